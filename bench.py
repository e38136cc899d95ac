"""Decode-attention throughput of the low-rank latent-KV path on one MI355X.

One step = append one token's latents to every sequence (quantise + pack)
and one decode step over the whole cache of the layer, on synthetic inputs
shaped like a LLaMA-7B-class attention layer serving a vision-language
decode (batch 16, 32 heads, head_dim 128, rank-32 per-head latents, int8 per
token, 4096 cached tokens of which 576 are image-prefix tokens, 128 decode
steps).  Prints one JSON line.

The layer's cache (156 MB) is smaller than MI355X's 256 MiB last-level cache,
so the timed steps cycle through copies of it, as the layers of a model do:
every launch reads its cache from HBM (MALL-cold).  The same launches on one
copy back to back are reported beside it as the warm figures.

  value        whole-job tokens/s = batch * steps * copies / wall time
  roofline     the decode kernel's algorithmic HBM bytes per launch divided
               by its average duration (HIP events on the launch stream
               around the graph of the timed launches)
  cpu_baseline the CPU oracle (plain fp64) timed on this host's threads on
               step 0 of whole batch rows (all of them when they fit about
               20 thread-seconds), scaled to the whole step
  parity       the GPU's step 0 against those oracle outputs, per (layer,
               b, h), with the decode tolerance of the parity tests
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "latent_kv_attention_lr_amd", "csrc", "kernels.hip")
PROJECT_SOURCE = os.path.join(ROOT, "latent_kv_attention_lr_amd", "csrc", "project.hip")
FFN_SOURCE = os.path.join(ROOT, "latent_kv_attention_lr_amd", "csrc", "ffn.hip")
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def measured_traffic(workload_name, kernel_form):
    """HBM bytes per decode launch from committed counter runs, if they were
    taken on the current kernel source (else None)."""
    import glob
    import hashlib
    src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    for f in glob.glob(os.path.join(TRAFFIC_DIR, "traffic_*.json")):
        d = json.load(open(f))
        if d.get("workload") == workload_name and d.get("decode_form") == kernel_form \
                and d.get("kernels_hip_sha256") == src:
            return d["hbm_bytes_per_launch"]
    return None


def measured_projection_traffic(workload_name):
    """HBM bytes per latent-generation launch from committed counter runs, if
    they were taken on the current projection source (else None)."""
    import hashlib
    src = hashlib.sha256(open(PROJECT_SOURCE, "rb").read()).hexdigest()
    f = os.path.join(TRAFFIC_DIR, f"traffic_{workload_name}_project.json")
    if os.path.exists(f):
        d = json.load(open(f))
        if d.get("project_hip_sha256") == src:
            return d["hbm_bytes_per_launch"]
    return None


def measured_ffn_traffic(workload_name):
    """HBM bytes per FFN step from committed counter runs on the current ffn.hip (else None)."""
    import hashlib
    src = hashlib.sha256(open(FFN_SOURCE, "rb").read()).hexdigest()
    f = os.path.join(TRAFFIC_DIR, f"traffic_{workload_name}_ffn.json")
    if os.path.exists(f):
        d = json.load(open(f))
        if d.get("ffn_hip_sha256") == src:
            return d["hbm_bytes_per_step"]
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=384,
                    help="untimed steps before the timed ones: up to 8 launched eagerly, the rest as "
                         "replays of the timed steps' graph (the GPU takes some 40 ms of sustained "
                         "load to reach its steady clocks)")
    ap.add_argument("--workload", type=int, default=1, help="index in the workload table")
    ap.add_argument("--explicit", action="store_true", help="time the explicit-reconstruction decode")
    ap.add_argument("--separate-append", action="store_true",
                    help="append and decode as two launches (default: one fused launch per step and layer)")
    ap.add_argument("--with-projection", action="store_true",
                    help="each step also generates the new token's latents from activations "
                         "(lr_attn_project_latent) before the fused append + decode")
    ap.add_argument("--no-projection-leg", action="store_true",
                    help="skip the separate latent-generation measurement")
    ap.add_argument("--allocate-ranks", type=int, default=0, metavar="MEAN",
                    help="replace the workload's rank table by the greedy allocation "
                         "(lr_attn_allocate_ranks) of synthetic component scores under a budget "
                         "of MEAN ranks per head and K/V")
    ap.add_argument("--ffn", action="store_true",
                    help="time the hybrid low-rank/dense W8A8 FFN decode (lr_ffn_decode) instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of the caches the timed steps cycle through (default: enough that "
                         "each launch reads its cache from HBM; 1 = one copy, partly cache-warm for "
                         "caches smaller than the 256 MiB last-level cache)")
    ap.add_argument("--wg-waves", type=int, default=0, choices=(0, 4, 8, 16),
                    help="wavefronts per decode work-group (0: the library's choice)")
    ap.add_argument("--no-warm-leg", action="store_true",
                    help="skip the warm measurement (one cache copy, launches back to back)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run warmup + this many steps (for rocprofv3); no CPU baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying one HIP graph")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (reads and writes that many "
                         "bytes), the reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# Warmup: the first steps are launched eagerly (module loads, first-touch
# allocations), the rest replay the graph of the timed steps.  From idle the
# GPU runs the first ~40 ms of a sustained load below its steady clocks
# (workload 1: the first two replays of the 128-step graph at 28.0 and 27.8
# us per launch, the third and later at 26.5), so the default warmup is three
# replays.
EAGER_WARMUP = 8


def warmup_passes(fn, steps_left, steps_per_pass):
    """Untimed calls of fn (one pass = steps_per_pass steps) until steps_left are done."""
    import torch
    while steps_left > 0:
        fn()
        steps_left -= max(steps_per_pass, 1)
    torch.cuda.synchronize()


def algorithmic_bytes(w, lens, rk, rv):
    """HBM bytes one decode launch must move at least: every cached code and
    scale of every (b, h) read once, both factor tensors, q and the output."""
    qf = w.qfmt
    per_tok = 0
    for h in range(w.n_heads):
        for r in (rk[h], rv[h]):
            rb = r if qf == 0 else r // 2
            sb = 4 if qf == 0 else 2 * ((r + 31) // 32)
            per_tok += rb + sb
    cache = sum(lens) * per_tok
    factors = (sum(rk) + sum(rv)) * w.head_dim * 2
    q_out = 2 * w.batch * w.n_heads * w.head_dim * 2
    return cache + factors + q_out, per_tok


def append_bytes(w, rk, rv):
    qf = w.qfmt
    row = 0
    for h in range(w.n_heads):
        for r in (rk[h], rv[h]):
            rb = r if qf == 0 else r // 2
            sb = 4 if qf == 0 else 2 * ((r + 31) // 32)
            row += 4 * r + rb + sb
    return w.batch * row


def projection_bytes(w, rk, rv, tokens):
    """Algorithmic HBM bytes of one latent-generation launch: the bf16 factors
    (E x sum r, K and V) once, the bf16 activations of the new tokens, and the
    fp32 latents written (the packed factors' zero rows past a multiple of 16
    are not counted)."""
    n = sum(rk) + sum(rv)
    return 2 * w.embed * n + 2 * tokens * w.embed + 4 * tokens * n


def host_threads():
    """Threads for the CPU baseline: the CPUs this process may run on, capped
    by OMP_NUM_THREADS where the host sets it (a shared host's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# fp64 multiply-adds per second of one host thread running the oracle
# (measured on an x86 host); only used to size the CPU sample beforehand
ORACLE_FMA_PER_S = 1.3e9
CPU_SAMPLE_THREAD_S = 20.0


def cpu_sample_units(w):
    """The (layer, b, h) units whose step-0 decode the oracle is timed on:
    whole batch rows (every layer and head of them), as many as fit about
    CPU_SAMPLE_THREAD_S thread-seconds of oracle work; all units when the
    whole step fits.  Every batch row does the same work, so the time of the
    rows scales exactly to the step."""
    T = w.context + 1
    row_fma = sum(T * (rk + rv) * w.head_dim
                  for l in range(w.n_layers) for rk, rv in zip(w.ranks_k[l], w.ranks_v[l]))
    rows = int(max(1, min(w.batch, CPU_SAMPLE_THREAD_S * ORACLE_FMA_PER_S // row_fma)))
    return [(l, b, h) for l in range(w.n_layers) for b in range(rows) for h in range(w.n_heads)], rows


def cpu_baseline(run, rows):
    """Time the oracle on step 0 of the sampled batch rows, on the host's threads."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    w = run.w
    units = sorted(run.keep)
    threads = host_threads()
    jobs = [run.unit_inputs(u, 0) for u in units]
    # one untimed unit pages the oracle library and the inputs in
    oracle.attend(w.qfmt, *jobs[0], run.scale)
    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        refs = list(pool.map(lambda j: oracle.attend(w.qfmt, *j, run.scale), jobs))
        wall = time.perf_counter() - t0
    step_s = wall * w.batch / rows
    whole = rows == w.batch
    units_total = w.n_layers * w.batch * w.n_heads
    return {"value": w.batch / step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"decode step 0 (T={run.context + 1}), {len(units)} of {units_total} "
                       f"(layer, b, h) units = batch rows 0..{rows - 1} of {w.batch}"
                       + ("" if whole else f", time scaled x{w.batch / rows:g} to the whole step "
                                           "(every batch row does the same work)")
                       + f"; fp64 explicit reconstruction; {wall:.2f} s wall on {threads} threads"),
            "extrapolated": not whole,
            "cpu_model": cpu_model(),
            "host_cpus_visible": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
            else os.cpu_count(),
            "step_s": step_s, "refs": dict(zip(units, refs))}


# Decode output tolerance with bf16 q, factors and output (the parity tests'):
# |o_gpu - o_ref| <= 1e-2 max|o_ref| + 1e-3, per (layer, b, h).
TOL_BF16 = (1e-2, 1e-3)


def parity_report(refs, got):
    """Step 0 of the GPU against the oracle outputs the CPU baseline computed
    (refs: unit -> fp64 [d]; got: layer -> fp64 [B, H, d])."""
    import numpy as np
    worst, max_abs, fails = 0.0, 0.0, 0
    for (l, b, h), ref in refs.items():
        err = float(np.max(np.abs(got[l][b, h] - ref)))
        bound = TOL_BF16[0] * float(np.max(np.abs(ref))) + TOL_BF16[1]
        worst, max_abs = max(worst, err / bound), max(max_abs, err)
        fails += err > bound
    return {"units": len(refs), "step": 0, "tolerance": "|o - o_ref| <= 1e-2 max|o_ref| + 1e-3 per (layer, b, h)",
            "worst_err_over_bound": worst, "max_abs_err": max_abs, "units_over_bound": fails,
            "source": "the oracle outputs of the cpu_baseline leg"}


def ffn_bench(args):
    """Hybrid FFN decode: `steps` evaluations of the LLaMA-7B-shaped hybrid FFN
    on 16 tokens, each four launches, in one HIP graph.  The packed weights
    (110 MB) fit the last-level cache, so the timed steps cycle through copies
    of them (each step reads its weights from HBM, as the layers of a model
    do); the same steps on one copy are reported as warm_*."""
    import torch
    import lrgen
    import latent_kv_attention_lr_amd as lrb
    from latent_kv_attention_lr_amd.ffn import FfnLayer
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    f = lrgen.FFN_WORKLOADS[0]
    steps = 128 if args.steps is None else args.steps
    warm = args.warmup
    print(f"[bench] setting up {f.name}", file=sys.stderr, flush=True)
    w = lrgen.ffn_weights(f)
    layer = FfnLayer(f.embed, f.hidden, f.n_lowrank, f.rank, device=dev)
    layer.set_weights(*w)
    xs = [lrgen.ffn_activations(lrgen.FfnWorkload(f.name, f.embed, f.hidden, f.n_lowrank, f.rank, f.tokens,
                                                   f.seed + 1 + s), f.tokens).to(dev) for s in range(4)]
    y = torch.empty(f.tokens, f.embed, dtype=torch.float32, device=dev)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    layer(xs[0], y)        # sizes the workspace
    R = choose_replicas(layer.weights.numel(), args.replicas)
    copies = [layer.weights] + [layer.weights.clone() for _ in range(R - 1)]
    ws = layer.workspace
    dp = ctypes_byref(layer.desc)

    def step(s, wt, st):
        rc = lrb._lib.lr_ffn_decode(dp, wt.data_ptr(), xs[s % 4].data_ptr(), f.tokens, y.data_ptr(),
                                    ws.data_ptr(), ws.numel(), st)
        if rc != 0:
            raise RuntimeError(f"lr_ffn_decode failed: {lrb.lr_attn_strerror(rc)}")

    def run(cs):
        def fn():
            st = torch.cuda.current_stream().cuda_stream
            for s in range(steps):
                for c in cs:
                    step(s, c, st)
        return fn

    eager_warm = min(warm, EAGER_WARMUP)
    for s in range(eager_warm):
        for c in copies:
            step(s, c, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    def graph_time(fn):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn()
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        warmup_passes(g.replay, warm - eager_warm - steps, steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    wall, ev = graph_time(run(copies))
    step_s = ev / (steps * R)
    E, F, S, r, T = f.embed, f.hidden, f.n_lowrank, f.rank, f.tokens
    Fp = (F + 63) // 64 * 64
    weight_bytes = (2 * (F - S) * E + 2 * r * E + 2 * S * r + E * F) + 4 * (2 * (F - S) + 2 * r + 2 * S + E)
    inter = 2 * (T * 2 * r * 4) + 2 * (T * F * 4) + 2 * (T * Fp + T * (Fp // 64) * 4)
    step_bytes = weight_bytes + T * E * 2 + T * E * 4 + inter
    achieved = step_bytes / step_s / 1e9
    result = {
        "metric": "hybrid low-rank/dense W8A8 FFN decode tokens/sec (1 GPU) + achieved HBM GB/s",
        "value": T * steps * R / wall, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": wall / (steps * R) * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8-weights,int8-activations,f32-acc", "data": "synthetic",
        "config": {"workload": f.name, "embed": E, "hidden": F, "lowrank_channels": S, "rank": r,
                   "tokens": T, "weights": "int8 per-row scale", "activations": "int8 per token per 64",
                   "launches_per_step": 4, "launch": "hip graph of all timed steps",
                   "weight_copies": R,
                   "mall": "cold: a weight byte is read again only after %.0f MB of weight reads"
                           % (R * layer.weights.numel() / 1e6)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_ffn_traffic(f.name),
                     "kernel": "k_ffn_quant + k_ffn_in + k_ffn_mid or k_ffn_mid_out + k_ffn_out (one step)",
                     "bytes_per_step": step_bytes,
                     "weight_bytes": weight_bytes, "avg_step_us": step_s * 1e6, "mall": "cold"},
    }
    if not args.no_warm_leg:
        wall_w, ev_w = graph_time(run([copies[0]]))
        result["roofline"]["warm_avg_step_us"] = ev_w / steps * 1e6
        result["roofline"]["warm_frac"] = step_bytes / (ev_w / steps) / 1e9 / PEAK_HBM_GBS
        result["warm_value"] = T * steps / wall_w
    del copies
    if not args.no_cpu_baseline:
        # the oracle as it stands (one call per step: it quantises the weights
        # and the activations, then evaluates in fp64; one thread), repeated
        # over whole steps until about 10 s of work are done
        import oracle
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        xh = [xx.float().cpu().numpy() for xx in xs]
        layer(xs[0], y)                   # the GPU's step for the first input, compared below
        torch.cuda.synchronize()
        y0 = y.double().cpu().numpy()
        n, cpu_wall, y_ref = 0, 0.0, None
        while n == 0 or cpu_wall < 10.0:
            t0 = time.perf_counter()
            yo = oracle.ffn(xh[n % len(xh)], *w)
            cpu_wall += time.perf_counter() - t0
            if n == 0:
                y_ref = yo
            n += 1
        result["cpu_baseline"] = {
            "value": T * n / cpu_wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole steps of {T} tokens (lro_ffn: W8A8 quantisation of weights and "
                      f"activations, then fp64), {cpu_wall:.2f} s on one thread",
            "cpu_model": cpu_model()}
        rel = abs(y0 - y_ref).max(axis=1) / abs(y_ref).max(axis=1)
        result["parity"] = {
            "tokens": T, "max_rel_err_per_token": float(rel.max()),
            "note": "one step of the GPU against the oracle output of the cpu_baseline leg, "
                    "|y - y_ref| / max|y_ref| per token; the parity tests bound each element "
                    "from the oracle's intermediates (fp32 sums, activation codes near a rounding boundary)"}
    print(json.dumps(result), flush=True)


def ctypes_byref(desc):
    import ctypes
    return ctypes.byref(desc)


MALL_BYTES = 256 << 20     # MI355X last-level cache (Infinity Cache)


def choose_replicas(total_cache_bytes, requested):
    """Copies of the layer stack's caches that the timed steps cycle through.
    Between two visits of one copy the other copies are read, so with at
    least twice the last-level cache of other bytes in between every launch
    reads its cache from HBM, as a layer of a deep model does.  Caches that
    are already that large need no copy."""
    if requested:
        return requested
    if total_cache_bytes >= 2 * MALL_BYTES:
        return 1
    return int(min(64, math.ceil(2 * MALL_BYTES / total_cache_bytes) + 1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; sharding across GPUs is described, not implemented "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.ffn:
        ffn_bench(args)
        return
    import torch
    import harness
    import lrgen
    import latent_kv_attention_lr_amd as lrb
    from latent_kv_attention_lr_amd import LR_DT_BF16

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = lrgen.workload(args.workload)
    alloc_info = None
    if args.allocate_ranks:
        from latent_kv_attention_lr_amd import lr_attn_allocate_ranks
        cost = w.embed + w.head_dim
        budget = w.n_layers * w.n_heads * 2 * args.allocate_ranks * cost
        scores = lrgen.component_scores(w.seed, w.n_layers, w.n_heads).numpy()
        t_alloc = time.perf_counter()
        rk, rv = lr_attn_allocate_ranks(scores, cost, budget)
        t_alloc = time.perf_counter() - t_alloc
        w.ranks_k, w.ranks_v, w.uniform_rank = rk.tolist(), rv.tolist(), None
        w.name += f"-allocated-mean{args.allocate_ranks}"
        alloc_info = {"entry_point": "lr_attn_allocate_ranks", "scores": "synthetic (lrgen.component_scores)",
                      "budget_params": budget, "mean_rank": args.allocate_ranks,
                      "rank_min": int(min(rk.min(), rv.min())), "rank_max": int(max(rk.max(), rv.max())),
                      "host_ms": t_alloc * 1e3}
    steps = w.steps if args.steps is None else args.steps
    warm = args.warmup
    if args.profile_steps:
        steps = args.profile_steps
    fused = not (args.explicit or args.separate_append)
    if args.with_projection and not fused:
        print("bench.py: --with-projection times the fused step only", file=sys.stderr)
        sys.exit(2)
    cpu_rows = 0
    keep = []
    if not (args.no_cpu_baseline or args.profile_steps):
        keep, cpu_rows = cpu_sample_units(w)
    eager_warm = min(warm, EAGER_WARMUP)
    nsteps_inputs = max(steps, eager_warm, 1)
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    run = harness.WorkloadRun(w, io_dtype=LR_DT_BF16, device=dev, keep=keep,
                              steps=nsteps_inputs, wg_waves=args.wg_waves).setup()
    sess = run.sess
    L = w.n_layers
    ctx = run.context
    B = w.batch
    scale = 1.0 / math.sqrt(w.head_dim)
    # every step's inputs are resident before timing: latents, q, pos, len
    per = []
    for s in range(nsteps_inputs):
        layers = []
        for l in range(L):
            ck, cv, q, pos = run.step_tensors(l, s)
            layers.append((ck, cv, q))
        ln = torch.full((B,), ctx + s + 1, dtype=torch.int32, device=dev)
        pos = torch.full((B,), ctx + s, dtype=torch.int32, device=dev)
        per.append((layers, pos, ln))
    out = torch.empty(B, w.n_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- copies of the prefilled caches: the timed steps visit copy 0, 1, ..,
    # R-1 of every layer in turn, so each launch finds its cache outside the
    # last-level cache (as layer l of a model does after the other layers ran)
    total_cache = sum(sess.caches[l].numel() for l in range(L))
    R = choose_replicas(total_cache, args.replicas)
    caches = [[sess.caches[l]] + [sess.caches[l].clone() for _ in range(R - 1)] for l in range(L)]
    reuse_bytes = R * total_cache     # cache bytes read between two reads of one byte
    torch.cuda.synchronize()

    # latent generation: per layer (and copy) the factors as [sum r, E] bf16
    # (A transposed), packed once; per step and layer the new tokens'
    # activations [B, E] bf16, and the fp32 latent buffers the projection writes
    proj = None
    want_proj = args.with_projection or not (args.no_projection_leg or args.profile_steps)
    if want_proj:
        packed = []
        for l in range(L):
            wk, wv = (lrgen.down_factors(w, l, kv, device=dev).t().contiguous().to(torch.bfloat16)
                      for kv in (0, 1))
            sess.set_projection(l, wk, wv)     # packed once per layer, as in serving
            del wk, wv
            packed.append(sess.proj[l][1])
        xs = [[torch.cat([lrgen.activations(w, l, b, ctx + s, ctx + s + 1, device=dev)
                          for b in range(B)]).to(torch.bfloat16).contiguous()
               for l in range(L)] for s in range(nsteps_inputs)]
        lat = [(torch.empty(B, sess.latent_elems(l, 0), dtype=torch.float32, device=dev),
                torch.empty(B, sess.latent_elems(l, 1), dtype=torch.float32, device=dev))
               for l in range(L)]
        # the split projection of the one-step path: parts per layer, partial sums
        parts = [lrb.lr_attn_project_parts(sess.plan, l, B, w.embed) for l in range(L)]
        plat = [(torch.empty(parts[l], B, sess.latent_elems(l, 0), dtype=torch.float32, device=dev),
                 torch.empty(parts[l], B, sess.latent_elems(l, 1), dtype=torch.float32, device=dev))
                for l in range(L)]
        step_ws = torch.empty(lrb.lr_attn_project_decode_workspace_bytes(sess.plan, sess.capacity, w.embed),
                              dtype=torch.uint8, device=dev)
        proj = (packed, xs, lat)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: {lrb.lr_attn_strerror(rc)}")

    lib = lrb._lib
    ws_ptr, ws_n = sess.workspace.data_ptr(), sess.workspace.numel()

    def project(l, s, st, wts=None):
        packed, xs, lat = proj
        check(lib.lr_attn_project_latent(sess.plan, l, xs[s][l].data_ptr(), B, w.embed,
                                         (wts or packed)[l].data_ptr(), lat[l][0].data_ptr(),
                                         lat[l][1].data_ptr(), st), "lr_attn_project_latent")
        return lat[l]

    def project_split(l, s, st, wts):
        packed, xs, lat = proj
        check(lib.lr_attn_project_latent_parts(sess.plan, l, xs[s][l].data_ptr(), B, w.embed,
                                               wts[l].data_ptr(), parts[l], plat[l][0].data_ptr(),
                                               plat[l][1].data_ptr(), st), "lr_attn_project_latent_parts")

    def one_step(l, s, r, st, wts):
        """Step s of layer l on cache copy r from activations: lr_attn_project_append_decode."""
        packed, xs, lat = proj
        layers, pos, ln = per[s]
        q = layers[l][2]
        check(lib.lr_attn_project_append_decode(
            sess.plan, l, caches[l][r].data_ptr(), xs[s][l].data_ptr(), w.embed, wts[l].data_ptr(),
            pos.data_ptr(), ln.data_ptr(), ctx + s + 1, q.data_ptr(), sess.bk[l].data_ptr(),
            sess.bv[l].data_ptr(), scale, out.data_ptr(), step_ws.data_ptr(), step_ws.numel(), st),
            "lr_attn_project_append_decode")

    def launch(l, s, r, st, append=True, project_first=False, wts=None):
        """Step s of layer l on cache copy r, on stream st: append the step's token and
        attend (one fused launch), or append and decode launches; with append=False
        (separate launches only) just the decode launch.  project_first: the whole
        step from activations (lr_attn_project_append_decode)."""
        if project_first:
            one_step(l, s, r, st, wts or proj[0])
            return
        layers, pos, ln = per[s]
        ck, cv, q = layers[l]
        cache = caches[l][r].data_ptr()
        common = (ln.data_ptr(), ctx + s + 1, q.data_ptr(), sess.bk[l].data_ptr(),
                  sess.bv[l].data_ptr(), scale, out.data_ptr(), ws_ptr, ws_n, st)
        if fused:
            check(lib.lr_attn_append_decode(sess.plan, l, cache, ck.data_ptr(), cv.data_ptr(),
                                            pos.data_ptr(), *common), "lr_attn_append_decode")
            return
        if append:
            check(lib.lr_attn_append_latent(sess.plan, l, cache, ck.data_ptr(), cv.data_ptr(),
                                            pos.data_ptr(), 1, st), "lr_attn_append_latent")
        fn = lib.lr_attn_decode_explicit if args.explicit else lib.lr_attn_decode
        check(fn(sess.plan, l, cache, *common), "decode")

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def steps_all(copies, **kw):
        def fn():
            st = cur()
            for s in range(steps):
                for l in range(L):
                    for r in copies:
                        launch(l, s, r, st, **kw)
        return fn

    print(f"[bench] warmup {warm} steps, {R} cache cop{'y' if R == 1 else 'ies'}", file=sys.stderr,
          flush=True)
    for s in range(eager_warm):
        st = cur()
        for l in range(L):
            for r in range(R):
                launch(l, s, r, st, project_first=args.with_projection)
    torch.cuda.synchronize()

    use_graph = not args.no_graph

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn()
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()                          # the first replay uploads the graph: untimed
        torch.cuda.synchronize()
        return g.replay

    def timed(fn):
        """(wall seconds, event seconds) of one call of fn, HIP events on the current stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    # ---- the timed steps: exactly `steps` steps of every cache copy from the
    # configured context, as one HIP graph, so the host issues nothing per step
    run_timed = steps_all(range(R), project_first=args.with_projection)
    timed_fn = capture(run_timed) if use_graph else run_timed   # capturing replays it once
    warmup_passes(timed_fn, warm - eager_warm - (steps if use_graph else 0), steps)
    wall, ev = timed(timed_fn)
    launches = steps * L * R
    print(f"[bench] timed {steps} steps x {R} copies in {wall * 1e3:.2f} ms "
          f"({'graph' if use_graph else 'eager'})", file=sys.stderr, flush=True)

    # ---- the decode kernel alone.  Fused: the timed launches are exactly the
    # decode launches (with their appends).  Otherwise the same decode launches
    # without the append launches, in a graph of their own.
    if fused and not args.with_projection:
        dec_s = ev / launches
    else:
        dec_only = steps_all(range(R), append=False)
        if fused:
            dec_only = steps_all(range(R))
        _, ev_d = timed(capture(dec_only) if use_graph else dec_only)
        dec_s = ev_d / launches
    rk_all, rv_all = w.ranks_k, w.ranks_v
    bytes_launch = 0.0
    per_tok_bytes = 0
    for s in range(steps):
        for l in range(L):
            b_, per_tok_bytes = algorithmic_bytes(w, [ctx + s + 1] * B, rk_all[l], rv_all[l])
            bytes_launch += b_ + (append_bytes(w, rk_all[l], rv_all[l]) if fused else 0)
    bytes_launch /= steps * L
    achieved = bytes_launch / dec_s / 1e9
    lat_dtype = "int8" if w.qfmt == 0 else "int4"
    result = {
        "metric": "decode attention tokens/sec (1 GPU) + achieved HBM GB/s as % of MI355X peak",
        "value": B * steps * R / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": wall / (steps * R) * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{lat_dtype}-latent,bf16-io,f32-acc",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "layers": L, "batch": B, "heads": w.n_heads, "head_dim": w.head_dim,
            "rank": ("greedy allocation" if alloc_info else "per-head table") if w.uniform_rank is None
                    else w.uniform_rank,
            "context": ctx, "image_prefix": w.prefix,
            "latents": "int8 per-token fp32 scale" if w.qfmt == 0 else "int4 group-32 fp16 scale",
            "q_factors_out": "bf16", "accumulation": "f32",
            "decode_form": "explicit" if args.explicit else "absorbed",
            "step": ("latent generation from activations, then append fused into the decode launch"
                     if args.with_projection else
                     "append fused into the decode launch" if fused else "append launch + decode launch"),
            "parallelism": "single GPU",
            "launch": "hip graph of all timed steps" if use_graph else "eager",
            "cache_copies": R,
            **({"wg_waves": args.wg_waves} if args.wg_waves else {}),
            "mall": ("cold: a cache byte is read again only after %.0f MB of cache reads "
                     "(last-level cache 268 MB)" % (reuse_bytes / 1e6)) if reuse_bytes >= 2 * MALL_BYTES
                    else ("partly warm: a cache byte is read again after %.0f MB of cache reads"
                          % (reuse_bytes / 1e6)),
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic(w.name, "explicit" if args.explicit else "absorbed"),
            "kernel": "k_decode_explicit" if args.explicit else "k_decode", "bytes_per_launch": bytes_launch,
            "bytes_per_token_per_bh": per_tok_bytes / w.n_heads,
            "avg_launch_us": dec_s * 1e6,
            "mall": "cold" if reuse_bytes >= 2 * MALL_BYTES else "partly warm",
        },
    }

    # ---- warm leg (outside the timed region): the same decode launches on one
    # cache copy back to back, so part of a cache smaller than the last-level
    # cache is still there from the previous step
    if not (args.no_warm_leg or args.profile_steps) and R > 1 and total_cache < MALL_BYTES:
        warm_fn = steps_all([0])
        wall_w, ev_w = timed(capture(warm_fn) if use_graph else warm_fn)
        if fused and not args.with_projection:
            warm_s = ev_w / (steps * L)
            result["roofline"]["warm_avg_launch_us"] = warm_s * 1e6
            result["roofline"]["warm_achieved"] = bytes_launch / warm_s / 1e9
            result["roofline"]["warm_frac"] = bytes_launch / warm_s / 1e9 / PEAK_HBM_GBS
        result["warm_value"] = B * steps / wall_w

    # ---- latent generation alone (outside the timed region): the projection
    # of each step's new tokens on copies of the packed factors, cycled so that
    # each launch reads its factors from HBM (cold), and on one copy back to
    # back (warm: the factors stay in the last-level cache)
    if proj is not None and not args.profile_steps:
        packed, xs, lat = proj
        nrep = max(1, min(steps, 64))
        pbytes = sum(projection_bytes(w, rk_all[l], rv_all[l], B) for l in range(L)) / L
        packed_total = sum(p.numel() * 2 for p in packed)
        Rp = choose_replicas(packed_total, 0)
        pcopies = [packed] + [[p.clone() for p in packed] for _ in range(Rp - 1)]

        def projections(copies, fn1):
            def fn():
                st = cur()
                for s in range(nrep):
                    for l in range(L):
                        for r in copies:
                            fn1(l, s, st, pcopies[r])
            return fn

        def cold_warm(fn1):
            _, ev_c = timed(capture(projections(range(Rp), fn1)) if use_graph else projections(range(Rp), fn1))
            _, ev_w = timed(capture(projections([0], fn1)) if use_graph else projections([0], fn1))
            return ev_c / (nrep * L * Rp), ev_w / (nrep * L)

        pc_s, pw_s = cold_warm(project_split)
        uc_s, uw_s = cold_warm(project)
        # parts partial sums are written and read once more by the decode launch
        pbytes_split = sum(projection_bytes(w, rk_all[l], rv_all[l], B * parts[l]) -
                           2 * B * parts[l] * w.embed + 2 * B * w.embed for l in range(L)) / L
        result["latent_generation"] = {
            "kernel": "k_project", "entry_point": "lr_attn_project_latent_parts",
            "parts": parts[0] if L == 1 else parts,
            "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "tokens_per_launch": B, "embed": w.embed,
            "bytes_per_launch": pbytes_split,
            "avg_launch_us": pc_s * 1e6, "achieved": pbytes_split / pc_s / 1e9,
            "frac": pbytes_split / pc_s / 1e9 / PEAK_HBM_GBS,
            "mall": "cold", "factor_copies": Rp,
            "warm_avg_launch_us": pw_s * 1e6, "warm_achieved": pbytes_split / pw_s / 1e9,
            "warm_frac": pbytes_split / pw_s / 1e9 / PEAK_HBM_GBS,
            "traffic": measured_projection_traffic(w.name),
            "flops_per_launch": 2.0 * B * w.embed * sum(sum(rk_all[l]) + sum(rv_all[l])
                                                        for l in range(L)) / L,
            "unsplit": {"entry_point": "lr_attn_project_latent", "bytes_per_launch": pbytes,
                        "avg_launch_us": uc_s * 1e6, "frac": pbytes / uc_s / 1e9 / PEAK_HBM_GBS,
                        "warm_avg_launch_us": uw_s * 1e6,
                        "warm_frac": pbytes / uw_s / 1e9 / PEAK_HBM_GBS},
        }
        # ---- a whole step from activations: latents generated from x, then
        # the fused append + decode, every layer's factors and cache cold
        if fused:
            def from_x():
                st = cur()
                for s in range(steps):
                    for l in range(L):
                        for r in range(R):
                            launch(l, s, r, st, project_first=True, wts=pcopies[r % Rp])
            wall_x, ev_x = timed(capture(from_x) if use_graph else from_x)
            step_x = ev_x / (steps * R)
            xbytes = bytes_launch + pbytes
            result["step_from_activations"] = {
                "entry_point": "lr_attn_project_append_decode",
                "tokens_per_s": B * steps * R / wall_x, "us_per_step": step_x * 1e6,
                "launches_per_layer": 2, "bytes_per_layer": xbytes,
                "achieved": xbytes * L / step_x / 1e9,
                "frac": xbytes * L / step_x / 1e9 / PEAK_HBM_GBS,
            }
        del pcopies

    # ---- practical read roof on this GPU (context for roofline.frac): a plain
    # streaming read of 1 GiB, which no last-level cache holds
    if not args.profile_steps:
        from latent_kv_attention_lr_amd import lr_attn_probe_read
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            lr_attn_probe_read(buf, buf.numel(), sink)
        _, ev_p = timed(lambda: [lr_attn_probe_read(buf, buf.numel(), sink) for _ in range(10)])
        probe_gbs = buf.numel() * 10 / ev_p / 1e9
        result["roofline"]["stream_read_probe"] = {
            "value": probe_gbs, "unit": "GB/s", "frac_of_peak": probe_gbs / PEAK_HBM_GBS,
            "kernel": "lr_attn_probe_read", "bytes": buf.numel(),
            "achieved_vs_probe": achieved / probe_gbs}
        del buf, sink

    if alloc_info:
        result["rank_allocation"] = alloc_info
    if keep:
        # step 0 once more on cache copy 0 (its token rewritten with the same
        # codes, the later steps' tokens beyond the length): the outputs the
        # oracle is compared with, per layer of the sampled units
        got = {}
        for l in sorted({u[0] for u in keep}):
            launch(l, 0, 0, cur(), project_first=False)
            got[l] = out.double().cpu().numpy()
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(run, cpu_rows)
        cb.pop("step_s")
        refs = cb.pop("refs")
        result["cpu_baseline"] = cb
        result["parity"] = parity_report(refs, got)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
