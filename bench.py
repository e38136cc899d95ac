"""Decode-attention throughput of the low-rank latent-KV path on one MI355X.

One step = append one token's latents to every sequence (quantise + pack)
and one decode step over the whole cache of the layer, on synthetic inputs
shaped like a LLaMA-7B-class attention layer serving a vision-language
decode (batch 16, 32 heads, head_dim 128, rank-32 per-head latents, int8 per
token, 4096 cached tokens of which 576 are image-prefix tokens, 128 decode
steps).  Prints one JSON line.

  value        whole-job tokens/s = batch * steps / wall time of the steps
  roofline     the decode kernel's algorithmic HBM bytes per launch divided
               by its average duration (HIP events on the launch stream)
  cpu_baseline the CPU oracle (plain fp64) timed on this host's cores on a
               sample of one step's (b, h) units, scaled to the whole step
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
    ap.add_argument("--warmup", type=int, default=8)
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
    ap.add_argument("--cold-steps", type=int, default=16,
                    help="extra untimed-in-value steps with the 256 MiB last-level cache flushed before each")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run warmup + this many steps (for rocprofv3); no CPU baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying one HIP graph")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (reads and writes that many "
                         "bytes), the reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


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


def cpu_baseline(run, n_units_target=128):
    """Time the oracle over a sample of step-0 units on the host's cores."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    w = run.w
    units = sorted(run.keep)[:n_units_target]
    jobs = [run.unit_inputs(u, 0) for u in units]
    threads = max(1, min(16, os.cpu_count() or 1))
    # repeat the sample until about 16 thread-seconds of oracle work are done
    passes, wall = 0, 0.0
    with ThreadPoolExecutor(threads) as pool:
        while passes == 0 or wall * threads < 16.0:
            t0 = time.perf_counter()
            list(pool.map(lambda j: oracle.attend(w.qfmt, *j, run.scale), jobs))
            wall += time.perf_counter() - t0
            passes += 1
    units_total = w.n_layers * w.batch * w.n_heads
    step_s = wall / passes * units_total / len(units)
    return {"value": w.batch / step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(units)} of {units_total} (b,h) units of decode step 0 "
                      f"(T={run.context + 1}), fp64 explicit reconstruction, {passes} passes; "
                      f"{wall:.2f} s wall on {threads} threads, per-pass time scaled "
                      f"x{units_total / len(units):.1f} to one step",
            "step_s": step_s}


def ffn_bench(args):
    """Hybrid FFN decode: `steps` evaluations of the LLaMA-7B-shaped hybrid FFN
    on 16 tokens, each seven launches, in one HIP graph."""
    import torch
    import lrgen
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
    layer(xs[0], y)
    for s in range(warm):
        layer(xs[s % 4], y)
    torch.cuda.synchronize()

    def run():
        for s in range(steps):
            layer(xs[s % 4], y)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run()
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = e0.elapsed_time(e1) / 1e3 / steps
    E, F, S, r, T = f.embed, f.hidden, f.n_lowrank, f.rank, f.tokens
    Fp = (F + 63) // 64 * 64
    weight_bytes = (2 * (F - S) * E + 2 * r * E + 2 * S * r + E * F) + 4 * (2 * (F - S) + 2 * r + 2 * S + E)
    inter = 2 * (T * 2 * r * 4) + 2 * (T * F * 4) + 2 * (T * Fp + T * (Fp // 64) * 4)
    step_bytes = weight_bytes + T * E * 2 + T * E * 4 + inter
    achieved = step_bytes / step_s / 1e9
    result = {
        "metric": "hybrid low-rank/dense W8A8 FFN decode tokens/sec (1 GPU) + achieved HBM GB/s",
        "value": T * steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": wall / steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": f.name, "embed": E, "hidden": F, "lowrank_channels": S, "rank": r,
                   "tokens": T, "weights": "int8 per-row scale", "activations": "int8 per token per 64",
                   "launches_per_step": 7, "launch": "hip graph of all timed steps"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_ffn_traffic(f.name),
                     "kernel": "k_ffn_quant + k_ffn_in + k_ffn_mid + "
                     "k_ffn_out + k_ffn_sum (one step)", "bytes_per_step": step_bytes,
                     "weight_bytes": weight_bytes, "avg_step_us": step_s * 1e6},
    }
    if not args.no_cpu_baseline:
        # the oracle as it stands (one call per step: it quantises the weights
        # and the activations, then evaluates in fp64; one thread), repeated
        # over whole steps until about 10 s of work are done
        import oracle
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        xh = [xx.float().cpu().numpy() for xx in xs]
        n, cpu_wall = 0, 0.0
        while n == 0 or cpu_wall < 10.0:
            t0 = time.perf_counter()
            oracle.ffn(xh[n % len(xh)], *w)
            cpu_wall += time.perf_counter() - t0
            n += 1
        result["cpu_baseline"] = {
            "value": T * n / cpu_wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole steps of {T} tokens (lro_ffn: W8A8 quantisation of weights and "
                      f"activations, then fp64), {cpu_wall:.2f} s on one thread"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU sharding is a design note, "
              "not an implemented path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.ffn:
        ffn_bench(args)
        return
    import torch
    import harness
    import lrgen
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
    n_cpu = 4 * w.n_heads if w.batch >= 4 else w.batch * w.n_heads
    keep = [] if (args.no_cpu_baseline or args.profile_steps) else \
        [(0, b, h) for b in range(min(w.batch, n_cpu // w.n_heads)) for h in range(w.n_heads)]
    nsteps_inputs = max(steps, warm, 1)
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    run = harness.WorkloadRun(w, io_dtype=LR_DT_BF16, device=dev, keep=keep,
                              steps=nsteps_inputs).setup()
    sess = run.sess
    L = w.n_layers
    ctx = run.context
    # every step's inputs are resident before timing: latents, q, pos, len
    per = []
    for s in range(nsteps_inputs):
        layers = []
        for l in range(L):
            ck, cv, q, pos = run.step_tensors(l, s)
            layers.append((ck, cv, q))
        ln = torch.full((w.batch,), ctx + s + 1, dtype=torch.int32, device=dev)
        pos = torch.full((w.batch,), ctx + s, dtype=torch.int32, device=dev)
        per.append((layers, pos, ln))
    out = torch.empty(w.batch, w.n_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    fused = not (args.explicit or args.separate_append)
    if args.with_projection and not fused:
        print("bench.py: --with-projection times the fused step only", file=sys.stderr)
        sys.exit(2)

    # latent generation: per layer the factors as [sum r, E] bf16 (A transposed),
    # per step and layer the new tokens' activations [B, E] bf16, and the fp32
    # latent buffers the projection writes
    proj = None
    if args.with_projection or not (args.no_projection_leg or args.profile_steps):
        for l in range(L):
            wk, wv = (lrgen.down_factors(w, l, kv, device=dev).t().contiguous().to(torch.bfloat16)
                      for kv in (0, 1))
            sess.set_projection(l, wk, wv)     # packed once per layer, as in serving
            del wk, wv
        wts = [sess.proj[l][1] for l in range(L)]
        xs = [[torch.cat([lrgen.activations(w, l, b, ctx + s, ctx + s + 1, device=dev)
                          for b in range(w.batch)]).to(torch.bfloat16).contiguous()
               for l in range(L)] for s in range(nsteps_inputs)]
        lat = [(torch.empty(w.batch, sess.latent_elems(l, 0), dtype=torch.float32, device=dev),
                torch.empty(w.batch, sess.latent_elems(l, 1), dtype=torch.float32, device=dev))
               for l in range(L)]
        proj = (wts, xs, lat)

    def one_layer(l, s, append=True, project=args.with_projection):
        """Step s of layer l: append the step's token and attend (one fused launch), or
        with append=False (separate launches only) just the decode launch."""
        layers, pos, ln = per[s]
        ck, cv, q = layers[l]
        if project:
            wts, xs, lat = proj
            ck, cv = sess.project(l, xs[s][l], ck=lat[l][0], cv=lat[l][1])
        if fused:
            sess.append_decode(l, ck.view(w.batch, -1), cv.view(w.batch, -1), pos, q, out,
                               ctx + s + 1, lengths=ln)
            return
        if append:
            sess.append(l, ck, cv, pos)
        sess.decode(l, q, out, ctx + s + 1, lengths=ln, explicit=args.explicit)

    def step(s):
        for l in range(L):
            one_layer(l, s)

    print(f"[bench] warmup {warm} steps", file=sys.stderr, flush=True)
    for s in range(warm):
        step(s)
    torch.cuda.synchronize()

    # ---- the timed steps: exactly `steps` steps from the configured context,
    # launched as one HIP graph (append + decode per step and layer) so the
    # host issues nothing per step.
    use_graph = not args.no_graph

    def timed_steps():
        for s in range(steps):
            step(s)

    def decodes_only():
        for s in range(steps):
            for l in range(L):
                one_layer(l, s, append=False, project=False)

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
        return g

    run_timed = capture(timed_steps).replay if use_graph else timed_steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_timed()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {steps} steps in {wall * 1e3:.2f} ms ({'graph' if use_graph else 'eager'})",
          file=sys.stderr, flush=True)

    # ---- the decode kernel alone: the same `steps` decode launches (each with
    # its step's lengths; fused: with its append) back to back, between two HIP
    # events on the launch stream; average launch duration = elapsed / launches.
    run_dec = capture(decodes_only).replay if use_graph else decodes_only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    run_dec()
    e1.record()
    torch.cuda.synchronize()
    dec_avg_s = e0.elapsed_time(e1) / (steps * L) / 1e3

    rk_all = w.ranks_k
    rv_all = w.ranks_v
    bytes_launch = 0.0
    per_tok_bytes = 0
    for s in range(steps):
        for l in range(L):
            b_, per_tok_bytes = algorithmic_bytes(w, [ctx + s + 1] * w.batch, rk_all[l], rv_all[l])
            bytes_launch += b_ + (append_bytes(w, rk_all[l], rv_all[l]) if fused else 0)
    bytes_launch /= steps * L
    achieved = bytes_launch / dec_avg_s / 1e9

    result = {
        "metric": "decode attention tokens/sec (1 GPU) + achieved HBM GB/s as % of MI355X peak",
        "value": w.batch * steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": wall / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "layers": L, "batch": w.batch, "heads": w.n_heads, "head_dim": w.head_dim,
            "rank": ("greedy allocation" if alloc_info else "per-head table") if w.uniform_rank is None
                    else w.uniform_rank,
            "context": ctx, "image_prefix": w.prefix,
            "latents": "int8 per-token fp32 scale" if w.qfmt == 0 else "int4 group-32 fp16 scale",
            "q_factors_out": "bf16", "accumulation": "f32",
            "decode_form": "explicit" if args.explicit else "absorbed",
            "step": "append fused into the decode launch" if fused else "append launch + decode launch",
            "parallelism": "single GPU",
            "launch": "hip graph of all timed steps" if use_graph else "eager",
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic(w.name, "explicit" if args.explicit else "absorbed"),
            "kernel": "k_decode_explicit" if args.explicit else "k_decode", "bytes_per_launch": bytes_launch,
            "bytes_per_token_per_bh": per_tok_bytes / w.n_heads,
            "avg_launch_us": dec_avg_s * 1e6,
        },
    }

    # ---- latent generation alone (outside the timed region): the projection
    # of each step's new tokens, every layer, back to back in a graph between
    # two HIP events (warm: the factors stay in the last-level cache), then
    # one launch at a time after a flush (cold, as when the factors of other
    # layers have been read in between).
    if proj is not None and not args.profile_steps:
        import latent_kv_attention_lr_amd as lrb
        wts, xs, lat = proj
        nrep = max(1, min(steps, 64))

        def proj_launch(s, l):
            # the current stream: torch's, or the capture stream inside capture()
            rc = lrb._lib.lr_attn_project_latent(
                sess.plan, l, xs[s][l].data_ptr(), w.batch, w.embed, wts[l].data_ptr(),
                lat[l][0].data_ptr(), lat[l][1].data_ptr(), torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"projection launch failed: {lrb.lr_attn_strerror(rc)}")

        def projections():
            for s in range(nrep):
                for l in range(L):
                    proj_launch(s, l)

        projections()
        run_proj = capture(projections).replay if use_graph else projections
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run_proj()
        e1.record()
        torch.cuda.synchronize()
        pw_s = e0.elapsed_time(e1) / (nrep * L) / 1e3
        pbytes = sum(projection_bytes(w, rk_all[l], rv_all[l], w.batch) for l in range(L)) / L
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        cold = []
        for s in range(min(16, nrep)):
            for l in range(L):
                flush.sum()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                proj_launch(s, l)
                b.record()
                cold.append((a, b))
        torch.cuda.synchronize()
        pc_s = sum(a.elapsed_time(b) for a, b in cold) / len(cold) / 1e3
        del flush
        result["latent_generation"] = {
            "kernel": "k_project", "entry_point": "lr_attn_project_latent",
            "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "tokens_per_launch": w.batch, "embed": w.embed,
            "bytes_per_launch": pbytes,
            "avg_launch_us": pw_s * 1e6, "achieved": pbytes / pw_s / 1e9,
            "frac": pbytes / pw_s / 1e9 / PEAK_HBM_GBS,
            "cold_avg_launch_us": pc_s * 1e6, "cold_achieved": pbytes / pc_s / 1e9,
            "cold_frac": pbytes / pc_s / 1e9 / PEAK_HBM_GBS,
            "traffic": measured_projection_traffic(w.name),
            "flops_per_launch": 2.0 * w.batch * w.embed * sum(sum(rk_all[l]) + sum(rv_all[l])
                                                              for l in range(L)) / L,
        }
        if args.with_projection:
            result["config"]["step"] = ("latent generation from activations, then append fused "
                                        "into the decode launch")

    # ---- MALL-cold decode timing (outside the timed region): flush first.
    # The launch between the two events goes straight to the C ABI with its
    # arguments prepared beforehand, so no host work sits between them.
    if args.cold_steps and not args.profile_steps:
        import latent_kv_attention_lr_amd as lrb
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)  # 512 MiB, read to evict
        stream = torch.cuda.current_stream().cuda_stream
        scale = 1.0 / math.sqrt(w.head_dim)
        cold = []
        for s in range(min(args.cold_steps, steps)):
            for l in range(L):
                layers, pos, ln = per[s]
                ck, cv, q = layers[l]
                common = (ln.data_ptr(), ctx + s + 1, q.data_ptr(), sess.bk[l].data_ptr(),
                          sess.bv[l].data_ptr(), scale, out.data_ptr(), sess.workspace.data_ptr(),
                          sess.workspace.numel(), stream)
                if fused:
                    fn, cargs = lrb._lib.lr_attn_append_decode, (
                        sess.plan, l, sess.caches[l].data_ptr(), ck.data_ptr(), cv.data_ptr(),
                        pos.data_ptr()) + common
                else:
                    sess.append(l, ck, cv, pos)
                    fn = lrb._lib.lr_attn_decode_explicit if args.explicit else lrb._lib.lr_attn_decode
                    cargs = (sess.plan, l, sess.caches[l].data_ptr()) + common
                flush.sum()                      # reads 512 MiB: the 256 MiB last-level cache holds none of the cache
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                rc = fn(*cargs)
                b.record()
                if rc != 0:
                    raise RuntimeError(f"decode launch failed: {lrb.lr_attn_strerror(rc)}")
                cold.append((a, b))
        torch.cuda.synchronize()
        cold_s = sum(a.elapsed_time(b) for a, b in cold) / len(cold) / 1e3
        result["roofline"]["cold_avg_launch_us"] = cold_s * 1e6
        result["roofline"]["cold_achieved"] = bytes_launch / cold_s / 1e9
        del flush

    # ---- practical read roof on this GPU (context for roofline.frac): a plain
    # streaming read of 1 GiB, which no last-level cache holds
    if not args.profile_steps:
        from latent_kv_attention_lr_amd import lr_attn_probe_read
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            lr_attn_probe_read(buf, buf.numel(), sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            lr_attn_probe_read(buf, buf.numel(), sink)
        e1.record()
        torch.cuda.synchronize()
        probe_gbs = buf.numel() * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
        result["roofline"]["stream_read_probe"] = {
            "value": probe_gbs, "unit": "GB/s", "frac_of_peak": probe_gbs / PEAK_HBM_GBS,
            "kernel": "lr_attn_probe_read", "bytes": buf.numel(),
            "achieved_vs_probe": achieved / probe_gbs}
        del buf, sink

    if alloc_info:
        result["rank_allocation"] = alloc_info
    if keep:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(run, n_cpu)
        cb.pop("step_s")
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
