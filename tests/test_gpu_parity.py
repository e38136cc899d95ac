"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* quantised latents: bit-exact codes and scale bits (hand-derived rows, random
  rows of every rank, and sampled rows of the five workloads' caches);
* decode outputs: |o_gpu - o_ref| <= 1e-2 max|o_ref| + 1e-3 (bf16) or
  <= 1e-4 max|o_ref| (fp32) on every unit of the small workload, on ragged
  and degenerate lengths, and on seeded samples of (layer, b, h) units of the
  four large workloads at their first, middle and last decode steps, in the
  launch configuration the benchmark uses.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import harness
import lrgen
import oracle
from latent_kv_attention_lr_amd import (LR_DT_BF16, LR_DT_F32, LR_EUNSUPPORTED, LR_Q_INT4_G32,
                                        LR_Q_INT8_TOKEN, LrAttnError, lr_attn_workspace_bytes)
from latent_kv_attention_lr_amd.session import DecodeSession
from gpu_util import TOL_BF16, TOL_F32, oracle_many, oracle_quant, read_codes, within

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def _val(v):
    return math.ldexp(v[0], v[1]) if isinstance(v, list) else float(v)


# ---------------------------------------------------------------------------
# quantise + append, bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_append_golden_rows_bitexact(fmt):
    cases = json.load(open(os.path.join(GOLD, "quant_cases.json")))[fmt]
    qfmt = LR_Q_INT8_TOKEN if fmt == "int8" else LR_Q_INT4_G32
    for c in cases:
        row = np.array([_val(v) for v in c["row"]], dtype=np.float32)
        r = len(row)
        say(f"append golden {fmt} {c['name']} r={r}")
        s = DecodeSession(1, 1, 1, 130, qfmt, LR_DT_BF16, [[r]], [[r]], device=DEV)
        ck = torch.from_numpy(row).view(1, 1, r).to(DEV)
        cv = torch.from_numpy(-row).view(1, 1, r).to(DEV)
        pos = torch.tensor([70], dtype=torch.int32, device=DEV)
        s.append(0, ck, cv, pos)
        torch.cuda.synchronize()
        cache = s.caches[0].cpu().numpy()
        hl = s.head_layout(0, 0)
        kq, ks = read_codes(cache, hl, qfmt, 0, [70], "k")
        vq, vs = read_codes(cache, hl, qfmt, 0, [70], "v")
        assert kq[0].tolist() == c["q"], c["why"]
        assert vq[0].tolist() == [-x for x in c["q"]], c["why"]
        if fmt == "int8":
            want = np.float32(np.abs(row).max()) / np.float32(127) if c["scale"] == "m/127" \
                else np.array([int(c["scale"], 16)], np.uint32).view(np.float32)[0]
            assert ks[0] == np.float32(want).view(np.uint32) and vs[0] == ks[0]
        else:
            assert [int(x) for x in ks[0]] == [int(h, 16) for h in c["scale"]]
            assert np.array_equal(vs, ks)


def _mixed_rows(rng, n, r):
    """Random rows over 40 binades, plus zero rows, rows with exact .5 ties at
    scale 1, and rows small enough that int4 group scales are fp16 subnormals
    or underflow."""
    c = rng.standard_normal((n, r)) * np.exp2(rng.integers(-30, 10, (n, 1)))
    c[0] = 0.0
    c[1] = np.round(rng.uniform(-126, 126, r)) + 0.5
    c[1, 0] = 127.0
    c[2] = np.round(rng.uniform(-6, 6, r)) + 0.5
    c[2, 0] = 7.0
    c[3] *= 1e-38
    c[4] = rng.standard_normal(r) * 1e-7
    c[5] = rng.standard_normal(r) * 3e-9
    return c.astype(np.float32)


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_append_random_rows_bitexact(qfmt):
    rng = np.random.default_rng(100 + qfmt)
    rk, rv = [8, 24, 48, 96, 128], [16, 40, 64, 88, 120]
    B, n_new, cap = 3, 70, 200
    s = DecodeSession(1, B, 5, cap, qfmt, LR_DT_BF16, [rk], [rv], device=DEV)
    ck = np.concatenate([_mixed_rows(rng, B * n_new, r) for r in rk], axis=1).reshape(B, n_new, sum(rk))
    cv = np.concatenate([_mixed_rows(rng, B * n_new, r) for r in rv], axis=1).reshape(B, n_new, sum(rv))
    pos = [0, 65, 180]  # row 2 runs past capacity: slots 200.. are dropped
    say(f"append random qfmt={qfmt}")
    s.append(0, torch.from_numpy(ck).to(DEV), torch.from_numpy(cv).to(DEV),
             torch.tensor(pos, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    cache = s.caches[0].cpu().numpy()
    ok, ov = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    for h in range(5):
        hl = s.head_layout(0, h)
        for b in range(B):
            n = min(n_new, cap - pos[b])
            slots = np.arange(pos[b], pos[b] + n)
            for kv, lat, off, r in (("k", ck, ok[h], rk[h]), ("v", cv, ov[h], rv[h])):
                got_q, got_s = read_codes(cache, hl, qfmt, b, slots, kv)
                want_q, want_s = oracle_quant(qfmt, lat[b, :n, off:off + r])
                assert np.array_equal(got_q, want_q), (h, b, kv)
                assert np.array_equal(got_s, want_s), (h, b, kv)
            if pos[b] + n_new > cap:  # the padding slots of the last tile stay untouched
                pad = np.arange(cap, 4 * 64)
                zq, zs = read_codes(cache, hl, qfmt, b, pad, "k")
                assert not zq.any() and not np.asarray(zs).any()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _check_units(run, units, s, tol, out):
    jobs = [run.unit_inputs(u, s) for u in units]
    refs = oracle_many(run.w.qfmt, jobs, run.scale)
    got = out.double().cpu().numpy()
    worst = 0.0
    for u, ref in zip(units, refs):
        _, b, h = u
        g = got[b, h]
        err = float(np.max(np.abs(g - ref)))
        bound = tol[0] * float(np.max(np.abs(ref))) + tol[1]
        worst = max(worst, err / bound)
        assert err <= bound, (u, s, err, bound)
    return worst


@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
def test_decode_small_workload_every_unit(io):
    w = lrgen.workload(0)
    units = [(0, 0, h) for h in range(w.n_heads)]
    say(f"decode small workload io={io}")
    run = harness.WorkloadRun(w, io_dtype=io, device=DEV, keep=units).setup()
    out = run.run_step(0, 0)
    torch.cuda.synchronize()
    _check_units(run, units, 0, TOL_BF16 if io == LR_DT_BF16 else TOL_F32, out)


def _session(qfmt, io, max_splits, rng, B, cap, rk, rv):
    """A session with random latents in every slot, random factors and q."""
    H = len(rk)
    s = DecodeSession(1, B, H, cap, qfmt, io, [rk], [rv], device=DEV, max_splits=max_splits)
    ck = (rng.standard_normal((B, cap, sum(rk))) * 1.3).astype(np.float32)
    cv = (rng.standard_normal((B, cap, sum(rv))) * 0.8).astype(np.float32)
    s.append(0, torch.from_numpy(ck).to(DEV), torch.from_numpy(cv).to(DEV),
             torch.zeros(B, dtype=torch.int32, device=DEV))
    dt = torch.bfloat16 if io == LR_DT_BF16 else torch.float32
    bk = (torch.from_numpy(rng.standard_normal((sum(rk), 128))) / 5).to(dt).to(DEV)
    bv = (torch.from_numpy(rng.standard_normal((sum(rv), 128))) / 5).to(dt).to(DEV)
    s.set_factors(0, bk.contiguous(), bv.contiguous())
    q = torch.from_numpy(rng.standard_normal((B, H, 128)) * 2).to(dt).to(DEV).contiguous()
    return s, rk, rv, ck, cv, bk, bv, q


def _ragged_session(qfmt, io, max_splits, rng):
    return _session(qfmt, io, max_splits, rng, 6, 700, [32, 8, 96], [64, 16, 40])


def _long_session(qfmt, io, max_splits, rng, rk=(32, 64), rv=(48, 64)):
    # 3 sequences x 2 heads over 8192 slots: few work-groups, so the launch
    # splits each context and merges the partials in a second kernel
    return _session(qfmt, io, max_splits, rng, 3, 8192, list(rk), list(rv))


# ranks 65-96: the int8 kernel puts two lanes on each token, except for a
# head whose ranks are at most 48 (the third), which keeps one lane per token
WIDE_RANKS = ((96, 40, 24), (72, 96, 48))


def _check_session(s, rk, rv, ck, cv, bk, bv, q, lens, qfmt, io, max_len, explicit=False):
    s.lengths.copy_(torch.tensor(lens, dtype=torch.int32))
    out = torch.full_like(q, float("nan"))
    s.decode(0, q, out, max_len=max_len, explicit=explicit)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    ok, ov = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    tol = TOL_BF16 if io == LR_DT_BF16 else TOL_F32
    qn, bkn, bvn = q.double().cpu().numpy(), bk.double().cpu().numpy(), bv.double().cpu().numpy()
    H = len(rk)
    jobs, keys = [], []
    for b, T in enumerate(lens):
        for h in range(H):
            jobs.append((ck[b, :T, ok[h]:ok[h] + rk[h]], cv[b, :T, ov[h]:ov[h] + rv[h]], qn[b, h],
                         bkn[ok[h]:ok[h] + rk[h]], bvn[ov[h]:ov[h] + rv[h]]))
            keys.append((b, h))
    refs = oracle_many(qfmt, jobs, 1 / math.sqrt(128))
    for (b, h), ref in zip(keys, refs):
        if lens[b] == 0:
            assert np.array_equal(got[b, h], np.zeros(128)), "empty context must give zeros"
        else:
            assert within(got[b, h], ref, tol), (b, h, lens[b])
    return out


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
@pytest.mark.parametrize("max_splits", [0, 1])
def test_decode_ragged_and_degenerate_lengths(qfmt, io, max_splits):
    rng = np.random.default_rng(7 + 2 * qfmt + io)
    say(f"decode ragged qfmt={qfmt} io={io} max_splits={max_splits}")
    sess = _ragged_session(qfmt, io, max_splits, rng)
    _check_session(*sess, [0, 1, 63, 64, 65, 700], qfmt, io, 700)


# Every tail width of the last 16-byte code chunk (int8 rows: 8 or 16 bytes;
# int4 rows: 4, 8, 12 or 16 bytes) and every int4 partial group, in the
# smallest, the paired-lane (int8) and the largest rank bucket.  In the 96
# bucket the int8 tail chunk falls to either lane of a token's pair, and the
# heads with both ranks at most 48 run one lane per token.
TAIL_RANKS = {
    32: ([8, 16, 24, 32], [24, 8, 32, 16]),
    96: ([8, 24, 40, 56, 72, 96, 16, 48, 88], [40, 16, 8, 88, 64, 8, 48, 24, 96]),
    128: ([8, 16, 24, 32, 56, 72, 112, 120], [120, 104, 88, 64, 48, 40, 16, 8]),
}


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
@pytest.mark.parametrize("bucket", [32, 96, 128])
def test_decode_every_row_tail_width(qfmt, io, bucket):
    rng = np.random.default_rng(90 + 4 * qfmt + 2 * io + (bucket == 128) + 8 * (bucket == 96))
    rk, rv = TAIL_RANKS[bucket]
    say(f"decode tail widths qfmt={qfmt} io={io} bucket={bucket}")
    sess = _session(qfmt, io, 0, rng, 4, 300, rk, rv)
    _check_session(*sess, [1, 64, 130, 300], qfmt, io, 300)
    if io == LR_DT_BF16:
        _check_session(*sess, [1, 64, 130, 300], qfmt, io, 300, explicit=True)


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_decode_explicit_ragged_and_degenerate_lengths(qfmt):
    rng = np.random.default_rng(50 + qfmt)
    say(f"decode explicit ragged qfmt={qfmt}")
    sess = _ragged_session(qfmt, LR_DT_BF16, 0, rng)
    _check_session(*sess, [0, 1, 63, 64, 65, 700], qfmt, LR_DT_BF16, 700, explicit=True)
    sess = _long_session(qfmt, LR_DT_BF16, 0, rng)
    _check_session(*sess, [100, 3001, 8192], qfmt, LR_DT_BF16, 8192, explicit=True)


def test_decode_explicit_rejects_fp32_io():
    rng = np.random.default_rng(1)
    s, rk, rv, ck, cv, bk, bv, q = _ragged_session(LR_Q_INT8_TOKEN, LR_DT_F32, 0, rng)
    with pytest.raises(LrAttnError) as e:
        s.decode(0, q, torch.empty_like(q), max_len=700, explicit=True)
    assert e.value.status == LR_EUNSUPPORTED


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
def test_decode_context_split_path(qfmt, io):
    rng = np.random.default_rng(30 + 2 * qfmt + io)
    sess = _long_session(qfmt, io, 0, rng)
    assert lr_attn_workspace_bytes(sess[0].plan, 8192) > 0, "this shape must split the context"
    say(f"decode split path qfmt={qfmt} io={io}")
    # one sequence within a single split, one ending inside a later split, one full
    _check_session(*sess, [100, 3001, 8192], qfmt, io, 8192)
    _check_session(*sess, [0, 8191, 2048], qfmt, io, 8192)
    sess = _long_session(qfmt, io, 0, rng, *WIDE_RANKS)
    assert lr_attn_workspace_bytes(sess[0].plan, 8192) > 0, "this shape must split the context"
    _check_session(*sess, [8192, 33, 4097], qfmt, io, 8192)


# Small heads in the paired-lane int8 buckets (both ranks at most 16, one lane
# per token, rows of at most one 16-byte chunk) beside a paired head and a
# one-lane head of rank 24 or 40 in the same launch; the lengths end on and
# around multiples of 3 and 4 tiles, leave some wavefronts without a step,
# and take the split and unsplit launches.
SMALL_RANKS = {
    128: ([128, 8, 16, 8, 16, 24], [8, 8, 16, 16, 8, 8]),
    96: ([96, 8, 16, 16, 40], [16, 8, 8, 16, 8]),
}
SMALL_LENS = [0, 1, 63, 64, 65, 192, 193, 256, 257, 700]


@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
@pytest.mark.parametrize("bucket", [96, 128])
def test_decode_small_heads_in_paired_buckets(io, bucket):
    qfmt = LR_Q_INT8_TOKEN
    rng = np.random.default_rng(140 + bucket + io)
    rk, rv = SMALL_RANKS[bucket]
    say(f"decode small heads io={io} bucket={bucket}")
    sess = _session(qfmt, io, 0, rng, len(SMALL_LENS), 700, rk, rv)
    _check_session(*sess, SMALL_LENS, qfmt, io, 700)
    # one split per work-group at most: the same heads, no context split
    sess = _session(qfmt, io, 1, rng, len(SMALL_LENS), 700, rk, rv)
    _check_session(*sess, SMALL_LENS, qfmt, io, 700)
    # context splits whose tile ranges need not be multiples of the step
    sess = _long_session(qfmt, io, 0, rng, (8, rk[0]), (16, rv[0]))
    assert lr_attn_workspace_bytes(sess[0].plan, 8192) > 0, "this shape must split the context"
    _check_session(*sess, [8192, 33, 4097], qfmt, io, 8192)
    _check_session(*sess, [100, 3001, 8191], qfmt, io, 8192)


def _fused_equals_separate(sess, lens, pos, max_len, seed):
    """append + decode and the fused append_decode write the same cache bytes
    and give the same outputs, bit for bit."""
    s, rk, rv, ck, cv, bk, bv, q = sess
    rng = np.random.default_rng(seed)
    B = s.batch
    nk = torch.from_numpy((rng.standard_normal((B, 1, sum(rk))) * 1.1).astype(np.float32)).to(DEV)
    nv = torch.from_numpy((rng.standard_normal((B, 1, sum(rv))) * 0.9).astype(np.float32)).to(DEV)
    posd = torch.tensor(pos, dtype=torch.int32, device=DEV)
    s.lengths.copy_(torch.tensor(lens, dtype=torch.int32))
    before = s.caches[0].clone()
    out_a = torch.full_like(q, float("nan"))
    s.append(0, nk, nv, posd)
    s.decode(0, q, out_a, max_len=max_len)
    torch.cuda.synchronize()
    cache_a = s.caches[0].clone()
    s.caches[0].copy_(before)
    out_b = torch.full_like(q, float("nan"))
    s.append_decode(0, nk.view(B, -1), nv.view(B, -1), posd, q, out_b, max_len=max_len)
    torch.cuda.synchronize()
    assert torch.equal(s.caches[0], cache_a), "fused append wrote different cache bytes"
    assert torch.equal(out_a, out_b), "fused decode differs from append + decode"
    return out_a


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
@pytest.mark.parametrize("io", [LR_DT_BF16, LR_DT_F32])
def test_append_decode_fused_equals_separate(qfmt, io):
    rng = np.random.default_rng(70 + 2 * qfmt + io)
    say(f"append_decode fused qfmt={qfmt} io={io}")
    sess = _ragged_session(qfmt, io, 0, rng)
    # the new token is the last attended one: slot 0, tile boundaries, the end
    lens = [1, 2, 64, 65, 300, 700]
    _fused_equals_separate(sess, lens, [n - 1 for n in lens], 700, 1)
    # slots outside the cache are skipped; a slot at or past len is written, not attended
    _fused_equals_separate(sess, [10, 700, 6, 50, 700, 1], [-1, 700, 5, 100, 699, 0], 700, 2)
    # context splits: the new token's tile in a later split of its (b, h)
    sess = _long_session(qfmt, io, 0, rng)
    lens = [100, 3001, 8192]
    _fused_equals_separate(sess, lens, [n - 1 for n in lens], 8192, 3)
    sess = _long_session(qfmt, io, 0, rng, *WIDE_RANKS)
    lens = [97, 4096, 8000]
    _fused_equals_separate(sess, lens, [n - 1 for n in lens], 8192, 4)
    if qfmt == LR_Q_INT8_TOKEN:   # small heads in the paired buckets: the new token at tile edges
        for bucket in (96, 128):
            rk, rv = SMALL_RANKS[bucket]
            sess = _session(qfmt, io, 0, rng, 6, 700, rk, rv)
            lens = [1, 65, 130, 195, 257, 700]
            _fused_equals_separate(sess, lens, [n - 1 for n in lens], 700, 5)
            _fused_equals_separate(sess, [64, 700, 6, 200, 700, 1], [0, 400, 5, 199, 699, 0], 700, 6)
        sess = _long_session(qfmt, io, 0, rng, (8, 128), (16, 8))
        lens = [100, 3001, 8192]
        _fused_equals_separate(sess, lens, [n - 1 for n in lens], 8192, 7)


def test_decode_max_len_clamps_longer_lengths():
    rng = np.random.default_rng(3)
    s, rk, rv, ck, cv, bk, bv, q = _ragged_session(LR_Q_INT8_TOKEN, LR_DT_F32, 0, rng)
    s.lengths.fill_(700)
    a = torch.empty_like(q)
    b = torch.empty_like(q)
    say("decode max_len clamp")
    s.decode(0, q, a, max_len=300)            # len 700 is clamped to max_len 300
    s.lengths.fill_(300)
    s.decode(0, q, b, max_len=300)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("which", ["ragged", "split"])
def test_decode_is_deterministic(which):
    rng = np.random.default_rng(11)
    mk = _ragged_session if which == "ragged" else _long_session
    s, rk, rv, ck, cv, bk, bv, q = mk(LR_Q_INT4_G32, LR_DT_BF16, 0, rng)
    cap = s.capacity
    s.lengths.fill_(cap)
    outs = []
    say(f"decode determinism {which}")
    for _ in range(3):
        o = torch.empty_like(q)
        s.decode(0, q, o, max_len=cap)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


# ---------------------------------------------------------------------------
# the four large workloads at full size, sampled units
# ---------------------------------------------------------------------------

STEPS_CHECKED = {1: [0, 63, 127], 2: [0, 63, 127], 3: [0], 4: [0, 31, 63]}
N_EXTRA = {1: 16, 2: 16, 3: 32, 4: 8}


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_workload_parity_full_size(idx):
    w = lrgen.workload(idx)
    units = harness.sample_units(w, N_EXTRA[idx], seed=1000 + idx)
    say(f"workload {idx} ({w.name}): setup, {len(units)} sampled units")
    run = harness.WorkloadRun(w, io_dtype=LR_DT_BF16, device=DEV, keep=units).setup()
    # quantised cache rows of the sampled units: bit-exact against the oracle
    rng = np.random.default_rng(idx)
    host_cache = {}
    for u in units[:: max(1, len(units) // 12)]:
        l, b, h = u
        hl = run.sess.head_layout(l, h)
        if l not in host_cache:
            host_cache[l] = run.sess.caches[l].cpu().numpy()
        cache = host_cache[l]
        ck, cv, _, _, _ = run.unit_inputs(u, run.steps - 1 if run.steps else 0)
        slots = np.unique(np.concatenate([rng.integers(0, run.context, 2048),
                                          np.arange(run.context - 3, run.context)]))
        for kv, lat in (("k", ck), ("v", cv)):
            got_q, got_s = read_codes(cache, hl, w.qfmt, b, slots, kv)
            want_q, want_s = oracle_quant(w.qfmt, lat[slots])
            assert np.array_equal(got_q, want_q), (u, kv)
            assert np.array_equal(got_s, want_s), (u, kv)
    del host_cache
    checked = STEPS_CHECKED[idx]
    worst = 0.0
    by_layer = {}
    for u in units:
        by_layer.setdefault(u[0], []).append(u)
    for l in range(w.n_layers):
        for s in range(w.steps):
            out = run.run_step(l, s)
            if s in checked and l in by_layer:
                torch.cuda.synchronize()
                say(f"workload {idx}: layer {l} step {s} check {len(by_layer[l])} units")
                worst = max(worst, _check_units(run, by_layer[l], s, TOL_BF16, out))
                if s == checked[0]:
                    _, _, q, _ = run.step_tensors(l, s)
                    ex = torch.empty_like(out)
                    run.sess.decode(l, q, ex, run.context + s + 1, explicit=True)
                    torch.cuda.synchronize()
                    say(f"workload {idx}: layer {l} step {s} explicit form")
                    worst = max(worst, _check_units(run, by_layer[l], s, TOL_BF16, ex))
    say(f"workload {idx}: worst error / bound = {worst:.3g}")


def test_graph_replay_matches_eager():
    """Append + decode steps captured in one HIP graph reproduce the eager
    outputs bit for bit on every replay (replays separated by eager work and
    synchronisations)."""
    w = lrgen.workload(0)
    steps = 4
    run = harness.WorkloadRun(w, io_dtype=LR_DT_BF16, device=DEV, steps=steps).setup()
    sess = run.sess
    ins = [run.step_tensors(0, s) for s in range(steps)]
    lens = [torch.full((w.batch,), run.context + s + 1, dtype=torch.int32, device=DEV)
            for s in range(steps)]
    outs = [torch.empty(w.batch, w.n_heads, 128, dtype=torch.bfloat16, device=DEV)
            for _ in range(steps)]

    def steps_fn():
        for s in range(steps):
            ck, cv, q, pos = ins[s]
            sess.append(0, ck, cv, pos)
            sess.decode(0, q, outs[s], run.context + s + 1, lengths=lens[s])

    say("graph: eager reference")
    steps_fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            steps_fn()
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s], ref[s]), (rep, s)


def test_probe_read_runs_and_leaves_memory_alone():
    """The streaming read probe (bandwidth context for the benchmark) reads
    every word of a buffer with a ragged tail and writes nothing else."""
    from latent_kv_attention_lr_amd import lr_attn_probe_read
    say("probe read")
    n = (1 << 20) + 48                      # not a multiple of the grid's 8 KiB stride
    buf = (torch.arange(n, device=DEV) % 251).to(torch.uint8)
    before = buf.clone()
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    lr_attn_probe_read(buf, n, sink)
    lr_attn_probe_read(buf, 16, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    # the sink is written only if the XOR of everything read equals the probe's
    # sentinel value; check that against the host's XOR of the same words
    words = before.cpu().numpy()[: n // 16 * 16].view("<u4")
    x = int(np.bitwise_xor.reduce(words))
    assert int(sink[0].item()) & 0xffffffff == (x if x == 0x9e3779b9 else 0)


# ---------------------------------------------------------------------------
# maximum sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_decode_all_128_heads(qfmt):
    """The largest head count a plan takes, with ranks 8..128 spread over the
    heads (K and V apart), so the layer runs the rank-128 kernel with every
    row width and, for int8, heads in both lane modes."""
    rng = np.random.default_rng(200 + qfmt)
    ranks = list(range(8, 129, 8))
    rk = [ranks[i % 16] for i in range(128)]
    rv = [ranks[(5 * i + 3) % 16] for i in range(128)]
    say(f"decode 128 heads qfmt={qfmt}")
    sess = _session(qfmt, LR_DT_BF16, 0, rng, 2, 200, rk, rv)
    _check_session(*sess, [200, 77], qfmt, LR_DT_BF16, 200)


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_decode_at_maximum_capacity(qfmt):
    """A context of 2^24 tokens, the largest capacity a plan takes: byte
    offsets past 4 GiB, hundreds of context splits and their merge.  Every K
    row is the same row, so all weights are equal; the V rows alternate
    between two rows, so the exact result is the oracle's for the two-token
    context made of those rows."""
    cap, r = 1 << 24, 128
    rng = np.random.default_rng(300 + qfmt)
    say(f"decode at capacity 2^24 qfmt={qfmt}")
    s = DecodeSession(1, 1, 1, cap, qfmt, LR_DT_BF16, [[r]], [[r]], device=DEV)
    assert lr_attn_workspace_bytes(s.plan, cap) > 0, "this shape must split the context"
    krow = (rng.standard_normal(r) * 1.3).astype(np.float32)
    vrows = (rng.standard_normal((2, r)) * 0.8).astype(np.float32)
    kd, vd = torch.from_numpy(krow).to(DEV), torch.from_numpy(vrows).to(DEV)
    chunk = 1 << 22
    for c0 in range(0, cap, chunk):
        ck = kd.view(1, 1, r).expand(1, chunk, r).contiguous()
        cv = vd.repeat(chunk // 2, 1).view(1, chunk, r)
        s.append(0, ck, cv, torch.tensor([c0], dtype=torch.int32, device=DEV))
        del ck, cv
    bk = (torch.from_numpy(rng.standard_normal((r, 128))) / 5).to(torch.bfloat16).to(DEV).contiguous()
    bv = (torch.from_numpy(rng.standard_normal((r, 128))) / 5).to(torch.bfloat16).to(DEV).contiguous()
    s.set_factors(0, bk, bv)
    q = torch.from_numpy(rng.standard_normal((1, 1, 128)) * 2).to(torch.bfloat16).to(DEV).contiguous()
    s.lengths.fill_(cap)
    out = torch.full_like(q, float("nan"))
    s.decode(0, q, out, cap)
    torch.cuda.synchronize()
    ref = oracle_many(qfmt, [(np.stack([krow, krow]), vrows, q.double().cpu().numpy()[0, 0],
                              bk.double().cpu().numpy(), bv.double().cpu().numpy())],
                      1 / math.sqrt(128))[0]
    assert within(out.double().cpu().numpy()[0, 0], ref, TOL_BF16)
    s.close()
