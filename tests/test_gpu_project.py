"""GPU parity of latent generation (c = x A on the matrix cores) and of the
generate-then-append entry point, through the C ABI, against the CPU oracle.

* inputs whose every fp32 sum is exact in any order (small integers, one-hot
  rows): bit-exact latents;
* random bf16 inputs of the workloads' shapes and distributions (outlier
  channels included): every latent within the worst-case fp32 summation bound
  2 (E-1) u sum_e |x_e a_e| (u = 2^-24; the factor 2 also covers additions
  that truncate), and an RMS error within 8 sqrt(E) u of the RMS latent, which
  a dropped or doubled term exceeds by orders of magnitude;
* lr_attn_project_append writes exactly the bytes of project + append; its
  codes are valid roundings of the oracle's latents; decode over a cache
  built from activations matches the oracle's whole chain within the decode
  tolerance.
"""
import math

import numpy as np
import pytest
import torch

import lrgen
import oracle
from latent_kv_attention_lr_amd import LR_DT_BF16, LR_Q_INT4_G32, LR_Q_INT8_TOKEN
from latent_kv_attention_lr_amd.session import DecodeSession
from gpu_util import TOL_BF16, read_codes, within

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U32 = 2.0 ** -24


def say(msg):
    print(msg, flush=True)


def _session(ranks_k, ranks_v, qfmt=LR_Q_INT8_TOKEN, batch=1, cap=64):
    return DecodeSession(1, batch, len(ranks_k), cap, qfmt, LR_DT_BF16, [list(ranks_k)],
                         [list(ranks_v)], device=DEV)


def _factors(E, ranks, key, std):
    """Down-projection factor A [E, sum r] ~ N(0, std^2), rounded to bf16 (fp32 array)."""
    n = E * sum(ranks)
    a = lrgen.normal(key, 0, n, std).view(E, sum(ranks)).to(torch.bfloat16).float()
    return a


def _set_factors(s, ak, av):
    """Pack A^K, A^V (fp32 arrays holding bf16 values, [E, N]) through the library."""
    wk = ak.t().contiguous().to(torch.bfloat16).to(DEV)
    wv = av.t().contiguous().to(torch.bfloat16).to(DEV)
    s.set_projection(0, wk, wv)
    return wk, wv


def _gpu_project(s, x_bf, ak, av):
    """Pack the factors, run lr_attn_project_latent, return host latents."""
    _set_factors(s, ak, av)
    ck, cv = s.project(0, x_bf.to(DEV).contiguous())
    torch.cuda.synchronize()
    return ck.cpu().numpy(), cv.cpu().numpy()


def _oracle_ref(x, a, rows=None):
    """The oracle's latents x A and the magnitudes |x| |A| that bound their rounding."""
    x64 = x.double().numpy() if rows is None else x.double().numpy()[rows]
    a64 = a.double().numpy()
    return oracle.latents(x64, a64), oracle.latents(np.abs(x64), np.abs(a64))


def _check_bound(got, x, a, rows=None, pre=None):
    """Worst-case and RMS rounding checks of fp32 latents against the oracle
    (pre: _oracle_ref(x, a, rows), when several results share it)."""
    E = x.shape[1]
    ref, mag = _oracle_ref(x, a, rows) if pre is None else pre
    g = got if rows is None else got[rows]
    err = np.abs(g.astype(np.float64) - ref)
    bound = 2.0 * (E - 1) * U32 * mag * 1.01 + U32 * np.abs(ref)
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    rms_ref = math.sqrt(float(np.mean(ref ** 2)))
    rms_err = math.sqrt(float(np.mean(err ** 2)))
    assert rms_err <= 8.0 * math.sqrt(E) * U32 * rms_ref, (rms_err, rms_ref)
    return ref


@pytest.mark.parametrize("E,T", [(32, 1), (96, 5), (1024, 16), (1024, 17), (1024, 40), (1024, 64),
                                 (1024, 65), (1024, 130), (4096, 3), (4128, 33), (2080, 48)])
def test_project_integer_inputs_bitexact(E, T):
    """Small-integer x and A (exact in bf16) keep every partial sum an integer
    below 2^24, so any summation order gives the exact product."""
    ranks_k, ranks_v = [8, 32, 24], [16, 40, 8]
    say(f"project integers E={E} T={T}")
    rng = np.random.default_rng(E * 1000 + T)
    s = _session(ranks_k, ranks_v)
    x = torch.from_numpy(rng.integers(-3, 4, (T, E)).astype(np.float32))
    ak = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_k))).astype(np.float32))
    av = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_v))).astype(np.float32))
    ck, cv = _gpu_project(s, x.to(torch.bfloat16), ak, av)
    assert np.array_equal(ck, oracle.latents(x.double().numpy(), ak.double().numpy()).astype(np.float32))
    assert np.array_equal(cv, oracle.latents(x.double().numpy(), av.double().numpy()).astype(np.float32))


@pytest.mark.parametrize("T", [49, 64, 100])
def test_project_two_tile_units_straddle_k_and_v(T):
    """From 49 tokens on, a work-group takes two row tiles.  With 3 K tiles and
    4 V tiles (the last one half full) one work-group holds K's last tile and
    V's first, and the last work-group's second tile is past the end: every
    latent still lands exactly where it belongs (integer inputs, exact)."""
    E, ranks_k, ranks_v = 1024, [8, 24, 16], [16, 8, 32]
    say(f"project two-tile units T={T}")
    rng = np.random.default_rng(T)
    s = _session(ranks_k, ranks_v)
    x = torch.from_numpy(rng.integers(-3, 4, (T, E)).astype(np.float32))
    ak = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_k))).astype(np.float32))
    av = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_v))).astype(np.float32))
    ck, cv = _gpu_project(s, x.to(torch.bfloat16), ak, av)
    assert np.array_equal(ck, oracle.latents(x.double().numpy(), ak.double().numpy()).astype(np.float32))
    assert np.array_equal(cv, oracle.latents(x.double().numpy(), av.double().numpy()).astype(np.float32))


def test_project_one_hot_rows_pick_factor_rows():
    """x_t = e_j gives row j of A exactly: every token and every latent lands
    at its own place (tokens across column tiles, rows across row tiles)."""
    E, ranks_k, ranks_v = 256, [32, 8, 56, 16, 8], [8, 8, 8, 8, 40]
    s = _session(ranks_k, ranks_v)
    idx = [(7 * t + 3) % E for t in range(70)]
    x = torch.zeros(len(idx), E)
    x[torch.arange(len(idx)), torch.tensor(idx)] = 1.0
    ak = _factors(E, ranks_k, lrgen.stream_key(9, 1), 1.0)
    av = _factors(E, ranks_v, lrgen.stream_key(9, 2), 1.0)
    ck, cv = _gpu_project(s, x.to(torch.bfloat16), ak, av)
    assert np.array_equal(ck, ak.numpy()[idx])
    assert np.array_equal(cv, av.numpy()[idx])


def test_pack_layout_matches_its_definition():
    """The packed buffer holds, for tile r, step c, lane l, element i: row
    16 r' + l % 16 of W^K (or W^V past the K tiles), column 32 c + 8 (l / 16)
    + i, zeros past the last row -- checked byte for byte."""
    E, ranks_k, ranks_v = 96, [8, 24, 40], [16, 8, 8]
    s = _session(ranks_k, ranks_v)
    rng = np.random.default_rng(7)
    wk = rng.integers(0, 1 << 16, (sum(ranks_k), E)).astype(np.uint16)
    wv = rng.integers(0, 1 << 16, (sum(ranks_v), E)).astype(np.uint16)
    wk_t = torch.from_numpy(wk.view(np.int16)).view(torch.bfloat16).to(DEV)
    wv_t = torch.from_numpy(wv.view(np.int16)).view(torch.bfloat16).to(DEV)
    s.set_projection(0, wk_t, wv_t)
    torch.cuda.synchronize()
    got = s.proj[0][1].view(torch.int16).cpu().numpy().view(np.uint16)
    want = []
    for w in (wk, wv):
        tiles = -(-w.shape[0] // 16)
        wpad = np.zeros((tiles * 16, E), np.uint16)
        wpad[:w.shape[0]] = w
        for r in range(tiles):
            for c in range(E // 32):
                for l in range(64):
                    row, col = 16 * r + l % 16, 32 * c + 8 * (l // 16)
                    want.append(wpad[row, col:col + 8])
    assert np.array_equal(got, np.concatenate(want))


def _workload_inputs(idx, T, layer=0):
    w = lrgen.workload(idx)
    x = torch.cat([lrgen.activations(w, layer, b, w.context, w.context + 1) for b in range(T)])
    ak = lrgen.down_factors(w, layer, 0).to(torch.bfloat16).float()
    av = lrgen.down_factors(w, layer, 1).to(torch.bfloat16).float()
    return w, x.to(torch.bfloat16), ak, av


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_project_workload_shapes_within_rounding_bound(idx):
    """Each workload's layer (E, ranks) with one new token per sequence, as in
    a decode step (batch tokens; workload 2 has its 20x outlier channels);
    oracle on every token for the small batches, on 8 sampled tokens else."""
    w = lrgen.workload(idx)
    say(f"project workload {idx} E={w.embed} T={w.batch}")
    w, x, ak, av = _workload_inputs(idx, w.batch)
    s = _session(w.ranks_k[0], w.ranks_v[0], w.qfmt, batch=w.batch)
    ck, cv = _gpu_project(s, x, ak, av)
    rows = None if w.batch <= 16 else np.random.default_rng(idx).choice(w.batch, 8, replace=False)
    _check_bound(ck, x.float(), ak, rows)
    _check_bound(cv, x.float(), av, rows)


def test_project_many_tokens_and_is_deterministic():
    """A prefill-sized call (several token blocks, a ragged last one) and
    bitwise-identical results on a second call."""
    E, ranks_k, ranks_v, T = 1024, [32] * 8, [24, 40] * 4, 1000
    s = _session(ranks_k, ranks_v)
    x = lrgen.normal(lrgen.stream_key(12, 0), 0, T * E, 1.0).view(T, E).to(torch.bfloat16)
    ak = _factors(E, ranks_k, lrgen.stream_key(12, 1), 1 / math.sqrt(E))
    av = _factors(E, ranks_v, lrgen.stream_key(12, 2), 1 / math.sqrt(E))
    ck, cv = _gpu_project(s, x, ak, av)
    rows = np.random.default_rng(0).choice(T, 24, replace=False)
    rows = np.concatenate([rows, [0, 63, 64, 999]])
    _check_bound(ck, x.float(), ak, rows)
    _check_bound(cv, x.float(), av, rows)
    ck2, cv2 = s.project(0, x.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(ck, ck2.cpu().numpy()) and np.array_equal(cv, cv2.cpu().numpy())


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_project_append_equals_project_then_append(qfmt):
    """The combined entry point writes exactly the bytes of the two calls,
    for one and for several new tokens per sequence."""
    E, ranks_k, ranks_v, B = 512, [8, 64, 32, 96], [40, 16, 128, 8], 3
    ak = _factors(E, ranks_k, lrgen.stream_key(13, 1), 1 / math.sqrt(E))
    av = _factors(E, ranks_v, lrgen.stream_key(13, 2), 1 / math.sqrt(E))
    for n_new in (1, 5, 70):
        say(f"project_append qfmt={qfmt} n_new={n_new}")
        x = lrgen.normal(lrgen.stream_key(13, n_new), 0, B * n_new * E, 1.0).view(B, n_new, E)
        x = x.to(torch.bfloat16).to(DEV)
        pos = torch.tensor([0, 3, 60][:B], dtype=torch.int32, device=DEV)
        a = _session(ranks_k, ranks_v, qfmt, batch=B, cap=140)
        b = _session(ranks_k, ranks_v, qfmt, batch=B, cap=140)
        _set_factors(a, ak, av)
        _set_factors(b, ak, av)
        a.project_append(0, x, pos)
        ck, cv = b.project(0, x)
        b.append(0, ck, cv, pos)
        torch.cuda.synchronize()
        assert torch.equal(a.caches[0], b.caches[0])


@pytest.mark.parametrize("qfmt", [LR_Q_INT8_TOKEN, LR_Q_INT4_G32])
def test_project_append_codes_are_roundings_of_oracle_latents(qfmt):
    """Codes and scales written from activations, against the oracle's
    latents c_ref: with e the latent error bound, each scale is within
    max(e)/L (plus its own rounding) of the oracle's, and each code within
    1/2 + e/s (plus the division's rounding) of clip(c_ref / s, -L, L), L =
    127 or 7."""
    w = lrgen.workload(2 if qfmt == LR_Q_INT4_G32 else 1)
    B = 16
    w, x, ak, av = _workload_inputs(w.index, B)
    ranks_k, ranks_v = w.ranks_k[0], w.ranks_v[0]
    s = _session(ranks_k, ranks_v, qfmt, batch=B, cap=64)
    _set_factors(s, ak, av)
    pos = torch.full((B,), 5, dtype=torch.int32, device=DEV)
    s.project_append(0, x.view(B, 1, -1).to(DEV), pos)
    torch.cuda.synchronize()
    cache = s.caches[0].cpu().numpy()
    E = w.embed
    x64 = x.double().numpy()
    lim = 127 if qfmt == LR_Q_INT8_TOKEN else 7
    srel = 2 * U32 if qfmt == LR_Q_INT8_TOKEN else 2.0 ** -10   # fp32 / fp16 scale rounding
    for kv, a, offs, ranks in (("k", ak, lrgen.head_offsets(ranks_k), ranks_k),
                               ("v", av, lrgen.head_offsets(ranks_v), ranks_v)):
        ref = oracle.latents(x64, a.double().numpy())
        mag = oracle.latents(np.abs(x64), np.abs(a.double().numpy()))
        bound = 2.0 * (E - 1) * U32 * mag * 1.01 + U32 * np.abs(ref)
        for h in range(0, len(ranks), 5):
            o, r = offs[h], ranks[h]
            hl = s.head_layout(0, h)
            for b in range(B):
                q, sc = read_codes(cache, hl, qfmt, b, [5], kv)
                c = ref[b, o:o + r]
                e = bound[b, o:o + r]
                if qfmt == LR_Q_INT8_TOKEN:
                    scale = np.full(r, float(sc.view(np.float32)[0]))
                    groups = [(0, r)]
                else:
                    g = np.array([oracle.f16_bits_to_f32(int(v)) for v in sc[0]], np.float64)
                    scale = np.repeat(g, 32)[:r]
                    groups = [(lo, min(r, lo + 32)) for lo in range(0, r, 32)]
                for lo, hi in groups:
                    s_ref = float(np.max(np.abs(c[lo:hi]))) / lim
                    tol = float(np.max(e[lo:hi])) / lim + srel * max(s_ref, scale[lo])
                    assert abs(scale[lo] - s_ref) <= tol, (kv, h, b, lo, scale[lo], s_ref)
                want = np.clip(c / scale, -lim, lim)
                slack = e / scale + 2 * lim * U32
                assert np.all(np.abs(q[0].astype(np.float64) - want) <= 0.5 + slack), (kv, h, b)


def _step_parts(s, E):
    """Projection parts of the fused step, read back from the workspace size
    (n_parts blocks of [batch][sum r] fp32 partials, K then V, 256-aligned)."""
    from latent_kv_attention_lr_amd import (lr_attn_project_decode_workspace_bytes,
                                            lr_attn_workspace_bytes)
    pbytes = (lr_attn_project_decode_workspace_bytes(s.plan, s.capacity, E)
              - lr_attn_workspace_bytes(s.plan, s.capacity))
    nk, nv = s.latent_elems(0, 0), s.latent_elems(0, 1)
    for parts in range(1, 9):
        r256 = lambda n: (n + 255) // 256 * 256
        if r256(parts * s.batch * nk * 4) + r256(parts * s.batch * nv * 4) == pbytes:
            return parts
    raise AssertionError(f"no part count gives {pbytes} bytes")


@pytest.mark.parametrize("E,B,ranks_k,ranks_v,parts", [
    (1024, 1, [8, 32, 24], [16, 40, 8], 4),
    (2080, 5, [8, 64, 32, 96], [40, 16, 128, 8], 8),
    (4096, 64, [8, 64, 32, 96], [40, 16, 128, 8], 1),
    (4096, 16, [32] * 32, [32] * 32, 4),
])
def test_project_append_decode_integer_inputs_equal_two_calls(E, B, ranks_k, ranks_v, parts):
    """With small-integer activations and factors every partial sum is exact,
    so the split projection's parts, added in order inside the fused append,
    give exactly lr_attn_project_latent's latents: cache bytes and outputs of
    the one-step entry point equal project_latent + append_decode bit for bit
    (part counts 1 to 8, one- and two-tile projection shapes)."""
    say(f"project_append_decode integers E={E} B={B} heads={len(ranks_k)}")
    rng = np.random.default_rng(E + B)
    H, ctx = len(ranks_k), 150
    a = _session(ranks_k, ranks_v, batch=B, cap=ctx + 1)
    b = _session(ranks_k, ranks_v, batch=B, cap=ctx + 1)
    assert _step_parts(a, E) == parts
    ak = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_k))).astype(np.float32))
    av = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_v))).astype(np.float32))
    for s in (a, b):
        _set_factors(s, ak, av)
    bk = torch.from_numpy(rng.standard_normal((sum(ranks_k), 128)) / 6).to(torch.bfloat16).to(DEV)
    bv = torch.from_numpy(rng.standard_normal((sum(ranks_v), 128)) / 6).to(torch.bfloat16).to(DEV)
    pk = torch.from_numpy(rng.standard_normal((B, ctx, sum(ranks_k))).astype(np.float32)).to(DEV)
    pv = torch.from_numpy(rng.standard_normal((B, ctx, sum(ranks_v))).astype(np.float32)).to(DEV)
    for s in (a, b):
        s.set_factors(0, bk, bv)
        s.append(0, pk, pv, torch.zeros(B, dtype=torch.int32, device=DEV))
    x = torch.from_numpy(rng.integers(-3, 4, (B, E)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    q = torch.from_numpy(rng.standard_normal((B, H, 128))).to(torch.bfloat16).to(DEV)
    pos = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    oa = torch.empty(B, H, 128, dtype=torch.bfloat16, device=DEV)
    ob = torch.empty_like(oa)
    a.lengths.fill_(ctx + 1)
    b.lengths.fill_(ctx + 1)
    a.project_append_decode(0, x, pos, q, oa, ctx + 1)
    ck, cv = b.project(0, x)
    b.append_decode(0, ck, cv, pos, q, ob, ctx + 1)
    torch.cuda.synchronize()
    assert torch.equal(a.caches[0], b.caches[0])
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_project_append_decode_full_layer_shape_matches_oracle_chain():
    """The one-step entry point at the int8 workload's layer shape (E 4096,
    batch 16, 32 heads of rank 32, four projection parts): random activations
    of the workload's distribution, a 300-token prefix generated the same way;
    sampled units match the oracle's chain x -> latents -> quantise -> attend."""
    w = lrgen.workload(1)
    E, H, B, ctx = w.embed, w.n_heads, w.batch, 300
    rk, rv = w.ranks_k[0], w.ranks_v[0]
    s = DecodeSession(1, B, H, ctx + 1, w.qfmt, LR_DT_BF16, [rk], [rv], device=DEV)
    assert _step_parts(s, E) == 4
    ak = lrgen.down_factors(w, 0, 0).to(torch.bfloat16).float()
    av = lrgen.down_factors(w, 0, 1).to(torch.bfloat16).float()
    bk = lrgen.up_factors(w, 0, 0).to(DEV).contiguous()
    bv = lrgen.up_factors(w, 0, 1).to(DEV).contiguous()
    s.set_factors(0, bk, bv)
    _set_factors(s, ak, av)
    xs = torch.stack([lrgen.activations(w, 0, b, 0, ctx + 1) for b in range(B)]).to(torch.bfloat16)
    s.project_append(0, xs[:, :ctx].contiguous().to(DEV), torch.zeros(B, dtype=torch.int32, device=DEV))
    q = lrgen.queries(w, 0, 0).to(DEV).contiguous()
    out = torch.empty(B, H, w.head_dim, dtype=torch.bfloat16, device=DEV)
    s.lengths.fill_(ctx + 1)
    s.project_append_decode(0, xs[:, ctx].contiguous().to(DEV),
                            torch.full((B,), ctx, dtype=torch.int32, device=DEV), q, out, ctx + 1)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    scale = 1.0 / math.sqrt(w.head_dim)
    offk, offv = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    for b in (0, 11):
        say(f"full-shape step, oracle chain row {b}")
        ref_k = oracle.latents(xs[b].double().numpy(), ak.double().numpy()).astype(np.float32)
        ref_v = oracle.latents(xs[b].double().numpy(), av.double().numpy()).astype(np.float32)
        for h in range(0, H, 3):
            ref = oracle.attend(w.qfmt, ref_k[:, offk[h]:offk[h] + rk[h]], ref_v[:, offv[h]:offv[h] + rv[h]],
                                q[b, h].double().cpu().numpy(),
                                bk[offk[h]:offk[h] + rk[h]].double().cpu().numpy(),
                                bv[offv[h]:offv[h] + rv[h]].double().cpu().numpy(), scale)
            assert within(got[b, h], ref, TOL_BF16), (b, h)


@pytest.mark.parametrize("idx,T", [(1, 16), (4, 8), (2, 64)])
def test_project_parts_sum_to_latents_within_rounding_bound(idx, T):
    """lr_attn_project_latent_parts at a workload's decode shape (one- and
    two-tile instances): one part is lr_attn_project_latent bit for bit; for
    2 to 8 parts the parts added in order stay within the fp32 summation bound
    of the oracle's latents."""
    from latent_kv_attention_lr_amd import lr_attn_project_latent_parts
    w, x, ak, av = _workload_inputs(idx, T)
    s = _session(w.ranks_k[0], w.ranks_v[0], w.qfmt, batch=1, cap=64)
    wk, wv = _set_factors(s, ak, av)
    xd = x.to(torch.bfloat16).to(DEV).contiguous()
    T, E = xd.shape
    nk, nv = s.latent_elems(0, 0), s.latent_elems(0, 1)
    ck1, cv1 = s.project(0, xd)
    xb = x.to(torch.bfloat16).float()
    pre_k, pre_v = _oracle_ref(xb, ak), _oracle_ref(xb, av)   # shared by every part count
    for parts in range(1, 9):
        say(f"project parts workload {idx} parts={parts}")
        pk = torch.empty(parts, T, nk, dtype=torch.float32, device=DEV)
        pv = torch.empty(parts, T, nv, dtype=torch.float32, device=DEV)
        lr_attn_project_latent_parts(s.plan, 0, xd, T, E, s.proj[0][1], parts, pk, pv)
        torch.cuda.synchronize()
        if parts == 1:
            assert torch.equal(pk[0], ck1) and torch.equal(pv[0], cv1)
        sk, sv = pk[0].clone(), pv[0].clone()
        for q in range(1, parts):
            sk += pk[q]
            sv += pv[q]
        _check_bound(sk.cpu().numpy(), xb, ak, pre=pre_k)
        _check_bound(sv.cpu().numpy(), xb, av, pre=pre_v)


@pytest.mark.parametrize("T", [1, 16, 40, 64, 100])
def test_project_parts_integer_inputs_sum_exactly(T):
    """Small-integer inputs: every part's sums are exact, so for any part
    count the parts added in order equal the oracle's latents exactly (one-,
    two- and three-block and two-tile instances, E of 65 steps so that parts
    are uneven)."""
    from latent_kv_attention_lr_amd import lr_attn_project_latent_parts
    ranks_k, ranks_v, E = [8, 64, 32, 96], [40, 16, 128, 8], 2080
    rng = np.random.default_rng(T)
    s = _session(ranks_k, ranks_v)
    x = torch.from_numpy(rng.integers(-3, 4, (T, E)).astype(np.float32))
    ak = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_k))).astype(np.float32))
    av = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_v))).astype(np.float32))
    _set_factors(s, ak, av)
    ref_k = oracle.latents(x.double().numpy(), ak.double().numpy()).astype(np.float32)
    ref_v = oracle.latents(x.double().numpy(), av.double().numpy()).astype(np.float32)
    xd = x.to(torch.bfloat16).to(DEV).contiguous()
    for parts in (1, 2, 3, 5, 8):
        say(f"project parts integers T={T} parts={parts}")
        pk = torch.empty(parts, T, sum(ranks_k), dtype=torch.float32, device=DEV)
        pv = torch.empty(parts, T, sum(ranks_v), dtype=torch.float32, device=DEV)
        lr_attn_project_latent_parts(s.plan, 0, xd, T, E, s.proj[0][1], parts, pk, pv)
        torch.cuda.synchronize()
        sk, sv = pk[0].clone(), pv[0].clone()
        for q in range(1, parts):
            sk += pk[q]
            sv += pv[q]
        assert np.array_equal(sk.cpu().numpy(), ref_k) and np.array_equal(sv.cpu().numpy(), ref_v)


@pytest.mark.parametrize("one_step", [False, True])
def test_decode_over_generated_latents_matches_oracle_chain(one_step):
    """Cache built by project_append from activations (prefill in chunks, then
    decode steps generating the new token's latents and attending with the
    fused append, as two calls or through the one-step entry point): outputs
    match the oracle's chain x -> latents -> quantise -> attend within the
    decode tolerance."""
    w = lrgen.workload(0)
    E, H, B, ctx, steps = w.embed, w.n_heads, 2, 100, 3
    rk, rv = w.ranks_k[0], w.ranks_v[0]
    s = DecodeSession(1, B, H, ctx + steps, w.qfmt, LR_DT_BF16, [rk], [rv], device=DEV)
    ak = lrgen.down_factors(w, 0, 0).to(torch.bfloat16).float()
    av = lrgen.down_factors(w, 0, 1).to(torch.bfloat16).float()
    bk = lrgen.up_factors(w, 0, 0).to(DEV).contiguous()
    bv = lrgen.up_factors(w, 0, 1).to(DEV).contiguous()
    s.set_factors(0, bk, bv)
    _set_factors(s, ak, av)
    xs = torch.stack([lrgen.activations(w, 0, b, 0, ctx + steps) for b in range(B)]).to(torch.bfloat16)
    for t0 in range(0, ctx, 40):
        t1 = min(ctx, t0 + 40)
        pos = torch.full((B,), t0, dtype=torch.int32, device=DEV)
        s.project_append(0, xs[:, t0:t1].contiguous().to(DEV), pos)
    ref_k = [oracle.latents(xs[b].double().numpy(), ak.double().numpy()).astype(np.float32) for b in range(B)]
    ref_v = [oracle.latents(xs[b].double().numpy(), av.double().numpy()).astype(np.float32) for b in range(B)]
    scale = 1.0 / math.sqrt(w.head_dim)
    offk, offv = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    for st in range(steps):
        T = ctx + st + 1
        q = lrgen.normal(lrgen.stream_key(w.seed, lrgen.TAG_Q, 0, st), 0, B * H * w.head_dim, 1.0)
        q = q.view(B, H, w.head_dim).to(torch.bfloat16).to(DEV).contiguous()
        pos = torch.full((B,), ctx + st, dtype=torch.int32, device=DEV)
        out = torch.empty(B, H, w.head_dim, dtype=torch.bfloat16, device=DEV)
        s.lengths.fill_(T)
        if one_step:
            s.project_append_decode(0, xs[:, ctx + st].contiguous().to(DEV), pos, q, out, T)
        else:
            ck, cv = s.project(0, xs[:, ctx + st].contiguous().to(DEV))
            s.append_decode(0, ck, cv, pos, q, out, T)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        for b in range(B):
            for h in range(H):
                ref = oracle.attend(w.qfmt, ref_k[b][:T, offk[h]:offk[h] + rk[h]],
                                    ref_v[b][:T, offv[h]:offv[h] + rv[h]],
                                    q[b, h].double().cpu().numpy(),
                                    bk[offk[h]:offk[h] + rk[h]].double().cpu().numpy(),
                                    bv[offv[h]:offv[h] + rv[h]].double().cpu().numpy(), scale)
                assert within(got[b, h], ref, TOL_BF16), (st, b, h)


@pytest.mark.parametrize("seed", range(16))
def test_project_random_shapes(seed):
    """Seeded random shapes: E a multiple of 32 (32..8192), 1..130 tokens, 1-8
    heads of random K and V ranks, a random part count.  Small-integer inputs
    give the oracle's latents exactly, unsplit and as parts added in order;
    Gaussian bf16 inputs stay within the rounding bounds."""
    from latent_kv_attention_lr_amd import lr_attn_project_latent_parts
    rng = np.random.default_rng(0x5EED2000 + seed)
    E = 32 * int(rng.integers(1, 257))
    T = int(rng.choice([1, 2, 15, 16, 17, 33, 48, 64, 65, 100, 130]))
    H = int(rng.integers(1, 9))
    ranks_k = [int(8 * rng.integers(1, 17)) for _ in range(H)]
    ranks_v = [int(8 * rng.integers(1, 17)) for _ in range(H)]
    parts = min(int(rng.integers(1, 9)), E // 32)
    say(f"project random {seed}: E={E} T={T} ranks_k={ranks_k} ranks_v={ranks_v} parts={parts}")
    s = _session(ranks_k, ranks_v)
    x = torch.from_numpy(rng.integers(-3, 4, (T, E)).astype(np.float32))
    ak = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_k))).astype(np.float32))
    av = torch.from_numpy(rng.integers(-3, 4, (E, sum(ranks_v))).astype(np.float32))
    ck, cv = _gpu_project(s, x.to(torch.bfloat16), ak, av)
    ref_k = oracle.latents(x.double().numpy(), ak.double().numpy()).astype(np.float32)
    ref_v = oracle.latents(x.double().numpy(), av.double().numpy()).astype(np.float32)
    assert np.array_equal(ck, ref_k) and np.array_equal(cv, ref_v)
    xd = x.to(torch.bfloat16).to(DEV).contiguous()
    pk = torch.empty(parts, T, sum(ranks_k), dtype=torch.float32, device=DEV)
    pv = torch.empty(parts, T, sum(ranks_v), dtype=torch.float32, device=DEV)
    lr_attn_project_latent_parts(s.plan, 0, xd, T, E, s.proj[0][1], parts, pk, pv)
    torch.cuda.synchronize()
    sk, sv = pk[0].clone(), pv[0].clone()
    for q in range(1, parts):
        sk += pk[q]
        sv += pv[q]
    assert np.array_equal(sk.cpu().numpy(), ref_k) and np.array_equal(sv.cpu().numpy(), ref_v)
    # Gaussian activations and factors (bf16 values)
    key = lrgen.stream_key(0x5EED2000 + seed, 1)
    xb = lrgen.normal(key, 0, T * E, 1.0).view(T, E).to(torch.bfloat16).float()
    ak = _factors(E, ranks_k, lrgen.stream_key(0x5EED2000 + seed, 2), 1.0 / math.sqrt(E))
    av = _factors(E, ranks_v, lrgen.stream_key(0x5EED2000 + seed, 3), 1.0 / math.sqrt(E))
    ck, cv = _gpu_project(s, xb.to(torch.bfloat16), ak, av)
    _check_bound(ck, xb, ak)
    _check_bound(cv, xb, av)


def test_project_append_decode_graph_replay_matches_eager():
    """Three steps from activations (generate, append, attend: two launches
    each) captured in one HIP graph: each replay writes the same cache bytes
    and outputs as the eager steps, with eager work and changed activations
    between replays."""
    rng = np.random.default_rng(61)
    ranks_k, ranks_v, E, B, ctx, steps = [8, 64, 32, 96], [40, 16, 128, 8], 2080, 5, 120, 3
    H = len(ranks_k)
    s = _session(ranks_k, ranks_v, batch=B, cap=ctx + steps)
    ak = _factors(E, ranks_k, lrgen.stream_key(61, 1), 1.0 / math.sqrt(E))
    av = _factors(E, ranks_v, lrgen.stream_key(61, 2), 1.0 / math.sqrt(E))
    _set_factors(s, ak, av)
    bk = torch.from_numpy(rng.standard_normal((sum(ranks_k), 128)) / 6).to(torch.bfloat16).to(DEV)
    bv = torch.from_numpy(rng.standard_normal((sum(ranks_v), 128)) / 6).to(torch.bfloat16).to(DEV)
    s.set_factors(0, bk, bv)
    pk = torch.from_numpy(rng.standard_normal((B, ctx, sum(ranks_k))).astype(np.float32)).to(DEV)
    pv = torch.from_numpy(rng.standard_normal((B, ctx, sum(ranks_v))).astype(np.float32)).to(DEV)
    s.append(0, pk, pv, torch.zeros(B, dtype=torch.int32, device=DEV))
    prefix = s.caches[0].clone()
    xs = [torch.empty(B, E, dtype=torch.bfloat16, device=DEV) for _ in range(steps)]
    qs = [torch.from_numpy(rng.standard_normal((B, H, 128))).to(torch.bfloat16).to(DEV) for _ in range(steps)]
    pos = [torch.full((B,), ctx + i, dtype=torch.int32, device=DEV) for i in range(steps)]
    lens = [torch.full((B,), ctx + i + 1, dtype=torch.int32, device=DEV) for i in range(steps)]
    outs = [torch.empty(B, H, 128, dtype=torch.bfloat16, device=DEV) for _ in range(steps)]

    def steps_fn():
        for i in range(steps):
            s.project_append_decode(0, xs[i], pos[i], qs[i], outs[i], ctx + steps, lengths=lens[i])

    def draw(seed):
        for i, x in enumerate(xs):
            x.copy_(torch.from_numpy(np.random.default_rng(seed + i).standard_normal((B, E))).to(torch.bfloat16))

    draw(1000)
    steps_fn()                                   # sizes the step workspace before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            steps_fn()
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        draw(2000 + 10 * rep)
        s.caches[0].copy_(prefix)
        steps_fn()                               # eager reference
        torch.cuda.synchronize()
        ref_out = [o.clone() for o in outs]
        ref_cache = s.caches[0].clone()
        s.caches[0].copy_(prefix)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"project_append_decode graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.caches[0], ref_cache), rep
        for i in range(steps):
            assert torch.equal(outs[i].view(torch.int16), ref_out[i].view(torch.int16)), (rep, i)
