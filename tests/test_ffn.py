"""Hybrid low-rank / dense W8A8 FFN (lr_ffn_*): host weight preparation
against the oracle's quantiser (CPU, bit for bit), argument errors (CPU), and
the decode through the GPU kernels against the oracle's fp64 FFN (GPU).

GPU tolerance, per token t and output e (ffn_bound): the kernels and the
oracle take the same quantisation decisions for x and the weights (same fp32
values, same rule); the latents z and the hidden h are formed in fp32 on the
GPU and in fp64 (then rounded to fp32) in the oracle.  So
  * y agrees to fp32 summation accuracy, 2e-5 max|y_ref[t]|, wherever no
    element of z or h sits within DELTA code units of a rounding boundary;
  * an h element within DELTA of a boundary may round the other way: its code
    moves by one, y[t][e] by at most one step s_h times |W_d[e][c]| (each such
    element is added to the bound);
  * a latent within DELTA of a boundary may take the other neighbouring code,
    which moves g or u of every low-rank channel: for each such latent the
    bound adds |y_alt[t] - y_ref[t]|, y_alt being the oracle's quantised tail
    (B z, SwiGLU, h quantisation, W_d h) rerun with that one code changed,
    plus the h flips possible around y_alt's own h (rare: DELTA = 2e-5 over a
    few thousand latents; such tokens are counted).
The boundary distances come from the oracle's own intermediates
(lro_ffn_trace).  A flip where the oracle's value is further than DELTA from
a boundary, a wrong group scale or index, or a dropped term exceeds this.
"""
import math

import numpy as np
import pytest

import lrgen
import oracle
import latent_kv_attention_lr_amd as lr

TOL_SUM = 2e-5     # fp32 summation, relative to max|y_ref| of the token
DELTA = 2e-5       # code units: how close to a rounding boundary counts as on it


def _near_boundary(a):
    """Distance of each activation's code value a / s from the nearest rounding
    boundary (k + 1/2), with the oracle's per-(token, 64-group) scales."""
    a = np.ascontiguousarray(a, np.float32)
    _, s = oracle.quant_act_groups(a)
    sg = np.repeat(s, 64, axis=1)[:, :a.shape[1]].astype(np.float64)
    v = np.abs(a.astype(np.float64)) / np.where(sg > 0, sg, 1.0)
    return np.abs(v - np.floor(v) - 0.5), sg


def _dequantised_rows(m):
    """Rows of m as the weight quantiser leaves them (codes x row scale, fp64)."""
    q, sc = oracle.quant_int8(np.ascontiguousarray(m, np.float32))
    return q.astype(np.float64) * sc.astype(np.float64)[:, None]


def _dequantised_acts(a):
    """Activations [T, K] as the group quantiser leaves them (fp64)."""
    q, sc = oracle.quant_act_groups(a)
    return q.astype(np.float64) * np.repeat(sc, 64, axis=1)[:, :a.shape[1]].astype(np.float64)


def _tail(zdq, g_dense, u_dense, bgd, bud, wdd, S):
    """The FFN after the latents' quantisation, for tokens with dequantised
    latents zdq [n, 2r]: low-rank g, u = B z; dense g, u given; h = silu(g) u
    rounded to fp32; y = W_d (h quantised).  Returns (y [n, E], h [n, F])."""
    r = zdq.shape[1] // 2
    g, u = g_dense.copy(), u_dense.copy()
    if S:
        g[:, :S] = zdq[:, :r] @ bgd.T
        u[:, :S] = zdq[:, r:] @ bud.T
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    return _dequantised_acts(h) @ wdd.T, h


def ffn_bound(x, w):
    """(y_ref [T, E], bound [T, E], tokens with a latent on a boundary)."""
    wg, wu, ag, au, bg, bu, wd = w
    y, z, g, u, h = oracle.ffn_trace(x, wg, wu, ag, au, bg, bu, wd)
    mh, sh = _near_boundary(h)
    absw = np.abs(wd.astype(np.float64)) * (1.0 + 1.0 / 254)   # dequantised |W_d| (RTN error <= s/2)
    bound = TOL_SUM * np.max(np.abs(y), axis=1, keepdims=True).repeat(y.shape[1], axis=1)
    flips = (mh < DELTA) * sh                                    # [T, F]: one code step where a flip can happen
    bound += flips @ absw.T
    z_tokens = []
    if z.shape[1]:
        mz, sz = _near_boundary(z)
        z_tokens = [t for t in range(z.shape[0]) if np.any(mz[t] < DELTA)]
    if z_tokens:
        S = bg.shape[0]
        bgd, bud, wdd = _dequantised_rows(bg), _dequantised_rows(bu), _dequantised_rows(wd)
        zdq = _dequantised_acts(z)
        # the tail reproduces the oracle's y before any code is changed
        y0, _ = _tail(zdq[z_tokens], g[z_tokens], u[z_tokens], bgd, bud, wdd, S)
        assert np.allclose(y0, y[z_tokens], rtol=1e-9, atol=1e-12 * float(np.max(np.abs(y))))
        for t in z_tokens:
            for k in np.flatnonzero(mz[t] < DELTA):
                v = float(z[t, k]) / float(sz[t, k])                    # the latent in code units
                code = float(np.rint(v))
                alt = zdq[t:t + 1].copy()
                alt[0, k] += (1.0 if v > code else -1.0) * float(sz[t, k])   # the other neighbouring code
                ya, ha = _tail(alt, g[t:t + 1], u[t:t + 1], bgd, bud, wdd, S)
                mha, sha = _near_boundary(ha)
                bound[t] += np.abs(ya[0] - y[t]) + (((mha < DELTA) * sha) @ absw.T)[0]
    return y, bound, z_tokens


def _desc(E, F, S, r):
    return lr.lr_ffn_desc(E, F, S, r, 0)


def _case(E, F, S, r, T, seed):
    f = lrgen.FfnWorkload("t", E, F, S, r, T, seed)
    return f, lrgen.ffn_weights(f), lrgen.ffn_activations(f, T)


@pytest.mark.parametrize("bad", [(32, 96, 0, 0), (100, 96, 0, 0), (8256, 96, 0, 0), (128, 90, 0, 0),
                                 (128, 96, 40, 64), (128, 96, 112, 64), (128, 96, 32, 0), (128, 96, 32, 96),
                                 (128, 96, 0, 64), (128, 96, 32, 4160)])
def test_ffn_rejects_bad_shapes(bad):
    assert lr.lr_ffn_weight_bytes(_desc(*bad)) == 0
    assert lr.lr_ffn_workspace_bytes(_desc(*bad), 4) == 0


def test_ffn_weight_and_workspace_sizes():
    E, F, S, r = 128, 96, 32, 64
    r256 = lambda n: -(-n // 256) * 256
    n1, n2, n3, Fp = 2 * (F - S) // 16 + 2 * r // 16, 2 * S // 16, E // 16, 128
    want = (r256(n1 * E * 16) + r256(n2 * r * 16) + r256(n3 * Fp * 16) + r256(n1 * 64) + r256(n2 * 64)
            + r256(n3 * 64))
    assert lr.lr_ffn_weight_bytes(_desc(E, F, S, r)) == want
    T = 5
    counters = 4 * 1 * (2 * r // 64 + Fp // 64 + E // 16)   # one token block, one chunk, 16-row tiles
    ws = (r256(counters) + r256(T * E) + r256(T * (E // 64) * 4) + r256(2 * T * 2 * r * 4) + r256(T * 2 * r)
          + r256(T * (2 * r // 64) * 4) + r256(T * F * 4) + r256(T * Fp) + r256(T * (Fp // 64) * 4))
    # (the two halves' partial latents; h rows already whole 128-byte lines;
    # no partial sums: the hidden dimension fits one chunk of the down projection)
    assert lr.lr_ffn_workspace_bytes(_desc(E, F, S, r), T) == ws
    assert lr.lr_ffn_workspace_bytes(_desc(E, F, S, r), 0) == 0


def _pass_tokens(E, F, S, r):
    """Tokens per pass of lr_ffn_decode, as documented with lr_ffn_workspace_bytes."""
    Fp = -(-F // 64) * 64
    chunks = 1 if Fp <= 2048 else -(-Fp // 4096)
    u = max(E // 16 * chunks, r // 8, Fp // 16, (F - S) // 16 + r // 16, S // 16)
    return 16 * max(1, (1 << 16) // u)


def test_ffn_workspace_holds_one_pass():
    """Above one pass of tokens the workspace stops growing; below it grows."""
    d = _desc(512, 8208, 4096, 256)
    p = _pass_tokens(512, 8208, 4096, 256)
    assert p == 2032
    assert lr.lr_ffn_workspace_bytes(d, p - 16) < lr.lr_ffn_workspace_bytes(d, p)
    assert lr.lr_ffn_workspace_bytes(d, p) == lr.lr_ffn_workspace_bytes(d, 2100)
    assert lr.lr_ffn_workspace_bytes(d, 1 << 20) == lr.lr_ffn_workspace_bytes(d, p)
    assert lr.lr_ffn_workspace_bytes(d, (1 << 20) + 1) == 0
    big = _desc(64, 1 << 20, 0, 0)   # the largest hidden size: passes of 16 tokens
    assert _pass_tokens(64, 1 << 20, 0, 0) == 16
    assert lr.lr_ffn_workspace_bytes(big, 1000) == lr.lr_ffn_workspace_bytes(big, 16)


def _unpack(buf, rows, K, Kp, tiles_off, tile, scales_off):
    """Codes [16][K] and scales [16] of packed tile `tile` (documented layout)."""
    tb = Kp * 16
    t = np.frombuffer(buf, dtype=np.int8, count=tb, offset=tiles_off + tile * tb).reshape(Kp // 64, 64, 16)
    codes = np.zeros((16, Kp), np.int8)
    for l in range(64):
        codes[l & 15].reshape(Kp // 64, 64)[:, 16 * (l >> 4):16 * (l >> 4) + 16] = t[:, l, :]
    sc = np.frombuffer(buf, dtype=np.float32, count=16, offset=scales_off + tile * 64)
    return codes[:, :K], sc


def test_prepared_weights_are_the_oracle_quantisation_packed():
    """Every tile of the host-prepared buffer unpacks to the oracle's int8 row
    codes and fp32 scales of the right rows (bit for bit), zeros past K."""
    E, F, S, r = 128, 96, 32, 64
    wg, wu, ag, au, bg, bu, wd = lrgen.ffn_weights(lrgen.FfnWorkload("t", E, F, S, r, 1, 3))
    buf = lr.lr_ffn_prepare_weights(_desc(E, F, S, r), wg, wu, ag, au, bg, bu, wd).tobytes()
    r256 = lambda n: -(-n // 256) * 256
    D, Fp = F - S, 128
    n1, n2, n3 = 2 * D // 16 + 2 * r // 16, 2 * S // 16, E // 16
    off_w2 = r256(n1 * E * 16)
    off_w3 = off_w2 + r256(n2 * r * 16)
    off_s1 = off_w3 + r256(n3 * Fp * 16)
    off_s2 = off_s1 + r256(n1 * 64)
    off_s3 = off_s2 + r256(n2 * 64)
    expect = []
    for p in range(D // 16):
        expect += [(wg, 16 * p), (wu, 16 * p)]
    A = np.concatenate([ag, au])
    expect += [(A, 16 * j) for j in range(2 * r // 16)]
    for tile, (M, row0) in enumerate(expect):
        q, s = _unpack(buf, None, E, E, 0, tile, off_s1)
        oq, os_ = oracle.quant_int8(M[row0:row0 + 16])
        assert np.array_equal(q, oq) and np.array_equal(s, os_), tile
    for p in range(S // 16):
        for k, M in enumerate((bg, bu)):
            q, s = _unpack(buf, None, r, r, off_w2, 2 * p + k, off_s2)
            oq, os_ = oracle.quant_int8(M[16 * p:16 * p + 16])
            assert np.array_equal(q, oq) and np.array_equal(s, os_)
    for e in range(E // 16):
        q, s = _unpack(buf, None, Fp, Fp, off_w3, e, off_s3)
        oq, os_ = oracle.quant_int8(wd[16 * e:16 * e + 16])
        assert np.array_equal(q[:, :F], oq) and np.all(q[:, F:] == 0) and np.array_equal(s, os_)


def test_ffn_argument_errors_before_launch():
    d = _desc(128, 96, 32, 64)
    FAKE = 1 << 20
    f = lr._lib.lr_ffn_decode
    import ctypes
    dp = ctypes.byref(d)
    assert f(None, FAKE, FAKE, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EINVAL
    assert f(dp, None, FAKE, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EINVAL
    assert f(dp, FAKE, None, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EINVAL
    assert f(dp, FAKE, FAKE, 4, None, FAKE, 1 << 30, None) == lr.LR_EINVAL
    assert f(dp, FAKE + 16, FAKE, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EINVAL   # weights 256-aligned
    assert f(dp, FAKE, FAKE + 8, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EINVAL    # x 16-aligned
    assert f(dp, FAKE, FAKE, -1, FAKE, FAKE, 1 << 30, None) == lr.LR_ERANGE
    assert f(dp, FAKE, FAKE, (1 << 20) + 1, FAKE, FAKE, 1 << 30, None) == lr.LR_ERANGE
    assert f(dp, FAKE, FAKE, 4, FAKE, None, 1 << 30, None) == lr.LR_EWORKSPACE
    need = lr.lr_ffn_workspace_bytes(d, 4)
    assert f(dp, FAKE, FAKE, 4, FAKE, FAKE, need - 1, None) == lr.LR_EWORKSPACE
    assert f(dp, FAKE, FAKE, 0, FAKE, None, 0, None) == lr.LR_OK                  # no-op
    bad = _desc(128, 96, 40, 64)
    assert f(ctypes.byref(bad), FAKE, FAKE, 4, FAKE, FAKE, 1 << 30, None) == lr.LR_EUNSUPPORTED
    w = lrgen.ffn_weights(lrgen.FfnWorkload("t", 128, 96, 32, 64, 1, 3))
    w[6] = w[6].copy()
    w[6][3, 5] = np.nan
    with pytest.raises(lr.LrAttnError):
        lr.lr_ffn_prepare_weights(d, *w)


@pytest.mark.parametrize("E,F,S,r,T", [(128, 96, 32, 64, 5), (512, 2064, 512, 128, 3)])
def test_ffn_bound_rejects_plausible_kernel_mistakes(E, F, S, r, T):
    """The GPU bound admits the oracle itself but not: one 64-group of h with
    its scale off by 128/127, or one hidden channel dropped (CPU)."""
    _, w, x = _case(E, F, S, r, T, seed=7)
    xf = x.float().numpy()
    y, bound, _ = ffn_bound(xf, w)
    assert np.all(np.abs(y - y) <= bound)
    _, _, _, _, h = oracle.ffn_trace(xf, *w)
    wd = w[6].astype(np.float64)
    t = T - 1
    g = 0
    part = wd[:, 64 * g:64 * g + 64] @ h[t, 64 * g:64 * g + 64].astype(np.float64)
    bad = y.copy()
    bad[t] += part / 127.0
    assert np.any(np.abs(bad - y) > bound)
    c = int(np.argmax(np.abs(h[t])))
    bad = y.copy()
    bad[t] -= wd[:, c] * float(h[t, c])
    assert np.any(np.abs(bad - y) > bound)


def test_ffn_bound_covers_a_boundary_latent_and_no_other():
    """A latent within DELTA of a rounding boundary may take its other code:
    the bound admits y with that code, and rejects the same one-step change
    of a latent of that token far from any boundary (CPU)."""
    E, F, S, r, T = 64, 5776, 544, 896, 40
    _, w, x = _case(E, F, S, r, T, seed=1007)
    xf = x.float().numpy()
    y, bound, z_tokens = ffn_bound(xf, w)
    assert z_tokens, "this seed has a latent on a rounding boundary"
    t = z_tokens[0]
    wg, wu, ag, au, bg, bu, wd = w
    _, z, g, u, _ = oracle.ffn_trace(xf, *w)
    mz, sz = _near_boundary(z)
    bgd, bud, wdd = _dequantised_rows(bg), _dequantised_rows(bu), _dequantised_rows(wd)
    zdq = _dequantised_acts(z)

    def y_with_step(k, sign):
        alt = zdq[t:t + 1].copy()
        alt[0, k] += sign * float(sz[t, k])
        return _tail(alt, g[t:t + 1], u[t:t + 1], bgd, bud, wdd, S)[0][0]

    k = int(np.flatnonzero(mz[t] < DELTA)[0])
    v = float(z[t, k]) / float(sz[t, k])
    assert np.all(np.abs(y_with_step(k, 1.0 if v > np.rint(v) else -1.0) - y[t]) <= bound[t])
    far = int(np.argmax(mz[t]))   # the latent of token t furthest from a rounding boundary
    assert mz[t, far] > 0.4
    assert np.any(np.abs(y_with_step(far, 1.0) - y[t]) > bound[t])


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------

def _run_gpu(E, F, S, r, T, seed, tokens=None):
    import torch
    from latent_kv_attention_lr_amd.ffn import FfnLayer
    f, w, x = _case(E, F, S, r, T, seed)
    layer = FfnLayer(E, F, S, r, device="cuda:0")
    layer.set_weights(*w)
    y = layer(x.to("cuda:0")).cpu().numpy()
    rows = range(T) if tokens is None else tokens
    ref, bound, z_tokens = ffn_bound(x.float().numpy()[list(rows)], w)
    return y[list(rows)], ref, bound, z_tokens, layer, x


def _check(y, ref, bound, z_tokens, what):
    err = np.abs(y.astype(np.float64) - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    rel = float(np.max(err / np.max(np.abs(ref), axis=1, keepdims=True)))
    print(f"{what}: worst error / bound {worst:.3f}, worst relative error {rel:.2e}, "
          f"tokens with a latent on a rounding boundary: {len(z_tokens)} of {len(y)}", flush=True)
    assert np.all(err <= bound), (what, np.argwhere(err > bound)[:5])
    return rel


@pytest.mark.gpu
@pytest.mark.parametrize("E,F,S,r,T", [(128, 96, 32, 64, 1), (128, 96, 32, 64, 5), (256, 160, 64, 128, 16),
                                       (256, 160, 64, 128, 17), (128, 96, 0, 0, 40), (128, 96, 96, 64, 3),
                                       (8192, 64, 16, 64, 2), (512, 8208, 4096, 256, 3),
                                       (512, 1296, 0, 0, 3), (512, 2064, 512, 128, 3), (512, 4112, 0, 0, 3),
                                       (256, 160, 64, 2048, 3), (256, 160, 64, 4096, 2)])
def test_ffn_decode_matches_oracle(E, F, S, r, T):
    """Small shapes across every path: T = 1 / ragged / several token blocks,
    all-dense and all-low-rank, the largest E, hidden sizes not a multiple of
    64, above one LDS chunk of the down projection, and between 1.3 K and 8 K
    (where LDS sized per launch once gave all-zero outputs); ranks 2048 and
    4096 take the medium and large LDS instances of the low-rank launch."""
    print(f"ffn E={E} F={F} S={S} r={r} T={T}", flush=True)
    y, ref, bound, z_tokens, _, _ = _run_gpu(E, F, S, r, T, seed=E + F + S + r + T)
    _check(y, ref, bound, z_tokens, f"E={E} F={F} S={S} r={r} T={T}")


@pytest.mark.gpu
def test_ffn_decode_full_size_and_deterministic():
    """The LLaMA-7B FFN workload (E 4096, hidden 11008, half low-rank at rank
    1024, 16 tokens): every token against the oracle; a second call is
    bitwise equal."""
    import torch
    f = lrgen.FFN_WORKLOADS[0]
    print(f"ffn full size {f.name}", flush=True)
    y, ref, bound, z_tokens, layer, x = _run_gpu(f.embed, f.hidden, f.n_lowrank, f.rank, f.tokens, seed=f.seed)
    _check(y, ref, bound, z_tokens, f.name)
    assert len(z_tokens) <= f.tokens // 4
    y2 = layer(x.to("cuda:0")).cpu().numpy()
    assert np.array_equal(y, y2)


@pytest.mark.gpu
def test_ffn_workspace_reuse_with_changing_inputs():
    """One layer (one workspace) called on alternating inputs x1, x2, x1, x2:
    the launches of a call pass the quantised activations, the latents and h
    to each other through the workspace, so a read of a value left by the
    previous call would show here.  Each output matches the oracle for its
    own input, and repeated inputs give bitwise equal outputs."""
    from latent_kv_attention_lr_amd.ffn import FfnLayer
    E, F, S, r, T = 512, 8208, 4096, 256, 17
    print(f"ffn reuse E={E} F={F} S={S} r={r} T={T}", flush=True)
    f, w, x1 = _case(E, F, S, r, T, seed=5)
    x2 = lrgen.ffn_activations(lrgen.FfnWorkload("t", E, F, S, r, T, 6), T)
    layer = FfnLayer(E, F, S, r, device="cuda:0")
    layer.set_weights(*w)
    outs = [layer(x.to("cuda:0")).cpu().numpy() for x in (x1, x2, x1, x2)]
    for x, y in ((x1, outs[0]), (x2, outs[1])):
        ref, bound, z_tokens = ffn_bound(x.float().numpy(), w)
        _check(y, ref, bound, z_tokens, "reuse")
    assert not np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])


@pytest.mark.gpu
def test_ffn_decode_in_several_passes():
    """2100 tokens of a shape whose pass is 2032 tokens: two passes through one
    workspace; tokens on both sides of the pass boundary and at both ends
    against the oracle."""
    E, F, S, r, T = 512, 8208, 4096, 256, 2100
    assert _pass_tokens(E, F, S, r) == 2032
    print(f"ffn passes E={E} F={F} S={S} r={r} T={T}", flush=True)
    rows = [0, 1, 777, 2030, 2031, 2032, 2033, 2099]
    y, ref, bound, z_tokens, _, _ = _run_gpu(E, F, S, r, T, seed=99, tokens=rows)
    _check(y, ref, bound, z_tokens, "two passes")


def _random_ffn_shape(seed):
    """E a multiple of 64 (64..4096), hidden a multiple of 16 (16..9000), a
    low-rank share from none to all (multiple of 16) at rank 64..1024 (a
    multiple of 64), 1..40 tokens."""
    rng = np.random.default_rng(0x5EEDF100 + seed)
    E = 64 * int(rng.integers(1, 65))
    F = 16 * int(rng.integers(1, 563))
    S = 16 * int(rng.integers(0, F // 16 + 1)) if rng.random() < 0.8 else 0
    r = 64 * int(rng.integers(1, 17)) if S > 0 else 0
    T = int(rng.choice([1, 2, 15, 16, 17, 31, 33, 40]))
    return E, F, S, r, T


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(16))
def test_ffn_decode_random_shapes(seed):
    """Seeded random shapes (sizes, low-rank share, rank, token count) against
    the oracle within ffn_bound."""
    E, F, S, r, T = _random_ffn_shape(seed)
    print(f"ffn random {seed}: E={E} F={F} S={S} r={r} T={T}", flush=True)
    y, ref, bound, z_tokens, _, _ = _run_gpu(E, F, S, r, T, seed=1000 + seed)
    _check(y, ref, bound, z_tokens, f"random {seed}: E={E} F={F} S={S} r={r} T={T}")


@pytest.mark.gpu
def test_ffn_graph_replay_matches_eager():
    """Two FFN calls sharing one workspace, captured in one HIP graph: every
    replay equals the eager calls bit for bit, with eager work and a changed
    input between replays (the step's counters are cleared by a kernel of the
    step itself, so nothing in the graph depends on state left by a replay)."""
    import torch
    from latent_kv_attention_lr_amd.ffn import FfnLayer
    E, F, S, r, T = 512, 8208, 4096, 256, 33       # every launch, three token blocks, three chunks
    f, w, x = _case(E, F, S, r, T, seed=404)
    layer = FfnLayer(E, F, S, r, device="cuda:0")
    layer.set_weights(*w)
    x1 = x.to("cuda:0").contiguous()
    x2 = (x.float() * 0.5).to(torch.bfloat16).to("cuda:0").contiguous()
    y1 = torch.empty(T, E, dtype=torch.float32, device="cuda:0")
    y2 = torch.empty_like(y1)
    ref2 = layer(x2).clone()                          # also sizes the workspace before capture
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            layer(x1, y1)
            layer(x2, y2)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        xr = lrgen.ffn_activations(lrgen.FfnWorkload("t", E, F, S, r, T, 500 + rep), T)
        x1.copy_(xr.to("cuda:0"))
        ref1 = layer(x1).clone()                      # eager work between replays
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"ffn graph replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, ref1), rep
        assert torch.equal(y2, ref2), rep
    y, bound, z_tokens = ffn_bound(x1.float().cpu().numpy(), w)   # and the last replay is right
    _check(y1.cpu().numpy(), y, bound, z_tokens, "graph replay")
