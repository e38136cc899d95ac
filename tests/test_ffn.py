"""Hybrid low-rank / dense W8A8 FFN (lr_ffn_*): host weight preparation
against the oracle's quantiser (CPU, bit for bit), argument errors (CPU), and
the decode through the GPU kernels against the oracle's fp64 FFN (GPU).

GPU tolerance: |y - y_ref| <= 2e-3 max|y_ref| per token row.  The kernels
and the oracle take the same quantisation decisions for x and the weights
(same fp32 values, same rule); the latents z and h are formed in fp32 on the
GPU and fp64 in the oracle, so a code of z or h sitting on a rounding
boundary may differ by one, which moves y by one step of that group's scale
times a weight (at most ~1/127 of that group's contribution).
"""
import math

import numpy as np
import pytest

import lrgen
import oracle
import latent_kv_attention_lr_amd as lr

TOL_FFN = 2e-3


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
    ws = (r256(T * E) + r256(T * (E // 64) * 4) + r256(T * 2 * r * 4) + r256(T * 2 * r)
          + r256(T * (2 * r // 64) * 4) + r256(T * F * 4) + r256(T * Fp) + r256(T * (Fp // 64) * 4))
    # (no partial sums: the hidden dimension fits one chunk of the down projection)
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
    ref = oracle.ffn(x.float().numpy()[list(rows)], *w)
    return y[list(rows)], ref, layer, x


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
    y, ref, _, _ = _run_gpu(E, F, S, r, T, seed=E + F + S + r + T)
    for t in range(T):
        err = float(np.max(np.abs(y[t] - ref[t])))
        assert err <= TOL_FFN * float(np.max(np.abs(ref[t]))), (t, err, float(np.max(np.abs(ref[t]))))


@pytest.mark.gpu
def test_ffn_decode_full_size_and_deterministic():
    """The LLaMA-7B FFN workload (E 4096, hidden 11008, half low-rank at rank
    1024, 16 tokens): every token against the oracle; a second call is
    bitwise equal."""
    import torch
    f = lrgen.FFN_WORKLOADS[0]
    print(f"ffn full size {f.name}", flush=True)
    y, ref, layer, x = _run_gpu(f.embed, f.hidden, f.n_lowrank, f.rank, f.tokens, seed=f.seed)
    worst = 0.0
    for t in range(f.tokens):
        err = float(np.max(np.abs(y[t] - ref[t]))) / float(np.max(np.abs(ref[t])))
        worst = max(worst, err)
        assert err <= TOL_FFN, (t, err)
    print(f"worst relative error {worst:.2e}", flush=True)
    y2 = layer(x.to("cuda:0")).cpu().numpy()
    assert np.array_equal(y, y2)


@pytest.mark.gpu
def test_ffn_decode_in_several_passes():
    """2100 tokens of a shape whose pass is 2032 tokens: two passes through one
    workspace; tokens on both sides of the pass boundary and at both ends
    against the oracle."""
    E, F, S, r, T = 512, 8208, 4096, 256, 2100
    assert _pass_tokens(E, F, S, r) == 2032
    print(f"ffn passes E={E} F={F} S={S} r={r} T={T}", flush=True)
    rows = [0, 1, 777, 2030, 2031, 2032, 2033, 2099]
    y, ref, _, _ = _run_gpu(E, F, S, r, T, seed=99, tokens=rows)
    for i, t in enumerate(rows):
        err = float(np.max(np.abs(y[i] - ref[i])))
        assert err <= TOL_FFN * float(np.max(np.abs(ref[i]))), (t, err)
