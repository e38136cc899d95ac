"""Rotation between the factors (block-Hadamard outlier smoothing).

CPU: the library's host transform (lr_attn_hadamard_rotate_rows, fast
Walsh-Hadamard butterflies) against the oracle's dense rotation (Sylvester
recursion, plain products); argument errors; and the quantisation error of
the oracle's own path with and without the rotation on the int4 workload's
layer shape, for the workload's iid factors and for SVD-like factors with a
decaying spectrum.

GPU: the same measurement through the product path -- rotated factors packed
for the projection and used by the decode, cache built from activations --
against the oracle's unquantised attention with the unrotated factors.
"""
import math

import numpy as np
import pytest
import torch

import lrgen
import oracle
import latent_kv_attention_lr_amd as lr

RANKS_K = [8, 24, 40, 48, 64, 96, 128, 16]
RANKS_V = [128, 16, 8, 96, 40, 64, 24, 48]


def _plan(rk=RANKS_K, rv=RANKS_V):
    return lr.lr_attn_plan_create(1, 2, len(rk), 64, lr.LR_Q_INT4_G32, lr.LR_DT_BF16, rk, rv)


@pytest.mark.parametrize("block", [8, 32, 128])
@pytest.mark.parametrize("kv", [0, 1])
def test_host_rotation_matches_oracle(kv, block):
    """Each head's rows replaced by S_h^T rows, S_h the oracle's block rotation:
    agreement to fp32 rounding of the same fp64 value."""
    p = _plan()
    try:
        ranks = RANKS_K if kv == 0 else RANKS_V
        rng = np.random.default_rng(10 * kv + block)
        rows = rng.standard_normal((sum(ranks), 37)).astype(np.float32)
        got = rows.copy()
        lr.lr_attn_hadamard_rotate_rows(p, 0, kv, block, got)
        o = 0
        for h, r in enumerate(ranks):
            s, g = oracle.block_rotation(r, block)
            assert lr.lr_attn_hadamard_block(p, 0, kv, h, block) == g
            want = s.T @ rows[o:o + r].astype(np.float64)
            tol = 2.0 ** -23 * np.max(np.abs(want))
            assert np.max(np.abs(got[o:o + r] - want)) <= tol, (h, r, g)
            o += r
    finally:
        lr.lr_attn_plan_destroy(p)


def test_host_rotation_twice_restores_and_keeps_products():
    """S^2 = I (Sylvester blocks are symmetric), and rotating both A^T and B
    keeps A B."""
    p = _plan()
    try:
        rng = np.random.default_rng(3)
        at = rng.standard_normal((sum(RANKS_K), 64)).astype(np.float32)   # A^T
        b = rng.standard_normal((sum(RANKS_K), 128)).astype(np.float32)   # B
        at2, b2 = at.copy(), b.copy()
        lr.lr_attn_hadamard_rotate_rows(p, 0, 0, 32, at2)
        lr.lr_attn_hadamard_rotate_rows(p, 0, 0, 32, b2)
        o = 0
        for r in RANKS_K:
            ab = at[o:o + r].T.astype(np.float64) @ b[o:o + r]
            ab2 = at2[o:o + r].T.astype(np.float64) @ b2[o:o + r]
            assert np.max(np.abs(ab2 - ab)) <= 1e-5 * np.max(np.abs(ab))
            o += r
        back = at2.copy()
        lr.lr_attn_hadamard_rotate_rows(p, 0, 0, 32, back)
        assert np.max(np.abs(back - at)) <= 1e-6 * np.max(np.abs(at))
        t = torch.from_numpy(at.copy())
        lr.lr_attn_hadamard_rotate_rows(p, 0, 0, 32, t)    # CPU torch tensors take the same path
        assert torch.equal(t, torch.from_numpy(at2))
    finally:
        lr.lr_attn_plan_destroy(p)


def test_host_rotation_argument_errors():
    p = _plan()
    try:
        f = lr._lib.lr_attn_hadamard_rotate_rows
        buf = np.zeros((sum(RANKS_K), 4), np.float32)
        ptr = buf.ctypes.data
        assert f(None, 0, 0, 32, ptr, 4) == lr.LR_EINVAL
        assert f(p, 0, 0, 32, None, 4) == lr.LR_EINVAL
        assert f(p, 1, 0, 32, ptr, 4) == lr.LR_ERANGE
        assert f(p, 0, 2, 32, ptr, 4) == lr.LR_EINVAL
        for blk in (0, 4, 12, 256):
            assert f(p, 0, 0, blk, ptr, 4) == lr.LR_EINVAL, blk
        assert f(p, 0, 0, 32, ptr, 0) == lr.LR_EINVAL
        assert lr.lr_attn_hadamard_block(p, 0, 0, 8, 32) == 0      # head out of range
        assert lr.lr_attn_hadamard_block(p, 0, 0, 0, 6) == 0       # block not a power of two
        with pytest.raises(ValueError):
            lr.lr_attn_hadamard_rotate_rows(p, 0, 0, 32, np.zeros((3, 4), np.float32))
    finally:
        lr.lr_attn_plan_destroy(p)


# ---------------------------------------------------------------------------
# quantisation error with and without the rotation (oracle path, CPU)
# ---------------------------------------------------------------------------

def _rel_err_oracle(w, alpha, heads, T, qfmt, seed, n_queries=32):
    """Relative RMS error over `heads` of the oracle's quantised attention,
    without and with the rotation, against its unquantised attention with the
    unrotated factors (fp64).  Returns (error without, error with)."""
    ak, bk = lrgen.svd_like_factors(w, 0, 0, alpha)
    av, bv = lrgen.svd_like_factors(w, 0, 1, alpha)
    x = lrgen.activations(w, 0, 0, 0, T).double().numpy()
    rng = np.random.default_rng(seed)
    num, den = [0.0, 0.0], 0.0
    offs = lrgen.head_offsets(w.ranks_k[0])
    scale = 1 / math.sqrt(w.head_dim)
    for h in heads:
        r, o = w.ranks_k[0][h], offs[h]
        A_k, B_k = ak[:, o:o + r].double().numpy(), bk[o:o + r].double().numpy()
        A_v, B_v = av[:, o:o + r].double().numpy(), bv[o:o + r].double().numpy()
        ck, cv = oracle.latents(x, A_k), oracle.latents(x, A_v)
        Ar_k, Br_k = oracle.rotate_factors(A_k, B_k, 32)
        Ar_v, Br_v = oracle.rotate_factors(A_v, B_v, 32)
        crk = oracle.latents(x, Ar_k).astype(np.float32)
        crv = oracle.latents(x, Ar_v).astype(np.float32)
        for _ in range(n_queries):
            q = rng.standard_normal(w.head_dim)
            ref = oracle.attend(oracle.QFMT_NONE, ck, cv, q, B_k, B_v, scale)
            den += float(np.sum(ref ** 2))
            got = oracle.attend(qfmt, ck.astype(np.float32), cv.astype(np.float32), q, B_k, B_v, scale)
            num[0] += float(np.sum((got - ref) ** 2))
            got = oracle.attend(qfmt, crk, crv, q, Br_k, Br_v, scale)
            num[1] += float(np.sum((got - ref) ** 2))
    return math.sqrt(num[0] / den), math.sqrt(num[1] / den)


def test_rotation_effect_on_quantisation_error_oracle():
    """Int4 workload layer shape (E = 4096, r = 64, outlier channels), 3 heads,
    128 tokens, 32 queries per head: the rotation leaves the error of the workload's iid factors
    unchanged (within 10 %) and lowers it for SVD-like factors (s_j ~ 1/j)."""
    w = lrgen.workload(2)
    heads = [0, 13, 27]
    e_iid = _rel_err_oracle(w, 0.0, heads, 128, oracle.QFMT_INT4, 1)
    e_svd = _rel_err_oracle(w, 1.0, heads, 128, oracle.QFMT_INT4, 1)
    print(f"int4 iid factors: {e_iid[0]:.4f} -> {e_iid[1]:.4f};  s_j~1/j: {e_svd[0]:.4f} -> {e_svd[1]:.4f}")
    assert 0.9 <= e_iid[1] / e_iid[0] <= 1.1
    assert e_svd[1] / e_svd[0] <= 0.85


# ---------------------------------------------------------------------------
# GPU: the product path
# ---------------------------------------------------------------------------

@pytest.mark.gpu
@pytest.mark.parametrize("alpha", [0.0, 1.0])
def test_rotation_through_the_gpu_path(alpha):
    """Int4 workload layer (E = 4096, 32 heads of rank 64, outlier channels),
    batch 2, 512 cached tokens generated from activations by the projection and
    appended, then 8 decode calls with different queries; every fourth head of
    both sequences against the oracle's unquantised attention with the
    unrotated fp64 factors.  The rotation leaves the error of iid factors
    unchanged within the sampling noise (ratio 0.8-1.15; 16 units x 8
    queries) and lowers it for SVD-like factors
    (s_j ~ 1/j).  Parity: on four units the output is within the decode
    tolerance of the oracle's int4 path with the same (rotated) factors."""
    from latent_kv_attention_lr_amd.session import DecodeSession
    dev = "cuda:0"
    w = lrgen.workload(2)
    B, T, H, d = 2, 512, w.n_heads, w.head_dim
    rk, rv = w.ranks_k[0], w.ranks_v[0]
    ak, bk = lrgen.svd_like_factors(w, 0, 0, alpha)
    av, bv = lrgen.svd_like_factors(w, 0, 1, alpha)
    xs = torch.stack([lrgen.activations(w, 0, b, 0, T) for b in range(B)])
    NQ = 8
    qs = lrgen.normal(lrgen.stream_key(w.seed, lrgen.TAG_Q, 7), 0, NQ * B * H * d, 1.0).view(NQ, B, H, d)
    scale = 1.0 / math.sqrt(d)
    # reference once: every checked (b, h) and query from bf16-rounded x and A
    # (what the GPU reads) and the unrotated fp32 B, unquantised, in fp64
    offk, offv = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    xb = xs.to(torch.bfloat16).double().numpy()
    akb = ak.to(torch.bfloat16).double().numpy()
    avb = av.to(torch.bfloat16).double().numpy()
    refs = []
    for b in range(B):
        for h in range(0, H, 4):
            ok, ov, r1, r2 = offk[h], offv[h], rk[h], rv[h]
            ck = oracle.latents(xb[b], np.ascontiguousarray(akb[:, ok:ok + r1]))
            cv = oracle.latents(xb[b], np.ascontiguousarray(avb[:, ov:ov + r2]))
            for i in range(NQ):
                refs.append((i, b, h, oracle.attend(oracle.QFMT_NONE, ck, cv, qs[i, b, h].double().numpy(),
                                                    bk[ok:ok + r1].double().numpy(),
                                                    bv[ov:ov + r2].double().numpy(), scale)))
    errs = {}
    for rotate in (False, True):
        print(f"rotation alpha={alpha} rotate={rotate}", flush=True)
        s = DecodeSession(1, B, H, T, w.qfmt, lr.LR_DT_F32, [rk], [rv], device=dev)
        at_k, at_v = ak.t().contiguous(), av.t().contiguous()
        fb_k, fb_v = bk.clone(), bv.clone()
        if rotate:
            for t_, kv in ((at_k, 0), (at_v, 1), (fb_k, 0), (fb_v, 1)):
                lr.lr_attn_hadamard_rotate_rows(s.plan, 0, kv, 32, t_)
        s.set_projection(0, at_k.to(torch.bfloat16).to(dev), at_v.to(torch.bfloat16).to(dev))
        s.set_factors(0, fb_k.to(dev), fb_v.to(dev))
        for t0 in range(0, T, 128):
            pos = torch.full((B,), t0, dtype=torch.int32, device=dev)
            s.project_append(0, xs[:, t0:t0 + 128].to(torch.bfloat16).contiguous().to(dev), pos)
        s.lengths.fill_(T)
        outs = []
        for i in range(NQ):
            out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
            s.decode(0, qs[i].contiguous().to(dev), out, T)
            outs.append(out)
        torch.cuda.synchronize()
        got = torch.stack(outs).cpu().numpy()
        num = den = 0.0
        for i, b, h, ref in refs:
            num += float(np.sum((got[i, b, h] - ref) ** 2))
            den += float(np.sum(ref ** 2))
        errs[rotate] = math.sqrt(num / den)
        # parity on a few units: the oracle's int4 path with the factors the GPU
        # used (rotated, A rounded to bf16), within the decode tolerance
        au_k = at_k.to(torch.bfloat16).double().numpy().T
        au_v = at_v.to(torch.bfloat16).double().numpy().T
        for b in range(B):
            for h in (0, 16):
                ok, ov, r1, r2 = offk[h], offv[h], rk[h], rv[h]
                ck = oracle.latents(xb[b], np.ascontiguousarray(au_k[:, ok:ok + r1])).astype(np.float32)
                cv = oracle.latents(xb[b], np.ascontiguousarray(au_v[:, ov:ov + r2])).astype(np.float32)
                want = oracle.attend(w.qfmt, ck, cv, qs[0, b, h].double().numpy(),
                                     fb_k[ok:ok + r1].double().numpy(), fb_v[ov:ov + r2].double().numpy(),
                                     scale)
                assert float(np.max(np.abs(got[0, b, h] - want))) <= 1e-2 * float(np.max(np.abs(want))) + 1e-3
    print(f"alpha={alpha}: relative RMS error {errs[False]:.5f} -> {errs[True]:.5f} "
          f"(ratio {errs[True] / errs[False]:.3f})", flush=True)
    if alpha == 0.0:
        assert 0.8 <= errs[True] / errs[False] <= 1.15
    else:
        assert errs[True] / errs[False] <= 0.85
