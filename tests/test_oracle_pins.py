"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each test checks it against a
hand-derived value (``tests/golden``), an independent library routine
(numpy's binary16 conversion, numpy's SVD), a closed form, or brute force,
chosen so that a dropped term, a wrong sign or index, a transposed factor or
a wrong rounding rule fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _val(v):
    return math.ldexp(v[0], v[1]) if isinstance(v, list) else float(v)


# --------------------------------------------------------------------------
# binary16 conversion (used for the int4 group scales)
# --------------------------------------------------------------------------

def test_fp16_golden_encodings():
    cases = json.load(open(os.path.join(GOLD, "fp16_rne.json")))["cases"]
    for c in cases:
        x = math.ldexp(c["m"], c["e"])
        assert oracle.f32_to_f16_bits(x) == int(c["bits"], 16), c["why"]


def test_fp16_matches_numpy_on_random_and_tie_values():
    rng = np.random.default_rng(7)
    mags = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))
    # exact ties: odd multiples of half an ulp at several binades, and in the subnormal range
    ties = []
    for e in range(-24, 16):
        ulp = math.ldexp(1.0, max(e - 10, -24))
        base = math.ldexp(1.0, e)
        for k in range(1, 8):
            ties.append(base + (2 * k + 1) * ulp / 2)
    xs = np.concatenate([mags, np.array(ties), -np.array(ties)]).astype(np.float32)
    xs = xs[np.isfinite(xs)]
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    mine = np.array([oracle.f32_to_f16_bits(float(v)) for v in xs], dtype=np.uint16)
    assert np.array_equal(ref, mine)


def test_fp16_decode_all_finite_patterns():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    finite = np.isfinite(vals)
    ref = vals[finite].astype(np.float32)
    mine = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits[finite]], dtype=np.float32)
    assert np.array_equal(ref.view(np.uint32), mine.view(np.uint32))


# --------------------------------------------------------------------------
# Quantisers
# --------------------------------------------------------------------------

QUANT = json.load(open(os.path.join(GOLD, "quant_cases.json")))


@pytest.mark.parametrize("case", QUANT["int8"], ids=lambda c: c["name"])
def test_quant_int8_golden(case):
    row = np.array([_val(v) for v in case["row"]], dtype=np.float32)
    q, s = oracle.quant_int8(row[None])
    assert q[0].tolist() == case["q"], case["why"]
    if case["scale"] == "m/127":
        want = np.float32(np.abs(row).max()) / np.float32(127.0)
    else:
        want = np.array([int(case["scale"], 16)], dtype=np.uint32).view(np.float32)[0]
    assert s[0].view(np.uint32) == np.float32(want).view(np.uint32)


@pytest.mark.parametrize("case", QUANT["int4"], ids=lambda c: c["name"])
def test_quant_int4_golden(case):
    row = np.array([_val(v) for v in case["row"]], dtype=np.float32)
    q, s = oracle.quant_int4(row[None])
    assert q[0].tolist() == case["q"], case["why"]
    assert [int(x) for x in s[0]] == [int(h, 16) for h in case["scale"]]


def _rows(n, r, seed):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((n, r)) * np.exp2(rng.integers(-6, 6, (n, 1)))
    return c.astype(np.float32)


@pytest.mark.parametrize("r", [8, 32, 40, 96, 128])
def test_quant_int8_error_bound_and_extremes(r):
    c = _rows(300, r, r)
    q, s = oracle.quant_int8(c)
    m = np.abs(c).max(axis=1)
    # the scale is the binary32 quotient m/127
    assert np.array_equal(s, (m.astype(np.float32) / np.float32(127.0)).astype(np.float32))
    # the largest-magnitude element maps to +-127 with its sign
    idx = np.abs(c).argmax(axis=1)
    assert np.array_equal(q[np.arange(len(c)), idx], np.sign(c[np.arange(len(c)), idx]) * 127)
    # round-to-nearest: |s*q - c| <= s/2 (fp64, exact products), codes inside [-127, 127]
    err = np.abs(s[:, None].astype(np.float64) * q - c.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))
    assert q.min() >= -127 and q.max() <= 127


@pytest.mark.parametrize("r", [8, 32, 48, 64, 96, 128])
def test_quant_int4_error_bound_and_groups(r):
    c = _rows(300, r, 100 + r)
    q, sb = oracle.quant_int4(c)
    ng = (r + 31) // 32
    assert sb.shape == (300, ng)
    s = sb.view(np.float16).astype(np.float64)
    for g in range(ng):
        lo, hi = 32 * g, min(r, 32 * g + 32)
        m = np.abs(c[:, lo:hi]).max(axis=1)
        # each group's scale is the binary16 value nearest m/7 (numpy's conversion)
        want = (m.astype(np.float32) / np.float32(7.0)).astype(np.float16)
        assert np.array_equal(sb[:, g], want.view(np.uint16))
        err = np.abs(s[:, g:g + 1] * q[:, lo:hi] - c[:, lo:hi].astype(np.float64))
        # |c/s| <= 7 (1 + 2^-10), so rounding stays within half a step and never clamps
        assert np.all(err <= s[:, g:g + 1] * (0.5 + 1e-6))
    assert q.min() >= -7 and q.max() <= 7


def test_quant_groups_are_independent():
    c = _rows(1, 64, 3)
    c2 = c.copy()
    c2[0, 40] = 1000.0  # inflates group 1 only
    q1, s1 = oracle.quant_int4(c)
    q2, s2 = oracle.quant_int4(c2)
    assert np.array_equal(q1[0, :32], q2[0, :32]) and s1[0, 0] == s2[0, 0]
    assert s1[0, 1] != s2[0, 1]


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _dense_mha(X, WK, WV, q, scale):
    """softmax(q (X W_K)^T * scale) (X W_V) for one head, brute force fp64."""
    K = X @ WK
    V = X @ WV
    z = (K @ q) * scale
    e = np.exp(z - z.max())
    p = e / e.sum()
    return p @ V


@pytest.mark.parametrize("T", [1, 2, 5, 7])
def test_full_rank_unquantised_equals_dense_mha(T):
    """At r = d with no quantisation, c_t = x_t A_h and k_t = c_t B_h rebuild
    x_t W_h exactly (W_h = A_h B_h from its SVD), so the oracle must equal
    dense multi-head attention (E=16, 2 heads, d=8)."""
    rng = np.random.default_rng(11 + T)
    E, H, d = 16, 2, 8
    X = rng.standard_normal((T, E))
    WK = rng.standard_normal((E, H * d)) / 4
    WV = rng.standard_normal((E, H * d)) / 4
    Q = rng.standard_normal((H, d))
    scale = 1 / math.sqrt(d)
    for h in range(H):
        wk, wv = WK[:, h * d:(h + 1) * d], WV[:, h * d:(h + 1) * d]
        fac = []
        for w in (wk, wv):
            U, S, Vt = np.linalg.svd(w, full_matrices=False)
            A = U * np.sqrt(S)              # E x d
            B = np.sqrt(S)[:, None] * Vt    # d x d
            fac.append((A, B))
        (AK, BK), (AV, BV) = fac
        got = oracle.attend_dequantised(X @ AK, X @ AV, Q[h], BK, BV, scale)
        want = _dense_mha(X, wk, wv, Q[h], scale)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_full_rank_through_generated_latents_equals_dense_mha():
    """The same pin with the latents made by the oracle's own latent generation
    (c = x A from the activations) rather than by a matrix product here."""
    rng = np.random.default_rng(23)
    E, H, d, T = 16, 2, 8, 6
    X = rng.standard_normal((T, E))
    WK = rng.standard_normal((E, H * d)) / 4
    WV = rng.standard_normal((E, H * d)) / 4
    Q = rng.standard_normal((H, d))
    scale = 1 / math.sqrt(d)
    fac = {}
    for name, W in (("k", WK), ("v", WV)):
        As, Bs = [], []
        for h in range(H):
            U, S, Vt = np.linalg.svd(W[:, h * d:(h + 1) * d], full_matrices=False)
            As.append(U * np.sqrt(S))
            Bs.append(np.sqrt(S)[:, None] * Vt)
        fac[name] = (np.concatenate(As, axis=1), Bs)   # heads side by side
    CK = oracle.latents(X, fac["k"][0])
    CV = oracle.latents(X, fac["v"][0])
    for h in range(H):
        got = oracle.attend_dequantised(CK[:, h * d:(h + 1) * d], CV[:, h * d:(h + 1) * d], Q[h],
                                        fac["k"][1][h], fac["v"][1][h], scale)
        want = _dense_mha(X, WK[:, h * d:(h + 1) * d], WV[:, h * d:(h + 1) * d], Q[h], scale)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_latents_exact_on_small_integers():
    """Integer inputs make every fp64 sum exact: the result must equal the
    brute-force integer product (non-square shapes catch a transposed factor,
    the full range of e catches a dropped term)."""
    rng = np.random.default_rng(3)
    for T, E, N in [(1, 1, 1), (3, 5, 2), (4, 7, 9), (2, 33, 17)]:
        x = rng.integers(-9, 10, size=(T, E))
        a = rng.integers(-9, 10, size=(E, N))
        want = [[sum(int(x[t, e]) * int(a[e, n]) for e in range(E)) for n in range(N)]
                for t in range(T)]
        got = oracle.latents(x.astype(np.float64), a.astype(np.float64))
        assert got.tolist() == [[float(v) for v in row] for row in want]


def test_latents_one_hot_rows_pick_factor_rows():
    """x_t = e_j gives c_t = row j of A, bit for bit."""
    rng = np.random.default_rng(4)
    E, N = 24, 40
    a = rng.standard_normal((E, N))
    idx = [0, 5, 23, 7]
    x = np.zeros((len(idx), E))
    x[np.arange(len(idx)), idx] = 1.0
    assert np.array_equal(oracle.latents(x, a), a[idx])


def test_latents_of_stacked_heads_are_per_head_latents():
    """Heads side by side in A give each head's own latent in its columns, and
    rows of x are independent tokens."""
    rng = np.random.default_rng(6)
    E, T = 32, 5
    ranks = [8, 16, 24]
    As = [rng.standard_normal((E, r)) for r in ranks]
    x = rng.standard_normal((T, E))
    full = oracle.latents(x, np.concatenate(As, axis=1))
    o = 0
    for A, r in zip(As, ranks):
        assert np.array_equal(full[:, o:o + r], oracle.latents(x, A))
        o += r
    for t in range(T):
        assert np.array_equal(full[t:t + 1], oracle.latents(x[t:t + 1], np.concatenate(As, axis=1)))


def test_eckart_young_truncation_error():
    """Per-head factors from a rank-r truncated SVD of a random W_h (E x d):
    rows of A_r B_r are rebuilt through the oracle's value path (T = 1, latent =
    row of A_r, so o = v_0 = c B^V), and ||W - A_r B_r||_F must equal
    sqrt(sum of the dropped sigma_i^2); the spectral error must equal sigma_{r+1}."""
    rng = np.random.default_rng(5)
    E, d = 24, 16
    W = rng.standard_normal((E, d))
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    q = rng.standard_normal(d)
    for r in range(1, d):
        A = U[:, :r] * np.sqrt(S[:r])
        B = np.sqrt(S[:r])[:, None] * Vt[:r]
        Wr = np.stack([
            oracle.attend_dequantised(A[j:j + 1], A[j:j + 1], q, B, B, 0.1) for j in range(E)])
        fro = np.linalg.norm(W - Wr)
        assert abs(fro - math.sqrt(np.sum(S[r:] ** 2))) <= 1e-10 * np.linalg.norm(W)
        spec = np.linalg.norm(W - Wr, 2)
        assert abs(spec - S[r]) <= 1e-10 * S[0]


def _unit(T, rk, rv, d, seed):
    rng = np.random.default_rng(seed)
    ck = rng.standard_normal((T, rk)).astype(np.float32)
    cv = rng.standard_normal((T, rv)).astype(np.float32)
    q = rng.standard_normal(d)
    bk = rng.standard_normal((rk, d)) / math.sqrt(rk)
    bv = rng.standard_normal((rv, d)) / math.sqrt(rv)
    return ck, cv, q, bk, bv


@pytest.mark.parametrize("qfmt", [oracle.QFMT_INT8, oracle.QFMT_INT4, oracle.QFMT_NONE])
def test_softmax_weights_sum_to_one(qfmt):
    ck, cv, q, bk, bv = _unit(37, 32, 48, 128, 1)
    _, p = oracle.attend(qfmt, ck, cv, q, bk, bv, 1 / math.sqrt(128), want_probs=True)
    assert abs(p.sum() - 1.0) <= 1e-12 and np.all(p > 0)


def test_single_token_returns_its_value():
    ck, cv, q, bk, bv = _unit(1, 16, 16, 32, 2)
    o = oracle.attend(oracle.QFMT_NONE, ck, cv, q, bk, bv, 0.3)
    assert np.max(np.abs(o - cv[0].astype(np.float64) @ bv)) <= 1e-13


def test_zero_query_gives_mean_value():
    ck, cv, q, bk, bv = _unit(9, 16, 24, 32, 3)
    o = oracle.attend(oracle.QFMT_NONE, ck, cv, np.zeros_like(q), bk, bv, 0.3)
    want = (cv.astype(np.float64) @ bv).mean(axis=0)
    assert np.max(np.abs(o - want)) <= 1e-13


def test_token_permutation_invariance():
    ck, cv, q, bk, bv = _unit(23, 32, 32, 64, 4)
    perm = np.random.default_rng(0).permutation(23)
    for qfmt in (oracle.QFMT_INT8, oracle.QFMT_INT4):
        a = oracle.attend(qfmt, ck, cv, q, bk, bv, 0.125)
        b = oracle.attend(qfmt, ck[perm], cv[perm], q, bk, bv, 0.125)
        assert np.max(np.abs(a - b)) <= 1e-13


def test_hand_worked_two_token_example():
    """d = 2, r = 1.  B^K = [[ln 3, 0]], q = [1, 0], scale 1: with latents
    c^K = (1, 0) the scores are (ln 3, 0), so p = (3/4, 1/4).  B^V = [[0, 1]]
    and c^V = (4, 8) give v = ((0, 4), (0, 8)), hence o = (0, 3 + 2) = (0, 5)."""
    o, p = oracle.attend_dequantised(np.array([[1.0], [0.0]]), np.array([[4.0], [8.0]]),
                                     np.array([1.0, 0.0]), np.array([[math.log(3.0), 0.0]]),
                                     np.array([[0.0, 1.0]]), 1.0, want_probs=True)
    assert np.allclose(p, [0.75, 0.25], atol=1e-15, rtol=0)
    assert np.allclose(o, [0.0, 5.0], atol=1e-14, rtol=0)


def test_scale_multiplies_scores():
    """Doubling the softmax scale equals doubling q."""
    ck, cv, q, bk, bv = _unit(15, 16, 16, 32, 9)
    a = oracle.attend(oracle.QFMT_INT8, ck, cv, q, bk, bv, 0.4)
    b = oracle.attend(oracle.QFMT_INT8, ck, cv, 2 * q, bk, bv, 0.2)
    assert np.max(np.abs(a - b)) <= 1e-13


def _dequant(qfmt, c):
    if qfmt == oracle.QFMT_INT8:
        q, s = oracle.quant_int8(c)
        return q.astype(np.float64) * s[:, None].astype(np.float64)
    q, sb = oracle.quant_int4(c)
    s = sb.view(np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(s, 32, axis=1)[:, :c.shape[1]]


@pytest.mark.parametrize("qfmt", [oracle.QFMT_INT8, oracle.QFMT_INT4])
def test_quantised_attend_is_dequantise_then_attend(qfmt):
    ck, cv, q, bk, bv = _unit(40, 48, 64, 128, 21)
    a = oracle.attend(qfmt, ck, cv, q, bk, bv, 1 / math.sqrt(128))
    b = oracle.attend_dequantised(_dequant(qfmt, ck), _dequant(qfmt, cv), q, bk, bv, 1 / math.sqrt(128))
    assert np.array_equal(a, b)


def test_absorbed_form_equals_explicit_oracle():
    """The GPU computes q' = scale q B^K^T, scores s_t = q' . c~^K_t, and
    o = (sum_t p_t c~^V_t) B^V.  In fp64 this must equal the oracle's explicit
    reconstruction."""
    for qfmt in (oracle.QFMT_INT8, oracle.QFMT_INT4):
        ck, cv, q, bk, bv = _unit(300, 32, 48, 128, 31 + qfmt)
        scale = 1 / math.sqrt(128)
        ctk, ctv = _dequant(qfmt, ck), _dequant(qfmt, cv)
        qp = scale * (bk @ q)
        s = ctk @ qp
        p = np.exp(s - s.max())
        p /= p.sum()
        o = (p @ ctv) @ bv
        ref = oracle.attend(qfmt, ck, cv, q, bk, bv, scale)
        assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_split_context_merge_equals_unsplit():
    """Flash-Decoding style partials (m_j, l_j, u_j) over any split of [0, T),
    merged with m = max m_j, l = sum e^(m_j - m) l_j, u = sum e^(m_j - m) u_j,
    give the unsplit result u / l."""
    ck, cv, q, bk, bv = _unit(257, 32, 32, 64, 41)
    scale = 0.125
    ctk, ctv = _dequant(oracle.QFMT_INT8, ck), _dequant(oracle.QFMT_INT8, cv)
    s = ctk @ (scale * (bk @ q))
    ref = oracle.attend(oracle.QFMT_INT8, ck, cv, q, bk, bv, scale)
    for cuts in ([0, 257], [0, 1, 257], [0, 64, 128, 192, 257], [0, 100, 101, 256, 257]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            m = s[a:b].max()
            e = np.exp(s[a:b] - m)
            parts.append((m, e.sum(), e @ ctv[a:b]))
        M = max(p[0] for p in parts)
        L = sum(math.exp(p[0] - M) * p[1] for p in parts)
        U = sum(math.exp(p[0] - M) * p[2] for p in parts)
        o = (U / L) @ bv
        assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_empty_context_gives_zero():
    o = oracle.attend(oracle.QFMT_INT8, np.zeros((0, 8), np.float32), np.zeros((0, 8), np.float32),
                      np.ones(16), np.ones((8, 16)), np.ones((8, 16)), 0.25)
    assert np.array_equal(o, np.zeros(16))


# --------------------------------------------------------------------------
# Rotation between the factors (Hadamard outlier smoothing)
# --------------------------------------------------------------------------

def test_hadamard_small_orders_by_hand():
    s2 = 1 / math.sqrt(2)
    assert np.array_equal(oracle.hadamard(1), np.array([[1.0]]))
    assert np.allclose(oracle.hadamard(2), np.array([[s2, s2], [s2, -s2]]), rtol=0, atol=1e-16)
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    assert np.array_equal(oracle.hadamard(4), h4)
    with pytest.raises(ValueError):
        oracle.hadamard(12)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_is_orthogonal_and_matches_scipy(n):
    import scipy.linalg
    h = oracle.hadamard(n)
    assert np.max(np.abs(h @ h.T - np.eye(n))) <= 1e-14
    assert np.all(np.abs(np.abs(h) * math.sqrt(n) - 1.0) <= 1e-14)
    assert np.allclose(h, scipy.linalg.hadamard(n) / math.sqrt(n), rtol=0, atol=1e-15)


@pytest.mark.parametrize("r,block,g", [(8, 32, 8), (16, 32, 16), (24, 32, 8), (40, 32, 8), (48, 32, 16),
                                       (64, 32, 32), (96, 32, 32), (128, 32, 32), (128, 128, 128),
                                       (96, 128, 32), (64, 8, 8)])
def test_block_rotation_structure(r, block, g):
    """Blocks of the largest power of two dividing r, capped at the block size;
    block-diagonal, orthogonal, zero off the blocks."""
    s, got = oracle.block_rotation(r, block)
    assert got == g
    assert np.max(np.abs(s @ s.T - np.eye(r))) <= 1e-14
    h = oracle.hadamard(g)
    for b0 in range(0, r, g):
        assert np.array_equal(s[b0:b0 + g, b0:b0 + g], h)
    mask = np.kron(np.eye(r // g), np.ones((g, g))).astype(bool)
    assert np.all(s[~mask] == 0.0)


def test_rotated_factors_keep_the_product_and_rotate_the_latent():
    """(A S)(S^T B) = A B, the latent becomes c S, and full-rank unquantised
    attention through the rotated factors still equals dense attention."""
    rng = np.random.default_rng(31)
    E, r, d, T = 64, 48, 48, 5
    a = rng.standard_normal((E, r))
    b = rng.standard_normal((r, d))
    ar, br = oracle.rotate_factors(a, b, 32)
    s, _ = oracle.block_rotation(r, 32)
    assert np.max(np.abs(ar @ br - a @ b)) <= 1e-12 * np.max(np.abs(a @ b))
    x = rng.standard_normal((T, E))
    assert np.max(np.abs(oracle.latents(x, ar) - oracle.latents(x, a) @ s)) <= 1e-12 * 10
    # full rank (r = d): rotated, unquantised attention equals dense attention
    W = rng.standard_normal((E, d)) / 4
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    A, B = U * np.sqrt(S), np.sqrt(S)[:, None] * Vt
    Ar, Br = oracle.rotate_factors(A, B, 32)
    q = rng.standard_normal(d)
    got = oracle.attend_dequantised(oracle.latents(x, Ar), oracle.latents(x, Ar), q, Br, Br, 0.2)
    want = _dense_mha(x, W, W, q, 0.2)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


# --------------------------------------------------------------------------
# Greedy global rank allocation
# --------------------------------------------------------------------------

def test_allocation_hand_worked():
    """Units with block sums (10, 2) and (6, 4) at step 2: from one block each
    (cost 4 of 6), the one block left goes to the larger next block (4 > 2);
    with room for both, both; with room for nothing more, none."""
    s = np.array([[5, 5, 1, 1], [3, 3, 2, 2.0]])
    assert oracle.allocate_ranks(s, 2, 1.0, 6).tolist() == [2, 4]
    assert oracle.allocate_ranks(s, 2, 1.0, 8).tolist() == [4, 4]
    assert oracle.allocate_ranks(s, 2, 1.0, 5.9).tolist() == [2, 2]
    with pytest.raises(ValueError):
        oracle.allocate_ranks(s, 2, 1.0, 3.9)


def test_allocation_ties_go_to_the_lowest_unit():
    s = np.ones((3, 32))
    assert oracle.allocate_ranks(s, 8, 1.0, 8 * 3 + 8 * 3).tolist() == [32, 8, 8]
    assert oracle.allocate_ranks(s, 8, 1.0, 8 * 3 + 8 * 4).tolist() == [32, 16, 8]


def _brute_force_best(block_vals, n_blocks, extra):
    """Best total block value over all prefix assignments using at most `extra`
    extra blocks (every unit keeps its first block)."""
    import itertools
    best = -1.0
    n = len(block_vals)
    for take in itertools.product(range(n_blocks), repeat=n):
        if sum(take) > extra:
            continue
        best = max(best, sum(sum(block_vals[u][1:1 + take[u]]) for u in range(n)))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_allocation_is_optimal_for_non_increasing_scores(seed):
    """With every unit's block values non-increasing (scores follow the
    singular values) and equal block costs, greedy picks the best prefix
    assignment: its total equals brute force over all assignments."""
    rng = np.random.default_rng(seed)
    n, step, m = 5, 2, 8                       # 5 units, 4 blocks each
    comp = -np.sort(-rng.exponential(1.0, (n, m)), axis=1) * rng.uniform(0.2, 3.0, (n, 1))
    blocks = comp.reshape(n, m // step, step).sum(axis=2)
    for extra in range(0, n * (m // step - 1) + 1, 3):
        ranks = oracle.allocate_ranks(comp, step, 1.0, step * (n + extra))
        assert int(ranks.sum()) == step * (n + min(extra, n * (m // step - 1)))
        got = sum(blocks[u, 1:ranks[u] // step].sum() for u in range(n))
        assert abs(got - _brute_force_best(blocks.tolist(), m // step, extra)) <= 1e-12


def test_allocation_grows_with_the_budget_and_respects_it():
    rng = np.random.default_rng(9)
    s = rng.exponential(1.0, (40, 128))          # not monotone within units
    prev = None
    for budget in np.linspace(40 * 8 * 136, 40 * 128 * 136, 13):
        r = oracle.allocate_ranks(s, 8, 136.0, budget)
        assert np.all(r % 8 == 0) and np.all(r >= 8) and np.all(r <= 128)
        assert r.sum() * 136.0 <= budget + 1e-9
        if prev is not None:
            assert np.all(r >= prev)
        prev = r
    assert np.all(oracle.allocate_ranks(s, 8, 136.0, 40 * 128 * 136) == 128)


# --------------------------------------------------------------------------
# Hybrid low-rank / dense FFN, W8A8
# --------------------------------------------------------------------------

def _silu(v):
    from scipy.special import expit
    return v * expit(v)


def test_activation_groups_are_int8_rows_of_64():
    """Per-token, per-64-group activation scales are the int8 row quantiser
    applied to each group (the last group shorter)."""
    rng = np.random.default_rng(2)
    a = (rng.standard_normal((3, 150)) * np.exp2(rng.integers(-8, 8, (3, 1)))).astype(np.float32)
    q, s = oracle.quant_act_groups(a)
    assert s.shape == (3, 3)
    for t in range(3):
        for g, (lo, hi) in enumerate([(0, 64), (64, 128), (128, 150)]):
            q1, s1 = oracle.quant_int8(a[t, lo:hi])
            assert np.array_equal(q[t, lo:hi], q1) and s[t, g] == s1


def _ffn_case(rng, T=3, E=64, F=48, S=16, r=8):
    f = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    return (f(T, E), f(F - S, E) / 8, f(F - S, E) / 8, f(r, E) / 8, f(r, E) / 8, f(S, r) / 3,
            f(S, r) / 3, f(E, F) / 7)


def test_ffn_unquantised_equals_brute_force():
    """Without quantisation the oracle is the hybrid SwiGLU FFN: low-rank
    channels through B A, dense ones through W, then W_d (numpy, fp64)."""
    rng = np.random.default_rng(4)
    x, wg, wu, ag, au, bg, bu, wd = [v.astype(np.float64) for v in _ffn_case(rng)]
    G = np.concatenate([bg @ ag, wg], axis=0)     # rows = hidden channels, low-rank first
    U = np.concatenate([bu @ au, wu], axis=0)
    h = (_silu(x @ G.T) * (x @ U.T)).astype(np.float32).astype(np.float64)
    want = h @ wd.T
    got = oracle.ffn(x, wg, wu, ag, au, bg, bu, wd, quantise=False)
    assert np.max(np.abs(got - want)) <= 1e-5 * np.max(np.abs(want))


def test_ffn_w8a8_error_is_the_rounding_of_h_on_grid_inputs():
    """All-dense (S = 0) with weights and x already on the int8 grid (integers
    times a power of two per activation group, every row / group reaching
    +-127, so every scale is a power of two and every code exact):
    the only error left is the RTN of h, so |y_q - y| <= sum_c |W_d[e][c]|
    (s_h(t, c) / 2 + fp32 rounding of h)."""
    rng = np.random.default_rng(8)
    T, E, F = 4, 128, 96

    def grid(rows, cols, group):
        m = rng.integers(-126, 127, (rows, cols)).astype(np.float32)
        for lo in range(0, cols, group):
            m[:, lo] = 127.0
        return m
    # x group g scaled by 2^(g - 1): scales 1/2, 1 differ per group, codes stay exact
    x = grid(T, E, 64) * np.repeat(np.exp2(np.arange(E // 64) - 1.0), 64)[None, :].astype(np.float32)
    wg, wu = grid(F, E, E), grid(F, E, E)
    wd = grid(E, F, F)
    z0 = np.zeros((0, E), np.float32)
    zs = np.zeros((0, 0), np.float32)
    yq = oracle.ffn(x, wg, wu, z0, z0, zs, zs, wd, quantise=True)
    y = oracle.ffn(x, wg, wu, z0, z0, zs, zs, wd, quantise=False)
    # h as the oracle forms it (fp32), its group scales, and the bound
    g = x.astype(np.float64) @ wg.T.astype(np.float64)
    u = x.astype(np.float64) @ wu.T.astype(np.float64)
    h = (_silu(g) * u).astype(np.float32)
    _, sh = oracle.quant_act_groups(h)
    bound = np.zeros((T, E))
    for c in range(F):
        bound += np.abs(wd[:, c])[None, :] * (sh[:, c // 64] / 2 + 2.0 ** -24 * np.abs(h[:, c]))[:, None]
    assert np.all(np.abs(yq - y) <= bound * 1.0001 + 1e-9)
    assert np.max(np.abs(yq - y)) > 0          # the rounding of h does show


def test_ffn_w8a8_scales_exactly_with_the_down_projection():
    """Doubling W_d doubles y exactly (codes unchanged, scales doubled)."""
    rng = np.random.default_rng(12)
    x, wg, wu, ag, au, bg, bu, wd = _ffn_case(rng, T=2, E=128, F=80, S=32, r=64)
    y1 = oracle.ffn(x, wg, wu, ag, au, bg, bu, wd)
    y2 = oracle.ffn(x, wg, wu, ag, au, bg, bu, wd * 2)
    assert np.array_equal(y2, 2 * y1)


def test_ffn_identity_low_rank_branch_reproduces_the_dense_branch():
    """S = F low-rank channels with A = I (r = E) and B = W give the dense
    branch's result with W (x on the grid, so the latent z is x itself up to
    the fp32 rounding of 127 * fl(1/127))."""
    rng = np.random.default_rng(13)
    T, E, F = 3, 64, 32
    x = rng.integers(-126, 127, (T, E)).astype(np.float32)
    x[:, 0] = 127.0
    W_g = (rng.standard_normal((F, E)) / 8).astype(np.float32)
    W_u = (rng.standard_normal((F, E)) / 8).astype(np.float32)
    wd = (rng.standard_normal((E, F)) / 7).astype(np.float32)
    I = np.eye(E, dtype=np.float32)
    z0 = np.zeros((0, E), np.float32)
    dense = oracle.ffn(x, W_g, W_u, z0, z0, np.zeros((0, 0), np.float32), np.zeros((0, 0), np.float32), wd)
    lowrank = oracle.ffn(x, np.zeros((0, E), np.float32), np.zeros((0, E), np.float32), I, I, W_g, W_u, wd)
    assert np.max(np.abs(lowrank - dense)) <= 1e-5 * np.max(np.abs(dense))


def test_ffn_trace_intermediates_unquantised_equal_brute_force():
    """lro_ffn_trace without quantisation: z = fp32(A x), g, u = the
    pre-activations of the hybrid layout (low-rank channels first, through
    B z), h = fp32(silu(g) u), all against a numpy brute force; its y is
    lro_ffn's bit for bit."""
    rng = np.random.default_rng(21)
    x, wg, wu, ag, au, bg, bu, wd = _ffn_case(rng, T=3, E=64, F=48, S=16, r=8)
    y, z, g, u, h = oracle.ffn_trace(x, wg, wu, ag, au, bg, bu, wd, quantise=False)
    x64 = x.astype(np.float64)
    zg = (x64 @ ag.T.astype(np.float64)).astype(np.float32)
    zu = (x64 @ au.T.astype(np.float64)).astype(np.float32)
    assert np.max(np.abs(z - np.concatenate([zg, zu], axis=1))) <= 2.0 ** -23 * np.max(np.abs(z))
    G = np.concatenate([zg.astype(np.float64) @ bg.T.astype(np.float64), x64 @ wg.T.astype(np.float64)], axis=1)
    U = np.concatenate([zu.astype(np.float64) @ bu.T.astype(np.float64), x64 @ wu.T.astype(np.float64)], axis=1)
    assert np.max(np.abs(g - G)) <= 1e-12 * np.max(np.abs(G))
    assert np.max(np.abs(u - U)) <= 1e-12 * np.max(np.abs(U))
    assert np.max(np.abs(h - (_silu(G) * U).astype(np.float32))) <= 2.0 ** -22 * np.max(np.abs(h))
    for q in (False, True):
        assert np.array_equal(oracle.ffn_trace(x, wg, wu, ag, au, bg, bu, wd, quantise=q)[0],
                              oracle.ffn(x, wg, wu, ag, au, bg, bu, wd, quantise=q))


def test_ffn_w8a8_low_rank_branch_with_two_latent_groups_equals_dense_branch():
    """All channels low-rank at rank r = E = 128 with A = 127 I and B on the
    int8 grid, against all channels dense with W = 127 B: the latent z = 127 x
    has two groups of 64 whose scales differ (x's groups are scaled by 1 and
    1/4), every scale is exact, so the quantised low-rank path must give the
    dense path's y bit for bit -- a wrong latent group index or scale breaks
    the equality."""
    rng = np.random.default_rng(22)
    T, E, F = 4, 128, 64

    def grid(rows, cols, group, scales):
        m = rng.integers(-126, 127, (rows, cols)).astype(np.float32)
        for lo in range(0, cols, group):
            m[:, lo] = 127.0
        return m * np.repeat(np.asarray(scales, np.float32), group)[None, :]
    x = grid(T, E, 64, [1.0, 0.25])
    bg = grid(F, E, E, [2.0 ** -3])
    bu = grid(F, E, E, [2.0 ** -2])
    wd = (rng.standard_normal((E, F)) / 8).astype(np.float32)
    A = (127.0 * np.eye(E)).astype(np.float32)
    none_e = np.zeros((0, E), np.float32)
    lowrank, z, _, _, _ = oracle.ffn_trace(x, none_e, none_e, A, A, bg, bu, wd)
    dense = oracle.ffn(x, 127 * bg, 127 * bu, none_e, none_e, np.zeros((0, 0), np.float32),
                       np.zeros((0, 0), np.float32), wd)
    assert np.array_equal(z[:, :E], 127 * x) and np.array_equal(z[:, E:], 127 * x)
    _, zs = oracle.quant_act_groups(z[:, :E])
    assert np.all(zs[:, 0] == 4 * zs[:, 1])          # the two latent groups have different scales
    assert np.array_equal(lowrank, dense)
