"""Greedy global rank allocation (lr_attn_allocate_ranks, host C++ with a
heap) against the oracle's plain round-by-round scan, bit for bit on the
integer rank tables; argument errors; and, on the GPU, decode over a plan
built from an allocated table (ranks 8..128 in one layer) against the oracle.
"""
import math

import numpy as np
import pytest

import lrgen
import oracle
import latent_kv_attention_lr_amd as lr

E, D = 4096, 128
COST = E + D


def _oracle_table(scores, budget):
    L, H, _, m = scores.shape
    r = oracle.allocate_ranks(scores.reshape(L * H * 2, m).astype(np.float64), 8, float(COST), float(budget))
    r = r.reshape(L, H, 2)
    return r[:, :, 0], r[:, :, 1]


@pytest.mark.parametrize("mean_rank", [8, 12, 24, 48, 52, 96, 128])
def test_allocation_matches_oracle_at_model_scale(mean_rank):
    """32 layers x 32 heads x K/V x 128 components of synthetic scores (the
    shape of a LLaMA-7B attention stack), budget = mean_rank per head and K/V."""
    s = lrgen.component_scores(11, 32, 32).numpy()
    budget = 32 * 32 * 2 * mean_rank * COST
    rk, rv = lr.lr_attn_allocate_ranks(s, COST, budget)
    ok, ov = _oracle_table(s, budget)
    assert np.array_equal(rk, ok) and np.array_equal(rv, ov)
    assert (rk.sum() + rv.sum()) * COST <= budget
    assert (rk.sum() + rv.sum()) == 32 * 32 * 2 * mean_rank      # blocks all fit exactly


@pytest.mark.parametrize("seed", range(5))
def test_allocation_matches_oracle_on_random_and_tied_scores(seed):
    rng = np.random.default_rng(seed)
    L, H, m = 3, 5, [32, 64, 128][seed % 3]
    cases = [rng.exponential(1.0, (L, H, 2, m)),                          # not monotone
             -np.sort(-rng.exponential(1.0, (L, H, 2, m)), axis=3),       # monotone
             np.ones((L, H, 2, m)),                                        # all tied
             np.round(rng.uniform(0, 3, (L, H, 2, m)))]                   # many ties
    for s in cases:
        s = s.astype(np.float32)
        for extra in (0, 1, 7, 30, 10 ** 6):
            budget = (L * H * 2 + extra) * 8 * COST + int(rng.integers(0, 8 * COST))
            rk, rv = lr.lr_attn_allocate_ranks(s, COST, budget)
            ok, ov = _oracle_table(s, budget)
            assert np.array_equal(rk, ok) and np.array_equal(rv, ov), (seed, extra)


def test_allocated_table_builds_a_plan():
    s = lrgen.component_scores(3, 4, 32).numpy()
    rk, rv = lr.lr_attn_allocate_ranks(s, COST, 4 * 32 * 2 * 52 * COST)
    p = lr.lr_attn_plan_create(4, 8, 32, 1024, lr.LR_Q_INT8_TOKEN, lr.LR_DT_BF16, rk.ravel().tolist(),
                               rv.ravel().tolist())
    try:
        for layer in range(4):
            assert lr.lr_attn_latent_elems(p, layer, 0) == int(rk[layer].sum())
    finally:
        lr.lr_attn_plan_destroy(p)


def test_allocation_argument_errors():
    f = lr._lib.lr_attn_allocate_ranks
    s = np.ones((1, 2, 2, 16), np.float32)
    out = np.zeros(2, np.int32)
    ptr, op = s.ctypes.data, out.ctypes.data
    ok_budget = 4 * 8 * COST
    assert f(1, 2, 16, ptr, COST, ok_budget, op, op) == lr.LR_OK
    assert f(0, 2, 16, ptr, COST, ok_budget, op, op) == lr.LR_EINVAL
    assert f(1, 2, 16, None, COST, ok_budget, op, op) == lr.LR_EINVAL
    assert f(1, 2, 16, ptr, COST, ok_budget, None, op) == lr.LR_EINVAL
    assert f(1, 2, 16, ptr, 0, ok_budget, op, op) == lr.LR_EINVAL
    for m in (0, 4, 12, 136):
        assert f(1, 2, m, ptr, COST, ok_budget, op, op) == lr.LR_EUNSUPPORTED, m
    assert f(1, 2, 16, ptr, COST, ok_budget - 1, op, op) == lr.LR_ERANGE
    s[0, 1, 1, 3] = np.nan
    assert f(1, 2, 16, ptr, COST, ok_budget, op, op) == lr.LR_EINVAL
    s[0, 1, 1, 3] = np.inf
    assert f(1, 2, 16, ptr, COST, ok_budget, op, op) == lr.LR_EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("qfmt", [lr.LR_Q_INT8_TOKEN, lr.LR_Q_INT4_G32])
def test_decode_on_an_allocated_rank_table(qfmt):
    """One layer of 32 heads with ranks from the allocator (8..128, K and V
    apart; budget = mean rank 52), batch 4, 700 cached tokens: every (b, h)
    against the oracle, within the decode tolerance."""
    import torch
    from latent_kv_attention_lr_amd.session import DecodeSession
    from gpu_util import TOL_BF16, oracle_many, within
    dev = "cuda:0"
    s = lrgen.component_scores(5, 1, 32).numpy()
    rk, rv = lr.lr_attn_allocate_ranks(s, COST, 32 * 2 * 52 * COST)
    rk, rv = rk[0].tolist(), rv[0].tolist()
    assert min(rk + rv) == 8 and max(rk + rv) >= 96
    B, H, T = 4, 32, 700
    sess = DecodeSession(1, B, H, T, qfmt, lr.LR_DT_BF16, [rk], [rv], device=dev)
    key = lrgen.stream_key(77, qfmt)
    ck = lrgen.normal(key, 0, B * T * sum(rk), 1.0).view(B, T, sum(rk)).to(dev)
    cv = lrgen.normal(key, 1 << 30, B * T * sum(rv), 1.0).view(B, T, sum(rv)).to(dev)
    bk = (lrgen.normal(key, 1 << 31, sum(rk) * D, 0.1)).view(sum(rk), D).to(torch.bfloat16).to(dev)
    bv = (lrgen.normal(key, 3 << 30, sum(rv) * D, 0.1)).view(sum(rv), D).to(torch.bfloat16).to(dev)
    q = lrgen.normal(key, 1 << 32, B * H * D, 1.0).view(B, H, D).to(torch.bfloat16).to(dev)
    sess.set_factors(0, bk.contiguous(), bv.contiguous())
    sess.append(0, ck.contiguous(), cv.contiguous(), torch.zeros(B, dtype=torch.int32, device=dev))
    lens = torch.tensor([700, 1, 333, 64], dtype=torch.int32, device=dev)
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
    sess.decode(0, q, out, T, lengths=lens)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    offk, offv = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    jobs, idx = [], []
    for b, n in enumerate(lens.tolist()):
        for h in range(H):
            jobs.append((ck[b, :n, offk[h]:offk[h] + rk[h]].cpu().numpy(),
                         cv[b, :n, offv[h]:offv[h] + rv[h]].cpu().numpy(),
                         q[b, h].double().cpu().numpy(),
                         bk[offk[h]:offk[h] + rk[h]].double().cpu().numpy(),
                         bv[offv[h]:offv[h] + rv[h]].double().cpu().numpy()))
            idx.append((b, h))
    refs = oracle_many(qfmt, jobs, 1 / math.sqrt(D))
    for (b, h), ref in zip(idx, refs):
        assert within(got[b, h], ref, TOL_BF16), (b, h, rk[h], rv[h])


@pytest.mark.gpu
@pytest.mark.parametrize("table", ["allocated", "rank64"])
def test_decode_with_three_wavefront_work_groups(table):
    """32 sequences x 32 heads = 1024 (b, h) units in an int8 layer whose
    kernel holds three wavefronts per SIMD (an allocated table with ranks up
    to 128, or every rank 64): the automatic launch takes three-wavefront
    work-groups (four per compute unit, all resident).  Every (b, h) against
    the oracle, ragged lengths."""
    import torch
    from latent_kv_attention_lr_amd.session import DecodeSession
    from gpu_util import TOL_BF16, oracle_many, within
    dev = "cuda:0"
    qfmt = lr.LR_Q_INT8_TOKEN
    if table == "allocated":
        s = lrgen.component_scores(9, 1, 32).numpy()
        rk, rv = lr.lr_attn_allocate_ranks(s, COST, 32 * 2 * 52 * COST)
        rk, rv = rk[0].tolist(), rv[0].tolist()
        assert max(rk + rv) > 96
    else:
        rk, rv = [64] * 32, [64] * 32
    B, H, T = 32, 32, 200
    print(f"three-wavefront groups: {table}, B={B} H={H} T={T}", flush=True)
    sess = DecodeSession(1, B, H, T, qfmt, lr.LR_DT_BF16, [rk], [rv], device=dev)
    key = lrgen.stream_key(91, 3 if table == "allocated" else 4)
    ck = lrgen.normal(key, 0, B * T * sum(rk), 1.0).view(B, T, sum(rk)).to(dev)
    cv = lrgen.normal(key, 1 << 30, B * T * sum(rv), 1.0).view(B, T, sum(rv)).to(dev)
    bk = (lrgen.normal(key, 1 << 31, sum(rk) * D, 0.1)).view(sum(rk), D).to(torch.bfloat16).to(dev)
    bv = (lrgen.normal(key, 3 << 30, sum(rv) * D, 0.1)).view(sum(rv), D).to(torch.bfloat16).to(dev)
    q = lrgen.normal(key, 1 << 32, B * H * D, 1.0).view(B, H, D).to(torch.bfloat16).to(dev)
    sess.set_factors(0, bk.contiguous(), bv.contiguous())
    sess.append(0, ck.contiguous(), cv.contiguous(), torch.zeros(B, dtype=torch.int32, device=dev))
    lens_l = [T - 5 * b if b % 3 else 1 + 6 * b for b in range(B)]   # 1..200
    lens = torch.tensor(lens_l, dtype=torch.int32, device=dev)
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
    sess.decode(0, q, out, T, lengths=lens)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    offk, offv = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
    ckh, cvh, qh, bkh, bvh = ck.cpu().numpy(), cv.cpu().numpy(), q.double().cpu().numpy(), \
        bk.double().cpu().numpy(), bv.double().cpu().numpy()
    jobs, idx = [], []
    for b, n in enumerate(lens_l):
        for h in range(H):
            jobs.append((ckh[b, :n, offk[h]:offk[h] + rk[h]], cvh[b, :n, offv[h]:offv[h] + rv[h]], qh[b, h],
                         bkh[offk[h]:offk[h] + rk[h]], bvh[offv[h]:offv[h] + rv[h]]))
            idx.append((b, h))
    refs = oracle_many(qfmt, jobs, 1 / math.sqrt(D))
    for (b, h), ref in zip(idx, refs):
        assert within(got[b, h], ref, TOL_BF16), (b, h, rk[h], rv[h])
