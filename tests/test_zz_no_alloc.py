"""The allocation-free fused append + decode (lr_attn_append_decode_noalloc)
through the C ABI, against lr_attn_append_decode, which takes the caller's
workspace.  Two calls in a row, the second on a smaller input (fewer
sequences, a shorter context, another rank and format), both on launches that
split the context so that the split partials live in the library's device
array: each call's output and cache bytes must equal the workspace entry
point's bit for bit (same kernels, same launch shape), and its output must be
within the decode tolerance of the oracle."""
import math

import numpy as np
import pytest
import torch

from latent_kv_attention_lr_amd import (LR_DT_BF16, LR_Q_INT4_G32, LR_Q_INT8_TOKEN,
                                        lr_attn_append_decode, lr_attn_append_decode_noalloc,
                                        lr_attn_workspace_bytes)
from latent_kv_attention_lr_amd.session import DecodeSession
from gpu_util import TOL_BF16, oracle_many, within

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def _case(batch, heads, ctx, rank, qfmt, seed):
    """A prefilled session (ctx random tokens), the new token's latents, q and factors."""
    g = torch.Generator().manual_seed(seed)
    s = DecodeSession(1, batch, heads, ctx + 1, qfmt, LR_DT_BF16, [[rank] * heads], [[rank] * heads],
                      device=DEV)
    n = heads * rank
    ck = torch.randn(batch, ctx + 1, n, generator=g)
    cv = torch.randn(batch, ctx + 1, n, generator=g)
    s.append(0, ck[:, :ctx].contiguous().to(DEV), cv[:, :ctx].contiguous().to(DEV),
             torch.zeros(batch, dtype=torch.int32, device=DEV))
    bk = (torch.randn(n, 128, generator=g) / math.sqrt(rank)).to(torch.bfloat16)
    bv = (torch.randn(n, 128, generator=g) / math.sqrt(rank)).to(torch.bfloat16)
    q = torch.randn(batch, heads, 128, generator=g).to(torch.bfloat16)
    s.set_factors(0, bk.to(DEV), bv.to(DEV))
    return s, ck, cv, q


def _one_call(batch, heads, ctx, rank, qfmt, seed):
    say(f"noalloc case batch={batch} heads={heads} ctx={ctx} rank={rank} qfmt={qfmt}")
    s, ck, cv, q = _case(batch, heads, ctx, rank, qfmt, seed)
    T = ctx + 1
    need = lr_attn_workspace_bytes(s.plan, T)
    assert need > 0, "the case must split the context (partials in the scratch array)"
    pos = torch.full((batch,), ctx, dtype=torch.int32, device=DEV)
    ln = torch.full((batch,), T, dtype=torch.int32, device=DEV)
    ckn = ck[:, ctx].contiguous().to(DEV)
    cvn = cv[:, ctx].contiguous().to(DEV)
    qd = q.to(DEV)
    cache_ref = s.caches[0].clone()
    out_ref = torch.empty(batch, heads, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(out_ref, float("nan"))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(128)
    lr_attn_append_decode(s.plan, 0, cache_ref, ckn, cvn, pos, ln, T, qd, s.bk[0], s.bv[0], scale,
                          out_ref, ws, ws.numel())
    lr_attn_append_decode_noalloc(s.plan, 0, s.caches[0], ckn, cvn, pos, ln, T, qd, s.bk[0], s.bv[0],
                                  scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "output differs from the workspace entry point"
    assert torch.equal(s.caches[0], cache_ref), "cache bytes differ from the workspace entry point"
    # and the oracle on every (b, h) unit
    bk64, bv64 = s.bk[0].double().cpu().numpy(), s.bv[0].double().cpu().numpy()
    jobs, idx = [], []
    for b in range(batch):
        for h in range(heads):
            o = h * rank
            jobs.append((ck[b, :T, o:o + rank].numpy(), cv[b, :T, o:o + rank].numpy(),
                         q[b, h].double().numpy(), bk64[o:o + rank], bv64[o:o + rank]))
            idx.append((b, h))
    refs = oracle_many(qfmt, jobs, scale)
    got = out.double().cpu().numpy()
    for (b, h), ref in zip(idx, refs):
        assert within(got[b, h], ref, TOL_BF16), (b, h, float(np.max(np.abs(got[b, h] - ref))))
    s.close()


def test_noalloc_equals_workspace_entry_point_twice_second_smaller():
    _one_call(batch=2, heads=4, ctx=8000, rank=32, qfmt=LR_Q_INT8_TOKEN, seed=11)
    _one_call(batch=1, heads=4, ctx=6000, rank=64, qfmt=LR_Q_INT4_G32, seed=12)
