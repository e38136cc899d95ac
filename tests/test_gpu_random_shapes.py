"""GPU parity on seeded random shapes: every (b, h) of a random plan against
the CPU oracle, through the C ABI.

Each case draws a latent format and I/O type, a batch of 1-6 sequences,
1-32 heads with their own K and V ranks (multiples of 8 up to 128, so every
register bucket, paired and single lanes, and mixed-rank layers occur), a
capacity, ragged lengths (empty, one token, tile edges, full), the launch
shape knobs (wavefronts per work-group, context-split cap) and max_len.  It
checks the absorbed decode (and, with bf16 I/O, the explicit form) against
the oracle within the decode tolerance, and that the fused append + decode
writes the same cache bytes and gives the same outputs, bit for bit, as the
separate append and decode.
"""
import math

import numpy as np
import pytest
import torch

import lrgen
from latent_kv_attention_lr_amd import LR_DT_BF16, LR_DT_F32, LR_Q_INT4_G32, LR_Q_INT8_TOKEN
from latent_kv_attention_lr_amd.session import DecodeSession
from gpu_util import TOL_BF16, TOL_F32, oracle_many, within

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 64


def _case(seed):
    rng = np.random.default_rng(0x5EED1000 + seed)
    c = {"qfmt": int(rng.choice([LR_Q_INT8_TOKEN, LR_Q_INT4_G32])),
         "io": int(rng.choice([LR_DT_BF16, LR_DT_F32])),
         "B": int(rng.integers(1, 7)),
         "H": int(rng.choice([1, 2, 3, 5, 8, 13, 32]))}
    top = int(rng.choice([32, 64, 96, 128]))          # the layer's register bucket
    c["rk"] = [int(8 * rng.integers(1, top // 8 + 1)) for _ in range(c["H"])]
    c["rv"] = [int(8 * rng.integers(1, top // 8 + 1)) for _ in range(c["H"])]
    # at most ~6 M latent values on the host
    per_tok = c["B"] * (sum(c["rk"]) + sum(c["rv"]))
    cap_max = max(1, min(2500, 6_000_000 // per_tok))
    c["cap"] = int(rng.integers(1, cap_max + 1))
    edges = [0, 1, 63, 64, 65, c["cap"]]
    c["lens"] = [int(min(c["cap"], rng.choice(edges) if rng.random() < 0.5 else rng.integers(0, c["cap"] + 1)))
                 for _ in range(c["B"])]
    c["max_len"] = int(rng.choice([c["cap"], max(1, max(c["lens"]))]))
    c["wg_waves"] = int(rng.choice([0, 0, 4, 8, 16]))
    c["max_splits"] = int(rng.choice([0, 0, 1, 2, 5]))
    c["explicit"] = c["io"] == LR_DT_BF16 and bool(rng.random() < 0.5)
    c["pos"] = [int(rng.integers(-1, c["cap"] + 1)) for _ in range(c["B"])]
    return c, rng


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_decode_matches_oracle(seed):
    c, rng = _case(seed)
    print(f"random shape {seed}: {c}", flush=True)
    B, H, cap = c["B"], c["H"], c["cap"]
    rk, rv = c["rk"], c["rv"]
    s = DecodeSession(1, B, H, cap, c["qfmt"], c["io"], [rk], [rv], device=DEV,
                      max_splits=c["max_splits"], wg_waves=c["wg_waves"])
    try:
        ck = (rng.standard_normal((B, cap, sum(rk))) * 1.2).astype(np.float32)
        cv = (rng.standard_normal((B, cap, sum(rv))) * 0.9).astype(np.float32)
        s.append(0, torch.from_numpy(ck).to(DEV), torch.from_numpy(cv).to(DEV),
                 torch.zeros(B, dtype=torch.int32, device=DEV))
        dt = torch.bfloat16 if c["io"] == LR_DT_BF16 else torch.float32
        bk = (torch.from_numpy(rng.standard_normal((sum(rk), 128))) / 6).to(dt).to(DEV).contiguous()
        bv = (torch.from_numpy(rng.standard_normal((sum(rv), 128))) / 6).to(dt).to(DEV).contiguous()
        s.set_factors(0, bk, bv)
        q = (torch.from_numpy(rng.standard_normal((B, H, 128)) * 2)).to(dt).to(DEV).contiguous()
        lens, max_len = c["lens"], c["max_len"]
        s.lengths.copy_(torch.tensor(lens, dtype=torch.int32))
        forms = [False] + ([True] if c["explicit"] else [])
        outs = {}
        for explicit in forms:
            out = torch.full_like(q, float("nan"))
            s.decode(0, q, out, max_len=max_len, explicit=explicit)
            torch.cuda.synchronize()
            outs[explicit] = out.double().cpu().numpy()
        ok, ov = lrgen.head_offsets(rk), lrgen.head_offsets(rv)
        qn, bkn, bvn = q.double().cpu().numpy(), bk.double().cpu().numpy(), bv.double().cpu().numpy()
        jobs, keys = [], []
        for b in range(B):
            T = min(lens[b], max_len)
            for h in range(H):
                jobs.append((ck[b, :T, ok[h]:ok[h] + rk[h]], cv[b, :T, ov[h]:ov[h] + rv[h]], qn[b, h],
                             bkn[ok[h]:ok[h] + rk[h]], bvn[ov[h]:ov[h] + rv[h]]))
                keys.append((b, h, T))
        refs = oracle_many(c["qfmt"], jobs, 1 / math.sqrt(128))
        tol = TOL_BF16 if c["io"] == LR_DT_BF16 else TOL_F32
        for explicit, got in outs.items():
            for (b, h, T), ref in zip(keys, refs):
                if T == 0:
                    assert np.array_equal(got[b, h], np.zeros(128)), (seed, explicit, b, h)
                else:
                    assert within(got[b, h], ref, tol), (seed, explicit, b, h, T, rk[h], rv[h])

        # fused append + decode == append, then decode (cache bytes and outputs)
        nk = torch.from_numpy((rng.standard_normal((B, 1, sum(rk))) * 1.1).astype(np.float32)).to(DEV)
        nv = torch.from_numpy((rng.standard_normal((B, 1, sum(rv))) * 0.9).astype(np.float32)).to(DEV)
        pos = torch.tensor(c["pos"], dtype=torch.int32, device=DEV)
        before = s.caches[0].clone()
        out_a = torch.full_like(q, float("nan"))
        s.append(0, nk, nv, pos)
        s.decode(0, q, out_a, max_len=max_len)
        torch.cuda.synchronize()
        cache_a = s.caches[0].clone()
        s.caches[0].copy_(before)
        out_b = torch.full_like(q, float("nan"))
        s.append_decode(0, nk.view(B, -1), nv.view(B, -1), pos, q, out_b, max_len=max_len)
        torch.cuda.synchronize()
        assert torch.equal(s.caches[0], cache_a), (seed, "fused append wrote different cache bytes")
        assert torch.equal(out_a, out_b), (seed, "fused decode differs from append + decode")
    finally:
        s.close()
