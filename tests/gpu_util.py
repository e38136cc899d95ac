"""Helpers shared by the GPU tests: reading the documented cache layout back
on the host, running the oracle on a thread pool, and the tolerance rule."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))

# Output tolerance: |o_gpu - o_ref| <= 1e-2 * max|o_ref| + 1e-3 with bf16 q,
# factors and output; <= 1e-4 * max|o_ref| with fp32 ones.
TOL_BF16 = (1e-2, 1e-3)
TOL_F32 = (1e-4, 0.0)


def within(got: np.ndarray, ref: np.ndarray, tol) -> bool:
    rel, ab = tol
    return float(np.max(np.abs(got - ref))) <= rel * float(np.max(np.abs(ref))) + ab


def read_codes(cache: np.ndarray, hl: dict, qfmt: int, b: int, slots: np.ndarray, kv: str):
    """Codes and scale bit patterns of ``slots`` of sequence ``b`` from a cache
    buffer copied to the host, using the byte layout of include/lr_attn.h.
    Returns (codes int8 [n, r], scales: uint32 [n] for int8 or uint16 [n, groups])."""
    r = hl["rank_" + kv]
    rb = hl["row_bytes_" + kv]
    tb = hl["tile_bytes_" + kv]
    slots = np.asarray(slots, dtype=np.int64)
    tile = hl[kv + "_offset"] + b * hl["plane_bytes_" + kv] + (slots // 64) * tb
    lane = slots % 64
    cols = []
    for c in range((rb + 15) // 16):
        w = min(16, rb - 16 * c)
        base = tile + 1024 * c + w * lane
        cols.append(cache[base[:, None] + np.arange(w)[None, :]])
    raw = np.concatenate(cols, axis=1)  # [n, rb] uint8
    if qfmt == oracle.QFMT_INT8:
        codes = raw.view(np.int8)
        sb = cache[(tile + 64 * rb + 4 * lane)[:, None] + np.arange(4)[None, :]]
        scales = sb.copy().view(np.uint32)[:, 0]
    else:
        lo = (raw & 0xF).astype(np.int8)
        hi = (raw >> 4).astype(np.int8)
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        codes = np.empty((len(slots), 2 * rb), np.int8)
        codes[:, 0::2] = lo
        codes[:, 1::2] = hi
        ng = (r + 31) // 32
        sc = []
        for g in range(ng):
            off = tile + 64 * rb + 2 * (64 * g + lane)
            sc.append(cache[off[:, None] + np.arange(2)[None, :]].copy().view(np.uint16)[:, 0])
        scales = np.stack(sc, axis=1)
    return codes[:, :r], scales


def oracle_quant(qfmt: int, c: np.ndarray):
    """Oracle codes and scale bit patterns for rows ``c`` (fp32 [n, r])."""
    if qfmt == oracle.QFMT_INT8:
        q, s = oracle.quant_int8(c)
        return q, s.view(np.uint32)
    return oracle.quant_int4(c)


def oracle_many(qfmt: int, jobs, scale: float):
    """Run the oracle on a list of (ck, cv, q, bk, bv) in parallel threads."""
    futs = [POOL.submit(oracle.attend, qfmt, ck, cv, q, bk, bv, scale) for (ck, cv, q, bk, bv) in jobs]
    return [f.result() for f in futs]
