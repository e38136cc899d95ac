"""ctypes binding of the CPU oracle (``liblr_oracle.so``).

TEST INFRASTRUCTURE: only ``tests/``, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
loads it, and it never loads the GPU library.

The oracle computes the plain definition of the decode step of per-head
low-rank attention over a quantised latent cache (WSVD page, "Fine-grained
per-head SVD" and "System implementation (fused kernel)"; LASER page, "Hybrid
SVD-quantisation", RTN): quantise each latent row, dequantise it, rebuild
k_t = c~^K_t B^K_h and v_t = c~^V_t B^V_h, then softmax attention, in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lr_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liblr_oracle.so")
_SAN_PATH = os.path.join(_HERE, "liblr_oracle_san.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source; a
# process that loads it must preload the gcc sanitizer runtimes
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]

QFMT_INT8, QFMT_INT4, QFMT_NONE = 0, 1, 2


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with g++ (IEEE fp32/fp64, no contraction, no
    fast-math); sanitize=True builds liblr_oracle_san.so with ASan and UBSan."""
    path = _SAN_PATH if sanitize else _LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return path


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("LR_ORACLE_LIB") or _LIB_PATH   # e.g. the sanitizer build
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.lro_f32_to_f16.argtypes = [ctypes.c_float]
        L.lro_f32_to_f16.restype = ctypes.c_uint16
        L.lro_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.lro_f16_to_f32.restype = ctypes.c_float
        L.lro_quant_int8.argtypes = [P, ctypes.c_int, P, P]
        L.lro_quant_int8.restype = None
        L.lro_quant_int4.argtypes = [P, ctypes.c_int, P, P]
        L.lro_quant_int4.restype = None
        L.lro_quant_int8_rows.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.lro_quant_int8_rows.restype = None
        L.lro_quant_int4_rows.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.lro_quant_int4_rows.restype = None
        L.lro_attend.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, P, P, P, P, P, ctypes.c_double, P, P]
        L.lro_attend.restype = ctypes.c_int
        L.lro_attend_dequantised.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             P, P, P, P, P, ctypes.c_double, P, P]
        L.lro_attend_dequantised.restype = ctypes.c_int
        L.lro_latents.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
        L.lro_latents.restype = ctypes.c_int
        L.lro_hadamard.argtypes = [ctypes.c_int, P]
        L.lro_hadamard.restype = ctypes.c_int
        L.lro_block_rotation.argtypes = [ctypes.c_int, ctypes.c_int, P]
        L.lro_block_rotation.restype = ctypes.c_int
        L.lro_rotate_factors.argtypes = [ctypes.c_int] * 4 + [P] * 4
        L.lro_rotate_factors.restype = ctypes.c_int
        L.lro_allocate_ranks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_double,
                                         ctypes.c_double, P]
        L.lro_allocate_ranks.restype = ctypes.c_int
        L.lro_quant_act_groups.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.lro_quant_act_groups.restype = None
        L.lro_ffn.argtypes = [ctypes.c_int] * 6 + [P] * 9
        L.lro_ffn.restype = ctypes.c_int
        L.lro_ffn_trace.argtypes = [ctypes.c_int] * 6 + [P] * 13
        L.lro_ffn_trace.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def f32_to_f16_bits(x: float) -> int:
    return int(lib().lro_f32_to_f16(ctypes.c_float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().lro_f16_to_f32(ctypes.c_uint16(h)))


def quant_int8(c: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Rows of ``c`` (fp32 [..., r]) -> (int8 values [..., r], fp32 scales [...])."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    r = c.shape[-1]
    rows = c.reshape(-1, r)
    q = np.empty(rows.shape, dtype=np.int8)
    s = np.empty(rows.shape[0], dtype=np.float32)
    lib().lro_quant_int8_rows(_ptr(rows), rows.shape[0], r, _ptr(q), _ptr(s))
    return q.reshape(c.shape), s.reshape(c.shape[:-1])


def quant_int4(c: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Rows of ``c`` (fp32 [..., r]) -> (values in [-7, 7] as int8 [..., r],
    fp16 scale bit patterns uint16 [..., ceil(r/32)])."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    r = c.shape[-1]
    ng = (r + 31) // 32
    rows = c.reshape(-1, r)
    q = np.empty(rows.shape, dtype=np.int8)
    s = np.empty((rows.shape[0], ng), dtype=np.uint16)
    lib().lro_quant_int4_rows(_ptr(rows), rows.shape[0], r, _ptr(q), _ptr(s))
    return q.reshape(c.shape), s.reshape(c.shape[:-1] + (ng,))


def attend(qfmt: int, ck: np.ndarray, cv: np.ndarray, q: np.ndarray, bk: np.ndarray,
           bv: np.ndarray, scale: float, want_probs: bool = False):
    """One attention unit: fp32 latents ck [T, rk], cv [T, rv]; q [d]; B^K [rk, d];
    B^V [rv, d] (q and B widened exactly to fp64).  Returns o [d] (fp64), and the
    softmax weights [T] when ``want_probs``."""
    ck = np.ascontiguousarray(ck, dtype=np.float32)
    cv = np.ascontiguousarray(cv, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float64)
    bk = np.ascontiguousarray(bk, dtype=np.float64)
    bv = np.ascontiguousarray(bv, dtype=np.float64)
    T, rk = ck.shape
    T2, rv = cv.shape
    d = q.shape[0]
    assert T == T2 and bk.shape == (rk, d) and bv.shape == (rv, d)
    out = np.zeros(d, dtype=np.float64)
    probs = np.zeros(max(T, 1), dtype=np.float64) if want_probs else None
    rc = lib().lro_attend(qfmt, T, rk, rv, d, _ptr(ck), _ptr(cv), _ptr(q), _ptr(bk), _ptr(bv),
                          float(scale), _ptr(out), _ptr(probs) if want_probs else None)
    if rc != 0:
        raise ValueError("lro_attend rejected its arguments")
    return (out, probs[:T]) if want_probs else out


def attend_dequantised(ctk: np.ndarray, ctv: np.ndarray, q: np.ndarray, bk: np.ndarray,
                       bv: np.ndarray, scale: float, want_probs: bool = False):
    """One attention unit from already dequantised fp64 latents ctk [T, rk], ctv [T, rv]."""
    ctk = np.ascontiguousarray(ctk, dtype=np.float64)
    ctv = np.ascontiguousarray(ctv, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    bk = np.ascontiguousarray(bk, dtype=np.float64)
    bv = np.ascontiguousarray(bv, dtype=np.float64)
    T, rk = ctk.shape
    T2, rv = ctv.shape
    d = q.shape[0]
    assert T == T2 and bk.shape == (rk, d) and bv.shape == (rv, d)
    out = np.zeros(d, dtype=np.float64)
    probs = np.zeros(max(T, 1), dtype=np.float64) if want_probs else None
    rc = lib().lro_attend_dequantised(T, rk, rv, d, _ptr(ctk), _ptr(ctv), _ptr(q), _ptr(bk),
                                      _ptr(bv), float(scale), _ptr(out),
                                      _ptr(probs) if want_probs else None)
    if rc != 0:
        raise ValueError("lro_attend_dequantised rejected its arguments")
    return (out, probs[:T]) if want_probs else out


def latents(x: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Latent generation c = x A in fp64: x [T, E], A [E, N] (heads side by side)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    T, E = x.shape
    E2, N = a.shape
    assert E == E2
    c = np.zeros((T, N), dtype=np.float64)
    if lib().lro_latents(T, E, N, _ptr(x), _ptr(a), _ptr(c)) != 0:
        raise ValueError("lro_latents rejected its arguments")
    return c


def hadamard(n: int) -> np.ndarray:
    """Normalised Sylvester-Hadamard matrix of order n (a power of two)."""
    h = np.zeros((n, n), dtype=np.float64)
    if lib().lro_hadamard(n, _ptr(h)) != 0:
        raise ValueError("n must be a power of two")
    return h


def block_rotation(r: int, block: int) -> Tuple[np.ndarray, int]:
    """(S, g): the r x r block-diagonal Hadamard rotation of a rank-r head and its block."""
    s = np.zeros((r, r), dtype=np.float64)
    g = lib().lro_block_rotation(r, block, _ptr(s))
    if g < 0:
        raise ValueError("bad rank or block")
    return s, g


def rotate_factors(a: np.ndarray, b: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """(A S, S^T B) for one head: A [E, r], B [r, d]."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    E, r = a.shape
    r2, d = b.shape
    assert r == r2
    ao = np.zeros_like(a)
    bo = np.zeros_like(b)
    if lib().lro_rotate_factors(E, r, d, block, _ptr(a), _ptr(b), _ptr(ao), _ptr(bo)) < 0:
        raise ValueError("lro_rotate_factors rejected its arguments")
    return ao, bo


def allocate_ranks(scores: np.ndarray, step: int, cost_per_component: float, budget: float) -> np.ndarray:
    """Greedy rank allocation: scores [n_units, max_rank] (fp64) -> ranks [n_units] (int)."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    n, m = scores.shape
    ranks = np.zeros(n, dtype=np.int32)
    rc = lib().lro_allocate_ranks(n, m, step, _ptr(scores), float(cost_per_component), float(budget),
                                  _ptr(ranks))
    if rc == -2:
        raise ValueError("budget below one block per unit")
    if rc != 0:
        raise ValueError("lro_allocate_ranks rejected its arguments")
    return ranks


def quant_act_groups(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Activations [T, K] -> (int8 codes [T, K], fp32 scales [T, ceil(K/64)]), one
    scale per token per group of 64 elements."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    T, K = a.shape
    q = np.empty((T, K), np.int8)
    s = np.empty((T, (K + 63) // 64), np.float32)
    lib().lro_quant_act_groups(_ptr(a), T, K, _ptr(q), _ptr(s))
    return q, s


def ffn(x, wg, wu, ag, au, bg, bu, wd, quantise: bool = True) -> np.ndarray:
    """Hybrid FFN: x [T, E]; dense rows wg, wu [F-S, E]; factors ag, au [r, E],
    bg, bu [S, r]; wd [E, F] (all fp32 values).  Returns y [T, E] in fp64."""
    arrs = [np.ascontiguousarray(v, dtype=np.float32) for v in (x, wg, wu, ag, au, bg, bu, wd)]
    x, wg, wu, ag, au, bg, bu, wd = arrs
    T, E = x.shape
    F = wd.shape[1]
    S = bg.shape[0]
    r = ag.shape[0]
    assert wg.shape == (F - S, E) and wu.shape == (F - S, E) and wd.shape == (E, F)
    assert ag.shape == (r, E) and au.shape == (r, E) and bg.shape == (S, r) and bu.shape == (S, r)
    y = np.zeros((T, E), np.float64)
    rc = lib().lro_ffn(0 if quantise else 1, T, E, F, S, r, *[_ptr(v) for v in arrs], _ptr(y))
    if rc != 0:
        raise ValueError("lro_ffn rejected its arguments")
    return y


def ffn_trace(x, wg, wu, ag, au, bg, bu, wd, quantise: bool = True):
    """ffn() and its intermediates: (y [T, E] fp64, z [T, 2r] fp32 latents (gate
    then up), g, u [T, F] fp64 pre-activations, h [T, F] fp32)."""
    arrs = [np.ascontiguousarray(v, dtype=np.float32) for v in (x, wg, wu, ag, au, bg, bu, wd)]
    x, wg, wu, ag, au, bg, bu, wd = arrs
    T, E = x.shape
    F = wd.shape[1]
    S = bg.shape[0]
    r = ag.shape[0]
    y = np.zeros((T, E), np.float64)
    z = np.zeros((T, 2 * r), np.float32)
    g = np.zeros((T, F), np.float64)
    u = np.zeros((T, F), np.float64)
    h = np.zeros((T, F), np.float32)
    rc = lib().lro_ffn_trace(0 if quantise else 1, T, E, F, S, r, *[_ptr(v) for v in arrs], _ptr(y), _ptr(z),
                             _ptr(g), _ptr(u), _ptr(h))
    if rc != 0:
        raise ValueError("lro_ffn_trace rejected its arguments")
    return y, z, g, u, h
