"""Thin Python binding of ``liblr_attn.so`` (the C ABI in ``include/lr_attn.h``).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  Functions keep the C names; tensor arguments are
torch tensors on the GPU (only their device pointers are passed), streams
default to torch's current stream.  If the library has not been built the
import fails: there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# LR_ATTN_LIB selects another build of the same library (the sanitizer build)
LIB_PATH = os.environ.get("LR_ATTN_LIB") or os.path.join(_HERE, "liblr_attn.so")

LR_OK, LR_EINVAL, LR_EUNSUPPORTED, LR_ERANGE, LR_EWORKSPACE, LR_EHIP = range(6)
LR_Q_INT8_TOKEN, LR_Q_INT4_G32 = 0, 1
LR_DT_BF16, LR_DT_F32 = 0, 1
LR_HEAD_DIM = 128
LR_TILE_TOKENS = 64


class LrAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lr_attn_strerror(status)
        if status == LR_EHIP:
            msg += f" (hipError {lr_attn_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")


class lr_attn_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("qfmt", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("wg_waves", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rank_k", ctypes.POINTER(ctypes.c_int32)),
                ("rank_v", ctypes.POINTER(ctypes.c_int32))]


class lr_attn_head_layout(ctypes.Structure):
    _fields_ = [("k_offset", ctypes.c_uint64), ("v_offset", ctypes.c_uint64),
                ("plane_bytes_k", ctypes.c_uint64), ("plane_bytes_v", ctypes.c_uint64),
                ("rank_k", ctypes.c_int32), ("rank_v", ctypes.c_int32),
                ("row_bytes_k", ctypes.c_int32), ("row_bytes_v", ctypes.c_int32),
                ("scale_bytes_k", ctypes.c_int32), ("scale_bytes_v", ctypes.c_int32),
                ("tile_bytes_k", ctypes.c_int32), ("tile_bytes_v", ctypes.c_int32),
                ("latent_offset_k", ctypes.c_int32), ("latent_offset_v", ctypes.c_int32),
                ("factor_offset_k", ctypes.c_int64), ("factor_offset_v", ctypes.c_int64)]


class lr_ffn_desc(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_lowrank", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def _load() -> ctypes.CDLL:
    # torch (device memory and streams) brings its own HIP runtime.  It must be
    # loaded first so that the library binds to that same runtime (both carry
    # the soname libamdhip64.so.7); two runtimes in one process do not share
    # devices, streams or allocations.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python latent_kv_attention_lr_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    rt = _hip_runtimes()
    if len(rt) > 1:
        raise ImportError(f"more than one HIP runtime is loaded ({rt}); import torch before "
                          "anything that loads /opt/rocm's libamdhip64")
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    plan_pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "lr_attn_plan_create": (ctypes.c_int, [ctypes.POINTER(lr_attn_desc), plan_pp]),
        "lr_attn_plan_destroy": (None, [P]),
        "lr_attn_cache_bytes": (SZ, [P, I32]),
        "lr_attn_latent_elems": (SZ, [P, I32, I32]),
        "lr_attn_factor_elems": (SZ, [P, I32, I32]),
        "lr_attn_head_layout_get": (ctypes.c_int, [P, I32, I32, ctypes.POINTER(lr_attn_head_layout)]),
        "lr_attn_workspace_bytes": (SZ, [P, I32]),
        "lr_attn_append_latent": (ctypes.c_int, [P, I32, P, P, P, P, I32, P]),
        "lr_attn_decode": (ctypes.c_int, [P, I32, P, P, I32, P, P, P, ctypes.c_float, P, P, SZ, P]),
        "lr_attn_decode_explicit": (ctypes.c_int, [P, I32, P, P, I32, P, P, P, ctypes.c_float, P, P, SZ, P]),
        "lr_attn_append_decode": (ctypes.c_int, [P, I32, P, P, P, P, P, I32, P, P, P, ctypes.c_float,
                                                 P, P, SZ, P]),
        "lr_attn_append_decode_noalloc": (ctypes.c_int, [P, I32, P, P, P, P, P, I32, P, P, P,
                                                         ctypes.c_float, P, P]),
        "lr_attn_packed_projection_elems": (SZ, [P, I32, I32]),
        "lr_attn_pack_projection": (ctypes.c_int, [P, I32, I32, P, P, P, P]),
        "lr_attn_project_latent": (ctypes.c_int, [P, I32, P, I32, I32, P, P, P, P]),
        "lr_attn_project_workspace_bytes": (SZ, [P, I32]),
        "lr_attn_project_append": (ctypes.c_int, [P, I32, P, P, I32, P, P, I32, P, SZ, P]),
        "lr_attn_project_latent_parts": (ctypes.c_int, [P, I32, P, I32, I32, P, I32, P, P, P]),
        "lr_attn_project_parts": (I32, [P, I32, I32, I32]),
        "lr_attn_project_decode_workspace_bytes": (SZ, [P, I32, I32]),
        "lr_attn_project_append_decode": (ctypes.c_int, [P, I32, P, P, I32, P, P, P, I32, P, P, P,
                                                         ctypes.c_float, P, P, SZ, P]),
        "lr_attn_hadamard_block": (I32, [P, I32, I32, I32, I32]),
        "lr_attn_hadamard_rotate_rows": (ctypes.c_int, [P, I32, I32, I32, P, ctypes.c_int64]),
        "lr_attn_allocate_ranks": (ctypes.c_int, [I32, I32, I32, P, ctypes.c_int64, ctypes.c_int64, P, P]),
        "lr_ffn_weight_bytes": (SZ, [ctypes.POINTER(lr_ffn_desc)]),
        "lr_ffn_workspace_bytes": (SZ, [ctypes.POINTER(lr_ffn_desc), I32]),
        "lr_ffn_prepare_weights": (ctypes.c_int, [ctypes.POINTER(lr_ffn_desc)] + [P] * 8),
        "lr_ffn_decode": (ctypes.c_int, [ctypes.POINTER(lr_ffn_desc), P, P, I32, P, P, SZ, P]),
        "lr_attn_probe_read": (ctypes.c_int, [P, SZ, P, P]),
        "lr_attn_check_count": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint64)]),
        "lr_attn_check_shrink": (ctypes.c_int, [ctypes.c_uint64]),
        "lr_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "lr_attn_last_hip_error": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_lib = _load()


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor, or an int/None passed through."""
    if x is None or isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != LR_OK:
        raise LrAttnError(status, where)


def lr_attn_strerror(status: int) -> str:
    return _lib.lr_attn_strerror(status).decode()


def lr_attn_last_hip_error() -> int:
    return int(_lib.lr_attn_last_hip_error())


def lr_attn_plan_create(n_layers: int, batch: int, n_heads: int, capacity: int, qfmt: int,
                        io_dtype: int, rank_k: Sequence[int], rank_v: Sequence[int],
                        head_dim: int = LR_HEAD_DIM, max_splits: int = 0,
                        wg_waves: int = 0) -> int:
    """Returns an opaque plan handle (int); raises LrAttnError on a bad description."""
    n = n_layers * n_heads
    rk = (ctypes.c_int32 * max(n, 1))(*[int(r) for r in rank_k])
    rv = (ctypes.c_int32 * max(n, 1))(*[int(r) for r in rank_v])
    d = lr_attn_desc(n_layers, batch, n_heads, head_dim, capacity, qfmt, io_dtype, max_splits,
                     wg_waves, 0, ctypes.cast(rk, ctypes.POINTER(ctypes.c_int32)),
                     ctypes.cast(rv, ctypes.POINTER(ctypes.c_int32)))
    h = ctypes.c_void_p()
    _check(_lib.lr_attn_plan_create(ctypes.byref(d), ctypes.byref(h)), "lr_attn_plan_create")
    return h.value


def lr_attn_plan_destroy(plan: int) -> None:
    _lib.lr_attn_plan_destroy(plan)


def lr_attn_cache_bytes(plan: int, layer: int) -> int:
    return int(_lib.lr_attn_cache_bytes(plan, layer))


def lr_attn_latent_elems(plan: int, layer: int, kv: int) -> int:
    return int(_lib.lr_attn_latent_elems(plan, layer, kv))


def lr_attn_factor_elems(plan: int, layer: int, kv: int) -> int:
    return int(_lib.lr_attn_factor_elems(plan, layer, kv))


def lr_attn_head_layout_get(plan: int, layer: int, head: int) -> Dict[str, int]:
    out = lr_attn_head_layout()
    _check(_lib.lr_attn_head_layout_get(plan, layer, head, ctypes.byref(out)), "lr_attn_head_layout_get")
    return {name: getattr(out, name) for name, _ in lr_attn_head_layout._fields_}


def lr_attn_workspace_bytes(plan: int, max_len: int) -> int:
    return int(_lib.lr_attn_workspace_bytes(plan, max_len))


def lr_attn_append_latent(plan: int, layer: int, cache, ck, cv, pos, n_new: int, stream=None) -> None:
    _check(_lib.lr_attn_append_latent(plan, layer, _ptr(cache), _ptr(ck), _ptr(cv), _ptr(pos),
                                      n_new, _stream(stream)), "lr_attn_append_latent")


def lr_attn_decode(plan: int, layer: int, cache, length, max_len: int, q, bk, bv,
                   softmax_scale: float, out, workspace, ws_bytes: int, stream=None) -> None:
    _check(_lib.lr_attn_decode(plan, layer, _ptr(cache), _ptr(length), max_len, _ptr(q), _ptr(bk),
                               _ptr(bv), softmax_scale, _ptr(out), _ptr(workspace), ws_bytes,
                               _stream(stream)), "lr_attn_decode")


def lr_attn_append_decode(plan: int, layer: int, cache, ck, cv, pos, lengths, max_len: int, q, bk,
                          bv, softmax_scale: float, out, workspace=None, ws_bytes: int = 0,
                          stream=None) -> None:
    """lr_attn_append_latent (one token per sequence) then lr_attn_decode, fused."""
    _check(_lib.lr_attn_append_decode(plan, layer, _ptr(cache), _ptr(ck), _ptr(cv), _ptr(pos),
                                      _ptr(lengths), max_len, _ptr(q), _ptr(bk), _ptr(bv),
                                      float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes,
                                      _stream(stream)), "lr_attn_append_decode")


def lr_attn_append_decode_noalloc(plan: int, layer: int, cache, ck, cv, pos, lengths, max_len: int,
                                  q, bk, bv, softmax_scale: float, out, stream=None) -> None:
    """lr_attn_append_decode with the library's own device scratch: allocates nothing."""
    _check(_lib.lr_attn_append_decode_noalloc(plan, layer, _ptr(cache), _ptr(ck), _ptr(cv), _ptr(pos),
                                              _ptr(lengths), max_len, _ptr(q), _ptr(bk), _ptr(bv),
                                              float(softmax_scale), _ptr(out), _stream(stream)),
           "lr_attn_append_decode_noalloc")


def lr_attn_decode_explicit(plan: int, layer: int, cache, length, max_len: int, q, bk, bv,
                            softmax_scale: float, out, workspace, ws_bytes: int, stream=None) -> None:
    _check(_lib.lr_attn_decode_explicit(plan, layer, _ptr(cache), _ptr(length), max_len, _ptr(q),
                                        _ptr(bk), _ptr(bv), softmax_scale, _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
           "lr_attn_decode_explicit")


def lr_attn_packed_projection_elems(plan: int, layer: int, embed: int) -> int:
    return int(_lib.lr_attn_packed_projection_elems(plan, layer, embed))


def lr_attn_pack_projection(plan: int, layer: int, embed: int, wk, wv, packed, stream=None) -> None:
    """Pack the factors wk/wv ([latent_elems, embed] bf16, A transposed) for the projection."""
    _check(_lib.lr_attn_pack_projection(plan, layer, embed, _ptr(wk), _ptr(wv), _ptr(packed),
                                        _stream(stream)), "lr_attn_pack_projection")


def lr_attn_project_latent(plan: int, layer: int, x, n_tokens: int, embed: int, packed, ck, cv,
                           stream=None) -> None:
    """ck/cv [n_tokens, latent_elems] (fp32) = x [n_tokens, embed] (bf16) times the
    packed factors."""
    _check(_lib.lr_attn_project_latent(plan, layer, _ptr(x), n_tokens, embed, _ptr(packed),
                                       _ptr(ck), _ptr(cv), _stream(stream)),
           "lr_attn_project_latent")


def lr_attn_project_workspace_bytes(plan: int, n_new: int) -> int:
    return int(_lib.lr_attn_project_workspace_bytes(plan, n_new))


def lr_attn_project_append(plan: int, layer: int, cache, x, embed: int, packed, pos, n_new: int,
                           workspace, ws_bytes: int, stream=None) -> None:
    """lr_attn_project_latent of x [batch, n_new, embed] then lr_attn_append_latent."""
    _check(_lib.lr_attn_project_append(plan, layer, _ptr(cache), _ptr(x), embed, _ptr(packed),
                                       _ptr(pos), n_new, _ptr(workspace), ws_bytes, _stream(stream)),
           "lr_attn_project_append")


def lr_attn_project_latent_parts(plan: int, layer: int, x, n_tokens: int, embed: int, packed,
                                 n_parts: int, ck, cv, stream=None) -> None:
    """Latents of x as n_parts partial sums over ranges of E (blocks of ck, cv)."""
    _check(_lib.lr_attn_project_latent_parts(plan, layer, _ptr(x), n_tokens, embed, _ptr(packed),
                                             n_parts, _ptr(ck), _ptr(cv), _stream(stream)),
           "lr_attn_project_latent_parts")


def lr_attn_project_parts(plan: int, layer: int, n_tokens: int, embed: int) -> int:
    return int(_lib.lr_attn_project_parts(plan, layer, n_tokens, embed))


def lr_attn_project_decode_workspace_bytes(plan: int, max_len: int, embed: int) -> int:
    return int(_lib.lr_attn_project_decode_workspace_bytes(plan, max_len, embed))


def lr_attn_project_append_decode(plan: int, layer: int, cache, x, embed: int, packed, pos, lengths,
                                  max_len: int, q, bk, bv, softmax_scale: float, out, workspace,
                                  ws_bytes: int, stream=None) -> None:
    """Latent generation from x, quantised append and decode: one step of a layer."""
    _check(_lib.lr_attn_project_append_decode(plan, layer, _ptr(cache), _ptr(x), embed, _ptr(packed),
                                              _ptr(pos), _ptr(lengths), max_len, _ptr(q), _ptr(bk),
                                              _ptr(bv), float(softmax_scale), _ptr(out),
                                              _ptr(workspace), ws_bytes, _stream(stream)),
           "lr_attn_project_append_decode")


def lr_attn_hadamard_block(plan: int, layer: int, kv: int, head: int, block: int) -> int:
    return int(_lib.lr_attn_hadamard_block(plan, layer, kv, head, block))


def lr_attn_hadamard_rotate_rows(plan: int, layer: int, kv: int, block: int, rows) -> None:
    """Fold the per-head block-Hadamard rotation into host fp32 rows
    [latent_elems(kv), cols] in place (a numpy array or a CPU torch tensor)."""
    import numpy as np
    if isinstance(rows, np.ndarray):
        if rows.dtype != np.float32 or rows.ndim != 2 or not rows.flags.c_contiguous:
            raise ValueError("rows must be a C-contiguous float32 [latent_elems, cols] array")
        ptr, cols = rows.ctypes.data, rows.shape[1]
    else:
        import torch
        if rows.device.type != "cpu" or rows.dtype != torch.float32 or rows.dim() != 2 \
                or not rows.is_contiguous():
            raise ValueError("rows must be a contiguous CPU float32 [latent_elems, cols] tensor")
        ptr, cols = rows.data_ptr(), rows.shape[1]
    if rows.shape[0] != lr_attn_latent_elems(plan, layer, kv):
        raise ValueError("rows must have latent_elems(kv) rows")
    _check(_lib.lr_attn_hadamard_rotate_rows(plan, layer, kv, block, ptr, cols),
           "lr_attn_hadamard_rotate_rows")


def lr_attn_allocate_ranks(scores, cost_per_rank: int, budget: int):
    """Greedy rank table from component scores (numpy float32 [L, H, 2, max_rank]):
    returns (rank_k, rank_v) as int32 arrays [L, H]."""
    import numpy as np
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if scores.ndim != 4 or scores.shape[2] != 2:
        raise ValueError("scores must be [n_layers, n_heads, 2, max_rank]")
    L, H, _, m = scores.shape
    rk = np.zeros((L, H), dtype=np.int32)
    rv = np.zeros((L, H), dtype=np.int32)
    _check(_lib.lr_attn_allocate_ranks(L, H, m, scores.ctypes.data, int(cost_per_rank), int(budget),
                                       rk.ctypes.data, rv.ctypes.data), "lr_attn_allocate_ranks")
    return rk, rv


def lr_ffn_weight_bytes(desc: lr_ffn_desc) -> int:
    return int(_lib.lr_ffn_weight_bytes(ctypes.byref(desc)))


def lr_ffn_workspace_bytes(desc: lr_ffn_desc, n_tokens: int) -> int:
    return int(_lib.lr_ffn_workspace_bytes(ctypes.byref(desc), n_tokens))


def lr_ffn_prepare_weights(desc: lr_ffn_desc, wg, wu, ag, au, bg, bu, wd):
    """Quantise and pack host fp32 weights (numpy) -> numpy uint8 buffer."""
    import numpy as np
    arrs = []
    for a in (wg, wu, ag, au, bg, bu, wd):
        arrs.append(None if a is None or a.size == 0 else np.ascontiguousarray(a, dtype=np.float32))
    out = np.zeros(lr_ffn_weight_bytes(desc), dtype=np.uint8)
    ptrs = [None if a is None else a.ctypes.data for a in arrs]
    _check(_lib.lr_ffn_prepare_weights(ctypes.byref(desc), *ptrs, out.ctypes.data), "lr_ffn_prepare_weights")
    return out


def lr_ffn_decode(desc: lr_ffn_desc, weights, x, n_tokens: int, y, workspace, ws_bytes: int,
                  stream=None) -> None:
    _check(_lib.lr_ffn_decode(ctypes.byref(desc), _ptr(weights), _ptr(x), n_tokens, _ptr(y),
                              _ptr(workspace), ws_bytes, _stream(stream)), "lr_ffn_decode")


def lr_attn_check_count() -> int:
    """Checked build only: cache accesses found outside their buffer since
    the last call on this device (then reset to 0).  Raises LrAttnError
    (LR_EUNSUPPORTED) in the release library."""
    n = ctypes.c_uint64(0)
    _check(_lib.lr_attn_check_count(ctypes.byref(n)), "lr_attn_check_count")
    return int(n.value)


def lr_attn_check_shrink(nbytes: int) -> None:
    """Checked build only: later launches test cache accesses against each
    cache's bytes less ``nbytes`` (0 restores the full extent)."""
    _check(_lib.lr_attn_check_shrink(nbytes), "lr_attn_check_shrink")


def lr_attn_probe_read(src, nbytes: int, sink, stream=None) -> None:
    """Measurement aid: stream ``nbytes`` of device memory ``src`` with a plain
    read kernel (``sink``: a device int32/uint32 the kernel practically never
    writes)."""
    _check(_lib.lr_attn_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "lr_attn_probe_read")
