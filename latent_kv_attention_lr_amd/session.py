"""Device state of a stack of low-rank latent-KV attention layers.

A ``DecodeSession`` owns, per layer, the quantised latent cache and the B^K /
B^V factor tensors, plus one split workspace and the per-sequence lengths.
torch provides the device allocations and the stream; all computation is in
``liblr_attn.so`` through the binding.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import torch

from . import (LR_DT_BF16, LR_DT_F32, LR_HEAD_DIM, lr_attn_append_decode, lr_attn_append_latent,
               lr_attn_cache_bytes,
               lr_attn_decode, lr_attn_decode_explicit, lr_attn_factor_elems,
               lr_attn_head_layout_get, lr_attn_latent_elems, lr_attn_plan_create,
               lr_attn_pack_projection, lr_attn_packed_projection_elems, lr_attn_plan_destroy,
               lr_attn_project_append, lr_attn_project_append_decode,
               lr_attn_project_decode_workspace_bytes, lr_attn_project_latent,
               lr_attn_project_workspace_bytes, lr_attn_workspace_bytes)


class DecodeSession:
    def __init__(self, n_layers: int, batch: int, n_heads: int, capacity: int, qfmt: int,
                 io_dtype: int, ranks_k: Sequence[Sequence[int]], ranks_v: Sequence[Sequence[int]],
                 device="cuda", max_splits: int = 0, wg_waves: int = 0):
        self.n_layers, self.batch, self.n_heads, self.capacity = n_layers, batch, n_heads, capacity
        self.qfmt, self.io_dtype = qfmt, io_dtype
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:   # "cuda" means the current device
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.ranks_k = [list(r) for r in ranks_k]
        self.ranks_v = [list(r) for r in ranks_v]
        flat_k = [r for row in self.ranks_k for r in row]
        flat_v = [r for row in self.ranks_v for r in row]
        self.plan = lr_attn_plan_create(n_layers, batch, n_heads, capacity, qfmt, io_dtype,
                                        flat_k, flat_v, max_splits=max_splits, wg_waves=wg_waves)
        self.torch_dtype = torch.bfloat16 if io_dtype == LR_DT_BF16 else torch.float32
        self.caches: List[torch.Tensor] = [
            torch.zeros(lr_attn_cache_bytes(self.plan, l), dtype=torch.uint8, device=self.device)
            for l in range(n_layers)]
        self.bk: List[Optional[torch.Tensor]] = [None] * n_layers
        self.bv: List[Optional[torch.Tensor]] = [None] * n_layers
        self.ws_bytes = lr_attn_workspace_bytes(self.plan, capacity)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.lengths = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self._proj_ws: Optional[torch.Tensor] = None   # latents of project_append, grown on demand
        self._step_ws: Optional[torch.Tensor] = None   # workspace of project_append_decode
        self.proj: List[Optional[tuple]] = [None] * n_layers   # (embed, packed factors) per layer

    def close(self) -> None:
        plan = getattr(self, "plan", None)
        if plan:
            lr_attn_plan_destroy(plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: module globals may be gone
            pass

    # -- layout -------------------------------------------------------------
    def latent_elems(self, layer: int, kv: int) -> int:
        return lr_attn_latent_elems(self.plan, layer, kv)

    def factor_elems(self, layer: int, kv: int) -> int:
        return lr_attn_factor_elems(self.plan, layer, kv)

    def head_layout(self, layer: int, head: int) -> dict:
        return lr_attn_head_layout_get(self.plan, layer, head)

    # -- state --------------------------------------------------------------
    def set_factors(self, layer: int, bk: torch.Tensor, bv: torch.Tensor) -> None:
        for t, kv in ((bk, 0), (bv, 1)):
            if t.numel() != self.factor_elems(layer, kv) or t.dtype != self.torch_dtype:
                raise ValueError("factor tensor has the wrong size or dtype")
            if t.device != self.device or not t.is_contiguous():
                raise ValueError("factor tensor must be contiguous on the session device")
        self.bk[layer] = bk
        self.bv[layer] = bv

    def append(self, layer: int, ck: torch.Tensor, cv: torch.Tensor, pos: torch.Tensor,
               stream=None) -> None:
        """Quantise and write fp32 latents ck/cv [B, n_new, latent_elems] at pos[b].."""
        n_new = ck.shape[1]
        if ck.dtype != torch.float32 or cv.dtype != torch.float32:
            raise ValueError("latents must be fp32")
        if ck.shape != (self.batch, n_new, self.latent_elems(layer, 0)) or \
                cv.shape != (self.batch, n_new, self.latent_elems(layer, 1)):
            raise ValueError("latent tensors have the wrong shape")
        if not (ck.is_contiguous() and cv.is_contiguous()) or ck.device != self.device or cv.device != self.device:
            raise ValueError("latent tensors must be contiguous on the session device")
        self._check_pos(pos)
        lr_attn_append_latent(self.plan, layer, self.caches[layer], ck, cv, pos, n_new, stream)

    def decode(self, layer: int, q: torch.Tensor, out: torch.Tensor, max_len: int,
               lengths: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
               explicit: bool = False, stream=None) -> None:
        """out[b, h] = attention of q[b, h] over the first lengths[b] cached tokens."""
        if self.bk[layer] is None:
            raise ValueError("factors of this layer are not set")
        shape = (self.batch, self.n_heads, LR_HEAD_DIM)
        if q.shape != shape or out.shape != shape or q.dtype != self.torch_dtype or out.dtype != self.torch_dtype:
            raise ValueError("q/out must be [B, H, 128] of the session dtype")
        if not (q.is_contiguous() and out.is_contiguous()):
            raise ValueError("q and out must be contiguous")
        scale = 1.0 / math.sqrt(LR_HEAD_DIM) if softmax_scale is None else softmax_scale
        fn = lr_attn_decode_explicit if explicit else lr_attn_decode
        fn(self.plan, layer, self.caches[layer], self.lengths if lengths is None else lengths,
           max_len, q, self.bk[layer], self.bv[layer], scale, out, self.workspace,
           self.workspace.numel(), stream)

    def append_decode(self, layer: int, ck: torch.Tensor, cv: torch.Tensor, pos: torch.Tensor,
                      q: torch.Tensor, out: torch.Tensor, max_len: int,
                      lengths: Optional[torch.Tensor] = None,
                      softmax_scale: Optional[float] = None, stream=None) -> None:
        """append() of one token per sequence, then decode(), in one fused call."""
        if self.bk[layer] is None:
            raise ValueError("factors of this layer are not set")
        if ck.dtype != torch.float32 or cv.dtype != torch.float32:
            raise ValueError("latents must be fp32")
        if ck.numel() != self.batch * self.latent_elems(layer, 0) or \
                cv.numel() != self.batch * self.latent_elems(layer, 1):
            raise ValueError("latent tensors must hold one token per sequence")
        shape = (self.batch, self.n_heads, LR_HEAD_DIM)
        if q.shape != shape or out.shape != shape or q.dtype != self.torch_dtype or out.dtype != self.torch_dtype:
            raise ValueError("q/out must be [B, H, 128] of the session dtype")
        if not all(t.is_contiguous() for t in (ck, cv, pos, q, out)):
            raise ValueError("all tensors must be contiguous")
        scale = 1.0 / math.sqrt(LR_HEAD_DIM) if softmax_scale is None else softmax_scale
        lr_attn_append_decode(self.plan, layer, self.caches[layer], ck, cv, pos,
                              self.lengths if lengths is None else lengths, max_len, q,
                              self.bk[layer], self.bv[layer], scale, out, self.workspace,
                              self.workspace.numel(), stream)

    # -- latent generation ---------------------------------------------------
    def set_projection(self, layer: int, wk: torch.Tensor, wv: torch.Tensor) -> None:
        """Pack the down-projection factors of a layer, given as wk/wv
        [latent_elems, embed] bf16 (A transposed), into a session-owned buffer."""
        if wk.dim() != 2 or wv.dim() != 2 or wk.shape[1] != wv.shape[1]:
            raise ValueError("factors must be [latent_elems, embed] with one embed")
        E = wk.shape[1]
        if wk.dtype != torch.bfloat16 or wv.dtype != torch.bfloat16:
            raise ValueError("factors must be bf16")
        if wk.shape[0] != self.latent_elems(layer, 0) or wv.shape[0] != self.latent_elems(layer, 1):
            raise ValueError("factors must be [latent_elems, embed] (A transposed)")
        if not all(t.is_contiguous() and t.device == self.device for t in (wk, wv)):
            raise ValueError("factors must be contiguous on the session device")
        packed = torch.empty(lr_attn_packed_projection_elems(self.plan, layer, E), dtype=torch.bfloat16,
                             device=self.device)
        lr_attn_pack_projection(self.plan, layer, E, wk, wv, packed)
        self.proj[layer] = (E, packed)

    def _check_pos(self, pos: torch.Tensor) -> None:
        """pos: the first slot of every sequence, int32 [batch] on the device."""
        if pos.dtype != torch.int32 or pos.numel() != self.batch or not pos.is_contiguous() \
                or pos.device != self.device:
            raise ValueError(f"pos must be contiguous int32 [{self.batch}] on the session device")

    def _projection_input(self, layer: int, x: torch.Tensor) -> int:
        if self.proj[layer] is None:
            raise ValueError("projection factors of this layer are not set")
        E = self.proj[layer][0]
        if x.dtype != torch.bfloat16 or x.shape[-1] != E:
            raise ValueError("x must be bf16 with the embed of the packed factors")
        if not (x.is_contiguous() and x.device == self.device):
            raise ValueError("x must be contiguous on the session device")
        return E

    def project(self, layer: int, x: torch.Tensor, ck: Optional[torch.Tensor] = None,
                cv: Optional[torch.Tensor] = None, stream=None):
        """fp32 latents of x [..., embed]: (x A^K, x A^V); returns (ck, cv)
        shaped [..., latent_elems]."""
        E = self._projection_input(layer, x)
        lead = tuple(x.shape[:-1])
        n = x.numel() // E
        if ck is None:
            ck = torch.empty(lead + (self.latent_elems(layer, 0),), dtype=torch.float32, device=self.device)
        if cv is None:
            cv = torch.empty(lead + (self.latent_elems(layer, 1),), dtype=torch.float32, device=self.device)
        if ck.numel() != n * self.latent_elems(layer, 0) or cv.numel() != n * self.latent_elems(layer, 1) \
                or ck.dtype != torch.float32 or cv.dtype != torch.float32 \
                or not (ck.is_contiguous() and cv.is_contiguous()):
            raise ValueError("ck/cv must be contiguous fp32 with one latent vector per row of x")
        lr_attn_project_latent(self.plan, layer, x, n, E, self.proj[layer][1], ck, cv, stream)
        return ck, cv

    def project_append(self, layer: int, x: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
        """Generate the latents of x [B, n_new, embed] and append them at pos[b].."""
        E = self._projection_input(layer, x)
        if x.dim() != 3 or x.shape[0] != self.batch:
            raise ValueError("x must be [batch, n_new, embed]")
        self._check_pos(pos)
        n_new = x.shape[1]
        need = lr_attn_project_workspace_bytes(self.plan, n_new) if n_new > 0 else 0
        if need > 0 and (self._proj_ws is None or self._proj_ws.numel() < need):
            self._proj_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = self._proj_ws
        lr_attn_project_append(self.plan, layer, self.caches[layer], x, E, self.proj[layer][1], pos,
                               n_new, ws, 0 if ws is None else ws.numel(), stream)

    def project_append_decode(self, layer: int, x: torch.Tensor, pos: torch.Tensor, q: torch.Tensor,
                              out: torch.Tensor, max_len: int, lengths: Optional[torch.Tensor] = None,
                              softmax_scale: Optional[float] = None, stream=None) -> None:
        """One decode step from activations x [batch, embed]: generate the new
        token's latents, append them at pos[b] and attend (two launches)."""
        E = self._projection_input(layer, x)
        if x.numel() != self.batch * E:
            raise ValueError("x must hold one token per sequence: [batch, embed]")
        self._check_pos(pos)
        if self.bk[layer] is None:
            raise ValueError("factors of this layer are not set")
        shape = (self.batch, self.n_heads, LR_HEAD_DIM)
        if q.shape != shape or out.shape != shape or q.dtype != self.torch_dtype or out.dtype != self.torch_dtype:
            raise ValueError("q/out must be [B, H, 128] of the session dtype")
        if not (q.is_contiguous() and out.is_contiguous()):
            raise ValueError("q and out must be contiguous")
        need = lr_attn_project_decode_workspace_bytes(self.plan, self.capacity, E)
        if self._step_ws is None or self._step_ws.numel() < need:
            self._step_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = self._step_ws
        scale = 1.0 / math.sqrt(LR_HEAD_DIM) if softmax_scale is None else softmax_scale
        lr_attn_project_append_decode(self.plan, layer, self.caches[layer], x, E, self.proj[layer][1],
                                      pos, self.lengths if lengths is None else lengths, max_len, q,
                                      self.bk[layer], self.bv[layer], scale, out, ws, ws.numel(), stream)
