"""Set up a synthetic decode workload on the GPU (tests, benchmark, smoke check).

It draws the workload's inputs with ``lrgen`` (activations, factors, queries),
makes the fp32 latents with a plain fp32 projection on the device, and drives
the library through ``DecodeSession``: prefill of the context, then decode
steps that append one token per sequence and attend.  The fp32 latents of
chosen (layer, b, h) units are copied to the host so the CPU oracle can be
fed exactly the same inputs.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np
import torch

import lrgen
from latent_kv_attention_lr_amd import LR_DT_BF16, LR_DT_F32
from latent_kv_attention_lr_amd.session import DecodeSession

Unit = Tuple[int, int, int]  # (layer, b, h)


class WorkloadRun:
    def __init__(self, w: lrgen.Workload, io_dtype: int = LR_DT_BF16, device="cuda",
                 keep: Iterable[Unit] = (), max_splits: int = 0, steps: Optional[int] = None,
                 context: Optional[int] = None, chunk_tokens: int = 1024, wg_waves: int = 0):
        self.w = w
        self.io_dtype = io_dtype
        self.device = torch.device(device)
        self.steps = w.steps if steps is None else steps
        self.context = w.context if context is None else context
        self.capacity = self.context + self.steps
        self.chunk = chunk_tokens
        self.dtype = torch.bfloat16 if io_dtype == LR_DT_BF16 else torch.float32
        self.sess = DecodeSession(w.n_layers, w.batch, w.n_heads, self.capacity, w.qfmt, io_dtype,
                                  w.ranks_k, w.ranks_v, device=self.device, max_splits=max_splits,
                                  wg_waves=wg_waves)
        self.keep = sorted(set(keep))
        self.kept: Dict[Unit, List[List[np.ndarray]]] = {u: [[], []] for u in self.keep}
        self.off_k = [lrgen.head_offsets(r) for r in w.ranks_k]
        self.off_v = [lrgen.head_offsets(r) for r in w.ranks_v]
        self.step_ck: List[Optional[torch.Tensor]] = [None] * w.n_layers
        self.step_cv: List[Optional[torch.Tensor]] = [None] * w.n_layers
        self.step_q: List[Optional[torch.Tensor]] = [None] * w.n_layers
        self.scale = 1.0 / math.sqrt(w.head_dim)

    # -- inputs ---------------------------------------------------------------
    def _latents_all_rows(self, layer: int, t0: int, t1: int, ak, av):
        # every batch row's activations in one draw, one fp32 product for K and one for V
        x = lrgen.activations_rows(self.w, layer, 0, self.w.batch, t0, t1, device=self.device)
        return torch.matmul(x, ak).contiguous(), torch.matmul(x, av).contiguous()

    def _keep(self, layer: int, ck: torch.Tensor, cv: torch.Tensor) -> None:
        units = [u for u in self.keep if u[0] == layer]
        if not units:
            return
        rows = sorted({b for (_, b, _) in units})
        # one copy per kept batch row of the chunk, sliced per head on the host
        hk = {b: ck[b].cpu().numpy() for b in rows}
        hv = {b: cv[b].cpu().numpy() for b in rows}
        for (l, b, h) in units:
            rk, rv = self.w.ranks_k[l][h], self.w.ranks_v[l][h]
            ok, ov = self.off_k[l][h], self.off_v[l][h]
            self.kept[(l, b, h)][0].append(hk[b][:, ok:ok + rk])
            self.kept[(l, b, h)][1].append(hv[b][:, ov:ov + rv])

    def setup(self) -> "WorkloadRun":
        """Factors, prefill of the context, and the inputs of every decode step."""
        w, dev = self.w, self.device
        for l in range(w.n_layers):
            ak = lrgen.down_factors(w, l, 0, device=dev)
            av = lrgen.down_factors(w, l, 1, device=dev)
            bk = lrgen.up_factors(w, l, 0, dtype=self.dtype, device=dev).contiguous()
            bv = lrgen.up_factors(w, l, 1, dtype=self.dtype, device=dev).contiguous()
            self.sess.set_factors(l, bk, bv)
            for t0 in range(0, self.context, self.chunk):
                t1 = min(self.context, t0 + self.chunk)
                ck, cv = self._latents_all_rows(l, t0, t1, ak, av)
                pos = torch.full((w.batch,), t0, dtype=torch.int32, device=dev)
                self.sess.append(l, ck, cv, pos)
                self._keep(l, ck, cv)
            if self.steps > 0:
                ck, cv = self._latents_all_rows(l, self.context, self.context + self.steps, ak, av)
                self.step_ck[l], self.step_cv[l] = ck, cv
                self._keep(l, ck, cv)
                self.step_q[l] = torch.stack([
                    lrgen.queries(w, l, s, dtype=self.dtype, device=dev) for s in range(self.steps)])
            del ak, av
        torch.cuda.synchronize()
        self.sess.lengths.fill_(self.context)
        return self

    # -- steps ----------------------------------------------------------------
    def step_tensors(self, layer: int, s: int):
        """Contiguous per-step inputs: ck, cv [B, 1, Σr]; q [B, H, d]; pos [B]."""
        ck = self.step_ck[layer][:, s:s + 1].contiguous()
        cv = self.step_cv[layer][:, s:s + 1].contiguous()
        q = self.step_q[layer][s].contiguous()
        pos = torch.full((self.w.batch,), self.context + s, dtype=torch.int32, device=self.device)
        return ck, cv, q, pos

    def run_step(self, layer: int, s: int, out: Optional[torch.Tensor] = None,
                 explicit: bool = False, fused: bool = True) -> torch.Tensor:
        """Append step s's token to every sequence, then attend over context + s + 1
        (one fused call unless explicit or fused=False)."""
        ck, cv, q, pos = self.step_tensors(layer, s)
        self.sess.lengths.fill_(self.context + s + 1)
        if out is None:
            out = torch.empty(self.w.batch, self.w.n_heads, self.w.head_dim, dtype=self.dtype,
                              device=self.device)
        if fused and not explicit:
            self.sess.append_decode(layer, ck.view(self.w.batch, -1), cv.view(self.w.batch, -1),
                                    pos, q, out, self.context + s + 1)
        else:
            self.sess.append(layer, ck, cv, pos)
            self.sess.decode(layer, q, out, self.context + s + 1, explicit=explicit)
        return out

    # -- oracle inputs ----------------------------------------------------------
    def unit_inputs(self, unit: Unit, s: int):
        """Exactly the fp32 latents, q and factors the GPU saw for ``unit`` at step s
        (T = context + s + 1 tokens), widened to fp64 where the oracle wants it."""
        l, b, h = unit
        ks, vs = self.kept[unit]
        T = self.context + s + 1
        ck = np.concatenate(ks, axis=0)[:T]
        cv = np.concatenate(vs, axis=0)[:T]
        rk, rv = self.w.ranks_k[l][h], self.w.ranks_v[l][h]
        ok, ov = self.off_k[l][h], self.off_v[l][h]
        q = self.step_q[l][s][b, h].double().cpu().numpy()
        bk = self.sess.bk[l][ok:ok + rk].double().cpu().numpy()
        bv = self.sess.bv[l][ov:ov + rv].double().cpu().numpy()
        return ck, cv, q, bk, bv


def sample_units(w: lrgen.Workload, n: int, seed: int, layers: Optional[List[int]] = None) -> List[Unit]:
    """A seeded sample of (layer, b, h) units that includes every head of one batch row."""
    rng = np.random.default_rng(seed)
    layers = list(range(w.n_layers)) if layers is None else layers
    units = set()
    b0 = int(rng.integers(w.batch))
    l0 = layers[int(rng.integers(len(layers)))]
    for h in range(w.n_heads):
        units.add((l0, b0, h))
    while len(units) < w.n_heads + n:
        units.add((layers[int(rng.integers(len(layers)))], int(rng.integers(w.batch)),
                   int(rng.integers(w.n_heads))))
    return sorted(units)
