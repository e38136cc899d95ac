"""Device state of one hybrid low-rank / dense W8A8 FFN layer: the packed
int8 weights and a workspace, held in torch allocations; all computation is
in liblr_attn.so (lr_ffn_prepare_weights on the host, lr_ffn_decode on the
GPU)."""
from __future__ import annotations

import torch

from . import (lr_ffn_decode, lr_ffn_desc, lr_ffn_prepare_weights, lr_ffn_weight_bytes,
               lr_ffn_workspace_bytes)


class FfnLayer:
    def __init__(self, embed: int, hidden: int, n_lowrank: int, rank: int, device="cuda"):
        self.desc = lr_ffn_desc(embed, hidden, n_lowrank, rank, 0)
        if lr_ffn_weight_bytes(self.desc) == 0:
            raise ValueError("unsupported FFN shape")
        self.E, self.F, self.S, self.r = embed, hidden, n_lowrank, rank
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:   # "cuda" means the current device
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.weights = None
        self.workspace = torch.empty(256, dtype=torch.uint8, device=self.device)

    def set_weights(self, wg, wu, ag, au, bg, bu, wd) -> None:
        """fp32 host arrays (numpy): wg, wu [F-S, E]; ag, au [r, E]; bg, bu [S, r]; wd [E, F]."""
        packed = lr_ffn_prepare_weights(self.desc, wg, wu, ag, au, bg, bu, wd)
        self.weights = torch.from_numpy(packed).to(self.device)

    def __call__(self, x: torch.Tensor, y: torch.Tensor = None, stream=None) -> torch.Tensor:
        """y [T, E] fp32 = FFN(x [T, E] bf16), launched on `stream` (default:
        torch's current stream).  The layer's one workspace is reused by every
        call, so calls on different streams must not overlap."""
        if self.weights is None:
            raise ValueError("weights are not set")
        if (x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.E or not x.is_contiguous()
                or x.device != self.device):
            raise ValueError(f"x must be contiguous bf16 [T, {self.E}] on {self.device}")
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, self.E, dtype=torch.float32, device=self.device)
        elif (y.dtype != torch.float32 or tuple(y.shape) != (T, self.E) or not y.is_contiguous()
              or y.device != self.device):
            raise ValueError(f"y must be contiguous fp32 [{T}, {self.E}] on {self.device}")
        need = lr_ffn_workspace_bytes(self.desc, T) if T > 0 else 0
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        lr_ffn_decode(self.desc, self.weights, x, T, y, self.workspace, self.workspace.numel(), stream)
        return y
