"""Seeded synthetic inputs for the low-rank latent-KV decode step.

This module draws every random tensor that the GPU path and the CPU oracle
consume, and nothing else: it holds none of the method's arithmetic (no
quantisation, no reconstruction, no attention).  Both sides are always fed
the very same tensors produced here.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used as a counter-based
generator: draw ``i`` of a stream with 64-bit key ``k`` is ``mix64(k + (i+1)·γ)``
with γ = 0x9E3779B97F4A7C15, which is exactly the i-th output of a SplitMix64
generator seeded with ``k``.  Normals use the Box–Muller transform in fp64
(Box and Muller, 1958) on two consecutive draws, then rounding to fp32.
Everything is written with torch int64/float64 elementwise ops so the same
code runs on the CPU and on the GPU; int64 multiplication wraps modulo 2**64
and the right shifts are made logical with a mask.

The workload table (``WORKLOADS``) describes the five decode workloads: the
shapes of LLaMA-7B-class attention layers as used by the WSVD and LASER
vision-language-model decode experiments (image-prefix plus text contexts),
with per-head rank-r factors ``W_h ≈ A_h B_h`` and latents ``c = x A_h``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
_U64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Two's-complement int64 view of an unsigned 64-bit constant."""
    v &= _U64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for the tensor version)."""
    z &= _U64
    z = ((z ^ (z >> 30)) * MIX1) & _U64
    z = ((z ^ (z >> 27)) * MIX2) & _U64
    return z ^ (z >> 31)


def _lshr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output function on an int64 tensor (bit pattern = uint64)."""
    z = (z ^ _lshr(z, 30)) * _s64(MIX1)
    z = (z ^ _lshr(z, 27)) * _s64(MIX2)
    return z ^ _lshr(z, 31)


def stream_key(seed: int, *ids: int) -> int:
    """64-bit key of the stream named by ``(seed, *ids)``."""
    k = mix64_int(seed + GAMMA)
    for v in ids:
        k = mix64_int(k + ((v + 1) * GAMMA))
    return k


def raw_draws(key: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Draws ``start .. start+count-1`` of stream ``key`` as int64 bit patterns."""
    i = torch.arange(start + 1, start + 1 + count, dtype=torch.int64, device=device)
    return mix64(i * _s64(GAMMA) + _s64(key))


def uniform53(z: torch.Tensor) -> torch.Tensor:
    """Top 53 bits of a draw as a float64 in [0, 1)."""
    return _lshr(z, 11).to(torch.float64) * (2.0 ** -53)


_CHUNK = 1 << 24


def normal(key: int, start: int, count: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """Elements ``start .. start+count-1`` of a N(0, std²) stream, as fp32.

    Element ``i`` uses draws ``2i`` and ``2i+1``:  sqrt(-2 ln U1) cos(2π U2)
    with U1 in (0, 1] and U2 in [0, 1), evaluated in fp64, times ``std``,
    rounded once to fp32.
    """
    out = torch.empty(count, dtype=torch.float32, device=device)
    done = 0
    while done < count:
        n = min(_CHUNK, count - done)
        z = raw_draws(key, 2 * (start + done), 2 * n, device).view(n, 2)
        u1 = 1.0 - uniform53(z[:, 0])
        u2 = uniform53(z[:, 1])
        g = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
        out[done:done + n] = (g * std).to(torch.float32)
        done += n
    return out


def normal_keyed(keys: torch.Tensor, idx: torch.Tensor, std) -> torch.Tensor:
    """Element-wise streams: element ``e`` is element ``idx[e]`` of the
    N(0, std²) stream with key ``keys[e]`` -- exactly the value ``normal()``
    gives for that stream and index -- as fp32.  ``keys`` (int64 bit
    patterns), ``idx`` and ``std`` (a float or a float64 tensor) broadcast to
    one shape; one pass of element-wise kernels draws the whole tensor."""
    keys, idx = torch.broadcast_tensors(keys, idx)
    if isinstance(std, torch.Tensor):
        std = std.to(torch.float64).expand(keys.shape).reshape(-1)
    shape = keys.shape
    k = keys.reshape(-1)
    i = idx.reshape(-1)
    out = torch.empty(k.numel(), dtype=torch.float32, device=k.device)
    step = _CHUNK
    for lo in range(0, k.numel(), step):
        hi = min(k.numel(), lo + step)
        kk, ii = k[lo:hi], i[lo:hi]
        z0 = mix64((2 * ii + 1) * _s64(GAMMA) + kk)     # draw 2i of the stream
        z1 = mix64((2 * ii + 2) * _s64(GAMMA) + kk)     # draw 2i + 1
        u1 = 1.0 - uniform53(z0)
        u2 = uniform53(z1)
        g = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
        out[lo:hi] = (g * (std[lo:hi] if isinstance(std, torch.Tensor) else std)).to(torch.float32)
    return out.view(shape)


def uniform_index(key: int, start: int, count: int, n: int) -> List[int]:
    """``count`` integers uniform on ``{0, .., n-1}``: floor(U53 · n)."""
    u = uniform53(raw_draws(key, start, count))
    return [int(math.floor(float(v) * n)) for v in u]


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

TAG_X, TAG_AK, TAG_AV, TAG_BK, TAG_BV, TAG_Q, TAG_OUTLIER, TAG_RANK = range(1, 9)

QFMT_INT8 = 0   # symmetric int8, one fp32 scale per (token, head)
QFMT_INT4 = 1   # symmetric int4, one fp16 scale per group of 32 ranks


@dataclass
class Workload:
    """One synthetic decode workload (shapes, distributions, seed)."""
    name: str
    index: int
    n_layers: int
    batch: int
    n_heads: int
    head_dim: int
    embed: int
    qfmt: int
    context: int          # tokens cached before the first decode step
    prefix: int           # leading image-prefix tokens (x ~ N(0, prefix_var))
    prefix_var: float
    text_var: float
    steps: int
    n_outliers: int = 0   # x channels with std multiplied by outlier_scale
    outlier_scale: float = 20.0
    uniform_rank: Optional[int] = None   # rank of every head (K and V), or None = drawn
    rank_choices: Tuple[int, ...] = ()
    seed: int = 0
    ranks_k: List[List[int]] = field(default_factory=list)
    ranks_v: List[List[int]] = field(default_factory=list)

    def __post_init__(self):
        self.seed = 0x5EED0000 + self.index
        if self.uniform_rank is not None:
            self.ranks_k = [[self.uniform_rank] * self.n_heads for _ in range(self.n_layers)]
            self.ranks_v = [[self.uniform_rank] * self.n_heads for _ in range(self.n_layers)]
        else:
            m = self.n_layers * self.n_heads
            key = stream_key(self.seed, TAG_RANK)
            idx = uniform_index(key, 0, 2 * m, len(self.rank_choices))
            flat_k = [self.rank_choices[i] for i in idx[:m]]
            flat_v = [self.rank_choices[i] for i in idx[m:]]
            H = self.n_heads
            self.ranks_k = [flat_k[l * H:(l + 1) * H] for l in range(self.n_layers)]
            self.ranks_v = [flat_v[l * H:(l + 1) * H] for l in range(self.n_layers)]

    @property
    def capacity(self) -> int:
        return self.context + self.steps

    def x_std(self, t: int) -> float:
        return math.sqrt(self.prefix_var if t < self.prefix else self.text_var)


def _mk() -> List[Workload]:
    return [
        Workload("single-layer-b1-h8-r32-int8-ctx512", 0, n_layers=1, batch=1, n_heads=8,
                 head_dim=128, embed=1024, qfmt=QFMT_INT8, context=512, prefix=0,
                 prefix_var=1.0, text_var=1.0, steps=1, uniform_rank=32),
        Workload("llama7b-layer-b16-r32-int8-ctx4096", 1, n_layers=1, batch=16, n_heads=32,
                 head_dim=128, embed=4096, qfmt=QFMT_INT8, context=4096, prefix=576,
                 prefix_var=1.5, text_var=1.0, steps=128, uniform_rank=32),
        Workload("llama7b-layer-b64-r64-int4g32-ctx8192-outliers", 2, n_layers=1, batch=64,
                 n_heads=32, head_dim=128, embed=4096, qfmt=QFMT_INT4, context=8192, prefix=576,
                 prefix_var=1.5, text_var=1.0, steps=128, n_outliers=4, uniform_rank=64),
        Workload("laser-32layer-b32-rank8to96-int8-ctx2048", 3, n_layers=32, batch=32,
                 n_heads=32, head_dim=128, embed=4096, qfmt=QFMT_INT8, context=2048, prefix=576,
                 prefix_var=1.5, text_var=1.0, steps=1,
                 rank_choices=tuple(range(8, 97, 8))),
        Workload("long-context-b8-r48-int4g32-ctx32768", 4, n_layers=1, batch=8, n_heads=32,
                 head_dim=128, embed=4096, qfmt=QFMT_INT4, context=32768, prefix=2304,
                 prefix_var=1.5, text_var=1.0, steps=64, uniform_rank=48),
    ]


WORKLOADS: List[Workload] = _mk()


def workload(i: int) -> Workload:
    return _mk()[i]


# ---------------------------------------------------------------------------
# Tensors of a workload
# ---------------------------------------------------------------------------

def outlier_channels(w: Workload, layer: int) -> List[int]:
    """Distinct x channels whose std is scaled by ``outlier_scale`` (fixed per layer)."""
    if w.n_outliers == 0:
        return []
    key = stream_key(w.seed, TAG_OUTLIER, layer)
    chosen: List[int] = []
    i = 0
    while len(chosen) < w.n_outliers:
        c = uniform_index(key, i, 1, w.embed)[0]
        i += 1
        if c not in chosen:
            chosen.append(c)
    return chosen


def activations(w: Workload, layer: int, b: int, t0: int, t1: int, device="cpu") -> torch.Tensor:
    """x[t0:t1] of batch row ``b`` at ``layer``: fp32 [t1-t0, E].

    Tokens ``t < prefix`` are image-prefix tokens with variance ``prefix_var``,
    the rest (including decode-step tokens) have ``text_var``.  Outlier
    channels have their std multiplied by ``outlier_scale`` for every token.
    """
    E = w.embed
    key = stream_key(w.seed, TAG_X, layer, b)
    x = normal(key, t0 * E, (t1 - t0) * E, 1.0, device).view(t1 - t0, E)
    scale = torch.full((t1 - t0, 1), math.sqrt(w.text_var), dtype=torch.float32, device=device)
    npre = max(0, min(t1, w.prefix) - t0)
    if npre > 0:
        scale[:npre] = math.sqrt(w.prefix_var)
    x = x * scale
    oc = outlier_channels(w, layer)
    if oc:
        x[:, oc] *= w.outlier_scale
    return x


def _head_blocks(w: Workload, layer: int, kv: int, tag: int, device):
    """Per latent column c of a layer's K or V latents: its head's stream key,
    the column's index within the head, and the head's rank (int64 [Σ_h r_h])."""
    ranks = w.ranks_k[layer] if kv == 0 else w.ranks_v[layer]
    keys, local, rank = [], [], []
    for h, r in enumerate(ranks):
        keys += [_s64(stream_key(w.seed, tag, layer, h))] * r
        local += list(range(r))
        rank += [r] * r
    as_t = lambda v: torch.tensor(v, dtype=torch.int64, device=device)
    return as_t(keys), as_t(local), as_t(rank)


def activations_rows(w: Workload, layer: int, b0: int, b1: int, t0: int, t1: int,
                     device="cpu") -> torch.Tensor:
    """activations() of batch rows b0 .. b1-1 at once: fp32 [b1-b0, t1-t0, E],
    the same values as the rows drawn one by one."""
    E = w.embed
    keys = torch.tensor([_s64(stream_key(w.seed, TAG_X, layer, b)) for b in range(b0, b1)],
                        dtype=torch.int64, device=device)[:, None, None]
    t = torch.arange(t0, t1, dtype=torch.int64, device=device)[None, :, None]
    e = torch.arange(E, dtype=torch.int64, device=device)[None, None, :]
    x = normal_keyed(keys, t * E + e, 1.0)
    scale = torch.full((1, t1 - t0, 1), math.sqrt(w.text_var), dtype=torch.float32, device=device)
    npre = max(0, min(t1, w.prefix) - t0)
    if npre > 0:
        scale[:, :npre] = math.sqrt(w.prefix_var)
    x = x * scale
    oc = outlier_channels(w, layer)
    if oc:
        x[:, :, oc] *= w.outlier_scale
    return x


def down_factors(w: Workload, layer: int, kv: int, device="cpu") -> torch.Tensor:
    """A for K (kv=0) or V (kv=1): fp32 [E, Σ_h r_h], head h in its own column block,
    each A_h ~ N(0, 1/E) elementwise (block h is stream (seed, A, layer, h) in
    row-major order: element (e, j) is stream element e r_h + j)."""
    keys, local, rank = _head_blocks(w, layer, kv, TAG_AK if kv == 0 else TAG_AV, device)
    e = torch.arange(w.embed, dtype=torch.int64, device=device)[:, None]
    return normal_keyed(keys[None, :], e * rank[None, :] + local[None, :], 1.0 / math.sqrt(w.embed))


def up_factors(w: Workload, layer: int, kv: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """B for K or V: [Σ_h r_h, d] with head h's r_h×d block B_h ~ N(0, 1/r_h),
    drawn in fp32 and rounded to ``dtype`` (block h is stream (seed, B, layer,
    h) in row-major order)."""
    keys, local, rank = _head_blocks(w, layer, kv, TAG_BK if kv == 0 else TAG_BV, device)
    d = torch.arange(w.head_dim, dtype=torch.int64, device=device)[None, :]
    std = torch.tensor([1.0 / math.sqrt(int(r)) for r in rank.tolist()], dtype=torch.float64,
                       device=device)[:, None]
    return normal_keyed(keys[:, None], local[:, None] * w.head_dim + d, std).to(dtype)


def svd_like_factors(w: Workload, layer: int, kv: int, alpha: float = 1.0,
                     device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Factors shaped like a truncated SVD, A_h = G_h diag(sqrt(s)), B_h =
    diag(sqrt(s)) G'_h, with G, G' the workload's own draws (down_factors,
    fp32 up_factors) and singular values s_j proportional to (j + 1)^-alpha,
    normalised to mean 1 per head.  Returns (A [E, sum r] fp32, B [sum r, d] fp32).
    alpha = 0 gives the workload's iid factors."""
    ranks = w.ranks_k[layer] if kv == 0 else w.ranks_v[layer]
    a = down_factors(w, layer, kv, device)
    b = up_factors(w, layer, kv, dtype=torch.float32, device=device)
    scale = []
    for r in ranks:
        s = torch.arange(1, r + 1, dtype=torch.float64) ** (-alpha)
        scale.append(torch.sqrt(s / s.mean()))
    sc = torch.cat(scale).to(torch.float32).to(device)
    return a * sc[None, :], b * sc[:, None]


TAG_SCORE = 9


def component_scores(seed: int, n_layers: int, n_heads: int, max_rank: int = 128) -> torch.Tensor:
    """Synthetic importance scores standing in for empirical-Fisher ones:
    fp32 [n_layers, n_heads, 2 (K, V), max_rank], component j of a head scored
    g_l * a_h * (j + 1)^(-2 b_h) * n_j -- a per-layer sensitivity g_l and a
    per-head gain a_h (both exp(N(0, 0.5^2))), a per-head spectral decay b_h
    uniform in [0.3, 1.2] (squared singular values), and a per-component
    factor n_j = exp(N(0, 0.2^2)) so that scores are only roughly monotone."""
    key = stream_key(seed, TAG_SCORE)
    L, H, m = n_layers, n_heads, max_rank
    g = torch.exp(0.5 * normal(key, 0, L).double()).view(L, 1, 1, 1)
    a = torch.exp(0.5 * normal(key, L, L * H * 2).double()).view(L, H, 2, 1)
    u = uniform53(raw_draws(key, 10 ** 9, L * H * 2)).view(L, H, 2, 1)
    b = 0.3 + 0.9 * u
    j = torch.arange(1, m + 1, dtype=torch.float64).view(1, 1, 1, m)
    n = torch.exp(0.2 * normal(key, L + L * H * 2, L * H * 2 * m).double()).view(L, H, 2, m)
    return (g * a * j ** (-2.0 * b) * n).to(torch.float32)


TAG_FFN = 10


@dataclass
class FfnWorkload:
    """One synthetic hybrid-FFN decode workload: LLaMA-7B FFN shape."""
    name: str
    embed: int
    hidden: int
    n_lowrank: int
    rank: int
    tokens: int
    seed: int


FFN_WORKLOADS = [
    FfnWorkload("llama7b-ffn-b16-hybrid50-r1024-w8a8", 4096, 11008, 5504, 1024, 16, 0x5EEDF000),
]


def ffn_weights(f: FfnWorkload):
    """fp32 weights of the hybrid FFN (numpy, row-major, rows = outputs):
    wg, wu [F-S, E] ~ N(0, 1/E); ag, au [r, E] ~ N(0, 1/E); bg, bu [S, r] ~
    N(0, 1/r); wd [E, F] ~ N(0, 1/F).  Each drawn from its own stream."""
    E, F, S, r = f.embed, f.hidden, f.n_lowrank, f.rank
    shapes = [(F - S, E, E), (F - S, E, E), (r, E, E), (r, E, E), (S, r, r), (S, r, r), (E, F, F)]
    out = []
    for i, (a, b, fan) in enumerate(shapes):
        key = stream_key(f.seed, TAG_FFN, i)
        out.append(normal(key, 0, a * b, 1.0 / math.sqrt(max(fan, 1))).view(a, b).numpy())
    return out


def ffn_activations(f: FfnWorkload, tokens: int, device="cpu") -> torch.Tensor:
    """x [tokens, E] ~ N(0, 1), rounded to bf16."""
    key = stream_key(f.seed, TAG_FFN, 100)
    return normal(key, 0, tokens * f.embed, 1.0, device).view(tokens, f.embed).to(torch.bfloat16)


def queries(w: Workload, layer: int, step: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """q for one decode step: [B, H, d] ~ N(0, 1), rounded to ``dtype``."""
    key = stream_key(w.seed, TAG_Q, layer, step)
    n = w.batch * w.n_heads * w.head_dim
    return normal(key, 0, n, 1.0, device).view(w.batch, w.n_heads, w.head_dim).to(dtype)


def latents(w: Workload, layer: int, b: int, t0: int, t1: int,
            a_k: torch.Tensor, a_v: torch.Tensor, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 latents c = x·A for tokens [t0, t1) of batch row ``b`` (K and V).

    This is synthesis of the inputs (the projection that produces the cached
    latents), done by a plain fp32 matmul; it is not part of the decode step.
    """
    x = activations(w, layer, b, t0, t1, device)
    return x @ a_k, x @ a_v


def head_offsets(ranks: Sequence[int]) -> List[int]:
    out, acc = [], 0
    for r in ranks:
        out.append(acc)
        acc += r
    return out
