// layout.h -- internal: cache layout arithmetic and the per-layer head table.
// Used by the host plan code and by the kernels, so both sides compute the
// same byte offsets.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/lr_attn.h"

#if defined(__HIPCC__)
#define LR_HD __host__ __device__ __forceinline__
#else
#define LR_HD inline
#endif

namespace lr {

constexpr int kTile = LR_TILE_TOKENS;   // tokens per tile == lanes per wavefront
constexpr int kChunk = 16;              // bytes one lane loads per chunk
constexpr int kHeadDim = LR_HEAD_DIM;
constexpr int kRegionAlign = 256;
constexpr int kPartStride = LR_MAX_RANK + 2;  // floats per split partial: m, l, u[r]

LR_HD int row_bytes(int qfmt, int r) { return qfmt == LR_Q_INT8_TOKEN ? r : r / 2; }
LR_HD int n_groups(int r) { return (r + 31) / 32; }
LR_HD int scale_bytes(int qfmt, int r) { return qfmt == LR_Q_INT8_TOKEN ? 4 : 2 * n_groups(r); }
LR_HD int tile_bytes(int qfmt, int r) { return kTile * (row_bytes(qfmt, r) + scale_bytes(qfmt, r)); }
LR_HD int n_tiles(int capacity) { return (capacity + kTile - 1) / kTile; }

// Per-layer table handed to every kernel by value (kernel-argument segment).
// Offsets of the K and V regions are in units of kRegionAlign bytes; head h's
// plane of sequence b starts at region + b * n_tiles(capacity) * tile_bytes.
// Every field is a 32-bit word: with narrower fields the compiler may fold a
// 2-byte-aligned element address into the base of a scalar load, and the
// scalar unit ignores the low two bits of that base.
struct HeadTab {
  uint32_t kreg[LR_MAX_HEADS];
  uint32_t vreg[LR_MAX_HEADS];
  uint32_t ranks[LR_MAX_HEADS];    // r_k | r_v << 16
  uint32_t loff[LR_MAX_HEADS];     // latent (== factor row) offset: K | V << 16
  uint32_t order[LR_MAX_HEADS];    // dispatch order: heads by bytes per token, largest first
  uint32_t xorder[LR_MAX_HEADS];   // the same heads dealt to the 8 XCDs: entry 8r + x is XCD x's r-th head
};

}  // namespace lr
