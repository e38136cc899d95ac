// project.hip -- latent generation on the matrix cores: the per-head latents
// c^K = x A^K_h and c^V = x A^V_h of new tokens (WSVD page, "Fine-grained
// per-head SVD": each head keeps its own rank-r latent of the embedding; LASER
// page, "System implementation": latent activations are generated inside a GPU
// kernel), in fp32 from bf16 activations and factors, for the quantised append
// that follows.
//
// At decode sizes (one token per sequence, a few dozen tokens) the product is
// bound by moving the factors (2 E bytes per latent dimension) from HBM and by
// feeding every work-group the same small activation block; two layout
// choices follow from measurement on MI355X:
//   * the factors are packed once (k_pack) so that the 16 x 32 operand block
//     of one MFMA step is 1 KB contiguous: lane l of the packed block holds
//     row l & 15, elements 8 (l >> 4) .. 8 (l >> 4) + 7 of the step.  Read in
//     row-major order the same step touches 16 rows at 64 bytes each, which
//     measured 1.7x slower;
//   * activations are read with plain coalesced 16-byte loads into LDS, a
//     phase of at most 128 KB at a time, and the MFMA operands are read from
//     there; the next phase's factors and activations are loaded into
//     registers while the current phase is multiplied.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "check.h"
#include "plan.h"

namespace {

using lr::Bounds;   // the checked build's bounds test (check.h)
using lr::checked;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 128 * 1024 + 64 * 16;   // largest activation phase + row padding

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// The packed factors are read once per launch (each work-group its own row
// tiles and part of E): non-temporal loads, as for the decode's cache.
#ifndef LR_PROJECT_NT_LOADS
#define LR_PROJECT_NT_LOADS 1
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const uint16_t* p) {
  if constexpr (LR_PROJECT_NT_LOADS) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return uint4{v.x, v.y, v.z, v.w};
  } else {
    return ld16(p);
  }
}

struct ProjArgs {
  const uint16_t* x;   // bf16 [T][E]
  const uint16_t* wp;  // packed factors: [k_tiles + v_tiles][E / 32][64 lanes][8]
  float* ck;           // fp32 [n_parts][T][nk]
  float* cv;           // fp32 [n_parts][T][nv]
  int32_t T, E, nk, nv;
  int32_t k_tiles, row_tiles;   // 16-row tiles of W^K; of W^K and W^V together
  int32_t t_blocks, tb_stride;  // token blocks; token blocks per grid pass
  int32_t units;                // work-groups per token block and part: ceil(row_tiles / RT)
  int32_t n_parts;              // E is split into this many ranges of steps, each summed
                                // into its own output block (1: the whole sum)
  Bounds bx, bw, bk, bv;        // extents of x, wp, ck, cv (checked build)
};

// Work-group (RT 16-row tiles, block of 16 NT tokens, part q of E):
//   c_q[t][n] = sum_{e in part q} x[t][e] w[n][e]
// where part q covers steps [q S / n_parts, (q + 1) S / n_parts) of the
// S = E / 32 MFMA steps (one part: all of E, and c_0 = c),
// with v_mfma_f32_16x16x32_bf16 (latent rows = MFMA rows, tokens = columns;
// lane (i, g) = (lane & 15, lane >> 4) supplies row/column i, elements 8 g ..
// 8 g + 7 of a step, and receives rows 4 g .. 4 g + 3 of column i).  E is
// walked in phases of PS = NW * SPW steps; in a phase wavefront w multiplies
// steps w SPW .. w SPW + SPW - 1, its partial tile is summed with the other
// wavefronts' through LDS in wavefront order at the end, so the result is the
// same on every call.  Rows and tokens past the ends are never stored.
template <int NT, int NW, int SPW, int RT>
__global__ __launch_bounds__(NW * 64) void k_project(ProjArgs a) {
  constexpr int TOK = 16 * NT;                 // tokens per block
  constexpr int PS = NW * SPW;                 // steps per phase
  constexpr int EP = 32 * PS;                  // embedding elements per phase
  constexpr int RS = EP * 2 + 16;              // LDS bytes per token row (padded)
  constexpr int XV = TOK * EP / 8;             // 16-byte activation pieces per phase
  constexpr int XPT = (XV + NW * 64 - 1) / (NW * 64);
  // LDS: one activation phase, reused for the wavefront partials at the end;
  // sized per instance so that small instances leave room for more
  // work-groups per compute unit
  constexpr int LDSB = TOK * RS > NW * RT * NT * 64 * 16 ? TOK * RS : NW * RT * NT * 64 * 16;
  static_assert(LDSB <= kLdsBytes, "activation phase exceeds LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDSB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int li = lane & 15, lg = lane >> 4;
  const int unit = blockIdx.x % a.units;
  const int part = (blockIdx.x / a.units) % a.n_parts;
  const int all_steps = a.E >> 5;
  const int sb = int(int64_t(part) * all_steps / a.n_parts);
  const int steps = int(int64_t(part + 1) * all_steps / a.n_parts) - sb;   // >= 1
  const int phases = (steps + PS - 1) / PS;
  const uint16_t* xs = a.x + 32 * sb;          // the part's first element of every token row
  const size_t osk = size_t(part) * a.T * a.nk, osv = size_t(part) * a.T * a.nv;
  // row tiles RT unit .. RT unit + RT - 1 (a tile past the last is loaded as
  // the last and never stored)
  const uint16_t* wl[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
    wl[r] = a.wp + (size_t(min(RT * unit + r, a.row_tiles - 1)) * all_steps + sb) * 512 + 8 * lane;

  for (int tb = blockIdx.x / (a.units * a.n_parts); tb < a.t_blocks; tb += a.tb_stride) {
    const int t0 = TOK * tb;
    uint4 wb[2][RT][SPW];
    uint4 xb[XPT];
    // factors of phase p for this wavefront's steps (clamped: a step past E is
    // loaded at the last step and not multiplied)
    auto load_w = [&](int p, uint4 (&dst)[RT][SPW]) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int u = 0; u < SPW; ++u)
          dst[r][u] = ld16_stream(checked(a.bw, wl[r] + size_t(min(p * PS + wid * SPW + u, steps - 1)) * 512, 16));
    };
    // activations of phase p, piece q = row * (EP / 8) + col: token t0 + row,
    // elements p EP + 8 col .. + 7 (clamped into the row and the token range)
    auto load_x = [&](int p) {
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int q = min(tid + m * NW * 64, XV - 1);
        const int row = q / (EP / 8), col = q % (EP / 8);
        xb[m] = ld16(checked(a.bx, xs + size_t(min(t0 + row, a.T - 1)) * a.E + min(p * EP + 8 * col, 32 * steps - 8), 16));
      }
    };
    auto store_x = [&]() {
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int q = tid + m * NW * 64;
        if (q < XV) *reinterpret_cast<uint4*>(lds + (q / (EP / 8)) * RS + 16 * (q % (EP / 8))) = xb[m];
      }
    };
    f32x4_t acc[RT][NT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[r][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int p, const uint4 (&w)[RT][SPW]) {
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        const int cl = wid * SPW + u;
        if (p * PS + cl < steps) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const bf16x8_t bv = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4*>(lds + (16 * j + li) * RS + 64 * cl + 16 * lg));
#pragma unroll
            for (int r = 0; r < RT; ++r)
              acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w[r][u]), bv,
                                                                  acc[r][j], 0, 0, 0);
          }
        }
      }
    };

    // two phases per trip so that the factor registers alternate statically
    load_w(0, wb[0]);
    load_x(0);
    for (int p = 0; p < phases; p += 2) {
      store_x();
      __syncthreads();
      if (p + 1 < phases) {
        load_w(p + 1, wb[1]);
        load_x(p + 1);
      }
      compute(p, wb[0]);
      __syncthreads();
      if (p + 1 < phases) {
        store_x();
        __syncthreads();
        if (p + 2 < phases) {
          load_w(p + 2, wb[0]);
          load_x(p + 2);
        }
        compute(p + 1, wb[1]);
        __syncthreads();
      }
    }

    f32x4_t* s_red = reinterpret_cast<f32x4_t*>(lds);   // [NW][RT][NT][64]
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int j = 0; j < NT; ++j) s_red[((wid * RT + r) * NT + j) * 64 + lane] = acc[r][j];
    __syncthreads();
    // tile r, token tt, row nn: consecutive threads on consecutive rows of one token
    for (int i = tid; i < RT * NT * 256; i += NW * 64) {
      const int r = i / (NT * 256), ii = i % (NT * 256);
      const int tt = ii >> 4, nn = ii & 15;
      const int j = tt >> 4, src = (tt & 15) + 16 * (nn >> 2), e = nn & 3;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_red[((w * RT + r) * NT + j) * 64 + src][e];
      const int rt = RT * unit + r;
      const bool isv = rt >= a.k_tiles;
      const int t = t0 + tt, n = 16 * (isv ? rt - a.k_tiles : rt) + nn, N = isv ? a.nv : a.nk;
      if (rt < a.row_tiles && t < a.T && n < N)
        *checked(isv ? a.bv : a.bk, (isv ? a.cv + osv : a.ck + osk) + size_t(t) * N + n, 4) = v;
    }
    __syncthreads();
  }
}

// Packing of the factors: piece q (16 bytes) of the packed buffer is lane l =
// q % 64 of step c = (q / 64) % (E / 32) of tile r = q / (64 E / 32): row
// 16 r' + (l & 15) of W^K (r < k_tiles, r' = r) or W^V (r' = r - k_tiles),
// elements 32 c + 8 (l >> 4) .. + 7; rows past the end are zeros.
__global__ __launch_bounds__(256) void k_pack(const uint16_t* wk, const uint16_t* wv, uint16_t* wp, int32_t E,
                                              int32_t nk, int32_t nv, int32_t k_tiles, size_t pieces, Bounds bwk,
                                              Bounds bwv, Bounds bwp) {
  const int steps = E >> 5;
  for (size_t q = size_t(blockIdx.x) * 256 + threadIdx.x; q < pieces; q += size_t(gridDim.x) * 256) {
    const int l = int(q & 63);
    const size_t cq = q >> 6;
    const int c = int(cq % steps);
    const int r = int(cq / steps);
    const bool isv = r >= k_tiles;
    const int row = 16 * (isv ? r - k_tiles : r) + (l & 15);
    const int N = isv ? nv : nk;
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (row < N) v = ld16(checked(isv ? bwv : bwk, (isv ? wv : wk) + size_t(row) * E + 32 * c + 8 * (l >> 4), 16));
    *checked(bwp, reinterpret_cast<uint4*>(wp + 8 * q), 16) = v;
  }
}

}  // namespace

namespace lr {

size_t packed_projection_elems(const lr_attn_plan& p, int32_t layer, int32_t embed) {
  const auto& L = p.layers[layer];
  return size_t((L.sum_rk + 15) / 16 + (L.sum_rv + 15) / 16) * 16 * size_t(embed);
}

int launch_pack_projection(const lr_attn_plan& p, int32_t layer, int32_t embed, const void* wk,
                           const void* wv, void* packed, void* stream) {
  const auto& L = p.layers[layer];
  const size_t pieces = packed_projection_elems(p, layer, embed) / 8;
  const size_t groups = (pieces + 255) / 256;
  const unsigned grid = unsigned(groups < 65536 ? groups : 65536);
  hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(wk), static_cast<const uint16_t*>(wv),
                     static_cast<uint16_t*>(packed), embed, L.sum_rk, L.sum_rv, (L.sum_rk + 15) / 16,
                     pieces, Bounds{static_cast<const uint8_t*>(wk), checked_extent(size_t(L.sum_rk) * embed * 2)},
                     Bounds{static_cast<const uint8_t*>(wv), checked_extent(size_t(L.sum_rv) * embed * 2)},
                     Bounds{static_cast<const uint8_t*>(packed), checked_extent(pieces * 16)});
  return int(hipGetLastError());
}

namespace {
// Launch shape of the projection without an E split: token-block size in
// 16-token tiles, whether work-groups take two row tiles, work-groups per
// token block, token blocks.
struct ProjShape {
  int nt;
  bool two;
  int units, t_blocks;
};
ProjShape proj_shape(const lr_attn_plan::Layer& L, int32_t n_tokens) {
  // Up to 48 tokens: one block of 16, 32 or 48 tokens per work-group and one
  // row tile.  From 49 tokens on: blocks of 32 tokens and two row tiles per
  // work-group, so that every staged activation serves 32 latent rows (the
  // LDS re-reads of the activations bound this case: 64 tokens at E = 4096
  // over 4096 rows measured 15.4 us with 64-token blocks and one tile, 12.7 us
  // so).  Larger calls loop over token blocks.
  const int row_tiles = (L.sum_rk + 15) / 16 + (L.sum_rv + 15) / 16;
  const int col_tiles = (n_tokens + 15) / 16;   // n_tokens >= 1
  ProjShape s;
  s.two = col_tiles >= 4;
  s.nt = s.two ? 2 : col_tiles;
  s.units = s.two ? (row_tiles + 1) / 2 : row_tiles;
  s.t_blocks = (col_tiles + s.nt - 1) / s.nt;
  return s;
}
}  // namespace

// Work-groups a split projection aims for: at decode sizes the product moves
// each work-group's factor block (tens of KB) in about one memory round trip,
// so it needs every compute unit busy with two or more resident work-groups,
// not long work-groups.  Only the one-tile, 16-token instance is split: its
// split parts use the 33 KB activation phase, so several work-groups share a
// compute unit.  Measured on MI355X, MALL-cold (copies of the factors
// cycled), E = 4096, us per launch for 1 / 2 / 3 / 4 / 8 parts:
//   16 tokens, 128 row tiles  8.6 / 6.4 / 9.1 / 6.0 / 7.8
//    8 tokens, 192 row tiles  9.0 / 9.8 / 12.7 / 8.3 / 10.8
// while 32 and 64 tokens were fastest unsplit (11.3 and 14.7 us; 12.4 and
// 16.8 with two parts): their larger activation blocks leave one work-group
// per compute unit, so more work-groups only add rounds.  Uneven parts (3)
// lose to the powers of two.
#ifndef LR_PROJECT_TARGET_WGS
#define LR_PROJECT_TARGET_WGS 512
#endif

int project_parts(const lr_attn_plan& p, int32_t layer, int32_t n_tokens, int32_t embed) {
  const ProjShape s = proj_shape(p.layers[layer], n_tokens);
  if (s.two || s.nt != 1) return 1;
  const int64_t wgs = int64_t(s.units) * s.t_blocks;
  const int64_t cap = std::min<int64_t>(kMaxProjectParts, embed / 32 / 8);   // >= 8 steps a part
  int64_t parts = 1;
  while (parts * 2 <= cap && parts * wgs < LR_PROJECT_TARGET_WGS) parts *= 2;
  return int(parts);
}

int launch_project(const lr_attn_plan& p, int32_t layer, const void* x, int32_t n_tokens,
                   int32_t embed, const void* packed, float* ck, float* cv, void* stream,
                   int32_t n_parts) {
  const auto& L = p.layers[layer];
  ProjArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.wp = static_cast<const uint16_t*>(packed);
  a.ck = ck;
  a.cv = cv;
  a.T = n_tokens;
  a.E = embed;
  a.nk = L.sum_rk;
  a.nv = L.sum_rv;
  a.k_tiles = (L.sum_rk + 15) / 16;
  a.row_tiles = a.k_tiles + (L.sum_rv + 15) / 16;
  const ProjShape sh = proj_shape(L, n_tokens);
  a.units = sh.units;
  a.t_blocks = sh.t_blocks;
  a.n_parts = n_parts;
  a.bx = Bounds{static_cast<const uint8_t*>(x), checked_extent(size_t(n_tokens) * embed * 2)};
  a.bw = Bounds{static_cast<const uint8_t*>(packed), checked_extent(packed_projection_elems(p, layer, embed) * 2)};
  a.bk = Bounds{reinterpret_cast<const uint8_t*>(ck), checked_extent(size_t(n_parts) * n_tokens * L.sum_rk * 4)};
  a.bv = Bounds{reinterpret_cast<const uint8_t*>(cv), checked_extent(size_t(n_parts) * n_tokens * L.sum_rv * 4)};
  const int max_tb = (1 << 20) / (a.units * n_parts);   // at most 2^20 work-groups
  a.tb_stride = a.t_blocks < max_tb ? a.t_blocks : max_tb;
  const dim3 grid(unsigned(a.units) * unsigned(n_parts) * unsigned(a.tb_stride));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // activation phases of 2048 elements up to 32 tokens (1024 where a part
  // has at most 32 steps), 1024 above
  const bool short_part = (embed / 32) / n_parts <= 32;
  if (sh.two) hipLaunchKernelGGL((k_project<2, 8, 4, 2>), grid, dim3(512), 0, s, a);
  else if (sh.nt == 1 && short_part) hipLaunchKernelGGL((k_project<1, 8, 4, 1>), grid, dim3(512), 0, s, a);
  else if (sh.nt == 1) hipLaunchKernelGGL((k_project<1, 8, 8, 1>), grid, dim3(512), 0, s, a);
  else if (sh.nt == 2 && short_part) hipLaunchKernelGGL((k_project<2, 8, 4, 1>), grid, dim3(512), 0, s, a);
  else if (sh.nt == 2) hipLaunchKernelGGL((k_project<2, 8, 8, 1>), grid, dim3(512), 0, s, a);
  else hipLaunchKernelGGL((k_project<3, 8, 4, 1>), grid, dim3(512), 0, s, a);
  return int(hipGetLastError());
}

int project_check_take(unsigned long long* count) {
#if LR_ATTN_CHECK
  const unsigned long long zero = 0;
  hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_check_count), sizeof *count, 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_check_count), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  return int(e);
#else
  *count = 0;
  return 0;
#endif
}

}  // namespace lr
