// ffn.hip -- decode step of the hybrid low-rank / dense SwiGLU FFN with W8A8
// round-to-nearest quantisation (LASER page, "Hybrid SVD-quantisation for
// FFNs": SVD-friendly hidden channels of the gate and up projections go
// through low-rank factors, the rest stay dense, both branches RTN-quantised;
// "System implementation": the fused FFN kernels cover the input projection,
// the latent activations, SwiGLU and quantisation / dequantisation).
//
//   hidden channels [0, S):  g = B_g (A_g x),  u = B_u (A_u x)   (rank r)
//   hidden channels [S, F):  g = W_g x,        u = W_u x
//   h = silu(g) * u,         y = W_d h
//
// Weights are int8 with one fp32 scale per row; activations (x, the latents
// z = A x, h) are int8 with one fp32 scale per token and per group of 64
// elements along the reduction dimension -- the k extent of one
// v_mfma_i32_16x16x64_i8, so every product is an exact integer sum per group,
// converted and scaled once per group in fp32.  Four launches:
//   k_ffn_quant x -> codes and group scales; clears the step's counters
//   k_ffn_in    the latents z = [A_g; A_u] x, each 64-latent group in two
//               work-groups over the halves of E; the second to finish adds
//               the halves and quantises the group.  Dense pairs:
//               h = silu(g) u
//   k_ffn_mid   low-rank pairs: h = silu(g) u
//   k_ffn_out   y = W_d h, the hidden dimension split in chunks of 4096
//               across work-groups; the last chunk of a row tile to finish
//               adds the chunks' partial sums in chunk order
// When the last chunks of the down projection hold no low-rank channel,
// their work-groups join the low-rank pairs' launch (k_ffn_mid_out) and
// k_ffn_out takes the others.
// The last pair work-group of each 64-channel group of h (in k_ffn_in or
// k_ffn_mid) quantises the group.  Each activation is quantised once (one
// wavefront per token and group); the GEMM launches copy 16 tokens' codes into
// LDS with coalesced loads.
// At decode sizes every launch streams its int8 weights once from HBM (packed
// so that one MFMA step of 16 rows x 64 k is 1 KB contiguous: lane l holds row
// l & 15, k = 16 (l >> 4) .. + 15) against a block of at most 16 tokens.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "check.h"
#include "ffn_lds.h"
#include "plan.h"

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The weights are read once per step, but the streaming hint did not pay
// here (MALL-cold 47.6 vs 47.7 us per step, warm 45.8 vs 42.9 us): the FFN
// step is bound by launch and memory latency, not by the stream, so plain
// loads are the default.
#ifndef LR_FFN_NT_LOADS
#define LR_FFN_NT_LOADS 0
#endif

using namespace lr::ffnlds;   // LDS layout and instances (ffn_lds.h)
using lr::Bounds;             // the checked build's bounds test (check.h)
using lr::checked;
constexpr int kThreads = kWaves * 64;
// LDS: the codes and group scales of 16 tokens (E in k_ffn_in, two blocks of
// r in k_ffn_mid, one chunk of k_ffn_out), then 2 x 16 x 16 fp32 of reduced
// outputs; the partial-tile reduction reuses the code area once the products
// are done.  Sizes are static, one per template instance, the smallest that
// fits the shape (so that two to four work-groups share a compute unit):
// sizing dynamic LDS per launch measured all-zero outputs from k_ffn_out for
// hidden sizes between 1.3 K and 8 K on MI355X, with no access past the
// requested size that we could find.

// The int8 quantiser of one group: s = max|v| / 127, q = clamp(rne(v / s)),
// 0 when s == 0 (correctly rounded fp32 division, round half to even).
__device__ __forceinline__ int code(float v, float s) {
  return s != 0.0f ? int(fminf(fmaxf(rintf(v / s), -127.0f), 127.0f)) : 0;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ float wave_absmax(float v) {
  float m = fabsf(v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Quantise x: src [T][K] bf16 (row stride ld elements) -> codes dst [T][Kp]
// (Kp = K rounded up to 64; zeros past K) and scales sc [T][Kp / 64].  One
// wavefront per (token, group of 64), one element per lane; the group's
// max|v| is a wavefront reduction.  The launch also clears the n_cnt
// counters that the step's later launches count into.
// The extents the checked build tests the launches' accesses against.
struct FfnBounds {
  Bounds w, ws, x, y;   // packed weights, workspace, input x, output y
};

__global__ __launch_bounds__(256) void k_ffn_quant(const uint16_t* src, int64_t ld, int32_t K, int32_t T, int32_t Kp,
                                                   int8_t* dst, float* sc, int32_t* cnt, int32_t n_cnt, FfnBounds fb) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_cnt; i += gridDim.x * 256) *checked(fb.ws, cnt + i, 4) = 0;
  const int groups = Kp / 64;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= T * groups) return;
  const int t = wave / groups, g = wave % groups, k = 64 * g + lane;
  const float v = k < K ? __uint_as_float(uint32_t(*checked(fb.x, src + t * ld + k, 2)) << 16) : 0.0f;
  const float s = wave_absmax(v) / 127.0f;
  *checked(fb.ws, dst + size_t(t) * Kp + k, 1) = int8_t(code(v, s));
  if (lane == 0) *checked(fb.ws, sc + size_t(t) * groups + g, 4) = s;
}

// Copy codes of tokens t0 .. t0 + 15 (clamped to T - 1), columns c0 .. c0 +
// kn - 1 of an int8 matrix (row stride ld, kn a multiple of 64) and their
// group scales (row stride ld / 64) into an LDS block: codes [16][rs], scales
// [16][kn / 64].  Loads go straight from memory into LDS (one wavefront load
// writes a lane's 16 or 4 bytes at the wavefront's LDS base + 16 or 4 x
// lane), so the copy holds no registers while the weights are in flight;
// `staged` then waits for them and passes a barrier.
#ifndef LR_FFN_LDS_DMA
#define LR_FFN_LDS_DMA 1
#endif
using lds_ptr = __attribute__((address_space(3))) void*;
__device__ void stage_codes(const Bounds& bws, const int8_t* codes, const float* scales, int64_t ld, int c0, int kn,
                            int T, int t0, int8_t* act, float* scale, int rs) {
  const int pieces = kn / 16, gn = kn / 64;
  if constexpr (LR_FFN_LDS_DMA) {
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int segs = (pieces + 63) / 64, gsegs = (gn + 63) / 64;
    for (int job = wid; job < 16 * segs; job += kWaves) {   // one 1 KB row segment per wavefront load
      const int tt = job / segs, sg = job % segs, t = min(t0 + tt, T - 1), piece = 64 * sg + lane;
      if (piece < pieces)
        __builtin_amdgcn_global_load_lds(checked(bws, codes + t * ld + c0 + 16 * piece, 16),
                                         (lds_ptr)(act + tt * rs + 1024 * sg), 16, 0, 0);
    }
    for (int job = wid; job < 16 * gsegs; job += kWaves) {
      const int tt = job / gsegs, sg = job % gsegs, t = min(t0 + tt, T - 1), g = 64 * sg + lane;
      if (g < gn)
        __builtin_amdgcn_global_load_lds(checked(bws, scales + t * (ld / 64) + c0 / 64 + g, 4),
                                         (lds_ptr)(scale + tt * gn + 64 * sg), 4, 0, 0);
    }
  } else {
    for (int i = threadIdx.x; i < 16 * pieces; i += kThreads) {
      const int tt = i / pieces, col = i % pieces, t = min(t0 + tt, T - 1);
      *reinterpret_cast<uint4*>(act + tt * rs + 16 * col) =
          *checked(bws, reinterpret_cast<const uint4*>(codes + t * ld + c0 + 16 * col), 16);
    }
    for (int i = threadIdx.x; i < 16 * gn; i += kThreads) {
      const int tt = i / gn, g = i % gn, t = min(t0 + tt, T - 1);
      scale[i] = *checked(bws, scales + t * (ld / 64) + c0 / 64 + g, 4);
    }
  }
}

// After stage_codes: this wavefront's loads (the copies into LDS among them)
// are complete, then a barrier -- the staged block is complete for all.
__device__ __forceinline__ void staged() {
  if constexpr (LR_FFN_LDS_DMA) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
}

// acc[r] += over this wavefront's steps c in [c0, c1) of tile r: the int8
// MFMA of the step (exact integer sums over 64 k) times the activation scale
// of the lane's token for that group (g = c - gbase in the LDS block).  The
// first batch of weight loads is issued before `stage` runs (stage fills LDS
// and ends with a barrier), so their latency overlaps the staging.
template <int RT, typename Stage>
__device__ __forceinline__ void gemm_steps(const Bounds& bw, const uint8_t* const (&wt)[RT], int c0, int c1, int gbase,
                                           const int8_t* const (&act)[RT], const float* const (&scale)[RT],
                                           int rs, int groups, f32x4_t (&acc)[RT], Stage stage) {
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  constexpr int U = RT > 2 ? 4 : 8;   // steps of weights in flight per batch (registers: U x RT x 4)
  i32x4_t a[U][RT];
  auto load = [&](int c) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const i32x4_t* p =
            checked(bw, reinterpret_cast<const i32x4_t*>(wt[r] + size_t(min(c + u, c1 - 1)) * 1024 + 16 * lane), 16);
        if constexpr (LR_FFN_NT_LOADS) a[u][r] = __builtin_nontemporal_load(p);
        else a[u][r] = *p;
      }
  };
  if (c0 < c1) load(c0);
  stage();
  for (int c = c0; c < c1; c += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u < c1) {
        const int g = c + u - gbase;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const i32x4_t b = *reinterpret_cast<const i32x4_t*>(act[r] + li * rs + 64 * g + 16 * lg);
          const i32x4_t p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][r], b, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
          const float sc = scale[r][li * groups + g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r][e] += float(p[e]) * sc;
        }
      }
    }
    if (c + U < c1) load(c + U);
  }
}

// Sum the wavefronts' partial tiles in wavefront order into out[r][token][row]
// (LDS, 16 x 16 fp32 per tile); lane (i, g) of a partial holds rows 4 g ..
// 4 g + 3 of token i.  Ends with a barrier: out is then readable by all.
template <int RT>
__device__ void reduce_tiles(f32x4_t (&acc)[RT], uint8_t* smem, float* out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __syncthreads();
  f32x4_t* s_red = reinterpret_cast<f32x4_t*>(smem);   // [kWaves][RT][64]
#pragma unroll
  for (int r = 0; r < RT; ++r) s_red[(wid * RT + r) * 64 + lane] = acc[r];
  __syncthreads();
  for (int i = tid; i < RT * 256; i += kThreads) {
    const int r = i >> 8, tt = (i >> 4) & 15, nn = i & 15;
    const int src = tt + 16 * (nn >> 2), e = nn & 3;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += s_red[(w * RT + r) * 64 + src][e];
    out[i] = v;
  }
  __syncthreads();
}

// ---- the last work-group of a group finishes it ---------------------------
// A group of work (the two halves of a latent group, the pair work-groups
// of a 64-channel group of h, the chunks of a down-projection row tile) is
// finished by whichever of its work-groups completes last, with no wait:
// each counts itself on a counter (agent-scope atomic) once its share is
// stored, and the one that brings the count to the group's size reads the
// others' shares.  Each XCD has its own L2 and the workspace is ordinary
// device memory, so the shares are written with device-coherent stores
// (relaxed agent-scope atomic stores, written through), every wavefront
// waits until its stores are acknowledged before the count, and the buffers
// are laid out so that no cache line holds parts of two groups: no cache
// then holds a line of a share from before it was complete (a kernel
// boundary writes back and invalidates them), and plain loads read it.
// (Agent-scope fences would do it too, but each writes back or invalidates
// a whole L2; measured many times slower.)
template <typename V>
__device__ __forceinline__ void put(V* p, V v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Every wavefront waits for its stores (they count in vmcnt on this
// architecture), then thread 0 counts the work-group's share; returns, to
// every thread, whether it completed the group of `size`.
__device__ bool count_last(const Bounds& bws, int32_t* c, int size, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(checked(bws, c, 4), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == size - 1;
  __syncthreads();
  return *s_flag != 0;
}

// Quantise one 64-channel group g of h (rows of Fh floats, zeros past F)
// for tokens t0 .. t0 + 15: one wavefront per token, a lane per channel.
__device__ void quantise_h_group(const Bounds& bws, const float* h, int Fh, int F, int8_t* hq, float* hs, int Fp,
                                 int T, int t0, int g) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, ch = 64 * g + lane;
  for (int tt = wid; tt < 16; tt += kWaves) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float v = ch < F ? *checked(bws, h + size_t(t) * Fh + ch, 4) : 0.0f;
    const float s = wave_absmax(v) / 127.0f;
    *checked(bws, hq + size_t(t) * Fp + ch, 1) = int8_t(code(v, s));
    if (lane == 0) *checked(bws, hs + size_t(t) * (Fp / 64) + g, 4) = s;
  }
}

// Pair work-group's 16 channels ch0 .. ch0 + 15 of h are stored: count them
// into their group; the last quantises it.
struct HArgs {
  float* h;                   // [T][Fh] (Fh: F rounded up to 32, whole cache lines per group)
  int8_t* hq;                 // [T][Fp]
  float* hs;                  // [T][Fp / 64]
  int32_t* hcnt;              // [TB][Fp / 64] pair work-groups done per group
  int32_t Fh, Fp;
};
__device__ void h_stored(const Bounds& bws, const HArgs& ha, int F, int T, int t0, int ch0, int* s_flag) {
  const int g = ch0 >> 6, G = ha.Fp / 64;
  if (count_last(bws, ha.hcnt + (t0 / 16) * G + g, min(64, F - 64 * g) / 16, s_flag))
    quantise_h_group(bws, ha.h, ha.Fh, F, ha.hq, ha.hs, ha.Fp, T, t0, g);
}

static_assert(in_extent(2048) <= kLdsS && in_extent(4096) <= kLdsM && in_extent(8192) <= kLdsL &&
                  mid_extent(1024) <= kLdsS && mid_extent(2048) <= kLdsM && mid_extent(4096) <= kLdsL,
              "LDS instances");

struct InArgs {
  const int8_t* xq;           // [T][E] codes of x
  const float* xs;            // [T][E / 64]
  const uint8_t* w;           // packed tiles: dense pairs (gate, up), then latent rows of [A_g; A_u]
  const float* ws;            // row scales in tile order
  HArgs ha;
  float* zp;                  // [2][T][2 r] the two halves' partial latents (before row scales)
  int32_t* zcnt;              // [TB][lat_groups] halves done per latent group
  int8_t* zq;                 // [T][2 r] codes of the latents z = [A_g; A_u] x
  float* zs;                  // [T][2 r / 64] their group scales
  int32_t T, E, F, S, pairs, lat_groups;   // pairs = (F - S) / 16; lat_groups = 2 r / 64
  FfnBounds fb;
};

// Launch 2: work-group = (latent half-group or dense pair, block of 16
// tokens).  Latent group j (64 latents, four 16-row tiles, one activation
// group of z) is split over E: work-group (j, q) sums the steps of half q.
// The latent work-groups come first in the grid.
template <int LDS>
__global__ __launch_bounds__(kThreads) void k_ffn_in(InArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ int s_flag;
  const int steps = a.E / 64;
  float* outv = reinterpret_cast<float*>(smem + code_area(block_bytes(a.E)));
  const int units = a.pairs + 2 * a.lat_groups;
  const int unit = blockIdx.x % units, t0 = 16 * (blockIdx.x / units);
  int8_t* act = reinterpret_cast<int8_t*>(smem);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit < 2 * a.lat_groups) {   // uniform: latent group j, half q; tiles 2 pairs + 4 j ..
    const int j = unit >> 1, q = unit & 1;
    const int h0 = steps / 2, c0 = q ? h0 : 0, n = q ? steps - h0 : h0;   // this half's steps
    const int rs = row_stride(64 * n);
    float* scale = reinterpret_cast<float*>(smem + scale_offset(64 * n));
    const int tile0 = 2 * a.pairs + 4 * j;
    const uint8_t* wt[4];
    const int8_t* acts[4];
    const float* scs[4];
    f32x4_t acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wt[r] = a.w + size_t(tile0 + r) * steps * 1024;
      acts[r] = act;
      scs[r] = scale;
      acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    gemm_steps<4>(a.fb.w, wt, c0 + n * wid / kWaves, c0 + n * (wid + 1) / kWaves, c0, acts, scs, rs, n, acc, [&]() {
      stage_codes(a.fb.ws, a.xq, a.xs, a.E, 64 * c0, 64 * n, a.T, t0, act, scale, rs);
      staged();
    });
    reduce_tiles<4>(acc, smem, outv);
    // this half's sums, lane = latent 16 r + nn of the group, one wavefront per token
    const int zr = 64 * a.lat_groups, r = lane >> 4, nn = lane & 15;   // zr = 2 r floats per token
    for (int tt = wid; tt < 16; tt += kWaves) {
      const int t = t0 + tt;
      if (t < a.T) put(checked(a.fb.ws, a.zp + (size_t(q) * a.T + t) * zr + 64 * j + lane, 4), outv[(r * 16 + tt) * 16 + nn]);
    }
    if (!count_last(a.fb.ws, a.zcnt + (t0 / 16) * a.lat_groups + j, 2, &s_flag)) return;
    // the second half to finish: z = (half 0 + half 1) x row scale, quantised per token
    for (int tt = wid; tt < 16; tt += kWaves) {
      const int t = t0 + tt;
      if (t >= a.T) break;
      const size_t o = size_t(t) * zr + 64 * j + lane;
      const float v = (*checked(a.fb.ws, a.zp + o, 4) + *checked(a.fb.ws, a.zp + size_t(a.T) * zr + o, 4)) *
                      *checked(a.fb.w, a.ws + 16 * (tile0 + r) + nn, 4);
      const float s = wave_absmax(v) / 127.0f;
      *checked(a.fb.ws, a.zq + o, 1) = int8_t(code(v, s));
      if (lane == 0) *checked(a.fb.ws, a.zs + size_t(t) * a.lat_groups + j, 4) = s;
    }
    return;
  }
  const int rs = row_stride(a.E);
  float* scale = reinterpret_cast<float*>(smem + scale_offset(a.E));
  const int p = unit - 2 * a.lat_groups;   // dense pair p: tiles (gate, up) = 2 p, 2 p + 1
  const int tile0 = 2 * p;
  const uint8_t* wt[2] = {a.w + size_t(tile0) * steps * 1024, a.w + size_t(tile0 + 1) * steps * 1024};
  const int8_t* acts[2] = {act, act};
  const float* scs[2] = {scale, scale};
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  gemm_steps<2>(a.fb.w, wt, steps * wid / kWaves, steps * (wid + 1) / kWaves, 0, acts, scs, rs, steps, acc, [&]() {
    stage_codes(a.fb.ws, a.xq, a.xs, a.E, 0, a.E, a.T, t0, act, scale, rs);
    staged();
  });
  reduce_tiles<2>(acc, smem, outv);
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    const int tt = i >> 4, nn = i & 15, t = t0 + tt;
    if (t >= a.T) continue;
    const float v0 = outv[i] * *checked(a.fb.w, a.ws + 16 * tile0 + nn, 4);
    const float v1 = outv[256 + i] * *checked(a.fb.w, a.ws + 16 * (tile0 + 1) + nn, 4);
    put(checked(a.fb.ws, a.ha.h + size_t(t) * a.ha.Fh + a.S + 16 * p + nn, 4), silu_mul(v0, v1));   // channel S + 16 p + nn
  }
  h_stored(a.fb.ws, a.ha, a.F, a.T, t0, a.S + 16 * p, &s_flag);
}

struct MidArgs {
  const int8_t* zq;           // [T][2 r] codes of the latents
  const float* zs;            // [T][2 r / 64]
  const uint8_t* w;           // packed pairs (B_g, B_u), k = r
  const float* ws;
  HArgs ha;                   // h channels [0, S)
  int32_t T, r, F, pairs;     // pairs = S / 16
  FfnBounds fb;
};

// Launch 3: work-group = (low-rank pair p, block of 16 tokens); B_g reads the
// gate latents (columns [0, r) of z), B_u the up latents ([r, 2 r)).  blk
// indexes the (pair, token block) units of the launch (launched only when
// pairs >= 1); smem holds at least mid_extent(r) bytes.
__device__ void mid_unit(const MidArgs& a, uint8_t* smem, int* s_flag, int blk) {
  const int rs = row_stride(a.r), steps = a.r / 64;
  float* outv = reinterpret_cast<float*>(smem + code_area(2 * block_bytes(a.r)));
  const int unit = blk % a.pairs, t0 = 16 * (blk / a.pairs);
  int8_t* act[2];
  float* sc[2];
  for (int half = 0; half < 2; ++half) {
    uint8_t* base = smem + half * block_bytes(a.r);
    act[half] = reinterpret_cast<int8_t*>(base);
    sc[half] = reinterpret_cast<float*>(base + scale_offset(a.r));
  }
  const int tile0 = 2 * unit;
  const uint8_t* wt[2] = {a.w + size_t(tile0) * steps * 1024, a.w + size_t(tile0 + 1) * steps * 1024};
  const int8_t* acts[2] = {act[0], act[1]};
  const float* scs[2] = {sc[0], sc[1]};
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  gemm_steps<2>(a.fb.w, wt, steps * wid / kWaves, steps * (wid + 1) / kWaves, 0, acts, scs, rs, steps, acc, [&]() {
    for (int half = 0; half < 2; ++half)
      stage_codes(a.fb.ws, a.zq, a.zs, 2 * a.r, half * a.r, a.r, a.T, t0, act[half], sc[half], rs);
    staged();
  });
  reduce_tiles<2>(acc, smem, outv);
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    const int tt = i >> 4, nn = i & 15, t = t0 + tt;
    if (t < a.T)
      put(checked(a.fb.ws, a.ha.h + size_t(t) * a.ha.Fh + 16 * unit + nn, 4),
          silu_mul(outv[i] * *checked(a.fb.w, a.ws + 16 * tile0 + nn, 4),
                   outv[256 + i] * *checked(a.fb.w, a.ws + 16 * (tile0 + 1) + nn, 4)));
  }
  h_stored(a.fb.ws, a.ha, a.F, a.T, t0, 16 * unit, s_flag);
}

template <int LDS>
__global__ __launch_bounds__(kThreads) void k_ffn_mid(MidArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ int s_flag;
  mid_unit(a, smem, &s_flag, blockIdx.x);
}

struct OutArgs {
  const int8_t* hq;           // [T][Fp]
  const float* hs;            // [T][Fp / 64]
  const uint8_t* w;           // packed W_d tiles, k = Fp
  const float* ws;
  float* y;                   // [T][E]
  float* yp;                  // partials [splits][T][E] when splits > 1
  int32_t* ycnt;              // [TB][units] chunks done per row tile
  int32_t T, E, Fp, units, splits;   // units = E / (16 RT); splits = ceil(Fp / CHUNK)
  int32_t split0, nsplit;     // the chunks this launch takes: split0 .. split0 + nsplit - 1
  FfnBounds fb;
};

// Launch 4: work-group = (RT tiles of 16 rows of W_d, one CHUNK of the hidden
// dimension, block of 16 tokens); its chunk of h's codes comes through LDS
// once for all RT tiles.  With several chunks each work-group stores its
// scaled partial sum, and the last chunk of the row tile to finish adds them
// in chunk order (RT = 2 then: a token's 32 rows are one 128-byte line).
// blk indexes the (row unit, chunk of split0 .., token block) units of the
// launch; smem holds at least out_extent(CHUNK, RT) bytes.
template <int CHUNK, int RT>
__device__ void out_unit(const OutArgs& a, uint8_t* smem, int* s_flag, int blk) {
  static_assert(RT <= 2, "two row tiles at most");
  const int unit = blk % a.units, split = a.split0 + (blk / a.units) % a.nsplit;
  const int t0 = 16 * (blk / (a.units * a.nsplit));
  const int steps = a.Fp / 64, kc = min(CHUNK, a.Fp);
  float* outv = reinterpret_cast<float*>(smem + code_area(block_bytes(kc)));
  const uint8_t* wt[RT];
  const int8_t* acts[RT];
  const float* scs[RT];
  f32x4_t acc[RT];
  int8_t* act = reinterpret_cast<int8_t*>(smem);
  const int k0 = split * CHUNK, kn = min(CHUNK, a.Fp - k0), gn = kn / 64, rs = row_stride(kn);
  float* scale = reinterpret_cast<float*>(smem + scale_offset(kn));
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    wt[r] = a.w + size_t(RT * unit + r) * steps * 1024;
    acts[r] = act;
    scs[r] = scale;
    acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cb = k0 / 64;
  gemm_steps<RT>(a.fb.w, wt, cb + gn * wid / kWaves, cb + gn * (wid + 1) / kWaves, cb, acts, scs, rs, gn, acc, [&]() {
    stage_codes(a.fb.ws, a.hq, a.hs, a.Fp, k0, kn, a.T, t0, act, scale, rs);
    staged();
  });
  reduce_tiles<RT>(acc, smem, outv);
  if (a.splits == 1) {
    for (int i = threadIdx.x; i < RT * 256; i += kThreads) {
      const int r = i >> 8, tt = (i >> 4) & 15, nn = i & 15, t = t0 + tt, row = 16 * (RT * unit + r) + nn;
      if (t < a.T) *checked(a.fb.y, a.y + size_t(t) * a.E + row, 4) = outv[i] * *checked(a.fb.w, a.ws + row, 4);
    }
    return;
  }
  const size_t n = size_t(a.T) * a.E;
  for (int i = threadIdx.x; i < RT * 256; i += kThreads) {
    const int r = i >> 8, tt = (i >> 4) & 15, nn = i & 15, t = t0 + tt, row = 16 * (RT * unit + r) + nn;
    if (t < a.T) put(checked(a.fb.ws, a.yp + split * n + size_t(t) * a.E + row, 4), outv[i] * *checked(a.fb.w, a.ws + row, 4));
  }
  if (!count_last(a.fb.ws, a.ycnt + (t0 / 16) * a.units + unit, a.splits, s_flag)) return;
  for (int i = threadIdx.x; i < RT * 256; i += kThreads) {   // y = sum over chunks s = 0, 1, ... in order
    const int r = i >> 8, tt = (i >> 4) & 15, nn = i & 15, t = t0 + tt, row = 16 * (RT * unit + r) + nn;
    if (t >= a.T) continue;
    const size_t o = size_t(t) * a.E + row;
    float v = 0.0f;
    for (int c = 0; c < a.splits; ++c) v += *checked(a.fb.ws, a.yp + c * n + o, 4);
    *checked(a.fb.y, a.y + o, 4) = v;
  }
}

template <int LDS, int CHUNK, int RT>
__global__ __launch_bounds__(kThreads) void k_ffn_out(OutArgs a) {
  static_assert(out_extent(CHUNK, RT) <= LDS, "chunk exceeds LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ int s_flag;
  out_unit<CHUNK, RT>(a, smem, &s_flag, blockIdx.x);
}

// Launch 3 when the last chunks of the down projection hold no low-rank
// channel: their units need only what launch 2 produced (the dense channels
// of h), so they run beside the low-rank pairs (a latency-bound launch that
// leaves HBM mostly idle) -- the first n_mid work-groups are pair units, the
// rest those chunks' units; launch 4 then takes the remaining chunks.
template <int LDS, int CHUNK, int RT>
__global__ __launch_bounds__(kThreads) void k_ffn_mid_out(MidArgs ma, OutArgs oa, int32_t n_mid) {
  static_assert(out_extent(CHUNK, RT) <= LDS, "chunk exceeds LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ int s_flag;
  if (int(blockIdx.x) < n_mid) mid_unit(ma, smem, &s_flag, blockIdx.x);
  else out_unit<CHUNK, RT>(oa, smem, &s_flag, int(blockIdx.x) - n_mid);
}

}  // namespace

namespace lr {

int launch_ffn(const FfnLayout& f, const void* weights, const void* x, int32_t n_tokens, float* y,
               void* workspace, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* w = static_cast<const uint8_t*>(weights);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + f.ws_xq);
  float* xs = reinterpret_cast<float*>(ws + f.ws_xs);
  int8_t* zq = reinterpret_cast<int8_t*>(ws + f.ws_zq);
  float* zs = reinterpret_cast<float*>(ws + f.ws_zs);
  const int T = n_tokens;
  const unsigned tb = unsigned((T + 15) / 16);
  const OutShape osh = out_shape(f.Fp);
  // the workspace (partial sums, counters) must be laid out for the same chunks
  if (osh.splits != f.out_splits || osh.rt != f.out_rt) return int(hipErrorInvalidValue);
  const int chunk = osh.chunk, splits = osh.splits, rt = osh.rt, out_units = f.E / (16 * rt);
  const int G = f.Fp / 64, lat_groups = 2 * f.r / 64;
  // counters: halves per latent group, pair work-groups per group of h, chunks per row tile
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + f.ws_cnt);
  int32_t* zcnt = cnt;
  int32_t* hcnt = zcnt + tb * lat_groups;
  int32_t* ycnt = hcnt + tb * G;
  const int n_cnt = int(tb) * (lat_groups + G + out_units);
  if (size_t(n_cnt) * 4 > f.ws_cnt_bytes) return int(hipErrorInvalidValue);
  HArgs ha{reinterpret_cast<float*>(ws + f.ws_h), reinterpret_cast<int8_t*>(ws + f.ws_hq),
           reinterpret_cast<float*>(ws + f.ws_hs), hcnt, f.h_ld, f.Fp};
  const FfnBounds fb{Bounds{w, checked_extent(f.weight_bytes)}, Bounds{ws, checked_extent(f.ws_bytes)},
                     Bounds{static_cast<const uint8_t*>(x), checked_extent(size_t(T) * f.E * 2)},
                     Bounds{reinterpret_cast<const uint8_t*>(y), checked_extent(size_t(T) * f.E * 4)}};
  int err = 0;

  const unsigned qgrid = unsigned((T * (f.E / 64) + 3) / 4);
  hipLaunchKernelGGL(k_ffn_quant, dim3(qgrid), dim3(256), 0, s, static_cast<const uint16_t*>(x), int64_t(f.E), f.E, T,
                     f.E, xq, xs, cnt, n_cnt, fb);
  if ((err = int(hipGetLastError())) != 0) return err;
  InArgs ia{xq, xs, w + f.off_w1, reinterpret_cast<const float*>(w + f.off_s1), ha,
            reinterpret_cast<float*>(ws + f.ws_zp), zcnt, zq, zs, T, f.E, f.F, f.S, (f.F - f.S) / 16, lat_groups, fb};
  if (ia.pairs + ia.lat_groups > 0) {
    const dim3 g(unsigned(ia.pairs + 2 * ia.lat_groups) * tb), b(kThreads);
    const int lds = instance_for(in_extent(f.E));   // the smallest instance that holds it
    if (lds == kLdsS) hipLaunchKernelGGL(k_ffn_in<kLdsS>, g, b, 0, s, ia);
    else if (lds == kLdsM) hipLaunchKernelGGL(k_ffn_in<kLdsM>, g, b, 0, s, ia);
    else if (lds == kLdsL) hipLaunchKernelGGL(k_ffn_in<kLdsL>, g, b, 0, s, ia);
    else return int(hipErrorInvalidConfiguration);
    if ((err = int(hipGetLastError())) != 0) return err;
  }
  // Chunks of 4096 (2048 for small hidden sizes); with several chunks a
  // work-group takes two row tiles, so each staged chunk of h serves 32 rows
  // of W_d (measured best on the LLaMA-7B FFN among chunks of 1, 2, 4 and 8 K
  // with one or two tiles).
  OutArgs oa{ha.hq, ha.hs, w + f.off_w3, reinterpret_cast<const float*>(w + f.off_s3), y,
             reinterpret_cast<float*>(ws + f.ws_yp), ycnt, T, f.E, f.Fp, out_units, splits, 0, splits, fb};
  // chunks from c_ind on hold no channel of a group of h with low-rank
  // channels: they can run beside the low-rank pairs (k_ffn_mid_out)
#ifndef LR_FFN_MERGE_OUT
#define LR_FFN_MERGE_OUT 1
#endif
  const int c_ind = ((f.S + 63) / 64 * 64 + chunk - 1) / chunk;
  const bool merge = LR_FFN_MERGE_OUT && f.S > 0 && splits > 1 && chunk == 4096 && rt == 2 && c_ind < splits;
  if (f.S > 0) {
    MidArgs ma{zq, zs, w + f.off_w2, reinterpret_cast<const float*>(w + f.off_s2), ha, T, f.r, f.F, f.S / 16, fb};
    const dim3 b(kThreads);
    if (merge) {
      OutArgs o3 = oa;
      o3.split0 = c_ind;
      o3.nsplit = splits - c_ind;
      oa.nsplit = c_ind;
      const int n_mid = ma.pairs * int(tb);
      const dim3 g(unsigned(n_mid) + unsigned(out_units) * unsigned(o3.nsplit) * tb);
      const int lds = instance_for(std::max(mid_extent(f.r), out_extent(4096, 2)));
      if (lds == kLdsM) hipLaunchKernelGGL((k_ffn_mid_out<kLdsM, 4096, 2>), g, b, 0, s, ma, o3, n_mid);
      else if (lds == kLdsL) hipLaunchKernelGGL((k_ffn_mid_out<kLdsL, 4096, 2>), g, b, 0, s, ma, o3, n_mid);
      else return int(hipErrorInvalidConfiguration);
    } else {
      const dim3 g(unsigned(ma.pairs) * tb);
      const int lds = instance_for(mid_extent(f.r));
      if (lds == kLdsS) hipLaunchKernelGGL(k_ffn_mid<kLdsS>, g, b, 0, s, ma);
      else if (lds == kLdsM) hipLaunchKernelGGL(k_ffn_mid<kLdsM>, g, b, 0, s, ma);
      else if (lds == kLdsL) hipLaunchKernelGGL(k_ffn_mid<kLdsL>, g, b, 0, s, ma);
      else return int(hipErrorInvalidConfiguration);
    }
    if ((err = int(hipGetLastError())) != 0) return err;
  }
  const dim3 g(unsigned(oa.units) * unsigned(oa.nsplit) * tb), b(kThreads);
  if (chunk == 2048) hipLaunchKernelGGL((k_ffn_out<kLdsS, 2048, 1>), g, b, 0, s, oa);
  else if (rt == 1) hipLaunchKernelGGL((k_ffn_out<kLdsM, 4096, 1>), g, b, 0, s, oa);
  else hipLaunchKernelGGL((k_ffn_out<kLdsM, 4096, 2>), g, b, 0, s, oa);
  return int(hipGetLastError());
}

int ffn_check_take(unsigned long long* count) {
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
