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
// converted and scaled once per group in fp32.  Five launches (six when h
// spans several chunks):
//   k_ffn_quant x -> codes and group scales
//   k_ffn_in    the latents z = [A_g; A_u] x, quantised by the work-group
//               that owns each 64-latent group; dense pairs: h = silu(g) u
//   k_ffn_mid   low-rank pairs: h = silu(g) u
//   k_ffn_quant h -> codes and group scales
//   k_ffn_out   y = W_d h, the hidden dimension split in chunks of 4096 across
//               work-groups (k_ffn_sum adds the chunks' partial sums in order)
// Each activation is quantised once (one wavefront per token and group); the
// GEMM launches copy 16 tokens' codes into LDS with coalesced loads.
// At decode sizes every launch streams its int8 weights once from HBM (packed
// so that one MFMA step of 16 rows x 64 k is 1 KB contiguous: lane l holds row
// l & 15, k = 16 (l >> 4) .. + 15) against a block of at most 16 tokens.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Quantise activations: src [T][K] (bf16 or fp32, row stride ld elements) ->
// codes dst [T][Kp] (Kp = K rounded up to 64; zeros past K) and scales
// sc [T][Kp / 64].  One wavefront per (token, group of 64), one element per
// lane; the group's max|v| is a wavefront reduction.
template <bool BF16>
__global__ __launch_bounds__(256) void k_ffn_quant(const void* src, int64_t ld, int32_t K, int32_t T, int32_t Kp,
                                                   int8_t* dst, float* sc) {
  const int groups = Kp / 64;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= T * groups) return;
  const int t = wave / groups, g = wave % groups, k = 64 * g + lane;
  float v = 0.0f;
  if (k < K) {
    if constexpr (BF16) v = __uint_as_float(uint32_t(static_cast<const uint16_t*>(src)[t * ld + k]) << 16);
    else v = static_cast<const float*>(src)[t * ld + k];
  }
  float m = fabsf(v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = m / 127.0f;
  dst[size_t(t) * Kp + k] = int8_t(code(v, s));
  if (lane == 0) sc[size_t(t) * groups + g] = s;
}

// Copy codes of tokens t0 .. t0 + 15 (clamped to T - 1), columns c0 .. c0 +
// kn - 1 of an int8 matrix (row stride ld, kn a multiple of 64) and their
// group scales (row stride ld / 64) into an LDS block: codes [16][rs], scales
// [16][kn / 64].  Coalesced 16-byte loads.
__device__ void stage_codes(const int8_t* codes, const float* scales, int64_t ld, int c0, int kn, int T, int t0,
                            int8_t* act, float* scale, int rs) {
  const int pieces = kn / 16, gn = kn / 64;
  for (int i = threadIdx.x; i < 16 * pieces; i += kThreads) {
    const int tt = i / pieces, col = i % pieces, t = min(t0 + tt, T - 1);
    *reinterpret_cast<uint4*>(act + tt * rs + 16 * col) =
        *reinterpret_cast<const uint4*>(codes + t * ld + c0 + 16 * col);
  }
  for (int i = threadIdx.x; i < 16 * gn; i += kThreads) {
    const int tt = i / gn, g = i % gn, t = min(t0 + tt, T - 1);
    scale[i] = scales[t * (ld / 64) + c0 / 64 + g];
  }
}

// acc[r] += over this wavefront's steps c in [c0, c1) of tile r: the int8
// MFMA of the step (exact integer sums over 64 k) times the activation scale
// of the lane's token for that group (g = c - gbase in the LDS block).  The
// first batch of weight loads is issued before `stage` runs (stage fills LDS
// and ends with a barrier), so their latency overlaps the staging.
template <int RT, typename Stage>
__device__ __forceinline__ void gemm_steps(const uint8_t* const (&wt)[RT], int c0, int c1, int gbase,
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
        const i32x4_t* p = reinterpret_cast<const i32x4_t*>(wt[r] + size_t(min(c + u, c1 - 1)) * 1024 + 16 * lane);
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

static_assert(in_extent(2048) <= kLdsS && in_extent(4096) <= kLdsM && in_extent(8192) <= kLdsL &&
                  mid_extent(1024) <= kLdsS && mid_extent(2048) <= kLdsM && mid_extent(4096) <= kLdsL,
              "LDS instances");

struct InArgs {
  const int8_t* xq;           // [T][E] codes of x
  const float* xs;            // [T][E / 64]
  const uint8_t* w;           // packed tiles: dense pairs (gate, up), then latent rows of [A_g; A_u]
  const float* ws;            // row scales in tile order
  float* h;                   // [T][F]
  int8_t* zq;                 // [T][2 r] codes of the latents z = [A_g; A_u] x
  float* zs;                  // [T][2 r / 64] their group scales
  int32_t T, E, F, S, pairs, lat_groups;   // pairs = (F - S) / 16; lat_groups = 2 r / 64
};

// Launch 2: work-group = (latent group j or dense pair p, block of 16 tokens).
// The latent groups come first in the grid (their work-groups carry twice a
// pair's weights) and each owns one whole activation group of z -- 64
// latents, four 16-row tiles -- so it quantises z itself (the int8 rule of
// k_ffn_quant on the same fp32 values) and no separate launch is needed.
template <int LDS>
__global__ __launch_bounds__(kThreads) void k_ffn_in(InArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  const int rs = row_stride(a.E), steps = a.E / 64;
  float* outv = reinterpret_cast<float*>(smem + code_area(block_bytes(a.E)));
  const int units = a.pairs + a.lat_groups;
  const int unit = blockIdx.x % units, t0 = 16 * (blockIdx.x / units);
  int8_t* act = reinterpret_cast<int8_t*>(smem);
  float* scale = reinterpret_cast<float*>(smem + scale_offset(a.E));
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  auto stage = [&]() {
    stage_codes(a.xq, a.xs, a.E, 0, a.E, a.T, t0, act, scale, rs);
    __syncthreads();
  };
  if (unit < a.lat_groups) {   // uniform: latent group j = unit, tiles 2 pairs + 4 j ..
    const int tile0 = 2 * a.pairs + 4 * unit;
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
    gemm_steps<4>(wt, steps * wid / kWaves, steps * (wid + 1) / kWaves, 0, acts, scs, rs, steps, acc, stage);
    reduce_tiles<4>(acc, smem, outv);
    // one wavefront per token (two tokens each): lane = latent 16 r + nn of the group
    const int r = lane >> 4, nn = lane & 15;
    for (int tt = wid; tt < 16; tt += kWaves) {
      const int t = t0 + tt;
      const float v = outv[(r * 16 + tt) * 16 + nn] * a.ws[16 * (tile0 + r) + nn];
      float m = fabsf(v);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      const float s = m / 127.0f;
      if (t < a.T) {
        const int zrow = 2 * (a.lat_groups * 32);   // codes per token: 2 r
        a.zq[size_t(t) * zrow + 64 * unit + lane] = int8_t(code(v, s));
        if (lane == 0) a.zs[size_t(t) * a.lat_groups + unit] = s;
      }
    }
    return;
  }
  const int p = unit - a.lat_groups;   // dense pair p: tiles (gate, up) = 2 p, 2 p + 1
  const int tile0 = 2 * p;
  const uint8_t* wt[2] = {a.w + size_t(tile0) * steps * 1024, a.w + size_t(tile0 + 1) * steps * 1024};
  const int8_t* acts[2] = {act, act};
  const float* scs[2] = {scale, scale};
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  gemm_steps<2>(wt, steps * wid / kWaves, steps * (wid + 1) / kWaves, 0, acts, scs, rs, steps, acc, stage);
  reduce_tiles<2>(acc, smem, outv);
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    const int tt = i >> 4, nn = i & 15, t = t0 + tt;
    if (t >= a.T) continue;
    const float v0 = outv[i] * a.ws[16 * tile0 + nn], v1 = outv[256 + i] * a.ws[16 * (tile0 + 1) + nn];
    a.h[size_t(t) * a.F + a.S + 16 * p + nn] = silu_mul(v0, v1);   // channel S + 16 p + nn
  }
}

struct MidArgs {
  const int8_t* zq;           // [T][2 r] codes of the latents
  const float* zs;            // [T][2 r / 64]
  const uint8_t* w;           // packed pairs (B_g, B_u), k = r
  const float* ws;
  float* h;                   // [T][F], channels [0, S)
  int32_t T, r, F, pairs;     // pairs = S / 16
};

// Launch 4: work-group = (low-rank pair p, block of 16 tokens); B_g reads the
// gate latents (columns [0, r) of z), B_u the up latents ([r, 2 r)).
template <int LDS>
__global__ __launch_bounds__(kThreads) void k_ffn_mid(MidArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  const int rs = row_stride(a.r), steps = a.r / 64;
  float* outv = reinterpret_cast<float*>(smem + code_area(2 * block_bytes(a.r)));
  const int unit = blockIdx.x % a.pairs, t0 = 16 * (blockIdx.x / a.pairs);   // launched only when pairs >= 1
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
  gemm_steps<2>(wt, steps * wid / kWaves, steps * (wid + 1) / kWaves, 0, acts, scs, rs, steps, acc, [&]() {
    for (int half = 0; half < 2; ++half)
      stage_codes(a.zq, a.zs, 2 * a.r, half * a.r, a.r, a.T, t0, act[half], sc[half], rs);
    __syncthreads();
  });
  reduce_tiles<2>(acc, smem, outv);
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    const int tt = i >> 4, nn = i & 15, t = t0 + tt;
    if (t < a.T)
      a.h[size_t(t) * a.F + 16 * unit + nn] =
          silu_mul(outv[i] * a.ws[16 * tile0 + nn], outv[256 + i] * a.ws[16 * (tile0 + 1) + nn]);
  }
}

struct OutArgs {
  const int8_t* hq;           // [T][Fp]
  const float* hs;            // [T][Fp / 64]
  const uint8_t* w;           // packed W_d tiles, k = Fp
  const float* ws;
  float* y;                   // [T][E] when splits == 1, else partials [splits][T][E]
  int32_t T, E, Fp, units, splits;   // units = E / (16 RT); splits = ceil(Fp / CHUNK)
};

// Launch 6: work-group = (RT tiles of 16 rows of W_d, one CHUNK of the hidden
// dimension, block of 16 tokens); its chunk of h's codes comes through LDS
// once for all RT tiles.  With several chunks each work-group writes its
// scaled partial sum, and k_ffn_sum adds them in chunk order.
template <int LDS, int CHUNK, int RT>
__global__ __launch_bounds__(kThreads) void k_ffn_out(OutArgs a) {
  static_assert(out_extent(CHUNK, RT) <= LDS && RT <= 2, "chunk exceeds LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  const int unit = blockIdx.x % a.units, split = (blockIdx.x / a.units) % a.splits;
  const int t0 = 16 * (blockIdx.x / (a.units * a.splits));
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
  gemm_steps<RT>(wt, cb + gn * wid / kWaves, cb + gn * (wid + 1) / kWaves, cb, acts, scs, rs, gn, acc, [&]() {
    stage_codes(a.hq, a.hs, a.Fp, k0, kn, a.T, t0, act, scale, rs);
    __syncthreads();
  });
  reduce_tiles<RT>(acc, smem, outv);
  float* dst = a.y + size_t(a.splits > 1 ? split : 0) * a.T * a.E;
  for (int i = threadIdx.x; i < RT * 256; i += kThreads) {
    const int r = i >> 8, tt = (i >> 4) & 15, nn = i & 15, t = t0 + tt, row = 16 * (RT * unit + r) + nn;
    if (t < a.T) dst[size_t(t) * a.E + row] = outv[i] * a.ws[row];
  }
}

// y[i] = sum over splits s = 0, 1, ... of yp[s][i] (in that order).
__global__ __launch_bounds__(256) void k_ffn_sum(const float* yp, float* y, int32_t n, int32_t splits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += yp[size_t(s) * n + i];
  y[i] = v;
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
  float* h = reinterpret_cast<float*>(ws + f.ws_h);
  int8_t* hq = reinterpret_cast<int8_t*>(ws + f.ws_hq);
  float* hs = reinterpret_cast<float*>(ws + f.ws_hs);
  const int T = n_tokens;
  const unsigned tb = unsigned((T + 15) / 16);
  auto quant_grid = [&](int Kp) { return dim3(unsigned((T * (Kp / 64) + 3) / 4)); };
  int err = 0;

  hipLaunchKernelGGL(k_ffn_quant<true>, quant_grid(f.E), dim3(256), 0, s, x, int64_t(f.E), f.E, T, f.E, xq, xs);
  if ((err = int(hipGetLastError())) != 0) return err;
  InArgs ia{xq, xs, w + f.off_w1, reinterpret_cast<const float*>(w + f.off_s1), h, zq, zs, T, f.E, f.F, f.S,
            (f.F - f.S) / 16, 2 * f.r / 64};
  if (ia.pairs + ia.lat_groups > 0) {
    const dim3 g(unsigned(ia.pairs + ia.lat_groups) * tb), b(kThreads);
    const int lds = instance_for(in_extent(f.E));   // the smallest instance that holds it
    if (lds == kLdsS) hipLaunchKernelGGL(k_ffn_in<kLdsS>, g, b, 0, s, ia);
    else if (lds == kLdsM) hipLaunchKernelGGL(k_ffn_in<kLdsM>, g, b, 0, s, ia);
    else if (lds == kLdsL) hipLaunchKernelGGL(k_ffn_in<kLdsL>, g, b, 0, s, ia);
    else return int(hipErrorInvalidConfiguration);
    if ((err = int(hipGetLastError())) != 0) return err;
  }
  if (f.S > 0) {
    MidArgs ma{zq, zs, w + f.off_w2, reinterpret_cast<const float*>(w + f.off_s2), h, T, f.r, f.F, f.S / 16};
    const dim3 g(unsigned(ma.pairs) * tb), b(kThreads);
    const int lds = instance_for(mid_extent(f.r));
    if (lds == kLdsS) hipLaunchKernelGGL(k_ffn_mid<kLdsS>, g, b, 0, s, ma);
    else if (lds == kLdsM) hipLaunchKernelGGL(k_ffn_mid<kLdsM>, g, b, 0, s, ma);
    else if (lds == kLdsL) hipLaunchKernelGGL(k_ffn_mid<kLdsL>, g, b, 0, s, ma);
    else return int(hipErrorInvalidConfiguration);
    if ((err = int(hipGetLastError())) != 0) return err;
  }
  hipLaunchKernelGGL(k_ffn_quant<false>, quant_grid(f.Fp), dim3(256), 0, s, h, int64_t(f.F), f.F, T, f.Fp, hq, hs);
  if ((err = int(hipGetLastError())) != 0) return err;
  // Chunks of 4096 (2048 for small hidden sizes); with several chunks a
  // work-group takes two row tiles, so each staged chunk of h serves 32 rows
  // of W_d (measured best on the LLaMA-7B FFN among chunks of 1, 2, 4 and 8 K
  // with one or two tiles).
  const OutShape osh = out_shape(f.Fp);
  const int chunk = osh.chunk, splits = osh.splits, rt = osh.rt;
  float* yp = reinterpret_cast<float*>(ws + f.ws_yp);
  OutArgs oa{hq, hs, w + f.off_w3, reinterpret_cast<const float*>(w + f.off_s3), splits > 1 ? yp : y, T, f.E, f.Fp,
             f.E / (16 * rt), splits};
  const dim3 g(unsigned(oa.units) * unsigned(splits) * tb), b(kThreads);
  if (chunk == 2048) hipLaunchKernelGGL((k_ffn_out<kLdsS, 2048, 1>), g, b, 0, s, oa);
  else if (rt == 1) hipLaunchKernelGGL((k_ffn_out<kLdsM, 4096, 1>), g, b, 0, s, oa);
  else hipLaunchKernelGGL((k_ffn_out<kLdsM, 4096, 2>), g, b, 0, s, oa);
  if ((err = int(hipGetLastError())) != 0) return err;
  if (splits > 1) {
    const int n = T * f.E;
    hipLaunchKernelGGL(k_ffn_sum, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, yp, y, n, splits);
  }
  return int(hipGetLastError());
}

}  // namespace lr
