// project.hip -- latent generation on the matrix cores: the per-head latents
// c^K = x A^K_h and c^V = x A^V_h of new tokens (WSVD page, "Fine-grained
// per-head SVD": each head keeps its own rank-r latent of the embedding; LASER
// page, "System implementation": latent activations are generated inside a GPU
// kernel), in fp32 from bf16 activations and factors, for the quantised append
// that follows.
//
// The factors come as W = A^T, one row of E values per latent dimension (the
// layout of a linear layer's weight), heads concatenated in the order of the
// latent vector; both MFMA operands are then contiguous 16-byte loads.  At
// decode sizes (a few dozen tokens) the product is bound by reading W once from
// HBM: 2 E bytes per latent dimension, against 2 T flops per byte.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProjWaves = 8;     // wavefronts per work-group, each on 1/8 of E
constexpr int kMaxColTiles = 4;   // 16-token column tiles per work-group

struct ProjArgs {
  const uint16_t* x;   // bf16 [T][E]
  const uint16_t* wk;  // bf16 [nk][E]
  const uint16_t* wv;  // bf16 [nv][E]
  float* ck;           // fp32 [T][nk]
  float* cv;           // fp32 [T][nv]
  int32_t T, E, nk, nv;
  int32_t k_tiles, row_tiles;     // 16-row tiles of W^K, of W^K and W^V together
  int32_t t_blocks, tb_stride;    // token blocks of 16 NT; blocks per grid column
};

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Work-group (row tile, token block): c[t][n] = sum_e x[t][e] w[n][e] for 16
// latent rows n and 16 NT tokens t, with v_mfma_f32_16x16x32_bf16 -- latent
// rows are the MFMA rows, tokens its columns.  Lane (i, g) = (lane & 15,
// lane >> 4) supplies row i of w and of each x column tile, eight consecutive
// embedding elements 8 g .. 8 g + 7 of every 32-wide step (the same elements
// on both sides, which is all the product needs), and receives rows 4 g .. 4 g
// + 3 of column i.  The eight wavefronts take contiguous eighths of the
// embedding; their partial tiles are summed through LDS in wavefront order, so
// the result is the same on every call.  Rows and tokens past the ends are
// read at the last valid row and never stored.
template <int NT>
__global__ __launch_bounds__(kProjWaves * 64) void k_project(ProjArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int li = lane & 15, lg = lane >> 4;
  const int rt = blockIdx.x % a.row_tiles;
  const bool isv = rt >= a.k_tiles;
  const int n0 = 16 * (isv ? rt - a.k_tiles : rt);
  const int N = isv ? a.nv : a.nk;
  const uint16_t* wr = (isv ? a.wv : a.wk) + size_t(min(n0 + li, N - 1)) * a.E + 8 * lg;
  float* out = isv ? a.cv : a.ck;

  const int steps = a.E >> 5, per = (steps + kProjWaves - 1) / kProjWaves;
  const int c0 = wid * per, c1 = min(steps, c0 + per);

  __shared__ f32x4_t s_red[kProjWaves][NT][64];
  for (int tb = blockIdx.x / a.row_tiles; tb < a.t_blocks; tb += a.tb_stride) {
    const int t0 = 16 * NT * tb;
    const uint16_t* xr[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xr[j] = a.x + size_t(min(t0 + 16 * j + li, a.T - 1)) * a.E + 8 * lg;

    f32x4_t acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // U steps of loads are issued before their products, so that U (NT + 1)
    // 16-byte loads per lane are in flight; the remainder goes one step at a time.
    constexpr int U = NT <= 2 ? 8 : 4;
    int c = c0;
    for (; c + U <= c1; c += U) {
      bf16x8_t av[U], bv[U][NT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        av[u] = load8(wr + 32 * (c + u));
#pragma unroll
        for (int j = 0; j < NT; ++j) bv[u][j] = load8(xr[j] + 32 * (c + u));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the products
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][j], acc[j], 0, 0, 0);
    }
    for (; c < c1; ++c) {
      const bf16x8_t av = load8(wr + 32 * c);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, load8(xr[j] + 32 * c), acc[j], 0, 0, 0);
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) s_red[wid][j][lane] = acc[j];
    __syncthreads();
    // one output per thread per pass: token tt of the block, row nn of the tile,
    // consecutive threads on consecutive rows of one token
    for (int i = tid; i < NT * 256; i += kProjWaves * 64) {
      const int tt = i >> 4, nn = i & 15;
      const int j = tt >> 4, src = (tt & 15) + 16 * (nn >> 2), e = nn & 3;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kProjWaves; ++w) v += s_red[w][j][src][e];
      const int t = t0 + tt, n = n0 + nn;
      if (t < a.T && n < N) out[size_t(t) * N + n] = v;
    }
    __syncthreads();
  }
}

}  // namespace

namespace lr {

int launch_project(const lr_attn_plan& p, int32_t layer, const void* x, int32_t n_tokens,
                   int32_t embed, const void* wk, const void* wv, float* ck, float* cv,
                   void* stream) {
  const auto& L = p.layers[layer];
  ProjArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.wk = static_cast<const uint16_t*>(wk);
  a.wv = static_cast<const uint16_t*>(wv);
  a.ck = ck;
  a.cv = cv;
  a.T = n_tokens;
  a.E = embed;
  a.nk = L.sum_rk;
  a.nv = L.sum_rv;
  a.k_tiles = (L.sum_rk + 15) / 16;
  a.row_tiles = a.k_tiles + (L.sum_rv + 15) / 16;
  const int col_tiles = (n_tokens + 15) / 16;
  const int nt = col_tiles < kMaxColTiles ? col_tiles : kMaxColTiles;
  a.t_blocks = (col_tiles + nt - 1) / nt;
  // at most 2^20 work-groups; the rest of the token blocks are looped over
  const int max_tb = (1 << 20) / a.row_tiles;
  a.tb_stride = a.t_blocks < max_tb ? a.t_blocks : max_tb;
  const dim3 grid(unsigned(a.row_tiles) * unsigned(a.tb_stride)), block(kProjWaves * 64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (nt) {
    case 1: hipLaunchKernelGGL(k_project<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_project<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_project<3>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_project<4>, grid, block, 0, s, a); break;
  }
  return int(hipGetLastError());
}

}  // namespace lr
