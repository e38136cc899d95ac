// kernels.hip -- gfx950 kernels of the low-rank latent-KV decode step.
//
//   k_append          quantise fp32 latents (int8 per token / int4 per group
//                     of 32, round half to even) and write them into the
//                     tiled cache planes.
//   k_decode          absorbed decode: q' = scale * q B^K_h^T, stream the
//                     K/V latent codes of each (b, h) once from HBM, online
//                     softmax in registers, accumulate the V latent, merge the
//                     context splits, apply B^V_h once.
//   k_ws_init         zero the split counters of a workspace.
//
// Cache tiles hold 64 tokens, one per lane of a wavefront; every lane load
// is a 16-byte chunk and a wavefront load instruction reads 1 KiB of
// contiguous memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace lr {
namespace {

constexpr float kTau = 8.0f;          // lazy rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// element I/O
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                         // round half to even
  return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {  // bf16
  static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}

// ---------------------------------------------------------------------------
// wavefront reductions with DPP (result in lane 63)
// ---------------------------------------------------------------------------

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}

// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror make
// every lane hold its 16-lane row total; row_bcast15 / row_bcast31 then fold
// the four rows into lane 63.
__device__ __forceinline__ float wave_sum63(float v) {
  v += dpp<0xb1>(v, 0.f);
  v += dpp<0x4e>(v, 0.f);
  v += dpp<0x141>(v, 0.f);
  v += dpp<0x140>(v, 0.f);
  v += dpp<0x142, 0xa>(v, 0.f);
  v += dpp<0x143, 0xc>(v, 0.f);
  return v;
}

__device__ __forceinline__ float wave_max63(float v) {
  const float ninf = -__builtin_inff();
  v = fmaxf(v, dpp<0xb1>(v, ninf));
  v = fmaxf(v, dpp<0x4e>(v, ninf));
  v = fmaxf(v, dpp<0x141>(v, ninf));
  v = fmaxf(v, dpp<0x140>(v, ninf));
  v = fmaxf(v, dpp<0x142, 0xa>(v, ninf));
  v = fmaxf(v, dpp<0x143, 0xc>(v, ninf));
  return v;
}

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// append: quantise + pack
// ---------------------------------------------------------------------------

struct AppendArgs {
  uint8_t* cache;
  const float* ck;
  const float* cv;
  const int32_t* pos;
  int32_t B, H, n_new, capacity, n_tiles, sum_rk, sum_rv;
  int64_t rows;
};

// int8: 16 values -> 16 bytes (or 8 -> 8 for a half chunk)
template <int NV>
__device__ __forceinline__ void pack_int8(const float* src, float s, uint32_t* w) {
#pragma unroll
  for (int j = 0; j < NV / 4; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(src + 4 * j);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int q = 0;
      if (s != 0.0f) q = int(fminf(fmaxf(rintf(vv[k] / s), -127.0f), 127.0f));
      word |= (uint32_t(q) & 0xffu) << (8 * k);
    }
    w[j] = word;
  }
}

// int4: NV values (8..32) of one group -> NV/2 bytes, element 2j in the low nibble
template <int NV>
__device__ __forceinline__ void pack_int4(const float* src, float s, uint32_t* w) {
#pragma unroll
  for (int j = 0; j < NV / 8; ++j) {
    const float4 a = *reinterpret_cast<const float4*>(src + 8 * j);
    const float4 b = *reinterpret_cast<const float4*>(src + 8 * j + 4);
    const float vv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int q = 0;
      if (s != 0.0f) q = int(fminf(fmaxf(rintf(vv[k] / s), -7.0f), 7.0f));
      word |= (uint32_t(q) & 0xfu) << (4 * k);
    }
    w[j] = word;
  }
}

template <int NV>
__device__ __forceinline__ float absmax(const float* src, float m) {
#pragma unroll
  for (int j = 0; j < NV / 4; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(src + 4 * j);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  return m;
}

template <int QF>
__global__ __launch_bounds__(256) void k_append(AppendArgs a, HeadTab ht) {
  int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= a.rows) return;
  // row order: (kv, h, b, j) with j fastest so neighbouring threads write
  // neighbouring token slots of one plane
  const int j = int(idx % a.n_new);
  idx /= a.n_new;
  const int b = int(idx % a.B);
  idx /= a.B;
  const int h = int(idx % a.H);
  const int kv = int(idx / a.H);
  const int slot = a.pos[b] + j;
  if (slot < 0 || slot >= a.capacity) return;
  const uint32_t rr = ht.ranks[h], lo = ht.loff[h];
  const int r = int(kv ? rr >> 16 : rr & 0xffffu);
  const int sum_r = kv ? a.sum_rv : a.sum_rk;
  const float* src = (kv ? a.cv : a.ck) + (int64_t(b) * a.n_new + j) * sum_r + int(kv ? lo >> 16 : lo & 0xffffu);
  const int rb = row_bytes(QF, r);
  const int tb = tile_bytes(QF, r);
  uint8_t* tile = a.cache + uint64_t(kv ? ht.vreg[h] : ht.kreg[h]) * kRegionAlign +
                  (uint64_t(b) * a.n_tiles + (slot >> 6)) * tb;
  const int lane = slot & 63;

  if constexpr (QF == LR_Q_INT8_TOKEN) {
    float m = 0.0f;
    for (int c = 0; c < r; c += 8) m = absmax<8>(src + c, m);
    const float s = m / 127.0f;
    *reinterpret_cast<float*>(tile + 64 * rb + 4 * lane) = s;
    for (int c = 0; 16 * c < r; ++c) {
      uint32_t w[4];
      if (16 * c + 16 <= r) {
        pack_int8<16>(src + 16 * c, s, w);
        *reinterpret_cast<uint4*>(tile + 1024 * c + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        pack_int8<8>(src + 16 * c, s, w);
        *reinterpret_cast<uint2*>(tile + 1024 * c + 8 * lane) = make_uint2(w[0], w[1]);
      }
    }
  } else {
    for (int g = 0; 32 * g < r; ++g) {
      const int nv = min(32, r - 32 * g);
      const float* gs = src + 32 * g;
      float m = 0.0f;
      for (int c = 0; c < nv; c += 8) m = absmax<8>(gs + c, m);
      const _Float16 sh = _Float16(m / 7.0f);
      const float s = float(sh);
      *reinterpret_cast<uint16_t*>(tile + 64 * rb + 2 * (64 * g + lane)) = __builtin_bit_cast(uint16_t, sh);
      uint32_t w[4];
      uint8_t* dst = tile + 1024 * g;
      if (nv == 32) {
        pack_int4<32>(gs, s, w);
        *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
      } else if (nv == 24) {
        pack_int4<24>(gs, s, w);
        *reinterpret_cast<uint3*>(dst + 12 * lane) = make_uint3(w[0], w[1], w[2]);
      } else if (nv == 16) {
        pack_int4<16>(gs, s, w);
        *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(w[0], w[1]);
      } else {
        pack_int4<8>(gs, s, w);
        *reinterpret_cast<uint32_t*>(dst + 4 * lane) = w[0];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode (absorbed form)
// ---------------------------------------------------------------------------

struct DecodeArgs {
  const uint8_t* cache;
  const int32_t* len;
  const void* q;
  const void* bk;
  const void* bv;
  void* out;
  float* part;       // workspace partials [B*H][n_split][kPartStride]
  int32_t* cnt;      // workspace counters [B*H]
  float qscale;      // softmax scale * log2(e)
  int32_t B, H, n_tiles, max_len, n_split, tps;
};

// Codes of one 64-token tile for this lane: NC chunks of 16 bytes.  The
// runtime row width rb (bytes) may end inside the bucket; missing chunks are
// zero and the tail chunk may be 4, 8 or 12 bytes wide.
template <int NC>
__device__ __forceinline__ void load_codes(const uint8_t* tile, int lane, int rb, uint32_t* w) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int wc = rb - 16 * c;
    const uint8_t* p = tile + 1024 * c;
    if (wc >= 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 16 * lane);
      w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
    } else if (wc == 12) {
      const uint3 v = *reinterpret_cast<const uint3*>(p + 12 * lane);
      w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = 0;
    } else if (wc == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + 8 * lane);
      w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = 0; w[4 * c + 3] = 0;
    } else if (wc == 4) {
      w[4 * c] = *reinterpret_cast<const uint32_t*>(p + 4 * lane);
      w[4 * c + 1] = 0; w[4 * c + 2] = 0; w[4 * c + 3] = 0;
    } else {
      w[4 * c] = 0; w[4 * c + 1] = 0; w[4 * c + 2] = 0; w[4 * c + 3] = 0;
    }
  }
}

__device__ __forceinline__ float i8(uint32_t w, int k) { return float(int8_t(w >> (8 * k))); }
__device__ __forceinline__ float i4(uint32_t w, int k) { return float(int32_t(w << (28 - 4 * k)) >> 28); }

// sum_k qp[k] * code_k over one chunk (16 int8 or 32 int4 values)
template <int QF>
__device__ __forceinline__ float dot_chunk(const uint32_t* w, const float* qp) {
  float acc = 0.0f;
  if constexpr (QF == LR_Q_INT8_TOKEN) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc = fmaf(qp[k], i8(w[k >> 2], k & 3), acc);
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) acc = fmaf(qp[k], i4(w[k >> 3], k & 7), acc);
  }
  return acc;
}

template <int QF>
__device__ __forceinline__ void acc_chunk(float* u, const uint32_t* w, float wt) {
  if constexpr (QF == LR_Q_INT8_TOKEN) {
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = fmaf(wt, i8(w[k >> 2], k & 3), u[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) u[k] = fmaf(wt, i4(w[k >> 3], k & 7), u[k]);
  }
}

template <int QF, typename IOT, int R, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode(DecodeArgs a, HeadTab ht) {
  constexpr int VPC = QF == LR_Q_INT8_TOKEN ? 16 : 32;  // values per 16-byte chunk
  constexpr int NC = R / VPC;                            // chunks per row in the bucket
  constexpr int NG = QF == LR_Q_INT8_TOKEN ? 1 : NC;     // scales per token
  using E = Elem<IOT>;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  int idx = blockIdx.x;
  const int split = idx % a.n_split;
  idx /= a.n_split;
  const int b = idx % a.B;
  const int h = uniform_i(int(ht.order[idx / a.B]));
  const uint32_t rr = uniform_i(int(ht.ranks[h])), lo = uniform_i(int(ht.loff[h]));
  const int rk = int(rr & 0xffffu), rv = int(rr >> 16);
  const int loff_k = int(lo & 0xffffu), loff_v = int(lo >> 16);
  const uint32_t kreg = uniform_i(int(ht.kreg[h])), vreg = uniform_i(int(ht.vreg[h]));
  const int rbk = row_bytes(QF, rk), rbv = row_bytes(QF, rv);
  const int tbk = tile_bytes(QF, rk), tbv = tile_bytes(QF, rv);
  const int len = min(max(a.len[b], 0), a.max_len);
  const int ntiles = (len + 63) >> 6;
  const int n_live = max(1, (ntiles + a.tps - 1) / a.tps);
  if (split >= n_live) return;
  const int t0 = split * a.tps, t1 = min(ntiles, t0 + a.tps);
  const int unit = b * a.H + h;

  __shared__ float s_q[R];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_u[NW][R];
  __shared__ int s_last;

  // ---- q'_i = scale * log2(e) * sum_j q_j B^K_h[i][j]  (one wavefront per i)
  {
    const IOT* qrow = reinterpret_cast<const IOT*>(a.q) + size_t(unit) * kHeadDim;
    const float q0 = E::ld(qrow, 2 * lane), q1 = E::ld(qrow, 2 * lane + 1);
    const IOT* bkh = reinterpret_cast<const IOT*>(a.bk) + size_t(loff_k) * kHeadDim;
    for (int i = wid; i < R; i += NW) {
      float v = 0.0f;
      if (i < rk) {
        v = q0 * E::ld(bkh, size_t(i) * kHeadDim + 2 * lane);
        v = fmaf(q1, E::ld(bkh, size_t(i) * kHeadDim + 2 * lane + 1), v);
        v = wave_sum63(v);
      }
      if (lane == 63) s_q[i] = v * a.qscale;
    }
  }
  __syncthreads();
  float qp[R];
#pragma unroll
  for (int i = 0; i < R; ++i) qp[i] = uniform(s_q[i]);

  // ---- stream this split's tiles: one token per lane, online softmax
  const uint8_t* kplane = a.cache + uint64_t(kreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbk;
  const uint8_t* vplane = a.cache + uint64_t(vreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbv;
  float m = -__builtin_inff(), l = 0.0f;
  float u[R];
#pragma unroll
  for (int i = 0; i < R; ++i) u[i] = 0.0f;

  for (int t = t0 + wid; t < t1; t += NW) {
    const uint8_t* kt = kplane + size_t(t) * tbk;
    const uint8_t* vt = vplane + size_t(t) * tbv;
    const bool valid = t * 64 + lane < len;
    uint32_t kw[4 * NC], vw[4 * NC];
    load_codes<NC>(kt, lane, rbk, kw);
    load_codes<NC>(vt, lane, rbv, vw);
    float sk[NG], sv[NG];
    if constexpr (QF == LR_Q_INT8_TOKEN) {
      sk[0] = *reinterpret_cast<const float*>(kt + 64 * rbk + 4 * lane);
      sv[0] = *reinterpret_cast<const float*>(vt + 64 * rbv + 4 * lane);
    } else {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sk[g] = 32 * g < rk ? half_bits_to_f32(*reinterpret_cast<const uint16_t*>(kt + 64 * rbk + 2 * (64 * g + lane))) : 0.0f;
        sv[g] = 32 * g < rv ? half_bits_to_f32(*reinterpret_cast<const uint16_t*>(vt + 64 * rbv + 2 * (64 * g + lane))) : 0.0f;
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c * VPC < rk) {
        const float part = dot_chunk<QF>(kw + 4 * c, qp + c * VPC);
        if constexpr (QF == LR_Q_INT8_TOKEN) s += part;
        else s = fmaf(sk[c], part, s);
      }
    }
    if constexpr (QF == LR_Q_INT8_TOKEN) s *= sk[0];
    s = valid ? s : -__builtin_inff();
    if (s > m + kTau) {  // rare after the first tile: rescale the running sums
      const float al = __builtin_amdgcn_exp2f(m - s);
      l *= al;
#pragma unroll
      for (int i = 0; i < R; ++i) u[i] *= al;
      m = s;
    }
    const float p = valid ? __builtin_amdgcn_exp2f(s - m) : 0.0f;
    l += p;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c * VPC < rv) {
        const float wt = valid ? p * sv[QF == LR_Q_INT8_TOKEN ? 0 : c] : 0.0f;
        acc_chunk<QF>(u + c * VPC, vw + 4 * c, wt);
      }
    }
  }

  // ---- merge the 64 lanes, then the NW wavefronts
  {
    const float M = lane63(wave_max63(m));
    const float f = (m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    const float lw = wave_sum63(l * f);
    if (lane == 63) { s_m[wid] = M; s_l[wid] = lw; }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (i < rv) {
        const float ui = wave_sum63(u[i] * f);
        if (lane == 63) s_u[wid][i] = ui;
      }
    }
  }
  __syncthreads();
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w]);
  float fw[NW];
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    fw[w] = (s_m[w] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w] - M);
    L = fmaf(fw[w], s_l[w], L);
  }
  float ui = 0.0f;
  if (tid < rv) {
#pragma unroll
    for (int w = 0; w < NW; ++w) ui = fmaf(fw[w], s_u[w][tid], ui);
  }

  if (n_live > 1) {
    // ---- publish this split's partial; the last split of (b, h) merges all
    float* part = a.part + (size_t(unit) * a.n_split + split) * kPartStride;
    if (tid == 0) { part[0] = M; part[1] = L; }
    if (tid < rv) part[2 + tid] = ui;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(a.cnt + unit, 1) == n_live - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* pu = a.part + size_t(unit) * a.n_split * kPartStride;
    M = -__builtin_inff();
    for (int s2 = 0; s2 < n_live; ++s2) M = fmaxf(M, pu[size_t(s2) * kPartStride]);
    L = 0.0f;
    ui = 0.0f;
    for (int s2 = 0; s2 < n_live; ++s2) {
      const float* ps = pu + size_t(s2) * kPartStride;
      const float fs = __builtin_amdgcn_exp2f(ps[0] - M);  // every live split saw a token
      L = fmaf(fs, ps[1], L);
      if (tid < rv) ui = fmaf(fs, ps[2 + tid], ui);
    }
    if (tid == 0) a.cnt[unit] = 0;  // leave the counter ready for the next call
  }

  // ---- o = (u / l) B^V_h
  __syncthreads();
  if (tid < rv) s_u[0][tid] = (L > 0.0f) ? ui / L : 0.0f;
  __syncthreads();
  const IOT* bvh = reinterpret_cast<const IOT*>(a.bv) + size_t(loff_v) * kHeadDim;
  IOT* o = reinterpret_cast<IOT*>(a.out) + size_t(unit) * kHeadDim;
  for (int j = tid; j < kHeadDim; j += NW * 64) {
    float acc = 0.0f;
    for (int i = 0; i < rv; ++i) acc = fmaf(s_u[0][i], E::ld(bvh, size_t(i) * kHeadDim + j), acc);
    E::st(o, j, acc);
  }
}

__global__ void k_ws_init(uint32_t* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int rank_bucket(int r) { return r <= 32 ? 32 : r <= 64 ? 64 : r <= 96 ? 96 : 128; }

template <int QF, typename IOT, int R>
hipError_t launch_decode_t(dim3 grid, hipStream_t st, const DecodeArgs& a, const HeadTab& t) {
  hipLaunchKernelGGL((k_decode<QF, IOT, R, 4>), grid, dim3(256), 0, st, a, t);
  return hipGetLastError();
}

template <int QF, typename IOT>
hipError_t dispatch_rank(int bucket, dim3 grid, hipStream_t st, const DecodeArgs& a, const HeadTab& t) {
  switch (bucket) {
    case 32: return launch_decode_t<QF, IOT, 32>(grid, st, a, t);
    case 64: return launch_decode_t<QF, IOT, 64>(grid, st, a, t);
    case 96: return launch_decode_t<QF, IOT, 96>(grid, st, a, t);
    default: return launch_decode_t<QF, IOT, 128>(grid, st, a, t);
  }
}

}  // namespace

int launch_append(const lr_attn_plan& p, int32_t layer, void* cache, const float* ck,
                  const float* cv, const int32_t* pos, int32_t n_new, void* stream) {
  const auto& L = p.layers[layer];
  AppendArgs a;
  a.cache = static_cast<uint8_t*>(cache);
  a.ck = ck;
  a.cv = cv;
  a.pos = pos;
  a.B = p.desc.batch;
  a.H = p.desc.n_heads;
  a.n_new = n_new;
  a.capacity = p.desc.capacity;
  a.n_tiles = p.n_tiles;
  a.sum_rk = L.sum_rk;
  a.sum_rv = L.sum_rv;
  a.rows = int64_t(2) * a.H * a.B * n_new;
  const dim3 grid(unsigned((a.rows + 255) / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.desc.qfmt == LR_Q_INT8_TOKEN)
    hipLaunchKernelGGL(k_append<LR_Q_INT8_TOKEN>, grid, dim3(256), 0, st, a, L.tab);
  else
    hipLaunchKernelGGL(k_append<LR_Q_INT4_G32>, grid, dim3(256), 0, st, a, L.tab);
  return int(hipGetLastError());
}

int launch_decode(const lr_attn_plan& p, int32_t layer, const void* cache, const int32_t* len,
                  int32_t max_len, const void* q, const void* bk, const void* bv, float scale,
                  void* out, void* workspace, void* stream, bool explicit_form) {
  if (explicit_form) return int(hipErrorNotSupported);
  const auto& L = p.layers[layer];
  const Split sp = choose_split(p, max_len);
  DecodeArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.len = len;
  a.q = q;
  a.bk = bk;
  a.bv = bv;
  a.out = out;
  const size_t units = size_t(p.desc.batch) * p.desc.n_heads;
  a.cnt = static_cast<int32_t*>(workspace);
  a.part = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + (units * 4 + 255) / 256 * 256)
                     : nullptr;
  a.qscale = scale * kLog2e;
  a.B = p.desc.batch;
  a.H = p.desc.n_heads;
  a.n_tiles = p.n_tiles;
  a.max_len = max_len;
  a.n_split = sp.n_split;
  a.tps = sp.tiles_per_split;
  const dim3 grid(unsigned(units * sp.n_split));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int bucket = rank_bucket(L.rk_max > L.rv_max ? L.rk_max : L.rv_max);
  hipError_t e;
  if (p.desc.qfmt == LR_Q_INT8_TOKEN) {
    e = p.desc.io_dtype == LR_DT_BF16 ? dispatch_rank<LR_Q_INT8_TOKEN, uint16_t>(bucket, grid, st, a, L.tab)
                                      : dispatch_rank<LR_Q_INT8_TOKEN, float>(bucket, grid, st, a, L.tab);
  } else {
    e = p.desc.io_dtype == LR_DT_BF16 ? dispatch_rank<LR_Q_INT4_G32, uint16_t>(bucket, grid, st, a, L.tab)
                                      : dispatch_rank<LR_Q_INT4_G32, float>(bucket, grid, st, a, L.tab);
  }
  return int(e);
}

int launch_workspace_init(void* workspace, size_t bytes, void* stream) {
  const int64_t n = int64_t(bytes / 4);
  hipLaunchKernelGGL(k_ws_init, dim3(unsigned((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace), n);
  return int(hipGetLastError());
}

}  // namespace lr
