// kernels.hip -- gfx950 kernels of the low-rank latent-KV decode step.
//
//   k_append          quantise fp32 latents (int8 per token / int4 per group
//                     of 32, round half to even) and write them into the
//                     tiled cache planes.
//   k_decode          absorbed decode: q' = scale * q B^K_h^T, stream the
//                     K/V latent codes of each (b, h) once from HBM, online
//                     softmax in registers, accumulate the V latent, merge the
//                     context splits, apply B^V_h once.
//   k_merge           merge the context-split partials of each (b, h) and
//                     apply B^V_h (only when a launch splits the context).
//
// Cache tiles hold 64 tokens, one per lane of a wavefront; every lane load
// is a 16-byte chunk and a wavefront load instruction reads 1 KiB of
// contiguous memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "check.h"
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

// Sum over the 64 lanes of 32 values per lane, transposed: each step pairs
// lanes across one lane bit, every lane keeps half of its values and adds
// its partner's copy of that half, so 32 values cost 31 adds plus the moves.
// Bits 5 and 4 use the gfx950 half-wave swaps, bits 3, 1, 0 DPP with
// selects, and a last DPP add folds bit 2.  Afterwards lane l with
// (l & 4) == 0 holds the total of value (l & 3) | ((l >> 1) & 0x1c).
// (Both swap results are read into unsigned locals first: bit-casting the
// second element of the returned pair directly is miscompiled to a second
// read of the first.)
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return __uint_as_float(r0) + __uint_as_float(r1);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return __uint_as_float(r0) + __uint_as_float(r1);
}
// The same over each 32-lane half separately, 16 values per lane (bit 5 is
// not reduced): lane l with (l & 4) == 0 holds its half's total of value
// (l & 3) | ((l >> 1) & 0xc).
__device__ __forceinline__ float half_sum16_transposed(float* x, int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = swap_sum16(x[k], x[k + 8]);       // keeps k + 8 bit4
  {
    const bool hi = lane & 8;                                            // row_ror:8 = lane ^ 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float send = hi ? x[k] : x[k + 4], keep = hi ? x[k + 4] : x[k];
      x[k] = keep + dpp<0x128>(send, 0.0f);
    }
  }
  {
    const bool hi = lane & 2;                                            // quad_perm [2,3,0,1]
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float send = hi ? x[k] : x[k + 2], keep = hi ? x[k + 2] : x[k];
      x[k] = keep + dpp<0x4e>(send, 0.0f);
    }
  }
  {
    const bool hi = lane & 1;                                            // quad_perm [1,0,3,2]
    const float send = hi ? x[0] : x[1], keep = hi ? x[1] : x[0];
    x[0] = keep + dpp<0xb1>(send, 0.0f);
  }
  return x[0] + dpp<0x12c>(x[0], 0.0f);                                  // row_ror:12 reads lane i + 4
}
__device__ __forceinline__ float wave_sum32_transposed(float* x, int lane) {
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = swap_sum32(x[k], x[k + 16]);     // keeps k + 16 bit5
  return half_sum16_transposed(x, lane);
}
__device__ __forceinline__ int transposed_index(int lane) { return (lane & 3) | ((lane >> 1) & 0x1c); }

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A zero the compiler cannot see through: an address offset by it cannot be
// hoisted out of a loop, so loop-invariant LDS reads stay where they are used
// instead of occupying registers for the whole loop.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// append: quantise + pack
// ---------------------------------------------------------------------------

struct AppendArgs {
  uint8_t* cache;
  uint64_t cache_bytes;
  const float* ck;
  const float* cv;
  const int32_t* pos;
  int32_t B, H, n_new, capacity, n_tiles, sum_rk, sum_rv;
  int64_t rows;
};

// max over the 16 lanes of a DPP row (every lane receives the result)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xb1>(v, 0.f));
  v = fmaxf(v, dpp<0x4e>(v, 0.f));
  v = fmaxf(v, dpp<0x141>(v, 0.f));
  v = fmaxf(v, dpp<0x140>(v, 0.f));
  return v;
}
// max over the 4 lanes of a quad
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp<0xb1>(v, 0.f));
  v = fmaxf(v, dpp<0x4e>(v, 0.f));
  return v;
}

// One lane's segment of a latent row: 8 values quantised round-half-even
// against the row's (int8) or its group's (int4) absmax scale.  The absmax is
// reduced with DPP inside the 16-lane row (int8) or the quad that holds one
// group of 32 ranks (int4), so every lane of those rows must take part.
struct SegCodes {
  uint32_t w[2];   // int8: 8 bytes; int4: 8 nibbles in w[0]
  float s;         // the scale as stored (int4: fp16 widened)
  uint16_t sh;     // int4: the fp16 scale bits
};

template <int QF>
__device__ __forceinline__ SegCodes quantise_seg(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  m = QF == LR_Q_INT8_TOKEN ? row16_max(m) : quad_max(m);
  SegCodes c;
  c.w[0] = 0u;
  c.w[1] = 0u;
  c.sh = 0;
  if constexpr (QF == LR_Q_INT8_TOKEN) {
    c.s = m / 127.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = c.s != 0.0f ? int(fminf(fmaxf(rintf(v[k] / c.s), -127.0f), 127.0f)) : 0;
      c.w[k >> 2] |= (uint32_t(q) & 0xffu) << (8 * (k & 3));
    }
  } else {
    const _Float16 sh = _Float16(m / 7.0f);
    c.s = float(sh);
    c.sh = __builtin_bit_cast(uint16_t, sh);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = c.s != 0.0f ? int(fminf(fmaxf(rintf(v[k] / c.s), -7.0f), 7.0f)) : 0;
      c.w[0] |= (uint32_t(q) & 0xfu) << (4 * k);
    }
  }
  return c;
}

// Store one lane's quantised segment (seg = lane within its 16-lane row) at
// token slot t of its tile; rb = the row's code bytes.
template <int QF>
__device__ __forceinline__ void store_seg(const Bounds& bd, uint8_t* tile, int rb, int t, int seg, const SegCodes& c) {
  if constexpr (QF == LR_Q_INT8_TOKEN) {
    const int ch = seg >> 1;                      // 16-byte chunk of this lane's 8 bytes
    const int wc = min(16, rb - 16 * ch);         // chunk width: 16, or 8 for the tail
    *checked(bd, reinterpret_cast<uint2*>(tile + 1024 * ch + wc * t + 8 * (seg & 1)), 8) = make_uint2(c.w[0], c.w[1]);
    if (seg == 0) *checked(bd, reinterpret_cast<float*>(tile + 64 * rb + 4 * t), 4) = c.s;
  } else {
    const int g = seg >> 2;                       // group of 32 ranks == 16-byte chunk
    const int wc = min(16, rb - 16 * g);          // 16, or 4, 8, 12 for the tail group
    *checked(bd, reinterpret_cast<uint32_t*>(tile + 1024 * g + wc * t + 4 * (seg & 3)), 4) = c.w[0];
    if ((seg & 3) == 0) *checked(bd, reinterpret_cast<uint16_t*>(tile + 64 * rb + 2 * (64 * g + t)), 2) = c.sh;
  }
}

// One latent row (one token, one head, K or V) per 16 lanes; lane s of the row
// owns values [8s, 8s + 8), so a row of rank r uses r/8 lanes.
template <int QF>
__global__ __launch_bounds__(256) void k_append(AppendArgs a, HeadTab ht) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int seg = threadIdx.x & 15;
  int64_t idx = gid >> 4;                 // row: (kv, h, b, j), j fastest
  const bool row_ok = idx < a.rows;
  if (!row_ok) idx = 0;                   // keep the lanes of a row together for DPP
  const int j = int(idx % a.n_new);
  idx /= a.n_new;
  const int b = int(idx % a.B);
  idx /= a.B;
  const int h = int(idx % a.H);
  const int kv = int(idx / a.H);
  const uint32_t rr = ht.ranks[h], lo = ht.loff[h];
  const int r = int(kv ? rr >> 16 : rr & 0xffffu);
  const int slot = a.pos[b] + j;
  const bool active = row_ok && 8 * seg < r && slot >= 0 && slot < a.capacity;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int sum_r = kv ? a.sum_rv : a.sum_rk;
    const float* src = (kv ? a.cv : a.ck) + (int64_t(b) * a.n_new + j) * sum_r +
                       int(kv ? lo >> 16 : lo & 0xffffu) + 8 * seg;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  }
  const SegCodes c = quantise_seg<QF>(v);
  if (!active) return;
  uint8_t* tile = a.cache + uint64_t(kv ? ht.vreg[h] : ht.kreg[h]) * kRegionAlign +
                  (uint64_t(b) * a.n_tiles + (slot >> 6)) * tile_bytes(QF, r);
  store_seg<QF>(Bounds{a.cache, a.cache_bytes}, tile, row_bytes(QF, r), slot & 63, seg, c);
}

// ---------------------------------------------------------------------------
// decode (absorbed form)
// ---------------------------------------------------------------------------

struct DecodeArgs {
  const uint8_t* cache;
  uint64_t cache_bytes;   // the cache buffer's bytes (cache and wcache are the same buffer)
  const int32_t* len;
  const void* q;
  const void* bk;
  const void* bv;
  void* out;
  float* part;       // workspace partials [B*H][n_split][kPartStride] (split launches only)
  float qscale;      // softmax scale * log2(e)
  int32_t B, H, n_tiles, max_len, n_split, tps;
  // 1: keep each head's work-groups on one XCD (see unit_of); 0: plain order
  int32_t xcd_groups;
  // fused append (ck == nullptr: none): quantise and write one token per
  // sequence at slot pos[b] before attending; its latents are the sum, in
  // block order, of n_parts blocks [B][sum_r] of ck (cv)
  uint8_t* wcache;
  const float* ck;
  const float* cv;
  const int32_t* pos;
  int32_t capacity, sum_rk, sum_rv, n_parts;
};

// Sequence b and head h of work-group (unit) idx.  Work-group i runs on XCD
// i % 8, each XCD with its own L2.  With xcd_groups, the B work-groups of one
// head all land on one XCD (heads dealt to the XCDs by xorder), so each L2
// fetches only its own heads' factors; otherwise (b, h) in dispatch order.
__device__ __forceinline__ void unit_of(const DecodeArgs& a, const HeadTab& ht, int idx, int& b, int& h) {
  int hp;
  if (a.xcd_groups) {
    const int x = idx & 7, k = idx >> 3;
    hp = (k / a.B) * 8 + x;
    b = k % a.B;
  } else {
    b = idx % a.B;
    hp = idx / a.B;
  }
  h = uniform_i(int(a.xcd_groups ? ht.xorder[hp] : ht.order[hp]));
}

// Codes of one 64-token tile for this lane: NC chunks of 16 bytes.  The
// runtime row width rb (bytes) may end inside the bucket.  Every load is
// issued unconditionally at an in-bounds address, so that no load sits under a
// branch: a conditional load makes the compiler merge old and new register
// values at the loop latch and wait there for every load in flight.  A tail
// chunk (4, 8 or 12 bytes per lane) is read 16 bytes wide: the extra words are
// neighbouring lanes' codes, or the tile's scales for the last lane; a chunk
// past the row reads the tile's first bytes.  Those codes are finite and only
// meet q' entries that are zero (K) or accumulators that are never read (V).
// With lm = 2 lanes per token, lane half hf takes the row's chunks hf,
// hf + 2, hf + 4, ... (NC of them) of token `tok`; with lm = 1 chunks 0..NC-1.
#ifndef LR_DECODE_NT_LOADS
#define LR_DECODE_NT_LOADS 1
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Cache bytes are read once per launch: non-temporal loads (the cache
// policy's streaming hint) let them pass through the caches without
// displacing what is reused.
__device__ __forceinline__ u32x4_t ld_stream16(const uint8_t* p) {
  if constexpr (LR_DECODE_NT_LOADS) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else return *reinterpret_cast<const u32x4_t*>(p);
}
template <typename T>
__device__ __forceinline__ T ld_stream(const uint8_t* p) {
  if constexpr (LR_DECODE_NT_LOADS) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

template <int NC>
__device__ __forceinline__ void load_codes(const Bounds& bd, const uint8_t* tile, int tok, int lm, int hf, int rb,
                                           uint32_t* w) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int cg = lm * c + hf;
    const int wc = rb - 16 * cg;
    const int off = wc > 0 ? 1024 * cg + min(wc, 16) * tok : 0;
    const u32x4_t v = ld_stream16(checked(bd, tile + off, 16));
    w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
  }
}

__device__ __forceinline__ float i8(uint32_t w, int k) { return float(int8_t(w >> (8 * k))); }
__device__ __forceinline__ float i4(uint32_t w, int k) { return float(int32_t(w << (28 - 4 * k)) >> 28); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

// Eight two's-complement nibbles -> four packed fp16 pairs of exact codes.
// (w & m) ^ k with k = 0x6408 / 0x6480 per half puts 1024 + (n ^ 8) = 1032 + c
// (or 1024 + 16 (c + 8)) in each fp16 half, and one packed add removes the
// bias.  Pairs: (c0, c4), (16 c1, 16 c5), (c2, c6), (16 c3, 16 c7).
__device__ __forceinline__ void nibbles_to_h2(uint32_t w, half2_t* o) {
  const uint32_t w8 = w >> 8;
  const half2_t b1 = {_Float16(-1032.0f), _Float16(-1032.0f)};
  const half2_t b16 = {_Float16(-1152.0f), _Float16(-1152.0f)};
  o[0] = as_h2((w & 0x000F000Fu) ^ 0x64086408u) + b1;
  o[1] = as_h2((w & 0x00F000F0u) ^ 0x64806480u) + b16;
  o[2] = as_h2((w8 & 0x000F000Fu) ^ 0x64086408u) + b1;
  o[3] = as_h2((w8 & 0x00F000F0u) ^ 0x64806480u) + b16;
}

// Everything one lane needs from one 64-token tile: its token's K and V codes
// and scales.
template <int NC, int NG>
struct TileRegs {
  uint32_t kw[4 * NC], vw[4 * NC];
  float sk[NG], sv[NG];
};

// Groups past the row (int4) re-read the last group's scale: it only
// multiplies partial sums over zero q' entries or unread accumulators.
template <int QF, int NC, int NG>
__device__ __forceinline__ void load_k(const Bounds& bd, const uint8_t* kt, int tok, int lm, int hf, int rk, int rbk,
                                       TileRegs<NC, NG>& x) {
  load_codes<NC>(bd, kt, tok, lm, hf, rbk, x.kw);
  if constexpr (QF == LR_Q_INT8_TOKEN) {
    x.sk[0] = ld_stream<float>(checked(bd, kt + 64 * rbk + 4 * tok, 4));
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
      x.sk[g] = half_bits_to_f32(
          ld_stream<uint16_t>(checked(bd, kt + 64 * rbk + 2 * (64 * min(g, (rk - 1) >> 5) + tok), 2)));
  }
}

template <int QF, int NC, int NG>
__device__ __forceinline__ void load_v(const Bounds& bd, const uint8_t* vt, int tok, int lm, int hf, int rv, int rbv,
                                       TileRegs<NC, NG>& x) {
  load_codes<NC>(bd, vt, tok, lm, hf, rbv, x.vw);
  if constexpr (QF == LR_Q_INT8_TOKEN) {
    x.sv[0] = ld_stream<float>(checked(bd, vt + 64 * rbv + 4 * tok, 4));
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
      x.sv[g] = half_bits_to_f32(
          ld_stream<uint16_t>(checked(bd, vt + 64 * rbv + 2 * (64 * min(g, (rv - 1) >> 5) + tok), 2)));
  }
}

// The absorbed query q' as 32-bit words: fp32 values, or (packed int4 path)
// fp16 pairs in the order nibbles_to_h2 produces.  Small operands live in
// scalar registers (uniform across the wavefront); large ones are read from
// LDS with broadcast loads where they are used.
template <int QW, bool IN_REGS>
struct QOperand {
  uint32_t r[IN_REGS ? QW : 1];
  const uint32_t* lds;
  __device__ __forceinline__ uint32_t word(int i) const {
    if constexpr (IN_REGS) return r[i];
    else return lds[i];
  }
  __device__ __forceinline__ float f(int i) const { return __uint_as_float(word(i)); }
};

// One work-group per (b, h, split).  NW wavefronts take the split's steps
// round-robin: a step is one 64-token tile with one token per lane, or (two
// lanes per token, below) half a tile.  Without context splitting the group
// finishes the output itself; with it, the group writes its partial (m, l, u)
// and k_merge combines them.
//
// int8 codes: the score is sum_i q'_i c_i (one SDWA convert + one FMA per
// value), the V latent u_i += w c_i.  int4 codes with bf16 I/O: codes become
// exact fp16 pairs (nibbles_to_h2), scores use 2-way fp16 dot products with
// fp32 accumulation against q' rounded to fp16, and u accumulates with mixed
// fp16 x fp32 FMAs.  int4 with fp32 I/O keeps q' in fp32 (bit-field extract +
// convert + FMA) so it can be held to the tighter tolerance.
//
// LPT = 2 (int8, ranks above 64): two lanes share a token, each holding
// every other 16-byte chunk of its row and half of the V accumulators; the
// two partial scores meet with one half-wave swap, so both lanes run the same
// softmax.  A wavefront then takes 32 tokens per step with half the
// registers, which doubles the wavefronts a compute unit can hold.  A head
// whose rows fit in half of the bucket keeps one lane per token in the same
// registers (64 tokens, twice the bytes per step: light heads are bound by
// the bytes each wavefront has in flight).  The choice is per work-group.
//
// Waves per SIMD the register allocation must allow (decode_waves_per_simd:
// enough bytes in flight per CU to cover HBM latency without spilling).
template <int QF, int R, int LPT>
constexpr int decode_occupancy() {
  static_assert(LPT == (pair_lanes(QF, R) ? 2 : 1), "lanes per token follow the bucket");
  return decode_waves_per_simd(QF, R);
}

template <int QF, typename IOT, int R, int NW, int LPT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(decode_occupancy<QF, R, LPT>(), decode_occupancy<QF, R, LPT>())))
void k_decode(DecodeArgs a, HeadTab ht) {
  constexpr bool INT8 = QF == LR_Q_INT8_TOKEN;
  constexpr bool PACKED = !INT8 && sizeof(IOT) == 2;
  // bf16 I/O: K scores as integer dot products of the codes against q' held
  // as NLV integer levels of the codes' width -- two int8 levels against int8
  // codes (v_dot4: 4 codes per instruction), four int4 levels against int4
  // codes (v_dot8: 8 codes per instruction).  fp32 I/O keeps fp32 q'.
#ifndef LR_DECODE_DOT4
#define LR_DECODE_DOT4 1
#endif
#ifndef LR_DECODE_DOT8
#define LR_DECODE_DOT8 1
#endif
  constexpr bool DOT = (INT8 ? LR_DECODE_DOT4 : LR_DECODE_DOT8) && sizeof(IOT) == 2;
  constexpr int CPW = INT8 ? 4 : 8;                    // codes per 32-bit word
  constexpr int NLV = INT8 ? 2 : 4;                    // integer levels of q'
  constexpr float QLIM = INT8 ? 127.0f : 7.0f;         // largest code of a level
  constexpr float QSTEP = INT8 ? 254.0f : 14.0f;       // ratio of consecutive level scales
  constexpr int QD = R / CPW;                          // 32-bit words of one level
  constexpr bool QD_IN_REGS = DOT && NLV * QD <= 32 && LPT == 1;
  constexpr int VPC = INT8 ? 16 : 32;                  // values per 16-byte chunk
  constexpr int NC = R / VPC;                          // chunks per row in the bucket
  constexpr int NCL = NC / LPT;                        // chunks per lane
  constexpr int NG = INT8 ? 1 : NC;                    // scales per token
  constexpr int QW = PACKED ? R / 2 : R;               // 32-bit words of q'
  constexpr bool Q_IN_REGS = !DOT && R <= 32 && LPT == 1;   // 32 scalar registers at most
  constexpr int RPW = (R + NW - 1) / NW;               // B rows per wavefront
  constexpr bool PREFETCH_BV = RPW <= 4;
  static_assert(LPT == 1 || (LPT == 2 && INT8 && NC % 2 == 0), "two lanes per token: int8 only");
  using E = Elem<IOT>;

  // wid is uniform: step indices and loop control live in scalar registers
  const int tid = threadIdx.x, wid = uniform_i(tid >> 6), lane = tid & 63;
  int idx = blockIdx.x;
  const int split = idx % a.n_split;
  idx /= a.n_split;
  int b, h;
  unit_of(a, ht, idx, b, h);
  const uint32_t rr = uniform_i(int(ht.ranks[h])), lo = uniform_i(int(ht.loff[h]));
  const int rk = int(rr & 0xffffu), rv = int(rr >> 16);
  const int loff_k = int(lo & 0xffffu), loff_v = int(lo >> 16);
  const uint32_t kreg = uniform_i(int(ht.kreg[h])), vreg = uniform_i(int(ht.vreg[h]));
  const int rbk = row_bytes(QF, rk), rbv = row_bytes(QF, rv);
  const int tbk = tile_bytes(QF, rk), tbv = tile_bytes(QF, rv);
  // lanes per token in this work-group (uniform), lane half, log2 of the
  // tokens per wavefront step, and this lane's token within a step
  const int lm = (LPT == 2 && max(rk, rv) > R / 2) ? 2 : 1;
  const int hf = lm == 2 ? lane >> 5 : 0, tsh = lm == 2 ? 5 : 6;
  const int tok = lane & ((1 << tsh) - 1);
  // len and the fused append's slot are read together, so that both arrive
  // in one round trip: read after the return below, the slot put one more
  // cold load latency in front of every load of the work-group (MALL-cold
  // workload 1, 28.1 against 26.6 us for the same launch without the
  // append).  Without an append a.pos is a.len.
  const int len_in = a.len[b], pos_in = a.pos[b];
  asm volatile("" ::"s"(len_in), "s"(pos_in));   // both here: the slot is not sunk into the branch below
  const int len = min(max(len_in, 0), a.max_len);
  const int ntiles = (len + 63) >> 6;
  const int n_live = max(1, (ntiles + a.tps - 1) / a.tps);
  if (split >= n_live) return;
  const int t0 = split * a.tps, t1 = min(ntiles, t0 + a.tps);
  const int unit = b * a.H + h;

  __shared__ float s_q[R];
  __shared__ uint32_t s_qw[PACKED ? QW : 1];
  __shared__ uint32_t s_qd[DOT && !QD_IN_REGS ? NLV * QD : 1];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_u[NW][R];
  __shared__ float s_o[NW][kHeadDim];

  // ---- fused append: the new token of sequence b (slot pos[b]); its
  //      latents are fetched first so their latency overlaps the prologue
  int tnew = -1, lnew = 0;                             // tile and lane of the new token
  const int nkv = (lane >> 4) & 1, nseg = lane & 15;   // wavefront 0: K row, V row
  bool nactive = false;
  float nv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (a.ck) {
    const int pos = pos_in;
    if (pos >= 0 && pos < a.capacity) {
      tnew = pos >> 6;
      lnew = pos & 63;
    }
    nactive = wid == 0 && tnew >= 0 && lane < 32 && 8 * nseg < (nkv ? rv : rk);
    if (nactive) {
      const float* src = nkv ? a.cv + size_t(b) * a.sum_rv + loff_v : a.ck + size_t(b) * a.sum_rk + loff_k;
      const size_t pstride = size_t(a.B) * (nkv ? a.sum_rv : a.sum_rk);
      const float4 x0 = *reinterpret_cast<const float4*>(src + 8 * nseg);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 8 * nseg + 4);
      nv[0] = x0.x; nv[1] = x0.y; nv[2] = x0.z; nv[3] = x0.w;
      nv[4] = x1.x; nv[5] = x1.y; nv[6] = x1.z; nv[7] = x1.w;
      for (int q = 1; q < a.n_parts; ++q) {   // further partial sums, added in order
        const float4 y0 = *reinterpret_cast<const float4*>(src + q * pstride + 8 * nseg);
        const float4 y1 = *reinterpret_cast<const float4*>(src + q * pstride + 8 * nseg + 4);
        nv[0] += y0.x; nv[1] += y0.y; nv[2] += y0.z; nv[3] += y0.w;
        nv[4] += y1.x; nv[5] += y1.y; nv[6] += y1.z; nv[7] += y1.w;
      }
    }
  }

  // ---- loads first, in the order their data is needed: q and this
  //      wavefront's B^K rows, the first tile, this wavefront's B^V rows.  Row
  //      indices are clamped instead of tested so no load sits under a branch.
  const IOT* qrow = reinterpret_cast<const IOT*>(a.q) + size_t(unit) * kHeadDim;
  const float q0 = E::ld(qrow, 2 * lane), q1 = E::ld(qrow, 2 * lane + 1);
  const IOT* bkh = reinterpret_cast<const IOT*>(a.bk) + size_t(loff_k) * kHeadDim;
  float b0[RPW], b1[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const size_t i = min(wid + k * NW, rk - 1);
    b0[k] = E::ld(bkh, i * kHeadDim + 2 * lane);
    b1[k] = E::ld(bkh, i * kHeadDim + 2 * lane + 1);
  }
  const Bounds bd{a.cache, a.cache_bytes};
  const uint8_t* kplane = a.cache + uint64_t(kreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbk;
  const uint8_t* vplane = a.cache + uint64_t(vreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbv;
  // wavefront steps of 64 / lm tokens (step s: tile s / lm); a wavefront
  // with no step of its own reads the split's last one (or tile 0) and ignores it
  const int s0 = t0 * lm, s1 = min(t1 * lm, (len + (1 << tsh) - 1) >> tsh);
  auto step_tile = [&](int st) { return size_t(st >> (lm - 1)); };
  auto step_tok = [&](int st) { return ((st & (lm - 1)) << tsh) + tok; };
  TileRegs<NCL, NG> cur;
  int t = s0 + wid;
  {
    const int sl = min(t, max(s1 - 1, 0));
    load_k<QF>(bd, kplane + step_tile(sl) * tbk, step_tok(sl), lm, hf, rk, rbk, cur);
    load_v<QF>(bd, vplane + step_tile(sl) * tbv, step_tok(sl), lm, hf, rv, rbv, cur);
  }
  const IOT* bvh = reinterpret_cast<const IOT*>(a.bv) + size_t(loff_v) * kHeadDim;
  float bv0[RPW], bv1[RPW];
  if constexpr (PREFETCH_BV) {
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const size_t i = min(wid + k * NW, rv - 1);
      bv0[k] = E::ld(bvh, i * kHeadDim + 2 * lane);
      bv1[k] = E::ld(bvh, i * kHeadDim + 2 * lane + 1);
    }
  }

  // ---- q'_i = scale * log2(e) * sum_j q_j B^K_h[i][j]: wavefront w takes
  //      rows i = w, w + NW, ..., lane j columns 2j and 2j+1; q'_i = 0 past r_k
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = wid + k * NW;
    if (i < R) {
      const float v = wave_sum63(fmaf(q1, b1[k], q0 * b0[k]));
      if (lane == 63) s_q[i] = i < rk ? v * a.qscale : 0.0f;
    }
  }

  // ---- fused append (continued): wavefront 0 quantises the new token's K row
  //      (lanes 0-15) and V row (lanes 16-31) exactly as the append kernel
  //      does and parks the codes in LDS in tile-register order for the
  //      wavefront that meets their slot; split 0 writes them to the cache
  //      when it is done (store_new)
  __shared__ uint32_t s_nw[2][4 * NC];
  __shared__ float s_ns[2][NG];
  if (wid == 0 && tnew >= 0) {
    const SegCodes nc = quantise_seg<QF>(nv);
    if (lane < 32 && 8 * nseg < R) {
      if constexpr (INT8) {
        s_nw[nkv][4 * (nseg >> 1) + 2 * (nseg & 1)] = nc.w[0];
        s_nw[nkv][4 * (nseg >> 1) + 2 * (nseg & 1) + 1] = nc.w[1];
        if (nseg == 0) s_ns[nkv][0] = nc.s;
      } else {
        s_nw[nkv][4 * (nseg >> 2) + (nseg & 3)] = nc.w[0];
        if ((nseg & 3) == 0) s_ns[nkv][nseg >> 2] = nc.s;
      }
    }
  }
  __syncthreads();
  QOperand<QW, Q_IN_REGS> qo;
  if constexpr (PACKED && !DOT) {
    // word 4j + k of the packed operand pairs values 8j + k and 8j + k + 4,
    // divided by 16 for odd k (those nibbles sit 4 bits higher)
    if (tid < QW) {
      const int j = tid >> 2, k = tid & 3;
      const float sc = (k & 1) ? 0.0625f : 1.0f;
      const half2_t hp = {_Float16(s_q[8 * j + k] * sc), _Float16(s_q[8 * j + k + 4] * sc)};
      s_qw[tid] = __builtin_bit_cast(uint32_t, hp);
    }
    __syncthreads();
    qo.lds = s_qw;
  } else {
    qo.lds = reinterpret_cast<const uint32_t*>(s_q);
  }
  if constexpr (Q_IN_REGS) {
#pragma unroll
    for (int i = 0; i < QW; ++i) qo.r[i] = uniform_i(int(qo.lds[i]));
  }
  // DOT: q' ~= sum_L qsc[L] q_L with integer levels q_1 = rne(q' / qsc[0]),
  // qsc[0] = max|q'| / QLIM, each next level rounding the remaining residual
  // on a QSTEP times finer scale (codes clamped to +-QLIM).  The error is at
  // most about max|q'| / 64516 per entry for two int8 levels and max|q'| /
  // 38416 for four int4 levels (entries past r_k stay 0).  Every wavefront
  // derives the same words; lane k packs word k of every level.
  float qsc[NLV];
  uint32_t qdw[QD_IN_REGS ? NLV * QD : 1];
  if constexpr (DOT) {
    float mq = 0.0f;
#pragma unroll
    for (int i = 0; i < R; i += 64)
      if (i + lane < R) mq = fmaxf(mq, fabsf(s_q[i + lane]));
    mq = lane63(wave_max63(mq));
    qsc[0] = mq / QLIM;
#pragma unroll
    for (int L = 1; L < NLV; ++L) qsc[L] = qsc[L - 1] / QSTEP;
    uint32_t wq[NLV];
#pragma unroll
    for (int L = 0; L < NLV; ++L) wq[L] = 0u;
    if (lane < QD && qsc[NLV - 1] != 0.0f) {
#pragma unroll
      for (int k = 0; k < CPW; ++k) {
        float v = s_q[CPW * lane + k];
#pragma unroll
        for (int L = 0; L < NLV; ++L) {
          const float c = fminf(fmaxf(rintf(v / qsc[L]), -QLIM), QLIM);
          v = fmaf(-qsc[L], c, v);
          wq[L] |= (uint32_t(int(c)) & (INT8 ? 0xffu : 0xfu)) << ((INT8 ? 8 : 4) * k);
        }
      }
    }
    if constexpr (QD_IN_REGS) {
#pragma unroll
      for (int L = 0; L < NLV; ++L)
#pragma unroll
        for (int k = 0; k < QD; ++k) qdw[L * QD + k] = uint32_t(__builtin_amdgcn_readlane(int(wq[L]), k));
    } else {
      if (wid == 0 && lane < QD) {
#pragma unroll
        for (int L = 0; L < NLV; ++L) s_qd[L * QD + lane] = wq[L];
      }
      __syncthreads();
    }
  }

  // The fused append's cache write is the work-group's last act (store_new
  // below): this launch takes the new token's codes from LDS, and on gfx950
  // stores count in the same vmcnt as loads, so a store issued before the
  // loop makes every later load wait of wavefront 0 wait for it as well, and
  // a store queued behind the stream of reads completes late.  A barrier also
  // waits for outstanding stores, so the write follows the last barrier.
  auto store_new = [&]() {
    if (split == 0 && nactive) {
      SegCodes c{};
      if constexpr (INT8) {
        c.w[0] = s_nw[nkv][4 * (nseg >> 1) + 2 * (nseg & 1)];
        c.w[1] = s_nw[nkv][4 * (nseg >> 1) + 2 * (nseg & 1) + 1];
        c.s = s_ns[nkv][0];
      } else {
        c.w[0] = s_nw[nkv][4 * (nseg >> 2) + (nseg & 3)];
        c.sh = __builtin_bit_cast(uint16_t, _Float16(s_ns[nkv][nseg >> 2]));   // exact: an fp16 value
      }
      uint8_t* tile = a.wcache + uint64_t(nkv ? vreg : kreg) * kRegionAlign +
                      (uint64_t(b) * a.n_tiles + tnew) * (nkv ? tbv : tbk);
      store_seg<QF>(Bounds{a.wcache, a.cache_bytes}, tile, nkv ? rbv : rbk, lnew, nseg, c);
    }
  };

  // ---- stream this split's steps (one token per lane or lane pair), online softmax
  float m = -__builtin_inff(), l = 0.0f;
  constexpr int LR = R / LPT;                          // V accumulators per lane
  float u[LR];
#pragma unroll
  for (int i = 0; i < LR; ++i) u[i] = 0.0f;

  // One step of this wavefront; PF: also fetch the wavefront's next step into
  // the registers just consumed.  The last step is peeled off (PF false) so
  // that no load is in flight when the loop ends: the merge below waits for
  // every outstanding load before it can use the prefetched B^V rows.
  auto tile_step = [&](const int t, auto pf) {
    constexpr bool PF = decltype(pf)::value;
    const bool valid = (t << tsh) + tok < len;
    if ((t << tsh) + tok == tnew * 64 + lnew) {   // fused append: the new token's codes come from LDS
      const int z = opaque_zero();     // keeps these reads here, not hoisted out of the loop
#pragma unroll
      for (int i = 0; i < 4 * NCL; ++i) {
        const int j = 4 * (lm * (i >> 2) + hf) + (i & 3);
        cur.kw[i] = s_nw[0][j + z];
        cur.vw[i] = s_nw[1][j + z];
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        cur.sk[g] = s_ns[0][g + z];
        cur.sv[g] = s_ns[1][g + z];
      }
    }
    if constexpr (!Q_IN_REGS) qo.lds = (PACKED ? s_qw : reinterpret_cast<const uint32_t*>(s_q)) + opaque_zero();
    const uint32_t* qdl = s_qd;
    if constexpr (DOT && !QD_IN_REGS) qdl = s_qd + opaque_zero();
    // word k of level L of the integer q'
    auto qword = [&](int L, int k) -> uint32_t {
      if constexpr (QD_IN_REGS) return qdw[(L * QD + k) % (QD_IN_REGS ? NLV * QD : 1)];
      else return qdl[L * QD + k];
    };
    float s = 0.0f;
    int acc8[NLV];   // int8 DOT: integer sums against each level, over the whole row
#pragma unroll
    for (int L = 0; L < NLV; ++L) acc8[L] = 0;
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      if (lm * c * VPC < rk) {   // uniform: tested on the lower half's chunk
        float part = 0.0f;
        if constexpr (DOT && INT8) {
          const int cg = lm * c + hf;
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int L = 0; L < NLV; ++L)
              acc8[L] = __builtin_amdgcn_sdot4(int(qword(L, 4 * cg + k)), int(cur.kw[4 * c + k]), acc8[L], false);
        } else if constexpr (DOT) {   // int4: one group of 32 ranks per chunk, its own scale
          // every word of the chunk: past r_k the q' words are 0 in every
          // level, so the codes read there add exactly 0 (a per-word rank
          // test costs a copy and a select per accumulator and word)
          int a4[NLV];
#pragma unroll
          for (int L = 0; L < NLV; ++L) a4[L] = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int L = 0; L < NLV; ++L)
              a4[L] = __builtin_amdgcn_sdot8(int(qword(L, 4 * c + j)), int(cur.kw[4 * c + j]), a4[L], false);
#pragma unroll
          for (int L = 0; L < NLV; ++L) part = fmaf(qsc[L], float(a4[L]), part);   // |a4| < 2^11: exact
          s = fmaf(cur.sk[c], part, s);
        } else if constexpr (INT8) {
          const int cg = lm * c + hf;
#pragma unroll
          for (int k = 0; k < 16; ++k) part = fmaf(qo.f(16 * cg + k), i8(cur.kw[4 * c + (k >> 2)], k & 3), part);
          s += part;
        } else if constexpr (PACKED) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (32 * c + 8 * j < rk) {
              half2_t hp[4];
              nibbles_to_h2(cur.kw[4 * c + j], hp);
#pragma unroll
              for (int k = 0; k < 4; ++k)
                part = __builtin_amdgcn_fdot2(hp[k], as_h2(qo.word(16 * c + 4 * j + k)), part, false);
            }
          }
          s = fmaf(cur.sk[c], part, s);
        } else {
#pragma unroll
          for (int k = 0; k < 32; ++k) part = fmaf(qo.f(32 * c + k), i4(cur.kw[4 * c + (k >> 3)], k & 7), part);
          s = fmaf(cur.sk[c], part, s);
        }
      }
    }
    if constexpr (DOT && INT8) {   // |sums| < 2^21: exact in fp32
      float t = 0.0f;
#pragma unroll
      for (int L = NLV - 1; L >= 0; --L) t = fmaf(qsc[L], float(acc8[L]), t);
      s = t;
    }
    if constexpr (LPT == 2) {   // both lanes of a token: the full score
      const float both = swap_sum32(s, s);
      s = lm == 2 ? both : s;
    }
    if constexpr (INT8) s *= cur.sk[0];
    const int tn = t + NW;   // K regs are free now: the next step's K codes
    if constexpr (PF) load_k<QF>(bd, kplane + step_tile(tn) * tbk, step_tok(tn), lm, hf, rk, rbk, cur);
    s = valid ? s : -__builtin_inff();
    if (s > m + kTau) {  // rare after the first tile: rescale the running sums
      const float al = __builtin_amdgcn_exp2f(m - s);
      l *= al;
#pragma unroll
      for (int i = 0; i < LR; ++i) u[i] *= al;
      m = s;
    }
    const float p = valid ? __builtin_amdgcn_exp2f(s - m) : 0.0f;
    l += p;
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      if (lm * c * VPC < rv) {
        const float wt = valid ? p * cur.sv[INT8 ? 0 : c] : 0.0f;
        if constexpr (INT8) {
#pragma unroll
          for (int k = 0; k < 16; ++k) u[16 * c + k] = fmaf(wt, i8(cur.vw[4 * c + (k >> 2)], k & 3), u[16 * c + k]);
        } else if constexpr (PACKED) {
          const float wt16 = wt * 0.0625f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (32 * c + 8 * j < rv) {
              half2_t hp[4];
              nibbles_to_h2(cur.vw[4 * c + j], hp);
              float* uu = u + 32 * c + 8 * j;
              uu[0] = fmaf(float(hp[0].x), wt, uu[0]);
              uu[4] = fmaf(float(hp[0].y), wt, uu[4]);
              uu[1] = fmaf(float(hp[1].x), wt16, uu[1]);
              uu[5] = fmaf(float(hp[1].y), wt16, uu[5]);
              uu[2] = fmaf(float(hp[2].x), wt, uu[2]);
              uu[6] = fmaf(float(hp[2].y), wt, uu[6]);
              uu[3] = fmaf(float(hp[3].x), wt16, uu[3]);
              uu[7] = fmaf(float(hp[3].y), wt16, uu[7]);
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < 32; ++k) u[32 * c + k] = fmaf(wt, i4(cur.vw[4 * c + (k >> 3)], k & 7), u[32 * c + k]);
        }
      }
    }
    if constexpr (PF) load_v<QF>(bd, vplane + step_tile(tn) * tbv, step_tok(tn), lm, hf, rv, rbv, cur);
  };
  for (; t + NW < s1; t += NW) tile_step(t, std::true_type{});
  if (t < s1) tile_step(t, std::false_type{});

  // ---- merge the lanes of each wavefront, publish per wavefront: the V
  //      latent in transposed groups of 32 ranks, or with two lanes per token
  //      16-rank chunks per half (one LDS write per lane)
  {
    const float Mw = lane63(wave_max63(m));
    const float f = (m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m - Mw);
    const float lw = wave_sum63(hf ? 0.0f : l * f);   // each token's l counted once
    if (lane == 63) { s_m[wid] = Mw; s_l[wid] = lw; }
    if constexpr (LPT == 1) {
#pragma unroll
      for (int g = 0; g < R; g += 32) {
        if (g < rv) {
          float x[32];
#pragma unroll
          for (int k = 0; k < 32; ++k) x[k] = u[g + k] * f;
          const float sum = wave_sum32_transposed(x, lane);
          if ((lane & 4) == 0) s_u[wid][g + transposed_index(lane)] = sum;
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        if (lm * c * 16 < rv) {
          float x[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) x[k] = u[16 * c + k] * f;
          if (lm == 1) {   // one token per lane: the halves hold the same ranks
#pragma unroll
            for (int k = 0; k < 16; ++k) x[k] = swap_sum32(x[k], x[k]);
          }
          const float sum = half_sum16_transposed(x, lane);
          if ((lane & 4) == 0 && (lm == 2 || lane < 32))
            s_u[wid][16 * (lm * c + hf) + ((lane & 3) | ((lane >> 1) & 0xc))] = sum;
        }
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

  if (a.n_split > 1) {  // partial for k_merge (the kernel boundary orders it)
    float* part = a.part + (size_t(unit) * a.n_split + split) * kPartStride;
    if (tid == 0) { part[0] = M; part[1] = L; }
    if (tid < rv) {
      float ui = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ui = fmaf(fw[w], s_u[w][tid], ui);
      part[2 + tid] = ui;
    }
    store_new();
    return;
  }

  // ---- o = (u / l) B^V_h: wavefront w finishes u_i for its rows
  //      i = w, w + NW, ... and multiplies them into columns 2j, 2j+1
  const float inv_l = L > 0.0f ? 1.0f / L : 0.0f;
  if constexpr (!PREFETCH_BV) {
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int i = wid + k * NW;
      bv0[k] = E::ld(bvh, size_t(min(i, rv - 1)) * kHeadDim + 2 * lane);
      bv1[k] = E::ld(bvh, size_t(min(i, rv - 1)) * kHeadDim + 2 * lane + 1);
    }
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = wid + k * NW;
    if (i < rv) {
      float ui = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ui = fmaf(fw[w], s_u[w][i], ui);
      ui *= inv_l;
      a0 = fmaf(ui, bv0[k], a0);
      a1 = fmaf(ui, bv1[k], a1);
    }
  }
  s_o[wid][2 * lane] = a0;
  s_o[wid][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < kHeadDim) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += s_o[w][tid];
    E::st(reinterpret_cast<IOT*>(a.out) + size_t(unit) * kHeadDim, tid, acc);
  }
  store_new();
}

// o[j] = sum_i v[i] B^V_h[i][j] for j < 128, v = u / l already in LDS (s_v),
// for the split merge.  Wavefront w takes rows i = w, w + NW, ... < rv and
// lane j columns 2j, 2j+1; the NW partial rows meet in LDS (s_o).
template <typename IOT, int R, int NW>
__device__ __forceinline__ void project_out(const float* s_v, float (*s_o)[kHeadDim], int rv,
                                            const IOT* bvh, IOT* o, int tid) {
  constexpr int RPW = (R + NW - 1) / NW;
  const int wid = tid >> 6, lane = tid & 63;
  float b0[RPW], b1[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = wid + k * NW;
    b0[k] = Elem<IOT>::ld(bvh, size_t(min(i, rv - 1)) * kHeadDim + 2 * lane);
    b1[k] = Elem<IOT>::ld(bvh, size_t(min(i, rv - 1)) * kHeadDim + 2 * lane + 1);
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = wid + k * NW;
    if (i < rv) {
      a0 = fmaf(s_v[i], b0[k], a0);
      a1 = fmaf(s_v[i], b1[k], a1);
    }
  }
  s_o[wid][2 * lane] = a0;
  s_o[wid][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < kHeadDim) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += s_o[w][tid];
    Elem<IOT>::st(o, tid, acc);
  }
}

// Flash-Decoding merge of the split partials of one (b, h), then o = (u/l) B^V_h:
//   M = max_s m_s,  l = sum_s 2^(m_s - M) l_s,  u = sum_s 2^(m_s - M) u_s.
template <typename IOT>
__global__ __launch_bounds__(512) void k_merge(DecodeArgs a, HeadTab ht) {
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int b = unit / a.H, h = unit % a.H;
  const int rv = int(uniform_i(int(ht.ranks[h])) >> 16);
  const int loff_v = int(uniform_i(int(ht.loff[h])) >> 16);
  const int len = min(max(a.len[b], 0), a.max_len);
  const int n_live = max(1, ((len + 63) / 64 + a.tps - 1) / a.tps);
  const float* pu = a.part + size_t(unit) * a.n_split * kPartStride;
  __shared__ float s_v[LR_MAX_RANK];
  __shared__ float s_o[8][kHeadDim];
  float M = -__builtin_inff();
  for (int s = 0; s < n_live; ++s) M = fmaxf(M, pu[size_t(s) * kPartStride]);
  float L = 0.0f, ui = 0.0f;
  for (int s = 0; s < n_live; ++s) {
    const float* ps = pu + size_t(s) * kPartStride;
    const float fs = (ps[0] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ps[0] - M);
    L = fmaf(fs, ps[1], L);
    if (tid < rv) ui = fmaf(fs, ps[2 + tid], ui);
  }
  if (tid < rv) s_v[tid] = (L > 0.0f) ? ui / L : 0.0f;
  __syncthreads();
  project_out<IOT, LR_MAX_RANK, 8>(s_v, s_o, rv, reinterpret_cast<const IOT*>(a.bv) + size_t(loff_v) * kHeadDim,
                                   reinterpret_cast<IOT*>(a.out) + size_t(unit) * kHeadDim, tid);
}

// ---------------------------------------------------------------------------
// decode, explicit reconstruction (matrix cores)
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t f32_to_bf16_exact(float v) { return __float_as_uint(v) >> 16; }

// 8 codes (ranks k0 .. k0+7 of this lane's token) as the bf16 B operand of
// v_mfma_f32_32x32x16_bf16; codes of magnitude <= 127 are exact in bf16.
template <int QF>
__device__ __forceinline__ bf16x8_t codes_to_bf16(const uint32_t* w, int k0) {
  float v[8];
  if constexpr (QF == LR_Q_INT8_TOKEN) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = i8(w[(k0 + e) >> 2], (k0 + e) & 3);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = i4(w[(k0 + e) >> 3], (k0 + e) & 7);
  }
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = f32_to_bf16_exact(v[2 * e]) | (f32_to_bf16_exact(v[2 * e + 1]) << 16);
  return __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
}

// Codes of ranks [16 kb + 8 hl, +8) of token ti of a tile (kb: 16-rank block,
// hl: which half of the block this lane holds), zero beyond the row width.
template <int QF>
__device__ __forceinline__ void load_codes8(const Bounds& bd, const uint8_t* tile, int rb, int kb, int hl, int ti,
                                            uint32_t* w) {
  if constexpr (QF == LR_Q_INT8_TOKEN) {
    const int c = kb, wc = min(16, rb - 16 * c), off = 8 * hl;   // 8 bytes
    if (off + 8 <= wc) {
      const uint2 v = *checked(bd, reinterpret_cast<const uint2*>(tile + 1024 * c + wc * ti + off), 8);
      w[0] = v.x; w[1] = v.y;
    } else { w[0] = 0; w[1] = 0; }
  } else {
    const int c = kb >> 1, wc = min(16, rb - 16 * c), off = 8 * (kb & 1) + 4 * hl;   // 4 bytes
    w[0] = off + 4 <= wc ? *checked(bd, reinterpret_cast<const uint32_t*>(tile + 1024 * c + wc * ti + off), 4) : 0u;
    w[1] = 0;
  }
}

// One work-group per (b, h); NW wavefronts take 64-token tiles round-robin and
// treat each as two halves of 32 tokens.  For every 32-row block of d,
// K^T = B^K^T C^T and V^T = B^V^T C^T are formed with
// v_mfma_f32_32x32x16_bf16 (B^T staged in LDS, codes as exact bf16): lane l
// then holds 16 rows of column (token) l % 32.  Scores are the dot of K^T with
// q over d (two lanes per token, halves added with a cross-half swap), and
// o^T accumulates p_t V^T.  int4 group scales are applied per group to the
// fp32 accumulators, so nothing is rounded beyond fp32.
template <int QF, int R, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_explicit(DecodeArgs a, HeadTab ht) {
  constexpr bool INT8 = QF == LR_Q_INT8_TOKEN;
  constexpr int VPC = INT8 ? 16 : 32;
  constexpr int NC = R / VPC;
  constexpr int NG = INT8 ? 1 : NC;
  constexpr int KB = R / 16;                 // 16-rank blocks
  constexpr int LDR = R + 8;                 // padded LDS row (bf16 elements)
  using E = Elem<uint16_t>;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  int b, h;
  unit_of(a, ht, int(blockIdx.x), b, h);
  const uint32_t rr = uniform_i(int(ht.ranks[h])), lo = uniform_i(int(ht.loff[h]));
  const int rk = int(rr & 0xffffu), rv = int(rr >> 16);
  const int loff_k = int(lo & 0xffffu), loff_v = int(lo >> 16);
  const uint32_t kreg = uniform_i(int(ht.kreg[h])), vreg = uniform_i(int(ht.vreg[h]));
  const int rbk = row_bytes(QF, rk), rbv = row_bytes(QF, rv);
  const int tbk = tile_bytes(QF, rk), tbv = tile_bytes(QF, rv);
  const int len = min(max(a.len[b], 0), a.max_len);
  const int ntiles = (len + 63) >> 6;
  const int unit = b * a.H + h;

  __shared__ uint16_t s_bt[2][kHeadDim * LDR];   // B^K^T, B^V^T: [d][rank]
  __shared__ float s_q[kHeadDim];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_o[NW][kHeadDim];

  // ---- stage B^K^T and B^V^T (zero beyond the ranks) and q * scale * log2(e)
  {
    const uint16_t* bk = reinterpret_cast<const uint16_t*>(a.bk) + size_t(loff_k) * kHeadDim;
    const uint16_t* bv = reinterpret_cast<const uint16_t*>(a.bv) + size_t(loff_v) * kHeadDim;
    for (int e = tid; e < R * kHeadDim; e += NW * 64) {
      const int k = e / kHeadDim, d = e % kHeadDim;
      s_bt[0][d * LDR + k] = k < rk ? bk[size_t(k) * kHeadDim + d] : uint16_t(0);
      s_bt[1][d * LDR + k] = k < rv ? bv[size_t(k) * kHeadDim + d] : uint16_t(0);
    }
    if (tid < kHeadDim)
      s_q[tid] = E::ld(reinterpret_cast<const uint16_t*>(a.q) + size_t(unit) * kHeadDim, tid) * a.qscale;
  }
  __syncthreads();

  const Bounds bd{a.cache, a.cache_bytes};
  const uint8_t* kplane = a.cache + uint64_t(kreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbk;
  const uint8_t* vplane = a.cache + uint64_t(vreg) * kRegionAlign + uint64_t(b) * a.n_tiles * tbv;
  const int hl = lane >> 5, col = lane & 31;
  float m = -__builtin_inff(), l = 0.0f;
  float o[4][16];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

  for (int t = wid; t < ntiles; t += NW) {
    const uint8_t* kt = kplane + size_t(t) * tbk;
    const uint8_t* vt = vplane + size_t(t) * tbv;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const int ti = 32 * half + col;              // token of this lane within the tile
      const bool valid = t * 64 + ti < len;
      uint32_t kw[KB][2], vw[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        load_codes8<QF>(bd, kt, rbk, kb, hl, ti, kw[kb]);
        load_codes8<QF>(bd, vt, rbv, kb, hl, ti, vw[kb]);
      }
      float sk[NG], sv[NG];
      if constexpr (INT8) {
        sk[0] = *checked(bd, reinterpret_cast<const float*>(kt + 64 * rbk + 4 * ti), 4);
        sv[0] = *checked(bd, reinterpret_cast<const float*>(vt + 64 * rbv + 4 * ti), 4);
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          sk[g] = 32 * g < rk ? half_bits_to_f32(*checked(bd, reinterpret_cast<const uint16_t*>(kt + 64 * rbk + 2 * (64 * g + ti)), 2)) : 0.0f;
          sv[g] = 32 * g < rv ? half_bits_to_f32(*checked(bd, reinterpret_cast<const uint16_t*>(vt + 64 * rbv + 2 * (64 * g + ti)), 2)) : 0.0f;
        }
      }
      // ---- k_t rebuilt block by block, dotted with q
      float s = 0.0f;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        float kd[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) kd[r] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          f32x16_t acc = {};
#pragma unroll
          for (int kb = (INT8 ? 0 : 2 * g); kb < (INT8 ? KB : 2 * g + 2); ++kb) {
            if (16 * kb < rk) {
              const bf16x8_t bt = __builtin_bit_cast(bf16x8_t,
                  *reinterpret_cast<const uint4*>(&s_bt[0][(32 * db + col) * LDR + 16 * kb + 8 * hl]));
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bt, codes_to_bf16<QF>(kw[kb], 0), acc, 0, 0, 0);
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) kd[r] = fmaf(sk[g], acc[r], kd[r]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s = fmaf(kd[r], s_q[32 * db + 8 * (r >> 2) + 4 * hl + (r & 3)], s);
      }
      s += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (lane ^ 32), __builtin_bit_cast(int, s)));
      s = valid ? s : -__builtin_inff();
      if (s > m + kTau) {
        const float al = __builtin_amdgcn_exp2f(m - s);
        l *= al;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= al;
        m = s;
      }
      const float p = valid ? __builtin_amdgcn_exp2f(s - m) : 0.0f;
      l += p;
      // ---- v_t rebuilt block by block, accumulated with weight p_t
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          f32x16_t acc = {};
#pragma unroll
          for (int kb = (INT8 ? 0 : 2 * g); kb < (INT8 ? KB : 2 * g + 2); ++kb) {
            if (16 * kb < rv) {
              const bf16x8_t bt = __builtin_bit_cast(bf16x8_t,
                  *reinterpret_cast<const uint4*>(&s_bt[1][(32 * db + col) * LDR + 16 * kb + 8 * hl]));
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bt, codes_to_bf16<QF>(vw[kb], 0), acc, 0, 0, 0);
            }
          }
          const float wt = valid ? p * sv[g] : 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] = fmaf(wt, acc[r], o[db][r]);
        }
      }
    }
  }

  // ---- merge: lanes of one half hold the same tokens' d-rows; both halves
  //      saw the same scores, so m and l are taken from the lower half
  const float Mw = lane63(wave_max63(m));
  const float f = (m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m - Mw);
  const float lw = wave_sum63(hl == 1 ? l * f : 0.0f);
  if (lane == 63) { s_m[wid] = Mw; s_l[wid] = lw; }
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = o[db][r] * f;                       // sum over the 32 lanes of this half
      v += dpp<0xb1>(v, 0.f);
      v += dpp<0x4e>(v, 0.f);
      v += dpp<0x141>(v, 0.f);
      v += dpp<0x140>(v, 0.f);
      v += dpp<0x142, 0xa>(v, 0.f);                 // lanes 31 and 63 hold the half sums
      if (col == 31) s_o[wid][32 * db + 8 * (r >> 2) + 4 * hl + (r & 3)] = v;
    }
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float fw = (s_m[w] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w] - M);
      L = fmaf(fw, s_l[w], L);
      acc = fmaf(fw, s_o[w][tid], acc);
    }
    E::st(reinterpret_cast<uint16_t*>(a.out) + size_t(unit) * kHeadDim, tid, L > 0.0f ? acc / L : 0.0f);
  }
}

template <int QF, typename IOT, int R>
hipError_t launch_decode_r(int waves, dim3 grid, hipStream_t st, const DecodeArgs& a, const HeadTab& t) {
  constexpr int LPT = pair_lanes(QF, R) ? 2 : 1;
  if constexpr (max_wg_waves(QF, R) == 16) {
    if (waves == 16) {
      hipLaunchKernelGGL((k_decode<QF, IOT, R, 16, LPT>), grid, dim3(1024), 0, st, a, t);
      return hipGetLastError();
    }
  }
  if constexpr (decode_waves_per_simd(QF, R) == 3) {
    if (waves == 3) {   // four work-groups per compute unit (choose_split)
      hipLaunchKernelGGL((k_decode<QF, IOT, R, 3, LPT>), grid, dim3(192), 0, st, a, t);
      return hipGetLastError();
    }
  }
  if (waves == 8) hipLaunchKernelGGL((k_decode<QF, IOT, R, 8, LPT>), grid, dim3(512), 0, st, a, t);
  else hipLaunchKernelGGL((k_decode<QF, IOT, R, 4, LPT>), grid, dim3(256), 0, st, a, t);
  return hipGetLastError();
}

template <int QF, typename IOT>
hipError_t launch_decode_q(int bucket, int waves, dim3 grid, hipStream_t st, const DecodeArgs& a,
                           const HeadTab& t) {
  switch (bucket) {
    case 32: return launch_decode_r<QF, IOT, 32>(waves, grid, st, a, t);
    case 64: return launch_decode_r<QF, IOT, 64>(waves, grid, st, a, t);
    case 96: return launch_decode_r<QF, IOT, 96>(waves, grid, st, a, t);
    default: return launch_decode_r<QF, IOT, 128>(waves, grid, st, a, t);
  }
}

// Split partials of lr_attn_append_decode_noalloc, for callers that cannot
// allocate: one array per device (each GPU the library runs on holds its own
// copy until the process ends), shared by every such call on that device.
// choose_split keeps units x splits below 2048, so the partials of any plan
// need at most 2048 x kPartStride x 4 bytes (1.06 MB).  In host code the name
// `scratch` is not a device address: only the address that
// hipGetSymbolAddress returns for it (scratch_address) is passed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

}  // namespace

uint64_t g_check_shrink = 0;
uint64_t checked_extent(size_t bytes) { return g_check_shrink < bytes ? uint64_t(bytes) - g_check_shrink : 0; }

int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {   // once per device, with that device current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return 0;
}

int launch_append(const lr_attn_plan& p, int32_t layer, void* cache, const float* ck,
                  const float* cv, const int32_t* pos, int32_t n_new, void* stream) {
  const auto& L = p.layers[layer];
  AppendArgs a;
  a.cache = static_cast<uint8_t*>(cache);
  a.cache_bytes = checked_extent(L.cache_bytes);
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
  const dim3 grid(unsigned((a.rows * 16 + 255) / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.desc.qfmt == LR_Q_INT8_TOKEN)
    hipLaunchKernelGGL(k_append<LR_Q_INT8_TOKEN>, grid, dim3(256), 0, st, a, L.tab);
  else
    hipLaunchKernelGGL(k_append<LR_Q_INT4_G32>, grid, dim3(256), 0, st, a, L.tab);
  return int(hipGetLastError());
}

// Eight-wavefront work-groups (two wavefronts per SIMD, 256 VGPRs each) only
// for the 32 bucket: from rank 64 up the kernel's accumulators and code
// registers exceed 256 VGPRs and spill, so those buckets always take four
// (explicit_split chooses accordingly).
template <int QF, int RR>
void launch_explicit_r(int waves, dim3 grid, hipStream_t st, const DecodeArgs& a, const HeadTab& t) {
  if constexpr (RR == 32) {
    if (waves == 8) {
      hipLaunchKernelGGL((k_decode_explicit<QF, RR, 8>), grid, dim3(512), 0, st, a, t);
      return;
    }
  }
  hipLaunchKernelGGL((k_decode_explicit<QF, RR, 4>), grid, dim3(256), 0, st, a, t);
}

template <int QF>
hipError_t launch_explicit_q(int bucket, int waves, dim3 grid, hipStream_t st, const DecodeArgs& a,
                             const HeadTab& t) {
  switch (bucket) {
    case 32: launch_explicit_r<QF, 32>(waves, grid, st, a, t); break;
    case 64: launch_explicit_r<QF, 64>(waves, grid, st, a, t); break;
    case 96: launch_explicit_r<QF, 96>(waves, grid, st, a, t); break;
    default: launch_explicit_r<QF, 128>(waves, grid, st, a, t); break;
  }
  return hipGetLastError();
}

int launch_decode(const lr_attn_plan& p, int32_t layer, const void* cache, const int32_t* len,
                  int32_t max_len, const void* q, const void* bk, const void* bv, float scale,
                  void* out, void* workspace, void* stream, bool explicit_form,
                  const AppendInputs* app) {
  const auto& L = p.layers[layer];
  const Split sp = explicit_form ? explicit_split(p, layer, max_len) : choose_split(p, layer, max_len);
  DecodeArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.cache_bytes = checked_extent(L.cache_bytes);
  a.len = len;
  a.q = q;
  a.bk = bk;
  a.bv = bv;
  a.out = out;
  a.part = static_cast<float*>(workspace);
  a.qscale = scale * kLog2e;
  a.B = p.desc.batch;
  a.H = p.desc.n_heads;
  a.n_tiles = p.n_tiles;
  a.max_len = max_len;
  a.n_split = sp.n_split;
  a.tps = sp.tiles_per_split;
  a.xcd_groups = (sp.n_split == 1 && p.desc.n_heads % 8 == 0) ? 1 : 0;
  a.wcache = app ? static_cast<uint8_t*>(app->cache) : nullptr;
  a.ck = app ? app->ck : nullptr;
  a.cv = app ? app->cv : nullptr;
  a.pos = app ? app->pos : len;     // read by every launch beside len (unused without ck)
  a.capacity = p.desc.capacity;
  a.sum_rk = L.sum_rk;
  a.sum_rv = L.sum_rv;
  a.n_parts = app ? app->n_parts : 1;
  const unsigned units = unsigned(p.desc.batch) * unsigned(p.desc.n_heads);
  const dim3 grid(units * unsigned(sp.n_split));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int bucket = layer_bucket(L);
  const bool bf = p.desc.io_dtype == LR_DT_BF16;
  hipError_t e;
  if (explicit_form) {
    e = p.desc.qfmt == LR_Q_INT8_TOKEN ? launch_explicit_q<LR_Q_INT8_TOKEN>(bucket, sp.waves, grid, st, a, L.tab)
                                       : launch_explicit_q<LR_Q_INT4_G32>(bucket, sp.waves, grid, st, a, L.tab);
    return int(e);
  }
  if (p.desc.qfmt == LR_Q_INT8_TOKEN)
    e = bf ? launch_decode_q<LR_Q_INT8_TOKEN, uint16_t>(bucket, sp.waves, grid, st, a, L.tab)
           : launch_decode_q<LR_Q_INT8_TOKEN, float>(bucket, sp.waves, grid, st, a, L.tab);
  else
    e = bf ? launch_decode_q<LR_Q_INT4_G32, uint16_t>(bucket, sp.waves, grid, st, a, L.tab)
           : launch_decode_q<LR_Q_INT4_G32, float>(bucket, sp.waves, grid, st, a, L.tab);
  if (e != hipSuccess || sp.n_split == 1) return int(e);
  if (bf) hipLaunchKernelGGL(k_merge<uint16_t>, dim3(units), dim3(512), 0, st, a, L.tab);
  else hipLaunchKernelGGL(k_merge<float>, dim3(units), dim3(512), 0, st, a, L.tab);
  return int(hipGetLastError());
}

}  // namespace lr

extern "C" {

lr_status lr_attn_check_count(uint64_t* count) {
#if LR_ATTN_CHECK
  if (!count) return LR_EINVAL;
  unsigned long long v = 0, vf = 0, vp = 0;
  const unsigned long long zero = 0;
  int e = int(hipMemcpyFromSymbol(&v, HIP_SYMBOL(lr::g_check_count), sizeof v, 0, hipMemcpyDeviceToHost));
  if (e == 0) e = int(hipMemcpyToSymbol(HIP_SYMBOL(lr::g_check_count), &zero, sizeof zero, 0, hipMemcpyHostToDevice));
  if (e == 0) e = lr::ffn_check_take(&vf);       // the FFN kernels' counter (ffn.hip)
  if (e == 0) e = lr::project_check_take(&vp);   // latent generation's (project.hip)
  if (e != 0) {
    lr::set_last_hip_error(e);
    return LR_EHIP;
  }
  *count = v + vf + vp;
  return LR_OK;
#else
  (void)count;
  return LR_EUNSUPPORTED;
#endif
}

lr_status lr_attn_check_shrink(uint64_t bytes) {
#if LR_ATTN_CHECK
  lr::g_check_shrink = bytes;
  return LR_OK;
#else
  (void)bytes;
  return LR_EUNSUPPORTED;
#endif
}

}  // extern "C"
