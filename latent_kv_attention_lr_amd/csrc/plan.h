// plan.h -- internal: the plan object and the launch functions the C ABI calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "layout.h"

struct lr_attn_plan {
  lr_attn_desc desc;                 // copy; rank pointers cleared
  int32_t n_tiles;                   // tiles per plane = ceil(capacity / 64)
  struct Layer {
    lr::HeadTab tab;
    std::vector<lr_attn_head_layout> heads;
    size_t cache_bytes;
    int32_t sum_rk, sum_rv, rk_max, rv_max;
  };
  std::vector<Layer> layers;
};

namespace lr {

// Shape of a decode launch.
struct Split {
  int32_t n_split;          // work-groups per (b, h): context splits
  int32_t tiles_per_split;  // 64-token tiles per work-group
  int32_t waves;            // wavefronts per work-group: 3, 4, 8 or 16
};
// Register bucket of a layer: the largest rank rounded up to 32, 64, 96 or 128.
inline int layer_bucket(const lr_attn_plan::Layer& L) {
  const int r = L.rk_max > L.rv_max ? L.rk_max : L.rv_max;
  return r <= 32 ? 32 : r <= 64 ? 64 : r <= 96 ? 96 : 128;
}
// Buckets whose decode kernel puts two lanes on each token (int8 ranks above
// 64): half the registers per lane, twice the wavefronts per compute unit.
constexpr bool pair_lanes(int qfmt, int bucket) { return qfmt == LR_Q_INT8_TOKEN && bucket > 64; }
// Wavefronts per SIMD each bucket's decode kernel is compiled for (its
// register budget): enough bytes in flight per compute unit to cover HBM
// latency without spilling.
constexpr int decode_waves_per_simd(int qfmt, int bucket) {
  return pair_lanes(qfmt, bucket) ? (bucket <= 96 ? 4 : 3)
                                  : bucket <= 32 ? 5 : bucket <= 64 ? (qfmt == LR_Q_INT8_TOKEN ? 3 : 4) : 2;
}
// Compute units of the GPU the library is built for (MI355X, gfx950).
constexpr int kComputeUnits = 256;
// Largest work-group of a bucket's decode kernel: 16 wavefronts where 128
// VGPRs per lane suffice (four wavefronts per SIMD), else 8.
constexpr int max_wg_waves(int qfmt, int bucket) {
  return (bucket <= 32 || (bucket <= 64 && qfmt == LR_Q_INT4_G32) || (pair_lanes(qfmt, bucket) && bucket <= 96))
             ? 16 : 8;
}
Split choose_split(const lr_attn_plan& p, int32_t layer, int32_t max_len);
// The explicit-reconstruction kernel never splits the context: 4 or 8 waves.
Split explicit_split(const lr_attn_plan& p, int32_t layer, int32_t max_len);
size_t workspace_bytes(const lr_attn_plan& p, int32_t max_len);

// Kernel launchers (kernels.hip).  Arguments are already validated.  Each
// returns the hipError_t of the launch (0 on success).
int launch_append(const lr_attn_plan& p, int32_t layer, void* cache, const float* ck,
                  const float* cv, const int32_t* pos, int32_t n_new, void* stream);
// The token a fused append writes before the decode attends (one per sequence).
struct AppendInputs {
  void* cache;
  const float* ck;
  const float* cv;
  const int32_t* pos;
  // ck, cv hold n_parts blocks of [batch][sum_r] partial sums (stride batch x
  // sum_r), added in block order to give the latents
  int32_t n_parts = 1;
};
int launch_decode(const lr_attn_plan& p, int32_t layer, const void* cache, const int32_t* len,
                  int32_t max_len, const void* q, const void* bk, const void* bv, float scale,
                  void* out, void* workspace, void* stream, bool explicit_form,
                  const AppendInputs* app = nullptr);
// project.hip: packing of the down-projection factors (row-major W [sum_r][E]
// bf16 -> MFMA step blocks) and fp32 latents ck [n_tokens][sum_rk] = x W^K^T
// (cv likewise) from bf16 x [n_tokens][embed].  n_tokens >= 1, embed % 32 == 0.
size_t packed_projection_elems(const lr_attn_plan& p, int32_t layer, int32_t embed);
int launch_pack_projection(const lr_attn_plan& p, int32_t layer, int32_t embed, const void* wk,
                           const void* wv, void* packed, void* stream);
// With n_parts > 1, E is split into n_parts ranges and part q's sums are
// written at ck + q * n_tokens * sum_rk (cv likewise); their sum in part
// order is the latent.  project_parts: the part count the fused step uses.
constexpr int kMaxProjectParts = 8;
int project_parts(const lr_attn_plan& p, int32_t layer, int32_t n_tokens, int32_t embed);
int launch_project(const lr_attn_plan& p, int32_t layer, const void* x, int32_t n_tokens,
                   int32_t embed, const void* packed, float* ck, float* cv, void* stream,
                   int32_t n_parts = 1);
// Hybrid FFN (ffn.hip, ffn_host.cpp): byte offsets of the packed weight
// sections and, for a call on T tokens, of the workspace buffers.
struct FfnLayout {
  int32_t E, F, S, r, Fp;                            // Fp = F rounded up to 64
  size_t off_w1, off_w2, off_w3, off_s1, off_s2, off_s3, weight_bytes;
  size_t ws_cnt, ws_cnt_bytes;                      // counters of the launches' last-to-finish work-groups
  int32_t h_ld;                                      // row stride of h in floats (F rounded up to 32)
  int32_t out_splits, out_rt;                        // down-projection chunks and row tiles the workspace is sized for
  size_t ws_xq, ws_xs, ws_zp, ws_zq, ws_zs, ws_h, ws_hq, ws_hs, ws_yp, ws_bytes;
};
// Records a HIP error for lr_attn_last_hip_error (this thread).
void set_last_hip_error(int err);
int launch_ffn(const FfnLayout& f, const void* weights, const void* x, int32_t n_tokens, float* y,
               void* workspace, void* stream);
// Device scratch of the allocation-free decode entry point (kernels.hip): a
// static device array of kScratchBytes; scratch_address gives the current
// device's copy (looked up once per device).  Returns a hipError_t.
constexpr size_t kScratchBytes = LR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
int scratch_address(void** out);
// The checked build (check.h): the extent the kernels test a buffer's
// accesses against -- its bytes less what lr_attn_check_shrink takes off (a
// test hook; 0 by default) -- and, from ffn.hip and project.hip, their
// kernels' counts of accesses outside their buffers, read and reset (each
// returns a hipError_t).
uint64_t checked_extent(size_t bytes);
int ffn_check_take(unsigned long long* count);
int project_check_take(unsigned long long* count);
// probe.hip: stream bytes / 16 16-byte words from src (read only).
int launch_probe_read(const void* src, size_t bytes, void* sink, void* stream);

}  // namespace lr
