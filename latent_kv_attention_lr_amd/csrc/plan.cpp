// plan.cpp -- host side of the C ABI: plan construction, layout queries,
// argument validation and the context-split policy.  Nothing here touches the
// GPU except through the launchers in kernels.hip.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <numeric>

#include "plan.h"

namespace {

thread_local int32_t g_last_hip = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool rank_ok(int32_t r) { return r >= 8 && r <= LR_MAX_RANK && r % 8 == 0; }

lr_status hip_status(int err) {
  if (err == 0) return LR_OK;
  g_last_hip = err;
  return LR_EHIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

namespace lr {
void set_last_hip_error(int err) { g_last_hip = err; }
}  // namespace lr

namespace lr {

Split choose_split(const lr_attn_plan& p, int32_t layer, int32_t max_len) {
  // Wavefronts per (b, h) work-group: 4, doubled while fewer than 4096
  // wavefronts (16 per CU) would be in flight -- up to 16 where 128 VGPRs
  // suffice, else 8.  Small work-groups let several run per compute unit out
  // of phase (one group's prologue and merge overlap another's streaming) and
  // let many (b, h) units fit in fewer rounds of resident work-groups:
  // MALL-cold on MI355X, 32-layer mixed-rank workload (1024 units) 48.2 /
  // 53.2 / 72.0 us per layer with 4 / 8 / 16 wavefronts, int4 rank-64 batch-64
  // workload (2048 units) 208 / 212 / 265 us.  Beyond 4096 wavefronts with
  // the largest work-group the context of each (b, h) is split
  // Flash-Decoding style and a second kernel merges the partials (every
  // split keeps at least two tiles per wavefront).
  //
  // Buckets compiled for three wavefronts per SIMD hold only three
  // four-wavefront work-groups per compute unit (768 on the GPU), so there
  // the target is the 3072 wavefronts the GPU holds, and between 769 and
  // 1024 (b, h) units the work-groups take three wavefronts: four per CU, all
  // resident in one round.  (Measured on MI355X, 32-layer workload with a
  // greedily allocated rank table, ranks 8..128: with four-wavefront groups
  // the 256 lightest heads waited for the first round and then streamed
  // almost alone for the last quarter of the launch.)
  Split s;
  const int64_t units = static_cast<int64_t>(p.desc.batch) * p.desc.n_heads;
  const int64_t tiles = ceil_div(max_len, kTile);
  const int bucket = layer_bucket(p.layers[layer]);
  const int nw_max = max_wg_waves(p.desc.qfmt, bucket);
  const int wps = decode_waves_per_simd(p.desc.qfmt, bucket);
  const int64_t target = wps == 3 ? int64_t(kComputeUnits) * 4 * wps : 4096;   // wavefronts in flight wanted
  int nw = 4;
  if (p.desc.wg_waves > 0) {
    nw = std::min(p.desc.wg_waves, nw_max);
  } else {
    while (nw < nw_max && units * nw < target) nw *= 2;
    while (nw > 4 && (nw / 2) >= tiles) nw /= 2;   // no wavefront without a tile
    if (wps == 3 && nw == 4 && units * 4 > target && units * 3 <= target) nw = 3;
  }
  s.waves = nw;
  int64_t n = 1;
  if (units * nw < target) {
    n = ceil_div(target, units * nw);
    n = std::min<int64_t>(n, tiles / (2 * nw));
  }
  if (p.desc.max_splits > 0) n = std::min<int64_t>(n, p.desc.max_splits);
  n = std::max<int64_t>(n, 1);
  const int64_t tps = ceil_div(tiles, n);
  s.tiles_per_split = static_cast<int32_t>(tps);
  s.n_split = static_cast<int32_t>(ceil_div(tiles, tps));
  return s;
}

Split explicit_split(const lr_attn_plan& p, int32_t layer, int32_t max_len) {
  // eight wavefronts only in the 32 bucket (above it the kernel would spill
  // at two wavefronts per SIMD)
  Split s;
  const int64_t units = static_cast<int64_t>(p.desc.batch) * p.desc.n_heads;
  const int64_t tiles = ceil_div(max_len, kTile);
  const bool eight_ok = layer_bucket(p.layers[layer]) == 32;
  s.waves = (eight_ok && units * 4 < 4096 && tiles >= 8) ? 8 : 4;
  if (p.desc.wg_waves == 4 || (p.desc.wg_waves == 8 && eight_ok)) s.waves = p.desc.wg_waves;
  s.n_split = 1;
  s.tiles_per_split = static_cast<int32_t>(tiles);
  return s;
}

size_t workspace_bytes(const lr_attn_plan& p, int32_t max_len) {
  const size_t units = static_cast<size_t>(p.desc.batch) * p.desc.n_heads;
  size_t need = 0;
  for (int l = 0; l < p.desc.n_layers; ++l) {
    const Split s = choose_split(p, l, max_len);
    if (s.n_split > 1)
      need = std::max(need, units * s.n_split * kPartStride * sizeof(float));
  }
  return (need + 255) / 256 * 256;
}

}  // namespace lr

extern "C" {

lr_status lr_attn_plan_create(const lr_attn_desc* d, lr_attn_plan** out) {
  if (!d || !out) return LR_EINVAL;
  *out = nullptr;
  if (!d->rank_k || !d->rank_v) return LR_EINVAL;
  if (d->n_layers < 1 || d->batch < 1 || d->n_heads < 1 || d->capacity < 1) return LR_EINVAL;
  if (d->qfmt != LR_Q_INT8_TOKEN && d->qfmt != LR_Q_INT4_G32) return LR_EINVAL;
  if (d->io_dtype != LR_DT_BF16 && d->io_dtype != LR_DT_F32) return LR_EINVAL;
  if (d->max_splits < 0) return LR_EINVAL;
  if (d->wg_waves != 0 && d->wg_waves != 4 && d->wg_waves != 8 && d->wg_waves != 16) return LR_EINVAL;
  if (d->reserved != 0) return LR_EINVAL;
  if (d->head_dim != LR_HEAD_DIM) return LR_EUNSUPPORTED;
  if (d->n_heads > LR_MAX_HEADS) return LR_EUNSUPPORTED;
  if (d->capacity > (1 << 24)) return LR_ERANGE;
  if (static_cast<int64_t>(d->batch) * d->n_heads > (1 << 24)) return LR_ERANGE;
  const int64_t n = static_cast<int64_t>(d->n_layers) * d->n_heads;
  for (int64_t i = 0; i < n; ++i)
    if (!rank_ok(d->rank_k[i]) || !rank_ok(d->rank_v[i])) return LR_EUNSUPPORTED;

  lr_attn_plan* p = new (std::nothrow) lr_attn_plan();
  if (!p) return LR_EINVAL;
  p->desc = *d;
  p->desc.rank_k = nullptr;
  p->desc.rank_v = nullptr;
  p->n_tiles = lr::n_tiles(d->capacity);
  const int H = d->n_heads;
  p->layers.resize(d->n_layers);
  for (int l = 0; l < d->n_layers; ++l) {
    auto& L = p->layers[l];
    std::memset(&L.tab, 0, sizeof(L.tab));
    L.heads.resize(H);
    uint64_t off = 0;
    int32_t lk = 0, lv = 0;
    L.rk_max = L.rv_max = 0;
    for (int h = 0; h < H; ++h) {
      const int rk = d->rank_k[static_cast<int64_t>(l) * H + h];
      const int rv = d->rank_v[static_cast<int64_t>(l) * H + h];
      auto& hl = L.heads[h];
      hl.rank_k = rk;
      hl.rank_v = rv;
      hl.row_bytes_k = lr::row_bytes(d->qfmt, rk);
      hl.row_bytes_v = lr::row_bytes(d->qfmt, rv);
      hl.scale_bytes_k = lr::scale_bytes(d->qfmt, rk);
      hl.scale_bytes_v = lr::scale_bytes(d->qfmt, rv);
      hl.tile_bytes_k = lr::tile_bytes(d->qfmt, rk);
      hl.tile_bytes_v = lr::tile_bytes(d->qfmt, rv);
      hl.plane_bytes_k = static_cast<uint64_t>(p->n_tiles) * hl.tile_bytes_k;
      hl.plane_bytes_v = static_cast<uint64_t>(p->n_tiles) * hl.tile_bytes_v;
      hl.latent_offset_k = lk;
      hl.latent_offset_v = lv;
      hl.factor_offset_k = static_cast<int64_t>(lk) * LR_HEAD_DIM;
      hl.factor_offset_v = static_cast<int64_t>(lv) * LR_HEAD_DIM;
      hl.k_offset = off;
      off += (hl.plane_bytes_k * d->batch + lr::kRegionAlign - 1) / lr::kRegionAlign * lr::kRegionAlign;
      hl.v_offset = off;
      off += (hl.plane_bytes_v * d->batch + lr::kRegionAlign - 1) / lr::kRegionAlign * lr::kRegionAlign;
      if (off / lr::kRegionAlign > 0xffffffffull) { delete p; return LR_ERANGE; }
      L.tab.kreg[h] = static_cast<uint32_t>(hl.k_offset / lr::kRegionAlign);
      L.tab.vreg[h] = static_cast<uint32_t>(hl.v_offset / lr::kRegionAlign);
      L.tab.ranks[h] = static_cast<uint32_t>(rk) | (static_cast<uint32_t>(rv) << 16);
      L.tab.loff[h] = static_cast<uint32_t>(lk) | (static_cast<uint32_t>(lv) << 16);
      lk += rk;
      lv += rv;
      L.rk_max = std::max(L.rk_max, rk);
      L.rv_max = std::max(L.rv_max, rv);
    }
    L.sum_rk = lk;
    L.sum_rv = lv;
    L.cache_bytes = off;
    // Heavy heads (more bytes per token) are dispatched first so the tail of
    // the launch is made of light work-groups (non-uniform ranks).
    std::vector<int> order(H);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      const int wa = L.heads[a].tile_bytes_k + L.heads[a].tile_bytes_v;
      const int wb = L.heads[b].tile_bytes_k + L.heads[b].tile_bytes_v;
      return wa > wb;
    });
    for (int i = 0; i < H; ++i) L.tab.order[i] = static_cast<uint32_t>(order[i]);
    // The same order dealt to the XCDs in a snake (0..7, then 7..0, ...): equal
    // head counts per XCD and near-equal bytes (used when H % 8 == 0).
    for (int i = 0; i < H; ++i) {
      const int r = i / 8, x = i % 8;
      const int src = (H % 8 == 0) ? r * 8 + ((r & 1) ? 7 - x : x) : i;
      L.tab.xorder[i] = static_cast<uint32_t>(order[src]);
    }
  }
  *out = p;
  return LR_OK;
}

void lr_attn_plan_destroy(lr_attn_plan* p) { delete p; }

size_t lr_attn_cache_bytes(const lr_attn_plan* p, int32_t layer) {
  if (!p || layer < 0 || layer >= p->desc.n_layers) return 0;
  return p->layers[layer].cache_bytes;
}

size_t lr_attn_latent_elems(const lr_attn_plan* p, int32_t layer, int32_t kv) {
  if (!p || layer < 0 || layer >= p->desc.n_layers || (kv != 0 && kv != 1)) return 0;
  return static_cast<size_t>(kv == 0 ? p->layers[layer].sum_rk : p->layers[layer].sum_rv);
}

size_t lr_attn_factor_elems(const lr_attn_plan* p, int32_t layer, int32_t kv) {
  return lr_attn_latent_elems(p, layer, kv) * LR_HEAD_DIM;
}

lr_status lr_attn_head_layout_get(const lr_attn_plan* p, int32_t layer, int32_t head,
                                  lr_attn_head_layout* out) {
  if (!p || !out) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers || head < 0 || head >= p->desc.n_heads)
    return LR_ERANGE;
  *out = p->layers[layer].heads[head];
  return LR_OK;
}

size_t lr_attn_workspace_bytes(const lr_attn_plan* p, int32_t max_len) {
  if (!p || max_len < 1 || max_len > p->desc.capacity) return 0;
  return lr::workspace_bytes(*p, max_len);
}

namespace {
// The append launch has 32 threads per (kv, head, sequence, token) row in one
// grid dimension, which holds fewer than 2^32 threads: batch x heads x n_new
// is limited to 2^26.
bool append_fits(const lr_attn_plan& p, int32_t n_new) {
  return int64_t(p.desc.batch) * p.desc.n_heads * n_new <= (int64_t(1) << 26);
}
}  // namespace

lr_status lr_attn_append_latent(const lr_attn_plan* p, int32_t layer, void* cache, const float* ck,
                                const float* cv, const int32_t* pos, int32_t n_new, void* stream) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (n_new < 0) return LR_EINVAL;
  if (n_new > p->desc.capacity || !append_fits(*p, n_new)) return LR_ERANGE;
  if (!cache || !ck || !cv || !pos) return LR_EINVAL;
  if (!aligned(cache, 256) || !aligned(ck, 16) || !aligned(cv, 16) || !aligned(pos, 4))
    return LR_EINVAL;
  if (n_new == 0) return LR_OK;
  return hip_status(lr::launch_append(*p, layer, cache, ck, cv, pos, n_new, stream));
}

namespace {

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Bytes of the fp32 latents of n tokens of one layer, K then V, each 256-aligned.
size_t latent_ws_bytes(const lr_attn_plan::Layer& L, size_t n) {
  return round256(n * L.sum_rk * sizeof(float)) + round256(n * L.sum_rv * sizeof(float));
}

lr_status check_project(const lr_attn_plan* p, int32_t layer, const void* x, int32_t embed,
                        const void* packed) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (embed < 32 || embed % 32 != 0) return LR_EINVAL;
  if (!x || !packed) return LR_EINVAL;
  if (!aligned(x, 16) || !aligned(packed, 16)) return LR_EINVAL;
  return LR_OK;
}

}  // namespace

size_t lr_attn_packed_projection_elems(const lr_attn_plan* p, int32_t layer, int32_t embed) {
  if (!p || layer < 0 || layer >= p->desc.n_layers || embed < 32 || embed % 32 != 0) return 0;
  return lr::packed_projection_elems(*p, layer, embed);
}

lr_status lr_attn_pack_projection(const lr_attn_plan* p, int32_t layer, int32_t embed, const void* wk,
                                  const void* wv, void* packed, void* stream) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (embed < 32 || embed % 32 != 0) return LR_EINVAL;
  if (!wk || !wv || !packed) return LR_EINVAL;
  if (!aligned(wk, 16) || !aligned(wv, 16) || !aligned(packed, 16)) return LR_EINVAL;
  return hip_status(lr::launch_pack_projection(*p, layer, embed, wk, wv, packed, stream));
}

lr_status lr_attn_project_latent(const lr_attn_plan* p, int32_t layer, const void* x,
                                 int32_t n_tokens, int32_t embed, const void* packed, float* ck,
                                 float* cv, void* stream) {
  const lr_status st = check_project(p, layer, x, embed, packed);
  if (st != LR_OK) return st;
  if (n_tokens < 0 || !ck || !cv || !aligned(ck, 16) || !aligned(cv, 16)) return LR_EINVAL;
  if (n_tokens == 0) return LR_OK;
  return hip_status(lr::launch_project(*p, layer, x, n_tokens, embed, packed, ck, cv, stream));
}

int32_t lr_attn_project_parts(const lr_attn_plan* p, int32_t layer, int32_t n_tokens, int32_t embed) {
  if (!p || layer < 0 || layer >= p->desc.n_layers || n_tokens < 1 || embed < 32 || embed % 32 != 0)
    return 0;
  return lr::project_parts(*p, layer, n_tokens, embed);
}

lr_status lr_attn_project_latent_parts(const lr_attn_plan* p, int32_t layer, const void* x,
                                       int32_t n_tokens, int32_t embed, const void* packed,
                                       int32_t n_parts, float* ck, float* cv, void* stream) {
  const lr_status st = check_project(p, layer, x, embed, packed);
  if (st != LR_OK) return st;
  if (n_tokens < 0 || !ck || !cv || !aligned(ck, 16) || !aligned(cv, 16)) return LR_EINVAL;
  if (n_parts < 1 || n_parts > lr::kMaxProjectParts || n_parts > embed / 32) return LR_EINVAL;
  if (n_tokens == 0) return LR_OK;
  return hip_status(lr::launch_project(*p, layer, x, n_tokens, embed, packed, ck, cv, stream, n_parts));
}

size_t lr_attn_project_workspace_bytes(const lr_attn_plan* p, int32_t n_new) {
  if (!p || n_new < 1 || n_new > p->desc.capacity) return 0;
  size_t best = 0;
  const size_t n = static_cast<size_t>(p->desc.batch) * static_cast<size_t>(n_new);
  for (const auto& L : p->layers) best = std::max(best, latent_ws_bytes(L, n));
  return best;
}

lr_status lr_attn_project_append(const lr_attn_plan* p, int32_t layer, void* cache, const void* x,
                                 int32_t embed, const void* packed, const int32_t* pos,
                                 int32_t n_new, void* ws, size_t ws_bytes, void* stream) {
  const lr_status st = check_project(p, layer, x, embed, packed);
  if (st != LR_OK) return st;
  if (n_new < 0) return LR_EINVAL;
  if (n_new > p->desc.capacity || !append_fits(*p, n_new)) return LR_ERANGE;
  if (!cache || !pos || !aligned(cache, 256) || !aligned(pos, 4)) return LR_EINVAL;
  if (n_new == 0) return LR_OK;
  const auto& L = p->layers[layer];
  const size_t n = static_cast<size_t>(p->desc.batch) * static_cast<size_t>(n_new);
  if (n > static_cast<size_t>(INT32_MAX)) return LR_ERANGE;
  if (!ws || ws_bytes < latent_ws_bytes(L, n)) return LR_EWORKSPACE;
  if (!aligned(ws, 256)) return LR_EINVAL;
  float* ck = static_cast<float*>(ws);
  float* cv = reinterpret_cast<float*>(static_cast<char*>(ws) + round256(n * L.sum_rk * sizeof(float)));
  const lr_status s1 = hip_status(lr::launch_project(*p, layer, x, static_cast<int32_t>(n), embed,
                                                     packed, ck, cv, stream));
  if (s1 != LR_OK) return s1;
  return hip_status(lr::launch_append(*p, layer, cache, ck, cv, pos, n_new, stream));
}

namespace {
// A launch's threads are counted in 32 bits: the decode grid (units x splits
// work-groups of waves x 64 threads) and the merge grid (units x 512) must
// each hold fewer than 2^32 threads.
bool decode_fits(const lr_attn_plan& p, int32_t layer, int32_t max_len, bool explicit_form) {
  const lr::Split s = explicit_form ? lr::explicit_split(p, layer, max_len) : lr::choose_split(p, layer, max_len);
  const uint64_t units = static_cast<uint64_t>(p.desc.batch) * static_cast<uint64_t>(p.desc.n_heads);
  const uint64_t limit = 0xffffffffull;
  if (units * static_cast<uint64_t>(s.n_split) * static_cast<uint64_t>(s.waves) * 64u > limit) return false;
  return s.n_split == 1 || units * 512u <= limit;
}
}  // namespace

// Every check of a decode call, in the order the errors are reported.
static lr_status decode_check(const lr_attn_plan* p, int32_t layer, const void* cache,
                              const int32_t* len, int32_t max_len, const void* q, const void* bk,
                              const void* bv, float scale, void* out, void* ws, size_t ws_bytes,
                              bool explicit_form) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (max_len < 1 || max_len > p->desc.capacity) return LR_ERANGE;
  if (!cache || !len || !q || !bk || !bv || !out) return LR_EINVAL;
  if (!std::isfinite(scale)) return LR_EINVAL;
  if (!aligned(cache, 256) || !aligned(len, 4) || !aligned(q, 16) || !aligned(bk, 16) ||
      !aligned(bv, 16) || !aligned(out, 16))
    return LR_EINVAL;
  if (explicit_form && p->desc.io_dtype != LR_DT_BF16) return LR_EUNSUPPORTED;
  if (!decode_fits(*p, layer, max_len, explicit_form)) return LR_ERANGE;
  const size_t need = explicit_form ? 0 : lr::workspace_bytes(*p, max_len);
  if (need > 0 && (!ws || ws_bytes < need)) return LR_EWORKSPACE;
  if (ws && !aligned(ws, 16)) return LR_EINVAL;
  return LR_OK;
}

static lr_status decode_common(const lr_attn_plan* p, int32_t layer, const void* cache,
                               const int32_t* len, int32_t max_len, const void* q,
                               const void* bk, const void* bv, float scale, void* out,
                               void* ws, size_t ws_bytes, void* stream, bool explicit_form,
                               const lr::AppendInputs* app = nullptr) {
  const lr_status st = decode_check(p, layer, cache, len, max_len, q, bk, bv, scale, out, ws,
                                    ws_bytes, explicit_form);
  if (st != LR_OK) return st;
  const size_t need = explicit_form ? 0 : lr::workspace_bytes(*p, max_len);
  return hip_status(lr::launch_decode(*p, layer, cache, len, max_len, q, bk, bv, scale, out,
                                      need > 0 ? ws : nullptr, stream, explicit_form, app));
}

lr_status lr_attn_decode(const lr_attn_plan* p, int32_t layer, const void* cache,
                         const int32_t* len, int32_t max_len, const void* q, const void* bk,
                         const void* bv, float scale, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  return decode_common(p, layer, cache, len, max_len, q, bk, bv, scale, out, ws, ws_bytes, stream,
                       false);
}

lr_status lr_attn_append_decode(const lr_attn_plan* p, int32_t layer, void* cache, const float* ck,
                                const float* cv, const int32_t* pos, const int32_t* len,
                                int32_t max_len, const void* q, const void* bk, const void* bv,
                                float scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (!ck || !cv || !pos) return LR_EINVAL;
  if (!aligned(ck, 16) || !aligned(cv, 16) || !aligned(pos, 4)) return LR_EINVAL;
  const lr::AppendInputs app{cache, ck, cv, pos};
  return decode_common(p, layer, cache, len, max_len, q, bk, bv, scale, out, ws, ws_bytes, stream,
                       false, &app);
}

namespace {
// Bytes of the projection partials of one decode step of a layer (one token
// per sequence): n_parts blocks of [batch][sum_r] fp32, K then V, 256-aligned.
size_t step_partials_bytes(const lr_attn_plan& p, int32_t layer, int32_t embed) {
  const size_t parts = static_cast<size_t>(lr::project_parts(p, layer, p.desc.batch, embed));
  return latent_ws_bytes(p.layers[layer], parts * static_cast<size_t>(p.desc.batch));
}
}  // namespace

size_t lr_attn_project_decode_workspace_bytes(const lr_attn_plan* p, int32_t max_len, int32_t embed) {
  if (!p || max_len < 1 || max_len > p->desc.capacity || embed < 32 || embed % 32 != 0) return 0;
  size_t best = 0;
  for (int32_t l = 0; l < p->desc.n_layers; ++l) best = std::max(best, step_partials_bytes(*p, l, embed));
  return best + lr::workspace_bytes(*p, max_len);
}

lr_status lr_attn_project_append_decode(const lr_attn_plan* p, int32_t layer, void* cache,
                                        const void* x, int32_t embed, const void* packed,
                                        const int32_t* pos, const int32_t* len, int32_t max_len,
                                        const void* q, const void* bk, const void* bv, float scale,
                                        void* out, void* ws, size_t ws_bytes, void* stream) {
  lr_status st = check_project(p, layer, x, embed, packed);
  if (st != LR_OK) return st;
  if (!pos || !aligned(pos, 4)) return LR_EINVAL;
  if (!ws || !aligned(ws, 256)) return ws ? LR_EINVAL : LR_EWORKSPACE;
  const size_t pbytes = step_partials_bytes(*p, layer, embed);
  if (ws_bytes < pbytes) return LR_EWORKSPACE;
  void* dws = static_cast<char*>(ws) + pbytes;
  st = decode_check(p, layer, cache, len, max_len, q, bk, bv, scale, out, dws, ws_bytes - pbytes, false);
  if (st != LR_OK) return st;
  const auto& L = p->layers[layer];
  const int32_t B = p->desc.batch;
  const int32_t parts = lr::project_parts(*p, layer, B, embed);
  float* pk = static_cast<float*>(ws);
  float* pv = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       round256(static_cast<size_t>(parts) * B * L.sum_rk * sizeof(float)));
  st = hip_status(lr::launch_project(*p, layer, x, B, embed, packed, pk, pv, stream, parts));
  if (st != LR_OK) return st;
  lr::AppendInputs app{cache, pk, pv, pos, parts};
  const size_t need = lr::workspace_bytes(*p, max_len);
  return hip_status(lr::launch_decode(*p, layer, cache, len, max_len, q, bk, bv, scale, out,
                                      need > 0 ? dws : nullptr, stream, false, &app));
}

lr_status lr_attn_append_decode_noalloc(const lr_attn_plan* p, int32_t layer, void* cache,
                                        const float* ck, const float* cv, const int32_t* pos,
                                        const int32_t* len, int32_t max_len, const void* q,
                                        const void* bk, const void* bv, float scale, void* out,
                                        void* stream) {
  if (!p) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if (max_len < 1 || max_len > p->desc.capacity) return LR_ERANGE;
  if (lr::workspace_bytes(*p, max_len) > lr::kScratchBytes) return LR_EWORKSPACE;
  void* ws = nullptr;
  const int e = lr::scratch_address(&ws);
  if (e != 0) return hip_status(e);
  return lr_attn_append_decode(p, layer, cache, ck, cv, pos, len, max_len, q, bk, bv, scale, out,
                               ws, lr::kScratchBytes, stream);
}

lr_status lr_attn_decode_explicit(const lr_attn_plan* p, int32_t layer, const void* cache,
                                  const int32_t* len, int32_t max_len, const void* q,
                                  const void* bk, const void* bv, float scale, void* out,
                                  void* ws, size_t ws_bytes, void* stream) {
  return decode_common(p, layer, cache, len, max_len, q, bk, bv, scale, out, ws, ws_bytes, stream,
                       true);
}

const char* lr_attn_strerror(lr_status s) {
  switch (s) {
    case LR_OK: return "ok";
    case LR_EINVAL: return "invalid argument";
    case LR_EUNSUPPORTED: return "unsupported configuration";
    case LR_ERANGE: return "index or length out of range";
    case LR_EWORKSPACE: return "workspace missing or too small";
    case LR_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t lr_attn_last_hip_error(void) { return g_last_hip; }

lr_status lr_attn_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes < 16 || !aligned(src, 16) || !aligned(sink, 4)) return LR_EINVAL;
  return hip_status(lr::launch_probe_read(src, bytes, sink, stream));
}

}  // extern "C"
