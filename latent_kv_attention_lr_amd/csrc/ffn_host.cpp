// ffn_host.cpp -- host side of the hybrid low-rank / dense W8A8 FFN (LASER
// page, "Hybrid SVD-quantisation for FFNs"): description checks, weight
// quantisation (int8, one fp32 scale per row, round to nearest even) and
// packing into matrix-core step blocks, workspace sizes, the decode call.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "ffn_lds.h"
#include "plan.h"

namespace {

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

lr_status ffn_layout(const lr_ffn_desc* d, lr::FfnLayout* f) {
  if (!d) return LR_EINVAL;
  if (d->reserved != 0) return LR_EINVAL;
  if (d->embed < 64 || d->embed > 8192 || d->embed % 64 != 0) return LR_EUNSUPPORTED;
  if (d->hidden < 16 || d->hidden % 16 != 0 || d->hidden > (1 << 20)) return LR_EUNSUPPORTED;
  if (d->n_lowrank < 0 || d->n_lowrank > d->hidden || d->n_lowrank % 16 != 0) return LR_EUNSUPPORTED;
  if (d->n_lowrank > 0 ? (d->rank < 64 || d->rank > 4096 || d->rank % 64 != 0) : d->rank != 0)
    return LR_EUNSUPPORTED;
  f->E = d->embed;
  f->F = d->hidden;
  f->S = d->n_lowrank;
  f->r = d->rank;
  f->Fp = (d->hidden + 63) / 64 * 64;
  const size_t D = size_t(f->F - f->S);
  const size_t n1 = 2 * D / 16 + 2 * size_t(f->r) / 16, n2 = 2 * size_t(f->S) / 16, n3 = size_t(f->E) / 16;
  const size_t b1 = n1 * size_t(f->E) * 16, b2 = n2 * size_t(f->r) * 16, b3 = n3 * size_t(f->Fp) * 16;
  f->off_w1 = 0;
  f->off_w2 = align256(b1);
  f->off_w3 = f->off_w2 + align256(b2);
  f->off_s1 = f->off_w3 + align256(b3);
  f->off_s2 = f->off_s1 + align256(n1 * 16 * 4);
  f->off_s3 = f->off_s2 + align256(n2 * 16 * 4);
  f->weight_bytes = f->off_s3 + align256(n3 * 16 * 4);
  return LR_OK;
}

void ffn_workspace(lr::FfnLayout* f, size_t T) {
  const size_t E = size_t(f->E), r2 = 2 * size_t(f->r), F = size_t(f->F), Fp = size_t(f->Fp);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  const lr::ffnlds::OutShape osh = lr::ffnlds::out_shape(f->Fp);   // the down projection's chunks
  const size_t splits = size_t(osh.splits), rt = size_t(osh.rt), TB = (T + 15) / 16;
  f->out_splits = osh.splits;
  f->out_rt = osh.rt;
  // counters, per block of 16 tokens: halves done per latent group, pair
  // work-groups done per group of h, chunks done per down-projection row tile
  f->ws_cnt_bytes = 4 * TB * (r2 / 64 + Fp / 64 + E / (16 * rt));
  f->ws_cnt = take(f->ws_cnt_bytes);
  f->ws_xq = take(T * E);
  f->ws_xs = take(T * (E / 64) * 4);
  f->ws_zp = take(2 * T * r2 * 4);   // the two halves' partial latents
  f->ws_zq = take(T * r2);
  f->ws_zs = take(T * (r2 / 64) * 4);
  // h rows padded to whole 128-byte lines, so a line never holds two groups
  f->h_ld = int32_t((F + 31) / 32 * 32);
  f->ws_h = take(T * size_t(f->h_ld) * 4);
  f->ws_hq = take(T * Fp);
  f->ws_hs = take(T * (Fp / 64) * 4);
  f->ws_yp = take(splits > 1 ? splits * T * E * 4 : 0);   // partial sums of the down projection
  f->ws_bytes = o;
}

// Tokens per pass of the launches: a multiple of 16 such that no launch of a
// pass has more than 2^16 work-groups.  Work-groups per 16 tokens, per launch:
// quantise x E / 16; k_ffn_in (F - S) / 16 + r / 16; k_ffn_mid S / 16;
// k_ffn_out at most E / 16 per chunk.  (The bound keeps the terms r / 8 and
// Fp / 16 of launches since merged, so pass sizes are unchanged.)
size_t ffn_pass_tokens(const lr::FfnLayout& f) {
  const size_t E = size_t(f.E), F = size_t(f.F), S = size_t(f.S), r = size_t(f.r), Fp = size_t(f.Fp);
  const size_t chunks = size_t(lr::ffnlds::out_shape(f.Fp).splits);
  const size_t u = std::max({E / 16 * chunks, r / 8, Fp / 16, (F - S) / 16 + r / 16, S / 16});
  return 16 * std::max<size_t>(1, (size_t(1) << 16) / u);
}

// One row: s = max|w| / 127 (fp32), codes clamp(rne(w / s), -127, 127), 0 if s == 0.
float quant_row(const float* w, int n, int8_t* q) {
  float m = 0.0f;
  for (int i = 0; i < n; ++i) m = std::fmax(m, std::fabs(w[i]));
  const float s = m / 127.0f;
  for (int i = 0; i < n; ++i) {
    float v = s != 0.0f ? std::rint(w[i] / s) : 0.0f;
    v = v < -127.0f ? -127.0f : (v > 127.0f ? 127.0f : v);
    q[i] = static_cast<int8_t>(v);
  }
  return s;
}

// Quantise rows row0 .. row0 + 15 of M [rows][K] and pack them as one tile of
// Kp / 64 steps: byte j of lane l of step c is row row0 + (l & 15), column
// 64 c + 16 (l >> 4) + j (zero past K); scales to sc[0 .. 15].
void pack_tile(const float* M, int rows, int K, int Kp, int row0, uint8_t* dst, float* sc) {
  std::vector<int8_t> q(size_t(16) * Kp, 0);
  for (int i = 0; i < 16; ++i) {
    const int row = row0 + i;
    sc[i] = row < rows ? quant_row(M + size_t(row) * K, K, q.data() + size_t(i) * Kp) : 0.0f;
  }
  for (int c = 0; c < Kp / 64; ++c)
    for (int l = 0; l < 64; ++l)
      std::memcpy(dst + size_t(c) * 1024 + 16 * l, q.data() + size_t(l & 15) * Kp + 64 * c + 16 * (l >> 4), 16);
}

}  // namespace

extern "C" {

size_t lr_ffn_weight_bytes(const lr_ffn_desc* d) {
  lr::FfnLayout f;
  return ffn_layout(d, &f) == LR_OK ? f.weight_bytes : 0;
}

size_t lr_ffn_workspace_bytes(const lr_ffn_desc* d, int32_t n_tokens) {
  lr::FfnLayout f;
  if (ffn_layout(d, &f) != LR_OK || n_tokens < 1 || n_tokens > (1 << 20)) return 0;
  ffn_workspace(&f, std::min(size_t(n_tokens), ffn_pass_tokens(f)));
  return f.ws_bytes;
}

lr_status lr_ffn_prepare_weights(const lr_ffn_desc* d, const float* wg, const float* wu, const float* ag,
                                 const float* au, const float* bg, const float* bu, const float* wd,
                                 void* out) {
  lr::FfnLayout f;
  const lr_status st = ffn_layout(d, &f);
  if (st != LR_OK) return st;
  const int D = f.F - f.S;
  if (!out || !wd || (D > 0 && (!wg || !wu)) || (f.S > 0 && (!ag || !au || !bg || !bu))) return LR_EINVAL;
  auto finite = [](const float* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
      if (!std::isfinite(p[i])) return false;
    return true;
  };
  if (!finite(wd, size_t(f.E) * f.F) || (D > 0 && (!finite(wg, size_t(D) * f.E) || !finite(wu, size_t(D) * f.E))) ||
      (f.S > 0 && (!finite(ag, size_t(f.r) * f.E) || !finite(au, size_t(f.r) * f.E) ||
                   !finite(bg, size_t(f.S) * f.r) || !finite(bu, size_t(f.S) * f.r))))
    return LR_EINVAL;
  uint8_t* o = static_cast<uint8_t*>(out);
  std::memset(o, 0, f.weight_bytes);
  // section 1: dense pairs (W_g, W_u rows of channels S + 16 p ..), then [A_g; A_u]
  const size_t t1 = size_t(f.E) * 16;
  float* s1 = reinterpret_cast<float*>(o + f.off_s1);
  size_t tile = 0;
  for (int p = 0; p < D / 16; ++p) {
    pack_tile(wg, D, f.E, f.E, 16 * p, o + f.off_w1 + tile * t1, s1 + 16 * tile);
    ++tile;
    pack_tile(wu, D, f.E, f.E, 16 * p, o + f.off_w1 + tile * t1, s1 + 16 * tile);
    ++tile;
  }
  for (int j = 0; j < 2 * f.r / 16; ++j, ++tile) {
    const bool up = 16 * j >= f.r;
    pack_tile(up ? au : ag, f.r, f.E, f.E, 16 * j - (up ? f.r : 0), o + f.off_w1 + tile * t1, s1 + 16 * tile);
  }
  // section 2: low-rank pairs (B_g, B_u rows of channels 16 p ..), k = r
  const size_t t2 = size_t(f.r) * 16;
  float* s2 = reinterpret_cast<float*>(o + f.off_s2);
  tile = 0;
  for (int p = 0; p < f.S / 16; ++p) {
    pack_tile(bg, f.S, f.r, f.r, 16 * p, o + f.off_w2 + tile * t2, s2 + 16 * tile);
    ++tile;
    pack_tile(bu, f.S, f.r, f.r, 16 * p, o + f.off_w2 + tile * t2, s2 + 16 * tile);
    ++tile;
  }
  // section 3: W_d rows, k = F padded to Fp
  const size_t t3 = size_t(f.Fp) * 16;
  float* s3 = reinterpret_cast<float*>(o + f.off_s3);
  for (int e = 0; e < f.E / 16; ++e) pack_tile(wd, f.E, f.F, f.Fp, 16 * e, o + f.off_w3 + e * t3, s3 + 16 * e);
  return LR_OK;
}

lr_status lr_ffn_decode(const lr_ffn_desc* d, const void* weights, const void* x, int32_t n_tokens, float* y,
                        void* workspace, size_t ws_bytes, void* stream) {
  lr::FfnLayout f;
  const lr_status st = ffn_layout(d, &f);
  if (st != LR_OK) return st;
  if (n_tokens < 0 || n_tokens > (1 << 20)) return LR_ERANGE;
  if (!weights || !x || !y) return LR_EINVAL;
  auto al = [](const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
  if (!al(weights, 256) || !al(x, 16) || !al(y, 16)) return LR_EINVAL;
  if (n_tokens == 0) return LR_OK;
  const size_t T = size_t(n_tokens), pass = ffn_pass_tokens(f);
  ffn_workspace(&f, std::min(T, pass));
  if (!workspace || ws_bytes < f.ws_bytes) return LR_EWORKSPACE;
  if (!al(workspace, 256)) return LR_EINVAL;
  // passes run in order on one stream and reuse the workspace
  for (size_t t0 = 0; t0 < T; t0 += pass) {
    const int err = lr::launch_ffn(f, weights, static_cast<const uint16_t*>(x) + t0 * size_t(f.E),
                                   int32_t(std::min(pass, T - t0)), y + t0 * size_t(f.E), workspace, stream);
    if (err != 0) {
      lr::set_last_hip_error(err);
      return LR_EHIP;
    }
  }
  return LR_OK;
}

}  // extern "C"
