// rotate.cpp -- outlier smoothing between the factors (WSVD page,
// "Quantisation": orthogonal transforms, S_1 a Hadamard matrix, smooth channel
// outliers of the latent; LASER page, "Hybrid SVD-quantisation": a rotation is
// inserted between the SVD factors before round-to-nearest quantisation).
//
// With S orthogonal, A B = (A S)(S^T B): folding S into the factors once
// changes the cached latent to c S and leaves every kernel as it is.  S is
// block-diagonal per head with normalised Hadamard blocks H_g (g the largest
// power of two dividing the head's rank, capped by the caller); H_g is
// symmetric, so S^T = S and both factors take the same row transform.  It is
// applied here on the host, in fp64, with the fast Walsh-Hadamard butterflies
// (x, y) -> (x + y, x - y), which multiply by the Sylvester-ordered H_g.

#include <cmath>
#include <vector>

#include "plan.h"

namespace {

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

}  // namespace

extern "C" {

int32_t lr_attn_hadamard_block(const lr_attn_plan* p, int32_t layer, int32_t kv, int32_t head,
                               int32_t block) {
  if (!p || layer < 0 || layer >= p->desc.n_layers || (kv != 0 && kv != 1) || head < 0 ||
      head >= p->desc.n_heads || !pow2(block) || block < 8 || block > LR_HEAD_DIM)
    return 0;
  const auto& hl = p->layers[layer].heads[head];
  const int r = kv == 0 ? hl.rank_k : hl.rank_v;
  int g = 1;
  while (g * 2 <= block && r % (g * 2) == 0) g *= 2;
  return g;
}

lr_status lr_attn_hadamard_rotate_rows(const lr_attn_plan* p, int32_t layer, int32_t kv,
                                       int32_t block, float* rows, int64_t cols) {
  if (!p || !rows) return LR_EINVAL;
  if (layer < 0 || layer >= p->desc.n_layers) return LR_ERANGE;
  if ((kv != 0 && kv != 1) || !pow2(block) || block < 8 || block > LR_HEAD_DIM || cols < 1)
    return LR_EINVAL;
  const auto& L = p->layers[layer];
  std::vector<double> buf;
  for (int h = 0; h < p->desc.n_heads; ++h) {
    const auto& hl = L.heads[h];
    const int r = kv == 0 ? hl.rank_k : hl.rank_v;
    const int off = kv == 0 ? hl.latent_offset_k : hl.latent_offset_v;
    const int g = lr_attn_hadamard_block(p, layer, kv, h, block);
    const double sc = 1.0 / std::sqrt(static_cast<double>(g));
    buf.assign(static_cast<size_t>(g) * static_cast<size_t>(cols), 0.0);
    for (int b0 = 0; b0 < r; b0 += g) {
      float* blk = rows + static_cast<int64_t>(off + b0) * cols;
      for (size_t i = 0; i < buf.size(); ++i) buf[i] = blk[i];
      for (int len = 1; len < g; len *= 2)
        for (int i0 = 0; i0 < g; i0 += 2 * len)
          for (int i = i0; i < i0 + len; ++i) {
            double* x = buf.data() + static_cast<size_t>(i) * cols;
            double* y = buf.data() + static_cast<size_t>(i + len) * cols;
            for (int64_t c = 0; c < cols; ++c) {
              const double a = x[c], b = y[c];
              x[c] = a + b;
              y[c] = a - b;
            }
          }
      for (size_t i = 0; i < buf.size(); ++i) blk[i] = static_cast<float>(buf[i] * sc);
    }
  }
  return LR_OK;
}

}  // extern "C"
