// lr_oracle.cpp -- CPU oracle for the decode step of per-head low-rank
// attention over a quantised latent KV cache.
//
// TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the package
// smoke check and the benchmark's CPU-baseline leg may load this library.  It
// shares no code, header, table or helper with the GPU library.
//
// It computes the plain definition, slowly and in the pages' order:
//   * per head h, keys and values are kept only as rank-r latents c_t = x_t A_h,
//     generated from the activations by lro_latents (WSVD page, "Fine-grained
//     per-head SVD": each head owns a small latent and its own factors,
//     W_h ~ A_h B_h);
//   * the latents are stored at low precision with round-to-nearest
//     quantisation (LASER page, "Hybrid SVD-quantisation ... RTN"; WSVD page,
//     "Quantisation": W8A8 / W8A4 activations);
//   * at decode time K_h and V_h are rebuilt from the latents through B_h and
//     ordinary softmax attention is taken: Q K^T, softmax, times V (WSVD page,
//     "System implementation (fused kernel)": low-rank reconstruction followed
//     by the QK product, softmax and V product).
// It never uses the absorbed form, never tiles, never splits the context and
// keeps every floating-point step after quantisation in fp64.  The quantiser
// works in fp32 because its fp32 arithmetic is its definition:
//   int8, per token:  m = max|c_i|, s = m / 127 (fp32 division),
//                     q_i = clamp(rne(c_i / s), -127, 127), or 0 when s == 0.
//   int4, group 32:   per group g of up to 32 consecutive ranks,
//                     s_g = fp16_rne(m_g / 7), q_i = clamp(rne(c_i / s_g), -7, 7),
//                     or 0 when s_g == 0 (also when m_g/7 underflows in fp16).
// Readings of points the pages leave open (tie rule, clamp range, what is
// divided, scale dtypes, group tail) are the plainest ones: round half to
// even, symmetric ranges, division by the stored scale, fp32 per-token scale,
// fp16 per-group scale, a short last group with its own scale.
//
// Build: g++ -O2 -fno-fast-math -ffp-contract=off -shared -fPIC (SSE math).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace

extern "C" {

// IEEE-754 binary32 -> binary16, round to nearest, ties to even; subnormal
// results are produced, magnitudes that round beyond 65504 give infinity, NaN
// stays NaN.  Written from the format definition: a binary16 value is
// (-1)^s * 2^(e-15) * (1 + f/1024) for 1 <= e <= 30, and 2^-14 * f/1024 for e = 0.
uint16_t lro_f32_to_f16(float x) {
  uint32_t bits;
  std::memcpy(&bits, &x, 4);
  const uint16_t sign = static_cast<uint16_t>((bits >> 16) & 0x8000u);
  if (std::isnan(x)) return static_cast<uint16_t>(sign | 0x7e00u);
  const double a = std::fabs(static_cast<double>(x));  // exact widening
  if (std::isinf(x) || a >= 65520.0) return static_cast<uint16_t>(sign | 0x7c00u);
  if (a < std::ldexp(1.0, -14)) {
    // subnormal range: value = n * 2^-24, n = rne(a / 2^-24); n == 1024 is the
    // smallest normal and has exactly that bit pattern.
    const double n = std::nearbyint(a / std::ldexp(1.0, -24));
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(n));
  }
  int k;
  (void)std::frexp(a, &k);            // a = f * 2^k, f in [0.5, 1)
  int e = k - 1;                      // a in [2^e, 2^(e+1))
  double n = std::nearbyint(a / std::ldexp(1.0, e - 10));  // in [1024, 2048]
  if (n == 2048.0) { n = 1024.0; e += 1; }
  if (e > 15) return static_cast<uint16_t>(sign | 0x7c00u);
  return static_cast<uint16_t>(sign | ((e + 15) << 10) | (static_cast<int>(n) - 1024));
}

// binary16 -> binary32, exact.
float lro_f16_to_f32(uint16_t h) {
  const int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0) v = std::ldexp(static_cast<double>(f), -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = std::ldexp(1024.0 + f, e - 25);
  return static_cast<float>(s ? -v : v);
}

// Symmetric int8 quantisation of one latent row with one fp32 scale.
void lro_quant_int8(const float* c, int r, int8_t* q, float* scale) {
  float m = 0.0f;
  for (int i = 0; i < r; ++i) m = std::fmax(m, std::fabs(c[i]));
  const float s = m / 127.0f;
  *scale = s;
  for (int i = 0; i < r; ++i) {
    if (s == 0.0f) { q[i] = 0; continue; }
    q[i] = static_cast<int8_t>(clampf(std::nearbyint(c[i] / s), -127.0f, 127.0f));
  }
}

// Symmetric int4 quantisation of one latent row, one fp16 scale per group of
// 32 consecutive ranks (the last group may be shorter).  q holds one value
// per element in [-7, 7]; scales holds ceil(r/32) binary16 bit patterns.
void lro_quant_int4(const float* c, int r, int8_t* q, uint16_t* scales) {
  for (int g = 0; g * 32 < r; ++g) {
    const int lo = g * 32, hi = (lo + 32 < r) ? lo + 32 : r;
    float m = 0.0f;
    for (int i = lo; i < hi; ++i) m = std::fmax(m, std::fabs(c[i]));
    const uint16_t sh = lro_f32_to_f16(m / 7.0f);
    scales[g] = sh;
    const float s = lro_f16_to_f32(sh);
    for (int i = lo; i < hi; ++i) {
      if (s == 0.0f) { q[i] = 0; continue; }
      q[i] = static_cast<int8_t>(clampf(std::nearbyint(c[i] / s), -7.0f, 7.0f));
    }
  }
}

// The two quantisers applied to n consecutive rows of r values (a plain loop).
void lro_quant_int8_rows(const float* c, int n, int r, int8_t* q, float* scales) {
  for (int i = 0; i < n; ++i)
    lro_quant_int8(c + static_cast<size_t>(i) * r, r, q + static_cast<size_t>(i) * r, scales + i);
}

void lro_quant_int4_rows(const float* c, int n, int r, int8_t* q, uint16_t* scales) {
  const int ng = (r + 31) / 32;
  for (int i = 0; i < n; ++i)
    lro_quant_int4(c + static_cast<size_t>(i) * r, r, q + static_cast<size_t>(i) * r,
                   scales + static_cast<size_t>(i) * ng);
}

// Latent generation (WSVD page, "Fine-grained per-head SVD": the cached
// latent of token t for head h is c_t = x_t A_h, A_h the E x r down-projection
// factor):  c[t][n] = sum_e x[t][e] * a[e][n]  for x [T][E], a [E][N], in fp64,
// e ascending.  Heads side by side in a (head h's r_h columns after those of
// heads 0 .. h-1) give every head's latent of a token at once.
// Returns 0, or -1 on bad sizes.
int lro_latents(int T, int E, int N, const double* x, const double* a, double* c) {
  if (T < 0 || E < 1 || N < 1) return -1;
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int e = 0; e < E; ++e)
        acc += x[static_cast<size_t>(t) * E + e] * a[static_cast<size_t>(e) * N + n];
      c[static_cast<size_t>(t) * N + n] = acc;
    }
  }
  return 0;
}

// Outlier smoothing by an orthogonal rotation between the factors (WSVD page,
// "Quantisation": orthogonal S_1, S_2 with S_1 a Hadamard matrix smooth
// channel outliers of the latent; LASER page, "Hybrid SVD-quantisation": a
// rotation inserted between the SVD factors before RTN).  With S orthogonal,
// W = A B = (A S)(S^T B): the latent becomes c S and the product is unchanged.
//
// Normalised Sylvester-Hadamard matrix of order n (a power of two):
// H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]], then scaled by 1/sqrt(n), so
// that H H^T = I.  Returns 0, or -1 if n is not a power of two.
int lro_hadamard(int n, double* h) {
  if (n < 1 || (n & (n - 1)) != 0) return -1;
  h[0] = 1.0;
  for (int k = 1; k < n; k *= 2) {
    // grow the top-left k x k block (row stride n) into 2k x 2k
    for (int i = 0; i < k; ++i)
      for (int j = 0; j < k; ++j) {
        const double v = h[static_cast<size_t>(i) * n + j];
        h[static_cast<size_t>(i) * n + j + k] = v;
        h[static_cast<size_t>(i + k) * n + j] = v;
        h[static_cast<size_t>(i + k) * n + j + k] = -v;
      }
  }
  const double sc = 1.0 / std::sqrt(static_cast<double>(n));
  for (size_t i = 0; i < static_cast<size_t>(n) * n; ++i) h[i] *= sc;
  return 0;
}

// The rotation of a rank-r head: block-diagonal with blocks H_g, g the
// largest power of two that divides r and does not exceed `block` (a power of
// two); s is r x r.  Returns g, or -1 on bad arguments.
int lro_block_rotation(int r, int block, double* s) {
  if (r < 1 || block < 1 || (block & (block - 1)) != 0) return -1;
  int g = 1;
  while (g * 2 <= block && r % (g * 2) == 0) g *= 2;
  std::vector<double> h(static_cast<size_t>(g) * g);
  lro_hadamard(g, h.data());
  for (size_t i = 0; i < static_cast<size_t>(r) * r; ++i) s[i] = 0.0;
  for (int b0 = 0; b0 < r; b0 += g)
    for (int i = 0; i < g; ++i)
      for (int j = 0; j < g; ++j)
        s[static_cast<size_t>(b0 + i) * r + b0 + j] = h[static_cast<size_t>(i) * g + j];
  return g;
}

// The rotated factors of one head: a_out = a S (E x r), b_out = S^T b (r x d),
// S = lro_block_rotation(r, block), by plain products in fp64.  Returns g, or -1.
int lro_rotate_factors(int E, int r, int d, int block, const double* a, const double* b,
                       double* a_out, double* b_out) {
  if (E < 1 || d < 1) return -1;
  std::vector<double> s(static_cast<size_t>(r) * r);
  const int g = lro_block_rotation(r, block, s.data());
  if (g < 0) return -1;
  for (int e = 0; e < E; ++e)
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int i = 0; i < r; ++i) acc += a[static_cast<size_t>(e) * r + i] * s[static_cast<size_t>(i) * r + j];
      a_out[static_cast<size_t>(e) * r + j] = acc;
    }
  for (int i = 0; i < r; ++i)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < r; ++j) acc += s[static_cast<size_t>(j) * r + i] * b[static_cast<size_t>(j) * d + c];
      b_out[static_cast<size_t>(i) * d + c] = acc;
    }
  return g;
}

// Greedy global rank allocation (LASER page, "Loss-aware cross-layer rank
// allocation": singular components are chosen greedily by importance score
// per parameter cost until a parameter budget is met, giving non-uniform
// ranks across layers and heads).  Units: (layer, head, K or V), n_units of
// them, each with up to max_rank components scored scores[u * max_rank + j]
// (component j of unit u, in the head's singular-value order).  Readings:
// a unit's rank is a prefix of its components, taken in blocks of `step`
// components (the kernels' rank granularity) whose score is the sum of the
// block's component scores; every unit starts at one block; a block costs
// step * cost_per_component parameters.  Each round takes, over all units,
// the next block with the highest score per parameter (ties: the lowest unit
// index), as long as it fits in what is left of the budget; the first block
// that does not fit ends the allocation.  ranks[u] receives the rank.
// Returns 0, or -1 on bad sizes, -2 if the budget is below one block per unit.
int lro_allocate_ranks(int n_units, int max_rank, int step, const double* scores,
                       double cost_per_component, double budget, int* ranks) {
  if (n_units < 1 || step < 1 || max_rank < step || max_rank % step != 0 || !(cost_per_component > 0))
    return -1;
  const double block_cost = step * cost_per_component;
  double used = n_units * block_cost;
  if (used > budget) return -2;
  for (int u = 0; u < n_units; ++u) ranks[u] = step;
  for (;;) {
    int best = -1;
    double best_v = 0.0;
    for (int u = 0; u < n_units; ++u) {
      if (ranks[u] >= max_rank) continue;
      double v = 0.0;
      for (int j = ranks[u]; j < ranks[u] + step; ++j) v += scores[static_cast<size_t>(u) * max_rank + j];
      v /= block_cost;
      if (best < 0 || v > best_v) { best = u; best_v = v; }
    }
    if (best < 0 || used + block_cost > budget) break;
    ranks[best] += step;
    used += block_cost;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Hybrid low-rank / dense FFN with W8A8 round-to-nearest quantisation (LASER
// page, "Hybrid SVD-quantisation for FFNs": SVD-friendly hidden channels of
// the gate and up projections go through low-rank factors, the others stay
// dense, and both branches are RTN-quantised; "System implementation": the
// fused FFN kernel covers the input projection, the latent activations,
// SwiGLU and quantisation / dequantisation).  Readings of what the pages
// leave open: a LLaMA-style SwiGLU FFN y = W_d (silu(W_g x) * (W_u x)); hidden
// channels [0, S) are the low-rank ones, W_g[S] ~ B_g A_g and W_u[S] ~ B_u A_u
// with one rank r; W_d stays dense; weights are int8 with one fp32 scale per
// row, activations (x, the latents z = A x, and h) are int8 with one fp32 scale
// per token and per group of 64 consecutive elements along the reduction
// dimension (the last group may be shorter); both use the int8 quantiser
// above (s = max|v| / 127, rne, clamp).  Every dot product is taken group by
// group: (exact integer sum) * activation scale, summed over groups, times the
// weight scale.  z and h are rounded to fp32 before they are quantised.
// qmode 0 = W8A8 as above, 1 = no quantisation anywhere (plain fp64 FFN).

// Activations a [T][K] -> codes [T][K], scales [T][ceil(K / 64)].
void lro_quant_act_groups(const float* a, int T, int K, int8_t* q, float* s) {
  const int ng = (K + 63) / 64;
  for (int t = 0; t < T; ++t)
    for (int g = 0; g < ng; ++g) {
      const int lo = 64 * g, n = (lo + 64 <= K ? 64 : K - lo);
      lro_quant_int8(a + static_cast<size_t>(t) * K + lo, n, q + static_cast<size_t>(t) * K + lo,
                     s + static_cast<size_t>(t) * ng + g);
    }
}

namespace {

// A quantised matrix (rows x cols, per-row scales) or its plain values.
struct QMat {
  int rows = 0, cols = 0;
  std::vector<int8_t> q;
  std::vector<float> s;
  const float* w = nullptr;
};

QMat make_qmat(const float* w, int rows, int cols, int qmode) {
  QMat m;
  m.rows = rows;
  m.cols = cols;
  m.w = w;
  if (qmode == 0) {
    m.q.resize(static_cast<size_t>(rows) * cols);
    m.s.resize(rows);
    lro_quant_int8_rows(w, rows, cols, m.q.data(), m.s.data());
  }
  return m;
}

// out[t][n] = sum_k W[n][k] act[t][k] for an activation matrix act [T][K] given
// as fp32 values; with qmode 0 the activations are quantised per (t, group)
// and the products follow the group-by-group dequantisation above.
void qmatmul(const QMat& W, const float* act, int T, int qmode, double* out) {
  const int K = W.cols, N = W.rows, ng = (K + 63) / 64;
  if (qmode == 1) {
    for (int t = 0; t < T; ++t)
      for (int n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
          acc += static_cast<double>(W.w[static_cast<size_t>(n) * K + k]) * act[static_cast<size_t>(t) * K + k];
        out[static_cast<size_t>(t) * N + n] = acc;
      }
    return;
  }
  std::vector<int8_t> aq(static_cast<size_t>(T) * K);
  std::vector<float> as(static_cast<size_t>(T) * ng);
  lro_quant_act_groups(act, T, K, aq.data(), as.data());
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int g = 0; g < ng; ++g) {
        long long isum = 0;
        for (int k = 64 * g; k < K && k < 64 * g + 64; ++k)
          isum += static_cast<long long>(W.q[static_cast<size_t>(n) * K + k]) * aq[static_cast<size_t>(t) * K + k];
        acc += static_cast<double>(isum) * as[static_cast<size_t>(t) * ng + g];
      }
      out[static_cast<size_t>(t) * N + n] = acc * W.s[n];
    }
}

}  // namespace

namespace {

// The hybrid FFN of lro_ffn; when the trace pointers are given it also
// stores what it computed on the way: the latents z (fp32 as quantised, gate
// then up, [T][2r]), the gate and up pre-activations g, u (fp64, [T][F]) and
// h (fp32 as quantised, [T][F]).
int ffn_eval(int qmode, int T, int E, int F, int S, int r, const float* x, const float* wg,
             const float* wu, const float* ag, const float* au, const float* bg, const float* bu,
             const float* wd, double* y, float* z_out, double* g_out, double* u_out, float* h_out) {
  if (T < 0 || E < 1 || F < 1 || S < 0 || S > F || (S > 0 && r < 1) || qmode < 0 || qmode > 1) return -1;
  const int D = F - S;
  std::vector<double> g(static_cast<size_t>(T) * F), u(static_cast<size_t>(T) * F);
  std::vector<double> tmp;
  // dense channels S..F-1
  if (D > 0) {
    tmp.resize(static_cast<size_t>(T) * D);
    qmatmul(make_qmat(wg, D, E, qmode), x, T, qmode, tmp.data());
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < D; ++c) g[static_cast<size_t>(t) * F + S + c] = tmp[static_cast<size_t>(t) * D + c];
    qmatmul(make_qmat(wu, D, E, qmode), x, T, qmode, tmp.data());
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < D; ++c) u[static_cast<size_t>(t) * F + S + c] = tmp[static_cast<size_t>(t) * D + c];
  }
  // low-rank channels 0..S-1: latent z = A x (rounded to fp32), then B z
  if (S > 0) {
    std::vector<double> z(static_cast<size_t>(T) * r);
    std::vector<float> z32(static_cast<size_t>(T) * r);
    tmp.resize(static_cast<size_t>(T) * S);
    const float* A[2] = {ag, au};
    const float* B[2] = {bg, bu};
    std::vector<double>* dst[2] = {&g, &u};
    for (int i = 0; i < 2; ++i) {
      qmatmul(make_qmat(A[i], r, E, qmode), x, T, qmode, z.data());
      for (size_t k = 0; k < z.size(); ++k) z32[k] = static_cast<float>(z[k]);
      if (z_out)
        for (int t = 0; t < T; ++t)
          for (int k = 0; k < r; ++k)
            z_out[(static_cast<size_t>(t) * 2 + i) * r + k] = z32[static_cast<size_t>(t) * r + k];
      qmatmul(make_qmat(B[i], S, r, qmode), z32.data(), T, qmode, tmp.data());
      for (int t = 0; t < T; ++t)
        for (int c = 0; c < S; ++c) (*dst[i])[static_cast<size_t>(t) * F + c] = tmp[static_cast<size_t>(t) * S + c];
    }
  }
  // SwiGLU: h = silu(g) * u, silu(v) = v / (1 + exp(-v)); rounded to fp32
  std::vector<float> h(static_cast<size_t>(T) * F);
  for (size_t k = 0; k < h.size(); ++k) h[k] = static_cast<float>(g[k] / (1.0 + std::exp(-g[k])) * u[k]);
  if (g_out) std::copy(g.begin(), g.end(), g_out);
  if (u_out) std::copy(u.begin(), u.end(), u_out);
  if (h_out) std::copy(h.begin(), h.end(), h_out);
  qmatmul(make_qmat(wd, E, F, qmode), h.data(), T, qmode, y);
  return 0;
}

}  // namespace

// Hybrid FFN on T tokens: x [T][E] (the activations' fp32 values), hidden F,
// S low-rank channels of rank r.  Weights (row-major fp32, rows = outputs):
// wg, wu [F - S][E] (dense gate / up rows of channels S..F-1), ag, au [r][E],
// bg, bu [S][r], wd [E][F].  y [T][E] in fp64.  Returns 0, or -1 on bad sizes.
int lro_ffn(int qmode, int T, int E, int F, int S, int r, const float* x, const float* wg,
            const float* wu, const float* ag, const float* au, const float* bg, const float* bu,
            const float* wd, double* y) {
  return ffn_eval(qmode, T, E, F, S, r, x, wg, wu, ag, au, bg, bu, wd, y, nullptr, nullptr, nullptr,
                  nullptr);
}

// lro_ffn that also returns its intermediates: z [T][2r] (fp32 latents, gate
// then up), g, u [T][F] (fp64 pre-activations), h [T][F] (fp32).
int lro_ffn_trace(int qmode, int T, int E, int F, int S, int r, const float* x, const float* wg,
                  const float* wu, const float* ag, const float* au, const float* bg,
                  const float* bu, const float* wd, double* y, float* z, double* g, double* u,
                  float* h) {
  return ffn_eval(qmode, T, E, F, S, r, x, wg, wu, ag, au, bg, bu, wd, y, z, g, u, h);
}

// Quantise and dequantise one row: out_i = scale * q_i in fp64 (exact).
// qfmt: 0 = int8 per token, 1 = int4 group 32, 2 = no quantisation (out = c).
static void dequantised_row(int qfmt, const float* c, int r, double* out) {
  if (qfmt == 2) {
    for (int i = 0; i < r; ++i) out[i] = static_cast<double>(c[i]);
    return;
  }
  std::vector<int8_t> q(r);
  if (qfmt == 0) {
    float s;
    lro_quant_int8(c, r, q.data(), &s);
    for (int i = 0; i < r; ++i) out[i] = static_cast<double>(s) * q[i];
  } else {
    std::vector<uint16_t> sc((r + 31) / 32);
    lro_quant_int4(c, r, q.data(), sc.data());
    for (int i = 0; i < r; ++i) out[i] = static_cast<double>(lro_f16_to_f32(sc[i / 32])) * q[i];
  }
}

// One attention unit (one layer, one sequence, one head) over T tokens whose
// latents are already dequantised (fp64):
//   ctk [T][rk], ctv [T][rv]   dequantised latents c~^K_t, c~^V_t
//   q  [d]                     query
//   bk [rk][d], bv [rv][d]     up-projection factors B^K_h, B^V_h
//   out [d]                    o = sum_t p_t v_t
//   probs [T] (optional)       the softmax weights p_t
// k_t = c~^K_t B^K and v_t = c~^V_t B^V are rebuilt explicitly, one token at a
// time; z_t = (q . k_t) * scale; p = softmax(z), taken as exp(z_t - max z)
// over the sum of the same; o = sum_t p_t v_t.  T == 0 gives o = 0.
// Returns 0, or -1 on bad sizes.
int lro_attend_dequantised(int T, int rk, int rv, int d, const double* ctk, const double* ctv,
                           const double* q, const double* bk, const double* bv, double scale,
                           double* out, double* probs) {
  if (T < 0 || rk < 1 || rv < 1 || d < 1) return -1;
  for (int j = 0; j < d; ++j) out[j] = 0.0;
  if (T == 0) return 0;

  std::vector<double> vec(d), z(T);
  for (int t = 0; t < T; ++t) {
    const double* c = ctk + static_cast<size_t>(t) * rk;
    for (int j = 0; j < d; ++j) {           // k_t = c~ B^K
      double acc = 0.0;
      for (int i = 0; i < rk; ++i) acc += c[i] * bk[static_cast<size_t>(i) * d + j];
      vec[j] = acc;
    }
    double dot = 0.0;
    for (int j = 0; j < d; ++j) dot += q[j] * vec[j];
    z[t] = dot * scale;
  }
  double zmax = z[0];
  for (int t = 1; t < T; ++t) zmax = z[t] > zmax ? z[t] : zmax;
  double denom = 0.0;
  for (int t = 0; t < T; ++t) denom += std::exp(z[t] - zmax);
  for (int t = 0; t < T; ++t) {
    const double p = std::exp(z[t] - zmax) / denom;
    if (probs) probs[t] = p;
    const double* c = ctv + static_cast<size_t>(t) * rv;
    for (int j = 0; j < d; ++j) {           // v_t = c~ B^V, accumulated with weight p_t
      double acc = 0.0;
      for (int i = 0; i < rv; ++i) acc += c[i] * bv[static_cast<size_t>(i) * d + j];
      out[j] += p * acc;
    }
  }
  return 0;
}

// The same unit from fp32 latents ck [T][rk], cv [T][rv]: every row is first
// quantised with qfmt (0 = int8 per token, 1 = int4 group 32, 2 = none) and
// dequantised, then lro_attend_dequantised runs.  Returns 0, or -1.
int lro_attend(int qfmt, int T, int rk, int rv, int d, const float* ck, const float* cv,
               const double* q, const double* bk, const double* bv, double scale,
               double* out, double* probs) {
  if (T < 0 || rk < 1 || rv < 1 || d < 1 || qfmt < 0 || qfmt > 2) return -1;
  std::vector<double> ctk(static_cast<size_t>(T) * rk), ctv(static_cast<size_t>(T) * rv);
  for (int t = 0; t < T; ++t) {
    dequantised_row(qfmt, ck + static_cast<size_t>(t) * rk, rk, ctk.data() + static_cast<size_t>(t) * rk);
    dequantised_row(qfmt, cv + static_cast<size_t>(t) * rv, rv, ctv.data() + static_cast<size_t>(t) * rv);
  }
  return lro_attend_dequantised(T, rk, rv, d, ctk.data(), ctv.data(), q, bk, bv, scale, out, probs);
}

}  // extern "C"
