// alloc.cpp -- greedy global rank allocation (LASER page, "Loss-aware
// cross-layer rank allocation": singular components are taken greedily by
// importance score per parameter cost until a parameter budget is met, which
// gives non-uniform ranks across layers and heads).
//
// The output is a rank table for lr_attn_plan_create: ranks come in blocks of
// 8 components (the kernels' rank granularity) scored by the sum of their
// components' scores, every (layer, head, K or V) keeps at least one block,
// and a head's rank is always a prefix of its components.  A max-heap holds
// each unit's next block; the best block is taken while it fits the budget.

#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "plan.h"

namespace {

constexpr int kStep = 8;

struct Cand {
  double value;   // block score / block cost
  int32_t unit;
};
// priority_queue keeps the largest first: higher value, then the lower unit
struct Worse {
  bool operator()(const Cand& a, const Cand& b) const {
    return a.value < b.value || (a.value == b.value && a.unit > b.unit);
  }
};

}  // namespace

extern "C" {

lr_status lr_attn_allocate_ranks(int32_t n_layers, int32_t n_heads, int32_t max_rank,
                                 const float* scores, int64_t cost_per_rank, int64_t budget,
                                 int32_t* rank_k, int32_t* rank_v) {
  if (n_layers < 1 || n_heads < 1 || !scores || !rank_k || !rank_v || cost_per_rank < 1)
    return LR_EINVAL;
  if (max_rank < kStep || max_rank > LR_HEAD_DIM || max_rank % kStep != 0) return LR_EUNSUPPORTED;
  const int64_t n_units = int64_t(n_layers) * n_heads * 2;
  if (n_units > (int64_t(1) << 24)) return LR_ERANGE;
  const size_t n_scores = size_t(n_units) * size_t(max_rank);
  for (size_t i = 0; i < n_scores; ++i)
    if (!std::isfinite(scores[i])) return LR_EINVAL;
  const int64_t block_cost = int64_t(kStep) * cost_per_rank;
  if (budget < n_units * block_cost) return LR_ERANGE;

  auto block_value = [&](int64_t u, int r) {
    const float* s = scores + size_t(u) * size_t(max_rank) + size_t(r);
    double v = 0.0;
    for (int j = 0; j < kStep; ++j) v += double(s[j]);
    return v / double(block_cost);
  };
  std::vector<int32_t> ranks(size_t(n_units), kStep);
  std::priority_queue<Cand, std::vector<Cand>, Worse> heap;
  for (int64_t u = 0; u < n_units; ++u)
    if (kStep < max_rank) heap.push({block_value(u, kStep), int32_t(u)});
  int64_t used = n_units * block_cost;
  while (!heap.empty()) {
    const Cand c = heap.top();
    if (used + block_cost > budget) break;
    heap.pop();
    ranks[size_t(c.unit)] += kStep;
    used += block_cost;
    if (ranks[size_t(c.unit)] < max_rank) heap.push({block_value(c.unit, ranks[size_t(c.unit)]), c.unit});
  }
  for (int64_t i = 0; i < int64_t(n_layers) * n_heads; ++i) {
    rank_k[i] = ranks[size_t(2 * i)];
    rank_v[i] = ranks[size_t(2 * i + 1)];
  }
  return LR_OK;
}

}  // extern "C"
