// Host-side planning for the Stem sparse-prefill path: argument checks,
// block layout of a packed batch, the Token Position-Decay budget table and
// the order in which query blocks are handed to the attention kernel.
// Touches no HIP API, so it runs (and is tested) on machines without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "stem.h"
#include "stem_internal.h"

namespace {

int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

int64_t tri(int64_t n) { return n * (n + 1) / 2; }

// Number of blocks chosen by the metric for local query block i of a
// sequence with nb blocks, before the k_min floor and the causal cap
// (gist.science/es 2.A and gist.science/fr 2.A: position-dependent top-k,
// high for early positions and decaying later).  Evaluated in double
// precision with the C library exp and ceil; every product and sum is its
// own statement so that no fused multiply-add changes the rounding.
double kdyn_raw(int64_t i, int64_t nb, const stem_params &p) {
  if (p.budget_mode == STEM_BUDGET_LINEAR || p.budget_mode == STEM_BUDGET_LINEAR_FRACTION) {
    const double f = nb <= 1 ? 0.0 : static_cast<double>(i) / static_cast<double>(nb - 1);
    const double a = p.k_start * (1.0 - f);
    const double b = p.mu * p.k_start;
    const double c = b * f;
    const double x = a + c;
    if (p.budget_mode == STEM_BUDGET_LINEAR) return std::ceil(x);
    // a share of the row's i + 1 causal key blocks
    const double y = x * static_cast<double>(i + 1);
    return std::ceil(y);
  }
  const double e = std::exp(-static_cast<double>(i) / p.tau);
  const double x = p.rho0 * e * static_cast<double>(i + 1);
  return std::ceil(x);
}

int32_t budget_of(int64_t i, int64_t nb, const stem_params &p) {
  if (i < p.sink_blocks) return static_cast<int32_t>(i + 1);
  const double c = kdyn_raw(i, nb, p);
  // k_dyn = max(k_min, ceil(x)), then k_i = min(i + 1, S + 1 + k_dyn)
  int64_t kdyn;
  if (c >= static_cast<double>(i + 1)) {
    kdyn = i + 1;  // saturates below anyway; avoids overflow for huge x
  } else if (c <= 0.0) {
    kdyn = 0;
  } else {
    kdyn = static_cast<int64_t>(c);
  }
  kdyn = std::max<int64_t>(kdyn, p.k_min);
  const int64_t k = std::min<int64_t>(i + 1, int64_t(p.sink_blocks) + 1 + kdyn);
  return static_cast<int32_t>(k);
}

}  // namespace

extern "C" int stem_plan(const stem_problem *pr, const stem_params *pa,
                         stem_plan_info *info, void *plan_host, int64_t capacity) {
  if (!pr || !pa || !info) return STEM_EINVAL;
  if (pr->num_seqs < 1 || !pr->cu_seqlens) return STEM_EINVAL;
  if (pr->num_q_heads < 1 || pr->num_kv_heads < 1) return STEM_EINVAL;
  if (pr->num_q_heads % pr->num_kv_heads != 0) return STEM_EINVAL;
  if (pr->dtype != STEM_F32 && pr->dtype != STEM_BF16) return STEM_EUNSUPPORTED;
  if (pr->head_dim != 64 && pr->head_dim != 128) return STEM_EUNSUPPORTED;
  if (pr->block != 64 && pr->block != 128) return STEM_EUNSUPPORTED;
  if (pa->sink_blocks < 0 || pa->k_min < 0) return STEM_EINVAL;
  if (pa->budget_mode == STEM_BUDGET_EXP) {
    if (!std::isfinite(pa->rho0) || pa->rho0 < 0.0) return STEM_EINVAL;
    if (!std::isfinite(pa->tau) || !(pa->tau > 0.0)) return STEM_EINVAL;
  } else if (pa->budget_mode == STEM_BUDGET_LINEAR) {
    if (!std::isfinite(pa->k_start) || pa->k_start < 0.0) return STEM_EINVAL;
    if (!(pa->mu >= 0.0 && pa->mu <= 1.0)) return STEM_EINVAL;
  } else if (pa->budget_mode == STEM_BUDGET_LINEAR_FRACTION) {
    if (!(pa->k_start >= 0.0 && pa->k_start <= 1.0)) return STEM_EINVAL;
    if (!(pa->mu >= 0.0 && pa->mu <= 1.0)) return STEM_EINVAL;
  } else {
    return STEM_EINVAL;
  }
  if (pa->metric_mode != STEM_METRIC_OUTPUT_AWARE && pa->metric_mode != STEM_METRIC_ADDITIVE &&
      pa->metric_mode != STEM_METRIC_ROUTING)
    return STEM_EINVAL;
  if (!std::isfinite(pa->beta) || pa->beta < 0.0) return STEM_EINVAL;

  const int32_t ns = pr->num_seqs;
  const int32_t *cu = pr->cu_seqlens;
  if (cu[0] != 0) return STEM_EINVAL;
  int64_t nbT = 0, tri_total = 0;
  int32_t max_nb = 0;
  for (int32_t s = 0; s < ns; ++s) {
    if (cu[s + 1] < cu[s]) return STEM_EINVAL;
    const int64_t len = int64_t(cu[s + 1]) - cu[s];
    const int64_t nb = (len + pr->block - 1) / pr->block;
    nbT += nb;
    tri_total += tri(nb);
    max_nb = std::max<int32_t>(max_nb, static_cast<int32_t>(nb));
  }
  const int64_t T = cu[ns];
  if (max_nb > STEM_MAX_SEQ_BLOCKS) return STEM_EUNSUPPORTED;
  // element offsets of Q [T, Hq, d] must fit the kernels' 64-bit math, and
  // block numbers / token numbers are int32 in the plan
  if (nbT > INT32_MAX / 2 || T > INT32_MAX) return STEM_EUNSUPPORTED;
  // one attention / selection work item per (query head, query block)
  if (int64_t(pr->num_q_heads) * nbT > INT32_MAX) return STEM_EUNSUPPORTED;

  std::vector<int32_t> budget(static_cast<size_t>(nbT));
  int64_t executed = 0;
  int32_t kmax = 0;
  {
    int64_t b = 0;
    for (int32_t s = 0; s < ns; ++s) {
      const int64_t nb = (int64_t(cu[s + 1]) - cu[s] + pr->block - 1) / pr->block;
      for (int64_t i = 0; i < nb; ++i, ++b) {
        budget[b] = budget_of(i, nb, *pa);
        executed += budget[b];
        kmax = std::max(kmax, budget[b]);
      }
    }
  }

  stem_plan_info in;
  std::memset(&in, 0, sizeof(in));
  in.magic = STEM_PLAN_MAGIC;
  in.num_seqs = ns;
  in.num_q_heads = pr->num_q_heads;
  in.num_kv_heads = pr->num_kv_heads;
  in.head_dim = pr->head_dim;
  in.block = pr->block;
  in.dtype = pr->dtype;
  in.sink_blocks = pa->sink_blocks;
  in.kmax = kmax;
  in.max_seq_blocks = max_nb;
  in.metric_mode = pa->metric_mode;
  in.beta = pa->beta;
  in.total_tokens = T;
  in.total_blocks = nbT;
  in.score_elems_per_head = tri_total;
  in.executed_blocks_per_head = executed;
  int64_t off = 0;
  in.off_cu_seqlens = off;  off = align16(off + 4 * int64_t(ns + 1));
  in.off_cu_blocks = off;   off = align16(off + 4 * int64_t(ns + 1));
  in.off_tri = off;         off = align16(off + 8 * int64_t(ns + 1));
  in.off_blk_seq = off;     off = align16(off + 4 * nbT);
  in.off_budget = off;      off = align16(off + 4 * nbT);
  in.off_order = off;       off = align16(off + 4 * nbT);
  in.plan_bytes = off;
  *info = in;
  if (!plan_host) return STEM_OK;
  if (capacity < in.plan_bytes) return STEM_ESPACE;

  char *base = static_cast<char *>(plan_host);
  std::memset(base, 0, static_cast<size_t>(in.plan_bytes));
  int32_t *p_cu = reinterpret_cast<int32_t *>(base + in.off_cu_seqlens);
  int32_t *p_cub = reinterpret_cast<int32_t *>(base + in.off_cu_blocks);
  int64_t *p_tri = reinterpret_cast<int64_t *>(base + in.off_tri);
  int32_t *p_seq = reinterpret_cast<int32_t *>(base + in.off_blk_seq);
  int32_t *p_bud = reinterpret_cast<int32_t *>(base + in.off_budget);
  int32_t *p_ord = reinterpret_cast<int32_t *>(base + in.off_order);
  int64_t b = 0, t = 0;
  p_cub[0] = 0;
  p_tri[0] = 0;
  for (int32_t s = 0; s < ns; ++s) {
    p_cu[s] = cu[s];
    const int64_t nb = (int64_t(cu[s + 1]) - cu[s] + pr->block - 1) / pr->block;
    for (int64_t i = 0; i < nb; ++i) p_seq[b + i] = s;
    b += nb;
    t += tri(nb);
    p_cub[s + 1] = static_cast<int32_t>(b);
    p_tri[s + 1] = t;
  }
  p_cu[ns] = cu[ns];
  // (an empty vector may hand out a null data pointer, which memcpy must
  // not receive even for zero bytes)
  if (!budget.empty()) std::memcpy(p_bud, budget.data(), sizeof(int32_t) * budget.size());
  // attention work order: most kept blocks first (longest-job-first keeps
  // the tail of the grid short); a final partial block counts as less work.
  std::vector<int32_t> order(static_cast<size_t>(nbT));
  std::iota(order.begin(), order.end(), 0);
  auto cost = [&](int32_t g) {
    const int32_t s = p_seq[g];
    const int64_t i = g - p_cub[s];
    const int64_t len = int64_t(cu[s + 1]) - cu[s];
    const int64_t rows = std::min<int64_t>(pr->block, len - i * pr->block);
    return int64_t(budget[g]) * 2 * pr->block - (pr->block - rows);
  };
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return cost(x) > cost(y); });
  if (!order.empty()) std::memcpy(p_ord, order.data(), sizeof(int32_t) * order.size());
  return STEM_OK;
}

extern "C" const char *stem_status_str(int status) {
  switch (status) {
    case STEM_OK: return "ok";
    case STEM_EINVAL: return "invalid argument";
    case STEM_EUNSUPPORTED: return "unsupported configuration";
    case STEM_EHIP: return "HIP runtime error";
    case STEM_ESPACE: return "plan buffer too small";
    default: return "unknown status";
  }
}
