// C entry points of libstem: argument checks on the host, then one kernel
// launch each on the caller's stream.  See include/stem.h for the contract.
#include <cstdint>

#include "stem.h"
#include "stem_device.h"
#include "stem_internal.h"

using namespace stem;

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_info(const stem_plan_info *in, const void *plan_dev) {
  if (!in || in->magic != STEM_PLAN_MAGIC) return STEM_EINVAL;
  if (in->num_q_heads < 1 || in->num_kv_heads < 1 || in->num_q_heads % in->num_kv_heads) return STEM_EINVAL;
  if (in->head_dim != 64 && in->head_dim != 128) return STEM_EUNSUPPORTED;
  if (in->block != 64 && in->block != 128) return STEM_EUNSUPPORTED;
  if (in->dtype != STEM_F32 && in->dtype != STEM_BF16) return STEM_EUNSUPPORTED;
  if (in->total_blocks < 0 || in->total_tokens < 0) return STEM_EINVAL;
  // the size limits stem_plan enforces (a plan edited afterwards could exceed them)
  if (in->total_tokens > INT32_MAX || in->total_blocks > INT32_MAX / 2 ||
      int64_t(in->num_q_heads) * in->total_blocks > INT32_MAX ||
      in->max_seq_blocks > STEM_MAX_SEQ_BLOCKS)
    return STEM_EUNSUPPORTED;
  if (in->metric_mode < STEM_METRIC_OUTPUT_AWARE || in->metric_mode > STEM_METRIC_ROUTING)
    return STEM_EINVAL;
  if (in->total_blocks > 0 && (!plan_dev || !aligned(plan_dev, 16))) return STEM_EINVAL;
  return STEM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? STEM_OK : STEM_EHIP; }

}  // namespace

extern "C" int stem_pool(const stem_plan_info *in, const void *plan_dev, const void *q,
                         const void *k, const void *v, float *qbar, float *kbar,
                         float *vnorm, int32_t vnorm_mode, void *stream) {
  int rc = check_info(in, plan_dev);
  if (rc) return rc;
  if (vnorm_mode != STEM_VNORM_MEAN && vnorm_mode != STEM_VNORM_MAX) return STEM_EINVAL;
  if (in->total_blocks == 0) return STEM_OK;
  if (!q || !k || !v || !qbar || !kbar || !vnorm) return STEM_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qbar, 16) ||
      !aligned(kbar, 16) || !aligned(vnorm, 4))
    return STEM_EINVAL;
  return hip_status(launch_pool(*in, make_plan_dev(*in, plan_dev), q, k, v, qbar, kbar, vnorm,
                                vnorm_mode, static_cast<hipStream_t>(stream)));
}

extern "C" int stem_score(const stem_plan_info *in, const void *plan_dev, const float *qbar,
                          const float *kbar, const float *vnorm, float *scores, void *stream) {
  int rc = check_info(in, plan_dev);
  if (rc) return rc;
  if (in->total_blocks == 0) return STEM_OK;
  if (!qbar || !kbar || !vnorm || !scores) return STEM_EINVAL;
  if (!aligned(qbar, 16) || !aligned(kbar, 16) || !aligned(vnorm, 4) || !aligned(scores, 4))
    return STEM_EINVAL;
  return hip_status(launch_score(*in, make_plan_dev(*in, plan_dev), qbar, kbar, vnorm, scores,
                                 static_cast<hipStream_t>(stream)));
}

extern "C" int stem_score_antidiag(const stem_plan_info *in, const void *plan_dev, const void *q,
                                   const void *k, const float *vnorm, int32_t stride,
                                   float *scores, void *stream) {
  int rc = check_info(in, plan_dev);
  if (rc) return rc;
  if (stride < 1 || stride > in->block || (stride & (stride - 1))) return STEM_EINVAL;
  if (in->total_blocks == 0) return STEM_OK;
  if (!q || !k || !vnorm || !scores) return STEM_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vnorm, 4) || !aligned(scores, 4))
    return STEM_EINVAL;
  if (in->dtype == STEM_BF16) {
    if (int64_t(in->num_q_heads) * antidiag_units_per_head(*in, stride) > INT32_MAX / 2)
      return STEM_EUNSUPPORTED;
    // token rows of one tile must be addressable with 32-bit offsets
    if (int64_t(256) * stride * in->num_q_heads * in->head_dim * 2 + 64 > (int64_t(1) << 32))
      return STEM_EUNSUPPORTED;
  }
  return hip_status(launch_score_antidiag(*in, make_plan_dev(*in, plan_dev), q, k, vnorm, stride,
                                          scores, static_cast<hipStream_t>(stream)));
}

extern "C" int stem_select(const stem_plan_info *in, const void *plan_dev, const float *scores,
                           int32_t *idx, int32_t *count, void *stream) {
  int rc = check_info(in, plan_dev);
  if (rc) return rc;
  if (in->total_blocks == 0) return STEM_OK;
  if (!scores || !idx || !count || in->kmax < 1) return STEM_EINVAL;
  if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(count, 4)) return STEM_EINVAL;
  return hip_status(launch_select(*in, make_plan_dev(*in, plan_dev), scores, idx, count,
                                  static_cast<hipStream_t>(stream)));
}

extern "C" int stem_sparse_attn(const stem_plan_info *in, const void *plan_dev, const void *q,
                                const void *k, const void *v, const int32_t *idx,
                                const int32_t *count, void *out, int32_t out_dtype, float *lse,
                                void *stream) {
  int rc = check_info(in, plan_dev);
  if (rc) return rc;
  if (out_dtype != STEM_F32 && out_dtype != STEM_BF16) return STEM_EUNSUPPORTED;
  if (in->total_blocks == 0) return STEM_OK;
  if (!q || !k || !v || !idx || !count || !out || in->kmax < 1) return STEM_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(idx, 4) || !aligned(count, 4) || (lse && !aligned(lse, 4)))
    return STEM_EINVAL;
  return hip_status(launch_attn(*in, make_plan_dev(*in, plan_dev), q, k, v, idx, count, out,
                                out_dtype, lse, static_cast<hipStream_t>(stream)));
}
