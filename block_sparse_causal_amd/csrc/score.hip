// Output-Aware Metric on pooled blocks (gist.science/es 2.B and
// gist.science/fr 2.B: routing relevance of a key block combined with the
// magnitude of its values), in the multiplicative form
//   m_ij = softmax_{j <= i}(qbar_i . kbar_j / sqrt(d)) * vnorm_j
// which orders key blocks of a row exactly like the pages' additive form
// s_ij + beta * log ||V_j||^2 with beta = 1/2.
//
// One wavefront owns 32 consecutive query-block rows of one (query head,
// sequence) and walks the causal key blocks 32 at a time.  The pooled dot
// products are an f32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32,
// computing the transposed tile keys x queries so that each lane holds one
// query row's values and row statistics never leave the lane pair l, l^32).
// Pass 1 stores the scaled logits into the output and keeps an online row
// max / sum; pass 2 re-reads the lane's own values and rewrites them as
// exp(x - max) / sum * vnorm.  f32 throughout.
#include "stem_device.h"

namespace stem {
namespace {

struct ScoreArgs {
  const float *qbar, *kbar, *vnorm;
  float *scores;
  PlanDev pd;
  int32_t Hq, Hkv, nbT, num_seqs;
  int64_t per_head;
  float scale;
};

template <int D>
__global__ __launch_bounds__(64) void score_kernel(ScoreArgs a) {
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x;
  const int n = lane & 31;        // query row inside the tile / key row of the A operand
  const int hi = lane >> 5;       // which half of the head dimension this lane feeds
  const int h = blockIdx.y;
  const int g = h / (a.Hq / a.Hkv);

  // tile -> (sequence, row tile), heaviest (last) row tiles first
  int t = blockIdx.x;
  int s = 0, nb = 0;
  for (s = 0; s < a.num_seqs; ++s) {
    nb = a.pd.cu_blocks[s + 1] - a.pd.cu_blocks[s];
    const int tiles = (nb + 31) >> 5;
    if (t < tiles) break;
    t -= tiles;
  }
  if (s >= a.num_seqs) return;
  const int tiles = (nb + 31) >> 5;
  const int rt = tiles - 1 - t;
  const int b0 = a.pd.cu_blocks[s];
  const int i0 = rt * 32;
  const int qi = i0 + n;
  const bool qvalid = qi < nb;
  const int64_t rowbase = int64_t(h) * a.per_head + a.pd.tri[s] +
                          (int64_t(qi) * (qi + 1)) / 2;

  // B operand: qbar row qi, contraction index c <-> dim hi*HALF + c
  float qv[HALF];
  {
    const float *src = a.qbar + (int64_t(h) * a.nbT + b0 + (qvalid ? qi : 0)) * D + hi * HALF;
#pragma unroll
    for (int c = 0; c < HALF; c += 4) {
      f32x4 x = qvalid ? *reinterpret_cast<const f32x4 *>(src + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      qv[c] = x[0]; qv[c + 1] = x[1]; qv[c + 2] = x[2]; qv[c + 3] = x[3];
    }
  }

  float mrun = -INFINITY, lrun = 0.f;
  const int last_row = min(i0 + 31, nb - 1);
  const int jt_end = last_row / 32;
  for (int jt = 0; jt <= jt_end; ++jt) {
    const int j0 = jt * 32;
    const int kr = j0 + n;
    const bool kvalid = kr < nb;
    const float *ksrc = a.kbar + (int64_t(g) * a.nbT + b0 + (kvalid ? kr : 0)) * D + hi * HALF;
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < HALF; c += 4) {
      f32x4 kx = kvalid ? *reinterpret_cast<const f32x4 *>(ksrc + c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kx[e], qv[c + e], acc, 0, 0, 0);
    }
    // acc[r] = logit(key j0 + 8(r/4) + 4hi + r%4, query qi)
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const bool ok = qvalid && j <= qi;
      const float x = acc[r] * a.scale;
      acc[r] = ok ? x : -INFINITY;
      if (ok) a.scores[rowbase + j] = x;
      bm = fmaxf(bm, acc[r]);
    }
    const float mnew = fmaxf(mrun, bm);
    if (mnew != -INFINITY) {
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += expf(acc[r] - mnew);
      lrun = lrun * expf(mrun - mnew) + ps;
      mrun = mnew;
    }
  }
  // combine the two lanes that share a query row
  const float mo = __shfl_xor(mrun, 32);
  const float lo = __shfl_xor(lrun, 32);
  const float M = fmaxf(mrun, mo);
  const float L = (mrun == -INFINITY ? 0.f : lrun * expf(mrun - M)) +
                  (mo == -INFINITY ? 0.f : lo * expf(mo - M));
  if (!qvalid) return;
  const float invL = 1.0f / L;
  const float *w = a.vnorm + int64_t(g) * a.nbT + b0;
  for (int jt = 0; jt <= jt_end; ++jt) {
    const int j0 = jt * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (j <= qi) {
        const float x = a.scores[rowbase + j];
        a.scores[rowbase + j] = expf(x - M) * invL * w[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_score(const stem_plan_info &in, PlanDev pd, const float *qbar,
                        const float *kbar, const float *vnorm, float *scores,
                        hipStream_t st) {
  if (in.total_blocks == 0) return hipSuccess;
  // number of 32-row tiles summed over sequences, computed from the host copy
  // of the layout is not available here; bound it by nbT/32 + num_seqs
  const int64_t tiles = in.total_blocks / 32 + in.num_seqs;
  ScoreArgs a;
  a.qbar = qbar; a.kbar = kbar; a.vnorm = vnorm; a.scores = scores;
  a.pd = pd;
  a.Hq = in.num_q_heads; a.Hkv = in.num_kv_heads;
  a.nbT = static_cast<int32_t>(in.total_blocks);
  a.num_seqs = in.num_seqs;
  a.per_head = in.score_elems_per_head;
  a.scale = 1.0f / sqrtf(static_cast<float>(in.head_dim));
  dim3 grid(static_cast<unsigned>(tiles), in.num_q_heads);
  if (in.head_dim == 128)
    hipLaunchKernelGGL((score_kernel<128>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((score_kernel<64>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace stem
