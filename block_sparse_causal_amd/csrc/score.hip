// Block metric on pooled blocks (gist.science/es 2.B and gist.science/fr
// 2.B: routing relevance of a key block combined with the magnitude of its
// values).  Three forms, chosen by the plan:
//   output-aware  m_ij = softmax_{j <= i}(s_ij) * vnorm_j
//   additive      m_ij = s_ij + beta * max(0, log vnorm_j^2)
//   routing       m_ij = softmax_{j <= i}(s_ij)
// with s_ij = qbar_i . kbar_j / sqrt(d).  Inside a row the output-aware form
// orders key blocks exactly like the additive one with beta = 1/2.
//
// One workgroup owns 32 consecutive query-block rows of one (query head,
// sequence); its 8 wavefronts split the causal key blocks 32 at a time
// (round robin) and merge their row statistics through LDS.  The pooled dot
// products are an f32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32,
// computing the transposed tile keys x queries so that each lane holds one
// query row's values and row statistics never leave the lane pair l, l^32).
// Softmax forms: pass 1 keeps an online row max / sum (and the scaled
// logits, in registers or parked in the output); pass 2 writes
// exp(x - max) / sum (* vnorm).  The additive form needs no row statistics
// and is written in pass 1.  f32 throughout; exponentials use the hardware
// exp2 (relative error ~1e-6).
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
  float beta;
};

constexpr int kScoreWaves = 8;

template <int D, int MODE>
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(ScoreArgs a) {
  constexpr int HALF = D / 2;
  __shared__ float st_m[kScoreWaves][64];
  __shared__ float st_l[kScoreWaves][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
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

  // pass 1: wavefront wv takes key tiles wv, wv + 8, ...; an online row
  // max / sum is kept per lane.  The scaled logits of the first kKeep tiles
  // stay in registers; those of later tiles are parked in the output and
  // re-read in pass 2.
  constexpr int kKeep = 4;
  float mrun = -INFINITY, lrun = 0.f;
  const int last_row = min(i0 + 31, nb - 1);
  const int jt_end = last_row / 32;
  f32x16 keep[kKeep];
  auto load_k = [&](int jt, f32x4 (&kx)[HALF / 4]) {
    const int kr = jt * 32 + n;
    const bool kvalid = jt <= jt_end && kr < nb;
    const float *ksrc = a.kbar + (int64_t(g) * a.nbT + b0 + (kvalid ? kr : 0)) * D + hi * HALF;
#pragma unroll
    for (int c = 0; c < HALF / 4; ++c)
      kx[c] = kvalid ? *reinterpret_cast<const f32x4 *>(ksrc + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  int slot = 0;
  for (int jt = wv; jt <= jt_end; jt += kScoreWaves, ++slot) {
    f32x4 kcur[HALF / 4];
    load_k(jt, kcur);
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < HALF / 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kcur[c][e], qv[4 * c + e], acc, 0, 0, 0);
    const int j0 = jt * 32;
    // acc[r] = logit(key j0 + 8(r/4) + 4hi + r%4, query qi)
    if constexpr (MODE == STEM_METRIC_ADDITIVE) {
      const float *w = a.vnorm + int64_t(g) * a.nbT + b0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qvalid && j <= qi) {
          // log(w^2) as 2 log w: no overflow for large w; log 0 = -inf -> 0
          const float bonus = fmaxf(0.f, 2.f * logf(w[j]));
          a.scores[rowbase + j] = fmaf(a.beta, bonus, acc[r] * a.scale);
        }
      }
      continue;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      acc[r] = (qvalid && j <= qi) ? acc[r] * a.scale : -INFINITY;
      bm = fmaxf(bm, acc[r]);
    }
    const float mnew = fmaxf(mrun, bm);
    if (mnew != -INFINITY) {
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += __expf(acc[r] - mnew);
      lrun = lrun * __expf(mrun - mnew) + ps;
      mrun = mnew;
    }
    if (slot < kKeep) {
#pragma unroll
      for (int k = 0; k < kKeep; ++k)
        if (k == slot) keep[k] = acc;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qvalid && j <= qi) a.scores[rowbase + j] = acc[r];
      }
    }
  }
  if constexpr (MODE == STEM_METRIC_ADDITIVE) return;
  // combine the statistics of the 8 wavefronts and of the two lanes that
  // share a query row
  st_m[wv][lane] = mrun;
  st_l[wv][lane] = lrun;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kScoreWaves; ++v) M = fmaxf(M, fmaxf(st_m[v][lane], st_m[v][lane ^ 32]));
  float L = 0.f;
#pragma unroll
  for (int v = 0; v < kScoreWaves; ++v) {
    const float m0 = st_m[v][lane], m1 = st_m[v][lane ^ 32];
    if (m0 != -INFINITY) L += st_l[v][lane] * __expf(m0 - M);
    if (m1 != -INFINITY) L += st_l[v][lane ^ 32] * __expf(m1 - M);
  }
  if (!qvalid) return;
  // pass 2: write this wavefront's values as exp(x - M) / L (* vnorm)
  const float invL = 1.0f / L;
  const float *w = a.vnorm + int64_t(g) * a.nbT + b0;
  slot = 0;
  for (int jt = wv; jt <= jt_end; jt += kScoreWaves, ++slot) {
    const int j0 = jt * 32;
    f32x16 x;
    if (slot < kKeep) {
#pragma unroll
      for (int k = 0; k < kKeep; ++k)
        if (k == slot) x = keep[k];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (j <= qi) {
        const float v = slot < kKeep ? x[r] : a.scores[rowbase + j];
        const float p = __expf(v - M) * invL;
        a.scores[rowbase + j] = MODE == STEM_METRIC_ROUTING ? p : p * w[j];
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
  a.beta = static_cast<float>(in.beta);
  dim3 grid(static_cast<unsigned>(tiles), in.num_q_heads);
  const dim3 block(64 * kScoreWaves);
  const bool d128 = in.head_dim == 128;
  switch (in.metric_mode) {
    case STEM_METRIC_ADDITIVE:
      if (d128) hipLaunchKernelGGL((score_kernel<128, STEM_METRIC_ADDITIVE>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((score_kernel<64, STEM_METRIC_ADDITIVE>), grid, block, 0, st, a);
      break;
    case STEM_METRIC_ROUTING:
      if (d128) hipLaunchKernelGGL((score_kernel<128, STEM_METRIC_ROUTING>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((score_kernel<64, STEM_METRIC_ROUTING>), grid, block, 0, st, a);
      break;
    default:
      if (d128)
        hipLaunchKernelGGL((score_kernel<128, STEM_METRIC_OUTPUT_AWARE>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((score_kernel<64, STEM_METRIC_OUTPUT_AWARE>), grid, block, 0, st, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace stem
