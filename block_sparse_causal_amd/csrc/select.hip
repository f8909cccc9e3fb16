// Token Position-Decay top-k block selection (gist.science/es
// "Implementacion" steps 2-3; gist.science/nl "Implementatie" steps 2-3).
//
// One 64-wide wavefront per (query head, query block) row, rows dispatched
// longest first; the per-row selection is select_row (select_row.h).  The
// kept blocks are written in ascending order and the list is padded with -1
// to kmax entries.
#include "select_row.h"
#include "stem_device.h"
#include "stem_internal.h"

namespace stem {
namespace {

struct SelectArgs {
  const float *scores;
  int32_t *idx, *count;
  PlanDev pd;
  int32_t Hq, nbT, kmax, sinks;
  int64_t per_head;
};

template <int E>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  // per wavefront: the few candidates that can still reach the top
  __shared__ uint32_t ckey[4][64];
  __shared__ int32_t cpos[4][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  // rows in reverse order: the longest rows (last query blocks) go first
  const int64_t nrows = int64_t(a.Hq) * a.nbT;
  const int64_t row = nrows - 1 - (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (row < 0) return;
  const int h = static_cast<int>(row / a.nbT);
  const int b = static_cast<int>(row % a.nbT);
  const int s = a.pd.blk_seq[b];
  const int i = b - a.pd.cu_blocks[s];
  const int k_i = a.pd.budget[b];
  int32_t *out = a.idx + row * a.kmax;
  if (lane == 0) a.count[row] = k_i;
  const float *mrow = a.scores + int64_t(h) * a.per_head + a.pd.tri[s] +
                      (int64_t(i) * (i + 1)) / 2;
  select_row<E>(mrow, i, k_i, a.sinks, ckey[wv], cpos[wv], [&](int p, int j) { out[p] = j; });
  for (int p = k_i + lane; p < a.kmax; p += 64) out[p] = -1;
}

}  // namespace

hipError_t launch_select(const stem_plan_info &in, PlanDev pd, const float *scores,
                         int32_t *idx, int32_t *count, hipStream_t st) {
  const int64_t rows = int64_t(in.num_q_heads) * in.total_blocks;
  if (rows == 0) return hipSuccess;
  SelectArgs a;
  a.scores = scores; a.idx = idx; a.count = count;
  a.pd = pd;
  a.Hq = in.num_q_heads;
  a.nbT = static_cast<int32_t>(in.total_blocks);
  a.kmax = in.kmax;
  a.sinks = in.sink_blocks;
  a.per_head = in.score_elems_per_head;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const int ncand = in.max_seq_blocks;  // upper bound of candidates per row
  if (ncand <= 64)
    hipLaunchKernelGGL((select_kernel<1>), grid, dim3(256), 0, st, a);
  else if (ncand <= 128)
    hipLaunchKernelGGL((select_kernel<2>), grid, dim3(256), 0, st, a);
  else if (ncand <= 256)
    hipLaunchKernelGGL((select_kernel<4>), grid, dim3(256), 0, st, a);
  else if (ncand <= 512)
    hipLaunchKernelGGL((select_kernel<8>), grid, dim3(256), 0, st, a);
  else if (ncand <= 1024)
    hipLaunchKernelGGL((select_kernel<16>), grid, dim3(256), 0, st, a);
  else if (ncand <= 2048)
    hipLaunchKernelGGL((select_kernel<32>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((select_kernel<64>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

static_assert(STEM_MAX_SEQ_BLOCKS <= 64 * 64, "select keeps <= 64 keys per lane");

}  // namespace stem
