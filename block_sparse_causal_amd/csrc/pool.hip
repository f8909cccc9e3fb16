// Block downsampling (stage 1 of the method: block-level Q, K and V
// magnitude; gist.science/es "Implementacion" step 1, gist.science/nl
// "Implementatie" step 1).
//
// One workgroup reduces the tokens of one block for a slice of one tensor's
// columns (a "column" is one (head, dim) element of a token row).  Token rows
// of Q/K/V are contiguous, so a wavefront reads 64 x 16 B = 1 KiB contiguous
// per token: the kernel is a single coalesced streaming pass over Q, K and V
// and is bound by HBM bandwidth.  The loads are non-temporal: every byte is
// read once here, and not allocating it in the caches keeps them for the
// later stages' working set.  When a tensor has fewer than 256 16-byte
// column vectors (few KV heads), the spare threads take interleaved tokens
// and the partial sums are combined through LDS.
//
// Outputs: qbar [Hq, nbT, d] and kbar [Hkv, nbT, d] hold block means
// (f32); vnorm [Hkv, nbT] holds the mean (or max) over the block's tokens of
// the per-token L2 norm of V, computed in f32 from the 16 B slices of one
// head row, summed across the lanes that hold that row by a DPP scan.
#include "stem_device.h"

namespace stem {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

struct PoolArgs {
  const void *q, *k, *v;
  float *qbar, *kbar, *vnorm;
  PlanDev pd;
  int32_t Hq, Hkv, block, nbT;
  int32_t q_chunks, kv_chunks;
  int32_t vnorm_max;
};

template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
  static constexpr int N = 8;
  __device__ static void to_f32(const u32x4 &r, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(r[e] << 16);
      f[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
    }
  }
};
template <>
struct Vec<false> {
  static constexpr int N = 4;
  __device__ static void to_f32(const u32x4 &r, float (&f)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(r[e]);
  }
};

// Data-parallel-primitive (DPP) move of x from another lane, 0 where the
// source lies outside the row (16 lanes) or the row is masked off.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               ROW_MASK, 0xF, true));
}

// Sum of x over each group of L consecutive lanes (L = 8, 16 or 32), left in
// the group's last lane: an inclusive scan within 16-lane rows (row_shr by
// 1, 2, 4, 8) and, for L = 32, row 15's partial broadcast into the next row.
template <int L>
__device__ __forceinline__ float group_sum_last(float x) {
  x += dpp<0x111>(x);
  x += dpp<0x112>(x);
  x += dpp<0x114>(x);
  if constexpr (L >= 16) x += dpp<0x118>(x);
  if constexpr (L >= 32) x += dpp<0x142, 0xA>(x);
  return x;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs a) {
  constexpr int VEC = Vec<BF16>::N;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int LANES_PER_HEAD = D / VEC;  // 8, 16 or 32: divides 64
  static_assert(LANES_PER_HEAD == 8 || LANES_PER_HEAD == 16 || LANES_PER_HEAD == 32, "lanes per head row");
  __shared__ float red[kThreads * (VEC + 1)];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int unit = blockIdx.y;
  int tensor, H;
  if (unit < a.q_chunks) {
    tensor = 0; H = a.Hq;
  } else if (unit < a.q_chunks + a.kv_chunks) {
    tensor = 1; H = a.Hkv; unit -= a.q_chunks;
  } else {
    tensor = 2; H = a.Hkv; unit -= a.q_chunks + a.kv_chunks;
  }
  const int s = a.pd.blk_seq[b];
  const int ib = b - a.pd.cu_blocks[s];
  const int64_t tok0 = int64_t(a.pd.cu_seqlens[s]) + int64_t(ib) * a.block;
  const int n = min(int64_t(a.block), int64_t(a.pd.cu_seqlens[s + 1]) - tok0);

  const int col_vecs = H * D / VEC;
  const int cv0 = unit * kThreads;
  const int cv_count = min(kThreads, col_vecs - cv0);
  const int tsplit = kThreads / cv_count;
  const int cv = tid % cv_count;
  const int ts = tid / cv_count;
  const bool active = ts < tsplit;

  const char *base = static_cast<const char *>(tensor == 0 ? a.q : (tensor == 1 ? a.k : a.v));
  const int64_t row_bytes = int64_t(H) * D * ESZ;
  const char *src = base + tok0 * row_bytes + int64_t(cv0 + cv) * 16;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  float nacc = 0.f;

  for (int t0 = 0; t0 < n; t0 += tsplit * kUnroll) {
    u32x4 raw[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + ts + u * tsplit;
      ok[u] = active && t < n;
      if (ok[u]) {
        raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + int64_t(t) * row_bytes));
      } else {
        raw[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float f[VEC];
      Vec<BF16>::to_f32(raw[u], f);
      if (tensor == 2) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) sq = fmaf(f[e], f[e], sq);
        // sum over the lanes holding this head's row, in its last lane
        // (every lane of the wavefront takes part)
        sq = group_sum_last<LANES_PER_HEAD>(sq);
        const float nrm = sqrtf(sq);
        if (ok[u]) nacc = a.vnorm_max ? fmaxf(nacc, nrm) : nacc + nrm;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += f[e];
      }
    }
  }

  // combine the token-interleaved partial results
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[tid * VEC + e] = acc[e];
  red[kThreads * VEC + tid] = nacc;
  __syncthreads();
  if (ts != 0) return;
  for (int r = 1; r < tsplit; ++r) {
    const int o = r * cv_count + cv;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += red[o * VEC + e];
    const float x = red[kThreads * VEC + o];
    nacc = a.vnorm_max ? fmaxf(nacc, x) : nacc + x;
  }
  const int col = (cv0 + cv) * VEC;
  const int h = col / D;
  const int d0 = col % D;
  const float inv_n = 1.0f / float(n);
  if (tensor == 2) {
    if (d0 == D - VEC) a.vnorm[int64_t(h) * a.nbT + b] = a.vnorm_max ? nacc : nacc * inv_n;
    return;
  }
  float *dst = (tensor == 0 ? a.qbar : a.kbar) + (int64_t(h) * a.nbT + b) * D + d0;
#pragma unroll
  for (int e = 0; e < VEC; e += 4) {
    f32x4 o4 = {acc[e] / float(n), acc[e + 1] / float(n), acc[e + 2] / float(n),
                acc[e + 3] / float(n)};
    *reinterpret_cast<f32x4 *>(dst + e) = o4;
  }
}

}  // namespace

hipError_t launch_pool(const stem_plan_info &in, PlanDev pd, const void *q,
                       const void *k, const void *v, float *qbar, float *kbar,
                       float *vnorm, int vnorm_mode, hipStream_t st) {
  if (in.total_blocks == 0) return hipSuccess;
  const int vec = in.dtype == STEM_BF16 ? 8 : 4;
  PoolArgs a;
  a.q = q; a.k = k; a.v = v;
  a.qbar = qbar; a.kbar = kbar; a.vnorm = vnorm;
  a.pd = pd;
  a.Hq = in.num_q_heads;
  a.Hkv = in.num_kv_heads;
  a.block = in.block;
  a.nbT = static_cast<int32_t>(in.total_blocks);
  a.q_chunks = (in.num_q_heads * in.head_dim / vec + kThreads - 1) / kThreads;
  a.kv_chunks = (in.num_kv_heads * in.head_dim / vec + kThreads - 1) / kThreads;
  a.vnorm_max = vnorm_mode == STEM_VNORM_MAX;
  dim3 grid(static_cast<unsigned>(in.total_blocks), a.q_chunks + 2 * a.kv_chunks);
  if (in.dtype == STEM_BF16) {
    if (in.head_dim == 128)
      hipLaunchKernelGGL((pool_kernel<true, 128>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((pool_kernel<true, 64>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (in.head_dim == 128)
      hipLaunchKernelGGL((pool_kernel<false, 128>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((pool_kernel<false, 64>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace stem
