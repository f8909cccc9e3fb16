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
// (round robin) and merge their row statistics through LDS.  Work items are
// dispatched row tile major (every head's heaviest tiles first), which keeps
// the triangular work from leaving a tail of heavy tiles at the end.
// The pooled dot products are an f32 GEMM on the matrix cores
// (v_mfma_f32_32x32x2_f32, computing the transposed tile keys x queries so
// that each lane holds one query row's values and row statistics never leave
// the lane pair l, l^32).  Operands are staged per wavefront in LDS by
// coalesced global->LDS DMA of whole 32-row tiles (the next key tile's DMA
// overlaps the current tile's products), and results leave through a
// per-wavefront LDS transpose so that every store covers 32 consecutive
// keys of a row.
// For bf16 inputs the products run on the bf16 matrix cores with each f32
// operand split into a bf16 high part and a bf16 remainder (three products,
// f32 accumulation, relative error about 2^-16 of the product magnitudes);
// f32 inputs keep the f32 products.
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

// 32 rows of D floats in LDS, row-major with the 16-byte chunks of row r
// XOR-swizzled by r % 16: the matrix-core operand reads (lane (n, hi) reads
// row n, chunks hi D/8 .. hi D/8 + D/8 - 1) are free of bank conflicts.
template <int D>
struct RowTile {
  static constexpr int CPR = D / 4;          // chunks per row
  static constexpr int LOADS = 32 * CPR / 64;
  // DMA rows base + row_of(r) * D (r = 0..31; row_of clamps) into this tile
  template <typename F>
  __device__ __forceinline__ static void load(uint32_t lds, int lane, const float *base, F &&row_of) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int q = it * 64 + lane;
      const int r = q / CPR, pc = q % CPR;
      const int lc = pc ^ (r % 16);
      dma16(base, static_cast<uint32_t>(row_of(r)) * (D * 4) + lc * 16, lds + it * 1024);
    }
  }
  __device__ __forceinline__ static f32x4 read(const char *tile, int row, int chunk) {
    return *reinterpret_cast<const f32x4 *>(tile + row * (D * 4) + ((chunk ^ (row % 16)) * 16));
  }
};

// A 32 x 32 tile in matrix-core layout (lane (n, hi) element r holds query
// row n, key column 8 (r / 4) + 4 hi + r % 4) is written to global memory
// row by row: it goes through this wavefront's 4 KiB of LDS (16-byte chunks
// of row r XOR-swizzled by r % 8), and each store then covers two query
// rows of 32 consecutive keys.
struct TileIO {
  float *t;
  int lane, n, hi;
  __device__ __forceinline__ int at(int row, int col) const {
    return row * 32 + ((((col >> 2) ^ (row & 7)) << 2) | (col & 3));
  }
  __device__ __forceinline__ void put(const f32x16 &acc) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) t[at(n, 8 * (r >> 2) + 4 * hi + (r & 3))] = acc[r];
  }
  __device__ __forceinline__ float get(int it) const { return t[at(2 * it + (lane >> 5), lane & 31)]; }
};

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (both round to nearest
// even): hi.hi' + hi.lo' + lo.hi' equals the f32 product x.x' up to the
// dropped lo.lo' term and the rounding of lo, both about 2^-16 of |x x'|.
__device__ __forceinline__ void split_bf16(const f32x8 &x, bf16x8 &h, bf16x8 &l) {
  h = __builtin_convertvector(x, bf16x8);
  l = __builtin_convertvector(x - __builtin_convertvector(h, f32x8), bf16x8);
}

// SPLIT: the pooled dot products as three bf16 matrix products of the split
// operands (v_mfma_f32_32x32x16_bf16, f32 accumulation), for bf16 inputs;
// otherwise one f32 product (v_mfma_f32_32x32x2_f32).
template <int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(ScoreArgs a) {
  constexpr int HALF = D / 2;
  constexpr int KTILE = 32 * D * 4;          // bytes of one staged 32-row tile
  // [8 operand tiles][8 transpose tiles]; after the first pass the operand
  // tiles hold the row statistics
  __shared__ __attribute__((aligned(16))) char lds[kScoreWaves * KTILE + kScoreWaves * 4096];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;        // query row inside the tile / key row of the A operand
  const int hi = lane >> 5;       // which half of the head dimension this lane feeds
  // work item = (row tile t, head h), t major, so that every head's
  // heaviest row tiles are dispatched first
  const int h = blockIdx.x % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  char *ktile = lds + wv * KTILE;
  const uint32_t ktile_addr = lds_addr_of(ktile);
  const TileIO io{reinterpret_cast<float *>(lds + kScoreWaves * KTILE + wv * 4096), lane, n, hi};
  float *st_m = reinterpret_cast<float *>(lds);                       // [8][64]
  float *st_l = st_m + kScoreWaves * 64;                              // [8][64]
  float *row_m = st_l + kScoreWaves * 64;                             // [32]
  float *row_il = row_m + 32;                                         // [32]

  // tile -> (sequence, row tile), heaviest (last) row tiles first
  int t = blockIdx.x / a.Hq;
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
  float *out_hs = a.scores + int64_t(h) * a.per_head + a.pd.tri[s];
  const float *w = a.vnorm + int64_t(g) * a.nbT + b0;
  const float *qrows = a.qbar + (int64_t(h) * a.nbT + b0) * D;
  const float *krows = a.kbar + (int64_t(g) * a.nbT + b0) * D;

  // Row-major pass over a tile: element (row 2 it + lane / 32, key j0 + lane % 32)
  // exists when the row is a valid query block and the key is causal.
  auto for_rows = [&](int j0, auto &&fn) {
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int row = 2 * it + (lane >> 5);
      const int qr = i0 + row;
      const int j = j0 + (lane & 31);
      if (qr < nb && j <= qr) fn(it, row, j, (int64_t(qr) * (qr + 1)) / 2 + j);
    }
  };

  // B operand: qbar row qi, contraction index c <-> dim hi*HALF + c (rows
  // past the sequence read its last row; their logits are masked)
  float qv[HALF];
  RowTile<D>::load(ktile_addr, lane, qrows, [&](int r) { return min(i0 + r, nb - 1); });
  wait_vm();
#pragma unroll
  for (int c = 0; c < HALF / 4; ++c) {
    const f32x4 x = RowTile<D>::read(ktile, n, hi * (HALF / 4) + c);
    qv[4 * c] = x[0]; qv[4 * c + 1] = x[1]; qv[4 * c + 2] = x[2]; qv[4 * c + 3] = x[3];
  }

  // split operand of the bf16 products: contraction chunk c covers dims
  // hi*HALF + 8c .. + 7, the same dims in both operands
  bf16x8 qh[SPLIT ? HALF / 8 : 1], ql[SPLIT ? HALF / 8 : 1];
  if constexpr (SPLIT) {
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = qv[8 * c + e];
      split_bf16(x, qh[c], ql[c]);
    }
  }

  // pass 1: wavefront wv takes key tiles wv, wv + 8, ...; an online row
  // max / sum is kept per lane.  The scaled logits of the first kKeep tiles
  // stay in registers; those of later tiles are parked in the output and
  // re-read in pass 2.  The next tile's DMA overlaps this tile's products.
  constexpr int kKeep = 4;
  float mrun = -INFINITY, lrun = 0.f;
  const int last_row = min(i0 + 31, nb - 1);
  const int jt_end = last_row / 32;
  auto load_k = [&](int jt) {
    RowTile<D>::load(ktile_addr, lane, krows, [&](int r) { return min(jt * 32 + r, nb - 1); });
  };
  f32x16 keep[kKeep];
  int slot = 0;
  // the operand reads of qv must be done before the tile is overwritten
  wait_lgkm();
  if (wv <= jt_end) load_k(wv);
  for (int jt = wv; jt <= jt_end; jt += kScoreWaves, ++slot) {
    wait_vm();
    f32x4 kcur[HALF / 4];
#pragma unroll
    for (int c = 0; c < HALF / 4; ++c) kcur[c] = RowTile<D>::read(ktile, n, hi * (HALF / 4) + c);
    wait_lgkm();   // operands in registers: the tile may be refilled
    if (jt + kScoreWaves <= jt_end) load_k(jt + kScoreWaves);
    f32x16 acc = {};
    if constexpr (SPLIT) {
#pragma unroll
      for (int c = 0; c < HALF / 8; ++c) {
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = kcur[2 * c][e]; x[4 + e] = kcur[2 * c + 1][e]; }
        bf16x8 kh, kl;
        split_bf16(x, kh, kl);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[c], acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < HALF / 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kcur[c][e], qv[4 * c + e], acc, 0, 0, 0);
    }
    const int j0 = jt * 32;
    // acc[r] = logit(key j0 + 8(r/4) + 4hi + r%4, query qi)
    if constexpr (MODE == STEM_METRIC_ADDITIVE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] *= a.scale;
      io.put(acc);
      for_rows(j0, [&](int it, int, int j, int64_t off) {
        // log(w^2) as 2 log w: no overflow for large w; log 0 = -inf -> 0
        const float bonus = fmaxf(0.f, 2.f * logf(w[j]));
        out_hs[off] = fmaf(a.beta, bonus, io.get(it));
      });
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
      io.put(acc);
      for_rows(j0, [&](int it, int, int, int64_t off) { out_hs[off] = io.get(it); });
    }
  }
  if constexpr (MODE == STEM_METRIC_ADDITIVE) return;
  // combine the statistics of the 8 wavefronts and of the two lanes that
  // share a query row (the operand tiles are free once every wavefront is
  // past its last product)
  __syncthreads();
  st_m[wv * 64 + lane] = mrun;
  st_l[wv * 64 + lane] = lrun;
  __syncthreads();
  if (wv == 0 && hi == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kScoreWaves; ++v) M = fmaxf(M, fmaxf(st_m[v * 64 + n], st_m[v * 64 + n + 32]));
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < kScoreWaves; ++v) {
      const float m0 = st_m[v * 64 + n], m1 = st_m[v * 64 + n + 32];
      if (m0 != -INFINITY) L += st_l[v * 64 + n] * __expf(m0 - M);
      if (m1 != -INFINITY) L += st_l[v * 64 + n + 32] * __expf(m1 - M);
    }
    row_m[n] = M;
    row_il[n] = 1.0f / L;
  }
  __syncthreads();
  // pass 2: write this wavefront's values as exp(x - M) / L (* vnorm)
  auto final_value = [&](float x, int row, int j) {
    const float p = __expf(x - row_m[row]) * row_il[row];
    return MODE == STEM_METRIC_ROUTING ? p : p * w[j];
  };
  slot = 0;
  for (int jt = wv; jt <= jt_end; jt += kScoreWaves, ++slot) {
    const int j0 = jt * 32;
    if (slot < kKeep) {
#pragma unroll
      for (int k = 0; k < kKeep; ++k)
        if (k == slot) io.put(keep[k]);
      for_rows(j0, [&](int it, int row, int j, int64_t off) {
        out_hs[off] = final_value(io.get(it), row, j);
      });
    } else {
      for_rows(j0, [&](int, int row, int j, int64_t off) {
        out_hs[off] = final_value(out_hs[off], row, j);
      });
    }
  }
}

template <int D, int MODE>
void launch_score_d_mode(bool split, dim3 grid, dim3 block, hipStream_t st, const ScoreArgs &a) {
  if (split) hipLaunchKernelGGL((score_kernel<D, MODE, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((score_kernel<D, MODE, false>), grid, block, 0, st, a);
}

template <int D>
void launch_score_d(int mode, bool split, dim3 grid, dim3 block, hipStream_t st, const ScoreArgs &a) {
  if (mode == STEM_METRIC_ADDITIVE) launch_score_d_mode<D, STEM_METRIC_ADDITIVE>(split, grid, block, st, a);
  else if (mode == STEM_METRIC_ROUTING) launch_score_d_mode<D, STEM_METRIC_ROUTING>(split, grid, block, st, a);
  else launch_score_d_mode<D, STEM_METRIC_OUTPUT_AWARE>(split, grid, block, st, a);
}

void launch_score_kernel(bool d128, int mode, bool split, dim3 grid, dim3 block, hipStream_t st,
                         const ScoreArgs &a) {
  if (d128) launch_score_d<128>(mode, split, grid, block, st, a);
  else launch_score_d<64>(mode, split, grid, block, st, a);
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
  dim3 grid(static_cast<unsigned>(tiles * in.num_q_heads));
  const dim3 block(64 * kScoreWaves);
  const bool d128 = in.head_dim == 128;
  const int mode = in.metric_mode == STEM_METRIC_ADDITIVE || in.metric_mode == STEM_METRIC_ROUTING
                       ? in.metric_mode : STEM_METRIC_OUTPUT_AWARE;
  const bool split = in.dtype == STEM_BF16;
  launch_score_kernel(d128, mode, split, grid, block, st, a);
  return hipGetLastError();
}

}  // namespace stem
