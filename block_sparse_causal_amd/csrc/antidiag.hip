// Block metric from anti-diagonal samples of the token logits
// (gist.science/fr, "Resume technique" 2.C step 1: the block metric is
// computed with anti-diagonal sampling).  For stride S (a power of two
// dividing the block size B), the tokens of a sequence form groups of S
// positions; the sample of query group r and key group c is the mean of
// q.k / sqrt(d) along the anti-diagonal of their S x S token tile (query
// position rS + S-1-u with key position cS + u), over the pairs whose tokens
// exist and whose key is not after the query.  The block logit t_ij is the
// log of the mean of exp(sample) over the samples of query block i and key
// block j; it then takes the place of the pooled logit in the metric, whose
// forms are unchanged (output-aware, additive, routing).
//
// Kernel 1 (antidiag_kernel): the samples are a causal matrix product per
// query head, Q' K'^T / S, where row r of Q' is the concatenation of the
// query tokens rS + S-1, rS + S-2, ..., rS of that head and row c of K' the
// key tokens cS, ..., cS + S-1 (depth S d).  One workgroup computes one
// 128 x 128 tile of groups with bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// f32 accumulation): 4 wavefronts of 64 x 64, operands staged through LDS
// 64 dimensions of one token position u at a time (16 KiB per operand per
// stage, double buffered, the next stage's global loads in flight while the
// current one is multiplied).  Block pairs never straddle a tile (128 groups
// are a whole number of blocks), so the tile finishes its block logits
// itself: samples go to LDS, a first pass reduces each (group row, key
// block) segment to a max and a sum of exponentials, a second pass combines
// the rows of each query block.
//
// Only the diagonal tile of each row of tiles holds samples whose
// anti-diagonal crosses the causal boundary (r = c): there the pairs with
// u >= ceil(S/2) have the key after the query, so those entries are frozen
// once the products of u < ceil(S/2) are accumulated.  Tokens past the end of
// a sequence load as zeros; each sample is divided by its own pair count.
//
// Kernel 2 (antidiag_metric_kernel): one wavefront per metric row turns the
// row's block logits into the metric in place (row softmax times V magnitude,
// the additive form, or the softmax alone).
#include "stem_device.h"

namespace stem {
namespace {

constexpr int kTile = 128;             // groups per tile side
constexpr int kRowBytes = 128;         // one staged row: 64 bf16 dimensions
constexpr int kOpBytes = kTile * kRowBytes;   // 16 KiB per operand per stage

struct AdArgs {
  const char *q, *k;
  float *out;
  PlanDev pd;
  int32_t Hq, Hkv, G, block, stride, num_seqs;
  int32_t units_per_head;     // bound on tile pairs per head (extra units exit)
  int64_t per_head;           // packed triangle elements per head
  float scale;                // 1 / sqrt(d)
};

// Locate tile pair u of the head's work: sequence s, row tile rt, column tile
// ct.  Pairs are numbered per sequence in bands of two row tiles, column tile
// major inside a band, so that work in flight together shares both operands.
__device__ __forceinline__ bool decode_unit(const AdArgs &a, int u, int &s, int &rt, int &ct) {
  for (s = 0; s < a.num_seqs; ++s) {
    const int len = a.pd.cu_seqlens[s + 1] - a.pd.cu_seqlens[s];
    const int ng = (len + a.stride - 1) / a.stride;
    const int nt = (ng + kTile - 1) / kTile;
    const int pairs = nt * (nt + 1) / 2;
    if (u >= pairs) { u -= pairs; continue; }
    for (int b = 0;; ++b) {
      const int r0 = 2 * b;
      const bool two = r0 + 1 < nt;
      const int cnt = two ? 2 * (r0 + 1) + 1 : r0 + 1;
      if (u >= cnt) { u -= cnt; continue; }
      if (!two) { rt = r0; ct = u; }
      else if (u < 2 * (r0 + 1)) { ct = u >> 1; rt = r0 + (u & 1); }
      else { ct = r0 + 1; rt = r0 + 1; }
      return true;
    }
  }
  return false;
}

// Number of anti-diagonal pairs behind the sample of groups (r, c), c <= r,
// for a sequence of len tokens (0: no sample).
__device__ __forceinline__ int pair_count(int r, int c, int S, int len) {
  const int m = min(S, len - r * S);       // tokens in query group r
  if (c < r) return m;
  const int half = (S + 1) >> 1;           // u < half: key not after query
  return max(0, min(m - 1, half - 1) - (S - m) + 1);
}

template <int D>
__global__ __launch_bounds__(256) void antidiag_kernel(AdArgs a) {
  constexpr int HALVES = D / 64;
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * kOpBytes];

  // XCD-aware numbering: consecutive workgroup ids go round robin over the 8
  // XCDs, so each XCD receives a contiguous range of units (grid % 8 == 0)
  const int id = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int grp_units = a.G * a.units_per_head;
  const int hk = id / grp_units;
  const int v = id - hk * grp_units;
  const int h = hk * a.G + v % a.G;         // heads of one KV group adjacent
  int s, rt, ct;
  if (hk >= a.Hkv || !decode_unit(a, v / a.G, s, rt, ct)) return;

  const int S = a.stride;
  const int t0 = a.pd.cu_seqlens[s];
  const int len = a.pd.cu_seqlens[s + 1] - t0;
  const int ng = (len + S - 1) / S;
  const int r0 = rt * kTile, c0 = ct * kTile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, n32 = lane & 31;

  // ---- staging roles: thread loads rows lrow + 32 p (p = 0..3), 16-byte chunk lch
  const int lrow = tid >> 3, lch = tid & 7;
  const int64_t qrow = int64_t(a.Hq) * D * 2, krow = int64_t(a.Hkv) * D * 2;
  const uint32_t st_off = uint32_t(lrow * kRowBytes + ((lch ^ (lrow & 7)) << 4));
  const int nst = S * HALVES;

  u32x4 ra[4], rb[4];
  auto load = [&](int st) {
    const int u = st / HALVES, half = st % HALVES;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qp = (r0 + lrow + 32 * p) * S + S - 1 - u;
      const int kp = (c0 + lrow + 32 * p) * S + u;
      const char *qa = a.q + (int64_t(t0) + qp) * qrow + int64_t(h) * D * 2 + half * 128 + lch * 16;
      const char *ka = a.k + (int64_t(t0) + kp) * krow + int64_t(hk) * D * 2 + half * 128 + lch * 16;
      ra[p] = qp < len ? *reinterpret_cast<const u32x4 *>(qa) : u32x4{0u, 0u, 0u, 0u};
      rb[p] = kp < len ? *reinterpret_cast<const u32x4 *>(ka) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
    char *A = lds + buf * 2 * kOpBytes, *Bm = A + kOpBytes;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<u32x4 *>(A + st_off + p * 32 * kRowBytes) = ra[p];
      *reinterpret_cast<u32x4 *>(Bm + st_off + p * 32 * kRowBytes) = rb[p];
    }
  };

  // ---- products: wavefront (wr, wc) owns rows wr*64.. and columns wc*64..
  const int wr = w >> 1, wc = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](int buf) {
    const char *A = lds + buf * 2 * kOpBytes, *Bm = A + kOpBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = ((2 * kk + hi) ^ (n32 & 7)) << 4;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        af[m] = *reinterpret_cast<const bf16x8 *>(A + (wr * 64 + m * 32 + n32) * kRowBytes + chunk);
#pragma unroll
      for (int n = 0; n < 2; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8 *>(Bm + (wc * 64 + n * 32 + n32) * kRowBytes + chunk);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
    }
  };

  // diagonal entries (row == column) of the diagonal 32 x 32 products: lane
  // (n32, hi) holds the one at element e_diag, if any
  const bool diag_wave = rt == ct && wr == wc;
  const int xd = n32 - 4 * hi;
  const bool has_diag = xd >= 0 && (xd & 4) == 0;
  const int e_diag = ((xd >> 3) << 2) | (xd & 3);
  const int st_freeze = ((S + 1) >> 1) * HALVES - 1;
  float frozen[2] = {0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) load(st + 1);
    compute(st & 1);
    if (diag_wave && st == st_freeze) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e == e_diag) frozen[m] = acc[m][m][e];
    }
    if (st + 1 < nst) store((st + 1) & 1);
    __syncthreads();
  }
  if (diag_wave && has_diag) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e == e_diag) acc[m][m][e] = frozen[m];
  }

  // ---- samples to LDS: f32 [128][128], -inf where there is no sample
  float *smp = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wr * 64 + m * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        const int cl = wc * 64 + n * 32 + n32;
        const int r = r0 + rl, c = c0 + cl;
        const int cnt = (r < ng && c <= r) ? pair_count(r, c, S, len) : 0;
        smp[rl * kTile + cl] = cnt > 0 ? acc[m][n][e] * (a.scale / float(cnt)) : -INFINITY;
      }
  __syncthreads();

  // ---- pass 1: each (row, key block) segment -> max and sum of exp(x - max),
  // left in the segment's first two slots
  const int gpb = a.block / S;             // groups per block
  const int nbt = kTile / max(gpb, 1);     // blocks per tile side (gpb <= 128)
  constexpr float kLog2e = 1.4426950408889634f;
  if (gpb > 1) {
    for (int it = tid; it < kTile * nbt; it += 256) {
      const int rl = it / nbt, jb = it - rl * nbt;
      float *seg = smp + rl * kTile + jb * gpb;
      float mx = -INFINITY;
      for (int x = 0; x < gpb; ++x) mx = fmaxf(mx, seg[x]);
      float sum = 0.f;
      if (mx != -INFINITY)
        for (int x = 0; x < gpb; ++x) sum += exp2f((seg[x] - mx) * kLog2e);
      seg[0] = mx;
      seg[1] = sum;
    }
    __syncthreads();
  }

  // ---- pass 2: combine the rows of each query block; write t_ij
  const int nrow_g = ng - r0;              // valid group rows in this tile (> 0)
  const int b_r0 = r0 / gpb, b_c0 = c0 / gpb;
  const int nb = a.pd.cu_blocks[s + 1] - a.pd.cu_blocks[s];
  float *orow = a.out + int64_t(h) * a.per_head + a.pd.tri[s];
  for (int it = tid; it < nbt * nbt; it += 256) {
    const int ib = it / nbt, jb = it - ib * nbt;
    const int i = b_r0 + ib, j = b_c0 + jb;
    if (i >= nb || j > i) continue;
    float mx = -INFINITY;
    const int rows = min(gpb, nrow_g - ib * gpb);
    for (int x = 0; x < rows; ++x) mx = fmaxf(mx, smp[(ib * gpb + x) * kTile + jb * gpb]);
    float t = -INFINITY;
    if (mx != -INFINITY) {
      float sum = 0.f;
      for (int x = 0; x < rows; ++x) {
        const float *seg = smp + (ib * gpb + x) * kTile + jb * gpb;
        const float l = gpb > 1 ? seg[1] : (seg[0] != -INFINITY ? 1.f : 0.f);
        if (seg[0] != -INFINITY) sum += l * exp2f((seg[0] - mx) * kLog2e);
      }
      // samples of the pair: every column of block j for each row when
      // j < i; the causal triangle plus the diagonal samples when j == i
      int ns;
      if (j < i) {
        ns = rows * gpb;
      } else {
        ns = rows * (rows - 1) / 2;
        for (int x = 0; x < rows; ++x) {
          const int r = r0 + ib * gpb + x;
          ns += pair_count(r, r, S, len) > 0;
        }
      }
      t = mx + __logf(sum / float(ns));
    }
    orow[int64_t(i) * (i + 1) / 2 + j] = t;
  }
}

// ---- metric rows from block logits, in place
struct MetricArgs {
  float *scores;
  const float *vnorm;
  PlanDev pd;
  int32_t Hq, Hkv, nbT, mode;
  int64_t per_head;
  float beta;
};

__global__ __launch_bounds__(256) void antidiag_metric_kernel(MetricArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= int64_t(a.Hq) * a.nbT) return;
  const int h = int(row / a.nbT), b = int(row - int64_t(h) * a.nbT);
  const int s = a.pd.blk_seq[b];
  const int i = b - a.pd.cu_blocks[s];
  const int b0 = a.pd.cu_blocks[s];
  const int hk = h / (a.Hq / a.Hkv);
  float *x = a.scores + int64_t(h) * a.per_head + a.pd.tri[s] + int64_t(i) * (i + 1) / 2;
  const float *wv = a.vnorm + int64_t(hk) * a.nbT + b0;
  const int n = i + 1;
  constexpr float kLog2e = 1.4426950408889634f;
  if (a.mode == STEM_METRIC_ADDITIVE) {
    for (int j = lane; j < n; j += 64) {
      const float wj = wv[j];
      const float bonus = wj > 0.f ? fmaxf(0.f, __logf(wj * wj)) : 0.f;
      x[j] = x[j] + a.beta * bonus;
    }
    return;
  }
  // online max / sum over the row, then one wavefront reduction
  float mx = -INFINITY, sum = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float t = x[j];
    if (t == -INFINITY) continue;
    if (t > mx) { sum = sum * exp2f((mx - t) * kLog2e) + 1.f; mx = t; }
    else sum += exp2f((t - mx) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o), os = __shfl_xor(sum, o);
    const float nm = fmaxf(mx, om);
    sum = (mx == -INFINITY ? 0.f : sum * exp2f((mx - nm) * kLog2e)) +
          (om == -INFINITY ? 0.f : os * exp2f((om - nm) * kLog2e));
    mx = nm;
  }
  const float inv = mx == -INFINITY ? 0.f : 1.f / sum;
  const bool oam = a.mode == STEM_METRIC_OUTPUT_AWARE;
  for (int j = lane; j < n; j += 64) {
    const float t = x[j];
    const float p = t == -INFINITY ? 0.f : exp2f((t - mx) * kLog2e) * inv;
    x[j] = oam ? p * wv[j] : p;
  }
}

}  // namespace

int64_t antidiag_units_per_head(const stem_plan_info &in, int stride) {
  const int64_t gpb = in.block / stride;
  const int64_t ntmax = (int64_t(in.max_seq_blocks) * gpb + kTile - 1) / kTile;
  const int64_t nt_sum = (in.total_blocks * gpb + kTile - 1) / kTile + in.num_seqs;
  return (ntmax + 1) * nt_sum / 2 + 1;
}

hipError_t launch_score_antidiag(const stem_plan_info &in, PlanDev pd, const void *q,
                                 const void *k, const float *vnorm, int stride,
                                 float *scores, hipStream_t st) {
  if (in.total_blocks == 0) return hipSuccess;
  AdArgs a;
  a.q = static_cast<const char *>(q);
  a.k = static_cast<const char *>(k);
  a.out = scores;
  a.pd = pd;
  a.Hq = in.num_q_heads;
  a.Hkv = in.num_kv_heads;
  a.G = in.num_q_heads / in.num_kv_heads;
  a.block = in.block;
  a.stride = stride;
  a.num_seqs = in.num_seqs;
  a.units_per_head = static_cast<int32_t>(antidiag_units_per_head(in, stride));
  a.per_head = in.score_elems_per_head;
  a.scale = 1.0f / sqrtf(float(in.head_dim));
  const int64_t units = int64_t(in.num_q_heads) * a.units_per_head;
  const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
  if (in.head_dim == 128)
    hipLaunchKernelGGL(antidiag_kernel<128>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(antidiag_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  MetricArgs m;
  m.scores = scores;
  m.vnorm = vnorm;
  m.pd = pd;
  m.Hq = in.num_q_heads;
  m.Hkv = in.num_kv_heads;
  m.nbT = static_cast<int32_t>(in.total_blocks);
  m.mode = in.metric_mode;
  m.per_head = in.score_elems_per_head;
  m.beta = static_cast<float>(in.beta);
  const int64_t rows = int64_t(in.num_q_heads) * in.total_blocks;
  hipLaunchKernelGGL(antidiag_metric_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256),
                     0, st, m);
  return hipGetLastError();
}

}  // namespace stem
