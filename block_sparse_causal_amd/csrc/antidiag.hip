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
// key tokens cS, ..., cS + S-1 (depth S d).  One workgroup of 4 wavefronts
// computes a tile of 256 query groups x 128 key groups on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16, f32 accumulation), each wavefront 64 rows
// x 128 columns (eight 32 x 32 products: 6 KiB of LDS operand reads per 8
// products).  Operands arrive by global->LDS DMA, 32 dimensions of one token
// position u per stage (24 KiB), three stage buffers with the loads two
// stages ahead; two workgroups share a CU, so one's epilogue overlaps the
// other's products.  Block pairs never straddle a tile (its sides are whole
// numbers of blocks), so the tile finishes its block logits itself, in
// registers: the Q' operand rows are read in a permuted order that leaves
// each lane holding 16 consecutive group rows of one column, so within each
// 32 x 32 product the samples of a block pair (or of its 32 x 32 part,
// combined through LDS when blocks hold more than 32 groups) reduce to a max
// and a sum of exponentials in the lane and across lanes by DPP.
//
// Only the tiles on the diagonal hold samples whose anti-diagonal crosses the
// causal boundary (r = c): there the pairs with u >= ceil(S/2) have the key
// after the query, so those entries are frozen once the products of
// u < ceil(S/2) are accumulated.  Token rows past the end of a sequence are
// clamped to its last token and their samples masked; in the tiles holding a
// short last group, the staged rows of its missing tokens are zeroed, so each
// sample sums exactly its own pairs and is divided by its own pair count.
//
// f32 inputs take antidiag_f32_kernel instead: one workgroup per metric row,
// each thread forming whole samples from f32 dot products.
//
// Kernel 2 (antidiag_metric_kernel): one wavefront per metric row turns the
// row's block logits into the metric in place (row softmax times V magnitude,
// the additive form, or the softmax alone).
#include <type_traits>

#include "stem_device.h"

namespace stem {
namespace {

// f(std::integral_constant<int, I>()) for I = FIRST .. LAST - 1
template <int FIRST, int LAST, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (FIRST < LAST) {
    f(std::integral_constant<int, FIRST>{});
    static_for<FIRST + 1, LAST>(f);
  }
}

// Two DMAs (see dma16x4) in one asm block: M0 saved and restored once.
__device__ __forceinline__ void dma16x2(const void *g0, uint32_t v0, uint32_t l0,
                                        const void *g1, uint32_t v1, uint32_t l1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v0), "v"(v1), "s"(g0), "s"(g1), "s"(l0), "s"(l1)
      : "memory");
}

constexpr int kTM = 256;                 // query groups per tile
constexpr int kTN = 128;                 // key groups per tile
constexpr int kSRow = 64;                // bytes per staged row: 32 bf16 dimensions
constexpr int kAB = kTM * kSRow;         // 16 KiB of Q' per stage
constexpr int kStage = kAB + kTN * kSRow;   // + 8 KiB of K'
constexpr int kNBuf = 3;
constexpr int kDmaA = kAB / 1024 / 4;    // 1 KiB DMAs per wavefront per stage: 4 for Q'
constexpr int kDmaB = kTN * kSRow / 1024 / 4;   // and 2 for K'
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AdArgs {
  const char *q, *k;
  float *out;
  PlanDev pd;
  int32_t Hq, Hkv, G, block, stride, num_seqs;
  int32_t units_per_head;     // bound on tile pairs per head (extra units exit)
  int64_t per_head;           // packed triangle elements per head
  float scale;                // 1 / sqrt(d)
};

// Tile pairs of a sequence with ng groups: row tile rt pairs with column
// tiles 0 .. min(2 rt + 1, ntc - 1), so rt(rt + 1) pairs precede row tile rt.
__device__ __forceinline__ int seq_pairs(int ng) {
  const int ntr = (ng + kTM - 1) / kTM, ntc = (ng + kTN - 1) / kTN;
  return ntr * (ntr + 1) - (2 * ntr - ntc);
}

// Locate tile pair u of the head's work (sequence s, row tile rt, column
// tile ct); column tiles are innermost, so work in flight together shares
// its row tile of Q'.
__device__ __forceinline__ bool decode_unit(const AdArgs &a, int u, int &s, int &rt, int &ct) {
  for (s = 0; s < a.num_seqs; ++s) {
    const int len = a.pd.cu_seqlens[s + 1] - a.pd.cu_seqlens[s];
    const int pairs = seq_pairs((len + a.stride - 1) / a.stride);
    if (u >= pairs) { u -= pairs; continue; }
    int x = int((sqrtf(4.0f * float(u) + 1.0f) - 1.0f) * 0.5f);
    while (x * (x + 1) > u) --x;
    while ((x + 1) * (x + 2) <= u) ++x;
    rt = x;
    ct = u - x * (x + 1);
    return true;
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

// Samples of block pair (i, j) of a sequence with ng groups (gpb groups per
// block): every column of block j for each of block i's rows when j < i; the
// causal triangle plus the diagonal samples that hold a pair when j == i.
__device__ __forceinline__ int pair_samples(int i, int j, int gpb, int ng, int S, int len) {
  const int rows = min(gpb, ng - i * gpb);
  if (j < i) return rows * gpb;
  int ns = rows * (rows - 1) / 2;
  for (int x = 0; x < rows; ++x) ns += pair_count(i * gpb + x, i * gpb + x, S, len) > 0;
  return ns;
}

// Data-parallel-primitive (DPP) move of x within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
// op(x[l], x[l ^ 32]) in every lane l (only blocks of 32 or more groups
// need it)
template <bool MAX>
__device__ __forceinline__ float halves(float x) {
  const float y = __shfl_xor(x, 32);
  return MAX ? fmaxf(x, y) : x + y;
}

// Combine x over groups of G consecutive lanes (G = 1 .. 32) within each
// half of the wavefront: butterflies of quad permutes and row mirrors.
template <int G, bool MAX>
__device__ __forceinline__ float lane_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (G >= 2) x = op(x, dpp<0xB1>(x));     // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x = op(x, dpp<0x4E>(x));     // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x = op(x, dpp<0x141>(x));    // row_half_mirror
  if constexpr (G >= 16) x = op(x, dpp<0x140>(x));   // row_mirror
  if constexpr (G >= 32) x = op(x, __shfl_xor(x, 16));
  return x;
}

// Max and sum of exp2(y - max) over groups of G x G samples of one 32 x 32
// product (G = 1 .. 32).  The products' rows are permuted (see the operand
// reads) so that lane (n, hi) holds rows 16 hi + e, e = 0..15, of column n:
// a group's G rows (G <= 16) lie in one lane, its G columns in G consecutive
// lanes.  On return mx[k], sm[k] hold the result of the lane's k-th row
// group (k < NR) in every lane of the group's columns (and, for G = 32, of
// both halves).
template <int G>
struct Groups {
  static constexpr int EG = G < 16 ? G : 16;   // elements of a group in one lane
  static constexpr int NR = 16 / EG;
  __device__ __forceinline__ static void reduce(const float (&y)[16], float (&mx)[NR], float (&sm)[NR]) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      float v = y[k * EG];
#pragma unroll
      for (int e = 1; e < EG; ++e) v = fmaxf(v, y[k * EG + e]);
      if constexpr (G == 32) v = halves<true>(v);
      mx[k] = lane_reduce<G, true>(v);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      float v = 0.f;
      if (mx[k] != -INFINITY) {
#pragma unroll
        for (int e = 0; e < EG; ++e) v += exp2f(y[k * EG + e] - mx[k]);
      }
      if constexpr (G == 32) v = halves<false>(v);
      sm[k] = lane_reduce<G, false>(v);
    }
  }
};

// LDS chunk swizzles of staged rows (4 chunks of 16 bytes per 64-byte row):
// eight lanes reading one logical chunk of rows {0..3, 16..19} + 4 j (Q',
// permuted) or of rows 0..7 + 8 j (K') hit eight different bank groups.
__device__ __forceinline__ int swz_a(int row) { return ((row >> 1) & 1) | ((row >> 3) & 2); }
__device__ __forceinline__ int swz_b(int row) { return (row >> 1) & 3; }

// Group size of the epilogue, and whether a group is a whole block pair
// (blocks of at most 32 groups) or a 32 x 32 part of one.
template <int G, bool WHOLE>
struct GroupTag {
  static constexpr int kG = G;
  static constexpr bool kWhole = WHOLE;
};

template <int D>
__global__ __launch_bounds__(256, 2) void antidiag_kernel(AdArgs a) {
  constexpr int QTR = D / 32;              // 32-dimension stages per token position
  __shared__ __attribute__((aligned(16))) char lds[kNBuf * kStage];

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
  const int r0 = rt * kTM, c0 = ct * kTN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, n32 = lane & 31;
  const int nst = S * QTR;

  // ---- DMA roles: DMA k of a stage moves 16 staged rows (1 KiB); lane L
  // lands at row 16 k + L / 4, LDS chunk L % 4, which holds the row's logical
  // chunk (L % 4) ^ swizzle(row) (swz_a for Q' rows, swz_b for K' rows): the
  // operand reads below are free of bank conflicts
  const int64_t qrow = int64_t(a.Hq) * D * 2, krow = int64_t(a.Hkv) * D * 2;
  const int drow = lane >> 2;
  const char *qtile = a.q + (int64_t(t0) + int64_t(r0) * S) * qrow + int64_t(h) * D * 2;
  const char *ktile = a.k + (int64_t(t0) + int64_t(c0) * S) * krow + int64_t(hk) * D * 2;
  const int qlim = len - 1 - r0 * S, klim = len - 1 - c0 * S;   // last token, tile-relative
  const uint32_t lds0 = lds_addr_of(lds);
  // whole tiles (every token of the tile's groups exists): the clamps never
  // bind, each lane's byte offsets are constants and the token position u
  // moves the scalar bases only
  static_assert(kDmaA == 4 && kDmaB == 2, "DMA batches");
  const bool qfull = (r0 + kTM) * S <= len, kfull = (c0 + kTN) * S <= len;
  uint32_t qoff[kDmaA], koff[kDmaB];
#pragma unroll
  for (int x = 0; x < kDmaA; ++x) {
    const int row = 16 * (w + 4 * x) + drow;
    qoff[x] = uint32_t(row * S + S - 1) * uint32_t(qrow) + (((lane & 3) ^ swz_a(row)) * 16);
  }
#pragma unroll
  for (int x = 0; x < kDmaB; ++x) {
    const int row = 16 * (w + 4 * x) + drow;
    koff[x] = uint32_t(row * S) * uint32_t(krow) + (((lane & 3) ^ swz_b(row)) * 16);
  }
  auto issue = [&](int st, int buf) {
    const int u = st / QTR, qt = st - u * QTR;
    const uint32_t sb = lds0 + buf * kStage;
    if (qfull && kfull) {
      const char *ga = qtile + qt * 64 - int64_t(u) * qrow;
      const char *gb = ktile + qt * 64 + int64_t(u) * krow;
      dma16x4(ga, qoff[0], sb + (w + 0) * 1024, ga, qoff[1], sb + (w + 4) * 1024,
              ga, qoff[2], sb + (w + 8) * 1024, ga, qoff[3], sb + (w + 12) * 1024);
      dma16x2(gb, koff[0], sb + kAB + (w + 0) * 1024, gb, koff[1], sb + kAB + (w + 4) * 1024);
      return;
    }
#pragma unroll
    for (int x = 0; x < kDmaA; ++x) {
      const int row = 16 * (w + 4 * x) + drow;
      const int chunk = (lane & 3) ^ swz_a(row);
      const int tok = min(row * S + S - 1 - u, qlim);
      dma16(qtile + qt * 64, uint32_t(tok) * uint32_t(qrow) + chunk * 16, sb + (w + 4 * x) * 1024);
    }
#pragma unroll
    for (int x = 0; x < kDmaB; ++x) {
      const int row = 16 * (w + 4 * x) + drow;
      const int chunk = (lane & 3) ^ swz_b(row);
      const int tok = min(row * S + u, klim);
      dma16(ktile + qt * 64, uint32_t(tok) * uint32_t(krow) + chunk * 16,
            sb + kAB + (w + 4 * x) * 1024);
    }
  };

  // a short last group in this tile: its missing tokens' staged rows are
  // zeroed after they land (query row r_last for u < S - m, key row c_last
  // for u >= m, m = tokens in the last group)
  const int m_last = len - (ng - 1) * S;
  const bool partial = m_last < S && ((ng - 1 >= r0 && ng - 1 < r0 + kTM) ||
                                      (ng - 1 >= c0 && ng - 1 < c0 + kTN));

  // ---- products: wavefront w owns rows 64 w .. 64 w + 63, all 128 columns
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // rows wholly above the causal boundary or past the sequence: no products
  const bool idle = r0 + 64 * w + 63 < c0 || r0 + 64 * w >= ng;
  // Q' operand rows are read permuted: the product's row 8 a + 4 h + c
  // (a = 0..3, h, c = 0..3) takes Q' row 16 h + 4 a + c of its 32, so that
  // lane (n, hi) ends up holding rows 16 hi + e of column n
  const int prow = 16 * ((n32 >> 2) & 1) + 4 * (n32 >> 3) + (n32 & 3);
  auto compute = [&](int buf) {
    const char *A = lds + buf * kStage, *Bm = A + kAB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ca = ((2 * kk + hi) ^ swz_a(prow)) << 4;
      const int cb = ((2 * kk + hi) ^ swz_b(n32)) << 4;
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        af[m] = *reinterpret_cast<const bf16x8 *>(A + (64 * w + 32 * m + prow) * kSRow + ca);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8 *>(Bm + (32 * n + n32) * kSRow + cb);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
    }
  };

  // diagonal entries (r == c): product (m, ndg + m) of this wavefront, lane
  // (n32, hi) holding the one at element e_diag = n32 - 16 hi if any
  const int ndg = 2 * w - 4 * (ct - 2 * rt);
  const bool diag_wave = ndg > -2 && ndg < 4;
  const int e_diag = n32 - 16 * hi;
  const bool has_diag = e_diag >= 0 && e_diag < 16;
  const int st_freeze = ((S + 1) >> 1) * QTR - 1;
  float frozen[2] = {0.f, 0.f};

  issue(0, 0);
  issue(1, 1);                             // nst >= 2 (S >= 1, D >= 64)
  auto stage = [&](int st, auto btag) {
    constexpr int buf = decltype(btag)::value;
    if (st + 1 < nst) __builtin_amdgcn_s_waitcnt(0x0F70 | (kDmaA + kDmaB));
    else wait_vm();
    __syncthreads();
    if (partial) {
      const int u = st / QTR;
      char *A = lds + buf * kStage;
      if (tid < 4 && u < S - m_last && ng - 1 >= r0 && ng - 1 < r0 + kTM)
        *reinterpret_cast<u32x4 *>(A + (ng - 1 - r0) * kSRow + tid * 16) = u32x4{0u, 0u, 0u, 0u};
      if (tid >= 4 && tid < 8 && u >= m_last && ng - 1 >= c0 && ng - 1 < c0 + kTN)
        *reinterpret_cast<u32x4 *>(A + kAB + (ng - 1 - c0) * kSRow + (tid - 4) * 16) =
            u32x4{0u, 0u, 0u, 0u};
      wait_lgkm();
      __syncthreads();
    }
    if (st + 2 < nst) issue(st + 2, (buf + 2) % kNBuf);
    if (!idle) compute(buf);
    if (diag_wave && st == st_freeze) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          if (n == ndg + m)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (e == e_diag) frozen[m] = acc[m][n][e];
    }
  };
  // unrolled over the buffers: every buffer offset is a constant
  for (int st = 0; st < nst; st += kNBuf)
    static_for<0, kNBuf>([&](auto b) {
      if (st + decltype(b)::value < nst) stage(st + decltype(b)::value, b);
    });
  if (diag_wave && has_diag) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (n == ndg + m)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (e == e_diag) acc[m][n][e] = frozen[m];
  }

  // ---- block logits
  const int gpb = a.block / S;             // groups per block (1 .. 128)
  const int nb = a.pd.cu_blocks[s + 1] - a.pd.cu_blocks[s];
  float *orow = a.out + int64_t(h) * a.per_head + a.pd.tri[s];
  // every sample of the tile exists and counts S pairs: all key groups before
  // all query groups, all query groups full
  const bool interior = c0 + kTN <= r0 && (r0 + kTM) * S <= len;
  const float lscale = a.scale * kLog2e;   // samples kept in log2 units
  const float fscale = lscale / float(S);

  auto finish = [&](auto grp) __attribute__((always_inline)) {
    using Gr = decltype(grp);
    constexpr int G = Gr::kG;
    using R = Groups<G>;
    // one 32 x 32 product at a time (a loop, not unrolled: the code stays
    // small; the product is first copied out with constant indices)
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
      const int m = t >> 2, n = t & 3;
      float x[16];
      switch (t) {
#define STEM_AD_TAKE(T)                                              \
  case T:                                                            \
    _Pragma("unroll") for (int e = 0; e < 16; ++e) x[e] = acc[T >> 2][T & 3][e]; \
    break;
        STEM_AD_TAKE(0) STEM_AD_TAKE(1) STEM_AD_TAKE(2) STEM_AD_TAKE(3)
        STEM_AD_TAKE(4) STEM_AD_TAKE(5) STEM_AD_TAKE(6) STEM_AD_TAKE(7)
#undef STEM_AD_TAKE
      }
      const int rb = r0 + 64 * w + 32 * m + 16 * hi, cb = c0 + 32 * n;
      // samples in log2 units: y = acc * scale * log2(e) / pairs
      if (idle) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = -INFINITY;
      } else if (interior) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] *= fscale;
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = rb + e, c = cb + n32;
          const int cnt = (r < ng && c <= r) ? pair_count(r, c, S, len) : 0;
          x[e] = cnt > 0 ? x[e] * (lscale / float(cnt)) : -INFINITY;
        }
      }
      float mx[R::NR], sm[R::NR];
      R::reduce(x, mx, sm);
      if constexpr (G < 32 || Gr::kWhole) {
        // whole block pairs: lanes at the first column of a group write
        if (n32 % G == 0 && (G < 32 || hi == 0)) {
#pragma unroll
          for (int k = 0; k < R::NR; ++k) {
            const int i = (rb + k * R::EG) / G, j = (cb + n32) / G;
            if (i < nb && j <= i) {
              float tv = -INFINITY;
              if (mx[k] != -INFINITY) {
                const int ns = interior ? G * G : pair_samples(i, j, G, ng, S, len);
                tv = (mx[k] + __log2f(sm[k] / float(ns))) * kLn2;
              }
              orow[int64_t(i) * (i + 1) / 2 + j] = tv;
            }
          }
        }
      } else {
        // blocks of more than 32 groups: partial results of this 32 x 32
        // product, combined below
        if (lane == 0) {
          f32x2 *part = reinterpret_cast<f32x2 *>(lds);
          part[(2 * w + m) * 4 + n] = f32x2{mx[0], sm[0]};
        }
      }
    }
  };
  switch (gpb) {
    case 1: finish(GroupTag<1, true>{}); return;
    case 2: finish(GroupTag<2, true>{}); return;
    case 4: finish(GroupTag<4, true>{}); return;
    case 8: finish(GroupTag<8, true>{}); return;
    case 16: finish(GroupTag<16, true>{}); return;
    case 32: finish(GroupTag<32, true>{}); return;
    default: break;
  }
  // gpb = 64 or 128: 32 x 32 partials through LDS (the staging area is free
  // once every wavefront has passed this barrier)
  __syncthreads();
  finish(GroupTag<32, false>{});
  __syncthreads();
  const f32x2 *part = reinterpret_cast<const f32x2 *>(lds);
  const int pr = kTM / gpb, pc = kTN / gpb, per = gpb / 32;
  if (tid < pr * pc) {
    const int ib = tid / pc, jb = tid - ib * pc;
    const int i = r0 / gpb + ib, j = c0 / gpb + jb;
    if (i < nb && j <= i) {
      float mx = -INFINITY;
      for (int x = 0; x < per; ++x)
        for (int y = 0; y < per; ++y) mx = fmaxf(mx, part[(ib * per + x) * 4 + jb * per + y][0]);
      float t = -INFINITY;
      if (mx != -INFINITY) {
        float sum = 0.f;
        for (int x = 0; x < per; ++x)
          for (int y = 0; y < per; ++y) {
            const f32x2 pv = part[(ib * per + x) * 4 + jb * per + y];
            if (pv[0] != -INFINITY) sum += pv[1] * exp2f(pv[0] - mx);
          }
        t = (mx + __log2f(sum / float(pair_samples(i, j, gpb, ng, S, len)))) * kLn2;
      }
      orow[int64_t(i) * (i + 1) / 2 + j] = t;
    }
  }
}

// ---- f32 inputs: one workgroup per (query head, query block) row, each
// thread forming whole samples from f32 dot products (the f32 workloads are
// small; no matrix cores), block pairs reduced with an online max / sum
// merged across the workgroup.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mn));
  m = mn;
}

template <int D>
__global__ __launch_bounds__(256) void antidiag_f32_kernel(AdArgs a) {
  __shared__ float red_m[4], red_s[4];
  __shared__ int red_n[4];
  const int nbT = a.pd.cu_blocks[a.num_seqs];
  const int h = int(blockIdx.x / unsigned(nbT)), b = int(blockIdx.x - unsigned(h) * unsigned(nbT));
  const int s = a.pd.blk_seq[b];
  const int i = b - a.pd.cu_blocks[s];
  const int S = a.stride, gpb = a.block / S;
  const int t0 = a.pd.cu_seqlens[s];
  const int len = a.pd.cu_seqlens[s + 1] - t0;
  const int ng = (len + S - 1) / S;
  const int hk = h / a.G;
  const float *q = reinterpret_cast<const float *>(a.q) + (int64_t(t0) * a.Hq + h) * D;
  const float *k = reinterpret_cast<const float *>(a.k) + (int64_t(t0) * a.Hkv + hk) * D;
  const int64_t qs = int64_t(a.Hq) * D, ks = int64_t(a.Hkv) * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float *orow = a.out + int64_t(h) * a.per_head + a.pd.tri[s] + int64_t(i) * (i + 1) / 2;
  for (int j = 0; j <= i; ++j) {
    float m = -INFINITY, sm = 0.f;
    int ns = 0;
    for (int x = tid; x < gpb * gpb; x += 256) {
      const int r = i * gpb + x / gpb, c = j * gpb + x % gpb;
      if (r >= ng || c > r) continue;
      float acc = 0.f;
      int cnt = 0;
      for (int u = 0; u < S; ++u) {
        const int qp = r * S + S - 1 - u, kp = c * S + u;
        if (qp >= len || kp >= len || kp > qp) continue;
        const float *qv = q + qp * qs, *kv = k + kp * ks;
        for (int e = 0; e < D; ++e) acc = fmaf(qv[e], kv[e], acc);
        ++cnt;
      }
      if (cnt == 0) continue;
      lse_merge(m, sm, acc * (a.scale / float(cnt)), 1.f);
      ++ns;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
      ns += __shfl_xor(ns, o);
      lse_merge(m, sm, m2, s2);
    }
    if (lane == 0) { red_m[w] = m; red_s[w] = sm; red_n[w] = ns; }
    __syncthreads();
    if (tid == 0) {
      float mt = red_m[0], st = red_s[0];
      int nt = red_n[0];
      for (int x = 1; x < 4; ++x) { lse_merge(mt, st, red_m[x], red_s[x]); nt += red_n[x]; }
      orow[j] = nt > 0 ? mt + __logf(st / float(nt)) : -INFINITY;
    }
    __syncthreads();
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
  // per sequence ntr (ntr + 1) pairs at most, ntr = row tiles of 256 groups
  const int64_t gpb = in.block / stride;
  const int64_t ntr_max = (int64_t(in.max_seq_blocks) * gpb + kTM - 1) / kTM;
  const int64_t ntr_sum = (in.total_blocks * gpb + kTM - 1) / kTM + in.num_seqs;
  return (ntr_max + 1) * ntr_sum + 1;
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
  a.units_per_head = in.dtype == STEM_BF16 ? static_cast<int32_t>(antidiag_units_per_head(in, stride)) : 0;
  a.per_head = in.score_elems_per_head;
  a.scale = 1.0f / sqrtf(float(in.head_dim));
  if (in.dtype == STEM_F32) {
    // one workgroup per (head, block) row; Hq * nbT < 2^31 (plan limit)
    const dim3 grid(static_cast<unsigned>(in.total_blocks * in.num_q_heads));
    if (in.head_dim == 128)
      hipLaunchKernelGGL(antidiag_f32_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(antidiag_f32_kernel<64>, grid, dim3(256), 0, st, a);
  } else {
    const int64_t units = int64_t(in.num_q_heads) * a.units_per_head;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    if (in.head_dim == 128)
      hipLaunchKernelGGL(antidiag_kernel<128>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(antidiag_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  }
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
