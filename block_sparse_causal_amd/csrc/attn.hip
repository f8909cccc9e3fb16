// Block-sparse causal attention over the kept blocks (the method's final
// stage: exact softmax and aggregation over the selected blocks only;
// gist.science/es "Implementacion" step 3, gist.science/fr 2.C step 3).
//
// Work unit: one (query head h, query block i) row = B query tokens, one
// workgroup of B/32 wavefronts, each wavefront owning 32 query tokens.  At
// B = 64 (bf16 inputs, lists of at most 32 blocks) a work unit is a pair of
// query heads of one KV head (with an odd number of query heads per KV head
// the last one runs as single-head units in a second launch):
// four wavefronts, two per head, stream the union of the two heads' lists
// through one set of stage buffers, which lets three workgroups (three
// wavefronts per SIMD) share a CU as at B = 128.  The
// workgroup walks the row's kept key blocks in ascending order; each key
// block (B tokens of K and V) is staged in LDS once and consumed by all
// wavefronts.  Per wavefront and key block:
//   S^T = K Q^T   on the matrix cores (keys x queries, so that every lane
//                 holds values of a single query token: the online-softmax
//                 statistics never leave the lane pair l, l^32)
//   online softmax in f32 (exp2 with the 1/sqrt(d) scale folded in)
//   O^T += V^T P^T on the matrix cores, P taken straight from the S^T
//                 accumulators (the contraction order over keys is permuted
//                 identically in both operands, so no data moves between
//                 lanes).
// bf16 inputs use v_mfma_f32_32x32x16_bf16 with f32 accumulation; f32 inputs
// use v_mfma_f32_32x32x2_f32.  The token-level causal mask is applied only
// when the key block is the diagonal block; the missing rows of a final
// partial block repeat its last valid row in LDS and are masked.
//
// Grid order: workgroups are issued round-robin over the 8 XCDs of the chip,
// each with its own L2.  Work item L is placed so that contiguous ranges of
// L land on one XCD, and L enumerates (KV head, query block by decreasing
// work, query head within the group): the query heads sharing a KV head and
// the neighbouring rows (which keep mostly the same key blocks) then hit
// the same L2.  With fewer than 8 KV heads (a divisor of 8), each KV head is
// shared by 8 / Hkv XCDs that take its query blocks' ranks in turn, so that
// every XCD gets the same mix of long and short rows (contiguous halves of
// the work order would give one XCD the long rows and the other the short).
#include <type_traits>

#include "stem_device.h"

namespace stem {
namespace {

constexpr int kXcds = 8;
constexpr float kRescaleBound = 256.f;  // lazy rescale: largest per-lane chunk weight sum (2^8)

struct AttnArgs {
  const void *q, *k, *v;
  const int32_t *idx, *count;
  void *out;
  float *lse;
  PlanDev pd;
  int32_t Hq, Hkv, nbT, kmax;
  int64_t T;
  int32_t n_items;     // Hq * nbT
  int32_t per_xcd;     // work items per XCD
  int32_t split;       // XCDs sharing one KV head (1: contiguous ranges)
  int32_t hpi;         // query heads per work item (1, or 2 for head pairs)
  int32_t hoff, hgrp;  // query heads hoff .. hoff + hgrp - 1 of each KV head's group
  float scale;         // 1 / sqrt(d)
  float scale_log2;    // log2(e) / sqrt(d)
};

struct Row {
  int h, g, b, i, nkeep;
  int64_t seq_start;
  int seq_len;
  const int32_t *list;
  int h2, nkeep2;          // head pairs: the second head (-1: none) and its list
  const int32_t *list2;
};

__device__ __forceinline__ bool decode_item(const AttnArgs &a, Row &r) {
  const int x = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int PG = a.hgrp / a.hpi;            // work items per (KV head, row)
  int p;
  if (a.split > 1) {
    // XCD k: KV head k / split, ranks congruent to k % split, in order
    const int k = x % kXcds, j = x / kXcds;
    const int rank = k % a.split + a.split * (j / PG);
    if (rank >= a.nbT) return false;
    r.g = k / a.split;
    r.b = a.pd.order[rank];
    p = j % PG;
  } else {
    const int L = (x % kXcds) * a.per_xcd + x / kXcds;
    if (L >= a.n_items) return false;
    const int per_g = PG * a.nbT;
    r.g = L / per_g;
    const int rem = L % per_g;
    r.b = a.pd.order[rem / PG];
    p = rem % PG;
  }
  r.h = r.g * G + a.hoff + a.hpi * p;
  r.h2 = a.hpi == 2 ? r.h + 1 : -1;
  const int s = a.pd.blk_seq[r.b];
  r.i = r.b - a.pd.cu_blocks[s];
  r.seq_start = a.pd.cu_seqlens[s];
  r.seq_len = a.pd.cu_seqlens[s + 1] - a.pd.cu_seqlens[s];
  const int64_t rowid = int64_t(r.h) * a.nbT + r.b;
  r.nkeep = min(a.count[rowid], a.kmax);
  r.list = a.idx + rowid * a.kmax;
  r.nkeep2 = 0;
  r.list2 = r.list;
  if (r.h2 >= 0) {
    const int64_t rowid2 = int64_t(r.h2) * a.nbT + r.b;
    r.nkeep2 = min(a.count[rowid2], a.kmax);
    r.list2 = a.idx + rowid2 * a.kmax;
  }
  return true;
}

// ---------------------------------------------------------------------------
// bf16 inputs
//
// Workgroup = B/32 wavefronts for one (head, query block) row, wavefront w
// owning queries 32w .. 32w+31.  Each kept key block is streamed through
// LDS in stages of 32 keys, filled by direct global->LDS DMA
// (global_load_lds_dwordx4, no registers) ahead of the compute.  At
// B = 128 three stage buffers (48 KiB at d = 128) keep the DMA two stages
// ahead, and with at most 168 VGPRs per wavefront three workgroups share a
// CU (three wavefronts per SIMD): their barriers are independent, so one's
// softmax, LDS reads and DMA waits overlap the others' MFMAs.  At B = 64
// single-head (two-wavefront) workgroups need more than 170 VGPRs, so two
// wavefronts per SIMD (four workgroups per CU) is the register bound; two
// stage buffers (32 KiB at d = 128) fit four workgroups, three would leave
// LDS for only three.  B = 64 head-pair workgroups (PAIR) have the B = 128
// shape (four wavefronts, two loads per thread and operand, three stage
// buffers) and the same 168-VGPR bound, so three of them share a CU.
//
// K and V stages are row-major with an XOR swizzle of the 16-byte chunks:
// K operand reads (ds_read_b128 of one key row) and V operand reads
// (ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one
// head-dim column, i.e. V^T) are free of bank conflicts.
//
// Selection lists are ascending and end with the diagonal block (the only
// block that needs the token-level causal mask, and the only one that can
// be a partial block): the unmasked step runs for the stages of every other
// block, and the masked step for a short tail holding the last block's
// stages.

__device__ __forceinline__ int swz_k(int row, int nch) { return (row / (16 / nch)) % nch; }
__device__ __forceinline__ int swz_v(int row, int nch) {
  return nch == 16 ? 4 * (row % 4) : 4 * ((row / 2) % 2);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kStageKeys = 32;   // keys per LDS stage

// Stage buffers: 3 (DMA two stages ahead, 48 KiB at d = 128) for B = 128,
// where three 4-wavefront workgroups then share a CU; 2 for B = 64, where
// registers allow four 2-wavefront workgroups per CU and three buffers
// would leave LDS for only three.
template <int B>
constexpr int stage_bufs() { return B == 128 ? 3 : 2; }

// Lane id (0..63) computed by v_mbcnt in inline assembly: a value the compiler
// cannot hoist or reuse from an earlier computation.
__device__ __forceinline__ int opaque_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// f(std::integral_constant<int, I>()) for I = FIRST .. LAST - 1
template <int FIRST, int LAST, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (FIRST < LAST) {
    f(std::integral_constant<int, FIRST>{});
    static_for<FIRST + 1, LAST>(f);
  }
}

template <int B, int D, int QW, bool OUT_BF16, bool PAIR>
__global__ __launch_bounds__((PAIR ? 2 : 1) * B / QW * 64)
__attribute__((amdgpu_waves_per_eu(QW == 32 ? (B == 128 || PAIR ? 3 : 2) : 1, QW == 32 ? (B == 128 || PAIR ? 3 : 2) : 1)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int QT = QW / 32;          // 32-query tiles per wavefront
  // head pairs: two query heads of one KV head share a workgroup, wavefronts
  // 0 .. B/QW - 1 on the first head and the rest on the second; the K/V
  // stages stream the union of the two heads' lists, and a wavefront skips
  // the blocks its head does not keep
  constexpr int NW = (PAIR ? 2 : 1) * B / QW;   // wavefronts
  constexpr int NT = NW * 64;          // threads
  constexpr int SK = kStageKeys;       // keys per stage
  constexpr int NBUF = PAIR ? 3 : stage_bufs<B>(); // stage buffers
  constexpr int NPB = B / SK;          // stages per key block
  constexpr int KT = SK / 32;          // 32-key MFMA tiles per stage
  constexpr int DT = D / 32;           // 32-dim output tiles
  constexpr int DC = D / 16;           // 16-dim contraction chunks for S
  constexpr int NCH = D / 8;           // 16-byte chunks per row
  constexpr int ROWB = D * 2;          // bytes per K/V row
  constexpr int TILEB = SK * ROWB;     // bytes per K or V stage
  constexpr int LOADS = TILEB / 16 / NT;
  static_assert(LOADS * 16 * NT == TILEB, "a stage must split into 16-byte loads");
  static_assert(NT % NCH == 0, "a load step covers whole rows");
  // [K buf 0..NBUF-1][V buf 0..NBUF-1]
  __shared__ __attribute__((aligned(16))) char lds[2 * NBUF * TILEB];

  Row r;
  if (!decode_item(a, r)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hi = lane >> 5;
  const int Hq = a.Hq, Hkv = a.Hkv;
  const uint32_t lds_base = lds_addr_of(lds);
  constexpr int WPH = B / QW;                    // wavefronts per head
  const int wq = PAIR ? w % WPH : w;             // query slot of this wavefront
  const int wh = PAIR ? w / WPH : 0;             // which head of the item
  const int myh = wh == 0 ? r.h : r.h2;          // -1: no second head

  // Q fragments of this wavefront's QW queries (B operand of S^T = K Q^T):
  // tile qt holds queries w*QW + 32qt + n
  int qloc[QT];
  bf16x8 qf[QT][DC];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    qloc[qt] = r.i * B + wq * QW + qt * 32 + n;
    const bool qvalid = qloc[qt] < r.seq_len && myh >= 0;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((r.seq_start + (qvalid ? qloc[qt] : 0)) * Hq + max(myh, 0)) * int64_t(D) + hi * 8;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      u32x4 x = qvalid ? *reinterpret_cast<const u32x4 *>(qp + c * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[qt][c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  wait_vm();  // Q resident before the loop: no wait on it inside

  f32x16 oacc[QT][DT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x16{};
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
  }
  const float cl2 = a.scale_log2;

  // Stage keys [key0, key0 + SK) of block j into buffer `buf` (asynchronous).
  // Thread tid moves 16-byte chunk slot q = it*NT + tid: row q / NCH,
  // physical chunk q % NCH, which holds logical chunk (q % NCH) ^ swizzle.
  // The byte offsets inside a stage do not depend on the block and are
  // computed once.  Rows past the end of a final partial block read its last
  // valid row instead (those keys are masked).
  constexpr int ROWSTEP = NT / NCH;
  const int row0 = tid / NCH;
  const int pc0 = tid % NCH;
  const uint32_t rowbytes = static_cast<uint32_t>(Hkv) * D * 2;   // between token rows
  // Load step it moves rows row0 + it*ROWSTEP: the row advance goes into the
  // scalar base, and the swizzle of those rows equals that of row0 except
  // for the K chunk bit 3 when ROWSTEP is an odd multiple of 8 (D = 128,
  // B = 64), so two lane offsets cover every step.
  const uint32_t koff0 = row0 * rowbytes + (pc0 ^ swz_k(row0, NCH)) * 16;
  const uint32_t voff0 = row0 * rowbytes + (pc0 ^ swz_v(row0, NCH)) * 16;
  static_assert(NCH != 16 || ROWSTEP % 8 == 0, "K swizzle period");
  static_assert(NCH != 8 || ROWSTEP % 16 == 0, "K swizzle period");
  auto koff_of = [&](int it) {
    return (NCH == 16 && ((it * ROWSTEP) & 8)) ? (koff0 ^ 128u) : koff0;
  };
  // K and V rows of this KV head at the sequence's first token
  const int64_t eseq = (r.seq_start * Hkv + r.g) * int64_t(D);
  const char *kseq = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + eseq);
  const char *vseq = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + eseq);
  // Stage `part` of block j into buffer `buf`.  Every call issues exactly
  // 2 LOADS DMA instructions (the stage waits count on it): a stage that lies
  // past the end of the sequence (keys all masked, buffer not read) loads
  // the sequence's first row instead.
  auto issue = [&](int j, int part, int buf) {
    int first = j * B + part * SK;                       // first key (local position)
    int nrows = min(SK, r.seq_len - first);               // may be <= 0 past the end
    if (nrows <= 0) { first = 0; nrows = 1; }
    const size_t off = size_t(static_cast<uint32_t>(first)) * rowbytes;
    const char *kblk = kseq + off;
    const char *vblk = vseq + off;
    const uint32_t l0 = lds_base + w * 64 * 16;  // this wavefront's 1 KiB slab
    if (nrows == SK) {
      if constexpr (LOADS % 2 == 0) {
        // two load steps (K and V each) per asm block
#pragma unroll
        for (int it = 0; it < LOADS; it += 2) {
          const char *kb = kblk + size_t(it) * ROWSTEP * rowbytes;
          const char *vb = vblk + size_t(it) * ROWSTEP * rowbytes;
          const size_t step = size_t(ROWSTEP) * rowbytes;
          dma16x4(kb, koff_of(it), l0 + it * NT * 16 + buf * TILEB,
                  vb, voff0, l0 + it * NT * 16 + (NBUF + buf) * TILEB,
                  kb + step, koff_of(it + 1), l0 + (it + 1) * NT * 16 + buf * TILEB,
                  vb + step, voff0, l0 + (it + 1) * NT * 16 + (NBUF + buf) * TILEB);
        }
      } else {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
          const char *kb = kblk + size_t(it) * ROWSTEP * rowbytes;
          const char *vb = vblk + size_t(it) * ROWSTEP * rowbytes;
          dma16(kb, koff_of(it), l0 + it * NT * 16 + buf * TILEB);
          dma16(vb, voff0, l0 + it * NT * 16 + (NBUF + buf) * TILEB);
        }
      }
    } else if (nrows > 0) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int row = row0 + it * ROWSTEP;
        const uint32_t rb = min(row, nrows - 1) * rowbytes;
        dma16(kblk, rb + (pc0 ^ swz_k(row, NCH)) * 16, l0 + it * NT * 16 + buf * TILEB);
        dma16(vblk, rb + (pc0 ^ swz_v(row, NCH)) * 16, l0 + it * NT * 16 + (NBUF + buf) * TILEB);
      }
    }
  };


  // One stage held in buffer `buf`, first key at local position key0: the S
  // tile, the next stages' DMA, the softmax and the PV products.  Three
  // wavefronts of independent workgroups share each SIMD, so one's softmax
  // and LDS reads overlap another's matrix products.  Every K and V^T
  // operand read from LDS feeds QT matrix products.
  auto step = [&](auto mask_tag, int buf, int key0, auto &&after_s) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // The masked step runs only in the short tail; it derives its lane
    // constants from a lane id the compiler cannot keep from before the main
    // loop, so that nothing of the tail's addressing stays live through it.
    const int ln = MASK ? opaque_lane_id() : lane;
    const int n = ln & 31, hi = ln >> 5;
    const int vrow = 4 * hi + ((ln & 15) >> 2);
    const int vd = 16 * ((ln >> 4) & 1) + 4 * (ln & 3);
    const int vsub = ((vd & 7) >> 2) * 8;
    if constexpr (MASK) {
      // nothing visible to this wavefront in this stage (future keys or
      // past the end of the sequence): skip it (wave-uniform)
      if (key0 > r.i * B + wq * QW + QW - 1 || key0 >= r.seq_len) { after_s(); return; }
    }
    const char *Kb = lds + buf * TILEB;
    const char *Vb = lds + (NBUF + buf) * TILEB;
    // S^T = K Q^T for keys key0 + 32u .. +31
    f32x16 sacc[KT][QT];
#pragma unroll
    for (int u = 0; u < KT; ++u) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sacc[u][qt] = f32x16{};
      const int kr = u * 32 + n;
      const char *krow = Kb + kr * ROWB;
      const int ksw = swz_k(kr, NCH);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 kx = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(krow + (((2 * c + hi) ^ ksw) * 16)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[u][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qf[qt][c], sacc[u][qt], 0, 0, 0);
      }
    }
    after_s();  // the next stage's DMA goes out while the matrix cores work
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      if constexpr (MASK) {
        // key position <= query position, and inside the sequence
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int lim = min(r.i * B + wq * QW + qt * 32 + n, r.seq_len - 1) - (key0 + u * 32 + 4 * hi);
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (8 * (q >> 2) + (q & 3) > lim) sacc[u][qt][q] = -INFINITY;
        }
      }
      // V^T fragments of this chunk (contraction step hc covers keys
      // kb0 + 4hi + {0..3} and kb0 + 8 + 4hi + {0..3}, kb0 = 32u + 16hc;
      // ds_read_b64_tr_b16 gives lane (n, hi) V[kb0 + 4hi + e][dt*32 + n])
      auto readv = [&](int hc, bf16x8 (&vf)[DT]) {
        const int r0 = u * 32 + 16 * hc + vrow;
        const char *p0 = Vb + r0 * ROWB + vsub;
        const char *p1 = p0 + 8 * ROWB;
        const int sw0 = swz_v(r0, NCH), sw1 = swz_v(r0 + 8, NCH);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int ch = (dt * 32 + vd) >> 3;
          const v4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0 + ((ch ^ sw0) * 16)));
          const v4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p1 + ((ch ^ sw1) * 16)));
          vf[dt] = __builtin_bit_cast(bf16x8, (v8i16){v0[0], v0[1], v0[2], v0[3],
                                                      v1[0], v1[1], v1[2], v1[3]});
        }
      };
      bf16x8 vf0[DT], vf1[DT];
      readv(0, vf0);
      // Online softmax against a lazily moved reference maximum mrun: the
      // weights are exp2((s - mrun) * c); the reference is raised only when
      // some weight of the chunk would exceed 2^8 (their per-lane sum is then
      // above 2^8 as well).  A row that has seen no key yet has mrun = -inf,
      // which makes its weights +inf or NaN and sends it down the same rare
      // path.  The row sum is taken over the bf16-rounded weights, the ones
      // that multiply V.
      bf16x8 pf[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float ps;
        auto weights = [&](float msc) {
#pragma unroll
          for (int hc = 0; hc < 2; ++hc) {
            f32x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[u][qt][8 * hc + e], cl2, -msc));
            pf[qt][hc] = __builtin_convertvector(pv, bf16x8);
          }
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          float sum = 0.f;
#pragma unroll
          for (int hc = 0; hc < 2; ++hc)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sum = __builtin_amdgcn_fdot2_f32_bf16(
                  bf16x2{pf[qt][hc][2 * e], pf[qt][hc][2 * e + 1]}, one, sum, false);
          ps = sum;
        };
        weights(mrun[qt] * cl2);
        if (__ballot(!(ps <= kRescaleBound))) {
          float bm = -INFINITY;
#pragma unroll
          for (int q = 0; q < 16; ++q) bm = fmaxf(bm, sacc[u][qt][q]);
          // the lane id comes from inline assembly so that the common path
          // keeps no copy of it
          bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_ds_bpermute(
                             (opaque_lane_id() ^ 32) << 2, __float_as_int(bm))));
          const float mnew = fmaxf(mrun[qt], bm);
          const float alpha =
              mnew == mrun[qt] ? 1.f : __builtin_amdgcn_exp2f((mrun[qt] - mnew) * cl2);
          lrun[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= alpha;
          mrun[qt] = mnew;
          // rows with every key so far masked keep mrun = -inf and weight 0
          weights(mnew == -INFINITY ? INFINITY : mnew * cl2);
        }
        lrun[qt] += ps;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf0[dt], pf[qt][0], oacc[qt][dt], 0, 0, 0);
      readv(1, vf1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf1[dt], pf[qt][1], oacc[qt][dt], 0, 0, 0);
    }
  };

  // Kept block numbers, 64 at a time in one register (lane e holds entry
  // chunk + e); entries outside [0, i] are clamped so that no access leaves
  // the sequence.
  // head pairs: the union of the two ascending lists (at most 32 entries
  // each), every entry tagged with the heads that keep it (bit 28: first,
  // bit 29: second), built by each wavefront in its own LDS slot of the last
  // stage buffer (whose first DMA goes out after the first stage's barrier)
  constexpr uint32_t kBlockMask = (1u << 28) - 1;
  int nkeep = r.nkeep;
  int chunk = 0;
  int listv = lane < nkeep ? min(max(r.list[lane], 0), r.i) : 0;
  if constexpr (PAIR) {
    const int n0 = r.nkeep, n1 = r.nkeep2;
    const int x0 = lane < n0 ? min(max(r.list[lane], 0), r.i) : 0;
    const int x1 = lane < n1 ? min(max(r.list2[lane], 0), r.i) : 0;
    // second-list entries: also in the first list? how many first-list
    // entries are smaller?
    bool dup1 = false;
    int lt0 = 0;
    for (int j = 0; j < n0; ++j) {
      const int y = __builtin_amdgcn_readlane(x0, j);
      dup1 |= y == x1;
      lt0 += y < x1;
    }
    const uint64_t dupm = __ballot(lane < n1 && dup1);
    // first-list entries: how many second-list-only entries are smaller,
    // and is it kept by the second head too?
    bool in1 = false;
    int lt1 = 0;
    for (int j = 0; j < n1; ++j) {
      const int y = __builtin_amdgcn_readlane(x1, j);
      in1 |= y == x0;
      lt1 += (y < x0) && !((dupm >> j) & 1);
    }
    int32_t *slot = reinterpret_cast<int32_t *>(lds + (NBUF - 1) * TILEB) + w * 64;
    if (lane < n0) slot[lane + lt1] = x0 | (1 << 28) | (in1 ? (1 << 29) : 0);
    const int dups_below = __popcll(dupm & ((uint64_t(1) << lane) - 1));
    if (lane < n1 && !dup1) slot[lt0 + lane - dups_below] = x1 | (1 << 29);
    nkeep = n0 + n1 - __popcll(dupm);
    wait_lgkm();
    // with ascending lists every slot below nkeep is written once; lists out
    // of order can leave slots unwritten, so the block part is clamped again
    // (no access outside the sequence, whatever the slot holds)
    const uint32_t e = uint32_t(slot[lane]);
    listv = lane < nkeep ? int((e & ~kBlockMask) | min(e & kBlockMask, uint32_t(r.i))) : 0;
  }
  // entry t of the stream (packed with the head tags for head pairs)
  auto entry = [&](int t) {
    if constexpr (PAIR) {
      return __builtin_amdgcn_readlane(listv, t);
    } else {
      if (t >= chunk + 64) {
        chunk += 64;
        listv = chunk + lane < nkeep ? min(max(r.list[chunk + lane], 0), r.i) : 0;
      }
      return __builtin_amdgcn_readlane(listv, t - chunk);
    }
  };
  const int mybit = 28 + wh;

  // Stage s covers keys [p*SK, p*SK + SK) of entry s / NPB (p = s % NPB) and
  // lives in buffer s % NBUF; its DMA is issued NBUF - 1 stages ahead.
  if (nkeep > 0) {
    const int nst = nkeep * NPB;
    int jq[NBUF];   // block of the stages s .. s + NBUF - 1
#pragma unroll
    for (int e = 0; e < NBUF; ++e) jq[e] = 0;
#pragma unroll
    for (int e = 0; e < NBUF - 1; ++e)
      if (e < nst) { jq[e] = entry(e / NPB); issue(jq[e] & kBlockMask, e % NPB, e); }
    auto body = [&](int st, auto btag, auto mtag) {
      constexpr int buf = decltype(btag)::value;
      // this stage's DMA has landed once at most the later stages' loads
      // (2 LOADS each, always) are in flight
      if (NBUF > 2 && st + NBUF - 2 < nst) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LOADS * (NBUF - 2)));
      else wait_vm();
      __syncthreads();
      const int key0 = int(jq[0] & kBlockMask) * B + (st % NPB) * SK;
      const int nxt = st + NBUF - 1;
      auto after = [&] {
        if (nxt < nst) {
          jq[NBUF - 1] = entry(nxt / NPB);
          issue(jq[NBUF - 1] & kBlockMask, nxt % NPB, (buf + NBUF - 1) % NBUF);
        }
      };
      // head pairs: a block the wavefront's head does not keep only moves
      // the ring on
      if constexpr (PAIR) {
        // head pairs: the next stage's DMA first, then this stage's products
        // only if this wavefront's head keeps the block
        after();
        if ((jq[0] >> mybit) & 1) step(mtag, buf, key0, [] {});
      } else {
        step(mtag, buf, key0, after);
      }
#pragma unroll
      for (int e = 0; e + 1 < NBUF; ++e) jq[e] = jq[e + 1];
    };
    // The loop is unrolled over the buffers so that every buffer offset is
    // a constant.  Stages before the last key block need no mask; the last
    // block's stages (and up to NBUF - 1 before them) run the masked step.
    const int nu = nst - NPB;
    int st = 0;
    for (; st + NBUF <= nu; st += NBUF)
      static_for<0, NBUF>([&](auto b) { body(st + decltype(b)::value, b, std::false_type{}); });
    for (; st < nst; st += NBUF)
      static_for<0, NBUF>([&](auto b) {
        if (st + decltype(b)::value < nst) body(st + decltype(b)::value, b, std::true_type{});
      });
  }

  // ---- finalize: O^T lane layout = query n, dims dt*32 + 8(q/4) + 4hi + q%4
  // bf16 output: each wavefront's 32 x D tile goes through LDS (rows
  // XOR-swizzled by 16-byte chunk), and every store then writes 16 bytes
  // per lane, one whole 2D-byte row per D/8 lanes.
  if constexpr (OUT_BF16 && QT == 1 && 32 * D * 2 * NW <= 2 * NBUF * TILEB) {
    __syncthreads();   // every wavefront is done with the stage buffers
    // lane constants again from an opaque lane id: none of them has to be
    // kept through the main loop
    const int lane = opaque_lane_id();
    const int n = lane & 31, hi = lane >> 5;
    char *ot = lds + w * (32 * D * 2);
    if (myh < 0) return;
    const float ltot = lrun[0] + __shfl_xor(lrun[0], 32);
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * hi;
        const uint32_t lo = pack_bf16x2(oacc[0][dt][4 * rg] * inv, oacc[0][dt][4 * rg + 1] * inv);
        const uint32_t up = pack_bf16x2(oacc[0][dt][4 * rg + 2] * inv, oacc[0][dt][4 * rg + 3] * inv);
        const int phys = ((d0 >> 3) ^ (n % NCH));
        *reinterpret_cast<uint2 *>(ot + n * (D * 2) + phys * 16 + (d0 & 4) * 2) = uint2{lo, up};
      }
    constexpr int ROWS_PER_STORE = 64 / NCH;      // 4 (d = 128) or 8 (d = 64)
#pragma unroll
    for (int it = 0; it < 32 / ROWS_PER_STORE; ++it) {
      const int row = it * ROWS_PER_STORE + lane / NCH;
      const int c = lane % NCH;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(ot + row * (D * 2) + ((c ^ (row % NCH)) * 16));
      const int qpos = r.i * B + wq * QW + row;
      if (qpos < r.seq_len)
        // non-temporal: O is not read again here, and keeping it out of L2
        // leaves room for the K/V blocks that neighbouring rows reuse
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.out) +
                                   ((r.seq_start + qpos) * Hq + myh) * int64_t(D) + c * 8));
    }
    const int q0 = r.i * B + wq * QW + n;
    if (a.lse && hi == 0 && q0 < r.seq_len)
      a.lse[int64_t(myh) * a.T + r.seq_start + q0] = mrun[0] * a.scale + logf(ltot);
    return;
  }
  if (myh < 0) return;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float ltot = lrun[qt] + __shfl_xor(lrun[qt], 32);
    if (qloc[qt] >= r.seq_len) continue;
    const float inv = 1.0f / ltot;
    const int64_t orow = ((r.seq_start + qloc[qt]) * Hq + myh) * int64_t(D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * hi;
        const float o0 = oacc[qt][dt][4 * rg] * inv, o1 = oacc[qt][dt][4 * rg + 1] * inv;
        const float o2 = oacc[qt][dt][4 * rg + 2] * inv, o3 = oacc[qt][dt][4 * rg + 3] * inv;
        if (OUT_BF16) {
          uint32_t *op = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.out) + orow + d0);
          op[0] = pack_bf16x2(o0, o1);
          op[1] = pack_bf16x2(o2, o3);
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + orow + d0) = f32x4{o0, o1, o2, o3};
        }
      }
    if (a.lse && hi == 0)
      a.lse[int64_t(myh) * a.T + r.seq_start + qloc[qt]] = mrun[qt] * a.scale + logf(ltot);
  }
}

// ---------------------------------------------------------------------------
// f32 inputs (f32 matrix cores; K and V stay row-major in LDS)

template <int B, int D, bool OUT_BF16>
__global__ __launch_bounds__(B * 2) void attn_f32_kernel(AttnArgs a) {
  constexpr int NT = (B / 32) * 64;
  constexpr int LD = D + 1;            // row stride in LDS (floats)
  constexpr int KT = B / 32;
  constexpr int DT = D / 32;
  constexpr int HALF = D / 2;
  __shared__ float Ks[B * LD];
  __shared__ float Vs[B * LD];

  Row r;
  if (!decode_item(a, r)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hi = lane >> 5;
  const int Hq = a.Hq, Hkv = a.Hkv;

  const int qloc = r.i * B + w * 32 + n;
  const bool qvalid = qloc < r.seq_len;
  // contraction step c <-> dim hi*HALF + c
  float qv[HALF];
  {
    const float *qp = static_cast<const float *>(a.q) +
                      ((r.seq_start + (qvalid ? qloc : 0)) * Hq + r.h) * int64_t(D) + hi * HALF;
#pragma unroll
    for (int c = 0; c < HALF; c += 4) {
      f32x4 x = qvalid ? *reinterpret_cast<const f32x4 *>(qp + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      qv[c] = x[0]; qv[c + 1] = x[1]; qv[c + 2] = x[2]; qv[c + 3] = x[3];
    }
  }
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float mrun = -INFINITY, lrun = 0.f;
  const float cl2 = a.scale_log2;
  const float *kbase = static_cast<const float *>(a.k);
  const float *vbase = static_cast<const float *>(a.v);

  for (int t = 0; t < r.nkeep; ++t) {
    const int j = __builtin_amdgcn_readfirstlane(r.list[t]);
    if (j < 0 || j > r.i) continue;
    const int key0 = j * B;
    const int nvalid = min(B, r.seq_len - key0);
    const int64_t tok0 = r.seq_start + key0;
    if (t > 0) __syncthreads();
    for (int c = tid; c < B * (D / 4); c += NT) {
      const int key = c / (D / 4);
      const int d4 = (c % (D / 4)) * 4;
      f32x4 xk = f32x4{0.f, 0.f, 0.f, 0.f}, xv = f32x4{0.f, 0.f, 0.f, 0.f};
      if (key < nvalid) {
        const int64_t off = ((tok0 + key) * Hkv + r.g) * int64_t(D) + d4;
        xk = *reinterpret_cast<const f32x4 *>(kbase + off);
        xv = *reinterpret_cast<const f32x4 *>(vbase + off);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Ks[key * LD + d4 + e] = xk[e];
        Vs[key * LD + d4 + e] = xv[e];
      }
    }
    __syncthreads();

    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sacc[kt] = f32x16{};
      const float *kp = &Ks[(kt * 32 + n) * LD + hi * HALF];
#pragma unroll
      for (int c = 0; c < HALF; ++c)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[c], qv[c], sacc[kt], 0, 0, 0);
    }
    if (j == r.i || nvalid < B) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int kk = kt * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
          if (key0 + kk > qloc || kk >= nvalid) sacc[kt][q] = -INFINITY;
        }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) bm = fmaxf(bm, sacc[kt][q]);
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mnew = fmaxf(mrun, bm);
    const float alpha = exp2f((mrun - mnew) * cl2);
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float p = exp2f((sacc[kt][q] - mnew) * cl2);
        sacc[kt][q] = p;
        ps += p;
      }
    lrun = fmaf(lrun, alpha, ps);
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    // O^T += V^T P^T with contraction step q <-> key kt*32 + 8(q/4) + 4hi + q%4
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int key = kt * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * LD + dt * 32 + n], sacc[kt][q],
                                                          oacc[dt], 0, 0, 0);
      }
  }

  const float ltot = lrun + __shfl_xor(lrun, 32);
  if (!qvalid) return;
  const float inv = 1.0f / ltot;
  const int64_t orow = ((r.seq_start + qloc) * Hq + r.h) * int64_t(D);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + 8 * rg + 4 * hi;
      const float o0 = oacc[dt][4 * rg] * inv, o1 = oacc[dt][4 * rg + 1] * inv;
      const float o2 = oacc[dt][4 * rg + 2] * inv, o3 = oacc[dt][4 * rg + 3] * inv;
      if (OUT_BF16) {
        uint32_t *op = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.out) + orow + d0);
        op[0] = pack_bf16x2(o0, o1);
        op[1] = pack_bf16x2(o2, o3);
      } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + orow + d0) = f32x4{o0, o1, o2, o3};
      }
    }
  if (a.lse && hi == 0) a.lse[int64_t(r.h) * a.T + r.seq_start + qloc] = mrun * a.scale + logf(ltot);
}

template <template <int, int, bool> class K>
struct Dummy;

// queries per wavefront of the bf16 kernel
constexpr int kQW = 32;

template <bool BF16IN, int B, int D, bool OB>
hipError_t launch_one(const AttnArgs &a, dim3 grid, hipStream_t st) {
  if constexpr (B == 64 && BF16IN) {
    if (a.hpi == 2) {
      hipLaunchKernelGGL((attn_bf16_kernel<B, D, kQW, OB, true>), grid, dim3(2 * B / kQW * 64), 0, st, a);
      return hipGetLastError();
    }
  }
  if (BF16IN)
    hipLaunchKernelGGL((attn_bf16_kernel<B, D, kQW, OB, false>), grid, dim3(B / kQW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<B, D, OB>), grid, dim3(B * 2), 0, st, a);
  return hipGetLastError();
}

template <bool BF16IN, int B, int D>
hipError_t launch_b_d(const AttnArgs &a, dim3 grid, bool out_bf16, hipStream_t st) {
  return out_bf16 ? launch_one<BF16IN, B, D, true>(a, grid, st)
                  : launch_one<BF16IN, B, D, false>(a, grid, st);
}

template <bool BF16IN>
hipError_t launch_dtype(const AttnArgs &a, dim3 grid, int B, int D, bool out_bf16, hipStream_t st) {
  if (B == 128 && D == 128) return launch_b_d<BF16IN, 128, 128>(a, grid, out_bf16, st);
  if (B == 128 && D == 64) return launch_b_d<BF16IN, 128, 64>(a, grid, out_bf16, st);
  if (B == 64 && D == 128) return launch_b_d<BF16IN, 64, 128>(a, grid, out_bf16, st);
  return launch_b_d<BF16IN, 64, 64>(a, grid, out_bf16, st);
}

}  // namespace

hipError_t launch_attn(const stem_plan_info &in, PlanDev pd, const void *q,
                       const void *k, const void *v, const int32_t *idx,
                       const int32_t *count, void *out, int out_dtype, float *lse,
                       hipStream_t st) {
  const int64_t items = int64_t(in.num_q_heads) * in.total_blocks;
  if (items == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.k = k; a.v = v;
  a.idx = idx; a.count = count;
  a.out = out; a.lse = lse;
  a.pd = pd;
  a.Hq = in.num_q_heads; a.Hkv = in.num_kv_heads;
  a.nbT = static_cast<int32_t>(in.total_blocks);
  a.kmax = in.kmax;
  a.T = in.total_tokens;
  // Head pairs for bf16 inputs at B = 64 with lists of at most 32 entries
  // (their union fits one register).  With an odd number of query heads per
  // KV head, the last head of every group takes a second launch of
  // single-head work items.
  const int G = in.num_q_heads / in.num_kv_heads;
  const bool pairs = in.dtype == STEM_BF16 && in.block == 64 && in.kmax <= 32 && G >= 2;
  auto setup = [&](int hpi, int hoff, int hgrp) {
    a.hpi = hpi; a.hoff = hoff; a.hgrp = hgrp;
    const int PG = hgrp / hpi;
    const int64_t units = int64_t(in.num_kv_heads) * PG * in.total_blocks;
    a.n_items = static_cast<int32_t>(units);
    if (in.num_kv_heads < kXcds && kXcds % in.num_kv_heads == 0) {
      a.split = kXcds / in.num_kv_heads;
      a.per_xcd = static_cast<int32_t>(PG * ((in.total_blocks + a.split - 1) / a.split));
    } else {
      a.split = 1;
      a.per_xcd = static_cast<int32_t>((units + kXcds - 1) / kXcds);
    }
  };
  a.scale = 1.0f / sqrtf(static_cast<float>(in.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  const bool ob = out_dtype == STEM_BF16;
  auto launch = [&]() {
    const dim3 grid(static_cast<unsigned>(int64_t(a.per_xcd) * kXcds));
    if (in.dtype == STEM_BF16) return launch_dtype<true>(a, grid, in.block, in.head_dim, ob, st);
    return launch_dtype<false>(a, grid, in.block, in.head_dim, ob, st);
  };
  if (!pairs) {
    setup(1, 0, G);
    return launch();
  }
  setup(2, 0, G - G % 2);
  hipError_t e = launch();
  if (e != hipSuccess || G % 2 == 0) return e;
  setup(1, G - 1, 1);
  return launch();
}

}  // namespace stem
