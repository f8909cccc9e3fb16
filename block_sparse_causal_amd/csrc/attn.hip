// Block-sparse causal attention over the kept blocks (the method's final
// stage: exact softmax and aggregation over the selected blocks only;
// gist.science/es "Implementacion" step 3, gist.science/fr 2.C step 3).
//
// Work unit: one (query head h, query block i) row = B query tokens, one
// workgroup of B/32 wavefronts, each wavefront owning 32 query tokens.  The
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
// when the key block is the diagonal block; a final partial block is
// zero-filled in LDS and masked.
//
// Grid order: workgroups are issued round-robin over the 8 XCDs of the chip,
// each with its own L2.  Work item L is placed so that contiguous ranges of
// L land on one XCD, and L enumerates (KV head, query block by decreasing
// work, query head within the group): the query heads sharing a KV head and
// the neighbouring rows (which keep mostly the same key blocks) then hit
// the same L2.
#include "stem_device.h"

namespace stem {
namespace {

constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold, log2 units

struct AttnArgs {
  const void *q, *k, *v;
  const int32_t *idx, *count;
  void *out;
  float *lse;
  PlanDev pd;
  int32_t Hq, Hkv, nbT, kmax;
  int64_t T;
  int32_t n_items;     // Hq * nbT
  int32_t per_xcd;     // ceil(n_items / 8)
  float scale;         // 1 / sqrt(d)
  float scale_log2;    // log2(e) / sqrt(d)
};

struct Row {
  int h, g, b, i, nkeep;
  int64_t seq_start;
  int seq_len;
  const int32_t *list;
};

__device__ __forceinline__ bool decode_item(const AttnArgs &a, Row &r) {
  const int x = blockIdx.x;
  const int L = (x % kXcds) * a.per_xcd + x / kXcds;
  if (L >= a.n_items) return false;
  const int G = a.Hq / a.Hkv;
  const int per_g = G * a.nbT;
  r.g = L / per_g;
  const int rem = L % per_g;
  r.b = a.pd.order[rem / G];
  r.h = r.g * G + rem % G;
  const int s = a.pd.blk_seq[r.b];
  r.i = r.b - a.pd.cu_blocks[s];
  r.seq_start = a.pd.cu_seqlens[s];
  r.seq_len = a.pd.cu_seqlens[s + 1] - a.pd.cu_seqlens[s];
  const int64_t rowid = int64_t(r.h) * a.nbT + r.b;
  r.nkeep = min(a.count[rowid], a.kmax);
  r.list = a.idx + rowid * a.kmax;
  return true;
}

// ---------------------------------------------------------------------------
// bf16 inputs

// Two wavefronts per SIMD: while one runs softmax on the vector ALU the other
// keeps the matrix cores busy, and one workgroup's global loads overlap the
// other's compute.  That caps a wavefront at 256 registers.
template <int B, int D, bool OUT_BF16>
__global__ __launch_bounds__(B * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NW = B / 32;           // wavefronts
  constexpr int NT = NW * 64;          // threads
  constexpr int LDK = D + 8;           // K row stride in LDS (bf16 elements)
  constexpr int LDV = B + 2;           // V^T row stride in LDS (bf16 elements)
  constexpr int DT = D / 32;           // 32-dim output tiles
  constexpr int DC = D / 16;           // 16-dim contraction chunks for S
  __shared__ __attribute__((aligned(16))) uint16_t Ks[B * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LDV];

  Row r;
  if (!decode_item(a, r)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hi = lane >> 5;
  const int Hq = a.Hq, Hkv = a.Hkv;

  // this lane's query token (local position) and its Q fragment
  const int qloc = r.i * B + w * 32 + n;
  const bool qvalid = qloc < r.seq_len;
  bf16x8 qf[DC];
  {
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((r.seq_start + (qvalid ? qloc : 0)) * Hq + r.h) * int64_t(D) + hi * 8;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      u32x4 x = qvalid ? *reinterpret_cast<const u32x4 *>(qp + c * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float mrun = -INFINITY, lrun = 0.f;
  const float cl2 = a.scale_log2;

  const uint16_t *kbase = static_cast<const uint16_t *>(a.k);
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v);

  for (int t = 0; t < r.nkeep; ++t) {
    const int j = __builtin_amdgcn_readfirstlane(r.list[t]);
    if (j < 0 || j > r.i) continue;                       // not a causal block of this row
    const int key0 = j * B;                               // local position of first key
    const int nvalid = min(B, r.seq_len - key0);
    const int64_t tok0 = r.seq_start + key0;

    // ---- stage K (row-major) and V (transposed) into LDS
    if (t > 0) __syncthreads();
#pragma unroll
    for (int it = 0; it < (B * D / 8) / NT; ++it) {
      const int c = tid + it * NT;
      const int key = c / (D / 8);
      const int dc = c % (D / 8);
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (key < nvalid)
        x = *reinterpret_cast<const u32x4 *>(kbase + ((tok0 + key) * Hkv + r.g) * int64_t(D) + dc * 8);
      *reinterpret_cast<u32x4 *>(&Ks[key * LDK + dc * 8]) = x;
    }
#pragma unroll
    for (int it = 0; it < (B / 2 * D / 8) / NT; ++it) {
      const int c = tid + it * NT;
      const int kp = c / (D / 8);
      const int dc = c % (D / 8);
      u32x4 x0 = u32x4{0u, 0u, 0u, 0u}, x1 = u32x4{0u, 0u, 0u, 0u};
      if (2 * kp < nvalid)
        x0 = *reinterpret_cast<const u32x4 *>(vbase + ((tok0 + 2 * kp) * Hkv + r.g) * int64_t(D) + dc * 8);
      if (2 * kp + 1 < nvalid)
        x1 = *reinterpret_cast<const u32x4 *>(vbase + ((tok0 + 2 * kp + 1) * Hkv + r.g) * int64_t(D) + dc * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(x1[e], x0[e], 0x05040100u);  // (x0.lo, x1.lo)
        const uint32_t hi2 = __builtin_amdgcn_perm(x1[e], x0[e], 0x07060302u); // (x0.hi, x1.hi)
        *reinterpret_cast<uint32_t *>(&Vt[(dc * 8 + 2 * e) * LDV + 2 * kp]) = lo;
        *reinterpret_cast<uint32_t *>(&Vt[(dc * 8 + 2 * e + 1) * LDV + 2 * kp]) = hi2;
      }
    }
    __syncthreads();

    // ---- the key block in chunks of 64 keys (two 32-key sub-tiles)
#pragma unroll
    for (int kc = 0; kc < B / 64; ++kc) {
      // S^T = K Q^T for this chunk
      f32x16 sacc[2];
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kt = kc * 2 + u;
          const u32x4 kx = *reinterpret_cast<const u32x4 *>(&Ks[(kt * 32 + n) * LDK + c * 16 + hi * 8]);
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qf[c],
                                                            sacc[u], 0, 0, 0);
        }
      }
      // masks: token causality inside the diagonal block, ragged tail
      if (j == r.i || nvalid < B) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int kk = (kc * 2 + u) * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
            if (key0 + kk > qloc || kk >= nvalid) sacc[u][q] = -INFINITY;
          }
      }
      // online softmax (row statistics shared by lanes l and l^32).  The
      // reference maximum only moves when some row's chunk maximum exceeds
      // it by more than 2^8 in the exp2 domain: probabilities then stay
      // <= 256 and the rescale of the output accumulators is skipped for
      // most chunks.
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 16; ++q) bm = fmaxf(bm, sacc[u][q]);
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      if (__ballot((bm - mrun) * cl2 > kRescaleLog2) != 0) {
        const float mnew = fmaxf(mrun, bm);   // finite: every row sees at least one key
        const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * cl2);
        lrun *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        mrun = mnew;
      }
      const float msc = mrun * cl2;
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u][q], cl2, -msc));
          sacc[u][q] = p;
          ps += p;
        }
      lrun += ps;
      // O^T += V^T P^T; contraction step (kt, hc) covers keys
      //   kt*32 + 16hc + {4hi..4hi+3} and kt*32 + 16hc + 8 + {4hi..4hi+3}
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kt = kc * 2 + u;
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
          const f32x8 pv = {sacc[u][8 * hc + 0], sacc[u][8 * hc + 1], sacc[u][8 * hc + 2],
                            sacc[u][8 * hc + 3], sacc[u][8 * hc + 4], sacc[u][8 * hc + 5],
                            sacc[u][8 * hc + 6], sacc[u][8 * hc + 7]};
          const bf16x8 pf = __builtin_convertvector(pv, bf16x8);
          const int kb = kt * 32 + 16 * hc + 4 * hi;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint16_t *vp = &Vt[(dt * 32 + n) * LDV + kb];
            u32x4 vx;
            vx[0] = *reinterpret_cast<const uint32_t *>(vp);
            vx[1] = *reinterpret_cast<const uint32_t *>(vp + 2);
            vx[2] = *reinterpret_cast<const uint32_t *>(vp + 8);
            vx[3] = *reinterpret_cast<const uint32_t *>(vp + 10);
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vx), pf,
                                                               oacc[dt], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- finalize: O^T lane layout = query n, dims dt*32 + 8(q/4) + 4hi + q%4
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

template <bool BF16IN, int B, int D, bool OB>
hipError_t launch_one(const AttnArgs &a, dim3 grid, hipStream_t st) {
  if (BF16IN)
    hipLaunchKernelGGL((attn_bf16_kernel<B, D, OB>), grid, dim3(B * 2), 0, st, a);
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
  a.n_items = static_cast<int32_t>(items);
  a.per_xcd = static_cast<int32_t>((items + kXcds - 1) / kXcds);
  a.scale = 1.0f / sqrtf(static_cast<float>(in.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid(static_cast<unsigned>(int64_t(a.per_xcd) * kXcds));
  const bool ob = out_dtype == STEM_BF16;
  if (in.dtype == STEM_BF16) return launch_dtype<true>(a, grid, in.block, in.head_dim, ob, st);
  return launch_dtype<false>(a, grid, in.block, in.head_dim, ob, st);
}

}  // namespace stem
