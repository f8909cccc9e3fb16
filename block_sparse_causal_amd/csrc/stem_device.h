// Device-side helpers and the launch interface between the C entry points
// (stem_api.hip) and the kernels (pool.hip, score.hip, select.hip,
// attn.hip).  gfx950 (CDNA4) only: 64-wide wavefronts, MFMA matrix cores.
#ifndef STEM_DEVICE_H
#define STEM_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stem.h"

namespace stem {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plan arrays on the device (see stem_plan_info for their meaning).
struct PlanDev {
  const int32_t *cu_seqlens;
  const int32_t *cu_blocks;
  const int64_t *tri;
  const int32_t *blk_seq;
  const int32_t *budget;
  const int32_t *order;
};

inline PlanDev make_plan_dev(const stem_plan_info &in, const void *base) {
  const char *b = static_cast<const char *>(base);
  PlanDev p;
  p.cu_seqlens = reinterpret_cast<const int32_t *>(b + in.off_cu_seqlens);
  p.cu_blocks = reinterpret_cast<const int32_t *>(b + in.off_cu_blocks);
  p.tri = reinterpret_cast<const int64_t *>(b + in.off_tri);
  p.blk_seq = reinterpret_cast<const int32_t *>(b + in.off_blk_seq);
  p.budget = reinterpret_cast<const int32_t *>(b + in.off_budget);
  p.order = reinterpret_cast<const int32_t *>(b + in.off_order);
  return p;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// One wavefront-wide 16-byte-per-lane DMA from global memory into LDS:
// lane l's 16 bytes land at LDS byte address lds_addr + 16 l.  Issued from
// inline assembly so that the compiler does not track the LDS write (it
// would otherwise wait for an in-flight prefetch before every unrelated LDS
// read); callers order it explicitly with s_waitcnt vmcnt (and a barrier
// when other wavefronts read the data).  The global address is a
// wave-uniform base (SGPRs) plus a 32-bit per-lane byte offset; M0, which
// carries the LDS address, is saved and restored.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}

// Four such DMAs in one asm block: M0 is saved and restored once for the
// four instead of once per instruction (DMA k: base gk, lane offset vk, LDS
// address lk).
__device__ __forceinline__ void dma16x4(const void *g0, uint32_t v0, uint32_t l0,
                                        const void *g1, uint32_t v1, uint32_t l1,
                                        const void *g2, uint32_t v2, uint32_t l2,
                                        const void *g3, uint32_t v3, uint32_t l3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %6\n\t"
      "s_mov_b32 m0, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %7\n\t"
      "s_mov_b32 m0, %12\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %8\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(g0), "s"(g1), "s"(g2), "s"(g3),
        "s"(l0), "s"(l1), "s"(l2), "s"(l3)
      : "memory");
}

// s_waitcnt vmcnt(0) / lgkmcnt(0) alone, as builtins so that the compiler's
// own wait-count bookkeeping sees them.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// LDS byte address (what M0 and ds_* instructions take) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_pool(const stem_plan_info &in, PlanDev pd, const void *q,
                       const void *k, const void *v, float *qbar, float *kbar,
                       float *vnorm, int vnorm_mode, hipStream_t st);
hipError_t launch_score(const stem_plan_info &in, PlanDev pd, const float *qbar,
                        const float *kbar, const float *vnorm, float *scores,
                        hipStream_t st);
// Anti-diagonal sampled metric (antidiag.hip): block logits from the token
// logits, then the metric in place; units_per_head bounds its tile pairs.
int64_t antidiag_units_per_head(const stem_plan_info &in, int stride);
hipError_t launch_score_antidiag(const stem_plan_info &in, PlanDev pd, const void *q,
                                 const void *k, const float *vnorm, int stride,
                                 float *scores, hipStream_t st);
hipError_t launch_select(const stem_plan_info &in, PlanDev pd, const float *scores,
                         int32_t *idx, int32_t *count, hipStream_t st);
hipError_t launch_attn(const stem_plan_info &in, PlanDev pd, const void *q,
                       const void *k, const void *v, const int32_t *idx,
                       const int32_t *count, void *out, int out_dtype, float *lse,
                       hipStream_t st);

}  // namespace stem

#endif
