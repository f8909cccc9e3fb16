// Token Position-Decay top-k selection of one (query head, query block) row
// by one 64-wide wavefront (gist.science/es "Implementacion" steps 2-3;
// gist.science/nl "Implementatie" steps 2-3; initial blocks are always kept
// because every later token aggregates them, gist.science/es section 1 and
// gist.science/fr section 1).  Shared by the selection kernel and the
// attention kernel's fused-selection prologue.
//
// The row's candidate metrics are read once (coalesced) into registers as
// order-preserving 32-bit keys.  Thresholds are found by a bitwise bisection
// (from the highest bit in which the largest and smallest key differ) whose
// counts come from wavefront ballots (v_cmp straight into a scalar mask,
// popcount on the scalar unit).  Fast path (budget <= 64): the take-th
// largest of the 64 per-lane maxima bounds the threshold from below; the few
// keys that reach it are compacted, in block order, into one register per
// lane and the exact threshold is found there with one ballot per bit.
// Otherwise the bisection runs over every key.  Keys above the threshold are
// kept; keys equal to it are kept in ascending block order until the budget
// is met, which is exactly "larger metric first, equal metrics to the
// smaller block number".  Kept blocks come out in ascending order: the
// forced sink blocks, the selected ones, the forced diagonal block.
#ifndef STEM_SELECT_ROW_H
#define STEM_SELECT_ROW_H

#include "stem_device.h"

namespace stem {

// Order-preserving key: larger float -> larger key; -0 == +0; NaN -> 1
// (below every number); 0 is reserved for "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Largest T with #{lanes l: v_l >= T} >= need (need >= 1 lanes hold v >= lo,
// every v that counts is >= lo >= 1 and <= hi): bitwise bisection from the
// highest bit in which lo and hi differ.
__device__ __forceinline__ uint32_t kth_largest(uint32_t v, uint32_t lo, uint32_t hi, int need) {
  const uint32_t diff = lo ^ hi;
  const int top = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t T = top < 0 ? hi : (top >= 31 ? 0u : (hi & ~((2u << top) - 1u)));
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    if (__popcll(__ballot(v >= cand)) >= need) T = cand;
  }
  return T;
}

// Row i (0-based query block within its sequence) with budget k_i and S
// sink blocks; mrow holds the row's i + 1 metric values (key blocks 0 .. i),
// read only when the budget leaves a choice; E 64-lane chunks cover the
// candidates S .. i - 1.  ckey / cpos: 64 entries of LDS scratch of this
// wavefront.  emit(p, j) is called once for every kept position
// p = 0 .. k_i - 1 with its block j, each call by one lane.
template <int E, typename Emit>
__device__ __forceinline__ void select_row(const float *mrow, int i, int k_i, int S,
                                           uint32_t *ckey, int32_t *cpos, Emit &&emit) {
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int nforced = i < S ? i + 1 : S + 1;
  const int ncand = i < S ? 0 : i - S;
  const int take = k_i - nforced;
  if (take >= ncand) {  // every causal block is kept
    for (int p = lane; p <= i; p += 64) emit(p, p);
    return;
  }
  // candidates j = S + lane + 64 e; every load is issued before any use
  float mv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = S + lane + 64 * e;
    mv[e] = j < i ? mrow[j] : 0.f;
  }
  uint32_t key[E];
  uint32_t kmx = 0u, kmn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = S + lane + 64 * e < i;
    key[e] = c ? order_key(mv[e]) : 0u;
    kmx = c ? max(kmx, key[e]) : kmx;
    kmn = c ? min(kmn, key[e]) : kmn;
  }
  const int ne = (ncand + 63) >> 6;  // chunks holding candidates (wave-uniform)
  // Fast path.  L = the take-th largest of the 64 per-lane maxima is a lower
  // bound of the take-th largest key (take lanes each hold a key >= L).  When
  // at most 64 keys reach L they are compacted, in block order, into one
  // register per lane and the exact threshold is found there.
  if (take >= 1 && take <= 64) {
    uint32_t lmax = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) lmax = max(lmax, key[e]);
    uint32_t wmax = lmax, wmin = lmax ? lmax : 0xffffffffu;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      wmax = max(wmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmax), o)));
      wmin = min(wmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmin), o)));
    }
    const uint32_t L = kth_largest(lmax, wmin, wmax, take);
    int nc = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < ne) nc += __popcll(__ballot(key[e] >= L));
    if (nc <= 64) {
      int base = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e >= ne) break;
        const bool c = key[e] >= L;
        const uint64_t m = __ballot(c);
        if (c) {
          const int p = base + static_cast<int>(lanes_below(m));
          ckey[p] = key[e];
          cpos[p] = S + lane + 64 * e;
        }
        base += __popcll(m);
      }
      const uint32_t ck = lane < nc ? ckey[lane] : 0u;
      const int cj = lane < nc ? cpos[lane] : 0;
      const uint32_t T = kth_largest(ck, L, wmax, take);
      const int gt = __popcll(__ballot(ck > T));
      const uint64_t eqm = __ballot(ck == T);
      const bool sel = ck > T || (ck == T && static_cast<int>(lanes_below(eqm)) < take - gt);
      const uint64_t sm = __ballot(sel);
      if (sel) emit(S + static_cast<int>(lanes_below(sm)), cj);
      for (int p = lane; p < S; p += 64) emit(p, p);
      if (lane == 0) emit(S + take, i);
      return;
    }
  }
  // largest T with #{key >= T} >= take (take >= 1 here, and all
  // candidates have key >= 1, so T >= 1 and padding never qualifies).
  // T lies between the row's smallest and largest key, so the bits above
  // their highest differing bit are already known.
  uint32_t T = 0;
  if (take > 0) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmx = max(kmx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmx), o)));
      kmn = min(kmn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmn), o)));
    }
    const uint32_t diff = kmx ^ kmn;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    T = top < 0 ? kmx : (top >= 31 ? 0u : (kmx & ~((2u << top) - 1u)));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
      if (cnt >= take) T = cand;
    }
  } else {
    T = 0xffffffffu;  // nothing to take: no key passes "> T", none ties
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
  const int need_eq = take > 0 ? take - gt : 0;

  int pos = S, eq_seen = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= ne) break;
    const bool is_eq = take > 0 && key[e] == T;
    const uint64_t eqm = __ballot(is_eq);
    const int rank = eq_seen + static_cast<int>(lanes_below(eqm));
    eq_seen += __popcll(eqm);
    const bool sel = key[e] > T || (is_eq && rank < need_eq);
    const uint64_t sm = __ballot(sel);
    if (sel) emit(pos + static_cast<int>(lanes_below(sm)), S + lane + 64 * e);
    pos += __popcll(sm);
  }
  for (int p = lane; p < S; p += 64) emit(p, p);
  if (lane == 0) emit(S + take, i);
}

}  // namespace stem

#endif
