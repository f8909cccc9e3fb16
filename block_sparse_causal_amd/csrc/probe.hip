// Measurement probes: the ceilings the path's kernels are compared with,
// re-measured on the device at hand (not part of the prefill path).
//
//   stem_probe_mfma      back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD
//                        (four independent accumulators per wavefront, many
//                        short workgroups so the load balances across the
//                        CUs), operands either random bf16
//                        values in [-1, 1) or small constants.  The chip's
//                        matrix-core rate depends on how much the operands
//                        toggle: its power limit, not the issue rate, caps it
//                        on random data.
//   stem_probe_hbm_read  one streaming pass of 16-byte non-temporal loads over
//                        a caller buffer (the pattern of the HBM-bound pool),
//                        64 KiB per workgroup.
//
// The caller times a launch (HIP events on the stream) and divides the
// reported work by it.
#include "stem_device.h"

namespace stem {
namespace {

constexpr int kProbeBlocksPerCU = 16;  // workgroups of 4 wavefronts per CU
constexpr int kProbeIters = 512;       // loop trips per wavefront
constexpr int kProbeChains = 4;        // independent accumulators per wavefront

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  return x ^ (x >> 16);
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float *sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kProbeChains], b[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = mix32((blockIdx.x * 256u + threadIdx.x) * 64u + j * 8u + e);
      a[j][e] = (__bf16)(RANDOM ? (h & 0xffffu) / 32768.f - 1.f : 0.001f * (lane + e));
      b[j][e] = (__bf16)(RANDOM ? (h >> 16) / 32768.f - 1.f : 0.002f * e);
    }
  f32x16 c[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) c[j] = f32x16{};
  for (int i = 0; i < kProbeIters; ++i) {
#pragma unroll
    for (int r = 0; r < kProbeChains; ++r)
#pragma unroll
      for (int j = 0; j < kProbeChains; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + r) % kProbeChains],
                                                       b[(j + 2 * r) % kProbeChains], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  // keeps the products live; the sink receives one value per workgroup
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

constexpr int kReadLoads = 16;                         // 16-byte loads per thread
constexpr int64_t kReadChunk = 256 * kReadLoads * 16;  // bytes per workgroup

// Each workgroup reads one contiguous 64 KiB chunk: all its loads are in
// flight before the first use, and the grid covers the buffer once.
__global__ __launch_bounds__(256) void hbm_probe_kernel(const u32x4 *p, int64_t n, uint32_t *sink) {
  __shared__ uint32_t part[4];
  const int64_t base = int64_t(blockIdx.x) * 256 * kReadLoads + threadIdx.x;
  u32x4 v[kReadLoads];
#pragma unroll
  for (int u = 0; u < kReadLoads; ++u) {
    const int64_t i = base + int64_t(u) * 256;
    v[u] = i < n ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kReadLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  // XOR of the workgroup's words, one sink word per workgroup: the XOR of
  // the sink is the XOR of every 32-bit word read (a check of the pass)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace
}  // namespace stem

using namespace stem;

extern "C" int stem_probe_mfma(int32_t random_operands, float *sink, int64_t sink_floats,
                               double *flops, void *stream) {
  int dev = 0, cus = 0;
  if (!sink || !flops) return STEM_EINVAL;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return STEM_EHIP;
  const int blocks = cus * kProbeBlocksPerCU;
  if (sink_floats < blocks) return STEM_EINVAL;
  *flops = double(blocks) * 4 * kProbeIters * kProbeChains * kProbeChains * (32.0 * 32 * 16 * 2);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (random_operands)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(blocks), dim3(256), 0, st, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(blocks), dim3(256), 0, st, sink);
  return hipGetLastError() == hipSuccess ? STEM_OK : STEM_EHIP;
}

extern "C" int stem_probe_hbm_read(const void *buf, int64_t bytes, uint32_t *sink,
                                   int64_t sink_words, void *stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return STEM_EINVAL;
  const int64_t blocks = (bytes + kReadChunk - 1) / kReadChunk;
  if (blocks > INT32_MAX || sink_words < blocks) return STEM_EINVAL;
  hipLaunchKernelGGL(hbm_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? STEM_OK : STEM_EHIP;
}
