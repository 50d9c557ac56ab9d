// peak.hip -- measured ceilings of this GPU, the denominators the benchmark reports beside the
// datasheet figures: the HBM read bandwidth that 16-byte nontemporal loads sustain (the load form
// the row passes use) and the bf16 matrix-core issue rate of the 32x32x16 MFMA with 4 x 4
// independent accumulators per wave (the LM-head product's instruction stream), with no memory
// traffic beside it.  Neither is a step of the verify.
#include "launch.h"

namespace psispec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every 16-byte word of the buffer read once: block b reads its own contiguous segment, each
// thread eight consecutive-per-wave 16-byte words per round (eight loads in flight), as the row
// passes stream a row chunk; one xor of what was read per block keeps the loads.
__global__ __launch_bounds__(kThreads) void k_peak_read(const u32x4* __restrict__ p, int64_t n,
                                                        uint32_t* __restrict__ out) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = min(n, lo + per);
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 7 * kThreads < hi; i += 8 * kThreads) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < hi; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t s[kThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

// `iters` rounds of 16 back-to-back MFMAs per wave on register operands; the accumulators' sum is
// written per thread so that nothing is dropped.
__global__ __launch_bounds__(kThreads) void k_peak_mfma(int64_t iters, float* __restrict__ out) {
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = (__bf16)(1.0f / (float)(1 + ((threadIdx.x + i + e) & 7)));
      b[i][e] = (__bf16)(1.0f / (float)(1 + ((threadIdx.x + 3 * i + e) & 7)));
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_peak_read(const void* buf, size_t bytes, uint32_t* out, int blocks,
                            hipStream_t stream) {
  PSISPEC_LAUNCH("peak_read", k_peak_read, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                 static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(int64_t iters, float* out, int blocks, hipStream_t stream) {
  PSISPEC_LAUNCH("peak_mfma", k_peak_mfma, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters,
                 out);
  return hipGetLastError();
}

}  // namespace psispec
