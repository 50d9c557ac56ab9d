// rows.hip -- the HBM pass over every logits row: temperature-softmax statistics, and the nucleus
// (top-p) threshold.
//
// Every p and q row of a call is read once here (the data-parallel part of the verify: [alphalab]
// walkthrough step 3 -- the AR scores the whole block in one pass and every position gets its
// test).  A workgroup streams one chunk of one row with 16-byte loads and keeps an online
// (max, sum of exp) pair per lane; the pair of each (row, chunk) goes to the workspace and is
// combined in a fixed order by the consumers, so results do not depend on scheduling.
#include "launch.h"

namespace psispec {
namespace {

template <typename T>
struct Elems;
template <>
struct Elems<bf16_t> {
  static constexpr int kPerVec = 8;
  __device__ static void unpack(const u32x4& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};
template <>
struct Elems<float> {
  static constexpr int kPerVec = 4;
  __device__ static void unpack(const u32x4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

// Fold n values into the online pair (m, s), s = sum exp2((x - m) * c).  m starts at a finite floor
// so that -inf entries contribute exp2(-inf) = 0 and NaN/+inf entries turn s into NaN.
template <int n>
__device__ inline void fold(const float (&f)[n], float& m, float& s, float c) {
  float vm = f[0];
#pragma unroll
  for (int j = 1; j < n; ++j) vm = fmaxf(vm, f[j]);
  if (vm > m) {
    s *= __builtin_amdgcn_exp2f((m - vm) * c);
    m = vm;
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < n; ++j) acc += __builtin_amdgcn_exp2f((f[j] - m) * c);
  s += acc;
}

__device__ inline void block_reduce_pair(float& m, float& s, float c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    os_combine(m, s, m2, s2, c);
  }
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0];
    s = ss[0];
    for (int w = 1; w < kThreads / 64; ++w) os_combine(m, s, sm[w], ss[w], c);
  }
}

template <typename T, int kUnroll>
__global__ __launch_bounds__(kThreads) void k_rowstats(RowSet rs, int nchunk, int chunk_elems,
                                                       float c, float2* __restrict__ part,
                                                       int vec_ok) {
  const int64_t task = blockIdx.x;
  const int64_t row = task / nchunk;
  const int chunk = (int)(task - row * nchunk);
  if (row_skipped(rs, row)) return;
  const T* rp = row_ptr<T>(rs, row);
  const int start = chunk * chunk_elems;
  const int end = min(rs.V, start + chunk_elems);
  float m = kNegBig, s = 0.f;
  int tail = start;
  if (vec_ok) {
    constexpr int E = Elems<T>::kPerVec;
    const int nvec = (end - start) / E;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rp + start);
    int i = threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < nvec; i += kUnroll * kThreads) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(vp + i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float f[E];
        Elems<T>::unpack(v[u], f);
        fold(f, m, s, c);
      }
    }
    for (; i < nvec; i += kThreads) {
      float f[E];
      Elems<T>::unpack(vp[i], f);
      fold(f, m, s, c);
    }
    tail = start + nvec * E;
  }
  for (int x = tail + threadIdx.x; x < end; x += kThreads) {
    const float f[1] = {to_f32(rp[x])};
    fold(f, m, s, c);
  }
  block_reduce_pair(m, s, c);
  if (threadIdx.x == 0) part[task] = make_float2(m, s);
}

// ---------------------------------------------------------------------------------------------
// Nucleus threshold by a mass-weighted radix select over the order keys of the logits, 8 bits per
// round (2 rounds for bf16, 4 for fp32).  Masses are fixed-point integers (pi * 2^56) summed with
// integer atomics, so the result is independent of the order of the atomics.  Only tokens with
// pi >= pi_min = (1 - top_p) / (4 V) take part: all smaller tokens together hold less than
// (1 - top_p) / 4, so the group at which the running mass reaches top_p is never among them.
// ---------------------------------------------------------------------------------------------
__device__ inline void row_stats_from_parts(const float2* part, int64_t row, int nchunk, float c,
                                            float& lmax, double& Z) {
  lmax = kNegBig;
  for (int k = 0; k < nchunk; ++k) lmax = fmaxf(lmax, part[row * nchunk + k].x);
  Z = 0.0;
  for (int k = 0; k < nchunk; ++k) {
    const float2 pk = part[row * nchunk + k];
    Z += (double)pk.y * exp2((double)(pk.x - lmax) * (double)c);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_topp(RowSet rs, int nchunk, float c, double top_p,
                                                   float pi_min, const float2* __restrict__ part,
                                                   ToppStat* __restrict__ topp) {
  constexpr bool kHalf = sizeof(T) == 2;
  constexpr int kKeyBits = kHalf ? 16 : 32;
  constexpr int kRounds = kKeyBits / 8;
  const int64_t row = blockIdx.x;
  if (row_skipped(rs, row)) return;
  const T* rp = row_ptr<T>(rs, row);
  float lmax;
  double Z;
  row_stats_from_parts(part, row, nchunk, c, lmax, Z);
  if (!(lmax > kNegBig) || !(lmax < __builtin_huge_valf()) || !(Z > 0.0) || !(Z < 1e300)) {
    if (threadIdx.x == 0) topp[row] = ToppStat{-__builtin_huge_valf(), 0, 1.0};
    return;
  }
  const float invZ = (float)(1.0 / Z);
  const double target = top_p * 0x1.0p56;

  __shared__ unsigned long long hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_above, s_kept;
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_above = 0;
    s_kept = 0;
  }
  for (int round = 0; round < kRounds; ++round) {
    const int shift = kKeyBits - 8 * (round + 1);
    hist[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int x = threadIdx.x; x < rs.V; x += kThreads) {
      const T e = rp[x];
      const float l = to_f32(e);
      uint32_t key;
      if constexpr (kHalf) {
        key = order_key16(e.bits);
      } else {
        key = order_key(l);
      }
      if (round > 0 && (key >> (shift + 8)) != (prefix >> (shift + 8))) continue;
      const float pi = __builtin_amdgcn_exp2f((l - lmax) * c) * invZ;
      if (!(pi >= pi_min) || pi == 0.f) continue;
      const unsigned long long w = (unsigned long long)((double)pi * 0x1.0p56);
      atomicAdd(&hist[(key >> shift) & 255u], w);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long above = s_above, run = above;
      int b = 255;
      int lowest = -1;
      for (; b >= 0; --b) {
        if (hist[b]) lowest = b;
        if ((double)(run + hist[b]) >= target) break;
        run += hist[b];
      }
      if (b < 0) b = lowest < 0 ? 0 : lowest;  // rounding left the mass short: lowest kept bin
      s_above = run;
      s_kept = run + hist[b];
      s_prefix = prefix | ((uint32_t)b << shift);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float thr = kHalf ? key16_to_float(s_prefix) : key_to_float(s_prefix);
    topp[row] = ToppStat{thr, 0, (double)s_kept * 0x1.0p-56};
  }
}

}  // namespace

hipError_t launch_rowstats(const RowSet& rs, psispec_dtype dtype, int nchunk, int chunk_elems,
                           float c, float2* part, hipStream_t stream) {
  const int64_t tasks = (rs.nP + rs.nQ) * (int64_t)nchunk;
  if (tasks == 0) return hipSuccess;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)rs.V * es) % 16 == 0 && ((uintptr_t)rs.p % 16) == 0 &&
                     ((uintptr_t)rs.q % 16) == 0 && (chunk_elems % 8) == 0;
  timing_begin("rowstats", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL((k_rowstats<bf16_t, 4>), dim3((unsigned)tasks), dim3(kThreads), 0, stream,
                       rs, nchunk, chunk_elems, c, part, vec_ok);
  else
    hipLaunchKernelGGL((k_rowstats<float, 4>), dim3((unsigned)tasks), dim3(kThreads), 0, stream,
                       rs, nchunk, chunk_elems, c, part, vec_ok);
  timing_end("rowstats", stream);
  return hipGetLastError();
}

hipError_t launch_topp(const RowSet& rs, psispec_dtype dtype, int nchunk, float c, double top_p,
                       const float2* part, ToppStat* topp, hipStream_t stream) {
  const int64_t rows = rs.nP + rs.nQ;
  if (rows == 0) return hipSuccess;
  double pmin = (1.0 - top_p) / (4.0 * (double)rs.V);
  if (pmin < 1e-30) pmin = 0.0;
  timing_begin("topp", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_topp<bf16_t>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs, nchunk,
                       c, top_p, (float)pmin, part, topp);
  else
    hipLaunchKernelGGL(k_topp<float>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs, nchunk,
                       c, top_p, (float)pmin, part, topp);
  timing_end("topp", stream);
  return hipGetLastError();
}

}  // namespace psispec
