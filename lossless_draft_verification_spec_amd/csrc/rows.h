// rows.h -- device code of the HBM row pass, shared by the row-pass kernel and the fused verify.
//
// A workgroup streams one chunk of one row with 16-byte loads and keeps an online
// (max, sum of exp) pair per lane; the pair of each (row, chunk) goes to the workspace and is
// combined in a fixed order by the consumers, so results do not depend on scheduling.
#pragma once

#include "internal.h"

namespace psispec {
namespace {

template <typename T>
struct Elems;
template <>
struct Elems<bf16_t> {
  static constexpr int kPerVec = 8;
  __device__ static void unpack(const u32x4& v, float* f) {  // f[0..8)
    f[0] = bf16_lo(v.x);
    f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y);
    f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z);
    f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w);
    f[7] = bf16_hi(v.w);
  }
};
template <>
struct Elems<float> {
  static constexpr int kPerVec = 4;
  __device__ static void unpack(const u32x4& v, float* f) {  // f[0..4)
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

// Fold n values into the online pair (m, s), s = sum exp2((x - m) * c).  m starts at a finite floor
// so that -inf entries contribute exp2(-inf) = 0 and NaN/+inf entries turn s into NaN (a row with a
// NaN is rejected by its sum, whatever its maximum).  The rescale runs every time: its factor is
// exp2(0) = 1 exactly when the maximum did not move, and it costs less than the compare and the
// selects of a conditional one.
template <int n>
__device__ inline void fold(const float (&f)[n], float& m, float& s, float c) {
  float mn = m;
#pragma unroll
  for (int j = 0; j < n; ++j) mn = fmaxf(mn, f[j]);
  float acc = __builtin_amdgcn_exp2f((f[0] - mn) * c);
#pragma unroll
  for (int j = 1; j < n; ++j) acc += __builtin_amdgcn_exp2f((f[j] - mn) * c);
  s = s * __builtin_amdgcn_exp2f((m - mn) * c) + acc;
  m = mn;
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

// One chunk of one row: the block's online pair (max, sum exp2((x - max) c)) over logits
// [chunk * chunk_elems, min(V, (chunk + 1) * chunk_elems)), written by thread 0 to *out.  Called by
// every thread of a kThreads block (it contains block barriers).
template <typename T, int kUnroll>
__device__ inline void rowstats_task(const RowSet& rs, int64_t row, int chunk, int chunk_elems,
                                     float c, float2* out, int vec_ok) {
  static_assert(kUnroll % 2 == 0, "vectors are folded in pairs");
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
      // two vectors per fold: one rescale per 2E values
#pragma unroll
      for (int u = 0; u < kUnroll; u += 2) {
        float f[2 * E];
        Elems<T>::unpack(v[u], f);
        Elems<T>::unpack(v[u + 1], f + E);
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
  if (threadIdx.x == 0) *out = make_float2(m, s);
}

}  // namespace
}  // namespace psispec
