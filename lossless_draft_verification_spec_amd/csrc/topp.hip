// topp.hip -- the nucleus (top-p) threshold and kept mass of every row.
//
// [alphalab] §"想跑 Uno" lists top-p among the run settings; the nucleus is tie-inclusive (every
// token whose logit equals the boundary logit is kept) and the kept distribution is renormalised.
#include "launch.h"

namespace psispec {
namespace {

constexpr int kToppUnroll = 8;   // 16-byte loads in flight per thread
constexpr int kCandQueue = 256;  // candidate logits queued per wave before they are processed

template <typename T>
__device__ inline T neg_inf();
template <>
__device__ inline float neg_inf<float>() { return -__builtin_huge_valf(); }
template <>
__device__ inline bf16_t neg_inf<bf16_t>() { return bf16_t{0xff80u}; }

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
                                                   ToppStat* __restrict__ topp,
                                                   const RowStat* __restrict__ pre, int vec_ok) {
  constexpr bool kHalf = sizeof(T) == 2;
  constexpr int kKeyBits = kHalf ? 16 : 32;
  constexpr int kRounds = kKeyBits / 8;
  const int64_t row = blockIdx.x;
  if (row_skipped(rs, row)) return;
  const T* rp = row_ptr<T>(rs, row);
  float lmax;
  double Z;
  if (pre) {  // statistics already combined
    lmax = pre[row].lmax;
    Z = pre[row].Z;
  } else {
    row_stats_from_parts(part, row, nchunk, c, lmax, Z);
  }
  if (!(lmax > kNegBig) || !(lmax < __builtin_huge_valf()) || !(Z > 0.0) || !(Z < 1e300)) {
    if (threadIdx.x == 0) topp[row] = ToppStat{-__builtin_huge_valf(), 0, 1.0};
    return;
  }
  const float invZ = (float)(1.0 / Z);
  const double target = top_p * 0x1.0p56;
  // Logits below l_cut cannot pass the pi >= pi_min test (pi = exp2((l - lmax) c) / Z): a
  // comparison rejects them without an exp.  The cut sits a margin below the exact bound, so the
  // exact test below still decides every token near it.
  const float l_cut = pi_min > 0.f
      ? (float)((double)lmax + (log2((double)pi_min) + log2(Z)) / (double)c - 1e-3 * (1.0 + fabs((double)lmax)))
      : -__builtin_huge_valf();

  // one histogram per wave (the candidates' keys crowd into few bins), summed in wave order
  __shared__ unsigned long long hist[kThreads / 64][256];
  __shared__ float s_cand[kThreads / 64][kCandQueue];
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_above, s_kept;
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_above = 0;
    s_kept = 0;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int E = 16 / (int)sizeof(T);
  const int nvec = vec_ok ? rs.V / E : 0;
  for (int round = 0; round < kRounds; ++round) {
    const int shift = kKeyBits - 8 * (round + 1);
    for (int w = 0; w < kThreads / 64; ++w) hist[w][threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    // Candidates (few percent of the tokens, crowding into a few bins) are compacted per wave into
    // an LDS queue and processed 64 at a time, so the exp and the histogram atomics run on full
    // waves instead of on the scattered lanes of every token.
    int fill = 0;  // queue length, the same in every lane
    auto flush = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int k = lane; k < fill; k += 64) {
        const float l = s_cand[wave][k];
        const uint32_t key = kHalf ? order_key16((uint16_t)(__float_as_uint(l) >> 16)) : order_key(l);
        const float pi = __builtin_amdgcn_exp2f((l - lmax) * c) * invZ;
        if (!(pi >= pi_min) || pi == 0.f) continue;
        const unsigned long long w = (unsigned long long)((double)pi * 0x1.0p56);
        atomicAdd(&hist[wave][(key >> shift) & 255u], w);
      }
      __builtin_amdgcn_wave_barrier();
      fill = 0;
    };
    auto take = [&](T e) {
      const float l = to_f32(e);
      bool cand = l >= l_cut;
      if (round > 0 && cand) {
        uint32_t key;
        if constexpr (kHalf) {
          key = order_key16(e.bits);
        } else {
          key = order_key(l);
        }
        cand = (key >> (shift + 8)) == (prefix >> (shift + 8));
      }
      const uint64_t m = __ballot(cand);
      if (cand) s_cand[wave][fill + __builtin_popcountll(m & ((1ull << lane) - 1ull))] = l;
      fill += __builtin_popcountll(m);
      if (fill > kCandQueue - 64) flush();
    };
    const u32x4* vp = reinterpret_cast<const u32x4*>(rp);
    int i = threadIdx.x;
    // eight 16-byte loads in flight per thread, then their tokens; the loop bound is the same for
    // every lane of a wave (the queue needs the whole wave in every step)
    for (; i - lane + 63 + (kToppUnroll - 1) * kThreads < nvec; i += kToppUnroll * kThreads) {
      u32x4 v[kToppUnroll];
#pragma unroll
      for (int u = 0; u < kToppUnroll; ++u) v[u] = __builtin_nontemporal_load(vp + i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kToppUnroll; ++u) {
        const T* ev = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
        for (int k = 0; k < E; ++k) take(ev[k]);
      }
    }
    // the rest: every lane of the wave takes part in each step (a token past the row is -inf)
    const int nvec_w = (nvec + kThreads - 1) / kThreads * kThreads;
    for (; i < nvec_w; i += kThreads) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (i < nvec) v = __builtin_nontemporal_load(vp + i);
      const T* ev = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int k = 0; k < E; ++k) take(i < nvec ? ev[k] : neg_inf<T>());
    }
    const int tail = nvec * E;
    const int V_w = tail + (rs.V - tail + kThreads - 1) / kThreads * kThreads;
    for (int x = tail + threadIdx.x; x < V_w; x += kThreads) take(x < rs.V ? rp[x] : neg_inf<T>());
    flush();
    __syncthreads();
    {
      unsigned long long tot = 0;
      for (int w = 0; w < kThreads / 64; ++w) tot += hist[w][threadIdx.x];
      hist[0][threadIdx.x] = tot;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long above = s_above, run = above;
      int b = 255;
      int lowest = -1;
      for (; b >= 0; --b) {
        if (hist[0][b]) lowest = b;
        if ((double)(run + hist[0][b]) >= target) break;
        run += hist[0][b];
      }
      if (b < 0) b = lowest < 0 ? 0 : lowest;  // rounding left the mass short: lowest kept bin
      s_above = run;
      s_kept = run + hist[0][b];
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

hipError_t launch_topp(const RowSet& rs, psispec_dtype dtype, int nchunk, float c, double top_p,
                       const float2* part, ToppStat* topp, hipStream_t stream,
                       const RowStat* rowstat) {
  const int64_t rows = rs.nP + rs.nQ;
  if (rows == 0) return hipSuccess;
  double pmin = (1.0 - top_p) / (4.0 * (double)rs.V);
  if (pmin < 1e-30) pmin = 0.0;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)rs.V * es) % 16 == 0 && ((size_t)rs.pstride * es) % 16 == 0 &&
                     ((uintptr_t)rs.p % 16) == 0 &&
                     ((uintptr_t)rs.q % 16) == 0;
  timing_begin("topp", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_topp<bf16_t>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs, nchunk,
                       c, top_p, (float)pmin, part, topp, rowstat, vec_ok);
  else
    hipLaunchKernelGGL(k_topp<float>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs, nchunk,
                       c, top_p, (float)pmin, part, topp, rowstat, vec_ok);
  timing_end("topp", stream);
  return hipGetLastError();
}

}  // namespace psispec
