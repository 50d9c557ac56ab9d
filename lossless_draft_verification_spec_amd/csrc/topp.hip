// topp.hip -- the nucleus (top-p) threshold and kept mass of every row.
//
// [alphalab] §"想跑 Uno" lists top-p among the run settings; the nucleus is tie-inclusive (every
// token whose logit equals the boundary logit is kept) and the kept distribution is renormalised.
#include "launch.h"

namespace psispec {
namespace {

constexpr int kToppUnroll = 8;   // 16-byte loads in flight per thread
constexpr int kCandQueue = 256;  // candidate logits queued per wave before they are processed
constexpr int kExactBins = 1024; // distinct bf16 candidate values counted in one pass
static_assert(kExactBins % kThreads == 0, "bins split evenly over the threads");

template <typename T>
__device__ inline T neg_inf();
template <>
__device__ inline float neg_inf<float>() { return -__builtin_huge_valf(); }
template <>
__device__ inline bf16_t neg_inf<bf16_t>() { return bf16_t{0xff80u}; }

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

// ---------------------------------------------------------------------------------------------
// bf16 rows whose candidate logits take at most kExactBins distinct values (the usual case: the
// candidates lie within a few binades of the row maximum) are settled in one pass over the row.
// Bin b counts the tokens whose bf16 key is khi - b; a value's mass is its count times the same
// fixed-point pi the radix select adds per token, so threshold and kept mass are the integers the
// radix select reaches, found with one read of the row instead of two.
// ---------------------------------------------------------------------------------------------
__device__ void topp_exact_bf16(const RowSet& rs, int64_t row, const bf16_t* __restrict__ rp,
                                int vec_ok, float lmax, float invZ, float c, float pi_min,
                                float l_cut, double target, uint32_t khi,
                                ToppStat* __restrict__ topp) {
  __shared__ uint32_t cnt[kThreads / 64][kExactBins];
  __shared__ unsigned long long s_wtot[kThreads / 64];
  __shared__ unsigned long long s_kept;
  __shared__ int s_bin, s_lowest;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int k = threadIdx.x; k < (kThreads / 64) * kExactBins; k += kThreads) (&cnt[0][0])[k] = 0u;
  if (threadIdx.x == 0) {
    s_bin = -1;
    s_lowest = -1;
  }
  __syncthreads();
  uint32_t* mine = cnt[wave];
  auto count = [&](bf16_t e) {
    if (to_f32(e) >= l_cut) {
      const uint32_t bin = khi - order_key16(e.bits == 0x8000u ? (uint16_t)0 : e.bits);
      if (bin < (uint32_t)kExactBins) atomicAdd(&mine[bin], 1u);
    }
  };
  constexpr int E = 8;
  const int nvec = vec_ok ? rs.V / E : 0;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp);
  int i = threadIdx.x;
  for (; i + (kToppUnroll - 1) * kThreads < nvec; i += kToppUnroll * kThreads) {
    u32x4 v[kToppUnroll];
#pragma unroll
    for (int u = 0; u < kToppUnroll; ++u) v[u] = __builtin_nontemporal_load(vp + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kToppUnroll; ++u) {
      const bf16_t* ev = reinterpret_cast<const bf16_t*>(&v[u]);
#pragma unroll
      for (int k = 0; k < E; ++k) count(ev[k]);
    }
  }
  for (; i < nvec; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(vp + i);
    const bf16_t* ev = reinterpret_cast<const bf16_t*>(&v);
#pragma unroll
    for (int k = 0; k < E; ++k) count(ev[k]);
  }
  for (int x = nvec * E + threadIdx.x; x < rs.V; x += kThreads) count(rp[x]);
  __syncthreads();

  // the mass of every value, then each thread's run of kPerThread consecutive bins
  constexpr int kPerThread = kExactBins / kThreads;
  const int b0 = threadIdx.x * kPerThread;
  unsigned long long w[kPerThread], s = 0;
  int lowest = -1;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int b = b0 + j;
    uint32_t n = 0;
    for (int v = 0; v < kThreads / 64; ++v) n += cnt[v][b];
    w[j] = 0;
    if (n != 0u && (uint32_t)b <= khi) {
      const float l = key16_to_float(khi - (uint32_t)b);
      const float pi = __builtin_amdgcn_exp2f((l - lmax) * c) * invZ;
      if (pi >= pi_min && pi != 0.f)
        w[j] = (unsigned long long)n * (unsigned long long)((double)pi * 0x1.0p56);
    }
    if (w[j]) lowest = b;
    s += w[j];
  }
  // exclusive prefix of the runs in bin order (value order, largest first)
  unsigned long long incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) s_wtot[wave] = incl;
  if (lowest >= 0) atomicMax(&s_lowest, lowest);
  __syncthreads();
  unsigned long long pre = incl - s, total = 0;
  for (int v = 0; v < kThreads / 64; ++v) {
    if (v < wave) pre += s_wtot[v];
    total += s_wtot[v];
  }
  // the first bin at which the running mass reaches top_p; exactly one run holds it
  if ((double)pre < target) {
    unsigned long long run = pre;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if ((double)(run + w[j]) >= target) {
        s_bin = b0 + j;
        s_kept = run + w[j];
        break;
      }
      run += w[j];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float thr;
    unsigned long long kept;
    if (s_bin >= 0) {
      thr = key16_to_float(khi - (uint32_t)s_bin);
      kept = s_kept;
    } else if (s_lowest >= 0) {  // rounding left the mass short: every kept token
      thr = key16_to_float(khi - (uint32_t)s_lowest);
      kept = total;
    } else {
      thr = key16_to_float(0u);
      kept = 0;
    }
    topp[row] = ToppStat{thr, 0, (double)kept * 0x1.0p-56};
  }
}

// ---------------------------------------------------------------------------------------------
// Nucleus threshold by a mass-weighted radix select over the order keys of the logits, 8 bits per
// round (2 rounds for bf16, 4 for fp32).  Masses are fixed-point integers (pi * 2^56) summed with
// integer atomics, so the result is independent of the order of the atomics.  Only tokens with
// pi >= pi_min = (1 - top_p) / (4 V) take part: all smaller tokens together hold less than
// (1 - top_p) / 4, so the group at which the running mass reaches top_p is never among them.
// ---------------------------------------------------------------------------------------------
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
  if constexpr (kHalf) {
    // -0 and +0 are one logit value: both take the key of +0
    const uint32_t khi = order_key16((uint16_t)(__float_as_uint(lmax + 0.f) >> 16));
    if (l_cut > -__builtin_huge_valf()) {
      // every candidate (l >= l_cut) has a key of at least klo: truncating l_cut to bf16 moves it
      // down for l_cut > 0 and up by less than one bf16 step for l_cut < 0
      const uint32_t kt = order_key16((uint16_t)(__float_as_uint(l_cut) >> 16));
      const uint32_t klo = kt > 0 ? kt - 1 : 0;
      if (khi >= klo && khi - klo < (uint32_t)kExactBins) {
        topp_exact_bf16(rs, row, rp, vec_ok, lmax, invZ, c, pi_min, l_cut, target, khi, topp);
        return;
      }
    }
  }
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
      const float l = to_f32(e) + 0.f;  // -0 -> +0: one value, one key
      bool cand = l >= l_cut;
      if (round > 0 && cand) {
        const uint32_t key = kHalf ? order_key16((uint16_t)(__float_as_uint(l) >> 16)) : order_key(l);
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
      if (b < 0) {  // rounding left the mass short: every kept token, down to the lowest bin
        b = lowest < 0 ? 0 : lowest;
        run -= hist[0][b];
      }
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
