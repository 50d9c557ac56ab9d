// topp.hip -- the nucleus (top-p) threshold and kept mass of every row.
//
// [alphalab] §"想跑 Uno" lists top-p among the run settings; the nucleus is tie-inclusive (every
// token whose logit equals the boundary logit is kept) and the kept distribution is renormalised.
#include "launch.h"
#include "rows.h"

namespace psispec {
namespace {

constexpr int kToppUnroll = 8;   // 16-byte loads in flight per thread
constexpr int kCandQueue = 256;  // candidate logits queued per wave before they are processed
constexpr int kFusedUnroll = 2;  // 16-byte loads in flight per thread in the fused row pass
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
// Common set-up of a row's nucleus search.  Only tokens with pi >= pi_min = (1 - top_p) / (4 V)
// take part: all smaller tokens together hold less than (1 - top_p) / 4, so the value at which the
// running mass reaches top_p is never among them.  Logits below l_cut cannot pass that test
// (pi = exp2((l - lmax) c) / Z): a comparison rejects them without an exp.  The cut sits a margin
// below the exact bound, so the exact test still decides every token near it.  Masses are
// fixed-point integers (pi * 2^56), so sums do not depend on their order.
// ---------------------------------------------------------------------------------------------
struct ToppSetup {
  float invZ, l_cut;
  double target;
};

// false (and the row's degenerate result written) for a row without a finite maximum or sum
__device__ inline bool topp_setup(float lmax, double Z, float c, double top_p, float pi_min,
                                  int64_t row, ToppStat* topp, ToppSetup& st) {
  if (!(lmax > kNegBig) || !(lmax < __builtin_huge_valf()) || !(Z > 0.0) || !(Z < 1e300)) {
    if (threadIdx.x == 0) topp[row] = ToppStat{-__builtin_huge_valf(), 0, 1.0};
    return false;
  }
  st.invZ = (float)(1.0 / Z);
  st.target = top_p * 0x1.0p56;
  st.l_cut = pi_min > 0.f ? (float)((double)lmax + (log2((double)pi_min) + log2(Z)) / (double)c -
                                    1e-3 * (1.0 + fabs((double)lmax)))
                          : -__builtin_huge_valf();
  return true;
}

// bf16 rows whose candidates (l >= l_cut) take at most kExactBins distinct values -- the usual
// case, the candidates lying within a few binades of the row maximum -- are settled from one count
// per value.  Bin b counts the tokens whose bf16 order key is khi - b, khi the key of the maximum
// (-0 and +0 are one value: the bin of -0 is merged into that of +0).
__device__ inline bool exact_window(float lmax, float l_cut, uint32_t& khi) {
  khi = order_key16((uint16_t)(__float_as_uint(lmax + 0.f) >> 16));
  if (!(l_cut > -__builtin_huge_valf())) return false;
  // every candidate has a key of at least klo: truncating l_cut to bf16 moves it down for
  // l_cut > 0 and up by less than one bf16 step for l_cut < 0
  const uint32_t kt = order_key16((uint16_t)(__float_as_uint(l_cut) >> 16));
  const uint32_t klo = kt > 0 ? kt - 1 : 0;
  return khi >= klo && khi - klo < (uint32_t)kExactBins;
}

// Threshold and kept mass from the per-value counts (count_of(b) for bins 0 .. kExactBins-1; a bin
// may also count tokens below l_cut, which take no part).  A value's mass is its count times the
// same fixed-point pi that the radix select adds token by token, so both reach the same integers.
template <class CountOf>
__device__ __attribute__((always_inline)) void settle_exact(CountOf count_of, int64_t row,
                                                            float lmax, const ToppSetup& st,
                                                            float c, float pi_min, uint32_t khi,
                                                            ToppStat* __restrict__ topp) {
  __shared__ unsigned long long s_wtot[kThreads / 64];
  __shared__ unsigned long long s_kept;
  __shared__ int s_bin, s_lowest;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) {
    s_bin = -1;
    s_lowest = -1;
  }
  __syncthreads();  // also: every count is in place

  // the mass of every value, then each thread's run of kPerThread consecutive bins
  constexpr int kPerThread = kExactBins / kThreads;
  const int b0 = threadIdx.x * kPerThread;
  unsigned long long w[kPerThread], s = 0;
  int lowest = -1;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int b = b0 + j;
    w[j] = 0;
    if ((uint32_t)b <= khi) {
      const uint32_t key = khi - (uint32_t)b;
      uint32_t n = 0;
      if (key != 0x7fffu) {  // -0 is counted with +0
        n = count_of(b);
        if (key == 0x8000u && b + 1 < kExactBins) n += count_of(b + 1);
      }
      const float l = key16_to_float(key);
      if (n != 0u && l >= st.l_cut) {
        const float pi = __builtin_amdgcn_exp2f((l - lmax) * c) * st.invZ;
        if (pi >= pi_min && pi != 0.f)
          w[j] = (unsigned long long)n * (unsigned long long)((double)pi * 0x1.0p56);
      }
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
  if ((double)pre < st.target) {
    unsigned long long run = pre;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if ((double)(run + w[j]) >= st.target) {
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

// One read of the row: the count of every candidate value, one histogram per wave.
__device__ __attribute__((always_inline)) void count_candidates_bf16(
    const RowSet& rs, const bf16_t* __restrict__ rp, int vec_ok, float l_cut, uint32_t khi,
    uint32_t* __restrict__ cnt) {
  const int wave = threadIdx.x >> 6;
  for (int k = threadIdx.x; k < (kThreads / 64) * kExactBins; k += kThreads) cnt[k] = 0u;
  __syncthreads();
  uint32_t* mine = cnt + wave * kExactBins;
  auto count = [&](bf16_t e) {
    if (to_f32(e) >= l_cut) {
      const uint32_t bin = khi - order_key16(e.bits);
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
}

// ---------------------------------------------------------------------------------------------
// Rows outside the exact window (fp32 rows, flat bf16 rows): a mass-weighted radix select over
// the order keys of the logits, 8 bits per round (2 rounds for bf16, 4 for fp32), one read of the
// row per round.  Candidates (few percent of the tokens, crowding into a few bins) are compacted
// per wave into an LDS queue and processed 64 at a time, so the exp and the histogram atomics run
// on full waves instead of on the scattered lanes of every token.
// ---------------------------------------------------------------------------------------------
template <typename T>
__device__ __attribute__((always_inline)) void topp_radix(
    const RowSet& rs, int64_t row, const T* __restrict__ rp, int vec_ok, float lmax,
    const ToppSetup& st, float c, float pi_min, ToppStat* __restrict__ topp,
    unsigned char* __restrict__ buf) {
  constexpr bool kHalf = sizeof(T) == 2;
  constexpr int kKeyBits = kHalf ? 16 : 32;
  constexpr int kRounds = kKeyBits / 8;
  // one histogram per wave, summed in wave order, then the candidate queues
  unsigned long long(*hist)[256] = reinterpret_cast<unsigned long long(*)[256]>(buf);
  float(*s_cand)[kCandQueue] = reinterpret_cast<float(*)[kCandQueue]>(
      buf + sizeof(unsigned long long) * 256 * (kThreads / 64));
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_above, s_kept;
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_above = 0;
    s_kept = 0;
  }
  const float invZ = st.invZ, l_cut = st.l_cut;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int E = 16 / (int)sizeof(T);
  const int nvec = vec_ok ? rs.V / E : 0;
  for (int round = 0; round < kRounds; ++round) {
    const int shift = kKeyBits - 8 * (round + 1);
    for (int w = 0; w < kThreads / 64; ++w) hist[w][threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
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
        if ((double)(run + hist[0][b]) >= st.target) break;
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

constexpr int kRadixBytes = (int)(sizeof(unsigned long long) * 256 + sizeof(float) * kCandQueue) *
                            (kThreads / 64);
constexpr int kCountBytes = (int)sizeof(uint32_t) * kExactBins * (kThreads / 64);
constexpr int kToppBuf = kRadixBytes > kCountBytes ? kRadixBytes : kCountBytes;

// The nucleus of every row after the row pass (statistics from its per-chunk pairs, or combined).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_topp(RowSet rs, int nchunk, float c, double top_p,
                                                   float pi_min, const float2* __restrict__ part,
                                                   ToppStat* __restrict__ topp,
                                                   const RowStat* __restrict__ pre, int vec_ok) {
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kToppBuf];
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
  ToppSetup st;
  if (!topp_setup(lmax, Z, c, top_p, pi_min, row, topp, st)) return;
  if constexpr (sizeof(T) == 2) {
    uint32_t khi;
    if (exact_window(lmax, st.l_cut, khi)) {
      uint32_t* cnt = reinterpret_cast<uint32_t*>(s_buf);
      count_candidates_bf16(rs, rp, vec_ok, st.l_cut, khi, cnt);
      settle_exact(
          [&](int b) {
            uint32_t n = 0;
            for (int w = 0; w < kThreads / 64; ++w) n += cnt[w * kExactBins + b];
            return n;
          },
          row, lmax, st, c, pi_min, khi, topp);
      return;
    }
  }
  topp_radix<T>(rs, row, rp, vec_ok, lmax, st, c, pi_min, topp, s_buf);
}

// ---------------------------------------------------------------------------------------------
// Row pass and nucleus in one read (bf16, one workgroup per row).  Beside the online (max, sum of
// exp) pair of every lane, each wave counts its positive tokens per bf16 value in a window of
// kExactBins keys below the wave's running maximum m_w, anchored anew (the counts shifted along)
// when that maximum rises.  A token is counted when it lies above the wave's running bound
//   g(m_w) = m_w + log2(pi_min) / c - 2e-3 (1 + |m_w|)
// and inside the window.  g never exceeds the row's l_cut (g rises with m_w, m_w <= lmax, Z >= 1
// and l_cut carries a margin of 1e-3 (1 + |lmax|)), so when l_cut > 0 and the row's candidates fit
// the window below lmax, every candidate was counted, once.  The row's pair goes to the workspace
// as its one chunk.  Other rows read the row again for the radix select.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_rowstats_topp(RowSet rs, float c, double top_p,
                                                            float pi_min,
                                                            float2* __restrict__ part,
                                                            ToppStat* __restrict__ topp,
                                                            int vec_ok) {
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kToppBuf];
  __shared__ uint32_t s_khw[kThreads / 64];
  __shared__ float2 s_pair;
  const int64_t row = blockIdx.x;
  if (row_skipped(rs, row)) return;
  const bf16_t* rp = row_ptr<bf16_t>(rs, row);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(s_buf);
  for (int k = threadIdx.x; k < (kThreads / 64) * kExactBins; k += kThreads) cnt[k] = 0u;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* mine = cnt + wave * kExactBins;
  const double drop = log2((double)pi_min) / (double)c;  // pi_min > 0 on this path
  float m = kNegBig, s = 0.f;  // the lane's online pair
  // the wave's anchor (wave-uniform): its value and key, the lowest counted value and the bin
  // offset kp (a counted token of bits b goes to bin kp - b)
  float mw = kNegBig, cut_f = __builtin_huge_valf();
  uint32_t khw = 0, kp = 0;

  // Raise the anchor to the wave's running maximum, shifting the counts along (the first anchor
  // clears them); a ballot finds the rare steps in which some lane passed it.  Only positive tokens
  // are counted (the exact window is used for rows whose l_cut is positive), down to the highest
  // of g(m_w), the smallest positive bf16 and the bottom of the window.
  auto anchor = [&]() __attribute__((always_inline)) {
    if (__ballot(m > mw) == 0ull) return;
    float wm = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, 64));
    wm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wm)));  // uniform: a scalar
    const uint32_t kn = order_key16((uint16_t)(__float_as_uint(wm + 0.f) >> 16));
    const uint32_t d = mw > kNegBig ? kn - khw : (uint32_t)kExactBins;
    // 64 bins at a time from the top: a block's sources lie below the bins already written, and
    // within a block every lane reads before any lane writes (one instruction each)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int k = kExactBins / 64 - 1; k >= 0; --k) {
      const uint32_t b = (uint32_t)(k * 64 + lane);
      const uint32_t moved = b >= d ? mine[b - d] : 0u;
      mine[b] = moved;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    mw = wm;
    khw = kn;
    const float g = (float)((double)wm + drop - 2e-3 * (1.0 + fabs((double)wm)));
    uint32_t klow = order_key16((uint16_t)(__float_as_uint(g) >> 16));
    klow = klow > 0 ? klow - 1 : 0;
    klow = max(klow, 0x8001u);
    if (kn >= (uint32_t)kExactBins) klow = max(klow, kn - (uint32_t)(kExactBins - 1));
    if (klow <= kn) {
      cut_f = key16_to_float(klow);
      kp = kn - 0x8000u;
    } else {
      cut_f = __builtin_huge_valf();
    }
  };

  constexpr int E = 8;
  // one step over U vectors: lane maximum and rescale, anchor, counts, then the sum of exps
  auto step = [&](const u32x4* v, int U) __attribute__((always_inline)) {
    float mn = m;
    for (int u = 0; u < U; ++u) {
      float f[E];
      Elems<bf16_t>::unpack(v[u], f);
#pragma unroll
      for (int j = 0; j < E; ++j) mn = fmaxf(mn, f[j]);
    }
    s *= __builtin_amdgcn_exp2f((m - mn) * c);  // 1 when the maximum did not move
    m = mn;
    anchor();
    float acc = 0.f;
    for (int u = 0; u < U; ++u) {
      float f[E];
      Elems<bf16_t>::unpack(v[u], f);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (f[2 * e] >= cut_f) atomicAdd(&mine[kp - (v[u][e] & 0xffffu)], 1u);
        if (f[2 * e + 1] >= cut_f) atomicAdd(&mine[kp - (v[u][e] >> 16)], 1u);
      }
#pragma unroll
      for (int j = 0; j < E; ++j) acc += __builtin_amdgcn_exp2f((f[j] - m) * c);
    }
    s += acc;
  };

  const int nvec = vec_ok ? rs.V / E : 0;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp);
  int i = threadIdx.x;
  // the loop bounds are the same for every lane of a wave (the anchor is a wave reduction)
  for (; i - lane + 63 + (kFusedUnroll - 1) * kThreads < nvec; i += kFusedUnroll * kThreads) {
    u32x4 v[kFusedUnroll];
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) v[u] = __builtin_nontemporal_load(vp + i + u * kThreads);
    step(v, kFusedUnroll);
  }
  // the rest, a token past the row being -inf (no mass, never counted)
  const u32x4 pad = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
  const int nvec_w = (nvec + kThreads - 1) / kThreads * kThreads;
  for (; i < nvec_w; i += kThreads) {
    const u32x4 v[1] = {i < nvec ? __builtin_nontemporal_load(vp + i) : pad};
    step(v, 1);
  }
  const int tail = nvec * E;
  const int V_w = tail + (rs.V - tail + kThreads * E - 1) / (kThreads * E) * (kThreads * E);
  for (int x = tail + threadIdx.x * E; x < V_w; x += kThreads * E) {
    // eight tokens per lane, -inf past the row
    uint32_t wd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = x + 2 * e < rs.V ? (uint32_t)rp[x + 2 * e].bits : 0xff80u;
      const uint32_t hi = x + 2 * e + 1 < rs.V ? (uint32_t)rp[x + 2 * e + 1].bits : 0xff80u;
      wd[e] = lo | (hi << 16);
    }
    const u32x4 v[1] = {u32x4{wd[0], wd[1], wd[2], wd[3]}};
    step(v, 1);
  }
  if (lane == 0) s_khw[wave] = mw > kNegBig ? khw : 0xffffffffu;  // no anchor: nothing counted

  // the row's pair (its one chunk), then its statistics as every consumer of the pair forms them
  block_reduce_pair(m, s, c);
  if (threadIdx.x == 0) {
    s_pair = make_float2(m, s);
    part[row] = s_pair;
  }
  __syncthreads();
  float lmax;
  double Z;
  row_stats_from_parts(&s_pair, 0, 1, c, lmax, Z);
  ToppSetup st;
  if (!topp_setup(lmax, Z, c, top_p, pi_min, row, topp, st)) return;
  uint32_t khi;
  if (st.l_cut > 0.f && exact_window(lmax, st.l_cut, khi)) {  // every candidate counted
    settle_exact(
        [&](int b) {
          uint32_t n = 0;
          for (int w = 0; w < kThreads / 64; ++w) {
            const uint32_t kw = s_khw[w];
            if (kw == 0xffffffffu) continue;
            const int bw = b - (int)(khi - kw);  // the wave's bin of the same key
            if (bw >= 0) n += cnt[w * kExactBins + bw];
          }
          return n;
        },
        row, lmax, st, c, pi_min, khi, topp);
    return;
  }
  topp_radix<bf16_t>(rs, row, rp, vec_ok, lmax, st, c, pi_min, topp, s_buf);
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
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("topp", k_topp<bf16_t>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs,
                   nchunk, c, top_p, (float)pmin, part, topp, rowstat, vec_ok);
  else
    PSISPEC_LAUNCH("topp", k_topp<float>, dim3((unsigned)rows), dim3(kThreads), 0, stream, rs,
                   nchunk, c, top_p, (float)pmin, part, topp, rowstat, vec_ok);
  return hipGetLastError();
}

hipError_t launch_rowstats_topp(const RowSet& rs, float c, double top_p, float2* part,
                                ToppStat* topp, hipStream_t stream) {
  const int64_t rows = rs.nP + rs.nQ;
  if (rows == 0) return hipSuccess;
  const double pmin = (1.0 - top_p) / (4.0 * (double)rs.V);
  if (!(pmin >= 1e-30)) return hipErrorInvalidValue;
  const int vec_ok = ((size_t)rs.V * 2) % 16 == 0 && ((size_t)rs.pstride * 2) % 16 == 0 &&
                     ((uintptr_t)rs.p % 16) == 0 && ((uintptr_t)rs.q % 16) == 0;
  PSISPEC_LAUNCH("rowstats_topp", k_rowstats_topp, dim3((unsigned)rows), dim3(kThreads), 0, stream,
                 rs, c, top_p, (float)pmin, part, topp, vec_ok);
  return hipGetLastError();
}

}  // namespace psispec
