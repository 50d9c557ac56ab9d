// decide.h -- device code of the linear accept test, shared by its kernel and the fused verify.
#pragma once

#include "launch.h"

namespace psispec {
namespace {

constexpr int kMaxB = 64;
constexpr int kStagePairs = (2 * kMaxB + 1) * 16;  // row pairs of a request staged in LDS

__device__ inline int row_status(float lmax, double Z) {
  const bool ok = (lmax > kNegBig) && (lmax < __builtin_huge_valf()) && (Z > 0.0) && (Z < 1e300);
  return ok ? 0 : PSISPEC_ST_NONFINITE;
}

// Statistics of one row from its per-chunk pairs, reduced by one wave64 in a fixed order: lane l
// takes chunks l, l+64, ...; then a butterfly.  Every lane returns the row's (lmax, Z).
__device__ inline void combine_row_wave(const float2* pr, int nchunk, float c, float& lmax,
                                        double& Z) {
  const int t = threadIdx.x & 63;
  lmax = kNegBig;
  for (int k = t; k < nchunk; k += 64) lmax = fmaxf(lmax, pr[k].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
  Z = 0.0;
  for (int k = t; k < nchunk; k += 64)
    Z += (double)pr[k].y * exp2((double)(pr[k].x - lmax) * (double)c);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Z += __shfl_xor(Z, off, 64);
}

// Accept test and first-rejection scan of request r (wave 0 of the calling block does the work;
// every thread of the block must call it: it contains one block barrier).
template <typename T>
__device__ inline void decide_linear_request(const LinearArgs& a, int r) {
  const int t = threadIdx.x;
  const int B = a.B, Bp1 = a.B + 1, V = a.V;
  const int64_t prow0 = (int64_t)r * Bp1;
  const int64_t qrow0 = a.rs.nP + (int64_t)r * B;
  const bool first_from_target = (a.flags & PSISPEC_FIRST_FROM_TARGET) != 0;

  __shared__ float s_lmax[2 * kMaxB + 1];
  __shared__ double s_Z[2 * kMaxB + 1];
  __shared__ int s_st[2 * kMaxB + 1];
  __shared__ float2 s_pair[kStagePairs];
  // a row's statistics: to the workspace (unless quiet) and to the caller's LDS copy (local row j)
  auto put_stat = [&](int j, int64_t row, const RowStat& rs) {
    if (!a.quiet) a.rowstat[row] = rs;
    if (a.rowstat_local) a.rowstat_local[j] = rs;
  };

  // 1. finish the row statistics (rows 0..B of p, then rows 0..B-1 of q).  When the request's pairs
  //    fit in LDS: one lane per row; else (LM-head column tiles at large B) the wave reduces each
  //    row's chunks in a fixed order.
  if (t >= 64) {
    // other waves of a larger block only join the barrier
  } else if (a.rowstat_ready) {
    // statistics already combined (one wave per row, by combine_row_wave)
    for (int j = t; j < 2 * B + 1; j += 64) {
      const int64_t row = j <= B ? prow0 + j : qrow0 + (j - Bp1);
      if (j > B && first_from_target && j == Bp1) {
        s_lmax[j] = 0.f;
        s_Z[j] = 1.0;
        s_st[j] = 0;
        continue;
      }
      const RowStat rw = a.rowstat[row];
      s_lmax[j] = rw.lmax;
      s_Z[j] = rw.Z;
      s_st[j] = rw.st;
      if (a.rowstat_local) a.rowstat_local[j] = rw;
    }
  } else if ((2 * B + 1) * a.nchunk <= kStagePairs) {
    // the request's pairs: p rows then q rows, each a contiguous run of the workspace, loaded by
    // the whole wave in one round
    const int np = Bp1 * a.nchunk, nq = B * a.nchunk;
    for (int i = t; i < np + nq; i += 64)
      s_pair[i] = i < np ? a.part[prow0 * a.nchunk + i] : a.part[qrow0 * a.nchunk + (i - np)];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int j = t; j < 2 * B + 1; j += 64) {
      const int64_t row = j <= B ? prow0 + j : qrow0 + (j - Bp1);
      if (j > B && first_from_target && j == Bp1) {
        s_lmax[j] = 0.f;
        s_Z[j] = 1.0;
        s_st[j] = 0;
        continue;
      }
      const float2* pr = s_pair + j * a.nchunk;
      float lmax = kNegBig;
      for (int k = 0; k < a.nchunk; ++k) lmax = fmaxf(lmax, pr[k].x);
      double Z = 0.0;
      for (int k = 0; k < a.nchunk; ++k) {
        const float2 pk = pr[k];
        Z += (double)pk.y * exp2((double)(pk.x - lmax) * (double)a.c);
      }
      const int st = row_status(lmax, Z);
      s_lmax[j] = lmax;
      s_Z[j] = Z;
      s_st[j] = st;
      put_stat(j, row, RowStat{lmax, st, Z});
    }
  } else {
    for (int j = 0; j < 2 * B + 1; ++j) {
      const int64_t row = j <= B ? prow0 + j : qrow0 + (j - Bp1);
      if (j > B && first_from_target && j == Bp1) {
        if (t == 0) {
          s_lmax[j] = 0.f;
          s_Z[j] = 1.0;
          s_st[j] = 0;
        }
        continue;
      }
      float lmax;
      double Z;
      combine_row_wave(a.part + row * a.nchunk, a.nchunk, a.c, lmax, Z);
      if (t == 0) {
        const int st = row_status(lmax, Z);
        s_lmax[j] = lmax;
        s_Z[j] = Z;
        s_st[j] = st;
        put_stat(j, row, RowStat{lmax, st, Z});
      }
    }
  }
  __syncthreads();
  if (t >= 64) return;

  // 2. ratio and accept bit of position t
  int st = 0;
  for (int j = t; j < 2 * B + 1; j += 64) st |= s_st[j];
  bool acc = false;
  int32_t d = -1;
  if (t < B) {
    d = a.draft[(int64_t)r * B + t];
    double ratio;
    const bool bad_tok = d < 0 || d >= V;
    if (bad_tok) st |= PSISPEC_ST_BAD_TOKEN;
    if (first_from_target && t == 0) {
      ratio = 1.0;  // the AR's own sample: always kept ([alphalab] walkthrough step 1)
    } else if (bad_tok) {
      ratio = 0.0;
    } else {
      float lp, lq;
      if (a.gath) {
        lp = a.gath[prow0 + t];
        lq = a.gath[qrow0 + t];
      } else {
        lp = to_f32(row_ptr<T>(a.rs, prow0 + t)[d]);
        lq = to_f32(row_ptr<T>(a.rs, qrow0 + t)[d]);
      }
      double pa = exp(((double)lp - (double)s_lmax[t]) * a.inv_T) / s_Z[t];
      double qb = exp(((double)lq - (double)s_lmax[Bp1 + t]) * a.inv_T) / s_Z[Bp1 + t];
      if (a.use_topp) {
        const ToppStat tp = a.topp[prow0 + t];
        const ToppStat tq = a.topp[qrow0 + t];
        pa = lp >= tp.thr ? pa / tp.M : 0.0;
        qb = lq >= tq.thr ? qb / tq.M : 0.0;
      }
      if (qb > 0.0) {
        ratio = fmin(1.0, pa / qb);
      } else {
        ratio = pa > 0.0 ? 1.0 : 0.0;
        st |= PSISPEC_ST_Q_ZERO;
      }
    }
    const double u = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)t,
                                     kPurposeAccept, a.step);
    acc = u < ratio;
    if (a.ratios && !a.quiet) a.ratios[(int64_t)r * B + t] = (float)ratio;
  }
  const uint64_t mask = __ballot(acc);
  const uint64_t full = B == 64 ? ~0ull : ((1ull << B) - 1ull);
  const int k = (mask & full) == full ? B : __builtin_ctzll(~mask);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) st |= __shfl_xor(st, off, 64);

  // 3. kept prefix; slot k is filled by the final draw, later slots are discarded (-1)
  if (!a.quiet) {
    if (t < B) a.out_tokens[(int64_t)r * Bp1 + t] = t < k ? d : -1;
    if (t == 0) a.out_tokens[(int64_t)r * Bp1 + B] = -1;  // block-end slot: the draw fills it if k == B
  }
  if (t == 0) {
    if (!a.quiet) {
      a.accept_len[r] = k;
      if (a.accept_mask) a.accept_mask[r] = mask & full;
    }
    DrawDesc dd;
    dd.prow = (int32_t)(prow0 + k);
    dd.qrow = k < B ? (int32_t)(qrow0 + k) : -1;
    dd.pos = k;
    dd.st = st;
    dd.nexcl = 0;
    dd.out_idx = (int32_t)((int64_t)r * Bp1 + k);
    dd.ph_req = r;
    dd.purpose = kPurposeDraw;
    dd.factor = 1.0;
    if (!a.quiet) a.desc[r] = dd;
    if (a.desc_local) *a.desc_local = dd;
  }
}


}  // namespace
}  // namespace psispec
