// drafts.hip -- the drafting step: one token per (request, position) drawn from its own row.
//
// [alphalab] walkthrough steps 1-2: the AR path samples the first token of the block and the
// diffusion path proposes the others in parallel.  Every drafted token is one inverse-CDF draw from
// its row after the temperature and the nucleus, because the verify divides by exactly that q'.
// Position 0 of the Uno layout comes from the request's AR row, every other position from its q
// row.  The Philox counter of a draw is (request, position, DRAFT, step).
//
// Bounded fp32 draw.  The exact fp64 pass of the verify's final draw costs about thirty fp64
// operations per token; most draws do not need it.  k_draft_bounds reads each row once in fp32:
// per sub-chunk of 1024 tokens the maximum kept logit m, s = sum of 2^((l - m) c) (hardware exp2,
// fp64 sum) and A = sum of |(l - m) c| 2^((l - m) c).  Every fp32 term has relative error below
//   kKappa1 |(l - m) c| (rounding of l - m, of c = log2(e) / T and of their product) + kKappa2
//   (the exp2 instruction; measured below 1.5 x 2^-24 over [-150, 0] on gfx950, flushing to 0
//   below 2^-126),
// so the sub-chunk mass in the row frame, exp((m - M) / T) s, is known within
//   e = exp((m - M) / T) (kKappa1 A + kKappa2 s + 1024 x 2^-126)  (+ fp64 rounding).
// k_draft_select sums the masses and bounds (fixed order), locates v = u S among the sub-chunks,
// and computes the exact fp64 weights of the chosen sub-chunk.  With E the total bound and E_P the
// bound of the sub-chunks before it, the offset of v in the sub-chunk is known within
// delta = u E + E_P; if no cumulative-weight breakpoint of the sub-chunk (nor its two ends) lies
// within delta of it, every value in that interval selects the same token, which is then the token
// of the exact computation.  Otherwise the draw is listed for the exact fp64 kernels of the
// verify's final draw, which then run over the listed draws only.
//
// With top-p the nucleus threshold comes first: the HBM row pass, k_draft_rows (per drafted token,
// the row statistics combined from the pass's per-chunk pairs, one wave, fixed order, and the
// description of its draw) and the nucleus kernel.
#include <limits.h>

#include "launch.h"
#include "decide.h"
#include "draw.h"

namespace psispec {
namespace {

__global__ __launch_bounds__(64) void k_draft_rows(RowSet rs, int B, int first_from_target,
                                                   const float2* __restrict__ part, int nchunk,
                                                   float c, RowStat* __restrict__ rowstat,
                                                   DrawDesc* __restrict__ desc) {
  const int j = blockIdx.x;  // drafted token r * B + i
  const int r = j / B, i = j - r * B;
  // position 0 of the Uno layout comes from the request's AR row (p rows, one per request)
  const int64_t row = (first_from_target && i == 0) ? (int64_t)r : rs.nP + (int64_t)j;
  float lmax;
  double Z;
  combine_row_wave(part + row * nchunk, nchunk, c, lmax, Z);
  if (threadIdx.x == 0) {
    const int st = row_status(lmax, Z);
    rowstat[row] = RowStat{lmax, st, Z};
    DrawDesc d;
    d.prow = (int32_t)row;
    d.qrow = -1;
    d.pos = i;
    d.st = st;
    d.nexcl = 0;
    d.out_idx = j;
    d.ph_req = r;
    d.purpose = kPurposeDraft;
    d.factor = 1.0;
    desc[j] = d;
  }
}

constexpr int kSubPerWave = 2;                              // sub-chunks a wave sums
constexpr int kSubPerBlock = kSubPerWave * (kThreads / 64);  // 8
constexpr float kKappa1 = 0x1.0p-22f;   // per unit |(l - m) c|: three roundings of 2^-24, times ln 2
constexpr float kKappa2 = 0x1.0p-22f;   // exp2 instruction, relative (measured < 1.5 x 2^-24)
constexpr double kFlushSub = 0x1.0p-116;  // 1024 terms that may flush to 0, each below 2^-126
constexpr float kClampT = 200.f;        // |t| cap in A (terms with |t| > 126 are 0 or flushed)

__device__ inline int64_t draft_row(const DraftArgs& a, int j) {
  const int r = j / a.B, i = j - r * a.B;
  return (a.first_from_target && i == 0) ? (int64_t)r : a.rs.nP + (int64_t)j;
}

// Block j * nblk + b sums sub-chunks 8b .. 8b+7 of drafted token j's row, two per wave (both
// loaded before either is summed).
template <typename T, bool kTopp>
__global__ __launch_bounds__(kThreads) void k_draft_bounds(DraftArgs a, int nblk, int vec_ok) {
  const int j = blockIdx.x / nblk;
  const int blk = blockIdx.x - j * nblk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = draft_row(a, j);
  const T* rp = row_ptr<T>(a.rs, row);
  float thr = -__builtin_huge_valf();
  if constexpr (kTopp) thr = a.topp[row].thr;
  const int sub0 = blk * kSubPerBlock + wave * kSubPerWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.count = 0;  // the select that follows appends to it
  float f[kSubPerWave][kPerLane];
#pragma unroll
  for (int u = 0; u < kSubPerWave; ++u)
    if (sub0 + u < a.nsub)
      load_run<T, kPerLane>(rp, (sub0 + u) * kSub + lane * kPerLane, a.V, vec_ok, f[u]);
#pragma unroll
  for (int u = 0; u < kSubPerWave; ++u) {
    const int sub = sub0 + u;
    if (sub >= a.nsub) break;
    float m = kNegBig;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      if constexpr (kTopp) {
        if (!(f[u][e] >= thr)) f[u][e] = -__builtin_huge_valf();  // outside the nucleus
      }
      m = fmaxf(m, f[u][e]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    double s = 0.0;
    float A = 0.f;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const float t = (f[u][e] - m) * a.c;  // <= 0; NaN for NaN or +inf logits (a bad row)
      const float w = __builtin_amdgcn_exp2f(t);
      s += (double)w;
      A = fmaf(fminf(-t, kClampT), w, A);
    }
    s = wave_sum(s);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) A += __shfl_xor(A, off, 64);
    if (lane == 0) a.rec[(int64_t)j * a.nsub + sub] = BoundRec{s, m, A};
  }
}

// One block per drafted token.
template <typename T, bool kTopp>
__global__ __launch_bounds__(kThreads) void k_draft_select(DraftArgs a) {
  __shared__ double tbl[kExpTable];
  __shared__ double s_mass[kMassLds];
  __shared__ double s_err[kMassLds];
  __shared__ double s_wave[kThreads / 64];
  __shared__ float s_max[kThreads / 64];
  __shared__ int s_pick[kThreads / 64], s_amb[kThreads / 64];
  __shared__ int s_sub;
  __shared__ double s_P, s_EP;
  exp_table_fill(tbl);
  const int j = blockIdx.x;
  const int r = j / a.B, i = j - r * a.B;
  const int64_t row = draft_row(a, j);
  const BoundRec* rec = a.rec + (int64_t)j * a.nsub;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // 1. the row's largest kept logit
  float M = kNegBig;
  for (int k = t; k < a.nsub; k += kThreads) M = fmaxf(M, rec[k].m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) s_max[wave] = M;
  if (t == 0) s_sub = -1;
  __syncthreads();
  M = s_max[0];
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, s_max[w]);

  // 2. sub-chunk masses and their error bounds in the frame of M
  for (int k = t; k < a.nsub; k += kThreads) {
    const BoundRec b = rec[k];
    const double sc = exp_tang(((double)b.m - (double)M) * a.inv_T, tbl);
    s_mass[k] = b.s * sc;
    s_err[k] = ((double)kKappa1 * 1.001 * (double)b.A + ((double)kKappa2 + 1e-13) * b.s +
                kFlushSub) * sc;
  }
  __syncthreads();

  // 3. each thread owns a contiguous run of sub-chunks; fixed-order block scans of mass and bound
  const int per = (a.nsub + kThreads - 1) / kThreads;
  const int j0 = min(a.nsub, t * per), j1 = min(a.nsub, j0 + per);
  double mine = 0.0, emine = 0.0;
  for (int k = j0; k < j1; ++k) {
    mine += s_mass[k];
    emine += s_err[k];
  }
  double lo, hi, elo, ehi;
  const double S = block_scan(mine, s_wave, &lo, &hi);
  const double E = block_scan(emine, s_wave, &elo, &ehi);
  int st = kTopp ? a.desc[j].st : 0;
  const bool finite_row = (M > kNegBig) && (M < __builtin_huge_valf()) && (S > 0.0) && (S < 1e300);
  if (!finite_row) {
    // NaN/+inf logits or no finite logit: the token is unspecified (0)
    if (t == 0) {
      a.out_tokens[j] = 0;
      if (a.status) a.status[j] = st | PSISPEC_ST_NONFINITE;
    }
    return;
  }
  const double u = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)i,
                                  kPurposeDraft, a.step);
  const double v = u * S;
  if (lo <= v && v < hi) {  // exactly one thread owns v
    double C = lo, CE = elo;
    int k = j0;
    for (; k < j1; ++k) {
      if (C + s_mass[k] > v) break;
      C += s_mass[k];
      CE += s_err[k];
    }
    if (k == j1) {  // rounding: the run ends before v; its last sub-chunk (the test below decides)
      --k;
      C -= s_mass[k];
      CE -= s_err[k];
    }
    s_sub = k;
    s_P = C;
    s_EP = CE;
  }
  __syncthreads();
  const int sub = s_sub;
  int amb = sub < 0;  // v rounded to S: left to the exact pass
  int tok = INT_MAX;
  if (sub >= 0) {
    // 4. exact fp64 weights of the chosen sub-chunk (4 tokens per thread) and the breakpoint test
    const double delta = 1.01 * (u * E + s_EP) + 1e-12 * S;
    const double rin = v - s_P;
    const T* rp = row_ptr<T>(a.rs, row);
    const float thr = kTopp ? a.topp[row].thr : -__builtin_huge_valf();
    const int x0 = sub * kSub + t * 4;
    float fl[4];
    load_run<T, 4>(rp, x0, a.V, false, fl);
    double w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = term(fl[e], M, thr, a.inv_T, tbl);
    double l0, h0;
    const double W = block_scan(w[0] + w[1] + w[2] + w[3], s_wave, &l0, &h0);
    double C = l0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      C += w[e];
      if (w[e] > 0.0) {
        if (fabs(C - rin) <= delta) amb = 1;
        if (C > rin && tok == INT_MAX) tok = x0 + e;
      }
    }
    if (rin - delta < 0.0 || rin + delta >= W) amb = 1;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    tok = min(tok, __shfl_xor(tok, off, 64));
    amb = max(amb, __shfl_xor(amb, off, 64));
  }
  if (lane == 0) {
    s_pick[wave] = tok;
    s_amb[wave] = amb;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 0; w < kThreads / 64; ++w) {
      tok = min(tok, s_pick[w]);
      amb = max(amb, s_amb[w]);
    }
    if (!amb && tok != INT_MAX) {
      a.out_tokens[j] = tok;
      if (a.status) a.status[j] = st;
    } else {
      a.list[atomicAdd(a.count, 1)] = j;
      if (!kTopp) {  // with top-p the row pass and k_draft_rows wrote both already
        a.rowstat[row] = RowStat{M, st, 0.0};
        DrawDesc d;
        d.prow = (int32_t)row;
        d.qrow = -1;
        d.pos = i;
        d.st = st;
        d.nexcl = 0;
        d.out_idx = j;
        d.ph_req = r;
        d.purpose = kPurposeDraft;
        d.factor = 1.0;
        a.desc[j] = d;
      }
    }
  }
}

}  // namespace

hipError_t launch_draft_bounded(const DraftArgs& a, psispec_dtype dtype, hipStream_t stream) {
  const int64_t jobs = (int64_t)a.batch * a.B;
  if (jobs == 0) return hipSuccess;
  const int nblk = (a.nsub + kSubPerBlock - 1) / kSubPerBlock;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)a.V * es) % 16 == 0 && ((size_t)a.rs.pstride * es) % 16 == 0 &&
                     ((uintptr_t)a.rs.p % 16) == 0 && ((uintptr_t)a.rs.q % 16) == 0;
  const dim3 grid((unsigned)(jobs * nblk)), block(kThreads);
  if (dtype == PSISPEC_BF16) {
    if (a.use_topp)
      PSISPEC_LAUNCH("draft_bounds", (k_draft_bounds<bf16_t, true>), grid, block, 0, stream, a,
                     nblk, vec_ok);
    else
      PSISPEC_LAUNCH("draft_bounds", (k_draft_bounds<bf16_t, false>), grid, block, 0, stream, a,
                     nblk, vec_ok);
  } else {
    if (a.use_topp)
      PSISPEC_LAUNCH("draft_bounds", (k_draft_bounds<float, true>), grid, block, 0, stream, a, nblk,
                     vec_ok);
    else
      PSISPEC_LAUNCH("draft_bounds", (k_draft_bounds<float, false>), grid, block, 0, stream, a,
                     nblk, vec_ok);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sgrid((unsigned)jobs);
  if (dtype == PSISPEC_BF16) {
    if (a.use_topp)
      PSISPEC_LAUNCH("draft_select", (k_draft_select<bf16_t, true>), sgrid, block, 0, stream, a);
    else
      PSISPEC_LAUNCH("draft_select", (k_draft_select<bf16_t, false>), sgrid, block, 0, stream, a);
  } else {
    if (a.use_topp)
      PSISPEC_LAUNCH("draft_select", (k_draft_select<float, true>), sgrid, block, 0, stream, a);
    else
      PSISPEC_LAUNCH("draft_select", (k_draft_select<float, false>), sgrid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_draft_rows(const RowSet& rs, int batch, int B, int first_from_target,
                             const float2* part, int nchunk, float c, RowStat* rowstat,
                             DrawDesc* desc, hipStream_t stream) {
  const int64_t jobs = (int64_t)batch * B;
  if (jobs == 0) return hipSuccess;
  PSISPEC_LAUNCH("draft_rows", k_draft_rows, dim3((unsigned)jobs), dim3(64), 0, stream, rs, B,
                 first_from_target, part, nchunk, c, rowstat, desc);
  return hipGetLastError();
}

}  // namespace psispec
