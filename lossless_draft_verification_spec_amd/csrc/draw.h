// draw.h -- device code of the fp64 final draw, shared by its kernels and the fused verify.
#pragma once

#include "launch.h"

namespace psispec {
namespace {

constexpr int kPerLane = kSub / 64;  // tokens per lane in k_draw_weights (16)

// Load n consecutive logits starting at x0 (x0 a multiple of n); tokens past V read as -inf.
// Whole 16-byte vectors when the row allows it, else element by element.
template <typename T, int n>
__device__ inline void load_run(const T* row, int x0, int V, bool vec_ok, float (&f)[n]) {
  constexpr int E = 16 / (int)sizeof(T);
  if constexpr (n % E == 0) {
    if (vec_ok && x0 + n <= V) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(row + x0);
#pragma unroll
      for (int v = 0; v < n / E; ++v) {
        const u32x4 w = vp[v];
        if constexpr (sizeof(T) == 2) {
          f[8 * v + 0] = __uint_as_float(w.x << 16);
          f[8 * v + 1] = __uint_as_float(w.x & 0xffff0000u);
          f[8 * v + 2] = __uint_as_float(w.y << 16);
          f[8 * v + 3] = __uint_as_float(w.y & 0xffff0000u);
          f[8 * v + 4] = __uint_as_float(w.z << 16);
          f[8 * v + 5] = __uint_as_float(w.z & 0xffff0000u);
          f[8 * v + 6] = __uint_as_float(w.w << 16);
          f[8 * v + 7] = __uint_as_float(w.w & 0xffff0000u);
        } else {
          f[4 * v + 0] = __uint_as_float(w.x);
          f[4 * v + 1] = __uint_as_float(w.y);
          f[4 * v + 2] = __uint_as_float(w.z);
          f[4 * v + 3] = __uint_as_float(w.w);
        }
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < n; ++e) f[e] = (x0 + e < V) ? to_f32(row[x0 + e]) : -__builtin_huge_valf();
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ inline int wave_max(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

struct RowView {
  float lmax_p, thr_p, lmax_q, thr_q;
};

__device__ inline RowView row_view(const DrawArgs& a, const DrawDesc& d) {
  RowView v;
  v.lmax_p = a.rowstat[d.prow].lmax;
  v.thr_p = a.use_topp ? a.topp[d.prow].thr : -__builtin_huge_valf();
  if (d.qrow >= 0) {
    v.lmax_q = a.rowstat[d.qrow].lmax;
    v.thr_q = a.use_topp ? a.topp[d.qrow].thr : -__builtin_huge_valf();
  } else {
    v.lmax_q = 0.f;
    v.thr_q = 0.f;
  }
  return v;
}

// exp((l - lmax) / T) for a kept token, 0 outside the nucleus (and for l = -inf or NaN): 2^(t/256)
// with t = l c256 - lmax c256 by one fused multiply-add (c256 and lmax c256 are loop invariants).
// kTopp = false skips the nucleus test (thr = -inf keeps every finite logit).
template <bool kTopp = true>
__device__ inline double term(float l, float lmax, float thr, double inv_T, const double* tbl) {
  const double c256 = inv_T * k256Log2e;
  const double e = exp2_256(fma((double)l, c256, -((double)lmax * c256)), tbl);
  if constexpr (!kTopp) return e;
  return l >= thr ? e : 0.0;
}

constexpr double kBand = 1e-5;  // relative band of uncertain residual signs
constexpr int kEsLds = 512;     // chunk normaliser pairs staged in LDS by the select

__device__ inline bool excluded(int x, const int* excl, int nexcl) {
  for (int i = 0; i < nexcl; ++i)
    if (excl[i] == x) return true;
  return false;
}

// factor E_p / E_q as estimated from the HBM pass's normalisers (sums over the kept tokens): the
// residual max(0, p' - factor q') is positive where e_p > rho e_q, rho = factor E_p / E_q
__device__ inline double rho_estimate(const DrawArgs& a, const DrawDesc& d) {
  double ep = a.rowstat[d.prow].Z, eq = a.rowstat[d.qrow].Z;
  if (a.use_topp) {
    ep *= a.topp[d.prow].M;
    eq *= a.topp[d.qrow].M;
  }
  return d.factor * ep / eq;
}

// Draw chunk c of request r (every thread of a kThreads block calls it).
template <typename T, bool kTopp>
__device__ inline void draw_pass_task(const DrawArgs& a, int r, int c, int vec_ok) {
  __shared__ double tbl[kExpTable];
  __shared__ int s_excl[1024];
  __shared__ double2 s_part[kThreads / 64];
  exp_table_fill(tbl);
  const DrawDesc d = a.desc[r];
  const RowView v = row_view(a, d);
  const T* prow = row_ptr<T>(a.rs, d.prow);
  const bool has_q = d.qrow >= 0;
  const T* qrow = has_q ? row_ptr<T>(a.rs, d.qrow) : nullptr;
  const int nexcl = has_q ? 0 : min(d.nexcl, 1024);
  for (int i = threadIdx.x; i < nexcl; i += kThreads)
    s_excl[i] = a.excl[(int64_t)r * a.excl_stride + i];
  const double rho = has_q ? rho_estimate(a, d) : 0.0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub_per_chunk = a.chunk_elems_draw / kSub;
  double Ep = 0.0, Eq = 0.0;
  for (int j = wave; j < sub_per_chunk; j += kThreads / 64) {
    const int sub = c * sub_per_chunk + j;
    if (sub >= a.nsub) break;
    const int x0 = sub * kSub + lane * kPerLane;
    float fp[kPerLane], fq[kPerLane];
    load_run<T, kPerLane>(prow, x0, a.V, vec_ok, fp);
    double Ap = 0.0, Aq = 0.0;
    int unc = 0;
    uint32_t umask = 0;
    if (has_q) {
      load_run<T, kPerLane>(qrow, x0, a.V, vec_ok, fq);
      // four tokens' fp64 chains at a time: fewer VGPRs than a full unroll, more waves per SIMD
#pragma unroll 4
      for (int e = 0; e < kPerLane; ++e) {
        const double ep = term<kTopp>(fp[e], v.lmax_p, v.thr_p, a.inv_T, tbl);
        const double eq = term<kTopp>(fq[e], v.lmax_q, v.thr_q, a.inv_T, tbl);
        Ep += ep;
        Eq += eq;
        const double diff = ep - rho * eq, band = kBand * (ep + rho * eq);
        if (diff > band) {
          Ap += ep;
          Aq += eq;
        } else if (diff >= -band && ep > 0.0) {
          ++unc;
          umask |= 1u << e;
        }
      }
      // pack this sub-chunk's uncertain tokens, in token order, into one pool segment
      int before = unc;  // inclusive prefix over lanes, then made exclusive
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(before, off, 64);
        if (lane >= off) before += y;
      }
      const int total = __shfl(before, 63, 64);
      before -= unc;
      int seg = -1;
      if (total > 0) {
        if (lane == 0) seg = atomicAdd(a.ucount + r, total);
        seg = __shfl(seg, 0, 64);
        if (seg + total > kUncPool) seg = -1;  // pool full: this sub-chunk is summed token by token
        if (seg >= 0 && umask) {
          double2* dst = a.upool + (int64_t)r * kUncPool + seg + before;
          // the few uncertain tokens re-read their logits (cached): no register copy of the run
          for (uint32_t m = umask; m; m &= m - 1) {
            const int x = x0 + __builtin_ctz(m);
            *dst++ = make_double2(term<kTopp>(to_f32(prow[x]), v.lmax_p, v.thr_p, a.inv_T, tbl),
                                  term<kTopp>(to_f32(qrow[x]), v.lmax_q, v.thr_q, a.inv_T, tbl));
          }
        }
      }
      if (lane == 0) a.suboff[(int64_t)r * a.nsub + sub] = seg;
    } else {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        double ep = term<kTopp>(fp[e], v.lmax_p, v.thr_p, a.inv_T, tbl);
        if (nexcl && excluded(x0 + e, s_excl, nexcl)) ep = 0.0;
        Ap += ep;
      }
    }
    Ap = wave_sum(Ap);
    Aq = wave_sum(Aq);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) unc += __shfl_xor(unc, off, 64);
    if (lane == 0) {
      a.suba[(int64_t)r * a.nsub + sub] = make_double2(Ap, Aq);
      a.subn[(int64_t)r * a.nsub + sub] = unc;
    }
  }
  if (!has_q) return;
  Ep = wave_sum(Ep);
  Eq = wave_sum(Eq);
  if (lane == 0) s_part[wave] = make_double2(Ep, Eq);
  __syncthreads();
  if (threadIdx.x == 0) {
    double sp = 0.0, sq = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) {
      sp += s_part[w].x;
      sq += s_part[w].y;
    }
    a.esum[(int64_t)r * a.nchunk_draw + c] = make_double2(sp, sq);
  }
}

// Fixed-order scan of one double per thread across the block.  Returns the exclusive prefix in
// *lo and the inclusive prefix in *hi with hi of thread t bit-identical to lo of thread t+1, so
// the intervals [lo, hi) tile [0, total) exactly; returns the block total.
__device__ inline double block_scan(double x, double* s_wave, double* lo, double* hi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  __syncthreads();
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  double off_w = 0.0;
  for (int k = 0; k < wave; ++k) off_w += s_wave[k];
  double tot = off_w;
  for (int k = wave; k < kThreads / 64; ++k) tot += s_wave[k];
  *lo = off_w + excl;
  *hi = off_w + incl;
  return tot;
}

// Weights of the 4 consecutive tokens x0..x0+3 (one thread's share of a sub-chunk).
//   mode 0: residual max(0, e_p rEp - e_q rEq);  mode 1: e_p with removed tokens;  mode 2: e_p.
template <typename T>
__device__ inline void weights4(const T* prow, const T* qrow, int x0, int V, const RowView& v,
                                int mode, double rEp, double rEq, double inv_T, const double* tbl,
                                const int* excl, int nexcl, double (&w)[4]) {
  float fp[4], fq[4];
  load_run<T, 4>(prow, x0, V, false, fp);
  if (mode == 0) load_run<T, 4>(qrow, x0, V, false, fq);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double ep = term(fp[e], v.lmax_p, v.thr_p, inv_T, tbl);
    if (mode == 0) {
      const double x = ep * rEp - term(fq[e], v.lmax_q, v.thr_q, inv_T, tbl) * rEq;
      w[e] = x > 0.0 ? x : 0.0;
    } else if (mode == 1) {
      w[e] = (nexcl && excluded(x0 + e, excl, nexcl)) ? 0.0 : ep;
    } else {
      w[e] = ep;
    }
  }
}

template <typename T>
__device__ inline double subchunk_mass(const T* prow, const T* qrow, int sub, int V,
                                       const RowView& v, int mode, double rEp, double rEq,
                                       double inv_T, const double* tbl, const int* excl, int nexcl,
                                       double* s_wave) {
  double w[4];
  weights4<T>(prow, qrow, sub * kSub + threadIdx.x * 4, V, v, mode, rEp, rEq, inv_T, tbl, excl,
              nexcl, w);
  double lo, hi;
  return block_scan(w[0] + w[1] + w[2] + w[3], s_wave, &lo, &hi);
}

// Final draw of request r (every thread of a kThreads block calls it).
template <typename T>
__device__ inline void draw_select_request(const DrawArgs& a, int r) {
  __shared__ double tbl[kExpTable];
  __shared__ int s_excl[1024];
  __shared__ double s_wave[kThreads / 64];
  __shared__ int s_pick[kThreads / 64];
  __shared__ int s_last[kThreads / 64];
  __shared__ int s_sub, s_flagged, s_list[1024];
  __shared__ double s_base;
  __shared__ double2 s_es[kEsLds];
  __shared__ double s_mass[kMassLds];
  exp_table_fill(tbl);
  // Loads that need no descriptor go out with it: this request's chunk normalisers and this
  // thread's first sub-chunk record (every record when nsub <= kThreads).
  const double2* es = a.esum + (int64_t)r * a.nchunk_draw;
  const double2* suba = a.suba + (int64_t)r * a.nsub;
  const int32_t* subn = a.subn + (int64_t)r * a.nsub;
  const int32_t* suboff = a.suboff + (int64_t)r * a.nsub;
  const int t0 = threadIdx.x;
  const double2 es_first = t0 < a.nchunk_draw ? es[t0] : make_double2(0.0, 0.0);
  double2 A_first = make_double2(0.0, 0.0);
  int n_first = 0, seg_first = -1;
  if (t0 < a.nsub) {
    A_first = suba[t0];
    n_first = subn[t0];
    seg_first = suboff[t0];
  }
  const DrawDesc d = a.desc[r];
  if (d.out_idx < 0) {
    if (threadIdx.x == 0 && a.status) a.status[r] = d.st;
    return;
  }
  int st = d.st;
  const RowView v = row_view(a, d);
  const T* prow = row_ptr<T>(a.rs, d.prow);
  const bool has_q = d.qrow >= 0;
  const T* qrow = has_q ? row_ptr<T>(a.rs, d.qrow) : nullptr;
  const int nexcl = has_q ? 0 : min(d.nexcl, 1024);
  for (int i = threadIdx.x; i < nexcl; i += kThreads)
    s_excl[i] = a.excl[(int64_t)r * a.excl_stride + i];
  if (threadIdx.x == 0) s_flagged = 0;
  double rEp = 1.0, rEq = 0.0, rho = 0.0;
  bool band_ok = true;
  if (has_q) {
    // the chunks' partial normalisers, loaded in parallel and summed in chunk order
    const bool in_lds = a.nchunk_draw <= kEsLds;
    if (in_lds) {
      for (int k = threadIdx.x; k < a.nchunk_draw; k += kThreads)
        s_es[k] = k == t0 ? es_first : es[k];
      __syncthreads();
    }
    double Ep = 0.0, Eq = 0.0;
    for (int k = 0; k < a.nchunk_draw; ++k) {
      const double2 e = in_lds ? s_es[k] : es[k];
      Ep += e.x;
      Eq += e.y;
    }
    rEp = 1.0 / Ep;
    rEq = d.factor / Eq;
    rho = d.factor * Ep / Eq;
    band_ok = fabs(rho / rho_estimate(a, d) - 1.0) <= 0.25 * kBand;
  }
  const int mode = has_q ? 0 : 1;
  // sub-chunk masses: in LDS up to kMassLds sub-chunks, else in the workspace
  double* mass = a.nsub <= kMassLds ? s_mass : a.subsum + (int64_t)r * a.nsub;
  __syncthreads();

  // 1. mass of every sub-chunk: the positive-token sums plus its uncertain tokens (their pool
  //    segment is in token order, so the sum order is fixed); token-by-token sums only for
  //    sub-chunks whose segment did not fit and when the classification is void
  const double2* pool = a.upool ? a.upool + (int64_t)r * kUncPool : nullptr;
  for (int j = threadIdx.x; j < a.nsub; j += kThreads) {
    const bool first = j == t0;
    const double2 A = first ? A_first : suba[j];
    if (!has_q) {
      mass[j] = A.x;
      continue;
    }
    const int n = first ? n_first : subn[j];
    const int seg = n > 0 ? (first ? seg_first : suboff[j]) : 0;
    if (band_ok && seg >= 0) {
      double m = (A.x - rho * A.y) * rEp;
      m = m > 0.0 ? m : 0.0;
      for (int i = 0; i < n; ++i) {
        const double2 t = pool[seg + i];
        const double w = t.x * rEp - t.y * rEq;
        if (w > 0.0) m += w;
      }
      mass[j] = m;
    } else {
      const int slot = atomicAdd(&s_flagged, 1);
      if (slot < 1024) s_list[slot] = j;
    }
  }
  __syncthreads();
  const int nflag = s_flagged;
  if (nflag > 1024) {
    for (int j = 0; j < a.nsub; ++j) {
      const double m = subchunk_mass<T>(prow, qrow, j, a.V, v, mode, rEp, rEq, a.inv_T, tbl, s_excl,
                                        nexcl, s_wave);
      if (threadIdx.x == 0) mass[j] = m;
    }
  } else {
    for (int i = 0; i < nflag; ++i) {
      const int j = s_list[i];
      const double m = subchunk_mass<T>(prow, qrow, j, a.V, v, mode, rEp, rEq, a.inv_T, tbl, s_excl,
                                        nexcl, s_wave);
      if (threadIdx.x == 0) mass[j] = m;
    }
  }
  __syncthreads();

  // 2. locate u' S among the sub-chunks: each thread owns a contiguous run of them
  const double u = philox_uniform(a.seed, a.request_base + (uint32_t)d.ph_req, (uint32_t)d.pos,
                                  (uint32_t)d.purpose, a.step);
  const int per = (a.nsub + kThreads - 1) / kThreads;
  const int j0 = min(a.nsub, threadIdx.x * per), j1 = min(a.nsub, j0 + per);
  double mine = 0.0;
  for (int j = j0; j < j1; ++j) mine += mass[j];
  double lo, hi;
  double S = block_scan(mine, s_wave, &lo, &hi);
  int wmode = mode;
  if (!(S > 0.0)) {
    // Zero residual mass (not reachable in exact arithmetic): draw from the target row itself.
    st |= PSISPEC_ST_RESID_ZERO;
    wmode = 2;
    for (int j = 0; j < a.nsub; ++j) {
      const double m = subchunk_mass<T>(prow, qrow, j, a.V, v, 2, 1.0, 0.0, a.inv_T, tbl, s_excl,
                                        0, s_wave);
      if (threadIdx.x == 0) mass[j] = m;
    }
    __syncthreads();
    mine = 0.0;
    for (int j = j0; j < j1; ++j) mine += mass[j];
    S = block_scan(mine, s_wave, &lo, &hi);
  }
  if (threadIdx.x == 0) {
    s_sub = a.nsub;
    s_base = 0.0;
  }
  __syncthreads();
  double vv = u * S;
  if (lo <= vv && vv < hi) {  // exactly one thread owns vv
    double C = lo;
    int j = j0;
    for (; j < j1; ++j) {
      if (C + mass[j] > vv) break;
      C += mass[j];
    }
    if (j == j1) {  // rounding: the run ends before vv; its last sub-chunk
      --j;
      C -= mass[j];
    }
    s_sub = j;
    s_base = C;
  }
  __syncthreads();
  if (s_sub == a.nsub) {
    // u' S rounded to S: the last token of positive weight of the row (last sub-chunk with mass)
    if (threadIdx.x == 0) {
      int j = a.nsub - 1;
      while (j > 0 && !(mass[j] > 0.0)) --j;
      s_sub = j;
    }
    vv = __builtin_huge_val();
    __syncthreads();
  }
  const int sub = s_sub;

  // 3. the token inside the sub-chunk: block scan of its 1024 weights
  const int x0 = sub * kSub + threadIdx.x * 4;
  double w[4];
  weights4<T>(prow, qrow, x0, a.V, v, wmode, rEp, rEq, a.inv_T, tbl, s_excl, nexcl, w);
  int lastpos = -1;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (w[e] > 0.0) lastpos = x0 + e;
  double l0, h0;
  block_scan(w[0] + w[1] + w[2] + w[3], s_wave, &l0, &h0);
  double C = s_base + l0;
  int tokv = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    C += w[e];
    if (w[e] > 0.0 && C > vv && tokv == 0x7fffffff) tokv = x0 + e;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    tokv = min(tokv, __shfl_xor(tokv, off, 64));
    lastpos = max(lastpos, __shfl_xor(lastpos, off, 64));
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    s_pick[threadIdx.x >> 6] = tokv;
    s_last[threadIdx.x >> 6] = lastpos;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int token = 0x7fffffff, last = -1;
    for (int k = 0; k < kThreads / 64; ++k) {
      token = min(token, s_pick[k]);
      last = max(last, s_last[k]);
    }
    if (token == 0x7fffffff) token = last >= 0 ? last : 0;  // rounding at the sub-chunk's end
    a.out_tokens[d.out_idx] = token;
    if (a.status) a.status[r] = st;
  }
}

}  // namespace
}  // namespace psispec
