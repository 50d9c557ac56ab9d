// draw.hip -- the final token draw of a verify call, in fp64.
//
// At the first rejected position k the replacement token is drawn from the residual
// max(0, p'_k - q'_k) renormalised; after a full accept the extra token is drawn from the
// block-end row p'_B ([alphalab] walkthrough step 4 and the paragraph after it).  The tree draw
// uses p' of the stopping node with the rejected children's tokens removed.  The draw is an
// inverse CDF by ascending token id: c = min{x : C_x > u' S}, C_x = sum_{y <= x} w_y, S = sum w,
// with u' the Philox uniform of (request, position, draw).
//
// The draw decides an integer from floating point, so it is computed in fp64 end to end
// (normalisers, weights and prefix sums): three kernels, all with fixed-order reductions.
//   k_draw_norm:    per (request, chunk) partial sums of exp((l - lmax) / T) over the kept tokens
//                   of the stopping p row (and q row);
//   k_draw_weights: per (request, sub-chunk of 1024 tokens) residual mass and last positive token;
//   k_draw_select:  per request, locate the sub-chunk holding u' S, then a block prefix scan over
//                   its 1024 weights.
#include "launch.h"

namespace psispec {
namespace {

template <typename T>
__device__ inline double term(const T* row, int x, float lmax, float thr, double inv_T) {
  const float l = to_f32(row[x]);
  if (!(l >= thr)) return 0.0;
  return exp(((double)l - (double)lmax) * inv_T);
}

// fixed-order block sum of one double per thread (wave shuffles, then waves in order)
__device__ inline double block_sum(double v, double* scratch) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kThreads / 64; ++w) s += scratch[w];
  return s;
}

__device__ inline int block_max_int(int v, int* scratch) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  int m = scratch[0];
  for (int w = 1; w < kThreads / 64; ++w) m = max(m, scratch[w]);
  return m;
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

template <typename T>
__global__ __launch_bounds__(kThreads) void k_draw_norm(DrawArgs a) {
  const int r = blockIdx.x / a.nchunk_draw;
  const int c = blockIdx.x - r * a.nchunk_draw;
  const DrawDesc d = a.desc[r];
  const RowView v = row_view(a, d);
  const T* prow = row_ptr<T>(a.rs, d.prow);
  const T* qrow = d.qrow >= 0 ? row_ptr<T>(a.rs, d.qrow) : nullptr;
  const int start = c * a.chunk_elems_draw;
  const int end = min(a.V, start + a.chunk_elems_draw);
  double ep = 0.0, eq = 0.0;
  for (int x = start + threadIdx.x; x < end; x += kThreads) {
    ep += term(prow, x, v.lmax_p, v.thr_p, a.inv_T);
    if (qrow) eq += term(qrow, x, v.lmax_q, v.thr_q, a.inv_T);
  }
  __shared__ double scratch[kThreads / 64];
  ep = block_sum(ep, scratch);
  eq = block_sum(eq, scratch);
  if (threadIdx.x == 0) a.esum[(int64_t)r * a.nchunk_draw + c] = make_double2(ep, eq);
}

// Residual weight of token x: max(0, p'(x) - q'(x)), or p'(x) without a q row; removed tokens 0.
template <typename T>
__device__ inline double weight(const T* prow, const T* qrow, int x, const RowView& v, double Ep,
                                double Eq, double inv_T, const int* excl, int nexcl) {
  for (int i = 0; i < nexcl; ++i)
    if (excl[i] == x) return 0.0;
  const double pp = term(prow, x, v.lmax_p, v.thr_p, inv_T) / Ep;
  if (!qrow) return pp;
  const double qq = term(qrow, x, v.lmax_q, v.thr_q, inv_T) / Eq;
  const double w = pp - qq;
  return w > 0.0 ? w : 0.0;
}

__device__ inline void normalisers(const DrawArgs& a, int r, double& Ep, double& Eq) {
  Ep = 0.0;
  Eq = 0.0;
  for (int k = 0; k < a.nchunk_draw; ++k) {
    const double2 e = a.esum[(int64_t)r * a.nchunk_draw + k];
    Ep += e.x;
    Eq += e.y;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_draw_weights(DrawArgs a) {
  const int r = blockIdx.x / a.nchunk_draw;
  const int c = blockIdx.x - r * a.nchunk_draw;
  const DrawDesc d = a.desc[r];
  const RowView v = row_view(a, d);
  const T* prow = row_ptr<T>(a.rs, d.prow);
  const T* qrow = d.qrow >= 0 ? row_ptr<T>(a.rs, d.qrow) : nullptr;
  __shared__ int s_excl[1024];
  __shared__ double scratch[kThreads / 64];
  __shared__ int iscratch[kThreads / 64];
  const int nexcl = min(d.nexcl, 1024);
  for (int i = threadIdx.x; i < nexcl; i += kThreads) s_excl[i] = a.excl[(int64_t)r * a.excl_stride + i];
  __syncthreads();
  double Ep, Eq;
  normalisers(a, r, Ep, Eq);
  const int sub_per_chunk = a.chunk_elems_draw / kSub;
  for (int j = 0; j < sub_per_chunk; ++j) {
    const int sub = c * sub_per_chunk + j;
    if (sub >= a.nsub) break;
    const int base = sub * kSub + threadIdx.x * 4;
    double acc = 0.0;
    int last = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = base + e;
      if (x < a.V) {
        const double w = weight(prow, qrow, x, v, Ep, Eq, a.inv_T, s_excl, nexcl);
        acc += w;
        if (w > 0.0) last = x;
      }
    }
    const double S = block_sum(acc, scratch);
    const int L = block_max_int(last, iscratch);
    if (threadIdx.x == 0) {
      a.subsum[(int64_t)r * a.nsub + sub] = S;
      a.sublast[(int64_t)r * a.nsub + sub] = L;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_draw_select(DrawArgs a) {
  const int r = blockIdx.x;
  const DrawDesc d = a.desc[r];
  __shared__ int s_excl[1024];
  __shared__ double s_wave[kThreads / 64];
  __shared__ double scratch[kThreads / 64];
  __shared__ int iscratch[kThreads / 64];
  __shared__ int s_sub, s_fallback;
  __shared__ double s_base, s_v;
  int st = d.st;
  if (d.out_idx < 0) {
    if (threadIdx.x == 0 && a.status) a.status[r] = st;
    return;
  }
  const RowView v = row_view(a, d);
  const T* prow = row_ptr<T>(a.rs, d.prow);
  const T* qrow = d.qrow >= 0 ? row_ptr<T>(a.rs, d.qrow) : nullptr;
  const int nexcl = min(d.nexcl, 1024);
  for (int i = threadIdx.x; i < nexcl; i += kThreads) s_excl[i] = a.excl[(int64_t)r * a.excl_stride + i];
  double Ep, Eq;
  normalisers(a, r, Ep, Eq);
  const double* subsum = a.subsum + (int64_t)r * a.nsub;
  const int32_t* sublast = a.sublast + (int64_t)r * a.nsub;
  const double u = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)d.pos,
                                  kPurposeDraw, a.step);
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int j = 0; j < a.nsub; ++j) S += subsum[j];
    s_fallback = !(S > 0.0);
    s_v = u * S;
  }
  __syncthreads();
  if (s_fallback) {
    // Zero residual mass (not reachable in exact arithmetic): draw from the target row instead.
    st |= PSISPEC_ST_RESID_ZERO;
    qrow = nullptr;
  }
  // Sub-chunk sums for the fallback are recomputed here; the normal path reuses k_draw_weights'.
  if (threadIdx.x == 0 && !s_fallback) {
    const double vv = s_v;
    double C = 0.0;
    int j = 0;
    for (; j < a.nsub; ++j) {
      if (C + subsum[j] > vv) break;
      C += subsum[j];
    }
    s_sub = j;
    s_base = C;
  }
  if (s_fallback) {
    // S over the p row, then the sub-chunk walk, both by the whole block in fixed order
    double S = 0.0;
    for (int sub = 0; sub < a.nsub; ++sub) {
      const int x0 = sub * kSub + threadIdx.x * 4;
      double acc = 0.0;
      for (int e = 0; e < 4; ++e)
        if (x0 + e < a.V) acc += weight(prow, qrow, x0 + e, v, Ep, Eq, a.inv_T, s_excl, 0);
      S += block_sum(acc, scratch);
    }
    const double vv = u * S;
    double C = 0.0;
    int j = 0;
    for (; j < a.nsub; ++j) {
      const int x0 = j * kSub + threadIdx.x * 4;
      double acc = 0.0;
      for (int e = 0; e < 4; ++e)
        if (x0 + e < a.V) acc += weight(prow, qrow, x0 + e, v, Ep, Eq, a.inv_T, s_excl, 0);
      const double Sj = block_sum(acc, scratch);
      if (C + Sj > vv) break;
      C += Sj;
    }
    if (threadIdx.x == 0) {
      s_sub = j;
      s_base = C;
      s_v = vv;
    }
  }
  __syncthreads();
  const int sub = s_sub;
  const int use_excl = s_fallback ? 0 : nexcl;
  int tokv = 0x7fffffff;
  int lastpos = -1;
  if (sub < a.nsub) {
    // weights of this thread's 4 consecutive tokens and their running sums
    const int x0 = sub * kSub + threadIdx.x * 4;
    double w[4];
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = (x0 + e < a.V) ? weight(prow, qrow, x0 + e, v, Ep, Eq, a.inv_T, s_excl, use_excl) : 0.0;
      run += w[e];
      if (w[e] > 0.0) lastpos = x0 + e;
    }
    // exclusive scan of the per-thread totals: inclusive wave scan, then wave offsets in order
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    double off_w = 0.0;
    for (int k = 0; k < wave; ++k) off_w += s_wave[k];
    double C = s_base + off_w + (incl - run);
    const double vv = s_v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      C += w[e];
      if (w[e] > 0.0 && C > vv && tokv == 0x7fffffff) tokv = x0 + e;
    }
  } else {
    __syncthreads();
  }
  // first token past v in the sub-chunk (min over threads)
  int tmin = tokv;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tmin = min(tmin, __shfl_xor(tmin, off, 64));
  __shared__ int s_min[kThreads / 64];
  if ((threadIdx.x & 63) == 0) s_min[threadIdx.x >> 6] = tmin;
  const int lastsub = block_max_int(lastpos, iscratch);
  if (threadIdx.x == 0) {
    int token = 0x7fffffff;
    for (int k = 0; k < kThreads / 64; ++k) token = min(token, s_min[k]);
    if (token == 0x7fffffff) {
      // rounding put u' S at or past the end of the chosen interval: last positive token there,
      // else the last positive token of the row
      token = lastsub;
      if (token < 0 && !s_fallback)
        for (int j = a.nsub - 1; j >= 0 && token < 0; --j) token = sublast[j];
      if (token < 0) token = 0;
    }
    a.out_tokens[d.out_idx] = token;
    if (a.status) a.status[r] = st;
  }
}

}  // namespace

hipError_t launch_draw(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)a.batch * a.nchunk_draw);
  timing_begin("draw_norm", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_draw_norm<bf16_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(k_draw_norm<float>, dim3(grid), dim3(kThreads), 0, stream, a);
  timing_end("draw_norm", stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_begin("draw_weights", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_draw_weights<bf16_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(k_draw_weights<float>, dim3(grid), dim3(kThreads), 0, stream, a);
  timing_end("draw_weights", stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_begin("draw_select", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_draw_select<bf16_t>, dim3(a.batch), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(k_draw_select<float>, dim3(a.batch), dim3(kThreads), 0, stream, a);
  timing_end("draw_select", stream);
  return hipGetLastError();
}

}  // namespace psispec
