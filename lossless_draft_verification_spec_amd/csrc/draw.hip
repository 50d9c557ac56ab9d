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
// (normalisers, weights and prefix sums) with a table-driven fp64 exp; all reductions run in a
// fixed order.  Two steps:
//   k_draw_pass:   one fp64 pass over the stopping row(s): a block per chunk of 4096 spw tokens,
//                  each wave taking spw sub-chunks of 1024 tokens in turn (spw = 1, 2, 4 or 8: more
//                  when the draws alone fill the chip, which spreads each block's set-up over more
//                  tokens), 16 consecutive tokens per lane.  Without a q row (bonus draw, tree
//                  draw) the weights need no normaliser: w = exp((l - lmax) / T) over the kept,
//                  not removed tokens, and the pass stores each sub-chunk's mass.  With a q row
//                  the sign of p'(x) - q'(x) = (e_p(x) - rho e_q(x)) / E_p, rho = E_p / E_q, is
//                  decided with the ratio of the normalisers from the HBM pass (relative error
//                  below ~1e-6), as a comparison of exponents (t_p - t_q against 256 log2 rho);
//                  tokens within a 1e-5 band of the sign change are uncertain: each wave packs the
//                  exact (e_p, e_q) of its sub-chunk's uncertain tokens, in token order, into a
//                  segment of its chunk's slice of the request's pool.  The pass stores per
//                  sub-chunk the sums A_p, A_q of e_p, e_q over the positive tokens and the
//                  segment, and per chunk the partial normalisers E_p, E_q.  The linear verify,
//                  and the trees of at most 64 nodes (tree.hip, treeq.hip), run the same pass
//                  fused after their accept test or walk (k_decide_draw and its tree forms).
//   k_draw_select: per request, the exact E_p, E_q give rho; each sub-chunk's mass is
//                  (A_p - rho A_q) / E_p plus the residual weights of its uncertain tokens (added
//                  in token order); it is recomputed token by token only when the slice overflowed
//                  or rho strays from the HBM-pass ratio by more than a quarter of the band (which
//                  voids the classification); a block scan over the
//                  masses locates u' S, then a block scan over that sub-chunk's 1024 weights
//                  picks the token.
#include "launch.h"
#include "decide.h"
#include "draw.h"

namespace psispec {
namespace {

// kList: the draws are a device-side list (the grid loops over its entries); a separate
// instantiation, since the loop keeps registers live that the one-task-per-block form does not need
template <typename T, bool kTopp, bool kList>
__global__ __launch_bounds__(kThreads, kList ? 4 : kDrawPassWaves) void k_draw_pass(DrawArgs a, int vec_ok) {
  if constexpr (!kList) {
    const int r = blockIdx.x / a.nchunk_draw;
    draw_pass_task<T, kTopp>(a, r, blockIdx.x - r * a.nchunk_draw, vec_ok);
    return;
  }
  // listed draws only: the grid loops over (list entry, chunk) pairs
  const int n = *a.count * a.nchunk_draw;
  for (int w = blockIdx.x; w < n; w += gridDim.x) {
    const int e = w / a.nchunk_draw;
    draw_pass_task<T, kTopp>(a, a.list[e], w - e * a.nchunk_draw, vec_ok);
    __syncthreads();  // the next task refills the block's LDS
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_draw_select(DrawArgs a) {
  if (!a.list) {
    draw_select_request<T>(a, blockIdx.x);
    return;
  }
  const int n = *a.count;
  for (int e = blockIdx.x; e < n; e += gridDim.x) {
    draw_select_request<T>(a, a.list[e]);
    __syncthreads();
  }
}

// The linear verify's accept test fused with the draw pass: block (r, c) runs request r's accept
// test (wave 0, on the row pass's pairs) into LDS, then draws chunk c of the stopping row(s) from
// those copies.  The test is repeated by each of the request's nchunk_draw blocks (a few hundred
// bytes of pairs and two gathered logits per position); the chunk-0 block also writes the call's
// outputs, the row statistics and the description that the select reads.  Against an accept-test
// launch followed by the draw pass this saves a launch and the pass's dependent reads of the
// description and then of the stopping rows' statistics.
template <typename T, bool kTopp>
__global__ __launch_bounds__(kThreads, kDrawPassWaves) void k_decide_draw(LinearArgs la, DrawArgs da,
                                                                          int vec_ok) {
  __shared__ double tbl[kExpTable];
  __shared__ RowStat s_rs[2 * kMaxB + 1];
  __shared__ DrawDesc s_d;
  exp_table_fill(tbl);  // read after the barriers below
  const int r = blockIdx.x / da.nchunk_draw;
  const int c = blockIdx.x - r * da.nchunk_draw;
  LinearArgs l = la;
  l.rowstat_local = s_rs;
  l.desc_local = &s_d;
  l.quiet = c != 0;
  decide_linear_request<T>(l, r);
  __syncthreads();  // the description and the statistics are in LDS
  const DrawDesc d = s_d;
  const int k = d.pos, qj = la.B + 1 + k;  // local rows of the stopping p and q rows
  const bool has_q = d.qrow >= 0;
  RowView v;
  v.lmax_p = s_rs[k].lmax;
  v.thr_p = kTopp ? la.topp[d.prow].thr : -__builtin_huge_valf();
  v.lmax_q = has_q ? s_rs[qj].lmax : 0.f;
  v.thr_q = has_q ? (kTopp ? la.topp[d.qrow].thr : -__builtin_huge_valf()) : 0.f;
  double rho = 0.0;
  if (has_q) {  // as rho_estimate computes it from the workspace copies
    double ep = s_rs[k].Z, eq = s_rs[qj].Z;
    if (kTopp) {
      ep *= la.topp[d.prow].M;
      eq *= la.topp[d.qrow].M;
    }
    rho = d.factor * ep / eq;
  }
  draw_pass_run<T, kTopp>(da, r, c, vec_ok, d, v, rho, tbl);
}

constexpr unsigned kListPassBlocks = 1024;   // grid of the pass over listed draws
constexpr unsigned kListSelectBlocks = 256;  // grid of the select over listed draws


}  // namespace

int draw_vec_ok(const DrawArgs& a, psispec_dtype dtype) {
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  return ((size_t)a.V * es) % 16 == 0 && ((size_t)a.rs.pstride * es) % 16 == 0 &&
         ((uintptr_t)a.rs.p % 16) == 0 && ((uintptr_t)a.rs.q % 16) == 0;
}

hipError_t launch_draw_select(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream) {
  unsigned sgrid = (unsigned)a.batch;
  if (a.list) sgrid = sgrid < kListSelectBlocks ? sgrid : kListSelectBlocks;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("draw_select", k_draw_select<bf16_t>, dim3(sgrid), dim3(kThreads), 0, stream, a);
  else
    PSISPEC_LAUNCH("draw_select", k_draw_select<float>, dim3(sgrid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_draw(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  unsigned grid = (unsigned)((int64_t)a.batch * a.nchunk_draw);
  if (a.list) grid = grid < kListPassBlocks ? grid : kListPassBlocks;
  const int vec_ok = draw_vec_ok(a, dtype);
  const bool bf = dtype == PSISPEC_BF16, tp = a.use_topp, li = a.list != nullptr;
  auto kern = bf ? (tp ? (li ? k_draw_pass<bf16_t, true, true> : k_draw_pass<bf16_t, true, false>)
                       : (li ? k_draw_pass<bf16_t, false, true> : k_draw_pass<bf16_t, false, false>))
                 : (tp ? (li ? k_draw_pass<float, true, true> : k_draw_pass<float, true, false>)
                       : (li ? k_draw_pass<float, false, true> : k_draw_pass<float, false, false>));
  PSISPEC_LAUNCH("draw_pass", kern, dim3(grid), dim3(kThreads), 0, stream, a, vec_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw_select(a, dtype, stream);
}

hipError_t launch_decide_draw(const LinearArgs& la, const DrawArgs& da, psispec_dtype dtype,
                              hipStream_t stream) {
  if (da.batch == 0) return hipSuccess;
  if (da.list || la.gath || la.rowstat_ready || la.batch != da.batch || la.use_topp != da.use_topp)
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((int64_t)da.batch * da.nchunk_draw);
  const int vec_ok = draw_vec_ok(da, dtype);
  const bool bf = dtype == PSISPEC_BF16, tp = da.use_topp;
  auto kern = bf ? (tp ? k_decide_draw<bf16_t, true> : k_decide_draw<bf16_t, false>)
                 : (tp ? k_decide_draw<float, true> : k_decide_draw<float, false>);
  PSISPEC_LAUNCH("decide_draw", kern, dim3(grid), dim3(kThreads), 0, stream, la, da, vec_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw_select(da, dtype, stream);
}

}  // namespace psispec
