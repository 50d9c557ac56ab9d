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
// fixed order.  Two kernels:
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
//                  segment of a per-request pool.  The pass stores per sub-chunk the sums A_p, A_q
//                  of e_p, e_q over the positive tokens and the segment, and per chunk the partial
//                  normalisers E_p, E_q.
//   k_draw_select: per request, the exact E_p, E_q give rho; each sub-chunk's mass is
//                  (A_p - rho A_q) / E_p plus the residual weights of its uncertain tokens (added
//                  in token order); it is recomputed token by token only when the pool overflowed
//                  or rho strays from the HBM-pass ratio by more than a quarter of the band (which
//                  voids the classification); a block scan over the
//                  masses locates u' S, then a block scan over that sub-chunk's 1024 weights
//                  picks the token.
#include "launch.h"
#include "draw.h"

namespace psispec {
namespace {

// at least this many waves per SIMD: a fully unrolled run of 16 token pairs would otherwise take
// ~190 VGPRs (two waves per SIMD); capped, the compiler interleaves fewer exps per wave and the
// other waves hide the table reads
constexpr int kDrawPassWaves = 5;

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

constexpr unsigned kListPassBlocks = 1024;   // grid of the pass over listed draws
constexpr unsigned kListSelectBlocks = 256;  // grid of the select over listed draws


}  // namespace

hipError_t launch_draw(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  unsigned grid = (unsigned)((int64_t)a.batch * a.nchunk_draw);
  unsigned sgrid = (unsigned)a.batch;
  if (a.list) {
    grid = grid < kListPassBlocks ? grid : kListPassBlocks;
    sgrid = sgrid < kListSelectBlocks ? sgrid : kListSelectBlocks;
  }
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)a.V * es) % 16 == 0 &&
                     ((size_t)a.rs.pstride * es) % 16 == 0 && ((uintptr_t)a.rs.p % 16) == 0 &&
                     ((uintptr_t)a.rs.q % 16) == 0;
  const bool bf = dtype == PSISPEC_BF16, tp = a.use_topp, li = a.list != nullptr;
  auto kern = bf ? (tp ? (li ? k_draw_pass<bf16_t, true, true> : k_draw_pass<bf16_t, true, false>)
                       : (li ? k_draw_pass<bf16_t, false, true> : k_draw_pass<bf16_t, false, false>))
                 : (tp ? (li ? k_draw_pass<float, true, true> : k_draw_pass<float, true, false>)
                       : (li ? k_draw_pass<float, false, true> : k_draw_pass<float, false, false>));
  PSISPEC_LAUNCH("draw_pass", kern, dim3(grid), dim3(kThreads), 0, stream, a, vec_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("draw_select", k_draw_select<bf16_t>, dim3(sgrid), dim3(kThreads), 0, stream, a);
  else
    PSISPEC_LAUNCH("draw_select", k_draw_select<float>, dim3(sgrid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace psispec
