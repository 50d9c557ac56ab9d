// linear.hip -- per-request accept test and first-rejection scan of the linear verify.
//
// One wave64 per request.  Lanes first finish the row statistics of the request's 2B+1 rows from
// the per-chunk pairs of the HBM pass (fixed order), then lane i scores draft i:
// ratio_i = min(1, p'_i(d_i) / q'_i(d_i)) in fp64, accept_i = u_i < ratio_i with u_i the Philox
// uniform of (request, i, accept).  A wave ballot gives every accept bit at once; the first zero
// bit is the first rejection k ([alphalab] walkthrough steps 3-4: keep the longest accepted run
// from the start, discard everything after the first rejection).  The final draw (correction at
// k < B, bonus from the block-end row at k = B) is left to the fp64 draw kernels.
//
// Small calls (a request's rows within kSmallVerifyBytes, no nucleus) are launch-latency bound: four
// launches of a few microseconds each for a few kilobytes of logits.  k_verify_small runs a
// request's whole verify in one block instead: its rows' statistics (one wave per row, each row one
// chunk), then the same device functions as the separate kernels, in the same order (accept test,
// draw pass chunk by chunk, select).  The pairs are reduced by one wave instead of a block, so they
// may differ from the separate kernels' in the last bit; every later step is the same code.
#include "launch.h"
#include "decide.h"
#include "draw.h"
#include "rows.h"

namespace psispec {
namespace {

template <typename T>
__global__ __launch_bounds__(64) void k_decide_linear(LinearArgs a) {
  decide_linear_request<T>(a, blockIdx.x);
}

__global__ __launch_bounds__(64) void k_combine_rows(RowSet rs, const float2* __restrict__ part,
                                                    int nchunk, float c,
                                                    RowStat* __restrict__ rowstat) {
  const int64_t row = blockIdx.x;
  if (row_skipped(rs, row)) return;
  float lmax;
  double Z;
  combine_row_wave(part + row * nchunk, nchunk, c, lmax, Z);
  if (threadIdx.x == 0) rowstat[row] = RowStat{lmax, row_status(lmax, Z), Z};
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_verify_small(LinearArgs la, DrawArgs da,
                                                           float2* __restrict__ part,
                                                           int vec_ok_draw) {
  const int r = blockIdx.x;
  const int B = la.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the request's rows, one wave per row (the launcher checks that a row is one chunk)
  for (int j = wave; j < 2 * B + 1; j += kThreads / 64) {
    const int64_t row = j <= B ? (int64_t)r * (B + 1) + j : la.rs.nP + (int64_t)r * B + (j - B - 1);
    if (row_skipped(la.rs, row)) continue;
    const T* rp = row_ptr<T>(la.rs, row);
    float m = kNegBig, s = 0.f;
    for (int x = lane; x < la.V; x += 64) {
      const float f[1] = {to_f32(rp[x])};
      fold(f, m, s, la.c);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(m, off, 64);
      const float s2 = __shfl_xor(s, off, 64);
      os_combine(m, s, m2, s2, la.c);
    }
    if (lane == 0) part[row] = make_float2(m, s);
  }
  __syncthreads();  // every pair is written
  decide_linear_request<T>(la, r);  // its first barrier follows the pair reads
  __syncthreads();                   // the descriptor is written
  for (int ch = 0; ch < da.nchunk_draw; ++ch) {
    draw_pass_task<T, false>(da, r, ch, vec_ok_draw);
    __syncthreads();  // the chunk's sums are written; the next chunk refills the LDS
  }
  draw_select_request<T>(da, r);
}

}  // namespace

hipError_t launch_verify_small(const LinearArgs& la, const DrawArgs& da, float2* part,
                               psispec_dtype dtype, hipStream_t stream) {
  if (la.batch == 0) return hipSuccess;
  if (la.nchunk != 1 || la.use_topp) return hipErrorInvalidValue;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const RowSet& rs = la.rs;
  const int aligned = ((size_t)rs.V * es) % 16 == 0 && ((size_t)rs.pstride * es) % 16 == 0 &&
                      ((uintptr_t)rs.p % 16) == 0 && ((uintptr_t)rs.q % 16) == 0;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("verify_small", k_verify_small<bf16_t>, dim3((unsigned)la.batch),
                   dim3(kThreads), 0, stream, la, da, part, aligned);
  else
    PSISPEC_LAUNCH("verify_small", k_verify_small<float>, dim3((unsigned)la.batch),
                   dim3(kThreads), 0, stream, la, da, part, aligned);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const RowSet& rs, const float2* part, int nchunk, float c,
                               RowStat* rowstat, hipStream_t stream) {
  const int64_t rows = rs.nP + rs.nQ;
  if (rows == 0) return hipSuccess;
  PSISPEC_LAUNCH("combine_rows", k_combine_rows, dim3((unsigned)rows), dim3(64), 0, stream, rs,
                 part, nchunk, c, rowstat);
  return hipGetLastError();
}

hipError_t launch_decide_linear(const LinearArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("decide_linear", k_decide_linear<bf16_t>, dim3(a.batch), dim3(64), 0, stream, a);
  else
    PSISPEC_LAUNCH("decide_linear", k_decide_linear<float>, dim3(a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace psispec
