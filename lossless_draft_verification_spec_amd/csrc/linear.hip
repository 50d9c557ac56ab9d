// linear.hip -- per-request accept test and first-rejection scan of the linear verify.
//
// One wave64 per request.  Lanes first finish the row statistics of the request's 2B+1 rows from
// the per-chunk pairs of the HBM pass (fixed order), then lane i scores draft i:
// ratio_i = min(1, p'_i(d_i) / q'_i(d_i)) in fp64, accept_i = u_i < ratio_i with u_i the Philox
// uniform of (request, i, accept).  A wave ballot gives every accept bit at once; the first zero
// bit is the first rejection k ([alphalab] walkthrough steps 3-4: keep the longest accepted run
// from the start, discard everything after the first rejection).  The final draw (correction at
// k < B, bonus from the block-end row at k = B) is left to the fp64 draw kernels.
#include "launch.h"
#include "decide.h"

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

}  // namespace

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
