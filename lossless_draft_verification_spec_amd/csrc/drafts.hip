// drafts.hip -- the drafting step: one token per (request, position) drawn from its own row.
//
// [alphalab] walkthrough steps 1-2: the AR path samples the first token of the block and the
// diffusion path proposes the others in parallel.  Every drafted token is one inverse-CDF draw from
// its row after the temperature and the nucleus, because the verify divides by exactly that q'.
// The draws reuse the kernels of the verify's final draw (the HBM row pass for the statistics, the
// nucleus kernel, the fp64 draw pass and select).  This file holds the step between them: per
// drafted token, the row's statistics are combined from the row pass's per-chunk pairs (one wave,
// fixed order) and the draw is described: its row, its Philox counter (request, position, DRAFT,
// step) and its output slot.
#include "launch.h"
#include "decide.h"

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
    desc[j] = d;
  }
}

}  // namespace

hipError_t launch_draft_rows(const RowSet& rs, int batch, int B, int first_from_target,
                             const float2* part, int nchunk, float c, RowStat* rowstat,
                             DrawDesc* desc, hipStream_t stream) {
  const int64_t jobs = (int64_t)batch * B;
  if (jobs == 0) return hipSuccess;
  timing_begin("draft_rows", stream);
  hipLaunchKernelGGL(k_draft_rows, dim3((unsigned)jobs), dim3(64), 0, stream, rs, B,
                     first_from_target, part, nchunk, c, rowstat, desc);
  timing_end("draft_rows", stream);
  return hipGetLastError();
}

}  // namespace psispec
