// rows.hip -- the HBM pass over every logits row: temperature-softmax statistics.
//
// Every p and q row of a call is read once here (the data-parallel part of the verify: [alphalab]
// walkthrough step 3 -- the AR scores the whole block in one pass and every position gets its
// test).  A workgroup streams one chunk of one row with 16-byte loads and keeps an online
// (max, sum of exp) pair per lane; the pair of each (row, chunk) goes to the workspace and is
// combined in a fixed order by the consumers, so results do not depend on scheduling.
#include "launch.h"
#include "rows.h"

namespace psispec {
namespace {

template <typename T, int kUnroll>
__global__ __launch_bounds__(kThreads) void k_rowstats(RowSet rs, int nchunk, int chunk_elems,
                                                       float c, float2* __restrict__ part,
                                                       int vec_ok) {
  const int64_t task = blockIdx.x;
  const int64_t row = task / nchunk;
  const int chunk = (int)(task - row * nchunk);
  if (row_skipped(rs, row)) return;
  rowstats_task<T, kUnroll>(rs, row, chunk, chunk_elems, c, part + task, vec_ok);
}

}  // namespace

hipError_t launch_rowstats(const RowSet& rs, psispec_dtype dtype, int nchunk, int chunk_elems,
                           float c, float2* part, hipStream_t stream) {
  const int64_t tasks = (rs.nP + rs.nQ) * (int64_t)nchunk;
  if (tasks == 0) return hipSuccess;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)rs.V * es) % 16 == 0 && ((size_t)rs.pstride * es) % 16 == 0 &&
                     ((uintptr_t)rs.p % 16) == 0 &&
                     ((uintptr_t)rs.q % 16) == 0 && (chunk_elems % 8) == 0;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("rowstats", (k_rowstats<bf16_t, 8>), dim3((unsigned)tasks), dim3(kThreads), 0,
                   stream, rs, nchunk, chunk_elems, c, part, vec_ok);
  else
    PSISPEC_LAUNCH("rowstats", (k_rowstats<float, 8>), dim3((unsigned)tasks), dim3(kThreads), 0,
                   stream, rs, nchunk, chunk_elems, c, part, vec_ok);
  return hipGetLastError();
}

}  // namespace psispec
