// kv.hip -- the KV commit after a verify.
//
// [lanes] "헤드냐, LoRA냐": drafting and verifying share one KV line per sequence; the AR verifies
// and appends.  [alphalab] walkthrough step 4: the accepted prefix is kept, everything after the
// first rejection is discarded and drafted again next round.  Reading: the verify forward wrote
// the KV rows of the block's blk positions at positions len .. len+blk-1 of the request's line; the
// kept rows (block positions keep[0..n-1], strictly increasing: the accepted prefix, or a tree's
// accepted path, whose node indices increase from parent to child) move to len .. len+n-1 in that
// order and the length grows by n.  The rows past the new length are free again (the rollback needs
// no data movement).
//
// The move is in place and hazard-free in increasing i: the source of row i is at keep[i] >= i, and
// every later source is at keep[j] >= j > i, so no store overwrites a row still to be read.  Each
// thread owns two 16-byte slices of every row (a sweep of 1-8 slices and 2-8 rows per round picked
// 2 x 4); it loads its slices of up to four kept rows, then stores them, and rows already in place
// (keep[i] == i, the whole linear case) are not touched.
#include "launch.h"

namespace psispec {
namespace {

constexpr int kKvThreads = 256;
constexpr int kKvSlices = 2;                            // 16-byte slices of a row per thread
constexpr int kKvTile = kKvThreads * 16 * kKvSlices;   // bytes of a row per block
constexpr int kKvBatch = 4;                             // rows loaded before they are stored

// Request r's commit is valid: n in [0, blk] (and <= keep_stride), len in [0, Lmax - blk], keep
// strictly increasing in [0, blk).  The kept positions go to s_keep.  Every thread of the block
// returns the same answer (one block barrier inside).
__device__ inline bool kv_request_ok(const KvArgs& a, int r, int* s_keep) {
  // the count, the length and the kept positions in one round of loads
  const int n = a.n_keep[r], L = a.len[r];
  const int nk = a.keep ? min(a.keep_stride, a.blk) : 0;
  for (int i = threadIdx.x; i < nk; i += blockDim.x) s_keep[i] = a.keep[(int64_t)r * a.keep_stride + i];
  __syncthreads();
  bool bad = n < 0 || n > a.blk || L < 0 || L > a.Lmax - a.blk || (a.keep && n > a.keep_stride);
  if (!bad) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int k = a.keep ? s_keep[i] : i;
      const int kp = i == 0 ? -1 : (a.keep ? s_keep[i - 1] : i - 1);
      if (k < 0 || k >= a.blk || k <= kp) bad = true;
    }
  }
  const bool ok = !__syncthreads_or(bad);
  if (ok && !a.keep) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) s_keep[i] = i;
    __syncthreads();
  }
  return ok;
}

// Block (r, tile) moves bytes [tile * kKvTile, (tile + 1) * kKvTile) of request r's kept rows; a
// thread owns kKvSlices slices, kKvThreads * 16 bytes apart.
__global__ __launch_bounds__(kKvThreads) void k_kv_commit(KvArgs a, int ntiles) {
  __shared__ int s_keep[kMaxKvBlock];
  const int r = blockIdx.x / ntiles;
  const int tile = blockIdx.x - r * ntiles;
  if (!kv_request_ok(a, r, s_keep)) return;
  const int n = a.n_keep[r], L = a.len[r];
  char* base = static_cast<char*>(a.kv) + (int64_t)r * a.line_stride + (int64_t)L * a.row_bytes +
               (int64_t)tile * kKvTile + (int64_t)threadIdx.x * 16;
  const int64_t lim = a.row_bytes - (int64_t)tile * kKvTile - (int64_t)threadIdx.x * 16;
  for (int i0 = 0; i0 < n; i0 += kKvBatch) {
    u32x4 v[kKvBatch][kKvSlices] = {};
#pragma unroll
    for (int u = 0; u < kKvBatch; ++u) {
      const int i = i0 + u;
      if (i < n && s_keep[i] != i) {
        const char* src = base + (int64_t)s_keep[i] * a.row_bytes;
#pragma unroll
        for (int k = 0; k < kKvSlices; ++k)
          if ((int64_t)k * kKvThreads * 16 < lim)
            v[u][k] = *reinterpret_cast<const u32x4*>(src + k * kKvThreads * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kKvBatch; ++u) {
      const int i = i0 + u;
      if (i < n && s_keep[i] != i) {
        char* dst = base + (int64_t)i * a.row_bytes;
#pragma unroll
        for (int k = 0; k < kKvSlices; ++k)
          if ((int64_t)k * kKvThreads * 16 < lim)
            *reinterpret_cast<u32x4*>(dst + k * kKvThreads * 16) = v[u][k];
      }
    }
  }
}

// After every tile of the copy: the new lengths and the status words (one block per request).
__global__ __launch_bounds__(64) void k_kv_len(KvArgs a) {
  __shared__ int s_keep[kMaxKvBlock];
  const int r = blockIdx.x;
  const bool ok = kv_request_ok(a, r, s_keep);
  if (threadIdx.x == 0) {
    if (ok) a.len[r] = a.len[r] + a.n_keep[r];
    if (a.status) a.status[r] = ok ? 0 : PSISPEC_ST_BAD_KEEP;
  }
}

}  // namespace

hipError_t launch_kv_commit(const KvArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int ntiles = (int)((a.row_bytes + kKvTile - 1) / kKvTile);
  PSISPEC_LAUNCH("kv_commit", k_kv_commit, dim3((unsigned)((int64_t)a.batch * ntiles)),
                 dim3(kKvThreads), 0, stream, a, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PSISPEC_LAUNCH("kv_len", k_kv_len, dim3((unsigned)a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace psispec
