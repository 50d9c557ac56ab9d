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
// Small calls (a request's rows within kSmallVerifyBytes, no nucleus) are latency bound: four
// launches of a few microseconds each for a few kilobytes of logits.  k_verify_small runs a
// request's whole verify in one block instead: it copies the request's rows into LDS (one round
// of loads), computes their statistics (each row one chunk, reduced by a wave, or by 16 lanes when
// there are more rows than waves), then runs the same device functions as the separate kernels, in
// the same order (accept test, draw pass chunk by chunk, select), on the request as a one-request
// call whose rows, pairs, statistics, descriptor and draw records are LDS arrays: the steps hand
// over through LDS, not through global memory.  The pairs are reduced by a
// wave or 16 lanes instead of a block, so they may differ from the separate kernels' in the last
// bit; every later step is the same code.
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

// DPP lane exchanges for the one-block verify's row reductions: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror and row_mirror pair the 16 lanes of a DPP row symmetrically, so after
// the four steps every lane of the row holds the row's result; for a whole wave the four rows are
// then combined in order.
template <int kCtrl>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, true));
}
__device__ inline float lane_f32(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ inline float row16_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return fmaxf(v, dpp_f32<0x140>(v));
}
__device__ inline float row16_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}
__device__ inline float wave_max_f32(float v) {
  v = row16_max_f32(v);
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ inline float wave_sum_f32(float v) {
  v = row16_sum_f32(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// LDS records of the one-block verify beside its rows: the draw's chunk and sub-chunk records (a
// request's rows within kSmallVerifyBytes have at most 6 sub-chunks of 1024 tokens)
constexpr int kSmallChunks = 8, kSmallSubs = 8;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_verify_small(LinearArgs la, DrawArgs da, int vec_ok) {
  __shared__ __attribute__((aligned(16))) unsigned char s_rows[kSmallVerifyBytes];
  __shared__ float2 s_pairs[2 * kMaxB + 1];
  __shared__ RowStat s_rowstat[2 * kMaxB + 1];
  __shared__ DrawDesc s_desc[1];
  __shared__ double2 s_esum[kSmallChunks], s_suba[kSmallSubs];
  __shared__ int32_t s_subn[kSmallSubs], s_suboff[kSmallSubs];
  __shared__ double s_subsum[kSmallSubs];
  const int r = blockIdx.x;
  const int B = la.B, V = la.V, nrows = 2 * B + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T* rows = reinterpret_cast<T*>(s_rows);
  // the request's global row of local row j (p rows 0..B, then q rows 0..B-1)
  auto grow = [&](int j) -> int64_t {
    return j <= B ? (int64_t)r * (B + 1) + j : la.rs.nP + (int64_t)r * B + (j - B - 1);
  };
  // 1. the request's rows into LDS (one round of loads; a skipped row is not read)
  if (vec_ok) {
    constexpr int E = 16 / (int)sizeof(T);
    const int nv = V / E;
    for (int i = threadIdx.x; i < nrows * nv; i += kThreads) {
      const int j = i / nv, x = i - j * nv;
      const int64_t row = grow(j);
      if (row_skipped(la.rs, row)) continue;
      reinterpret_cast<u32x4*>(rows + (size_t)j * V)[x] =
          reinterpret_cast<const u32x4*>(row_ptr<T>(la.rs, row))[x];
    }
  } else {
    for (int i = threadIdx.x; i < nrows * V; i += kThreads) {
      const int j = i / V, x = i - j * V;
      const int64_t row = grow(j);
      if (!row_skipped(la.rs, row)) rows[i] = row_ptr<T>(la.rs, row)[x];
    }
  }
  // 2. the same device functions as the separate kernels, on this request alone (request 0 of a
  //    one-request call whose rows, statistics, descriptor and draw records live in LDS; the
  //    Philox request word and the outputs keep their place in the whole call)
  LinearArgs l1 = la;
  l1.rs.p = rows;
  l1.rs.q = rows + (size_t)(B + 1) * V;
  l1.rs.nP = B + 1;
  l1.rs.nQ = B;
  l1.rs.pstride = V;
  l1.draft = la.draft + (int64_t)r * B;
  l1.batch = 1;
  l1.request_base = la.request_base + (uint32_t)r;
  l1.part = s_pairs;
  l1.rowstat = s_rowstat;
  l1.rowstat_ready = 0;
  l1.desc = s_desc;
  l1.accept_len = la.accept_len + r;
  l1.out_tokens = la.out_tokens + (int64_t)r * (B + 1);
  l1.ratios = la.ratios ? la.ratios + (int64_t)r * B : nullptr;
  l1.accept_mask = la.accept_mask ? la.accept_mask + r : nullptr;
  DrawArgs d1 = da;
  d1.rs = l1.rs;
  d1.batch = 1;
  d1.request_base = l1.request_base;
  d1.rowstat = s_rowstat;
  d1.desc = s_desc;
  d1.esum = s_esum;
  d1.suba = s_suba;
  d1.subn = s_subn;
  d1.suboff = s_suboff;
  d1.subsum = s_subsum;
  d1.upool = da.upool ? da.upool + (int64_t)r * kUncPool : nullptr;
  d1.out_tokens = da.out_tokens + (int64_t)r * (B + 1);
  d1.status = da.status ? da.status + r : nullptr;
  __syncthreads();  // the rows are staged
  // 3. the rows' pairs (the launcher checks that a row is one chunk): with more rows than waves,
  //    each 16-lane row of the block reduces one logit row in one round (all lanes take part in the
  //    DPP steps; a lane past the rows or in a skipped row holds (floor, 0)); else one wave per row
  if (nrows > kThreads / 64) {
    const int grp = threadIdx.x >> 4, l16 = threadIdx.x & 15;
    for (int j0 = 0; j0 < nrows; j0 += kThreads / 16) {
      const int j = j0 + grp;
      const bool live = j < nrows && !row_skipped(l1.rs, j);
      float m = kNegBig, s = 0.f;
      if (live) {
        const T* rp = row_ptr<T>(l1.rs, j);
        for (int x = l16; x < V; x += 16) {
          const float f[1] = {to_f32(rp[x])};
          fold(f, m, s, la.c);
        }
      }
      const float M = row16_max_f32(m);
      const float S = row16_sum_f32(s * __builtin_amdgcn_exp2f((m - M) * la.c));
      if (live && l16 == 0) s_pairs[j] = make_float2(M, S);
    }
  } else {
    for (int j = wave; j < nrows; j += kThreads / 64) {
      if (row_skipped(l1.rs, j)) continue;
      const T* rp = row_ptr<T>(l1.rs, j);
      float m = kNegBig, s = 0.f;
      for (int x = lane; x < V; x += 64) {
        const float f[1] = {to_f32(rp[x])};
        fold(f, m, s, la.c);
      }
      // the wave's pair: its maximum, then every lane's sum rescaled to it and added up (a lane
      // without tokens holds (floor, 0) and adds 0; a NaN sum stays NaN)
      const float M = wave_max_f32(m);
      const float S = wave_sum_f32(s * __builtin_amdgcn_exp2f((m - M) * la.c));
      if (lane == 0) s_pairs[j] = make_float2(M, S);
    }
  }
  __syncthreads();  // every pair is written
  decide_linear_request<T>(l1, 0);  // its first barrier follows the pair reads
  __syncthreads();                  // the descriptor is written
  const int vec_lds = ((size_t)V * sizeof(T)) % 16 == 0;  // LDS rows are 16-byte aligned then
  for (int ch = 0; ch < d1.nchunk_draw; ++ch) {
    draw_pass_task<T, false, true>(d1, 0, ch, vec_lds);
    __syncthreads();  // the chunk's sums are written; the next chunk refills the LDS
  }
  draw_select_request<T>(d1, 0);
}

}  // namespace

hipError_t launch_verify_small(const LinearArgs& la, const DrawArgs& da, psispec_dtype dtype,
                               hipStream_t stream) {
  if (la.batch == 0) return hipSuccess;
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  if (la.nchunk != 1 || la.use_topp || la.gath || la.B < 1 || la.B > kMaxB ||
      (size_t)(2 * la.B + 1) * (size_t)la.V * es > kSmallVerifyBytes ||
      da.nchunk_draw > kSmallChunks || da.nsub > kSmallSubs)
    return hipErrorInvalidValue;
  const RowSet& rs = la.rs;
  const int aligned = ((size_t)rs.V * es) % 16 == 0 && ((size_t)rs.pstride * es) % 16 == 0 &&
                      ((uintptr_t)rs.p % 16) == 0 && ((uintptr_t)rs.q % 16) == 0;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("verify_small", k_verify_small<bf16_t>, dim3((unsigned)la.batch),
                   dim3(kThreads), 0, stream, la, da, aligned);
  else
    PSISPEC_LAUNCH("verify_small", k_verify_small<float>, dim3((unsigned)la.batch),
                   dim3(kThreads), 0, stream, la, da, aligned);
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
