// lmhead.hip -- the LM head feeding the verify: logits = H W (+ LoRA on the draft rows) on MFMA.
//
// [lanes] §"헤드냐, LoRA냐": the draft path is the frozen AR weights plus a low-rank LoRA delta, the
// verify path the frozen AR weights alone; [alphalab] walkthrough step 2 (draft rows through the
// LoRA path) and step 3 (the AR scores the block).  Only the output projection is built here:
//   p rows (AR):    logits[m]  = h_ar[m] . W
//   q rows (draft): logits[m]  = h_dr[m] . W + s (h_dr[m] . A) . B
// The product is the one dense contraction of the verify step, so it runs on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  The weight is taken in its usual storage, one
// contiguous row of H values per token (W_t[V][H]), so both MFMA operands are contiguous along the
// contraction and go to LDS without a transpose.
//
// Tiling: a 256x256 output tile per 256-thread workgroup (four wave64s, 128x128 each = 4x4 MFMA
// tiles), K steps of 64 double-buffered in LDS (144 KB), 16-byte global loads staged through
// registers.  Tiles are ordered so that the workgroups of one XCD sweep the M tiles of the same
// W column block together, so each W block comes from HBM once and is reused through that XCD's L2.
// The LoRA delta rides in the same MFMA loop as extra contraction columns: t = s (h_dr . A) is
// computed in fp64 and split into two bf16 parts t_hi + t_lo (relative error 2^-17, far below the
// fp32 accumulation error of the H-long product), and the extra steps multiply [t_hi | t_lo] by
// [B | B] (zeros for the AR rows and the padding).  The epilogue writes the fp32 logits and emits
// per (row, column tile) the online softmax pair (max, sum exp) that the verify's decide and draw
// kernels consume in place of the HBM row pass.
#include "launch.h"

namespace psispec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LROW = BK + 8;  // bf16 elements per LDS row (16-byte pad: conflict-free 16-byte reads)
constexpr int A_STAGE = BM * LROW, B_STAGE = BN * LROW;
constexpr int kXcd = 8;

__device__ inline uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Extra contraction columns of row m (grid over all M rows): zeros for the AR rows (m < nP); for
// draft row i = m - nP, t_j = s sum_h h_dr[i][h] A_t[j][h] (fp64 sum) stored as bf16 t_hi (columns
// 0..r-1) and t_lo = t - t_hi (columns r..2r-1), zero up to kx.
__global__ __launch_bounds__(kThreads) void k_lora_aug_rows(const uint16_t* __restrict__ hd,
                                                            const uint16_t* __restrict__ at, int nP,
                                                            int K, int r, int kx, float scale,
                                                            uint16_t* __restrict__ taug) {
  const int m = blockIdx.x;
  uint16_t* out = taug + (int64_t)m * kx;
  if (m < nP) {
    for (int j = threadIdx.x; j < kx; j += kThreads) out[j] = 0;
    return;
  }
  const uint16_t* x = hd + (int64_t)(m - nP) * K;
  for (int j = threadIdx.x + 2 * r; j < kx; j += kThreads) out[j] = 0;
  // all ranks in one pass over h: each thread owns 8-element chunks of h (K is a multiple of 64)
  // and keeps up to 16 fp64 partial sums per round
  const int nc = K >> 3;
  for (int j0 = 0; j0 < r; j0 += 16) {
    const int nj = min(16, r - j0);
    double acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0;
    for (int c = threadIdx.x; c < nc; c += kThreads) {
      const u32x4 xw = *reinterpret_cast<const u32x4*>(x + 8 * c);
      double xv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[2 * e] = (double)__uint_as_float(xw[e] << 16);
        xv[2 * e + 1] = (double)__uint_as_float(xw[e] & 0xffff0000u);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (q < nj) {
          const u32x4 aw = *reinterpret_cast<const u32x4*>(at + (int64_t)(j0 + q) * K + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[q] += xv[2 * e] * (double)__uint_as_float(aw[e] << 16);
            acc[q] += xv[2 * e + 1] * (double)__uint_as_float(aw[e] & 0xffff0000u);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[q] += __shfl_xor(acc[q], off, 64);
    }
    __shared__ double s_acc[kThreads / 64][16];
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) s_acc[threadIdx.x >> 6][q] = acc[q];
    }
    __syncthreads();
    if (threadIdx.x < nj) {
      double tot = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) tot += s_acc[w][threadIdx.x];
      const int j = j0 + threadIdx.x;
      const float tf = (float)(tot * (double)scale);
      const uint16_t hi = bf16_rne(tf);
      out[j] = hi;
      out[r + j] = bf16_rne(tf - __uint_as_float((uint32_t)hi << 16));
    }
    __syncthreads();
  }
}

// Extra contraction columns of vocab column n: [B_t[n][0..r) | B_t[n][0..r) | 0 ...] up to kx.
__global__ __launch_bounds__(kThreads) void k_lora_aug_cols(const uint16_t* __restrict__ bt, int N,
                                                            int r, int kx,
                                                            uint16_t* __restrict__ baug) {
  // one thread per 8-column chunk of an augmented row (kx is a multiple of 64)
  const int cpr = kx >> 3;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)N * cpr) return;
  const int n = (int)(idx / cpr);
  const int j0 = 8 * (int)(idx - (int64_t)n * cpr);
  const uint16_t* src = bt + (int64_t)n * r;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t v2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = j0 + 2 * e + k;
      v2[k] = j < r ? src[j] : (j < 2 * r ? src[j - r] : 0u);
    }
    w[e] = v2[0] | (v2[1] << 16);
  }
  *reinterpret_cast<u32x4*>(baug + (int64_t)n * kx + j0) = u32x4{w[0], w[1], w[2], w[3]};
}

__global__ __launch_bounds__(kThreads, 1) void k_lmhead_gemm(LMHeadArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_STAGE + B_STAGE)];
  // XCD-aware tile order: workgroup ids are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, M tiles fastest, so the XCD's workgroups share W column blocks.
  const int ntile = a.mtiles * a.ntiles;
  const int per_xcd = (int)((gridDim.x + kXcd - 1) / kXcd);
  const int tile = (int)(blockIdx.x % kXcd) * per_xcd + (int)(blockIdx.x / kXcd);
  if (tile >= ntile) return;
  const int tm = tile % a.mtiles, tn = tile / a.mtiles;
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K;

  // global -> register staging: 8 A and 8 B 16-byte chunks per thread per K step; rows past the
  // end are clamped (loaded, never stored).  Steps past K read the LoRA columns (kx of them): row m
  // of taug (zeros for the AR rows) and row n of baug.  Row pointers are fixed per thread, so the
  // loop only adds the step offset (kt is uniform: the two phases are a scalar branch).
  const uint16_t* pa[8];
  const uint16_t* pb[8];
  int ma[8], nb[8];
  const int kc = (t & 7) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ma[i] = min(m0 + (t >> 3) + 32 * i, a.M - 1);
    nb[i] = min(n0 + (t >> 3) + 32 * i, a.N - 1);
    pa[i] = (ma[i] < a.nP ? a.h_ar + (int64_t)ma[i] * K : a.h_dr + (int64_t)(ma[i] - a.nP) * K) + kc;
    pb[i] = a.w_t + (int64_t)nb[i] * K + kc;
  }
  const int KT = K / BK, KTX = KT + a.kx / BK;
  u32x4 ra[8], rb[8];
  auto gload = [&](int kt) {
    if (kt < KT) {
      const int ko = kt * BK;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + ko);
        rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + ko);
      }
    } else {
      const int ko = (kt - KT) * BK + kc;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(a.taug + (int64_t)ma[i] * a.kx + ko);
        rb[i] = *reinterpret_cast<const u32x4*>(a.baug + (int64_t)nb[i] * a.kx + ko);
      }
    }
  };
  const int lofs = (t >> 3) * LROW + kc;  // + 32*i*LROW
  auto lstore = [&](int buf) {
    uint16_t* As = smem + buf * (A_STAGE + B_STAGE);
    uint16_t* Bs = As + A_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(As + lofs + 32 * i * LROW) = ra[i];
      *reinterpret_cast<u32x4*>(Bs + lofs + 32 * i * LROW) = rb[i];
    }
  };
  gload(0);
  lstore(0);
  __syncthreads();

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int frag = (lane & 31) * LROW + 8 * (lane >> 5);
  for (int kt = 0; kt < KTX; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KTX) gload(kt + 1);
    const uint16_t* As = smem + buf * (A_STAGE + B_STAGE) + (wm * 128) * LROW + frag;
    const uint16_t* Bs = smem + buf * (A_STAGE + B_STAGE) + A_STAGE + (wn * 128) * LROW + frag;
    // fragments of substep ks+1 are read from LDS while the 16 MFMAs of substep ks run
    bf16x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[0][i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * LROW);
      fb[0][i] = *reinterpret_cast<const bf16x8*>(Bs + i * 32 * LROW);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[cur ^ 1][i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * LROW + (ks + 1) * 16);
          fb[cur ^ 1][i] = *reinterpret_cast<const bf16x8*>(Bs + i * 32 * LROW + (ks + 1) * 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads of ks+1 ahead of the MFMAs of ks
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < KTX) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------------------------
  // Element (i, j, v) of this lane sits at row m0 + wm*128 + i*32 + 8*(v/4) + 4*(lane/32) + v%4,
  // column n0 + wn*128 + j*32 + lane%32.  One 64-row slice (i fixed) at a time goes through LDS:
  // then 4 threads per row store 64 columns each with 16-byte writes and fold them into the row's
  // online pair (max, sum exp) for this column tile.
  constexpr int SROW = BN + 4;
  float* S = reinterpret_cast<float*>(smem);  // [64][SROW]
  const float c = a.c;
  const int lr = t >> 2, qq = t & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        S[rr * SROW + wn * 128 + j * 32 + (lane & 31)] = acc[i][j][v];
      }
    __syncthreads();
    const int m = m0 + (lr < 32 ? i * 32 + lr : 128 + i * 32 + (lr - 32));
    const int nbase = n0 + qq * 64;
    const float* src = S + lr * SROW + qq * 64;
    float mx = kNegBig, sm = 0.f;
    float4 buf[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      buf[k] = *reinterpret_cast<const float4*>(src + 4 * k);
      const float x[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = (nbase + 4 * k + e < a.N) ? x[e] : -__builtin_huge_valf();
        if (xv > mx) {
          sm *= exp2f((mx - xv) * c);
          mx = xv;
        }
        sm += exp2f((xv - mx) * c);
      }
    }
    if (m < a.M) {
      float* dst = a.logits + (int64_t)m * a.N + nbase;
      if (nbase + 64 <= a.N && (a.N & 3) == 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k) *reinterpret_cast<float4*>(dst + 4 * k) = buf[k];
      } else {
        for (int k = 0; k < 64; ++k)
          if (nbase + k < a.N) dst[k] = src[k];
      }
    }
#pragma unroll
    for (int off = 1; off <= 2; off <<= 1) {
      const float m2 = __shfl_xor(mx, off, 64);
      const float s2 = __shfl_xor(sm, off, 64);
      os_combine(mx, sm, m2, s2, c);
    }
    if (qq == 0 && m < a.M) a.part[(int64_t)m * a.ntiles + tn] = make_float2(mx, sm);
    __syncthreads();
  }
}

}  // namespace

int lmhead_tile_n() { return BN; }

hipError_t launch_lmhead(const LMHeadArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.kx > 0) {
    timing_begin("lora_aug", stream);
    hipLaunchKernelGGL(k_lora_aug_rows, dim3((unsigned)a.M), dim3(kThreads), 0, stream, a.h_dr,
                       a.lora_at, a.nP, a.K, a.r, a.kx, a.lora_scale, a.taug);
    const int64_t n = (int64_t)a.N * (a.kx >> 3);
    hipLaunchKernelGGL(k_lora_aug_cols, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a.lora_bt, a.N, a.r, a.kx, a.baug);
    timing_end("lora_aug", stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int ntile = a.mtiles * a.ntiles;
  const unsigned grid = (unsigned)((ntile + kXcd - 1) / kXcd * kXcd);
  timing_begin("lmhead_gemm", stream);
  hipLaunchKernelGGL(k_lmhead_gemm, dim3(grid), dim3(kThreads), 0, stream, a);
  timing_end("lmhead_gemm", stream);
  return hipGetLastError();
}

}  // namespace psispec
