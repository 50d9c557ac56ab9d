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

constexpr int BM = 256, BN = 256, BK = 32, NSTAGE = 4;
constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per LDS stage: A tile then B tile (32 KB)
constexpr int kDma = BM * BK * 2 / 1024 / 4;  // 1 KB direct-to-LDS blocks per wave per operand
constexpr int kXcd = 8;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer resource: 32-bit data, no swizzle

__device__ inline uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Row m of the augmented A operand (grid over all M rows), KX = K + kx columns: the hidden state
// (h_ar row m for m < nP, h_dr row m - nP after), then the extra contraction columns: zeros for the
// AR rows; for draft row i = m - nP, t_j = s sum_h h_dr[i][h] A_t[j][h] (fp64 sum) stored as bf16
// t_hi (columns K..K+r-1) and t_lo = t - t_hi (columns K+r..K+2r-1), zero up to KX.
__global__ __launch_bounds__(kThreads) void k_build_a(const uint16_t* __restrict__ har,
                                                      const uint16_t* __restrict__ hd,
                                                      const uint16_t* __restrict__ at, int nP,
                                                      int K, int r, int kx, float scale,
                                                      uint16_t* __restrict__ aaug) {
  const int m = blockIdx.x;
  const int KX = K + kx;
  uint16_t* row = aaug + (int64_t)m * KX;
  const uint16_t* x = m < nP ? har + (int64_t)m * K : hd + (int64_t)(m - nP) * K;
  const int nc = K >> 3;  // K is a multiple of 64: whole 16-byte chunks
  for (int c = threadIdx.x; c < nc; c += kThreads)
    *reinterpret_cast<u32x4*>(row + 8 * c) = *reinterpret_cast<const u32x4*>(x + 8 * c);
  uint16_t* out = row + K;
  if (m < nP) {
    for (int j = threadIdx.x; j < kx; j += kThreads) out[j] = 0;
    return;
  }
  for (int j = threadIdx.x + 2 * r; j < kx; j += kThreads) out[j] = 0;
  // all ranks in one pass over h: each thread owns 8-element chunks of h and keeps up to 16 fp64
  // partial sums per round
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

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory operations are in
// flight, leaving the LDS and export counters unconstrained.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__global__ __launch_bounds__(kThreads, 1) void k_lmhead_gemm(LMHeadArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NSTAGE * STAGE];
  // XCD-aware tile order: workgroup ids are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, M tiles fastest, so the XCD's workgroups share W column blocks.
  const int ntile = a.mtiles * a.ntiles;
  const int per_xcd = (int)((gridDim.x + kXcd - 1) / kXcd);
  const int tile = (int)(blockIdx.x % kXcd) * per_xcd + (int)(blockIdx.x / kXcd);
  if (tile >= ntile) return;
  const int tm = tile % a.mtiles, tn = tile / a.mtiles;
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS bases go to M0
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K;

  // Operands stream HBM -> LDS with 16-byte direct-to-LDS buffer loads, NSTAGE-1 K steps ahead of
  // the MFMAs.  Each load instruction fills one 1 KB block: 16 rows of 32 bf16, lane l writing row
  // l/4, 16-byte slot l%4.  Slot s of row r holds the row's K chunk s ^ f(r), f(r) = r2 | (r1^r3)<<1
  // (r_k = bit k of r): the 16-byte fragment reads then hit distinct banks both within each group
  // of 8 rows on 32 banks and within each group of 16 rows on 64 banks.  The buffer resources
  // cover only this tile's valid rows: rows past M or N, and the steps past the end (a zero-length
  // resource), land as zeros.  A is the augmented [M][K + kx] matrix; B is W_t for the first K/32
  // steps and the augmented LoRA columns [N][kx] after.
  const int KX = K + a.kx;
  const int rows_a = min(BM, a.M - m0), rows_b = min(BN, a.N - n0);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.aaug + (int64_t)m0 * KX), (short)0, rows_a * KX * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w_t + (int64_t)n0 * K), (short)0, rows_b * K * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.baug + (int64_t)n0 * a.kx), (short)0, rows_b * a.kx * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.w_t, (short)0, 0, kRsrcWord3);
  const int drow = wave * kDma * 16 + (lane >> 2);  // + 16 i
  const int gch = (lane & 3) ^ (((lane >> 4) & 1) | ((((lane >> 3) ^ (lane >> 5)) & 1) << 1));
  const int va = drow * KX * 2 + 16 * gch;
  const int vw = drow * K * 2 + 16 * gch;
  const int vx = drow * a.kx * 2 + 16 * gch;
  const int KT = K / BK, KTX = KT + a.kx / BK;
  auto dma = [&](int kt) {
    uint16_t* As = smem + (kt % NSTAGE) * STAGE + wave * kDma * 512;
    uint16_t* Bs = As + BM * BK;
    const bool live = kt < KTX, main = kt < KT;
    const __amdgpu_buffer_rsrc_t ra = live ? rs_a : rs_0;
    const __amdgpu_buffer_rsrc_t rb = live ? (main ? rs_w : rs_x) : rs_0;
    const int oa = va + kt * (BK * 2);
    const int ob = main ? vw + kt * (BK * 2) : vx + (kt - KT) * (BK * 2);
    const int sa = 16 * KX * 2, sb = 16 * (main ? K : a.kx) * 2;
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(As + i * 512), 16, oa + i * sa, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(Bs + i * 512), 16, ob + i * sb, 0, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // fragment of MFMA row/column l%32, K chunk 2 ks + l/32 (8 bf16), through the slot swizzle
  const int xr = ((lane >> 2) & 1) | ((((lane >> 1) ^ (lane >> 3)) & 1) << 1);
  const int fofs0 = (lane & 31) * BK + 8 * ((lane >> 5) ^ xr);
  const int fofs1 = (lane & 31) * BK + 8 * ((2 + (lane >> 5)) ^ xr);
  bf16x8 fa[2][4], fb[2][4];
  auto fread = [&](int kt, int ks, bf16x8(&ra)[4], bf16x8(&rb)[4]) {
    const uint16_t* As = smem + (kt % NSTAGE) * STAGE + (wm * 128) * BK + (ks ? fofs1 : fofs0);
    const uint16_t* Bs = As + BM * BK + (wn - wm) * 128 * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * BK);
      rb[i] = *reinterpret_cast<const bf16x8*>(Bs + i * 32 * BK);
    }
  };
  auto mfma16 = [&](const bf16x8(&ra)[4], const bf16x8(&rb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i], rb[j], acc[i][j], 0, 0, 0);
  };

#pragma unroll
  for (int k = 0; k < NSTAGE - 1; ++k) dma(k);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSTAGE - 2) * 2 * kDma));  // step 0 landed
  __builtin_amdgcn_s_barrier();
  fread(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < KTX; ++kt) {
    // One barrier per step.  Past it, step kt+1 has landed for every wave (each waited for its own
    // loads of it) and every wave is done with step kt-1, whose stage the loads of step
    // kt+NSTAGE-1 then overwrite.  Everything else in the step is free to overlap the MFMAs.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSTAGE - 3) * 2 * kDma));
    __builtin_amdgcn_s_barrier();
    fread(kt, 1, fa[1], fb[1]);
    dma(kt + NSTAGE - 1);
    mfma16(fa[0], fb[0]);
    fread(kt + 1, 0, fa[0], fb[0]);
    mfma16(fa[1], fb[1]);
    // issue order: one fragment read after each of the first 8 MFMAs, one DMA load after each of
    // the next 8, then the reads of step kt+1 between the first 8 MFMAs of substep 1
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (direct-to-LDS)
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the zero-filling tail loads also write LDS
  __syncthreads();

  // ---- epilogue -------------------------------------------------------------------------------
  // Element (i, j, v) of this lane sits at row m0 + wm*128 + i*32 + 8*(v/4) + 4*(lane/32) + v%4,
  // column n0 + wn*128 + j*32 + lane%32.  One 64-row slice (i fixed) at a time goes through LDS:
  // then 4 threads per row reduce 64 columns each to the segment's (max, sum exp2((x - max) c)),
  // combined over the row's 4 segments, and each wave stores 16 of the slice's rows, one row of
  // 256 columns per 1 KB coalesced instruction.
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
    const int nvalid = a.N - (n0 + qq * 64);  // columns of this segment inside the row (may be <= 0)
    const float* src = S + lr * SROW + qq * 64;
    float4 buf[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) buf[k] = *reinterpret_cast<const float4*>(src + 4 * k);
    // segment max and sum, four independent chains each (a finite floor: a segment past the row's
    // end gives (floor, 0)); the chains are combined in a fixed order
    float mq[4] = {kNegBig, kNegBig, kNegBig, kNegBig};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float x[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * k + e < nvalid) mq[e] = fmaxf(mq[e], x[e]);
    }
    const float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float x[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * k + e < nvalid) sq[e] += __builtin_amdgcn_exp2f((x[e] - mx) * c);
    }
    float sm = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    float mxc = mx;
#pragma unroll
    for (int off = 1; off <= 2; off <<= 1) {
      const float m2 = __shfl_xor(mxc, off, 64);
      const float s2 = __shfl_xor(sm, off, 64);
      os_combine(mxc, sm, m2, s2, c);
    }
    if (qq == 0 && m < a.M) a.part[(int64_t)m * a.ntiles + tn] = make_float2(mxc, sm);
    // logits: one wave writes one row's 256 columns per instruction (16 rows per wave)
    const int ncol = min(BN, a.N - n0);
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
      const int sr = wave * 16 + q;  // slice row
      const int mr = m0 + (sr < 32 ? i * 32 + sr : 128 + i * 32 + (sr - 32));
      if (mr >= a.M) continue;
      const float4 v4 = *reinterpret_cast<const float4*>(S + sr * SROW + 4 * lane);
      float* dst = a.logits + (int64_t)mr * a.N + n0 + 4 * lane;
      if (4 * lane + 4 <= ncol && (a.N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = v4;
      } else {
        const float e4[4] = {v4.x, v4.y, v4.z, v4.w};
        for (int e = 0; e < 4; ++e)
          if (4 * lane + e < ncol) dst[e] = e4[e];
      }
    }
    __syncthreads();
  }
}

}  // namespace

int lmhead_tile_n() { return BN; }
int lmhead_tile_m() { return BM; }

hipError_t launch_lmhead(const LMHeadArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  timing_begin("build_a", stream);
  hipLaunchKernelGGL(k_build_a, dim3((unsigned)a.M), dim3(kThreads), 0, stream, a.h_ar, a.h_dr,
                     a.lora_at, a.nP, a.K, a.r, a.kx, a.lora_scale, a.aaug);
  if (a.kx > 0) {
    const int64_t n = (int64_t)a.N * (a.kx >> 3);
    hipLaunchKernelGGL(k_lora_aug_cols, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a.lora_bt, a.N, a.r, a.kx, a.baug);
  }
  timing_end("build_a", stream);
  {
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
