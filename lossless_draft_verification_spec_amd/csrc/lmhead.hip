// lmhead.hip -- the LM head feeding the verify: logits = h W (+ LoRA on the draft rows) on MFMA.
//
// [lanes] §"헤드냐, LoRA냐": the draft path is the frozen AR weights plus a low-rank LoRA delta, the
// verify path the frozen AR weights alone; [alphalab] walkthrough step 2 (draft rows through the
// LoRA path) and step 3 (the AR scores the block).  Only the output projection is built here:
//   p rows (AR):    logits[m] = h_ar[m] . W
//   q rows (draft): logits[m] = h_dr[m] . W + s (h_dr[m] . A) . B
// with W [H][V], A [H][r], B [r][V] (bf16, V contiguous in W and B).  The product is the one dense
// contraction of the verify step, so it runs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).
//
// Operands.  The A operand (hidden states plus LoRA columns) is staged by k_build_a in a K-step
// blocked layout, [K/32][Mpad][32]: the 32 contraction columns of one K step of a whole M tile are
// one contiguous block, so every load of it fills whole cache lines.  The LoRA delta rides in the
// same MFMA loop as extra contraction columns: t = s (h_dr . A) is summed in fp64, rounded to fp32
// and split into bf16 t_hi + t_lo (relative error 2^-17, far below the fp32 accumulation error of
// the H-long product); the extra K steps multiply [t_hi | t_lo | 0] by the rows [B | B | 0]
// (zeros for the AR rows).  W and B are read in place, V contiguous: each K step of a tile is 32
// rows of BN contiguous columns.  The MFMA wants eight consecutive contraction values of one
// column per lane, so the B fragments come out of LDS through gfx950's transposing read
// (ds_read_b64_tr_b16: a 16-lane group reads a 4 x 16 block and each lane receives one column's
// four values).
//
// Tiling.  A 256 x 256 output tile per 512-thread workgroup: eight wave64s (two per SIMD), each
// owning a 128 x 64 block (4 x 2 MFMA tiles of 32 x 32), so one wave's MFMAs overlap the other's
// LDS reads.  K steps of 32 go through NSTAGE LDS stages filled by 16-byte direct-to-LDS buffer
// loads NSTAGE-1 steps ahead (no register staging), one barrier per step.  When the rows end in a
// band of at most 128, that band uses 128 x 512 tiles instead (the same staging and the same
// 128 x 64 wave blocks, eight side by side), so the short band costs half the tiles of a padded
// 256-row band.  Tiles form column groups (256 columns, or 512 with a short last band) with the
// M tiles fastest; workgroup ids are dealt round-robin to the 8 XCDs, and each XCD takes a
// contiguous range of groups, so the workgroups that share a W column block run on one XCD at
// the same time and share it through that XCD's L2.
//
// Epilogue.  The logits are not stored.  Per row and 256-column segment it emits the softmax pair
// (max, sum exp2((x - max) log2e / T)) that the verify combines in place of an HBM row pass, and
// the logit at the row's draft token (its one column tile writes it), which the accept test
// needs.  Storing the logits is an option, used for the stopping rows that the final draw reads
// (recomputed by a second launch over just those rows: the same kernel and K order give the same
// bits) and for a caller who asks for them.
#include <type_traits>

#include "launch.h"

namespace psispec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int BK = 32;                  // contraction columns per K step
constexpr int kXcd = 8;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer resource: 32-bit data, no swizzle

__device__ inline uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// The transposing LDS read.  The restrict-qualified (inlined) parameter gives the access an alias
// scope, so the compiler does not add a wait for every direct-to-LDS load in flight before it: the
// kernel orders those loads and the reads itself (explicit vmcnt waits and a barrier per K step).
__device__ __attribute__((always_inline)) inline bf16x4 tr_read(const lds_bf16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

__device__ inline float bf16_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Row m of the staged A operand ([KTX][Mpad][32], KTX = (K + kx) / 32): the hidden state of source
// row src (h_ar row src for src < nP, h_dr row src - nP after; zeros for src < 0), then the extra
// contraction columns: zeros for the AR rows; for a draft row, t_j = s sum_h h[h] A[h][j] (fp64
// sum, rounded to fp32) stored as bf16 t_hi (columns K..K+r-1) and t_lo = t - t_hi (columns
// K+r..K+2r-1), zero up to K + kx.  Source rows: m itself (m < nP + nQ), or with a draw list the
// stopping rows of request m / 2 (row 2r = p row of the draw, 2r + 1 = its q row); that form also
// rewrites the draw's descriptor and row statistics for the recomputed rows (2r and 2r + 1).
struct BuildArgs {
  const uint16_t* h_ar;
  const uint16_t* h_dr;
  const uint16_t* lora_a;  // [K][r]
  float lora_scale;
  int nP, nQ, K, r, kx, Mpad;
  int nrows;               // rows with a source (the rest of Mpad is zero)
  const DrawDesc* desc;    // null: identity rows
  const RowStat* rowstat;
  DrawDesc* desc2;
  RowStat* rowstat2;
  uint16_t* ablk;
};

__global__ __launch_bounds__(kThreads) void k_build_a(BuildArgs a) {
  const int m = blockIdx.x;
  int src = -1;
  if (m < a.nrows) {
    if (!a.desc) {
      src = m;
    } else {
      const DrawDesc d = a.desc[m >> 1];
      src = (m & 1) ? d.qrow : d.prow;
      if (threadIdx.x == 0) {
        if (src >= 0) a.rowstat2[m] = a.rowstat[src];
        if ((m & 1) == 0) {
          DrawDesc d2 = d;
          d2.prow = m;
          d2.qrow = d.qrow >= 0 ? m + 1 : -1;
          a.desc2[m >> 1] = d2;
        }
      }
    }
  }
  const int64_t kstride = (int64_t)a.Mpad * BK;  // elements from one K step's block to the next
  uint16_t* dst = a.ablk + (int64_t)m * BK;
  const int nc = a.K >> 3;  // 16-byte chunks of the hidden state
  const uint16_t* x = src < 0 ? nullptr
                    : src < a.nP ? a.h_ar + (int64_t)src * a.K
                                 : a.h_dr + (int64_t)(src - a.nP) * a.K;
  for (int c = threadIdx.x; c < nc; c += kThreads) {
    const u32x4 v = x ? *reinterpret_cast<const u32x4*>(x + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(dst + (c >> 2) * kstride + 8 * (c & 3)) = v;
  }
  if (a.kx == 0) return;
  uint16_t* ext = dst + (a.K / BK) * kstride;  // the extra columns: one or more K steps
  const bool draft_row = src >= a.nP;
  for (int j = threadIdx.x + (draft_row ? 2 * a.r : 0); j < a.kx; j += kThreads)
    ext[(j / BK) * kstride + (j % BK)] = 0;
}

// The LoRA columns of the draft rows of the staged A operand (rows as k_build_a takes them; other
// rows return at once).
__global__ __launch_bounds__(kThreads) void k_build_lora(BuildArgs a) {
  const int m = blockIdx.x;
  if (m >= a.nrows) return;
  int src = m;
  if (a.desc) {
    const DrawDesc d = a.desc[m >> 1];
    src = (m & 1) ? d.qrow : d.prow;
  }
  if (src < a.nP) return;  // an AR row (or none): its extra columns are zero
  const int64_t kstride = (int64_t)a.Mpad * BK;
  uint16_t* ext = a.ablk + (int64_t)m * BK + (a.K / BK) * kstride;
  auto put = [&](int j, uint16_t v) { ext[(j / BK) * kstride + (j % BK)] = v; };
  const uint16_t* x = a.h_dr + (int64_t)(src - a.nP) * a.K;
  // t_j = s sum_h x[h] A[h][j], 16 ranks at a time: each thread takes 8 consecutive h per round
  // (x from one 16-byte word, A's 8 rows loaded together), summed in h order in fp64; the
  // threads' sums are reduced in a fixed order (wave butterflies, then the 4 waves).
  __shared__ double s_acc[kThreads / 64][16];
  const bool vec = (a.r % 8) == 0 && ((uintptr_t)a.lora_a % 16) == 0;
  for (int j0 = 0; j0 < a.r; j0 += 16) {
    const int nj = min(16, a.r - j0);
    double acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0;
    for (int h0 = 8 * threadIdx.x; h0 < a.K; h0 += 8 * kThreads) {
      const u32x4 xw = *reinterpret_cast<const u32x4*>(x + h0);
      u32x4 raw[8][2];
      if (vec) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint16_t* row = a.lora_a + (int64_t)(h0 + k) * a.r + j0;
#pragma unroll
          for (int w = 0; w < 2; ++w)
            raw[k][w] = 8 * w < nj ? *reinterpret_cast<const u32x4*>(row + 8 * w)
                                   : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int w = 0; w < 2; ++w)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q0 = 8 * w + 2 * e;
              const uint16_t* row = a.lora_a + (int64_t)(h0 + k) * a.r + j0;
              const uint32_t lo = q0 < nj ? row[q0] : 0u, hi = q0 + 1 < nj ? row[q0 + 1] : 0u;
              raw[k][w][e] = lo | (hi << 16);
            }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t xk = xw[k >> 1];
        const double xd = (double)__uint_as_float((k & 1) ? (xk & 0xffff0000u) : (xk << 16));
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[8 * w + 2 * e] += xd * (double)__uint_as_float(raw[k][w][e] << 16);
            acc[8 * w + 2 * e + 1] += xd * (double)__uint_as_float(raw[k][w][e] & 0xffff0000u);
          }
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[q] += __shfl_xor(acc[q], off, 64);
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) s_acc[threadIdx.x >> 6][q] = acc[q];
    }
    __syncthreads();
    if (threadIdx.x < nj) {
      double tot = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) tot += s_acc[w][threadIdx.x];
      const int jj = j0 + threadIdx.x;
      const float tf = (float)(tot * (double)a.lora_scale);
      const uint16_t hi = bf16_rne(tf);
      put(jj, hi);
      put(a.r + jj, bf16_rne(tf - bf16_f(hi)));
    }
    __syncthreads();
  }
}

struct GemmArgs {
  const uint16_t* ablk;    // [KTX][Mpad][32]
  const uint16_t* w;       // [K][N]
  const uint16_t* lora_b;  // [r][N] or null
  int M, Mpad, N, K, r, KT, KTX;
  // Tiles: full 256-row bands of 256 x 256 tiles; a last band of at most 128 rows takes 128 x 512
  // tiles instead (no MFMA work on padding rows).  Tiles are numbered by column group (256 columns,
  // or 512 with such a band), bands fastest within a group, the 128 x 512 tile last.
  int fbands;              // full bands (256 x 256 tiles)
  int tailB;               // 1: a last band of 128 x 512 tiles
  int gcols;               // columns per group: 256, or 512 with tailB
  int per_group;           // tiles per group: fbands (x2 with tailB) + tailB
  int ngroups;
  int ntiles;              // 256-column tiles of a row (row pairs per row)
  float c;                 // log2(e) / T for the row pairs
  float2* part;            // [M][ntiles] row pairs, or null
  const int32_t* draft;    // gather: draft token of each row (linear layout), or null
  int B, nP;
  float* gath;             // [M] logit at the row's draft token
  float* out0;             // logit store, or null: row m < split -> out0 + m N,
  float* out1;             //                        else out1 + (m - split) N
  int split;
};

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory operations are in
// flight, leaving the LDS and export counters unconstrained.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

constexpr int NSTAGE = 4;            // LDS stages
constexpr int kGT = 512;             // threads per workgroup: two waves per SIMD
constexpr int WTM = 128, WTN = 64;   // output tile of one wave
template <int BM_, int BN_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_;
};
using ShapeFull = TileShape<256, 256>;  // full bands
using ShapeTail = TileShape<128, 512>;  // a last band of at most 128 rows
constexpr int kStageMax = (128 + 512) * BK;  // bf16 elements of the larger stage

// One output tile of shape Shp at (m0, n0).
template <class Shp>
__device__ __attribute__((always_inline)) inline void gemm_tile(const GemmArgs& a, Shp, int m0,
                                                                int n0, uint16_t* smem) {
  constexpr int BM = Shp::BM, BN = Shp::BN;
  constexpr int kWaves = kGT / 64;
  constexpr int WN = BN / WTN, WM = BM / WTM;
  static_assert(WM * WN == kWaves, "the wave tiles cover the output tile");
  constexpr int NI = WTM / 32, NJ = WTN / 32;  // 32 x 32 MFMA blocks of a wave tile
  constexpr int STAGE = kStageMax;             // bf16 elements per LDS stage: A block, then B block
  static_assert((BM + BN) * BK <= STAGE, "a stage holds the tile's K step");
  constexpr int nA = BM / 16 / kWaves;         // 1 KB direct-to-LDS loads per wave per step (A)
  constexpr int nB = BN / 16 / kWaves;         // idem (B)
  constexpr int D = nA + nB;
  constexpr int R = NI + 2 * NJ;               // fragment reads per wave per substep
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS bases go to M0
  const int wm = wave / WN, wn = wave % WN;

  // ---- loads ---------------------------------------------------------------------------------
  // A: one load fills 16 rows x 64 B (lane l: row l/4, 16-byte slot l%4).  Slot s of row r holds
  // the row's chunk s ^ f(r), f(r) = r2 | (r1 ^ r3) << 1 (r_k = bit k of r), which keeps the
  // 16-byte fragment reads conflict-free.  The whole K step of the tile is one contiguous block.
  // B: one load fills 512 contiguous columns of the step's 32 rows (BN = 256: two rows).  Slot s
  // of row k holds the row's 8-column chunk s ^ ((k & 3) << 2): the transposing reads of four
  // consecutive rows then fall on distinct banks.  W and the LoRA rows are read through buffer
  // resources whose range ends with the matrix: rows past the end read as zeros (the padding of a
  // last partial K step); columns past N of a last column tile read neighbouring data that only
  // feeds the discarded output columns.
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.ablk, (short)0, (int)((uint32_t)a.KTX * (uint32_t)a.Mpad * 64u), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.ablk, (short)0, 0, kRsrcWord3);
  const int arow = lane >> 2;
  const int ach = (lane & 3) ^ (((arow >> 2) & 1) | ((((arow >> 1) ^ (arow >> 3)) & 1) << 1));
  const int va = (wave * nA * 16 + arow) * 64 + 16 * ach;  // + 1024 i
  int vb[nB], cbo[nB], lrow[nB];
#pragma unroll
  for (int i = 0; i < nB; ++i) {
    const int e = (wave * nB + i) * 512 + lane * 8;  // element within the step's B block
    const int kr = e / BN, s = (e % BN) >> 3;
    cbo[i] = (s ^ ((kr & 3) << 2)) * 16;
    vb[i] = kr * a.N * 2 + cbo[i];
    lrow[i] = kr;
  }
  const int64_t wtotal = (int64_t)a.K * a.N;
  const int64_t lleft = a.lora_b ? 2 * ((int64_t)a.r * a.N - n0) : 0;
  const int nrow2 = a.N * 2;
  // A K step's loads.  kW: a step of W (no branch, so that the loads interleave with the MFMAs of
  // one basic block); otherwise any step: W, a LoRA step, or past the end (zero-length resource).
  auto dma = [&](int kt, auto kW) {
    uint16_t* As = smem + (kt % NSTAGE) * STAGE + wave * nA * 512;
    uint16_t* Bs = smem + (kt % NSTAGE) * STAGE + BM * BK + wave * nB * 512;
    const bool live = decltype(kW)::value || kt < a.KTX;
    const __amdgpu_buffer_rsrc_t ra = live ? rs_a : rs_0;
    const int soa = live ? (kt * a.Mpad + m0) * 64 : 0;
#pragma unroll
    for (int i = 0; i < nA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(As + i * 512), 16, va + i * 1024,
                                               soa, 0, 0);
    const int64_t wbase = (int64_t)kt * BK * a.N + n0;
    const int64_t wleft = 2 * (wtotal - wbase);
    const auto w_rsrc = [&]() {
      return __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.w + wbase), (short)0,
          (int)(uint32_t)(wleft > 0xffffffffll ? 0xffffffffll : wleft), kRsrcWord3);
    };
    if constexpr (decltype(kW)::value) {
      const __amdgpu_buffer_rsrc_t rb = w_rsrc();
#pragma unroll
      for (int i = 0; i < nB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(Bs + i * 512), 16, vb[i], 0, 0, 0);
    } else if (kt < a.KT) {
      const __amdgpu_buffer_rsrc_t rb = w_rsrc();
#pragma unroll
      for (int i = 0; i < nB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(Bs + i * 512), 16, vb[i], 0, 0, 0);
    } else {
      const int64_t left = live ? lleft : 0;
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.lora_b ? a.lora_b + n0 : a.w), (short)0, (int)(uint32_t)left, kRsrcWord3);
      const int jb = (kt - a.KT) * BK;
#pragma unroll
      for (int i = 0; i < nB; ++i) {
        // extra column j of a LoRA step: LoRA row j (t_hi), j - r (t_lo), none past 2r
        const int j = jb + lrow[i];
        const int lr = j < a.r ? j : j - a.r;
        const int off = j < 2 * a.r ? lr * nrow2 + cbo[i] : (int)left;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(Bs + i * 512), 16, off, 0, 0, 0);
      }
    }
  };
  using kWStep = std::integral_constant<bool, true>;
  using kAnyStep = std::integral_constant<bool, false>;

  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // ---- fragments -----------------------------------------------------------------------------
  // A: MFMA row l%32, contraction chunk 2 ks + l/32 (8 values), through the slot swizzle.
  const int xr = ((lane >> 2) & 1) | ((((lane >> 1) ^ (lane >> 3)) & 1) << 1);
  const int fofs0 = (lane & 31) * BK + 8 * ((lane >> 5) ^ xr);
  const int fofs1 = (lane & 31) * BK + 8 * ((2 + (lane >> 5)) ^ xr);
  // B: lane l of 16-lane group g reads 8 bytes at contraction row 8 (g / 2) + 4 h + (l % 16) / 4,
  // columns 16 (g % 2) + 4 (l % 4) .. +3 of the MFMA column block; it receives column
  // 16 (g % 2) + l % 16 at four consecutive contraction rows.  Byte offsets within the stage's B
  // block, per column block j (h and ks are immediate offsets).
  const int g = lane >> 4, q = lane & 15;
  int bofs[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int k = 8 * (g >> 1) + (q >> 2);
    const int n = wn * WTN + 32 * j + 16 * (g & 1) + 4 * (q & 3);
    const int chunk = (n >> 3) ^ ((k & 3) << 2);
    bofs[j] = k * BN * 2 + chunk * 16 + (n & 7) * 2;
  }
  bf16x8 fa[2][NI], fb[2][NJ];
  auto fread = [&](int kt, int ks, bf16x8(&ra)[NI], bf16x8(&rb)[NJ]) {
    const uint16_t* As = smem + (kt % NSTAGE) * STAGE + (wm * WTM) * BK + (ks ? fofs1 : fofs0);
    const char* Bs = reinterpret_cast<const char*>(smem + (kt % NSTAGE) * STAGE + BM * BK) +
                     ks * 16 * BN * 2;
#pragma unroll
    for (int i = 0; i < NI; ++i) ra[i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bf16x4 lo = tr_read((const lds_bf16x4*)(Bs + bofs[j]));
      const bf16x4 hi = tr_read((const lds_bf16x4*)(Bs + bofs[j] + 4 * BN * 2));
      rb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto mfma_sub = [&](const bf16x8(&ra)[NI], const bf16x8(&rb)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i], rb[j], acc[i][j], 0, 0, 0);
  };

  const int KTX = a.KTX;
#pragma unroll
  for (int k = 0; k < NSTAGE - 1; ++k) dma(k, kAnyStep{});
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSTAGE - 2) * D));  // step 0 landed
  __builtin_amdgcn_s_barrier();
  fread(0, 0, fa[0], fb[0]);
  auto step = [&](int kt, auto kW) {
    // One barrier per step.  Past it, step kt+1 has landed for every wave (each waited for its own
    // loads of it) and every wave is done with step kt-1, whose stage the loads of step
    // kt+NSTAGE-1 then overwrite.  Everything else in the step is free to overlap the MFMAs.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSTAGE - 3) * D));
    __builtin_amdgcn_s_barrier();
    fread(kt, 1, fa[1], fb[1]);
    dma(kt + NSTAGE - 1, kW);
    mfma_sub(fa[0], fb[0]);
    fread(kt + 1, 0, fa[0], fb[0]);
    mfma_sub(fa[1], fb[1]);
    // issue order: the fragment reads of substep 1 between the MFMAs of substep 0; the step's
    // loads and the reads of step kt+1 between the MFMAs of substep 1
#pragma unroll
    for (int k = 0; k < NI * NJ; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
      if (k < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
#pragma unroll
    for (int k = 0; k < NI * NJ; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
      if (k < D) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read (to LDS)
      if (k < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
  };
  // steps whose look-ahead loads are W steps, then the last NSTAGE-1 steps of W and the LoRA steps
  const int kt_w = a.KT - (NSTAGE - 1);
  int kt = 0;
  for (; kt < kt_w; ++kt) step(kt, kWStep{});
  for (; kt < KTX; ++kt) step(kt, kAnyStep{});
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the zero-filling tail loads also write LDS
  __syncthreads();

  // ---- epilogue -------------------------------------------------------------------------------
  // Element (i, j, v) of this lane sits at row m0 + wm*WTM + i*32 + 8*(v/4) + 4*(lane/32) + v%4,
  // column n0 + wn*WTN + j*32 + lane%32.  One slice (i fixed: WM*32 rows) at a time goes through
  // LDS; then TPR threads per row reduce COLS columns each to the segment's
  // (max, sum exp2((x - max) c)), combined over the row's segments in a fixed order.
  constexpr int SR = WM * 32;         // rows per slice
  constexpr int TPR = kGT / SR;       // threads per row
  constexpr int COLS = BN / TPR;      // columns per thread
  constexpr int SROW = BN + 4;
  static_assert(SR * SROW * sizeof(float) <= NSTAGE * STAGE * sizeof(uint16_t),
                "a slice fits in the stages' LDS");
  float* S = reinterpret_cast<float*>(smem);  // [SR][SROW]
  const float c = a.c;
  const int lr = t / TPR, qq = t % TPR;
  const int ncol = min(BN, a.N - n0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        S[rr * SROW + wn * WTN + j * 32 + (lane & 31)] = acc[i][j][v];
      }
    __syncthreads();
    auto slice_row = [&](int sr) { return m0 + (sr >> 5) * WTM + i * 32 + (sr & 31); };
    const int m = slice_row(lr);
    const int nvalid = ncol - qq * COLS;  // columns of this segment inside the row (may be <= 0)
    const float* src = S + lr * SROW + qq * COLS;
    float4 buf[COLS / 4];
#pragma unroll
    for (int k = 0; k < COLS / 4; ++k) buf[k] = *reinterpret_cast<const float4*>(src + 4 * k);
    if (a.part) {
      // segment max and sum, four independent chains each (a finite floor: a segment past the
      // row's end gives (floor, 0)); the chains are combined in a fixed order
      float mq[4] = {kNegBig, kNegBig, kNegBig, kNegBig};
#pragma unroll
      for (int k = 0; k < COLS / 4; ++k) {
        const float x[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * k + e < nvalid) mq[e] = fmaxf(mq[e], x[e]);
      }
      const float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
      float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < COLS / 4; ++k) {
        const float x[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * k + e < nvalid) sq[e] += __builtin_amdgcn_exp2f((x[e] - mx) * c);
      }
      float sm = (sq[0] + sq[1]) + (sq[2] + sq[3]);
      float mxc = mx;
      // one pair per 256 columns (the threads of one 256-column segment, fixed order)
      constexpr int TPS = 256 / COLS;
#pragma unroll
      for (int off = 1; off < TPS; off <<= 1) {
        const float m2 = __shfl_xor(mxc, off, 64);
        const float s2 = __shfl_xor(sm, off, 64);
        os_combine(mxc, sm, m2, s2, c);
      }
      const int seg = n0 / 256 + qq / TPS;
      if (qq % TPS == 0 && m < a.M && seg < a.ntiles)
        a.part[(int64_t)m * a.ntiles + seg] = make_float2(mxc, sm);
    }
    if (a.gath && m < a.M) {
      // the logit at this row's draft token, by the thread whose segment holds it
      int d = -1;
      if (m < a.nP) {
        const int rq = m / (a.B + 1), pos = m - rq * (a.B + 1);
        if (pos < a.B) d = a.draft[(int64_t)rq * a.B + pos];
      } else {
        d = a.draft[m - a.nP];
      }
      const int o = d - (n0 + qq * COLS);
      if (d >= 0 && d < a.N && o >= 0 && o < COLS) a.gath[m] = src[o];
    }
    if (a.out0) {
      // logits: each wave stores SR / kWaves rows of the slice, 256 columns per instruction
      for (int k = 0; k < SR / kWaves; ++k) {
        const int sr = wave * (SR / kWaves) + k;
        const int mr = slice_row(sr);
        if (mr >= a.M) continue;
        float* dst = mr < a.split ? a.out0 + (int64_t)mr * a.N : a.out1 + (int64_t)(mr - a.split) * a.N;
#pragma unroll
        for (int cb = 0; cb < BN; cb += 256) {
          const int col = cb + 4 * lane;
          const float4 v4 = *reinterpret_cast<const float4*>(S + sr * SROW + col);
          if (col + 4 <= ncol) {
            *reinterpret_cast<float4*>(dst + n0 + col) = v4;
          } else {
            const float e4[4] = {v4.x, v4.y, v4.z, v4.w};
            for (int e = 0; e < 4; ++e)
              if (col + e < ncol) dst[n0 + col + e] = e4[e];
          }
        }
      }
    }
    __syncthreads();
  }
}


__global__ __launch_bounds__(kGT, 1) void k_lmhead_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NSTAGE * kStageMax];
  const int per_xcd = (int)(gridDim.x / kXcd);
  const int tile = (int)(blockIdx.x % kXcd) * per_xcd + (int)(blockIdx.x / kXcd);
  if (tile >= a.ngroups * a.per_group) return;
  const int grp = tile / a.per_group, idx = tile - grp * a.per_group;
  const bool tail = a.tailB && idx == a.per_group - 1;
  int m0, n0;
  if (tail) {
    m0 = a.fbands * 256;
    n0 = grp * a.gcols;
  } else {
    m0 = (idx % a.fbands) * 256;
    n0 = grp * a.gcols + (idx / a.fbands) * 256;
  }
  if (n0 >= a.N) return;
  if (tail)
    gemm_tile(a, ShapeTail{}, m0, n0, smem);
  else
    gemm_tile(a, ShapeFull{}, m0, n0, smem);
}

constexpr int kBM = 256, kBN = 256;

int lmhead_mpad(int rows) { return (rows + kBM - 1) / kBM * kBM; }

}  // namespace

int lmhead_tile_n() { return kBN; }

int lmhead_kx(int r) { return r > 0 ? (2 * r + BK - 1) / BK * BK : 0; }

size_t lmhead_ablk_bytes(int rows, int K, int r) {
  return (size_t)lmhead_mpad(rows) * (size_t)(K + lmhead_kx(r)) * 2;
}

namespace {

hipError_t run_gemm(const LMHeadArgs& a, const uint16_t* ablk, int rows, float2* part,
                    const int32_t* draft, int B, float* gath, float* out0, float* out1, int split,
                    hipStream_t stream, const char* name) {
  GemmArgs g{};
  g.ablk = ablk;
  g.w = a.w;
  g.lora_b = a.lora_b;
  g.M = rows;
  g.Mpad = lmhead_mpad(rows);
  g.N = a.N;
  g.K = a.K;
  g.r = a.r;
  g.KT = a.K / BK;
  g.KTX = (a.K + lmhead_kx(a.r)) / BK;
  g.fbands = rows / 256;
  const int rem = rows - 256 * g.fbands;
  g.tailB = rem > 0 && rem <= 128;
  if (rem > 128) g.fbands += 1;  // a last band of more than 128 rows: a padded full band
  g.gcols = g.tailB ? 512 : 256;
  g.per_group = g.tailB ? 2 * g.fbands + 1 : g.fbands;
  g.ngroups = (a.N + g.gcols - 1) / g.gcols;
  g.ntiles = (a.N + kBN - 1) / kBN;
  g.c = a.c;
  g.part = part;
  g.draft = draft;
  g.B = B;
  g.nP = a.nP;
  g.gath = gath;
  g.out0 = out0;
  g.out1 = out1;
  g.split = split;
  const int ntile = g.ngroups * g.per_group;
  const unsigned grid = (unsigned)((ntile + kXcd - 1) / kXcd * kXcd);
  PSISPEC_LAUNCH(name, k_lmhead_gemm, dim3(grid), dim3(kGT), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_main(const LMHeadArgs& a, uint16_t* ablk, const int32_t* draft, int B,
                              float2* part, float* gath, float* out_p, float* out_q,
                              hipStream_t stream) {
  const int M = a.nP + a.nQ;
  if (M == 0) return hipSuccess;
  BuildArgs b{};
  b.h_ar = a.h_ar;
  b.h_dr = a.h_dr;
  b.lora_a = a.lora_a;
  b.lora_scale = a.lora_scale;
  b.nP = a.nP;
  b.nQ = a.nQ;
  b.K = a.K;
  b.r = a.r;
  b.kx = lmhead_kx(a.r);
  b.Mpad = lmhead_mpad(M);
  b.nrows = M;
  b.ablk = ablk;
  PSISPEC_LAUNCH("build_a", k_build_a, dim3((unsigned)b.Mpad), dim3(kThreads), 0, stream, b);
  if (b.kx > 0 && b.r > 0)
    PSISPEC_LAUNCH("build_a_lora", k_build_lora, dim3((unsigned)b.nrows), dim3(kThreads), 0,
                   stream, b);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return run_gemm(a, ablk, M, part, draft, B, gath, out_p, out_q, a.nP, stream, "lmhead_gemm");
}

hipError_t launch_lmhead_rows(const LMHeadArgs& a, uint16_t* ablk, int batch, const DrawDesc* desc,
                              const RowStat* rowstat, DrawDesc* desc2, RowStat* rowstat2,
                              float* out, hipStream_t stream) {
  const int rows = 2 * batch;
  if (rows == 0) return hipSuccess;
  BuildArgs b{};
  b.h_ar = a.h_ar;
  b.h_dr = a.h_dr;
  b.lora_a = a.lora_a;
  b.lora_scale = a.lora_scale;
  b.nP = a.nP;
  b.nQ = a.nQ;
  b.K = a.K;
  b.r = a.r;
  b.kx = lmhead_kx(a.r);
  b.Mpad = lmhead_mpad(rows);
  b.nrows = rows;
  b.desc = desc;
  b.rowstat = rowstat;
  b.desc2 = desc2;
  b.rowstat2 = rowstat2;
  b.ablk = ablk;
  PSISPEC_LAUNCH("build_rows", k_build_a, dim3((unsigned)b.Mpad), dim3(kThreads), 0, stream, b);
  if (b.kx > 0 && b.r > 0)
    PSISPEC_LAUNCH("build_rows_lora", k_build_lora, dim3((unsigned)b.nrows), dim3(kThreads), 0,
                   stream, b);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return run_gemm(a, ablk, rows, nullptr, nullptr, 0, nullptr, out, out, rows, stream,
                  "lmhead_rows");
}

}  // namespace psispec
