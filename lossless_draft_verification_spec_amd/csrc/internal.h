// internal.h -- types and device helpers shared by the HIP kernels of libpsispec (gfx950 only).
//
// Citations use page titles and sections:
//   [alphalab] "Uno Ψ-Spec 是什麼？Diffusion-Augmented LLM 如何保留 AR 分布、一次驗證多個 Token"
//   [lanes]    "Uno / Ψ-Spec — 같은 모델 안에서 초안 뽑고 AR로 도장 찍기"
//   [philox]   Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psispec.h"

namespace psispec {

constexpr int kThreads = 256;       // workgroup size of the streaming kernels (4 wave64)
constexpr int kSub = 1024;          // tokens per sub-chunk of the fp64 residual prefix sums
constexpr int kUncPool = 8192;     // uncertain-sign residual tokens kept per request
constexpr int kMassLds = 2048;     // sub-chunk masses a select keeps in LDS (V <= 2M tokens)
constexpr float kNegBig = -3.40282346638528859812e+38f;  // running-max floor (finite: -inf - floor = -inf)

enum : uint32_t { kPurposeAccept = 0, kPurposeDraw = 1, kPurposeDraft = 2 };

// Rows of one call: rows [0, nP) live in p, pstride elements apart; rows [nP, nP + nQ) in q, V
// elements apart; each row holds V contiguous elements.
struct RowSet {
  const void* p;
  const void* q;
  int64_t nP;
  int64_t nQ;
  int V;
  int qB;          // q rows per request (linear: B), used to skip position-0 q rows
  int skip_q0;     // 1: q rows at position 0 are not read (first-from-target layout)
  int64_t pstride; // elements from one p row to the next (V for packed rows)
};

// Per-row softmax statistics of the raw logits: lmax = max logit, Z = sum exp((l - lmax) / T).
struct RowStat {
  float lmax;
  int32_t st;
  double Z;
};

// Per-row nucleus: tokens with logit >= thr are kept; M = their mass under softmax(l / T).
struct ToppStat {
  float thr;
  int32_t pad;
  double M;
};

// What the final draw of a request needs: the stopping row of p (and of q, or -1), the Philox
// position of the draw, the tokens removed from the residual (tree: rejected children) and the
// weight of q in the residual.
struct DrawDesc {
  int32_t prow;
  int32_t qrow;
  int32_t pos;      // Philox counter word 1 for the draw
  int32_t st;       // status bits found before the draw
  int32_t nexcl;    // number of excluded tokens
  int32_t out_idx;  // where the drawn token goes in out_tokens (flat index), -1 = nowhere
  int32_t ph_req;   // Philox counter word 0 is request_base + ph_req
  int32_t purpose;  // Philox counter word 2
  double factor;    // with a q row: the residual is max(0, p' - factor q') (1 for the linear rule)
};

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 [philox]: ten rounds; each multiplies counter words 0 and 2 by the two published
// multipliers, swaps, and xors the high halves with words 1/3 and the round key; the key advances
// by the two published Weyl increments between rounds.
// ---------------------------------------------------------------------------------------------
__device__ inline uint4 philox4x32_10(uint4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t a = ctr.x, c = ctr.z;
    const uint32_t hi_a = __umulhi(0xD2511F53u, a), lo_a = 0xD2511F53u * a;
    const uint32_t hi_c = __umulhi(0xCD9E8D57u, c), lo_c = 0xCD9E8D57u * c;
    ctr = make_uint4(hi_c ^ ctr.y ^ k0, lo_c, hi_a ^ ctr.w ^ k1, lo_a);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return ctr;
}

// u in [0, 1): the 53 high bits of (word0 << 32 | word1) scaled by 2^-53 (exact in fp64).
__device__ inline double philox_uniform(uint64_t seed, uint32_t request, uint32_t position,
                                        uint32_t purpose, uint32_t step) {
  const uint4 x = philox4x32_10(make_uint4(request, position, purpose, step),
                                (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32));
  const uint64_t bits = ((uint64_t)x.x << 32) | (uint64_t)x.y;
  return (double)(bits >> 11) * 0x1.0p-53;
}

// ---------------------------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
  uint16_t bits;
};

// Barrier of a one-wave block: its lanes' LDS writes before this point are seen by their LDS
// reads after it (one wave's LDS operations complete in order; the fences keep the compiler from
// moving accesses across).  Unlike __syncthreads it does not wait for the wave's global loads in
// flight, so a gather issued earlier keeps going while the wave works on LDS.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bf16 -> float: the 16 bits on top of a float (a shift or a mask).  Written as conversions so that
// the compiler takes the values as canonical and forms three-operand maxima from them without
// quieting every input first.
__device__ inline float bf16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(__bf16, b); }
__device__ inline float bf16_lo(uint32_t w) { return bf16_bits_to_f32((uint16_t)w); }
__device__ inline float bf16_hi(uint32_t w) { return bf16_bits_to_f32((uint16_t)(w >> 16)); }

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16_t x) { return bf16_bits_to_f32(x.bits); }

template <typename T>
__device__ inline const T* row_ptr(const RowSet& rs, int64_t row) {
  if (row < rs.nP) return static_cast<const T*>(rs.p) + row * rs.pstride;
  return static_cast<const T*>(rs.q) + (row - rs.nP) * (int64_t)rs.V;
}

__device__ inline bool row_skipped(const RowSet& rs, int64_t row) {
  return rs.skip_q0 && row >= rs.nP && ((row - rs.nP) % rs.qB) == 0;
}

// order-preserving integer key of a logit (larger logit <-> larger key)
__device__ inline uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline uint32_t order_key16(uint16_t b) {
  return (b & 0x8000u) ? (uint32_t)(~b & 0xffffu) : (uint32_t)(b | 0x8000u);
}
__device__ inline float key_to_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ inline float key16_to_float(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
  return __uint_as_float(b << 16);
}

// ---------------------------------------------------------------------------------------------
// fp64 exp by Tang's table-driven method (P. T. P. Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989), with 256 table
// entries: x = (256 m + j) ln2/256 + r, |r| <= ln2/512, exp(x) = 2^m * 2^(j/256) * exp(r), exp(r) - 1
// by its degree-4 Taylor polynomial (truncation below 4e-17 relative).  tbl[j] = 2^(j/256) lives in
// LDS (filled by exp_table_fill).  Inputs are <= 0 here (logit minus row maximum); below -745 the
// result underflows to 0.  Branch-free: the clamped argument is always evaluated and the result
// selected, so a wave's lanes never split on it.
// ---------------------------------------------------------------------------------------------
constexpr int kExpTable = 256;
__device__ inline void exp_table_fill(double* tbl) {
  for (int j = threadIdx.x; j < kExpTable; j += blockDim.x) tbl[j] = exp2((double)j / kExpTable);
}

__device__ inline double exp_tang(double x, const double* tbl) {
  const double xc = fmax(x, -745.0);
  const double kInvL = 369.3299304675746;    // 256 / ln 2
  const double kL1 = 0.0027076061740622863;  // ln 2 / 256 rounded to double
  const double kL2 = 9.058776616587108e-20;  // ln 2 / 256 - kL1
  const double kf = rint(xc * kInvL);
  const int k = (int)kf;
  double r = fma(-kf, kL1, xc);
  r = fma(-kf, kL2, r);
  double t = fma(r, 1.0 / 24.0, 1.0 / 6.0);
  t = fma(r, t, 0.5);
  t = fma(r, t, 1.0);
  const double p = r * t;  // exp(r) - 1
  const double tj = tbl[k & (kExpTable - 1)];
  const double v = ldexp(fma(tj, p, tj), k >> 8);
  return x > -745.0 ? v : 0.0;
}

// 2^(t/256) for t = 256 log2(e) (l - lmax) / T formed by one fused multiply-add,
// t = l c256 - lmax c256: with r = t - rint(t) (exact, |r| <= 1/2), 2^(t/256) = 2^m 2^(j/256) 2^(r/256)
// and 2^(r/256) - 1 = x (1 + x/2 + x^2/6 + x^3/24 + ...) (x = r ln 2/256, |x| <= a = ln 2/512) by a
// cubic: in the bracket, x^3 is replaced by its Chebyshev economization on [-a, a], (3/4) a^2 x, so
// the cubic is x + (1/2 + a^2/32) x^2 + x^3/6; it vanishes at r = 0 (integer t stays exact) and its
// relative error is below 3.5e-14 (one multiply-add fewer than the degree-4 Taylor polynomial,
// error 4e-17).  Same table as exp_tang.  Relative error against
// exp((l - lmax) / T): below 5e-14 for |l - lmax| / T up to 80, 2.2e-13 at 4600 (the rounding of
// lmax c256 scales with it), as exp_tang's own argument rounding does.  Branch-free and
// select-free: t is clamped at
// -300000 (which also maps -inf and NaN there), where the final scaling by 2^(-1172) rounds to 0;
// results below 2^-1074 round to 0 or to a subnormal as the scaling rounds them (0 from
// t < -275200, i.e. exp(x) for x < -745.13, as the fp64 exp itself).
constexpr double k256Log2e = 369.3299304675746;  // 256 / ln 2
__device__ inline double exp2_256(double t, const double* tbl) {
  const double c1 = 0.0027076061740622863;   // c = ln 2 / 256
  const double c2 = 3.6655660167967044e-06;  // (1/2 + a^2/32) c^2 = c^2 / 2 + c^4 / 128
  const double c3 = 3.3083026805413713e-09;  // c^3 / 6
  const double tc = fmax(t, -300000.0);
  const double kf = rint(tc);
  const int k = (int)kf;
  const double r = tc - kf;
  double s = fma(r, c3, c2);
  s = fma(r, s, c1);
  const double p = r * s;  // 2^(r/256) - 1
  const double tj = tbl[k & (kExpTable - 1)];
  return ldexp(fma(tj, p, tj), k >> 8);
}

// online softmax accumulation: (m, s) with s = sum exp2((x - m) * c)
__device__ inline void os_combine(float& m, float& s, float m2, float s2, float c) {
  const float mn = fmaxf(m, m2);
  s = s * exp2f((m - mn) * c) + s2 * exp2f((m2 - mn) * c);
  m = mn;
}

template <typename F>
__device__ inline void wave_allreduce(F& v, F (*op)(F, F)) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, 64));
}

}  // namespace psispec
