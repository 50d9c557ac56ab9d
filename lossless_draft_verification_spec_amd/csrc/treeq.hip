// treeq.hip -- tree verify with candidates drawn from the draft (recursive rejection).
//
// [alphalab] §"Linear 與 Tree sampler" leaves the candidate rule open.  When the children of node v
// were drawn independently from v's draft distribution q'_v, the lossless rule is recursive
// rejection: with r_0 = p'_v, child i is kept with probability min(1, r_{i-1}(x_i) / q'_v(x_i)); a
// rejection replaces the residual by max(0, r_{i-1} - q'_v) renormalised; with no child kept one
// token is drawn from the last residual.
//
// The residual after i rejections is max(0, p' - c_i q') / S_i with c_0 = 0, c_1 = 1,
// c_{i+1} = c_i + S_i and S_i = sum_x max(0, p'(x) - c_i q'(x)): by induction, where p' > c_i q' the
// next subtraction leaves p' - (c_i + S_i) q', and elsewhere both sides are 0.  So a node with m
// children needs its exact normalisers and S_1 .. S_{m-1}, one fp64 pass over its p and q rows per
// level (k_tree_chain; level 0 gives the normalisers and, from the row pass's estimate of their
// ratio, most of S_1, which k_tree_resolve completes), then its chain (k_tree_chain_final).  The
// accept tests need one gathered token per child (k_decide_tree_sampled), and the final draw is the
// residual draw of the linear rule with q weighted by c_m (or, at a leaf, the draw from p').
#include "launch.h"
#include "draw.h"

namespace psispec {
namespace {

constexpr int kChainWaves = kThreads / 64;  // one 1024-token sub-chunk per wave

// a b - c d with each product rounded on its own (no fused multiply-add), as the definition's
// separately rounded terms: p' = c q' then gives exactly 0
__device__ inline double sub_products(double a, double b, double c, double d) {
#pragma clang fp contract(off)
  return a * b - c * d;
}

// Sum of the n entries p[0], p[stride], ... by one full wave in a fixed order: lane l adds entries
// l, l+64, ... in turn, then a butterfly (every lane ends with the same bits).  Every kernel that
// recombines a node's partial sums uses it, so they all see identical values.
__device__ inline double wave_sum_fixed(const double* p, int n, int stride) {
  const int l = threadIdx.x & 63;
  double s = 0.0;
  for (int k = l; k < n; k += 64) s += p[(int64_t)k * stride];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

__device__ inline const double* e_part_of(const TreeQArgs& a, int64_t g) {
  return reinterpret_cast<const double*>(a.e_part + g * a.nchunk_c);
}
__device__ inline const double* s_part_of(const TreeQArgs& a, int level, int64_t g) {
  return a.s_part + ((int64_t)(level - 1) * a.rs.nP + g) * a.nchunk_c;
}

// Children per node row: one block per request counts the parents (entries outside -1 .. N-1 are
// counted for no row; the decide rejects them).
__global__ __launch_bounds__(256) void k_tree_children(TreeQArgs a) {
  __shared__ int s_cnt[1025];
  const int r = blockIdx.x, N = a.N;
  for (int j = threadIdx.x; j <= N; j += 256) s_cnt[j] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < N; j += 256) {
    const int v = a.parent[(int64_t)r * N + j];
    if (v >= -1 && v < N) atomicAdd(&s_cnt[v + 1], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j <= N; j += 256) a.nchild[(int64_t)r * (N + 1) + j] = s_cnt[j];
}

// kappa = E_p / E_q estimated from the row pass (its fp32 sums, times the nucleus masses).  Level 0
// classifies a token as surely inside the support of max(0, p' - q') when e_p > kappa (1 + d) e_q,
// surely outside when e_p <= kappa (1 - d) e_q (the tests on the fp64 terms themselves: 0 and 0, as
// past a row's end, is outside), and keeps the indices of the few in between; the resolve accepts
// the split only when the exact ratio lies well inside the band (within d / 4), so a wrong estimate
// costs a recomputation, never a wrong sum.
constexpr double kBandRel = 1.0 / 65536.0;
__device__ inline double kappa_est(const TreeQArgs& a, int64_t g) {
  double zp = a.rowstat[g].Z, zq = a.rowstat[a.rs.nP + g].Z;
  if (a.use_topp) {
    zp *= a.topp[g].M;
    zq *= a.topp[a.rs.nP + g].M;
  }
  return zp / zq;
}

// Work item (g, chunk) of a level: node row g = r (N+1) + v + 1, 4096 tokens of its p and q rows.
// Level 0, nodes with >= 2 children: the chunk's sums of e_p and e_q, and the split of S_1's terms
// above (BandPart).  Level 1: only the chunks whose split the resolve did not accept, the chunk's
// sum of max(0, p' - q').  Level i >= 2, nodes with >= i+1 children: the chunk's sum of
// max(0, p' - c_i q').  A fixed grid loops over the items: a block looks up the children counts of
// up to kThreads of its items in one round of loads and then works through the items that have
// work only, so levels without work cost a launch and one load.
template <typename T, bool kFirst>
__global__ __launch_bounds__(kThreads) void k_tree_chain(TreeQArgs a, int level, int vec_ok) {
  __shared__ double tbl[kExpTable];
  __shared__ int s_cnt, s_nband;
  __shared__ double s_sum[kChainWaves][4];
  __shared__ double s_inv[2], s_c;
  __shared__ int s_items[kThreads];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t items = a.rs.nP * (int64_t)a.nchunk_c;

  // the item's pass over its 4096 tokens (every thread of the block; block barriers inside)
  auto do_item = [&](int64_t g, int chunk) {
    const int64_t prow = g, qrow = a.rs.nP + g, item = g * a.nchunk_c + chunk;
    // the item's loads first (tokens, row statistics), in flight while wave 0 sums the node's parts
    const int x0 = chunk * a.chunk_elems_c + wave * kSub + lane * kPerLane;
    float fp[kPerLane], fq[kPerLane];
    load_run<T, kPerLane>(row_ptr<T>(a.rs, prow), x0, a.V, vec_ok, fp);
    load_run<T, kPerLane>(row_ptr<T>(a.rs, qrow), x0, a.V, vec_ok, fq);
    const float lmp = a.rowstat[prow].lmax, lmq = a.rowstat[qrow].lmax;
    const float thp = a.use_topp ? a.topp[prow].thr : -__builtin_huge_valf();
    const float thq = a.use_topp ? a.topp[qrow].thr : -__builtin_huge_valf();
    double klo = 0.0, khi = 0.0;
    if constexpr (kFirst) {
      const double k = kappa_est(a, g);
      klo = k * (1.0 - kBandRel);
      khi = k * (1.0 + kBandRel);
      if (threadIdx.x == 0) s_nband = 0;
    } else if (wave == 0) {
      // the node's normalisers and c_level = 1 + S_1 + ... + S_{level-1}: every array's entries
      // loaded in one round, then summed in wave_sum_fixed's order (lane l: entries l, l+64, ...;
      // then the butterfly)
      const double* ep = e_part_of(a, g);
      double se = 0.0, sq = 0.0, ss[kMaxSampledChildren - 1];
#pragma unroll
      for (int j = 0; j < kMaxSampledChildren - 1; ++j) ss[j] = 0.0;
      for (int k = lane; k < a.nchunk_c; k += 64) {
        se += ep[2 * (int64_t)k];
        sq += ep[2 * (int64_t)k + 1];
#pragma unroll
        for (int j = 0; j < kMaxSampledChildren - 1; ++j)
          if (j + 1 < level) ss[j] += s_part_of(a, j + 1, g)[k];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        se += __shfl_xor(se, off, 64);
        sq += __shfl_xor(sq, off, 64);
#pragma unroll
        for (int j = 0; j < kMaxSampledChildren - 1; ++j)
          if (j + 1 < level) ss[j] += __shfl_xor(ss[j], off, 64);
      }
      double ci = 1.0;
#pragma unroll
      for (int j = 0; j < kMaxSampledChildren - 1; ++j)
        if (j + 1 < level) ci += ss[j];
      if (lane == 0) {
        s_inv[0] = 1.0 / se;
        s_inv[1] = 1.0 / sq;
        s_c = ci;
      }
    }
    __syncthreads();
    const double invEp = kFirst ? 0.0 : s_inv[0], invEq = kFirst ? 0.0 : s_inv[1];
    const double ci = kFirst ? 0.0 : s_c;
    double sp = 0.0, sq = 0.0, pa = 0.0, qa = 0.0;
    if constexpr (kFirst) {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        const double ep = term(fp[e], lmp, thp, a.inv_T, tbl);
        const double eq = term(fq[e], lmq, thq, a.inv_T, tbl);
        sp += ep;
        sq += eq;
        if (ep > khi * eq) {
          pa += ep;
          qa += eq;
        } else if (!(ep <= klo * eq)) {  // rare: an in-between token (or a NaN term)
          const int k = atomicAdd(&s_nband, 1);
          if (k < kBandSlots) a.band[item].x[k] = x0 + e;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        const double ep = term(fp[e], lmp, thp, a.inv_T, tbl);
        const double eq = term(fq[e], lmq, thq, a.inv_T, tbl);
        const double x = sub_products(ep, invEp, ci, eq * invEq);
        sp += x > 0.0 ? x : 0.0;
      }
    }
    sp = wave_sum(sp);
    sq = wave_sum(sq);
    if constexpr (kFirst) {
      pa = wave_sum(pa);
      qa = wave_sum(qa);
    }
    if (lane == 0) {
      s_sum[wave][0] = sp;
      s_sum[wave][1] = sq;
      s_sum[wave][2] = pa;
      s_sum[wave][3] = qa;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double tp = 0.0, tq = 0.0, ta = 0.0, tb = 0.0;
      for (int k = 0; k < kChainWaves; ++k) {
        tp += s_sum[k][0];
        tq += s_sum[k][1];
        ta += s_sum[k][2];
        tb += s_sum[k][3];
      }
      if constexpr (kFirst) {
        a.e_part[item] = make_double2(tp, tq);
        a.band[item].pa = ta;
        a.band[item].qa = tb;
        a.band[item].n = s_nband;
      } else {
        a.s_part[((int64_t)(level - 1) * a.rs.nP + g) * a.nchunk_c + chunk] = tp;
      }
    }
    __syncthreads();  // the next item reuses the block's LDS
  };

  if constexpr (kFirst) {  // one item per block (no loop: 95 instead of 111 VGPRs, 5 waves/SIMD)
    const int64_t w = blockIdx.x;
    const int64_t g = w / a.nchunk_c;
    const int m = a.nchild[g];
    if (m < 2 || m > a.max_children) return;
    exp_table_fill(tbl);  // read after do_item's first barrier
    do_item(g, (int)(w - g * a.nchunk_c));
    return;
  }
  bool filled = false;  // the exp table, filled once the block has an item (empty levels skip it)
  // items blockIdx.x + k gridDim.x, kThreads at a time: their children counts (and at level 1 the
  // resolve's flags) in one round
  const int mmin = level < 2 ? 2 : level + 1;
  const int64_t stride = gridDim.x;
  for (int64_t base = blockIdx.x; base < items; base += stride * kThreads) {
    if (threadIdx.x == 0) s_cnt = 0;
    __syncthreads();
    // index j runs chunk-major (node row j mod nP, chunk j / nP): one node's chunks land in
    // blocks (g + c nP) mod gridDim.x, distinct for all c < gridDim.x when gridDim.x is a prime
    // that does not divide nP (the launcher picks such a grid)
    const int64_t j = base + (int64_t)threadIdx.x * stride;
    if (j < items) {
      const int64_t g = j % a.rs.nP;
      const int m = a.nchild[g];
      // the resolve's flag, read for every item; used where m >= 2 only
      const int redo = level == 1 ? a.fb[g * a.nchunk_c + j / a.rs.nP] : 1;
      if (m >= mmin && m <= a.max_children && redo) s_items[atomicAdd(&s_cnt, 1)] = threadIdx.x;
    }
    __syncthreads();
    const int nit = s_cnt;
    if (nit > 0 && !filled) {  // read after do_item's first barrier
      exp_table_fill(tbl);
      filled = true;
    }
    for (int it = 0; it < nit; ++it) {
      const int64_t j2 = base + (int64_t)s_items[it] * stride;
      do_item(j2 % a.rs.nP, (int)(j2 / a.rs.nP));
    }
    __syncthreads();  // s_cnt and s_items are reset by the next round
  }
}

// One wave per node row with two or more children: its exact normalisers (wave_sum_fixed's order),
// then per chunk S_1's part from level 0's split: the sure terms' sums scaled, plus the kept
// in-between tokens (their e_p and e_q recomputed as level 0 computes them) in index order.  A
// chunk whose split cannot be used (ratio outside the checked band, or more in-between tokens than
// were kept) is flagged for the full level-1 pass.
template <typename T>
__global__ __launch_bounds__(64) void k_tree_resolve(TreeQArgs a) {
  __shared__ double tbl[kExpTable];
  exp_table_fill(tbl);
  const int64_t g = blockIdx.x;
  const int m = a.nchild[g];
  if (m < 2 || m > a.max_children) return;
  const int lane = threadIdx.x;
  const int64_t prow = g, qrow = a.rs.nP + g;
  const T* pr = row_ptr<T>(a.rs, prow);
  const T* qr = row_ptr<T>(a.rs, qrow);
  const float lmp = a.rowstat[prow].lmax, lmq = a.rowstat[qrow].lmax;
  const float thp = a.use_topp ? a.topp[prow].thr : -__builtin_huge_valf();
  const float thq = a.use_topp ? a.topp[qrow].thr : -__builtin_huge_valf();
  const double* ep = e_part_of(a, g);
  double se = 0.0, sq = 0.0;
  for (int k = lane; k < a.nchunk_c; k += 64) {
    se += ep[2 * (int64_t)k];
    sq += ep[2 * (int64_t)k + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    se += __shfl_xor(se, off, 64);
    sq += __shfl_xor(sq, off, 64);
  }
  const double invEp = 1.0 / se, invEq = 1.0 / sq;
  const double kt = kappa_est(a, g), kappa = se / sq;
  const bool ok = kappa > kt * (1.0 - 0.25 * kBandRel) && kappa < kt * (1.0 + 0.25 * kBandRel);
  double* s1 = a.s_part + g * a.nchunk_c;
  for (int k = lane; k < a.nchunk_c; k += 64) {
    const int64_t item = g * a.nchunk_c + k;
    const BandPart& b = a.band[item];
    const int n = b.n;
    int redo = 1;
    if (ok && n <= kBandSlots) {
      double s = sub_products(b.pa, invEp, 1.0, b.qa * invEq);
      s = s > 0.0 ? s : 0.0;
      int xs[kBandSlots];
#pragma unroll
      for (int j = 0; j < kBandSlots; ++j) xs[j] = j < n ? b.x[j] : 0x7fffffff;
      // index order (the atomic slots are taken in no fixed order): a sorting network
#pragma unroll
      for (int i = 0; i < kBandSlots; ++i)
#pragma unroll
        for (int j = (i & 1); j + 1 < kBandSlots; j += 2) {
          const int lo = min(xs[j], xs[j + 1]), hi = max(xs[j], xs[j + 1]);
          xs[j] = lo;
          xs[j + 1] = hi;
        }
#pragma unroll
      for (int j = 0; j < kBandSlots; ++j) {
        if (j < n) {
          const double ep = term(to_f32(pr[xs[j]]), lmp, thp, a.inv_T, tbl);
          const double eq = term(to_f32(qr[xs[j]]), lmq, thq, a.inv_T, tbl);
          const double x = sub_products(ep, invEp, 1.0, eq * invEq);
          s += x > 0.0 ? x : 0.0;
        }
      }
      s1[k] = s;
      redo = 0;
    }
    a.fb[item] = redo;
  }
}

// One wave per node row with children: its normalisers and its residual chain (NodeChain).
__global__ __launch_bounds__(64) void k_tree_chain_final(TreeQArgs a) {
  const int64_t g = blockIdx.x;
  const int m = a.nchild[g];
  if (m < 1 || m > a.max_children) return;
  const int64_t nP = a.rs.nP;
  const int lane = threadIdx.x;
  // the normalisers (two or more children) and S_1 .. S_{m-1}: every array's entries in one round of
  // loads, then summed in wave_sum_fixed's order (lane l: entries l, l+64, ...; then the butterfly)
  const double* ep = e_part_of(a, g);
  double se = 0.0, sq = 0.0, S[kMaxSampledChildren];
#pragma unroll
  for (int k = 0; k < kMaxSampledChildren; ++k) S[k] = 0.0;
  for (int k = lane; k < a.nchunk_c; k += 64) {
    if (m >= 2) {
      se += ep[2 * (int64_t)k];
      sq += ep[2 * (int64_t)k + 1];
    }
#pragma unroll
    for (int j = 1; j < kMaxSampledChildren; ++j)
      if (j < m) S[j] += s_part_of(a, j, g)[k];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    se += __shfl_xor(se, off, 64);
    sq += __shfl_xor(sq, off, 64);
#pragma unroll
    for (int j = 1; j < kMaxSampledChildren; ++j)
      if (j < m) S[j] += __shfl_xor(S[j], off, 64);
  }
  if (lane != 0) return;
  double Ep = se, Eq = sq;
  if (m < 2) {  // one child: the HBM pass's normalisers suffice for its ratio
    Ep = a.rowstat[g].Z;
    Eq = a.rowstat[nP + g].Z;
    if (a.use_topp) {
      Ep *= a.topp[g].M;
      Eq *= a.topp[nP + g].M;
    }
  }
  NodeChain ch;
  ch.Ep = Ep;
  ch.Eq = Eq;
  ch.c[0] = 0.0;
  ch.S[0] = 1.0;
  ch.stuck = kMaxSampledChildren + 1;
#pragma unroll
  for (int k = 1; k <= kMaxSampledChildren; ++k) {
    if (k > m) {
      ch.c[k] = 0.0;
      ch.S[k] = 0.0;
      continue;
    }
    if (ch.stuck <= k) {  // a zero residual earlier: the residual stays
      ch.c[k] = ch.c[k - 1];
      ch.S[k] = ch.S[k - 1];
      continue;
    }
    ch.c[k] = ch.c[k - 1] + ch.S[k - 1];
    const double Sk = k < m ? S[k] : 1.0;  // S_m is never used: the final draw normalises itself
    if (!(Sk > 0.0)) {
      ch.stuck = k;
      ch.c[k] = ch.c[k - 1];
      ch.S[k] = ch.S[k - 1];
    } else {
      ch.S[k] = Sk;
    }
  }
  a.chain[g] = ch;
}

// p'(x) or q'(x) of one gathered token: exp((l - lmax) / T) / E over the nucleus
template <typename T>
__device__ inline double gathered_prob(const TreeQArgs& a, int64_t row, int tok, double E) {
  const float l = to_f32(row_ptr<T>(a.rs, row)[tok]);
  if (a.use_topp && !(l >= a.topp[row].thr)) return 0.0;
  return exp(((double)l - (double)a.rowstat[row].lmax) * a.inv_T) / E;
}

// Structure, node ratios, the walk and the draw description of request r, by one wave (threads
// 0..63 of the calling block; it syncs with wave barriers only).  kMaxN: most nodes per tree (its
// LDS arrays).  desc_local: the fused kernel's LDS copy of the description (with quiet, the only
// output: another block of the request writes the call's).
template <typename T, int kMaxN>
__device__ inline void decide_tree_sampled_request(const TreeQArgs& a, int r, bool quiet,
                                                   DrawDesc* desc_local) {
  const int t = threadIdx.x;
  const int N = a.N, V = a.V;
  const int64_t row0 = (int64_t)r * (N + 1);
  const int64_t nP = a.rs.nP;
  const int32_t* par = a.parent + (int64_t)r * N;
  const int32_t* tok = a.node_tokens + (int64_t)r * N;

  __shared__ int32_t s_par[kMaxN], s_tok[kMaxN];
  __shared__ double s_u[kMaxN], s_ratio[kMaxN];
  __shared__ int s_st;

  for (int j = t; j < N; j += 64) {
    s_par[j] = par[j];
    s_tok[j] = tok[j];
    s_u[j] = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)(j + 1), kPurposeAccept,
                            a.step);
  }
  wave_sync();

  // 1. structure: parents precede children, depth within max_depth, at most a.max_children
  //    children per node (the level-0 pass counted them); row statistics of the request's rows
  int bad = 0, st = 0;
  for (int j = t; j < N; j += 64) {
    const int pj = s_par[j];
    if (pj < -1 || pj >= j) {
      bad = 1;
      continue;
    }
    int d = 1, pnode = pj;
    while (pnode >= 0 && d <= a.max_depth) {
      const int q = s_par[pnode];
      if (q < -1 || q >= pnode) break;
      ++d;
      pnode = q;
    }
    if (d > a.max_depth) bad = 1;
  }
  for (int j = t; j <= N; j += 64) {
    if (a.nchild[row0 + j] > a.max_children) bad = 1;
    st |= a.rowstat[row0 + j].st | a.rowstat[nP + row0 + j].st;
  }
  {
    const uint64_t bm = __ballot(bad);
    if (t == 0) s_st = bm ? PSISPEC_ST_BAD_PARENT : 0;
  }

  // 2. node ratios: child j is the i-th child of v (siblings in index order)
  for (int j = t; j < N; j += 64) {
    const int v = s_par[j], tj = s_tok[j];
    double ratio = 0.0;
    if (tj < 0 || tj >= V) {
      st |= PSISPEC_ST_BAD_TOKEN;
    } else if (v >= -1 && v < j) {
      int i = 1;
      for (int s = 0; s < j; ++s) i += s_par[s] == v;
      const int64_t g = row0 + v + 1;
      if (i <= a.max_children) {
        const NodeChain& ch = a.chain[g];
        const double pp = gathered_prob<T>(a, g, tj, ch.Ep);
        const double qq = gathered_prob<T>(a, nP + g, tj, ch.Eq);
        double R = sub_products(pp, 1.0, ch.c[i - 1], qq);  // residual after i-1 rejections
        R = R > 0.0 ? R : 0.0;
        const double S = ch.S[i - 1];
        if (qq > 0.0) {
          ratio = fmin(1.0, (R / S) / qq);
        } else {
          ratio = R > 0.0 ? 1.0 : 0.0;
          st |= PSISPEC_ST_Q_ZERO;
        }
      }
    }
    s_ratio[j] = ratio;
    if (a.node_ratios && !quiet) a.node_ratios[(int64_t)r * N + j] = (float)ratio;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) st |= __shfl_xor(st, off, 64);
  wave_sync();

  // 3. the walk: at each node the children in index order, 64 at a time; the first accepted
  //    child (ballot) is the next node
  const int Dp1 = a.max_depth + 1;
  int32_t* nodes = a.accept_nodes + (int64_t)r * a.max_depth;
  int32_t* out = a.out_tokens + (int64_t)r * Dp1;
  int cur = -1, dep = 0;
  st |= s_st;
  if (!(s_st & PSISPEC_ST_BAD_PARENT)) {
    for (;;) {
      int next = -1, rejected = 0;
      for (int c0 = 0; c0 < N && next < 0; c0 += 64) {
        const int c = c0 + t;
        const bool child = c < N && s_par[c] == cur;
        const uint64_t am = __ballot(child && s_u[c] < s_ratio[c]);
        const uint64_t cm = __ballot(child);
        if (am) {
          next = c0 + __builtin_ctzll(am);
          rejected += __builtin_popcountll(cm & ((1ull << (next - c0)) - 1ull));
        } else {
          rejected += __builtin_popcountll(cm);
        }
      }
      {
        const int m = a.nchild[row0 + cur + 1];
        if (m >= 1 && rejected >= a.chain[row0 + cur + 1].stuck) st |= PSISPEC_ST_RESID_ZERO;
      }
      if (next < 0) break;
      if (t == 0 && !quiet) {
        nodes[dep] = next;
        out[dep] = s_tok[next];
      }
      ++dep;
      cur = next;
    }
  }
  if (t == 0) {
    if (!quiet) {
      for (int i = dep; i < a.max_depth; ++i) nodes[i] = -1;
      for (int i = dep; i < Dp1; ++i) out[i] = -1;
      a.accept_len[r] = dep;
    }
    const int64_t g = row0 + cur + 1;
    const int m = (s_st & PSISPEC_ST_BAD_PARENT) ? 0 : a.nchild[g];
    DrawDesc dd;
    dd.prow = (int32_t)g;
    dd.qrow = m >= 1 ? (int32_t)(nP + g) : -1;  // every child rejected: residual of c_m q'
    dd.pos = cur + 1;
    dd.st = st;
    dd.nexcl = 0;
    dd.out_idx = (s_st & PSISPEC_ST_BAD_PARENT) ? -1 : (int32_t)((int64_t)r * Dp1 + dep);
    dd.ph_req = r;
    dd.purpose = kPurposeDraw;
    dd.factor = m >= 1 ? a.chain[g].c[m] : 1.0;
    if (!quiet) a.desc[r] = dd;
    if (desc_local) *desc_local = dd;
  }
}

template <typename T>
__global__ __launch_bounds__(64) void k_decide_tree_sampled(TreeQArgs a) {
  decide_tree_sampled_request<T, 1024>(a, blockIdx.x, false, nullptr);
}

// The sampled tree's walk fused with its draw pass (trees of at most 64 nodes): block (r, c) runs
// request r's walk in wave 0 into an LDS copy of the draw description, then draws chunk c of the
// stopping rows; the chunk-0 block also writes the call's outputs and the description the select
// reads.  One launch fewer than the walk followed by the pass, and no read of the description.
template <typename T, bool kTopp>
__global__ __launch_bounds__(kThreads, kDrawPassWaves) void k_decide_tree_sampled_draw(
    TreeQArgs ta, DrawArgs da, int vec_ok) {
  __shared__ double tbl[kExpTable];
  __shared__ DrawDesc s_d;
  exp_table_fill(tbl);  // read after the barriers below
  const int r = blockIdx.x / da.nchunk_draw;
  const int c = blockIdx.x - r * da.nchunk_draw;
  if (threadIdx.x < 64) decide_tree_sampled_request<T, 64>(ta, r, c != 0, &s_d);
  __syncthreads();  // the description is in LDS
  const DrawDesc d = s_d;
  draw_pass_run<T, kTopp>(da, r, c, vec_ok, d, row_view(da, d),
                          d.qrow >= 0 ? rho_estimate(da, d) : 0.0, tbl);
}

}  // namespace

hipError_t launch_tree_children(const TreeQArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  PSISPEC_LAUNCH("tree_children", k_tree_children, dim3((unsigned)a.batch), dim3(256), 0, stream,
                 a);
  return hipGetLastError();
}

hipError_t launch_tree_resolve(const TreeQArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("tree_resolve", k_tree_resolve<bf16_t>, dim3((unsigned)a.rs.nP), dim3(64), 0,
                   stream, a);
  else
    PSISPEC_LAUNCH("tree_resolve", k_tree_resolve<float>, dim3((unsigned)a.rs.nP), dim3(64), 0,
                   stream, a);
  return hipGetLastError();
}

hipError_t launch_tree_chain_pass(const TreeQArgs& a, int level, psispec_dtype dtype,
                                  hipStream_t stream) {
  int64_t blocks = a.rs.nP * (int64_t)a.nchunk_c;
  if (blocks == 0) return hipSuccess;
  // a fixed grid loops over the work items: about 2048 blocks at level 1 (every chunk of every node
  // with two or more children when the level-0 split is refused), about 509 from level 2 on (nodes
  // with three or more children: fewer items, and a launch without work is cheaper).  The grid is
  // a prime that does not divide nP, so that the chunks of one node go to different blocks.
  if (level > 0) {
    static const int64_t kGrid1[] = {2039, 2029, 2027}, kGrid2[] = {509, 503, 499};
    const int64_t* cand = level == 1 ? kGrid1 : kGrid2;
    int64_t grid = cand[0];
    for (int i = 0; i < 3; ++i)
      if (a.rs.nP % cand[i] != 0) {
        grid = cand[i];
        break;
      }
    if (blocks > grid) blocks = grid;
  }
  const size_t es = dtype == PSISPEC_BF16 ? 2 : 4;
  const int vec_ok = ((size_t)a.V * es) % 16 == 0 && ((uintptr_t)a.rs.p % 16) == 0 &&
                     ((uintptr_t)a.rs.q % 16) == 0;
  auto kern = dtype == PSISPEC_BF16 ? (level == 0 ? k_tree_chain<bf16_t, true> : k_tree_chain<bf16_t, false>)
                                    : (level == 0 ? k_tree_chain<float, true> : k_tree_chain<float, false>);
  PSISPEC_LAUNCH("tree_chain", kern, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, level,
                 vec_ok);
  return hipGetLastError();
}

hipError_t launch_decide_tree_sampled_draw(const TreeQArgs& ta, const DrawArgs& da,
                                           psispec_dtype dtype, hipStream_t stream) {
  if (ta.batch == 0) return hipSuccess;
  if (ta.N > 64 || da.list || ta.batch != da.batch || ta.use_topp != da.use_topp)
    return hipErrorInvalidValue;
  PSISPEC_LAUNCH("tree_chain_final", k_tree_chain_final, dim3((unsigned)ta.rs.nP), dim3(64), 0,
                 stream, ta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)da.batch * da.nchunk_draw);
  const int vec_ok = draw_vec_ok(da, dtype);
  const bool bf = dtype == PSISPEC_BF16, tp = da.use_topp;
  auto kern = bf ? (tp ? k_decide_tree_sampled_draw<bf16_t, true>
                       : k_decide_tree_sampled_draw<bf16_t, false>)
                 : (tp ? k_decide_tree_sampled_draw<float, true>
                       : k_decide_tree_sampled_draw<float, false>);
  PSISPEC_LAUNCH("decide_tree_sampled_draw", kern, dim3(grid), dim3(kThreads), 0, stream, ta, da,
                 vec_ok);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw_select(da, dtype, stream);
}

hipError_t launch_decide_tree_sampled(const TreeQArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  PSISPEC_LAUNCH("tree_chain_final", k_tree_chain_final, dim3((unsigned)a.rs.nP), dim3(64), 0,
                 stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("decide_tree_sampled", k_decide_tree_sampled<bf16_t>, dim3(a.batch), dim3(64), 0,
                   stream, a);
  else
    PSISPEC_LAUNCH("decide_tree_sampled", k_decide_tree_sampled<float>, dim3(a.batch), dim3(64), 0,
                   stream, a);
  return hipGetLastError();
}

}  // namespace psispec
