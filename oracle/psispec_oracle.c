/*
 * psispec_oracle.c -- plain CPU oracle of the Psi-Spec verify step (fp64, single-threaded).
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark to check the GPU library.  It shares no code with the HIP library and is never called by
 * it.  Everything is written for a reader to check against the sources by eye: no blocking, no
 * fusion, sums run sequentially by ascending token id, all arithmetic in fp64 on exactly widened
 * inputs.  Source citations are in psispec_oracle.h ([alphalab], [lanes], [philox]).
 *
 * What the method computes (restated in our words):
 *   - A frozen AR model scores a block of B drafted tokens in one pass and the verifier applies a
 *     rejection test position by position, keeping only the longest run of accepted positions from
 *     the start ([alphalab] walkthrough, step 3; [lanes] "Ψ-Spec이 한 스텝에서 하는 일").
 *   - At the first rejected position a replacement token is drawn from a corrected residual
 *     distribution and every later draft is discarded ([alphalab] walkthrough, step 4).
 *   - If all B drafts pass, one extra token is drawn from the logits at the end of the block
 *     ([alphalab] walkthrough, paragraph after step 4).
 *   - The result is distributed exactly as the AR model ([lanes] "Ψ-Spec이 한 스텝에서 하는 일";
 *     [alphalab] "為什麼 lossless 不等於答案完全一樣？").  The pages never print the rule; we take the
 *     speculative-sampling rule of the lineage they cite (Leviathan et al. 2023, [lanes] "어디서
 *     왔나"): accept draft x with probability min(1, p(x)/q(x)); on rejection sample from
 *     max(0, p - q) renormalised.
 */
#include "psispec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------
 * Philox4x32-10 [philox]: ten rounds of the 4x32 Philox S-box.  Each round multiplies counter words
 * 0 and 2 by the two published multipliers, swaps and xors the high halves with the other words and
 * the round key; the key is bumped by the two published Weyl constants between rounds.
 * ---------------------------------------------------------------------------------------------- */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

void psispec_oracle_philox(uint64_t seed, const uint32_t ctr[4], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* Uniform from words 0 and 1 of the block: the top 53 bits of (x0 << 32 | x1), scaled by 2^-53.
 * Exact in fp64 and always in [0, 1). */
double psispec_oracle_uniform(uint64_t seed, uint32_t request, uint32_t position, uint32_t purpose,
                              uint32_t step) {
  uint32_t ctr[4] = {request, position, purpose, step};
  uint32_t x[4];
  psispec_oracle_philox(seed, ctr, x);
  uint64_t bits = ((uint64_t)x[0] << 32) | (uint64_t)x[1];
  return (double)(bits >> 11) * 0x1.0p-53;
}

/* ------------------------------------------------------------------------------------------------
 * Row transform: temperature softmax, then the optional nucleus (top-p) truncation.
 * ---------------------------------------------------------------------------------------------- */
static double widen(const void* row, int dtype, size_t x) {
  if (dtype == ORC_F32) return (double)((const float*)row)[x];
  if (dtype == ORC_F64) return ((const double*)row)[x];
  /* bf16: the 16 stored bits are the top half of an fp32 */
  uint32_t bits = (uint32_t)((const uint16_t*)row)[x] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_size(int dtype) {
  return dtype == ORC_F32 ? 4u : (dtype == ORC_BF16 ? 2u : 8u);
}

typedef struct {
  double l;
  int x;
} logit_at;

static int by_logit_desc(const void* a, const void* b) {
  const logit_at* u = (const logit_at*)a;
  const logit_at* v = (const logit_at*)b;
  if (u->l > v->l) return -1;
  if (u->l < v->l) return 1;
  return (u->x > v->x) - (u->x < v->x);
}

/*
 * pi[x] = exp(z_x - m) / Z with z = l / T, m = max z, Z = sum exp(z - m) (temperature is a fixed
 * sampling setting: [alphalab] "為什麼 lossless 不等於答案完全一樣？" and the run-card list in
 * "想跑 Uno").
 *
 * Nucleus (top_p < 1): tokens are grouped by equal logit and the groups taken by decreasing logit;
 * the kept set is every token whose logit is at least that of the first group at which the running
 * mass reaches top_p (ties are kept whole), and pi is renormalised over it.  The boundary margin is
 * min(top_p - mass before that group, mass including it - top_p).
 */
int psispec_oracle_row_probs(const void* row, int dtype, int V, double T, double top_p, double* pi,
                             double* topp_margin) {
  if (topp_margin) *topp_margin = INFINITY;
  double m = -INFINITY;
  int bad = 0;
  for (int x = 0; x < V; ++x) {
    double l = widen(row, dtype, (size_t)x);
    if (isnan(l) || l == INFINITY) bad = 1;
    double z = l / T;
    if (z > m) m = z;
  }
  if (bad || m == -INFINITY) {
    for (int x = 0; x < V; ++x) pi[x] = 0.0;
    return ORC_ST_NONFINITE;
  }
  double Z = 0.0;
  for (int x = 0; x < V; ++x) {
    double z = widen(row, dtype, (size_t)x) / T;
    pi[x] = exp(z - m);
    Z += pi[x];
  }
  for (int x = 0; x < V; ++x) pi[x] = pi[x] / Z;
  if (!(top_p < 1.0)) return 0;

  logit_at* order = (logit_at*)malloc(sizeof(logit_at) * (size_t)V);
  for (int x = 0; x < V; ++x) {
    order[x].l = widen(row, dtype, (size_t)x);
    order[x].x = x;
  }
  qsort(order, (size_t)V, sizeof(logit_at), by_logit_desc);
  double cum = 0.0, before = 0.0, threshold = order[V - 1].l;
  int i = 0;
  while (i < V) {
    int j = i;
    double group = 0.0;
    while (j < V && order[j].l == order[i].l) {
      group += pi[order[j].x];
      ++j;
    }
    before = cum;
    cum += group;
    if (cum >= top_p) {
      threshold = order[i].l;
      break;
    }
    i = j;
  }
  free(order);
  if (topp_margin) {
    double a = top_p - before, b = cum - top_p;
    *topp_margin = a < b ? a : b;
  }
  double M = 0.0;
  for (int x = 0; x < V; ++x)
    if (widen(row, dtype, (size_t)x) >= threshold) M += pi[x];
  for (int x = 0; x < V; ++x) pi[x] = (widen(row, dtype, (size_t)x) >= threshold) ? pi[x] / M : 0.0;
  return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Inverse-CDF draw: c = min{x : C_x > v}, C_x = sum_{y<=x} w_y (ascending token id), v = u * S.
 * If rounding leaves v >= C_{V-1}, the last token with positive weight is taken.  The margin is the
 * distance of v to the nearer edge of the chosen interval, divided by S.
 * ---------------------------------------------------------------------------------------------- */
static int inverse_cdf(const double* w, int V, double S, double u, double* margin) {
  double v = u * S, C = 0.0, prev = 0.0;
  int last_pos = -1;
  for (int x = 0; x < V; ++x) {
    prev = C;
    C += w[x];
    if (w[x] > 0.0) last_pos = x;
    if (C > v) {
      if (margin) {
        double a = v - prev, b = C - v;
        *margin = (a < b ? a : b) / S;
      }
      return x;
    }
  }
  if (margin) *margin = 0.0;
  return last_pos;
}

/* ------------------------------------------------------------------------------------------------
 * Linear verify ([alphalab] walkthrough steps 3-4 and the full-accept paragraph; [alphalab] "Linear 與
 * Tree sampler": one candidate per position).  Row layout per request: p rows 0..B (row B is the
 * block-end row), q rows 0..B-1, drafted token d_i scored by p row i and q row i.
 * ---------------------------------------------------------------------------------------------- */
int psispec_oracle_verify_linear(const void* p, const void* q, int dtype, const int32_t* draft,
                                 int batch, int B, int V, double T, double top_p, uint64_t seed,
                                 uint32_t step, uint32_t request_base, uint32_t flags,
                                 const double* u_accept, const double* u_resample,
                                 int32_t* accept_len, int32_t* out_tokens, double* ratios,
                                 uint64_t* accept_mask, int32_t* status, double* margin_accept,
                                 double* margin_sample, double* margin_topp, double* resid_w,
                                 double* resid_S) {
  if (!p || !draft || !accept_len || !out_tokens) return ORC_EINVAL;
  if (batch < 0 || B < 1 || B > 64 || V < 1) return ORC_EINVAL;
  if (!(T > 0.0) || !isfinite(T) || !(top_p > 0.0) || !(top_p <= 1.0)) return ORC_EINVAL;
  int first_from_target = (flags & ORC_FIRST_FROM_TARGET) != 0;
  if (!q && !(first_from_target && B == 1)) return ORC_EINVAL;
  size_t es = elem_size(dtype);
  double* pp = (double*)malloc(sizeof(double) * (size_t)V);
  double* qq = (double*)malloc(sizeof(double) * (size_t)V);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);

  for (int r = 0; r < batch; ++r) {
    const char* prow0 = (const char*)p + (size_t)r * (size_t)(B + 1) * (size_t)V * es;
    const char* qrow0 = q ? (const char*)q + (size_t)r * (size_t)B * (size_t)V * es : NULL;
    const int32_t* d = draft + (size_t)r * (size_t)B;
    uint32_t req = request_base + (uint32_t)r;
    int st = 0;
    double rat[64];

    /* ratio_i = min(1, p'_i(d_i) / q'_i(d_i)) for every position (data-parallel, all B). */
    for (int i = 0; i < B; ++i) {
      double mp = INFINITY, mq = INFINITY;
      int sp = psispec_oracle_row_probs(prow0 + (size_t)i * V * es, dtype, V, T, top_p, pp, &mp);
      st |= sp;
      if (margin_topp) margin_topp[(size_t)r * (2 * B + 1) + i] = mp;
      int bad_tok = d[i] < 0 || d[i] >= V;
      if (bad_tok) st |= ORC_ST_BAD_TOKEN;
      if (first_from_target && i == 0) {
        /* Uno layout: position 0 is the AR's own sample, so it is always kept ([alphalab]
         * walkthrough, step 1); the q row of position 0 is not read. */
        rat[i] = 1.0;
        if (margin_topp) margin_topp[(size_t)r * (2 * B + 1) + (B + 1) + i] = INFINITY;
        continue;
      }
      int sq = psispec_oracle_row_probs(qrow0 + (size_t)i * V * es, dtype, V, T, top_p, qq, &mq);
      st |= sq;
      if (margin_topp) margin_topp[(size_t)r * (2 * B + 1) + (B + 1) + i] = mq;
      if (bad_tok) {
        rat[i] = 0.0;
        continue;
      }
      double a = pp[d[i]], b = qq[d[i]];
      if (b > 0.0) {
        double ab = a / b;
        rat[i] = ab < 1.0 ? ab : 1.0;
      } else {
        rat[i] = a > 0.0 ? 1.0 : 0.0;
        st |= ORC_ST_Q_ZERO;
      }
    }
    {
      double mB = INFINITY;
      st |= psispec_oracle_row_probs(prow0 + (size_t)B * V * es, dtype, V, T, top_p, pp, &mB);
      if (margin_topp) margin_topp[(size_t)r * (2 * B + 1) + B] = mB;
    }

    /* accept_i = u_i < ratio_i (strict, u in [0,1)); k = first rejected position, or B. */
    int k = B;
    uint64_t mask = 0;
    for (int i = 0; i < B; ++i) {
      double u = u_accept ? u_accept[(size_t)r * B + i]
                          : psispec_oracle_uniform(seed, req, (uint32_t)i, ORC_PURPOSE_ACCEPT, step);
      int acc = u < rat[i];
      if (acc) mask |= (uint64_t)1 << i;
      if (!acc && k == B) k = i;
      if (margin_accept) margin_accept[(size_t)r * B + i] = fabs(u - rat[i]);
      if (ratios) ratios[(size_t)r * B + i] = rat[i];
    }

    /* Correction at k < B: w = max(0, p'_k - q'_k); bonus at k = B: w = p'_B. */
    double S = 0.0;
    psispec_oracle_row_probs(prow0 + (size_t)k * V * es, dtype, V, T, top_p, pp, NULL);
    if (k < B) {
      psispec_oracle_row_probs(qrow0 + (size_t)k * V * es, dtype, V, T, top_p, qq, NULL);
      for (int x = 0; x < V; ++x) {
        double diff = pp[x] - qq[x];
        w[x] = diff > 0.0 ? diff : 0.0;
        S += w[x];
      }
      if (!(S > 0.0)) {
        /* unreachable in exact arithmetic (p' = q' always accepts); documented fallback */
        st |= ORC_ST_RESID_ZERO;
        S = 0.0;
        for (int x = 0; x < V; ++x) {
          w[x] = pp[x];
          S += w[x];
        }
      }
    } else {
      for (int x = 0; x < V; ++x) {
        w[x] = pp[x];
        S += w[x];
      }
    }
    double u2 = u_resample ? u_resample[r]
                           : psispec_oracle_uniform(seed, req, (uint32_t)k, ORC_PURPOSE_RESAMPLE, step);
    double msample = 0.0;
    int c = inverse_cdf(w, V, S, u2, &msample);

    accept_len[r] = k;
    int32_t* out = out_tokens + (size_t)r * (B + 1);
    for (int i = 0; i < B + 1; ++i) out[i] = -1;
    for (int i = 0; i < k; ++i) out[i] = d[i];
    out[k] = c;
    if (accept_mask) accept_mask[r] = mask;
    if (status) status[r] = st;
    if (margin_sample) margin_sample[r] = msample;
    if (resid_w) memcpy(resid_w + (size_t)r * V, w, sizeof(double) * (size_t)V);
    if (resid_S) resid_S[r] = S;
  }
  free(pp);
  free(qq);
  free(w);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * Drafting ([alphalab] walkthrough steps 1-2: the AR path samples the first token of the block, the
 * diffusion path proposes the remaining ones in parallel; [lanes] "Ψ-Spec이 한 스텝에서 하는 일": the
 * same model drafts the block).  Each drafted token is one inverse-CDF draw from its row after the
 * same temperature and nucleus transform the verify applies (the verify is lossless only when the
 * drafts come from exactly the q' it divides by).  Row of position i: with FIRST_FROM_TARGET and
 * i = 0 the AR row of the request (ar + r * ar_stride elements), else q row i of the request
 * (q[batch][B][V]; row 0 is then not read).  The uniform is the Philox value at
 * (request_base + r, i, DRAFT, step), or u_draw[r][i] when given.
 * ---------------------------------------------------------------------------------------------- */
int psispec_oracle_sample_drafts(const void* ar, int64_t ar_stride, const void* q, int dtype,
                                 int batch, int B, int V, double T, double top_p, uint64_t seed,
                                 uint32_t step, uint32_t request_base, uint32_t flags,
                                 const double* u_draw, int32_t* tokens, int32_t* status,
                                 double* margin_sample, double* margin_topp) {
  if (!tokens || batch < 0 || B < 1 || B > 64 || V < 1) return ORC_EINVAL;
  if (!(T > 0.0) || !isfinite(T) || !(top_p > 0.0) || !(top_p <= 1.0)) return ORC_EINVAL;
  int first_from_target = (flags & ORC_FIRST_FROM_TARGET) != 0;
  if (first_from_target && (!ar || ar_stride < V)) return ORC_EINVAL;
  if (!q && !(first_from_target && B == 1)) return ORC_EINVAL;
  size_t es = elem_size(dtype);
  double* pi = (double*)malloc(sizeof(double) * (size_t)V);
  for (int r = 0; r < batch; ++r) {
    for (int i = 0; i < B; ++i) {
      const char* row;
      if (first_from_target && i == 0)
        row = (const char*)ar + (size_t)r * (size_t)ar_stride * es;
      else
        row = (const char*)q + ((size_t)r * (size_t)B + (size_t)i) * (size_t)V * es;
      double mt = INFINITY;
      int st = psispec_oracle_row_probs(row, dtype, V, T, top_p, pi, &mt);
      double S = 0.0;
      for (int x = 0; x < V; ++x) S += pi[x];
      double u = u_draw ? u_draw[(size_t)r * B + i]
                        : psispec_oracle_uniform(seed, request_base + (uint32_t)r, (uint32_t)i,
                                                 ORC_PURPOSE_DRAFT, step);
      double ms = 0.0;
      int c = inverse_cdf(pi, V, S, u, &ms);
      tokens[(size_t)r * B + i] = c;
      if (status) status[(size_t)r * B + i] = st;
      if (margin_sample) margin_sample[(size_t)r * B + i] = ms;
      if (margin_topp) margin_topp[(size_t)r * B + i] = mt;
    }
  }
  free(pi);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * Tree verify ([alphalab] "Linear 與 Tree sampler": several likely candidates per position, pruned to
 * a finite prefix tree that is verified at once).  The pages give no rule; we take the lossless rule
 * for candidates chosen deterministically (top-k): at node v with distribution pi_v, children are
 * tried in ascending node index; child c is kept with probability res(tok_c) / R, where res is pi_v
 * with the tokens of already-rejected siblings removed and R its remaining mass; a rejected child's
 * token is removed from res.  If no child is kept (or v is a leaf) one token is drawn from res.
 * This is the linear rule with a point-mass proposal on tok_c.
 *
 * Rows per request: row 0 = root, row j+1 = node j.  parent[j] in [-1, j-1] (-1 = root).
 * Uniforms: accept of node c at (request, c+1, ACCEPT); final draw at (request, row, RESAMPLE).
 * ---------------------------------------------------------------------------------------------- */
int psispec_oracle_verify_tree(const void* p, int dtype, const int32_t* parent,
                               const int32_t* node_tokens, int batch, int N, int V, int max_depth,
                               double T, double top_p, uint64_t seed, uint32_t step,
                               uint32_t request_base, const double* u_accept,
                               const double* u_resample, int32_t* accept_len, int32_t* accept_nodes,
                               int32_t* out_tokens, double* node_ratios, int32_t* status,
                               double* margin_accept, double* margin_sample, double* margin_topp,
                               double* resid_w, double* resid_S) {
  if (!p || !parent || !node_tokens || !accept_len || !accept_nodes || !out_tokens) return ORC_EINVAL;
  if (batch < 0 || N < 1 || V < 1 || max_depth < 1) return ORC_EINVAL;
  if (!(T > 0.0) || !isfinite(T) || !(top_p > 0.0) || !(top_p <= 1.0)) return ORC_EINVAL;
  size_t es = elem_size(dtype);
  double* pi = (double*)malloc(sizeof(double) * (size_t)V);
  double* res = (double*)malloc(sizeof(double) * (size_t)V);
  int* depth = (int*)malloc(sizeof(int) * (size_t)N);
  double* ratio = (double*)malloc(sizeof(double) * (size_t)N);

  for (int r = 0; r < batch; ++r) {
    const char* rows = (const char*)p + (size_t)r * (size_t)(N + 1) * (size_t)V * es;
    const int32_t* par = parent + (size_t)r * N;
    const int32_t* tok = node_tokens + (size_t)r * N;
    uint32_t req = request_base + (uint32_t)r;
    int st = 0;

    /* structure check: parents precede children, depth within max_depth */
    for (int j = 0; j < N; ++j) {
      if (par[j] < -1 || par[j] >= j) {
        st |= ORC_ST_BAD_PARENT;
        depth[j] = 1;
        continue;
      }
      depth[j] = par[j] < 0 ? 1 : depth[par[j]] + 1;
      if (depth[j] > max_depth) st |= ORC_ST_BAD_PARENT;
    }

    /* Row transforms of every row (for margins and status), and data-parallel node ratios: each
     * node's ratio assumes every earlier sibling was rejected. */
    for (int row = 0; row <= N; ++row) {
      double mt = INFINITY;
      st |= psispec_oracle_row_probs(rows + (size_t)row * V * es, dtype, V, T, top_p, pi, &mt);
      if (margin_topp) margin_topp[(size_t)r * (N + 1) + row] = mt;
      int v = row - 1; /* node whose children are scored by this row (-1 = root) */
      memcpy(res, pi, sizeof(double) * (size_t)V);
      double R = 1.0;
      for (int c = 0; c < N; ++c) {
        if (par[c] != v) continue;
        double rc = 0.0;
        if (tok[c] < 0 || tok[c] >= V) {
          st |= ORC_ST_BAD_TOKEN;
        } else {
          rc = R > 0.0 ? res[tok[c]] / R : 0.0;
          if (rc > 1.0) rc = 1.0;
          R -= res[tok[c]];
          res[tok[c]] = 0.0;
        }
        ratio[c] = rc;
      }
    }
    for (int c = 0; c < N; ++c) {
      if (node_ratios) node_ratios[(size_t)r * N + c] = ratio[c];
      if (margin_accept) margin_accept[(size_t)r * N + c] = INFINITY;
    }

    int32_t* nodes = accept_nodes + (size_t)r * max_depth;
    int32_t* out = out_tokens + (size_t)r * (max_depth + 1);
    for (int i = 0; i < max_depth; ++i) nodes[i] = -1;
    for (int i = 0; i < max_depth + 1; ++i) out[i] = -1;
    if (st & ORC_ST_BAD_PARENT) {
      accept_len[r] = 0;
      if (status) status[r] = st;
      if (margin_sample) margin_sample[r] = INFINITY;
      if (resid_S) resid_S[r] = 0.0;
      continue;
    }

    /* the walk */
    int cur = -1, dep = 0;
    for (;;) {
      int row = cur + 1;
      psispec_oracle_row_probs(rows + (size_t)row * V * es, dtype, V, T, top_p, pi, NULL);
      memcpy(res, pi, sizeof(double) * (size_t)V);
      int next = -1;
      for (int c = 0; c < N; ++c) {
        if (par[c] != cur) continue;
        double u = u_accept ? u_accept[(size_t)r * N + c]
                            : psispec_oracle_uniform(seed, req, (uint32_t)(c + 1), ORC_PURPOSE_ACCEPT,
                                                     step);
        if (margin_accept) margin_accept[(size_t)r * N + c] = fabs(u - ratio[c]);
        if (u < ratio[c]) {
          next = c;
          break;
        }
        if (tok[c] >= 0 && tok[c] < V) res[tok[c]] = 0.0;
      }
      if (next >= 0) {
        nodes[dep] = next;
        out[dep] = tok[next];
        ++dep;
        cur = next;
        continue;
      }
      /* final draw from the residual of the stopping node (a leaf gives the bonus token) */
      double S = 0.0;
      for (int x = 0; x < V; ++x) S += res[x];
      if (!(S > 0.0)) {
        st |= ORC_ST_RESID_ZERO;
        memcpy(res, pi, sizeof(double) * (size_t)V);
        S = 0.0;
        for (int x = 0; x < V; ++x) S += res[x];
      }
      double u2 = u_resample ? u_resample[r]
                             : psispec_oracle_uniform(seed, req, (uint32_t)row, ORC_PURPOSE_RESAMPLE,
                                                      step);
      double ms = 0.0;
      out[dep] = inverse_cdf(res, V, S, u2, &ms);
      if (margin_sample) margin_sample[r] = ms;
      if (resid_w) memcpy(resid_w + (size_t)r * V, res, sizeof(double) * (size_t)V);
      if (resid_S) resid_S[r] = S;
      break;
    }
    accept_len[r] = dep;
    if (status) status[r] = st;
  }
  free(pi);
  free(res);
  free(depth);
  free(ratio);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * LM-head logits in fp64 ([lanes] "헤드냐, LoRA냐": the draft path adds a LoRA delta to the frozen AR
 * weights; here only the output projection).  out[i][v] = sum_h h[i][h] W[h][v], plus, when A is
 * given, scale * sum_j (sum_h h[i][h] A[h][j]) Bl[j][v].  Sums run by ascending index.
 * ---------------------------------------------------------------------------------------------- */
static double bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int psispec_oracle_lmhead_logits(const uint16_t* h, const uint16_t* W, const uint16_t* A,
                                 const uint16_t* Bl, double scale, int M, int H, int V, int r,
                                 double* out) {
  if (!h || !W || !out || M < 0 || H < 1 || V < 1) return ORC_EINVAL;
  if (A && (!Bl || r < 1)) return ORC_EINVAL;
  double* hrow = (double*)malloc(sizeof(double) * (size_t)H);
  double* t = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
  for (int i = 0; i < M; ++i) {
    double* o = out + (size_t)i * V;
    for (int k = 0; k < H; ++k) hrow[k] = bf16_to_double(h[(size_t)i * H + k]);
    for (int v = 0; v < V; ++v) o[v] = 0.0;
    for (int k = 0; k < H; ++k) {
      const uint16_t* wrow = W + (size_t)k * V;
      double hk = hrow[k];
      for (int v = 0; v < V; ++v) o[v] += hk * bf16_to_double(wrow[v]);
    }
    if (A) {
      for (int j = 0; j < r; ++j) {
        double s = 0.0;
        for (int k = 0; k < H; ++k) s += hrow[k] * bf16_to_double(A[(size_t)k * r + j]);
        t[j] = s;
      }
      for (int j = 0; j < r; ++j) {
        const uint16_t* brow = Bl + (size_t)j * V;
        for (int v = 0; v < V; ++v) o[v] += scale * t[j] * bf16_to_double(brow[v]);
      }
    }
  }
  free(hrow);
  free(t);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * Tree verify with sampled candidates ([alphalab] "Linear 與 Tree sampler" leaves the candidate rule
 * open).  Reading: the children of node v were drawn independently from v's draft distribution
 * q'_v (row v+1 of q; row 0 for the root), in ascending node index.  The lossless rule for such
 * candidates is recursive rejection: with r_0 = p'_v, child i (the i-th child of v) is kept with
 * probability min(1, r_{i-1}(x_i) / q'_v(x_i)); when it is rejected the residual becomes
 * r_i = max(0, r_{i-1} - q'_v) renormalised.  If no child is kept (or v is a leaf) one token is drawn
 * from r_m, m the number of children.  q'_v(x_i) = 0 (x_i could not have been drawn): the ratio is 1
 * when r_{i-1}(x_i) > 0, else 0, and status Q_ZERO is set; a zero residual mass (unreachable in
 * exact arithmetic: r_{i-1} = q'_v accepts every candidate) keeps r_{i-1} and sets RESID_ZERO.
 * Node ratios are computed for every node as if all its earlier siblings were rejected.
 * Uniforms as in the deterministic tree: child c at (request, c+1, ACCEPT), the draw at (request,
 * row of the stopping node, RESAMPLE).  margin_topp: [batch][2(N+1)], p rows then q rows.
 * ---------------------------------------------------------------------------------------------- */
static double residual_step(double* res, const double* qv, int V) {
  double Z = 0.0;
  for (int x = 0; x < V; ++x) {
    double d = res[x] - qv[x];
    res[x] = d > 0.0 ? d : 0.0;
    Z += res[x];
  }
  if (Z > 0.0)
    for (int x = 0; x < V; ++x) res[x] = res[x] / Z;
  return Z;
}

int psispec_oracle_verify_tree_sampled(const void* p, const void* q, int dtype,
                                       const int32_t* parent, const int32_t* node_tokens,
                                       int batch, int N, int V, int max_depth, double T,
                                       double top_p, uint64_t seed, uint32_t step,
                                       uint32_t request_base, const double* u_accept,
                                       const double* u_resample, int32_t* accept_len,
                                       int32_t* accept_nodes, int32_t* out_tokens,
                                       double* node_ratios, int32_t* status,
                                       double* margin_accept, double* margin_sample,
                                       double* margin_topp, double* resid_w, double* resid_S) {
  if (!p || !q || !parent || !node_tokens || !accept_len || !accept_nodes || !out_tokens)
    return ORC_EINVAL;
  if (batch < 0 || N < 1 || V < 1 || max_depth < 1) return ORC_EINVAL;
  if (!(T > 0.0) || !isfinite(T) || !(top_p > 0.0) || !(top_p <= 1.0)) return ORC_EINVAL;
  size_t es = elem_size(dtype);
  double* pi = (double*)malloc(sizeof(double) * (size_t)V);
  double* qv = (double*)malloc(sizeof(double) * (size_t)V);
  double* res = (double*)malloc(sizeof(double) * (size_t)V);
  int* depth = (int*)malloc(sizeof(int) * (size_t)N);
  double* ratio = (double*)malloc(sizeof(double) * (size_t)N);

  for (int r = 0; r < batch; ++r) {
    const char* prows = (const char*)p + (size_t)r * (size_t)(N + 1) * (size_t)V * es;
    const char* qrows = (const char*)q + (size_t)r * (size_t)(N + 1) * (size_t)V * es;
    const int32_t* par = parent + (size_t)r * N;
    const int32_t* tok = node_tokens + (size_t)r * N;
    uint32_t req = request_base + (uint32_t)r;
    int st = 0;

    for (int j = 0; j < N; ++j) {
      if (par[j] < -1 || par[j] >= j) {
        st |= ORC_ST_BAD_PARENT;
        depth[j] = 1;
        continue;
      }
      depth[j] = par[j] < 0 ? 1 : depth[par[j]] + 1;
      if (depth[j] > max_depth) st |= ORC_ST_BAD_PARENT;
    }

    /* data-parallel node ratios: the residual sequence of every node with children */
    for (int row = 0; row <= N; ++row) {
      double mp = INFINITY, mq = INFINITY;
      st |= psispec_oracle_row_probs(prows + (size_t)row * V * es, dtype, V, T, top_p, pi, &mp);
      st |= psispec_oracle_row_probs(qrows + (size_t)row * V * es, dtype, V, T, top_p, qv, &mq);
      if (margin_topp) {
        margin_topp[(size_t)r * 2 * (N + 1) + row] = mp;
        margin_topp[(size_t)r * 2 * (N + 1) + (N + 1) + row] = mq;
      }
      int v = row - 1;
      memcpy(res, pi, sizeof(double) * (size_t)V);
      for (int c = 0; c < N; ++c) {
        if (par[c] != v) continue;
        double rc = 0.0;
        if (tok[c] < 0 || tok[c] >= V) {
          st |= ORC_ST_BAD_TOKEN;
        } else if (qv[tok[c]] > 0.0) {
          rc = res[tok[c]] / qv[tok[c]];
          if (rc > 1.0) rc = 1.0;
        } else {
          rc = res[tok[c]] > 0.0 ? 1.0 : 0.0;
          st |= ORC_ST_Q_ZERO;
        }
        ratio[c] = rc;
        /* the residual if this child is rejected (the next sibling's test uses it) */
        double* keep = (double*)malloc(sizeof(double) * (size_t)V);
        memcpy(keep, res, sizeof(double) * (size_t)V);
        if (!(residual_step(res, qv, V) > 0.0)) memcpy(res, keep, sizeof(double) * (size_t)V);
        free(keep);
      }
    }
    for (int c = 0; c < N; ++c) {
      if (node_ratios) node_ratios[(size_t)r * N + c] = ratio[c];
      if (margin_accept) margin_accept[(size_t)r * N + c] = INFINITY;
    }

    int32_t* nodes = accept_nodes + (size_t)r * max_depth;
    int32_t* out = out_tokens + (size_t)r * (max_depth + 1);
    for (int i = 0; i < max_depth; ++i) nodes[i] = -1;
    for (int i = 0; i < max_depth + 1; ++i) out[i] = -1;
    if (st & ORC_ST_BAD_PARENT) {
      accept_len[r] = 0;
      if (status) status[r] = st;
      if (margin_sample) margin_sample[r] = INFINITY;
      if (resid_S) resid_S[r] = 0.0;
      continue;
    }

    /* the walk: at each node the children in index order against the current residual */
    int cur = -1, dep = 0;
    for (;;) {
      int row = cur + 1;
      psispec_oracle_row_probs(prows + (size_t)row * V * es, dtype, V, T, top_p, pi, NULL);
      psispec_oracle_row_probs(qrows + (size_t)row * V * es, dtype, V, T, top_p, qv, NULL);
      memcpy(res, pi, sizeof(double) * (size_t)V);
      int next = -1;
      for (int c = 0; c < N; ++c) {
        if (par[c] != cur) continue;
        double u = u_accept ? u_accept[(size_t)r * N + c]
                            : psispec_oracle_uniform(seed, req, (uint32_t)(c + 1), ORC_PURPOSE_ACCEPT,
                                                     step);
        if (margin_accept) margin_accept[(size_t)r * N + c] = fabs(u - ratio[c]);
        if (u < ratio[c]) {
          next = c;
          break;
        }
        double* keep = (double*)malloc(sizeof(double) * (size_t)V);
        memcpy(keep, res, sizeof(double) * (size_t)V);
        if (!(residual_step(res, qv, V) > 0.0)) {
          st |= ORC_ST_RESID_ZERO;
          memcpy(res, keep, sizeof(double) * (size_t)V);
        }
        free(keep);
      }
      if (next >= 0) {
        nodes[dep] = next;
        out[dep] = tok[next];
        ++dep;
        cur = next;
        continue;
      }
      double S = 0.0;
      for (int x = 0; x < V; ++x) S += res[x];
      double u2 = u_resample ? u_resample[r]
                             : psispec_oracle_uniform(seed, req, (uint32_t)row, ORC_PURPOSE_RESAMPLE,
                                                      step);
      double ms = 0.0;
      out[dep] = inverse_cdf(res, V, S, u2, &ms);
      if (margin_sample) margin_sample[r] = ms;
      if (resid_w) memcpy(resid_w + (size_t)r * V, res, sizeof(double) * (size_t)V);
      if (resid_S) resid_S[r] = S;
      break;
    }
    accept_len[r] = dep;
    if (status) status[r] = st;
  }
  free(pi);
  free(qv);
  free(res);
  free(depth);
  free(ratio);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * KV commit after a verify ([lanes] "헤드냐, LoRA냐": the draft and the verify share one KV line per
 * sequence, the AR verifies and appends; [alphalab] walkthrough step 4: the accepted prefix is kept,
 * everything after the first rejection is discarded and drafted again next round).  Reading: the
 * verify forward wrote the KV rows of the block's blk positions at positions len .. len+blk-1 of the
 * request's line; the kept rows (their block positions keep[0..n-1], strictly increasing) move to
 * len .. len+n-1 in that order, len grows by n, and the rows past the new length are free again.
 * The rows are opaque bytes.  A request whose n, keep or len is invalid (n outside [0, blk],
 * keep not strictly increasing within [0, blk), len < 0 or len + blk > Lmax) is left unchanged and
 * flagged.
 * ---------------------------------------------------------------------------------------------- */
int psispec_oracle_kv_commit(void* kv, int64_t line_stride, int64_t row_bytes, int Lmax, int blk,
                             const int32_t* keep, int keep_stride, const int32_t* n_keep,
                             int32_t* len, int32_t* status, int batch) {
  if (!kv || !n_keep || !len || batch < 0 || row_bytes < 1 || Lmax < 1 || blk < 1 || blk > Lmax)
    return ORC_EINVAL;
  if (keep && keep_stride < 1) return ORC_EINVAL;
  unsigned char* old = (unsigned char*)malloc((size_t)blk * (size_t)row_bytes);
  for (int r = 0; r < batch; ++r) {
    int n = n_keep[r], L = len[r];
    int ok = n >= 0 && n <= blk && L >= 0 && L <= Lmax - blk && (!keep || n <= keep_stride);
    for (int i = 0; ok && keep && i < n; ++i) {
      int k = keep[(size_t)r * keep_stride + i];
      if (k < 0 || k >= blk) ok = 0;
      if (i > 0 && k <= keep[(size_t)r * keep_stride + i - 1]) ok = 0;
    }
    if (status) status[r] = ok ? 0 : ORC_ST_BAD_KEEP;
    if (!ok) continue;
    unsigned char* block = (unsigned char*)kv + (size_t)r * (size_t)line_stride +
                           (size_t)L * (size_t)row_bytes;
    memcpy(old, block, (size_t)blk * (size_t)row_bytes);
    for (int i = 0; i < n; ++i) {
      int k = keep ? keep[(size_t)r * keep_stride + i] : i;
      memcpy(block + (size_t)i * (size_t)row_bytes, old + (size_t)k * (size_t)row_bytes,
             (size_t)row_bytes);
    }
    len[r] = L + n;
  }
  free(old);
  return ORC_OK;
}
