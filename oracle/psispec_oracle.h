/*
 * psispec_oracle.h -- declarations of the CPU oracle for the Psi-Spec verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded fp64 reference used to check the
 * GPU library.  Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no source with the HIP library (lossless_draft_verification_spec_amd/csrc) and
 * the HIP library never calls it.
 *
 * Sources (cited by page title and section; the pages are web articles about Uno / Psi-Spec):
 *   [alphalab]  "Uno Psi-Spec 是什麼？Diffusion-Augmented LLM 如何保留 AR 分布、一次驗證多個 Token",
 *               sections "Uno Ψ-Spec 怎麼運作？完整走一次四個 Token" (the B=4 walkthrough),
 *               "為什麼 lossless 不等於答案完全一樣？" and "Linear 與 Tree sampler".
 *   [lanes]     "Uno / Ψ-Spec — 같은 모델 안에서 초안 뽑고 AR로 도장 찍기",
 *               sections "Ψ-Spec이 한 스텝에서 하는 일" and "어디서 왔나" (Leviathan et al. 2023 lineage).
 *   [philox]    Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
 */
#ifndef PSISPEC_ORACLE_H
#define PSISPEC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of logits rows */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* oracle-only: fp64 logits produced by the oracle's own LM-head GEMM */

/* sampling flags */
#define ORC_FIRST_FROM_TARGET 1u

/* Philox purposes (counter word 2) */
#define ORC_PURPOSE_ACCEPT 0u
#define ORC_PURPOSE_RESAMPLE 1u
#define ORC_PURPOSE_DRAFT 2u

/* per-request status bits (data errors, never abort) */
#define ORC_ST_NONFINITE 1   /* a row read by the request holds NaN/+Inf or no finite logit */
#define ORC_ST_BAD_TOKEN 2   /* a draft/node token outside [0, V) */
#define ORC_ST_Q_ZERO 4      /* draft probability of a drafted token is zero */
#define ORC_ST_RESID_ZERO 8  /* residual mass zero at a rejection: fell back to the target row */
#define ORC_ST_BAD_PARENT 16 /* tree: parent[j] not in [-1, j-1] or depth beyond max_depth */
#define ORC_ST_BAD_KEEP 32   /* KV commit: kept count, kept positions or length invalid */

/* return codes */
#define ORC_OK 0
#define ORC_EINVAL -1

/* Philox4x32-10 block: out = Philox(key = (lo32(seed), hi32(seed)), counter = ctr). */
void psispec_oracle_philox(uint64_t seed, const uint32_t ctr[4], uint32_t out[4]);

/* 53-bit uniform in [0,1) from the Philox block at counter (request, position, purpose, step). */
double psispec_oracle_uniform(uint64_t seed, uint32_t request, uint32_t position, uint32_t purpose,
                              uint32_t step);

/* Probabilities of one logits row after temperature and (optional) nucleus truncation.
 * pi[V] receives them; *topp_margin (nullable) the nucleus boundary margin; returns status bits. */
int psispec_oracle_row_probs(const void* row, int dtype, int V, double T, double top_p, double* pi,
                             double* topp_margin);

int psispec_oracle_verify_linear(const void* p, const void* q, int dtype, const int32_t* draft,
                                 int batch, int B, int V, double T, double top_p, uint64_t seed,
                                 uint32_t step, uint32_t request_base, uint32_t flags,
                                 const double* u_accept, const double* u_resample,
                                 int32_t* accept_len, int32_t* out_tokens, double* ratios,
                                 uint64_t* accept_mask, int32_t* status, double* margin_accept,
                                 double* margin_sample, double* margin_topp, double* resid_w,
                                 double* resid_S);

/* Tree verify with candidates drawn from q (recursive rejection); q [batch][N+1][V] like p;
 * margin_topp [batch][2(N+1)]. */
int psispec_oracle_verify_tree_sampled(const void* p, const void* q, int dtype,
                                       const int32_t* parent, const int32_t* node_tokens,
                                       int batch, int N, int V, int max_depth, double T,
                                       double top_p, uint64_t seed, uint32_t step,
                                       uint32_t request_base, const double* u_accept,
                                       const double* u_resample, int32_t* accept_len,
                                       int32_t* accept_nodes, int32_t* out_tokens,
                                       double* node_ratios, int32_t* status,
                                       double* margin_accept, double* margin_sample,
                                       double* margin_topp, double* resid_w, double* resid_S);

/* Drafting: tokens[r][i] ~ p'(row) by inverse CDF with the Philox value at (request, i, DRAFT, step)
 * (or u_draw[r][i]); row = AR row r (ar + r * ar_stride elements) for i = 0 with FIRST_FROM_TARGET,
 * else q[r][i].  status/margins [batch][B], nullable. */
int psispec_oracle_sample_drafts(const void* ar, int64_t ar_stride, const void* q, int dtype,
                                 int batch, int B, int V, double T, double top_p, uint64_t seed,
                                 uint32_t step, uint32_t request_base, uint32_t flags,
                                 const double* u_draw, int32_t* tokens, int32_t* status,
                                 double* margin_sample, double* margin_topp);

int psispec_oracle_verify_tree(const void* p, int dtype, const int32_t* parent,
                               const int32_t* node_tokens, int batch, int N, int V, int max_depth,
                               double T, double top_p, uint64_t seed, uint32_t step,
                               uint32_t request_base, const double* u_accept,
                               const double* u_resample, int32_t* accept_len, int32_t* accept_nodes,
                               int32_t* out_tokens, double* node_ratios, int32_t* status,
                               double* margin_accept, double* margin_sample, double* margin_topp,
                               double* resid_w, double* resid_S);

/* fp64 LM-head logits: out[M][V] = h[M][H] * W[H][V] (+ (h*A)[M][r] * Bl[r][V] * scale when A != NULL).
 * h, W, A, Bl are bf16 bit patterns. */
int psispec_oracle_lmhead_logits(const uint16_t* h, const uint16_t* W, const uint16_t* A,
                                 const uint16_t* Bl, double scale, int M, int H, int V, int r,
                                 double* out);

/* KV commit: in line r (kv + r * line_stride bytes, rows of row_bytes), the block's rows at
 * len[r] + keep[r][i] (keep NULL: i) move to len[r] + i for i < n_keep[r]; len[r] += n_keep[r].
 * status [batch] nullable. */
int psispec_oracle_kv_commit(void* kv, int64_t line_stride, int64_t row_bytes, int Lmax, int blk,
                             const int32_t* keep, int keep_stride, const int32_t* n_keep,
                             int32_t* len, int32_t* status, int batch);

#ifdef __cplusplus
}
#endif
#endif
