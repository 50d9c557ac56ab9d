/*
 * psispec.h -- C ABI of the Psi-Spec verify step on MI355X (gfx950).
 *
 * The verify step of Uno's Psi-Spec sampler: a frozen AR model has scored a block of B drafted
 * tokens (plus the row after the block) in one pass; the verifier applies an acceptance test to the
 * drafts in order, keeps the longest accepted run from the start, draws a replacement token from a
 * corrected residual distribution at the first rejection and discards the rest, or draws one extra
 * token from the block-end row when every draft passes.  Sources, cited by page title and section:
 *
 *   [alphalab] "Uno Ψ-Spec 是什麼？Diffusion-Augmented LLM 如何保留 AR 分布、一次驗證多個 Token":
 *              §"Uno Ψ-Spec 怎麼運作？完整走一次四個 Token" (steps 1-4 and the full-accept paragraph),
 *              §"為什麼 lossless 不等於答案完全一樣？" (the output law equals the AR's),
 *              §"Linear 與 Tree sampler" (one candidate per position vs a pruned prefix tree).
 *   [lanes]    "Uno / Ψ-Spec — 같은 모델 안에서 초안 뽑고 AR로 도장 찍기":
 *              §"Ψ-Spec이 한 스텝에서 하는 일" (frozen AR verifies, longest prefix kept),
 *              §"어디서 왔나" (speculative sampling of Leviathan et al. 2023 as the lineage).
 *
 * The pages print no formula.  The rule implemented is the speculative-sampling rule of that
 * lineage: accept draft d at position i when u_i < min(1, p'_i(d) / q'_i(d)); at the first rejected
 * position k draw from max(0, p'_k - q'_k) renormalised; after a full accept draw from p'_B.  p' and
 * q' are softmax(logits / temperature), optionally truncated to the tie-inclusive nucleus of mass
 * top_p and renormalised.  Uniforms come from Philox4x32-10 (Salmon et al., SC'11) with key = seed
 * and counter = (request_base + request, position, purpose, step); u = top 53 bits of
 * (word0 << 32 | word1) times 2^-53.  Purposes: 0 = accept test, 1 = final draw, 2 = drafting.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; rows are contiguous with V elements.
 *     The library never allocates or frees: its scratch lives in the caller's `workspace`
 *     (device memory, >= the size returned by the matching *_workspace query, 256-byte aligned).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream), never
 *     synchronise the host, and are reentrant.  Concurrent calls need distinct workspaces.
 *     Outputs are a pure function of the inputs and (seed, step, request_base): reruns are bitwise
 *     identical.
 *   - Host-detectable errors (null pointers, bad sizes, temperature <= 0 or not finite, top_p
 *     outside (0, 1], bad dtype, small workspace) return a negative code and launch nothing;
 *     a failed launch returns PSISPEC_EHIP.
 *   - Data errors found on the device never abort: they set bits in status[request] and leave that
 *     request's other outputs unspecified (but in bounds).  When an input error is flagged
 *     (NONFINITE, BAD_TOKEN, BAD_PARENT) the remaining status bits are unspecified as well.
 */
#ifndef PSISPEC_H
#define PSISPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PSISPEC_OK = 0,
  PSISPEC_EINVAL = -1,       /* bad pointer, size or sampling parameter */
  PSISPEC_EDTYPE = -2,       /* unsupported element type */
  PSISPEC_EWORKSPACE = -3,   /* workspace missing, too small or misaligned */
  PSISPEC_EHIP = -4,         /* a HIP call or kernel launch failed */
  PSISPEC_EUNSUPPORTED = -5, /* a mode that is not implemented */
  PSISPEC_ESCRATCH = -6      /* sizes beyond the fixed scratch of the no-allocation entry point */
} psispec_status;

typedef enum { PSISPEC_F32 = 0, PSISPEC_BF16 = 1 } psispec_dtype;

/* flags */
#define PSISPEC_FIRST_FROM_TARGET 1u /* Uno layout: position 0 is the AR's own sample and is always
                                        kept ([alphalab] walkthrough step 1); q row 0 is not read */
/* Tree verify with q_logits only: PSISPEC_MAX_CHILDREN(k), 1 <= k <= 8, says that no node has more
   than k children (the drafter's branching), so the residual chain is built for k children only
   and its passes for more are not launched.  A node with more than k children is then reported
   with PSISPEC_ST_BAD_PARENT.  0 (not given) means 8.  Every other call rejects these bits. */
#define PSISPEC_MAX_CHILDREN_SHIFT 4
#define PSISPEC_MAX_CHILDREN_MASK (0xfu << PSISPEC_MAX_CHILDREN_SHIFT)
#define PSISPEC_MAX_CHILDREN(k) ((uint32_t)(k) << PSISPEC_MAX_CHILDREN_SHIFT)

/* per-request status bits */
#define PSISPEC_ST_NONFINITE 1   /* a row read by the request holds NaN/+Inf or no finite logit */
#define PSISPEC_ST_BAD_TOKEN 2   /* a drafted / node token outside [0, V) */
#define PSISPEC_ST_Q_ZERO 4      /* the draft probability of a drafted token is 0 (ratio set to
                                    1 if the target probability is positive, else 0) */
#define PSISPEC_ST_RESID_ZERO 8  /* residual mass 0 at a rejection: drew from the target row */
#define PSISPEC_ST_BAD_PARENT 16 /* tree: parent[j] outside [-1, j-1] or depth beyond max_depth */
#define PSISPEC_ST_BAD_KEEP 32   /* KV commit: kept count, kept positions or length invalid */

typedef struct {
  double temperature;    /* > 0 and finite: logits are divided by it */
  double top_p;          /* (0, 1]; 1 disables the nucleus truncation */
  uint64_t seed;         /* Philox key */
  uint32_t step;         /* Philox counter word 3 */
  uint32_t request_base; /* global id of request 0 (counter word 0 = request_base + request) */
  uint32_t flags;        /* PSISPEC_FIRST_FROM_TARGET, PSISPEC_MAX_CHILDREN(k) or 0 */
  uint32_t reserved;     /* must be 0 */
} psispec_sampling;

/*
 * Linear verify ([alphalab] §"Linear 與 Tree sampler": one candidate per position;
 * walkthrough steps 3-4 and the full-accept paragraph).
 *
 *   p_logits     [batch][B+1][V]  target (AR) logits; row i scores draft i, row B is the block end
 *   q_logits     [batch][B][V]    draft logits; row i is the distribution draft i was drawn from
 *   dtype        element type of p_logits and q_logits (PSISPEC_F32 or PSISPEC_BF16)
 *   draft_tokens [batch][B] int32 drafted tokens
 *   B            1..64;  V >= 1;  batch >= 0 (0 launches nothing)
 *   s            host pointer to the sampling parameters
 * Outputs (device):
 *   accept_len   [batch] int32    k = number of leading drafts kept, in [0, B]
 *   out_tokens   [batch][B+1]     d_0..d_{k-1}, then the correction (k < B) or bonus (k = B) token,
 *                                 then -1; k+1 tokens are committed
 *   ratios       [batch][B] f32   min(1, p'_i(d_i)/q'_i(d_i)) for every i (also past k); nullable
 *   accept_mask  [batch] u64      bit i set when u_i < ratio_i (every i); nullable
 *   status       [batch] int32    PSISPEC_ST_* bits; nullable
 */
size_t psispec_verify_linear_workspace(int32_t batch, int32_t B, int32_t V, psispec_dtype dtype);

psispec_status psispec_verify_linear(const void* p_logits, const void* q_logits, psispec_dtype dtype,
                                     const int32_t* draft_tokens, int32_t batch, int32_t B,
                                     int32_t V, const psispec_sampling* s, int32_t* accept_len,
                                     int32_t* out_tokens, float* ratios, uint64_t* accept_mask,
                                     int32_t* status, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Linear verify for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): psispec_verify_linear with the same
 * arguments, outputs, determinism and errors, but no workspace argument.  Its scratch is a fixed
 * 64 MiB array in device memory that the library holds on every GPU it runs on until the process
 * ends; the call allocates nothing.  Sizes whose workspace (psispec_verify_linear_workspace)
 * exceeds 64 MiB return PSISPEC_ESCRATCH and launch nothing (batch 256 fits at any B up to 64
 * and V up to 262,144; batch 512 at B = 8, V = 151,936 does not).  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (two streams, two host threads) race and must be
 * ordered by the caller.  Nothing in the array needs to start at zero; it keeps the last call's
 * contents.  (While psispec_timing_enable is on, the library's timing hooks create HIP events.)
 */
psispec_status psispec_verify_linear_noalloc(const void* p_logits, const void* q_logits,
                                             psispec_dtype dtype, const int32_t* draft_tokens,
                                             int32_t batch, int32_t B, int32_t V,
                                             const psispec_sampling* s, int32_t* accept_len,
                                             int32_t* out_tokens, float* ratios,
                                             uint64_t* accept_mask, int32_t* status, void* stream);

/*
 * Tree verify ([alphalab] §"Linear 與 Tree sampler": several likely candidates per position,
 * pruned to a finite prefix tree verified at once).  The rule for candidates chosen
 * deterministically (e.g. top-k of the draft): at node v, children are tried in ascending node
 * index; child c is kept when u_c < res(tok_c) / R, where res is p'_v with the tokens of the
 * already rejected siblings removed and R = 1 - their mass; a rejected child's token is removed
 * from res; when no child is kept (or v is a leaf) one token is drawn from res.  Node ratios are
 * computed for every node as if all its earlier siblings were rejected.
 *
 * With q_logits (candidates drawn from the draft), the rule is recursive rejection: at node v the
 * children were drawn independently from q'_v, in ascending node index; child i is kept when
 * u < min(1, r_{i-1}(tok) / q'_v(tok)), r_0 = p'_v, and a rejection replaces the residual by
 * max(0, r_{i-1} - q'_v) renormalised; with no child kept one token is drawn from the last
 * residual.  At most 8 children per node (PSISPEC_ST_BAD_PARENT otherwise).
 *
 *   p_logits     [batch][N+1][V]  row 0 = root, row j+1 = node j
 *   q_logits     NULL (candidates chosen, e.g. top-k of the draft), or [batch][N+1][V] draft logits
 *                whose row v+1 (row 0: the root) is the distribution node v's children were drawn
 *                from (the tree's shape must not depend on the drawn tokens)
 *   parent       [batch][N] int32 parent node of node j, -1 = root, must be < j
 *   node_tokens  [batch][N] int32 token of node j
 *   N            1..1024 nodes per request;  V >= 1;  batch >= 0 (0 launches nothing)
 *   max_depth    bound on the depth of any node (1..64)
 * Uniforms: node c's test at (request, c+1, accept); the final draw at (request, row, draw) where
 * row is the stopping node's row.
 * Outputs (device):
 *   accept_len   [batch] int32            depth of the kept path
 *   accept_nodes [batch][max_depth]       the kept nodes in order, then -1
 *   out_tokens   [batch][max_depth+1]     their tokens, then the drawn token, then -1
 *   node_ratios  [batch][N] f32           nullable
 *   status       [batch] int32            nullable
 * The workspace query covers both rules.
 */
size_t psispec_verify_tree_workspace(int32_t batch, int32_t N, int32_t V, psispec_dtype dtype);

psispec_status psispec_verify_tree(const void* p_logits, const void* q_logits, psispec_dtype dtype,
                                   const int32_t* parent, const int32_t* node_tokens, int32_t batch,
                                   int32_t N, int32_t V, int32_t max_depth,
                                   const psispec_sampling* s, int32_t* accept_len,
                                   int32_t* accept_nodes, int32_t* out_tokens, float* node_ratios,
                                   int32_t* status, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Drafting step ([alphalab] walkthrough steps 1-2: the AR path samples the first token of the
 * block, the diffusion path proposes the others in parallel).  Draws d_0..d_{B-1} of every request,
 * each from its row after the transform the verify applies (softmax(logits / temperature), then the
 * nucleus of mass top_p, renormalised): the verify is lossless only for drafts drawn from exactly
 * that q'.  Each draw is an inverse CDF by ascending token id with the Philox uniform of
 * (request_base + request, i, purpose 2 = draft, step), decided as in exact arithmetic: an fp32 pass
 * with a rigorous error bound settles a draw when the bound cannot change it, the others are drawn
 * in fp64 like the verify's final draw.
 *
 *   ar_logits    AR rows, read only with PSISPEC_FIRST_FROM_TARGET (may be NULL otherwise): the row
 *                of request r starts at element r * ar_stride; d_0 is drawn from it.  ar_stride >= V
 *                ((B+1)*V reads row 0 of the verify's p_logits [batch][B+1][V]; V reads packed
 *                [batch][V] rows)
 *   q_logits     [batch][B][V] draft rows; d_i is drawn from row i.  With PSISPEC_FIRST_FROM_TARGET
 *                row 0 is not read, and q_logits may be NULL when B = 1
 *   dtype        element type of ar_logits and q_logits (PSISPEC_F32 or PSISPEC_BF16)
 *   B            1..64;  V >= 1;  batch >= 0 (0 launches nothing)
 *   s            host pointer to the sampling parameters (the verify's temperature and top_p)
 * Outputs (device):
 *   draft_tokens [batch][B] int32   in [0, V)
 *   status       [batch][B] int32   PSISPEC_ST_NONFINITE when the row holds NaN/+Inf or no finite
 *                                   logit (that token is then unspecified); nullable
 * Rows that are 16-byte aligned with V * element size and ar_stride * element size multiples of 16
 * are read with 16-byte loads; any other layout is read element by element.
 */
size_t psispec_sample_drafts_workspace(int32_t batch, int32_t B, int32_t V, psispec_dtype dtype);

psispec_status psispec_sample_drafts(const void* ar_logits, int64_t ar_stride,
                                     const void* q_logits, psispec_dtype dtype, int32_t batch,
                                     int32_t B, int32_t V, const psispec_sampling* s,
                                     int32_t* draft_tokens, int32_t* status, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * KV commit after a verify ([lanes] §"헤드냐, LoRA냐": drafting and verifying share one KV line per
 * sequence, the AR verifies and appends; [alphalab] walkthrough step 4: the accepted prefix is kept,
 * the rest is discarded and drafted again).  The verify forward has written the KV rows of the
 * block's blk positions at positions len[r] .. len[r]+blk-1 of line r.  The kept rows, block
 * positions keep[r][0..n_keep[r]-1], move to len[r] .. len[r]+n_keep[r]-1 in that order and
 * len[r] grows by n_keep[r]; the rows past the new length are free (rolled back, untouched).
 *
 *   kv           device; line r starts at kv + r * line_stride bytes, position t at
 *                + t * row_bytes; rows are opaque bytes (any layout of layers, heads and K/V)
 *   line_stride  bytes, multiple of 16, >= Lmax * row_bytes
 *   row_bytes    bytes per position, a multiple of 16;  kv 16-byte aligned
 *   Lmax         positions per line;  blk: 1..min(Lmax, 1024) block positions
 *   keep         [batch][keep_stride] int32 kept block positions, strictly increasing in [0, blk)
 *                (the tree verify's accept_nodes as they are, keep_stride = max_depth), or NULL:
 *                the first n_keep positions (the linear verify: nothing moves)
 *   n_keep       [batch] int32 in [0, blk] (and <= keep_stride): the verify's accept_len
 *   len          [batch] int32, in/out, with len + blk <= Lmax
 *   status       [batch] int32, nullable: PSISPEC_ST_BAD_KEEP when n_keep, keep or len is invalid;
 *                that request's line and length are then left unchanged
 * Asynchronous on `stream`; no workspace.  Host-detectable errors return PSISPEC_EINVAL.
 */
psispec_status psispec_kv_commit(void* kv, int64_t line_stride, int64_t row_bytes, int32_t Lmax,
                                 int32_t blk, const int32_t* keep, int32_t keep_stride,
                                 const int32_t* n_keep, int32_t* len, int32_t* status,
                                 int32_t batch, void* stream);

/*
 * LM head + linear verify ([lanes] §"헤드냐, LoRA냐": the draft path is the frozen AR weights plus a
 * low-rank LoRA delta; [alphalab] walkthrough steps 2-3: the draft rows go through the LoRA path, the
 * AR path scores the block).  Computes, on the bf16 matrix cores with fp32 accumulation,
 *   p logits (AR rows)    = h_ar . W
 *   q logits (draft rows) = h_draft . W + lora_scale (h_draft . A) . B
 * and runs the linear verify on them (same sampling, outputs, statuses and Philox keys as
 * psispec_verify_linear on those fp32 logits).  The logits are not written to memory: the matrix
 * product's epilogue hands the verify each row's softmax statistics and the logit at each draft
 * token, and the one or two rows that the final draw reads (p_k and q_k at the first rejection k,
 * or the block-end row p_B) are recomputed, bit-identical, into the workspace.
 *
 *   h_ar      bf16 [batch][B+1][H]  final hidden states of the AR rows (row B = block end)
 *   h_draft   bf16 [batch][B][H]    final hidden states of the draft rows
 *   W         bf16 [H][V]           the LM-head weight (V contiguous)
 *   lora_A    bf16 [H][r]           the LoRA down-projection; NULL when r = 0
 *   lora_B    bf16 [r][V]           the LoRA up-projection (V contiguous); NULL when r = 0
 *   H         multiple of 64, at most 2^20;  V multiple of 8;  0 <= r <= 64;  B 1..64
 *   p_logits_dbg, q_logits_dbg
 *             fp32 [batch][B+1][V] and [batch][B][V], or both NULL (the logits are never
 *             materialised).  When given, the logits are also stored there and the final draw
 *             reads them instead of recomputing its rows.  With top_p < 1 both are required (the
 *             nucleus needs every row's values a second time): PSISPEC_EUNSUPPORTED otherwise.
 * h_ar, h_draft, W, lora_B and the logit buffers must be 16-byte aligned (PSISPEC_EINVAL
 * otherwise).  All inputs are read-only and caller-owned; the call is asynchronous on `stream`.
 * The product h_draft . A is formed in fp64 and enters the matrix product as a bf16 pair
 * (hi + lo, relative error 2^-17).
 */
size_t psispec_lmhead_verify_workspace(int32_t batch, int32_t B, int32_t H, int32_t V, int32_t r);

psispec_status psispec_lmhead_verify(const void* h_ar, const void* h_draft, const void* W,
                                     const void* lora_A, const void* lora_B, float lora_scale,
                                     int32_t batch, int32_t B, int32_t H, int32_t V, int32_t r,
                                     const int32_t* draft_tokens, const psispec_sampling* s,
                                     int32_t* accept_len, int32_t* out_tokens, float* ratios,
                                     uint64_t* accept_mask, int32_t* status, float* p_logits_dbg,
                                     float* q_logits_dbg, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Message for a return code (static string). */
const char* psispec_strerror(psispec_status code);

/*
 * Measured ceilings (for benchmarks; not steps of the verify).  psispec_peak_read reads every
 * 16-byte word of `buf` (device, 16-byte aligned, `bytes` long; make it larger than the 256 MB
 * last-level cache) once with nontemporal loads, each of `blocks` workgroups of 256 threads
 * streaming its own contiguous segment, and writes one word per block to out[blocks]:
 * bytes / kernel time is the sustained read bandwidth.  psispec_peak_mfma runs `iters` rounds of 16 independent v_mfma_f32_32x32x16_bf16 per
 * wave in `blocks` workgroups of four waves, with no memory traffic, and writes one float per
 * thread to out[blocks * 256]: blocks * 4 * iters * 16 * 32768 / kernel time is the bf16 matrix-core
 * issue rate at the clock the chip holds under that load.  Both are asynchronous on `stream`;
 * the kernels appear in the timing records as "peak_read" and "peak_mfma".
 */
psispec_status psispec_peak_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                                 void* stream);
psispec_status psispec_peak_mfma(int64_t iters, float* out, int32_t blocks, void* stream);

/*
 * Kernel timing (for benchmarks).  While enabled, every kernel launch of the library records a
 * start and a stop event through its own dispatch (hipExtLaunchKernelGGL) on the call's stream:
 * the events measure the kernel itself, as a profiler's kernel trace does.  psispec_timing_read synchronises those events and
 * returns, per kernel name, the summed device milliseconds and the launch count since the last
 * enable; it returns the number of kernels written (at most max_kernels).  names receives
 * max_kernels fixed slots of 64 bytes (NUL-terminated).
 */
psispec_status psispec_timing_enable(int32_t on);
int32_t psispec_timing_read(char* names, float* total_ms, int32_t* launches, int32_t max_kernels);

#ifdef __cplusplus
}
#endif
#endif /* PSISPEC_H */
