// launch.h -- host-side launchers of the kernels (one per .hip translation unit).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "internal.h"

namespace psispec {

// Kernel timing (api.hip).  While timing is enabled, timing_take hands out two events and
// timing_push files them under a kernel name; PSISPEC_LAUNCH launches through
// hipExtLaunchKernelGGL, whose dispatch records the events at the kernel's own start and end.
bool timing_take(hipEvent_t* start, hipEvent_t* stop);
void timing_push(const char* name, hipEvent_t start, hipEvent_t stop);

#define PSISPEC_LAUNCH(name, kernel, grid, block, shm, stream, ...)                           \
  do {                                                                                         \
    hipEvent_t psispec_e0_ = nullptr, psispec_e1_ = nullptr;                                   \
    const bool psispec_on_ = ::psispec::timing_take(&psispec_e0_, &psispec_e1_);              \
    hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, psispec_e0_, psispec_e1_, 0,       \
                          __VA_ARGS__);                                                        \
    if (psispec_on_) ::psispec::timing_push(name, psispec_e0_, psispec_e1_);                   \
  } while (0)

// rows.hip
hipError_t launch_rowstats(const RowSet& rs, psispec_dtype dtype, int nchunk, int chunk_elems,
                           float c, float2* part, hipStream_t stream);
hipError_t launch_topp(const RowSet& rs, psispec_dtype dtype, int nchunk, float c, double top_p,
                       const float2* part, ToppStat* topp, hipStream_t stream,
                       const RowStat* rowstat = nullptr);
// bf16 rows, top_p < 1 with (1 - top_p) / (4 V) >= 1e-30: the row pass (one pair per row, nchunk 1)
// and the nucleus in one read of every row
hipError_t launch_rowstats_topp(const RowSet& rs, float c, double top_p, float2* part,
                                ToppStat* topp, hipStream_t stream);

// linear.hip
struct LinearArgs {
  RowSet rs;
  const int32_t* draft;
  int batch, B, V, nchunk;
  float c;            // log2(e) / T in fp32 (main-pass exponent scale)
  double inv_T;       // 1 / T in fp64
  int use_topp;
  uint64_t seed;
  uint32_t step, request_base, flags;
  const float2* part;
  const ToppStat* topp;
  RowStat* rowstat;
  int rowstat_ready;  // rowstat already holds every row's statistics (launch_combine_rows)
  const float* gath;  // logit at each row's draft token (LM-head epilogue), or null: read the rows
  DrawDesc* desc;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* ratios;
  uint64_t* accept_mask;
  // the accept test fused with the draw pass: the statistics of the request's rows (local row j:
  // p rows 0..B, then q rows) and its draw description also go to these LDS copies; quiet: no
  // output, statistic or description is written to global memory (another block of the request
  // writes them)
  RowStat* rowstat_local;
  DrawDesc* desc_local;
  int quiet;
};
hipError_t launch_decide_linear(const LinearArgs& a, psispec_dtype dtype, hipStream_t stream);
// Row statistics from many per-chunk pairs (the LM-head column tiles), one wave per row.
hipError_t launch_combine_rows(const RowSet& rs, const float2* part, int nchunk, float c,
                               RowStat* rowstat, hipStream_t stream);

// drafts.hip -- the drafting step
// Per drafted token: its row's statistics from the row-pass pairs and its draw description.
hipError_t launch_draft_rows(const RowSet& rs, int batch, int B, int first_from_target,
                             const float2* part, int nchunk, float c, RowStat* rowstat,
                             DrawDesc* desc, hipStream_t stream);
// One sub-chunk of a drafted token's row as summed by the bounded fp32 pass: m = max kept logit,
// s = sum of 2^((l - m) c) over the kept tokens (fp32 terms, fp64 sum), A = sum of |(l - m) c| times
// those terms (the argument-rounding part of the error bound).
struct BoundRec {
  double s;
  float m;
  float A;
};
struct DraftArgs {
  RowSet rs;
  int batch, B, V, nsub, first_from_target;
  float c;              // log2(e) / T in fp32
  double inv_T;         // 1 / T in fp64
  int use_topp;
  uint64_t seed;
  uint32_t step, request_base;
  const ToppStat* topp;
  RowStat* rowstat;     // written for the draws left to the exact pass
  DrawDesc* desc;       // idem
  BoundRec* rec;        // [batch*B][nsub]
  int32_t* list;        // [batch*B] the draws left to the exact pass, in no particular order
  int32_t* count;       // their number (zeroed by the bounded pass)
  int32_t* out_tokens;  // [batch*B]
  int32_t* status;      // [batch*B] or null
};
// The bounded fp32 pass and the select that settles every draw whose bound allows it.
hipError_t launch_draft_bounded(const DraftArgs& a, psispec_dtype dtype, hipStream_t stream);

// tree.hip
struct TreeArgs {
  RowSet rs;
  const int32_t* parent;
  const int32_t* node_tokens;
  int batch, N, V, max_depth, nchunk;
  float c;
  double inv_T;
  int use_topp;
  uint64_t seed;
  uint32_t step, request_base;
  const float2* part;
  const ToppStat* topp;
  RowStat* rowstat;
  DrawDesc* desc;
  int32_t* excl;      // [batch][N] excluded tokens of the stopping node
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  float* node_ratios;
};
hipError_t launch_decide_tree(const TreeArgs& a, psispec_dtype dtype, hipStream_t stream);
// Trees of at most 64 nodes: the walk and the draw pass in one launch (block (r, c) walks request r
// and draws chunk c of its stopping row; the chunk-0 block writes the outputs), then the select.
struct DrawArgs;
hipError_t launch_decide_tree_draw(const TreeArgs& ta, const DrawArgs& da, psispec_dtype dtype,
                                   hipStream_t stream);
struct TreeQArgs;
// Sampled candidates, trees of at most 64 nodes: the chains, then the walk and the draw pass in one
// launch, then the select.
hipError_t launch_decide_tree_sampled_draw(const TreeQArgs& ta, const DrawArgs& da,
                                           psispec_dtype dtype, hipStream_t stream);

// treeq.hip -- tree verify with candidates drawn from the draft (recursive rejection)
constexpr int kMaxSampledChildren = 8;  // children per node under the sampled rule
// Per node: exact normalisers of its p and q rows and the residual chain: after k rejections the
// residual is max(0, p' - c[k] q') / S[k], c[0] = 0, S[0] = 1, c[k] = c[k-1] + S[k-1] and
// S[k] = sum_x max(0, p'(x) - c[k] q'(x)).  A zero residual (S[k] = 0, unreachable in exact
// arithmetic) keeps the previous one: then c[j], S[j] = c[k-1], S[k-1] for every j >= k, and
// stuck = k (else kMaxSampledChildren + 1).
struct NodeChain {
  double Ep, Eq;
  double S[kMaxSampledChildren + 1];
  double c[kMaxSampledChildren + 1];
  int stuck;
};
// Level 0's split of one chunk's terms of S_1 = sum_x max(0, p'(x) - q'(x)) (see k_tree_chain)
constexpr int kBandSlots = 8;  // in-between tokens kept per chunk
struct BandPart {
  double pa, qa;            // sums of e_p and e_q over the chunk's tokens surely in the support
  int32_t n;                // in-between tokens seen (more than kBandSlots: the chunk is redone)
  int32_t x[kBandSlots];    // their indices (the first kBandSlots seen, in no fixed order)
};
struct TreeQArgs {
  RowSet rs;                // p rows [0, nP), q rows [nP, 2 nP), nP = batch (N+1)
  const int32_t* parent;
  const int32_t* node_tokens;
  int batch, N, V, max_depth;
  int nchunk_c, chunk_elems_c;  // chain passes: 4096-token chunks of a row
  double inv_T;
  int use_topp;
  uint64_t seed;
  uint32_t step, request_base;
  const RowStat* rowstat;   // every p and q row (combined)
  const ToppStat* topp;
  int max_children;         // most children per node: the caller's bound, else kMaxSampledChildren
  int32_t* nchild;          // [nP] children per node row (written by k_tree_children)
  double2* e_part;          // [nP][nchunk_c] (sum e_p, sum e_q) over the kept tokens
  double* s_part;           // [kMaxSampledChildren - 1][nP][nchunk_c] residual masses
  BandPart* band;           // [nP][nchunk_c] level 0's split of S_1
  int32_t* fb;              // [nP][nchunk_c] 1: the level-1 pass recomputes the chunk
  NodeChain* chain;         // [nP]
  DrawDesc* desc;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  float* node_ratios;
};
hipError_t launch_tree_children(const TreeQArgs& a, hipStream_t stream);
hipError_t launch_tree_chain_pass(const TreeQArgs& a, int level, psispec_dtype dtype,
                                  hipStream_t stream);
hipError_t launch_tree_resolve(const TreeQArgs& a, psispec_dtype dtype, hipStream_t stream);
hipError_t launch_decide_tree_sampled(const TreeQArgs& a, psispec_dtype dtype, hipStream_t stream);

// draw.hip -- the fp64 inverse-CDF draw shared by the verify entry points and the drafting step
struct DrawArgs {
  RowSet rs;
  int batch, V, nchunk_draw, chunk_elems_draw, nsub;
  double inv_T;
  int use_topp;
  uint64_t seed;
  uint32_t step, request_base;
  const RowStat* rowstat;
  const ToppStat* topp;
  const DrawDesc* desc;
  const int32_t* excl;
  int excl_stride;
  double2* esum;      // [batch][nchunk_draw] partial normalisers (E_p, E_q)
  double2* suba;      // [batch][nsub] per sub-chunk sums of e_p, e_q over positive tokens
  int32_t* subn;      // [batch][nsub] uncertain-sign tokens per sub-chunk
  int32_t* suboff;    // [batch][nsub] pool offset of the sub-chunk's uncertain tokens, -1 = none kept
  double2* upool;     // [batch][kUncPool] exact (e_p, e_q) of uncertain-sign tokens, chunk c
                      // of a draw in entries [c s, (c + 1) s), s = kUncPool / nchunk_draw
  double* subsum;     // [batch][nsub] sub-chunk masses (written by the select)
  int32_t* out_tokens;
  int32_t* status;
  // null: every draw r < batch.  Otherwise only the draws list[0 .. *count - 1] (draws already
  // settled elsewhere are skipped); a fixed grid then loops over them.
  const int32_t* list;
  const int32_t* count;
};
hipError_t launch_draw(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream);
// The linear verify's accept test and draw pass in one launch (block (r, c) decides request r and
// draws chunk c; the chunk-0 block writes the outputs), then the select.
hipError_t launch_decide_draw(const LinearArgs& la, const DrawArgs& da, psispec_dtype dtype,
                              hipStream_t stream);
// The select alone, and whether the pass may read the rows with 16-byte loads.
hipError_t launch_draw_select(const DrawArgs& a, psispec_dtype dtype, hipStream_t stream);
int draw_vec_ok(const DrawArgs& a, psispec_dtype dtype);

// linear.hip -- small linear verifies (no nucleus, one chunk per row) in one launch: one block per
// request stages its rows in LDS, computes their pairs, then runs the accept test, the draw pass
// and the select on LDS copies of the rows and records.  Used when a request's rows hold at most
// kSmallVerifyBytes.
constexpr size_t kSmallVerifyBytes = 32768;
hipError_t launch_verify_small(const LinearArgs& la, const DrawArgs& da, psispec_dtype dtype,
                               hipStream_t stream);

// kv.hip -- the KV commit after a verify
constexpr int kMaxKvBlock = 1024;  // block positions of a commit (B or N)
struct KvArgs {
  void* kv;               // line r at kv + r * line_stride bytes; position t at + t * row_bytes
  int64_t line_stride;    // bytes
  int64_t row_bytes;      // bytes per position (multiple of 16)
  int Lmax, blk;          // positions per line; block positions written by the verify forward
  const int32_t* keep;    // [batch][keep_stride] kept block positions, or null (the prefix)
  int keep_stride;
  const int32_t* n_keep;  // [batch]
  int32_t* len;           // [batch] in/out
  int32_t* status;        // [batch] or null
  int batch;
};
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t stream);

// lmhead.hip -- LM head on MFMA feeding the linear verify
struct LMHeadArgs {
  const uint16_t* h_ar;    // bf16 [nP][K]
  const uint16_t* h_dr;    // bf16 [nQ][K]
  const uint16_t* w;       // bf16 [K][N]
  const uint16_t* lora_a;  // bf16 [K][r] or null
  const uint16_t* lora_b;  // bf16 [r][N] or null
  float lora_scale;
  int nP, nQ, N, K, r;
  float c;                 // log2(e) / T for the epilogue's row pairs
};
int lmhead_tile_n();
int lmhead_kx(int r);  // extra contraction columns of the LoRA delta (2r rounded up to 32)
// bytes of the staged A operand for `rows` rows
size_t lmhead_ablk_bytes(int rows, int K, int r);
// Every row: per (row, column tile) online (max, sum exp) pairs [nP + nQ][ntiles], the logit at
// each row's draft token (gath [nP + nQ]; p row B of a request has none) and, when out_p is not
// null, the logits (p rows to out_p [nP][N], q rows to out_q [nQ][N]).
hipError_t launch_lmhead_main(const LMHeadArgs& a, uint16_t* ablk, const int32_t* draft, int B,
                              float2* part, float* gath, float* out_p, float* out_q,
                              hipStream_t stream);
// The stopping rows of every draw: row 2r = desc[r].prow, 2r + 1 = desc[r].qrow (if any), logits
// to out [2 batch][N]; desc2 / rowstat2 describe the draws over those rows.
hipError_t launch_lmhead_rows(const LMHeadArgs& a, uint16_t* ablk, int batch, const DrawDesc* desc,
                              const RowStat* rowstat, DrawDesc* desc2, RowStat* rowstat2,
                              float* out, hipStream_t stream);

// peak.hip -- measured ceilings (read bandwidth, bf16 MFMA issue rate)
hipError_t launch_peak_read(const void* buf, size_t bytes, uint32_t* out, int blocks,
                            hipStream_t stream);
hipError_t launch_peak_mfma(int64_t iters, float* out, int blocks, hipStream_t stream);

}  // namespace psispec
