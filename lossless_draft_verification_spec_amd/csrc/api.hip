// api.hip -- the C ABI of libpsispec: argument checks, workspace layout, launch order, timing.
//
// Launch order of a verify call (all on the caller's stream, no host synchronisation):
//   rowstats  -- one HBM pass over every p and q row: per (row, chunk) online (max, sum exp);
//   topp      -- (top_p < 1) nucleus threshold and mass per row;
//   decide    -- per request: ratios, accept bits, first rejection (linear) or the tree walk;
//   draw      -- fp64 normalisers, residual sub-chunk sums, inverse-CDF select of the final token.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

namespace psispec {
namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kDrawBlocks = 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int nchunk, chunk_elems;          // main pass split of a row
  int nchunk_draw, chunk_elems_draw, nsub;
  size_t off_part, off_rowstat, off_topp, off_desc, off_excl, off_esum, off_suba, off_subn,
      off_subsum, off_suboff, off_upool, off_rec, off_list, off_extra;
  size_t total;
};

// Row split of the HBM pass: chunks of about 128 KiB (a workgroup keeps 32 KiB of 16-byte loads in
// flight, about four rounds per chunk); calls with few rows get smaller chunks (down to 16 KiB) so
// that about 2048 workgroups (8 per CU) stream at once; chunk starts stay 16-byte aligned
// (multiples of 64 elements).
// rows: rows of the HBM pass; batch: draws (one per request, or one per drafted token); pool: the
// draws have a q row (residual draws keep a pool of uncertain-sign tokens).
// bounded: the drafting step's fp32 sub-chunk records and its list of unsettled draws.
// wide_draw: the draw pass may give each wave several sub-chunks (not for the sampled-tree chain
// passes, which share the draw chunking and keep one sub-chunk per wave, nor for the drafting
// step, whose exact pass runs over the few listed draws and wants many small tasks).
Plan make_plan(int64_t rows, int64_t batch, int V, size_t es, int excl_stride, int fixed_nchunk = 0,
               bool pool = true, bool bounded = false, bool wide_draw = true) {
  Plan pl{};
  const size_t row_bytes = (size_t)V * es;
  int nchunk = (int)((row_bytes + 131071) / 131072);
  if (rows > 0) {
    const int64_t want = (2048 + rows - 1) / rows;
    const int64_t most = std::max<int64_t>(1, (int64_t)(row_bytes / 16384));
    nchunk = (int)std::max<int64_t>(nchunk, std::min(want, most));
  }
  if (nchunk < 1) nchunk = 1;
  int ce = (V + nchunk - 1) / nchunk;
  ce = (ce + 63) / 64 * 64;
  pl.nchunk = (V + ce - 1) / ce;
  pl.chunk_elems = ce;
  if (fixed_nchunk > 0) {  // row pairs produced elsewhere: one per column tile of the LM-head
                           // epilogue, or one per row of the fused row pass and nucleus
    pl.nchunk = fixed_nchunk;
    pl.chunk_elems = 0;
  }
  pl.nsub = (V + kSub - 1) / kSub;
  // draw pass: 1024-token sub-chunks, spw per wave of a block.  spw grows (2, 4, 8) while the
  // draws still make about kDrawBlocks blocks (about one round of the draw pass's resident blocks),
  // which spreads each block's set-up (exp table, descriptor, normaliser ratio) over more tokens
  // and shortens the select's chunk sums without leaving CUs idle: spw = 2 at batch 64, 4 at 128,
  // 8 at 256.
  int spw = 1;
  while (wide_draw && spw < 8 &&
         batch * (int64_t)((pl.nsub + 2 * spw * (kThreads / 64) - 1) / (2 * spw * (kThreads / 64))) >=
             kDrawBlocks)
    spw *= 2;
  pl.chunk_elems_draw = spw * (kThreads / 64) * kSub;
  pl.nchunk_draw = (V + pl.chunk_elems_draw - 1) / pl.chunk_elems_draw;
  size_t off = 0;
  pl.off_part = off;
  off = align_up(off + sizeof(float2) * (size_t)rows * pl.nchunk);
  pl.off_rowstat = off;
  off = align_up(off + sizeof(RowStat) * (size_t)rows);
  pl.off_topp = off;
  off = align_up(off + sizeof(ToppStat) * (size_t)rows);
  pl.off_desc = off;
  off = align_up(off + sizeof(DrawDesc) * (size_t)batch);
  pl.off_excl = off;
  off = align_up(off + sizeof(int32_t) * (size_t)batch * (size_t)excl_stride);
  pl.off_esum = off;
  off = align_up(off + sizeof(double2) * (size_t)batch * pl.nchunk_draw);
  pl.off_suba = off;
  off = align_up(off + sizeof(double2) * (size_t)batch * pl.nsub);
  pl.off_subn = off;
  off = align_up(off + sizeof(int32_t) * (size_t)batch * pl.nsub);
  pl.off_subsum = off;
  off = align_up(off + sizeof(double) * (size_t)batch * pl.nsub);
  pl.off_suboff = off;
  off = align_up(off + sizeof(int32_t) * (size_t)batch * pl.nsub);
  pl.off_upool = off;
  off = align_up(off + (pool ? sizeof(double2) * (size_t)batch * kUncPool : 0));
  pl.off_rec = off;
  off = align_up(off + (bounded ? sizeof(BoundRec) * (size_t)batch * pl.nsub : 0));
  // the count, then (256 bytes on) the list of draws left to the exact pass
  pl.off_list = off;
  off = align_up(off + (bounded ? kAlign + sizeof(int32_t) * (size_t)batch : 0));
  pl.total = off;
  pl.off_extra = off;
  return pl;
}

size_t elem_size(psispec_dtype d) { return d == PSISPEC_BF16 ? 2 : 4; }

// The row pass and the nucleus share one read of every row (one workgroup per row, the row's pair
// as its one chunk) for bf16 rows under top-p, when the rows are many enough to fill the chip.
constexpr int64_t kFuseRows = 256;
bool fuse_topp(psispec_dtype dtype, int64_t rows, int V, double top_p) {
  return dtype == PSISPEC_BF16 && top_p < 1.0 && (1.0 - top_p) / (4.0 * (double)V) >= 1e-30 &&
         rows >= kFuseRows;
}

// Tree verify with sampled candidates: the rows of p and q, then per node row its children count,
// the chain passes' partial sums and its residual chain.
struct TreeQPlan {
  Plan pl;
  size_t off_nchild, off_epart, off_spart, off_band, off_fb, off_chain, total;
};

TreeQPlan make_treeq_plan(int batch, int N, int V, size_t es) {
  TreeQPlan tp{};
  const int64_t nP = (int64_t)batch * (N + 1);
  tp.pl = make_plan(2 * nP, batch, V, es, N, 0, true, false, false);
  const size_t nc = (size_t)tp.pl.nchunk_draw;
  size_t off = tp.pl.total;
  tp.off_nchild = off;
  off = align_up(off + sizeof(int32_t) * (size_t)nP);
  tp.off_epart = off;
  off = align_up(off + sizeof(double2) * (size_t)nP * nc);
  tp.off_spart = off;
  off = align_up(off + sizeof(double) * (size_t)(kMaxSampledChildren - 1) * (size_t)nP * nc);
  tp.off_band = off;
  off = align_up(off + sizeof(BandPart) * (size_t)nP * nc);
  tp.off_fb = off;
  off = align_up(off + sizeof(int32_t) * (size_t)nP * nc);
  tp.off_chain = off;
  off = align_up(off + sizeof(NodeChain) * (size_t)nP);
  tp.total = off;
  return tp;
}

// children_bound: the call accepts PSISPEC_MAX_CHILDREN (the tree verify)
bool sampling_ok(const psispec_sampling* s, bool children_bound = false) {
  if (!s) return false;
  if (!(s->temperature > 0.0) || !isfinite(s->temperature)) return false;
  if (!(s->top_p > 0.0) || !(s->top_p <= 1.0)) return false;
  if (s->reserved != 0) return false;
  const uint32_t known =
      PSISPEC_FIRST_FROM_TARGET | (children_bound ? PSISPEC_MAX_CHILDREN_MASK : 0u);
  if (s->flags & ~known) return false;
  if (((s->flags & PSISPEC_MAX_CHILDREN_MASK) >> PSISPEC_MAX_CHILDREN_SHIFT) >
      (uint32_t)kMaxSampledChildren)
    return false;
  return true;
}

template <typename P>
P* carve(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// ----------------------------------------------------------------------------------------------
// kernel timing
// ----------------------------------------------------------------------------------------------
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> pool;
  std::vector<std::string> names;
  std::vector<double> total_ms;
  std::vector<int> launches;
};

Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain(Timing& t) {
  for (auto& tl : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(tl.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, tl.start, tl.stop) != hipSuccess)
      ms = 0.f;
    size_t i = 0;
    for (; i < t.names.size(); ++i)
      if (t.names[i] == tl.name) break;
    if (i == t.names.size()) {
      t.names.push_back(tl.name);
      t.total_ms.push_back(0.0);
      t.launches.push_back(0);
    }
    t.total_ms[i] += ms;
    t.launches[i] += 1;
    t.pool.push_back(tl.start);
    t.pool.push_back(tl.stop);
  }
  t.pending.clear();
}

}  // namespace

bool timing_take(hipEvent_t* start, hipEvent_t* stop) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return false;
  *start = take_event(t);
  *stop = take_event(t);
  if (!*start || !*stop) {
    if (*start) t.pool.push_back(*start);
    if (*stop) t.pool.push_back(*stop);
    *start = *stop = nullptr;
    return false;
  }
  return true;
}

void timing_push(const char* name, hipEvent_t start, hipEvent_t stop) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.pending.push_back(TimedLaunch{name, start, stop});
  if (t.pending.size() > 4096) drain(t);
}

}  // namespace psispec

using namespace psispec;

namespace {

// Tree verify with candidates drawn from q (recursive rejection): row pass over the p and q rows,
// their statistics and nuclei, the chain passes (level 0: exact normalisers; level i: residual mass
// after i rejections), the walk, and the final draw of the stopping node's residual.
psispec_status verify_tree_sampled(const void* p_logits, const void* q_logits, psispec_dtype dtype,
                                   const int32_t* parent, const int32_t* node_tokens, int32_t batch,
                                   int32_t N, int32_t V, int32_t max_depth,
                                   const psispec_sampling* s, int32_t* accept_len,
                                   int32_t* accept_nodes, int32_t* out_tokens, float* node_ratios,
                                   int32_t* status, void* workspace, size_t workspace_bytes,
                                   void* stream_ptr) {
  const int64_t nP = (int64_t)batch * (N + 1);
  const TreeQPlan tp = make_treeq_plan(batch, N, V, elem_size(dtype));
  const Plan& pl = tp.pl;
  if (!workspace || workspace_bytes < tp.total || ((uintptr_t)workspace % kAlign) != 0)
    return PSISPEC_EWORKSPACE;
  if (2 * nP * pl.nchunk > INT32_MAX || nP * pl.nchunk_draw > INT32_MAX) return PSISPEC_EINVAL;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const double T = s->temperature;
  const float c = (float)(1.4426950408889634074 / T);
  const bool use_topp = s->top_p < 1.0;
  RowSet rs{p_logits, q_logits, nP, nP, V, N + 1, 0, V};
  float2* part = carve<float2>(workspace, pl.off_part);
  RowStat* rowstat = carve<RowStat>(workspace, pl.off_rowstat);
  ToppStat* topp = carve<ToppStat>(workspace, pl.off_topp);
  DrawDesc* desc = carve<DrawDesc>(workspace, pl.off_desc);
  if (launch_rowstats(rs, dtype, pl.nchunk, pl.chunk_elems, c, part, stream) != hipSuccess)
    return PSISPEC_EHIP;
  if (launch_combine_rows(rs, part, pl.nchunk, c, rowstat, stream) != hipSuccess)
    return PSISPEC_EHIP;
  if (use_topp && launch_topp(rs, dtype, pl.nchunk, c, s->top_p, part, topp, stream, rowstat) !=
                      hipSuccess)
    return PSISPEC_EHIP;

  TreeQArgs ta{};
  ta.rs = rs;
  ta.parent = parent;
  ta.node_tokens = node_tokens;
  ta.batch = batch;
  ta.N = N;
  ta.V = V;
  ta.max_depth = max_depth;
  ta.nchunk_c = pl.nchunk_draw;
  ta.chunk_elems_c = pl.chunk_elems_draw;
  ta.inv_T = 1.0 / T;
  ta.use_topp = use_topp;
  ta.seed = s->seed;
  ta.step = s->step;
  ta.request_base = s->request_base;
  ta.rowstat = rowstat;
  ta.topp = topp;
  ta.nchild = carve<int32_t>(workspace, tp.off_nchild);
  ta.e_part = carve<double2>(workspace, tp.off_epart);
  ta.s_part = carve<double>(workspace, tp.off_spart);
  ta.band = carve<BandPart>(workspace, tp.off_band);
  ta.fb = carve<int32_t>(workspace, tp.off_fb);
  ta.chain = carve<NodeChain>(workspace, tp.off_chain);
  ta.desc = desc;
  ta.accept_len = accept_len;
  ta.accept_nodes = accept_nodes;
  ta.out_tokens = out_tokens;
  ta.node_ratios = node_ratios;
  // the caller's bound on children per node, if given: the levels past it would find no work
  const int bound = (int)((s->flags & PSISPEC_MAX_CHILDREN_MASK) >> PSISPEC_MAX_CHILDREN_SHIFT);
  ta.max_children = bound > 0 ? bound : kMaxSampledChildren;
  if (launch_tree_children(ta, stream) != hipSuccess) return PSISPEC_EHIP;
  for (int level = 0; level < ta.max_children; ++level) {
    if (level == 1 && launch_tree_resolve(ta, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
    if (launch_tree_chain_pass(ta, level, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  }

  DrawArgs da{};
  da.rs = rs;
  da.batch = batch;
  da.V = V;
  da.nchunk_draw = pl.nchunk_draw;
  da.chunk_elems_draw = pl.chunk_elems_draw;
  da.nsub = pl.nsub;
  da.inv_T = 1.0 / T;
  da.use_topp = use_topp;
  da.seed = s->seed;
  da.step = s->step;
  da.request_base = s->request_base;
  da.rowstat = rowstat;
  da.topp = topp;
  da.desc = desc;
  da.excl = nullptr;
  da.excl_stride = 0;
  da.esum = carve<double2>(workspace, pl.off_esum);
  da.subsum = carve<double>(workspace, pl.off_subsum);
  da.suba = carve<double2>(workspace, pl.off_suba);
  da.subn = carve<int32_t>(workspace, pl.off_subn);
  da.suboff = carve<int32_t>(workspace, pl.off_suboff);
  da.upool = carve<double2>(workspace, pl.off_upool);
  da.out_tokens = out_tokens;
  da.status = status;
  if (N <= 64)  // the walk runs in each draw block: one launch fewer
    return launch_decide_tree_sampled_draw(ta, da, dtype, stream) == hipSuccess ? PSISPEC_OK
                                                                               : PSISPEC_EHIP;
  if (launch_decide_tree_sampled(ta, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  if (launch_draw(da, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

}  // namespace

namespace {

// Scratch of psispec_verify_linear_noalloc: a fixed array in device memory (one copy per GPU
// the library runs on, held until the process ends).  Host code uses only the device address
// that hipGetSymbolAddress returns for it, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  static std::mutex mu;
  static std::vector<void*> per_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    per_device[dev] = ptr;
  }
  return per_device[dev];
}

}  // namespace

extern "C" {

const char* psispec_strerror(psispec_status code) {
  switch (code) {
    case PSISPEC_OK: return "ok";
    case PSISPEC_EINVAL: return "invalid argument (pointer, size or sampling parameter)";
    case PSISPEC_EDTYPE: return "unsupported element type";
    case PSISPEC_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case PSISPEC_EHIP: return "HIP launch or runtime error";
    case PSISPEC_EUNSUPPORTED: return "mode not implemented";
    case PSISPEC_ESCRATCH:
      return "sizes need more scratch than the no-allocation entry point's fixed array holds";
  }
  return "unknown status";
}

psispec_status psispec_peak_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                                 void* stream) {
  if (!buf || !out || blocks < 1 || bytes < 16 || ((uintptr_t)buf % 16) != 0) return PSISPEC_EINVAL;
  if (launch_peak_read(buf, bytes, out, blocks, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PSISPEC_EHIP;
  return PSISPEC_OK;
}

psispec_status psispec_peak_mfma(int64_t iters, float* out, int32_t blocks, void* stream) {
  if (!out || blocks < 1 || iters < 1) return PSISPEC_EINVAL;
  if (launch_peak_mfma(iters, out, blocks, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PSISPEC_EHIP;
  return PSISPEC_OK;
}

psispec_status psispec_timing_enable(int32_t on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  drain(t);
  t.on = on != 0;
  t.names.clear();
  t.total_ms.clear();
  t.launches.clear();
  return PSISPEC_OK;
}

int32_t psispec_timing_read(char* names, float* total_ms, int32_t* launches, int32_t max_kernels) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  drain(t);
  int32_t n = 0;
  for (size_t i = 0; i < t.names.size() && n < max_kernels; ++i, ++n) {
    if (names) {
      strncpy(names + 64 * n, t.names[i].c_str(), 63);
      names[64 * n + 63] = '\0';
    }
    if (total_ms) total_ms[n] = (float)t.total_ms[i];
    if (launches) launches[n] = t.launches[i];
  }
  return n;
}

size_t psispec_verify_linear_workspace(int32_t batch, int32_t B, int32_t V, psispec_dtype dtype) {
  if (batch < 0 || B < 1 || B > 64 || V < 1) return 0;
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return 0;
  const int64_t rows = (int64_t)batch * (2 * B + 1);
  return make_plan(rows, batch, V, elem_size(dtype), 0).total + kAlign;
}

size_t psispec_verify_tree_workspace(int32_t batch, int32_t N, int32_t V, psispec_dtype dtype) {
  if (batch < 0 || N < 1 || N > 1024 || V < 1) return 0;
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return 0;
  const int64_t rows = (int64_t)batch * (N + 1);
  // sized for both rules (candidates chosen, or drawn from q)
  const size_t det = make_plan(rows, batch, V, elem_size(dtype), N).total;
  const size_t smp = make_treeq_plan(batch, N, V, elem_size(dtype)).total;
  return (det > smp ? det : smp) + kAlign;
}

psispec_status psispec_verify_linear(const void* p_logits, const void* q_logits, psispec_dtype dtype,
                                     const int32_t* draft_tokens, int32_t batch, int32_t B,
                                     int32_t V, const psispec_sampling* s, int32_t* accept_len,
                                     int32_t* out_tokens, float* ratios, uint64_t* accept_mask,
                                     int32_t* status, void* workspace, size_t workspace_bytes,
                                     void* stream_ptr) {
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return PSISPEC_EDTYPE;
  if (batch < 0 || B < 1 || B > 64 || V < 1) return PSISPEC_EINVAL;
  if (!sampling_ok(s)) return PSISPEC_EINVAL;
  if (batch == 0) return PSISPEC_OK;
  if (!p_logits || !q_logits || !draft_tokens || !accept_len || !out_tokens) return PSISPEC_EINVAL;
  const int64_t nP = (int64_t)batch * (B + 1), nQ = (int64_t)batch * B;
  const bool fuse = fuse_topp(dtype, nP + nQ, V, s->top_p);
  const Plan pl = make_plan(nP + nQ, batch, V, elem_size(dtype), 0, fuse ? 1 : 0);
  if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace % kAlign) != 0)
    return PSISPEC_EWORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const double T = s->temperature;
  const float c = (float)(1.4426950408889634074 / T);
  const bool use_topp = s->top_p < 1.0;

  RowSet rs{p_logits, q_logits, nP, nQ, V, B, (s->flags & PSISPEC_FIRST_FROM_TARGET) ? 1 : 0, V};
  float2* part = carve<float2>(workspace, pl.off_part);
  RowStat* rowstat = carve<RowStat>(workspace, pl.off_rowstat);
  ToppStat* topp = carve<ToppStat>(workspace, pl.off_topp);
  DrawDesc* desc = carve<DrawDesc>(workspace, pl.off_desc);

  LinearArgs la{};
  la.rs = rs;
  la.draft = draft_tokens;
  la.batch = batch;
  la.B = B;
  la.V = V;
  la.nchunk = pl.nchunk;
  la.c = c;
  la.inv_T = 1.0 / T;
  la.use_topp = use_topp;
  la.seed = s->seed;
  la.step = s->step;
  la.request_base = s->request_base;
  la.flags = s->flags;
  la.part = part;
  la.topp = topp;
  la.rowstat = rowstat;
  la.desc = desc;
  la.accept_len = accept_len;
  la.out_tokens = out_tokens;
  la.ratios = ratios;
  la.accept_mask = accept_mask;

  DrawArgs da{};
  da.rs = rs;
  da.batch = batch;
  da.V = V;
  da.nchunk_draw = pl.nchunk_draw;
  da.chunk_elems_draw = pl.chunk_elems_draw;
  da.nsub = pl.nsub;
  da.inv_T = 1.0 / T;
  da.use_topp = use_topp;
  da.seed = s->seed;
  da.step = s->step;
  da.request_base = s->request_base;
  da.rowstat = rowstat;
  da.topp = topp;
  da.desc = desc;
  da.excl = nullptr;
  da.excl_stride = 0;
  da.esum = carve<double2>(workspace, pl.off_esum);
  da.subsum = carve<double>(workspace, pl.off_subsum);
  da.suba = carve<double2>(workspace, pl.off_suba);
  da.subn = carve<int32_t>(workspace, pl.off_subn);
  da.suboff = carve<int32_t>(workspace, pl.off_suboff);
  da.upool = carve<double2>(workspace, pl.off_upool);
  da.out_tokens = out_tokens;
  da.status = status;

  // a few kilobytes of logits per request: one launch does the whole verify
  if (!use_topp && pl.nchunk == 1 &&
      (size_t)(2 * B + 1) * (size_t)V * elem_size(dtype) <= kSmallVerifyBytes)
    return launch_verify_small(la, da, dtype, stream) == hipSuccess
               ? PSISPEC_OK
               : PSISPEC_EHIP;

  if (fuse) {
    if (launch_rowstats_topp(rs, c, s->top_p, part, topp, stream) != hipSuccess) return PSISPEC_EHIP;
  } else {
    if (launch_rowstats(rs, dtype, pl.nchunk, pl.chunk_elems, c, part, stream) != hipSuccess)
      return PSISPEC_EHIP;
    if (use_topp && launch_topp(rs, dtype, pl.nchunk, c, s->top_p, part, topp, stream) !=
                        hipSuccess)
      return PSISPEC_EHIP;
  }
  if (launch_decide_draw(la, da, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

psispec_status psispec_verify_linear_noalloc(const void* p_logits, const void* q_logits,
                                             psispec_dtype dtype, const int32_t* draft_tokens,
                                             int32_t batch, int32_t B, int32_t V,
                                             const psispec_sampling* s, int32_t* accept_len,
                                             int32_t* out_tokens, float* ratios,
                                             uint64_t* accept_mask, int32_t* status,
                                             void* stream) {
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return PSISPEC_EDTYPE;
  if (batch < 0 || B < 1 || B > 64 || V < 1) return PSISPEC_EINVAL;
  if (batch == 0) return sampling_ok(s) ? PSISPEC_OK : PSISPEC_EINVAL;
  const size_t need = psispec_verify_linear_workspace(batch, B, V, dtype);
  if (need == 0) return PSISPEC_EINVAL;
  if (need > kNoAllocScratchBytes) return PSISPEC_ESCRATCH;
  void* ws = noalloc_scratch();
  if (!ws) return PSISPEC_EHIP;
  return psispec_verify_linear(p_logits, q_logits, dtype, draft_tokens, batch, B, V, s,
                               accept_len, out_tokens, ratios, accept_mask, status, ws,
                               kNoAllocScratchBytes, stream);
}

psispec_status psispec_verify_tree(const void* p_logits, const void* q_logits, psispec_dtype dtype,
                                   const int32_t* parent, const int32_t* node_tokens, int32_t batch,
                                   int32_t N, int32_t V, int32_t max_depth,
                                   const psispec_sampling* s, int32_t* accept_len,
                                   int32_t* accept_nodes, int32_t* out_tokens, float* node_ratios,
                                   int32_t* status, void* workspace, size_t workspace_bytes,
                                   void* stream_ptr) {
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return PSISPEC_EDTYPE;
  if (batch < 0 || N < 1 || N > 1024 || V < 1 || max_depth < 1 || max_depth > 64)
    return PSISPEC_EINVAL;
  if (!sampling_ok(s, true) || (s->flags & PSISPEC_FIRST_FROM_TARGET)) return PSISPEC_EINVAL;
  if (!q_logits && (s->flags & PSISPEC_MAX_CHILDREN_MASK)) return PSISPEC_EINVAL;
  if (batch == 0) return PSISPEC_OK;
  if (!p_logits || !parent || !node_tokens || !accept_len || !accept_nodes || !out_tokens)
    return PSISPEC_EINVAL;
  if (q_logits)
    return verify_tree_sampled(p_logits, q_logits, dtype, parent, node_tokens, batch, N, V,
                               max_depth, s, accept_len, accept_nodes, out_tokens, node_ratios,
                               status, workspace, workspace_bytes, stream_ptr);
  const int64_t nP = (int64_t)batch * (N + 1);
  const Plan pl = make_plan(nP, batch, V, elem_size(dtype), N);
  if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace % kAlign) != 0)
    return PSISPEC_EWORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const double T = s->temperature;
  const float c = (float)(1.4426950408889634074 / T);
  const bool use_topp = s->top_p < 1.0;

  RowSet rs{p_logits, nullptr, nP, 0, V, 1, 0, V};
  float2* part = carve<float2>(workspace, pl.off_part);
  RowStat* rowstat = carve<RowStat>(workspace, pl.off_rowstat);
  ToppStat* topp = carve<ToppStat>(workspace, pl.off_topp);
  DrawDesc* desc = carve<DrawDesc>(workspace, pl.off_desc);
  int32_t* excl = carve<int32_t>(workspace, pl.off_excl);

  if (launch_rowstats(rs, dtype, pl.nchunk, pl.chunk_elems, c, part, stream) != hipSuccess)
    return PSISPEC_EHIP;
  if (use_topp && launch_topp(rs, dtype, pl.nchunk, c, s->top_p, part, topp, stream) != hipSuccess)
    return PSISPEC_EHIP;

  TreeArgs ta{};
  ta.rs = rs;
  ta.parent = parent;
  ta.node_tokens = node_tokens;
  ta.batch = batch;
  ta.N = N;
  ta.V = V;
  ta.max_depth = max_depth;
  ta.nchunk = pl.nchunk;
  ta.c = c;
  ta.inv_T = 1.0 / T;
  ta.use_topp = use_topp;
  ta.seed = s->seed;
  ta.step = s->step;
  ta.request_base = s->request_base;
  ta.part = part;
  ta.topp = topp;
  ta.rowstat = rowstat;
  ta.desc = desc;
  ta.excl = excl;
  ta.accept_len = accept_len;
  ta.accept_nodes = accept_nodes;
  ta.out_tokens = out_tokens;
  ta.node_ratios = node_ratios;

  DrawArgs da{};
  da.rs = rs;
  da.batch = batch;
  da.V = V;
  da.nchunk_draw = pl.nchunk_draw;
  da.chunk_elems_draw = pl.chunk_elems_draw;
  da.nsub = pl.nsub;
  da.inv_T = 1.0 / T;
  da.use_topp = use_topp;
  da.seed = s->seed;
  da.step = s->step;
  da.request_base = s->request_base;
  da.rowstat = rowstat;
  da.topp = topp;
  da.desc = desc;
  da.excl = excl;
  da.excl_stride = N;
  da.esum = carve<double2>(workspace, pl.off_esum);
  da.subsum = carve<double>(workspace, pl.off_subsum);
  da.suba = carve<double2>(workspace, pl.off_suba);
  da.subn = carve<int32_t>(workspace, pl.off_subn);
  da.suboff = carve<int32_t>(workspace, pl.off_suboff);
  da.upool = carve<double2>(workspace, pl.off_upool);
  da.out_tokens = out_tokens;
  da.status = status;
  if (N <= 64)  // the walk runs in each draw block: one launch fewer
    return launch_decide_tree_draw(ta, da, dtype, stream) == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
  if (launch_decide_tree(ta, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  if (launch_draw(da, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

// Drafting step: rows of the HBM pass are the AR rows (one per request, Uno layout) and the q rows;
// the plan is sized for both so that the workspace query needs no flags.
size_t psispec_sample_drafts_workspace(int32_t batch, int32_t B, int32_t V, psispec_dtype dtype) {
  if (batch < 0 || B < 1 || B > 64 || V < 1) return 0;
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return 0;
  const int64_t rows = (int64_t)batch * (B + 1), jobs = (int64_t)batch * B;
  return make_plan(rows, jobs, V, elem_size(dtype), 0, 0, false, true, false).total + kAlign;
}

psispec_status psispec_sample_drafts(const void* ar_logits, int64_t ar_stride,
                                     const void* q_logits, psispec_dtype dtype, int32_t batch,
                                     int32_t B, int32_t V, const psispec_sampling* s,
                                     int32_t* draft_tokens, int32_t* status, void* workspace,
                                     size_t workspace_bytes, void* stream_ptr) {
  if (dtype != PSISPEC_F32 && dtype != PSISPEC_BF16) return PSISPEC_EDTYPE;
  if (batch < 0 || B < 1 || B > 64 || V < 1) return PSISPEC_EINVAL;
  if (!sampling_ok(s)) return PSISPEC_EINVAL;
  if (batch == 0) return PSISPEC_OK;
  const bool fft = (s->flags & PSISPEC_FIRST_FROM_TARGET) != 0;
  if (!draft_tokens) return PSISPEC_EINVAL;
  if (fft && (!ar_logits || ar_stride < V)) return PSISPEC_EINVAL;
  if (!q_logits && !(fft && B == 1)) return PSISPEC_EINVAL;
  const int64_t rows_plan = (int64_t)batch * (B + 1), jobs = (int64_t)batch * B;
  const int64_t rows_pass = (fft ? batch : 0) + (q_logits ? jobs : 0);
  const bool fuse = fuse_topp(dtype, rows_pass, V, s->top_p);
  const Plan pl =
      make_plan(rows_plan, jobs, V, elem_size(dtype), 0, fuse ? 1 : 0, false, true, false);
  if (rows_plan * pl.nchunk > INT32_MAX || jobs * pl.nchunk_draw > INT32_MAX) return PSISPEC_EINVAL;
  if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace % kAlign) != 0)
    return PSISPEC_EWORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const double T = s->temperature;
  const float c = (float)(1.4426950408889634074 / T);
  const bool use_topp = s->top_p < 1.0;

  // p rows: the AR row of each request (Uno layout only); q rows: [batch][B], position 0 skipped
  // in the Uno layout
  const int64_t nP = fft ? batch : 0, nQ = q_logits ? jobs : 0;
  RowSet rs{fft ? ar_logits : nullptr, q_logits, nP, nQ, V, B, fft ? 1 : 0,
            fft ? ar_stride : (int64_t)V};
  float2* part = carve<float2>(workspace, pl.off_part);
  RowStat* rowstat = carve<RowStat>(workspace, pl.off_rowstat);
  ToppStat* topp = carve<ToppStat>(workspace, pl.off_topp);
  DrawDesc* desc = carve<DrawDesc>(workspace, pl.off_desc);

  // The bounded fp32 pass settles most draws (sub-chunk masses in LDS: V <= 2M tokens); the exact
  // fp64 draw takes the rest.  The row statistics are needed first only for the nucleus, or when
  // every draw takes the exact path.
  const bool bounded = pl.nsub <= kMassLds;
  int32_t* count = carve<int32_t>(workspace, pl.off_list);
  int32_t* list = carve<int32_t>(workspace, pl.off_list + kAlign);
  if (fuse) {  // the nucleus comes with the pairs
    if (launch_rowstats_topp(rs, c, s->top_p, part, topp, stream) != hipSuccess) return PSISPEC_EHIP;
    if (launch_draft_rows(rs, batch, B, fft ? 1 : 0, part, pl.nchunk, c, rowstat, desc, stream) !=
        hipSuccess)
      return PSISPEC_EHIP;
  } else if (use_topp || !bounded) {
    if (launch_rowstats(rs, dtype, pl.nchunk, pl.chunk_elems, c, part, stream) != hipSuccess)
      return PSISPEC_EHIP;
    if (launch_draft_rows(rs, batch, B, fft ? 1 : 0, part, pl.nchunk, c, rowstat, desc, stream) !=
        hipSuccess)
      return PSISPEC_EHIP;
    if (use_topp && launch_topp(rs, dtype, pl.nchunk, c, s->top_p, part, topp, stream, rowstat) !=
                        hipSuccess)
      return PSISPEC_EHIP;
  }
  if (bounded) {
    DraftArgs fa{};
    fa.rs = rs;
    fa.batch = batch;
    fa.B = B;
    fa.V = V;
    fa.nsub = pl.nsub;
    fa.first_from_target = fft ? 1 : 0;
    fa.c = c;
    fa.inv_T = 1.0 / T;
    fa.use_topp = use_topp;
    fa.seed = s->seed;
    fa.step = s->step;
    fa.request_base = s->request_base;
    fa.topp = topp;
    fa.rowstat = rowstat;
    fa.desc = desc;
    fa.rec = carve<BoundRec>(workspace, pl.off_rec);
    fa.list = list;
    fa.count = count;
    fa.out_tokens = draft_tokens;
    fa.status = status;
    if (launch_draft_bounded(fa, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  }

  DrawArgs da{};
  da.rs = rs;
  da.batch = (int)jobs;
  da.V = V;
  da.nchunk_draw = pl.nchunk_draw;
  da.chunk_elems_draw = pl.chunk_elems_draw;
  da.nsub = pl.nsub;
  da.inv_T = 1.0 / T;
  da.use_topp = use_topp;
  da.seed = s->seed;
  da.step = s->step;
  da.request_base = s->request_base;
  da.rowstat = rowstat;
  da.topp = topp;
  da.desc = desc;
  da.excl = nullptr;
  da.excl_stride = 0;
  da.esum = carve<double2>(workspace, pl.off_esum);
  da.subsum = carve<double>(workspace, pl.off_subsum);
  da.suba = carve<double2>(workspace, pl.off_suba);
  da.subn = carve<int32_t>(workspace, pl.off_subn);
  da.suboff = carve<int32_t>(workspace, pl.off_suboff);
  da.upool = nullptr;  // draws without a q row keep no pool
  da.out_tokens = draft_tokens;
  da.status = status;
  da.list = bounded ? list : nullptr;  // the draws the bounded pass could not settle
  da.count = bounded ? count : nullptr;
  if (launch_draw(da, dtype, stream) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

psispec_status psispec_kv_commit(void* kv, int64_t line_stride, int64_t row_bytes, int32_t Lmax,
                                 int32_t blk, const int32_t* keep, int32_t keep_stride,
                                 const int32_t* n_keep, int32_t* len, int32_t* status,
                                 int32_t batch, void* stream_ptr) {
  if (batch < 0 || Lmax < 1 || blk < 1 || blk > Lmax || blk > kMaxKvBlock) return PSISPEC_EINVAL;
  if (row_bytes < 16 || row_bytes % 16 || line_stride % 16 || line_stride < (int64_t)Lmax * row_bytes)
    return PSISPEC_EINVAL;
  if (keep && keep_stride < 1) return PSISPEC_EINVAL;
  if (batch == 0) return PSISPEC_OK;
  if (!kv || !n_keep || !len || ((uintptr_t)kv % 16) != 0) return PSISPEC_EINVAL;
  if ((int64_t)batch * ((row_bytes + 4095) / 4096) > INT32_MAX) return PSISPEC_EINVAL;  // grid size
  KvArgs a{};
  a.kv = kv;
  a.line_stride = line_stride;
  a.row_bytes = row_bytes;
  a.Lmax = Lmax;
  a.blk = blk;
  a.keep = keep;
  a.keep_stride = keep_stride;
  a.n_keep = n_keep;
  a.len = len;
  a.status = status;
  a.batch = batch;
  if (launch_kv_commit(a, static_cast<hipStream_t>(stream_ptr)) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// LM head + linear verify
// ---------------------------------------------------------------------------------------------
namespace {

// Workspace of the LM-head verify: the linear verify's plan over the M = batch (2B+1) rows (one
// row pair per column tile), the logit at each row's draft token, the staged A operand (reused
// by the stopping-row pass once the main pass is done), and for the final draw the recomputed
// stopping rows with their descriptors and statistics.
struct LMPlan {
  Plan pl;
  size_t off_gath, off_ablk, off_desc2, off_rowstat2, off_rows, total;
  int ntiles;
};

LMPlan make_lm_plan(int batch, int B, int H, int V, int r) {
  LMPlan lp{};
  const int nP = batch * (B + 1), nQ = batch * B, M = nP + nQ;
  lp.ntiles = (V + lmhead_tile_n() - 1) / lmhead_tile_n();
  lp.pl = make_plan((int64_t)M, batch, V, 4, 0, lp.ntiles);
  size_t off = lp.pl.total;
  lp.off_gath = off;
  off = align_up(off + sizeof(float) * (size_t)M);
  lp.off_ablk = off;
  const size_t a_main = lmhead_ablk_bytes(M, H, r), a_rows = lmhead_ablk_bytes(2 * batch, H, r);
  off = align_up(off + (a_main > a_rows ? a_main : a_rows));
  lp.off_desc2 = off;
  off = align_up(off + sizeof(DrawDesc) * (size_t)batch);
  lp.off_rowstat2 = off;
  off = align_up(off + sizeof(RowStat) * (size_t)(2 * batch));
  lp.off_rows = off;
  off = align_up(off + sizeof(float) * (size_t)(2 * batch) * (size_t)V);
  lp.total = off + kAlign;
  return lp;
}

bool lm_shape_ok(int32_t batch, int32_t B, int32_t H, int32_t V, int32_t r) {
  if (batch < 0 || B < 1 || B > 64 || V < 8 || V % 8 || H < 64 || H % 64 || H > (1 << 20) ||
      r < 0 || r > 64)
    return false;
  // 32-bit offsets: rows of the staged operand, a K step of W, the per-call row count
  const int64_t M = (int64_t)batch * (2 * B + 1);
  if (M > (1 << 24) || (int64_t)V * 64 > INT32_MAX || M * (H + 128) * 2 > INT32_MAX) return false;
  return true;
}

}  // namespace

extern "C" {

size_t psispec_lmhead_verify_workspace(int32_t batch, int32_t B, int32_t H, int32_t V, int32_t r) {
  if (!lm_shape_ok(batch, B, H, V, r)) return 0;
  return make_lm_plan(batch, B, H, V, r).total;
}

psispec_status psispec_lmhead_verify(const void* h_ar, const void* h_draft, const void* W,
                                     const void* lora_A, const void* lora_B, float lora_scale,
                                     int32_t batch, int32_t B, int32_t H, int32_t V, int32_t r,
                                     const int32_t* draft_tokens, const psispec_sampling* s,
                                     int32_t* accept_len, int32_t* out_tokens, float* ratios,
                                     uint64_t* accept_mask, int32_t* status, float* p_logits_dbg,
                                     float* q_logits_dbg, void* workspace, size_t workspace_bytes,
                                     void* stream_ptr) {
  if (!lm_shape_ok(batch, B, H, V, r)) return PSISPEC_EINVAL;
  if (!sampling_ok(s) || !isfinite(lora_scale)) return PSISPEC_EINVAL;
  if (batch == 0) return PSISPEC_OK;
  if (!h_ar || !h_draft || !W || !draft_tokens || !accept_len || !out_tokens) return PSISPEC_EINVAL;
  if (r > 0 && (!lora_A || !lora_B)) return PSISPEC_EINVAL;
  if ((p_logits_dbg == nullptr) != (q_logits_dbg == nullptr)) return PSISPEC_EINVAL;
  if (((uintptr_t)h_ar | (uintptr_t)h_draft | (uintptr_t)W | (uintptr_t)lora_B |
       (uintptr_t)p_logits_dbg | (uintptr_t)q_logits_dbg) % 16)
    return PSISPEC_EINVAL;
  const bool use_topp = s->top_p < 1.0;
  const bool materialise = p_logits_dbg != nullptr;
  if (use_topp && !materialise) return PSISPEC_EUNSUPPORTED;
  const LMPlan lp = make_lm_plan(batch, B, H, V, r);
  if (!workspace || workspace_bytes < lp.total || ((uintptr_t)workspace % kAlign) != 0)
    return PSISPEC_EWORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const double T = s->temperature;
  const float c = (float)(1.4426950408889634074 / T);
  const int nP = batch * (B + 1), nQ = batch * B;
  const Plan& pl = lp.pl;
  float2* part = carve<float2>(workspace, pl.off_part);
  float* gath = carve<float>(workspace, lp.off_gath);
  uint16_t* ablk = carve<uint16_t>(workspace, lp.off_ablk);

  LMHeadArgs ha{};
  ha.h_ar = static_cast<const uint16_t*>(h_ar);
  ha.h_dr = static_cast<const uint16_t*>(h_draft);
  ha.w = static_cast<const uint16_t*>(W);
  ha.lora_a = static_cast<const uint16_t*>(lora_A);
  ha.lora_b = static_cast<const uint16_t*>(lora_B);
  ha.lora_scale = lora_scale;
  ha.nP = nP;
  ha.nQ = nQ;
  ha.N = V;
  ha.K = H;
  ha.r = r;
  ha.c = c;
  if (launch_lmhead_main(ha, ablk, draft_tokens, B, part, gath, p_logits_dbg, q_logits_dbg,
                         stream) != hipSuccess)
    return PSISPEC_EHIP;

  // the accept test on the epilogue's row pairs (one per column tile) and gathered logits; the rows
  // themselves are read only when the caller materialised them (the nucleus, the final draw)
  RowSet rs{p_logits_dbg, q_logits_dbg, nP, nQ, V, B,
            (s->flags & PSISPEC_FIRST_FROM_TARGET) ? 1 : 0, V};
  RowStat* rowstat = carve<RowStat>(workspace, pl.off_rowstat);
  ToppStat* topp = carve<ToppStat>(workspace, pl.off_topp);
  DrawDesc* desc = carve<DrawDesc>(workspace, pl.off_desc);
  if (launch_combine_rows(rs, part, pl.nchunk, c, rowstat, stream) != hipSuccess)
    return PSISPEC_EHIP;
  if (use_topp && launch_topp(rs, PSISPEC_F32, pl.nchunk, c, s->top_p, part, topp, stream,
                              rowstat) != hipSuccess)
    return PSISPEC_EHIP;
  LinearArgs la{};
  la.rs = rs;
  la.draft = draft_tokens;
  la.batch = batch;
  la.B = B;
  la.V = V;
  la.nchunk = pl.nchunk;
  la.c = c;
  la.inv_T = 1.0 / T;
  la.use_topp = use_topp;
  la.seed = s->seed;
  la.step = s->step;
  la.request_base = s->request_base;
  la.flags = s->flags;
  la.part = part;
  la.topp = topp;
  la.rowstat = rowstat;
  la.rowstat_ready = 1;
  la.gath = gath;
  la.desc = desc;
  la.accept_len = accept_len;
  la.out_tokens = out_tokens;
  la.ratios = ratios;
  la.accept_mask = accept_mask;
  if (launch_decide_linear(la, PSISPEC_F32, stream) != hipSuccess) return PSISPEC_EHIP;

  DrawArgs da{};
  da.rs = rs;
  da.batch = batch;
  da.V = V;
  da.nchunk_draw = pl.nchunk_draw;
  da.chunk_elems_draw = pl.chunk_elems_draw;
  da.nsub = pl.nsub;
  da.inv_T = 1.0 / T;
  da.use_topp = use_topp;
  da.seed = s->seed;
  da.step = s->step;
  da.request_base = s->request_base;
  da.rowstat = rowstat;
  da.topp = topp;
  da.desc = desc;
  if (!materialise) {
    // recompute the stopping rows: p_k and q_k of request r become rows 2r and 2r + 1
    float* rows = carve<float>(workspace, lp.off_rows);
    DrawDesc* desc2 = carve<DrawDesc>(workspace, lp.off_desc2);
    RowStat* rowstat2 = carve<RowStat>(workspace, lp.off_rowstat2);
    if (launch_lmhead_rows(ha, ablk, batch, desc, rowstat, desc2, rowstat2, rows, stream) !=
        hipSuccess)
      return PSISPEC_EHIP;
    da.rs = RowSet{rows, rows, 2 * (int64_t)batch, 0, V, 1, 0, V};
    da.rowstat = rowstat2;
    da.desc = desc2;
  }
  da.excl = nullptr;
  da.excl_stride = 0;
  da.esum = carve<double2>(workspace, pl.off_esum);
  da.suba = carve<double2>(workspace, pl.off_suba);
  da.subn = carve<int32_t>(workspace, pl.off_subn);
  da.suboff = carve<int32_t>(workspace, pl.off_suboff);
  da.upool = carve<double2>(workspace, pl.off_upool);
  da.subsum = carve<double>(workspace, pl.off_subsum);
  da.out_tokens = out_tokens;
  da.status = status;
  if (launch_draw(da, PSISPEC_F32, stream) != hipSuccess) return PSISPEC_EHIP;
  return PSISPEC_OK;
}

}  // extern "C"
