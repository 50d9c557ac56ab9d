// tree.hip -- node ratios and the walk of the tree verify.
//
// [alphalab] §"Linear 與 Tree sampler": several likely candidates per position are pruned into a
// finite prefix tree that is verified at once.  For candidates chosen deterministically (top-k),
// the lossless rule is the linear rule with a point-mass proposal on each candidate: at node v,
// children in ascending node index, child c kept when u_c < res(tok_c) / R where res is p'_v with
// the tokens of the earlier (rejected) siblings removed and R = 1 - their mass.  Every node's ratio
// is computed data-parallel as if all its earlier siblings were rejected; one lane then walks from
// the root with the Philox uniforms of (request, c+1, accept) and records the stopping node and the
// tokens its rejected children remove from the residual.  The draw itself runs in the fp64 draw
// kernels.
#include "launch.h"
#include "draw.h"

namespace psispec {
namespace {

constexpr int kMaxNodes = 1024;
constexpr int kStagePairs = 4096;  // row pairs of a request staged in LDS (more: read in place)
constexpr int kSmallNodes = 64;    // trees the accept walk fused with the draw pass takes
constexpr int kSmallPairs = 1024;  // row pairs it stages in LDS (more: read in place)

__device__ inline int row_status(float lmax, double Z) {
  const bool ok = (lmax > kNegBig) && (lmax < __builtin_huge_valf()) && (Z > 0.0) && (Z < 1e300);
  return ok ? 0 : PSISPEC_ST_NONFINITE;
}

// p'_row(tok) from the token's logit l (read up front by the caller)
__device__ inline double node_prob(const TreeArgs& a, int64_t row, float lmax, double Z, float l) {
  double pr = exp(((double)l - (double)lmax) * a.inv_T) / Z;
  if (a.use_topp) {
    const ToppStat tp = a.topp[row];
    pr = l >= tp.thr ? pr / tp.M : 0.0;
  }
  return pr;
}

// What the draw pass of the fused kernel takes from the walk, in LDS: the draw description, the
// stopping row's maximum logit and the tokens its rejected children remove.
struct TreeWalkLocal {
  DrawDesc desc;
  float lmax;
  int32_t excl[kSmallNodes];
};

// Node ratios and the walk of request r, by one wave (threads 0..63 of the calling block; it syncs
// with wave barriers only).  kMaxN: most nodes per tree (its LDS arrays); loc: the fused kernel's
// LDS copies (with quiet, the only output: another block of the request writes the call's).
template <typename T, int kMaxN, int kPairs>
__device__ inline void decide_tree_request(const TreeArgs& a, int r, bool quiet, TreeWalkLocal* loc) {
  const int t = threadIdx.x;
  const int N = a.N, V = a.V;
  const int64_t row0 = (int64_t)r * (N + 1);
  const int32_t* par = a.parent + (int64_t)r * N;
  const int32_t* tok = a.node_tokens + (int64_t)r * N;

  __shared__ float s_lmax[kMaxN + 1];
  __shared__ double s_Z[kMaxN + 1];
  __shared__ double s_ratio[kMaxN];
  __shared__ int s_st;
  __shared__ int32_t s_par[kMaxN], s_tok[kMaxN];
  __shared__ double s_u[kMaxN];
  __shared__ double s_pown[kMaxN];
  __shared__ int s_first[kMaxN];
  __shared__ float2 s_pair[kPairs];

  // 0. the tree, every node's accept uniform (Philox of (request, c+1, accept)) and the row pairs,
  //    loaded or computed by the whole wave up front; then the logit of each node's token in its
  //    parent's row, gathered into the lane that scores the node.  The block is one wave and syncs
  //    with wave barriers, which do not wait for the gathers: they stay in flight through the row
  //    statistics and the structure check, and only the ratios wait for them.
  for (int j = t; j < N; j += 64) {
    s_par[j] = par[j];
    s_tok[j] = tok[j];
    s_u[j] = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)(j + 1), kPurposeAccept,
                            a.step);
  }
  const bool staged = (int64_t)(N + 1) * a.nchunk <= kPairs;
  if (staged)
    for (int i = t; i < (N + 1) * a.nchunk; i += 64) s_pair[i] = a.part[row0 * a.nchunk + i];
  wave_sync();
  constexpr int kGl = kMaxN / 64;  // nodes per lane
  float gl[kGl];                       // node t + 64 k's token logit
#pragma unroll
  for (int k = 0; k < kGl; ++k) {
    const int j = t + 64 * k;
    gl[k] = 0.f;
    if (j < N) {
      const int v = s_par[j], tj = s_tok[j];
      if (tj >= 0 && tj < V && v >= -1 && v < j) gl[k] = to_f32(row_ptr<T>(a.rs, row0 + v + 1)[tj]);
    }
  }

  // 1. row statistics of the root and node rows (pairs in chunk order)
  int st = 0;
  // (LDS and global pairs in separate branches: a pointer that may be either would be read by
  // flat loads, whose waits also wait for the gathers)
  auto pair_stats = [&](const float2* pr, float& lmax, double& Z) {
    lmax = kNegBig;
    for (int k = 0; k < a.nchunk; ++k) lmax = fmaxf(lmax, pr[k].x);
    Z = 0.0;
    for (int k = 0; k < a.nchunk; ++k) {
      const float2 pk = pr[k];
      Z += (double)pk.y * exp2((double)(pk.x - lmax) * (double)a.c);
    }
  };
  for (int j = t; j <= N; j += 64) {
    const int64_t row = row0 + j;
    float lmax;
    double Z;
    if (staged)
      pair_stats(s_pair + j * a.nchunk, lmax, Z);
    else
      pair_stats(a.part + row * a.nchunk, lmax, Z);
    const int rs = row_status(lmax, Z);
    st |= rs;
    s_lmax[j] = lmax;
    s_Z[j] = Z;
    if (!quiet) a.rowstat[row] = RowStat{lmax, rs, Z};
  }
  // 2. structure: parents precede children, depth within max_depth.  Each lane climbs its node's
  //    parent chain (indices strictly decrease along a valid chain; a chain that meets an invalid
  //    parent stops there, and that node's own lane flags it).
  {
    int bad = 0;
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
    if (t < 64) {
      const uint64_t bm = __ballot(bad);
      if (t == 0) s_st = bm ? PSISPEC_ST_BAD_PARENT : 0;
    }
  }
  wave_sync();

  // 3. data-parallel node ratios.  An earlier sibling s of node j has the same parent row, so the
  //    probability it removes from j's residual is s's own probability p_own[s]: one gather per
  //    node, all in parallel, then the sibling sums read LDS.
#pragma unroll
  for (int k = 0; k < kGl; ++k) {
    const int j = t + 64 * k;
    if (j >= N) break;
    const int v = s_par[j], tj = s_tok[j];
    s_pown[j] = (tj >= 0 && tj < V && v >= -1 && v < j)
                    ? node_prob(a, row0 + v + 1, s_lmax[v + 1], s_Z[v + 1], gl[k])
                    : 0.0;
  }
  // first[s]: no earlier sibling of s carries s's token (each distinct removed token counts once).
  // With N <= 64, node s sits in lane s: one ballot per distinct parent gives every lane the mask
  // of its siblings, and each lane then visits only its earlier siblings, in index order (LDS
  // reads), so R takes the same subtractions in index order as the general form below.
  wave_sync();
  if (kMaxN <= 64 || N <= 64) {
    const int pj = t < N ? s_par[t] : -2, tj = t < N ? s_tok[t] : -1;
    uint64_t sib = 0;
    for (uint64_t todo = __ballot(t < N); todo;) {
      const int v = __builtin_amdgcn_readlane(pj, __builtin_ctzll(todo));
      const bool same = t < N && pj == v;
      const uint64_t m = __ballot(same);
      if (same) sib = m;
      todo &= ~m;
    }
    const uint64_t earlier = sib & ((1ull << t) - 1ull);  // t < 64
    int first = 1;
    for (uint64_t m = earlier; m; m &= m - 1) first &= s_tok[__builtin_ctzll(m)] != tj;
    if (t < N) s_first[t] = first;
    wave_sync();
    double ratio = 0.0;
    if (t < N) {
      if (tj < 0 || tj >= V) st |= PSISPEC_ST_BAD_TOKEN;
    }
    double res = t < N ? s_pown[t] : 0.0, R = 1.0;
    for (uint64_t m = earlier; m; m &= m - 1) {  // earlier siblings, in index order
      const int s2 = __builtin_ctzll(m);
      const int ts = s_tok[s2];
      if (ts < 0 || ts >= V) continue;
      if (ts == tj)
        res = 0.0;  // same token rejected earlier: already removed from the residual
      else if (s_first[s2])
        R -= s_pown[s2];
    }
    if (t < N) {
      if (tj >= 0 && tj < V && pj >= -1 && pj < t) ratio = R > 0.0 ? fmin(1.0, res / R) : 0.0;
      s_ratio[t] = ratio;
      if (a.node_ratios && !quiet) a.node_ratios[(int64_t)r * N + t] = (float)ratio;
    }
  } else if constexpr (kMaxN > 64) {
    for (int j = t; j < N; j += 64) {
      const int v = s_par[j], tj = s_tok[j];
      int first = 1;
#pragma unroll 8
      for (int s2 = 0; s2 < N; ++s2) first &= !(s2 < j && s_par[s2] == v && s_tok[s2] == tj);
      s_first[j] = first;
    }
    wave_sync();
    for (int j = t; j < N; j += 64) {
      const int v = s_par[j];
      double ratio = 0.0;
      const int tj = s_tok[j];
      if (tj < 0 || tj >= V) {
        st |= PSISPEC_ST_BAD_TOKEN;
      } else if (v >= -1 && v < j) {
        double res = s_pown[j];
        double R = 1.0;
#pragma unroll 8
        for (int s2 = 0; s2 < N; ++s2) {  // earlier siblings, in index order
          const int ts = s_tok[s2];
          if (s2 >= j || s_par[s2] != v || ts < 0 || ts >= V) continue;
          if (ts == tj)
            res = 0.0;  // same token rejected earlier: already removed from the residual
          else if (s_first[s2])
            R -= s_pown[s2];
        }
        ratio = R > 0.0 ? fmin(1.0, res / R) : 0.0;
      }
      s_ratio[j] = ratio;
      if (a.node_ratios && !quiet) a.node_ratios[(int64_t)r * N + j] = (float)ratio;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) st |= __shfl_xor(st, off, 64);
  wave_sync();

  // 4. the walk.  At each node the children are scanned in index order by the whole wave, 64 at a
  //    time: a ballot finds the first accepted child; the valid tokens of the children rejected
  //    before it are appended to the removed-token list in index order.
  const int Dp1 = a.max_depth + 1;
  int32_t* nodes = a.accept_nodes + (int64_t)r * a.max_depth;
  int32_t* out = a.out_tokens + (int64_t)r * Dp1;
  // the removed tokens: the fused kernel's LDS list (copied to the workspace after the walk unless
  // quiet), else the workspace
  int32_t* excl = loc ? loc->excl : a.excl + (int64_t)r * N;
  int cur = -1, dep = 0, nexcl = 0;
  if (t < 64) {
    st |= s_st;
    if (!(s_st & PSISPEC_ST_BAD_PARENT)) {
      for (;;) {
        int next = -1;
        nexcl = 0;
        for (int c0 = 0; c0 < N && next < 0; c0 += 64) {
          const int c = c0 + t;
          const bool child = c < N && s_par[c] == cur;
          const uint64_t am = __ballot(child && s_u[c] < s_ratio[c]);
          const int firstacc = am ? __builtin_ctzll(am) : 64;
          const uint64_t before = firstacc == 64 ? ~0ull : ((1ull << firstacc) - 1ull);
          const bool rej = child && t < firstacc && s_tok[c] >= 0 && s_tok[c] < V;
          const uint64_t rm = __ballot(rej) & before;
          if (rej) excl[nexcl + __builtin_popcountll(rm & ((1ull << t) - 1ull))] = s_tok[c];
          nexcl += __builtin_popcountll(rm);
          if (firstacc < 64) next = c0 + firstacc;
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
  }
  if (loc && !quiet) {
    wave_sync();  // the LDS list is complete
    for (int i = t; i < nexcl; i += 64) a.excl[(int64_t)r * N + i] = loc->excl[i];
  }
  if (t == 0) {
    if (!quiet) {
      for (int i = dep; i < a.max_depth; ++i) nodes[i] = -1;
      for (int i = dep; i < Dp1; ++i) out[i] = -1;
      a.accept_len[r] = dep;
    }
    DrawDesc dd;
    dd.prow = (int32_t)(row0 + cur + 1);
    dd.qrow = -1;
    dd.pos = cur + 1;
    dd.st = st;
    dd.nexcl = nexcl;
    dd.out_idx = (s_st & PSISPEC_ST_BAD_PARENT) ? -1 : (int32_t)((int64_t)r * Dp1 + dep);
    dd.ph_req = r;
    dd.purpose = kPurposeDraw;
    dd.factor = 1.0;
    if (!quiet) a.desc[r] = dd;
    if (loc) {
      loc->desc = dd;
      loc->lmax = s_lmax[cur + 1];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(64) void k_decide_tree(TreeArgs a) {
  decide_tree_request<T, kMaxNodes, kStagePairs>(a, blockIdx.x, false, nullptr);
}

// The chosen-candidate tree's walk fused with its draw pass (trees of at most kSmallNodes nodes):
// block (r, c) runs request r's walk in wave 0 into LDS, then draws chunk c of the stopping row from
// those copies; the chunk-0 block also writes the call's outputs and the records the select
// reads.  One launch fewer than the walk followed by the pass, and no dependent reads of the
// description, the row statistics and the removed tokens.
template <typename T, bool kTopp>
__global__ __launch_bounds__(kThreads, kDrawPassWaves) void k_decide_tree_draw(TreeArgs ta,
                                                                               DrawArgs da,
                                                                               int vec_ok) {
  __shared__ double tbl[kExpTable];
  __shared__ TreeWalkLocal loc;
  exp_table_fill(tbl);  // read after the barriers below
  const int r = blockIdx.x / da.nchunk_draw;
  const int c = blockIdx.x - r * da.nchunk_draw;
  if (threadIdx.x < 64) decide_tree_request<T, kSmallNodes, kSmallPairs>(ta, r, c != 0, &loc);
  __syncthreads();  // the description, the stopping row's maximum and the removed tokens are in LDS
  const DrawDesc d = loc.desc;
  RowView v;
  v.lmax_p = loc.lmax;
  v.thr_p = kTopp ? ta.topp[d.prow].thr : -__builtin_huge_valf();
  v.lmax_q = 0.f;
  v.thr_q = 0.f;
  DrawArgs dl = da;
  dl.excl = loc.excl;  // read at excl[r * excl_stride + i]: the LDS list
  dl.excl_stride = 0;
  draw_pass_run<T, kTopp>(dl, r, c, vec_ok, d, v, 0.0, tbl);
}

}  // namespace

hipError_t launch_decide_tree_draw(const TreeArgs& ta, const DrawArgs& da, psispec_dtype dtype,
                                   hipStream_t stream) {
  if (da.batch == 0) return hipSuccess;
  if (ta.N > kSmallNodes || da.list || ta.batch != da.batch || ta.use_topp != da.use_topp)
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((int64_t)da.batch * da.nchunk_draw);
  const int vec_ok = draw_vec_ok(da, dtype);
  const bool bf = dtype == PSISPEC_BF16, tp = da.use_topp;
  auto kern = bf ? (tp ? k_decide_tree_draw<bf16_t, true> : k_decide_tree_draw<bf16_t, false>)
                 : (tp ? k_decide_tree_draw<float, true> : k_decide_tree_draw<float, false>);
  PSISPEC_LAUNCH("decide_tree_draw", kern, dim3(grid), dim3(kThreads), 0, stream, ta, da, vec_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw_select(da, dtype, stream);
}

hipError_t launch_decide_tree(const TreeArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (dtype == PSISPEC_BF16)
    PSISPEC_LAUNCH("decide_tree", k_decide_tree<bf16_t>, dim3(a.batch), dim3(64), 0, stream, a);
  else
    PSISPEC_LAUNCH("decide_tree", k_decide_tree<float>, dim3(a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace psispec
