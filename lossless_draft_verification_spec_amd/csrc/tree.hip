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

namespace psispec {
namespace {

constexpr int kMaxNodes = 1024;
constexpr int kStagePairs = 4096;  // row pairs of a request staged in LDS (more: read in place)

__device__ inline int row_status(float lmax, double Z) {
  const bool ok = (lmax > kNegBig) && (lmax < __builtin_huge_valf()) && (Z > 0.0) && (Z < 1e300);
  return ok ? 0 : PSISPEC_ST_NONFINITE;
}

template <typename T>
__device__ inline double node_prob(const TreeArgs& a, int64_t row, float lmax, double Z, int tok) {
  const float l = to_f32(row_ptr<T>(a.rs, row)[tok]);
  double pr = exp(((double)l - (double)lmax) * a.inv_T) / Z;
  if (a.use_topp) {
    const ToppStat tp = a.topp[row];
    pr = l >= tp.thr ? pr / tp.M : 0.0;
  }
  return pr;
}

template <typename T>
__global__ __launch_bounds__(64) void k_decide_tree(TreeArgs a) {
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int N = a.N, V = a.V;
  const int64_t row0 = (int64_t)r * (N + 1);
  const int32_t* par = a.parent + (int64_t)r * N;
  const int32_t* tok = a.node_tokens + (int64_t)r * N;

  __shared__ float s_lmax[kMaxNodes + 1];
  __shared__ double s_Z[kMaxNodes + 1];
  __shared__ double s_ratio[kMaxNodes];
  __shared__ int s_st;
  __shared__ int32_t s_par[kMaxNodes], s_tok[kMaxNodes];
  __shared__ double s_u[kMaxNodes];
  __shared__ double s_pown[kMaxNodes];
  __shared__ int s_first[kMaxNodes];
  __shared__ float2 s_pair[kStagePairs];

  // 0. the tree, every node's accept uniform (Philox of (request, c+1, accept)) and the row pairs,
  //    loaded or computed by the whole wave up front: the serial steps below then read LDS only
  for (int j = t; j < N; j += 64) {
    s_par[j] = par[j];
    s_tok[j] = tok[j];
    s_u[j] = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)(j + 1), kPurposeAccept,
                            a.step);
  }
  const bool staged = (int64_t)(N + 1) * a.nchunk <= kStagePairs;
  if (staged)
    for (int i = t; i < (N + 1) * a.nchunk; i += 64) s_pair[i] = a.part[row0 * a.nchunk + i];
  __syncthreads();

  // 1. row statistics of the root and node rows (pairs in chunk order)
  int st = 0;
  for (int j = t; j <= N; j += 64) {
    const int64_t row = row0 + j;
    const float2* pr = staged ? s_pair + j * a.nchunk : a.part + row * a.nchunk;
    float lmax = kNegBig;
    for (int k = 0; k < a.nchunk; ++k) lmax = fmaxf(lmax, pr[k].x);
    double Z = 0.0;
    for (int k = 0; k < a.nchunk; ++k) {
      const float2 pk = pr[k];
      Z += (double)pk.y * exp2((double)(pk.x - lmax) * (double)a.c);
    }
    const int rs = row_status(lmax, Z);
    st |= rs;
    s_lmax[j] = lmax;
    s_Z[j] = Z;
    a.rowstat[row] = RowStat{lmax, rs, Z};
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
  __syncthreads();

  // 3. data-parallel node ratios.  An earlier sibling s of node j has the same parent row, so the
  //    probability it removes from j's residual is s's own probability p_own[s]: one gather per
  //    node, all in parallel, then the sibling sums read LDS.
  for (int j = t; j < N; j += 64) {
    const int v = s_par[j], tj = s_tok[j];
    s_pown[j] = (tj >= 0 && tj < V && v >= -1 && v < j)
                    ? node_prob<T>(a, row0 + v + 1, s_lmax[v + 1], s_Z[v + 1], tj)
                    : 0.0;
  }
  // first[s]: no earlier sibling of s carries s's token (each distinct removed token counts once).
  // With N <= 64, node s sits in lane s and the loops over the earlier siblings read its parent,
  // token, flag and probability from that lane (v_readlane, wave-uniform index: scalar values, no
  // LDS round trips); larger trees read LDS.  Either way R takes the same subtractions in index
  // order.
  __syncthreads();
  if (N <= 64) {
    const int pj = t < N ? s_par[t] : -2, tj = t < N ? s_tok[t] : -1;
    const double pown = t < N ? s_pown[t] : 0.0;
    const int pown_lo = __double2loint(pown), pown_hi = __double2hiint(pown);
    int first = 1;
    for (int s2 = 0; s2 < N; ++s2) {
      const int ps = __builtin_amdgcn_readlane(pj, s2), ts = __builtin_amdgcn_readlane(tj, s2);
      first &= !(s2 < t && ps == pj && ts == tj);
    }
    double ratio = 0.0;
    if (t < N) {
      if (tj < 0 || tj >= V) st |= PSISPEC_ST_BAD_TOKEN;
    }
    double res = pown, R = 1.0;
    for (int s2 = 0; s2 < N; ++s2) {  // earlier siblings, in index order
      const int ps = __builtin_amdgcn_readlane(pj, s2), ts = __builtin_amdgcn_readlane(tj, s2);
      const int fs = __builtin_amdgcn_readlane(first, s2);
      const double ws = __hiloint2double(__builtin_amdgcn_readlane(pown_hi, s2),
                                         __builtin_amdgcn_readlane(pown_lo, s2));
      if (s2 >= t || ps != pj || ts < 0 || ts >= V) continue;
      if (ts == tj)
        res = 0.0;  // same token rejected earlier: already removed from the residual
      else if (fs)
        R -= ws;
    }
    if (t < N) {
      if (tj >= 0 && tj < V && pj >= -1 && pj < t) ratio = R > 0.0 ? fmin(1.0, res / R) : 0.0;
      s_ratio[t] = ratio;
      if (a.node_ratios) a.node_ratios[(int64_t)r * N + t] = (float)ratio;
    }
  } else {
    for (int j = t; j < N; j += 64) {
      const int v = s_par[j], tj = s_tok[j];
      int first = 1;
#pragma unroll 8
      for (int s2 = 0; s2 < N; ++s2) first &= !(s2 < j && s_par[s2] == v && s_tok[s2] == tj);
      s_first[j] = first;
    }
    __syncthreads();
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
      if (a.node_ratios) a.node_ratios[(int64_t)r * N + j] = (float)ratio;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) st |= __shfl_xor(st, off, 64);
  __syncthreads();

  // 4. the walk.  At each node the children are scanned in index order by the whole wave, 64 at a
  //    time: a ballot finds the first accepted child; the valid tokens of the children rejected
  //    before it are appended to the removed-token list in index order.
  const int Dp1 = a.max_depth + 1;
  int32_t* nodes = a.accept_nodes + (int64_t)r * a.max_depth;
  int32_t* out = a.out_tokens + (int64_t)r * Dp1;
  int32_t* excl = a.excl + (int64_t)r * N;
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
        if (t == 0) {
          nodes[dep] = next;
          out[dep] = s_tok[next];
        }
        ++dep;
        cur = next;
      }
    }
  }
  if (t == 0) {
    for (int i = dep; i < a.max_depth; ++i) nodes[i] = -1;
    for (int i = dep; i < Dp1; ++i) out[i] = -1;
    a.accept_len[r] = dep;
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
    a.desc[r] = dd;
    a.ucount[r] = 0;
  }
}

}  // namespace

hipError_t launch_decide_tree(const TreeArgs& a, psispec_dtype dtype, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  timing_begin("decide_tree", stream);
  if (dtype == PSISPEC_BF16)
    hipLaunchKernelGGL(k_decide_tree<bf16_t>, dim3(a.batch), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(k_decide_tree<float>, dim3(a.batch), dim3(64), 0, stream, a);
  timing_end("decide_tree", stream);
  return hipGetLastError();
}

}  // namespace psispec
