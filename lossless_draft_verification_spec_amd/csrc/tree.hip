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
  __shared__ int s_depth[kMaxNodes];
  __shared__ int s_st;

  // 1. row statistics of the root and node rows
  int st = 0;
  for (int j = t; j <= N; j += 64) {
    const int64_t row = row0 + j;
    float lmax = kNegBig;
    for (int k = 0; k < a.nchunk; ++k) lmax = fmaxf(lmax, a.part[row * a.nchunk + k].x);
    double Z = 0.0;
    for (int k = 0; k < a.nchunk; ++k) {
      const float2 pk = a.part[row * a.nchunk + k];
      Z += (double)pk.y * exp2((double)(pk.x - lmax) * (double)a.c);
    }
    const int rs = row_status(lmax, Z);
    st |= rs;
    s_lmax[j] = lmax;
    s_Z[j] = Z;
    a.rowstat[row] = RowStat{lmax, rs, Z};
  }
  // 2. structure: parents precede children, depth within max_depth (one lane, N is small)
  if (t == 0) {
    int bad = 0;
    for (int j = 0; j < N; ++j) {
      const int pj = par[j];
      if (pj < -1 || pj >= j) {
        bad = 1;
        s_depth[j] = 1;
        continue;
      }
      s_depth[j] = pj < 0 ? 1 : s_depth[pj] + 1;
      if (s_depth[j] > a.max_depth) bad = 1;
    }
    s_st = bad ? PSISPEC_ST_BAD_PARENT : 0;
  }
  __syncthreads();

  // 3. data-parallel node ratios
  for (int j = t; j < N; j += 64) {
    const int v = par[j];
    double ratio = 0.0;
    const int tj = tok[j];
    if (tj < 0 || tj >= V) {
      st |= PSISPEC_ST_BAD_TOKEN;
    } else if (v >= -1 && v < j) {
      const int64_t row = row0 + v + 1;
      const float lmax = s_lmax[v + 1];
      const double Z = s_Z[v + 1];
      double res = node_prob<T>(a, row, lmax, Z, tj);
      double R = 1.0;
      for (int s = 0; s < j; ++s) {
        if (par[s] != v) continue;
        const int ts = tok[s];
        if (ts < 0 || ts >= V) continue;
        if (ts == tj) {
          res = 0.0;  // same token rejected earlier: already removed from the residual
          continue;
        }
        bool seen = false;  // subtract each distinct removed token once
        for (int s2 = 0; s2 < s; ++s2)
          if (par[s2] == v && tok[s2] == ts) {
            seen = true;
            break;
          }
        if (!seen) R -= node_prob<T>(a, row, lmax, Z, ts);
      }
      ratio = R > 0.0 ? fmin(1.0, res / R) : 0.0;
    }
    s_ratio[j] = ratio;
    if (a.node_ratios) a.node_ratios[(int64_t)r * N + j] = (float)ratio;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) st |= __shfl_xor(st, off, 64);
  __syncthreads();

  // 4. the walk (one lane)
  const int Dp1 = a.max_depth + 1;
  int32_t* nodes = a.accept_nodes + (int64_t)r * a.max_depth;
  int32_t* out = a.out_tokens + (int64_t)r * Dp1;
  int32_t* excl = a.excl + (int64_t)r * N;
  if (t == 0) {
    st |= s_st;
    int cur = -1, dep = 0, nexcl = 0;
    if (!(s_st & PSISPEC_ST_BAD_PARENT)) {
      for (;;) {
        int next = -1;
        nexcl = 0;
        for (int c = 0; c < N; ++c) {
          if (par[c] != cur) continue;
          const double u = philox_uniform(a.seed, a.request_base + (uint32_t)r, (uint32_t)(c + 1),
                                          kPurposeAccept, a.step);
          if (u < s_ratio[c]) {
            next = c;
            break;
          }
          if (tok[c] >= 0 && tok[c] < V) excl[nexcl++] = tok[c];
        }
        if (next < 0) break;
        nodes[dep] = next;
        out[dep] = tok[next];
        ++dep;
        cur = next;
      }
    }
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
