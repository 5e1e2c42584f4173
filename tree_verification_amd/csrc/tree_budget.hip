// Tree-budget calibration for gfx950: the expected acceptance length of token
// trees, and the goodput lookup that turns measured latencies into a tree size
// per batch size.
//
// Model ([chapter] "Worked Example: How Many Tokens Land Per Expensive
// Pass?", applied per node): drafted node v, when tested, is accepted with
// probability a[v], independently of every other test; a node's children are
// tried in ascending id and the first accepted one continues the walk.  So v
// is on the accepted path exactly when every edge (w -> parent) on its root
// path "fires", where edge w fires with probability
//   e[w] = a[w] * prod over earlier siblings s of w of (1 - a[s]),
// and reach[v] = prod of e over v's root path.  AL = 1 + sum_{v >= 1} reach[v]
// (a round emits the accepted nodes plus one more token).
//
// One wavefront per tree (n <= 128: node j lives in lane j % 64, slot j / 64).
// Each node's children are collected as bit masks (LDS atomics), which give
// every node its previous sibling; the products over earlier siblings and then
// over the root path are both taken by pointer jumping with lane shuffles
// (seven rounds cover any chain below 128), all in float64.

#include "tv_common.h"

#include <math.h>

namespace {

constexpr int kBudgetMaxNodes = 128;

struct BudgetParams {
  const int32_t* parent;
  const int32_t* n_nodes;
  const double* prob;
  double* reach;
  double* al;
  int32_t* status;
  int B, n_max;
};

__device__ __forceinline__ double shfl_d(double v, int src) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Products along links by pointer jumping: on return val[j] holds the product
// of val over j, link(j), link(link(j)), ... (node j: lane j % 64, slot j / 64;
// link -1 ends a chain).  Seven rounds cover chains shorter than 128.
__device__ __forceinline__ void jump_products(double (&val)[2], int (&link)[2]) {
  for (int r = 0; r < 7; ++r) {
    double nval[2];
    int nlink[2];
    for (int s = 0; s < 2; ++s) {
      const int j = link[s];
      const int src = j < 0 ? 0 : (j & 63);
      const double v0 = shfl_d(val[0], src), v1 = shfl_d(val[1], src);
      const int j0 = __shfl(link[0], src), j1 = __shfl(link[1], src);
      if (j >= 0) {
        nval[s] = val[s] * (j >= 64 ? v1 : v0);
        nlink[s] = j >= 64 ? j1 : j0;
      } else {
        nval[s] = val[s];
        nlink[s] = -1;
      }
    }
    for (int s = 0; s < 2; ++s) {
      val[s] = nval[s];
      link[s] = nlink[s];
    }
  }
}

// One wavefront (one workgroup) per tree.
__global__ __launch_bounds__(64) void expected_len_kernel(BudgetParams p) {
  __shared__ int par[kBudgetMaxNodes];
  __shared__ double a[kBudgetMaxNodes];
  __shared__ unsigned long long kids[kBudgetMaxNodes][2];   // children of each node, as bit masks
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int n = p.n_nodes[b];
  const size_t row = (size_t)b * p.n_max;

  int flags = 0;
  if (n < 1 || n > p.n_max) {
    flags = TV_REQ_BAD_NNODES;
  } else {
    bool bad_par = false, bad_prob = false;
    for (int s = 0; s < 2; ++s) {
      const int u = lane + 64 * s;
      if (u < n) {
        const int pu = p.parent[row + u];
        const double au = u > 0 ? p.prob[row + u] : 0.0;
        par[u] = pu;
        a[u] = au;
        kids[u][0] = 0ull;
        kids[u][1] = 0ull;
        bad_par |= (u == 0) ? (pu != -1) : (pu < 0 || pu >= u);
        bad_prob |= u > 0 && !(au >= 0.0 && au <= 1.0);   // NaN fails both compares
      }
    }
    if (__any(bad_par)) flags = TV_REQ_BAD_PARENT;
    else if (__any(bad_prob)) flags = TV_REQ_BAD_PROB;
  }
  if (flags) {
    for (int u = lane; u < p.n_max; u += 64) p.reach[row + u] = 0.0;
    if (lane == 0) {
      p.al[b] = 0.0;
      p.status[b] = flags;
    }
    return;
  }
  __syncthreads();
  for (int s = 0; s < 2; ++s) {
    const int v = lane + 64 * s;
    if (v >= 1 && v < n) atomicOr(&kids[par[v]][s], 1ull << lane);
  }
  __syncthreads();

  // previous sibling of each node, and the rejection of every earlier sibling
  // as a product along previous-sibling links
  const unsigned long long below = (1ull << lane) - 1ull;
  double val[2];
  int link[2];
  for (int s = 0; s < 2; ++s) {
    const int v = lane + 64 * s;
    val[s] = 1.0;
    link[s] = -1;
    if (v >= 1 && v < n) {
      const int pv = par[v];
      const unsigned long long m0 = s == 0 ? (kids[pv][0] & below) : kids[pv][0];
      const unsigned long long m1 = s == 0 ? 0ull : (kids[pv][1] & below);
      const int prev = m1 ? 64 + 63 - __clzll(m1) : (m0 ? 63 - __clzll(m0) : -1);
      if (prev >= 0) {
        val[s] = 1.0 - a[prev];
        link[s] = prev;
      }
    }
  }
  jump_products(val, link);
  // edge weight a[v] * rejection of the earlier siblings, then root-path products
  for (int s = 0; s < 2; ++s) {
    const int v = lane + 64 * s;
    if (v >= 1 && v < n) {
      val[s] *= a[v];
      link[s] = par[v];
    } else {
      val[s] = 1.0;
      link[s] = -1;
    }
  }
  jump_products(val, link);
  double part = 0.0;
  for (int s = 0; s < 2; ++s) {
    const int v = lane + 64 * s;
    if (v < p.n_max) p.reach[row + v] = v < n ? val[s] : 0.0;
    if (v >= 1 && v < n) part += val[s];
  }
  const double total = tv_wave_sum_d(part);
  if (lane == 0) {
    p.al[b] = 1.0 + total;
    p.status[b] = 0;
  }
}

}  // namespace

static int tree_expected_accept_length_impl(const tv_budget_desc* desc, const int32_t* parent, const int32_t* n_nodes,
                                           const double* accept_prob, double* reach, double* expected_len,
                                           int32_t* status, hipStream_t stream) {
  if (!desc || desc->batch < 0) return TV_ERR_INVALID_ARG;
  if (desc->n_max < 1 || desc->n_max > kBudgetMaxNodes) return TV_ERR_UNSUPPORTED;
  if (desc->batch == 0) return TV_OK;
  if (!parent || !n_nodes || !accept_prob || !reach || !expected_len || !status) return TV_ERR_INVALID_ARG;
  BudgetParams p;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.prob = accept_prob;
  p.reach = reach;
  p.al = expected_len;
  p.status = status;
  p.B = desc->batch;
  p.n_max = desc->n_max;
  hipLaunchKernelGGL(expected_len_kernel, dim3(desc->batch), dim3(64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_expected_accept_length(const tv_budget_desc* desc, const int32_t* parent, const int32_t* n_nodes,
                                           const double* accept_prob, double* reach, double* expected_len,
                                           int32_t* status, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_expected_accept_length");
  return tv_debug_finish("tree_expected_accept_length", tree_expected_accept_length_impl(desc, parent, n_nodes, accept_prob, reach, expected_len, status, stream), stream);
}

extern "C" int tree_budget_select(int32_t n_batch_sizes, int32_t n_shapes, const double* al, const double* itl,
                                  int32_t* best) {
  if (n_batch_sizes < 0 || n_shapes < 0) return TV_ERR_INVALID_ARG;
  if (n_batch_sizes == 0) return TV_OK;
  if (!itl || !best || (n_shapes > 0 && !al)) return TV_ERR_INVALID_ARG;
  for (int i = 0; i < n_batch_sizes; ++i) {
    int pick = -1;
    double top = -INFINITY;
    for (int s = 0; s < n_shapes; ++s) {
      const double t = itl[(size_t)i * n_shapes + s];
      if (!(t > 0.0 && isfinite(t))) continue;
      const double g = al[s] / t;
      if (g > top) {
        top = g;
        pick = s;
      }
    }
    best[i] = pick;
  }
  return TV_OK;
}
