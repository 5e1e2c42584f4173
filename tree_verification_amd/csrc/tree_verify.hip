// Token-tree verification for gfx950.
//
// Greedy ([guide] "Greedy Verification Algorithm"): one workgroup per (node,
// vocabulary chunk) computes the chunk's max / first argmax of the target row;
// the last workgroup to finish a request combines the chunks, picks for every
// node the first child whose token equals the node's argmax, and walks the
// root path (at most depth + 1 dependent steps).
//
// Stochastic ([guide] "Stochastic Verification Algorithm"; [chapter] the
// min(1, p/q) acceptance rule and the residual max(p - q, 0) / Z): each node's
// decision depends only on its own two rows, its children's tokens and their
// uniforms, so every node decides in parallel and the path is chased at the
// end.  At node u with children c_1, c_2, ... the residual after i rejections
// has the closed form
//     p^(i)(w) = max(p(w) - C_i q(w), 0) / D_i,
//     C_0 = 0, D_0 = 1,  C_{i+1} = C_i + D_i,  D_{i+1} = F(C_{i+1}),
//     F(c) = sum_w max(p(w) - c q(w), 0),
// (induction on the recursive residual; Z_{i+1} = F(C_{i+1}) / D_i), so a
// rejection costs one vocabulary pass evaluating F at a known point, and the
// accept test of c_{i+1} is  u * q(x) * D_i <= max(p(x) - C_i q(x), 0).
// A team of S workgroups shares each node: each owns a slice of vocabulary
// tiles, and the team meets at bounded barriers (cooperative launch keeps the
// whole grid resident, so a team's members always run together).  The final
// draw is a two-level inverse CDF: tile masses, then a scan inside one tile.
// Exponentials are float32 (expf), sums and the accept test float64.

#include "tv_common.h"

#include <math.h>

namespace {

constexpr int kVThreads = 512;
constexpr int kTileElems = kVThreads * 16;     // 8192 logits per tile (16 per thread)
constexpr int kGreedyThreads = 256;
constexpr int kGreedyChunk = kGreedyThreads * 32;
constexpr int kMaxNodes = 128;
constexpr int kMaxTiles = 64;                  // vocabulary up to 64 * 8192 = 524288
constexpr long long kSpinLimit = 1LL << 22;   // bounded waits: ~0.5 s worst case, then TV_REQ_TIMEOUT
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// small block reductions
// ---------------------------------------------------------------------------

template <int NT>
__device__ float block_max(float v, float* red) {
  v = tv_wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int NT>
__device__ double block_sum_d(double v, double* red) {
  v = tv_wave_sum_d(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < NT / 64; ++i) r += red[i];   // fixed order: identical in every workgroup
  return r;
}

template <int NT>
__device__ int block_or(int v, int* red) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  unsigned long long bal = __ballot(v != 0);
  __syncthreads();
  if (l == 0) red[w] = bal != 0ull;
  __syncthreads();
  int r = 0;
  for (int i = 0; i < NT / 64; ++i) r |= red[i];
  return r;
}

// 16 consecutive logits of one thread (elements at or past `bound` read as -inf);
// rows whose length is a multiple of 4 are 16-byte aligned and use vector loads.
__device__ __forceinline__ void load16(const float* row, int V, int bound, int e0, float* x) {
  if ((V & 3) == 0 && e0 + 16 <= bound) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tv_f32x4 a = *(const tv_f32x4*)(row + e0 + 4 * i);
      x[4 * i] = a[0];
      x[4 * i + 1] = a[1];
      x[4 * i + 2] = a[2];
      x[4 * i + 3] = a[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (e0 + i < bound) ? row[e0 + i] : kNegInf;
  }
}

// ===========================================================================
// greedy
// ===========================================================================

struct GreedyParams {
  const float* logits;
  const int32_t* tokens;
  const int32_t* parent;
  const int32_t* n_nodes;
  int32_t* path;
  int32_t* path_len;
  int32_t* out_tokens;
  int32_t* status;
  float* part_val;   // [B][n_max][chunks]
  int* part_idx;     // [B][n_max][chunks]
  int* part_bad;     // [B][n_max][chunks]
  int* counters;     // [B]
  int B, n_max, V, chunks;
};

__global__ __launch_bounds__(kGreedyThreads) void greedy_kernel(GreedyParams p) {
  __shared__ float s_val[kGreedyThreads / 64];
  __shared__ int s_idx[kGreedyThreads / 64];
  __shared__ int s_bad[kGreedyThreads / 64];
  __shared__ int s_last;
  __shared__ int s_arg[kMaxNodes];
  __shared__ int s_child[kMaxNodes];
  __shared__ int s_flags;

  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int lid = blockIdx.x;
  const int c = lid % p.chunks;
  const int u = (lid / p.chunks) % p.n_max;
  const int b = lid / (p.chunks * p.n_max);
  const int n = p.n_nodes[b];
  if (n < 1 || n > p.n_max) {
    if (u == 0 && c == 0 && t == 0) {
      p.status[b] = TV_REQ_BAD_NNODES;
      p.path_len[b] = 0;
    }
    return;
  }
  if (u >= n) return;

  // chunk max with the lowest index among equal maxima
  const float* row = p.logits + ((size_t)b * p.n_max + u) * p.V;
  const int lo = c * kGreedyChunk, hi = min(p.V, lo + kGreedyChunk);
  float best = kNegInf;
  int bidx = 0x7fffffff;
  int bad = 0;
  for (int e0 = lo + 16 * t; e0 < hi; e0 += 16 * kGreedyThreads) {
    float x[16];
    load16(row, p.V, hi, e0, x);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (e0 + i < hi) {
        bad |= !isfinite(x[i]);
        if (x[i] > best) {
          best = x[i];
          bidx = e0 + i;
        }
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(best, o);
    int oi = __shfl_xor(bidx, o);
    if (ov > best || (ov == best && oi < bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  unsigned long long anybad = __ballot(bad != 0);
  if (l == 0) {
    s_val[w] = best;
    s_idx[w] = bidx;
    s_bad[w] = anybad != 0ull;
  }
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kGreedyThreads / 64; ++i) {
      if (s_val[i] > best || (s_val[i] == best && s_idx[i] < bidx)) {
        best = s_val[i];
        bidx = s_idx[i];
      }
      s_bad[0] |= s_bad[i];
    }
    size_t slot = ((size_t)b * p.n_max + u) * p.chunks + c;
    p.part_val[slot] = best;
    p.part_idx[slot] = bidx;
    p.part_bad[slot] = s_bad[0];
    __threadfence();
    int prev = atomicAdd(&p.counters[b], 1);
    s_last = (prev == n * p.chunks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // last arrival for request b: per-node argmax, matching child, root path
  if (t == 0) s_flags = 0;
  __syncthreads();
  const int32_t* par = p.parent + (size_t)b * p.n_max;
  const int32_t* tok = p.tokens + (size_t)b * p.n_max;
  for (int v = t; v < n; v += kGreedyThreads) {
    float bv = kNegInf;
    int bi = 0x7fffffff, bb = 0;
    for (int cc = 0; cc < p.chunks; ++cc) {
      size_t slot = ((size_t)b * p.n_max + v) * p.chunks + cc;
      float cv = p.part_val[slot];
      int ci = p.part_idx[slot];
      bb |= p.part_bad[slot];
      if (cv > bv) {   // chunks in ascending order: the first chunk wins ties
        bv = cv;
        bi = ci;
      }
    }
    s_arg[v] = (bi == 0x7fffffff) ? 0 : bi;
    s_child[v] = 0x7fffffff;
    int pv = par[v];
    bool ok = (v == 0) ? (pv == -1) : (pv >= 0 && pv < v);
    if (!ok) atomicOr(&s_flags, TV_REQ_BAD_PARENT);
    if (bb) atomicOr(&s_flags, TV_REQ_NONFINITE);
  }
  __syncthreads();
  if (s_flags == 0) {
    for (int v = 1 + t; v < n; v += kGreedyThreads) {
      int pv = par[v];
      if (tok[v] == s_arg[pv]) atomicMin(&s_child[pv], v);
    }
  }
  __syncthreads();
  if (t == 0) {
    if (s_flags) {
      p.status[b] = s_flags;
      p.path_len[b] = 0;
    } else {
      int32_t* path = p.path + (size_t)b * p.n_max;
      int32_t* out = p.out_tokens + (size_t)b * p.n_max;
      int cur = 0, j = 0;
      path[0] = 0;
      while (s_child[cur] != 0x7fffffff && j + 1 < n) {
        int ch = s_child[cur];
        out[j] = tok[ch];
        path[++j] = ch;
        cur = ch;
      }
      out[j] = s_arg[cur];
      p.path_len[b] = j + 1;
      p.status[b] = 0;
    }
    p.counters[b] = 0;
  }
}

// ===========================================================================
// stochastic
// ===========================================================================

struct StochParams {
  const float* target;
  const float* draft;
  const int32_t* tokens;
  const int32_t* parent;
  const int32_t* n_nodes;
  const float* u_accept;
  const float* u_sample;
  int32_t* path;
  int32_t* path_len;
  int32_t* out_tokens;
  int32_t* status;
  // workspace
  float* tile_m;     // [nodes][2][tiles]   per-tile max of the target / draft row
  double* tile_s;    // [nodes][2][tiles]   per-tile sum exp((z - tile max) / T)
  double* tile_f;    // [nodes][3][tiles]   per-tile residual mass of the last passes
  int* acc_child;    // [nodes]
  int* final_tok;    // [nodes]
  int* node_flags;   // [nodes]
  int* arrive;       // [nodes]  team barrier counters
  int* depart;       // [nodes]
  int* req_done;     // [B]
  int B, n_max, V, tiles, S, slots;
  float invT;
  double invT_d;
};

struct StochSmem {
  float tm[2][kMaxTiles];     // tile maxima (target, draft) staged from the workspace
  double ts[2][kMaxTiles];    // tile exp-sums
  double tf[kMaxTiles];       // tile residual masses of the latest pass
  double tcur[kMaxTiles];     // tile masses of the current residual
  double red_d[kVThreads / 64];
  float red_f[kVThreads / 64];
  int red_i[kVThreads / 64];
  double scan[kVThreads / 64];
  int kids[kMaxNodes];
  int facc[kMaxNodes];        // request finalisation: accepted child and final token per node
  int ffin[kMaxNodes];
  int fflags;
  int nkids;
  int timeout;
  int sel;
  int last;
  int fin;
  int badtok;
};

// Team barrier: every member adds one arrival and waits for S * phase of them.
// Bounded: on expiry the request is flagged TV_REQ_TIMEOUT and the workgroup
// carries on (all later reads stay in bounds).
__device__ void team_barrier(const StochParams& p, StochSmem& sm, int k, int phase) {
  if (p.S == 1) {
    __syncthreads();
    return;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&p.arrive[k], 1);
    const int target = p.S * phase;
    long long it = 0;
    while (__hip_atomic_load(&p.arrive[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it > kSpinLimit) {
        sm.timeout = 1;
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

// Row statistics of one tile: max, then sum of expf((z - max) * invT) in float64.
__device__ void tile_stats(const StochParams& p, StochSmem& sm, const float* row, int tile, float* m_out,
                           double* s_out, int* bad) {
  const int t = threadIdx.x;
  const int e0 = tile * kTileElems + 16 * t;
  float x[16];
  load16(row, p.V, p.V, e0, x);
  float mx = kNegInf;
  int nb = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (e0 + i < p.V) {
      nb |= !isfinite(x[i]);
      mx = fmaxf(mx, x[i]);
    }
  }
  *bad |= nb;
  const float M = block_max<kVThreads>(mx, sm.red_f);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (e0 + i < p.V) s += (double)expf((x[i] - M) * p.invT);
  s = block_sum_d<kVThreads>(s, sm.red_d);
  *m_out = M;
  *s_out = s;
}

// Residual weights max(p - c q, 0) of 16 logits, float32 exponentials, float64 combination.
__device__ __forceinline__ void residual16(const StochParams& p, const float* zp, const float* zq, int e0,
                                           float Mp, float Mq, double ip, double iq, double c, double* w) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (e0 + i < p.V) {
      double pw = (double)expf((zp[i] - Mp) * p.invT) * ip;
      double qw = (double)expf((zq[i] - Mq) * p.invT) * iq;
      w[i] = fmax(pw - c * qw, 0.0);
    } else {
      w[i] = 0.0;
    }
  }
}

__global__ __launch_bounds__(kVThreads) void stochastic_kernel(StochParams p) {
  __shared__ StochSmem sm;
  const int t = threadIdx.x;
  const int slot = blockIdx.x / p.S, member = blockIdx.x % p.S;
  const int tiles_per = (p.tiles + p.S - 1) / p.S;
  const int my_t0 = member * tiles_per, my_t1 = min(p.tiles, my_t0 + tiles_per);
  const int total_nodes = p.B * p.n_max;
  for (int k = slot; k < total_nodes; k += p.slots) {
    const int b = k / p.n_max, u = k % p.n_max;
    const int n = p.n_nodes[b];
    if (n < 1 || n > p.n_max) {
      if (u == 0 && member == 0 && t == 0) {
        p.status[b] = TV_REQ_BAD_NNODES;
        p.path_len[b] = 0;
      }
      continue;
    }
    if (u >= n) continue;
    const int32_t* par = p.parent + (size_t)b * p.n_max;
    const int32_t* tok = p.tokens + (size_t)b * p.n_max;
    const float* zp = p.target + ((size_t)b * p.n_max + u) * p.V;
    const float* zq = p.draft + ((size_t)b * p.n_max + u) * p.V;

    // children of u in ascending id
    __syncthreads();
    if (t == 0) {
      int c = 0, badtok = 0;
      for (int v = 1; v < n; ++v) {
        if (par[v] == u) {
          sm.kids[c++] = v;
          badtok |= (tok[v] < 0 || tok[v] >= p.V);
        }
      }
      sm.nkids = c;
      sm.badtok = badtok;
      sm.timeout = 0;
    }
    __syncthreads();
    const int nk = sm.nkids;
    int flags = sm.badtok ? TV_REQ_BAD_TOKEN : 0;

    // phase 1: per-tile statistics of my slice
    int bad = 0;
    for (int tl = my_t0; tl < my_t1; ++tl) {
      float m;
      double s;
      tile_stats(p, sm, zp, tl, &m, &s, &bad);
      if (t == 0) {
        p.tile_m[((size_t)k * 2) * p.tiles + tl] = m;
        p.tile_s[((size_t)k * 2) * p.tiles + tl] = s;
      }
      if (nk > 0) {
        tile_stats(p, sm, zq, tl, &m, &s, &bad);
        if (t == 0) {
          p.tile_m[((size_t)k * 2 + 1) * p.tiles + tl] = m;
          p.tile_s[((size_t)k * 2 + 1) * p.tiles + tl] = s;
        }
      }
    }
    if (block_or<kVThreads>(bad, sm.red_i) && t == 0) atomicOr(&p.node_flags[k], TV_REQ_NONFINITE);
    int phase = 1;
    team_barrier(p, sm, k, phase++);
    // stage every member's tile statistics into LDS (one parallel round trip)
    for (int i = t; i < 2 * p.tiles; i += kVThreads) {
      const int r = i / p.tiles, tl = i % p.tiles;
      if (r == 0 || nk > 0) {
        sm.tm[r][tl] = p.tile_m[((size_t)k * 2 + r) * p.tiles + tl];
        sm.ts[r][tl] = p.tile_s[((size_t)k * 2 + r) * p.tiles + tl];
      }
    }
    __syncthreads();

    // row maxima and normalisers (every member, same order -> same values)
    float Mp = kNegInf, Mq = kNegInf;
    for (int tl = 0; tl < p.tiles; ++tl) {
      Mp = fmaxf(Mp, sm.tm[0][tl]);
      if (nk > 0) Mq = fmaxf(Mq, sm.tm[1][tl]);
    }
    double Sp = 0.0, Sq = 0.0;
    for (int tl = 0; tl < p.tiles; ++tl) {
      Sp += sm.ts[0][tl] * exp((double)(sm.tm[0][tl] - Mp) * p.invT_d);
      if (nk > 0) Sq += sm.ts[1][tl] * exp((double)(sm.tm[1][tl] - Mq) * p.invT_d);
    }
    const double ip = 1.0 / Sp, iq = nk > 0 ? 1.0 / Sq : 0.0;
    const double lse_p = (double)Mp * p.invT_d + log(Sp);
    const double lse_q = nk > 0 ? (double)Mq * p.invT_d + log(Sq) : 0.0;

    // decisions along the children, one vocabulary pass per rejection
    double Cres = 0.0, Dres = 1.0;
    int cur_buf = -1, buf = 0, accepted = -1;
    for (int i = 0; i < nk; ++i) {
      const int c = sm.kids[i];
      const int x = tok[c];
      if (flags & TV_REQ_BAD_TOKEN) break;
      const double px = exp((double)zp[x] * p.invT_d - lse_p);
      const double qx = exp((double)zq[x] * p.invT_d - lse_q);
      const double ua = (double)p.u_accept[(size_t)b * p.n_max + c];
      if (ua * qx * Dres <= fmax(px - Cres * qx, 0.0)) {
        accepted = c;
        break;
      }
      const double cn = Cres + Dres;
      for (int tl = my_t0; tl < my_t1; ++tl) {
        const int e0 = tl * kTileElems + 16 * t;
        float xp[16], xq[16];
        load16(zp, p.V, p.V, e0, xp);
        load16(zq, p.V, p.V, e0, xq);
        double w[16];
        residual16(p, xp, xq, e0, Mp, Mq, ip, iq, cn, w);
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) s += w[j];
        s = block_sum_d<kVThreads>(s, sm.red_d);
        if (t == 0) p.tile_f[((size_t)k * 3 + buf) * p.tiles + tl] = s;
      }
      team_barrier(p, sm, k, phase++);
      for (int i = t; i < p.tiles; i += kVThreads) sm.tf[i] = p.tile_f[((size_t)k * 3 + buf) * p.tiles + i];
      __syncthreads();
      double F = 0.0;
      for (int tl = 0; tl < p.tiles; ++tl) F += sm.tf[tl];
      // Z > 0: move to the new residual.  The next pass writes a buffer that is
      // neither the one just summed (a slower member may still be reading it)
      // nor the one holding the current residual's tile masses.
      const int just = buf;
      if (F > 0.0) {
        Cres = cn;
        Dres = F;
        cur_buf = buf;
        __syncthreads();
        for (int i = t; i < p.tiles; i += kVThreads) sm.tcur[i] = sm.tf[i];
      }
      buf = 0;
      while (buf == just || buf == cur_buf) ++buf;
    }

    bool writer = (member == 0);
    int result_tok = -1;
    if (accepted < 0 && !(flags & TV_REQ_BAD_TOKEN)) {
      // two-level inverse CDF: tile masses, then a scan inside the selected tile
      __syncthreads();
      const double us = (double)p.u_sample[(size_t)b * p.n_max + u];
      double total = 0.0;
      for (int tl = 0; tl < p.tiles; ++tl) {
        double mass = (cur_buf < 0) ? sm.ts[0][tl] * exp((double)(sm.tm[0][tl] - Mp) * p.invT_d) * ip
                                    : sm.tcur[tl];
        total += mass;
      }
      const double thr = us * total;
      double cum = 0.0, base = 0.0;
      int sel = -1, lastpos = 0;
      for (int tl = 0; tl < p.tiles; ++tl) {
        double mass = (cur_buf < 0) ? sm.ts[0][tl] * exp((double)(sm.tm[0][tl] - Mp) * p.invT_d) * ip
                                    : sm.tcur[tl];
        if (mass > 0.0) lastpos = tl;
        if (sel < 0 && cum + mass > thr) {
          sel = tl;
          base = cum;
        }
        cum += mass;
      }
      if (sel < 0) {
        sel = lastpos;
        base = cum;   // nothing crosses: the scan falls back to the last positive weight
      }
      writer = (sel >= my_t0 && sel < my_t1);
      if (writer) {
        const int e0 = sel * kTileElems + 16 * t;
        double w[16];
        if (cur_buf < 0) {
          float xp[16];
          load16(zp, p.V, p.V, e0, xp);
          const float Mt = sm.tm[0][sel];
          const double sc = exp((double)(Mt - Mp) * p.invT_d) * ip;
#pragma unroll
          for (int j = 0; j < 16; ++j) w[j] = (e0 + j < p.V) ? (double)expf((xp[j] - Mt) * p.invT) * sc : 0.0;
        } else {
          float xp[16], xq[16];
          load16(zp, p.V, p.V, e0, xp);
          load16(zq, p.V, p.V, e0, xq);
          residual16(p, xp, xq, e0, Mp, Mq, ip, iq, Cres, w);
        }
        double loc = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) loc += w[j];
        // exclusive scan of the per-thread totals (wave scan, then across waves)
        const int wv = t >> 6, ln = t & 63;
        double incl = loc;
        for (int o = 1; o < 64; o <<= 1) {
          double y = __shfl_up(incl, o);
          if (ln >= o) incl += y;
        }
        __syncthreads();
        if (ln == 63) sm.scan[wv] = incl;
        __syncthreads();
        double pre = base;
        for (int i2 = 0; i2 < wv; ++i2) pre += sm.scan[i2];
        pre += incl - loc;
        int found = 0x7fffffff, lastw = -1;
        double run = pre;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          run += w[j];
          if (found == 0x7fffffff && w[j] > 0.0 && run > thr) found = e0 + j;
          if (w[j] > 0.0) lastw = e0 + j;
        }
        if (t == 0) {
          sm.sel = 0x7fffffff;
          sm.last = -1;
        }
        __syncthreads();
        if (found != 0x7fffffff) atomicMin(&sm.sel, found);
        if (lastw >= 0) atomicMax(&sm.last, lastw);
        __syncthreads();
        result_tok = (sm.sel != 0x7fffffff) ? sm.sel : (sm.last >= 0 ? sm.last : sel * kTileElems);
      }
    }

    // publish the node's result; the last node of the request chases the path
    __syncthreads();
    if (writer && t == 0) {
      if (sm.timeout) flags |= TV_REQ_TIMEOUT;
      if (flags) atomicOr(&p.node_flags[k], flags);
      p.acc_child[k] = accepted;
      p.final_tok[k] = result_tok;
      __threadfence();
      int prev = atomicAdd(&p.req_done[b], 1);
      sm.fin = (prev == n - 1);
    }
    __syncthreads();
    // leave the team counters at zero: the last member to depart resets them
    if (p.S > 1 && t == 0) {
      int prev = atomicAdd(&p.depart[k], 1);
      if (prev == p.S - 1) {
        p.arrive[k] = 0;
        p.depart[k] = 0;
      }
    }
    if (writer && sm.fin) {
      __threadfence();   // acquire: every node of the request has published its result
      if (t == 0) sm.fflags = 0;
      __syncthreads();
      for (int v = t; v < n; v += kVThreads) {
        const size_t kv = (size_t)b * p.n_max + v;
        sm.facc[v] = p.acc_child[kv];
        sm.ffin[v] = p.final_tok[kv];
        const int pv = par[v];
        const bool ok = (v == 0) ? (pv == -1) : (pv >= 0 && pv < v);
        const int fl = p.node_flags[kv] | (ok ? 0 : TV_REQ_BAD_PARENT);
        if (fl) atomicOr(&sm.fflags, fl);
        p.node_flags[kv] = 0;
      }
      __syncthreads();
      if (t == 0) {
        // every flag raised on a row that was read (or a timeout) fails the request
        const int fl = sm.fflags;
        if (fl) {
          p.status[b] = fl;
          p.path_len[b] = 0;
        } else {
          int32_t* path = p.path + (size_t)b * p.n_max;
          int32_t* out = p.out_tokens + (size_t)b * p.n_max;
          int cur = 0, j = 0;
          path[0] = 0;
          for (;;) {
            const int ch = sm.facc[cur];
            if (ch <= cur || ch >= n || j + 1 >= n) break;
            out[j] = tok[ch];
            path[++j] = ch;
            cur = ch;
          }
          out[j] = sm.ffin[cur];
          p.path_len[b] = j + 1;
          p.status[b] = 0;
        }
        p.req_done[b] = 0;
      }
    }
    __syncthreads();
  }
}

// ===========================================================================
// host side
// ===========================================================================

int check_vdesc(const tv_verify_desc* d) {
  if (!d) return TV_ERR_INVALID_ARG;
  if (d->batch < 0 || d->vocab < 1) return TV_ERR_INVALID_ARG;
  if (d->n_max < 1 || d->n_max > kMaxNodes) return TV_ERR_UNSUPPORTED;
  if (!(d->temperature > 0.f) || !isfinite(d->temperature)) return TV_ERR_INVALID_ARG;
  return TV_OK;
}

struct VerifyLayout {
  size_t greedy_val, greedy_idx, greedy_bad, greedy_cnt, greedy_bytes;
  size_t tm, ts, tf, acc, fin, flg, arr, dep, req, stoch_bytes;
  int chunks, tiles;
};

VerifyLayout layout(const tv_verify_desc* d) {
  VerifyLayout L;
  const size_t nodes = (size_t)d->batch * d->n_max;
  L.chunks = (d->vocab + kGreedyChunk - 1) / kGreedyChunk;
  L.tiles = (d->vocab + kTileElems - 1) / kTileElems;
  size_t o = 0;
  L.greedy_val = o;
  o = tv_align_up(o + nodes * L.chunks * sizeof(float), 256);
  L.greedy_idx = o;
  o = tv_align_up(o + nodes * L.chunks * sizeof(int), 256);
  L.greedy_bad = o;
  o = tv_align_up(o + nodes * L.chunks * sizeof(int), 256);
  L.greedy_cnt = o;
  o = tv_align_up(o + (size_t)d->batch * sizeof(int), 256);
  L.greedy_bytes = o;
  o = 0;
  L.tm = o;
  o = tv_align_up(o + nodes * 2 * L.tiles * sizeof(float), 256);
  L.ts = o;
  o = tv_align_up(o + nodes * 2 * L.tiles * sizeof(double), 256);
  L.tf = o;
  o = tv_align_up(o + nodes * 3 * L.tiles * sizeof(double), 256);
  L.acc = o;
  o = tv_align_up(o + nodes * sizeof(int), 256);
  L.fin = o;
  o = tv_align_up(o + nodes * sizeof(int), 256);
  L.flg = o;
  o = tv_align_up(o + nodes * sizeof(int), 256);
  L.arr = o;
  o = tv_align_up(o + nodes * sizeof(int), 256);
  L.dep = o;
  o = tv_align_up(o + nodes * sizeof(int), 256);
  L.req = o;
  o = tv_align_up(o + (size_t)d->batch * sizeof(int), 256);
  L.stoch_bytes = o;
  return L;
}

int g_stoch_blocks_per_cu = -1;

}  // namespace

extern "C" size_t tree_verify_workspace_size(const tv_verify_desc* desc) {
  if (check_vdesc(desc) != TV_OK) return 0;
  VerifyLayout L = layout(desc);
  return L.greedy_bytes > L.stoch_bytes ? L.greedy_bytes : L.stoch_bytes;
}

extern "C" int tree_verify_greedy(const tv_verify_desc* desc, const float* target_logits,
                                  const int32_t* tokens, const int32_t* parent,
                                  const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* status, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!target_logits || !tokens || !parent || !n_nodes || !path || !path_len || !out_tokens || !status)
    return TV_ERR_INVALID_ARG;
  if (((uintptr_t)target_logits & 15) != 0) return TV_ERR_INVALID_ARG;
  VerifyLayout L = layout(desc);
  if (!workspace || workspace_bytes < L.greedy_bytes) return TV_ERR_WORKSPACE;
  GreedyParams p;
  p.logits = target_logits;
  p.tokens = tokens;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.path = path;
  p.path_len = path_len;
  p.out_tokens = out_tokens;
  p.status = status;
  p.part_val = (float*)((char*)workspace + L.greedy_val);
  p.part_idx = (int*)((char*)workspace + L.greedy_idx);
  p.part_bad = (int*)((char*)workspace + L.greedy_bad);
  p.counters = (int*)((char*)workspace + L.greedy_cnt);
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.V = desc->vocab;
  p.chunks = L.chunks;
  long long grid = (long long)desc->batch * desc->n_max * L.chunks;
  if (grid > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(greedy_kernel, dim3((unsigned)grid), dim3(kGreedyThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_verify_stochastic(const tv_verify_desc* desc, const float* target_logits,
                                      const float* draft_logits, const int32_t* tokens,
                                      const int32_t* parent, const int32_t* n_nodes,
                                      const float* u_accept, const float* u_sample, int32_t* path,
                                      int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!target_logits || !draft_logits || !tokens || !parent || !n_nodes || !u_accept || !u_sample ||
      !path || !path_len || !out_tokens || !status)
    return TV_ERR_INVALID_ARG;
  if ((((uintptr_t)target_logits | (uintptr_t)draft_logits) & 15) != 0) return TV_ERR_INVALID_ARG;
  VerifyLayout L = layout(desc);
  if (L.tiles > kMaxTiles) return TV_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.stoch_bytes) return TV_ERR_WORKSPACE;
  int cu = 0;
  rc = tv_device_cu_count(&cu);
  if (rc != TV_OK) return rc;
  if (g_stoch_blocks_per_cu < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stochastic_kernel, kVThreads, 0) != hipSuccess)
      return TV_ERR_HIP;
    g_stoch_blocks_per_cu = nb < 1 ? 1 : nb;
  }
  const long long capacity = (long long)g_stoch_blocks_per_cu * cu;
  const long long nodes = (long long)desc->batch * desc->n_max;
  // team size: enough members to fill the grid, at most one tile each, at most 16
  int S = 1;
  while (S * 2 <= 16 && S * 2 <= L.tiles && nodes * S * 2 <= capacity) S *= 2;
  long long slots = capacity / S;
  if (slots > nodes) slots = nodes;
  if (slots < 1) slots = 1;

  StochParams p;
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = tokens;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.u_accept = u_accept;
  p.u_sample = u_sample;
  p.path = path;
  p.path_len = path_len;
  p.out_tokens = out_tokens;
  p.status = status;
  char* ws = (char*)workspace;
  p.tile_m = (float*)(ws + L.tm);
  p.tile_s = (double*)(ws + L.ts);
  p.tile_f = (double*)(ws + L.tf);
  p.acc_child = (int*)(ws + L.acc);
  p.final_tok = (int*)(ws + L.fin);
  p.node_flags = (int*)(ws + L.flg);
  p.arrive = (int*)(ws + L.arr);
  p.depart = (int*)(ws + L.dep);
  p.req_done = (int*)(ws + L.req);
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.V = desc->vocab;
  p.tiles = L.tiles;
  p.S = S;
  p.slots = (int)slots;
  p.invT = 1.0f / desc->temperature;
  p.invT_d = 1.0 / (double)desc->temperature;
  void* args[] = {&p};
  hipError_t e = hipLaunchCooperativeKernel((const void*)stochastic_kernel, dim3((unsigned)(slots * S)),
                                            dim3(kVThreads), args, 0, stream);
  return e == hipSuccess ? TV_OK : TV_ERR_HIP;
}
