// Token-tree verification for gfx950.
//
// Workgroups hand values to one another only through 64-bit words read and
// written with agent-scope atomics (a word carries its own "written" or
// "complete" marks, so no ordering between different addresses is needed);
// everything else passes at kernel boundaries.  No workgroup issues a
// device-wide fence (on this part an agent-scope fence writes back and
// invalidates the XCD's whole L2).
//
// Both verifiers are one launch each (with a prepared workspace): the grid
// holds the per-node workgroups and then one workgroup per request that chases
// the accepted path.  Workgroups are dispatched in id order, so a chase
// workgroup takes a slot only after every per-node workgroup has one; it polls
// its request's published words (bounded) and clears them for the next call.
//
// Greedy ([guide] "Greedy Verification Algorithm"):
//   greedy_argmax_kernel  one workgroup per (node, 8192-logit chunk) reduces its
//                         chunk to one 64-bit key that orders by value, then by
//                         lower index (or a reserved value when the chunk holds
//                         a non-finite logit) and publishes it; the chase
//                         workgroups take each node's largest key, match
//                         children against the argmaxes and walk the root path.
//   greedy_chase_kernel   the same chase as a kernel of its own, for the static
//                         scratch of tree_verify_greedy_noalloc.
//
// Stochastic ([guide] "Stochastic Verification Algorithm"; [chapter] the
// min(1, p/q) acceptance rule and the residual max(p - q, 0) / Z):
//   stoch_node_kernel     a team of S workgroups per node, each member owning a
//                         slice of 4096-logit chunks: chunk maxima and sums of
//                         exp((z - max) / T) of the target row (and of the draft
//                         row for nodes with children), then for nodes with
//                         children the tests of the children in ascending id.
//                         At node u with children c_1, c_2, ... the residual
//                         after i rejections has the closed form
//                             p^(i)(w) = max(p(w) - C_i q(w), 0) / D_i,
//                             C_0 = 0, D_0 = 1, C_{i+1} = C_i + D_i,
//                             D_{i+1} = F(C_{i+1}),  F(c) = sum_w max(p(w) - c q(w), 0)
//                         (induction on the recursive residual, Z_{i+1} =
//                         F(C_{i+1}) / D_i; when F = 0 the residual is kept), so
//                         the accept test of c_{i+1} is
//                             u * q(x) * D_i <= max(p(x) - C_i q(x), 0)
//                         and a rejection costs one evaluation of F, split over
//                         the team.  Members publish float64 partials in 64-bit
//                         slots whose top bit marks them written, so a member
//                         waits only for its team's slots.  A member whose slice
//                         is at most two chunks keeps its exponentials on chip
//                         across rejections.  Each node also makes the draw it
//                         emits when no child is accepted: an inverse CDF over
//                         member masses, chunk masses, then one chunk.  Every
//                         member then ORs its part of the node's result into one
//                         64-bit word.  The chase workgroups read the words:
//                         status, the root path and its final token, and for
//                         verify-and-compact the accepted path's KV compaction
//                         ([guide] "Depth-First Flattening and KV Cache Reuse").
// Vocabulary exponentials are float32 (exp_t), as is each entry's residual
// bracket (residual_rel); sums, chunk factors and the accept test are float64.

#include "tv_common.h"
#include "tv_compact.h"

#include <math.h>
#include <mutex>

namespace {

constexpr int kMaxNodes = 128;
constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kGreedyThreads = 256;
constexpr int kGreedyChunk = kGreedyThreads * 32;   // 8192 logits per (node, chunk) unit

constexpr int kSThreads = 256;
constexpr int kChunk = kSThreads * 16;              // 4096 logits per chunk
constexpr int kMaxChunks = 128;                     // vocabulary up to 128 * 4096 = 524288
constexpr int kMaxTeam = 16;
constexpr int kResident = 2;                        // chunks a member holds in registers
constexpr long long kSpinLimit = 1LL << 19;         // bounded waits (~0.5 s), then TV_REQ_TIMEOUT
constexpr unsigned long long kWritten = 1ull << 63;  // marks a published exchange slot
constexpr int kPrioSteps = 3;                        // load-order classes: 0, 1, 2, 3+ children
constexpr long long kChaseSpinLimit = kSpinLimit << 2;   // a chase workgroup's bounded wait (~2 s)

// A verifier's workspace starts with the prepared-workspace header (kWsMagic,
// bytes cleared).  The verifiers' slots tell a published value from an empty
// one by their contents and every call leaves them at zero, so a workspace
// that was never initialised (or is too small for this call's layout) must
// not be used: such a request gets TV_REQ_BAD_WORKSPACE.

// Buffer resource over one logit row of V floats.  Buffer loads address the row
// with a 32-bit offset plus an immediate (one VGPR per batch of loads instead of a
// 64-bit address per load) and return 0 past the row's end instead of reading it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* row, int V) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, V * 4, 0x00020000);
}

// Issue the loads of 16 consecutive logits of one thread (elements past the
// row's end read as 0; callers mask them by index where the values are used).
// Nothing here consumes the data, so consecutive calls keep all their loads in
// flight together.  kVec: rows are 16-byte aligned (V a multiple of 4), so
// 16-byte loads are used and a 4-vector starting below V lies wholly inside
// the row.
template <bool kVec>
__device__ __forceinline__ void load16(__amdgpu_buffer_rsrc_t rs, int e0, float* x) {
  if (kVec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const tv_f32x4 a = __builtin_bit_cast(tv_f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * e0 + 16 * i, 0, 0));
      x[4 * i] = a[0];
      x[4 * i + 1] = a[1];
      x[4 * i + 2] = a[2];
      x[4 * i + 3] = a[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (e0 + i), 0, 0));
  }
}

// Children of u among nodes [1, n), ascending, written by one wave into kids[]
// with their tokens in ktok[]; returns the count to every lane (n <= 128: two
// ballots).  pv0 / pv1 and tk0 / tk1: parent and token of nodes 1 + l and
// 65 + l (parent -1 past the request).
__device__ __forceinline__ int collect_children(int pv0, int pv1, int tk0, int tk1, int u, int* kids, int* ktok) {
  const int l = threadIdx.x & 63;
  const bool k0 = pv0 == u, k1 = pv1 == u;
  const unsigned long long b0 = __ballot(k0), b1 = __ballot(k1);
  const unsigned long long below = (1ull << l) - 1ull;
  if (k0) {
    kids[__popcll(b0 & below)] = 1 + l;
    ktok[__popcll(b0 & below)] = tk0;
  }
  if (k1) {
    kids[__popcll(b0) + __popcll(b1 & below)] = 65 + l;
    ktok[__popcll(b0) + __popcll(b1 & below)] = tk1;
  }
  return __popcll(b0) + __popcll(b1);
}

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
  // [B][n_max][chunks] each chunk's largest (value, index) key, kGreedyBad when
  // the chunk holds NaN or +-inf, 0 while it is not written
  unsigned long long* keys;
  const unsigned long long* header;   // prepared workspace header (null: the static scratch)
  unsigned long long* header_w;       // the same, for invalidating it after an expired wait
  unsigned long long need;            // bytes this call's layout uses (header included)
  int B, n_max, V, chunks;
  int G;   // argmax workgroups; when the grid holds more, the B after them chase the paths
  long long chase_spin;   // polling rounds before a chase workgroup gives up (negative: at once)
};

// A chunk's slot when it holds a non-finite logit.  Every key of a finite
// value has its low word at 0x80000000 or above (index < 2^31), so neither 0
// nor this value is a key.
constexpr unsigned long long kGreedyBad = 1ull;

// Order-preserving key: larger value first, then lower index.  -0 and +0 tie.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// One (node, chunk) unit's logits held by a thread: 32 values, two runs of 16
// consecutive logits (elements lo + 16 t .. + 15 and lo + 4096 + 16 t .. + 15).
struct GreedyUnit {
  float x[32];
};

__device__ __forceinline__ int greedy_elem(int lo, int j) {
  return lo + 16 * (int)threadIdx.x + (j >= 16 ? 16 * kGreedyThreads + j - 16 : j);
}

template <bool kVec>
__device__ __forceinline__ void greedy_issue(const GreedyParams& p, int unit, GreedyUnit& u) {
  const int c = unit % p.chunks, k = unit / p.chunks;
  const __amdgpu_buffer_rsrc_t row = row_rsrc(p.logits + (size_t)k * p.V, p.V);
  const int e0 = c * kGreedyChunk + 16 * (int)threadIdx.x;
  load16<kVec>(row, e0, u.x);   // both halves issued before either is used
  load16<kVec>(row, e0 + 16 * kGreedyThreads, u.x + 16);
}

// Reduce a unit whose loads have been issued: the chunk's largest key and
// whether it holds a non-finite logit, written by thread 0 (`red` / `redbad`:
// one LDS slot per wave).
__device__ __forceinline__ void greedy_reduce(const GreedyParams& p, int unit, const GreedyUnit& x,
                                              unsigned long long* red, int* redbad, bool live) {
  const int c = unit % p.chunks;
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int lo = c * kGreedyChunk, hi = min(p.V, lo + kGreedyChunk);
  unsigned long long best = 0ull;
  if (live) {
    int bad = 0;
    if (hi - lo == kGreedyChunk) {
      // A full chunk: the largest value (three-input maxima), then the first of
      // the thread's entries (ascending index) that holds it; non-finite
      // entries are found by class.  With every entry finite the maximum is
      // exact and -0 / +0 compare equal, so this is the same key as below.
#pragma unroll
      for (int j = 0; j < 32; ++j) bad |= !isfinite(x.x[j]);
      const float m = fmaxf(tv_max16(x.x), tv_max16(x.x + 16));
      int jm = 31;
#pragma unroll
      for (int j = 30; j >= 0; --j) jm = x.x[j] == m ? j : jm;
      best = argmax_key(m, greedy_elem(lo, jm));
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int e = greedy_elem(lo, j);
        if (e < hi) {
          bad |= !isfinite(x.x[j]);
          const unsigned long long kx = argmax_key(x.x[j], e);
          best = kx > best ? kx : best;
        }
      }
    }
    best = tv_wave_max_u64(best);
    const bool anybad = __ballot(bad != 0) != 0ull;
    if (l == 0) {
      red[w] = best;
      redbad[w] = anybad ? 1 : 0;
    }
  }
  tv_lds_barrier();
  if (live && t == 0) {
    int fl = redbad[0];
    for (int i = 1; i < kGreedyThreads / 64; ++i) {
      best = red[i] > best ? red[i] : best;
      fl |= redbad[i];
    }
    const size_t k = (size_t)(unit / p.chunks);
    __hip_atomic_store(p.keys + k * p.chunks + c, fl ? kGreedyBad : best, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct GreedyChaseSmem {
  int arg[kMaxNodes], child[kMaxNodes], tok[kMaxNodes];
  int badpar, nonfinite, timeout;
};

__device__ __forceinline__ bool greedy_ws_ok(const GreedyParams& p) {
  if (!p.header) return true;
  const unsigned long long magic = p.header[0], bytes = p.header[1];   // both loads at once
  return (magic == kWsMagic) & (bytes >= p.need);
}

// The greedy chase of request b by one workgroup of at least kMaxNodes
// threads: each node's argmax (the largest of its chunks' keys), each node's
// first child whose token equals it, and the path from the root.  kPoll: the
// argmax workgroups of the same grid may still be running; thread t waits
// (bounded) until every chunk slot of node t is written and clears the slots
// it read for the next call.  Otherwise the slots were all written before this
// kernel started (and are overwritten by the next call).
template <bool kPoll>
__device__ void greedy_chase(const GreedyParams& p, GreedyChaseSmem& sm, int b) {
  const int t = threadIdx.x;
  const int32_t* par = p.parent + (size_t)b * p.n_max;
  const int32_t* tok = p.tokens + (size_t)b * p.n_max;
  const size_t kv = (size_t)b * p.n_max + t;
  const int n = p.n_nodes[b];
  const bool wsok = greedy_ws_ok(p);
  int pv = -1, tk = 0, flg = 0;
  if (t < p.n_max) {
    pv = par[t];
    tk = tok[t];
  }
  const bool mine = wsok && n >= 1 && n <= p.n_max && t < n;
  unsigned long long key = 0ull;
  bool done = true;
  if (mine) {
    unsigned long long* kp = p.keys + kv * p.chunks;
    for (int c0 = 0; c0 < p.chunks; c0 += 16) {
      unsigned long long kc[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) kc[c] = 0ull;
      if (kPoll && p.chase_spin < 0) {
        done = false;
        break;
      }
      for (long long it = 0;; ++it) {
        bool all = true;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          if (c0 + c < p.chunks && kc[c] == 0ull)
            kc[c] = kPoll ? __hip_atomic_load(kp + c0 + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kp[c0 + c];
          all = all && (c0 + c >= p.chunks || kc[c] != 0ull);
        }
        if (!kPoll || all) break;
        if (it >= p.chase_spin) {
          done = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        key = kc[c] > key ? kc[c] : key;
        flg |= kc[c] == kGreedyBad;
      }
      if (!done) break;
    }
    if (kPoll) {
      // A complete node's slots are cleared for the next call.  A node whose
      // slots were not all written in time may still be written: the
      // workspace header is invalidated instead, so that later calls report
      // TV_REQ_BAD_WORKSPACE until the workspace is prepared again.
      if (done) {
        for (int c = 0; c < p.chunks; ++c) kp[c] = 0ull;
      } else {
        p.header_w[0] = 0;
      }
    }
  }
  int st = 0;
  if (n < 1 || n > p.n_max) st = TV_REQ_BAD_NNODES;
  else if (!wsok) st = TV_REQ_BAD_WORKSPACE;
  if (st) {
    if (t == 0) {
      p.status[b] = st;
      p.path_len[b] = 0;
    }
    return;
  }
  if (t == 0) {
    sm.badpar = 0;
    sm.nonfinite = 0;
    sm.timeout = 0;
  }
  __syncthreads();
  if (t < n) {
    sm.arg[t] = (int)(0xFFFFFFFFu - (uint32_t)key);
    sm.child[t] = 0x7fffffff;
    sm.tok[t] = tk;
    if (flg) sm.nonfinite = 1;
    if (!done) sm.timeout = 1;
    if (!((t == 0) ? (pv == -1) : (pv >= 0 && pv < t))) sm.badpar = 1;
  }
  __syncthreads();
  const int fl = sm.badpar ? TV_REQ_BAD_PARENT
                           : (sm.timeout ? TV_REQ_TIMEOUT : (sm.nonfinite ? TV_REQ_NONFINITE : 0));
  if (fl == 0 && t >= 1 && t < n) {
    if (tk == sm.arg[pv]) atomicMin(&sm.child[pv], t);
  }
  __syncthreads();
  if (t == 0) {
    int len = 0;
    if (!fl) {
      int32_t* path = p.path + (size_t)b * p.n_max;
      int32_t* out = p.out_tokens + (size_t)b * p.n_max;
      int cur = 0, j = 0;
      path[0] = 0;
      while (sm.child[cur] != 0x7fffffff && j + 1 < n) {
        const int ch = sm.child[cur];
        out[j] = sm.tok[ch];
        path[++j] = ch;
        cur = ch;
      }
      out[j] = sm.arg[cur];
      len = j + 1;
    }
    p.status[b] = fl;
    p.path_len[b] = len;
  }
}

// One workgroup per (node, chunk) unit, and (when the grid holds more than the
// G units) one per request after them that chases its path.  In-order dispatch
// places the chase workgroups only after every unit has a slot.  Units of
// nodes past the request's size load nothing (the size is read before the
// row: a grid with many dead units, such as a batch of short chains padded to
// n_max, would otherwise stream their rows for nothing).  (A persistent grid
// with two units in flight per workgroup measured slower: 57.7 against 48.1 us
// for 512 nodes x 128256 logits.)
template <bool kVec>
__global__ __launch_bounds__(kGreedyThreads) void greedy_argmax_kernel(GreedyParams p) {
  __shared__ union {
    struct {
      unsigned long long red[kGreedyThreads / 64];
      int bad[kGreedyThreads / 64];
    } a;
    GreedyChaseSmem c;
  } sm;
  const int unit = blockIdx.x;
  const int k = unit / p.chunks;
  const int n = p.n_nodes[min(k / p.n_max, p.B - 1)];   // clamped for chase workgroups
  if (unit >= p.G) {
    greedy_chase<true>(p, sm.c, unit - p.G);
    return;
  }
  if (n > p.n_max || k % p.n_max >= n) return;
  GreedyUnit x;
  greedy_issue<kVec>(p, unit, x);
  greedy_reduce(p, unit, x, sm.a.red, sm.a.bad, true);
}

// The chase as a kernel of its own, after the argmax kernel (the static
// scratch of tree_verify_greedy_noalloc, which no call prepares).
__global__ __launch_bounds__(kMaxNodes) void greedy_chase_kernel(GreedyParams p) {
  __shared__ GreedyChaseSmem sm;
  greedy_chase<false>(p, sm, blockIdx.x);
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
  const unsigned long long* header;   // [2]: kWsMagic, bytes zero-filled by tree_verify_workspace_init
  unsigned long long* header_w;       // the same, for invalidating it after an expired wait
  unsigned long long need;            // bytes this call's layout uses (header included)
  unsigned long long* xch;   // [nodes][kMaxTeam]    member masses after child `node` is rejected
  unsigned long long* sxch;  // [nodes][chunks][4] chunk (max, sum) of the target and draft rows
  unsigned long long* nword; // [nodes]  the node's result (see kNw*), zero between calls
  int prio_ticks;            // load delay per missing child below kPrioSteps, 100 MHz ticks (0: none)
  int xcd_teams;             // 1: the whole grid is resident; a team's members share an XCD
  int B, n_max, V, chunks, S, per;   // per = chunks per team member
  float k2hi, k2lo;                  // log2(e) / T as a float32 head and tail
  double invT_d;
  int G;            // node workgroups; the B workgroups after them chase the paths
  int chase_mode;   // kChaseOnly, or the chase then the KV compaction of cpt
  long long chase_spin;   // polling rounds before a chase workgroup gives up (negative: at once)
  TvCompactArgs cpt;
};

// What the workgroups that follow the node workgroups do for their request:
// walk the path, or walk it and then compact the request's KV along it (bf16
// or float32 caches).
enum { kChaseOnly = 0, kChaseCompactBf16 = 1, kChaseCompactF32 = 2 };


// A node's result word, assembled by its team with one atomic OR per member:
// the draw made when no child is accepted (bits 0-31, from the member that
// owns it), the accepted child + 1 (bits 32-39, member 0), the node's status
// flags (bits 40-47, any member) and one bit per member that has finished
// (bits 48-63).  The word is complete once every member's bit is set.
constexpr int kNwAccShift = 32, kNwFlagShift = 40, kNwDoneShift = 48;

__device__ __forceinline__ bool ws_ok(const StochParams& p) {
  const unsigned long long magic = p.header[0], bytes = p.header[1];   // both loads at once
  return (magic == kWsMagic) & (bytes >= p.need);
}

// exp(d / T) for d <= 0 in float32: exp2 of d * log2(e) / T, with the product
// carried as head + tail (the tail from an exact fma residual) so that rounding
// the exponent does not cost accuracy.  Exponents below -150 give 0; a NaN or
// infinite d gives NaN (callers detect non-finite logits from the sums).
__device__ __forceinline__ float exp_t(float d, float k2hi, float k2lo) {
  const float h = d * k2hi;
  const float lo = fmaf(d, k2hi, -h) + d * k2lo;
  const float r = __builtin_amdgcn_exp2f(h);
  return fmaf(r, lo * 0.693147180559945309f, r);
}

// Weight of one vocabulary entry under max(p - c q, 0).  ep / eq are the
// float32 exponentials exp((z - m) / T) relative to the entry's chunk maxima of
// the target / draft row, and a = exp((m - M) / T) / S, b the same factor of the
// draft row, turn them into p and q.  So max(p - c q, 0) = a max(ep - rho eq, 0)
// with rho = c b / a for the whole chunk: the bracket is taken in float32 (one
// fma and one max per entry) and scaled by a in float64 once per thread.
__device__ __forceinline__ float residual_rel(float ep, float eq, float rho) {
  return fmaxf(fmaf(eq, -rho, ep), 0.f);
}

// rho of a chunk from b and ia = 1 / a (0 for a chunk whose target mass a
// underflowed: its weights are 0).
__device__ __forceinline__ float chunk_rho(double ia, double b, double c) {
  return (float)(c * b * ia);
}

// LDS of a request's chase.
struct ChaseSmem {
  int acc[kMaxNodes], fin[kMaxNodes], tok[kMaxNodes], path[kMaxNodes];
  int flags, badpar, len, bad;
};

constexpr int kStagedBlocks = kMaxNodes / 16 + 2;   // blocks holding n <= 128 positions (block size >= 16)

// A chase workgroup's LDS (it shares the node kernel's): the chase's arrays,
// and for the compaction the block-table entries it reads while it waits.
struct ChaseTailSmem {
  ChaseSmem c;
  int first_bad;
  int stage[kStagedBlocks];
};

template <bool kRes>
struct NodeSmem {
  static constexpr int MM = kRes ? kResident : kMaxChunks;   // chunks per member
  static constexpr int MC = kRes ? kMaxTeam * kResident : kMaxChunks;   // chunks of a row
  float red_f[kSThreads / 64][2 * kResident];   // per-wave maxima of a batch (chunk, row)
  double red_d[kSThreads / 64][2 * kResident];  // per-wave exponential sums of a batch
  float cm[2][MM];        // this member's chunk maxima (target, draft)
  double cs[2][MM];       // ... chunk sums of exp((z - chunk max) / T)
  double ca[2][MC];       // every chunk's factor exp((m - M) / T) / S (target, draft)
  double sc[MC];          // every chunk's target sum of exp((z - m) / T)
  double ia[MC];          // 1 / ca[0][c] (0 where ca[0][c] is 0)
  double part[kSThreads / 64][MM];   // per-wave residual sums of this member's chunks
  double rcur[MM];        // ... of the current residual
  double xcur[kMaxTeam];  // ... of the current residual
  double rowS[2];         // team exponential sums relative to the team maxima
  double Fx;              // team residual mass of the latest rejection
  double scan[kSThreads / 64];
  int wcross[kSThreads / 64], wlast[kSThreads / 64];   // per wave: first crossing lane, last lane with mass
  int kids[kMaxNodes], ktok[kMaxNodes];
  float kzp[kMaxNodes], kzq[kMaxNodes], kua[kMaxNodes];   // per child: logits of its token, its uniform
  double kpx[kMaxNodes], kqx[kMaxNodes];                   // ... and p(x), q(x) of that token
  int nk, bad, badtok, timeout, owner, sel, res_tok;
  double base, thr;
  // draft exponentials of the resident slice, [chunk][group of 4][thread]
  tv_f32x4 qe[kRes ? kResident * 4 * kSThreads : 1];
};

// Sum of 16 doubles, pairwise.
__device__ __forceinline__ double sum16_d(const double* x) {
  double a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] += a[i + 4];
  return (a[0] + a[2]) + (a[1] + a[3]);
}

// Sum of 16 floats, pairwise.
__device__ __forceinline__ float sum16(const float* x) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] += a[i + 4];
  return (a[0] + a[2]) + (a[1] + a[3]);
}

// Statistics of a batch of up to kResident chunks of the target row (and of the
// draft row when `both`): every chunk's maximum m and sum of exp((z - m) / T)
// over the workgroup, stored at local chunk index j0 + r.  The thread's logits
// are replaced by those exponentials.  Units (row, chunk) are taken in the order
// their loads were issued, each as soon as its own data has arrived.  Only the
// thread holding the row's end masks entries; elsewhere the 16 entries run
// without per-entry tests.  A non-finite logit makes its thread's sum NaN (the
// maximum skips NaN; NaN, +inf and -inf all reach a NaN exponential), which
// sets sm.bad.
template <bool kRes>
__device__ void batch_stats(NodeSmem<kRes>& sm, float (&xp)[kResident][16], float (&xq)[kResident][16], int nb,
                            bool both, int my_c0, int j0, int V, float k2hi, float k2lo) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  int bad = 0;
#pragma unroll
  for (int row = 0; row < 2; ++row) {
#pragma unroll
    for (int r = 0; r < kResident; ++r) {
      if (r < nb && (row == 0 || both)) {
        float* x = row ? xq[r] : xp[r];
        const int nv = V - ((my_c0 + j0 + r) * kChunk + 16 * t);   // entries of this thread inside the row
        float m;
        if (nv >= 16) {
          m = tv_max16(x);
        } else {
          m = kNegInf;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (e < nv) m = fmaxf(m, x[e]);
        }
        m = tv_wave_max(m);
        if (l == 0) sm.red_f[w][2 * r + row] = m;
        tv_lds_barrier();
        m = sm.red_f[0][2 * r + row];
        for (int i = 1; i < kSThreads / 64; ++i) m = fmaxf(m, sm.red_f[i][2 * r + row]);
        if (nv >= 16) {
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] = exp_t(x[e] - m, k2hi, k2lo);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] = e < nv ? exp_t(x[e] - m, k2hi, k2lo) : 0.f;
        }
        const float st = sum16(x);
        bad |= !isfinite(st);
        const double sw = tv_wave_sum_d((double)st);
        if (l == 0) sm.red_d[w][2 * r + row] = sw;
        if (t == 0) sm.cm[row][j0 + r] = m;
      }
    }
  }
  if (__ballot(bad != 0) != 0ull && l == 0) sm.bad = 1;
  tv_lds_barrier();
  if (t < 2 * nb) {
    double s = 0.0;
    for (int i = 0; i < kSThreads / 64; ++i) s += sm.red_d[i][t];
    sm.cs[t & 1][j0 + (t >> 1)] = s;
  }
  tv_lds_barrier();   // the next batch may overwrite red_f / red_d
}

// Publish one 64-bit word in slot `slot` (top bit marks it written).
__device__ __forceinline__ void xch_put(unsigned long long* slot, unsigned long long bits) {
  __hip_atomic_store(slot, bits | kWritten, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for a published slot (bounded); returns its payload, 0 after a timeout.
__device__ __forceinline__ unsigned long long xch_get(unsigned long long* slot, int* timeout) {
  unsigned long long v;
  long long it = 0;
  while (((v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & kWritten) == 0ull) {
    if (++it > kSpinLimit) {
      *timeout = 1;
      return 0ull;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return v & ~kWritten;
}

// Wait for up to N published slots at once (those with need[i]): every round
// re-reads all slots still missing with loads issued together, so the wait
// costs one round trip, not one per slot.  Payloads in v (0 after a timeout or
// when not needed).
template <int N>
__device__ __forceinline__ void xch_get_n(unsigned long long* const (&slot)[N], const bool (&need)[N],
                                          unsigned long long (&v)[N], int* timeout) {
  bool done[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    v[i] = 0ull;
    done[i] = !need[i];
  }
  for (long long it = 0;; ++it) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!done[i]) v[i] = __hip_atomic_load(slot[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (!done[i]) done[i] = (v[i] & kWritten) != 0ull;
      all = all && done[i];
    }
    if (all) break;
    if (it > kSpinLimit) {
      *timeout = 1;
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (!done[i]) v[i] = 0ull;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] &= ~kWritten;
}

// Inverse CDF inside one chunk: the smallest index whose running mass (from
// `base`) exceeds thr.  The thread ranges come from a wave scan of the
// per-thread sums and the waves' totals; the first thread with mass whose
// range ends past thr (found by ballots) walks its 16 weights.  When rounding
// leaves no such thread, or no weight of that thread crosses, the last
// positive weight at or before it is taken.  w: this thread's 16 weights.
// Returns the index to every thread.
template <class Smem>
__device__ int chunk_draw(Smem& sm, const double (&w)[16], int e0, double base, double thr, int fallback) {
  constexpr int NW = kSThreads / 64;
  const int t = threadIdx.x, wv = t >> 6, ln = t & 63;
  double loc;
  {
    double a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = w[2 * j] + w[2 * j + 1];
    loc = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  }
  const double incl = tv_wave_incl_scan_d(loc, ln);
  if (ln == 63) sm.scan[wv] = incl;
  tv_lds_barrier();
  double off = base;   // mass before this wave
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < wv) off += sm.scan[i];
  const double lo = off + (incl - loc);   // mass before this thread
  const uint64_t cross = __ballot(loc > 0.0 && lo + loc > thr), pos = __ballot(loc > 0.0);
  if (ln == 0) {
    sm.wcross[wv] = cross ? __builtin_ctzll(cross) : -1;
    sm.wlast[wv] = pos ? 63 - __builtin_clzll(pos) : -1;
  }
  tv_lds_barrier();
  int ct = -1;
#pragma unroll
  for (int i = NW - 1; i >= 0; --i)
    if (sm.wcross[i] >= 0) ct = 64 * i + sm.wcross[i];
  if (ct < 0) {
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (sm.wlast[i] >= 0) ct = 64 * i + sm.wlast[i];
  }
  if (ct < 0) return fallback;   // no mass in the chunk
  if (t == ct) {
    double run = lo;
    int found = -1, lastw = -1;
    for (int j = 0; j < 16; ++j) {
      run += w[j];
      if (w[j] > 0.0) {
        lastw = e0 + j;
        if (run > thr) {
          found = e0 + j;
          break;
        }
      }
    }
    sm.res_tok = found >= 0 ? found : lastw;
  }
  tv_lds_barrier();
  return sm.res_tok;
}

// First index of m[0..count) (in order, count <= 128) whose running sum from
// *base exceeds thr, with the running sum before it in *base; the last
// positive entry (0 when none) and the full sum when rounding leaves none.
// One wave, 64 entries per scan; every lane gets the result.
__device__ int wave_select_mass(const double* m, int count, double thr, double* base, int lane) {
  double b0 = *base;
  int lastpos = 0;
  for (int h0 = 0; h0 < count; h0 += 64) {
    const int i = h0 + lane;
    const double x = i < count ? m[i] : 0.0;
    const double incl = tv_wave_incl_scan_d(x, lane);
    const uint64_t hit = __ballot(i < count && b0 + incl > thr);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      *base = b0 + tv_readlane_d(incl - x, f);
      return h0 + f;
    }
    const uint64_t pos = __ballot(i < count && x > 0.0);
    if (pos) lastpos = h0 + 63 - __builtin_clzll(pos);
    b0 += tv_readlane_d(incl, 63);
  }
  *base = b0;
  return lastpos;
}

// What the chase reads of request b, one entry per thread (thread t < n holds
// node t's): its flags, accepted child and draw (from the node's result word),
// token and parent; done: the word was complete.
struct ChaseLoads {
  int fl, acc, fin, tk, pv, n;
  bool ws_ok, done;
};

// Issues the loads of request b's rows at once (rows are n_max long; entries
// past n are not used), then polls the result words of nodes 0 .. n-1 until
// every member of each node has ORed its part (at most p.chase_spin rounds; a
// negative limit polls none).  A word still incomplete when the wait expires
// is flagged TV_REQ_TIMEOUT and left as it is.
__device__ __forceinline__ ChaseLoads chase_gather(const StochParams& p, int b) {
  const int t = threadIdx.x;
  const size_t kv = (size_t)b * p.n_max + t;
  ChaseLoads c{0, -1, 0, 0, -1, 0, ws_ok(p), true};
  c.n = p.n_nodes[b];
  if (t < p.n_max) {
    c.tk = p.tokens[kv];
    c.pv = p.parent[kv];
  }
  const bool mine = c.ws_ok && c.n >= 1 && c.n <= p.n_max && t < c.n;
  const unsigned long long full = ((1ull << p.S) - 1ull) << kNwDoneShift;
  unsigned long long wv = 0;
  bool done = !mine;
  for (long long it = 0; p.chase_spin >= 0; ++it) {
    if (!done) {
      wv = __hip_atomic_load(p.nword + kv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done = (wv & full) == full;
    }
    if (__all(done) || it >= p.chase_spin) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (mine) {
    c.done = done;
    c.fl = (int)((wv >> kNwFlagShift) & 0xffu) | (done ? 0 : TV_REQ_TIMEOUT);
    c.acc = (int)((wv >> kNwAccShift) & 0xffu) - 1;
    c.fin = (int)(uint32_t)wv;
  }
  return c;
}

// The chase of request b by the whole workgroup (any size of at least
// kMaxNodes threads), from its entries in c: status, the accepted path and its
// final token, and the request's result words cleared for the next call.
// Returns (to every thread) the length of the path written, 0 when the request
// failed; the path is also left in sm.path.
__device__ int chase_request(const StochParams& p, ChaseSmem& sm, int b, const ChaseLoads& c) {
  const int t = threadIdx.x;
  const size_t kv = (size_t)b * p.n_max + t;
  const int n = c.n;
  // status and path_len are written once, by thread 0, at the end
  int st = 0;
  if (n < 1 || n > p.n_max) st = TV_REQ_BAD_NNODES;
  else if (!c.ws_ok) st = TV_REQ_BAD_WORKSPACE;   // nothing of the workspace is trusted, read or cleared
  if (st) {
    if (t == 0) {
      p.status[b] = st;
      p.path_len[b] = 0;
    }
    return 0;
  }
  if (t == 0) {
    sm.flags = 0;
    sm.badpar = 0;
  }
  __syncthreads();
  if (t < n) {
    // A complete word is cleared for the next call.  An incomplete one (its
    // team's waits expired) may still be ORed: the workspace header is
    // invalidated instead, so that later calls report TV_REQ_BAD_WORKSPACE
    // until the workspace is prepared again.
    if (c.done) p.nword[kv] = 0;
    else p.header_w[0] = 0;
    if (c.fl) atomicOr(&sm.flags, c.fl);
    sm.acc[t] = c.acc;
    sm.fin[t] = c.fin;
    sm.tok[t] = c.tk;
    if (!((t == 0) ? (c.pv == -1) : (c.pv >= 0 && c.pv < t))) sm.badpar = 1;
  }
  __syncthreads();
  if (t == 0) {
    st = sm.badpar ? TV_REQ_BAD_PARENT : sm.flags;
    int len = 0;
    if (!st) {
      int32_t* path = p.path + (size_t)b * p.n_max;
      int32_t* out = p.out_tokens + (size_t)b * p.n_max;
      int cur = 0, j = 0;
      path[0] = 0;
      sm.path[0] = 0;
      for (;;) {
        const int ch = sm.acc[cur];
        if (ch <= cur || ch >= n || j + 1 >= n) break;
        out[j] = sm.tok[ch];
        ++j;
        path[j] = ch;
        sm.path[j] = ch;
        cur = ch;
      }
      out[j] = sm.fin[cur];
      len = j + 1;
    }
    p.status[b] = st;
    p.path_len[b] = len;
    sm.len = len;
  }
  __syncthreads();
  return sm.len;
}


// What one member contributes to its node's result word (thread 0's copy is used).
struct NodeOut {
  int flags, acc, tok;
  bool drew;
};

// The work of member `member` of node k (request b, node u < n) up to its
// contribution to the node's result.
template <bool kRes, bool kVec>
__device__ __forceinline__ void node_body(const StochParams& p, NodeSmem<kRes>& sm, int k, int member, int b, int u,
                                          int n, int4 rows, NodeOut& o) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int my_c0 = min(member * p.per, p.chunks);
  const int nmine = min(my_c0 + p.per, p.chunks) - my_c0;   // at most kResident when kRes
  const float* zp_row = p.target + (size_t)k * p.V;
  const float* zq_row = p.draft + (size_t)k * p.V;
  const __amdgpu_buffer_rsrc_t zp_rs = row_rsrc(zp_row, p.V), zq_rs = row_rsrc(zq_row, p.V);

  // first batch of the slice: the target at once, the draft as soon as one
  // ballot over the parent row (read with the request's size, ahead of the
  // slice) shows that u has children.  rows: parent[1 + l], parent[65 + l] and
  // (wave 0) the tokens of those nodes, -1 / 0 past n.
  const int pv0 = rows.x, pv1 = rows.y;
  const int tk0 = rows.z, tk1 = rows.w;   // tokens, for the children's accept tests
  const float us = p.u_sample[k];
  float ep[kResident][16], eq[kResident][16];
  if (p.prio_ticks > 0) {
    // The whole grid is resident and every member's loads share HBM: a node with
    // fewer children (a shorter chain of rejections after its loads) issues its
    // loads later, so the rows of nodes with longer chains arrive first.  Timed
    // on the 100 MHz real-time counter.
    const int nkc = __popcll(__ballot(pv0 == u)) + __popcll(__ballot(pv1 == u));
    // the same order for instruction issue among the waves sharing a SIMD
    if (nkc >= 2)
      __builtin_amdgcn_s_setprio(2);
    else if (nkc == 1)
      __builtin_amdgcn_s_setprio(1);
    if (nkc < kPrioSteps) {
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      const unsigned long long d = (unsigned long long)p.prio_ticks * (unsigned long long)(kPrioSteps - nkc);
      while (__builtin_amdgcn_s_memrealtime() - t0 < d) __builtin_amdgcn_s_sleep(8);
    }
  }
#pragma unroll
  for (int r = 0; r < kResident; ++r)
    if (r < nmine) load16<kVec>(zp_rs, (my_c0 + r) * kChunk + 16 * t, ep[r]);
  const bool internal = (__ballot(pv0 == u) | __ballot(pv1 == u)) != 0ull;
  if (internal) {
#pragma unroll
    for (int r = 0; r < kResident; ++r)
      if (r < nmine) load16<kVec>(zq_rs, (my_c0 + r) * kChunk + 16 * t, eq[r]);
  }
  // wave 0: the children, and the logits and uniforms their accept tests read
  // (issued now, behind the slice's loads, so they arrive with them instead of
  // a round trip after the statistics)
  // (children past the first 64 are read after the statistics)
  float kzp_v = 0.f, kzq_v = 0.f, kua_v = 0.f;
  int badtok = 0;
  if (w == 0) {
    const int c = collect_children(pv0, pv1, tk0, tk1, u, sm.kids, sm.ktok);
    if (l == 0) {
      sm.nk = c;
      sm.bad = 0;
      sm.badtok = 0;
      sm.timeout = 0;
    }
    if (l < c) {
      const int x = sm.ktok[l];
      badtok = x < 0 || x >= p.V;
      const int xs = badtok ? 0 : x;
      kzp_v = zp_row[xs];
      kzq_v = zq_row[xs];
      kua_v = p.u_accept[(size_t)b * p.n_max + sm.kids[l]];
    }
  }
  // the children and the flags above are read by every wave (also when this
  // member's slice is empty and the statistics below run no barrier)
  tv_lds_barrier();

  // chunk statistics of this member's slice (batch_stats synchronises first)
  for (int j0 = 0; j0 < nmine; j0 += kResident) {
    if (j0 > 0) {
#pragma unroll
      for (int r = 0; r < kResident; ++r) {
        const int e0 = (my_c0 + min(j0 + r, nmine - 1)) * kChunk + 16 * t;
        load16<kVec>(zp_rs, e0, ep[r]);
        if (internal) load16<kVec>(zq_rs, e0, eq[r]);
      }
    }
    batch_stats(sm, ep, eq, min(kResident, nmine - j0), internal, my_c0, j0, p.V, p.k2hi, p.k2lo);
  }
  if (kRes && internal) {   // each thread later reads back only its own entries
#pragma unroll
    for (int r = 0; r < kResident; ++r)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        sm.qe[(r * 4 + g) * kSThreads + t] = tv_f32x4{eq[r][4 * g], eq[r][4 * g + 1], eq[r][4 * g + 2], eq[r][4 * g + 3]};
  }
  // From here on each step waits on the team: the waves issue ahead of the
  // statistics of workgroups still streaming their slices.
  __builtin_amdgcn_s_setprio(3);
  // publish this member's chunk statistics at once: words (m, s) of the target
  // row, then of the draft row, per chunk (a non-finite logit has made its
  // chunk's s NaN, which the team sums carry to every member)
  unsigned long long* sx = p.sxch + (size_t)k * p.chunks * 4;
  for (int i = t; i < 4 * nmine; i += kSThreads) {
    const int j = i >> 2, row = (i >> 1) & 1;
    if (row == 0 || internal)
      xch_put(sx + (size_t)(my_c0 + j) * 4 + (i & 3),
              (i & 1) ? (unsigned long long)__double_as_longlong(sm.cs[row][j]) : (unsigned long long)__float_as_uint(sm.cm[row][j]));
  }
  const int nk = sm.nk;
  if (t < nk) {
    if (t < 64) {
      sm.kzp[t] = kzp_v;
      sm.kzq[t] = kzq_v;
      sm.kua[t] = kua_v;
    } else {
      const int x = sm.ktok[t];
      badtok = x < 0 || x >= p.V;
      const int xs = badtok ? 0 : x;
      sm.kzp[t] = zp_row[xs];
      sm.kzq[t] = zq_row[xs];
      sm.kua[t] = p.u_accept[(size_t)b * p.n_max + sm.kids[t]];
    }
  }
  if (sm.bad) o.flags |= TV_REQ_NONFINITE;
  if (badtok) sm.badtok = 1;
  tv_lds_barrier();   // kzp / kzq / kua, badtok
  if (sm.badtok) {   // the request fails
    o.flags |= TV_REQ_BAD_TOKEN;
    return;
  }
  // Team statistics from every chunk's words: wave 0 the target row, wave 1 the
  // draft row (lanes take chunks l and l + 64): the row maximum M, the sum
  // S = sum_c s_c exp((m_c - M) / T) and each chunk's factor exp((m_c - M) / T) / S.
  // All members combine the same words in the same order, so they agree exactly.
  // Beside them, the lanes of the children (threads 128 + i) take the
  // exponentials of their tokens' logits relative to the maxima of the chunks
  // that hold them, so that p(x) and q(x) need one product after the barrier.
  if (w < 2 && (w == 0 || internal)) {
    unsigned long long* const sl[4] = {sx + (size_t)l * 4 + 2 * w, sx + (size_t)l * 4 + 2 * w + 1,
                                       sx + (size_t)(l + 64) * 4 + 2 * w, sx + (size_t)(l + 64) * 4 + 2 * w + 1};
    const bool nd[4] = {l < p.chunks, l < p.chunks, l + 64 < p.chunks, l + 64 < p.chunks};
    unsigned long long v[4];
    xch_get_n(sl, nd, v, &sm.timeout);
    const float m0 = nd[0] ? __uint_as_float((uint32_t)v[0]) : kNegInf;
    const float m1 = nd[2] ? __uint_as_float((uint32_t)v[2]) : kNegInf;
    const double s0 = __longlong_as_double((long long)v[1]), s1 = __longlong_as_double((long long)v[3]);
    const float M = tv_wave_max(fmaxf(m0, m1));
    const double e0 = l < p.chunks ? exp(((double)m0 - (double)M) * p.invT_d) : 0.0;
    const double e1 = l + 64 < p.chunks ? exp(((double)m1 - (double)M) * p.invT_d) : 0.0;
    const double S = tv_wave_sum_d(s0 * e0 + s1 * e1);
    const double iS = 1.0 / S;
    if (l < p.chunks) {
      const double a = e0 * iS;
      sm.ca[w][l] = a;
      if (w == 0) {
        sm.sc[l] = s0;
        sm.ia[l] = a > 0.0 ? 1.0 / a : 0.0;
      }
    }
    if (l + 64 < p.chunks) {
      const double a = e1 * iS;
      sm.ca[w][l + 64] = a;
      if (w == 0) {
        sm.sc[l + 64] = s1;
        sm.ia[l + 64] = a > 0.0 ? 1.0 / a : 0.0;
      }
    }
    if (l == 0) sm.rowS[w] = S;
  }
  const int ci = t - 2 * 64;   // every child's test operands at once
  const bool child_t = ci >= 0 && ci < nk;
  double ekp = 0.0, ekq = 0.0;
  int kc = 0;
  if (child_t) {
    kc = sm.ktok[ci] / kChunk;
    unsigned long long* const sl[2] = {sx + (size_t)kc * 4, sx + (size_t)kc * 4 + 2};
    const bool nd[2] = {true, internal};
    unsigned long long v[2];
    xch_get_n(sl, nd, v, &sm.timeout);
    ekp = exp(((double)sm.kzp[ci] - (double)__uint_as_float((uint32_t)v[0])) * p.invT_d);
    if (internal) ekq = exp(((double)sm.kzq[ci] - (double)__uint_as_float((uint32_t)v[1])) * p.invT_d);
  }
  tv_lds_barrier();
  const double Sp = sm.rowS[0], Sq = sm.rowS[1];
  if (!isfinite(Sp) || (internal && !isfinite(Sq))) return;   // some member saw a non-finite logit
  if (!internal && t < p.chunks) sm.ca[1][t] = 0.0;
  if (child_t) {   // p(x) = exp((z - m_c) / T) exp((m_c - M) / T) / S
    sm.kpx[ci] = ekp * sm.ca[0][kc];
    sm.kqx[ci] = internal ? ekq * sm.ca[1][kc] : 0.0;
  }
  tv_lds_barrier();

  // children in ascending id, one team-wide evaluation of F per rejection
  double Cres = 0.0, Dres = 1.0;
  int accepted = -1, cur = -1;
  for (int i = 0; i < nk; ++i) {
    const double px = sm.kpx[i], qx = sm.kqx[i];
    if ((double)sm.kua[i] * qx * Dres <= fmax(px - Cres * qx, 0.0)) {
      accepted = sm.kids[i];
      break;
    }
    const double cn = Cres + Dres;
    for (int j0 = 0; j0 < nmine; j0 += kResident) {
      if (!kRes) {   // re-read the batch and rebuild its exponentials
#pragma unroll
        for (int r = 0; r < kResident; ++r) {
          const int e0 = (my_c0 + min(j0 + r, nmine - 1)) * kChunk + 16 * t;
          load16<kVec>(zp_rs, e0, ep[r]);
          load16<kVec>(zq_rs, e0, eq[r]);
        }
#pragma unroll
        for (int r = 0; r < kResident; ++r) {
          const int jr = min(j0 + r, nmine - 1);
          const int e0 = (my_c0 + jr) * kChunk + 16 * t;
          const float mp = sm.cm[0][jr], mq = sm.cm[1][jr];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool in = e0 + e < p.V;
            ep[r][e] = in ? exp_t(ep[r][e] - mp, p.k2hi, p.k2lo) : 0.f;
            eq[r][e] = in ? exp_t(eq[r][e] - mq, p.k2hi, p.k2lo) : 0.f;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kResident; ++r) {
        if (j0 + r < nmine) {
          const double a = sm.ca[0][my_c0 + j0 + r];
          const float rho = chunk_rho(sm.ia[my_c0 + j0 + r], sm.ca[1][my_c0 + j0 + r], cn);
          float wv[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const tv_f32x4 q4 = kRes ? sm.qe[(r * 4 + g) * kSThreads + t]
                                     : tv_f32x4{eq[r][4 * g], eq[r][4 * g + 1], eq[r][4 * g + 2], eq[r][4 * g + 3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[4 * g + e] = residual_rel(ep[r][4 * g + e], q4[e], rho);
          }
          const double s = tv_wave_sum_d((double)sum16(wv) * a);   // pairwise: a short dependent chain
          if (l == 0) sm.part[w][j0 + r] = s;
        }
      }
    }
    tv_lds_barrier();   // the waves' partials
    // Wave 0: this member's chunk masses (lanes take chunks l and l + 64) and
    // their sum, published; lanes below S gather the team's masses and add
    // them with a fixed DPP tree, so every member obtains the same F.
    if (w == 0) {
      double r0 = 0.0, r1 = 0.0;
      if (l < nmine)
        for (int i2 = 0; i2 < kSThreads / 64; ++i2) r0 += sm.part[i2][l];
      if (l + 64 < nmine)
        for (int i2 = 0; i2 < kSThreads / 64; ++i2) r1 += sm.part[i2][l + 64];
      const double mine = tv_wave_sum_d(r0 + r1);
      unsigned long long* xs = p.xch + ((size_t)b * p.n_max + sm.kids[i]) * kMaxTeam;
      if (l == 0) xch_put(xs + member, (unsigned long long)__double_as_longlong(mine));
      double xv = 0.0;
      if (l < p.S) xv = __longlong_as_double((long long)xch_get(xs + l, &sm.timeout));
      const double F = tv_readlane_d(tv_row16_sum_d(xv), 0);
      if (F > 0.0) {   // the residual moves: keep its member and chunk masses
        if (l < p.S) sm.xcur[l] = xv;
        if (l < nmine) sm.rcur[l] = r0;
        if (l + 64 < nmine) sm.rcur[l + 64] = r1;
      }
      if (l == 0) sm.Fx = F;
    }
    tv_lds_barrier();
    const double F = sm.Fx;
    if (F > 0.0) {   // Z > 0: move to the new residual
      Cres = cn;
      Dres = F;
      cur = i;
    }
  }

  if (accepted < 0) {
    // the node's draw: inverse CDF over member masses, this member's chunk
    // masses, then inside one chunk; masses are those of p while no rejection
    // has moved the residual, else of the current residual
    if (cur < 0) {
      if (t < p.S) {   // member masses of p, parallel over members
        double x = 0.0;
        for (int c = t * p.per; c < min((t + 1) * p.per, p.chunks); ++c) x += sm.sc[c] * sm.ca[0][c];
        sm.xcur[t] = x;
      }
      if (t < nmine) sm.rcur[t] = sm.cs[0][t] * sm.ca[0][my_c0 + t];
    }
    tv_lds_barrier();
    if (w == 0) {   // member, then chunk, by wave scans
      const double x = l < p.S ? sm.xcur[l] : 0.0;
      const double total = tv_readlane_d(tv_wave_incl_scan_d(x, l), 63);
      const double thr = (double)us * total;
      double base = 0.0;
      const int ms = wave_select_mass(sm.xcur, p.S, thr, &base, l);
      const int sel = ms == member ? wave_select_mass(sm.rcur, nmine, thr, &base, l) : 0;
      if (l == 0) {
        sm.owner = ms;
        sm.sel = sel;
        sm.base = base;
        sm.thr = thr;
      }
    }
    tv_lds_barrier();
    if (sm.owner == member && nmine > 0) {
      const int j = min(sm.sel, nmine - 1);
      const int e0 = (my_c0 + j) * kChunk + 16 * t;
      const double a = sm.ca[0][my_c0 + j];
      const float rho = chunk_rho(sm.ia[my_c0 + j], sm.ca[1][my_c0 + j], Cres);
      const bool res = cur >= 0;
      double wts[16];
      if (kRes) {
        float pe[16], qe[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) pe[e] = (j == 0) ? ep[0][e] : ep[kResident - 1][e];
        if (res) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const tv_f32x4 q4 = sm.qe[(j * 4 + g) * kSThreads + t];
            qe[4 * g] = q4[0];
            qe[4 * g + 1] = q4[1];
            qe[4 * g + 2] = q4[2];
            qe[4 * g + 3] = q4[3];
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) wts[e] = (double)residual_rel(pe[e], qe[e], rho) * a;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) wts[e] = (double)pe[e] * a;
        }
      } else {
        float xp[16], xq[16];
        load16<kVec>(zp_rs, e0, xp);
        if (res) load16<kVec>(zq_rs, e0, xq);
        const float mp = sm.cm[0][j], mq = sm.cm[1][j];
        if (res) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            wts[e] = e0 + e < p.V ? (double)residual_rel(exp_t(xp[e] - mp, p.k2hi, p.k2lo),
                                                         exp_t(xq[e] - mq, p.k2hi, p.k2lo), rho) * a
                                  : 0.0;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) wts[e] = e0 + e < p.V ? (double)exp_t(xp[e] - mp, p.k2hi, p.k2lo) * a : 0.0;
        }
      }
      const int y = chunk_draw(sm, wts, e0, sm.base, sm.thr, (my_c0 + j) * kChunk);
      o.tok = y;
      o.drew = true;
    }
  }
  o.acc = accepted;
}

// The chase of request b by one of the B workgroups that follow the node
// workgroups in the grid.  Dispatched in id order, it takes a slot only after
// every node workgroup has one, so it never holds one a team needs.  It issues
// its loads at once (for the compaction also the block-table entries it checks
// and uses: every entry among those of positions [0, P + n), the path's last
// node being below n, and the entries of positions [P, P + n) kept for the
// moves), waits for the request's node words, walks the path, and in the
// verify-and-compact form then compacts the request's KV heads along it
// (tv_compact.h), so the path never round-trips through memory.
__device__ __forceinline__ void chase_tail(const StochParams& p, ChaseTailSmem& sm, int b) {
  const int t = threadIdx.x;
  int P = 0, stage0 = 0;
  if (p.chase_mode != kChaseOnly) {
    const TvCompactArgs& c = p.cpt;
    if (t == 0) sm.first_bad = kTvNoBadBlock;
    __syncthreads();
    const int n = p.n_nodes[b];
    P = c.prefix_len[b];
    if (n >= 1 && n <= p.n_max && P >= 0) {
      const int nblk_max = (int)min(((long long)P + n - 1) / c.bs + 1, (long long)c.max_blocks);
      stage0 = P / c.bs;
      const int32_t* trow = c.table + (size_t)b * c.max_blocks;
      for (int i = t; i < nblk_max; i += blockDim.x) {
        const int blk = trow[i];
        if (blk < 0 || blk >= c.num_blocks) atomicMin(&sm.first_bad, i);
        if (i >= stage0) sm.stage[i - stage0] = blk;
      }
    }
  }
  const int len = chase_request(p, sm.c, b, chase_gather(p, b));   // synchronises before it returns
  if (p.chase_mode == kChaseOnly) return;
  const TvTablePrefetch pre{sm.first_bad, stage0, sm.stage};
  // 8-byte moves (the caches are 8-byte aligned on this path)
  if (p.chase_mode == kChaseCompactBf16)
    tv_compact_heads<uint16_t, 4>(p.cpt, b, 0, p.cpt.Hkv, sm.c.path, len, P, &pre, &sm.c.bad);
  else
    tv_compact_heads<float, 2>(p.cpt, b, 0, p.cpt.Hkv, sm.c.path, len, P, &pre, &sm.c.bad);
}

// One team of S workgroups per node (team = blockIdx / S, members on consecutive
// ids), each member owning `per` consecutive chunks of the vocabulary.  Every
// member reads its slice of the target row (and of the draft row when the node
// has children) once; the team exchanges each slice's (max, sum), tests the
// children, and makes the node's draw for the case that no child is accepted
// (the chase uses it when the accepted path ends at this node).  Members
// wait only on their own team: with workgroups dispatched in id order every
// team becomes fully resident once the teams before it have left, and a wait
// that still expires flags TV_REQ_TIMEOUT instead of hanging.  kRes: every
// member's slice is at most kResident chunks and its exponentials stay on chip
// (target in registers, draft in LDS); otherwise each pass re-reads the slice.
// The resident variant runs four workgroups per CU (a 16-member team per node
// for up to 64 nodes on 256 CUs); the streaming variant keeps two batches of
// loads in flight and runs three.
template <bool kRes, bool kVec>
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(kRes ? 4 : 2))) void stoch_node_kernel(StochParams p) {
  __shared__ union {
    NodeSmem<kRes> node;
    ChaseTailSmem chase;
  } smu;
  // A node workgroup's first loads (its request's size, the workspace header)
  // are issued before it is known whether this is a chase workgroup: a
  // separate test ahead of them would delay every node workgroup by one more
  // dependent load.
  const bool chase = (int)blockIdx.x >= p.G;
  const int t = threadIdx.x;
  // With the whole grid resident, team members are numbered so that they run
  // on one XCD (workgroup i goes to XCD i mod 8), where their exchange hand-offs
  // are shorter.  Otherwise teams stay consecutive workgroup ids, which in-order
  // dispatch makes resident one after another.
  const int lid = p.xcd_teams ? tv_xcd_remap(blockIdx.x, p.G) : blockIdx.x;
  const int k = lid / p.S, member = lid % p.S;
  const int b = min(k / p.n_max, p.B - 1), u = k % p.n_max;   // b clamped for chase workgroups
  const int n = p.n_nodes[b];
  const bool wsok = ws_ok(p);
  // The parent and token rows are read whole (n_max entries, in bounds before n
  // is known), beside the request size, and masked by n afterwards.
  const int l = t & 63;
  const int32_t* par = p.parent + (size_t)b * p.n_max;
  const int32_t* tok = p.tokens + (size_t)b * p.n_max;
  const int pr0 = 1 + l < p.n_max ? par[1 + l] : -1;
  const int pr1 = 65 + l < p.n_max ? par[65 + l] : -1;
  const int tr0 = (t < 64 && 1 + l < p.n_max) ? tok[1 + l] : 0;
  const int tr1 = (t < 64 && 65 + l < p.n_max) ? tok[65 + l] : 0;
  asm volatile("" : : "v"(n), "v"((int)wsok), "v"(pr0), "v"(pr1), "v"(tr0), "v"(tr1));   // keeps the loads above the branch
  if (chase) {
    // The chase reads its arguments through an opaque copy of the argument
    // pointer, so that the compiler does not hoist them above this branch and
    // keep them live (in spilled scalar registers) through the node's work.
    const StochParams* kp = (const StochParams*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    chase_tail(*kp, smu.chase, (int)blockIdx.x - kp->G);
    return;
  }
  NodeSmem<kRes>& sm = smu.node;
  if (n < 1 || n > p.n_max || u >= n) return;
  if (!wsok) return;   // the chase reports it; no slot is read or written
  NodeOut o{0, -1, 0, false};
  const int4 rows = make_int4(1 + l < n ? pr0 : -1, 65 + l < n ? pr1 : -1, 1 + l < n ? tr0 : 0, 65 + l < n ? tr1 : 0);
  node_body<kRes, kVec>(p, sm, k, member, b, u, n, rows, o);
  __syncthreads();
  // The member's part of the node's result word.  The member whose OR
  // completes the word clears the node's exchange slots for the next call
  // (every member has finished with them): the exchange stores all come from
  // wave 0 and have landed before the OR.
  if (t == 0) {
    const int fl = o.flags | (sm.timeout ? TV_REQ_TIMEOUT : 0);
    const unsigned long long mine = 1ull << (kNwDoneShift + member);
    unsigned long long wv = mine | ((unsigned long long)(fl & 0xff) << kNwFlagShift);
    if (member == 0) wv |= (unsigned long long)(uint32_t)(o.acc + 1) << kNwAccShift;
    if (o.drew) wv |= (unsigned long long)(uint32_t)o.tok;
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned long long before = __hip_atomic_fetch_or(p.nword + k, wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long full = ((1ull << p.S) - 1ull) << kNwDoneShift;
    sm.bad = ((before | mine) & full) == full;   // reused: this member completed the node
  }
  __syncthreads();
  if (sm.bad) {   // the node's statistics words, and the rejection slots of its children
    tv_u32x4* sx = (tv_u32x4*)(p.sxch + (size_t)k * p.chunks * 4);
    const tv_u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = t; i < p.chunks * 2; i += kSThreads) sx[i] = z;
    for (int i = t; i < sm.nk * (kMaxTeam / 2); i += kSThreads) {
      tv_u32x4* xc = (tv_u32x4*)(p.xch + ((size_t)b * p.n_max + sm.kids[i / (kMaxTeam / 2)]) * kMaxTeam);
      xc[i % (kMaxTeam / 2)] = z;
    }
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
  size_t g_keys, greedy_bytes;
  size_t xch, sxch, nword, stoch_bytes;
  int gchunks, chunks;
};

VerifyLayout layout(const tv_verify_desc* d) {
  VerifyLayout L;
  const size_t nodes = (size_t)d->batch * d->n_max;
  L.gchunks = (d->vocab + kGreedyChunk - 1) / kGreedyChunk;
  L.chunks = (d->vocab + kChunk - 1) / kChunk;
  size_t o = kWsHeader;
  L.g_keys = o;
  o = tv_align_up(o + nodes * L.gchunks * sizeof(unsigned long long), 256);
  L.greedy_bytes = o;
  o = kWsHeader;
  L.xch = o;
  o = tv_align_up(o + nodes * kMaxTeam * sizeof(unsigned long long), 256);
  L.sxch = o;
  o = tv_align_up(o + nodes * (size_t)L.chunks * 4 * sizeof(unsigned long long), 256);
  L.nword = o;
  o = tv_align_up(o + nodes * sizeof(unsigned long long), 256);
  L.stoch_bytes = o;
  return L;
}

// Workgroups of the resident node kernel one CU holds at once (its registers
// and LDS decide; cached per device, 0 when the query fails).  The whole-grid
// schedule below needs every workgroup resident at the same time.
int resident_per_cu(bool vec) {
  constexpr int kDev = 64;
  static std::once_flag once[kDev][2];
  static int per[kDev][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) return 0;
  std::call_once(once[dev][vec], [dev, vec]() {
    int nb = 0;
    const hipError_t e =
        vec ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stoch_node_kernel<true, true>, kSThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stoch_node_kernel<true, false>, kSThreads, 0);
    per[dev][vec] = e == hipSuccess ? nb : 0;
  });
  return per[dev][vec];
}


struct TeamPlan {
  int S;     // workgroups per node
  int per;   // chunks per member
};

// Team size: enough members (a power of two, at most kMaxTeam and at most one
// per chunk) that every member's slice fits on chip (kResident chunks).  Teams
// need not all be resident at once: a team waits only on its own members,
// which sit on consecutive workgroup ids, so teams dispatched later simply
// start when earlier ones leave.
TeamPlan plan_team(int chunks) {
  TeamPlan tp;
  int S = 1;
  while (S * 2 <= kMaxTeam && S * 2 <= chunks && (chunks + S - 1) / S > kResident) S *= 2;
  tp.S = S;
  tp.per = (chunks + S - 1) / S;
  return tp;
}

}  // namespace

namespace {

// Zero-fills workspace bytes [kWsHeader, bytes) in 16-byte stores, then (one
// thread) writes the header; the next kernel sees both.
__global__ __launch_bounds__(256) void ws_init_kernel(unsigned char* ws, size_t bytes) {
  const size_t n16 = (bytes - kWsHeader) / 16;
  tv_u32x4* z = (tv_u32x4*)(ws + kWsHeader);
  const tv_u32x4 zero = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    z[i] = zero;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    unsigned long long* h = (unsigned long long*)ws;
    h[0] = kWsMagic;
    h[1] = kWsHeader + n16 * 16;
  }
}

}  // namespace

static int tree_verify_workspace_init_impl(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes < kWsHeader) return TV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return TV_ERR_INVALID_ARG;
  const size_t n16 = (workspace_bytes - kWsHeader) / 16;
  size_t grid = (n16 + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(ws_init_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (unsigned char*)workspace,
                     workspace_bytes);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_verify_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_verify_workspace_init");
  return tv_debug_finish("tree_verify_workspace_init", tree_verify_workspace_init_impl(workspace, workspace_bytes, stream), stream);
}

extern "C" size_t tree_verify_workspace_size(const tv_verify_desc* desc) {
  if (check_vdesc(desc) != TV_OK) return 0;
  VerifyLayout L = layout(desc);
  return L.greedy_bytes > L.stoch_bytes ? L.greedy_bytes : L.stoch_bytes;
}

// Scratch of tree_verify_greedy_noalloc (see below).
constexpr size_t kNoAllocScratchBytes = 4u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// Checks the arguments of a greedy verification and launches it with `ws`
// (at least greedy_bytes of the layout) as its scratch.  A prepared workspace
// (header given) takes one kernel whose grid ends with the chase workgroups;
// the static scratch (no header) takes the argmax kernel and then the chase
// kernel.
int launch_greedy(const tv_verify_desc* desc, const float* target_logits, const int32_t* tokens,
                  const int32_t* parent, const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                  int32_t* out_tokens, int32_t* status, char* ws, const VerifyLayout& L, bool prepared,
                  hipStream_t stream) {
  GreedyParams p;
  p.logits = target_logits;
  p.tokens = tokens;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.path = path;
  p.path_len = path_len;
  p.out_tokens = out_tokens;
  p.status = status;
  p.keys = (unsigned long long*)(ws + L.g_keys);
  p.header = prepared ? (const unsigned long long*)ws : nullptr;
  p.header_w = prepared ? (unsigned long long*)ws : nullptr;
  p.need = L.greedy_bytes;
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.V = desc->vocab;
  p.chunks = L.gchunks;
  const long long units = (long long)desc->batch * desc->n_max * L.gchunks;
  if (units + desc->batch > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  p.G = (int)units;
  p.chase_spin = tv_chase_spin_limit(kChaseSpinLimit);
  const unsigned grid = (unsigned)(prepared ? units + desc->batch : units);
  if ((desc->vocab & 3) == 0)
    hipLaunchKernelGGL(greedy_argmax_kernel<true>, dim3(grid), dim3(kGreedyThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(greedy_argmax_kernel<false>, dim3(grid), dim3(kGreedyThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  if (!prepared) hipLaunchKernelGGL(greedy_chase_kernel, dim3((unsigned)desc->batch), dim3(kMaxNodes), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

int check_greedy_args(const tv_verify_desc* desc, const float* target_logits, const int32_t* tokens,
                      const int32_t* parent, const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                      int32_t* out_tokens, int32_t* status) {
  if (!target_logits || !tokens || !parent || !n_nodes || !path || !path_len || !out_tokens || !status)
    return TV_ERR_INVALID_ARG;
  if (((uintptr_t)target_logits & 15) != 0) return TV_ERR_INVALID_ARG;
  return TV_OK;
}

// Scratch of tree_verify_greedy_noalloc: one static array per device (every
// GPU the library runs on holds its own copy until the process ends), reached
// from host code only through the device address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
constexpr int kMaxDevices = 64;

void* g_scratch[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device.
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TV_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_rc[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_rc[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_rc[dev] != hipSuccess || !g_scratch[dev]) return TV_ERR_HIP;
  *out = g_scratch[dev];
  return TV_OK;
}

}  // namespace

static int tree_verify_greedy_impl(const tv_verify_desc* desc, const float* target_logits,
                                  const int32_t* tokens, const int32_t* parent,
                                  const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* status, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  rc = check_greedy_args(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status);
  if (rc != TV_OK) return rc;
  VerifyLayout L = layout(desc);
  if (!workspace || workspace_bytes < L.greedy_bytes) return TV_ERR_WORKSPACE;
  return launch_greedy(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status,
                       (char*)workspace, L, true, stream);
}

extern "C" int tree_verify_greedy(const tv_verify_desc* desc, const float* target_logits,
                                  const int32_t* tokens, const int32_t* parent,
                                  const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* status, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_verify_greedy");
  if (tv_debug_enabled() && desc && desc->batch > 0) {
    tv_debug_trees("tree_verify_greedy", parent, n_nodes, desc->batch, desc->n_max, stream);
  }
  return tv_debug_finish("tree_verify_greedy", tree_verify_greedy_impl(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status, workspace, workspace_bytes, stream), stream);
}

extern "C" size_t tree_verify_greedy_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

static int tree_verify_greedy_noalloc_impl(const tv_verify_desc* desc, const float* target_logits,
                                          const int32_t* tokens, const int32_t* parent,
                                          const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                                          int32_t* out_tokens, int32_t* status, hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  rc = check_greedy_args(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status);
  if (rc != TV_OK) return rc;
  VerifyLayout L = layout(desc);
  if (L.greedy_bytes > kNoAllocScratchBytes) return TV_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != TV_OK) return rc;
  return launch_greedy(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status,
                       (char*)ws, L, false, stream);
}

extern "C" int tree_verify_greedy_noalloc(const tv_verify_desc* desc, const float* target_logits,
                                          const int32_t* tokens, const int32_t* parent,
                                          const int32_t* n_nodes, int32_t* path, int32_t* path_len,
                                          int32_t* out_tokens, int32_t* status, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_verify_greedy_noalloc");
  if (tv_debug_enabled() && desc && desc->batch > 0) {
    tv_debug_trees("tree_verify_greedy_noalloc", parent, n_nodes, desc->batch, desc->n_max, stream);
  }
  return tv_debug_finish("tree_verify_greedy_noalloc", tree_verify_greedy_noalloc_impl(desc, target_logits, tokens, parent, n_nodes, path, path_len, out_tokens, status, stream), stream);
}

namespace {

// Checks the arguments of a stochastic verification and launches its kernel:
// the node workgroups, then one workgroup per request that chases its path
// (and compacts its KV when cpt is given).
int launch_stoch_nodes(const tv_verify_desc* desc, const float* target_logits, const float* draft_logits,
                       const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                       const float* u_accept, const float* u_sample, int32_t* path, int32_t* path_len,
                       int32_t* out_tokens, int32_t* status, void* workspace, size_t workspace_bytes,
                       const TvCompactArgs* cpt, int cpt_bf16, hipStream_t stream) {
  StochParams p{};
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (!target_logits || !draft_logits || !tokens || !parent || !n_nodes || !u_accept || !u_sample ||
      !path || !path_len || !out_tokens || !status)
    return TV_ERR_INVALID_ARG;
  if ((((uintptr_t)target_logits | (uintptr_t)draft_logits) & 15) != 0) return TV_ERR_INVALID_ARG;
  VerifyLayout L = layout(desc);
  if (L.chunks > kMaxChunks) return TV_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.stoch_bytes) return TV_ERR_WORKSPACE;
  const long long nodes = (long long)desc->batch * desc->n_max;
  const TeamPlan tp = plan_team(L.chunks);
  const bool resident = tp.per <= kResident;

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
  p.header = (const unsigned long long*)ws;
  p.header_w = (unsigned long long*)ws;
  p.need = L.stoch_bytes;
  p.xch = (unsigned long long*)(ws + L.xch);
  p.sxch = (unsigned long long*)(ws + L.sxch);
  p.nword = (unsigned long long*)(ws + L.nword);
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.V = desc->vocab;
  p.chunks = L.chunks;
  p.S = tp.S;
  p.per = tp.per;
  p.invT_d = 1.0 / (double)desc->temperature;
  const double k2 = 1.4426950408889634074 * p.invT_d;   // log2(e) / T
  p.k2hi = (float)k2;
  p.k2lo = (float)(k2 - (double)p.k2hi);

  // node workgroups, then one chase workgroup per request
  const long long grid = nodes * tp.S;
  if (grid + desc->batch > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  p.G = (int)grid;
  p.chase_spin = tv_chase_spin_limit(kChaseSpinLimit);
  p.chase_mode = !cpt ? kChaseOnly : (cpt_bf16 ? kChaseCompactBf16 : kChaseCompactF32);
  if (cpt) p.cpt = *cpt;
  // When the whole grid is resident at once (four workgroups per CU), load order
  // follows the number of children: each class waits a quarter of the time the
  // target rows take to stream at about 5.5 TB/s (measured on MI355X: 1.5 us per
  // class at 64 nodes x 128256 logits took the slowest chain 2.3 us earlier).
  int cu = 0;
  p.prio_ticks = 0;
  p.xcd_teams = 0;
  const bool vec = (desc->vocab & 3) == 0;
  if (resident && tv_device_cu_count(&cu) == TV_OK && grid <= (long long)resident_per_cu(vec) * cu) {
    p.xcd_teams = 1;
    const double row_bytes = (double)nodes * (double)desc->vocab * 4.0;
    p.prio_ticks = (int)fmin(row_bytes / (4.0 * 5.5e12) * 1e8, 1000.0);
  }
  void (*kern)(StochParams) = resident ? (vec ? stoch_node_kernel<true, true> : stoch_node_kernel<true, false>)
                                        : (vec ? stoch_node_kernel<false, true> : stoch_node_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)(grid + desc->batch)), dim3(kSThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace

static int tree_verify_stochastic_impl(const tv_verify_desc* desc, const float* target_logits,
                                      const float* draft_logits, const int32_t* tokens,
                                      const int32_t* parent, const int32_t* n_nodes,
                                      const float* u_accept, const float* u_sample, int32_t* path,
                                      int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  return launch_stoch_nodes(desc, target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, path,
                            path_len, out_tokens, status, workspace, workspace_bytes, nullptr, 0, stream);
}

extern "C" int tree_verify_stochastic(const tv_verify_desc* desc, const float* target_logits,
                                      const float* draft_logits, const int32_t* tokens,
                                      const int32_t* parent, const int32_t* n_nodes,
                                      const float* u_accept, const float* u_sample, int32_t* path,
                                      int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_verify_stochastic");
  if (tv_debug_enabled() && desc && desc->batch > 0) {
    tv_debug_trees("tree_verify_stochastic", parent, n_nodes, desc->batch, desc->n_max, stream);
  }
  return tv_debug_finish("tree_verify_stochastic", tree_verify_stochastic_impl(desc, target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, path, path_len, out_tokens, status, workspace, workspace_bytes, stream), stream);
}

static int tree_verify_stochastic_compact_impl(const tv_verify_desc* desc, const tv_attn_desc* kv_desc,
                                              const float* target_logits, const float* draft_logits,
                                              const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                                              const float* u_accept, const float* u_sample, int32_t* path,
                                              int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                              void* k_cache, void* v_cache, const int32_t* block_table,
                                              const int32_t* prefix_len, int32_t* src_pos, int32_t* new_len,
                                              int32_t* kv_status, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  int rc = check_vdesc(desc);
  if (rc != TV_OK) return rc;
  rc = tv_compact_check_desc(kv_desc);
  if (rc != TV_OK) return rc;
  if (kv_desc->batch != desc->batch || kv_desc->n_max != desc->n_max) return TV_ERR_INVALID_ARG;
  if (desc->batch == 0) return TV_OK;
  if (!k_cache || !v_cache || !block_table || !prefix_len || !src_pos || !new_len) return TV_ERR_INVALID_ARG;
  if ((((uintptr_t)k_cache | (uintptr_t)v_cache) & 7) != 0) {
    // caches not aligned to 8 bytes: the compaction's own kernel, which moves
    // single elements, after the verification
    rc = launch_stoch_nodes(desc, target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, path,
                            path_len, out_tokens, status, workspace, workspace_bytes, nullptr, 0, stream);
    if (rc != TV_OK) return rc;
    return kv_compact_accepted(kv_desc, k_cache, v_cache, block_table, prefix_len, path, path_len, src_pos,
                               new_len, kv_status, stream);
  }
  const TvCompactArgs c =
      tv_compact_args(kv_desc, k_cache, v_cache, block_table, prefix_len, src_pos, new_len, kv_status);
  return launch_stoch_nodes(desc, target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, path,
                            path_len, out_tokens, status, workspace, workspace_bytes, &c, kv_desc->dtype == TV_BF16,
                            stream);
}

extern "C" int tree_verify_stochastic_compact(const tv_verify_desc* desc, const tv_attn_desc* kv_desc,
                                              const float* target_logits, const float* draft_logits,
                                              const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                                              const float* u_accept, const float* u_sample, int32_t* path,
                                              int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                              void* k_cache, void* v_cache, const int32_t* block_table,
                                              const int32_t* prefix_len, int32_t* src_pos, int32_t* new_len,
                                              int32_t* kv_status, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  TV_TRACE_SCOPE("tree_verify_stochastic_compact");
  if (tv_debug_enabled() && desc && kv_desc && desc->batch > 0) {
    tv_debug_trees("tree_verify_stochastic_compact", parent, n_nodes, desc->batch, desc->n_max, stream);
    tv_debug_kv("tree_verify_stochastic_compact", block_table, prefix_len, n_nodes, kv_desc->batch, kv_desc->max_blocks_per_seq, kv_desc->block_size, kv_desc->num_blocks, stream);
  }
  return tv_debug_finish("tree_verify_stochastic_compact", tree_verify_stochastic_compact_impl(desc, kv_desc, target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, path, path_len, out_tokens, status, k_cache, v_cache, block_table, prefix_len, src_pos, new_len, kv_status, workspace, workspace_bytes, stream), stream);
}
