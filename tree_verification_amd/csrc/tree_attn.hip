// Token-tree attention for gfx950.
//
// Operation ([guide] "Generalizing Attention to Tree Topologies", "The
// Topology-Aware 2D Causal Mask"): every tree node u of request b attends, for
// each q-head h, to all prefix keys [0, P) and to the tree keys at P + w for w
// in Anc(u) u {u}; q-head h reads KV head h / G.
//
// Decomposition.  The query rows of one (request, KV head) pair are the n*G
// (node, head-in-group) combinations; they all share the same keys, so the
// prefix part is a dense contraction.  A workgroup owns a tile of rows and a
// contiguous range of 32-key chunks (split-K over the prefix, FlashDecoding-
// style).  The split plan follows the requests' actual lengths, read on the
// device: a batch whose row tiles alone leave CUs idle is planned as a whole
// (every workgroup reads all requests' sizes and takes the same share of the
// batch's chunk-tiles, so long requests get more splits than short ones);
// otherwise every tile has the same number of splits and each request's own
// length sets its keys per split.  A block table sized for a longer context
// than the request uses costs nothing.  A workgroup that owns all keys of its
// tile writes the output directly.  Otherwise it writes its (m, l, O) partial
// to the workspace, publishes it (release fence, then one increment of the
// tile's counter), and the split that arrives last merges the tile's partials
// by log-sum-exp and writes the output (no workgroup ever waits for another;
// the merging one resets the counter, so every call leaves the counters zero).
//
// MFMA path (bf16): four MFMA waves own disjoint 16*NTW-row slices of the
// tile (rows past the request are padding) and a fifth, producer wave moves
// 32-key chunks of K and V straight from HBM into a four-slot LDS ring with
// global_load_lds_dwordx4, so the MFMA waves issue no memory operations while
// they compute.  The products are
//   S^T[key][row] = K Q^T  then  O^T[d][row] += V^T P^T,
// laid out so that a lane always owns one query row (lane % 16): the softmax
// state is lane-local, and the C layout of S^T feeds the B operand of the PV
// product without cross-lane moves.  Key bytes land exactly where lane l of
// every MFMA wave reads the K operand of v_mfma_f32_16x16x32_bf16 (ds_read_b128).
// Values are token-major in the cache and in LDS; the V^T operand (8
// consecutive keys of one d per lane) comes from two ds_read_b64_tr_b16 reads,
// the LDS transpose load of gfx950, over rows whose 16-byte pieces the DMA
// stores XOR-swizzled so that those reads are free of bank conflicts.  The
// running max moves only when a row's max grows by more than 8 (log2 units),
// which keeps most chunks free of rescaling.  Chunks of prefix keys only (no
// mask) take a branch-free body whose row sums come from a matrix product
// with ones; chunks holding tree keys or the request's end apply the mask.
//
// VALU path (fp32): the waves interleave 64-key chunks with lane = key for the
// scores and lane = d for PV, merged in LDS.
//
// Tree mask: a wavefront builds the ancestor bitmaps of all nodes (two 64-bit
// words per node, n <= 128) from the parent array by pointer jumping with lane
// shuffles, then tests one bit per (row, tree key).

#include "tv_common.h"

#include <math.h>
#include <mutex>

namespace {

constexpr int kThreads = 256;        // VALU path (fp32): four waves
constexpr int kMfmaWaves = 4;        // MFMA path: four waves own the rows of a tile (per key group) ...
// ... and one more per key group moves its K/V chunks: 5 waves, or 10 with two key groups
template <int KG>
constexpr int mfma_threads() { return 64 * (kMfmaWaves + 1) * KG; }
constexpr int kMaxNodes = 128;
constexpr int kMaxKeysPerSplit = 32768;   // NTW = 1 (two workgroups per CU); twice that for NTW = 2
constexpr int kMinSplitChunks = 4;        // a split owns at least 128 keys (or the whole request)
// LDS ring on the MFMA path: NS steps of KG chunks (one chunk per key group).
template <int KG>
constexpr int ring_steps() { return 4; }
// Keys one split may own, and the block-table entries a workgroup stages for
// them (block size 16 at least).
template <int NTW>
constexpr int max_keys_per_split() { return NTW == 1 ? kMaxKeysPerSplit : 2 * kMaxKeysPerSplit; }
template <int NTW>
constexpr int max_tab() { return max_keys_per_split<NTW>() / 16 + 2; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  const int32_t* parent;
  void* out;
  int32_t* status;
  void* part_o;     // [slots][rows_per_tile][D] O / l of each split times a power of two (fp16 or fp32)
  float4* part_ml;  // [slots][rows_per_tile] (m, l, the power of two's inverse, 0)
  int* counters;    // [slots]: splits of a tile published so far, at the tile's first slot
  const unsigned long long* header;   // [2] prepared-workspace header (magic, bytes cleared)
  unsigned long long need;            // workspace bytes this call's layout uses
  int coresident;   // 1: every workgroup of the grid is resident at once (the splits of a tile merge together)
  long long spin;   // polling rounds of the bounded wait for a tile's splits (negative: give up at once)
  int B, n_max, Hq, Hkv, G, D, bs, lbs, max_blocks, num_blocks;
  float scale_log2;
  int rows_per_tile, row_tiles;   // row tiles of one (request, KV head) at n_max nodes
  int balanced;     // 1: the batch is planned as a whole from its lengths; 0: `splits` per tile
  int splits;       // uniform plan: key splits per tile
  int nwg;          // balanced plan: workgroups it aims at
  int max_kps_ch;   // most 32-key chunks one split may own (the staged block table's reach)
  int grid;         // attention workgroups launched
};

struct AttnPlan {
  int rows_per_tile, row_tiles, ntw, kg, balanced, splits, nwg, max_kps_ch, grid, slots;
  size_t off_cnt, off_o, off_ml, bytes;
};

// ---------------------------------------------------------------------------
// split plan (computed on the device from the requests' sizes)
// ---------------------------------------------------------------------------

// Work shape of one request: row tiles in use and 32-key chunks of its P + n
// keys (both 0 when its sizes are malformed: such a request gets no split).
struct ReqShape {
  int P, n, rt, ch;
};

__device__ __forceinline__ ReqShape req_shape(const AttnParams& p, int P, int n) {
  ReqShape r;
  r.P = P;
  r.n = n;
  const bool ok = n >= 1 && n <= p.n_max && P >= 0 && (long long)P + n <= (long long)p.max_blocks * p.bs;
  r.rt = ok ? (n * p.G + p.rows_per_tile - 1) / p.rows_per_tile : 0;
  r.ch = ok ? (P + n + 31) / 32 : 0;
  return r;
}

// Status of a request whose sizes are malformed (0 otherwise).
__device__ __forceinline__ int shape_status(const AttnParams& p, int P, int n) {
  if (n < 1 || n > p.n_max) return TV_REQ_BAD_NNODES;
  if (P < 0 || (long long)P + n > (long long)p.max_blocks * p.bs) return TV_REQ_BAD_KV;
  return 0;
}

// Chunks per split of a request under the uniform plan.
__device__ __forceinline__ int uniform_kps(const AttnParams& p, int ch) {
  int k = (ch + p.splits - 1) / p.splits;
  k = max(k, kMinSplitChunks);
  return min(k, p.max_kps_ch);
}

// Wave-wide int32 sum and inclusive prefix sum over lanes (DPP and lane
// permutes, no LDS traffic).
__device__ __forceinline__ int wave_sum_i(int v) {
  return (int)tv_wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
  x += (int)tv_dpp<0x111>((uint32_t)x);   // row_shr:1 (lanes shifted in from outside the row read 0)
  x += (int)tv_dpp<0x112>((uint32_t)x);   // row_shr:2
  x += (int)tv_dpp<0x114>((uint32_t)x);   // row_shr:4
  x += (int)tv_dpp<0x118>((uint32_t)x);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// Sum over the batch of f(shape of request b) (each wave computes it; lane =
// request, 64 requests per step).  `mine` is the lane's request shape of the
// first step, loaded once by the caller (batches of at most 64 requests then
// need no further loads).
template <class F>
__device__ __forceinline__ int batch_sum(const AttnParams& p, int lane, const ReqShape& mine, F f) {
  int acc = wave_sum_i(lane < p.B ? f(mine) : 0);
  for (int b0 = 64; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    acc += wave_sum_i(b < p.B ? f(req_shape(p, p.prefix_len[b], p.n_nodes[b])) : 0);
  }
  return acc;
}

__device__ __forceinline__ ReqShape lane_shape(const AttnParams& p, int lane) {
  if (lane < p.B) return req_shape(p, p.prefix_len[lane], p.n_nodes[lane]);
  return ReqShape{0, 0, 0, 0};
}

// The balanced plan's chunks per split: the smallest kps for which the
// batch's splits (every tile's ceil(ch / kps)) fit p.nwg workgroups, at least
// kMinSplitChunks and at most p.max_kps_ch.  With W chunk-tiles over T tiles,
// kps >= W / nwg is necessary and kps >= W / (nwg - T) sufficient; a binary
// search over that range, each step one wave-wide sum over the batch.
__device__ int balanced_kps(const AttnParams& p, int lane, const ReqShape& mine) {
  const int W = batch_sum(p, lane, mine, [&](ReqShape r) { return p.Hkv * r.rt * r.ch; });
  const int T = batch_sum(p, lane, mine, [&](ReqShape r) { return p.Hkv * r.rt; });
  const int cap = p.max_kps_ch;
  int lo = (W + p.nwg - 1) / p.nwg;
  int hi = T < p.nwg ? (W + (p.nwg - T) - 1) / (p.nwg - T) : cap;
  lo = min(max(lo, kMinSplitChunks), cap);
  hi = min(max(hi, lo), cap);
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    const int total = batch_sum(p, lane, mine, [&](ReqShape r) { return p.Hkv * r.rt * ((r.ch + mid - 1) / mid); });
    if (total <= p.nwg) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// One workgroup's share of the plan.
struct SplitPlan {
  int b, g, rt, s;    // request, KV head, row tile, split
  int P, n;           // the request's sizes
  int rt_b;           // row tiles the request uses
  int splits;         // splits of each of its tiles
  int kps_ch;         // chunks per split
  int slot;           // partial slot of this split (its logical workgroup id)
  bool work;          // this workgroup owns a (tile, split)
  bool shape_ok;      // the request's sizes are well formed
};

// Logical workgroup -> (request, KV head, row tile, split).  Splits of one
// tile are consecutive logical ids, tiles of one request consecutive runs, and
// logical ids are numbered XCD-aware (tv_xcd_remap), so a tile's splits and
// the row tiles sharing its K/V run on one XCD.
__device__ SplitPlan plan_split(const AttnParams& p, int phys) {
  const int lane = threadIdx.x & 63;
  SplitPlan sp;
  sp.b = sp.g = sp.rt = sp.s = sp.P = sp.n = sp.rt_b = sp.splits = sp.kps_ch = sp.slot = 0;
  sp.work = false;
  sp.shape_ok = false;
  if (!p.balanced) {
    const int w = tv_xcd_remap(phys, p.grid);
    const int per_req = p.Hkv * p.row_tiles * p.splits;
    sp.b = w / per_req;
    int idx = w % per_req;
    sp.g = idx / (p.row_tiles * p.splits);
    idx %= p.row_tiles * p.splits;
    sp.rt = idx / p.splits;
    sp.s = idx % p.splits;
    sp.P = p.prefix_len[sp.b];
    sp.n = p.n_nodes[sp.b];
    const ReqShape r = req_shape(p, sp.P, sp.n);
    sp.shape_ok = r.rt > 0;
    sp.rt_b = r.rt;
    sp.kps_ch = uniform_kps(p, r.ch);
    sp.splits = r.ch > 0 ? (r.ch + sp.kps_ch - 1) / sp.kps_ch : 0;
    sp.slot = w;
    sp.work = sp.shape_ok && sp.rt < r.rt && sp.s < sp.splits;
    return sp;
  }
  // balanced: every wave walks the batch (sizes are L1/L2 hits after the first)
  const ReqShape mine = lane_shape(p, lane);
  const int kps = balanced_kps(p, lane, mine);
  const int total = batch_sum(p, lane, mine, [&](ReqShape r) { return p.Hkv * r.rt * ((r.ch + kps - 1) / kps); });
  sp.kps_ch = kps;
  if (phys >= total) return sp;
  const int w = tv_xcd_remap(phys, total);
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const ReqShape r = b0 == 0 ? mine : (b < p.B ? req_shape(p, p.prefix_len[b], p.n_nodes[b]) : ReqShape{0, 0, 0, 0});
    const int spl = (r.ch + kps - 1) / kps;
    const int cnt = b < p.B ? p.Hkv * r.rt * spl : 0;
    const int incl = wave_incl_scan_i(cnt, lane);
    const bool hit_lane = w >= base + incl - cnt && w < base + incl;
    const unsigned long long hit = __ballot(hit_lane);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      sp.b = b0 + src;
      sp.P = __shfl(r.P, src);
      sp.n = __shfl(r.n, src);
      sp.rt_b = __shfl(r.rt, src);
      sp.splits = __shfl(spl, src);
      int idx = w - (base + __shfl(incl - cnt, src));
      sp.g = idx / (sp.rt_b * sp.splits);
      idx %= sp.rt_b * sp.splits;
      sp.rt = idx / sp.splits;
      sp.s = idx % sp.splits;
      sp.slot = w;
      sp.shape_ok = true;
      sp.work = true;
      return sp;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  return sp;
}

template <int D>
struct Chunk {
  static constexpr int KK = D / 32;            // 32-wide d pieces of the QK^T contraction
  static constexpr int DT = D / 16;            // 16-wide d tiles of the PV product
  static constexpr int NBLK = 2 * KK + DT;     // 1 KB operand blocks per 32-key chunk
  static constexpr int BYTES = NBLK * 1024;
};

// ---------------------------------------------------------------------------
// shared state
// ---------------------------------------------------------------------------

struct CommonSmem {
  uint64_t anc[kMaxNodes][2];
  int par[kMaxNodes];
  int flag;
};

template <int D>
struct ValuSmem {
  float o[16][D + 4];           // unnormalised output rows (log2-domain softmax)
  float m[16];
  float l[16];
  float wm[4][16];              // per-wave partial m / l before the intra-workgroup merge
  float wl[4][16];
  float qs[16][D];
  float sc[4][16][64];          // per-wave probability strips
};

// ---------------------------------------------------------------------------
// ancestor bitmaps
// ---------------------------------------------------------------------------

// Wave-cooperative pointer jumping: node j lives in lane j % 64, slot j / 64.
// After round r every node holds its ancestors within distance < 2^r; seven
// rounds cover any depth below 128.
__device__ void build_ancestor_bitmaps(const int* par, int n, uint64_t (*anc)[2], int lane) {
  uint64_t lo[2], hi[2];
  int jmp[2];
  for (int s = 0; s < 2; ++s) {
    int u = lane + 64 * s;
    jmp[s] = (u < n && u > 0) ? par[u] : -1;
    lo[s] = (s == 0) ? (1ull << lane) : 0ull;
    hi[s] = (s == 1) ? (1ull << lane) : 0ull;
  }
  for (int r = 0; r < 7; ++r) {
    uint64_t nlo[2], nhi[2];
    int njmp[2];
    for (int s = 0; s < 2; ++s) {
      int j = jmp[s];
      int src = j < 0 ? 0 : (j & 63);
      uint64_t l0 = __shfl(lo[0], src), l1 = __shfl(lo[1], src);
      uint64_t h0 = __shfl(hi[0], src), h1 = __shfl(hi[1], src);
      int j0 = __shfl(jmp[0], src), j1 = __shfl(jmp[1], src);
      bool second = j >= 64;
      if (j >= 0) {
        nlo[s] = lo[s] | (second ? l1 : l0);
        nhi[s] = hi[s] | (second ? h1 : h0);
        njmp[s] = second ? j1 : j0;
      } else {
        nlo[s] = lo[s];
        nhi[s] = hi[s];
        njmp[s] = -1;
      }
    }
    for (int s = 0; s < 2; ++s) {
      lo[s] = nlo[s];
      hi[s] = nhi[s];
      jmp[s] = njmp[s];
    }
  }
  for (int s = 0; s < 2; ++s) {
    int u = lane + 64 * s;
    if (u < n) {
      anc[u][0] = lo[s];
      anc[u][1] = hi[s];
    }
  }
}

typedef __bf16 tv_bf16x2 __attribute__((ext_vector_type(2)));
typedef float tv_f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((tv_f32x2){lo, hi}, tv_bf16x2));
}

__device__ __forceinline__ tv_bf16x8 load_bf16x8(const uint16_t* ptr) {
  return __builtin_bit_cast(tv_bf16x8, *(const tv_u32x4*)ptr);
}

__device__ __forceinline__ bool anc_bit(uint64_t lo, uint64_t hi, int w) {
  return w < 64 ? ((lo >> w) & 1ull) : ((hi >> (w - 64)) & 1ull);
}

__device__ __forceinline__ bool block_ok(int blk, int num_blocks) {
  return blk >= 0 && blk < num_blocks;
}

// ---------------------------------------------------------------------------
// VALU path: up to 16 rows, any element type
// ---------------------------------------------------------------------------
//
// Same wave structure as the MFMA path (the four waves interleave 64-key
// chunks and merge at the end).  Scores: lane = key, the query rows are read
// from LDS as broadcasts.  PV: lane = d, probabilities are read back from a
// per-wave LDS strip four keys at a time.

template <bool kBF16>
__device__ __forceinline__ void load8(const void* base, size_t off, float* dst) {
  if (kBF16) {
    tv_u32x4 w = *(const tv_u32x4*)((const uint16_t*)base + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[2 * j] = __uint_as_float(w[j] << 16);
      dst[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    tv_f32x4 a = *(const tv_f32x4*)((const float*)base + off);
    tv_f32x4 c = *(const tv_f32x4*)((const float*)base + off + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j] = a[j];
      dst[4 + j] = c[j];
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ float val_at(const void* base, size_t off) {
  return kBF16 ? tv_bf16_bits_to_f32(((const uint16_t*)base)[off]) : ((const float*)base)[off];
}

template <bool kBF16, int D, int RV>
__device__ void attn_valu_rows(const AttnParams& p, ValuSmem<D>& sm, int b, int g, int r0, int rows,
                               int P, int k_begin, int k_end, bool tree_in_range, const uint64_t (*anc)[2]) {
  constexpr int DJ = D / 64;   // d values per lane in the PV phase
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int G = p.G;
  const int32_t* trow = p.table + (size_t)b * p.max_blocks;
  float m_r[RV], l_r[RV], o[RV][DJ];
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    m_r[r] = kNegInf;
    l_r[r] = 0.f;
#pragma unroll
    for (int j = 0; j < DJ; ++j) o[r][j] = 0.f;
  }
  float* ps = &sm.sc[wave][0][0];               // this wave's [16][64] probability strip
  const int nchunks = (k_end - k_begin + 63) / 64;
  for (int c = wave; c < nchunks; c += 4) {
    const int kb = k_begin + 64 * c;
    // scores: lane = key
    float s[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) s[r] = 0.f;
    const int key = kb + lane;
    bool valid = key < k_end;
    int blk = valid ? trow[key >> p.lbs] : -1;
    valid = valid && block_ok(blk, p.num_blocks);
    if (valid) {
      size_t base = ((((size_t)blk * p.Hkv + g) << p.lbs) + (key & (p.bs - 1))) * D;
#pragma unroll 2
      for (int d0 = 0; d0 < D; d0 += 8) {
        float kv[8];
        load8<kBF16>(p.k, base + d0, kv);
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          const tv_f32x4 qa = *(const tv_f32x4*)&sm.qs[r][d0];
          const tv_f32x4 qb = *(const tv_f32x4*)&sm.qs[r][d0 + 4];
          s[r] += qa[0] * kv[0] + qa[1] * kv[1] + qa[2] * kv[2] + qa[3] * kv[3] +
                  qb[0] * kv[4] + qb[1] * kv[5] + qb[2] * kv[6] + qb[3] * kv[7];
        }
      }
    }
    float alpha[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      bool ok = valid && r < rows;
      if (ok && key >= P) {
        const int node = (r0 + r) / G;
        ok = tree_in_range && anc_bit(anc[node][0], anc[node][1], key - P);
      }
      float v = ok ? s[r] : kNegInf;
      float cmax = tv_wave_max(v);
      float m_new = fmaxf(m_r[r], cmax);
      float m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha[r] = __builtin_amdgcn_exp2f(m_r[r] - m_use);
      float pv = __builtin_amdgcn_exp2f(v - m_use);
      l_r[r] = l_r[r] * alpha[r] + pv;
      m_r[r] = m_new;
      ps[r * 64 + lane] = pv;
    }
    // PV: lane = d; value rows are token-major, so each key's row is one
    // coalesced read across the wave (8 keys at a time, all inside one block)
#pragma unroll
    for (int r = 0; r < RV; ++r) {
#pragma unroll
      for (int j = 0; j < DJ; ++j) o[r][j] *= alpha[r];
    }
#pragma unroll 1
    for (int k8 = 0; k8 < 64; k8 += 8) {
      const int kk = kb + k8;
      if (kk >= k_end) break;
      const int vb = trow[kk >> p.lbs];
      if (!block_ok(vb, p.num_blocks)) continue;
      float vv[DJ][8];
      const size_t row0 = ((size_t)vb * p.Hkv + g) * p.bs + (kk & (p.bs - 1));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int j = 0; j < DJ; ++j)   // slots past the request hold no data
          vv[j][e] = kk + e < k_end ? val_at<kBF16>(p.v, (row0 + e) * D + lane + 64 * j) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const tv_f32x4 pa = *(const tv_f32x4*)&ps[r * 64 + k8];
        const tv_f32x4 pb = *(const tv_f32x4*)&ps[r * 64 + k8 + 4];
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          o[r][j] += pa[0] * vv[j][0] + pa[1] * vv[j][1] + pa[2] * vv[j][2] + pa[3] * vv[j][3] +
                     pb[0] * vv[j][4] + pb[1] * vv[j][5] + pb[2] * vv[j][6] + pb[3] * vv[j][7];
        }
      }
    }
  }
  // merge the four waves (same protocol as the MFMA path)
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    float lt = tv_wave_sum(l_r[r]);
    if (lane == 0) {
      sm.wm[wave][r] = m_r[r];
      sm.wl[wave][r] = lt;
    }
  }
  __syncthreads();
  if (t < RV) {
    float M = fmaxf(fmaxf(sm.wm[0][t], sm.wm[1][t]), fmaxf(sm.wm[2][t], sm.wm[3][t]));
    float L = 0.f;
    for (int w = 0; w < 4; ++w) {
      float mw = sm.wm[w][t];
      L += (mw == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mw - M) * sm.wl[w][t];
    }
    sm.m[t] = M;
    sm.l[t] = L;
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        float M = fmaxf(fmaxf(sm.wm[0][r], sm.wm[1][r]), fmaxf(sm.wm[2][r], sm.wm[3][r]));
        float sc = (m_r[r] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_r[r] - M);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          float v = sc * o[r][j];
          float* dst = &sm.o[r][lane + 64 * j];
          *dst = (w == 0) ? v : *dst + v;
        }
      }
    }
    __syncthreads();
  }
}

template <bool kBF16, int D>
__device__ void attn_valu(const AttnParams& p, ValuSmem<D>& sm, int b, int g, int r0, int rows,
                          int P, int k_begin, int k_end, bool tree_in_range, const uint64_t (*anc)[2]) {
  const int t = threadIdx.x;
  const int G = p.G;
  // query rows, pre-scaled into the log2 domain; rows past `rows` are zero
  for (int idx = t; idx < 16 * D; idx += kThreads) {
    int r = idx / D, d = idx % D;
    float v = 0.f;
    if (r < rows) {
      int qrow = r0 + r, node = qrow / G, hh = qrow % G;
      size_t off = (((size_t)b * p.n_max + node) * p.Hq + (size_t)g * G + hh) * D + d;
      v = kBF16 ? tv_bf16_bits_to_f32(((const uint16_t*)p.q)[off]) : ((const float*)p.q)[off];
    }
    sm.qs[r][d] = v * p.scale_log2;
  }
  __syncthreads();
  const int rv = (rows + 3) / 4;
  if (rv <= 1) attn_valu_rows<kBF16, D, 4>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range, anc);
  else if (rv == 2) attn_valu_rows<kBF16, D, 8>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range, anc);
  else if (rv == 3) attn_valu_rows<kBF16, D, 12>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range, anc);
  else attn_valu_rows<kBF16, D, 16>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range, anc);
}

// ---------------------------------------------------------------------------
// output and split-K merge
// ---------------------------------------------------------------------------

// Split partials hold the split's normalised output O / l (|O / l| <= max |v|:
// a convex combination of value rows) beside its (m, l).  For bf16 inputs they
// are stored as fp16 after multiplying each row by a power of two that brings
// its largest magnitude into [2^14, 2^15): every element then keeps fp16's 11
// significant bits relative to the row's largest one (no overflow for large
// values, no loss to subnormals for small ones), and the merge multiplies by
// the inverse, kept in the row's (m, l) record.  fp32 inputs keep fp32 (scale 1).
typedef _Float16 tv_f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 tv_f16x8 __attribute__((ext_vector_type(8)));

// Power of two for a row whose largest |O / l| is amax, and its inverse.
__device__ __forceinline__ float2 part_scale(float amax) {
  int e = __builtin_amdgcn_frexp_expf(amax);   // amax < 2^e (0 for amax = 0)
  e = max(e, -100);                            // keeps both factors normal floats
  return make_float2(ldexpf(1.f, 15 - e), ldexpf(1.f, e - 15));
}

// Partials cross workgroups that may run on different XCDs, whose L2 caches
// are not coherent with each other.  They are written and read as 64-bit
// device-scope (agent) accesses, which write through to and read from the
// device's coherent memory side, so no L2 write-back or invalidation is needed
// around the hand-off (see publish_split).
__device__ __forceinline__ void st_agent(void* ptr, uint64_t v) {
  __hip_atomic_store((uint64_t*)ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent(const void* ptr) {
  return __hip_atomic_load((uint64_t*)ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool kBF16>
__device__ __forceinline__ void store_part4(void* part_o, size_t off, tv_f32x4 v) {
  if (kBF16) {
    st_agent((_Float16*)part_o + off, __builtin_bit_cast(uint64_t, __builtin_convertvector(v, tv_f16x4)));
  } else {
    float* d = (float*)part_o + off;
    st_agent(d, __builtin_bit_cast(uint64_t, (tv_f32x2){v[0], v[1]}));
    st_agent(d + 2, __builtin_bit_cast(uint64_t, (tv_f32x2){v[2], v[3]}));
  }
}

template <bool kBF16>
__device__ __forceinline__ tv_f32x4 load_part4(const void* part_o, size_t off) {
  if (kBF16) return __builtin_convertvector(__builtin_bit_cast(tv_f16x4, ld_agent((const _Float16*)part_o + off)), tv_f32x4);
  const float* s = (const float*)part_o + off;
  const tv_f32x2 lo = __builtin_bit_cast(tv_f32x2, ld_agent(s)), hi = __builtin_bit_cast(tv_f32x2, ld_agent(s + 2));
  return (tv_f32x4){lo[0], lo[1], hi[0], hi[1]};
}

// A row's (m, l, inverse scale) record.
__device__ __forceinline__ void store_ml(float4* rec, float m, float l, float z) {
  st_agent(rec, __builtin_bit_cast(uint64_t, (tv_f32x2){m, l}));
  st_agent((float*)rec + 2, __builtin_bit_cast(uint64_t, (tv_f32x2){z, 0.f}));
}
__device__ __forceinline__ float4 load_ml(const float4* rec) {
  const tv_f32x2 a = __builtin_bit_cast(tv_f32x2, ld_agent(rec)), b = __builtin_bit_cast(tv_f32x2, ld_agent((const float*)rec + 2));
  return make_float4(a[0], a[1], b[0], 0.f);
}

template <bool kBF16, int D>
__device__ __forceinline__ void store_out4(const AttnParams& p, int b, int g, int qrow, int d, const float* v4) {
  int node = qrow / p.G, hh = qrow % p.G;
  size_t off = (((size_t)b * p.n_max + node) * p.Hq + (size_t)g * p.G + hh) * D + d;
  if (kBF16) {
    *(uint2*)((uint16_t*)p.out + off) = make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
  } else {
    *(tv_f32x4*)((float*)p.out + off) = (tv_f32x4){v4[0], v4[1], v4[2], v4[3]};
  }
}

// Split-K merge inside the attention grid.  Every split of a tile writes its
// partial and publishes it with one increment of the tile's counter (after a
// barrier that follows every wave's stores).  The workgroup whose increment
// completes the count has every other split's partial published before it,
// merges the tile's rows by log-sum-exp from the workspace, and resets the
// counter for the next call.  No workgroup waits
// for another, so nothing depends on which workgroups are resident together.
// A thread owns 8 d values of one row and walks the splits in batches whose
// loads are in flight together, rescaling its running sum when a batch raises
// the row's max.
constexpr int kMergeVec = 8;     // d values per thread
constexpr long long kMergeSpinLimit = 1LL << 19;   // bounded wait of a co-resident tile's splits (~0.5 s)
constexpr int kMergeBatch = 4;   // splits loaded together

template <bool kBF16>
__device__ __forceinline__ void load_part8(const void* part_o, size_t off, float (&o)[kMergeVec]) {
  const tv_f32x4 lo = load_part4<kBF16>(part_o, off), hi = load_part4<kBF16>(part_o, off + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = lo[i];
    o[4 + i] = hi[i];
  }
}

// True in the workgroup that completes the tile's count (for every thread of
// it).  Called by every thread after the partial stores; `flag` is LDS.  Each
// wave waits until its device-scope partial stores have completed, the
// barrier joins the waves, and one thread increments the tile's counter
// (device scope).  The partials are written and read with device-scope
// accesses (st_agent / ld_agent), so the stores that completed before the
// increment are what the merging workgroup's loads, issued after it observed
// the count, return; no cache write-back or invalidation is involved.
__device__ __forceinline__ bool publish_split(const AttnParams& p, int* flag, int first, int n_active, bool ws_ok) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    int last = 0;
    if (ws_ok) last = __hip_atomic_fetch_add(p.counters + first, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_active - 1;
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// Rows [r0, r0 + rows) of tile `first` (its splits' partials at slots first ..
// first + n_active - 1), by the NT threads of the merging workgroup.
template <bool kBF16, int D, int NT>
__device__ void merge_tile(const AttnParams& p, int first, int n_active, int b, int g, int r0, int rows) {
  constexpr int TPR = D / kMergeVec;
  for (int idx = threadIdx.x; idx < rows * TPR; idx += NT) {
    const int r = idx / TPR, d = kMergeVec * (idx % TPR);
    const size_t base = (size_t)first * p.rows_per_tile + r;
    float4 ml[kMergeBatch];
    float o[kMergeBatch][kMergeVec];
    float M = kNegInf, L = 0.f, acc[kMergeVec];
#pragma unroll
    for (int i = 0; i < kMergeVec; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < n_active; s0 += kMergeBatch) {
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s) {
        if (s0 + s < n_active) {
          const size_t pr = base + (size_t)(s0 + s) * p.rows_per_tile;
          ml[s] = load_ml(p.part_ml + pr);
          load_part8<kBF16>(p.part_o, pr * D + d, o[s]);
        }
      }
      float mb = kNegInf;
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s)
        if (s0 + s < n_active) mb = fmaxf(mb, ml[s].x);
      if (mb > M) {   // the batch raises the row's max: rescale what is summed so far
        const float sc = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - mb);
        L *= sc;
#pragma unroll
        for (int i = 0; i < kMergeVec; ++i) acc[i] *= sc;
        M = mb;
      }
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s) {
        if (s0 + s < n_active && ml[s].x != kNegInf) {
          const float w = __builtin_amdgcn_exp2f(ml[s].x - M) * ml[s].y;
          L += w;
          const float wo = w * ml[s].z;   // the stored row is O / l times 1 / ml.z
#pragma unroll
          for (int i = 0; i < kMergeVec; ++i) acc[i] += wo * o[s][i];
        }
      }
    }
    const float inv = 1.f / L;
    float v4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    store_out4<kBF16, D>(p, b, g, r0 + r, d, v4);
    float w4[4] = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    store_out4<kBF16, D>(p, b, g, r0 + r, d + 4, w4);
  }
}

// VALU path output: rows [r0, r0 + rows) are in LDS.
template <bool kBF16, int D, int RW>
__device__ void emit_valu(const AttnParams& p, CommonSmem& cm, ValuSmem<D>& sm, int slot, int n_active,
                          int b, int g, int r0, int rows) {
  const int t = threadIdx.x;
  if (n_active == 1) {
    for (int idx = t; idx < rows * (D / 4); idx += kThreads) {
      int r = idx / (D / 4), d = 4 * (idx % (D / 4));
      float inv = 1.f / sm.l[r];
      float v4[4] = {sm.o[r][d] * inv, sm.o[r][d + 1] * inv, sm.o[r][d + 2] * inv, sm.o[r][d + 3] * inv};
      store_out4<kBF16, D>(p, b, g, r0 + r, d, v4);
    }
    return;
  }
  const size_t prow = (size_t)slot * RW;
  for (int idx = t; idx < rows * (D / 4); idx += kThreads) {
    int r = idx / (D / 4), d = 4 * (idx % (D / 4));
    const float inv = sm.l[r] > 0.f ? 1.f / sm.l[r] : 0.f;
    store_part4<kBF16>(p.part_o, (prow + r) * D + d,
                       (tv_f32x4){sm.o[r][d] * inv, sm.o[r][d + 1] * inv, sm.o[r][d + 2] * inv, sm.o[r][d + 3] * inv});
  }
  if (t < rows) store_ml(p.part_ml + prow + t, sm.m[t], sm.l[t], 1.f);
}

// ---------------------------------------------------------------------------
// MFMA path: K/V chunks DMA'd into an LDS ring, 16*NTW rows per wave
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) const tv_u32x4* tv_lds_u32x4_ptr;

// 16 bytes from LDS address `addr` (ds_read_b128).
__device__ __forceinline__ tv_bf16x8 lds_read16(uint32_t addr) {
  return __builtin_bit_cast(tv_bf16x8, *(tv_lds_u32x4_ptr)(uintptr_t)addr);
}


// s_waitcnt that only waits for the vector-memory counter (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* tv_lds_ptr;

// One 32-key chunk, sent straight from HBM into its LDS slot by the producer
// wave with global_load_lds_dwordx4 (lane l's 16 bytes land at 16*l of the
// instruction's 1 KB).  A chunk starts at a multiple of 32 keys, so it spans
// at most two blocks (only with 16-token blocks: keys 0..15 then 16..31 of the
// chunk).  Each instruction reads from one of the chunk's two halves, whose
// base addresses are wave-uniform (a 64-bit scalar base plus a per-lane 32-bit
// offset fixed for the whole split); keys at or past k_end read whatever their
// (in-pool) block holds and are masked at use.
//   Keys: instruction (tt, kk) holds, at lane l, key 16*tt + l%16 of the chunk
// and d values 8*(l/16) + 32*kk .. + 7: the K operand lane l of every MFMA
// wave feeds to v_mfma_f32_16x16x32_bf16 for the keys of half tt
// (conflict-free ds_read_b128).
//   Values: 32 token-major rows of 2*D bytes.  Instruction j fills rows R*j ..
// R*j + R - 1 (R = 512 / D rows per KB); in row `key` the 16-byte piece of d
// values 8p .. 8p+7 sits at piece slot p ^ vswz<D>(key), an XOR swizzle that
// puts the pieces one ds_read_b64_tr_b16 reads (four keys x 16 d values per
// group of 16 lanes, eight consecutive keys per half-wave) on distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return D == 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
}

struct DmaLane {
  uint32_t koff;      // key instructions: this lane's row and d piece within a half
  uint32_t voff[2];   // value instruction j: this lane's row and swizzled piece, by j & 1
};

template <int D>
__device__ __forceinline__ DmaLane dma_lane(int lane) {
  const int l16 = lane & 15, h4 = lane >> 4;
  DmaLane dl;
  dl.koff = (uint32_t)(l16 * D * 2 + 16 * h4);
  constexpr int R = 512 / D, PPR = D / 8;   // value rows per instruction, 16-byte pieces per row
  const int r = lane / PPR, s = lane % PPR;
#pragma unroll
  for (int x = 0; x < 2; ++x)   // row R*j + r of the chunk; the swizzle depends on j only through j & 1
    dl.voff[x] = (uint32_t)(r * D * 2 + 16 * (s ^ vswz<D>(R * x + r)));
  return dl;
}

// Row indices of the two blocks of the chunk at key0 (the second clamped into
// the staged table; it is only read for keys past the request's end then).
__device__ __forceinline__ int2 chunk_rows(const int* tab, int tab0, int ntab, int key0, int lbs) {
  const int ia = (key0 >> lbs) - tab0;
  const int ib = min(((key0 + 16) >> lbs) - tab0, ntab - 1);
  return make_int2(__builtin_amdgcn_readfirstlane(tab[ia]), __builtin_amdgcn_readfirstlane(tab[ib]));
}

__device__ __forceinline__ tv_lds_ptr lds_at(uint32_t addr) { return (tv_lds_ptr)(uintptr_t)addr; }

// LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) { return (uint32_t)(uintptr_t)(tv_lds_ptr)ptr; }

template <int D>
__device__ __forceinline__ void dma_chunk(const AttnParams& p, const DmaLane& dl, int2 rows, int key0,
                                          uint32_t slot) {
  constexpr int KK = Chunk<D>::KK, DT = Chunk<D>::DT, R = 512 / D;
  const size_t row_bytes = (size_t)p.bs * D * 2;   // one (block, KV head) row, K and V alike
  const size_t kin = (size_t)(key0 & (p.bs - 1));  // the chunk's first in-block position
  // byte offsets of the chunk's two halves (keys 0..15 and 16..31)
  const size_t h0 = (size_t)(uint32_t)rows.x * row_bytes + kin * D * 2;
  const size_t h1 = p.bs == 16 ? (size_t)(uint32_t)rows.y * row_bytes : h0 + 16 * D * 2;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const char* kb = (const char*)p.k + (tt ? h1 : h0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      __builtin_amdgcn_global_load_lds((const void*)(kb + dl.koff + 64 * kk), lds_at(slot + (tt * KK + kk) * 1024),
                                       16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < DT; ++j) {
    const int row0 = R * j;   // the instruction's first row of the chunk
    const char* vb = (const char*)p.v + (row0 >= 16 ? h1 : h0);
    __builtin_amdgcn_global_load_lds((const void*)(vb + dl.voff[j & 1] + (row0 & 15) * D * 2),
                                     lds_at(slot + (2 * KK + j) * 1024), 16, 0, 0);
  }
}

typedef __bf16 tv_bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tv_bf16x4* tv_lds_bf16x4_ptr;

// V^T operand of d tile dt for v_mfma_f32_16x16x32_bf16.  The PV product
// contracts over the chunk's keys in the order the score tiles hold them: lane
// l's eight k entries are keys 4*(l/16) + 0..3 (score tile 0) and 16 + 4*(l/16)
// + 0..3 (score tile 1), so lane l needs V[those keys][d = 16*dt + l%16], as two
// transposed reads of four keys.  In each group of 16 lanes,
// ds_read_b64_tr_b16 hands lane j element j%4 of the 8 bytes lane 4*k + j/4
// addressed, as its element k; so lane i of group h addresses the four d
// values 16*dt + 4*(i%4) .. + 3 of key 16*e + 4*h + i/4 (one 8-byte half of a
// swizzled 16-byte piece).
template <int D>
__device__ __forceinline__ tv_bf16x8 lds_vop(uint32_t vreg, int dt, int lane) {
  const int h = lane >> 4, i = lane & 15;
  const int key0 = 4 * h + (i >> 2);
  const int f = vswz<D>(key0);   // the same for key0 + 16
  const uint32_t a0 = vreg + key0 * 2 * D + 16 * ((2 * dt + ((i & 3) >> 1)) ^ f) + 8 * (i & 1);
  const tv_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((tv_lds_bf16x4_ptr)(uintptr_t)a0);
  const tv_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((tv_lds_bf16x4_ptr)(uintptr_t)(a0 + 16 * 2 * D));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Running softmax state and output accumulators of one wave (16*NTW rows).
template <int D, int NTW>
struct WaveAcc {
  float m_run[NTW], l_run[NTW];     // l_run: this lane's share of the row sums of masked chunks
  tv_f32x4 oacc[Chunk<D>::DT][NTW];
  tv_f32x4 lacc[NTW];               // row sums of unmasked chunks, by a matrix product with ones
};

// Online-softmax step of one 16-row tile over a chunk whose 32 keys are all
// visible (no mask): the tile's running max moves only when the chunk's max
// exceeds it by more than kLazy (log2 units).  Each lane first tests its own
// eight scores; only when some lane's exceed the margin (rare) does the wave
// take the row maxima across lanes.  Returns the factor the tile's
// accumulators must be scaled by (1 when the max did not move) and the
// chunk's probabilities as the bf16 B operand of the PV product.  Written
// without short-circuit tests, so the common path is straight-line code.
constexpr float kLazy = 8.f;
__device__ __forceinline__ float softmax_plain(const tv_f32x4 (&sc)[2], float& m_run, float scale_log2,
                                               tv_bf16x8& pop) {
  const float lmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  float alpha = 1.f;
  if (__any((lmax * scale_log2 > m_run + kLazy) | (m_run == kNegInf))) {
    const float cmax = tv_rows_max(lmax) * scale_log2;
    const bool fresh = m_run == kNegInf;
    const bool move = (cmax > m_run + kLazy) | (fresh & (cmax != kNegInf));
    const float m_ref = move ? cmax : m_run;
    alpha = (move & !fresh) ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.f;
    m_run = m_ref;
  }
  const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
  float e[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) e[4 * tt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[tt][i], scale_log2, neg_m));
  const tv_u32x4 pw = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                       pack_bf16x2(e[6], e[7])};
  pop = __builtin_bit_cast(tv_bf16x8, pw);
  return alpha;
}

// A chunk of visible prefix keys (no mask).  With two 16-row tiles per wave
// the products of one tile can run under the other's softmax: both tiles'
// S^T = K Q^T first, then per tile its softmax, rescaling (a uniform branch,
// rare with the lazy max) and O^T += V^T P^T.  The row sums come from one more
// product per tile, with a V^T operand of ones: the sums of the same bf16
// probabilities the PV product uses, with no VALU additions.
template <int D, int NTW>
__device__ __forceinline__ void mfma_chunk_plain(uint32_t slot, const tv_bf16x8 (&qop)[NTW][D / 32],
                                                 WaveAcc<D, NTW>& a, float scale_log2, int lane) {
  constexpr int KK = Chunk<D>::KK, DT = Chunk<D>::DT;
  const tv_bf16x8 ones = __builtin_bit_cast(tv_bf16x8, (tv_u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  tv_bf16x8 kop[2][KK], vop[DT];
  tv_f32x4 sc[NTW][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kop[tt][kk] = lds_read16(slot + (tt * KK + kk) * 1024 + lane * 16);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      tv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[tt][kk], qop[nt][kk], acc, 0, 0, 0);
      sc[nt][tt] = acc;
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vop[dt] = lds_vop<D>(slot + 2 * KK * 1024, dt, lane);
  // LLVM's interleave strategy 3 for matrix products beside exponentials
  // (measured: 70B-shaped share 758 -> 733 us, ragged 70.1 -> 68.6 us)
  __builtin_amdgcn_iglp_opt(3);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    tv_bf16x8 pop;
    const float alpha = softmax_plain(sc[nt], a.m_run[nt], scale_log2, pop);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) a.oacc[dt][nt] *= alpha;
      a.lacc[nt] *= alpha;
      a.l_run[nt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      a.oacc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pop, a.oacc[dt][nt], 0, 0, 0);
    a.lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop, a.lacc[nt], 0, 0, 0);
    __builtin_amdgcn_iglp_opt(3);
  }
}

// One 32-key chunk from an LDS slot: S^T = K Q^T, masked online softmax, O^T += V^T P^T.
template <int D, int NTW>
__device__ __forceinline__ void mfma_chunk(uint32_t slot, const tv_bf16x8 (&qop)[NTW][D / 32],
                                           WaveAcc<D, NTW>& a, const uint64_t (&alo)[NTW],
                                           const uint64_t (&ahi)[NTW], int key0, int P, int k_end,
                                           float scale_log2, int lane) {
  constexpr int KK = Chunk<D>::KK, DT = Chunk<D>::DT;
  if (key0 + 32 <= P && key0 + 32 <= k_end) {   // prefix keys only: no mask
    mfma_chunk_plain<D, NTW>(slot, qop, a, scale_log2, lane);
    return;
  }
  const int h4 = lane >> 4;
  tv_bf16x8 kop[2][KK], vop[DT];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kop[tt][kk] = lds_read16(slot + (tt * KK + kk) * 1024 + lane * 16);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vop[dt] = lds_vop<D>(slot + 2 * KK * 1024, dt, lane);

  // phase 1: scores of every row tile (independent MFMA chains)
  tv_f32x4 sc[NTW][2];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      tv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[tt][kk], qop[nt][kk], acc, 0, 0, 0);
      sc[nt][tt] = acc;
    }
  }
  // The request's last chunk: value slots at or past k_end hold no data (zero
  // them so that 0 * garbage cannot reach the sum).  Lane l holds keys
  // key0 + 4*(l/16) + e (e < 4) and key0 + 16 + 4*(l/16) + e - 4 (e >= 4).
  const bool plain = key0 + 32 <= P && key0 + 32 <= k_end;   // prefix keys only: no mask
  if (key0 + 32 > k_end) {
    const int kv = key0 + 4 * h4;   // element e: key kv + e (e < 4) or kv + 12 + e (e >= 4)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      tv_u32x4 w = __builtin_bit_cast(tv_u32x4, vop[dt]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (kv + (e < 4 ? e : 12 + e) >= k_end) {
          if (e & 1) w[e >> 1] &= 0x0000FFFFu;
          else w[e >> 1] &= 0xFFFF0000u;
        }
      }
      vop[dt] = __builtin_bit_cast(tv_bf16x8, w);
    }
  }
  // phase 2: mask, online softmax.  Lane l holds keys key0 + 16*tt + 4*(l/16) + i
  // of query row l % 16.  The max is taken over the raw scores (the scale is
  // positive) and the scale is folded into the exponent's FMA.  The running max
  // only moves when a row's max grows by more than kLazy (log2 units), so the
  // accumulators are rescaled rarely; probabilities stay below 2^kLazy.
  tv_bf16x8 pop[NTW];
  float alpha[NTW];
  bool any_rescale = false;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    if (!plain) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * tt + 4 * h4 + i;
          bool ok = key < k_end;
          if (ok && key >= P) ok = anc_bit(alo[nt], ahi[nt], key - P);
          sc[nt][tt][i] = ok ? sc[nt][tt][i] : kNegInf;
        }
      }
    }
    float rmax = fmaxf(fmaxf(fmaxf(sc[nt][0][0], sc[nt][0][1]), fmaxf(sc[nt][0][2], sc[nt][0][3])),
                       fmaxf(fmaxf(sc[nt][1][0], sc[nt][1][1]), fmaxf(sc[nt][1][2], sc[nt][1][3])));
    rmax = tv_rows_max(rmax);
    const float cmax = rmax * scale_log2;   // -inf stays -inf
    const bool move = cmax > a.m_run[nt] + kLazy || (a.m_run[nt] == kNegInf && cmax != kNegInf);
    const float m_ref = move ? cmax : a.m_run[nt];
    alpha[nt] = (move && a.m_run[nt] != kNegInf) ? __builtin_amdgcn_exp2f(a.m_run[nt] - m_ref) : 1.f;
    any_rescale |= alpha[nt] != 1.f;
    a.m_run[nt] = m_ref;
    const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
    float e[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[4 * tt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nt][tt][i], scale_log2, neg_m));
    a.l_run[nt] = a.l_run[nt] * alpha[nt] + (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
    const tv_u32x4 pw = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                         pack_bf16x2(e[6], e[7])};
    pop[nt] = __builtin_bit_cast(tv_bf16x8, pw);
  }
  if (__any(any_rescale)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) a.oacc[dt][nt] *= alpha[nt];
      a.lacc[nt] *= alpha[nt];
    }
  }
  // phase 3: O^T += V^T P^T for every row tile
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      a.oacc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pop[nt], a.oacc[dt][nt], 0, 0, 0);
}

// Key group 1 hands its (m, L, O) to group 0 through LDS (the ring is free:
// every DMA has landed and the last barrier has passed).  Wave wr of each
// group uses ring slot wr: O as [dt][nt][lane], then (m, L) as [nt][lane].
// L is the row total.  Ends with group 0 holding the combined state.
template <int D, int NTW, int KG>
__device__ __forceinline__ void group_handoff(const uint32_t (&slot_lds)[ring_steps<KG>() * KG], WaveAcc<D, NTW>& a,
                                              float (&L)[NTW], bool producer, int kg, int wr, int lane) {
  constexpr int DT = Chunk<D>::DT;
  typedef __attribute__((address_space(3))) tv_f32x4* lds_f32x4_ptr;
  typedef __attribute__((address_space(3))) tv_f32x2* lds_f2_ptr;
  const uint32_t mine = wr == 0 ? slot_lds[0] : wr == 1 ? slot_lds[1] : wr == 2 ? slot_lds[2] : slot_lds[3];
  lds_f32x4_ptr xo = (lds_f32x4_ptr)(uintptr_t)mine;
  lds_f2_ptr xml = (lds_f2_ptr)(uintptr_t)(mine + DT * NTW * 64 * 16);
  static_assert(DT * NTW * 64 * 16 + NTW * 64 * 8 <= Chunk<D>::BYTES && kMfmaWaves <= ring_steps<KG>() * KG,
                "hand-off buffers fit the ring");
  tv_lds_barrier();
  if (!producer && kg == 1) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) xo[(dt * NTW + nt) * 64 + lane] = a.oacc[dt][nt];
      xml[nt * 64 + lane] = (tv_f32x2){a.m_run[nt], L[nt]};
    }
  }
  tv_lds_barrier();
  if (producer || kg != 0) return;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const tv_f32x2 mb = xml[nt * 64 + lane];
    const float M = fmaxf(a.m_run[nt], mb.x);
    const float fa = a.m_run[nt] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(a.m_run[nt] - M);
    const float fb = mb.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mb.x - M);
    a.m_run[nt] = M;
    L[nt] = L[nt] * fa + mb.y * fb;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) a.oacc[dt][nt] = a.oacc[dt][nt] * fa + xo[(dt * NTW + nt) * 64 + lane] * fb;
  }
}

// Output rows of one MFMA wave: lane l holds O[row rbase + 16*nt + l%16][16*dt + 4*(l/16) + i].
template <int D, int NTW>
__device__ __forceinline__ void write_rows(const AttnParams& p, const WaveAcc<D, NTW>& a, const float (&L)[NTW],
                                           int b, int g, int rbase, int R, int lane) {
  constexpr int DT = Chunk<D>::DT;
  const int l16 = lane & 15, h4 = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int qrow = rbase + 16 * nt + l16;
    if (qrow >= R) continue;
    const float inv = 1.f / L[nt];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float v4[4] = {a.oacc[dt][nt][0] * inv, a.oacc[dt][nt][1] * inv, a.oacc[dt][nt][2] * inv,
                     a.oacc[dt][nt][3] * inv};
      store_out4<true, D>(p, b, g, qrow, 16 * dt + 4 * h4, v4);
    }
  }
}

// Split partials of the MFMA path, in the waves' own register layout: for
// slot s, 16-row block rb (= row in tile / 16) and d-tile pair j, lane l's 16
// bytes are the fp16 values of oacc[2j][.] then oacc[2j+1][.] times the row's
// power of two (O / L scaled as part_scale gives); the row's (m, L, inverse
// power) record sits at part_ml[s * rows_per_tile + row].  Written and read
// with 16-byte device-scope buffer accesses (cache policy sc1).
constexpr int kSc1 = 16;   // buffer instruction cache-policy bit: device scope
template <int D>
__device__ __forceinline__ uint32_t part_off(int rows_per_tile, int s, int rb, int j, int lane) {
  return (uint32_t)((((s * (rows_per_tile / 16) + rb) * (Chunk<D>::DT / 2) + j) * 64 + lane) * 16);
}

template <int D, int NTW>
__device__ __forceinline__ void store_partial(const AttnParams& p, const WaveAcc<D, NTW>& a, const float (&L)[NTW],
                                              int slot, int wr, int row0, int lane) {
  constexpr int DT = Chunk<D>::DT;
  const int l16 = lane & 15, h4 = lane >> 4;
  const size_t slot_bytes = (size_t)p.rows_per_tile * D * 2;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((char*)p.part_o + slot * slot_bytes, (short)0,
                                                                      (int)slot_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(p.part_ml + (size_t)slot * p.rows_per_tile, (short)0,
                                                                      p.rows_per_tile * 16, 0x00020000);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float inv = L[nt] > 0.f ? 1.f / L[nt] : 0.f;
    float amax = 0.f;   // the row's largest |O / L| over its four lanes sets the stored power of two
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(a.oacc[dt][nt][i] * inv));
    amax = tv_rows_max(amax);
    const float2 sc = part_scale(amax);
    const float f = inv * sc.x;
    const int rb = wr * NTW + nt;
#pragma unroll
    for (int j = 0; j < DT / 2; ++j) {
      const tv_f16x4 lo = __builtin_convertvector(a.oacc[2 * j][nt] * f, tv_f16x4);
      const tv_f16x4 hi = __builtin_convertvector(a.oacc[2 * j + 1][nt] * f, tv_f16x4);
      const tv_u32x4 w = __builtin_bit_cast(tv_u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      __builtin_amdgcn_raw_buffer_store_b128(w, ro, part_off<D>(p.rows_per_tile, 0, rb, j, lane), 0, kSc1);
    }
    if (h4 == 0) {
      const tv_u32x4 w = __builtin_bit_cast(tv_u32x4, (tv_f32x4){a.m_run[nt], L[nt], sc.y, 0.f});
      __builtin_amdgcn_raw_buffer_store_b128(w, rm, (uint32_t)((row0 + 16 * nt + l16) * 16), 0, kSc1);
    }
  }
}

// Co-resident grids: every split of a tile merges a slice of the tile's rows
// once all of them have published.  Thread-owned units are the 16-byte pieces
// of the partial layout (row block rb, d-tile pair j, lane): 8 values of one
// row.  The fold order is the same as in merge_partials (split kg, kg + KG,
// ... per key group, then group 1 into group 0), so both ways of merging give
// the same values.
template <int D, int NTW, int KG, int NT>
__device__ __forceinline__ void merge_slice(const AttnParams& p, int first, int n_active, int own_s, int b, int g,
                                            int r0, int R) {
  constexpr int DT = Chunk<D>::DT, JP = DT / 2;
  const int RW = p.rows_per_tile, units = (RW / 16) * JP * 64;
  const int u_begin = (int)((long long)units * own_s / n_active), u_end = (int)((long long)units * (own_s + 1) / n_active);
  const size_t slot_bytes = (size_t)RW * D * 2;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((char*)p.part_o + first * slot_bytes, (short)0,
                                                                      (int)(slot_bytes * n_active), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(p.part_ml + (size_t)first * RW, (short)0,
                                                                      RW * 16 * n_active, 0x00020000);
  constexpr int PB = 8;   // splits whose loads are in flight together
  for (int u = u_begin + (int)threadIdx.x; u < u_end; u += NT) {
    const int lane = u & 63, j = (u >> 6) % JP, rb = (u >> 6) / JP;
    const int row = rb * 16 + (lane & 15);
    float m[KG], l[KG];
    tv_f32x4 lo[KG], hi[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      m[k] = kNegInf;
      l[k] = 0.f;
      lo[k] = hi[k] = (tv_f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < n_active; s0 += PB) {
      tv_u32x4 po[PB], pm[PB];
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int sp = s0 + q;
        if (sp < n_active) {
          pm[q] = __builtin_amdgcn_raw_buffer_load_b128(rm, (uint32_t)((sp * RW + row) * 16), 0, kSc1);
          po[q] = __builtin_amdgcn_raw_buffer_load_b128(ro, part_off<D>(RW, sp, rb, j, lane), 0, kSc1);
        }
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int sp = s0 + q;
        if (sp >= n_active) break;
        const int k = KG == 1 ? 0 : sp % KG;
        const tv_f32x4 ml = __builtin_bit_cast(tv_f32x4, pm[q]);
        if (ml[0] == kNegInf) continue;
        const float M = fmaxf(m[k], ml[0]);
        const float fa = m[k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[k] - M);
        const float fb = __builtin_amdgcn_exp2f(ml[0] - M);
        m[k] = M;
        l[k] = l[k] * fa + ml[1] * fb;
        const float w = fb * ml[1] * ml[2];
        const tv_f16x8 h = __builtin_bit_cast(tv_f16x8, po[q]);
        lo[k] = lo[k] * fa + __builtin_convertvector(__builtin_shufflevector(h, h, 0, 1, 2, 3), tv_f32x4) * w;
        hi[k] = hi[k] * fa + __builtin_convertvector(__builtin_shufflevector(h, h, 4, 5, 6, 7), tv_f32x4) * w;
      }
    }
    if constexpr (KG > 1) {
      const float M = fmaxf(m[0], m[1]);
      const float fa = m[0] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[0] - M);
      const float fb = m[1] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[1] - M);
      l[0] = l[0] * fa + l[1] * fb;
      lo[0] = lo[0] * fa + lo[1] * fb;
      hi[0] = hi[0] * fa + hi[1] * fb;
    }
    const int qrow = r0 + row;
    if (qrow >= R) continue;
    const float inv = 1.f / l[0];
    const int d0 = 32 * j + 4 * (lane >> 4);
    float v4[4] = {lo[0][0] * inv, lo[0][1] * inv, lo[0][2] * inv, lo[0][3] * inv};
    store_out4<true, D>(p, b, g, qrow, d0, v4);
    float w4[4] = {hi[0][0] * inv, hi[0][1] * inv, hi[0][2] * inv, hi[0][3] * inv};
    store_out4<true, D>(p, b, g, qrow, d0 + 16, w4);
  }
}

// Co-resident grids: count this split in, wait (bounded) until every split of
// the tile has published, merge this split's slice of rows, then count it out;
// the split that completes the second count resets the counter for the next
// call.  A wait that expires (or TV_CHASE_SPIN_LIMIT < 0) gives the request
// TV_REQ_TIMEOUT and invalidates the workspace header: the counter may be
// left mid-count, so later calls report TV_REQ_BAD_WORKSPACE until the
// workspace is prepared again.  No split's wait depends on a workgroup that
// is not resident: the whole grid is.
template <int D, int NTW, int KG, int NT>
__device__ void merge_together(const AttnParams& p, int* flag, int first, int n_active, int own_s, bool ws_ok, int b,
                               int g, int r0, int R) {
  int* cnt = p.counters + first;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = ws_ok;
    if (ok) {
      __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.spin < 0) {
        ok = 0;
      } else {
        long long it = 0;
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n_active) {
          if (++it > p.spin) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (!ok) {
        // The request's first workgroup stores the request's status in its
        // prologue and ORs this flag after that store when its own wait
        // expires; the other workgroups OR it only after their whole split,
        // with the grid resident at once well after that prologue.
        if (p.status) __hip_atomic_fetch_or(p.status + b, (int)TV_REQ_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store((unsigned long long*)p.header, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    *flag = ok;
  }
  __syncthreads();
  if (*flag == 0) return;
  merge_slice<D, NTW, KG, NT>(p, first, n_active, own_s, b, g, r0, R);
  if (threadIdx.x == 0 && __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 2 * n_active - 1)
    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merging workgroup: MFMA wave wr of key group kg folds the tile's split
// partials kg, kg + KG, ... (in that order) into its rows' state, PB splits
// at a time with all their loads in flight together.
template <int D, int NTW, int KG>
__device__ __forceinline__ void merge_partials(const AttnParams& p, WaveAcc<D, NTW>& a, float (&L)[NTW], int first,
                                               int n_active, int kg, int wr, int row0, int lane) {
  constexpr int DT = Chunk<D>::DT, PB = NTW == 1 ? 4 : 2;
  const int l16 = lane & 15;
  const size_t slot_bytes = (size_t)p.rows_per_tile * D * 2;
  const size_t tile_bytes = slot_bytes * n_active;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((char*)p.part_o + first * slot_bytes, (short)0,
                                                                      (int)tile_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(p.part_ml + (size_t)first * p.rows_per_tile,
                                                                      (short)0, p.rows_per_tile * 16 * n_active, 0x00020000);
  for (int s0 = kg; s0 < n_active; s0 += KG * PB) {
    tv_u32x4 po[PB][NTW][DT / 2], pm[PB][NTW];
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int s = s0 + KG * k;
      if (s < n_active) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int rb = wr * NTW + nt;
          pm[k][nt] = __builtin_amdgcn_raw_buffer_load_b128(rm, (uint32_t)((s * p.rows_per_tile + row0 + 16 * nt + l16) * 16),
                                                            0, kSc1);
#pragma unroll
          for (int j = 0; j < DT / 2; ++j)
            po[k][nt][j] = __builtin_amdgcn_raw_buffer_load_b128(ro, part_off<D>(p.rows_per_tile, s, rb, j, lane), 0, kSc1);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      if (s0 + KG * k >= n_active) break;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const tv_f32x4 ml = __builtin_bit_cast(tv_f32x4, pm[k][nt]);
        if (ml[0] == kNegInf) continue;   // no key of that split is visible to the row
        const float M = fmaxf(a.m_run[nt], ml[0]);
        const float fa = a.m_run[nt] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(a.m_run[nt] - M);
        const float fb = __builtin_amdgcn_exp2f(ml[0] - M);
        a.m_run[nt] = M;
        L[nt] = L[nt] * fa + ml[1] * fb;
        const float w = fb * ml[1] * ml[2];   // the stored row is O / L times 1 / ml[2]
#pragma unroll
        for (int j = 0; j < DT / 2; ++j) {
          const tv_f16x8 h = __builtin_bit_cast(tv_f16x8, po[k][nt][j]);
          const tv_f32x4 lo = __builtin_convertvector(__builtin_shufflevector(h, h, 0, 1, 2, 3), tv_f32x4);
          const tv_f32x4 hi = __builtin_convertvector(__builtin_shufflevector(h, h, 4, 5, 6, 7), tv_f32x4);
          a.oacc[2 * j][nt] = a.oacc[2 * j][nt] * fa + lo * w;
          a.oacc[2 * j + 1][nt] = a.oacc[2 * j + 1][nt] * fa + hi * w;
        }
      }
    }
  }
}

// The key range of one split, step by step through an LDS ring of NS steps
// of KG chunks.  With KG key groups, group k's four MFMA waves take the
// chunks c = KG*step + k, so two waves share each SIMD and one's softmax runs
// beside the other's matrix products; the groups' (m, l, O) are merged through
// LDS at the end.  The producer wave sent the first NS-1 steps in the prologue
// and read the block rows of the next chunks.  Per step: the producer waits
// for its DMAs of the step (later steps stay in flight); one barrier (the step
// has landed and every MFMA wave is done with the previous one); the producer
// sends step s+NS-1 into the previous step's slots and reads the block rows
// of the following step (used one step later, so the LDS read's latency stays
// hidden) while the MFMA waves compute.  Issuing a DMA stalls the issuing wave
// until the memory pipeline takes it, so keeping all of them on one wave lets
// the chunks' compute run under the transfer of later ones.  The slots are
// distinct LDS objects and the stage loop is unrolled, so the compiler sees
// which DMA writes which slot and adds no waits of its own before the slot
// reads (the MFMA waves have no memory operations in flight).
template <int D, int NTW, int KG, bool CO>
__device__ __attribute__((always_inline)) void attn_mfma(const AttnParams& p, CommonSmem& cm, const int* tab,
                                                         const uint32_t (&slot_lds)[ring_steps<KG>() * KG],
                                                         const tv_bf16x8 (&qop)[NTW][D / 32],
                                                         const DmaLane& dl, int2 next_rows, int slot,
                                                         int n_active, int b, int g, int r0, int R, int P,
                                                         int k_begin, int k_end, int tab0, int ntab,
                                                         bool tree_in_range, int own_s, bool ws_ok) {
  constexpr int DT = Chunk<D>::DT, NB = Chunk<D>::NBLK, NS = ring_steps<KG>();
  constexpr int NW = kMfmaWaves * KG;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15;
  const int G = p.G;
  const bool producer = wave >= NW;
  // key group of an MFMA wave, or the group whose chunks a producer moves
  const int kg = producer ? wave - NW : wave / kMfmaWaves, wr = wave % kMfmaWaves;
  const int rbase = producer ? R : r0 + wr * 16 * NTW;   // this wave's first row (none for a producer)
  const int nchunks = (k_end - k_begin + 31) / 32;
  const int nsteps = (nchunks + KG - 1) / KG;

  uint64_t alo[NTW], ahi[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int qrow = rbase + 16 * nt + l16;
    const int node = qrow < R ? qrow / G : 0;
    alo[nt] = tree_in_range ? cm.anc[node][0] : 0ull;
    ahi[nt] = tree_in_range ? cm.anc[node][1] : 0ull;
  }
  WaveAcc<D, NTW> a;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    a.m_run[nt] = kNegInf;
    a.l_run[nt] = 0.f;
    a.lacc[nt] = (tv_f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) a.oacc[dt][nt] = (tv_f32x4){0.f, 0.f, 0.f, 0.f};
  }

  for (int st0 = 0; st0 < nsteps; st0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int st = st0 + s;
      if (st >= nsteps) break;
      if (producer) {
        // this producer's chunks of steps st+1 .. st+NS-2 stay in flight when those are full steps
        if (st + NS - 2 < nsteps - 1) wait_vmcnt<(NS - 2) * NB>();
        else wait_vmcnt<0>();
      }
      tv_lds_barrier();
      const uint32_t sslot = KG == 1 ? slot_lds[s] : (kg ? slot_lds[s * KG + 1] : slot_lds[s * KG]);
      if (producer) {
        const int sn = st + NS - 1;   // the step sent now, into the previous step's slots
        const int ps = (s + NS - 1) % NS;
        const uint32_t dst = KG == 1 ? slot_lds[ps] : (kg ? slot_lds[ps * KG + 1] : slot_lds[ps * KG]);
        const int c = KG * sn + kg;
        if (c < nchunks) dma_chunk<D>(p, dl, next_rows, k_begin + 32 * c, dst);
        if (c + KG < nchunks) next_rows = chunk_rows(tab, tab0, ntab, k_begin + 32 * (c + KG), p.lbs);
      } else {
        const int c = KG * st + kg;
        if (c < nchunks && rbase < R)
          mfma_chunk<D, NTW>(sslot, qop, a, alo, ahi, k_begin + 32 * c, P, k_end, p.scale_log2, lane);
      }
    }
  }

  // row totals of l (a lane holds the sum over its own keys of each chunk)
  float L[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) L[nt] = tv_rows_sum(a.l_run[nt]) + a.lacc[nt][0];
  if constexpr (KG > 1) group_handoff<D, NTW, KG>(slot_lds, a, L, producer, kg, wr, lane);
  const bool writer = !producer && kg == 0;   // group 0 holds the workgroup's state now

  if (n_active == 1) {
    if (writer) write_rows<D, NTW>(p, a, L, b, g, rbase, R, lane);
    return;
  }
  // split partial, then the tile's count; the last split merges
  const int first = slot - own_s;   // the tile's splits are slots first .. first + n_active - 1
  if (writer) store_partial<D, NTW>(p, a, L, slot, wr, rbase - r0, lane);
  if constexpr (CO) {
    merge_together<D, NTW, KG, mfma_threads<KG>()>(p, &cm.flag, first, n_active, own_s, ws_ok, b, g, r0, R);
    return;
  }
  if (!publish_split(p, &cm.flag, first, n_active, ws_ok)) return;
  if (!producer) {
    // every split's stored partial, this one's included, in split order: the
    // result does not depend on which split arrived last
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      a.m_run[nt] = kNegInf;
      L[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) a.oacc[dt][nt] = (tv_f32x4){0.f, 0.f, 0.f, 0.f};
    }
    merge_partials<D, NTW, KG>(p, a, L, first, n_active, kg, wr, rbase - r0, lane);
  }
  if constexpr (KG > 1) group_handoff<D, NTW, KG>(slot_lds, a, L, producer, kg, wr, lane);
  if (writer) write_rows<D, NTW>(p, a, L, b, g, rbase, R, lane);
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + first, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------

// Launch bounds: NTW = 1 leaves room for two workgroups per CU (ten waves,
// under 80 KB of LDS each); wider tiles take more of the register file.
template <bool kBF16, int NTW, int KG>
constexpr int wg_per_cu() { return (kBF16 && (NTW > 1 || KG > 1)) ? 1 : 2; }

template <bool kBF16, int NTW, int KG>
constexpr int block_threads() { return kBF16 ? mfma_threads<KG>() : kThreads; }

// CO: the whole grid is resident at once, so the splits of a tile merge
// together (each a slice of the rows) instead of the last one merging alone.
template <bool kBF16, int D, int NTW, int KG, bool CO>
__global__ __launch_bounds__((block_threads<kBF16, NTW, KG>()), (wg_per_cu<kBF16, NTW, KG>())) void tree_attn_kernel(AttnParams p) {
  constexpr int RW = kBF16 ? 64 * NTW : 16;
  constexpr int NT = block_threads<kBF16, NTW, KG>();
  constexpr int NW = kMfmaWaves * KG;   // MFMA waves; the waves after them are the producers
  __shared__ CommonSmem cm;
  const int t = threadIdx.x;
  // balanced plans: workgroup 0 reports every request whose sizes are malformed
  // (no workgroup is planned for those)
  if (p.balanced && blockIdx.x == 0 && t < 64 && p.status) {
    for (int b0 = 0; b0 < p.B; b0 += 64) {
      const int bb = b0 + t;
      if (bb < p.B) {
        const int st = shape_status(p, p.prefix_len[bb], p.n_nodes[bb]);
        if (st) p.status[bb] = st;
      }
    }
  }
  const SplitPlan sp = plan_split(p, blockIdx.x);
  const int b = sp.b, g = sp.g, rt = sp.rt;
  const bool designated = sp.shape_ok && g == 0 && rt == 0 && sp.s == 0;
  if (!sp.shape_ok) {
    // uniform plans: the request's first workgroup reports malformed sizes
    if (!p.balanced && g == 0 && rt == 0 && sp.s == 0 && t == 0 && p.status)
      p.status[b] = shape_status(p, sp.P, sp.n);
    return;
  }
  if (!sp.work) return;
  const int P = sp.P, n = sp.n;
  const int32_t* trow = p.table + (size_t)b * p.max_blocks;
  const int kps = sp.kps_ch * 32;
  const int k_begin = sp.s * kps;
  const int tab0 = k_begin / p.bs;
  const int R = n * p.G;
  const int r0 = rt * RW;
  const int keys_total = P + n;
  const int n_active = sp.splits;
  const int k_end = min(k_begin + kps, keys_total);
  // A tile split over keys hands its partials over through the workspace's
  // counters, which must have been prepared: the header is loaded with the
  // prologue's other loads and checked after its barrier.
  unsigned long long hdr[2] = {kWsMagic, ~0ull};

  if constexpr (kBF16) {
    // the ring: distinct LDS objects, one chunk each
    constexpr int NSLOT = ring_steps<KG>() * KG;
    static_assert(NSLOT == 4 || NSLOT == 8, "one LDS object per ring slot");
    __shared__ alignas(16) unsigned char ring0[Chunk<D>::BYTES];
    __shared__ alignas(16) unsigned char ring1[Chunk<D>::BYTES];
    __shared__ alignas(16) unsigned char ring2[Chunk<D>::BYTES];
    __shared__ alignas(16) unsigned char ring3[Chunk<D>::BYTES];
    __shared__ int tab[max_tab<NTW>()];   // (block, KV head) row index per block of this split
    uint32_t slots[NSLOT];   // LDS addresses of the slots
    slots[0] = lds_addr(ring0);
    slots[1] = lds_addr(ring1);
    slots[2] = lds_addr(ring2);
    slots[3] = lds_addr(ring3);
    if constexpr (NSLOT == 8) {
      __shared__ alignas(16) unsigned char ring4[Chunk<D>::BYTES];
      __shared__ alignas(16) unsigned char ring5[Chunk<D>::BYTES];
      __shared__ alignas(16) unsigned char ring6[Chunk<D>::BYTES];
      __shared__ alignas(16) unsigned char ring7[Chunk<D>::BYTES];
      slots[4 % NSLOT] = lds_addr(ring4);
      slots[5 % NSLOT] = lds_addr(ring5);
      slots[6 % NSLOT] = lds_addr(ring6);
      slots[7 % NSLOT] = lds_addr(ring7);
    }

    // one round trip: parents, this split's block-table entries and this
    // wave's query operands (rows past the request are masked later)
    constexpr int KQ = D / 32;
    tv_bf16x8 qop[NTW][KQ];
    if ((t >> 6) < NW) {
      const int lane = t & 63, l16 = lane & 15, h4 = lane >> 4;
      const int rbase = r0 + ((t >> 6) % kMfmaWaves) * 16 * NTW;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int qrow = rbase + 16 * nt + l16;
        const int node = min(qrow / p.G, p.n_max - 1), hh = qrow % p.G;
        const uint16_t* qp =
            (const uint16_t*)p.q + (((size_t)b * p.n_max + node) * p.Hq + (size_t)g * p.G + hh) * D + 8 * h4;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) qop[nt][kk] = load_bf16x8(qp + 32 * kk);
      }
    }
    if (t < kMaxNodes) cm.par[t] = (t < p.n_max) ? p.parent[(size_t)b * p.n_max + t] : -1;
    if (n_active > 1) {
      hdr[0] = p.header[0];
      hdr[1] = p.header[1];
    }
    const int ntab = min(p.max_blocks - tab0, (kps + p.bs - 1) / p.bs + 1);
    for (int i = t; i < ntab; i += NT) {
      const int blk = trow[tab0 + i];
      // ids outside the pool (flagged by the request's validation) read block 0
      tab[i] = (block_ok(blk, p.num_blocks) ? blk : 0) * p.Hkv + g;
    }
    if (t == 0) cm.flag = 0;
    __syncthreads();   // also completes the query loads before any DMA is in flight
    const bool ws_ok = (hdr[0] == kWsMagic) & (hdr[1] >= p.need);

    // parent array: parent[0] = -1 and 0 <= parent[i] < i
    if (t < n) {
      const int pi = cm.par[t];
      const bool ok = (t == 0) ? (pi == -1) : (pi >= 0 && pi < t);
      if (!ok) cm.flag = 1;
    }
    tv_lds_barrier();
    if (cm.flag) {
      if (designated && t == 0 && p.status) p.status[b] = TV_REQ_BAD_PARENT;
      return;
    }
    // The first chunks go out now, so their latency overlaps the rest of the
    // prologue (the sizes are valid, so every key and block-table index stays
    // inside this split's staged table).  From here on no workgroup leaves
    // before its DMAs have landed, and the barriers are LDS-only.
    const DmaLane dl = dma_lane<D>(t & 63);
    constexpr int NS = ring_steps<KG>();
    int2 next_rows = make_int2(0, 0);
    if ((t >> 6) >= NW) {
      // producer k moves the chunks k, k + KG, ...: steps 0 .. NS-2 now, and
      // the block rows of its chunk of step NS-1 read ahead
      const int pk = (t >> 6) - NW;
      const int nchunks = (k_end - k_begin + 31) / 32;
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) {
        const int c = KG * i + pk;
        if (c < nchunks)
          dma_chunk<D>(p, dl, chunk_rows(tab, tab0, ntab, k_begin + 32 * c, p.lbs), k_begin + 32 * c,
                       KG == 1 ? slots[i] : (pk ? slots[i * KG + 1] : slots[i * KG]));
      }
      const int c = KG * (NS - 1) + pk;
      if (c < nchunks) next_rows = chunk_rows(tab, tab0, ntab, k_begin + 32 * c, p.lbs);
    }
    if (designated) {
      // every block id used by positions [0, P + n) must name a pool block
      const int nblk = (P + n + p.bs - 1) / p.bs;
      for (int i = t; i < nblk; i += NT)
        if (!block_ok(trow[i], p.num_blocks)) cm.flag = 1;
      tv_lds_barrier();
      if (t == 0 && p.status) p.status[b] = (cm.flag ? TV_REQ_BAD_KV : 0) | (ws_ok ? 0 : TV_REQ_BAD_WORKSPACE);
      // keep going: loads from bad blocks are redirected
    }
    const bool tree_in_range = k_end > P;
    if (tree_in_range && t < 64) build_ancestor_bitmaps(cm.par, n, cm.anc, t);
    tv_lds_barrier();
    attn_mfma<D, NTW, KG, CO>(p, cm, tab, slots, qop, dl, next_rows, sp.slot, n_active, b, g, r0, R, P, k_begin, k_end,
                          tab0, ntab, tree_in_range, sp.s, ws_ok);
  } else {
    __shared__ ValuSmem<D> vs;
    if (t < kMaxNodes) cm.par[t] = (t < p.n_max) ? p.parent[(size_t)b * p.n_max + t] : -1;
    if (n_active > 1) {
      hdr[0] = p.header[0];
      hdr[1] = p.header[1];
    }
    if (t == 0) cm.flag = 0;
    __syncthreads();
    const bool ws_ok = (hdr[0] == kWsMagic) & (hdr[1] >= p.need);
    if (t < n) {
      const int pi = cm.par[t];
      const bool ok = (t == 0) ? (pi == -1) : (pi >= 0 && pi < t);
      if (!ok) cm.flag = 1;
    }
    __syncthreads();
    if (cm.flag) {
      if (designated && t == 0 && p.status) p.status[b] = TV_REQ_BAD_PARENT;
      return;
    }
    if (designated) {
      const int nblk = (P + n + p.bs - 1) / p.bs;
      for (int i = t; i < nblk; i += NT)
        if (!block_ok(trow[i], p.num_blocks)) cm.flag = 1;
      __syncthreads();
      if (t == 0 && p.status) p.status[b] = (cm.flag ? TV_REQ_BAD_KV : 0) | (ws_ok ? 0 : TV_REQ_BAD_WORKSPACE);
    }
    const bool tree_in_range = k_end > P;
    if (tree_in_range && t < 64) build_ancestor_bitmaps(cm.par, n, cm.anc, t);
    __syncthreads();
    const int rows = min(RW, R - r0);
    attn_valu<false, D>(p, vs, b, g, r0, rows, P, k_begin, k_end, tree_in_range, cm.anc);
    emit_valu<false, D, RW>(p, cm, vs, sp.slot, n_active, b, g, r0, rows);
    if (n_active > 1 && publish_split(p, &cm.flag, sp.slot - sp.s, n_active, ws_ok)) {
      merge_tile<false, D, NT>(p, sp.slot - sp.s, n_active, b, g, r0, rows);
      if (t == 0) __hip_atomic_store(p.counters + sp.slot - sp.s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int check_desc(const tv_attn_desc* d) {
  if (!d) return TV_ERR_INVALID_ARG;
  if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->max_blocks_per_seq < 1 ||
      d->num_blocks < 1)
    return TV_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads) return TV_ERR_INVALID_ARG;
  if (d->n_max < 1 || d->n_max > kMaxNodes) return TV_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (d->dtype != TV_F32 && d->dtype != TV_BF16) return TV_ERR_UNSUPPORTED;
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64 && d->block_size != 128)
    return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

// Rows per MFMA workgroup: 64 * NTW.  Every MFMA wave reads each chunk's 16 KB
// of operands from LDS once per 16*NTW rows, so wider tiles spend less on LDS
// reads and re-read each chunk from HBM / L2 fewer times (once per row tile),
// but leave fewer tiles to spread over the CUs (more key splits to merge).
// NTW = 2 when its tiles alone cover a quarter of the CUs.
int choose_ntw(const tv_attn_desc* d, int cu) {
  if (d->dtype != TV_BF16) return 1;
  const long long R = (long long)d->n_max * (d->n_q_heads / d->n_kv_heads);
  const long long pairs = (long long)d->batch * d->n_kv_heads;
  if (R >= 128 && pairs * ((R + 127) / 128) * 4 >= cu) return 2;
  return 1;
}

// Key groups: two sets of MFMA waves on alternate chunks of a split, each
// with its own producer wave (64-row tiles only: 128-row tiles need more
// registers than two waves per SIMD leave).  Measured on MI355X: the 4096-key
// chains 200 -> 193 us; 128-row tiles with one group stay better for the
// 70B-shaped share (1005 against 1058 us as 64-row tiles with two groups, and
// 790 against 1107 us as 128-row tiles with two groups whose MFMA waves issue
// their own chunks' DMAs, a quarter each, without producer waves).
int choose_kg(const tv_attn_desc* d, int ntw) {
  return (d->dtype == TV_BF16 && ntw == 1) ? 2 : 1;
}

// Host half of the split plan: which plan the device follows and how many
// workgroups and partial slots it may use.  Keys per split are chosen on the
// device from the requests' lengths, so none of this depends on how long a
// context the block table could hold, beyond the staged-table limit of
// max_keys_per_split keys per split.
//   Uniform: every tile gets `splits` splits, enough to give each CU one
//   workgroup (and enough for the longest sequence the table can hold).
//   Balanced (batches whose tiles alone leave CUs idle): the device spreads the
//   batch's chunk-tiles over `nwg` = one workgroup per CU; the grid covers the
//   most splits that can produce (nwg + tiles, or tiles * min_splits when a
//   split's reach is the limit).
int make_plan(const tv_attn_desc* d, int cu, int ntw, AttnPlan* pl) {
  const int G = d->n_q_heads / d->n_kv_heads;
  const long long Rmax = (long long)d->n_max * G;
  pl->ntw = ntw;
  pl->rows_per_tile = d->dtype == TV_BF16 ? 64 * ntw : 16;
  pl->row_tiles = (int)((Rmax + pl->rows_per_tile - 1) / pl->rows_per_tile);
  const long long tiles = (long long)d->batch * d->n_kv_heads * pl->row_tiles;
  const long long cap_ch = ((long long)d->max_blocks_per_seq * d->block_size + 31) / 32;
  const long long max_kps_ch = (ntw == 1 ? max_keys_per_split<1>() : max_keys_per_split<2>()) / 32;
  const long long min_splits = (cap_ch + max_kps_ch - 1) / max_kps_ch;
  pl->max_kps_ch = (int)max_kps_ch;
  pl->nwg = cu;
  long long grid, slots;
  // the balanced plan's device sums stay in 32 bits (chunk-tiles of the batch)
  if (d->batch > 1 && tiles < cu && tiles * cap_ch < 0x7fffffffLL) {
    pl->balanced = 1;
    pl->splits = 0;
    grid = tiles * min_splits;   // bounds the device plan's split count
    if (cu + tiles > grid) grid = cu + tiles;
    slots = grid;
  } else {
    pl->balanced = 0;
    long long s = tiles > 0 ? (cu + tiles - 1) / tiles : 1;
    if (s < min_splits) s = min_splits;
    if (s < 1) s = 1;
    pl->splits = (int)s;
    grid = tiles * s;
    slots = s > 1 ? grid : 0;
  }
  if (grid > 0x7fffffff || slots > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  pl->grid = (int)grid;
  pl->slots = (int)slots;
  // workspace (only when some tile may be split): the prepared-workspace
  // header, one counter per slot, then the partials
  size_t bytes = 0;
  pl->off_cnt = pl->off_o = pl->off_ml = 0;
  if (slots > 0) {
    const size_t esz = d->dtype == TV_BF16 ? 2 : 4;   // partial O element: fp16 for bf16 inputs
    pl->off_cnt = kWsHeader;
    pl->off_o = tv_align_up(pl->off_cnt + (size_t)slots * sizeof(int), 256);
    pl->off_ml = tv_align_up(pl->off_o + (size_t)slots * pl->rows_per_tile * (size_t)d->head_dim * esz, 256);
    bytes = pl->off_ml + (size_t)slots * pl->rows_per_tile * sizeof(float4);
    // the partials are addressed through buffer resources with 32-bit sizes
    if (bytes >= (1ull << 31)) return TV_ERR_UNSUPPORTED;
  }
  pl->bytes = tv_align_up(bytes, 256);
  return TV_OK;
}

typedef void (*AttnKernel)(AttnParams);

// Workgroups of `k` one CU holds at once (registers and LDS decide; cached per
// device and kernel, 0 when the query fails).
int resident_per_cu(AttnKernel k, int threads) {
  static std::mutex mu;
  static struct { int dev; AttnKernel k; int nb; } cache[64];
  static int n_cache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_cache; ++i)
    if (cache[i].dev == dev && cache[i].k == k) return cache[i].nb;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, threads, 0) != hipSuccess) nb = 0;
  if (n_cache < 64) cache[n_cache++] = {dev, k, nb};
  return nb;
}

template <bool CO>
AttnKernel pick_kernel_co(const tv_attn_desc* d, int ntw, int kg) {
  const bool bf = d->dtype == TV_BF16;
  if (d->head_dim == 128) {
    if (!bf) return tree_attn_kernel<false, 128, 1, 1, false>;
    if (kg == 2) return tree_attn_kernel<true, 128, 1, 2, CO>;
    return ntw == 2 ? tree_attn_kernel<true, 128, 2, 1, CO> : tree_attn_kernel<true, 128, 1, 1, CO>;
  }
  if (!bf) return tree_attn_kernel<false, 64, 1, 1, false>;
  if (kg == 2) return tree_attn_kernel<true, 64, 1, 2, CO>;
  return ntw == 2 ? tree_attn_kernel<true, 64, 2, 1, CO> : tree_attn_kernel<true, 64, 1, 1, CO>;
}

AttnKernel pick_kernel(const tv_attn_desc* d, int ntw, int kg) { return pick_kernel_co<false>(d, ntw, kg); }

int plan_for(const tv_attn_desc* d, AttnPlan* pl, AttnKernel* kern) {
  int cu = 0;
  int rc = tv_device_cu_count(&cu);
  if (rc != TV_OK) return rc;
  const int ntw = choose_ntw(d, cu);
  const int kg = choose_kg(d, ntw);
  rc = make_plan(d, cu, ntw, pl);
  pl->kg = kg;
  if (kern) *kern = pick_kernel(d, ntw, kg);
  return rc;
}

}  // namespace

extern "C" size_t tree_attn_workspace_size(const tv_attn_desc* desc) {
  if (check_desc(desc) != TV_OK) return 0;
  AttnPlan pl;
  if (plan_for(desc, &pl, nullptr) != TV_OK) return 0;
  return pl.bytes;
}

static int tree_attn_forward_impl(const tv_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* prefix_len, const int32_t* n_nodes,
                                 const int32_t* parent, void* out, int32_t* status, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!q || !k_cache || !v_cache || !block_table || !prefix_len || !n_nodes || !parent || !out)
    return TV_ERR_INVALID_ARG;
  if ((((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15) != 0)
    return TV_ERR_INVALID_ARG;   // 16-byte vector loads and stores
  AttnPlan pl;
  AttnKernel kern = nullptr;
  rc = plan_for(desc, &pl, &kern);
  if (rc != TV_OK) return rc;
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes)) return TV_ERR_WORKSPACE;
  if (pl.bytes > 0 && ((uintptr_t)workspace & 255) != 0) return TV_ERR_INVALID_ARG;

  AttnParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.table = block_table;
  p.prefix_len = prefix_len;
  p.n_nodes = n_nodes;
  p.parent = parent;
  p.out = out;
  p.status = status;
  p.header = (const unsigned long long*)workspace;
  p.counters = (int*)((char*)workspace + pl.off_cnt);
  p.part_o = (char*)workspace + pl.off_o;
  p.part_ml = (float4*)((char*)workspace + pl.off_ml);
  p.need = pl.bytes;
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = desc->n_q_heads / desc->n_kv_heads;
  p.D = desc->head_dim;
  p.bs = desc->block_size;
  p.lbs = __builtin_ctz((unsigned)desc->block_size);
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  const float scale = desc->sm_scale > 0.f ? desc->sm_scale : 1.f / sqrtf((float)desc->head_dim);
  p.scale_log2 = scale * kLog2e;
  p.rows_per_tile = pl.rows_per_tile;
  p.row_tiles = pl.row_tiles;
  p.balanced = pl.balanced;
  p.splits = pl.splits;
  p.nwg = pl.nwg;
  p.max_kps_ch = pl.max_kps_ch;
  p.grid = pl.grid;
  p.spin = tv_chase_spin_limit(kMergeSpinLimit);
  p.coresident = 0;
  if (pl.grid > 0) {
    const int threads = desc->dtype != TV_BF16 ? kThreads : (pl.kg == 2 ? mfma_threads<2>() : mfma_threads<1>());
    if (pl.slots > 0 && desc->dtype == TV_BF16) {
      // the whole grid fits on the CUs at once: the splits of a tile merge together
      AttnKernel co = pick_kernel_co<true>(desc, pl.ntw, pl.kg);
      int cu = 0;
      if (tv_device_cu_count(&cu) == TV_OK && (long long)resident_per_cu(co, threads) * cu >= pl.grid) {
        p.coresident = 1;
        kern = co;
      }
    }
    hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(threads), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  }
  return TV_OK;
}

extern "C" int tree_attn_forward(const tv_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* prefix_len, const int32_t* n_nodes,
                                 const int32_t* parent, void* out, int32_t* status, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_attn_forward");
  if (tv_debug_enabled() && desc && desc->batch > 0) {
    tv_debug_trees("tree_attn_forward", parent, n_nodes, desc->batch, desc->n_max, stream);
    tv_debug_kv("tree_attn_forward", block_table, prefix_len, n_nodes, desc->batch, desc->max_blocks_per_seq, desc->block_size, desc->num_blocks, stream);
  }
  return tv_debug_finish("tree_attn_forward", tree_attn_forward_impl(desc, q, k_cache, v_cache, block_table, prefix_len, n_nodes, parent, out, status, workspace, workspace_bytes, stream), stream);
}
