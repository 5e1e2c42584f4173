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
// contiguous key range (split-K over the prefix, FlashDecoding-style); its four
// waves interleave 32-key chunks of that range and merge their online-softmax
// partials in LDS.  When a pair needs several key splits, each workgroup writes
// its (m, l, O) partial to the workspace and the last workgroup to arrive on the
// tile merges them by log-sum-exp and writes the output (no second kernel).
//
// Rows per pair >= 16 with bf16 inputs run on MFMA (v_mfma_f32_16x16x32_bf16):
//   S^T[key][row] = K Q^T  then  O^T[d][row] += V^T P^T,
// laid out so that a lane always owns one query row (lane % 16): the softmax
// state is lane-local, and the C layout of S^T feeds the B operand of the PV
// product without cross-lane moves.  Values are stored transposed per block
// ([D][block] per head) so the PV operand (8 consecutive keys of one d) is a
// single 16-byte load.  Fewer rows (or fp32 inputs) run on a VALU path.
//
// Tree mask: each wavefront builds the ancestor bitmaps of all nodes (two
// 64-bit words per node, n <= 128) from the parent array by pointer jumping
// with lane shuffles, then tests one bit per (row, tree key).

#include "tv_common.h"

#include <math.h>
#include <mutex>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNodes = 128;
constexpr int kMaxSplits = 32;   // key splits per (request, KV head, row tile)
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
  float* part_o;    // [tiles][splits][rows_per_tile][D]
  float* part_ml;   // [tiles][splits][rows_per_tile][2]
  int* counters;    // [tiles]
  int B, n_max, Hq, Hkv, G, D, bs, max_blocks, num_blocks;
  float scale_log2;
  int rows_per_tile, row_tiles, splits, keys_per_split, total;
};

struct AttnPlan {
  int rows_per_tile, row_tiles, splits, keys_per_split, nt;
  size_t off_ml, off_cnt, bytes;
};

// ---------------------------------------------------------------------------
// ancestor bitmaps
// ---------------------------------------------------------------------------

// Wave-cooperative pointer jumping: node j lives in lane j % 64, slot j / 64.
// After round r every node holds its ancestors within distance < 2^r; seven
// rounds cover any depth below 128.
__device__ void build_ancestor_bitmaps(const int32_t* par, int n, uint64_t (*anc)[2], int lane) {
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

__device__ __forceinline__ bool anc_bit(uint64_t lo, uint64_t hi, int w) {
  return w < 64 ? ((lo >> w) & 1ull) : ((hi >> (w - 64)) & 1ull);
}

__device__ __forceinline__ bool block_ok(int blk, int num_blocks) {
  return blk >= 0 && blk < num_blocks;
}

// ---------------------------------------------------------------------------
// shared state of one workgroup
// ---------------------------------------------------------------------------

template <int RPT, int D>
struct AttnSmem {
  uint64_t anc[kMaxNodes][2];
  float o[RPT][D + 4];          // unnormalised output rows (log2-domain softmax)
  float m[RPT];
  float l[RPT];
  float wm[4][RPT];             // per-wave partial m / l before the intra-workgroup merge
  float wl[4][RPT];
  // VALU path scratch
  float qs[16][D];
  float sc[4][16][64];          // per-wave probability strips; split weights of the merge later
  int flag;
};

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

template <bool kBF16, int D, int RPT, int RV>
__device__ void attn_valu_rows(const AttnParams& p, AttnSmem<RPT, D>& sm, int b, int g, int r0, int rows,
                               int P, int k_begin, int k_end, bool tree_in_range) {
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
    int blk = valid ? trow[key / p.bs] : -1;
    valid = valid && block_ok(blk, p.num_blocks);
    if (valid) {
      size_t base = (((size_t)blk * p.Hkv + g) * p.bs + key % p.bs) * D;
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
        ok = tree_in_range && anc_bit(sm.anc[node][0], sm.anc[node][1], key - P);
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
    // PV: lane = d (values are stored as [d][slot])
#pragma unroll
    for (int r = 0; r < RV; ++r) {
#pragma unroll
      for (int j = 0; j < DJ; ++j) o[r][j] *= alpha[r];
    }
#pragma unroll 1
    for (int k8 = 0; k8 < 64; k8 += 8) {
      const int kk = kb + k8;
      if (kk >= k_end) break;
      const int vb = trow[kk / p.bs];
      if (!block_ok(vb, p.num_blocks)) continue;
      float vv[DJ][8];
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        size_t off = (((size_t)vb * p.Hkv + g) * D + lane + 64 * j) * p.bs + kk % p.bs;
        load8<kBF16>(p.v, off, vv[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk + e >= k_end) vv[j][e] = 0.f;   // slots past the request hold no data
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

template <bool kBF16, int D, int RPT>
__device__ void attn_valu(const AttnParams& p, AttnSmem<RPT, D>& sm, int b, int g, int r0, int rows,
                          int P, int k_begin, int k_end, bool tree_in_range) {
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
  if (rv <= 1) attn_valu_rows<kBF16, D, RPT, 4>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range);
  else if (rv == 2) attn_valu_rows<kBF16, D, RPT, 8>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range);
  else if (rv == 3) attn_valu_rows<kBF16, D, RPT, 12>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range);
  else attn_valu_rows<kBF16, D, RPT, 16>(p, sm, b, g, r0, rows, P, k_begin, k_end, tree_in_range);
}

// ---------------------------------------------------------------------------
// MFMA path: 16*NT rows, bf16
// ---------------------------------------------------------------------------

__device__ __forceinline__ tv_bf16x8 load_bf16x8(const uint16_t* ptr) {
  return __builtin_bit_cast(tv_bf16x8, *(const tv_u32x4*)ptr);
}

template <int D, int NT>
__device__ void attn_mfma(const AttnParams& p, AttnSmem<16 * NT, D>& sm, int b, int g, int r0, int R,
                          int P, int n, int k_begin, int k_end, bool tree_in_range) {
  constexpr int KK = D / 32;   // 32-wide d chunks of the QK^T contraction
  constexpr int DT = D / 16;   // 16-wide d tiles of the PV product
  constexpr int RPT = 16 * NT;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, h4 = lane >> 4;
  const int G = p.G;
  const uint16_t* qg = (const uint16_t*)p.q;
  const uint16_t* kg = (const uint16_t*)p.k;
  const uint16_t* vg = (const uint16_t*)p.v;
  const int32_t* trow = p.table + (size_t)b * p.max_blocks;

  tv_bf16x8 qop[NT][KK];
  uint64_t alo[NT], ahi[NT];
  const tv_bf16x8 zero8 = {};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int qrow = r0 + 16 * nt + l16;
    bool ok = qrow < R;
    int node = ok ? qrow / G : 0, hh = ok ? qrow % G : 0;
    const uint16_t* qp = qg + (((size_t)b * p.n_max + node) * p.Hq + (size_t)g * G + hh) * D + 8 * h4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[nt][kk] = ok ? load_bf16x8(qp + 32 * kk) : zero8;
    alo[nt] = tree_in_range ? sm.anc[node][0] : 0ull;
    ahi[nt] = tree_in_range ? sm.anc[node][1] : 0ull;
  }

  float m_run[NT], l_run[NT];
  tv_f32x4 oacc[DT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt][nt] = (tv_f32x4){0.f, 0.f, 0.f, 0.f};
  }

  const int nchunks = (k_end - k_begin + 31) / 32;
  for (int c = wave; c < nchunks; c += 4) {
    const int key0 = k_begin + 32 * c;
    // K operand rows: S^T row i of tile t is key key0 + 8*(i/4) + 4*t + i%4, so the
    // C layout gives lane l the keys key0 + 8*(l/16) + 4*t + j (j = 0..3).
    tv_bf16x8 kop[2][KK];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int key = key0 + 8 * (l16 >> 2) + 4 * tt + (l16 & 3);
      bool ok = key < k_end;
      int blk = ok ? trow[key / p.bs] : -1;
      ok = ok && block_ok(blk, p.num_blocks);
      const uint16_t* kp = kg + (((size_t)(ok ? blk : 0) * p.Hkv + g) * p.bs + key % p.bs) * D + 8 * h4;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[tt][kk] = ok ? load_bf16x8(kp + 32 * kk) : zero8;
    }
    // V operand: lane l holds d = 16*dt + l%16 for keys key0 + 8*(l/16) .. +7
    tv_bf16x8 vop[DT];
    {
      int kv = key0 + 8 * h4;
      bool ok = kv < k_end;
      int blk = ok ? trow[kv / p.bs] : -1;
      ok = ok && block_ok(blk, p.num_blocks);
      const uint16_t* vp = vg + (((size_t)(ok ? blk : 0) * p.Hkv + g) * D + l16) * p.bs + kv % p.bs;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vop[dt] = ok ? load_bf16x8(vp + (size_t)16 * dt * p.bs) : zero8;
      if (ok && kv + 8 > k_end) {
        // the last keys of the request share a block with slots that hold no data
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          tv_u32x4 w = __builtin_bit_cast(tv_u32x4, vop[dt]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (kv + j >= k_end) {
              if (j & 1) w[j >> 1] &= 0x0000FFFFu;
              else w[j >> 1] &= 0xFFFF0000u;
            }
          }
          vop[dt] = __builtin_bit_cast(tv_bf16x8, w);
        }
      }
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      tv_f32x4 s[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        tv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[tt][kk], qop[nt][kk], acc, 0, 0, 0);
        s[tt] = acc;
      }
      // scale, mask, chunk max
      float cmax = kNegInf;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int key = key0 + 8 * h4 + 4 * tt + i;
          bool ok = key < k_end;
          if (ok && key >= P) ok = anc_bit(alo[nt], ahi[nt], key - P);
          float v = ok ? s[tt][i] * p.scale_log2 : kNegInf;
          s[tt][i] = v;
          cmax = fmaxf(cmax, v);
        }
      }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      float m_new = fmaxf(m_run[nt], cmax);
      float m_use = (m_new == kNegInf) ? 0.f : m_new;
      float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      m_run[nt] = m_new;
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          float e0 = __builtin_amdgcn_exp2f(s[tt][i] - m_use);
          float e1 = __builtin_amdgcn_exp2f(s[tt][i + 1] - m_use);
          psum += e0 + e1;
          pk[2 * tt + (i >> 1)] = (uint32_t)tv_f32_to_bf16_bits(e0) | ((uint32_t)tv_f32_to_bf16_bits(e1) << 16);
        }
      }
      l_run[nt] = l_run[nt] * alpha + psum;
      tv_u32x4 pw = {pk[0], pk[1], pk[2], pk[3]};
      tv_bf16x8 pop = __builtin_bit_cast(tv_bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        oacc[dt][nt] *= alpha;
        oacc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pop, oacc[dt][nt], 0, 0, 0);
      }
    }
  }

  // merge the four waves' partials: m and l first, then the rescaled O sums
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l_run[nt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    l_run[nt] = lt;
    if (h4 == 0) {
      sm.wm[wave][16 * nt + l16] = m_run[nt];
      sm.wl[wave][16 * nt + l16] = lt;
    }
  }
  __syncthreads();
  float wsc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r = 16 * nt + l16;
    float M = fmaxf(fmaxf(sm.wm[0][r], sm.wm[1][r]), fmaxf(sm.wm[2][r], sm.wm[3][r]));
    wsc[nt] = (m_run[nt] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - M);
  }
  if (t < RPT) {
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
      for (int nt = 0; nt < NT; ++nt) {
        int r = 16 * nt + l16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float* dst = &sm.o[r][16 * dt + 4 * h4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = wsc[nt] * oacc[dt][nt][i];
            dst[i] = (w == 0) ? v : dst[i] + v;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// output / split-K merge
// ---------------------------------------------------------------------------

template <bool kBF16, int D>
__device__ __forceinline__ void store_out4(const AttnParams& p, int b, int g, int qrow, int d, const float* v4) {
  int node = qrow / p.G, hh = qrow % p.G;
  size_t off = (((size_t)b * p.n_max + node) * p.Hq + (size_t)g * p.G + hh) * D + d;
  if (kBF16) {
    uint32_t lo = (uint32_t)tv_f32_to_bf16_bits(v4[0]) | ((uint32_t)tv_f32_to_bf16_bits(v4[1]) << 16);
    uint32_t hi = (uint32_t)tv_f32_to_bf16_bits(v4[2]) | ((uint32_t)tv_f32_to_bf16_bits(v4[3]) << 16);
    uint2 w = make_uint2(lo, hi);
    *(uint2*)((uint16_t*)p.out + off) = w;
  } else {
    *(tv_f32x4*)((float*)p.out + off) = (tv_f32x4){v4[0], v4[1], v4[2], v4[3]};
  }
}

template <bool kBF16, int D, int RPT>
__device__ void emit(const AttnParams& p, AttnSmem<RPT, D>& sm, int tile, int split, int n_active, int b,
                     int g, int r0, int rows) {
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
  // write this split's partial
  size_t prow = ((size_t)tile * p.splits + split) * RPT;
  for (int idx = t; idx < rows * (D / 4); idx += kThreads) {
    int r = idx / (D / 4), d = 4 * (idx % (D / 4));
    *(tv_f32x4*)(p.part_o + (prow + r) * D + d) = (tv_f32x4){sm.o[r][d], sm.o[r][d + 1], sm.o[r][d + 2], sm.o[r][d + 3]};
  }
  if (t < rows) {
    p.part_ml[(prow + t) * 2] = sm.m[t];
    p.part_ml[(prow + t) * 2 + 1] = sm.l[t];
  }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    int prev = atomicAdd(&p.counters[tile], 1);
    sm.flag = (prev == n_active - 1);
  }
  __syncthreads();
  if (!sm.flag) return;
  // acquire: the agent-scope fence invalidates this CU's L1 and the stale lines
  // of this XCD's L2, so the plain loads below see the other splits' partials
  __threadfence();
  // last arrival: log-sum-exp merge of the n_active partials of this tile
  const size_t base = (size_t)tile * p.splits * RPT;
  static_assert(kMaxSplits * RPT <= 4 * 16 * 64, "split weights must fit the scratch strips");
  float(*wgt)[RPT] = reinterpret_cast<float(*)[RPT]>(&sm.sc[0][0][0]);
  if (t < rows) {
    float M = kNegInf;
    for (int s = 0; s < n_active; ++s) M = fmaxf(M, p.part_ml[(base + (size_t)s * RPT + t) * 2]);
    float L = 0.f;
    for (int s = 0; s < n_active; ++s) {
      const float2 ml = *(const float2*)&p.part_ml[(base + (size_t)s * RPT + t) * 2];
      const float w = (ml.x == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      L += w * ml.y;
      wgt[s][t] = w;
    }
    sm.l[t] = L;
  }
  __syncthreads();
  for (int idx = t; idx < rows * (D / 4); idx += kThreads) {
    const int r = idx / (D / 4), d = 4 * (idx % (D / 4));
    tv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_active; ++s) {
      const size_t pr = base + (size_t)s * RPT + r;
      acc += wgt[s][r] * *(const tv_f32x4*)&p.part_o[pr * D + d];
    }
    const float inv = 1.f / sm.l[r];
    float v4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    store_out4<kBF16, D>(p, b, g, r0 + r, d, v4);
  }
  if (t == 0) p.counters[tile] = 0;   // leave the workspace ready for the next call
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------

template <bool kBF16, int D, int NT>
__global__ __launch_bounds__(kThreads) void tree_attn_kernel(AttnParams p) {
  constexpr int RPT = kBF16 ? 16 * NT : 16;
  __shared__ AttnSmem<RPT, D> sm;
  const int t = threadIdx.x;
  const int lid = tv_xcd_remap(blockIdx.x, p.total);
  const int tile = lid / p.splits, split = lid % p.splits;
  const int bg = tile / p.row_tiles, rt = tile % p.row_tiles;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const bool designated = (g == 0 && rt == 0 && split == 0);

  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  int flags = 0;
  if (n < 1 || n > p.n_max) flags |= TV_REQ_BAD_NNODES;
  else if (P < 0 || (long long)P + n > (long long)p.max_blocks * p.bs) flags |= TV_REQ_BAD_KV;
  if (flags) {
    if (designated && t == 0 && p.status) p.status[b] = flags;
    return;
  }
  const int32_t* par = p.parent + (size_t)b * p.n_max;
  // parent array: parent[0] = -1 and 0 <= parent[i] < i
  if (t == 0) sm.flag = 0;
  __syncthreads();
  if (t < n) {
    int pi = par[t];
    bool ok = (t == 0) ? (pi == -1) : (pi >= 0 && pi < t);
    if (!ok) sm.flag = 1;
  }
  __syncthreads();
  if (sm.flag) {
    if (designated && t == 0 && p.status) p.status[b] = TV_REQ_BAD_PARENT;
    return;
  }
  if (designated) {
    // every block id used by positions [0, P + n) must name a pool block
    const int32_t* trow = p.table + (size_t)b * p.max_blocks;
    int nblk = (P + n + p.bs - 1) / p.bs;
    __syncthreads();
    for (int i = t; i < nblk; i += kThreads)
      if (!block_ok(trow[i], p.num_blocks)) sm.flag = 1;
    __syncthreads();
    if (t == 0 && p.status) p.status[b] = sm.flag ? TV_REQ_BAD_KV : 0;
    // keep going: loads from bad blocks are skipped, and the other workgroups
    // of this tile count on this one in the split-K hand-off
  }

  const int R = n * p.G;
  const int r0 = rt * RPT;
  if (r0 >= R) return;
  const int keys_total = P + n;
  const int n_active = (keys_total + p.keys_per_split - 1) / p.keys_per_split;
  if (split >= n_active) return;
  const int k_begin = split * p.keys_per_split;
  const int k_end = min(k_begin + p.keys_per_split, keys_total);
  const bool tree_in_range = k_end > P;
  if (tree_in_range && t < 64) build_ancestor_bitmaps(par, n, sm.anc, t);
  __syncthreads();

  int rows = min(RPT, R - r0);
  if (kBF16 && R >= 16) {
    if constexpr (kBF16) attn_mfma<D, NT>(p, sm, b, g, r0, R, P, n, k_begin, k_end, tree_in_range);
  } else {
    attn_valu<kBF16, D, RPT>(p, sm, b, g, r0, min(rows, 16), P, k_begin, k_end, tree_in_range);
    rows = min(rows, 16);
  }
  emit<kBF16, D, RPT>(p, sm, tile, split, n_active, b, g, r0, rows);
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

// MFMA row tile: 16 * NT query rows per workgroup (bf16 only).
int choose_nt(const tv_attn_desc* d) {
  const long long Rmax = (long long)d->n_max * (d->n_q_heads / d->n_kv_heads);
  if (d->dtype != TV_BF16) return 1;
  return Rmax >= 64 ? 4 : (Rmax >= 32 ? 2 : 1);
}

int make_plan(const tv_attn_desc* d, int cu, int wg_per_cu, AttnPlan* pl) {
  const int G = d->n_q_heads / d->n_kv_heads;
  const long long Rmax = (long long)d->n_max * G;
  const int nt = choose_nt(d);
  pl->nt = nt;
  pl->rows_per_tile = d->dtype == TV_BF16 ? 16 * nt : 16;
  pl->row_tiles = (int)((Rmax + pl->rows_per_tile - 1) / pl->rows_per_tile);
  const long long max_keys = (long long)d->max_blocks_per_seq * d->block_size;
  const long long base = (long long)d->batch * d->n_kv_heads * pl->row_tiles;
  long long target = (long long)wg_per_cu * cu;
  long long splits = base > 0 ? (target + base - 1) / base : 1;
  long long max_splits = (max_keys + 127) / 128;
  if (max_splits > kMaxSplits) max_splits = kMaxSplits;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  long long kps = (max_keys + splits - 1) / splits;
  kps = (kps + 31) / 32 * 32;
  splits = (max_keys + kps - 1) / kps;
  if (kps > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  pl->splits = (int)splits;
  pl->keys_per_split = (int)kps;
  const size_t tiles = (size_t)base;
  size_t bytes = 0;
  if (pl->splits > 1) {
    bytes = tiles * pl->splits * pl->rows_per_tile * (size_t)d->head_dim * sizeof(float);
    pl->off_ml = tv_align_up(bytes, 256);
    bytes = pl->off_ml + tiles * pl->splits * pl->rows_per_tile * 2 * sizeof(float);
    pl->off_cnt = tv_align_up(bytes, 256);
    bytes = pl->off_cnt + tiles * sizeof(int);
  } else {
    pl->off_ml = pl->off_cnt = 0;
  }
  pl->bytes = tv_align_up(bytes, 256);
  return TV_OK;
}

typedef void (*AttnKernel)(AttnParams);

AttnKernel pick_kernel(const tv_attn_desc* d, int nt) {
  const bool bf = d->dtype == TV_BF16;
  if (d->head_dim == 128) {
    if (!bf) return tree_attn_kernel<false, 128, 1>;
    return nt == 4 ? tree_attn_kernel<true, 128, 4> : nt == 2 ? tree_attn_kernel<true, 128, 2> : tree_attn_kernel<true, 128, 1>;
  }
  if (!bf) return tree_attn_kernel<false, 64, 1>;
  return nt == 4 ? tree_attn_kernel<true, 64, 4> : nt == 2 ? tree_attn_kernel<true, 64, 2> : tree_attn_kernel<true, 64, 1>;
}

// Resident workgroups per CU of one kernel instance on the current device (cached).
int occupancy(AttnKernel k, int* out) {
  static std::mutex mu;
  static const void* keys[16];
  static int vals[16];
  static int dev_of[16];
  static int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TV_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (keys[i] == (const void*)k && dev_of[i] == dev) {
      *out = vals[i];
      return TV_OK;
    }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, kThreads, 0) != hipSuccess) return TV_ERR_HIP;
  if (nb < 1) nb = 1;
  if (n < 16) {
    keys[n] = (const void*)k;
    vals[n] = nb;
    dev_of[n] = dev;
    ++n;
  }
  *out = nb;
  return TV_OK;
}

int plan_for(const tv_attn_desc* d, AttnPlan* pl, AttnKernel* kern) {
  int cu = 0, occ = 0;
  int rc = tv_device_cu_count(&cu);
  if (rc != TV_OK) return rc;
  const int nt = choose_nt(d);
  AttnKernel k = pick_kernel(d, nt);
  rc = occupancy(k, &occ);
  if (rc != TV_OK) return rc;
  rc = make_plan(d, cu, occ, pl);
  if (kern) *kern = k;
  return rc;
}

}  // namespace

extern "C" size_t tree_attn_workspace_size(const tv_attn_desc* desc) {
  if (check_desc(desc) != TV_OK) return 0;
  AttnPlan pl;
  if (plan_for(desc, &pl, nullptr) != TV_OK) return 0;
  return pl.bytes;
}

extern "C" int tree_attn_forward(const tv_attn_desc* desc, const void* q, const void* k_cache,
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
  p.part_o = (float*)workspace;
  p.part_ml = (float*)((char*)workspace + pl.off_ml);
  p.counters = (int*)((char*)workspace + pl.off_cnt);
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = desc->n_q_heads / desc->n_kv_heads;
  p.D = desc->head_dim;
  p.bs = desc->block_size;
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  float scale = desc->sm_scale > 0.f ? desc->sm_scale : 1.f / sqrtf((float)desc->head_dim);
  p.scale_log2 = scale * kLog2e;
  p.rows_per_tile = pl.rows_per_tile;
  p.row_tiles = pl.row_tiles;
  p.splits = pl.splits;
  p.keys_per_split = pl.keys_per_split;
  long long total = (long long)desc->batch * desc->n_kv_heads * pl.row_tiles * pl.splits;
  if (total > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  p.total = (int)total;

  hipLaunchKernelGGL(kern, dim3(p.total), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}
