/*
 * tree_verify.h -- C interface of libtreeverify.so: token-tree attention,
 * token-tree verification and accepted-path KV compaction on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (web pages, section names as printed):
 *   [guide]   "SpecInfer Guide: Tree-Based Speculative LLM Serving"
 *   [chapter] "Inference Optimization Techniques: Speed and Efficiency"
 *   [cohere]  Cohere's blog post "hardware-aware dynamic speculative decoding"
 *
 * General rules for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     keeps no reference to them after the call is enqueued.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream);
 *     nothing is synchronised and nothing returns to the host.
 *   - The return value reports synchronous argument errors found on the host
 *     before anything is launched (TV_OK = 0, negative = error; nothing was
 *     enqueued).  Data errors in device arrays are reported per request in
 *     `status[b]` as a bitwise OR of TV_REQ_* flags; a request with a non-zero
 *     status has unspecified outputs but is never read or written out of
 *     bounds.
 *   - `workspace` is caller-owned device scratch (256-byte aligned) of at
 *     least the size the matching *_workspace_size() returns for the call's
 *     descriptor.  The verifiers', the attention's and the tree expansion's
 *     workspaces hold slots or counters that must start at zero: prepare
 *     each once with tree_verify_workspace_init (every call leaves them at
 *     zero again, so later calls need nothing).  A workspace that was not
 *     prepared, or was prepared with fewer bytes than the call needs, is
 *     detected on the device from its header and fails the requests that
 *     would use it with TV_REQ_BAD_WORKSPACE; nothing of it is read as
 *     exchange data.  Two calls that may run concurrently must use distinct
 *     workspaces.
 *   - Node ids: a tree of n nodes is a parent array with parent[0] = -1 (node 0
 *     is the root: the last token already emitted) and 0 <= parent[i] < i.
 *     Rows are padded to n_max; padding rows are neither read nor written.
 *   - Integer types are int32_t; bf16 tensors are passed as raw 16-bit words.
 *
 * Environment (read once per process, at the first call):
 *   TV_TRACE=1  every entry point is a named roctx range when the roctx
 *               library can be loaded (rocprofv3 --marker-trace records them);
 *               otherwise nothing happens.
 *   TV_DEBUG=1  entry points that take trees or block tables first copy them
 *               to the host and print each malformed request on stderr
 *               ("[tv debug] <entry>: request <b>: ..."), then launch as usual
 *               (the status flags are unchanged), and afterwards synchronise
 *               `stream`, returning TV_ERR_HIP when the GPU reported an error.
 *               This synchronises, so it must not be set for calls made under
 *               stream capture.
 *   TV_CHASE_SPIN_LIMIT=<n>  a test hook: the verifiers' path-chasing
 *               workgroups, the attention's key splits waiting for each
 *               other and the tree expansion's per-request workgroups give
 *               up after n polling rounds (default about 2 s, 0.5 s and 2 s
 *               worth) and report TV_REQ_TIMEOUT, invalidating the
 *               workspace; a negative n gives up without waiting.  Every
 *               workgroup still ends normally.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- synchronous status codes ------------------------------------------ */
enum {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad descriptor field */
  TV_ERR_UNSUPPORTED = -2,  /* head_dim, dtype, block_size or n_max outside the supported set */
  TV_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  TV_ERR_HIP = -4           /* a HIP runtime call failed (device query or launch) */
};

/* ---- per-request status flags (status[b], bitwise OR) -------------------- */
enum {
  TV_REQ_BAD_PARENT = 1,    /* parent[0] != -1 or some parent[i] outside [0, i) */
  TV_REQ_BAD_NNODES = 2,    /* n_nodes[b] outside [1, n_max] */
  TV_REQ_BAD_KV = 4,        /* prefix_len < 0, positions past the block table, or a block id outside the pool */
  TV_REQ_NONFINITE = 8,     /* a logit row that is read holds NaN or +-inf */
  TV_REQ_BAD_TOKEN = 16,    /* a child token outside [0, vocab) (stochastic verification) */
  TV_REQ_BAD_PATH = 32,     /* accepted path is not 0 followed by increasing node ids < n_max */
  TV_REQ_TIMEOUT = 64,      /* a bounded inter-workgroup wait expired (results unspecified) */
  TV_REQ_TREE_OVERFLOW = 128, /* a constructed tree would need more than n_max nodes */
  TV_REQ_BAD_LEN = 256,     /* a candidate length, frontier count or frontier node id out of range */
  TV_REQ_POOL_EXHAUSTED = 512, /* the block pool cannot serve an allocation, or a release would overfill it */
  TV_REQ_BAD_PROB = 1024,   /* an acceptance probability that is NaN or outside [0, 1] (tree budget) */
  TV_REQ_BAD_WORKSPACE = 2048 /* the call's workspace was not prepared by tree_verify_workspace_init (or is too small) */
};

/* ---- element types ------------------------------------------------------ */
enum { TV_F32 = 0, TV_BF16 = 1 };

/* ---- attention / cache descriptor --------------------------------------- */
typedef struct tv_attn_desc {
  int32_t batch;              /* B >= 0 requests */
  int32_t n_max;              /* node stride of q/out/parent/path, 1..128 */
  int32_t n_q_heads;          /* Hq >= 1 */
  int32_t n_kv_heads;         /* Hkv >= 1, divides Hq; q-head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* tokens per KV block: 16, 32, 64 or 128 */
  int32_t max_blocks_per_seq; /* row stride of block_table (>= 1) */
  int32_t num_blocks;         /* blocks in the pool; block ids outside [0, num_blocks) are data errors */
  int32_t dtype;              /* TV_F32 or TV_BF16: element type of q, k_cache, v_cache and out */
  float sm_scale;             /* softmax scale; <= 0 selects 1 / sqrt(head_dim) */
} tv_attn_desc;

/* Cache layout (both caches are indexed by physical block id):
 *   k_cache [num_blocks][Hkv][block_size][D]   token-major key rows
 *   v_cache [num_blocks][Hkv][block_size][D]   token-major value rows
 * Logical position p of request b lives in block block_table[b][p / block_size],
 * slot p % block_size.  A request's prefix occupies positions [0, P) and its
 * tree nodes positions [P, P + n) in node order ([guide] "Depth-First
 * Flattening and KV Cache Reuse": tree tokens append their K/V to the cache). */

/* Bytes of workspace tree_attn_forward needs for `desc` on the current device
 * (0 when no tile of the call is split over keys; then `workspace` may be NULL).
 * The workspace holds the split-K partials and one counter per tile: the last
 * split of a tile to finish merges the tile ([guide] "The Topology-Aware 2D
 * Causal Mask", FlashDecoding-style split-K).  Prepare it once with
 * tree_verify_workspace_init. */
size_t tree_attn_workspace_size(const tv_attn_desc* desc);

/* Tree attention ([guide] "Generalizing Attention to Tree Topologies" and "The
 * Topology-Aware 2D Causal Mask"): for request b, q-head h and node u < n_b,
 *   out[b][u][h] = sum_v alpha_v V_v,  alpha = softmax_v(sm_scale * q . K_v)
 * over the keys v in the prefix [0, P_b) and the tree positions P_b + w with w
 * equal to u or one of u's ancestors (parent walk of parent[b]).
 *   q      [B][n_max][Hq][D]     (dtype)
 *   out    [B][n_max][Hq][D]     (dtype) written for u < n_b only
 *   block_table [B][max_blocks_per_seq], prefix_len [B], n_nodes [B], parent [B][n_max]
 *   status [B] or NULL: TV_REQ_BAD_NNODES / _BAD_PARENT / _BAD_KV, and
 *     TV_REQ_BAD_WORKSPACE for a request whose tiles are split over keys when
 *     the workspace was not prepared (its output rows are then not written)
 * The caches are only read.  TV_ERR_WORKSPACE: workspace missing or too small;
 * TV_ERR_INVALID_ARG: q, caches or out not 16-byte aligned, or a workspace
 * not 256-byte aligned; TV_ERR_UNSUPPORTED: a call whose split partials would
 * need 2 GiB of workspace or more.  When every workgroup of the call is
 * resident at once, the key splits of a tile wait (bounded, see
 * TV_CHASE_SPIN_LIMIT) for each other before merging; a wait that expires
 * gives TV_REQ_TIMEOUT and invalidates the workspace header (a split of the
 * same call that reads the header after that reports TV_REQ_BAD_WORKSPACE for
 * its request instead, which needs the same remedy: prepare the workspace). */
int tree_attn_forward(const tv_attn_desc* desc, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* prefix_len,
                      const int32_t* n_nodes, const int32_t* parent, void* out, int32_t* status,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- verifier descriptor ------------------------------------------------- */
typedef struct tv_verify_desc {
  int32_t batch;        /* B >= 0 */
  int32_t n_max;        /* node stride, 1..128 */
  int32_t vocab;        /* V >= 1: row length of the logit arrays */
  float temperature;    /* > 0; logits are divided by it (stochastic verification only) */
} tv_verify_desc;

/* Outputs common to both verifiers, per request b (n = n_nodes[b]):
 *   path [B][n_max]       path[0] = 0, then the accepted nodes root to leaf
 *   path_len [B]          L + 1 = number of entries of path and of out_tokens
 *                         (0 when status[b] != 0)
 *   out_tokens [B][n_max] the L accepted tokens, then one correction/bonus token
 *                         ([chapter] "Worked Example ...": a round emits K + 1)
 *   status [B]            TV_REQ_* flags (required)
 * Teams of workgroups that cooperate on one node wait on each other through
 * bounded spins; if a wait expires (other work holding the GPU for a long
 * time) the request gets TV_REQ_TIMEOUT instead of hanging.  When the stochastic
 * verifier's path chase itself gives up waiting for a node, it also invalidates
 * the workspace: later calls report TV_REQ_BAD_WORKSPACE until
 * tree_verify_workspace_init prepares it again.
 * Entries past path_len are not written. */

/* Bytes of workspace either verifier needs for `desc`.  The two verifiers lay
 * their workspaces out differently: give each its own buffer. */
size_t tree_verify_workspace_size(const tv_verify_desc* desc);

/* Prepares a workspace (256-byte aligned, at least the *_workspace_size bytes
 * of the descriptors it will serve): zeroes it and writes the header the
 * kernels check.  Both verifiers and tree_attn_forward need it.  Enqueued on `stream`.
 * TV_ERR_WORKSPACE for a null or too small buffer, TV_ERR_INVALID_ARG when
 * it is not 256-byte aligned. */
int tree_verify_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification ([guide] "Greedy Verification Algorithm"): from the root,
 * t = argmax_w target_logits[b][u][w] (lowest index among equal maxima); move to
 * the first child c (ascending node id) with tokens[b][c] == t, else emit t and
 * stop.  A leaf emits its argmax.
 *   target_logits [B][n_max][V] float32 (rows u < n read); tokens, parent [B][n_max].
 * The workspace must have been prepared by tree_verify_workspace_init (each
 * call leaves it prepared); an unprepared one gives TV_REQ_BAD_WORKSPACE. */
int tree_verify_greedy(const tv_verify_desc* desc, const float* target_logits,
                       const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                       int32_t* path, int32_t* path_len, int32_t* out_tokens, int32_t* status,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* tree_verify_greedy without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch -- one 64-bit key per (node,
 * 8192-logit chunk) after a 256-byte header: 256 + 8 * B * n_max * ceil(V / 8192)
 * bytes, rounded up to a multiple of 256 -- lives
 * in a static array of tree_verify_greedy_noalloc_max_scratch() bytes (4 MiB)
 * that every GPU the library runs on holds until the process ends; the call
 * allocates nothing.  Descriptors needing more scratch return TV_ERR_WORKSPACE
 * before anything is enqueued.  Arguments, results and errors otherwise as
 * tree_verify_greedy.  Every call on one GPU shares that GPU's array: calls
 * that may overlap on one device (different streams, or host threads) race and
 * must be serialised by the caller.  Each call writes every scratch entry it
 * reads, so nothing carries over from the previous call. */
int tree_verify_greedy_noalloc(const tv_verify_desc* desc, const float* target_logits,
                               const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                               int32_t* path, int32_t* path_len, int32_t* out_tokens, int32_t* status,
                               hipStream_t stream);

/* Bytes of the static scratch behind tree_verify_greedy_noalloc. */
size_t tree_verify_greedy_noalloc_max_scratch(void);

/* Stochastic verification ([guide] "Stochastic Verification Algorithm";
 * [chapter] acceptance rule min(1, p/q) and residual max(p - q, 0) / Z).
 * At node u with p = softmax(target_u / T), q = softmax(draft_u / T), p' = p:
 * children c are tried in ascending id with proposal x = tokens[c]; c is
 * accepted when u_accept[b][c] * q(x) <= p'(x); a rejection replaces p' by
 * max(p' - q, 0) / Z (kept when Z = 0) before the next sibling is tried.  When
 * no child is accepted (always at a leaf) the final token is the smallest x
 * whose cumulative p' exceeds u_sample[b][u] * sum(p').
 *   draft_logits [B][n_max][V] float32: only rows of nodes that have children are read.
 *   u_accept, u_sample [B][n_max] float32 uniforms in [0, 1), supplied by the caller.
 * Decisions use float32 exponentials with float64 sums and a float64 accept test.
 * Supports vocab <= 524288 (TV_ERR_UNSUPPORTED beyond). */
int tree_verify_stochastic(const tv_verify_desc* desc, const float* target_logits,
                           const float* draft_logits, const int32_t* tokens,
                           const int32_t* parent, const int32_t* n_nodes, const float* u_accept,
                           const float* u_sample, int32_t* path, int32_t* path_len,
                           int32_t* out_tokens, int32_t* status, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Accepted-path KV compaction ([guide] "Depth-First Flattening and KV Cache
 * Reuse"; "PagedKV Allocation with Zero-Copy Pruning"): for j = 0..L,
 * K/V at position P + path[j] is moved to position P + j (all KV heads) and
 * new_len[b] = P + L + 1.  The move is in place and hazard-free (every source
 * is read before any destination is written).  A request with path_len 0 or a
 * malformed path is left untouched: new_len = prefix_len, src_pos = -1.
 *   path, path_len as produced by the verifiers; src_pos [B][n_max] receives
 *   P + path[j] for j < path_len and -1 elsewhere; new_len [B];
 *   status [B] or NULL: TV_REQ_BAD_PATH / TV_REQ_BAD_KV.
 * Only desc->batch, n_max, n_kv_heads, head_dim, block_size,
 * max_blocks_per_seq, num_blocks and dtype are used. */
int kv_compact_accepted(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* prefix_len,
                        const int32_t* path, const int32_t* path_len, int32_t* src_pos,
                        int32_t* new_len, int32_t* status, hipStream_t stream);

/* Verify-and-compact: tree_verify_stochastic followed by kv_compact_accepted of
 * the path it selects ([guide] "Stochastic Verification Algorithm", then
 * "Depth-First Flattening and KV Cache Reuse"), in one call whose last kernel
 * both walks the path and moves the K/V, so the path does not travel through
 * memory between two launches.  Every output equals that of the two calls in
 * sequence: path, path_len, out_tokens and status as tree_verify_stochastic
 * gives them; the caches, src_pos, new_len and kv_status (NULL allowed) as
 * kv_compact_accepted gives them for that path.  kv_desc->batch and n_max must
 * equal desc->batch and n_max (TV_ERR_INVALID_ARG otherwise); the workspace is
 * tree_verify_workspace_size(desc) bytes, as for tree_verify_stochastic.
 * The compaction moves 8 bytes at a time when both caches are 8-byte aligned;
 * otherwise it runs as a second kernel that moves single elements. */
int tree_verify_stochastic_compact(const tv_verify_desc* desc, const tv_attn_desc* kv_desc,
                                   const float* target_logits, const float* draft_logits,
                                   const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                                   const float* u_accept, const float* u_sample, int32_t* path,
                                   int32_t* path_len, int32_t* out_tokens, int32_t* status,
                                   void* k_cache, void* v_cache, const int32_t* block_table,
                                   const int32_t* prefix_len, int32_t* src_pos, int32_t* new_len,
                                   int32_t* kv_status, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---- speculative KV blocks -------------------------------------------------
 * [guide] "PagedKV Allocation with Zero-Copy Pruning": the tree's KV blocks are
 * taken from the paged pool and marked speculative; after verification the
 * blocks of the unselected branches return to the free pool in one metadata
 * update.  The pool is a stack of free block ids, free_ids[0 .. *free_count),
 * top at *free_count - 1.  Each call serves the batch in request order, pops or
 * pushes one contiguous segment of the stack and updates *free_count once.  A
 * request the pool cannot serve gets TV_REQ_POOL_EXHAUSTED and so does every
 * later request that needs blocks moved (requests moving none always succeed);
 * failed requests are left unchanged.  *free_count outside [0, num_blocks]
 * fails every request with TV_REQ_BAD_KV.  Only desc->batch, block_size,
 * max_blocks_per_seq and num_blocks are used.  One workgroup; no workspace. */

/* Allocation: request b's table maps n_blocks[b] blocks; it is extended to the
 * ceil((prefix_len[b] + n_nodes[b]) / block_size) blocks that hold its prefix
 * and its tree (the tree's K/V goes to positions prefix_len .. + n_nodes), the
 * new entries popped from the top of the stack one by one.  spec_from[b] = the
 * first speculative table index (the old n_blocks[b]; -1 when the request
 * failed).  TV_REQ_BAD_KV: negative prefix_len / n_nodes, n_blocks outside
 * [0, max_blocks], or more than max_blocks blocks needed.
 *   block_table [B][max_blocks] and n_blocks [B] in/out; free_ids [num_blocks] in;
 *   free_count [1] in/out; spec_from, status [B] out. */
int kv_alloc_tree_blocks(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                         const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* free_ids,
                         int32_t* free_count, int32_t* spec_from, int32_t* status, hipStream_t stream);

/* Release: request b keeps the ceil(new_len[b] / block_size) blocks that hold
 * its first new_len positions (new_len from kv_compact_accepted: prefix plus
 * accepted path) and pushes every later mapped block onto the stack, in table
 * order, setting its table entry to -1 and n_blocks[b] to the kept count.
 * TV_REQ_BAD_KV: new_len < 0, n_blocks outside [0, max_blocks], new_len beyond
 * the mapped blocks, or a block id to release outside [0, num_blocks).
 *   block_table [B][max_blocks], n_blocks [B] in/out; new_len [B] in;
 *   free_ids [num_blocks], free_count [1] in/out; status [B] out. */
int kv_release_blocks(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                      const int32_t* new_len, int32_t* free_ids, int32_t* free_count, int32_t* status,
                      hipStream_t stream);

/* ---- token-tree construction ---------------------------------------------
 * [guide] "Token Tree Construction: Expansion vs. Merge".  Both entry points
 * produce the parent-array trees the entry points above consume: node 0 is
 * the root (the last token already emitted) and parent[i] < i. */

typedef struct tv_merge_desc {
  int32_t batch;        /* B >= 0 */
  int32_t n_cand;       /* M: candidate sequences per request, 1..64 */
  int32_t max_len;      /* Lmax: candidate stride, 1..32 */
  int32_t n_max;        /* node stride of the output tree, 1..1024 */
} tv_merge_desc;

/* Merge-based construction ([guide] Method B, the merge condition "every node
 * of every candidate has a node of M with the same token sequence"): request
 * b's candidates (continuations drafted by several draft models) become one
 * tree whose node 0 carries root_token[b].  Every prefix of every candidate is
 * the token sequence of exactly one node; identical prefixes share it.  Nodes
 * are numbered in depth-first preorder, siblings in the order of the first
 * candidate that contains them.
 *   cand_tokens [B][M][Lmax] int32 (entries past cand_len are not read)
 *   cand_len [B][M] int32 in [0, Lmax]; root_token [B] int32
 * Outputs: tokens, parent [B][n_max] (entries past n_nodes[b] not written);
 *   n_nodes [B]; node_of [B][M][Lmax] or NULL: the node of each candidate
 *   position (-1 past cand_len); status [B]: TV_REQ_BAD_LEN (a cand_len out of
 *   range) or TV_REQ_TREE_OVERFLOW (more than n_max nodes needed), both with
 *   n_nodes = 0 and nothing else written.
 * No workspace.  TV_ERR_UNSUPPORTED outside the limits of the descriptor. */
int tree_merge_candidates(const tv_merge_desc* desc, const int32_t* cand_tokens,
                          const int32_t* cand_len, const int32_t* root_token, int32_t* tokens,
                          int32_t* parent, int32_t* n_nodes, int32_t* node_of, int32_t* status,
                          hipStream_t stream);

typedef struct tv_expand_desc {
  int32_t batch;        /* B >= 0 */
  int32_t f_max;        /* F >= 1: frontier stride (draft rows per request) */
  int32_t vocab;        /* V >= 1: row length of draft_logits */
  int32_t n_max;        /* node stride of the tree, 1..1024 */
  int32_t k;            /* expansion factor of this level, 1..16 and <= V */
} tv_expand_desc;

/* Bytes of workspace tree_expand_topk needs for `desc` (0 for an invalid one);
 * prepare it once with tree_verify_workspace_init. */
size_t tree_expand_workspace_size(const tv_expand_desc* desc);

/* One level of expansion-based construction ([guide] Method A, schedule
 * <k_1, ..., k_m>: call once per depth i with k = k_i and the draft model's
 * logits at the previous level's nodes).  Frontier node f < n_frontier[b] of
 * request b, in order, receives as children the k tokens of largest logit in
 * its draft row (best first; equal logits: lower token index first), appended
 * after the tree's last node: child r of frontier f gets id
 * n_nodes[b] + f * k + r.
 *   draft_logits [B][F][V] float32, 16-byte aligned: row f = logits at frontier[b][f]
 *   frontier [B][F] int32 node ids below n_nodes[b]; n_frontier [B] in [0, F]
 * In/out: tokens, parent [B][n_max]; n_nodes [B] (grows by n_frontier * k).
 * Out: new_frontier [B][F * k] (the appended ids, in order); n_new [B];
 *   status [B]: TV_REQ_BAD_NNODES (n_nodes outside [1, n_max]),
 *   TV_REQ_BAD_LEN (n_frontier or a frontier id out of range),
 *   TV_REQ_TREE_OVERFLOW (more than n_max nodes), TV_REQ_NONFINITE (a read
 *   row holds NaN or +-inf; reported only when the checks before it pass),
 *   TV_REQ_BAD_WORKSPACE, TV_REQ_TIMEOUT (a request's wait for its rows'
 *   partial results expired; the workspace is invalidated); with any of them
 *   nothing is appended and n_new = 0.
 * One launch: the per-chunk partial results pass through the prepared
 * workspace (256-byte aligned, else TV_ERR_INVALID_ARG) to one workgroup per
 * request in the same grid.  TV_ERR_UNSUPPORTED when V > 131072 at k = 16
 * (ceil(V / 8192) * k must stay <= 256). */
int tree_expand_topk(const tv_expand_desc* desc, const float* draft_logits, const int32_t* frontier,
                     const int32_t* n_frontier, int32_t* tokens, int32_t* parent, int32_t* n_nodes,
                     int32_t* new_frontier, int32_t* n_new, int32_t* status, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* ---- tree-budget calibration ----------------------------------------------
 * [chapter] "Worked Example: How Many Tokens Land Per Expensive Pass?" models
 * acceptance events as independent draws and counts the tokens one round
 * emits as T = K + 1 (K accepted drafts plus one correction or bonus token);
 * for a chain of gamma drafts with acceptance alpha, E[T] = (1 - alpha^(gamma+1))
 * / (1 - alpha).  [cohere] "Dynamic speculative decoding" picks the number of
 * drafts per batch size by goodput = AL / ITL (acceptance length over
 * inter-token latency) from offline measurements kept as a lookup table, and
 * [guide] "Dynamic Tree Budget Calibration" asks tree size to follow the batch
 * size.  The two calls below are that calculation for token trees. */

typedef struct tv_budget_desc {
  int32_t batch;        /* B >= 0 trees */
  int32_t n_max;        /* node stride, 1..128 */
} tv_budget_desc;

/* Expected acceptance length of each tree under the per-node independence
 * model: drafted node v, when it is tested, is accepted with probability
 * accept_prob[b][v], independently of every other test; the children of a node
 * are tested in ascending id and the first accepted one continues the walk
 * (the order of the verification walk, [guide] "Stochastic Verification
 * Algorithm").  For a chain with every probability alpha this is [chapter]'s
 * model exactly.
 *   parent [B][n_max] int32 (parent[0] = -1, 0 <= parent[i] < i); n_nodes [B]
 *   accept_prob [B][n_max] float64; entry 0 (the root, never tested) and
 *     entries past n_nodes[b] are not read.
 * Outputs (float64):
 *   reach [B][n_max]: P(node v lies on the accepted path); reach[b][0] = 1 and
 *     every entry from n_nodes[b] to n_max - 1 is written as 0;
 *   expected_len [B]: AL = E[T] = 1 + sum over v >= 1 of reach[b][v];
 *   status [B]: TV_REQ_BAD_NNODES, else TV_REQ_BAD_PARENT, else
 *     TV_REQ_BAD_PROB (a probability that is NaN or outside [0, 1]); a failed
 *     request gets expected_len = 0 and a reach row of zeros.
 * One wavefront per tree; no workspace.  Sums and products are float64 in an
 * order other than the walk's, so results agree with a sequential evaluation
 * to rounding (relative 1e-12 and better). */
int tree_expected_accept_length(const tv_budget_desc* desc, const int32_t* parent, const int32_t* n_nodes,
                                const double* accept_prob, double* reach, double* expected_len,
                                int32_t* status, hipStream_t stream);

/* Tree-size lookup table from measurements ([cohere] goodput): for each batch
 * size i, best[i] = the shape s with the largest al[s] / itl[i][s] among the
 * latencies that are positive and finite (equal goodputs keep the lower s;
 * -1 when there is none).  A host computation on HOST arrays: al [n_shapes]
 * (acceptance length of each candidate shape, e.g. from
 * tree_expected_accept_length), itl [n_batch_sizes][n_shapes] (measured step
 * latency, any unit), best [n_batch_sizes] out.  Nothing is launched.
 * TV_ERR_INVALID_ARG for a null array or a negative count. */
int tree_budget_select(int32_t n_batch_sizes, int32_t n_shapes, const double* al, const double* itl,
                       int32_t* best);

/* Human-readable name of a synchronous status code. */
const char* tv_status_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* TREE_VERIFY_H */
