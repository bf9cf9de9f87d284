/*
 * spec_verify.h -- C ABI of the tree-verification library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the target model's verification step of tree speculative decoding:
 *
 *   spec_tree_attention    tree-masked GQA attention of every draft-tree node against a paged
 *                          bf16 KV cache (split-K over the context, LSE merge of the splits)
 *   spec_chunk_salience    the attention mass that the verification queries put on each context
 *                          chunk, optionally accumulated over layers, with top-k chunk selection
 *   spec_accept_greedy     greedy longest-accepted-path acceptance
 *   spec_accept_rejection  exact rejection-sampling acceptance against the draft distribution
 *   spec_kv_commit         moves the accepted path's K/V next to the committed context and
 *                          advances the per-sequence lengths (the per-row rollback)
 *   spec_draft_gather      builds the draft model's compact KV from the selected context chunks
 *                          and the recent window, rotated at local positions
 *   spec_tree_bundle_order host-side preorder renumbering of a draft tree (bundles of leaves
 *                          under one branching node adjacent; subtrees as index ranges)
 *   spec_controller_*      host-side choice of the next draft depth from the online acceptance
 *                          rate and cost ratio
 *
 * Sources (web pages cited by title and section):
 *   [DS]  "DiffSpec: Accelerating Long Sequence Generation with Differential Speculative Decoding"
 *         (vllm-diffspec README): "What DiffSpec Does" items 2 and 5, "Architecture"
 *         (target-guided retrieval from paged target KV), "Configuration" (chunk size 64,
 *         up to 50 verifier tree nodes).
 *   [DSC] DiffSpec README (CGCL-codes), "Features": salience-aware chunk encoding, paged KV,
 *         the bundle scheduler.
 *   [AS]  "Adaptive Speculative Decoding": "Correctness first" (exact rejection sampling,
 *         greedy as its temperature-0 case), "The controller" (acceptance probability
 *         min(1, p/q); k drafts give up to k+1 tokens), "Layout" (per-row cache mask
 *         s <= lengths[b] + j).
 *   [VC]  vllm.cpp "Speculative decoding": "MTP" (accept-if-equal greedy verification),
 *         "Consuming it programmatically" (a versioned C ABI that refuses what it cannot
 *         honour, by name, instead of silently downgrading).
 *
 * Conventions for every entry point
 *   - Pointers are device pointers unless marked (host).  The caller owns all memory; the
 *     library never allocates, frees or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only
 *     enqueue work and return; there is no host<->device synchronisation, so calls may be
 *     captured in a HIP graph.
 *   - Host-visible arguments are validated before anything is enqueued.  On failure the call
 *     returns a spec_status other than SPEC_OK, enqueues nothing, and spec_last_error()
 *     (thread-local) names the argument and the accepted values.  A failed HIP launch returns
 *     SPEC_ERR_HIP with the HIP error text.
 *   - Device-side preconditions (listed per call) are not checked on the host.  Kernels clamp
 *     every index they derive from device data to the host bounds, so a violated
 *     precondition gives wrong results, never an out-of-bounds access.
 *   - Results are deterministic: fixed reduction orders, no floating-point atomics.
 *   - No C++ exception crosses this interface.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 5

/* Largest draft tree (nodes per sequence) any call accepts.  spec_tree_attention takes up to 256
 * nodes in index order, and up to this many when the tree is in preorder with subtree ends. */
#define SPEC_MAX_TREE_NODES 2048

typedef enum spec_status {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARGUMENT = 1, /* a null/misaligned pointer, a size out of range, inconsistent shapes */
  SPEC_ERR_UNSUPPORTED = 2,      /* a well-formed value this build does not implement (e.g. head_dim 96) */
  SPEC_ERR_WORKSPACE = 3,        /* workspace missing or smaller than the matching *_workspace_size() */
  SPEC_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  SPEC_ERR_STATE = 5             /* call order violated (salience without chunk partials) */
} spec_status;

typedef enum spec_dtype { SPEC_DTYPE_BF16 = 0, SPEC_DTYPE_F32 = 1 } spec_dtype;

/* Layout of the V cache inside a (page, kv_head) block; see spec_paged_kv. */
typedef enum spec_v_layout {
  SPEC_V_TOKEN_ROWS = 0,  /* like K: row t of the page at t * token_stride, head_dim contiguous */
  SPEC_V_DIM_MAJOR = 1    /* dim d at d * page_size, the page's tokens of that dim contiguous */
} spec_v_layout;

/* == SPEC_ABI_VERSION of the built library. */
int spec_abi_version(void);
/* Static text for a status code. */
const char* spec_status_string(int status);
/* (host) Thread-local text of the last failure on this thread; "" after a successful call. */
const char* spec_last_error(void);

/* ------------------------------------------------------------------------------------------
 * The SPEC_DEBUG build and the debug record  [AS "Correctness first": per-row bookkeeping errors;
 * VC "MTP": positive witnesses that every draft was really tested]
 *
 * libspec_verify_debug.so is this library built with SPEC_DEBUG.  In it, spec_tree_attention,
 * spec_accept_greedy and spec_accept_rejection first run device-side checks of the device
 * preconditions listed with each call, and the acceptance walks count what they did.  The results go
 * to a debug record of SPEC_DEBUG_RECORD_BYTES bytes at the end of the call's workspace, at byte
 * offset (the call's *_workspace_size) - SPEC_DEBUG_RECORD_BYTES, as uint32 words:
 *   [0] error bits (SPEC_DBG_*): 0 when every checked precondition holds
 *   [1] acceptance: rows of target logits whose reduction (greedy: argmax; rejection: row maximum)
 *       this call computed and its walk read; Σ_b N_b when the call ran whole
 *   [2] acceptance: draft tokens the walk tested against their parent's row; Σ_b (N_b - 1)
 *   [3] 0
 * (spec_tree_attention writes words 1..3 as 0.)  Every workspace size includes the record in both
 * builds; the release build never writes it.  A call whose preconditions fail still runs (its kernels
 * clamp indices, so nothing is read or written out of bounds); the record says what was wrong.  The
 * record is written on the call's stream: read it after the call completes.  spec_accept_greedy_noalloc
 * and the calls without a workspace run no checks.
 * ------------------------------------------------------------------------------------------ */
#define SPEC_DEBUG_RECORD_BYTES 256
#define SPEC_DBG_PARENTS (1u << 0)      /* parents[i] outside 0..i-1 (i > 0), or a root parent other than -1 */
#define SPEC_DBG_BLOCK_TABLE (1u << 1)  /* a block-table entry the call reads is outside 0..num_pages-1 */
#define SPEC_DBG_NODE_OFFSETS (1u << 2) /* node_offsets[0] != 0, decreasing, or a tree above max_nodes */
#define SPEC_DBG_CTX_LENS (1u << 3)     /* a ctx_lens entry outside 0..max_ctx_len */
#define SPEC_DBG_SUBTREE_END (1u << 4)  /* subtree_end[i] outside i+1..N (sequence-local) */
#define SPEC_DBG_TOKENS (1u << 5)       /* a non-root draft token outside 0..vocab-1 */
#define SPEC_DBG_UNIFORMS (1u << 6)     /* a u_accept (non-root) or u_sample entry outside [0, 1) */
#define SPEC_DBG_DRAFT_PROBS (1u << 7)  /* a draft probability negative or not finite */
#define SPEC_DBG_CHILDREN (1u << 8)     /* a node with more than max_children children */
#define SPEC_DBG_LOGITS (1u << 9)       /* a NaN target logit */

/* 1 in the SPEC_DEBUG build (libspec_verify_debug.so), 0 in the release build. */
int spec_debug_build(void);

/* ------------------------------------------------------------------------------------------
 * Paged KV cache [DSC "Features": paged KV with a block table; AS "Layout"].
 * Logical slot t of sequence b is page block_table[b * block_table_stride + t / page_size],
 * row t % page_size.  Element (page, kv_head, row, d) of K is at
 *   k_cache + page * page_stride + kv_head * head_stride + row * token_stride + d
 * (bf16 elements).  V uses the same page and head strides; inside a (page, kv_head) block it is
 *   v_layout = SPEC_V_TOKEN_ROWS:  v_cache + ... + row * token_stride + d          (like K)
 *   v_layout = SPEC_V_DIM_MAJOR:   v_cache + ... + d * page_size + row
 * i.e. [pages][kv_heads][page_size][head_dim] or [pages][kv_heads][head_dim][page_size] (the
 * layout of caches that store V transposed per page).  Results of the two layouts agree to fp32
 * rounding (the order of the key contraction differs).  With token_stride = head_dim and
 * head_stride = page_size * head_dim each (page, head) is one contiguous block (the fastest K
 * layout); other strides work if every row is 16-byte aligned.
 * page_stride and token_stride * page_size must stay below 2^31 elements (the pool may be larger).
 * Pages may be shared between sequences (copy-on-write prefixes): the library only reads them.
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_paged_kv {
  const void* k_cache;          /* bf16, 16-byte aligned */
  const void* v_cache;          /* bf16, 16-byte aligned */
  int64_t page_stride;          /* elements; multiple of 8 */
  int64_t head_stride;          /* elements; multiple of 8 */
  int64_t token_stride;         /* elements; multiple of 8, >= head_dim */
  int32_t page_size;            /* slots per page: a power of two in [8, 1024] (16 in the workloads) */
  int32_t num_pages;            /* (host) pages in the pool; an id outside [0, num_pages) is never dereferenced
                                   (a precondition violation: that page's keys then read as zeros) */
  const int32_t* block_table;   /* int32 [batch][block_table_stride] physical page ids */
  int32_t block_table_stride;   /* >= ceil((max_ctx_len + max_nodes) / page_size) */
  int32_t v_layout;             /* spec_v_layout */
} spec_paged_kv;

/* ------------------------------------------------------------------------------------------
 * spec_tree_attention  [DS "What DiffSpec Does" item 5; AS "Layout"]
 *
 * Every node of each sequence's draft tree is a query.  Node i of sequence b (L = ctx_lens[b]
 * committed tokens) sees the keys {0 .. L-1} and {L + j : j is i or an ancestor of i}; its own
 * K/V must already be written at logical slot L + i.  The ancestor relation comes from parents
 * (up to 256 nodes), or, when subtree_end is given, from index ranges: the tree is then in
 * preorder (every subtree a contiguous range of nodes, as spec_tree_bundle_order returns it) and
 * j is i or an ancestor of i iff j <= i < subtree_end[j] (up to SPEC_MAX_TREE_NODES nodes; parents
 * is not read).  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).  For a chain of drafts this is ordinary causal decode.
 *   out[n][h][:] = softmax(scale * q[n][h] . K^T) V  over the visible keys   (bf16, RNE)
 *   lse[n][h]    = natural log of the softmax denominator                     (fp32)
 * Arithmetic: bf16 products with fp32 accumulation; probabilities are rounded to bf16 before
 * the P.V product; split partials are merged in fp32.
 * With chunk_size > 0 the call also leaves, in the workspace, the per-(query row, context
 * chunk) partials that spec_chunk_salience reduces [DS "Architecture": chunks are scored from
 * the paged target KV without materialising the attention matrix].
 *
 * Device preconditions: 0 <= ctx_lens[b] <= max_ctx_len; node_offsets non-decreasing with
 * node_offsets[0] = 0 and at most max_nodes nodes per sequence; parents sequence-local with
 * parents[first node] = -1 and 0 <= parents[i] < i otherwise; with subtree_end, i < subtree_end[i]
 * <= the sequence's node count (values outside are clamped into that range); block-table ids <
 * num_pages.
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_tree_attention_args {
  int32_t batch;                /* >= 1 */
  int32_t num_q_heads;          /* >= 1, multiple of num_kv_heads */
  int32_t num_kv_heads;         /* >= 1 */
  int32_t head_dim;             /* 64 or 128 */
  int32_t max_nodes;            /* (host) bound on tree nodes per sequence: 1..256, or
                                   1..SPEC_MAX_TREE_NODES with subtree_end */
  int32_t max_ctx_len;          /* (host) bound on ctx_lens[b], >= 0 */
  const int32_t* ctx_lens;      /* int32 [batch] committed tokens before the root */
  const int32_t* node_offsets;  /* int32 [batch + 1] packed node ranges; the first node of a range is the root */
  const int32_t* parents;       /* int32 [total_nodes] sequence-local parent ids (may be NULL with subtree_end) */
  const int32_t* subtree_end;   /* int32 [total_nodes] sequence-local, one past each node's subtree
                                   (preorder trees), or NULL to take the ancestors from parents */
  const void* q;                /* bf16 [total_nodes][num_q_heads][head_dim], 16-byte aligned (post-RoPE) */
  spec_paged_kv kv;
  float scale;                  /* finite; usually 1/sqrt(head_dim) */
  void* out;                    /* bf16 [total_nodes][num_q_heads][head_dim], 16-byte aligned */
  float* lse;                   /* fp32 [total_nodes][num_q_heads] or NULL */
  int32_t chunk_size;           /* 0: no salience partials; else 16, 32 or a multiple of 64 */
  int32_t split_tiles;          /* 0: library choice; else KV tiles of 64 slots per split (tuning knob) */
  void* workspace;              /* 256-byte aligned, >= spec_tree_attention_workspace_size(args) bytes */
  size_t workspace_bytes;
} spec_tree_attention_args;

/* Workspace bytes needed by spec_tree_attention for these host bounds (0 if args are invalid;
 * spec_last_error() then says why).  Depends only on batch, head counts, head_dim, max_nodes,
 * max_ctx_len, chunk_size and split_tiles. */
size_t spec_tree_attention_workspace_size(const spec_tree_attention_args* args);
int spec_tree_attention(const spec_tree_attention_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_chunk_salience  [DS "What DiffSpec Does" item 2, "Architecture" (target-guided retrieval),
 * "Configuration" (diffspec_chunk_size); DSC "Features" (salience-aware chunk encoding)]
 *
 * For each sequence b and context chunk c = slots [c*chunk_size, min((c+1)*chunk_size, L)):
 *   mass[b][c] = (1 / (N_b * num_q_heads)) * sum over nodes i, query heads h, keys t in c of
 *                the attention probability p[i][h][t] of the preceding spec_tree_attention call
 * (probabilities are normalised over all visible keys, context and tree; tree keys belong to no
 * chunk).  accumulate = 1 adds to chunk_mass (summing over layers); 0 overwrites it.  Entries
 * c >= ceil(L / chunk_size) are written as 0 (overwrite) or left unchanged (accumulate).
 * With top_k > 0 it then writes, per sequence, the top_k chunks of chunk_mass (after the update)
 * ordered by (mass descending, chunk index ascending), padded with index -1 and mass 0.
 *
 * Must follow, on the same stream, the spec_tree_attention call made with *attn (same workspace,
 * chunk_size > 0) before that workspace is reused.  chunk_size == 0 there -> SPEC_ERR_STATE.
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_chunk_salience_args {
  const spec_tree_attention_args* attn;  /* (host) the arguments of the preceding attention call */
  float* chunk_mass;            /* fp32 [batch][max_chunks] */
  int32_t max_chunks;           /* >= ceil(attn->max_ctx_len / attn->chunk_size) */
  int32_t accumulate;           /* 0 or 1 */
  int32_t top_k;                /* 0 (none) .. min(max_chunks, 8192) */
  int32_t* topk_index;          /* int32 [batch][top_k] or NULL when top_k == 0 */
  float* topk_mass;             /* fp32 [batch][top_k] or NULL when top_k == 0 */
} spec_chunk_salience_args;

int spec_chunk_salience(const spec_chunk_salience_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_accept_greedy  [VC "MTP": accept a draft iff it equals the target's greedy choice;
 * AS "The controller": k drafts give up to k+1 tokens]
 *
 * a_u = argmax_v target_logits[u][v] (lowest v among exactly equal maxima).  Node j is accepted
 * iff its parent is accepted and draft_tokens[j] == a_parent(j); the root is always accepted.
 * The result is the deepest accepted node f (lowest node index among equally deep ones):
 *   out_num_accepted[b]   = depth(f)  (accepted draft tokens)
 *   out_path_nodes[b][:]  = sequence-local nodes root .. f, then -1
 *   out_tokens[b][:]      = draft tokens of path nodes 1.., then a_f (the bonus token), then -1
 * A path longer than max_path is reported as out_num_accepted[b] = -1 with -1 rows.
 *
 * Device preconditions: as for spec_tree_attention (node_offsets, parents); no NaN logits.
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_accept_greedy_args {
  int32_t batch;                /* >= 1 */
  int32_t vocab;                /* 1 .. 2^24 */
  int32_t max_nodes;            /* (host) bound on nodes per sequence, 1..SPEC_MAX_TREE_NODES */
  int32_t max_path;             /* (host) row length of the path/token outputs, >= 1 (max depth + 1) */
  const int32_t* node_offsets;  /* int32 [batch + 1] */
  const int32_t* parents;       /* int32 [total_nodes] sequence-local */
  const int32_t* draft_tokens;  /* int32 [total_nodes]; the root's entry is ignored */
  const void* target_logits;    /* [total_nodes][vocab] of logits_dtype; row u = target logits after node u */
  int32_t logits_dtype;         /* spec_dtype */
  int32_t* out_num_accepted;    /* int32 [batch] */
  int32_t* out_path_nodes;      /* int32 [batch][max_path] */
  int32_t* out_tokens;          /* int32 [batch][max_path] */
  void* workspace;              /* >= spec_accept_greedy_workspace_size(args) bytes, 256-byte aligned */
  size_t workspace_bytes;
} spec_accept_greedy_args;

size_t spec_accept_greedy_workspace_size(const spec_accept_greedy_args* args);
int spec_accept_greedy(const spec_accept_greedy_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_accept_greedy_noalloc  for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same operation, outputs, preconditions and errors as spec_accept_greedy, except that
 * args->workspace and args->workspace_bytes are ignored: the per-segment argmax keys live in a
 * library-owned device array of SPEC_GREEDY_NOALLOC_SCRATCH_BYTES bytes, one per GPU, which each GPU
 * the library runs on holds until the process ends.  A call whose workspace need
 * (spec_accept_greedy_workspace_size) exceeds that size returns SPEC_ERR_UNSUPPORTED before anything
 * is enqueued.  The call allocates nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks the array's address up once, with that device current.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (different streams, no ordering
 * between them) race; calls ordered on one stream do not.  Nothing in the array needs clearing: each
 * call writes every key it reads.
 * ------------------------------------------------------------------------------------------ */
#define SPEC_GREEDY_NOALLOC_SCRATCH_BYTES (4u << 20)

int spec_accept_greedy_noalloc(const spec_accept_greedy_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_accept_rejection  [AS "Correctness first", "The controller"; Leviathan et al. and
 * Chen et al. as cited there]
 *
 * p_u = softmax(target_logits[u]) and q_u = draft_probs[u] (the distribution u's children were
 * drawn from, i.i.d.).  Starting at the root u: res = p_u; visit the children c of u in increasing
 * node index with x = draft_tokens[c]:
 *   accept iff u_accept[c] * q_u(x) < res(x)  -> move to c and repeat;
 *   else res = max(0, res - q_u) / sum(max(0, res - q_u))   (kept unchanged if that sum is 0).
 * If no child is accepted, the bonus token is the smallest v with
 *   sum_{w <= v} res(w) > u_sample[u] * sum_w res(w).
 * With one child per node this is the chain rule of the page; with i.i.d. children the emitted
 * token has law p_u (lossless).  Outputs as for spec_accept_greedy.  A node with more than
 * max_children children is reported as out_num_accepted[b] = -1.
 * Arithmetic: every probability, residual and sum in fp64 (exp evaluated in fp64).
 *
 * Device preconditions: as for spec_accept_greedy; draft_probs rows non-negative; uniforms in [0,1).
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_accept_rejection_args {
  spec_accept_greedy_args base; /* topology, target logits, outputs, workspace */
  int32_t max_children;         /* (host) bound on children of any node, 1 .. max_nodes - 1 (0 if max_nodes == 1) */
  const float* draft_probs;     /* fp32 [total_nodes][vocab] */
  const float* u_accept;        /* fp32 [total_nodes]: uniform for the accept test of node c */
  const float* u_sample;        /* fp32 [total_nodes]: uniform for the bonus draw at stopping node u */
} spec_accept_rejection_args;

size_t spec_accept_rejection_workspace_size(const spec_accept_rejection_args* args);
int spec_accept_rejection(const spec_accept_rejection_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_kv_commit  [AS "Layout": a per-row length and a cache mask turn rollback into a length
 * update; AS "The controller": k drafts yield up to k + 1 tokens]
 *
 * The step after acceptance.  The verification forward wrote node i's K/V at slot ctx_lens[b] + i;
 * the accepted path (path_nodes[b][0] = root, then num_accepted[b] drafts, as returned by
 * spec_accept_greedy / spec_accept_rejection) is moved so that the committed tokens are
 * contiguous: for i = 1 .. num_accepted[b], in every layer and KV head, K and V of slot
 * ctx_lens[b] + path_nodes[b][i] are copied to slot ctx_lens[b] + i (through the block table; the
 * root already sits at ctx_lens[b]).  new_ctx_lens[b] = ctx_lens[b] + 1 + num_accepted[b].  Slots
 * past the new length keep stale values that no later call reads (attention reads only slots
 * below ctx_len plus the current tree's own slots).  The bonus token has no K/V yet: it is the
 * root of the next verification, at slot new_ctx_lens[b].
 * A sequence with num_accepted[b] < 0 (a path that did not fit max_path) is left untouched and
 * keeps its length.  Copies are exact (bytes).
 *
 * Device preconditions: path_nodes[b][i] is a node of sequence b at depth i (so i <= node <
 * max_nodes); entries that are not are skipped.  ctx_lens[b] + max_nodes slots are mapped by the
 * block table.
 * ------------------------------------------------------------------------------------------ */
#define SPEC_MAX_COMMIT_LAYERS 128

typedef struct spec_kv_commit_args {
  int32_t batch;                /* >= 1 */
  int32_t num_layers;           /* 1 .. SPEC_MAX_COMMIT_LAYERS */
  int32_t num_kv_heads;         /* >= 1 */
  int32_t head_dim;             /* 64 or 128 */
  int32_t max_nodes;            /* (host) bound on tree nodes per sequence, 1..SPEC_MAX_TREE_NODES */
  int32_t max_path;             /* row stride of path_nodes, >= 1 */
  const void* const* k_caches;  /* (host) [num_layers] device pointers (bf16, 16-byte aligned) */
  const void* const* v_caches;  /* (host) [num_layers] device pointers (bf16, 16-byte aligned) */
  int64_t page_stride;          /* elements, shared by every layer (as in spec_paged_kv) */
  int64_t head_stride;
  int64_t token_stride;
  int32_t page_size;            /* a power of two in [8, 1024] */
  int32_t num_pages;            /* (host) pages in each layer's pool */
  const int32_t* block_table;   /* int32 [batch][block_table_stride] */
  int32_t block_table_stride;
  int32_t v_layout;             /* spec_v_layout */
  const int32_t* ctx_lens;      /* int32 [batch] */
  const int32_t* num_accepted;  /* int32 [batch] */
  const int32_t* path_nodes;    /* int32 [batch][max_path] */
  int32_t* new_ctx_lens;        /* int32 [batch] out; may be ctx_lens itself, and may overlap num_accepted
                                   or path_nodes (then the lengths are written by a second launch) */
} spec_kv_commit_args;

int spec_kv_commit(const spec_kv_commit_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_draft_gather  [DS "What DiffSpec Does": item 2 (a bounded working set of important
 * long-range context for the draft) and the paragraph after the list (chunks chosen from the
 * target's paged KV, joined with a rolling recent window, rebuilt as a compact draft cache at
 * local positions); DS "Architecture" (dual-view draft cache: canonical pre-RoPE KV at absolute
 * positions, compact cache with local draft RoPE positions); DS "Configuration" (chunk size,
 * token budget)]
 *
 * Builds each sequence's compact draft KV from its canonical pre-RoPE draft cache (paged like the
 * target's).  With L = ctx_lens[b] and w0 = max(0, L - window), context token t < L is kept iff
 * t >= w0 or chunk t / chunk_size is among chunk_index[b][0 .. num_select) (ids outside
 * [0, ceil(L / chunk_size)), -1 padding and repeated ids select nothing more).  Kept tokens keep
 * their order; compact slot j holds the j-th of them:
 *   out_pos[b][j]      = t, its absolute position (-1 for j >= out_len[b], up to capacity)
 *   out_k[b][j][h][:]  = K[t][h][:] rotated at local position j (as stored for SPEC_ROPE_NONE)
 *   out_v[b][j][h][:]  = V[t][h][:] (bytes)
 *   out_len[b]         = kept tokens, <= num_select * chunk_size + window <= capacity
 * Rotation: pair i, i < head_dim / 2 (dims (i, i + head_dim/2) for SPEC_ROPE_HALF, (2i, 2i + 1)
 * for SPEC_ROPE_PAIRS), turns by the angle j * inv_freq[i]: (x, y) -> (x cos - y sin, y cos + x sin).
 * The angle is formed exactly and its cosine and sine evaluated in fp64; the rotation runs in
 * fp32 and rounds to bf16 (RNE).  K/V slots j >= out_len[b] are not written.
 * chunk_index may be the topk_index output of spec_chunk_salience (row stride top_k): its first
 * num_select entries are the num_select heaviest chunks.
 *
 * Device preconditions: 0 <= ctx_lens[b] <= max_ctx_len; block-table ids < kv.num_pages (a kept
 * row on an invalid page is written as zeros).
 * ------------------------------------------------------------------------------------------ */
typedef enum spec_rope {
  SPEC_ROPE_NONE = 0,   /* copy K as stored (the compact cache stays pre-RoPE) */
  SPEC_ROPE_HALF = 1,   /* pairs (i, i + head_dim/2): the rotate-half form of Llama and Qwen */
  SPEC_ROPE_PAIRS = 2   /* pairs (2i, 2i + 1): the interleaved form */
} spec_rope;

typedef struct spec_draft_gather_args {
  int32_t batch;                /* >= 1, <= 65535 */
  int32_t num_kv_heads;         /* >= 1 */
  int32_t head_dim;             /* 64 or 128 */
  int32_t max_ctx_len;          /* (host) bound on ctx_lens[b]; ceil(max_ctx_len / chunk_size) <= 2^18 */
  const int32_t* ctx_lens;      /* int32 [batch] */
  spec_paged_kv kv;             /* canonical pre-RoPE draft K/V at absolute positions;
                                   block_table_stride >= ceil(max_ctx_len / page_size) */
  int32_t chunk_size;           /* 1 .. 65536 tokens per chunk */
  int32_t window;               /* recent tokens always kept, >= 0 */
  int32_t num_select;           /* chunk ids read per sequence, 0 .. 8192 */
  const int32_t* chunk_index;   /* int32 [batch][chunk_index_stride]; NULL if num_select == 0 */
  int32_t chunk_index_stride;   /* >= num_select */
  int32_t capacity;             /* compact slots per sequence, >= num_select * chunk_size + window, <= 2^24 */
  int32_t rope;                 /* spec_rope */
  const float* inv_freq;        /* fp32 [head_dim / 2]; NULL for SPEC_ROPE_NONE */
  void* out_k;                  /* bf16 [batch][capacity][num_kv_heads][head_dim], 16-byte aligned */
  void* out_v;                  /* bf16 [batch][capacity][num_kv_heads][head_dim], 16-byte aligned */
  int32_t* out_pos;             /* int32 [batch][capacity] */
  int32_t* out_len;             /* int32 [batch] */
} spec_draft_gather_args;

int spec_draft_gather(const spec_draft_gather_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_read_probe  (a measurement helper, not a step of the method)
 *
 * Reads every byte of data once with 16-byte loads and writes the XOR of all its 32-bit words to
 * sink[0], so that no load is elided; sink[1 .. SPEC_READ_PROBE_SINK_WORDS) is scratch for the
 * per-work-group partials.  Timing it over a buffer much larger than the caches gives the streaming-read
 * rate that bounds the library's HBM-bound calls, a measured ceiling beside the HBM peak of the spec
 * sheet.  bytes must be a positive multiple of 16 and data 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
#define SPEC_READ_PROBE_SINK_WORDS 2049

int spec_read_probe(const void* data, size_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------------------------
 * spec_tree_bundle_order (host code, no GPU)  [DSC "Features": the bundle scheduler groups
 * draft-tree leaves by their branching ancestor for prefix-coherent target verification]
 *
 * Renumbers one draft tree (parents[0] = -1, 0 <= parents[i] < i, host memory) in depth-first
 * preorder from the root, the children of a node in increasing index.  Every subtree becomes one
 * contiguous range, and the leaves under one branching node become adjacent, so consecutive
 * verification rows share their prefix.  Outputs, in the new numbering (host arrays of num_nodes):
 *   order[i]        original index of the node placed at i (the permutation to apply to the
 *                   tree's queries, draft tokens and tree K/V slots)
 *   new_parents[i]  parent position (-1 for the root)                       (may be NULL)
 *   subtree_end[i]  one past the last position of i's subtree: j is an ancestor-or-self of i
 *                   iff j <= i < subtree_end[j] (the subtree_end of spec_tree_attention_args)
 *   bundle[i]       position of i's nearest proper ancestor with >= 2 children, 0 if none
 *                   (0 for the root)                                        (may be NULL)
 * Returns SPEC_OK, or SPEC_ERR_INVALID_ARGUMENT naming the first bad parent, or
 * SPEC_ERR_UNSUPPORTED above SPEC_MAX_TREE_NODES nodes.  Allocates nothing.
 * ------------------------------------------------------------------------------------------ */
int spec_tree_bundle_order(const int32_t* parents, int32_t num_nodes, int32_t* order, int32_t* new_parents,
                           int32_t* subtree_end, int32_t* bundle);

/* ------------------------------------------------------------------------------------------
 * Draft-depth controller (host code, no GPU)  [AS "The controller"; DS "Configuration": long-
 * context threshold and initial depth; DS "Architecture": adaptive verification starts long
 * contexts shallow]
 *
 * With acceptance rate a per drafted token and cost ratio c = t_draft / t_target, a round that
 * drafts k tokens yields (1 - a^(k+1)) / (1 - a) tokens (k + 1 when a = 1) and costs
 * (k + 1) * c + 1 target forwards.  spec_controller_choose returns the k in [1, k_max] with the
 * largest ratio (the smallest such k on ties).  a is an exponentially weighted mean decayed per
 * observed token: in a round that drafted k and accepted n, the n accepted drafts are 1s and, if
 * n < k, the first rejected draft is a 0 (later drafts were never tested).  c is an exponentially
 * weighted mean per round of the measured draft/target time ratio.  A sequence whose context is
 * at least long_ctx_threshold starts at depth long_ctx_depth (later rounds use the closed form).
 * All functions return SPEC_OK or SPEC_ERR_INVALID_ARGUMENT (naming the argument).
 * ------------------------------------------------------------------------------------------ */
typedef struct spec_depth_controller {
  double alpha;                 /* current estimate of the acceptance rate, in [0, 1] */
  double cost_ratio;            /* current estimate of c = t_draft / t_target, > 0 */
  double alpha_decay;           /* weight of one new token observation, in (0, 1] */
  double cost_decay;            /* weight of one new round's cost ratio, in (0, 1] */
  int32_t k_max;                /* >= 1 */
  int32_t k;                    /* depth for the next round */
  int64_t rounds;               /* rounds observed */
} spec_depth_controller;

int spec_controller_init(spec_depth_controller* ctl, int32_t k_max, double alpha0, double cost_ratio0,
                         double alpha_decay, double cost_decay, int64_t ctx_len, int64_t long_ctx_threshold,
                         int32_t long_ctx_depth);
/* expected tokens per target forward for depth k: ((1 - a^(k+1)) / (1 - a)) / ((k + 1) c + 1) */
double spec_controller_speedup(double alpha, double cost_ratio, int32_t k);
/* (host) the k in [1, k_max] maximising spec_controller_speedup (smallest on ties); 0 on bad input */
int32_t spec_controller_choose(double alpha, double cost_ratio, int32_t k_max);
/* one verified round: k drafted, n accepted (0 <= n <= k), measured draft and target times
 * (t_target > 0; t_draft >= 0, 0 keeps the cost estimate); updates alpha, cost_ratio and k */
int spec_controller_update(spec_depth_controller* ctl, int32_t drafted, int32_t accepted, double t_draft,
                           double t_target);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
