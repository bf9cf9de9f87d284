// Internal declarations shared by the host layer and the kernel launchers of libspec_verify.
// Not part of the public ABI (include/spec_verify.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace spec {

constexpr int kTile = 64;          // KV slots per attention tile
constexpr int kRingFloats = 2048;  // chunk values a 4-wave attention work-group holds between two writes
constexpr int kMaxNodes = 256;     // tree nodes per sequence with ancestor bit masks (4 x 64 bits)
constexpr int kMaxTreeNodes = SPEC_MAX_TREE_NODES;   // tree nodes per sequence otherwise
constexpr int kSegment = 8192;     // vocabulary elements per argmax work-group
constexpr int kRejSegment = 8192;  // vocabulary elements per rejection work-group
constexpr int kMaxTopK = 8192;     // chunks sorted by one work-group for top-k
constexpr int kMaxSplitPages = 1024;  // page ids of one attention split staged in LDS

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------------------------------
// tree attention: launch plan and workspace layout (a pure function of the host bounds)
// ------------------------------------------------------------------------------------------
struct AttnPlan {
  int G = 0;             // query heads per KV head
  int waves = 0;         // waves per work-group (4 or 8)
  int rb = 0;            // 16-row MFMA blocks per wave (2)
  int rows_wg = 0;       // query rows per work-group = waves * 32
  int row_groups = 0;    // work-groups sharing one KV range (rows of one KV head / rows_wg)
  int rows_pad = 0;      // row_groups * rows_wg
  int chunk_cs = 0;      // chunk_lse2 strides (floats) of a chunk and of a KV head; see AttnParams
  int chunk_hs = 0;
  int max_tiles = 0;     // ceil((max_ctx_len + max_nodes) / 64)
  int split_tiles = 0;   // tiles per split
  int max_splits = 0;    // ceil(max_tiles / split_tiles)
  int max_chunks = 0;    // ceil(max_ctx_len / chunk_size), 0 without salience
  size_t off_part_o = 0, off_part_ml = 0, off_chunk = 0, off_lse2 = 0, off_debug = 0, bytes = 0;
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t page_stride, head_stride, token_stride;
  int page_shift;
  int num_pages;
  int v_dim_major;       // 1: V pages store each dim's page_size tokens contiguously
  const int32_t* block_table;
  int bt_stride;
  const int32_t* ctx_lens;
  const int32_t* node_offsets;
  const int32_t* parents;
  const int32_t* subtree_end;   // preorder trees: ancestors as index ranges (NULL: bit masks from parents)
  int batch, Hq, Hkv, G, max_nodes, max_ctx;
  float scale_log2;      // scale * log2(e)
  int chunk_size, max_chunks;
  int split_tiles, max_splits, row_groups, rows_pad;
  int chunk_cs, chunk_hs;  // chunk_lse2 strides (floats) of a chunk and of a KV head
  float* part_o;         // [batch][Hkv][max_splits][rows_pad][D]
  float* part_ml;        // [batch][Hkv][max_splits][rows_pad][2]  (running max in log2 units, sum)
  float* chunk_lse2;     // per sequence max_chunks * Hkv * max_nodes * G floats; (chunk c, KV head h, row r =
                         // node * G + g, query head h * G + g) at c * chunk_cs + h * chunk_hs + r: chunk-major
                         // ([chunk][h][row]) when max_nodes * G is a multiple of 32, else [h][chunk][row]
  float* lse2;           // [batch][Hkv][max_nodes * G], rows ordered as in chunk_lse2
  uint16_t* out;         // bf16 [total_nodes][Hq][D]
  float* lse;            // [total_nodes][Hq] natural log, nullable
};

bool make_attn_plan(const spec_tree_attention_args* a, int num_cus, AttnPlan* plan);
hipError_t launch_tree_attention(const AttnParams& p, const AttnPlan& plan, int head_dim, hipStream_t s);

// ------------------------------------------------------------------------------------------
// chunk salience
// ------------------------------------------------------------------------------------------
struct SalienceParams {
  const int32_t* ctx_lens;
  const int32_t* node_offsets;
  int batch, Hq, Hkv, max_nodes, max_ctx, chunk_size;
  int ws_max_chunks;     // chunk stride of the attention workspace
  int chunk_cs, chunk_hs;  // its strides (floats) of a chunk and of a KV head
  const float* chunk_lse2;
  const float* lse2;
  float* chunk_mass;     // [batch][max_chunks]
  int max_chunks;
  int accumulate;
  int top_k;
  int32_t* topk_index;
  float* topk_mass;
};
hipError_t launch_chunk_salience(const SalienceParams& p, hipStream_t s);

// ------------------------------------------------------------------------------------------
// acceptance
// ------------------------------------------------------------------------------------------
struct AcceptParams {
  int batch, vocab, max_nodes, max_path, nseg, nsegr;
  const int32_t* node_offsets;
  const int32_t* parents;
  const int32_t* draft_tokens;
  const void* logits;
  int bf16;              // 1: bf16 logits, 0: fp32
  int32_t* out_num_accepted;
  int32_t* out_path_nodes;
  int32_t* out_tokens;
  unsigned long long* seg_key;   // [batch*max_nodes][nseg] packed (ordered value, ~index); rejection:
                                 // one per residual segment (nseg == nsegr)
  // rejection only
  int max_children;
  const float* draft_probs;
  const float* u_accept;
  const float* u_sample;
  unsigned long long* node_key;   // [batch*max_nodes] row maximum key
  double* seg_sum;       // [batch*max_nodes][max_children+1][nsegr] residual sums per segment
  int32_t* acc_ok;       // [batch*max_nodes] 1: the node's draft passed its accept test
  int32_t* bonus_tok;    // [batch*max_nodes] the token drawn from the node's last residual
  uint32_t* sync_cnt;    // [batch] sequence counters (finished nodes), then 1 error word
  uint32_t* dbg;         // the debug record (SPEC_DEBUG build: witness counters of the walk), else NULL
};
// byte offsets of the rejection workspace's arrays (seg_key first, at 0)
struct RejectionLayout {
  size_t off_node_key, off_seg_sum, off_acc_ok, off_bonus, off_sync, bytes;
};
RejectionLayout rejection_layout(int batch, int max_nodes, int nsegr, int max_children);
size_t greedy_keys_bytes(int batch, int max_nodes, int nseg);   // the segment-key array alone
size_t greedy_ws_bytes(int batch, int max_nodes, int nseg);     // keys + the debug record
size_t rejection_ws_bytes(int batch, int max_nodes, int nsegr, int max_children);
hipError_t launch_accept_greedy(const AcceptParams& p, hipStream_t s);

// ------------------------------------------------------------------------------------------
// KV commit
// ------------------------------------------------------------------------------------------
struct KvCommitParams {
  void* k[SPEC_MAX_COMMIT_LAYERS];
  void* v[SPEC_MAX_COMMIT_LAYERS];
  int batch, num_layers, Hkv, max_nodes, max_path;
  int64_t page_stride, head_stride, token_stride;
  int page_shift, num_pages, v_dim_major;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* ctx_lens;
  const int32_t* num_accepted;
  const int32_t* path_nodes;
  int32_t* new_ctx_lens;
  int lengths_in_commit;  // 1: new_ctx_lens shares no byte with ctx_lens, num_accepted or path_nodes, so the
                          //    move kernel writes it
};
hipError_t launch_kv_commit(const KvCommitParams& p, int head_dim, hipStream_t s);
hipError_t launch_accept_rejection(const AcceptParams& p, hipStream_t s);

// ------------------------------------------------------------------------------------------
// compact draft KV gather
// ------------------------------------------------------------------------------------------
constexpr int kMaxSelect = 8192;          // chunk ids read per sequence
constexpr int kMaxGatherChunks = 1 << 18; // chunks per sequence (the selection bitmap is 32 KB of LDS)
struct DraftGatherParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t page_stride, head_stride, token_stride;
  int page_shift, num_pages, v_dim_major;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* ctx_lens;
  int batch, Hkv, max_ctx, chunk_size, window, num_select;
  const int32_t* chunk_index;
  int ci_stride;
  int capacity;
  int nwords;            // 32-bit words of the selection bitmap: ceil(ceil(max_ctx / chunk_size) / 32)
  const float* inv_freq;
  uint16_t* out_k;       // bf16 [batch][capacity][Hkv][D]
  uint16_t* out_v;
  int32_t* out_pos;      // [batch][capacity]
  int32_t* out_len;      // [batch]
};
hipError_t launch_draft_gather(const DraftGatherParams& p, int head_dim, int rope, hipStream_t s);

// ------------------------------------------------------------------------------------------
// device-side precondition checks (run by the SPEC_DEBUG build only)
// ------------------------------------------------------------------------------------------
hipError_t launch_debug_attn_check(const AttnParams& p, uint32_t* rec, hipStream_t s);
hipError_t launch_debug_accept_check(const AcceptParams& p, uint32_t* rec, int rejection, hipStream_t s);

// ------------------------------------------------------------------------------------------
// streaming-read probe
// ------------------------------------------------------------------------------------------
constexpr int kProbeGrid = 2048;  // work-groups of the probe (8 per CU); the sink holds 1 + this many words
hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* sink, int grid, hipStream_t s);

}  // namespace spec
