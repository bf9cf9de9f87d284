// Host layer of libspec_verify: argument validation, launch plans, workspace layout and the
// extern "C" entry points declared in include/spec_verify.h.
//
// Every host-visible argument is checked before anything is enqueued, and a refusal names the
// argument and the accepted values (the vllm.cpp "Speculative decoding" documentation, section
// "Which keys the JSON accepts": refuse what cannot be honoured, by name, never downgrade silently).
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "spec_internal.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return SPEC_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SPEC_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

}  // namespace

namespace spec {
// status and thread-local message for the host-only functions (what == nullptr: success)
int host_fail(int status, const char* what) {
  if (!what) {
    g_err.clear();
    return SPEC_OK;
  }
  g_err = what;
  return status;
}
}  // namespace spec

namespace {

constexpr int kPlanCUs = 256;   // MI355X compute units; the plan is a pure function of the arguments

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Checks a paged KV description whose block table must map need_slots logical slots per sequence.
int check_kv(const spec_paged_kv& kv, int head_dim, int64_t need_slots, const char* need_text) {
  if (!kv.k_cache || !aligned(kv.k_cache, 16))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.k_cache: NULL or not 16-byte aligned");
  if (!kv.v_cache || !aligned(kv.v_cache, 16))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.v_cache: NULL or not 16-byte aligned");
  if (!kv.block_table) return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.block_table: NULL");
  if (kv.page_stride <= 0 || kv.page_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.page_stride: %lld, must be a positive multiple of 8",
                (long long)kv.page_stride);
  if (kv.head_stride < 0 || kv.head_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.head_stride: %lld, must be a non-negative multiple of 8",
                (long long)kv.head_stride);
  if (kv.token_stride < head_dim || kv.token_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.token_stride: %lld, must be a multiple of 8 and >= head_dim (%d)",
                (long long)kv.token_stride, head_dim);
  if (!pow2(kv.page_size) || kv.page_size < 8 || kv.page_size > 1024)
    return fail(SPEC_ERR_UNSUPPORTED, "kv.page_size: %d, must be a power of two in 8..1024", kv.page_size);
  if (kv.page_stride > INT32_MAX || kv.token_stride * kv.page_size > INT32_MAX)
    return fail(SPEC_ERR_UNSUPPORTED, "kv.page_stride and kv.token_stride * page_size must be < 2^31 elements");
  if (kv.num_pages < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.num_pages: %d, must be >= 1", kv.num_pages);
  if (kv.v_layout != SPEC_V_TOKEN_ROWS && kv.v_layout != SPEC_V_DIM_MAJOR)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.v_layout: %d, must be SPEC_V_TOKEN_ROWS (0) or SPEC_V_DIM_MAJOR (1)",
                kv.v_layout);
  const int64_t need_blocks = spec::ceil_div(need_slots, kv.page_size);
  if (kv.block_table_stride < need_blocks)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "kv.block_table_stride: %d, must be >= %s = %lld", kv.block_table_stride,
                need_text, (long long)need_blocks);
  return SPEC_OK;
}

// Checks everything about the attention arguments except the workspace.
int check_attn(const spec_tree_attention_args* a) {
  if (!a) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  if (a->batch < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "batch: %d, must be >= 1", a->batch);
  if (a->num_kv_heads < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "num_kv_heads: %d, must be >= 1", a->num_kv_heads);
  if (a->num_q_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "num_q_heads: %d, must be a positive multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim: %d, supported values are 64 and 128", a->head_dim);
  if (a->max_nodes < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "max_nodes: %d, must be >= 1", a->max_nodes);
  const int node_cap = a->subtree_end ? spec::kMaxTreeNodes : spec::kMaxNodes;
  if (a->max_nodes > node_cap)
    return fail(SPEC_ERR_UNSUPPORTED, "max_nodes: %d, supported range is 1..%d%s", a->max_nodes, node_cap,
                a->subtree_end ? "" : " (up to 2048 for trees in preorder, with subtree_end)");
  if (a->max_ctx_len < 0 || a->max_ctx_len > (1 << 30))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "max_ctx_len: %d, must be in 0..2^30", a->max_ctx_len);
  if ((int64_t)a->batch * a->max_nodes * a->num_q_heads > (1LL << 30))
    return fail(SPEC_ERR_UNSUPPORTED, "batch * max_nodes * num_q_heads: too large (limit 2^30)");
  if (!a->ctx_lens) return fail(SPEC_ERR_INVALID_ARGUMENT, "ctx_lens: NULL");
  if (!a->node_offsets) return fail(SPEC_ERR_INVALID_ARGUMENT, "node_offsets: NULL");
  if (!a->parents && !a->subtree_end)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "parents: NULL (needed unless subtree_end is given)");
  if (!a->q || !aligned(a->q, 16)) return fail(SPEC_ERR_INVALID_ARGUMENT, "q: NULL or not 16-byte aligned");
  if (!a->out || !aligned(a->out, 16)) return fail(SPEC_ERR_INVALID_ARGUMENT, "out: NULL or not 16-byte aligned");
  const int kst = check_kv(a->kv, a->head_dim, (int64_t)a->max_ctx_len + a->max_nodes,
                           "ceil((max_ctx_len + max_nodes) / page_size)");
  if (kst != SPEC_OK) return kst;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "scale: %g, must be finite and > 0", (double)a->scale);
  if (a->chunk_size < 0) return fail(SPEC_ERR_INVALID_ARGUMENT, "chunk_size: %d, must be >= 0", a->chunk_size);
  if (a->chunk_size != 0 && a->chunk_size != 16 && a->chunk_size != 32 && a->chunk_size % spec::kTile != 0)
    return fail(SPEC_ERR_UNSUPPORTED, "chunk_size: %d, supported values are 0, 16, 32 and multiples of 64",
                a->chunk_size);
  if (a->split_tiles < 0) return fail(SPEC_ERR_INVALID_ARGUMENT, "split_tiles: %d, must be >= 0", a->split_tiles);
  return SPEC_OK;
}

struct AttnLayout {
  spec::AttnPlan plan;
  size_t bytes = 0;
  int ws_max_chunks = 0;
};

AttnLayout attn_layout(const spec_tree_attention_args* a) {
  AttnLayout l;
  spec::make_attn_plan(a, kPlanCUs, &l.plan);
  l.ws_max_chunks = l.plan.max_chunks;
  l.bytes = l.plan.bytes;
  return l;
}

int check_workspace(void* ws, size_t have, size_t need, const char* what) {
  if (need == 0) return SPEC_OK;
  if (!ws) return fail(SPEC_ERR_WORKSPACE, "%s: workspace is NULL, %zu bytes are needed", what, need);
  if (!aligned(ws, 256)) return fail(SPEC_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", what);
  if (have < need) return fail(SPEC_ERR_WORKSPACE, "%s: workspace_bytes %zu < %zu needed", what, have, need);
  return SPEC_OK;
}

spec::AttnParams attn_params(const spec_tree_attention_args* a, const AttnLayout& l) {
  spec::AttnParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->kv.k_cache);
  p.v = static_cast<const uint16_t*>(a->kv.v_cache);
  p.page_stride = a->kv.page_stride;
  p.head_stride = a->kv.head_stride;
  p.token_stride = a->kv.token_stride;
  p.page_shift = log2i(a->kv.page_size);
  p.num_pages = a->kv.num_pages;
  p.v_dim_major = a->kv.v_layout == SPEC_V_DIM_MAJOR ? 1 : 0;
  p.block_table = a->kv.block_table;
  p.bt_stride = a->kv.block_table_stride;
  p.ctx_lens = a->ctx_lens;
  p.node_offsets = a->node_offsets;
  p.parents = a->parents;
  p.subtree_end = a->subtree_end;
  p.batch = a->batch;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = l.plan.G;
  p.max_nodes = a->max_nodes;
  p.max_ctx = a->max_ctx_len;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.chunk_size = a->chunk_size;
  p.max_chunks = l.plan.max_chunks;
  p.split_tiles = l.plan.split_tiles;
  p.max_splits = l.plan.max_splits;
  p.row_groups = l.plan.row_groups;
  p.rows_pad = l.plan.rows_pad;
  p.chunk_cs = l.plan.chunk_cs;
  p.chunk_hs = l.plan.chunk_hs;
  char* ws = static_cast<char*>(a->workspace);
  p.part_o = reinterpret_cast<float*>(ws + l.plan.off_part_o);
  p.part_ml = reinterpret_cast<float*>(ws + l.plan.off_part_ml);
  p.lse2 = reinterpret_cast<float*>(ws + l.plan.off_lse2);
  p.chunk_lse2 = reinterpret_cast<float*>(ws + l.plan.off_chunk);
  p.out = static_cast<uint16_t*>(a->out);
  p.lse = a->lse;
  return p;
}

int check_greedy(const spec_accept_greedy_args* a) {
  if (!a) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  if (a->batch < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "batch: %d, must be >= 1", a->batch);
  if (a->vocab < 1 || a->vocab > (1 << 24))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "vocab: %d, must be in 1..2^24", a->vocab);
  if (a->max_nodes < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "max_nodes: %d, must be >= 1", a->max_nodes);
  if (a->max_nodes > spec::kMaxTreeNodes)
    return fail(SPEC_ERR_UNSUPPORTED, "max_nodes: %d, supported range is 1..%d", a->max_nodes, spec::kMaxTreeNodes);
  if ((int64_t)a->batch * a->max_nodes > 65535)
    return fail(SPEC_ERR_UNSUPPORTED, "batch * max_nodes: %lld, limit 65535", (long long)a->batch * a->max_nodes);
  if (a->max_path < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "max_path: %d, must be >= 1", a->max_path);
  if (!a->node_offsets) return fail(SPEC_ERR_INVALID_ARGUMENT, "node_offsets: NULL");
  if (!a->parents) return fail(SPEC_ERR_INVALID_ARGUMENT, "parents: NULL");
  if (!a->draft_tokens) return fail(SPEC_ERR_INVALID_ARGUMENT, "draft_tokens: NULL");
  if (!a->target_logits) return fail(SPEC_ERR_INVALID_ARGUMENT, "target_logits: NULL");
  if (a->logits_dtype != SPEC_DTYPE_BF16 && a->logits_dtype != SPEC_DTYPE_F32)
    return fail(SPEC_ERR_UNSUPPORTED, "logits_dtype: %d, supported are SPEC_DTYPE_BF16 (0) and SPEC_DTYPE_F32 (1)",
                a->logits_dtype);
  if (!aligned(a->target_logits, a->logits_dtype == SPEC_DTYPE_BF16 ? 2 : 4))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "target_logits: not aligned to its element size");
  if (!a->out_num_accepted) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_num_accepted: NULL");
  if (!a->out_path_nodes) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_path_nodes: NULL");
  if (!a->out_tokens) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_tokens: NULL");
  return SPEC_OK;
}

int nseg_of(int vocab) { return (int)spec::ceil_div(vocab, spec::kSegment); }
int nsegr_of(int vocab) { return (int)spec::ceil_div(vocab, spec::kRejSegment); }

spec::AcceptParams accept_params(const spec_accept_greedy_args* a) {
  spec::AcceptParams p{};
  p.batch = a->batch;
  p.vocab = a->vocab;
  p.max_nodes = a->max_nodes;
  p.max_path = a->max_path;
  p.nseg = nseg_of(a->vocab);
  p.node_offsets = a->node_offsets;
  p.parents = a->parents;
  p.draft_tokens = a->draft_tokens;
  p.logits = a->target_logits;
  p.bf16 = a->logits_dtype == SPEC_DTYPE_BF16;
  p.out_num_accepted = a->out_num_accepted;
  p.out_path_nodes = a->out_path_nodes;
  p.out_tokens = a->out_tokens;
  p.seg_key = static_cast<unsigned long long*>(a->workspace);
  return p;
}

}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

#ifdef SPEC_DEBUG
int spec_debug_build(void) { return 1; }
#else
int spec_debug_build(void) { return 0; }
#endif

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARGUMENT: return "SPEC_ERR_INVALID_ARGUMENT";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
    case SPEC_ERR_STATE: return "SPEC_ERR_STATE";
    default: return "unknown spec_status";
  }
}

const char* spec_last_error(void) { return g_err.c_str(); }

size_t spec_tree_attention_workspace_size(const spec_tree_attention_args* args) {
  if (check_attn(args) != SPEC_OK) return 0;
  g_err.clear();
  return attn_layout(args).bytes;
}

int spec_tree_attention(const spec_tree_attention_args* args, void* stream) {
  int st = check_attn(args);
  if (st != SPEC_OK) return st;
  const AttnLayout l = attn_layout(args);
  st = check_workspace(args->workspace, args->workspace_bytes, l.bytes, "spec_tree_attention");
  if (st != SPEC_OK) return st;
  const spec::AttnParams p = attn_params(args, l);
#ifdef SPEC_DEBUG
  {
    uint32_t* rec = reinterpret_cast<uint32_t*>(static_cast<char*>(args->workspace) + l.plan.off_debug);
    const hipError_t de = spec::launch_debug_attn_check(p, rec, static_cast<hipStream_t>(stream));
    if (de != hipSuccess) return hip_fail(de, "spec_tree_attention debug checks");
  }
#endif
  const hipError_t e = spec::launch_tree_attention(p, l.plan, args->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_tree_attention launch");
  return ok();
}

int spec_chunk_salience(const spec_chunk_salience_args* args, void* stream) {
  if (!args) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  if (!args->attn) return fail(SPEC_ERR_INVALID_ARGUMENT, "attn: NULL");
  const spec_tree_attention_args* a = args->attn;
  int st = check_attn(a);
  if (st != SPEC_OK) return fail(st, "attn->%s", g_err.c_str());
  if (a->chunk_size == 0)
    return fail(SPEC_ERR_STATE, "attn->chunk_size is 0: the attention call left no chunk partials");
  const AttnLayout l = attn_layout(a);
  st = check_workspace(a->workspace, a->workspace_bytes, l.bytes, "spec_chunk_salience (attn workspace)");
  if (st != SPEC_OK) return st;
  const int need_chunks = (int)spec::ceil_div(a->max_ctx_len, a->chunk_size);
  if (!args->chunk_mass) return fail(SPEC_ERR_INVALID_ARGUMENT, "chunk_mass: NULL");
  if (args->max_chunks < need_chunks || args->max_chunks < 1)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "max_chunks: %d, must be >= max(1, ceil(max_ctx_len / chunk_size)) = %d",
                args->max_chunks, need_chunks > 1 ? need_chunks : 1);
  if (args->accumulate != 0 && args->accumulate != 1)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "accumulate: %d, must be 0 or 1", args->accumulate);
  if (args->top_k < 0) return fail(SPEC_ERR_INVALID_ARGUMENT, "top_k: %d, must be >= 0", args->top_k);
  if (args->top_k > 0) {
    if (args->top_k > args->max_chunks)
      return fail(SPEC_ERR_INVALID_ARGUMENT, "top_k: %d, must be <= max_chunks (%d)", args->top_k, args->max_chunks);
    if (need_chunks > spec::kMaxTopK || args->top_k > spec::kMaxTopK)
      return fail(SPEC_ERR_UNSUPPORTED, "top_k selection over %d chunks: at most %d chunks are supported",
                  need_chunks, spec::kMaxTopK);
    if (!args->topk_index) return fail(SPEC_ERR_INVALID_ARGUMENT, "topk_index: NULL with top_k > 0");
    if (!args->topk_mass) return fail(SPEC_ERR_INVALID_ARGUMENT, "topk_mass: NULL with top_k > 0");
  }
  spec::SalienceParams p{};
  p.ctx_lens = a->ctx_lens;
  p.node_offsets = a->node_offsets;
  p.batch = a->batch;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.max_nodes = a->max_nodes;
  p.max_ctx = a->max_ctx_len;
  p.chunk_size = a->chunk_size;
  p.ws_max_chunks = l.ws_max_chunks;
  p.chunk_cs = l.plan.chunk_cs;
  p.chunk_hs = l.plan.chunk_hs;
  char* ws = static_cast<char*>(a->workspace);
  p.chunk_lse2 = reinterpret_cast<const float*>(ws + l.plan.off_chunk);
  p.lse2 = reinterpret_cast<const float*>(ws + l.plan.off_lse2);
  p.chunk_mass = args->chunk_mass;
  p.max_chunks = args->max_chunks;
  p.accumulate = args->accumulate;
  p.top_k = args->top_k;
  p.topk_index = args->topk_index;
  p.topk_mass = args->topk_mass;
  if (l.ws_max_chunks == 0) {    // no context anywhere: masses are all zero
    p.ws_max_chunks = 1;
  }
  const hipError_t e = spec::launch_chunk_salience(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_chunk_salience launch");
  return ok();
}

size_t spec_accept_greedy_workspace_size(const spec_accept_greedy_args* args) {
  if (check_greedy(args) != SPEC_OK) return 0;
  g_err.clear();
  return spec::greedy_ws_bytes(args->batch, args->max_nodes, nseg_of(args->vocab));
}

int spec_accept_greedy(const spec_accept_greedy_args* args, void* stream) {
  int st = check_greedy(args);
  if (st != SPEC_OK) return st;
  const size_t need = spec::greedy_ws_bytes(args->batch, args->max_nodes, nseg_of(args->vocab));
  st = check_workspace(args->workspace, args->workspace_bytes, need, "spec_accept_greedy");
  if (st != SPEC_OK) return st;
  spec::AcceptParams p = accept_params(args);
#ifdef SPEC_DEBUG
  {
    p.dbg = reinterpret_cast<uint32_t*>(static_cast<char*>(args->workspace) + need - SPEC_DEBUG_RECORD_BYTES);
    const hipError_t de = spec::launch_debug_accept_check(p, p.dbg, 0, static_cast<hipStream_t>(stream));
    if (de != hipSuccess) return hip_fail(de, "spec_accept_greedy debug checks");
  }
#endif
  const hipError_t e = spec::launch_accept_greedy(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_accept_greedy launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// spec_accept_greedy_noalloc: the greedy call with its segment keys in a file-scope device array
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = SPEC_GREEDY_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;

// Each GPU the library runs on holds its own copy.  In host code `scratch` names a host-side stand-in,
// not a device address: only the per-device pointers from hipGetSymbolAddress are handed to kernels.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The device address of this device's `scratch`, looked up once per device (with that device current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "spec_accept_greedy_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(SPEC_ERR_UNSUPPORTED, "spec_accept_greedy_noalloc: device %d, supported are 0..%d", dev,
                kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "spec_accept_greedy_noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SPEC_ERR_HIP, "spec_accept_greedy_noalloc: hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_accept_greedy_noalloc(const spec_accept_greedy_args* args, void* stream) {
  int st = check_greedy(args);
  if (st != SPEC_OK) return st;
  const size_t need = spec::greedy_ws_bytes(args->batch, args->max_nodes, nseg_of(args->vocab));
  if (need > kScratchBytes)
    return fail(SPEC_ERR_UNSUPPORTED,
                "spec_accept_greedy_noalloc: batch * max_nodes * ceil(vocab / %d) keys need %zu bytes, more than the "
                "%zu-byte device array; use spec_accept_greedy with a workspace",
                spec::kSegment, need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != SPEC_OK) return st;
  spec::AcceptParams p = accept_params(args);
  p.seg_key = static_cast<unsigned long long*>(ws);
  const hipError_t e = spec::launch_accept_greedy(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_accept_greedy_noalloc launch");
  return ok();
}

static int check_rejection(const spec_accept_rejection_args* a) {
  if (!a) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  int st = check_greedy(&a->base);
  if (st != SPEC_OK) return fail(st, "base.%s", g_err.c_str());
  if (a->max_children < 0 || a->max_children > a->base.max_nodes - 1)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "max_children: %d, must be in 0..max_nodes-1 (%d)", a->max_children,
                a->base.max_nodes - 1);
  if (!a->draft_probs) return fail(SPEC_ERR_INVALID_ARGUMENT, "draft_probs: NULL");
  if (!a->u_accept) return fail(SPEC_ERR_INVALID_ARGUMENT, "u_accept: NULL");
  if (!a->u_sample) return fail(SPEC_ERR_INVALID_ARGUMENT, "u_sample: NULL");
  return SPEC_OK;
}

size_t spec_accept_rejection_workspace_size(const spec_accept_rejection_args* args) {
  if (check_rejection(args) != SPEC_OK) return 0;
  g_err.clear();
  return spec::rejection_ws_bytes(args->base.batch, args->base.max_nodes, nsegr_of(args->base.vocab),
                                  args->max_children);
}

int spec_accept_rejection(const spec_accept_rejection_args* args, void* stream) {
  int st = check_rejection(args);
  if (st != SPEC_OK) return st;
  const spec_accept_greedy_args& g = args->base;
  const int nsegr = nsegr_of(g.vocab);
  const size_t need = spec::rejection_ws_bytes(g.batch, g.max_nodes, nsegr, args->max_children);
  st = check_workspace(g.workspace, g.workspace_bytes, need, "spec_accept_rejection");
  if (st != SPEC_OK) return st;
  spec::AcceptParams p = accept_params(&g);
  p.max_children = args->max_children;
  p.draft_probs = args->draft_probs;
  p.u_accept = args->u_accept;
  p.u_sample = args->u_sample;
  p.nsegr = nsegr;
  p.nseg = nsegr;                                 // rejection keeps its segment maxima per residual segment
  char* ws = static_cast<char*>(g.workspace);
  const spec::RejectionLayout l = spec::rejection_layout(g.batch, g.max_nodes, nsegr, args->max_children);
  p.node_key = reinterpret_cast<unsigned long long*>(ws + l.off_node_key);
  p.seg_sum = reinterpret_cast<double*>(ws + l.off_seg_sum);
  p.acc_ok = reinterpret_cast<int32_t*>(ws + l.off_acc_ok);
  p.bonus_tok = reinterpret_cast<int32_t*>(ws + l.off_bonus);
  p.sync_cnt = reinterpret_cast<uint32_t*>(ws + l.off_sync);
#ifdef SPEC_DEBUG
  {
    p.dbg = reinterpret_cast<uint32_t*>(ws + need - SPEC_DEBUG_RECORD_BYTES);
    const hipError_t de = spec::launch_debug_accept_check(p, p.dbg, 1, static_cast<hipStream_t>(stream));
    if (de != hipSuccess) return hip_fail(de, "spec_accept_rejection debug checks");
  }
#endif
  const hipError_t e = spec::launch_accept_rejection(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_accept_rejection launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// spec_kv_commit
// ---------------------------------------------------------------------------------------------
namespace {

int check_commit(const spec_kv_commit_args* a) {
  if (!a) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  if (a->batch < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "batch: %d, must be >= 1", a->batch);
  if (a->num_layers < 1 || a->num_layers > SPEC_MAX_COMMIT_LAYERS)
    return fail(SPEC_ERR_UNSUPPORTED, "num_layers: %d, supported range is 1..%d", a->num_layers,
                SPEC_MAX_COMMIT_LAYERS);
  if (a->num_kv_heads < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "num_kv_heads: %d, must be >= 1", a->num_kv_heads);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim: %d, supported values are 64 and 128", a->head_dim);
  if (a->max_nodes < 1 || a->max_nodes > spec::kMaxTreeNodes)
    return fail(SPEC_ERR_UNSUPPORTED, "max_nodes: %d, supported range is 1..%d", a->max_nodes, spec::kMaxTreeNodes);
  if (a->max_path < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "max_path: %d, must be >= 1", a->max_path);
  if ((int64_t)a->batch * a->max_path > (1LL << 30) || (int64_t)a->batch > 65535)
    return fail(SPEC_ERR_UNSUPPORTED, "batch: %d, too large (limit 65535 sequences per call)", a->batch);
  if (!a->k_caches || !a->v_caches) return fail(SPEC_ERR_INVALID_ARGUMENT, "k_caches / v_caches: NULL");
  for (int l = 0; l < a->num_layers; ++l) {
    if (!a->k_caches[l] || !aligned(a->k_caches[l], 16))
      return fail(SPEC_ERR_INVALID_ARGUMENT, "k_caches[%d]: NULL or not 16-byte aligned", l);
    if (!a->v_caches[l] || !aligned(a->v_caches[l], 16))
      return fail(SPEC_ERR_INVALID_ARGUMENT, "v_caches[%d]: NULL or not 16-byte aligned", l);
  }
  if (a->page_stride <= 0 || a->page_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "page_stride: %lld, must be a positive multiple of 8",
                (long long)a->page_stride);
  if (a->head_stride < 0 || a->head_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "head_stride: %lld, must be a non-negative multiple of 8",
                (long long)a->head_stride);
  if (a->token_stride < a->head_dim || a->token_stride % 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "token_stride: %lld, must be a multiple of 8 and >= head_dim (%d)",
                (long long)a->token_stride, a->head_dim);
  if (!pow2(a->page_size) || a->page_size < 8 || a->page_size > 1024)
    return fail(SPEC_ERR_UNSUPPORTED, "page_size: %d, must be a power of two in 8..1024", a->page_size);
  if (a->num_pages < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "num_pages: %d, must be >= 1", a->num_pages);
  if (!a->block_table) return fail(SPEC_ERR_INVALID_ARGUMENT, "block_table: NULL");
  if (a->block_table_stride < 1)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "block_table_stride: %d, must be >= 1", a->block_table_stride);
  if (a->v_layout != SPEC_V_TOKEN_ROWS && a->v_layout != SPEC_V_DIM_MAJOR)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "v_layout: %d, must be SPEC_V_TOKEN_ROWS (0) or SPEC_V_DIM_MAJOR (1)",
                a->v_layout);
  if (!a->ctx_lens) return fail(SPEC_ERR_INVALID_ARGUMENT, "ctx_lens: NULL");
  if (!a->num_accepted) return fail(SPEC_ERR_INVALID_ARGUMENT, "num_accepted: NULL");
  if (!a->path_nodes) return fail(SPEC_ERR_INVALID_ARGUMENT, "path_nodes: NULL");
  if (!a->new_ctx_lens) return fail(SPEC_ERR_INVALID_ARGUMENT, "new_ctx_lens: NULL");
  return SPEC_OK;
}

}  // namespace

extern "C" int spec_kv_commit(const spec_kv_commit_args* a, void* stream) {
  const int st = check_commit(a);
  if (st != SPEC_OK) return st;
  spec::KvCommitParams p{};
  for (int l = 0; l < a->num_layers; ++l) {
    p.k[l] = const_cast<void*>(a->k_caches[l]);
    p.v[l] = const_cast<void*>(a->v_caches[l]);
  }
  p.batch = a->batch;
  p.num_layers = a->num_layers;
  p.Hkv = a->num_kv_heads;
  p.max_nodes = a->max_nodes;
  p.max_path = a->max_path;
  p.page_stride = a->page_stride;
  p.head_stride = a->head_stride;
  p.token_stride = a->token_stride;
  p.page_shift = log2i(a->page_size);
  p.num_pages = a->num_pages;
  p.v_dim_major = a->v_layout == SPEC_V_DIM_MAJOR ? 1 : 0;
  p.block_table = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.ctx_lens = a->ctx_lens;
  p.num_accepted = a->num_accepted;
  p.path_nodes = a->path_nodes;
  p.new_ctx_lens = a->new_ctx_lens;
  const hipError_t e = spec::launch_kv_commit(p, a->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_kv_commit launch");
  return ok();
}

namespace {

int check_gather(const spec_draft_gather_args* a) {
  if (!a) return fail(SPEC_ERR_INVALID_ARGUMENT, "args: NULL");
  if (a->batch < 1 || a->batch > 65535)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "batch: %d, must be in 1..65535", a->batch);
  if (a->num_kv_heads < 1) return fail(SPEC_ERR_INVALID_ARGUMENT, "num_kv_heads: %d, must be >= 1", a->num_kv_heads);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim: %d, supported values are 64 and 128", a->head_dim);
  if (a->max_ctx_len < 0 || a->max_ctx_len > (1 << 30))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "max_ctx_len: %d, must be in 0..2^30", a->max_ctx_len);
  if (a->chunk_size < 1 || a->chunk_size > 65536)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "chunk_size: %d, must be in 1..65536", a->chunk_size);
  if (spec::ceil_div(a->max_ctx_len, a->chunk_size) > spec::kMaxGatherChunks)
    return fail(SPEC_ERR_UNSUPPORTED, "max_ctx_len / chunk_size: %lld chunks, supported up to %d",
                (long long)spec::ceil_div(a->max_ctx_len, a->chunk_size), spec::kMaxGatherChunks);
  if (!a->ctx_lens) return fail(SPEC_ERR_INVALID_ARGUMENT, "ctx_lens: NULL");
  const int kst = check_kv(a->kv, a->head_dim, a->max_ctx_len, "ceil(max_ctx_len / page_size)");
  if (kst != SPEC_OK) return kst;
  if (a->window < 0) return fail(SPEC_ERR_INVALID_ARGUMENT, "window: %d, must be >= 0", a->window);
  if (a->num_select < 0 || a->num_select > spec::kMaxSelect)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "num_select: %d, must be in 0..%d", a->num_select, spec::kMaxSelect);
  if (a->num_select > 0 && !a->chunk_index)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "chunk_index: NULL with num_select = %d", a->num_select);
  if (a->num_select > 0 && a->chunk_index_stride < a->num_select)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "chunk_index_stride: %d, must be >= num_select (%d)",
                a->chunk_index_stride, a->num_select);
  const int64_t need = (int64_t)a->num_select * a->chunk_size + a->window;
  if (a->capacity < 1 || a->capacity > (1 << 24) || a->capacity < need)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "capacity: %d, must be in 1..2^24 and >= num_select * chunk_size + "
                "window = %lld", a->capacity, (long long)need);
  if ((int64_t)a->batch * a->capacity * a->num_kv_heads * a->head_dim > (1LL << 40))
    return fail(SPEC_ERR_UNSUPPORTED, "batch * capacity * num_kv_heads * head_dim: too large");
  if (a->rope != SPEC_ROPE_NONE && a->rope != SPEC_ROPE_HALF && a->rope != SPEC_ROPE_PAIRS)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "rope: %d, must be SPEC_ROPE_NONE (0), SPEC_ROPE_HALF (1) or "
                "SPEC_ROPE_PAIRS (2)", a->rope);
  if (a->rope != SPEC_ROPE_NONE && !a->inv_freq)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "inv_freq: NULL with rope = %d", a->rope);
  if (!a->out_k || !aligned(a->out_k, 16)) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_k: NULL or not 16-byte aligned");
  if (!a->out_v || !aligned(a->out_v, 16)) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_v: NULL or not 16-byte aligned");
  if (!a->out_pos) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_pos: NULL");
  if (!a->out_len) return fail(SPEC_ERR_INVALID_ARGUMENT, "out_len: NULL");
  return SPEC_OK;
}

}  // namespace

extern "C" int spec_draft_gather(const spec_draft_gather_args* a, void* stream) {
  const int st = check_gather(a);
  if (st != SPEC_OK) return st;
  spec::DraftGatherParams p{};
  p.k = static_cast<const uint16_t*>(a->kv.k_cache);
  p.v = static_cast<const uint16_t*>(a->kv.v_cache);
  p.page_stride = a->kv.page_stride;
  p.head_stride = a->kv.head_stride;
  p.token_stride = a->kv.token_stride;
  p.page_shift = log2i(a->kv.page_size);
  p.num_pages = a->kv.num_pages;
  p.v_dim_major = a->kv.v_layout == SPEC_V_DIM_MAJOR ? 1 : 0;
  p.block_table = a->kv.block_table;
  p.bt_stride = a->kv.block_table_stride;
  p.ctx_lens = a->ctx_lens;
  p.batch = a->batch;
  p.Hkv = a->num_kv_heads;
  p.max_ctx = a->max_ctx_len;
  p.chunk_size = a->chunk_size;
  p.window = a->window;
  p.num_select = a->num_select;
  p.chunk_index = a->chunk_index;
  p.ci_stride = a->chunk_index_stride;
  p.capacity = a->capacity;
  p.nwords = (int)((spec::ceil_div(a->max_ctx_len, a->chunk_size) + 31) / 32);
  p.inv_freq = a->inv_freq;
  p.out_k = static_cast<uint16_t*>(a->out_k);
  p.out_v = static_cast<uint16_t*>(a->out_v);
  p.out_pos = a->out_pos;
  p.out_len = a->out_len;
  const hipError_t e = spec::launch_draft_gather(p, a->head_dim, a->rope, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_draft_gather launch");
  return ok();
}

extern "C" int spec_read_probe(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  if (!data || !aligned(data, 16)) return fail(SPEC_ERR_INVALID_ARGUMENT, "data: NULL or not 16-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(SPEC_ERR_INVALID_ARGUMENT, "bytes: %zu, must be a positive multiple of 16", bytes);
  if (!sink || !aligned(sink, 4)) return fail(SPEC_ERR_INVALID_ARGUMENT, "sink: NULL or not 4-byte aligned");
  static_assert(SPEC_READ_PROBE_SINK_WORDS == spec::kProbeGrid + 1, "sink size");
  const hipError_t e = spec::launch_read_probe(data, (int64_t)bytes, sink, spec::kProbeGrid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_read_probe launch");
  return ok();
}
