// Device-side precondition checks of the SPEC_DEBUG build (libspec_verify_debug.so).
//
// Per-row bookkeeping (which cache slots a row may read, which node is whose parent) is where
// speculative decoders go wrong most often ("Adaptive Speculative Decoding", "Correctness first").
// The release library does not read its device inputs twice to check them: its kernels clamp every
// index derived from device data, so a violated precondition gives wrong values, never an access
// out of bounds.  The debug build runs these kernels before the call's own kernels; they check the
// preconditions the header lists and leave one error bit per kind of violation in the call's debug
// record (uint32 words at the end of its workspace):
//   [0] error bits (SPEC_DBG_*)      [1], [2] acceptance witnesses, cleared here, counted by the walk
// The acceptance checks also clear the per-row results the walk reads (segment keys for greedy, row
// maxima for rejection), so the walk's witness counts only rows reduced in this call.
// Every integer OR and add is exact, so the record is deterministic.
#include "spec_internal.h"

namespace spec {
namespace {

constexpr int kCheckThreads = 1024;

__device__ __forceinline__ void or_bits(uint32_t* lds_bits, uint32_t my) {
  if (my) atomicOr(lds_bits, my);
}

// One work-group: node offsets, context lengths, parents (or subtree ends) and every block-table entry
// the call reads.  Writes the whole record.
__global__ __launch_bounds__(kCheckThreads) void debug_attn_check_kernel(AttnParams p, uint32_t* rec) {
  __shared__ uint32_t bits;
  const int tid = threadIdx.x;
  if (tid == 0) bits = 0;
  __syncthreads();
  uint32_t my = 0;
  if (tid == 0 && p.node_offsets[0] != 0) my |= SPEC_DBG_NODE_OFFSETS;
  for (int b = tid; b < p.batch; b += kCheckThreads) {
    const int o0 = p.node_offsets[b], o1 = p.node_offsets[b + 1];
    if (o1 < o0 || o1 - o0 > p.max_nodes) my |= SPEC_DBG_NODE_OFFSETS;
    const int L = p.ctx_lens[b];
    if (L < 0 || L > p.max_ctx) my |= SPEC_DBG_CTX_LENS;
  }
  for (int b = 0; b < p.batch; ++b) {
    // the bounds the attention kernels use (clamped the same way)
    int n0 = p.node_offsets[b];
    int N = p.node_offsets[b + 1] - n0;
    N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
    n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
    int L = p.ctx_lens[b];
    L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
    for (int i = tid; i < N; i += kCheckThreads) {
      if (p.subtree_end) {
        const int e = p.subtree_end[n0 + i];
        if (e <= i || e > N) my |= SPEC_DBG_SUBTREE_END;
      }
      if (p.parents) {
        const int pi = p.parents[n0 + i];
        if (i == 0 ? pi != -1 : (pi < 0 || pi >= i)) my |= SPEC_DBG_PARENTS;
      }
    }
    const int64_t slots = (int64_t)L + N;
    const int64_t pages = (slots + (1 << p.page_shift) - 1) >> p.page_shift;
    const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
    for (int64_t j = tid; j < pages && j < p.bt_stride; j += kCheckThreads) {
      const int pg = bt[j];
      if (pg < 0 || pg >= p.num_pages) my |= SPEC_DBG_BLOCK_TABLE;
    }
  }
  or_bits(&bits, my);
  __syncthreads();
  if (tid < 4) rec[tid] = tid == 0 ? bits : 0u;
}

// One work-group: node offsets, parents, draft tokens, child counts and uniforms (rejection); clears the
// per-row results the walk reads.  Writes the whole record.
__global__ __launch_bounds__(kCheckThreads) void debug_accept_check_kernel(AcceptParams p, uint32_t* rec,
                                                                           int rejection) {
  __shared__ uint32_t bits;
  const int tid = threadIdx.x;
  if (tid == 0) bits = 0;
  __syncthreads();
  uint32_t my = 0;
  if (tid == 0 && p.node_offsets[0] != 0) my |= SPEC_DBG_NODE_OFFSETS;
  for (int b = tid; b < p.batch; b += kCheckThreads) {
    const int o0 = p.node_offsets[b], o1 = p.node_offsets[b + 1];
    if (o1 < o0 || o1 - o0 > p.max_nodes) my |= SPEC_DBG_NODE_OFFSETS;
  }
  // the per-row results the walk reads start this call at zero (no real key or maximum is zero)
  const int64_t rows = (int64_t)p.batch * p.max_nodes;
  if (rejection) {
    for (int64_t r = tid; r < rows; r += kCheckThreads) p.node_key[r] = 0ull;
  } else {
    for (int64_t r = tid; r < rows * p.nseg; r += kCheckThreads) p.seg_key[r] = 0ull;
  }
  for (int b = 0; b < p.batch; ++b) {
    int n0 = p.node_offsets[b];
    int N = p.node_offsets[b + 1] - n0;
    N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
    n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
    for (int i = tid; i < N; i += kCheckThreads) {
      const int pi = p.parents[n0 + i];
      if (i == 0 ? pi != -1 : (pi < 0 || pi >= i)) my |= SPEC_DBG_PARENTS;
      const int t = p.draft_tokens[n0 + i];
      if (i > 0 && (t < 0 || t >= p.vocab)) my |= SPEC_DBG_TOKENS;
      if (rejection) {
        const float us = p.u_sample[n0 + i];
        if (!(us >= 0.f && us < 1.f)) my |= SPEC_DBG_UNIFORMS;
        if (i > 0) {
          const float ua = p.u_accept[n0 + i];
          if (!(ua >= 0.f && ua < 1.f)) my |= SPEC_DBG_UNIFORMS;
        }
        int kids = 0;
        for (int j = i + 1; j < N; ++j) kids += p.parents[n0 + j] == i ? 1 : 0;
        if (kids > p.max_children) my |= SPEC_DBG_CHILDREN;
      }
    }
  }
  or_bits(&bits, my);
  __syncthreads();
  if (tid < 4) rec[tid] = tid == 0 ? bits : 0u;
}

// One work-group per row of logits: NaN target logits, and (rejection) draft probabilities that are
// negative or not finite.  ORs into the record written by debug_accept_check_kernel.
__global__ __launch_bounds__(256) void debug_rows_check_kernel(AcceptParams p, uint32_t* rec, int rejection) {
  __shared__ uint32_t bits;
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  int tn = p.node_offsets[p.batch];
  tn = tn < 0 ? 0 : (tn > p.batch * p.max_nodes ? p.batch * p.max_nodes : tn);
  if (u >= tn) return;
  if (tid == 0) bits = 0;
  __syncthreads();
  uint32_t my = 0;
  for (int v = tid; v < p.vocab; v += 256) {
    float l;
    if (p.bf16) l = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p.logits)[u * p.vocab + v] << 16);
    else l = reinterpret_cast<const float*>(p.logits)[u * p.vocab + v];
    if (l != l) my |= SPEC_DBG_LOGITS;
    if (rejection) {
      const float q = p.draft_probs[u * p.vocab + v];
      if (!(q >= 0.f && q <= 3.402823466e38f)) my |= SPEC_DBG_DRAFT_PROBS;
    }
  }
  or_bits(&bits, my);
  __syncthreads();
  if (tid == 0 && bits) atomicOr(rec, bits);
}

}  // namespace

hipError_t launch_debug_attn_check(const AttnParams& p, uint32_t* rec, hipStream_t s) {
  hipLaunchKernelGGL(debug_attn_check_kernel, dim3(1), dim3(kCheckThreads), 0, s, p, rec);
  return hipGetLastError();
}

hipError_t launch_debug_accept_check(const AcceptParams& p, uint32_t* rec, int rejection, hipStream_t s) {
  hipLaunchKernelGGL(debug_accept_check_kernel, dim3(1), dim3(kCheckThreads), 0, s, p, rec, rejection);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(debug_rows_check_kernel, dim3((unsigned)(p.batch * p.max_nodes)), dim3(256), 0, s, p, rec,
                     rejection);
  return hipGetLastError();
}

}  // namespace spec
