// Post-acceptance KV commit for gfx950: the accepted path's K/V rows move next to the committed
// context, and the per-sequence lengths advance ("Adaptive Speculative Decoding", section Layout:
// with a per-row length and a cache mask, rollback is a length update; here the accepted nodes of
// a tree are first made contiguous so that the committed prefix stays a plain prefix).
//
// One work-group per (sequence, layer, KV head).  Row i (depth i) moves from slot L + path[i] to
// slot L + i.  Since path[i] >= i, no move's source is the destination of an earlier or equal row,
// so rows are moved in increasing order, a batch of rows at a time: the whole batch is read into
// registers, then written (a source inside the batch may be another row's destination).  The new
// lengths are written by work-group (b, 0, 0) when they go to a buffer of their own; when they replace
// ctx_lens in place, a second launch writes them after every work-group has read the old ones.
#include "spec_internal.h"

namespace spec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCommitThreads = 128;
constexpr int kCommitRows = 16;

template <int D, int VT>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(KvCommitParams p) {
  constexpr int CPR = D / 8;                                  // 16-byte chunks per token row
  constexpr int RI = kCommitRows * CPR / kCommitThreads;      // row chunks per thread and batch
  constexpr int VI = kCommitRows * D / kCommitThreads;        // dim-major V elements per thread and batch
  const int b = blockIdx.x, layer = blockIdx.y, kvh = blockIdx.z;
  const int tid = threadIdx.x;
  const int L_in = p.ctx_lens[b], n_in = p.num_accepted[b];
  if (p.lengths_in_commit && layer == 0 && kvh == 0 && tid == 0)
    p.new_ctx_lens[b] = n_in >= 0 ? L_in + 1 + n_in : L_in;   // as kv_lengths_kernel
  int L = L_in;
  L = L < 0 ? 0 : L;
  int n = n_in;
  n = n < p.max_path - 1 ? n : p.max_path - 1;
  n = n < p.max_nodes - 1 ? n : p.max_nodes - 1;
  if (n <= 0) return;
  const int32_t* path = p.path_nodes + (int64_t)b * p.max_path;
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const int pmask = (1 << p.page_shift) - 1;
  const int64_t max_slot = (int64_t)p.bt_stride << p.page_shift;
  uint16_t* kb = static_cast<uint16_t*>(p.k[layer]) + (int64_t)kvh * p.head_stride;
  uint16_t* vb = static_cast<uint16_t*>(p.v[layer]) + (int64_t)kvh * p.head_stride;
  // element offset of (slot, element e of the row) or -1 when the slot has no valid page
  auto page_of = [&](int64_t slot) -> int64_t {
    if (slot < 0 || slot >= max_slot) return -1;
    const int pg = bt[slot >> p.page_shift];
    if (pg < 0 || pg >= p.num_pages) return -1;
    return (int64_t)pg * p.page_stride;
  };
  for (int i0 = 1; i0 <= n; i0 += kCommitRows) {
    u32x4 kval[RI], vval[VT ? 1 : RI];
    uint16_t vdm[VT ? VI : 1];
    // read phase
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      const int it = tid + kCommitThreads * q;
      const int row = i0 + it / CPR, c = it % CPR;
      const int node = row <= n ? path[row] : row;
      if (row <= n && node != row && node > row && node < p.max_nodes) {
        const int64_t slot = (int64_t)L + node;
        const int64_t pb = page_of(slot);
        if (pb >= 0) {
          const int64_t off = pb + (int64_t)(slot & pmask) * p.token_stride + 8 * c;
          kval[q] = *reinterpret_cast<const u32x4*>(kb + off);
          if (!VT) vval[q] = *reinterpret_cast<const u32x4*>(vb + off);
        }
      }
    }
    if (VT) {
#pragma unroll
      for (int q = 0; q < VI; ++q) {
        const int it = tid + kCommitThreads * q;
        const int row = i0 + it / D, d = it % D;
        const int node = row <= n ? path[row] : row;
        if (row <= n && node != row && node > row && node < p.max_nodes) {
          const int64_t slot = (int64_t)L + node;
          const int64_t pb = page_of(slot);
          if (pb >= 0) vdm[q] = vb[pb + ((int64_t)d << p.page_shift) + (slot & pmask)];
        }
      }
    }
    __syncthreads();                                          // every read of the batch is done
    // write phase (same conditions, destination slot L + row)
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      const int it = tid + kCommitThreads * q;
      const int row = i0 + it / CPR, c = it % CPR;
      const int node = row <= n ? path[row] : row;
      if (row <= n && node != row && node > row && node < p.max_nodes) {
        const int64_t src = (int64_t)L + node, slot = (int64_t)L + row;
        const int64_t pb = page_of(slot);
        if (pb >= 0 && page_of(src) >= 0) {
          const int64_t off = pb + (int64_t)(slot & pmask) * p.token_stride + 8 * c;
          *reinterpret_cast<u32x4*>(kb + off) = kval[q];
          if (!VT) *reinterpret_cast<u32x4*>(vb + off) = vval[q];
        }
      }
    }
    if (VT) {
#pragma unroll
      for (int q = 0; q < VI; ++q) {
        const int it = tid + kCommitThreads * q;
        const int row = i0 + it / D, d = it % D;
        const int node = row <= n ? path[row] : row;
        if (row <= n && node != row && node > row && node < p.max_nodes) {
          const int64_t src = (int64_t)L + node, slot = (int64_t)L + row;
          const int64_t pb = page_of(slot);
          if (pb >= 0 && page_of(src) >= 0) vb[pb + ((int64_t)d << p.page_shift) + (slot & pmask)] = vdm[q];
        }
      }
    }
    __syncthreads();                                          // writes done before the next batch reads
  }
}

__global__ __launch_bounds__(256) void kv_lengths_kernel(KvCommitParams p) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= p.batch) return;
  const int L = p.ctx_lens[b];
  const int n = p.num_accepted[b];
  p.new_ctx_lens[b] = n >= 0 ? L + 1 + n : L;
}

template <int D>
hipError_t launch_d(const KvCommitParams& p, hipStream_t s) {
  const dim3 grid(p.batch, p.num_layers, p.Hkv);
  if (p.v_dim_major) hipLaunchKernelGGL((kv_commit_kernel<D, 1>), grid, dim3(kCommitThreads), 0, s, p);
  else hipLaunchKernelGGL((kv_commit_kernel<D, 0>), grid, dim3(kCommitThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_commit(const KvCommitParams& p_in, int head_dim, hipStream_t s) {
  KvCommitParams p = p_in;
  // The move kernel's work-groups read ctx_lens, num_accepted and path_nodes of their sequence while
  // work-group (b, 0, 0) writes new_ctx_lens[b].  When new_ctx_lens shares no byte with any of the three,
  // that write can happen in the move kernel (no second launch); otherwise a second launch writes the
  // lengths after every work-group has read its inputs.
  auto disjoint = [&](const void* x, size_t xb) {
    const char *a = reinterpret_cast<const char*>(p.new_ctx_lens), *c = reinterpret_cast<const char*>(x);
    return a + sizeof(int32_t) * (size_t)p.batch <= c || c + xb <= a;
  };
  p.lengths_in_commit = (disjoint(p.ctx_lens, sizeof(int32_t) * (size_t)p.batch) &&
                         disjoint(p.num_accepted, sizeof(int32_t) * (size_t)p.batch) &&
                         disjoint(p.path_nodes, sizeof(int32_t) * (size_t)p.batch * p.max_path)) ? 1 : 0;
  hipError_t e = head_dim == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
  if (e != hipSuccess || p.lengths_in_commit) return e;
  hipLaunchKernelGGL(kv_lengths_kernel, dim3((unsigned)ceil_div(p.batch, 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace spec
