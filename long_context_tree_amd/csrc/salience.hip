// Per-chunk attention mass ("salience") and top-k chunk selection, for gfx950.
//
// The DiffSpec pages select target KV chunks by an attention-derived signal computed from the
// paged target KV without materialising the attention matrix ("DiffSpec: Accelerating Long
// Sequence Generation with Differential Speculative Decoding", "What DiffSpec Does" item 2 and
// "Architecture"; chunk size 64 in "Configuration"; "salience-aware chunk encoding" in the
// CGCL-codes README, "Features").  Here the signal is the attention probability mass that the
// verification queries put on each context chunk, averaged over tree nodes and query heads.
//
// The attention kernel leaves, per (query row, chunk), the log2-sum-exp of the row's scaled
// scores over the chunk, and the merge leaves each row's final log2-sum-exp.  The mass of chunk c
// is then  mean over rows of exp2(chunk_lse2[c][row] - lse2[row]).
//   pass 1  one wave per (chunk, block of 1024 rows): lanes stride the rows (coalesced), fixed-order
//           wave reduction -> partial[b][row block][c]
//   pass 2  sum of the row-block partials in order, scaled, written or accumulated
//   pass 3  (top_k > 0) one work-group per sequence: bitonic sort of (mass desc, index asc) keys in LDS
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "spec_internal.h"

namespace spec {
namespace {

constexpr int kRowsPerSplit = 1024;

__device__ __forceinline__ void seq_bounds(const SalienceParams& p, int b, int* N, int* L) {
  int n = p.node_offsets[b + 1] - p.node_offsets[b];
  *N = n < 0 ? 0 : (n > p.max_nodes ? p.max_nodes : n);
  int l = p.ctx_lens[b];
  *L = l < 0 ? 0 : (l > p.max_ctx ? p.max_ctx : l);
}

__global__ __launch_bounds__(256) void salience_partial_kernel(SalienceParams p) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rs = blockIdx.y, b = blockIdx.z;
  int N, L;
  seq_bounds(p, b, &N, &L);
  const int nch = (L + p.chunk_size - 1) / p.chunk_size;
  if (c >= nch) return;
  const int rows = N * p.Hq;
  const int stride = p.max_nodes * p.Hq;
  const int r0 = rs * kRowsPerSplit;
  const int r1 = min(rows, r0 + kRowsPerSplit);
  const float* x = p.chunk_lse2 + ((int64_t)b * p.ws_max_chunks + c) * stride;
  const float* l2 = p.lse2 + (int64_t)b * stride;
  float acc = 0.f;
  for (int r = r0 + lane; r < r1; r += 64) acc += __builtin_amdgcn_exp2f(x[r] - l2[r]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) p.partial[((int64_t)b * p.row_splits + rs) * p.ws_max_chunks + c] = acc;
}

__global__ __launch_bounds__(256) void salience_finalize_kernel(SalienceParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= p.max_chunks) return;
  int N, L;
  seq_bounds(p, b, &N, &L);
  const int nch = (L + p.chunk_size - 1) / p.chunk_size;
  float* dst = p.chunk_mass + (int64_t)b * p.max_chunks + c;
  if (c >= nch || N == 0) {
    if (!p.accumulate) *dst = 0.f;
    return;
  }
  const int rows = N * p.Hq;
  const int nrs = (rows + kRowsPerSplit - 1) / kRowsPerSplit;
  float tot = 0.f;
  for (int rs = 0; rs < nrs; ++rs) tot += p.partial[((int64_t)b * p.row_splits + rs) * p.ws_max_chunks + c];
  tot *= 1.0f / (float)rows;
  *dst = p.accumulate ? *dst + tot : tot;
}

__global__ __launch_bounds__(1024) void topk_kernel(SalienceParams p) {
  __shared__ unsigned long long keys[kMaxTopK];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int N, L;
  seq_bounds(p, b, &N, &L);
  int nch = (L + p.chunk_size - 1) / p.chunk_size;
  if (nch > p.max_chunks) nch = p.max_chunks;
  int n = 1;
  while (n < nch) n <<= 1;
  const float* mass = p.chunk_mass + (int64_t)b * p.max_chunks;
  for (int i = tid; i < n; i += 1024) {
    if (i < nch) {
      const uint32_t bits = __float_as_uint(mass[i]) & 0x7FFFFFFFu;   // masses are >= 0; drop a -0 sign
      keys[i] = ((unsigned long long)(~bits) << 32) | (uint32_t)i;
    } else {
      keys[i] = ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], c = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < p.top_k; i += 1024) {
    int32_t idx = -1;
    float m = 0.f;
    if (i < nch) {
      idx = (int32_t)(keys[i] & 0xFFFFFFFFu);
      m = __uint_as_float(~(uint32_t)(keys[i] >> 32));
    }
    p.topk_index[(int64_t)b * p.top_k + i] = idx;
    p.topk_mass[(int64_t)b * p.top_k + i] = m;
  }
}

}  // namespace

size_t salience_partial_bytes(int batch, int max_nodes, int Hq, int ws_max_chunks) {
  const int64_t row_splits = ceil_div((int64_t)max_nodes * Hq, kRowsPerSplit);
  return sizeof(float) * (size_t)batch * row_splits * ws_max_chunks;
}

hipError_t launch_chunk_salience(const SalienceParams& pin, hipStream_t s) {
  SalienceParams p = pin;
  p.row_splits = (int)ceil_div((int64_t)p.max_nodes * p.Hq, kRowsPerSplit);
  hipLaunchKernelGGL(salience_partial_kernel, dim3((unsigned)ceil_div(p.ws_max_chunks, 4), p.row_splits, p.batch),
                     dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(salience_finalize_kernel, dim3((unsigned)ceil_div(p.max_chunks, 256), p.batch), dim3(256), 0, s,
                     p);
  e = hipGetLastError();
  if (e != hipSuccess || p.top_k <= 0) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(p.batch), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace spec
