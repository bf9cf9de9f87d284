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
//   salience  one work-group per (sequence, chunk): a fixed-order sum over the rows of the chunk
//             (one contiguous run per KV head in the workspace), scaled, written or accumulated
//   top-k     (top_k > 0) one work-group per sequence: bitonic sort of (mass desc, index asc) keys in LDS
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "spec_internal.h"

namespace spec {
namespace {

constexpr int kChunksPerWG = 1;

__device__ __forceinline__ void seq_bounds(const SalienceParams& p, int b, int* N, int* L) {
  int n = p.node_offsets[b + 1] - p.node_offsets[b];
  *N = n < 0 ? 0 : (n > p.max_nodes ? p.max_nodes : n);
  int l = p.ctx_lens[b];
  *L = l < 0 ? 0 : (l > p.max_ctx ? p.max_ctx : l);
}

// One work-group per (sequence, kChunksPerWG chunks): for each chunk, every row's exp2(chunk_lse2 -
// lse2) is summed in a fixed order (each thread a fixed set of rows, then a butterfly in each wave, then
// the four waves in order), scaled by 1 / rows and written or accumulated.  The attention workspace keeps
// a chunk's rows, and the rows' final log2-sum-exps, as one run per KV head (row node * G + g is query
// head kvh * G + g); with G a multiple of 4 the reads are 16-byte loads.
__global__ __launch_bounds__(256) void salience_kernel(SalienceParams p) {
  __shared__ float red[4];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int N, L;
  seq_bounds(p, b, &N, &L);
  const int nch = (L + p.chunk_size - 1) / p.chunk_size;
  const int rows = N * p.Hq;
  const int G = p.Hq / p.Hkv;
  const int NG = N * G;                           // rows of one KV head
  const int RS = p.max_nodes * G;                 // lse2 rows per KV head
  const float* l2 = p.lse2 + (int64_t)b * p.Hkv * RS;
  const bool vec = (G & 3) == 0;                  // (NG and RS are then multiples of 4)
  for (int k = 0; k < kChunksPerWG; ++k) {
    const int c = blockIdx.x * kChunksPerWG + k;
    if (c >= p.max_chunks) return;
    float* dst = p.chunk_mass + (int64_t)b * p.max_chunks + c;
    if (c >= nch || N == 0) {
      if (tid == 0 && !p.accumulate) *dst = 0.f;
      continue;
    }
    const float* x = p.chunk_lse2 + (int64_t)b * p.ws_max_chunks * p.Hkv * RS + (int64_t)c * p.chunk_cs;   // head 0
    const float prev = (p.accumulate && tid == 0) ? *dst : 0.f;   // read now, used after the reduction
    float acc = 0.f;
    // element (h, j) of the runs: KV head h, row (4-row group) j; each thread takes the flattened
    // elements tid, tid + 256, ... in order, stepping (h, j) without a division
    const int per = vec ? NG >> 2 : NG;           // elements per KV head
    int h = 0, j = tid;
    while (per > 0 && j >= per && h < p.Hkv) {
      j -= per;
      ++h;
    }
    auto next = [&]() {
      j += 256;
      while (j >= per && h < p.Hkv) {
        j -= per;
        ++h;
      }
    };
    if (per > 0 && vec) {
      auto add4 = [&](const float4& a, const float4& m) {
        acc += (__builtin_amdgcn_exp2f(a.x - m.x) + __builtin_amdgcn_exp2f(a.y - m.y)) +
               (__builtin_amdgcn_exp2f(a.z - m.z) + __builtin_amdgcn_exp2f(a.w - m.w));
      };
      // up to four pairs of 16-byte loads in flight per round trip; the sum keeps the element order
      while (h < p.Hkv) {
        float4 a[4], m[4];
        int n = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (h < p.Hkv) {
            a[u] = *reinterpret_cast<const float4*>(x + (int64_t)h * p.chunk_hs + 4 * j);
            m[u] = *reinterpret_cast<const float4*>(l2 + h * RS + 4 * j);
            n = u + 1;
            next();
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (u < n) add4(a[u], m[u]);
      }
    } else if (per > 0) {
      for (; h < p.Hkv; next()) acc += __builtin_amdgcn_exp2f(x[(int64_t)h * p.chunk_hs + j] - l2[h * RS + j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    if (tid == 0) {
      const float tot = ((red[0] + red[1]) + (red[2] + red[3])) * (1.0f / (float)rows);
      *dst = p.accumulate ? prev + tot : tot;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Top-k for up to 2048 chunks: a bitonic sort of 2048 keys held in registers, two adjacent keys per
// thread (elements 2t and 2t+1 in thread t).  Stride 1 compares within a thread, strides 2..64 exchange
// with the partner thread t ^ (j/2) of the same wave by shuffles, and only strides >= 128 go through LDS.
__global__ __launch_bounds__(1024) void topk2048_kernel(SalienceParams p) {
  __shared__ unsigned long long keys[2048];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  int N, L;
  seq_bounds(p, b, &N, &L);
  int nch = (L + p.chunk_size - 1) / p.chunk_size;
  if (nch > p.max_chunks) nch = p.max_chunks;
  const float* mass = p.chunk_mass + (int64_t)b * p.max_chunks;
  unsigned long long e[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * t + h;
    e[h] = ~0ull;
    if (i < nch) {
      const uint32_t bits = __float_as_uint(mass[i]) & 0x7FFFFFFFu;   // masses are >= 0; drop a -0 sign
      e[h] = ((unsigned long long)(~bits) << 32) | (uint32_t)i;
    }
  }
  for (int k = 2; k <= 2048; k <<= 1) {
    const bool up = ((2 * t) & k) == 0;             // the same for both elements of the thread (k >= 2)
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j == 1) {
        const bool sw = (e[0] > e[1]) == up;
        const unsigned long long lo = sw ? e[1] : e[0], hi = sw ? e[0] : e[1];
        e[0] = lo;
        e[1] = hi;
        continue;
      }
      unsigned long long q[2];
      if (j < 128) {
        q[0] = shfl_xor_u64(e[0], j >> 1);
        q[1] = shfl_xor_u64(e[1], j >> 1);
      } else {
        __syncthreads();                              // earlier LDS reads are done
        keys[2 * t] = e[0];
        keys[2 * t + 1] = e[1];
        __syncthreads();
        q[0] = keys[(2 * t) ^ j];
        q[1] = keys[(2 * t + 1) ^ j];
      }
      const bool lower = (t & (j >> 1)) == 0;        // this thread holds the lower index of each pair
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned long long mn = e[h] < q[h] ? e[h] : q[h], mx = e[h] < q[h] ? q[h] : e[h];
        e[h] = (lower == up) ? mn : mx;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * t + h;
    if (i < p.top_k) {
      int32_t idx = -1;
      float m = 0.f;
      if (i < nch) {
        idx = (int32_t)(e[h] & 0xFFFFFFFFu);
        m = __uint_as_float(~(uint32_t)(e[h] >> 32));
      }
      p.topk_index[(int64_t)b * p.top_k + i] = idx;
      p.topk_mass[(int64_t)b * p.top_k + i] = m;
    }
  }
  for (int i = 2048 + t; i < p.top_k; i += 1024) {   // k above the chunk count: padding only
    p.topk_index[(int64_t)b * p.top_k + i] = -1;
    p.topk_mass[(int64_t)b * p.top_k + i] = 0.f;
  }
}

// Top-k for more chunks (up to 8192): the same sort through LDS.
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
  // Element i belongs to thread i mod 1024, so for strides j < 64 both elements of a pair belong to
  // one wave.  A stage reads what the previous stage wrote: after a stage of stride >= 64 (whose swaps
  // write elements owned by another wave) that needs a work-group barrier, so every stage of stride
  // >= 32 starts with one; a stage of stride < 32 follows one of stride < 64, whose writes all came
  // from its own wave, and the wave's LDS operations complete in order.
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 32) {
        __syncthreads();
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
      }
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
    }
  }
  __syncthreads();
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

hipError_t launch_chunk_salience(const SalienceParams& p, hipStream_t s) {
  hipLaunchKernelGGL(salience_kernel, dim3((unsigned)ceil_div(p.max_chunks, kChunksPerWG), p.batch), dim3(256), 0, s,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.top_k <= 0) return e;
  if (p.max_chunks <= 2048) hipLaunchKernelGGL(topk2048_kernel, dim3(p.batch), dim3(1024), 0, s, p);
  else hipLaunchKernelGGL(topk_kernel, dim3(p.batch), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace spec
