// Compact draft KV for gfx950: each sequence's selected context chunks and its recent window,
// gathered from the canonical pre-RoPE draft cache (paged) into a contiguous cache whose slot j holds
// the j-th kept token, K rotated at local position j ("DiffSpec: Accelerating Long Sequence
// Generation with Differential Speculative Decoding", vllm-diffspec README, "What DiffSpec Does" and
// "Architecture": the dual-view draft cache).
//
// One work-group per (8 compact slots, sequence).  Each work-group rebuilds, from the selection
// itself, the part of the slot -> position map it needs, so a single launch does everything:
//   1. a bitmap of the selected chunks that start before the window (w0 = max(0, L - window)), in
//      LDS; repeated ids set the same bit;
//   2. a block-wide prefix count of the bitmap words.  A marked chunk's rank among the marked ones
//      is its place in the compact order.  Every marked chunk but the highest is whole, and only
//      chunk ceil(w0 / chunk_size) - 1 can be cut by the window, so the P tokens that precede the
//      window follow from the count alone;
//   3. slot j < P holds offset j - r * chunk_size of the chunk of rank r = j / chunk_size; slot
//      P <= j < P + (L - w0) holds window position w0 + j - P.
// The copy gives each slot 32 threads, each moving two 16-byte pieces of one K row and of one V
// row.  For K, cos and sin of the slot's angles sit in LDS, evaluated once per work-group in fp64.
// The angle j * inv_freq[i] is exact in fp64 (24-bit by 24-bit product).
#include "spec_internal.h"

namespace spec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kGatherThreads = 256;
constexpr int kGatherSlots = 8;            // compact slots per work-group (32 threads each)

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// ROPE: 0 none, 1 pairs (i, i + D/2), 2 pairs (2i, 2i + 1).  VT: V stored dim-major inside a page.
template <int D, int ROPE, int VT>
__global__ __launch_bounds__(kGatherThreads) void draft_gather_kernel(DraftGatherParams p) {
  constexpr int TPR = D / 16;                 // threads per (slot, head) row: 16 elements each
  constexpr int HPI = 32 / TPR;               // heads per pass of a slot's 32 threads
  extern __shared__ uint32_t bits[];          // [p.nwords] marked chunks
  __shared__ int s_wave[kGatherThreads / 64];
  __shared__ int s_rank_chunk[kGatherSlots];
  __shared__ int s_pos[kGatherSlots];
  __shared__ float2 s_cs[ROPE ? kGatherSlots : 1][D / 2];

  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * kGatherSlots;
  const int cs = p.chunk_size;
  int L = p.ctx_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int w0 = L > p.window ? L - p.window : 0;
  int32_t* pos_row = p.out_pos + (int64_t)b * p.capacity;

  // slots past every possible selection hold nothing (the first work-group still writes the length)
  const int64_t bound = (int64_t)p.num_select * cs + (L - w0);
  if (j0 >= bound && blockIdx.x != 0) {
    if (tid < kGatherSlots && j0 + tid < p.capacity) pos_row[j0 + tid] = -1;
    return;
  }

  // 1. bitmap of the selected chunks that start before w0
  const int nc0 = (int)(((int64_t)w0 + cs - 1) / cs);
  const int nw = (nc0 + 31) >> 5;             // <= p.nwords since w0 <= max_ctx
  for (int w = tid; w < nw; w += kGatherThreads) bits[w] = 0u;
  __syncthreads();
  const int32_t* sel = p.chunk_index + (int64_t)b * p.ci_stride;
  for (int i = tid; i < p.num_select; i += kGatherThreads) {
    const int c = sel[i];
    if (c >= 0 && c < nc0) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  // 2. prefix count over the words, each thread owning a run of consecutive words
  const int per = (nw + kGatherThreads - 1) / kGatherThreads;
  const int wb = min(tid * per, nw), we = min(wb + per, nw);
  int cnt = 0;
  for (int w = wb; w < we; ++w) cnt += __popc(bits[w]);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kGatherThreads / 64; ++w) {
    before += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
  const int excl = before + incl - cnt;
  const bool last_cut = nc0 > 0 && ((bits[(nc0 - 1) >> 5] >> ((nc0 - 1) & 31)) & 1u);
  const int P = total * cs - (last_cut ? (int)((int64_t)nc0 * cs - w0) : 0);
  const int len = P + (L - w0);

  // ranks this work-group's slots need: r_lo .. r_hi (at most kGatherSlots of them)
  const int jl = min(j0 + kGatherSlots, P) - 1;     // last slot below P, if any
  if (j0 < P) {
    const int r_lo = j0 / cs, r_hi = jl / cs;
    int run = excl;
    for (int w = wb; w < we && run <= r_hi; ++w) {
      uint32_t word = bits[w];
      const int pc = __popc(word);
      if (run + pc > r_lo) {
        while (word) {
          const int bit = __ffs(word) - 1;
          if (run >= r_lo && run <= r_hi) s_rank_chunk[run - r_lo] = (w << 5) + bit;
          ++run;
          word &= word - 1;
        }
      } else {
        run += pc;
      }
    }
  }
  // cos and sin of the slots' angles
  if (ROPE) {
    for (int e = tid; e < kGatherSlots * (D / 2); e += kGatherThreads) {
      const int s = e / (D / 2), i = e % (D / 2);
      double sn, cn;
      sincos((double)(j0 + s) * (double)p.inv_freq[i], &sn, &cn);
      s_cs[ROPE ? s : 0][i] = make_float2((float)cn, (float)sn);
    }
  }
  __syncthreads();
  if (tid < kGatherSlots) {
    const int j = j0 + tid;
    int t = -1;
    if (j < P) {
      const int r = j / cs;
      t = s_rank_chunk[r - j0 / cs] * cs + (j - r * cs);
    } else if (j < len) {
      t = w0 + (j - P);
    }
    s_pos[tid] = t;
    if (j < p.capacity) pos_row[j] = t;
  }
  if (blockIdx.x == 0 && tid == 0) p.out_len[b] = len;
  __syncthreads();

  // 3. copy: thread (slot s, head hh of the pass, piece u)
  const int s = tid >> 5, sub = tid & 31, hh = sub / TPR, u = sub % TPR;
  const int t = s_pos[s];
  if (t < 0) return;
  const int j = j0 + s;
  const int pg = p.block_table[(int64_t)b * p.bt_stride + (t >> p.page_shift)];
  const bool valid = pg >= 0 && pg < p.num_pages;
  const int row = t & ((1 << p.page_shift) - 1);
  // element offsets of the thread's two 8-element pieces
  const int e0 = ROPE == 2 ? 16 * u : 8 * u;
  const int e1 = ROPE == 2 ? 16 * u + 8 : D / 2 + 8 * u;
  float2 cs8[ROPE ? 8 : 1];
  if (ROPE) {
#pragma unroll
    for (int m = 0; m < 8; ++m) cs8[m] = s_cs[s][8 * u + m];
  }
  for (int h0 = 0; h0 < p.Hkv; h0 += HPI) {
    const int h = h0 + hh;
    if (h >= p.Hkv) break;
    u32x4 k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0}, v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (valid) {
      const int64_t blk = (int64_t)pg * p.page_stride + (int64_t)h * p.head_stride;
      const uint16_t* kr = p.k + blk + (int64_t)row * p.token_stride;
      k0 = *reinterpret_cast<const u32x4*>(kr + e0);
      k1 = *reinterpret_cast<const u32x4*>(kr + e1);
      if (!VT) {
        const uint16_t* vr = p.v + blk + (int64_t)row * p.token_stride;
        v0 = *reinterpret_cast<const u32x4*>(vr + e0);
        v1 = *reinterpret_cast<const u32x4*>(vr + e1);
      } else {
        const uint16_t* vb = p.v + blk + row;
        uint32_t w[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          w[m] = (uint32_t)vb[(int64_t)(e0 + 2 * m) << p.page_shift] |
                 ((uint32_t)vb[(int64_t)(e0 + 2 * m + 1) << p.page_shift] << 16);
          w[4 + m] = (uint32_t)vb[(int64_t)(e1 + 2 * m) << p.page_shift] |
                     ((uint32_t)vb[(int64_t)(e1 + 2 * m + 1) << p.page_shift] << 16);
        }
        v0 = {w[0], w[1], w[2], w[3]};
        v1 = {w[4], w[5], w[6], w[7]};
      }
    }
    if (ROPE == 1) {
      // element m of piece 0 pairs with element m of piece 1 (dims 8u + m and D/2 + 8u + m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = bf_lo(k0[q]), x1 = bf_hi(k0[q]);
        const float y0 = bf_lo(k1[q]), y1 = bf_hi(k1[q]);
        const float2 c0 = cs8[2 * q], c1 = cs8[2 * q + 1];
        k0[q] = pack_bf16(x0 * c0.x - y0 * c0.y, x1 * c1.x - y1 * c1.y);
        k1[q] = pack_bf16(y0 * c0.x + x0 * c0.y, y1 * c1.x + x1 * c1.y);
      }
    } else if (ROPE == 2) {
      // each 32-bit word is one pair (2i, 2i + 1): pairs 8u .. 8u+3 in piece 0, 8u+4 .. 8u+7 in piece 1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = bf_lo(k0[q]), y = bf_hi(k0[q]);
        float2 c = cs8[q];
        k0[q] = pack_bf16(x * c.x - y * c.y, y * c.x + x * c.y);
        x = bf_lo(k1[q]);
        y = bf_hi(k1[q]);
        c = cs8[4 + q];
        k1[q] = pack_bf16(x * c.x - y * c.y, y * c.x + x * c.y);
      }
    }
    const int64_t orow = (((int64_t)b * p.capacity + j) * p.Hkv + h) * D;
    *reinterpret_cast<u32x4*>(p.out_k + orow + e0) = k0;
    *reinterpret_cast<u32x4*>(p.out_k + orow + e1) = k1;
    *reinterpret_cast<u32x4*>(p.out_v + orow + e0) = v0;
    *reinterpret_cast<u32x4*>(p.out_v + orow + e1) = v1;
  }
}

template <int D, int ROPE>
hipError_t launch_r(const DraftGatherParams& p, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(p.capacity, kGatherSlots), (unsigned)p.batch);
  const size_t lds = (size_t)p.nwords * 4;
  if (p.v_dim_major)
    hipLaunchKernelGGL((draft_gather_kernel<D, ROPE, 1>), grid, dim3(kGatherThreads), lds, s, p);
  else
    hipLaunchKernelGGL((draft_gather_kernel<D, ROPE, 0>), grid, dim3(kGatherThreads), lds, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DraftGatherParams& p, int rope, hipStream_t s) {
  if (rope == 1) return launch_r<D, 1>(p, s);
  if (rope == 2) return launch_r<D, 2>(p, s);
  return launch_r<D, 0>(p, s);
}

}  // namespace

hipError_t launch_draft_gather(const DraftGatherParams& p, int head_dim, int rope, hipStream_t s) {
  return head_dim == 128 ? launch_d<128>(p, rope, s) : launch_d<64>(p, rope, s);
}

}  // namespace spec
