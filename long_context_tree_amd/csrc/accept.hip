// Greedy and rejection-sampling acceptance over a draft tree, for gfx950.
//
// Greedy: a draft is accepted iff it equals the target's greedy choice at its parent (vllm.cpp
// "Speculative decoding", section MTP); on a tree the result is the deepest accepted node.
// Rejection: accept x ~ q with probability min(1, p(x)/q(x)); on rejection continue with the
// normalised residual max(0, res - q) ("Adaptive Speculative Decoding", sections "Correctness
// first" and "The controller"), generalised to siblings drawn i.i.d. from q.
//
// Both are HBM streams over the [nodes][vocab] logits (16-33 MB at vocab 128K), so the work is
// spread over (vocab segment x node) work-groups with fixed-order reductions:
//   argmax_seg        (greedy) per (node, 8192-token segment): the packed key (ordered value, ~index)
//                     maximum, i.e. the largest logit with the lowest index among exact ties
//   greedy_walk       (greedy) per sequence: every edge test in parallel, the deepest accepted node,
//                     the path and the argmax bonus token
//   rejection_kernel  (rejection) per (node, 8192-token segment), all levels of the node in one
//                     launch (see below), the walk by the sequence's last node to finish
#include <type_traits>

#include "spec_internal.h"

namespace spec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t ordered(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0) u = 0;                       // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long pack_key(float v, int idx) {
  return ((unsigned long long)ordered(v) << 32) | (uint32_t)(~(uint32_t)idx);
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)(~(uint32_t)(k & 0xFFFFFFFFu)); }

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Lane l's value from lane l ^ M within each half-wave (M < 32), by ds_swizzle in its bitmask mode:
// the lane pattern is an immediate, so no lane-address register stays live through a kernel.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  static_assert(M > 0 && M < 32, "bitmask-mode swizzles stay within 32 lanes");
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
}
template <int M>
__device__ __forceinline__ unsigned long long xor_lane_u64(unsigned long long v) {
  return ((unsigned long long)xor_lane<M>((uint32_t)(v >> 32)) << 32) | xor_lane<M>((uint32_t)v);
}
template <int M>
__device__ __forceinline__ double xor_lane_f64(double v) {
  return __builtin_bit_cast(double, xor_lane_u64<M>(__builtin_bit_cast(unsigned long long, v)));
}
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ double lane_f64(double v, int l) {
  return __builtin_bit_cast(double, lane_u64(__builtin_bit_cast(unsigned long long, v), l));
}

// Wave maximum of a u64 key: butterflies within each half-wave, then the two halves (lanes 0 and 32).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = umax64(v, xor_lane_u64<16>(v));
  v = umax64(v, xor_lane_u64<8>(v));
  v = umax64(v, xor_lane_u64<4>(v));
  v = umax64(v, xor_lane_u64<2>(v));
  v = umax64(v, xor_lane_u64<1>(v));
  return umax64(lane_u64(v, 0), lane_u64(v, 32));
}

// Wave fp64 sum in a fixed order: butterflies within each half-wave (the two lanes of a pair add the
// same two values, so every lane of a half holds the same bits), then half 0 + half 1.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += xor_lane_f64<16>(v);
  v += xor_lane_f64<8>(v);
  v += xor_lane_f64<4>(v);
  v += xor_lane_f64<2>(v);
  v += xor_lane_f64<1>(v);
  return lane_f64(v, 0) + lane_f64(v, 32);
}

__device__ __forceinline__ float load_logit(const AcceptParams& p, int64_t u, int v) {
  if (p.bf16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(p.logits)[u * p.vocab + v];
    return __uint_as_float((uint32_t)h << 16);
  }
  return reinterpret_cast<const float*>(p.logits)[u * p.vocab + v];
}

__device__ __forceinline__ int total_nodes(const AcceptParams& p) {
  int t = p.node_offsets[p.batch];
  const int cap = p.batch * p.max_nodes;
  return t < 0 ? 0 : (t > cap ? cap : t);
}

// Block-wide (256 threads) maximum of a u64 key; result valid in every thread.
__device__ unsigned long long block_max_u64(unsigned long long v) {
  __shared__ unsigned long long red[4];
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = lane_u64(umax64(umax64(red[0], red[1]), umax64(red[2], red[3])), 0);   // (uniform: scalar registers)
  __syncthreads();
  return v;
}

// Block-wide (256 threads) fp64 sum in a fixed order; result valid in every thread.
__device__ double block_sum_f64(double v) {
  __shared__ double red[4];
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = lane_f64((red[0] + red[1]) + (red[2] + red[3]), 0);   // (uniform: scalar registers)
  __syncthreads();
  return v;
}

// Block-wide (256 threads) exclusive prefix sum in fp64, in a fixed order (inclusive wave scan by
// shuffles, then the wave totals in order); every thread gets the sum of the values of lower threads,
// and *total the sum of all.
__device__ double block_scan_excl_f64(double v, double* total) {
  __shared__ double wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  double before = 0.0, all = 0.0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// ---- per (segment, node): maximum logit with the lowest index among exact ties ----
__global__ __launch_bounds__(256) void argmax_seg_kernel(AcceptParams p) {
  const int seg = blockIdx.x;
  const int64_t u = blockIdx.y;
  if (u >= total_nodes(p)) return;
  const int v0 = seg * kSegment;
  const int v1 = min(p.vocab, v0 + kSegment);
  unsigned long long best = 0;
  const int esz = p.bf16 ? 2 : 4;
  const int per = 16 / esz;                       // elements per 16-byte load
  const char* row = reinterpret_cast<const char*>(p.logits) + u * (int64_t)p.vocab * esz;
  const bool vec = ((((uintptr_t)row) & 15) == 0) && (v0 % per == 0);
  int v = v0;
  if (vec) {
    const int nvec = (v1 - v0) / per;
    // four loads in flight per round trip; an index past the end repeats the last load, whose keys
    // (value, index) are then seen twice, which leaves the maximum unchanged
    for (int i0 = threadIdx.x; i0 < nvec; i0 += 4 * 256) {
      u32x4 w[4];
      int base[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = min(i0 + 256 * j, nvec - 1);
        base[j] = v0 + i * per;
        w[j] = *reinterpret_cast<const u32x4*>(row + (int64_t)base[j] * esz);
      }
      // the largest value of this round first (one max per entry), then the lowest index holding it
      // (entries visited from the highest index down, so the last match is the lowest), and one packed key:
      // the same key as the per-entry maximum, since -0 == +0 here as in ordered()
      auto round_key = [&](auto ne_c, auto val) -> unsigned long long {
        constexpr int NE = decltype(ne_c)::value;   // entries per 16-byte load
        float mv = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < NE; ++e) mv = fmaxf(mv, val(j, e));
        int idx = 0x7FFFFFFF;
#pragma unroll
        for (int j = 3; j >= 0; --j)
#pragma unroll
          for (int e = NE - 1; e >= 0; --e)
            if (val(j, e) == mv) idx = base[j] + e;
        return pack_key(mv, idx);
      };
      if (p.bf16)
        best = umax64(best, round_key(std::integral_constant<int, 8>{}, [&](int j, int e) {
          return __uint_as_float((e & 1) ? (w[j][e >> 1] & 0xFFFF0000u) : (w[j][e >> 1] << 16));
        }));
      else
        best = umax64(best, round_key(std::integral_constant<int, 4>{},
                                      [&](int j, int e) { return __uint_as_float(w[j][e]); }));
    }
    v = v0 + nvec * per;
  }
  for (int i = v + threadIdx.x; i < v1; i += 256) best = umax64(best, pack_key(load_logit(p, u, i), i));
  best = block_max_u64(best);
  if (threadIdx.x == 0) p.seg_key[u * p.nseg + seg] = best;
}

// Child count and sibling rank (earlier siblings) of the nodes tid + 256 q, q < PER; flags a parent
// array that is not topological or a node with more than max_children children.  Without COUNT (greedy)
// only the parent-order checks run.
template <int PER, bool COUNT, typename PT>
__device__ __forceinline__ void child_ranks(const PT* par_s, int N, int tid, int max_children, int* rank_s,
                                            int* nch_s, int& bad_s) {
  int own_p[PER], rank[PER], nch[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    own_p[q] = i < N ? par_s[i] : -2;
    rank[q] = 0;
    nch[q] = 0;
    if (i < N && i > 0 && !(own_p[q] >= 0 && own_p[q] < i)) bad_s = 1;
    if (i == 0 && own_p[q] != -1) bad_s = 1;
  }
  // the counts (rejection only; greedy needs just the parent-order checks above)
  for (int j = 1; COUNT && j < N; ++j) {
    const int pj = par_s[j];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = tid + 256 * q;
      rank[q] += (j < i && pj == own_p[q]) ? 1 : 0;
      nch[q] += (pj == i) ? 1 : 0;
    }
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    if (i < N) {
      rank_s[i] = rank[q];
      nch_s[i] = nch[q];
      if (nch[q] > max_children) bad_s = 1;
    }
  }
}

// Outputs of a sequence whose tree, or whose call, could not be evaluated: num_accepted = -1.
__device__ __forceinline__ void write_invalid(const AcceptParams& p, int b, int tid) {
  for (int i = tid; i < p.max_path; i += 256) {
    p.out_path_nodes[(int64_t)b * p.max_path + i] = -1;
    p.out_tokens[(int64_t)b * p.max_path + i] = -1;
  }
  if (tid == 0) p.out_num_accepted[b] = -1;
}

// ---- greedy, per sequence: the walk and the bonus token ----
__global__ __launch_bounds__(256) void greedy_walk_kernel(AcceptParams p) {
  __shared__ int par_s[kMaxTreeNodes], tok_s[kMaxTreeNodes], nch_s[kMaxTreeNodes];
  __shared__ int rank_s[kMaxTreeNodes], amax_s[kMaxTreeNodes], path_s[kMaxTreeNodes];
  __shared__ int stop_s, depth_s, bad_s;
#ifdef SPEC_DEBUG
  __shared__ int dbg_rows_s, dbg_tests_s;   // witnesses: rows reduced in this call and read here, tests run
#endif
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  int32_t* o_path = p.out_path_nodes + (int64_t)b * p.max_path;
  int32_t* o_tok = p.out_tokens + (int64_t)b * p.max_path;
  if (N == 0) {
    write_invalid(p, b, tid);
    return;
  }
  if (tid == 0) bad_s = 0;
#ifdef SPEC_DEBUG
  if (tid == 0) dbg_rows_s = dbg_tests_s = 0;
  __syncthreads();
#endif
  for (int i = tid; i < N; i += 256) {
    par_s[i] = p.parents[n0 + i];
    tok_s[i] = p.draft_tokens[n0 + i];
    // four independent accumulators, unrolled so that 16 segment loads (the whole row at V = 128K) are
    // in flight together
    const unsigned long long* sk = p.seg_key + (int64_t)(n0 + i) * p.nseg;
    unsigned long long k0 = 0, k1 = 0, k2 = 0, k3 = 0;
    int s = 0;
#pragma unroll 4
    for (; s + 4 <= p.nseg; s += 4) {
      k0 = umax64(k0, sk[s]);
      k1 = umax64(k1, sk[s + 1]);
      k2 = umax64(k2, sk[s + 2]);
      k3 = umax64(k3, sk[s + 3]);
    }
    for (; s < p.nseg; ++s) k0 = umax64(k0, sk[s]);
    amax_s[i] = key_index(umax64(umax64(k0, k1), umax64(k2, k3)));
#ifdef SPEC_DEBUG
    // the debug checks cleared every key: a row counts when all its segment keys were written again
    bool fresh = true;
    for (int q = 0; q < p.nseg; ++q) fresh = fresh && sk[q] != 0ull;
    if (fresh) atomicAdd(&dbg_rows_s, 1);
#endif
  }
  __syncthreads();
  // the parent-order checks: each parent entry is read once and compared with the nodes this thread
  // owns (tid, tid + 256, ...): one node per thread for trees of <= 256 nodes, else up to 8
  if (N <= 256)
    child_ranks<1, false>(par_s, N, tid, 0x7FFFFFFF, rank_s, nch_s, bad_s);
  else
    child_ranks<kMaxTreeNodes / 256, false>(par_s, N, tid, 0x7FFFFFFF, rank_s, nch_s, bad_s);
  __syncthreads();
  if (bad_s) {
    write_invalid(p, b, tid);
    return;
  }
  // the edge tests, in parallel: a draft passes iff it is its parent's greedy token
  for (int c = 1 + tid; c < N; c += 256) {
    const int x = tok_s[c];
#ifdef SPEC_DEBUG
    atomicAdd(&dbg_tests_s, 1);
#endif
    rank_s[c] = (x >= 0 && x < p.vocab && x == amax_s[par_s[c]]) ? 1 : 0;
  }
  __syncthreads();
#ifdef SPEC_DEBUG
  if (tid == 0 && p.dbg) {
    atomicAdd(&p.dbg[1], (uint32_t)dbg_rows_s);
    atomicAdd(&p.dbg[2], (uint32_t)dbg_tests_s);
  }
#endif
  // node j is accepted iff every edge on its root path passed; keep the deepest accepted node, the lowest
  // index among equally deep ones
  unsigned long long best = 0;
  for (int j = tid; j < N; j += 256) {
    bool acc = true;
    int d = 0, x = j;
    while (x > 0 && d < N) {
      acc = acc && rank_s[x] != 0;
      x = par_s[x];
      ++d;
    }
    if (acc) best = umax64(best, ((unsigned long long)d << 32) | (uint32_t)(0xFFFFu - j));
  }
  best = block_max_u64(best);
  if (tid == 0) {
    const int f = 0xFFFF - (int)(best & 0xFFFFu);
    const int d = (int)(best >> 32);
    int x = f;
    for (int k = d; k >= 0; --k) {
      path_s[k] = x;
      x = k > 0 ? par_s[x] : x;
    }
    stop_s = f;
    depth_s = d;
  }
  __syncthreads();
  const int u = stop_s, depth = depth_s;
  if (depth + 1 > p.max_path) {
    write_invalid(p, b, tid);
    return;
  }
  const int bonus = amax_s[u];
  for (int i = tid; i < p.max_path; i += 256) {
    o_path[i] = i <= depth ? path_s[i] : -1;
    o_tok[i] = i < depth ? tok_s[path_s[i + 1]] : (i == depth ? bonus : -1);
  }
  if (tid == 0) p.out_num_accepted[b] = depth;
}

// ---------------------------------------------------------------------------------------------------
// Rejection acceptance in one pass over the rows ("Adaptive Speculative Decoding", "Correctness first").
//
// One work-group per (node, 8192-token segment) loads its segment of the node's logits once: 32
// consecutive entries per thread, held in registers as fp64 residual values from then on, beside the
// thread's 32 draft probabilities (fp32, read once, since every level subtracts the same row).  The
// grid of a 64-node tree at vocabulary 128K is 1024 work-groups, which must all be resident at once
// (four per compute unit, so at most 128 registers per lane).  The node's work-groups meet once per
// level, each publishing its segment's value into a slot of its own and polling the others':
//   sync 0: each segment's maximum m_s and sum exp(l - m_s) (fp64) -> the row maximum M = max m_s and
//           Z_0 = sum_s (sum exp(l - m_s)) exp(m_s - M); res_0 = exp(l - M) / Z_0, evaluated per thread
//           as exp(l - m_t) exp(m_t - M) / Z_0 with the thread's own maximum m_t (so that a thread's
//           exps wait for its own loads only)
//   sync r, r = 1 .. children: the segment sums of max(0, res_{r-1} - q) -> Z_r;
//           res_r = max(0, res_{r-1} - q) / Z_r, or res_{r-1} again if Z_r = 0
// Every exp is fp64 (exp_neg: table-driven, within ~2 ulp).
// The child of rank r (r earlier siblings) is tested against res_r at its token, by the thread that
// holds that token, as soon as res_r exists; after the last level the node's bonus token (the inverse
// CDF of its last residual at u_sample) is drawn by the work-group whose segment holds it.  Every node's
// draw is made, whether or not the walk ends there: the decisions of one node depend on that node's
// row alone.  The sequence counts its finished nodes; the last one walks the tree from the root (first
// accepted child of each node) and writes the outputs.
//
// Wave 0 of each work-group polls the node's slots and sums them in one fixed order, so all of a node's
// work-groups hold the same bits.  A node's work-groups are consecutive in the grid, and work-groups start in grid
// order, so the ones that wait only wait for ones that have started or will start when a finished
// work-group leaves: the waits end.  Each wait is also bounded; a wait that runs out (which the ordering
// above rules out) marks the call's error word, and the walk then writes num_accepted = -1.
// ---------------------------------------------------------------------------------------------------
constexpr int kRejPer = kRejSegment / 256;        // consecutive vocabulary entries per thread
static_assert(kRejPer % 8 == 0, "a run is whole 16-byte loads of bf16 logits and of fp32 probabilities");
constexpr int kSpinLimit = 1 << 18;               // polls of a counter before a wait gives up
constexpr int kPreTests = 16;                     // children whose test inputs are read before level 0

// exp(d) for d <= 0 in fp64, table-driven (P. T. P. Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989):
//   n = rint(d 256 / ln 2),  r = d - n (ln 2 / 256)  (|r| <= ln 2 / 512, the constant split in two
//   parts so that r carries no cancellation error),  exp(d) = 2^(n >> 8) * 2^((n & 255) / 256) * e^r,
// the middle factor from a 256-entry table (2^(j/256), built by every work-group at its start) and
// e^r from its degree-4 Taylor polynomial, whose truncation error at |r| <= ln 2 / 512 is below
// 4e-17 relative.  The result is within ~2 ulp of the exact value.  d below -746 gives +0 (as does
// exp: the true value is below half the smallest subnormal); NaN gives NaN.
constexpr int kExpTab = 256;
constexpr double kExpInvStep = 0x1.71547652b82fep+8;     // 256 / ln 2
constexpr double kExpStepHi = 0x1.62e42fefa39efp-9;      // ln 2 / 256, leading part
constexpr double kExpStepLo = 0x1.abc9e3b39803fp-64;     // ln 2 / 256 - kExpStepHi

__device__ __forceinline__ double exp_neg(double d, const double* tab) {
  d = d < -746.0 ? -746.0 : d;
  const double n = __builtin_rint(d * kExpInvStep);
  double r = __builtin_fma(-n, kExpStepHi, d);
  r = __builtin_fma(-n, kExpStepLo, r);
  double e = __builtin_fma(r, 1.0 / 24.0, 1.0 / 6.0);
  e = __builtin_fma(e, r, 0.5);
  e = __builtin_fma(e, r, 1.0);
  e = __builtin_fma(e, r, 1.0);
  const int ni = (int)n;
  return ldexp(tab[ni & (kExpTab - 1)] * e, ni >> 8);
}

// this thread's run [a0, a1) of row u of the draft probabilities (entries past a1 are 0).  They are read
// again at every residual level, from L2, rather than held in registers through the exps.
__device__ __forceinline__ void load_q_run(const AcceptParams& p, int64_t u, int a0, int a1, float (&qv)[kRejPer]) {
  const float* row = p.draft_probs + u * p.vocab + a0;
  if (a1 - a0 == kRejPer && ((uintptr_t)row & 15) == 0) {
    u32x4 w[kRejPer / 4];
#pragma unroll
    for (int j = 0; j < kRejPer / 4; ++j) w[j] = *reinterpret_cast<const u32x4*>(row + 4 * j);
#pragma unroll
    for (int j = 0; j < kRejPer / 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) qv[4 * j + k] = __uint_as_float(w[j][k]);
  } else {
#pragma unroll
    for (int i = 0; i < kRejPer; ++i) qv[i] = a0 + i < a1 ? row[i] : 0.f;
  }
}

// Values passed between work-groups are written and read with device-scope (sc1) stores and loads,
// which are coherent across the XCDs' L2 caches.  A writer waits for its stores to complete (vmcnt)
// before it counts its arrival, and a reader issues its loads only after it has seen the count, so the
// loads find the stores.  (Release and acquire fences at device scope would write back and invalidate
// the whole L2 on every arrival: measured ten times slower.)
__device__ __forceinline__ void store_dev_u64(unsigned long long* a, unsigned long long v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_f64(double* a, double v) {
  store_dev_u64(reinterpret_cast<unsigned long long*>(a), __builtin_bit_cast(unsigned long long, v));
}
__device__ __forceinline__ void store_dev_i32(int32_t* a, int32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_dev_u64(const unsigned long long* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_dev_f64(const double* a) {
  return __builtin_bit_cast(double, load_dev_u64(reinterpret_cast<const unsigned long long*>(a)));
}
__device__ __forceinline__ int load_dev_i32(const int32_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A work-group's value for one sync of its node: every thread's stores of the call so far complete
// (vmcnt), then thread 0 stores the value into the work-group's own slot.
__device__ __forceinline__ void publish_f64(double* slot, double v) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) store_dev_f64(slot, v);
}

// A uniform fp64 value in scalar registers (its bits from lane 0).
__device__ __forceinline__ double uniform_f64(double v) { return lane_f64(v, 0); }

// A sync of a node is its S work-groups' values: a slot holds kUnset until its work-group writes it (a
// real value is a sum of non-negative terms, or NaN from NaN inputs, never kUnset).  The waiters poll
// the S slots in parallel, so that the values arrive with the poll that sees them all.
constexpr double kUnset = -1.0;

// True when the call's error word is marked; read by one lane every 256 polls of a wait (the word is
// one address for the whole grid, so that reading it on every poll would queue at its memory channel).
__device__ __forceinline__ bool wait_abandoned(int it, const uint32_t* err) {
  if (it + 1 == kSpinLimit) return true;
  if ((it & 255) != 255) return false;
  const uint32_t e = (threadIdx.x & 63) == 0 ? __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  return __builtin_amdgcn_readfirstlane(e) != 0u;
}

// The total of one sync's S slots v[0 .. S).  Wave 0 polls them: with S <= 64, lane l watches slot l and
// stops reading it once it holds a value, so that a round reads only the slots still missing; else each
// round reads them all.  The total is summed in a fixed order (lane l: slots l, l + 64, ... in order,
// then the wave sum), so every work-group of the node gets the same bits, and reaches the other waves
// through LDS.  *mine: slot l's value in lane l of wave 0 (with S <= 64).  A wait that runs out marks
// *err (and once *err is marked no wait waits: the call's results are void anyway).
__device__ double wait_total(const double* v, int S, uint32_t* err, double* mine) {
  __shared__ double tot_s;
  const int tid = threadIdx.x;
  if (tid < 64) {
    double part = 0.0;
    if (S <= 64) {
      double x = 0.0;
      bool have = tid >= S;
      for (int it = 0;; ++it) {
        if (!have) {
          x = load_dev_f64(v + tid);
          have = x != kUnset;
        }
        if (__ballot(!have) == 0ull) break;
        if (wait_abandoned(it, err)) {
          if (tid == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      part = tid < S ? x : 0.0;
      *mine = part;
    } else {
      for (int it = 0;; ++it) {
        bool ok = true;
        part = 0.0;
        for (int s = tid; s < S; s += 64) {
          const double x = load_dev_f64(v + s);
          ok = ok && x != kUnset;
          part += x;
        }
        if (__ballot(!ok) == 0ull) break;
        if (wait_abandoned(it, err)) {
          if (tid == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    const double t = wave_sum_f64(part);
    if (tid == 0) tot_s = t;
  }
  __syncthreads();
  return uniform_f64(tot_s);                      // (read by every wave before the barriers of the next
                                                  // level's sum, after which tot_s is written again)
}

// Clears what the first sync of a rejection call reads (every row's segment keys and level-0 slots),
// the sequence counters and the error word.  The slots of later levels are cleared by their own
// work-groups before those publish level 0.
__global__ __launch_bounds__(256) void rej_clear_kernel(AcceptParams p) {
  const int64_t nk = (int64_t)p.batch * p.max_nodes * p.nsegr;
  const int64_t lvS = (int64_t)(p.max_children + 1) * p.nsegr;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < nk; i += gridDim.x * 256) {
    p.seg_key[i] = 0ull;
    p.seg_sum[(i / p.nsegr) * lvS + i % p.nsegr] = kUnset;
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < p.batch + 1; i += gridDim.x * 256) p.sync_cnt[i] = 0u;
}

// BF16: bf16 logits, kept packed (two to a register) until their exps are taken
template <bool BF16>
__global__ __launch_bounds__(256, 4) void rejection_kernel(AcceptParams p) {
  __shared__ int kids_s[kMaxTreeNodes];           // this node's children, in index order
  __shared__ int16_t par16_s[kMaxTreeNodes];      // the sequence's parents, for the walk
  __shared__ int wcnt_s[4];
  __shared__ int claim_s, last_s;
  __shared__ double base_s, thr_s;
  __shared__ double etab[kExpTab];                // 2^(j/256)
  __shared__ int ptok_s[kPreTests];               // the first children's tokens ...
  __shared__ float pua_s[kPreTests];              // ... their u_accept ...
  __shared__ double pthr_s[kPreTests];            // ... and u_accept * q_u(token)
  __shared__ float mt_s[256];                     // each thread's own maximum m_t, kept through sync 1
  // with S <= 64: segment l's key and its slot at level lvl, as wave 0 polled them
  __shared__ unsigned long long k0_s[64];
  __shared__ double sl_s[64];
  const int seg = blockIdx.x;
  const int S = p.nsegr;
  const int i = blockIdx.y;                       // the node within its sequence
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tn = total_nodes(p);
  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  const int64_t u = (int64_t)n0 + i;
  if (N == 0 || n0 + N > tn) {                    // (uniform) a sequence without a tree: -1
    if (seg == 0 && i == 0) write_invalid(p, b, tid);
    return;
  }
  if (i >= N) return;                             // (uniform) no such node: no counter counts this group
  uint32_t* seq_cnt = p.sync_cnt + b;
  uint32_t* err = p.sync_cnt + p.batch;
  const int lv = p.max_children + 1;
  const float us = p.u_sample[u];                 // the bonus draw's uniform (read now, used last)

  // ---- this node's children in index order (a child's rank is its position); the parents are kept
  // for the walk (a value outside -1 .. N-1 as -2, which the walk's checks reject) ----
  int nk = 0;
  for (int j0 = 0; j0 < N; j0 += 256) {
    const int j = j0 + tid;
    const int pj = j < N ? p.parents[n0 + j] : -2;
    if (j < N) par16_s[j] = (int16_t)(pj >= -1 && pj < N ? pj : -2);
    const bool kid = j > i && j < N && pj == i;
    const unsigned long long m = __ballot(kid);
    if (lane == 0) wcnt_s[wave] = __popcll(m);
    __syncthreads();
    int off = nk;
    for (int w = 0; w < wave; ++w) off += wcnt_s[w];
    if (kid) kids_s[off + __popcll(m & ((1ull << lane) - 1ull))] = j;
    nk += wcnt_s[0] + wcnt_s[1] + wcnt_s[2] + wcnt_s[3];
    __syncthreads();
  }
  const int nl = nk < p.max_children ? nk : p.max_children;   // residual levels past level 0 (more
                                                                // children than max_children: the walk
                                                                // reports the tree)
  // ---- the run's logits ----
  const int v0 = seg * kRejSegment, v1 = min(p.vocab, v0 + kRejSegment);
  const int a0 = min(v1, v0 + tid * kRejPer), a1 = min(v1, a0 + kRejPer);
  const int nv = a1 - a0;                         // entries of the run inside the vocabulary
  // the run's logits: BF16 packed two to a register, else fp32; entries past the end of the vocabulary
  // read as -inf, so that they change no maximum and take exp(-inf) = +0 at every level
  constexpr int LW = BF16 ? kRejPer / 2 : kRejPer;
  uint32_t lw[LW];
  {
    const bool whole = nv == kRejPer;
    const char* row = static_cast<const char*>(p.logits) + (u * p.vocab + a0) * (BF16 ? 2 : 4);
    if (whole && ((uintptr_t)row & 15) == 0) {
#pragma unroll
      for (int j = 0; j < LW / 4; ++j) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(row + 16 * j);
#pragma unroll
        for (int k = 0; k < 4; ++k) lw[4 * j + k] = w[k];
      }
    } else if (BF16) {
      const uint16_t* r16 = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
      for (int j = 0; j < LW; ++j) {
        const uint32_t lo = 2 * j < nv ? r16[2 * j] : 0xFF80u, hi = 2 * j + 1 < nv ? r16[2 * j + 1] : 0xFF80u;
        lw[j] = lo | (hi << 16);
      }
    } else {
      const uint32_t* r32 = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
      for (int j = 0; j < LW; ++j) lw[j] = j < nv ? r32[j] : 0xFF800000u;
    }
  }
  auto logit = [&](int k) -> float {
    if (BF16) return __uint_as_float((k & 1) ? (lw[k >> 1] & 0xFFFF0000u) : (lw[k >> 1] << 16));
    return __uint_as_float(lw[k]);
  };
  // the exp table, 2^(j/256), in LDS before any wave's first exp (this barrier waits for LDS only, not
  // for the loads in flight)
  etab[tid] = exp2((double)tid * (1.0 / kExpTab));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // the test inputs of the first kPreTests children, read during level 0 so that no level waits for
  // them: the token and u_accept now, q_u(token) once the token is in (after the level-0 publish); the
  // threshold u_accept * q_u(token) (fp64; 0 for a token outside the vocabulary) goes to LDS after sync 1
  const int npre = nk < kPreTests ? nk : kPreTests;
  int pre_x = -1;
  float pre_ua = 0.f, pre_q = 0.f;
  if (tid < npre) {
    const int c = kids_s[tid];
    pre_x = p.draft_tokens[n0 + c];
    pre_ua = p.u_accept[n0 + c];
  }

  double* ssum = p.seg_sum + u * lv * S;          // [level][segment]
  // this work-group's slots of levels 1 .. nl, cleared before it publishes level 0 (a work-group polls a
  // level's slots only after it has seen every level-0 value)
  for (int r = 1 + tid; r <= nl; r += 256) store_dev_f64(ssum + r * S + seg, kUnset);

  // ---- sync 1: the segment's maximum m_s (largest logit, lowest index among exact ties) and its
  // level-0 sum against it, sum exp(l - m_s) (fp64); then the row maximum M = max m_s and
  // Z_0 = sum_s (sum exp(l - m_s)) exp(m_s - M).  Each thread first takes its exps against its own
  // maximum m_t, so that they wait for its own loads only (no barrier before them); its sum is then
  // rescaled by exp(m_t - m_s), and its entries by exp(m_t - M) / Z_0 after the sync ----
  double res[kRejPer];
  unsigned long long mine_key;
  {
    float mv = -INFINITY;                         // m_t
#pragma unroll
    for (int k = 0; k < kRejPer; ++k) mv = fmaxf(mv, logit(k));
    uint32_t at_max = 0;                          // bit k: entry k holds the maximum
#pragma unroll
    for (int k = 0; k < kRejPer; ++k) at_max |= logit(k) == mv ? 1u << k : 0u;
    at_max &= nv >= kRejPer ? ~0u : (1u << nv) - 1u;
    const int kb = at_max ? __builtin_ctz(at_max) : 0;   // the lowest such entry
    double at = 0.0;
    if (mv > -INFINITY) {                         // else the run has no mass
      // the logits are unpacked again from lw here, and the exps are scheduled four at a time: the
      // unpacked copies from the maximum, or more exps in flight, would not fit beside res at the
      // occupancy the grid needs
#pragma unroll
      for (int j = 0; j < LW; ++j) asm volatile("" : "+v"(lw[j]));
      const double mt = mv;
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) {
        res[k] = exp_neg((double)logit(k) - mt, etab);
        at += res[k];
        if (k % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) res[k] = 0.0;
    }
    if (tid < npre) {                             // (out of registers through the sync)
      ptok_s[tid] = pre_x;
      pua_s[tid] = pre_ua;
    }
    mine_key = block_max_u64(nv > 0 ? pack_key(mv, a0 + kb) : 0ull);
    const double ms = (double)key_value(mine_key);
    const double acc = block_sum_f64(mv > -INFINITY ? at * exp_neg((double)mv - ms, etab) : 0.0);
    mt_s[tid] = mv;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      store_dev_f64(ssum + seg, acc);
      store_dev_u64(p.seg_key + u * S + seg, mine_key);
    }
  }
  if (tid < npre) {
    const int x = ptok_s[tid];
    if (x >= 0 && x < p.vocab) pre_q = p.draft_probs[u * p.vocab + x];
  }
  double M, z;
  float qv[kRejPer];
  {
    // wave 0 polls the S (key, sum) pairs as wait_total polls a level's slots, then takes the row
    // maximum M and Z_0 (lane l: segments l, l + 64, ... in order, then the wave sum), for every wave
    __shared__ double m_sh, z_sh;
    if (nl > 0) load_q_run(p, u, a0, a1, qv);
    if (tid < 64) {
      const unsigned long long* keys = p.seg_key + u * S;
      unsigned long long mk = 0;
      double part = 0.0;
      if (S <= 64) {
        unsigned long long kk = 0;
        double sm = 0.0;
        bool have = tid >= S;
        for (int it = 0;; ++it) {
          if (!have) {
            kk = load_dev_u64(keys + tid);
            sm = load_dev_f64(ssum + tid);
            have = kk != 0ull && sm != kUnset;
          }
          if (__ballot(!have) == 0ull) break;
          if (wait_abandoned(it, err)) {
            if (tid == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (tid >= S) kk = 0ull, sm = 0.0;
        mk = wave_max_u64(kk);
        M = (double)key_value(mk);
        const double ms = (double)key_value(kk);
        part = tid < S && ms > -INFINITY ? sm * exp_neg(ms - M, etab) : 0.0;
        k0_s[tid] = kk;
        sl_s[tid] = sm;
      } else {
        for (int it = 0;; ++it) {
          bool ok = true;
          mk = 0;
          for (int s2 = tid; s2 < S; s2 += 64) {
            const unsigned long long k2 = load_dev_u64(keys + s2);
            ok = ok && k2 != 0ull && load_dev_f64(ssum + s2) != kUnset;
            mk = umax64(mk, k2);
          }
          if (__ballot(!ok) == 0ull) break;
          if (wait_abandoned(it, err)) {
            if (tid == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        mk = wave_max_u64(mk);
        M = (double)key_value(mk);
        for (int s2 = tid; s2 < S; s2 += 64) {
          const double ms = (double)key_value(load_dev_u64(keys + s2));
          const double sm = load_dev_f64(ssum + s2);
          part += ms > -INFINITY ? sm * exp_neg(ms - M, etab) : 0.0;
        }
      }
      const double zz = wave_sum_f64(part);
      if (tid == 0) {
        m_sh = M;
        z_sh = zz;
        if (seg == 0) store_dev_u64(p.node_key + u, mk);
      }
    }
    if (tid < npre) pthr_s[tid] = (double)pua_s[tid] * (double)pre_q;
    __syncthreads();
    M = uniform_f64(m_sh);
    z = uniform_f64(z_sh);
    // res_0 = exp(l - m_t) exp(m_t - M) / Z_0
    const double rz = uniform_f64(z > 0.0 ? 1.0 / z : 0.0);
    const float mt = mt_s[tid];
    const double sc = mt > -INFINITY ? exp_neg((double)mt - M, etab) * rz : 0.0;
#pragma unroll
    for (int k = 0; k < kRejPer; ++k) res[k] *= sc;
  }
  int lvl = 0;                                    // the residual level res holds (the last with mass)
  double zl = z;

  // the child of rank r against res_r at its token, by the thread that holds the token; a token outside
  // the vocabulary is rejected, by segment 0
  auto test_child = [&](int r) {
    if (r >= nk) return;
    const int c = kids_s[r];
    int x;
    double thr;
    if (r < kPreTests) {
      x = ptok_s[r];
      thr = pthr_s[r];
    } else {
      x = p.draft_tokens[n0 + c];
      thr = x >= 0 && x < p.vocab ? (double)p.u_accept[n0 + c] * (double)p.draft_probs[u * p.vocab + x] : 0.0;
    }
    if (x < 0 || x >= p.vocab) {
      if (seg == 0 && tid == 0) {
        store_dev_i32(p.acc_ok + n0 + c, 0);
#ifdef SPEC_DEBUG
        if (p.dbg) atomicAdd(&p.dbg[2], 1u);
#endif
      }
      return;
    }
    if (x < a0 || x >= a1) return;
    const int kx = x - a0;
    double rv = 0.0;
#pragma unroll
    for (int k = 0; k < kRejPer; ++k)
      if (k == kx) rv = res[k];
    store_dev_i32(p.acc_ok + n0 + c, thr < rv ? 1 : 0);
#ifdef SPEC_DEBUG
    if (p.dbg) atomicAdd(&p.dbg[2], 1u);
#endif
  };
  test_child(0);

  // ---- syncs 2 + r: the residual levels ----
  // A thread whose run still has residual mass (part > 0) replaces res by
  // max(0, res - q) at once: the level's total is then > 0, and res_r is that times 1/Z_r.  A thread
  // without keeps res_{r-1}: res_r is 0 there when Z_r > 0, and Z_r == 0 keeps the previous level.
  for (int r = 1; r <= nl; ++r) {
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < kRejPer; ++k) part += fmax(0.0, res[k] - (double)qv[k]);
    const bool mass = part > 0.0;
    if (mass) {
      // (q is converted to fp64 again here rather than kept converted from the sum above: 32 more fp64
      // values live at once would cost a quarter of the register file, i.e. the occupancy)
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) asm volatile("" : "+v"(qv[k]));
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) res[k] = fmax(0.0, res[k] - (double)qv[k]);
    }
    const double acc = block_sum_f64(part);
    // a level's slots carry their own values: only the last one also vouches for the node's test
    // stores (the walk reads them once the node has counted itself)
    if (r == nl) publish_f64(ssum + r * S + seg, acc);
    else if (tid == 0) store_dev_f64(ssum + r * S + seg, acc);
    double s_mine = 0.0;
    z = wait_total(ssum + r * S, S, err, &s_mine);
    if (z > 0.0) {
      const double rz = uniform_f64(1.0 / z);
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) res[k] = mass ? res[k] * rz : 0.0;
      lvl = r;
      zl = z;
      if (tid < 64) sl_s[tid] = s_mine;
    }
    test_child(r);
  }

  // ---- the bonus draw from res (level lvl): the segment where the cumulative residual passes
  // u_sample * total (every work-group of the node finds the same one), then the entry inside it ----
  {
    const double* ss = ssum + lvl * S;
    const double rz = uniform_f64(1.0 / zl);
    // segment q's share of the residual: level 0's slots hold sums against the segment maximum
    // (with S <= 64, segment tid's values were kept from the polls; others are read again, with the
    // same bits)
    auto wseg = [&](int q) -> double {
      const bool kept = S <= 64 && q == tid;
      const double v = kept ? sl_s[tid] : load_dev_f64(ss + q);
      if (lvl > 0) return v * rz;
      const double ms = (double)key_value(kept ? k0_s[tid] : load_dev_u64(p.seg_key + u * S + q));
      return ms > -INFINITY ? v * exp_neg(ms - M, etab) * rz : 0.0;
    };
    // each thread owns a run of consecutive segments; a fixed-order block scan of the run totals gives
    // every run its starting point
    const int per_s = (S + 255) / 256;
    const int s0 = min(tid * per_s, S), s1 = min(s0 + per_s, S);
    double run_tot = 0.0;
    for (int q = s0; q < s1; ++q) run_tot += wseg(q);
    double tot;
    const double start = block_scan_excl_f64(run_tot, &tot);
    const double thr = (double)us * tot;
    if (tid == 0) {
      claim_s = 0x7FFFFFFF;
      base_s = 0.0;
      thr_s = thr;
    }
    __syncthreads();
    int my_q = -1;
    double my_base = 0.0;
    if (start <= thr && start + run_tot > thr) {
      double base = start;
      for (int q = s0; q < s1; ++q) {
        const double w = wseg(q);
        if (base + w > thr) {
          my_q = q;
          my_base = base;
          break;
        }
        base += w;
      }
      if (my_q < 0) {                             // rounding inside the run: its last segment with mass
        for (int q = s1 - 1; q >= s0; --q)
          if (load_dev_f64(ss + q) > 0.0) {
            my_q = q;
            break;
          }
        my_base = start;
        for (int q = s0; q < my_q; ++q) my_base += wseg(q);
      }
      if (my_q >= 0) atomicMin(&claim_s, my_q);   // rounding may let two runs claim: lowest wins
    }
    __syncthreads();
    if (my_q >= 0 && my_q == claim_s) base_s = my_base;
    if (tid == 0 && claim_s == 0x7FFFFFFF) {      // rounding left the threshold past the end: the last
      double base = tot;                          // segment with mass
      int sg = S - 1;
      for (int q = S - 1; q >= 0; --q) {
        const double w = wseg(q);
        base -= w;
        if (w > 0.0) {
          sg = q;
          break;
        }
      }
      claim_s = sg;
      base_s = base;
    }
    __syncthreads();
    if (claim_s == seg) {                         // (uniform) this segment holds the draw
      double mine = 0.0;
#pragma unroll
      for (int k = 0; k < kRejPer; ++k) mine += res[k];
      double seg_tot;
      const double lo = base_s + block_scan_excl_f64(mine, &seg_tot);
      const double th = thr_s;
      if (tid == 0) claim_s = 0x7FFFFFFF;
      __syncthreads();
      if (nv > 0 && lo + mine > th && lo <= th) {
        double run = lo;                          // (entries past the end hold +0: they pass nothing)
        int kp = nv - 1;
        bool found = false;
#pragma unroll
        for (int k = 0; k < kRejPer; ++k) {       // the first entry whose running sum passes thr
          if (found) continue;
          run += res[k];
          if (run > th) {
            kp = k;
            found = true;
          }
        }
        atomicMin(&claim_s, a0 + kp);             // rounding may let two threads claim: lowest wins
      }
      __syncthreads();
      if (claim_s == 0x7FFFFFFF) {                // rounding: the last entry with mass in the segment
        int last = -1;
#pragma unroll
        for (int k = 0; k < kRejPer; ++k)
          if (res[k] > 0.0) last = k;
        const unsigned long long lk = last >= 0 ? (unsigned long long)(a0 + last + 1) : 0ull;
        const unsigned long long mx = block_max_u64(lk);
        if (tid == 0) claim_s = mx > 0 ? (int)mx - 1 : v0;
        __syncthreads();
      }
      // the node is done: its tests were stored before its last sync, its draw just now.  The sequence
      // counts its finished nodes; the last one walks the tree.
      if (tid == 0) {
        store_dev_i32(p.bonus_tok + u, claim_s);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t old = __hip_atomic_fetch_add(seq_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = old + 1 == (uint32_t)N;
      }
      __syncthreads();
    } else {
      return;
    }
  }

  // ---- the last node of the sequence to finish walks its tree ----
  if (!last_s) return;
  {
    // (the parents were read into LDS at the start)
    __shared__ int first_s[kMaxTreeNodes], rank_s[kMaxTreeNodes], nch_s[kMaxTreeNodes], path_s[kMaxTreeNodes];
    __shared__ int bad_s, stop_s, depth_s;
    const int16_t* par_s = par16_s;
    if (tid == 0) bad_s = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
#ifdef SPEC_DEBUG
    int rows_seen = 0;
#endif
    for (int j = tid; j < N; j += 256) {
      first_s[j] = 0x7FFFFFFF;
#ifdef SPEC_DEBUG
      rows_seen += load_dev_u64(p.node_key + n0 + j) != 0ull ? 1 : 0;   // row maximum written in this call
#endif
    }
    __syncthreads();
#ifdef SPEC_DEBUG
    if (p.dbg) {
      const double seen = block_sum_f64((double)rows_seen);
      if (tid == 0) atomicAdd(&p.dbg[1], (uint32_t)seen);
    }
#endif
    if (N <= 256)
      child_ranks<1, true>(par_s, N, tid, p.max_children, rank_s, nch_s, bad_s);
    else
      child_ranks<kMaxTreeNodes / 256, true>(par_s, N, tid, p.max_children, rank_s, nch_s, bad_s);
    __syncthreads();
    if (bad_s) {
      write_invalid(p, b, tid);
      return;
    }
    // the first accepted child of each node (every earlier sibling was rejected)
    for (int c = 1 + tid; c < N; c += 256)
      if (load_dev_i32(p.acc_ok + n0 + c) != 0) atomicMin(&first_s[par_s[c]], c);
    __syncthreads();
    if (tid == 0) {
      int x = 0, d = 0;
      path_s[0] = 0;
      while (first_s[x] != 0x7FFFFFFF && d + 1 < kMaxTreeNodes) {
        x = first_s[x];
        path_s[++d] = x;
      }
      stop_s = x;
      depth_s = d;
    }
    __syncthreads();
    const int depth = depth_s;
    if (depth + 1 > p.max_path) {
      write_invalid(p, b, tid);
      return;
    }
    const int bonus = load_dev_i32(p.bonus_tok + n0 + stop_s);
    int32_t* o_path = p.out_path_nodes + (int64_t)b * p.max_path;
    int32_t* o_tok = p.out_tokens + (int64_t)b * p.max_path;
    for (int k = tid; k < p.max_path; k += 256) {
      o_path[k] = k <= depth ? path_s[k] : -1;
      o_tok[k] = k < depth ? p.draft_tokens[n0 + path_s[k + 1]] : (k == depth ? bonus : -1);
    }
    if (tid == 0) p.out_num_accepted[b] = depth;
  }
}

}  // namespace

// workspace: the call's arrays, then the debug record (last SPEC_DEBUG_RECORD_BYTES bytes)
size_t greedy_keys_bytes(int batch, int max_nodes, int nseg) {
  return align_up(sizeof(unsigned long long) * (size_t)batch * max_nodes * nseg, 256);
}

size_t greedy_ws_bytes(int batch, int max_nodes, int nseg) {
  return greedy_keys_bytes(batch, max_nodes, nseg) + SPEC_DEBUG_RECORD_BYTES;
}

RejectionLayout rejection_layout(int batch, int max_nodes, int nsegr, int max_children) {
  const size_t nodes = (size_t)batch * max_nodes, lv = (size_t)max_children + 1;
  RejectionLayout l;
  l.off_node_key = greedy_keys_bytes(batch, max_nodes, nsegr);
  l.off_seg_sum = l.off_node_key + align_up(sizeof(unsigned long long) * nodes, 256);
  l.off_acc_ok = l.off_seg_sum + align_up(sizeof(double) * nodes * lv * nsegr, 256);
  l.off_bonus = l.off_acc_ok + align_up(sizeof(int32_t) * nodes, 256);
  l.off_sync = l.off_bonus + align_up(sizeof(int32_t) * nodes, 256);
  l.bytes = l.off_sync + align_up(sizeof(uint32_t) * (batch + 1), 256) + SPEC_DEBUG_RECORD_BYTES;
  return l;
}

size_t rejection_ws_bytes(int batch, int max_nodes, int nsegr, int max_children) {
  return rejection_layout(batch, max_nodes, nsegr, max_children).bytes;
}

hipError_t launch_accept_greedy(const AcceptParams& p, hipStream_t s) {
  const unsigned rows = (unsigned)(p.batch * p.max_nodes);
  hipLaunchKernelGGL(argmax_seg_kernel, dim3(p.nseg, rows), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_walk_kernel, dim3(p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_accept_rejection(const AcceptParams& p, hipStream_t s) {
  const int n = p.batch * p.max_nodes * p.nsegr + p.batch + 1;
  hipLaunchKernelGGL(rej_clear_kernel, dim3((unsigned)min(ceil_div(n, 256), (int64_t)1024)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.bf16) hipLaunchKernelGGL(rejection_kernel<true>, dim3(p.nsegr, p.max_nodes, p.batch), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(rejection_kernel<false>, dim3(p.nsegr, p.max_nodes, p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace spec
