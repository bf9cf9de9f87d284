// Greedy and rejection-sampling acceptance over a draft tree, for gfx950.
//
// Greedy: a draft is accepted iff it equals the target's greedy choice at its parent (vllm.cpp
// "Speculative decoding", section MTP); on a tree the result is the deepest accepted node.
// Rejection: accept x ~ q with probability min(1, p(x)/q(x)); on rejection continue with the
// normalised residual max(0, res - q) ("Adaptive Speculative Decoding", sections "Correctness
// first" and "The controller"), generalised to siblings drawn i.i.d. from q.
//
// Both are HBM streams over the [nodes][vocab] logits (16-33 MB at vocab 128K), so the work is
// spread over (vocab segment x node) work-groups with fixed-order reductions, and only the tree
// walk itself runs in one work-group per sequence:
//   argmax_seg     (greedy) per (node, 8192-token segment): the packed key (ordered value, ~index)
//                  maximum, i.e. the largest logit with the lowest index among exact ties
//   max_sum_seg    (rejection) per (node, 2048-token segment): the same key, and level 0's
//                  sum exp(l - m_s) against the segment maximum m_s, from one read of the logits;
//                  segment 0 also counts the node's children.  node_max then takes the row maximum
//                  M and scales each sum by exp(m_s - M)
//   residual_pass  (rejection) level r >= 1, for nodes with >= r children: sum max(0, res_{r-1} - q),
//                  with res_{r-1} rebuilt per element from the earlier levels' normalisers
//                  (all fp64, exp evaluated in fp64), whose totals every work-group sums in one fixed
//                  order and segment 0 stores for the walk
// Each thread of the rejection passes loads its run of 8 consecutive entries before using any of them,
// so a pass costs one round trip to memory.
//   walk           per sequence: accept tests of every child in parallel (a child is tested only
//                  after all earlier siblings were rejected, so its residual level is its sibling
//                  rank), first accepted child per node by LDS atomic-min, walk from the root,
//                  then the bonus token (greedy: argmax; rejection: inverse CDF of the residual,
//                  segment found from the segment sums, then an in-segment scan)
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

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax64(v, shfl_xor_u64(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
  __syncthreads();
  return v;
}

// Block-wide (256 threads) fp64 sum in a fixed order; result valid in every thread.
__device__ double block_sum_f64(double v) {
  __shared__ double red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
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

__device__ __forceinline__ float row_max(const AcceptParams& p, int64_t u) { return key_value(p.node_key[u]); }

// Normaliser k of node u: Z[0] = sum exp(l - M); Z[k] = sum max(0, res_{k-1} - q) (fixed-order totals)
__device__ __forceinline__ double level_sum(const AcceptParams& p, int64_t u, int k) {
  return p.zsum[u * (p.max_children + 1) + k];
}

// ---- rejection: per node, the row-maximum key over the segments (one wave per node); then the
// level-0 segment sums, taken against each segment's own maximum m_s, are brought to the row maximum M:
// sum exp(l - m_s) * exp(m_s - M) ----
__global__ __launch_bounds__(64) void node_max_kernel(AcceptParams p) {
  const int64_t u = blockIdx.x;
  // seg_key has a row for every row of the grid: its reads go out together with the row-count read
  const int tn = total_nodes(p);
  // the first key and level-0 sum of each lane stay in registers for the rescale below
  const int s_first = threadIdx.x;
  double* s0 = p.seg_sum + u * (p.max_children + 1) * p.nsegr;
  const unsigned long long k_first = s_first < p.nseg ? p.seg_key[u * p.nseg + s_first] : 0ull;
  const double sum_first = s_first < p.nsegr ? s0[s_first] : 0.0;
  unsigned long long k = k_first;
  for (int s = s_first + 64; s < p.nseg; s += 64) k = umax64(k, p.seg_key[u * p.nseg + s]);
  if (u >= tn) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) k = umax64(k, shfl_xor_u64(k, off));
  if (threadIdx.x == 0) p.node_key[u] = k;
  const double M = (double)key_value(k);
  for (int s = s_first; s < p.nsegr; s += 64) {
    const double ms = (double)key_value(s == s_first ? k_first : p.seg_key[u * p.nseg + s]);
    const double sum = s == s_first ? sum_first : s0[s];
    s0[s] = ms > -INFINITY ? sum * exp(ms - M) : 0.0;
  }
}

// Total of residual level r of node u over its segments, summed by one wave in a fixed order (lanes
// stride the segments, then a butterfly): every caller gets the same bits.  Valid in every lane.
__device__ __forceinline__ double level_total_wave(const AcceptParams& p, int64_t u, int r) {
  const double* s = p.seg_sum + (u * (p.max_children + 1) + r) * p.nsegr;
  double z = 0.0;
  for (int i = threadIdx.x & 63; i < p.nsegr; i += 64) z += s[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  return z;
}

// A thread's run of kResPer consecutive vocabulary entries [a0, a1) of row u (a1 - a0 <= kResPer): the
// logits as fp32 and, if want_q, the draft probabilities.  Every load is issued before any value is
// used (one round trip to memory instead of one per entry); 16-byte loads where the run is whole and
// aligned.  Entries at and past a1 are left 0.
constexpr int kResPer = kResSegment / 256;
static_assert(kResPer % 8 == 0, "a run is whole 16-byte loads of bf16 logits and of fp32 probabilities");

__device__ __forceinline__ void load_run(const AcceptParams& p, int64_t u, int a0, int a1, bool want_q,
                                         float (&lg)[kResPer], float (&qv)[kResPer]) {
  const bool whole = a1 - a0 == kResPer;
  if (p.bf16) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(p.logits) + u * p.vocab + a0;
    if (whole && ((uintptr_t)row & 15) == 0) {
      u32x4 w[kResPer / 8];
#pragma unroll
      for (int j = 0; j < kResPer / 8; ++j) w[j] = *reinterpret_cast<const u32x4*>(row + 8 * j);
#pragma unroll
      for (int j = 0; j < kResPer / 8; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lg[8 * j + 2 * k] = __uint_as_float(w[j][k] << 16);
          lg[8 * j + 2 * k + 1] = __uint_as_float(w[j][k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
      for (int i = 0; i < kResPer; ++i) lg[i] = a0 + i < a1 ? __uint_as_float((uint32_t)row[i] << 16) : 0.f;
    }
  } else {
    const float* row = reinterpret_cast<const float*>(p.logits) + u * p.vocab + a0;
    if (whole && ((uintptr_t)row & 15) == 0) {
      u32x4 w[kResPer / 4];
#pragma unroll
      for (int j = 0; j < kResPer / 4; ++j) w[j] = *reinterpret_cast<const u32x4*>(row + 4 * j);
#pragma unroll
      for (int j = 0; j < kResPer / 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) lg[4 * j + k] = __uint_as_float(w[j][k]);
    } else {
#pragma unroll
      for (int i = 0; i < kResPer; ++i) lg[i] = a0 + i < a1 ? row[i] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < kResPer; ++i) qv[i] = 0.f;
  if (want_q) {
    const float* row = p.draft_probs + u * p.vocab + a0;
    if (whole && ((uintptr_t)row & 15) == 0) {
      u32x4 w[kResPer / 4];
#pragma unroll
      for (int j = 0; j < kResPer / 4; ++j) w[j] = *reinterpret_cast<const u32x4*>(row + 4 * j);
#pragma unroll
      for (int j = 0; j < kResPer / 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) qv[4 * j + k] = __uint_as_float(w[j][k]);
    } else {
#pragma unroll
      for (int i = 0; i < kResPer; ++i) qv[i] = a0 + i < a1 ? row[i] : 0.f;
    }
  }
}

// ---- rejection: per (node, residual segment) the maximum key and the level-0 sum sum exp(l - m_s)
// against the segment's own maximum m_s, from one read of the logits (the row maximum is not known
// yet; node_max_kernel rescales the sums to it) ----
__global__ __launch_bounds__(256) void max_sum_seg_kernel(AcceptParams p) {
  const int seg = blockIdx.x;
  const int i = blockIdx.y;                       // the node within its sequence
  const int b = blockIdx.z;
  const int tn = total_nodes(p);
  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  const int64_t u = (int64_t)n0 + i;
  if (i >= N || u >= tn) return;
  // segment 0 also counts the node's children (the later ones among the sequence's nodes whose parent
  // is i), for the residual passes; its parent reads go out with the logit reads
  int kids = 0;
  if (seg == 0)
    for (int j = 1 + (int)threadIdx.x; j < N && n0 + j < tn; j += 256) kids += (p.parents[n0 + j] == i && i < j) ? 1 : 0;
  const int v0 = seg * kResSegment;
  const int v1 = min(p.vocab, v0 + kResSegment);
  const int a0 = min(v1, v0 + (int)threadIdx.x * kResPer), a1 = min(v1, a0 + kResPer);
  float lg[kResPer], qv[kResPer];
  load_run(p, u, a0, a1, false, lg, qv);
  // this thread's largest logit, then the lowest index holding it (visited from the top down), packed once
  float mv = -INFINITY;
#pragma unroll
  for (int i = 0; i < kResPer; ++i)
    if (a0 + i < a1) mv = fmaxf(mv, lg[i]);
  int idx = a0;
#pragma unroll
  for (int i = kResPer - 1; i >= 0; --i)
    if (a0 + i < a1 && lg[i] == mv) idx = a0 + i;
  unsigned long long best = a0 < a1 ? pack_key(mv, idx) : 0ull;
  best = block_max_u64(best);
  const double m = (double)key_value(best);
  double acc = 0.0;                               // this thread's run, summed in order
  if (m > -INFINITY) {                            // a segment of -inf logits has no mass
    // branch-free: an entry past the end takes exp(-inf) = +0, which leaves the sum's bits unchanged,
    // and the eight exps share their constants and interleave
#pragma unroll
    for (int i = 0; i < kResPer; ++i) acc += exp(a0 + i < a1 ? (double)lg[i] - m : -INFINITY);
  }
  acc = block_sum_f64(acc);
  if (threadIdx.x == 0) {
    p.seg_key[u * p.nseg + seg] = best;
    p.seg_sum[u * (p.max_children + 1) * p.nsegr + seg] = acc;
  }
  if (seg == 0) {                                 // uniform in the work-group
    const double k = block_sum_f64((double)kids); // exact: at most max_nodes
    if (threadIdx.x == 0) p.n_children[u] = (int)k;
  }
}

// ---- rejection: one residual level r >= 1 for every node that needs it ----
__global__ __launch_bounds__(256) void residual_pass_kernel(AcceptParams p, int r) {
  const int seg = blockIdx.x;
  const int64_t u = blockIdx.y;
  // both reads are issued before either test (n_children has an entry for every row of the grid)
  const int tn = total_nodes(p);
  const int nc = p.n_children[u];
  if ((u >= tn) | (nc < r)) return;
  extern __shared__ double rz_s[];                // [max_children + 1] reciprocals of the earlier levels' totals
  const int v0 = seg * kResSegment;
  const int v1 = min(p.vocab, v0 + kResSegment);
  const int a0 = min(v1, v0 + (int)threadIdx.x * kResPer), a1 = min(v1, a0 + kResPer);
  float lg[kResPer], qv[kResPer];
  load_run(p, u, a0, a1, true, lg, qv);
  const double M = (double)row_max(p, u);
  double acc = 0.0;                               // this thread's run, summed in order
  {
    // the earlier levels' totals, summed here (wave w takes levels w, w + 4, ...; each in the order the
    // walk's totals use), kept as reciprocals: a product with the reciprocal differs from the quotient
    // by at most one fp64 rounding.  The first 9 are held in registers.
    for (int k = threadIdx.x >> 6; k < r; k += 4) {
      const double z = level_total_wave(p, u, k);
      if ((threadIdx.x & 63) == 0) {
        rz_s[k] = z > 0.0 ? 1.0 / z : 0.0;
        if (seg == 0) p.zsum[u * (p.max_children + 1) + k] = z;   // for the walk (the same bits in every pass)
      }
    }
    __syncthreads();
    // the first 9 in registers: every index below is a constant after unrolling (an array indexed by a
    // loop variable would live in scratch memory, one read per entry and level)
    double Z[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) Z[k] = k < r ? rz_s[k] : 0.0;
    // branch-free over the run: an entry past the end has q = 0 and exp(-inf) = +0, so it adds +0
#pragma unroll
    for (int i = 0; i < kResPer; ++i) {
      const double q = (double)qv[i];
      double res = exp(a0 + i < a1 ? (double)lg[i] - M : -INFINITY) * Z[0];
#pragma unroll
      for (int k = 1; k < 9; ++k) {
        if (k >= r) break;
        const double d = fmax(0.0, res - q);
        if (Z[k] > 0.0) res = d * Z[k];
      }
      for (int k = 9; k < r; ++k) {
        const double d = fmax(0.0, res - q);
        const double zk = rz_s[k];
        if (zk > 0.0) res = d * zk;
      }
      acc += fmax(0.0, res - q);
    }
  }
  acc = block_sum_f64(acc);
  if (threadIdx.x == 0) p.seg_sum[(u * (p.max_children + 1) + r) * p.nsegr + seg] = acc;
}

// Child count and sibling rank (earlier siblings) of the nodes tid + 256 q, q < PER; flags a parent
// array that is not topological or a node with more than max_children children.  Without COUNT (greedy)
// only the parent-order checks run.
template <int PER, bool COUNT>
__device__ __forceinline__ void child_ranks(const int* par_s, int N, int tid, int max_children, int* rank_s,
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

// ---- per sequence: the walk and the bonus token ----
template <bool REJECT>
__global__ __launch_bounds__(256) void walk_kernel(AcceptParams p) {
  __shared__ int par_s[kMaxTreeNodes], tok_s[kMaxTreeNodes], first_s[kMaxTreeNodes], nch_s[kMaxTreeNodes];
  __shared__ int rank_s[kMaxTreeNodes], amax_s[kMaxTreeNodes], path_s[kMaxTreeNodes];
  __shared__ int stop_s, depth_s, bad_s, seg_s, bonus_s;
  __shared__ double base_s, thr_s, zlast_s;
  __shared__ double zs[9];
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
    for (int i = tid; i < p.max_path; i += 256) { o_path[i] = -1; o_tok[i] = -1; }
    if (tid == 0) p.out_num_accepted[b] = -1;
    return;
  }
  if (tid == 0) bad_s = 0;
#ifdef SPEC_DEBUG
  if (tid == 0) dbg_rows_s = dbg_tests_s = 0;
  __syncthreads();
#endif
  for (int i = tid; i < N; i += 256) {
    int pi = p.parents[n0 + i];
    par_s[i] = pi;
    int t = p.draft_tokens[n0 + i];
    tok_s[i] = t;
    first_s[i] = 0x7FFFFFFF;
    if (!REJECT) {
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
#ifdef SPEC_DEBUG
    if (REJECT && p.node_key[n0 + i] != 0ull) atomicAdd(&dbg_rows_s, 1);   // row maximum written in this call
#endif
  }
  __syncthreads();
  // child counts and sibling ranks: each parent entry is read once and compared with the nodes this
  // thread owns (tid, tid + 256, ...): one node per thread for trees of <= 256 nodes, else up to 8
  if (N <= 256)
    child_ranks<1, REJECT>(par_s, N, tid, REJECT ? p.max_children : 0x7FFFFFFF, rank_s, nch_s, bad_s);
  else
    child_ranks<kMaxTreeNodes / 256, REJECT>(par_s, N, tid, REJECT ? p.max_children : 0x7FFFFFFF, rank_s, nch_s,
                                             bad_s);
  __syncthreads();
  if (bad_s) {
    for (int i = tid; i < p.max_path; i += 256) { o_path[i] = -1; o_tok[i] = -1; }
    if (tid == 0) p.out_num_accepted[b] = -1;
    return;
  }
  // accept tests of every child, in parallel
  for (int c = 1 + tid; c < N; c += 256) {
    const int u = par_s[c];
    const int x = tok_s[c];
    bool ok = false;
#ifdef SPEC_DEBUG
    atomicAdd(&dbg_tests_s, 1);
#endif
    if (x >= 0 && x < p.vocab) {
      if (!REJECT) {
        ok = (x == amax_s[u]);
      } else {
        const int64_t gu = n0 + u;
        const int r = rank_s[c];
        // every read of the test is issued before any is used: the first 9 level totals (entries past r
        // repeat level r, which exists, and are not used), the row maximum, q(x) and the logit
        double Z[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) Z[k] = level_sum(p, gu, k < r ? k : r);
        const double M = (double)row_max(p, gu);
        const double qx = (double)p.draft_probs[gu * p.vocab + x];
        const float lx = load_logit(p, gu, x);
#pragma unroll
        for (int k = 0; k < 9; ++k) Z[k] = Z[k] > 0.0 ? 1.0 / Z[k] : 0.0;   // reciprocals, as in the residual passes
        const double e = exp((double)lx - M);
        double res = e * Z[0];
        for (int k = 1; k <= r; ++k) {
          const double d = fmax(0.0, res - qx);
          const double zk = k < 9 ? Z[k] : (level_sum(p, gu, k) > 0.0 ? 1.0 / level_sum(p, gu, k) : 0.0);
          if (zk > 0.0) res = d * zk;
        }
        ok = (double)p.u_accept[n0 + c] * qx < res;
      }
    }
    if (REJECT) {
      if (ok) atomicMin(&first_s[u], c);
    } else {
      rank_s[c] = ok ? 1 : 0;                     // greedy: the edge test, reused below
    }
  }
  __syncthreads();
#ifdef SPEC_DEBUG
  if (tid == 0 && p.dbg) {
    atomicAdd(&p.dbg[1], (uint32_t)dbg_rows_s);
    atomicAdd(&p.dbg[2], (uint32_t)dbg_tests_s);
  }
#endif
  if (REJECT) {
    // sampling order: at each node move to its first accepted child
    if (tid == 0) {
      int u = 0, d = 0;
      path_s[0] = 0;
      while (first_s[u] != 0x7FFFFFFF && d + 1 < kMaxTreeNodes) {
        u = first_s[u];
        path_s[++d] = u;
      }
      stop_s = u;
      depth_s = d;
    }
  } else {
    // greedy: node j is accepted iff every edge on its root path passed; keep the deepest
    // accepted node, the lowest index among equally deep ones
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
  }
  __syncthreads();
  const int u = stop_s, depth = depth_s;
  if (depth + 1 > p.max_path) {
    for (int i = tid; i < p.max_path; i += 256) { o_path[i] = -1; o_tok[i] = -1; }
    if (tid == 0) p.out_num_accepted[b] = -1;
    return;
  }
  int bonus;
  if (!REJECT) {
    bonus = amax_s[u];
  } else {
    // inverse CDF of the residual left at u after all its children were rejected
    const int64_t gu = n0 + u;
    const int r = nch_s[u];
    // the totals of levels < r were stored by the residual passes; level r's (no pass follows it for this
    // node) is summed here by wave 0 in the passes' order, so it has the bits they would give it
    if (tid < 64) {
      const double z = level_total_wave(p, gu, r);
      if (tid == 0) {
        zlast_s = z;
        if (r < 9) zs[r] = z;
      }
    }
    if (tid < r && tid < 9) zs[tid] = level_sum(p, gu, tid);    // read in parallel
    __syncthreads();
    auto zsum_of = [&](int k) -> double { return k == r ? zlast_s : level_sum(p, gu, k); };
    if (tid == 0) {
      int lvl = 0;
      for (int k = 0; k <= r; ++k) {
        const double z = k < 9 ? zs[k] : zsum_of(k);
        if (z > 0.0 || k == 0) lvl = k;             // a zero residual keeps the previous level
      }
      seg_s = lvl;                                  // the level, handed to the block below
    }
    __syncthreads();
    {
      // the segment where the cumulative residual passes u * total: each thread owns a run of consecutive
      // segments; a fixed-order block scan of the run totals gives every run its starting point
      const int lvl = seg_s;
      const double* ss = p.seg_sum + (gu * (p.max_children + 1) + lvl) * p.nsegr;
      const double rz = 1.0 / zsum_of(lvl);
      const int per_s = (p.nsegr + 255) / 256;
      const int s0 = min(tid * per_s, p.nsegr), s1 = min(s0 + per_s, p.nsegr);
      double run_tot = 0.0;
      for (int q = s0; q < s1; ++q) run_tot += ss[q] * rz;
      double tot;
      const double start = block_scan_excl_f64(run_tot, &tot);
      const double thr = (double)p.u_sample[gu] * tot;
      if (tid == 0) {
        seg_s = 0x7FFFFFFF;
        base_s = 0.0;
        thr_s = thr;
        bonus_s = 0x7FFFFFFF;
      }
      __syncthreads();
      int my_q = -1;
      double my_base = 0.0;
      if (start <= thr && start + run_tot > thr) {
        double base = start;
        for (int q = s0; q < s1; ++q) {
          const double w = ss[q] * rz;
          if (base + w > thr) {
            my_q = q;
            my_base = base;
            break;
          }
          base += w;
        }
        if (my_q < 0) {                             // rounding inside the run: its last segment with mass
          for (int q = s1 - 1; q >= s0; --q)
            if (ss[q] > 0.0) {
              my_q = q;
              break;
            }
          my_base = start;
          for (int q = s0; q < my_q; ++q) my_base += ss[q] * rz;
        }
        if (my_q >= 0) atomicMin(&seg_s, my_q);     // rounding may let two runs claim: lowest wins
      }
      __syncthreads();
      if (my_q >= 0 && my_q == seg_s) base_s = my_base;
      if (tid == 0 && seg_s == 0x7FFFFFFF) {        // rounding left the threshold past the end: the last
        double base = tot;                          // segment with mass
        int seg = p.nsegr - 1;
        for (int q = p.nsegr - 1; q >= 0; --q) {
          base -= ss[q] * rz;
          if (ss[q] > 0.0) {
            seg = q;
            break;
          }
        }
        seg_s = seg;
        base_s = base;
      }
    }
    __syncthreads();
    const int seg = seg_s;
    const int v0 = seg * kResSegment;
    const int v1 = min(p.vocab, v0 + kResSegment);
    const int a0 = min(v1, v0 + tid * kResPer);
    const int a1 = min(v1, a0 + kResPer);
    float lg[kResPer], qr[kResPer];
    load_run(p, gu, a0, a1, true, lg, qr);
    const double M = (double)row_max(p, gu);
    const float* q = p.draft_probs + gu * (int64_t)p.vocab;
    double Z[9];
    for (int k = 0; k <= r && k < 9; ++k) Z[k] = zs[k] > 0.0 ? 1.0 / zs[k] : 0.0;
    auto res_from = [&](float l, float qf) -> double {
      const double qv = (double)qf;
      double res = exp((double)l - M) * Z[0];
      for (int k = 1; k <= r; ++k) {
        const double dd = fmax(0.0, res - qv);
        const double zk = k < 9 ? Z[k] : (zsum_of(k) > 0.0 ? 1.0 / zsum_of(k) : 0.0);
        if (zk > 0.0) res = dd * zk;
      }
      return res;
    };
    auto res_of = [&](int v) -> double { return res_from(load_logit(p, gu, v), q[v]); };
    // this thread's run of the residual, evaluated once and kept for the claim below
    double rv[kResPer];
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < kResPer; ++i) {             // an entry past the end gives +0 (q = 0, exp(-inf) = +0)
      rv[i] = res_from(a0 + i < a1 ? lg[i] : -INFINITY, qr[i]);
      mine += rv[i];
    }
    double seg_tot;
    const double lo = base_s + block_scan_excl_f64(mine, &seg_tot);
    const double thr = thr_s;
    if (a0 < a1 && lo + mine > thr && lo <= thr) {
      double run = lo;
      int pick = a1 - 1;
      bool found = false;
#pragma unroll
      for (int i = 0; i < kResPer; ++i) {         // the first entry whose running sum passes thr
        if (found || a0 + i >= a1) continue;
        run += rv[i];
        if (run > thr) {
          pick = a0 + i;
          found = true;
        }
      }
      atomicMin(&bonus_s, pick);                    // rounding may let two threads claim: lowest wins
    }
    __syncthreads();
    if (tid == 0 && bonus_s == 0x7FFFFFFF) {        // rounding: take the last token with mass in the segment
      int pick = v0;
      for (int v = v1 - 1; v >= v0; --v)
        if (res_of(v) > 0.0) { pick = v; break; }
      bonus_s = pick;
    }
    __syncthreads();
    bonus = bonus_s;
  }
  for (int i = tid; i < p.max_path; i += 256) {
    o_path[i] = i <= depth ? path_s[i] : -1;
    o_tok[i] = i < depth ? tok_s[path_s[i + 1]] : (i == depth ? bonus : -1);
  }
  if (tid == 0) p.out_num_accepted[b] = depth;
}

}  // namespace

// workspace: the call's arrays, then the debug record (last SPEC_DEBUG_RECORD_BYTES bytes)
size_t greedy_keys_bytes(int batch, int max_nodes, int nseg) {
  return align_up(sizeof(unsigned long long) * (size_t)batch * max_nodes * nseg, 256);
}

size_t greedy_ws_bytes(int batch, int max_nodes, int nseg) {
  return greedy_keys_bytes(batch, max_nodes, nseg) + SPEC_DEBUG_RECORD_BYTES;
}

size_t rejection_ws_bytes(int batch, int max_nodes, int nsegr, int max_children) {
  const size_t nodes = (size_t)batch * max_nodes, lv = (size_t)max_children + 1;
  return greedy_keys_bytes(batch, max_nodes, nsegr) + align_up(sizeof(unsigned long long) * nodes, 256) +
         align_up(sizeof(double) * nodes * lv * nsegr, 256) + align_up(sizeof(double) * nodes * lv, 256) +
         align_up(sizeof(int32_t) * nodes, 256) + SPEC_DEBUG_RECORD_BYTES;
}

hipError_t launch_accept_greedy(const AcceptParams& p, hipStream_t s) {
  const unsigned rows = (unsigned)(p.batch * p.max_nodes);
  hipLaunchKernelGGL(argmax_seg_kernel, dim3(p.nseg, rows), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk_kernel<false>, dim3(p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_accept_rejection(const AcceptParams& p, hipStream_t s) {
  const unsigned rows = (unsigned)(p.batch * p.max_nodes);
  hipLaunchKernelGGL(max_sum_seg_kernel, dim3(p.nsegr, p.max_nodes, p.batch), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(node_max_kernel, dim3(rows), dim3(64), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int r = 1; r <= p.max_children; ++r) {
    hipLaunchKernelGGL(residual_pass_kernel, dim3(p.nsegr, rows), dim3(256),
                       sizeof(double) * (size_t)(p.max_children + 1), s, p, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(walk_kernel<true>, dim3(p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace spec
