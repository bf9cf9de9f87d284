// Tree-masked GQA attention over a paged bf16 KV cache, for gfx950.
//
// Every draft-tree node is a query of one verification forward; it sees the whole committed
// context and its own ancestors in the tree ("DiffSpec: Accelerating Long Sequence Generation
// with Differential Speculative Decoding", "What DiffSpec Does" item 5: verification shares the
// prefixes of the speculative structure; the chain case is the per-row cache mask of "Adaptive
// Speculative Decoding", section Layout).
//
// Design (MI355X-first):
//  * Split-K flash decoding.  A work-group owns one (sequence, KV head, KV split) range and up to
//    256 query rows (all tree nodes x the GQA group of that KV head), so each 64-slot K/V tile is
//    read from HBM once and shared, through LDS, by every node and every query head of the group.
//    Wider trees use several row groups; their work-groups are placed on the same XCD (work-group
//    ids i and i+8 land on one XCD) so the second read of a tile hits that XCD's L2.
//  * The split's block-table slice is staged in LDS once; each 64-slot tile is then copied straight
//    from HBM into LDS (buffer loads with the LDS destination, 16 bytes per lane, one scalar buffer
//    descriptor per page whose range ends at the sequence's last slot), double-buffered, the next
//    tile in flight while the current one is computed.  Rows are XOR-swizzled in 16-byte chunks so
//    that the MFMA operand reads hit no LDS bank conflicts.  V may be stored like K (token rows; the
//    V^T operand then comes from transposing LDS reads) or dim-major (each dim's tokens of a page
//    contiguous; plain 16-byte reads).
//  * Both products run on MFMA v_mfma_f32_16x16x32_bf16: S^T = K Q^T (A = K rows from LDS,
//    B = Q from registers), then O^T = V^T P^T (A = V^T from LDS, B = P straight from the S^T
//    accumulators).  In this orientation each lane owns one query row in every fragment, so the
//    only cross-lane step of the online softmax is a 4-lane max (permlane swaps); the row sum is
//    kept per lane in fp32 and reduced once at the end.  Per-chunk sums of P come from one more
//    MFMA against a constant ones fragment (every output slot then holds the row's chunk sum).
//  * Lazy rescaling: the running max only moves when a tile's max exceeds it by more than 2^8, so the
//    O accumulators are rescaled on a handful of tiles per split.  The exps are taken against the
//    running max first; only a tile whose probabilities exceed 2^8 computes its max and redoes them.
//  * Keys >= ctx_len are tree slots: visible iff the key's node is an ancestor-or-self of the
//    row's node.  The relation comes from ancestor bit masks built in LDS from the parent array
//    (up to 256 nodes), or, for trees in preorder (the bundle order of the DiffSpec README,
//    "Features": leaves grouped by branching ancestor), from index ranges: j is an ancestor-or-self
//    of i iff j <= i < subtree_end[j] (up to 2048 nodes, one int per node in LDS).
//  * A work-group's split stops after the tree slot of its last row's node: an ancestor's index is
//    below its descendant's, so later tree tiles are masked for all of its rows.
//  * With chunk_size > 0 each tile also emits, per query row, the log2-sum-exp of the row's scores
//    over each context chunk; the salience pass turns these into attention mass once the row's
//    final log-sum-exp is known (no second pass over K).
//  * Splits write (max, sum, unnormalised O) partials; the merge kernel combines them (LSE merge).
#include <type_traits>

#include "spec_internal.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima
constexpr float kRescale = 8.0f;      // log2 headroom before the running max must move

__device__ __forceinline__ float max4g(float x) {   // max over lanes l, l^16, l^32, l^48
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ bf16x8 bf16_splat8(uint32_t lo_pair, uint32_t hi_pair) {
  const u32x4 v = {lo_pair, lo_pair, hi_pair, hi_pair};
  return __builtin_bit_cast(bf16x8, v);
}

// 16 bytes per lane from global memory straight into LDS (lane i writes dst + 16 * i), through a raw
// buffer descriptor over [base, base + num_bytes): offsets at or past num_bytes read zeros.  The buffer
// descriptor type only exists for the device target, so the host pass sees an empty body.
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t num_bytes, void* dst, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voffset, 0, 0, 0);
#endif
}

// CM: 0 = chunk sums per 64-slot tile (chunk_size 0 or a multiple of 64), 1 = per 32 slots, 2 = per 16 slots
// VT: 0 = V pages hold token rows (like K), 1 = V pages are dim-major (each dim's page_size tokens contiguous)
// PRE: the tree is in preorder and p.subtree_end gives the ancestor relation as index ranges.  It is a
// compile-time switch: with a run-time flag the compiler versioned the tile loop on it, and that
// build gave wrong results on the bit-mask path as well (cause not found), so the two mask sources are
// separate instantiations.
// SW: (4-wave work-groups, token-row V, 64-slot chunks, <= 64 rows per KV head) waves 1 and 2 load the
// tiles and wave 3 alone writes the chunk ring out.  Wave 3 issues no loads, so no step waits for its
// stores: with HBM busy with the KV stream, a store round trip is longer than a step.
template <int D, int W, int RB, int CM, int VT, int PRE, int SW = 0>
__global__ __launch_bounds__(W * 64, (W == 8 ? 1 : 2)) void tree_attn_kernel(AttnParams p) {
  static_assert(!SW || (W == 4 && CM == 0 && VT == 0), "the store wave is a variant of the 4-wave chunk ring");
  constexpr int NT = W * 64;
  constexpr int NLW = SW ? 2 : W;               // waves that load tiles
  constexpr int ROWS_WG = W * RB * 16;
  constexpr int KS = D / 32;                    // k-steps of the QK^T product
  constexpr int NB = D / 16;                    // 16-dim output blocks
  constexpr int CPR = D / 8;                    // 16-byte chunks per K/V row
  constexpr int TILE_EL = kTile * D;            // bf16 elements of one K (or V) tile
  constexpr int LOADS = 2 * kTile * CPR / (NLW * 64);   // 16-byte direct-to-LDS loads per loading thread and tile
  constexpr int KB = kTile * CPR / 64;          // 1 KiB blocks of a K (or V) tile
  constexpr int NS = CM == 2 ? 4 : (CM == 1 ? 2 : 1);   // row-sum fragments per row block
  // ancestor masks: a 4-wave work-group holds <= 128 rows, hence <= 128 nodes (two 64-bit words)
  constexpr int ANC_N = W == 8 ? kMaxNodes : 128;
  constexpr int ANC_W = ANC_N / 64;
  static_assert((2 * kTile * CPR) % (NLW * 64) == 0 && (kTile * CPR) % 64 == 0, "tile must split evenly");

  // K and V tiles, double-buffered, rows of D bf16 without padding; the 16-byte chunk c of key r sits at
  // position c ^ swz(r) of its row, which keeps both the MFMA operand reads and the transposing V reads
  // free of bank conflicts
  // two separate arrays (not one indexed by the buffer number) so that alias analysis can tell the
  // tile being read from the tile whose direct-to-LDS loads are still in flight
  __shared__ __attribute__((aligned(16))) uint16_t kv_a[2][TILE_EL];
  __shared__ __attribute__((aligned(16))) uint16_t kv_b[2][TILE_EL];
  // The tree relation: ancestor bit masks (PRE = 0) or, for preorder trees, each node's subtree end
  // (PRE = 1).  One instantiation only ever touches one of the two members.
  constexpr int END_N = ANC_N * ANC_W * 2;
  static_assert(W != 8 || END_N >= kMaxTreeNodes, "subtree ends of the largest tree must fit");
  union TreeRel {
    uint64_t anc[ANC_N][ANC_W];
    int end[END_N];
  };
  __shared__ TreeRel rel_lds;
  auto& anc_lds = rel_lds.anc;
  auto& end_lds = rel_lds.end;
  __shared__ int pg_lds[kMaxSplitPages];
  // Row r of a K tile keeps its 16-byte chunk c at position c ^ swz(r), row r of a token-row V tile at
  // c ^ swzv_rows(r).  The XOR patterns were chosen with the LDS bank-conflict counter: they leave the K
  // operand reads (rows kmap(j, 0..15), see below) and the transposing V reads without conflicts.
  auto swz = [](int r) -> int {
    if (VT) return D == 128 ? ((r & 3) | ((r >> 1) & 12)) : (((r >> 1) & 1) | ((r >> 2) & 6));
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
  };
  auto swzv_rows = [](int r) -> int { return D == 128 ? ((2 * r) & 15) : ((r >> 1) & 7); };

  // ---- which (row group, split, KV head, sequence): row groups of one KV range share an XCD ----
  const int RG = p.row_groups;
  const int n_units = p.batch * p.Hkv * p.max_splits;
  const int wg = blockIdx.x;
  const int rg = (wg >> 3) % RG;
  const int unit = ((wg >> 3) / RG) * 8 + (wg & 7);
  if (unit >= n_units) return;
  const int split = unit % p.max_splits;
  const int kvh = (unit / p.max_splits) % p.Hkv;
  const int b = unit / (p.max_splits * p.Hkv);

  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  int L = p.ctx_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int keys = L + N;
  const int n_tiles = (keys + kTile - 1) / kTile;
  const int t_begin = split * p.split_tiles;
  int t_end = min(n_tiles, t_begin + p.split_tiles);
  const int G = p.G;
  const int rows = N * G;
  const int row0 = rg * ROWS_WG;
  if (t_begin >= t_end || row0 >= rows) return;
  // an ancestor's index is below its descendant's, so tree slots past the work-group's last node are
  // masked for all of its rows: the split ends there (at least one tile stays, so that every split
  // the merge reads writes its partial; a fully masked tile leaves the neutral one)
  {
    const int last_node = (min(row0 + ROWS_WG, rows) - 1) / G;
    const int t_need = (L + last_node + 1 + kTile - 1) / kTile;
    t_end = max(t_begin + 1, min(t_end, t_need));
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps load descriptors scalar
  const bool loader = !SW || wave == 1 || wave == 2;            // this wave loads tiles
  const int lwave = SW ? (wave == 2 ? 1 : 0) : wave;            // its place among the loading waves
  const int lm = lane & 15, lg = lane >> 4;
  const int pshift = p.page_shift;

  // ---- the split's page ids (invalid or missing pages become -1) ----
  const int pg_first = (t_begin * kTile) >> pshift;
  const int pg_count = (((keys < t_end * kTile ? keys : t_end * kTile) - 1) >> pshift) - pg_first + 1;
  {
    const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
    for (int i = tid; i < pg_count; i += NT) {
      const int pg = bt_row[pg_first + i];
      pg_lds[i] = (pg >= 0 && pg < p.num_pages) ? pg : -1;
    }
  }

  // ---- ancestor-or-self bit masks of the tree nodes (only the split holding the tree slots) ----
  const bool has_tree = t_end * kTile > L;
  if (PRE && has_tree) {
    // a 4-wave work-group serves <= 128 rows, hence <= 128 nodes (< END_N)
    for (int i = tid; i < N && i < END_N; i += NT) {
      int e = p.subtree_end[n0 + i];
      end_lds[i] = e <= i ? i + 1 : (e > N ? N : e);
    }
  } else if (has_tree) {
    for (int i = tid; i < N && i < ANC_N; i += NT) {
      uint64_t m[ANC_W];
#pragma unroll
      for (int w = 0; w < ANC_W; ++w) m[w] = 0;
      int j = i;
      for (int step = 0; step < N && j >= 0 && j < ANC_N; ++step) {
#pragma unroll
        for (int w = 0; w < ANC_W; ++w) m[w] |= (j >> 6) == w ? 1ull << (j & 63) : 0ull;   // no dynamic index
        const int pj = p.parents[n0 + j];
        if (pj >= j) break;                       // not topological: stop the walk
        j = pj;
      }
#pragma unroll
      for (int w = 0; w < ANC_W; ++w) anc_lds[i][w] = m[w];
    }
  }

  // ---- this lane's query rows (row = node * G + head-in-group) and their Q fragments ----
  int node_r[RB];
  bool valid_r[RB];
  bf16x8 qreg[RB][KS];
  const bool wave_active = row0 + wave * RB * 16 < rows;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + (wave * RB + rb) * 16 + lm;
    valid_r[rb] = row < rows;
    node_r[rb] = valid_r[rb] ? row / G : 0;
    const int head = valid_r[rb] ? kvh * G + row % G : 0;
    const uint16_t* qp = p.q + ((int64_t)(n0 + node_r[rb]) * p.Hq + head) * D + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid_r[rb]) v = *reinterpret_cast<const u32x4*>(qp + 32 * kk);
      qreg[rb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();                                  // page ids visible before the first tile load

  // ---- tile loads: straight from HBM into LDS, 16 bytes per lane, lanes in LDS order ----
  // Load i of loading wave lwave fills LDS chunks [(lwave * LOADS + i) * 64, +64) of the K tile (first
  // half of the loads) or of the V tile: 64 / CPR consecutive keys of one page (page sizes >= 8), so each load is a
  // buffer load through a scalar descriptor of that page and each lane only adds a fixed offset (its
  // key's row and its swizzled source chunk).  The descriptor's byte range ends at the sequence's last
  // slot in the page, so slots past the sequence (and pages with an invalid id: empty range) read zeros.
  const uint16_t* kbase = p.k + (int64_t)kvh * p.head_stride;
  const uint16_t* vbase = p.v + (int64_t)kvh * p.head_stride;
  const uint32_t tstride = (uint32_t)p.token_stride;
  const int pmask = (1 << pshift) - 1;
  // Dim-major V tile in LDS: one block per page of the tile ([page in tile][dim][pe keys], pe = page size
  // capped at 64); a dim's row of pe keys holds pe / 8 chunks of 16 bytes, chunk c at c ^ vswz(dim).  An
  // operand read takes one chunk of 16 consecutive dims; this XOR pattern keeps it free of bank conflicts
  // for every pe (checked with the LDS bank-conflict counter).
  const int lpe = pshift < 6 ? pshift : 6;          // log2 pe
  const int lcr = lpe - 3;                          // log2 chunks per row
  auto vswz = [&](int d) -> int { return (d >> 1) & ((1 << lcr) - 1); };
  const int v_ipp_l = lpe + (D == 128 ? 7 : 6) - 9; // log2 of 1 KiB loads per page block
  uint32_t ld_voff[LOADS];                          // bytes from the page (or, for pages > 64 slots, tile) start
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int blk = lwave * LOADS + i;
    if (VT && blk >= KB) {
      // V load u = blk - KB fills 1 KiB of page block u >> v_ipp_l: dims from (u mod loads per page) * 512 / pe
      const int u = blk - KB;
      const int dim = ((u & ((1 << v_ipp_l) - 1)) << (9 - lpe)) + (lane >> lcr);
      const int c = (lane & ((1 << lcr) - 1)) ^ vswz(dim);
      ld_voff[i] = (uint32_t)((dim << pshift) + 8 * c) * 2u;
    } else {
      const int q = (blk * 64 + lane) % (kTile * CPR);
      const int kt = q / CPR;
      const int src = ((q % CPR) ^ (blk >= KB ? swzv_rows(kt) : swz(kt))) * 8;
      const int row = pshift > 6 ? kt : (kt & pmask);
      ld_voff[i] = ((uint32_t)row * tstride + (uint32_t)src) * 2u;
    }
  }
  // A wave's loads are all K or all V (KB is a multiple of LOADS), LOADS * 64 / CPR consecutive keys, in
  // groups of 16 keys (GL loads) that never straddle a page when pages hold >= 16 tokens.  Then one page-id
  // lookup and one buffer descriptor serve each group: one per tile step for an 8-wave work-group at
  // D = 128, two for a 4-wave one.
  constexpr int KPL = 64 / CPR;                     // keys per load
  constexpr int GL = 16 / KPL < LOADS ? 16 / KPL : LOADS;   // loads per 16-key group
  static_assert(KB % LOADS == 0 && LOADS % GL == 0, "a wave's loads must be all K or all V, in whole groups");
  const bool wave_is_v = lwave * LOADS >= KB;
  const bool grouped = !(VT && wave_is_v) && pshift >= 4;
  auto issue_tile = [&](int t, uint16_t (*kv)[TILE_EL]) __attribute__((always_inline)) {
    const int key0 = t * kTile;
    if (grouped) {
      int pgs[LOADS / GL];
#pragma unroll
      for (int g = 0; g < LOADS / GL; ++g) {      // page ids of the groups (LDS reads issued together)
        const int key_w = key0 + (((lwave * LOADS + g * GL) * 64) % (kTile * CPR)) / CPR;
        int pi = (key_w >> pshift) - pg_first;
        pi = pi < pg_count ? pi : pg_count - 1;
        pgs[g] = pg_lds[pi];
      }
#pragma unroll
      for (int g = 0; g < LOADS / GL; ++g) {
        const int key_w = key0 + (((lwave * LOADS + g * GL) * 64) % (kTile * CPR)) / CPR;
        const int pg = __builtin_amdgcn_readfirstlane(pgs[g]);
        const int first_key = pshift > 6 ? key0 : (key_w & ~pmask);
        const int span = pshift > 6 ? kTile : (1 << pshift);
        int valid = keys - first_key;
        valid = valid < 0 ? 0 : (valid > span ? span : valid);
        if (pg < 0) valid = 0;
        const uint32_t row0 = pshift > 6 ? (uint32_t)(key0 & pmask) * tstride : 0u;
        const uint16_t* b = (wave_is_v ? vbase : kbase) + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride + row0;
#pragma unroll
        for (int i = g * GL; i < (g + 1) * GL; ++i)
          buffer_load_lds16(b, (uint32_t)valid * tstride * 2u, &kv[wave_is_v ? 1 : 0][((lwave * LOADS + i) % KB) * 512],
                            ld_voff[i]);
      }
      return;
    }
    // every load reads one page: look all page ids up first (LDS reads issued together, one wait)
    int pgv[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = lwave * LOADS + i;
      const int key_w = (VT && blk >= KB) ? key0 + (((blk - KB) >> v_ipp_l) << lpe) : key0 + ((blk * 64) % (kTile * CPR)) / CPR;
      int pi = (key_w >> pshift) - pg_first;
      pi = pi < pg_count ? pi : pg_count - 1;
      pgv[i] = pg_lds[pi];
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = lwave * LOADS + i;
      const bool is_v = blk >= KB;
      uint16_t* dst = &kv[is_v ? 1 : 0][(blk % KB) * 512];
      const int pg = __builtin_amdgcn_readfirstlane(pgv[i]);
      if (VT && is_v) {
        // a descriptor over the page's whole dim-major block; slots past the sequence are not a byte
        // prefix of it, so they are cleared in the V fragments instead; an invalid page id reads zeros
        const uint32_t in_page = pshift > 6 ? (uint32_t)(key0 & pmask) * 2u : 0u;
        const uint16_t* b = vbase + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride;
        buffer_load_lds16(b, pg < 0 ? 0u : ((uint32_t)D << (pshift + 1)), dst, ld_voff[i] + in_page);
        continue;
      }
      // the descriptor starts at the page (or at the tile's first row inside a page longer than a tile)
      const int key_w = key0 + ((blk * 64) % (kTile * CPR)) / CPR;
      const int first_key = pshift > 6 ? key0 : (key_w & ~pmask);
      const int span = pshift > 6 ? kTile : (1 << pshift);
      int valid = keys - first_key;
      valid = valid < 0 ? 0 : (valid > span ? span : valid);
      if (pg < 0) valid = 0;
      const uint32_t row0 = pshift > 6 ? (uint32_t)(key0 & pmask) * tstride : 0u;
      const uint16_t* b = (is_v ? vbase : kbase) + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride + row0;
      buffer_load_lds16(b, (uint32_t)valid * tstride * 2u, dst, ld_voff[i]);
    }
  };

  // per-lane LDS element offsets of the MFMA operand reads.
  // Row r of S^T block j holds tile key kmap(j, r).  With dim-major V the keys are ordered so that the
  // P fragment of 32-key half h2 holds keys 32 h2 + 8 lg + e in element e, the order in which a 16-byte
  // row read of the V^T tile delivers them; with token-row V the order follows the transposing reads.
  auto kmap = [](int j, int r) -> int { return VT ? 32 * (j >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3) : 16 * j + r; };
  // tile key of element e of this lane's P fragment for half h2
  auto pkey = [&](int h2, int e) -> int { return VT ? 32 * h2 + 8 * lg + e : 32 * h2 + (e < 4 ? 4 * lg + e : 12 + 4 * lg + e); };
  // K rows kmap(j, lm), chunk 4kk + lg.  Blocks j and j + 2 are 32 keys apart with the same swizzle, and
  // with token-row V all four blocks share it, so only the offsets of blocks 0 and 1 are kept.
  int k_off[VT ? 2 : 1][KS];
#pragma unroll
  for (int jj = 0; jj < (VT ? 2 : 1); ++jj)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int r = kmap(jj, lm);
      k_off[jj][kk] = r * D + 8 * ((4 * kk + lg) ^ swz(r));
    }
  auto kaddr = [&](int j, int kk) -> int {
    return VT ? k_off[j & 1][kk] + (j >> 1) * 32 * D : k_off[0][kk] + 16 * j * D;
  };
  // V^T fragment reads.  Token-row V: transposing reads, lane (lg, lm) points at key 32*h2 + 4*lg + lm/4
  // (+16), dims 16*nb + 4*(lm%4).  Dim-major V: a 16-byte read of dim 16*nb + lm, keys 32*h2 + 8*lg + 0..7.
  int v_row[2], v_swz[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    if (VT) {
      const int key = 32 * h2 + 8 * lg;             // first of the lane's 8 keys
      v_row[h2] = ((key >> lpe) << (lpe + (D == 128 ? 7 : 6))) + (lm << lpe) +
                  8 * (((key & ((1 << lpe) - 1)) >> 3) ^ vswz(lm));
      v_swz[h2] = 0;
    } else {
      const int key = 32 * h2 + 4 * lg + (lm >> 2);
      v_row[h2] = key * D + 4 * (lm & 1);
      v_swz[h2] = swzv_rows(key);
    }
  }

  // constant A fragments for the chunk sums (bf16 1.0 = 0x3F80): all slots, or the slots of one 16-key block
  const bf16x8 ones = bf16_splat8(0x3F803F80u, 0x3F803F80u);
  const bf16x8 ones_lo = VT ? (lg < 2 ? ones : bf16_splat8(0u, 0u)) : bf16_splat8(0x3F803F80u, 0u);
  const bf16x8 ones_hi = VT ? (lg < 2 ? bf16_splat8(0u, 0u) : ones) : bf16_splat8(0u, 0x3F803F80u);

  f32x4 o[RB][NB];
  float m_r[RB], l_r[RB], cacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_r[rb] = kNegBig;
    l_r[rb] = 0.f;
    cacc[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale_log2;
  const int cs = p.chunk_size;
  // chunk of a context slot: a shift for power-of-two chunk sizes (no per-tile scalar division)
  const int cs_shift = (cs > 0 && (cs & (cs - 1)) == 0) ? __builtin_ctz((unsigned)cs) : -1;
  auto chunk_of = [&](int key) __attribute__((always_inline)) -> int { return cs_shift >= 0 ? key >> cs_shift : key / cs; };
  // chunk partials (layout in AttnParams): a wave's 32 rows of a chunk are contiguous, in lines that
  // only this work-group writes
  const int row_stride_chunk = p.chunk_cs;
  // chunk-partial rows: the lanes of group lg store row block lg (RB consecutive 16-row blocks, one store)
  const int st_rb = lg % RB;
  const int st_row = row0 + (wave * RB + st_rb) * 16 + lm;
  const bool st_ok = lg < RB && st_row < rows;
  float* cbase = p.chunk_lse2 + (int64_t)b * p.max_chunks * p.Hkv * p.max_nodes * G + (int64_t)kvh * p.chunk_hs +
                 (st_ok ? st_row : 0);

  // S (scores of the current tile) and P (its bf16 probabilities) live across the compute stages
  f32x4 s[RB][4];
  bf16x8 pb[RB][2];

  // stage 1: S^T = K . Q^T for tile t from the K tile at kt
  auto stage_qk = [&](int t, const uint16_t* kt) __attribute__((always_inline)) {
    const int key0 = t * kTile;
    (void)key0;
      // S^T[key][row] = K . Q^T
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments double-buffered across k-steps: the reads for step kk+1 are in flight while the
    // MFMAs of step kk run
    bf16x8 kf[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kf[0][j] = *reinterpret_cast<const bf16x8*>(kt + kaddr(j, 0));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) kf[(kk + 1) & 1][j] = *reinterpret_cast<const bf16x8*>(kt + kaddr(j, kk + 1));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk & 1][j], qreg[rb][kk], s[rb][j], 0, 0, 0);
    }
  };
  // stage 2a: in a tile that reaches past the context, mask the scores of slots a row may not see
  float mt[RB];
  auto stage_mask = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * kTile;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + kmap(j, 4 * lg + i);
            bool vis = key < L;
            if (!vis && key < keys && valid_r[rb]) {
              const int tj = key - L;           // < N (<= ANC_N, or <= END_N in preorder), and node_r < N
              if constexpr (PRE != 0)
                vis = tj <= node_r[rb] && node_r[rb] < end_lds[tj];
              else
                vis = (anc_lds[node_r[rb]][(tj >> 6) & (ANC_W - 1)] >> (tj & 63)) & 1ull;
            }
            if (!vis) s[rb][j][i] = -INFINITY;
          }
      }
    }
  };
  // stage 2b (only when stage 2c found a probability above 2^kRescale): the rows' tile maxima; true
  // (wave-uniform) when some row's running max must move (lazy rescaling: only when a tile's max exceeds
  // it by more than 2^kRescale)
  auto stage_max = [&]() __attribute__((always_inline)) -> bool {
    bool resc = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3]));
#pragma unroll
      for (int j = 1; j < 4; ++j)
        mx = fmaxf(fmaxf(mx, fmaxf(s[rb][j][0], s[rb][j][1])), fmaxf(s[rb][j][2], s[rb][j][3]));
      mt[rb] = max4g(mx) * c2;
      resc |= mt[rb] > m_r[rb] + kRescale;
    }
    return __builtin_amdgcn_ballot_w64(resc) != 0;
  };
  // stage 2b': move the running max of the rows that need it, rescaling O, l and the chunk accumulator
  auto stage_rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mnew = mt[rb] > m_r[rb] + kRescale ? mt[rb] : m_r[rb];
      const float alpha = __builtin_amdgcn_exp2f(m_r[rb] - mnew);
      l_r[rb] *= alpha;
      cacc[rb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[rb][nb] *= alpha;
      m_r[rb] = mnew;
    }
  };
  // stage 2c: probabilities against the running max (bf16 P fragments; esum: this lane's fp32 sum of them)
  float esum[RB];
  auto stage_exp = [&](bf16x8 (&pout)[RB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mneg = -m_r[rb];
      float e0 = 0.f, e1 = 0.f;                 // fp32 row sums of this lane's 16 probabilities
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = __builtin_amdgcn_exp2f(fmaf(s[rb][2 * h2][i], c2, mneg));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(s[rb][2 * h2 + 1][i], c2, mneg));
          e0 += x0;
          e1 += x1;
          v[i] = (__bf16)x0;
          v[4 + i] = (__bf16)x1;
        }
        pout[rb][h2] = v;
      }
      esum[rb] = e0 + e1;
    }
  };
  // stage 3a: O^T[dim][row] += V^T . P^T for the tile at key0 (V^T fragments from vt, two dim blocks
  // ahead of their MFMAs)
  auto pv_mfma = [&](int key0, const uint16_t* vt, const bf16x8 (&pin)[RB][2]) __attribute__((always_inline)) {
    (void)key0;
    auto vfrag = [&](int nb, int h2) __attribute__((always_inline)) -> bf16x8 {
      if (VT) return *reinterpret_cast<const bf16x8*>(vt + (nb << (lpe + 4)) + v_row[h2]);
      // token-row V: transposing reads
      typedef short i16x4 __attribute__((ext_vector_type(4)));
      const int c = 2 * nb + ((lm & 3) >> 1);
      const int off = v_row[h2] + 8 * (c ^ v_swz[h2]);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off + 16 * D));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 av = {lo2[0], lo2[1], hi2[0], hi2[1]};
      return __builtin_bit_cast(bf16x8, av);
    };
    // order (h2, nb, rb): the two MFMAs accumulating into one O fragment are 2 * NB apart, so no MFMA
    // waits on the previous one's result
    constexpr int NV = 2 * NB;
    constexpr int VPF = 2;                          // fragments read ahead of their MFMAs
    bf16x8 vf[8];
#pragma unroll
    for (int x = 0; x < VPF; ++x) vf[x] = vfrag(x % NB, x / NB);
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      if (x + VPF < NV) vf[(x + VPF) & 7] = vfrag((x + VPF) % NB, (x + VPF) / NB);
      const int nb = x % NB, h2 = x / NB;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[x & 7], pin[rb][h2], o[rb][nb], 0, 0, 0);
    }
  };
  // stage 3b: chunk sums of P (bf16 values, fp32 sums) on MFMA against constant ones: every output slot
  // of the fragment holds the row's sum, so no cross-lane reduction is needed.  edge: the tile holds
  // slots >= L, whose ones are cleared (chunk sums cover context keys only; P stays untouched).
  auto chunk_mfma = [&](int key0, const bf16x8 (&pin)[RB][2], bool edge, float (&csum)[RB][NS]) __attribute__((always_inline)) {
    bf16x8 a_all[2] = {ones, ones}, a_lo[2] = {ones_lo, ones_lo}, a_hi[2] = {ones_hi, ones_hi};
    if (edge) {
      // nv comes out of an opaque (volatile) statement, so the compares and selects below cannot be hoisted
      // out of this branch: hoisted, they would run on every tile (16 per half), not only in the edge tile
      int nv = L - key0;                              // context slots left in this tile
      asm volatile("" : "+s"(nv));
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (pkey(h2, e) >= nv) {
            a_all[h2][e] = (__bf16)0.0f;
            a_lo[h2][e] = (__bf16)0.0f;
            a_hi[h2][e] = (__bf16)0.0f;
          }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (CM == 0) {
        f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_all[0], pin[rb][0], z, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_all[1], pin[rb][1], c, 0, 0, 0);
        csum[rb][0] = c[0];
      } else if (CM == 1) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          csum[rb][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_all[h2], pin[rb][h2], z, 0, 0, 0)[0];
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          csum[rb][2 * h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[h2], pin[rb][h2], z, 0, 0, 0)[0];
          csum[rb][2 * h2 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[h2], pin[rb][h2], z, 0, 0, 0)[0];
        }
      }
    }
  };
  // Chunk partials computed in one step are stored at the start of the next one, after that step's tile
  // loads are issued: the wait that closes a step (for the next tile) then does not also wait for a store
  // issued just before it, which would add a store round trip to every tile.  pend_c: the first chunk of
  // the pending values, -1 when none (wave-uniform).  16-slot chunks (four values per tile) store at once:
  // holding four values more would spill registers.
  constexpr bool DEFER = CM != 2;
  float pend_v[NS];
  int pend_c = -1;
  // With chunks of >= 64 slots (one value per row and chunk end) and token-row V, the values collect in
  // LDS instead: a store issued inside a step would be waited for by the step's closing wait, and with HBM
  // busy with the KV stream a store round trip is long.  The LDS ring holds kRingFloats values,
  // [chunk end][row - row0] with RS rows per chunk end (the work-group holds every row of its KV head:
  // RS <= 128), i.e. in the layout's order of a chunk's rows.  When it is full, every thread of the
  // work-group writes it out after a step's closing barrier, 16 bytes per store where the rows allow, and
  // a second barrier keeps the next appends behind those reads; the stores land during the next step.
  // The rest goes out after the split.
  constexpr bool RING = CM == 0 && VT == 0 && W == 4;
  __shared__ __attribute__((aligned(16))) float cring[RING ? kRingFloats : 4];
  const int RS = p.max_nodes * G;                   // a chunk's rows of one KV head in the layout
  const int ring_cap = RING ? kRingFloats / RS : 0; // chunk ends the ring holds (>= 16)
  int ring_n = 0, ring_c0 = 0;                      // chunk ends in the ring, the first one's chunk
  float* const gbase = p.chunk_lse2 + (int64_t)b * p.max_chunks * p.Hkv * p.max_nodes * G + (int64_t)kvh * p.chunk_hs + row0;
  // (all threads) the ring's ring_n chunk ends -> chunk partials; rows past the sequence's own are not
  // written
  auto ring_flush = [&]() __attribute__((always_inline)) {
    const float* src = cring;
    const int n = ring_n * RS, nr = rows - row0;
    const int ft = SW ? lane : tid, fn = SW ? 64 : NT;   // the writing threads: the store wave, or all
    if ((RS & 3) == 0 && (nr & 3) == 0) {
      for (int i = 4 * ft; i < n; i += 4 * fn) {
        const int j = i / RS, r = i - j * RS;
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
        if (r < nr) *reinterpret_cast<f32x4*>(gbase + (int64_t)(ring_c0 + j) * row_stride_chunk + r) = v;
      }
    } else {
      for (int i = ft; i < n; i += fn) {
        const int j = i / RS, r = i - j * RS;
        if (r < nr) gbase[(int64_t)(ring_c0 + j) * row_stride_chunk + r] = src[i];
      }
    }
    ring_n = 0;
  };
  // the chunk that tile t closes (its last context tile), or -1
  auto close_of = [&](int t) __attribute__((always_inline)) -> int {
    const int key0 = t * kTile;
    if (cs <= 0 || key0 >= L) return -1;
    const int c = chunk_of(key0);
    return key0 + kTile >= min((c + 1) * cs, L) ? c : -1;
  };
  auto flush_chunks = [&]() __attribute__((always_inline)) {
    if (pend_c >= 0) {
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const int c = pend_c + q;
        if (st_ok && (CM == 0 || c * cs < L)) cbase[(int64_t)c * row_stride_chunk] = pend_v[q];
      }
      pend_c = -1;
    }
  };
  // stage 3c: per-chunk log2-sum-exp partials against the running max (one 128-byte store per chunk and
  // wave, deferred as above); with 64-slot (or longer) chunks the tile's sum is accumulated until the
  // chunk ends
  auto chunk_store = [&](int key0, const float (&csum)[RB][NS]) __attribute__((always_inline)) {
    if (CM == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) cacc[rb] += csum[rb][0];
      const int c = chunk_of(key0);
      const int cend = min((c + 1) * cs, L);
      if (key0 + kTile >= cend) {
        float v = m_r[0] + __builtin_amdgcn_logf(cacc[0]);
#pragma unroll
        for (int rb = 1; rb < RB; ++rb)
          if (st_rb == rb) v = m_r[rb] + __builtin_amdgcn_logf(cacc[rb]);
        if constexpr (RING) {
          // (the step's end counts the chunk end, in every wave)
          if (st_ok) cring[ring_n * RS + (st_row - row0)] = v;
        } else {
          pend_v[0] = v;
          pend_c = c;
          if (!DEFER) flush_chunks();
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) cacc[rb] = 0.f;
      }
    } else {
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        float v = m_r[0] + __builtin_amdgcn_logf(csum[0][q]);
#pragma unroll
        for (int rb = 1; rb < RB; ++rb)
          if (st_rb == rb) v = m_r[rb] + __builtin_amdgcn_logf(csum[rb][q]);
        pend_v[q] = v;
      }
      pend_c = chunk_of(key0);
      if (!DEFER) flush_chunks();
    }
  };
  // stage 3: P.V and the chunk partials of tile t, any tile
  auto stage_pv = [&](int t, const uint16_t* vt, const bf16x8 (&pin)[RB][2]) __attribute__((always_inline)) {
    const int key0 = t * kTile;
    pv_mfma(key0, vt, pin);
    if (cs > 0 && key0 < L) {
      float csum[RB][NS];
      chunk_mfma(key0, pin, key0 + kTile > L, csum);
      chunk_store(key0, csum);
    }
  };

  // one barrier per tile: tile t+1 loads straight into the other buffer while tile t is computed
  if (loader) issue_tile(t_begin, kv_a);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto step = [&](int t, uint16_t (*cur)[TILE_EL], uint16_t (*nxt)[TILE_EL]) __attribute__((always_inline)) {
    if (loader && t + 1 < t_end) issue_tile(t + 1, nxt);
    flush_chunks();
    if (VT && t * kTile + kTile > keys) {
      // the sequence's last tile: its dim-major V slots past the sequence hold whatever the page held
      // (they are not a byte prefix that the load's range check could clear), so they are zeroed in LDS
      // before any wave multiplies them by P = 0
      const int key0 = t * kTile;
      for (int i = tid; i < D * kTile; i += NT) {
        const int dim = i >> 6, key = i & 63;
        if (key0 + key >= keys)
          cur[1][((key >> lpe) << (lpe + (D == 128 ? 7 : 6))) + (dim << lpe) +
                 8 * (((key & ((1 << lpe) - 1)) >> 3) ^ vswz(dim)) + (key & 7)] = 0;
      }
      __syncthreads();
    }
    if (wave_active) {
      stage_qk(t, cur[0]);
      if (__builtin_expect(t * kTile + kTile > L, 0)) stage_mask(t);
      // The exps run against the running max with no tile max first.  A probability above 2^kRescale
      // makes its lane's sum exceed 2^kRescale (on a split's first tile, where the max is still -1e30,
      // every sum is infinite); only then are the tile maxima taken, the running max moved and the exps
      // redone.  That is the decision the tile max would give (they can differ only for a probability
      // that rounds to exactly 2^kRescale, where either is valid: the headroom only bounds how large a
      // probability may grow), on a handful of tiles per split, and it saves the max reduction and its
      // cross-lane steps on all the others.
      stage_exp(pb);
      bool big = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) big |= esum[rb] > 0x1p8f;
      static_assert(kRescale == 8.0f, "the sum test above is 2^kRescale");
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(big) != 0, 0)) {
        if (stage_max()) stage_rescale();
        stage_exp(pb);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l_r[rb] += esum[rb];
      stage_pv(t, cur[1], pb);
    }
    // this thread's loads of the next tile landed (the store wave has none, and does not wait for its stores)
    if (!SW || wave != 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (RING) {
      const int c = close_of(t);
      if (c >= 0) {
        ring_c0 = ring_n == 0 ? c : ring_c0;
        ++ring_n;
      }
      // the barriers wait for LDS only (a work-group fence would also wait for the ring's stores); after
      // the first the step's chunk ends are in the ring, and a full ring goes out, to land during the
      // next step
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (ring_n == ring_cap) {
        if (!SW || wave == 3) ring_flush();
        ring_n = 0;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    } else {
      __syncthreads();
    }
  };
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, kv_a, kv_b);
    if (t + 1 < t_end) step(t + 1, kv_b, kv_a);
  }

  flush_chunks();
  if (RING && ring_n > 0 && (!SW || wave == 3)) ring_flush();
  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_r[rb];                              // per-lane partial sums -> the row's sum
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_r[rb] = l;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!valid_r[rb]) continue;
    const int row = row0 + (wave * RB + rb) * 16 + lm;
    const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.rows_pad + row;
    if (lg == 0) {
      p.part_ml[base * 2 + 0] = m_r[rb];
      p.part_ml[base * 2 + 1] = l_r[rb];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4*>(&p.part_o[base * D + 16 * nb + 4 * lg]) = o[rb][nb];
  }
}

// LSE merge of the split partials: one wave per (node, query head) row, or (SPLIT4, for calls with few
// rows) one work-group per row whose four waves take a quarter of the splits each and combine through
// LDS, so that a few rows with many splits still spread over the CUs.  A split's D partial-output
// values are read as D/4 16-byte pieces, so one wave-wide load covers 64/(D/4) splits and a lane keeps
// up to kMergeLoads of them in flight: a row's splits arrive in a few round trips even when the rows are
// few (a chain's 160 rows at 128K context hold ~60 splits each), which is what bounds this kernel there.
constexpr int kMergeLoads = 8;
template <int D, bool SPLIT4>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int F = D / 4;                        // lanes per split, four dims each
  constexpr int P = 64 / F;                       // splits per wave-wide load
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rid = SPLIT4 ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + wave;   // (SPLIT4: uniform
                                                                                        // in the work-group)
  const int per_seq = p.max_nodes * p.Hq;
  const int b = (int)(rid / per_seq);
  if (b >= p.batch) return;
  const int rem = (int)(rid % per_seq);
  const int node = rem / p.Hq, head = rem % p.Hq;
  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  if (node >= N) return;
  int L = p.ctx_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int n_tiles = (L + N + kTile - 1) / kTile;
  const int nsp = (n_tiles + p.split_tiles - 1) / p.split_tiles;
  const int kvh = head / p.G;
  const int row = node * p.G + head % p.G;
  const int64_t base0 = ((int64_t)b * p.Hkv + kvh) * p.max_splits * p.rows_pad + row;
  const int sub = lane / F, d4 = lane % F;        // this lane's split within a load, and its four dims
  int s_lo = 0, s_hi = nsp;                       // this wave's splits
  if (SPLIT4) {
    const int q = (nsp + 3) / 4;
    s_lo = min(nsp, wave * q);
    s_hi = min(nsp, s_lo + q);
  }

  // every lane reads the (max, sum) of up to 64 splits at once; then per-split weights by shuffle
  float M = -INFINITY;
  for (int s = s_lo + lane; s < s_hi; s += 64) M = fmaxf(M, p.part_ml[(base0 + (int64_t)s * p.rows_pad) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float lsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_lo; s0 < s_hi; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f, lw = 0.f;
    if (s < s_hi) {
      const int64_t bs = base0 + (int64_t)s * p.rows_pad;
      w = __builtin_amdgcn_exp2f(p.part_ml[bs * 2] - M);
      lw = w * p.part_ml[bs * 2 + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
    lsum += lw;
    const int cnt = min(64, s_hi - s0);
    for (int i = 0; i < cnt; i += P * kMergeLoads) {
      f32x4 x[kMergeLoads];
      float wv[kMergeLoads];
#pragma unroll
      for (int u = 0; u < kMergeLoads; ++u) {
        const int j = i + u * P + sub;            // the split (within this block of 64) of load u
        wv[u] = __shfl(w, j & 63);
        wv[u] = j < cnt ? wv[u] : 0.f;
        x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < cnt)
          x[u] = *reinterpret_cast<const f32x4*>(&p.part_o[(base0 + (int64_t)(s0 + j) * p.rows_pad) * D + 4 * d4]);
      }
#pragma unroll
      for (int u = 0; u < kMergeLoads; ++u) acc += wv[u] * x[u];
    }
  }
  // the P lanes that hold the same four dims of different splits
#pragma unroll
  for (int off = F; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (SPLIT4) {
    // the four waves' (max, sum, O) against the largest max (a wave without splits has max -inf and
    // weight 0)
    __shared__ float m_s[4], l_s[4];
    __shared__ f32x4 a_s[4][F];
    if (lane == 0) {
      m_s[wave] = M;
      l_s[wave] = lsum;
    }
    if (sub == 0) a_s[wave][d4] = acc;
    __syncthreads();
    if (wave != 0) return;
    const float Mt = fmaxf(fmaxf(m_s[0], m_s[1]), fmaxf(m_s[2], m_s[3]));
    lsum = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = m_s[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_s[w] - Mt);
      lsum += sc * l_s[w];
      acc += sc * a_s[w][d4];
    }
    M = Mt;
  }
  const float inv = 1.0f / lsum;
  if (sub == 0) {
    uint16_t* op = p.out + ((int64_t)(n0 + node) * p.Hq + head) * D + 4 * d4;
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
  }
  if (lane == 0) {
    const float l2 = M + __builtin_amdgcn_logf(lsum);
    p.lse2[(int64_t)b * per_seq + (int64_t)kvh * p.max_nodes * p.G + row] = l2;   // [b][kvh][node * G + g]
    if (p.lse) p.lse[(int64_t)(n0 + node) * p.Hq + head] = l2 * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------------------------------
// Software-pipelined variant for wide trees: 8 waves of 32 query rows (256 rows per work-group),
// head_dim 128, V in token rows, chunk partials per 64-slot tile (or none).
//
// The per-tile work of tree_attn_kernel runs in phases: the QK^T MFMAs, then the softmax on the VALU,
// then the P.V MFMAs.  Both waves that share a SIMD reach the same phase at the same time (one barrier
// per tile), so the exps never run beside matrix work.  On gfx950 a wave's independent VALU
// instructions issue in the shadow of its MFMAs: at up to about two VALU instructions per 16x16x32
// MFMA they cost nearly nothing (measured with a throwaway microbenchmark).  This variant splits each
// 64-slot tile into two 32-key halves and runs, per tile t, two blocks of 34 MFMAs each with the exps of
// one half inside:
//   B1: QK^T of (t, half 1) and P.V + chunk sums of (t-1, half 1)  |  exps of (t, half 0)
//   B2: P.V + chunk sums of (t, half 0) and QK^T of (t+1, half 0)  |  exps of (t, half 1)
// so tile t+1's K tile must be in LDS during tile t.  K and V each have four LDS buffers: K(t+3) and
// V(t+2) load while tile t is computed, two steps ahead of their first use.  Scores, probabilities and accumulators keep the registers of
// tree_attn_kernel (the two score halves and the two probability halves are reused in turn).  The
// online softmax, the lazy rescaling and the chunk bookkeeping are those of tree_attn_kernel, taken per
// half-tile.  Every tile runs the same two blocks: a tile that holds tree slots masks its scores between
// them, the split's first tile multiplies a cleared V buffer by zero probabilities, and its last tile
// computes scores it never uses, so that no second copy of the step (and no register spill) is needed.
// On pages of >= 16 slots each wave's four direct-to-LDS loads of the next tiles go out one at a time
// inside block B1, so the vector memory path takes them beside the matrix work.
template <int PRE, int CH, int GRP>
__global__ __launch_bounds__(512, 1) void tree_attn_pipe_kernel(AttnParams p) {
  constexpr int D = 128, W = 8, RB = 2, NT = W * 64, ROWS_WG = W * RB * 16;
  constexpr int KS = D / 32;                    // k-steps of the QK^T product
  constexpr int NB = D / 16;                    // 16-dim output blocks
  constexpr int CPR = D / 8;                    // 16-byte chunks per K/V row
  constexpr int TILE_EL = kTile * D;
  constexpr int LOADS = 2 * kTile * CPR / NT;   // 16-byte loads per thread and tile step (K or V)
  constexpr int KB = kTile * CPR / 64;          // 1 KiB blocks of a K (or V) tile
  constexpr int ANC_N = kMaxNodes, ANC_W = ANC_N / 64, END_N = ANC_N * ANC_W * 2;
  static_assert(KB % LOADS == 0, "a wave's loads must be all K or all V");

  // four K and four V tile buffers, separate arrays so that alias analysis tells the buffers being read
  // from the ones whose direct-to-LDS loads are in flight
  __shared__ __attribute__((aligned(16))) uint16_t ka[TILE_EL], kb[TILE_EL], kc[TILE_EL], kd[TILE_EL];
  __shared__ __attribute__((aligned(16))) uint16_t va[TILE_EL], vb[TILE_EL], vc[TILE_EL], vd[TILE_EL];
  union TreeRel {
    uint64_t anc[ANC_N][ANC_W];
    int end[END_N];
  };
  __shared__ TreeRel rel_lds;
  auto& anc_lds = rel_lds.anc;
  auto& end_lds = rel_lds.end;
  __shared__ int pg_lds[kMaxSplitPages];
  auto swz = [](int r) -> int { return r & 15; };              // K rows
  auto swzv_rows = [](int r) -> int { return (2 * r) & 15; };  // V rows (read transposed)

  // ---- which (row group, split, KV head, sequence): as tree_attn_kernel ----
  const int RG = p.row_groups;
  const int n_units = p.batch * p.Hkv * p.max_splits;
  const int wg = blockIdx.x;
  const int rg = (wg >> 3) % RG;
  const int unit = ((wg >> 3) / RG) * 8 + (wg & 7);
  if (unit >= n_units) return;
  const int split = unit % p.max_splits;
  const int kvh = (unit / p.max_splits) % p.Hkv;
  const int b = unit / (p.max_splits * p.Hkv);
  int n0 = p.node_offsets[b];
  int N = p.node_offsets[b + 1] - n0;
  N = N < 0 ? 0 : (N > p.max_nodes ? p.max_nodes : N);
  n0 = n0 < 0 ? 0 : (n0 > (p.batch - 1) * p.max_nodes ? (p.batch - 1) * p.max_nodes : n0);
  int L = p.ctx_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int keys = L + N;
  const int n_tiles = (keys + kTile - 1) / kTile;
  const int t_begin = split * p.split_tiles;
  int t_end = min(n_tiles, t_begin + p.split_tiles);
  const int G = p.G;
  const int rows = N * G;
  const int row0 = rg * ROWS_WG;
  if (t_begin >= t_end || row0 >= rows) return;
  {
    const int last_node = (min(row0 + ROWS_WG, rows) - 1) / G;
    const int t_need = (L + last_node + 1 + kTile - 1) / kTile;
    t_end = max(t_begin + 1, min(t_end, t_need));
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lm = lane & 15, lg = lane >> 4;
  const int pshift = p.page_shift;

  const int pg_first = (t_begin * kTile) >> pshift;
  const int pg_count = (((keys < t_end * kTile ? keys : t_end * kTile) - 1) >> pshift) - pg_first + 1;
  {
    const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
    for (int i = tid; i < pg_count; i += NT) {
      const int pg = bt_row[pg_first + i];
      pg_lds[i] = (pg >= 0 && pg < p.num_pages) ? pg : -1;
    }
  }
  const bool has_tree = t_end * kTile > L;
  if (PRE && has_tree) {
    for (int i = tid; i < N && i < END_N; i += NT) {
      int e = p.subtree_end[n0 + i];
      end_lds[i] = e <= i ? i + 1 : (e > N ? N : e);
    }
  } else if (has_tree) {
    for (int i = tid; i < N && i < ANC_N; i += NT) {
      uint64_t m[ANC_W];
#pragma unroll
      for (int w = 0; w < ANC_W; ++w) m[w] = 0;
      int j = i;
      for (int step = 0; step < N && j >= 0 && j < ANC_N; ++step) {
#pragma unroll
        for (int w = 0; w < ANC_W; ++w) m[w] |= (j >> 6) == w ? 1ull << (j & 63) : 0ull;
        const int pj = p.parents[n0 + j];
        if (pj >= j) break;
        j = pj;
      }
#pragma unroll
      for (int w = 0; w < ANC_W; ++w) anc_lds[i][w] = m[w];
    }
  }

  // ---- this lane's query rows and their Q fragments ----
  int node_r[RB];
  bool valid_r[RB];
  bf16x8 qreg[RB][KS];
  const bool wave_active = row0 + wave * RB * 16 < rows;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + (wave * RB + rb) * 16 + lm;
    valid_r[rb] = row < rows;
    node_r[rb] = valid_r[rb] ? row / G : 0;
    const int head = valid_r[rb] ? kvh * G + row % G : 0;
    const uint16_t* qp = p.q + ((int64_t)(n0 + node_r[rb]) * p.Hq + head) * D + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid_r[rb]) v = *reinterpret_cast<const u32x4*>(qp + 32 * kk);
      qreg[rb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();                                  // page ids visible before the first tile load

  // ---- tile loads: waves 0..3 load K tiles, waves 4..7 V tiles (16 consecutive keys per wave) ----
  const uint16_t* kbase = p.k + (int64_t)kvh * p.head_stride;
  const uint16_t* vbase = p.v + (int64_t)kvh * p.head_stride;
  const uint32_t tstride = (uint32_t)p.token_stride;
  const int pmask = (1 << pshift) - 1;
  const bool wave_is_v = wave * LOADS >= KB;
  uint32_t ld_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int blk = wave * LOADS + i;
    const int q = (blk * 64 + lane) % (kTile * CPR);
    const int kt = q / CPR;
    const int src = ((q % CPR) ^ (blk >= KB ? swzv_rows(kt) : swz(kt))) * 8;
    const int row = pshift > 6 ? kt : (kt & pmask);
    ld_voff[i] = ((uint32_t)row * tstride + (uint32_t)src) * 2u;
  }
  constexpr int KPL = 64 / CPR;                     // keys per load (4)
  constexpr int GL = 16 / KPL < LOADS ? 16 / KPL : LOADS;
  // GRP: pages of >= 16 slots (a wave's 16 keys of a tile in one page).  A compile-time switch: a
  // run-time test around the loads inside a block is a branch, and the compiler then sinks the block's
  // exps below it, out of the MFMAs' shadow.
  constexpr bool grouped = GRP != 0;
  // this wave's share of tile t (K for waves 0..3, V for waves 4..7) into buf
  auto issue = [&](int t, uint16_t* buf) __attribute__((always_inline)) {
    const int key0 = t * kTile;
    const uint16_t* base = wave_is_v ? vbase : kbase;
    if (grouped) {
      int pgs[LOADS / GL];
#pragma unroll
      for (int g = 0; g < LOADS / GL; ++g) {
        const int key_w = key0 + (((wave * LOADS + g * GL) * 64) % (kTile * CPR)) / CPR;
        int pi = (key_w >> pshift) - pg_first;
        pi = pi < pg_count ? pi : pg_count - 1;
        pgs[g] = pg_lds[pi];
      }
#pragma unroll
      for (int g = 0; g < LOADS / GL; ++g) {
        const int key_w = key0 + (((wave * LOADS + g * GL) * 64) % (kTile * CPR)) / CPR;
        const int pg = __builtin_amdgcn_readfirstlane(pgs[g]);
        const int first_key = pshift > 6 ? key0 : (key_w & ~pmask);
        const int span = pshift > 6 ? kTile : (1 << pshift);
        int valid = keys - first_key;
        valid = valid < 0 ? 0 : (valid > span ? span : valid);
        if (pg < 0) valid = 0;
        const uint32_t rowb = pshift > 6 ? (uint32_t)(key0 & pmask) * tstride : 0u;
        const uint16_t* bp = base + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride + rowb;
#pragma unroll
        for (int i = g * GL; i < (g + 1) * GL; ++i)
          buffer_load_lds16(bp, (uint32_t)valid * tstride * 2u, buf + ((wave * LOADS + i) % KB) * 512, ld_voff[i]);
      }
      return;
    }
    int pgv[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = wave * LOADS + i;
      const int key_w = key0 + ((blk * 64) % (kTile * CPR)) / CPR;
      int pi = (key_w >> pshift) - pg_first;
      pi = pi < pg_count ? pi : pg_count - 1;
      pgv[i] = pg_lds[pi];
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = wave * LOADS + i;
      const int pg = __builtin_amdgcn_readfirstlane(pgv[i]);
      const int key_w = key0 + ((blk * 64) % (kTile * CPR)) / CPR;
      const int first_key = pshift > 6 ? key0 : (key_w & ~pmask);
      const int span = pshift > 6 ? kTile : (1 << pshift);
      int valid = keys - first_key;
      valid = valid < 0 ? 0 : (valid > span ? span : valid);
      if (pg < 0) valid = 0;
      const uint32_t rowb = pshift > 6 ? (uint32_t)(key0 & pmask) * tstride : 0u;
      const uint16_t* bp = base + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride + rowb;
      buffer_load_lds16(bp, (uint32_t)valid * tstride * 2u, buf + (blk % KB) * 512, ld_voff[i]);
    }
  };

  // The grouped path (pages of >= 16 slots: a wave's 16 keys sit in one page) split in two, so that the
  // loads can be spread over a block: the page lookup and the descriptor's base and byte range first
  // (valid = false gives an empty range: the loads then write zeros, into a buffer nobody reads), then
  // one 16-byte direct-to-LDS load at a time.
  constexpr int KEY_W = (((LOADS * 64) % (kTile * CPR)) / CPR);   // keys of a tile per wave (16)
  auto page_of_tile = [&](int t) __attribute__((always_inline)) -> int {   // this wave's page id in tile t
    int pi = ((t * kTile + KEY_W * (wave & 3)) >> pshift) - pg_first;
    pi = pi < pg_count ? pi : pg_count - 1;
    return pg_lds[pi < 0 ? 0 : pi];
  };
  // branch-free (it runs inside an interleaved block): the descriptor covers the tile's slots in the
  // page (pages longer than a tile) or the whole page from its first slot; a tile start is a multiple
  // of kTile, so key0 & pmask is zero for pages of <= kTile slots
  const int fk_mask = pshift > 6 ? ~(kTile - 1) : ~pmask;
  const int span = pshift > 6 ? kTile : (1 << pshift);
  auto plan_grouped = [&](int t, bool valid_tile, int pg_v, const uint16_t*& bp, uint32_t& bytes) __attribute__((always_inline)) {
    const int key0 = t * kTile;
    const int key_w = key0 + (((wave * LOADS) * 64) % (kTile * CPR)) / CPR;
    const int pg = __builtin_amdgcn_readfirstlane(pg_v);
    const int first_key = key_w & fk_mask;
    int valid = min(max(keys - first_key, 0), span);
    valid = (pg < 0 || !valid_tile) ? 0 : valid;
    const uint32_t rowb = (uint32_t)(key0 & pmask) * tstride;
    bp = (wave_is_v ? vbase : kbase) + (uint64_t)(uint32_t)(pg < 0 ? 0 : pg) * (uint32_t)p.page_stride + rowb;
    bytes = (uint32_t)valid * tstride * 2u;
  };
  auto load_one = [&](const uint16_t* bp, uint32_t bytes, uint16_t* buf, int i) __attribute__((always_inline)) {
    buffer_load_lds16(bp, bytes, buf + ((wave * LOADS + i) % KB) * 512, ld_voff[i]);
  };
  static_assert(LOADS / GL == 1, "one page group per wave and tile");

  // ---- operand offsets (as tree_attn_kernel with token-row V) ----
  int k_off[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) k_off[kk] = lm * D + 8 * ((4 * kk + lg) ^ swz(lm));
  // chunk c = 2 nb + b0 of the row at key sits at position c ^ swz: with swz = 2 sh + s0 that is
  // 2 (nb ^ sh) + (b0 ^ s0), so the offset of dim block nb is v_base[h] + (16 sh ^ 16 nb)
  int v_base[2], v_sh16[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int key = 32 * h2 + 4 * lg + (lm >> 2);
    const int sw = swzv_rows(key);
    v_base[h2] = key * D + 4 * (lm & 1) + 8 * (((lm & 3) >> 1) ^ (sw & 1));
    v_sh16[h2] = 16 * (sw >> 1);
  }
  const bf16x8 ones = bf16_splat8(0x3F803F80u, 0x3F803F80u);

  f32x4 o[RB][NB];
  float m_r[RB], l_r[RB], cacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_r[rb] = kNegBig;
    l_r[rb] = 0.f;
    cacc[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale_log2;
  const int cs = p.chunk_size;
  const int cs_shift = (cs > 0 && (cs & (cs - 1)) == 0) ? __builtin_ctz((unsigned)cs) : -1;
  auto chunk_of = [&](int key) __attribute__((always_inline)) -> int { return cs_shift >= 0 ? key >> cs_shift : key / cs; };
  // chunk partials (layout in AttnParams)
  const int row_stride_chunk = p.chunk_cs;
  const int st_rb = lg % RB;
  const int st_row = row0 + (wave * RB + st_rb) * 16 + lm;
  const bool st_ok = lg < RB && st_row < rows;
  float* cbase = p.chunk_lse2 + (int64_t)b * p.max_chunks * p.Hkv * p.max_nodes * G + (int64_t)kvh * p.chunk_hs +
                 (st_ok ? st_row : 0);

  // score halves (keys 0..31 and 32..63 of a tile) and probability halves, reused in turn
  f32x4 sA[RB][2], sB[RB][2];
  bf16x8 pA[RB], pB[RB];
  float eA[RB], eB[RB];                             // this lane's fp32 sums of a half's probabilities
  float csum[RB];

  // S^T half h of the tile in kt: rows of keys 32h .. 32h+31 (blocks j = 2h, 2h+1)
  auto qk_half = [&](const uint16_t* kt, int h, f32x4 (&s)[RB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) s[rb][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      bf16x8 kf[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        kf[jj] = *reinterpret_cast<const bf16x8*>(kt + k_off[kk] + 16 * (2 * h + jj) * D);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[jj], qreg[rb][kk], s[rb][jj], 0, 0, 0);
    }
  };
  // a half-tile's probabilities against the running max (bf16 P fragment, fp32 lane sum)
  auto exps_half = [&](const f32x4 (&s)[RB][2], bf16x8 (&pout)[RB], float (&esum)[RB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mneg = -m_r[rb];
      bf16x8 v;
      float e0 = 0.f, e1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[rb][0][i], c2, mneg));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[rb][1][i], c2, mneg));
        e0 = i == 0 ? x0 : e0 + x0;
        e1 = i == 0 ? x1 : e1 + x1;
        v[i] = (__bf16)x0;
        v[4 + i] = (__bf16)x1;
      }
      pout[rb] = v;
      esum[rb] = e0 + e1;
    }
  };
  // O^T += V^T . P^T for half h of the tile in vt
  auto pv_half = [&](const uint16_t* vt, int h, const bf16x8 (&pin)[RB]) __attribute__((always_inline)) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int off = v_base[h] + (v_sh16[h] ^ (16 * nb));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off + 16 * D));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 av = {lo2[0], lo2[1], hi2[0], hi2[1]};
      const bf16x8 vf = __builtin_bit_cast(bf16x8, av);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pin[rb], o[rb][nb], 0, 0, 0);
    }
  };
  // chunk sums of half h (ones of the context slots of the half: a = all ones inside the context)
  auto chunk_half = [&](const bf16x8 (&pin)[RB], const bf16x8& a) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      csum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pin[rb], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)[0];
  };
  // ones of half h of the tile at key0, cleared at slots >= L (chunk sums cover context slots only)
  auto ones_edge = [&](int key0, int h) -> bf16x8 {
    bf16x8 a = ones;
    int nv = L - key0;
    asm volatile("" : "+s"(nv));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pk = 32 * h + (e < 4 ? 4 * lg + e : 12 + 4 * lg + e);
      if (pk >= nv) a[e] = (__bf16)0.0f;
    }
    return a;
  };
  // tree mask of half h of tile t (keys >= L visible only to their descendants)
  auto mask_half = [&](int t, int h, f32x4 (&s)[RB][2]) __attribute__((always_inline)) {
    const int key0 = t * kTile;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * (2 * h + jj) + 4 * lg + i;
          bool vis = key < L;
          if (!vis && key < keys && valid_r[rb]) {
            const int tj = key - L;
            if constexpr (PRE != 0)
              vis = tj <= node_r[rb] && node_r[rb] < end_lds[tj];
            else
              vis = (anc_lds[node_r[rb]][(tj >> 6) & (ANC_W - 1)] >> (tj & 63)) & 1ull;
          }
          if (!vis) s[rb][jj][i] = -INFINITY;
        }
  };
  // after a half's exps: when some probability exceeds 2^kRescale (the running max is stale), take the
  // half's maxima, move the running max (rescaling O, l and the chunk accumulator) and redo the exps;
  // then add the half's sums to l
  auto settle_half = [&](const f32x4 (&s)[RB][2], bf16x8 (&pout)[RB], float (&esum)[RB]) __attribute__((always_inline)) {
    bool big = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) big |= esum[rb] > 0x1p8f;
    static_assert(kRescale == 8.0f, "the sum test above is 2^kRescale");
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(big) != 0, 0)) {
      bool resc = false;
      float mt[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3]));
        mx = fmaxf(fmaxf(mx, fmaxf(s[rb][1][0], s[rb][1][1])), fmaxf(s[rb][1][2], s[rb][1][3]));
        mt[rb] = max4g(mx) * c2;
        resc |= mt[rb] > m_r[rb] + kRescale;
      }
      if (__builtin_amdgcn_ballot_w64(resc) != 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float mnew = mt[rb] > m_r[rb] + kRescale ? mt[rb] : m_r[rb];
          const float alpha = __builtin_amdgcn_exp2f(m_r[rb] - mnew);
          l_r[rb] *= alpha;
          cacc[rb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[rb][nb] *= alpha;
          m_r[rb] = mnew;
        }
      }
      exps_half(s, pout, esum);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_r[rb] += esum[rb];
  };
  // chunk sums of a finished half join the accumulator; a 64-slot tile that ends a chunk stores the
  // chunk's log2-sum-exp per row (one 128-byte store per wave)
  auto chunk_add = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) cacc[rb] += csum[rb];
  };
  float st_val = 0.f;                               // a closed chunk's value, stored at the next step
  int st_c = -1;
  auto chunk_close = [&](int key0) __attribute__((always_inline)) {
    const int c = chunk_of(key0);
    const int cend = min((c + 1) * cs, L);
    if (key0 + kTile >= cend) {
      float v = m_r[0] + __builtin_amdgcn_logf(cacc[0]);
#pragma unroll
      for (int rb = 1; rb < RB; ++rb)
        if (st_rb == rb) v = m_r[rb] + __builtin_amdgcn_logf(cacc[rb]);
      st_val = v;
      st_c = c;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) cacc[rb] = 0.f;
    }
  };
  // the store of a closed chunk waits for the start of the next step, ahead of that step's tile loads,
  // so that the counted wait closing the step never waits for it
  auto chunk_flush = [&]() __attribute__((always_inline)) {
    if (CH && st_c >= 0) {
      if (st_ok) cbase[(int64_t)st_c * row_stride_chunk] = st_val;
      st_c = -1;
    }
  };

  // One interleaved block: 17 slots, each one MFMA pair (P.V of the V tile vt, half hv, with pin: dim
  // blocks 0..7; then the chunk sums of pin against a_chunk; then QK^T of the K tile kt, half hk: k-steps
  // 0..3 x key blocks 0..1), the LDS reads of the fragment two slots ahead, and one element's
  // probability (fma, exp, add, bf16 convert) of the half-tile scores sin.  sched_barrier pins the order:
  // about two VALU instructions per MFMA issue in the MFMAs' shadow.
  auto run_block = [&](const uint16_t* vt, int hv, const bf16x8 (&pin)[RB], const bf16x8& a_chunk,
                       const uint16_t* kt, int hk, f32x4 (&sout)[RB][2], const f32x4 (&sin)[RB][2],
                       bf16x8 (&pout)[RB], float (&esum)[RB], auto&& slot_hook) __attribute__((always_inline)) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    constexpr int NF = 17, AHEAD = 2;
    bf16x8 fr[AHEAD + 1];
    auto read_frag = [&](int f, bf16x8& out) __attribute__((always_inline)) {
      if (f < NB) {                                // V^T fragment of dim block f (two transposing reads)
        const int off = v_base[hv] + (v_sh16[hv] ^ (16 * f));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + off + 16 * D));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 av = {lo2[0], lo2[1], hi2[0], hi2[1]};
        out = __builtin_bit_cast(bf16x8, av);
      } else if (f > NB) {                         // K fragment of k-step kk, key block jj
        const int kk = (f - NB - 1) >> 1, jj = (f - NB - 1) & 1;
        out = *reinterpret_cast<const bf16x8*>(kt + k_off[kk] + 16 * (2 * hk + jj) * D);
      }
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) sout[rb][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float xs[RB][8];
#pragma unroll
    for (int f = 0; f < AHEAD; ++f) read_frag(f, fr[f]);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      slot_hook(f);
      if (f + AHEAD < NF) read_frag(f + AHEAD, fr[(f + AHEAD) % (AHEAD + 1)]);
      const bf16x8& cur = fr[f % (AHEAD + 1)];
      if (f < NB) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pin[rb], o[rb][f], 0, 0, 0);
      } else if (f == NB) {
        if (CH) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            csum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_chunk, pin[rb], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)[0];
        }
      } else {
        const int kk = (f - NB - 1) >> 1, jj = (f - NB - 1) & 1;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sout[rb][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qreg[rb][kk], sout[rb][jj], 0, 0, 0);
      }
      if (f < 2 * 8) {                             // element e of row block rb of the P fragment
        const int rb = f >> 3, e = f & 7;
        const float x = __builtin_amdgcn_exp2f(fmaf(sin[rb][e >> 2][e & 3], c2, -m_r[rb]));
        xs[rb][e] = x;
        esum[rb] = e == 0 ? x : esum[rb] + x;
        if (e & 1) {
          pout[rb][e - 1] = (__bf16)xs[rb][e - 1];
          pout[rb][e] = (__bf16)x;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the pipeline ----
  // Tiles load two steps ahead of their first use: during step t, K(t+3) and V(t+2).  On pages of >= 16
  // slots every wave issues exactly LOADS loads per step (empty-range loads past the split's end), and
  // direct-to-LDS loads complete in order among themselves, so the wait that closes step t,
  // vmcnt(LOADS), covers the loads of step t - 1 (K(t+2), V(t+1)) and leaves this step's in flight; a
  // chunk store counted in between only makes that wait longer.  Shorter pages wait for everything.
  auto kslot = [&](int i) __attribute__((always_inline)) -> uint16_t* {
    return i == 0 ? ka : (i == 1 ? kb : (i == 2 ? kc : kd));
  };
  auto vslot = [&](int i) __attribute__((always_inline)) -> uint16_t* {
    return i == 0 ? va : (i == 1 ? vb : (i == 2 ? vc : vd));
  };
  auto issue_tile = [&](int t, uint16_t* buf) __attribute__((always_inline)) {
    if (grouped) {
      const uint16_t* bp;
      uint32_t bytes;
      plan_grouped(t, t < t_end, page_of_tile(t), bp, bytes);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) load_one(bp, bytes, buf, i);
    } else if (t < t_end) {
      issue(t, buf);
    }
  };
  // The barrier that closes a step.  __syncthreads() would also wait for every load in flight (its
  // release fence covers the direct-to-LDS writes), so the wait and the barrier are written out: this
  // thread's LDS writes done (lgkmcnt), the older tile loads landed, then s_barrier.  The asm's memory
  // clobber keeps every memory access on its side of the barrier.
  auto step_barrier = [&]() __attribute__((always_inline)) {
    static_assert(LOADS == 4, "the counted wait below is LOADS");
    if (grouped) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // prologue: K(t0 .. t0+2) and V(t0 .. t0+1) issued, K(t0), K(t0+1) and V(t0) resident, V buffer 3 (the
  // V "tile t0 - 1" of the first step) cleared, then the scores of (t0, half 0).  The first step's P.V of
  // the previous tile multiplies that cleared buffer by P = 0; its chunk sums are zero and never stored.
  const int t0 = t_begin;
  if (!wave_is_v) {
    issue_tile(t0, ka);
    issue_tile(t0 + 1, kb);
    issue_tile(t0 + 2, kc);
  } else {
    issue_tile(t0, va);
    issue_tile(t0 + 1, vb);
  }
  for (int i = tid; i < TILE_EL / 8; i += NT) reinterpret_cast<u32x4*>(vd)[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) pB[rb] = bf16_splat8(0u, 0u);
  // the first step's load plan
  int pg_pre = 0;
  const uint16_t* ld_bp = nullptr;
  uint32_t ld_bytes = 0;
  if (grouped) {
    const int t_first = wave_is_v ? t0 + 2 : t0 + 3;
    plan_grouped(t_first, t_first < t_end, page_of_tile(t_first), ld_bp, ld_bytes);
  }
  step_barrier();
  if (wave_active) qk_half(ka, 0, sA);

  // Step of tile t; R = (t - t0) mod 4 selects the buffers: K(t) in slot R, K(t+1) in R+1, K(t+2) in R+2
  // (landing), K(t+3) loads into R+3; V(t-1) in slot R+3, V(t) in R, V(t+1) in R+1 (landing), V(t+2)
  // loads into R+2 (slots mod 4).  Every tile runs the same two interleaved blocks; a tile holding slots
  // >= L first masks its scores (between the blocks, where few registers are live), and the split's last
  // tile computes scores of a tile it never uses.
  auto step = [&](int t, auto r_c) __attribute__((always_inline)) {
    constexpr int R = decltype(r_c)::value;
    uint16_t* kcur = kslot(R);
    uint16_t* knext = kslot((R + 1) % 4);
    uint16_t* vprev = vslot((R + 3) % 4);
    uint16_t* vcur = vslot(R);
    // this wave's share of K(t+3) (waves 0..3) or V(t+2) (waves 4..7).  On the grouped path its four
    // loads go out one at a time at slots 2, 6, 10 and 14 of B1, so the vector memory path takes them
    // beside the matrix work; the next step's page id is read from LDS at the start of B2 and its load
    // plan made at the end of B2, away from the step boundary where all waves want the scalar unit.
    // (Loads placed in B2 as well, or shared by all waves as K and V halves, measured slower.)
    const int t_ld = wave_is_v ? t + 2 : t + 3;
    uint16_t* ld_buf = wave_is_v ? vslot((R + 2) % 4) : kslot((R + 3) % 4);
    chunk_flush();
    if (!grouped && t_ld < t_end) issue(t_ld, ld_buf);
    auto b1_hook = [&](int f) __attribute__((always_inline)) {
      if (grouped && (f & 3) == 2 && f < 16) load_one(ld_bp, ld_bytes, ld_buf, f >> 2);
    };
    auto b2_hook = [&](int f) __attribute__((always_inline)) {
      if (grouped && f == 0) pg_pre = page_of_tile(t_ld + 1);
      if (grouped && f == 16) plan_grouped(t_ld + 1, t_ld + 1 < t_end, pg_pre, ld_bp, ld_bytes);
    };
    const int key0 = t * kTile;
    const bool edge = key0 + kTile > L;             // holds slots >= L: the tree mask applies
    const bool prev_edge = key0 > L;                // tile t - 1 holds slots >= L
    if (wave_active) {
      if (__builtin_expect(edge, 0)) mask_half(t, 0, sA);
      const bf16x8 a_prev = (CH && __builtin_expect(prev_edge, 0)) ? ones_edge(key0 - kTile, 1) : ones;
      // B1: P.V and chunk sums of (t-1, half 1), QK^T of (t, half 1) | exps of (t, half 0)
      run_block(vprev, 1, pB, a_prev, kcur, 1, sB, sA, pA, eA, b1_hook);
      // the exps' sums feed the rescale check right here, so they stay inside the block above; the chunk
      // of tile t - 1 closes after it (a rescale scales the running max and the chunk sum together, so the
      // stored log2-sum-exp is the same).  At t0 the sums of the cleared "tile t0 - 1" are zero.
      if (CH) chunk_add();
      settle_half(sA, pA, eA);
      if (CH && t > t0 && key0 - kTile < L) chunk_close(key0 - kTile);
      if (__builtin_expect(edge, 0)) mask_half(t, 1, sB);
      const bf16x8 a_cur = (CH && __builtin_expect(edge, 0)) ? ones_edge(key0, 0) : ones;
      // B2: P.V and chunk sums of (t, half 0), QK^T of (t+1, half 0) | exps of (t, half 1)
      run_block(vcur, 0, pA, a_cur, knext, 0, sA, sB, pB, eB, b2_hook);
      if (CH) chunk_add();
      settle_half(sB, pB, eB);
    } else if (grouped) {
      // a wave without rows still loads its share of the tiles
#pragma unroll
      for (int i = 0; i < LOADS; ++i) load_one(ld_bp, ld_bytes, ld_buf, i);
      plan_grouped(t_ld + 1, t_ld + 1 < t_end, page_of_tile(t_ld + 1), ld_bp, ld_bytes);
    }
    step_barrier();                                 // K(t+2) / V(t+1) landed (this thread's loads)
  };
  for (int t = t0; t < t_end; t += 4) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_end) step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < t_end) step(t + 2, std::integral_constant<int, 2>{});
    if (t + 3 < t_end) step(t + 3, std::integral_constant<int, 3>{});
  }
  // the last tile's half 1: P.V, chunk sums and its chunk
  if (wave_active) {
    const int tl = t_end - 1;
    const uint16_t* vl = vslot((tl - t0) & 3);
    pv_half(vl, 1, pB);
    const int key0 = tl * kTile;
    chunk_flush();
    if (CH && key0 < L) {
      chunk_half(pB, key0 + kTile > L ? ones_edge(key0, 1) : ones);
      chunk_add();
      chunk_close(key0);
      chunk_flush();
    }
  }
  // the loads of tiles past the split's end are still in flight: they must land before the work-group's
  // LDS is handed to another work-group
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_r[rb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_r[rb] = l;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!valid_r[rb]) continue;
    const int row = row0 + (wave * RB + rb) * 16 + lm;
    const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.rows_pad + row;
    if (lg == 0) {
      p.part_ml[base * 2 + 0] = m_r[rb];
      p.part_ml[base * 2 + 1] = l_r[rb];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4*>(&p.part_o[base * D + 16 * nb + 4 * lg]) = o[rb][nb];
  }
}

template <int D, int W, int RB, int CM, int VT>
hipError_t launch_d_w(const AttnParams& p, const AttnPlan& plan, hipStream_t s) {
  const int n_units = p.batch * p.Hkv * p.max_splits;
  const int grid = (int)(ceil_div(n_units, 8) * 8 * plan.row_groups);
  if constexpr (D == 128 && W == 8 && CM == 0 && VT == 0) {
    // wide trees, head_dim 128, token-row V, 64-slot (or no) chunk partials: the software-pipelined kernel
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, p); };
    const bool grp = p.page_shift >= 4;
    if (p.subtree_end) {
      if (p.chunk_size > 0) grp ? go(tree_attn_pipe_kernel<1, 1, 1>) : go(tree_attn_pipe_kernel<1, 1, 0>);
      else grp ? go(tree_attn_pipe_kernel<1, 0, 1>) : go(tree_attn_pipe_kernel<1, 0, 0>);
    } else {
      if (p.chunk_size > 0) grp ? go(tree_attn_pipe_kernel<0, 1, 1>) : go(tree_attn_pipe_kernel<0, 1, 0>);
      else grp ? go(tree_attn_pipe_kernel<0, 0, 1>) : go(tree_attn_pipe_kernel<0, 0, 0>);
    }
  } else if constexpr (W == 4 && CM == 0 && VT == 0) {
    // <= 64 rows per KV head (one or two waves with rows): the variant with a store wave
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(grid), dim3(W * 64), 0, s, p); };
    const bool sw = p.max_nodes * p.G <= 64;
    if (p.subtree_end)
      sw ? go(tree_attn_kernel<D, W, RB, CM, VT, 1, 1>) : go(tree_attn_kernel<D, W, RB, CM, VT, 1, 0>);
    else
      sw ? go(tree_attn_kernel<D, W, RB, CM, VT, 0, 1>) : go(tree_attn_kernel<D, W, RB, CM, VT, 0, 0>);
  } else if (p.subtree_end)
    hipLaunchKernelGGL((tree_attn_kernel<D, W, RB, CM, VT, 1>), dim3(grid), dim3(W * 64), 0, s, p);
  else
    hipLaunchKernelGGL((tree_attn_kernel<D, W, RB, CM, VT, 0>), dim3(grid), dim3(W * 64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.batch * p.max_nodes * p.Hq;
  // few rows (under 1024: fewer than 256 work-groups of four rows): one work-group per row
  if (rows < 1024)
    hipLaunchKernelGGL((attn_merge_kernel<D, true>), dim3((unsigned)rows), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, false>), dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D, int CM, int VT>
hipError_t launch_d(const AttnParams& p, const AttnPlan& plan, hipStream_t s) {
  return plan.waves == 8 ? launch_d_w<D, 8, 2, CM, VT>(p, plan, s) : launch_d_w<D, 4, 2, CM, VT>(p, plan, s);
}

template <int D, int CM>
hipError_t launch_v(const AttnParams& p, const AttnPlan& plan, hipStream_t s) {
  return p.v_dim_major ? launch_d<D, CM, 1>(p, plan, s) : launch_d<D, CM, 0>(p, plan, s);
}

template <int D>
hipError_t launch_cm(const AttnParams& p, const AttnPlan& plan, hipStream_t s) {
  if (p.chunk_size == 16) return launch_v<D, 2>(p, plan, s);
  if (p.chunk_size == 32) return launch_v<D, 1>(p, plan, s);
  return launch_v<D, 0>(p, plan, s);
}

}  // namespace

bool make_attn_plan(const spec_tree_attention_args* a, int num_cus, AttnPlan* plan) {
  AttnPlan pl;
  pl.G = a->num_q_heads / a->num_kv_heads;
  const int rows = a->max_nodes * pl.G;
  // 32 rows per wave; 8 waves (256 rows) when a KV head has more than 128 rows, else 4
  pl.waves = rows > 128 ? 8 : 4;
  pl.rb = 2;
  pl.rows_wg = pl.waves * pl.rb * 16;
  pl.row_groups = (int)ceil_div(rows, pl.rows_wg);
  pl.rows_pad = pl.row_groups * pl.rows_wg;
  pl.max_tiles = (int)ceil_div((int64_t)a->max_ctx_len + a->max_nodes, kTile);
  const int align = (a->chunk_size >= kTile) ? a->chunk_size / kTile : 1;   // splits hold whole chunks
  // page ids of one split must fit the LDS staging array
  const int ps = a->kv.page_size > 0 ? a->kv.page_size : 1;
  const int64_t cap_tiles = ((int64_t)(kMaxSplitPages - 1) * ps) / kTile;
  int st = a->split_tiles;
  if (st <= 0) {
    // one round of work-groups: as many as the CUs hold at once (one 8-wave or two 4-wave work-groups
    // per CU), but at least 8 tiles per split.  A second round would add partials to write and merge
    // and per-work-group set-up, and a partial round leaves CUs idle at the end.
    const int64_t ranges = (int64_t)a->batch * a->num_kv_heads * pl.row_groups;
    const int64_t target = (int64_t)(num_cus > 0 ? num_cus : 256) * (pl.waves == 8 ? 1 : 2);
    int64_t want_splits = ceil_div(target, ranges);
    st = (int)ceil_div(pl.max_tiles, want_splits < 1 ? 1 : want_splits);
    if (st < 8) {
      // short contexts: 8 tiles per split, unless the work-groups would then fill less than half of that
      // round; the split length is then halved (down to 2 tiles) until they do, since a split's tiles run
      // one after another (a 4K-token chain: 18 against 24 us)
      st = 8;
      while (st > 2 && ranges * ceil_div(pl.max_tiles, st) < target / 2) st /= 2;
    }
  }
  if (st > cap_tiles) st = (int)cap_tiles;
  st = (int)(ceil_div(st, align) * align);
  if (st > cap_tiles) st = (int)((cap_tiles / align) * align);
  if (st < 1) st = align;
  pl.split_tiles = st;
  pl.max_splits = (int)ceil_div(pl.max_tiles, st);
  pl.max_chunks = a->chunk_size > 0 ? (int)ceil_div(a->max_ctx_len, a->chunk_size) : 0;
  size_t off = 0;
  pl.off_part_o = off;
  off = align_up(off + sizeof(float) * (size_t)a->batch * a->num_kv_heads * pl.max_splits * pl.rows_pad * a->head_dim, 256);
  pl.off_part_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)a->batch * a->num_kv_heads * pl.max_splits * pl.rows_pad, 256);
  pl.off_lse2 = off;
  off = align_up(off + sizeof(float) * (size_t)a->batch * a->max_nodes * a->num_q_heads, 256);
  pl.off_chunk = off;
  {
    // chunk partials: with whole 32-row blocks per KV head, chunk-major, so that a chunk's rows are one
    // run for the salience pass and a wave's 32 rows one 128-byte line; otherwise KV-head-major, so that
    // a work-group's values of consecutive chunks are one run (no line shared with another KV head)
    const int rs = a->max_nodes * pl.G;
    const bool chunk_major = rs % 32 == 0;
    pl.chunk_cs = chunk_major ? a->num_kv_heads * rs : rs;
    pl.chunk_hs = chunk_major ? rs : (pl.max_chunks > 0 ? pl.max_chunks : 1) * rs;
  }
  off = align_up(off + sizeof(float) * (size_t)a->batch * pl.max_chunks * a->num_kv_heads * a->max_nodes * pl.G, 256);
  pl.off_debug = off;                 // the debug record, last
  off += SPEC_DEBUG_RECORD_BYTES;
  pl.bytes = off;
  *plan = pl;
  return true;
}

hipError_t launch_tree_attention(const AttnParams& p, const AttnPlan& plan, int head_dim, hipStream_t s) {
  if (head_dim == 128) return launch_cm<128>(p, plan, s);
  return launch_cm<64>(p, plan, s);
}

}  // namespace spec
