// Data movement on gfx950: dispatch (gather-send fused with scatter-recv),
// the two hops of node-deduplicated dispatch, and the weighted combine.
//
// Work unit: a wave-item = one 64-chunk segment of one row (64 lanes x 16
// bytes = 1 KiB of consecutive bytes; the last segment of a row may be
// partial).  A row's token is wave-uniform, so every per-token value (expert
// ids, in-tile ranks, slots, weights) is loaded once per wave through the
// scalar unit and only the 16-byte row chunks use vector memory.  Each wave
// takes U wave-items and issues all of its loads before any store, to keep
// enough bytes in flight to cover HBM latency.  Source and destination rows
// are contiguous, so the row copies need no LDS staging.
//
//  gather   dispatch, single hop: each source row x[t] is read once and
//           written to its k receive rows (FUSCO article, "core innovation":
//           no pack buffer before the send, no reorder after the receive).
//           Also finishes slot_of / row_src from the in-tile ranks.  Small
//           plans use gather_scan, which also does the plan's scan.
//  stage_a  deduplicated dispatch, hop 1: x[t] is read once and written once
//           per distinct destination node, to that node's forwarder staging
//           row (FUSCO article, "load balancing and cross-node
//           deduplication").  Also finishes slot_of / row_src / stage_of /
//           stage_src.
//  stage_b  hop 2, intra-node fan-out: each staging row is read once and
//           written to every receive row of its token on that node.  The two
//           hops run chunk by chunk over consecutive tokens.
//  combine  out[t] = sum_j w[t,j] * y[slot_of[t,j]]: k row loads, one fp32
//           fused multiply-add per element and slot in ascending j starting
//           from 0, then round-to-nearest-even bf16 (or fp32) out (INC-MoE
//           abstract: combine back to each token's owner).  The hierarchical
//           form (combine_part, combine_nodes) and the fp8 payload follow
//           below.
#include "move_body.h"
#include "plan_body.h"

namespace moe {
namespace {

// Waves per gather_scan block when E <= 64 (olmoe dispatch: 4 -> 32.2 us,
// 8 -> 30.9, 16 -> 31.4), and when E > 64 (qwen3 dispatch: 4 -> 166 us,
// 8 -> 100, 16 -> 90).
constexpr int kGatherScanWaves = 8;
constexpr int kGatherScanWavesWide = 16;
// Wave-items (consecutive segments) per wave of gather_scan, E <= 64 (olmoe,
// two batches in flight: 1 -> 50.3 us a step, 2 -> 48.2, 3 -> 48.4, 4 ->
// 51.1), and E > 64 (qwen3, staggered: 1 -> 204.9 us, 2 -> 208.3, 4 -> 212.3).
constexpr int kGatherScanU = 2;
constexpr int kGatherScanUWide = 1;
// ... of the fp8 gather_scan (fp8 olmoe, two batches in flight: 1 -> 32.5 us,
// 2 -> 33.0, 4 -> 33.4), and its waves per block.
constexpr int kGatherScan8U = 1;
constexpr int kGatherScan8Waves = kGatherScanWaves;
// Wave-items per wave of stage_a.  DeepSeek-V3-like dispatch, one stream:
// 1 -> 679 us, 2 -> 694, 2 consecutive segments sharing their lookups -> 689,
// 4 consecutive -> 714.
constexpr int kStageAU = 1;
// Staging bytes per chunk of the deduplicated dispatch, at most.
// DeepSeek-V3-like dispatch, us with two batches in flight / one stream
// (before stage A skipped its unused lookups): no chunks 1217 / 1217,
// 512 MiB 1228 / 1187, 256 MiB 1178 / 1180, 224 MiB (8 chunks) 1142 / 1181,
// 128 MiB 1107 / 1265.
constexpr int64_t kChunkBytes = (int64_t)224 << 20;
// Partial bytes per chunk of the hierarchical combine, at most.
// DeepSeek-V3-like, us on one stream: whole batch 1235, 448 MiB (8 chunks)
// 1149, 224 MiB 1189, 112 MiB 1356.
constexpr int64_t kHierChunkBytes = (int64_t)448 << 20;

// The plan inputs a block of the folded-scan gather reads before it can place
// rows: its share of the tile-count matrix (entries tid + r * GB), and for
// each wave-item the in-tile rank and expert of its token's slots (lane
// j < k holds slot j).  The gather loads them before its row loads: a wave's
// loads complete in issue order, so data loaded after the rows could be used
// only once the rows had arrived, and the block would scan after its rows
// load instead of while they do.  Every one of these loads, and every row
// load after them, is issued by every lane (at a clamped address where the
// lane has nothing to load, its value then dropped): a load skipped on some
// path would leave the count of loads in flight unknown, and the wait for
// the plan inputs would become a wait for everything.
template <int GB>
__device__ __forceinline__ void load_tile_counts(const Dims& d, const Work& w,
                                                 int (&m)[kFusedScanInts / GB]) {
  const int n = d.nblk * d.E;
#pragma unroll
  for (int r = 0; r < kFusedScanInts / GB; ++r) {
    const int i = threadIdx.x + r * GB;
    const int v = w.tile_counts[min(i, n - 1)];
    m[r] = i < n ? v : 0;
  }
}

__device__ __forceinline__ void load_slot_inputs(const Dims& d, const int32_t* __restrict__ idx,
                                                 const Work& w, bool live, int t, int& l, int& e) {
  const int lane = threadIdx.x % kWave;
  const bool mine = live && lane < d.k;
  const int64_t at = (int64_t)(live ? t : 0) * d.k + min(lane, d.k - 1);
  const int lv = w.lr[at], ev = idx[at];
  l = mine ? lv : -1;
  e = mine ? ev : 0;
}

// The scan folded into the gather of a small plan (nblk * E <=
// kFusedScanInts; single band).  The block (GB threads, all of which call
// this) puts the tile counts it loaded (load_tile_counts) into LDS, sums each
// expert's column and scans the totals over the experts (one wave with lane
// shuffles when E <= 64) into s_off.  fused_slot then gives each token's
// receive rows: the expert's first row, plus its rows in earlier tiles, plus
// the slot's rank in its tile (the same rows route_scan's tile bases give).
template <int GB>
__device__ __forceinline__ void fused_scan_block(const Dims& d, const int (&m)[kFusedScanInts / GB],
                                                 int* s_mat, int* s_off, int* s_wsum,
                                                 int* s_part) {
  constexpr int kGBlock = GB;
  const int tid = threadIdx.x, lane = threadIdx.x % kWave;
  const int E = d.E, n = d.nblk * E;
#pragma unroll
  for (int r = 0; r < kFusedScanInts / GB; ++r)
    if (tid + r * GB < n) s_mat[tid + r * GB] = m[r];
  __syncthreads();
  if (E <= kWave) {
    // Up to 64 experts: kGBlock / E threads per expert sum parts of its
    // column, then one wave adds the parts and scans with lane shuffles.
    const int parts = min(kGBlock / E, d.nblk);
    if (tid < parts * E) {
      const int q = tid / E, e = tid - q * E;
      s_off[tid] = column_sum(s_mat, E, e, q * d.nblk / parts, (q + 1) * d.nblk / parts);
    }
    __syncthreads();
    if (tid < kWave) {
      int tot = 0;
      if (tid < E)
        for (int q = 0; q < parts; ++q) tot += s_off[q * E + tid];
      int incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (tid >= o) incl += y;
      }
      if (tid < E) s_off[tid] = incl - tot;  // parts are all read: each lane read only its column
    }
    __syncthreads();
  } else {
    // With at least two threads per expert, kGBlock / E threads sum parts of
    // its column into s_part (parts * E <= kGBlock entries) and the first E
    // threads add them; else each thread sums whole columns.  Then the block
    // scans the totals (block_exclusive_scan covers 4 * kPlanBlock entries
    // with its first kPlanWaves waves; any further waves carry zeros).
    const int parts = min(kGBlock / E, d.nblk);
    if (parts >= 2) {
      if (tid < parts * E) {
        const int q = tid / E, e = tid - q * E;
        s_part[tid] = column_sum(s_mat, E, e, q * d.nblk / parts, (q + 1) * d.nblk / parts);
      }
      __syncthreads();
      if (tid < E) {
        int tot = 0;
        for (int q = 0; q < parts; ++q) tot += s_part[q * E + tid];
        s_off[tid] = tot;
      }
    } else {
      for (int e = tid; e < E; e += kGBlock) s_off[e] = column_sum(s_mat, E, e, 0, d.nblk);
    }
    __syncthreads();
    block_exclusive_scan(s_off, E, s_wsum);
  }
}

// After fused_scan_block: lane j < k of the wave returns the receive row of
// slot j of token t from the slot's in-tile rank l and expert e
// (load_slot_inputs; -1 for a dropped slot or another lane).
__device__ __forceinline__ int fused_slot(const Dims& d, int l, int e, int t, const int* s_mat,
                                          const int* s_off) {
  if (l < 0) return -1;
  e = min(max(e, 0), d.E - 1);
  return s_off[e] + column_sum(s_mat, d.E, e, 0, t / d.tile) + l;
}

// Gather for plans whose tile-count matrix is small (nblk * E <=
// kFusedScanInts): every block first issues its row loads, then scans the raw
// tile counts in LDS (column totals, their exclusive scan over the experts,
// and the prefix over earlier tiles for the experts its tokens use) while
// those loads are in flight.  The plan's separate scan launch then leaves the
// critical path (it still runs, lazily, for anything that reads the plan
// arrays).  Each wave takes U consecutive segments, so a block's scan serves
// GW * U of them.  Same receive rows as gather_kernel.
template <int KMAX, int GW, int U>
__global__ __launch_bounds__(GW * kWave) void gather_scan_kernel(Dims d, const int32_t* __restrict__ idx,
                                                                 const u32x4* __restrict__ x,
                                                                 u32x4* __restrict__ recv, Work w,
                                                                 int base, int limit) {
  constexpr int kGBlock = GW * kWave;
  __shared__ int s_mat[kFusedScanInts];   // tile counts [nblk][E]
  __shared__ int s_off[MOE_MAX_EXPERTS];  // first receive row of each expert
  __shared__ int s_wsum[GW];
  __shared__ int s_part[GW * kWave];      // column parts (more than 64 experts)
  const int lane = threadIdx.x % kWave, tid = threadIdx.x;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const bool keep = keep_rows(rows, 2 * d.H);
  // wave-items g = base + (block * GW + wave) * U + u: U consecutive segments
  Item it[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = __builtin_amdgcn_readfirstlane(base + (blockIdx.x * GW + tid / kWave) * U + u);
    it[u].live = g < limit;
    it[u].t = it[u].live ? g / d.segs : 0;
    it[u].c = (g - it[u].t * d.segs) * kWave + lane;
    it[u].ok = it[u].live && it[u].c < d.chunks;
  }
  // plan inputs first, then the rows, all unconditional (load_tile_counts)
  int m[kFusedScanInts / kGBlock], sl[U], se[U];
  load_tile_counts<kGBlock>(d, w, m);
#pragma unroll
  for (int u = 0; u < U; ++u) load_slot_inputs(d, idx, w, it[u].live, it[u].t, sl[u], se[u]);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = load_x_chunk(&x[it[u].ok ? (int64_t)it[u].t * d.chunks + it[u].c : 0]);

  fused_scan_block<kGBlock>(d, m, s_mat, s_off, s_wsum, s_part);
  int mine = -1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u == 0 || it[u].t != it[u - 1].t)
      mine = fused_slot(d, sl[u], se[u], it[u].t, s_mat, s_off);
    int slot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) slot[j] = __builtin_amdgcn_readfirstlane(__shfl(mine, j));

    if (it[u].live && it[u].c == lane && lane < d.k) {  // the first segment publishes the slots
      w.slot_of[(int64_t)it[u].t * d.k + lane] = mine;
      if ((uint32_t)mine < rows) w.row_src[mine] = it[u].t;
    }
    if (it[u].ok) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if ((uint32_t)slot[j] < rows)
          store_row(&recv[(int64_t)slot[j] * d.chunks + it[u].c], v[u], keep);
    }
  }
}

// Hop 1 over wave-items [item0, item_end) (one chunk of tokens), block-chunk
// blk of them; keep: plain stores for the staging rows.
template <int KMAX, int U>
__device__ __forceinline__ void stage_a_body(const Dims& d, const int32_t* __restrict__ idx,
                                             const u32x4* __restrict__ x,
                                             u32x4* __restrict__ staging, const Work& w, int blk,
                                             int item0, int item_end, int keep) {
  const int lane = threadIdx.x % kWave;
  const uint32_t rows = (uint32_t)(d.T * d.k), srows = (uint32_t)d.smax;
  Item it[U];
  int slot[U][KMAX], p[U][KMAX];
  uint32_t lead[U];
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, item0, item_end, u);
    lead[u] = 0;
    // x first, so its latency overlaps the plan lookups (DeepSeek-V3-like
    // dispatch 715 -> 695 us); non-temporal here (826 -> 794 us with x read
    // from HBM), while the single-hop gather keeps plain loads
    if (it[u].ok) v[u] = load_chunk(&x[(int64_t)it[u].t * d.chunks + it[u].c]);
    if (it[u].live) {
      // only a row's first segment publishes the slots: the others skip
      // their lookups (DeepSeek-V3-like dispatch 756 -> 715 us)
      if (__builtin_amdgcn_readfirstlane(it[u].c - lane) == 0) {
        token_slots_serial<KMAX>(d, w, idx, it[u].t, slot[u]);
      } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) slot[u][j] = -1;
      }
      token_stages<KMAX>(d, w, it[u].t, p[u], lead[u]);
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) slot[u][j] = p[u][j] = -1;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (it[u].live && it[u].c == lane && lane < d.k) {
      const int64_t at = (int64_t)it[u].t * d.k + lane;
      const int s = lane_pick<KMAX>(slot[u], lane);
      const int q = lane_pick<KMAX>(p[u], lane);
      w.slot_of[at] = s;
      if ((uint32_t)s < rows) w.row_src[s] = it[u].t;
      w.stage_of[at] = q;
      if (((lead[u] >> lane) & 1u) && (uint32_t)q < srows) w.stage_src[q] = it[u].t;
    }
    if (it[u].ok) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (((lead[u] >> j) & 1u) && (uint32_t)p[u][j] < srows)
          store_row(&staging[(int64_t)p[u][j] * d.chunks + it[u].c], v[u], keep);
    }
  }
}

// Hop 2, one token per wave-item, over wave-items [item0, item_end),
// block-chunk blk of them: each of the token's staging rows (one per
// destination node) is read once and written to the token's slots on that
// node.
template <int KMAX, int U>
__device__ __forceinline__ void stage_b_body(const Dims& d, const u32x4* __restrict__ staging,
                                             u32x4* __restrict__ recv, const Work& w, int blk,
                                             int item0, int item_end) {
  const uint32_t rows = (uint32_t)(d.T * d.k), srows = (uint32_t)d.smax;
  const bool keep = keep_rows(rows, 2 * d.H);
  Item it[U];
  int slot[U][KMAX], p[U][KMAX];
  u32x4 v[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, item0, item_end, u);
    const int64_t at = (int64_t)it[u].t * d.k;
    int sj[KMAX], pj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {  // no branch between the loads: they issue together
      const int64_t a = slot_index(at, j, d.k);
      sj[j] = w.slot_of[a];
      pj[j] = w.stage_of[a];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool has = it[u].live && j < d.k;
      slot[u][j] = has ? sj[j] : -1;
      p[u][j] = has ? pj[j] : -1;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      bool first = (uint32_t)p[u][j] < srows;
#pragma unroll
      for (int jj = 0; jj < j; ++jj) first = first && p[u][jj] != p[u][j];
      if (first && it[u].ok) v[u][j] = load_chunk(&staging[(int64_t)p[u][j] * d.chunks + it[u].c]);
      if (!first) p[u][j] = p[u][j] < 0 ? -1 : -2 - p[u][j];  // later slot of a node: -2-row
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!it[u].ok) continue;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (p[u][j] < 0) continue;  // j is the first slot of its node: write all of the node's slots
#pragma unroll
      for (int jj = j; jj < KMAX; ++jj) {
        const bool same = jj == j || p[u][jj] == -2 - p[u][j];
        if (same && (uint32_t)slot[u][jj] < rows)
          store_row(&recv[(int64_t)slot[u][jj] * d.chunks + it[u].c], v[u][j], keep);
      }
    }
  }
}

template <int KMAX, int U>
__global__ __launch_bounds__(kBlock) void stage_a_kernel(Dims d, const int32_t* __restrict__ idx,
                                                         const u32x4* __restrict__ x,
                                                         u32x4* __restrict__ staging, Work w,
                                                         int item0, int item_end, int keep) {
  stage_a_body<KMAX, U>(d, idx, x, staging, w, blockIdx.x, item0, item_end, keep);
}

template <int KMAX, int U>
__global__ __launch_bounds__(kBlock) void stage_b_kernel(Dims d, const u32x4* __restrict__ staging,
                                                         u32x4* __restrict__ recv, Work w,
                                                         int item0, int item_end) {
  stage_b_body<KMAX, U>(d, staging, recv, w, blockIdx.x, item0, item_end);
}

// Hop 2 of chunk c in the first b_blocks blocks, hop 1 of chunk c + 1 in the
// others.  The GPU dispatches a grid's blocks in order, so hop 1's blocks
// start as hop 2's drain and fill its tail, and a chunk boundary costs one
// launch instead of two (DeepSeek-V3-like dispatch 712 -> 665 us a step,
// with the route plan).  The two hops touch disjoint rows and plan entries.
// Hop 2 takes one wave-item a wave here, so the kernel fits 8 waves per SIMD.
template <int KMAX>
__global__ __launch_bounds__(kBlock) void stage_ab_kernel(Dims d, const int32_t* __restrict__ idx,
                                                          const u32x4* __restrict__ x,
                                                          u32x4* __restrict__ staging,
                                                          u32x4* __restrict__ recv, Work w,
                                                          int b_blocks, int b_item0, int b_item_end,
                                                          int a_item0, int a_item_end, int keep) {
  if ((int)blockIdx.x < b_blocks)
    stage_b_body<KMAX, 1>(d, staging, recv, w, blockIdx.x, b_item0, b_item_end);
  else
    stage_a_body<KMAX, kStageAU>(d, idx, x, staging, w, blockIdx.x - b_blocks, a_item0, a_item_end,
                                 keep);
}

// ---- hierarchical combine over the deduplication's staging rows ------------
// Hop 1 (at the forwarder): one fp32 partial per staging row p = (token t,
// node n), the fused multiply-add chain over t's slots on n in ascending j.
// Token-major: a wave-item is a segment of token t, whose k rows are loaded
// once; each of t's staging rows gets its partial (a row all of whose slots
// were dropped gets zeros).
template <int KMAX>
__device__ __forceinline__ void combine_part_body(const Dims& d, const u32x4* __restrict__ y,
                                                  const float* __restrict__ wts,
                                                  f32x4* __restrict__ part, const Work& w, int blk,
                                                  int item0, int item_end, int keep) {
  const uint32_t rows = (uint32_t)(d.T * d.k), srows = (uint32_t)d.smax;
  const Item it = wave_item<1>(d, blk, item0, item_end, 0);
  const int64_t at = (int64_t)it.t * d.k;
  int slot[KMAX], p[KMAX];
  float wj[KMAX];
  u32x4 v[KMAX];
  {
    int sj[KMAX], pj[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {  // no branch between the loads: they issue together
      const int64_t a = slot_index(at, j, d.k);
      sj[j] = w.slot_of[a];
      pj[j] = w.stage_of[a];
      wt[j] = wts[a];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool has = it.live && j < d.k;
      slot[j] = has && (uint32_t)sj[j] < rows ? sj[j] : -1;
      p[j] = has && (uint32_t)pj[j] < srows ? pj[j] : -1;
      wj[j] = wt[j];
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (slot[j] >= 0 && it.ok) v[j] = load_chunk(&y[(int64_t)slot[j] * d.chunks + it.c]);
  if (!it.ok) return;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    bool first = p[j] >= 0;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) first = first && p[jj] != p[j];
    if (!first) continue;  // p[j] is done by its first slot
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int jj = j; jj < KMAX; ++jj) {
      if (p[jj] != p[j] || slot[jj] < 0) continue;
      float f[8];
      unpack_bf16(v[jj], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wj[jj], f[q], acc[q]);
    }
    f32x4* o = part + ((int64_t)p[j] * d.chunks + it.c) * 2;
    store_row(o, f32x4{acc[0], acc[1], acc[2], acc[3]}, keep);
    store_row(o + 1, f32x4{acc[4], acc[5], acc[6], acc[7]}, keep);
  }
}

// Hop 2 (at the owner): out[t] = sum of t's partials in ascending node order
// (one partial per node the token reached), then bf16 (nearest even) or fp32.
template <int KMAX, bool F32OUT>
__device__ __forceinline__ void combine_nodes_body(const Dims& d, const f32x4* __restrict__ part,
                                                   const Work& w, void* __restrict__ out, int blk,
                                                   int item0, int item_end) {
  const uint32_t srows = (uint32_t)d.smax;
  const Item it = wave_item<1>(d, blk, item0, item_end, 0);
  const int64_t at = (int64_t)it.t * d.k;
  int p[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool has = it.live && j < d.k;
    p[j] = has ? w.stage_of[at + j] : -1;
    if ((uint32_t)p[j] >= srows) p[j] = -1;
#pragma unroll
    for (int jj = 0; jj < j; ++jj)
      if (p[jj] == p[j]) p[j] = -1;  // a later slot of an already seen node
  }
  f32x4 a[KMAX], b[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (p[j] >= 0 && it.ok) {
      const f32x4* src = part + ((int64_t)p[j] * d.chunks + it.c) * 2;
      a[j] = __builtin_nontemporal_load(src);
      b[j] = __builtin_nontemporal_load(src + 1);
    }
  }
  if (!it.ok) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  // Add the partials in ascending node order.  Staging rows are grouped by
  // forwarder and forwarders are numbered node by node, so that is the
  // ascending order of the token's (distinct) partial rows: no expert ids or
  // rank divisions needed (DeepSeek-V3-like hierarchical combine 1148 ->
  // 1086 us against ranking by node).
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (p[j] < 0) continue;
      int rank = 0;
#pragma unroll
      for (int jj = 0; jj < KMAX; ++jj) rank += (p[jj] >= 0 && p[jj] < p[j]) ? 1 : 0;
      if (rank != r) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] += a[j][q];
        acc[4 + q] += b[j][q];
      }
    }
  }
  const int64_t i = (int64_t)it.t * d.chunks + it.c;
  if constexpr (F32OUT) {
    f32x4* o = reinterpret_cast<f32x4*>(out) + i * 2;
    store_chunk(o, f32x4{acc[0], acc[1], acc[2], acc[3]});
    store_chunk(o + 1, f32x4{acc[4], acc[5], acc[6], acc[7]});
  } else {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
    store_chunk(reinterpret_cast<u32x4*>(out) + i, r);
  }
}

template <int KMAX>
__global__ __launch_bounds__(kBlock) void combine_part_kernel(Dims d, const u32x4* __restrict__ y,
                                                              const float* __restrict__ wts,
                                                              f32x4* __restrict__ part, Work w,
                                                              int item0, int item_end, int keep) {
  combine_part_body<KMAX>(d, y, wts, part, w, blockIdx.x, item0, item_end, keep);
}

template <int KMAX, bool F32OUT>
__global__ __launch_bounds__(kBlock) void combine_nodes_kernel(Dims d, const f32x4* __restrict__ part,
                                                               Work w, void* __restrict__ out,
                                                               int item0, int item_end) {
  combine_nodes_body<KMAX, F32OUT>(d, part, w, out, blockIdx.x, item0, item_end);
}

// Hop 2 of chunk c in the first b_blocks blocks and hop 1 of chunk c + 1 in
// the others, as stage_ab_kernel: one launch per chunk boundary.
template <int KMAX, bool F32OUT>
__global__ __launch_bounds__(kBlock) void combine_pn_kernel(Dims d, const u32x4* __restrict__ y,
                                                            const float* __restrict__ wts,
                                                            f32x4* __restrict__ part, Work w,
                                                            void* __restrict__ out, int b_blocks,
                                                            int n_item0, int n_item_end, int p_item0,
                                                            int p_item_end, int keep) {
  if ((int)blockIdx.x < b_blocks)
    combine_nodes_body<KMAX, F32OUT>(d, part, w, out, blockIdx.x, n_item0, n_item_end);
  else
    combine_part_body<KMAX>(d, y, wts, part, w, blockIdx.x - b_blocks, p_item0, p_item_end, keep);
}

// ---- fp8 payload -----------------------------------------------------------
// OCP E4M3 codes; each row is cut into blocks of 128 elements (16 lanes x 8),
// each block scaled by the smallest power of two 2^e with amax <= 448 * 2^e.
// Scaling by a power of two is exact, so the only rounding is the code
// choice: the gfx950 conversion instruction, round to nearest even.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kFp8BlockChunks = 16;  // 16-byte bf16 chunks per scale block

// Block exponent of a block whose largest magnitude has the float bits
// `abits` (sign cleared): 0 for an all-zero block and for a block holding an
// infinity or a NaN (whose codes are then unspecified), else the smallest e
// with amax <= 448 * 2^e.
__device__ __forceinline__ int fp8_block_exp(uint32_t abits) {
  if (abits == 0u || abits >= 0x7f800000u) return 0;
  int p;
  const float m = frexpf(__uint_as_float(abits), &p);  // amax = m * 2^p, m in [0.5, 1)
  const int e = p - 9 + (m > 0.875f ? 1 : 0);
  return min(max(e, -126), 127);
}

// 8 floats (already scaled) -> 8 E4M3 codes, element i in byte i.
__device__ __forceinline__ u32x2 encode_e4m3x8(const float (&f)[8]) {
  u32x2 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h], f[4 * h + 1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h + 2], f[4 * h + 3], word, true);
    r[h] = (uint32_t)word;
  }
  return r;
}

__device__ __forceinline__ void decode_e4m3x8(u32x2 c, float (&f)[8]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], true);
    f[4 * h] = lo[0];
    f[4 * h + 1] = lo[1];
    f[4 * h + 2] = hi[0];
    f[4 * h + 3] = hi[1];
  }
}

// fp8 dispatch wave-items: each lane takes two 16-byte bf16 chunks (16
// elements), so a wave covers 128 chunks of a row and writes 16 bytes of codes
// per lane; a 128-element scale block is 8 lanes.  (The fp8 combine keeps one
// chunk per lane: twice the waves in flight measured faster there.)
constexpr int kFp8ItemChunks = 2 * kWave;
constexpr int kFp8BlockLanes = kFp8BlockChunks / 2;

struct Item8 {
  int t, c0;         // token, first of the lane's two chunks
  bool live, ok0, ok1;
};

template <int U>
__device__ __forceinline__ Item8 wave_item8(const Dims& d, int segs8, int blk, int base, int limit,
                                        int u) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = __builtin_amdgcn_readfirstlane(base + (blk * U + u) * kWaves + wave);
  Item8 it;
  it.live = g < limit;
  it.t = it.live ? g / segs8 : 0;
  const int seg = g - it.t * segs8;
  it.c0 = seg * kFp8ItemChunks + 2 * lane;
  it.ok0 = it.live && it.c0 < d.chunks;
  it.ok1 = it.live && it.c0 + 1 < d.chunks;
  return it;
}

// 16 codes of a lane at byte offset (row * H + c0 * 8): one 16-byte store when
// rows are 16-byte multiples (H % 16 == 0), else two 8-byte stores.
__device__ __forceinline__ void store_codes(uint8_t* base, int64_t row, const Dims& d,
                                            const Item8& it, u32x2 a, u32x2 b, bool keep) {
  uint8_t* p = base + row * d.H + (int64_t)it.c0 * 8;
  if ((d.H & 15) == 0) {
    const u32x4 v = {a[0], a[1], b[0], b[1]};
    store_row(reinterpret_cast<u32x4*>(p), v, keep);
  } else {
    if (it.ok0) store_row(reinterpret_cast<u32x2*>(p), a, keep);
    if (it.ok1) store_row(reinterpret_cast<u32x2*>(p + 8), b, keep);
  }
}

// The lane's 16 codes of its two chunks of a token row and its scale
// block's scale 2^e.
struct Fp8Piece {
  u32x2 a, b;
  float scale;
};

// The lane's two 16-byte chunks of token row it.t (zeros past the row).
__device__ __forceinline__ void load_piece(const Dims& d, const Item8& it,
                                           const u32x4* __restrict__ x, u32x4& v0, u32x4& v1) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int64_t xrow = (int64_t)it.t * d.chunks;
  v0 = it.ok0 ? load_x_chunk(&x[xrow + it.c0]) : zero;
  v1 = it.ok1 ? load_x_chunk(&x[xrow + it.c0 + 1]) : zero;
}

// Quantizes the lane's two chunks (block amax by an 8-lane reduction, so
// every lane of the wave must call it).
__device__ __forceinline__ Fp8Piece quantize_loaded(u32x4 v0, u32x4 v1) {
  float f0[8], f1[8];
  unpack_bf16(v0, f0);
  unpack_bf16(v1, f1);
  // The largest magnitude as float bits with the sign cleared: for
  // non-negative floats the integer order is the numeric order, and an
  // infinity or NaN compares above every finite value (a float max would
  // skip a NaN).
  uint32_t abits = 0u;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    abits = max(abits, max(__float_as_uint(f0[q]) & 0x7fffffffu, __float_as_uint(f1[q]) & 0x7fffffffu));
#pragma unroll
  for (int o = kFp8BlockLanes / 2; o > 0; o >>= 1)
    abits = max(abits, (uint32_t)__shfl_xor((int)abits, o, kFp8BlockLanes));
  const int e = fp8_block_exp(abits);
  const float inv = ldexpf(1.0f, -e);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f0[q] *= inv;
    f1[q] *= inv;
  }
  return Fp8Piece{encode_e4m3x8(f0), encode_e4m3x8(f1), ldexpf(1.0f, e)};
}

// 16 codes of a lane from byte offset (row * H + c0 * 8), the inverse of
// store_codes.
__device__ __forceinline__ void load_codes(const uint8_t* base, int64_t row, const Dims& d,
                                           const Item8& it, u32x2& a, u32x2& b) {
  const uint8_t* p = base + row * d.H + (int64_t)it.c0 * 8;
  if ((d.H & 15) == 0) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    a = u32x2{v[0], v[1]};
    b = u32x2{v[2], v[3]};
  } else {
    const u32x2 zero = {0u, 0u};
    a = it.ok0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)) : zero;
    b = it.ok1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + 8)) : zero;
  }
}

// Dispatch with an fp8 payload: each token row is read once, quantized once
// and its codes and block scales are written to the token's k receive rows.
template <int KMAX>
__global__ __launch_bounds__(kBlock) void gather_fp8_kernel(Dims d, const int32_t* __restrict__ idx,
                                                            const u32x4* __restrict__ x,
                                                            uint8_t* __restrict__ recv8,
                                                            float* __restrict__ rscale, Work w,
                                                            int base, int limit) {
  const int lane = threadIdx.x % kWave;
  const int segs8 = (d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  const Item8 it = wave_item8<1>(d, segs8, blockIdx.x, base, limit, 0);
  u32x4 v0, v1;  // x first, so its latency overlaps the slot lookups
  load_piece(d, it, x, v0, v1);
  int slot[KMAX];
  if (it.live) {
    token_slots<KMAX>(d, w, idx, it.t, slot);
  } else {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) slot[j] = -1;
  }
  const Fp8Piece q = quantize_loaded(v0, v1);
  const u32x2 ca = q.a, cb = q.b;
  const float scale = q.scale;
  const bool scale_lane = it.ok0 && (lane % kFp8BlockLanes) == 0;
  const int blk = it.c0 / kFp8BlockChunks;

  if (it.live && it.c0 == 2 * lane && lane < d.k) {  // first segment publishes the slots
    const int s = lane_pick<KMAX>(slot, lane);
    w.slot_of[(int64_t)it.t * d.k + lane] = s;
    if ((uint32_t)s < rows) w.row_src[s] = it.t;
  }
  if (it.ok0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if ((uint32_t)slot[j] < rows) {
        store_codes(recv8, slot[j], d, it, ca, cb, keep_rows((int64_t)d.T * d.k, d.H));
        if (scale_lane) rscale[(int64_t)slot[j] * nb + blk] = scale;
      }
    }
  }
}

// gather_fp8_kernel for small plans, with the scan folded in as in
// gather_scan_kernel (GW waves per block): the row loads are issued first,
// the scan runs while they are in flight.
template <int KMAX, int GW, int U>
__global__ __launch_bounds__(GW * kWave) void gather_fp8_scan_kernel(Dims d,
                                                                     const int32_t* __restrict__ idx,
                                                                     const u32x4* __restrict__ x,
                                                                     uint8_t* __restrict__ recv8,
                                                                     float* __restrict__ rscale,
                                                                     Work w, int base, int limit) {
  __shared__ int s_mat[kFusedScanInts];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[GW];
  __shared__ int s_part[GW * kWave];
  const int lane = threadIdx.x % kWave;
  const int segs8 = (d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  const bool keep = keep_rows(rows, d.H);
  Item8 it[U];  // wave-items g = base + (block * GW + wave) * U + u
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = __builtin_amdgcn_readfirstlane(base + (blockIdx.x * GW + threadIdx.x / kWave) * U + u);
    it[u].live = g < limit;
    it[u].t = it[u].live ? g / segs8 : 0;
    it[u].c0 = (g - it[u].t * segs8) * kFp8ItemChunks + 2 * lane;
    it[u].ok0 = it[u].live && it[u].c0 < d.chunks;
    it[u].ok1 = it[u].live && it[u].c0 + 1 < d.chunks;
  }
  // plan inputs first, then the rows, all unconditional (load_tile_counts)
  int m[kFusedScanInts / (GW * kWave)], sl[U], se[U];
  load_tile_counts<GW * kWave>(d, w, m);
#pragma unroll
  for (int u = 0; u < U; ++u) load_slot_inputs(d, idx, w, it[u].live, it[u].t, sl[u], se[u]);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v0[U], v1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t xrow = (int64_t)it[u].t * d.chunks;
    v0[u] = load_x_chunk(&x[it[u].ok0 ? xrow + it[u].c0 : 0]);
    v1[u] = load_x_chunk(&x[it[u].ok1 ? xrow + it[u].c0 + 1 : 0]);
  }
  fused_scan_block<GW * kWave>(d, m, s_mat, s_off, s_wsum, s_part);
  int mine = -1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u == 0 || it[u].t != it[u - 1].t)
      mine = fused_slot(d, sl[u], se[u], it[u].t, s_mat, s_off);
    int slot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) slot[j] = __builtin_amdgcn_readfirstlane(__shfl(mine, j));
    const u32x4 zero = {0u, 0u, 0u, 0u};  // lanes past the row quantize zeros
    const Fp8Piece q = quantize_loaded(it[u].ok0 ? v0[u] : zero, it[u].ok1 ? v1[u] : zero);
    const bool scale_lane = it[u].ok0 && (lane % kFp8BlockLanes) == 0;
    const int blk = it[u].c0 / kFp8BlockChunks;
    if (it[u].live && it[u].c0 == 2 * lane && lane < d.k) {  // first segment publishes the slots
      w.slot_of[(int64_t)it[u].t * d.k + lane] = mine;
      if ((uint32_t)mine < rows) w.row_src[mine] = it[u].t;
    }
    if (it[u].ok0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if ((uint32_t)slot[j] < rows) {
          store_codes(recv8, slot[j], d, it[u], q.a, q.b, keep);
          if (scale_lane) rscale[(int64_t)slot[j] * nb + blk] = q.scale;
        }
      }
    }
  }
}

// Node-deduplicated dispatch with an fp8 payload, hop 1: each token row is
// read and quantized once, and its codes and block scales go to one staging
// row per destination node.  Also finishes slot_of / row_src / stage_of /
// stage_src.
template <int KMAX>
__device__ __forceinline__ void stage_a_fp8_body(const Dims& d, const int32_t* __restrict__ idx,
                                                 const u32x4* __restrict__ x,
                                                 uint8_t* __restrict__ stage8,
                                                 float* __restrict__ sscale, const Work& w, int bx,
                                                 int item0, int item_end, int keep) {
  const int lane = threadIdx.x % kWave;
  const int segs8 = (d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks;
  const uint32_t rows = (uint32_t)(d.T * d.k), srows = (uint32_t)d.smax;
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  const Item8 it = wave_item8<1>(d, segs8, bx, item0, item_end, 0);
  u32x4 v0, v1;  // x first, so its latency overlaps the plan lookups
  load_piece(d, it, x, v0, v1);
  int slot[KMAX], p[KMAX];
  uint32_t lead = 0;
  if (it.live) {
    // only a row's first segment publishes the slots: the others skip them
    if (__builtin_amdgcn_readfirstlane(it.c0 - 2 * lane) == 0) {
      token_slots_serial<KMAX>(d, w, idx, it.t, slot);
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) slot[j] = -1;
    }
    token_stages<KMAX>(d, w, it.t, p, lead);
  } else {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) slot[j] = p[j] = -1;
  }
  const Fp8Piece q = quantize_loaded(v0, v1);
  const bool scale_lane = it.ok0 && (lane % kFp8BlockLanes) == 0;
  const int blk = it.c0 / kFp8BlockChunks;
  if (it.live && it.c0 == 2 * lane && lane < d.k) {  // first segment publishes the plan
    const int64_t at = (int64_t)it.t * d.k + lane;
    const int s = lane_pick<KMAX>(slot, lane);
    const int r = lane_pick<KMAX>(p, lane);
    w.slot_of[at] = s;
    if ((uint32_t)s < rows) w.row_src[s] = it.t;
    w.stage_of[at] = r;
    if (((lead >> lane) & 1u) && (uint32_t)r < srows) w.stage_src[r] = it.t;
  }
  if (it.ok0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (((lead >> j) & 1u) && (uint32_t)p[j] < srows) {
        store_codes(stage8, p[j], d, it, q.a, q.b, keep);
        if (scale_lane) sscale[(int64_t)p[j] * nb + blk] = q.scale;
      }
    }
  }
}

// Hop 2, one token per wave-item: each of the token's staging rows (codes and
// scales) is read once and written to the token's slots on that node.
template <int KMAX>
__device__ __forceinline__ void stage_b_fp8_body(const Dims& d, const uint8_t* __restrict__ stage8,
                                                 const float* __restrict__ sscale,
                                                 uint8_t* __restrict__ recv8,
                                                 float* __restrict__ rscale, const Work& w, int bx,
                                                 int item0, int item_end) {
  const int lane = threadIdx.x % kWave;
  const int segs8 = (d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks;
  const uint32_t rows = (uint32_t)(d.T * d.k), srows = (uint32_t)d.smax;
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  const Item8 it = wave_item8<1>(d, segs8, bx, item0, item_end, 0);
  const bool scale_lane = it.ok0 && (lane % kFp8BlockLanes) == 0;
  const int blk = it.c0 / kFp8BlockChunks;
  const int64_t at = (int64_t)it.t * d.k;
  int slot[KMAX], p[KMAX];
  u32x2 a[KMAX], b[KMAX];
  float sc[KMAX];
  int sj[KMAX], pj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {  // no branch between the loads: they issue together
    const int64_t a = slot_index(at, j, d.k);
    sj[j] = w.slot_of[a];
    pj[j] = w.stage_of[a];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool has = it.live && j < d.k;
    slot[j] = has ? sj[j] : -1;
    p[j] = has ? pj[j] : -1;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    bool first = (uint32_t)p[j] < srows;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) first = first && p[jj] != p[j];
    if (first && it.ok0) {
      load_codes(stage8, p[j], d, it, a[j], b[j]);
      if (scale_lane) sc[j] = sscale[(int64_t)p[j] * nb + blk];
    }
    if (!first) p[j] = p[j] < 0 ? -1 : -2 - p[j];  // later slot of a node: -2-row
  }
  if (!it.ok0) return;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (p[j] < 0) continue;  // j is the first slot of its node: write all of the node's slots
#pragma unroll
    for (int jj = j; jj < KMAX; ++jj) {
      const bool same = jj == j || p[jj] == -2 - p[j];
      if (same && (uint32_t)slot[jj] < rows) {
        store_codes(recv8, slot[jj], d, it, a[j], b[j], keep_rows((int64_t)d.T * d.k, d.H));
        if (scale_lane) rscale[(int64_t)slot[jj] * nb + blk] = sc[j];
      }
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(kBlock) void stage_a_fp8_kernel(Dims d, const int32_t* __restrict__ idx,
                                                             const u32x4* __restrict__ x,
                                                             uint8_t* __restrict__ stage8,
                                                             float* __restrict__ sscale, Work w,
                                                             int item0, int item_end, int keep) {
  stage_a_fp8_body<KMAX>(d, idx, x, stage8, sscale, w, blockIdx.x, item0, item_end, keep);
}

template <int KMAX>
__global__ __launch_bounds__(kBlock) void stage_b_fp8_kernel(Dims d, const uint8_t* __restrict__ stage8,
                                                             const float* __restrict__ sscale,
                                                             uint8_t* __restrict__ recv8,
                                                             float* __restrict__ rscale, Work w,
                                                             int item0, int item_end) {
  stage_b_fp8_body<KMAX>(d, stage8, sscale, recv8, rscale, w, blockIdx.x, item0, item_end);
}

// Hop 2 of chunk c and hop 1 of chunk c + 1 in one launch, as stage_ab_kernel.
template <int KMAX>
__global__ __launch_bounds__(kBlock) void stage_ab_fp8_kernel(Dims d, const int32_t* __restrict__ idx,
                                                              const u32x4* __restrict__ x,
                                                              uint8_t* __restrict__ stage8,
                                                              float* __restrict__ sscale,
                                                              uint8_t* __restrict__ recv8,
                                                              float* __restrict__ rscale, Work w,
                                                              int b_blocks, int b_item0,
                                                              int b_item_end, int a_item0,
                                                              int a_item_end, int keep) {
  if ((int)blockIdx.x < b_blocks)
    stage_b_fp8_body<KMAX>(d, stage8, sscale, recv8, rscale, w, blockIdx.x, b_item0, b_item_end);
  else
    stage_a_fp8_body<KMAX>(d, idx, x, stage8, sscale, w, blockIdx.x - b_blocks, a_item0,
                           a_item_end, keep);
}

// Combine of an fp8 payload: codes decoded and scaled (exact), then the same
// fp32 fused multiply-add chain as the bf16 combine.
template <int KMAX, int U, bool F32OUT>
__global__ __launch_bounds__(kCombine8Waves * kWave) void combine_fp8_kernel(Dims d, const u32x2* __restrict__ y8,
                                                             const float* __restrict__ yscale,
                                                             const float* __restrict__ wts,
                                                             const int32_t* __restrict__ slot_of,
                                                             void* __restrict__ out, int base,
                                                             int limit) {
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  Item it[U];
  int slot[U][KMAX];
  float wj[U][KMAX], sc[U][KMAX];
  u32x2 v[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U, kCombine8Waves>(d, blockIdx.x, base, limit, u);
    const int64_t at = (int64_t)it[u].t * d.k;
    const int blk = it[u].c / kFp8BlockChunks;
    int sj[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {  // no branch between the loads: they issue together
      const int64_t a = slot_index(at, j, d.k);
      sj[j] = slot_of[a];
      wt[j] = wts[a];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool has = it[u].live && j < d.k;
      slot[u][j] = has && (uint32_t)sj[j] < rows ? sj[j] : -1;
      wj[u][j] = has ? wt[j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (slot[u][j] >= 0 && it[u].ok) {
        v[u][j] = __builtin_nontemporal_load(&y8[(int64_t)slot[u][j] * d.chunks + it[u].c]);
        sc[u][j] = yscale[(int64_t)slot[u][j] * nb + blk];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!it[u].ok) continue;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (slot[u][j] < 0) continue;
      float f[8];
      decode_e4m3x8(v[u][j], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wj[u][j], f[q] * sc[u][j], acc[q]);
    }
    const int64_t i = (int64_t)it[u].t * d.chunks + it[u].c;
    if constexpr (F32OUT) {
      f32x4* o = reinterpret_cast<f32x4*>(out) + i * 2;
      const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
      const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
      store_chunk(o, a);
      store_chunk(o + 1, b);
    } else {
      u32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
      store_chunk(reinterpret_cast<u32x4*>(out) + i, r);
    }
  }
}

// Launches f(grid, base, limit) -> hipError_t over wave-items [0, items), at
// most kMaxLaunchItems a launch, per_block wave-items a block.
template <typename F>
hipError_t launch_ranges(int64_t items, int per_block, F f) {
  for (int64_t base = 0; base < items; base += kMaxLaunchItems) {
    const int64_t limit = std::min<int64_t>(items, base + kMaxLaunchItems);
    const hipError_t e =
        f(dim3((unsigned)((limit - base + per_block - 1) / per_block)), (int)base, (int)limit);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <template <int> class Launch, typename... A>
hipError_t by_topk(int k, A... a) {
  if (k <= 2) return Launch<2>::run(a...);
  if (k <= 4) return Launch<4>::run(a...);
  if (k <= 8) return Launch<8>::run(a...);
  return Launch<16>::run(a...);
}

template <int KMAX>
struct GatherLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                        const Work& w, hipStream_t s) {
    const int64_t items = (int64_t)d.T * d.segs;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    u32x4* rv = reinterpret_cast<u32x4*>(recv);
    if (d.fused_scan) {
      // larger blocks where the experts fit one wave: fewer blocks redo the scan
      if (d.E <= kWave)
        return launch_ranges(items, kGatherScanWaves * kGatherScanU, [&](dim3 g, int b, int l) {
          return launch(MOE_KERNEL_GATHER_SCAN, gather_scan_kernel<KMAX, kGatherScanWaves, kGatherScanU>,
                        g, dim3(kGatherScanWaves * kWave), 0, s, d, idx, xv, rv, w, b, l);
        });
      return launch_ranges(items, kGatherScanWavesWide * kGatherScanUWide, [&](dim3 g, int b, int l) {
        return launch(MOE_KERNEL_GATHER_SCAN,
                      gather_scan_kernel<KMAX, kGatherScanWavesWide, kGatherScanUWide>, g,
                      dim3(kGatherScanWavesWide * kWave), 0, s, d, idx, xv, rv, w, b, l);
      });
    }
    return launch_ranges(items, kWaves * kGatherU, [&](dim3 g, int b, int l) {
      return launch(MOE_KERNEL_GATHER, gather_kernel<KMAX, kGatherU>, g, dim3(kBlock), 0, s, d, idx,
                    xv, rv, w, b, l);
    });
  }
};

// Tokens per chunk of the deduplicated dispatch: even chunks, each with at
// most kChunkBytes of staging rows (row_bound bytes a token, at most).
inline int stage_chunk_tokens(const Dims& d, int64_t row_bound) {
  const int64_t n = std::max<int64_t>(1, ((int64_t)d.T * row_bound + kChunkBytes - 1) / kChunkBytes);
  return (int)(((int64_t)d.T + n - 1) / n);
}

// Deduplicated dispatch over chunks of consecutive tokens: hop 1, then hop
// 2, of each chunk after the previous chunk's.  A chunk's staging rows (at
// most tokens * min(k, N) rows) fit in the 256 MB MALL, so hop 2 reads rows
// hop 1 has just written (DeepSeek-V3-like, 8 chunks: dispatch 799 -> 756
// us on one stream).  Launches: hop 1 of chunk 0, then one stage_ab launch
// per chunk boundary (hop 2 of chunk c with hop 1 of chunk c + 1), then hop
// 2 of the last chunk.  The rows, and the plan arrays hop 1 finishes, of one
// chunk are disjoint from every other chunk's.  (Running hop 1 of chunk c +
// 1 on a second stream beside hop 2 of chunk c instead made both hops far
// slower, 0.30 and 0.49 of the HBM peak: two write-heavy grids at full width
// contend.)
template <int KMAX>
struct DedupLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* staging,
                        uint16_t* recv, const Work& w, hipStream_t s) {
    const int64_t row_bound = (int64_t)min(d.k, d.N) * 2 * d.H;  // staging bytes per token, at most
    const int chunk = stage_chunk_tokens(d, row_bound);
    const int nch = (d.T + chunk - 1) / chunk;
    const int keep = (int64_t)chunk * row_bound <= kKeepBytes;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    u32x4* sv = reinterpret_cast<u32x4*>(staging);
    u32x4* rv = reinterpret_cast<u32x4*>(recv);
    auto first = [&](int c) { return c * chunk * d.segs; };
    auto last = [&](int c) { return min(d.T, (c + 1) * chunk) * d.segs; };
    auto blocks = [](int items, int per_block) { return (items + per_block - 1) / per_block; };
    const int per_a = kWaves * kStageAU, per_b = kWaves * kStageU;
    hipError_t e = launch(MOE_KERNEL_STAGE_A, stage_a_kernel<KMAX, kStageAU>,
                          dim3(blocks(last(0) - first(0), per_a)), dim3(kBlock), 0, s, d, idx, xv, sv,
                          w, first(0), last(0), keep);
    for (int c = 0; c + 1 < nch && e == hipSuccess; ++c) {
      const int bb = blocks(last(c) - first(c), kWaves);  // one wave-item a wave
      const int ba = blocks(last(c + 1) - first(c + 1), per_a);
      e = launch(MOE_KERNEL_STAGE_AB, stage_ab_kernel<KMAX>, dim3(bb + ba), dim3(kBlock), 0, s, d,
                 idx, xv, sv, rv, w, bb, first(c), last(c), first(c + 1), last(c + 1), keep);
    }
    if (e == hipSuccess)
      e = launch(MOE_KERNEL_STAGE_B, stage_b_kernel<KMAX, kStageU>,
                 dim3(blocks(last(nch - 1) - first(nch - 1), per_b)), dim3(kBlock), 0, s, d,
                 static_cast<const u32x4*>(sv), rv, w, first(nch - 1), last(nch - 1));
    return e;
  }
};

template <int KMAX>
struct CombineLaunch {
  static hipError_t run(const Dims& d, const uint16_t* y, const float* wts, void* out, bool f32,
                        const Work& w, hipStream_t s) {
    const u32x4* yv = reinterpret_cast<const u32x4*>(y);
    const dim3 block(kCombineWaves * kWave);
    return launch_ranges((int64_t)d.T * d.segs, kCombineWaves * kCombineU, [&](dim3 g, int b, int l) {
      if (f32)
        return launch(MOE_KERNEL_COMBINE, combine_kernel<KMAX, kCombineU, true>, g, block, 0, s, d,
                      yv, wts, w.slot_of, out, b, l);
      return launch(MOE_KERNEL_COMBINE, combine_kernel<KMAX, kCombineU, false>, g, block, 0, s, d,
                    yv, wts, w.slot_of, out, b, l);
    });
  }
};

template <int KMAX>
struct GatherFp8Launch {
  static hipError_t run(const Dims& d, const int32_t* idx, const uint16_t* x, uint8_t* recv8,
                        float* rscale, const Work& w, hipStream_t s) {
    const int64_t items = (int64_t)d.T * ((d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks);
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    if (fp8_fused_scan(d))
      return launch_ranges(items, kGatherScan8Waves * kGatherScan8U, [&](dim3 g, int b, int l) {
        return launch(MOE_KERNEL_GATHER_FP8_SCAN,
                      gather_fp8_scan_kernel<KMAX, kGatherScan8Waves, kGatherScan8U>, g,
                      dim3(kGatherScan8Waves * kWave), 0, s, d, idx, xv, recv8, rscale, w, b, l);
      });
    return launch_ranges(items, kWaves, [&](dim3 g, int b, int l) {
      return launch(MOE_KERNEL_GATHER_FP8, gather_fp8_kernel<KMAX>, g, dim3(kBlock), 0, s, d, idx,
                    xv, recv8, rscale, w, b, l);
    });
  }
};

// Tokens per chunk of the deduplicated fp8 dispatch (codes and scales:
// min(k, N) * (H + 4 * nb) staging bytes a token, at most).
inline int stage_chunk_tokens_fp8(const Dims& d) {
  const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
  return stage_chunk_tokens(d, (int64_t)min(d.k, d.N) * (d.H + 4 * nb));
}

// The deduplicated fp8 dispatch in chunks of tokens, with the launches of
// DedupLaunch: hop 1 of chunk 0, hop 2 of chunk c with hop 1 of chunk c + 1,
// hop 2 of the last chunk.
template <int KMAX>
struct DedupFp8Launch {
  static hipError_t run(const Dims& d, const int32_t* idx, const uint16_t* x, uint8_t* stage8,
                        float* sscale, uint8_t* recv8, float* rscale, const Work& w,
                        hipStream_t s) {
    const int segs8 = (d.chunks + kFp8ItemChunks - 1) / kFp8ItemChunks;
    const int nb = (d.chunks + kFp8BlockChunks - 1) / kFp8BlockChunks;
    const int64_t row_bound = (int64_t)min(d.k, d.N) * (d.H + 4 * nb);  // codes + scales
    const int chunk = stage_chunk_tokens_fp8(d);
    const int nch = (d.T + chunk - 1) / chunk;
    const int keep = (int64_t)chunk * row_bound <= kKeepBytes;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    auto first = [&](int c) { return c * chunk * segs8; };
    auto last = [&](int c) { return min(d.T, (c + 1) * chunk) * segs8; };
    auto blocks = [](int items) { return (items + kWaves - 1) / kWaves; };
    hipError_t e = launch(MOE_KERNEL_STAGE_A_FP8, stage_a_fp8_kernel<KMAX>,
                          dim3(blocks(last(0) - first(0))), dim3(kBlock), 0, s, d, idx, xv, stage8,
                          sscale, w, first(0), last(0), keep);
    for (int c = 0; c + 1 < nch && e == hipSuccess; ++c) {
      const int bb = blocks(last(c) - first(c)), ba = blocks(last(c + 1) - first(c + 1));
      e = launch(MOE_KERNEL_STAGE_AB_FP8, stage_ab_fp8_kernel<KMAX>, dim3(bb + ba), dim3(kBlock), 0,
                 s, d, idx, xv, stage8, sscale, recv8, rscale, w, bb, first(c), last(c),
                 first(c + 1), last(c + 1), keep);
    }
    if (e == hipSuccess)
      e = launch(MOE_KERNEL_STAGE_B_FP8, stage_b_fp8_kernel<KMAX>,
                 dim3(blocks(last(nch - 1) - first(nch - 1))), dim3(kBlock), 0, s, d,
                 static_cast<const uint8_t*>(stage8), static_cast<const float*>(sscale), recv8,
                 rscale, w, first(nch - 1), last(nch - 1));
    return e;
  }
};

template <int KMAX>
struct CombineFp8Launch {
  static hipError_t run(const Dims& d, const uint8_t* y8, const float* yscale, const float* wts,
                        void* out, bool f32, const Work& w, hipStream_t s) {
    const u32x2* y = reinterpret_cast<const u32x2*>(y8);
    const dim3 block(kCombine8Waves * kWave);
    return launch_ranges((int64_t)d.T * d.segs, kCombine8Waves * kCombine8U, [&](dim3 g, int b, int l) {
      if (f32)
        return launch(MOE_KERNEL_COMBINE_FP8, combine_fp8_kernel<KMAX, kCombine8U, true>, g, block, 0,
                      s, d, y, yscale, wts, w.slot_of, out, b, l);
      return launch(MOE_KERNEL_COMBINE_FP8, combine_fp8_kernel<KMAX, kCombine8U, false>, g, block, 0,
                    s, d, y, yscale, wts, w.slot_of, out, b, l);
    });
  }
};

// Tokens per chunk of the hierarchical combine: even chunks, each with at
// most kHierChunkBytes of fp32 partial rows (min(k, N) rows a token, at most).
inline int hier_chunk_tokens(const Dims& d) {
  const int64_t row_bound = (int64_t)min(d.k, d.N) * 4 * d.H;
  const int64_t n = std::max<int64_t>(1, ((int64_t)d.T * row_bound + kHierChunkBytes - 1) / kHierChunkBytes);
  return (int)(((int64_t)d.T + n - 1) / n);
}

// The hierarchical combine in chunks of consecutive tokens: hop 1, then hop
// 2, of each chunk after the previous chunk's, so hop 2 reads partials hop 1
// has just written (at most kHierChunkBytes of partial rows a chunk,
// counting min(k, N) rows a token; the node-limited workload uses about
// half).  Launches as DedupLaunch: hop 1 of chunk 0, hop 2 of chunk c with
// hop 1 of chunk c + 1 (combine_pn), hop 2 of the last chunk.
template <int KMAX>
struct CombineHierLaunch {
  template <bool F32OUT>
  static hipError_t go(const Dims& d, const uint16_t* y, const float* wts, float* part, void* out,
                       const Work& w, hipStream_t s) {
    const int64_t row_bound = (int64_t)min(d.k, d.N) * 4 * d.H;  // partial bytes per token, at most
    const int chunk = hier_chunk_tokens(d);
    const int nch = (d.T + chunk - 1) / chunk;
    const int keep = (int64_t)chunk * row_bound <= kKeepBytes;
    const u32x4* yv = reinterpret_cast<const u32x4*>(y);
    f32x4* pp = reinterpret_cast<f32x4*>(part);
    auto first = [&](int c) { return c * chunk * d.segs; };
    auto last = [&](int c) { return min(d.T, (c + 1) * chunk) * d.segs; };
    auto blocks = [](int items) { return (items + kWaves - 1) / kWaves; };
    hipError_t e = launch(MOE_KERNEL_COMBINE_PART, combine_part_kernel<KMAX>,
                          dim3(blocks(last(0) - first(0))), dim3(kBlock), 0, s, d, yv, wts, pp, w,
                          first(0), last(0), keep);
    for (int c = 0; c + 1 < nch && e == hipSuccess; ++c) {
      const int bb = blocks(last(c) - first(c)), bp = blocks(last(c + 1) - first(c + 1));
      e = launch(MOE_KERNEL_COMBINE_PN, combine_pn_kernel<KMAX, F32OUT>, dim3(bb + bp), dim3(kBlock),
                 0, s, d, yv, wts, pp, w, out, bb, first(c), last(c), first(c + 1), last(c + 1),
                 keep);
    }
    if (e == hipSuccess)
      e = launch(MOE_KERNEL_COMBINE_NODES, combine_nodes_kernel<KMAX, F32OUT>,
                 dim3(blocks(last(nch - 1) - first(nch - 1))), dim3(kBlock), 0, s, d,
                 static_cast<const f32x4*>(pp), w, out, first(nch - 1), last(nch - 1));
    return e;
  }
  static hipError_t run(const Dims& d, const uint16_t* y, const float* wts,
                        float* part, void* out, bool f32, const Work& w, hipStream_t s) {
    return f32 ? go<true>(d, y, wts, part, out, w, s) : go<false>(d, y, wts, part, out, w, s);
  }
};

}  // namespace

hipError_t launch_combine_hier(const Dims& d, const uint16_t* y,
                               const float* wts, float* part, void* out, bool out_f32,
                               const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<CombineHierLaunch>(d.k, d, y, wts, part, out, out_f32, w, s);
}

hipError_t launch_gather_fp8(const Dims& d, const int32_t* idx, const uint16_t* x, uint8_t* recv8,
                             float* rscale, const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<GatherFp8Launch>(d.k, d, idx, x, recv8, rscale, w, s);
}

hipError_t launch_stage_fp8(const Dims& d, const int32_t* idx, const uint16_t* x,
                            uint8_t* stage8, float* sscale, uint8_t* recv8, float* rscale,
                            const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<DedupFp8Launch>(d.k, d, idx, x, stage8, sscale, recv8, rscale, w, s);
}

hipError_t launch_combine_fp8(const Dims& d, const uint8_t* y8, const float* yscale,
                              const float* wts, void* out, bool out_f32, const Work& w,
                              hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<CombineFp8Launch>(d.k, d, y8, yscale, wts, out, out_f32, w, s);
}

hipError_t launch_gather(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                         const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<GatherLaunch>(d.k, d, idx, x, recv, w, s);
}

int64_t chunk_tokens(const Dims& d, int call) {
  if (call == 1) return stage_chunk_tokens_fp8(d);
  if (call == 2) return hier_chunk_tokens(d);
  return stage_chunk_tokens(d, (int64_t)min(d.k, d.N) * 2 * d.H);
}

hipError_t launch_dedup_dispatch(const Dims& d, const int32_t* idx, const uint16_t* x,
                                 uint16_t* staging, uint16_t* recv, const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<DedupLaunch>(d.k, d, idx, x, staging, recv, w, s);
}

hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* wts, void* out,
                          bool out_f32, const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<CombineLaunch>(d.k, d, y, wts, out, out_f32, w, s);
}

}  // namespace moe
