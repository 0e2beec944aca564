// Device bodies of the route plan (per-tile counting with lane ballots, the
// per-band scan), shared by the route-plan kernels (route_plan.hip) and the
// banded pipeline (pipeline.hip).  See route_plan.hip for the method.
#pragma once

#include "moe_device.h"

namespace moe {
namespace {

// In-place exclusive scan of a[0..n) (n <= 4 * NT) by the whole block of NT
// threads; returns the total.  s_wsum: NT / 64 ints of LDS.
template <int NT = kPlanBlock>
__device__ __forceinline__ int block_exclusive_scan(int* a, int n, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int v[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid * 4 + i;
    v[i] = p < n ? a[p] : 0;
    sum += v[i];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int run = 0, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < NT / kWave; ++w2) {
    run += (w2 < wv) ? s_wsum[w2] : 0;
    total += s_wsum[w2];
  }
  run += incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid * 4 + i;
    if (p < n) a[p] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

// Sum of column c of a [nblk, W] tile-major matrix in LDS over tiles
// [b0, b1), with eight reads in flight at a time (one read and its wait per
// tile would make the sum a chain of LDS round trips).
__device__ __forceinline__ int column_sum(const int* s_mat, int W, int c, int b0, int b1) {
  int sum = 0, b = b0;
  for (; b + 8 <= b1; b += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_mat[(b + i) * W + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += v[i];
  }
  for (; b < b1; ++b) sum += s_mat[b * W + c];
  return sum;
}

// Writes the first row of tiles [b0, b1) of column c, the first of them at
// `run`, reading the counts eight at a time.
template <bool COH>
__device__ __forceinline__ void column_run(const int* s_mat, int W, int c, int b0, int b1, int run,
                                           int32_t* base) {
  int b = b0;
  for (; b + 8 <= b1; b += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_mat[(b + i) * W + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      st_plan<COH>(&base[(b + i) * W + c], run);
      run += v[i];
    }
  }
  for (; b < b1; ++b) {
    st_plan<COH>(&base[b * W + c], run);
    run += s_mat[b * W + c];
  }
}

// Column sums of a [nblk, W] tile-major matrix in LDS by a block of NT
// threads.  With W <= NT each column is cut into P = min(NT / W, nblk) parts
// of consecutive tiles, one part a thread (thread q * W + c takes part q of
// column c): the part sums go to s_part, are turned into exclusive prefixes
// over the column's parts in place, and the column totals go to tot[c].
// Returns P (0 when W > NT: then each thread sums whole columns and s_part is
// unused).  Ends with the block synchronised.
template <int NT>
__device__ __forceinline__ int column_parts(const int* s_mat, int W, int nblk, int* s_part,
                                            int* tot) {
  const int tid = threadIdx.x;
  if (W > NT) {
    for (int c = tid; c < W; c += NT) tot[c] = column_sum(s_mat, W, c, 0, nblk);
    __syncthreads();
    return 0;
  }
  const int P = max(1, min(NT / W, nblk));
  if (tid < P * W) {
    const int q = tid / W, c = tid - q * W;
    s_part[tid] = column_sum(s_mat, W, c, q * nblk / P, (q + 1) * nblk / P);
  }
  __syncthreads();
  if (tid < W) {
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int v = s_part[q * W + tid];
      s_part[q * W + tid] = run;
      run += v;
    }
    tot[tid] = run;
  }
  __syncthreads();
  return P;
}

// First row of every (tile, column) of a [nblk, W] matrix in LDS: column c
// starts at first(c), and each tile adds its count.  P and s_part as left by
// column_parts (P = 0: one thread per column).
template <bool COH, int NT, typename F>
__device__ __forceinline__ void column_bases(const int* s_mat, int W, int nblk, int P,
                                             const int* s_part, int32_t* base, F first) {
  const int tid = threadIdx.x;
  if (P == 0) {
    for (int c = tid; c < W; c += NT) column_run<COH>(s_mat, W, c, 0, nblk, first(c), base);
  } else if (tid < P * W) {
    const int q = tid / W, c = tid - q * W;
    column_run<COH>(s_mat, W, c, q * nblk / P, (q + 1) * nblk / P, first(c) + s_part[tid], base);
  }
}

// Scan of a [nblk, W] tile-major count matrix by a block of NT threads:
// column totals (to `totals` if given), exclusive offsets of the columns (to
// off[0..W]), and the first row of every (tile, column) (to base), all
// counted on from row0.  Leaves the offsets from 0 in s_tot; returns the
// grand total.  Needs W * nblk <= the LDS matrix; s_part holds NT ints.
template <bool COH = false, int NT = kPlanBlock>
__device__ __forceinline__ int scan_tiles(const int32_t* src, int32_t* base, int32_t* totals,
                                          int32_t* off, int W, int nblk, int row0, int* s_mat,
                                          int* s_tot, int* s_wsum, int* s_part) {
  const int tid = threadIdx.x, n = W * nblk;
#pragma unroll 16
  for (int i = tid; i < n; i += NT) s_mat[i] = ld_plan<COH>(&src[i]);
  __syncthreads();
  const int P = column_parts<NT>(s_mat, W, nblk, s_part, s_tot);
  if (totals)
    for (int c = tid; c < W; c += NT) totals[c] = s_tot[c];
  const int total = block_exclusive_scan<NT>(s_tot, W, s_wsum);
  column_bases<COH, NT>(s_mat, W, nblk, P, s_part, base, [&](int c) { return row0 + s_tot[c]; });
  for (int c = tid; c < W; c += NT) off[c] = row0 + s_tot[c];
  if (tid == 0) off[W] = row0 + total;
  __syncthreads();
  return total;
}

// LDS of one count tile: per-wave ballots [kPlanWaves * max(E, fkeys)] and
// running counts.  s_frun / s_node are used with node deduplication only.
struct CountLds {
  unsigned long long* mask;  // per-wave ballots                      [kPlanWaves * max(E, fkeys)]
  int* pre;                  // slots before each (wave, key) so far   [kPlanWaves * max(E, fkeys)]
  int* run;                  // tile's slots per expert so far        [E]
  int* frun;                 // tile's staging rows per key so far    [fkeys]
  int* node;                 // destination node of each expert       [E]
  int* bad;                  // [1]
};

// s_pre[w * W + c] = run[c] + the ballots of waves before w for key c: the
// number of the tile's slots with key c that come before wave w's tokens.
__device__ __forceinline__ void prefix_table(const unsigned long long* s_mask, int* s_pre,
                                             const int* s_run, int W) {
  for (int i = threadIdx.x; i < kPlanWaves * W; i += kPlanBlock) {
    const int wv = i / W, c = i - wv * W;
    // The ballots of all the earlier waves a wave can have are read together,
    // then those before wv added (a loop up to wv waited for each read).
    unsigned long long m[kPlanWaves - 1];
#pragma unroll
    for (int q = 0; q < kPlanWaves - 1; ++q) m[q] = s_mask[q * W + c];
    int n = s_run[c];
#pragma unroll
    for (int q = 0; q < kPlanWaves - 1; ++q) n += q < wv ? __popcll(m[q]) : 0;
    s_pre[i] = n;
  }
}

// One plan tile (tokens [tile * d.tile, (tile + 1) * d.tile)) by the whole
// block: in-tile ranks of every slot, the tile's per-expert counts and its
// bad-routing flag.
// COH: ranks, counts and flags are device-scope stores (read by other blocks
// of the same launch).
template <int KMAX, bool COH = false>
__device__ __forceinline__ void count_tile(const Dims& d, const int32_t* idx, const Work& w,
                                           int tile, const CountLds& L) {
  unsigned long long* s_mask = L.mask;
  int* s_pre = L.pre;
  int* s_run = L.run;
  int* s_frun = L.frun;
  int* s_node = L.node;
  int& s_bad = *L.bad;

  const int tid = threadIdx.x, wv = tid / kWave, lane = tid % kWave;
  const unsigned long long bit = 1ull << lane, below = bit - 1ull;
  const int E = d.E, R = d.R, k = d.k;

  for (int i = tid; i < E; i += kPlanBlock) {
    s_run[i] = 0;
    if (d.dedup) s_node[i] = split_part(i, d.ebase, d.erem) / d.G;
  }
  const int K = d.fkeys;
  if (d.dedup)
    for (int i = tid; i < K; i += kPlanBlock) s_frun[i] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  for (int pass = 0; pass < d.passes; ++pass) {
    const int t = tile * d.tile + pass * kPlanBlock + tid;
    const bool live = t < d.T;
    const int64_t at = (int64_t)t * k;
    for (int i = tid; i < kPlanWaves * E; i += kPlanBlock) s_mask[i] = 0;

    // Every id is loaded before any is used, with no per-token branch around
    // the loads (a dead token or an entry j >= k reads entry 0), so that they
    // are in flight together: behind branches, each load waited for the one
    // before it, eight HBM round trips for top-8 (a 256-token tile, after a
    // cache flush: 4.7-5.1 us of its 8-9 us).  A pass with no live token
    // reads nothing: an empty batch has no entry 0.
    int raw[KMAX];
    if (tile * d.tile + pass * kPlanBlock < d.T) {  // block-uniform
#pragma unroll
      for (int j = 0; j < KMAX; ++j) raw[j] = idx[live && j < k ? at + j : 0];
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) raw[j] = -1;
    }

    // An id outside [0, E) or repeated in the row is dropped (the first
    // occurrence of a repeat stays) and flags the routing as bad.
    int e[KMAX];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      int v = -1;
      if (live && j < k) {
        v = raw[j];
        if (v < 0 || v >= E) {
          bad = true;
          v = -1;
        }
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
          if (v >= 0 && e[jj] == v) {
            bad = true;
            v = -1;
          }
      }
      e[j] = v;
    }
    if (bad) s_bad = 1;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (e[j] >= 0) atomicOr(&s_mask[wv * E + e[j]], bit);
    __syncthreads();
    prefix_table(s_mask, s_pre, s_run, E);
    __syncthreads();
    // Both lookups of every slot are issued before any is used (a dropped
    // slot reads entry 0 and drops the value): behind per-slot branches each
    // slot's lookups waited for the slot before.
    int pre[KMAX];
    unsigned long long msk[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int c = wv * E + (e[j] >= 0 ? e[j] : 0);
      pre[j] = s_pre[c];
      msk[j] = s_mask[c];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (live && j < k) st_plan<COH>(&w.lr[at + j], e[j] >= 0 ? pre[j] + __popcll(msk[j] & below) : -1);
    for (int i = tid; i < E; i += kPlanBlock)
      s_run[i] = s_pre[(kPlanWaves - 1) * E + i] + __popcll(s_mask[(kPlanWaves - 1) * E + i]);

    if (d.dedup) {
      __syncthreads();
      for (int i = tid; i < kPlanWaves * K; i += kPlanBlock) s_mask[i] = 0;
      // Key of the first slot of each distinct destination node: the
      // forwarder rank n*G + owner(t) % G, or with load-aware forwarders the
      // (owner, node) pair n*R + owner (its forwarder is chosen by the scan).
      // Both are node-major, so a node's keys are contiguous.  Later slots
      // of the node point back to the first.
      const int owner = live ? split_part(t, d.tbase, d.trem) : 0;
      int nd[KMAX], key[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        nd[j] = e[j] >= 0 ? s_node[e[j]] : -1;
        key[j] = nd[j] < 0 ? -1 : d.load_aware ? nd[j] * R + owner : nd[j] * d.G + owner % d.G;
#pragma unroll
        for (int jj = j - 1; jj >= 0; --jj)
          if (nd[j] >= 0 && nd[jj] == nd[j]) key[j] = -2 - jj;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (key[j] >= 0) atomicOr(&s_mask[wv * K + key[j]], bit);
      __syncthreads();
      prefix_table(s_mask, s_pre, s_frun, K);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {  // all lookups first, as for the experts
        const int c = wv * K + (key[j] >= 0 ? key[j] : 0);
        pre[j] = s_pre[c];
        msk[j] = s_mask[c];
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (live && j < k) {
          w.fkey[at + j] = key[j];
          w.flr[at + j] = key[j] >= 0 ? pre[j] + __popcll(msk[j] & below) : -1;
        }
      }
      for (int i = tid; i < K; i += kPlanBlock)
        s_frun[i] = s_pre[(kPlanWaves - 1) * K + i] + __popcll(s_mask[(kPlanWaves - 1) * K + i]);
    }
    __syncthreads();
  }

  for (int i = tid; i < E; i += kPlanBlock) st_plan<COH>(&w.tile_counts[tile * E + i], s_run[i]);
  if (d.dedup)
    for (int i = tid; i < K; i += kPlanBlock) st_plan<COH>(&w.tile_fcounts[tile * K + i], s_frun[i]);
  if (d.load_aware) {
    // The tile's staging rows per node (the sum of the node's R keys, one
    // wave a node): the scan places the nodes one after another from these,
    // so that each node's keys can be scanned by a block of their own.
    for (int n = wv; n < d.N; n += kPlanWaves) {
      int v = 0;
      for (int s = lane; s < R; s += kWave) v += s_frun[n * R + s];
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) st_plan<COH>(&w.tile_ncounts[tile * d.N + n], v);
    }
  }
  if (tid == 0) st_plan<COH>(&w.tile_flags[tile], s_bad);
}

// Load-aware forwarders (FUSCO article, "load balancing and cross-node
// deduplication": forwarding follows the load and is spread evenly over a
// node's GPUs).  Keys are (owner s, node n) pairs, c = n * R + s; the load of
// a pair is its staging rows.  In each node the owners are ranked by load
// (more first, ties to the lower owner) and dealt to the node's G ranks in
// snake order, so the forwarder with local index g gets the R / G owners of
// ranks lap * G + g (even laps) and lap * G + G - 1 - g (odd laps).  Staging
// rows stay ordered by (forwarder, token); owners hold ascending token
// ranges, so inside a forwarder that is (owner, token).
//
// Node n by the whole block: a node's forwarders are ranks n * G .. n * G +
// G - 1, so its staging rows follow those of nodes 0 .. n - 1, whose number
// comes from the count's per-(tile, node) sums; the rest needs only node n's
// columns of the [tiles x pairs] matrix (R consecutive ones of the R * N), so
// the nodes are scanned by blocks of their own, side by side.  Each pair's first row is its
// forwarder's first row plus the loads of the forwarder's owners with a lower
// id: R / G terms, read through the node's owner-by-rank and load-by-rank
// tables.  With R <= 64 one wave ranks the owners, one lane an owner: a
// lane's rank counts the lanes ahead of it (R compares against values read
// from the other lanes).  Larger R ranks one owner a thread against the LDS
// load table.  Writes node n's entries of the forwarder table, stage_off and
// the (tile, pair) bases; the block of node 0 also writes D to ctrl.  Needs
// R * N <= 1024 (so R <= 512: load-aware plans have two nodes or more).
template <bool COH = false, int NT = kPlanBlock>
__device__ __forceinline__ void scan_load_aware(const Dims& d, const Work& w, int n, int* s_mat,
                                                int* s_tot, int* s_wsum, int* s_part) {
  constexpr int kMaxOwners = MOE_MAX_EXPERTS / 2;
  __shared__ int s_load[kMaxOwners];   // per owner: its staging rows in node n
  __shared__ int s_lbr[kMaxOwners];    // per rank: load of the owner of that rank
  __shared__ int s_order[kMaxOwners];  // per rank: owner of that rank
  __shared__ int s_rank[kMaxOwners];   // R > 64: per owner, its rank
  __shared__ int s_first[kMaxOwners];  // per owner: first staging row of (owner, n)
  __shared__ int s_g[kMaxOwners];      // per owner: local index of its forwarder
  __shared__ int s_red[2];             // staging rows of nodes before n, of all nodes
  const int tid = threadIdx.x, lane = tid % kWave, R = d.R, N = d.N, G = d.G, K = d.fkeys;
  const int nblk = d.nblk, laps = R / G;
  if (tid < 2) s_red[tid] = 0;
  // Node n's columns as a [tiles x owners] matrix, and the per-(tile, node)
  // sums, all loaded before any is used.
#pragma unroll 4
  for (int i = tid; i < nblk * R; i += NT) {
    const int b = i / R, s = i - b * R;
    s_mat[i] = ld_plan<COH>(&w.tile_fcounts[(int64_t)b * K + n * R + s]);
  }
  int before = 0, all = 0;
  for (int i = tid; i < nblk * N; i += NT) {
    const int v = ld_plan<COH>(&w.tile_ncounts[i]);
    all += v;
    before += (i % N) < n ? v : 0;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    before += __shfl_xor(before, o);
    all += __shfl_xor(all, o);
  }
  __syncthreads();
  if (lane == 0 && all != 0) {
    atomicAdd(&s_red[0], before);
    atomicAdd(&s_red[1], all);
  }
  const int P = column_parts<NT>(s_mat, R, nblk, s_part, s_load);
  if (R <= kWave) {
    if (tid < kWave) {
      const bool live = lane < R;
      const int l = live ? s_load[lane] : 0;
      // One key orders by load, then owner: a pair's load is at most the
      // owner's ceil(T / R) tokens, so l * R + R - 1 - lane < 2^32 and keys
      // are distinct.  Lanes past R hold key 0, which outranks no one.
      const uint32_t key = live ? (uint32_t)l * R + (R - 1 - lane) : 0u;
      int rank = 0;
#pragma unroll
      for (int j = 0; j < kWave; ++j)
        rank += (uint32_t)__builtin_amdgcn_readlane((int)key, j) > key ? 1 : 0;
      // The node's owners and loads by rank; only this wave reads them.
      if (live) {
        s_order[rank] = lane;
        s_lbr[rank] = l;
      }
      __builtin_amdgcn_wave_barrier();
      if (live) {
        const int lap = rank / G, pos = rank - lap * G;
        const int g = (lap & 1) ? G - 1 - pos : pos;
        int tot = 0, bef = 0;
        for (int l2 = 0; l2 < laps; ++l2) {
          const int r = l2 * G + ((l2 & 1) ? G - 1 - g : g);
          const int v = s_lbr[r];
          tot += v;
          bef += s_order[r] < lane ? v : 0;
        }
        if (lap == 0) s_tot[g] = tot;
        s_first[lane] = bef;
        s_g[lane] = g;
      }
    }
  } else {
    for (int s = tid; s < R; s += NT) {
      const int l = s_load[s];
      int rank = 0;
      for (int s2 = 0; s2 < R; ++s2) {
        const int l2 = s_load[s2];
        rank += (l2 > l || (l2 == l && s2 < s)) ? 1 : 0;
      }
      s_rank[s] = rank;
      s_order[rank] = s;
    }
    __syncthreads();
    // owner of the forwarder with local index g, lap `lap`
    auto owner = [&](int g, int lap) { return s_order[lap * G + ((lap & 1) ? G - 1 - g : g)]; };
    for (int g = tid; g < G; g += NT) {
      int tot = 0;
      for (int lap = 0; lap < laps; ++lap) tot += s_load[owner(g, lap)];
      s_tot[g] = tot;
    }
    for (int s = tid; s < R; s += NT) {
      const int rank = s_rank[s], lap = rank / G, pos = rank - lap * G;
      const int g = (lap & 1) ? G - 1 - pos : pos;
      int bef = 0;
      for (int l2 = 0; l2 < laps; ++l2) {
        const int o = owner(g, l2);
        bef += o < s ? s_load[o] : 0;
      }
      s_first[s] = bef;
      s_g[s] = g;
    }
  }
  __syncthreads();
  const int node_first = s_red[0], staged = s_red[1];
  block_exclusive_scan<NT>(s_tot, G, s_wsum);  // the node's forwarders, from the node's first row
  for (int g = tid; g < G; g += NT) w.stage_off[n * G + g] = node_first + s_tot[g];
  if (tid == 0 && n == N - 1) w.stage_off[R] = staged;
  if (tid == 0 && n == 0) w.ctrl[kCtrlStaged] = staged;
  for (int s = tid; s < R; s += NT) {
    const int g = s_g[s];
    s_first[s] += node_first + s_tot[g];
    w.fwd[s * N + n] = n * G + g;
  }
  __syncthreads();
  // First staging row of every (tile, pair) of node n: column s of the
  // node's matrix is pair n * R + s of the full one.
  if (P == 0) {
    for (int s = tid; s < R; s += NT) {
      int run = s_first[s];
      for (int b = 0; b < nblk; ++b) {
        st_plan<COH>(&w.tile_fbase[(int64_t)b * K + n * R + s], run);
        run += s_mat[b * R + s];
      }
    }
  } else if (tid < P * R) {
    const int q = tid / R, s = tid - q * R;
    int run = s_first[s] + s_part[tid];
    const int b1 = (q + 1) * nblk / P;
    for (int b = q * nblk / P; b < b1; ++b) {
      st_plan<COH>(&w.tile_fbase[(int64_t)b * K + n * R + s], run);
      run += s_mat[b * R + s];
    }
  }
}

// LDS of one band scan.
struct ScanLds {
  int* mat;   // count matrix of the band's tiles
  int* tot;   // [MOE_MAX_EXPERTS]
  int* wsum;  // [NT / 64]
  int* part;  // [NT] column parts
};

// One band by the whole block: scans its [tiles x experts] count matrix into
// base rows, the band's expert and rank offsets and its status.  The band's
// receive rows start at band * d.band * k.
template <bool COH = false, int NT = kPlanBlock>
__device__ __forceinline__ void scan_band(const Dims& d, const Work& w, int band,
                                          const ScanLds& L) {
  int* s_tot = L.tot;
  const int tid = threadIdx.x, E = d.E, R = d.R;
  const int t0 = band * d.tpb, nt = min(d.tpb, d.nblk - t0);
  const int row0 = band * d.band * d.k;
  const int rows = scan_tiles<COH, NT>(
      w.tile_counts + (int64_t)t0 * E, w.tile_base + (int64_t)t0 * E, w.counts + (int64_t)band * E,
      w.expert_off + (int64_t)band * (E + 1), E, nt, row0, L.mat, s_tot, L.wsum, L.part);
  int32_t* roff = w.rank_off + (int64_t)band * (R + 1);
  for (int r = tid; r <= R; r += NT) {
    const int first = r * d.ebase + min(r, d.erem);  // first expert of rank r
    roff[r] = row0 + (first < E ? s_tot[first] : rows);
  }
  int bad = 0;
  for (int b = tid; b < nt; b += NT) bad |= ld_plan<COH>(&w.tile_flags[t0 + b]);
  bad = __syncthreads_or(bad);
  if (tid == 0) w.band_status[band] = bad ? MOE_ERR_BAD_ROUTING : MOE_OK;
}

// The staging keys of a deduplicated plan (one band) by the whole block:
// the [tiles x keys] count matrix into staging base rows, the forwarder
// offsets and table, and the number of staging rows.  It reads nothing the
// expert-key scan writes, so the two run in separate blocks side by side.
// Load-aware forwarders take one block per node (`part` = the node); static
// ones one block (`part` = 0).
template <bool COH = false, int NT = kPlanBlock>
__device__ __forceinline__ void scan_stage_keys(const Dims& d, const Work& w, int part,
                                                const ScanLds& L) {
  if (d.load_aware) {
    scan_load_aware<COH, NT>(d, w, part, L.mat, L.tot, L.wsum, L.part);
    return;
  }
  const int tid = threadIdx.x;
  const int staged = scan_tiles<COH, NT>(w.tile_fcounts, w.tile_fbase, nullptr, w.stage_off, d.R,
                                         d.nblk, 0, L.mat, L.tot, L.wsum, L.part);
  for (int c = tid; c < d.R * d.N; c += NT) w.fwd[c] = (c % d.N) * d.G + (c / d.N) % d.G;
  if (tid == 0) w.ctrl[kCtrlStaged] = staged;
}

}  // namespace
}  // namespace moe
