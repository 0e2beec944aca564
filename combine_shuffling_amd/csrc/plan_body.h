// Device bodies of the route plan (per-tile counting with lane ballots, the
// per-band scan), shared by the route-plan kernels (route_plan.hip) and the
// banded pipeline (pipeline.hip).  See route_plan.hip for the method.
#pragma once

#include "moe_device.h"

namespace moe {
namespace {

// In-place exclusive scan of a[0..n) (n <= 4 * kPlanBlock) by the whole
// block; returns the total.  s_wsum: kPlanWaves ints of LDS.
__device__ int block_exclusive_scan(int* a, int n, int* s_wsum) {
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
  for (int w2 = 0; w2 < kPlanWaves; ++w2) {
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

// Scan of a [nblk, W] tile-major count matrix: column totals (to `totals` if
// given), exclusive offsets of the columns (to off[0..W]), and the first row
// of every (tile, column) (to base), all counted on from row0.  Leaves the
// offsets from 0 in s_tot; returns the grand total.  Needs W * nblk <=
// kScanLdsInts.
template <bool COH = false>
__device__ int scan_tiles(const int32_t* src, int32_t* base, int32_t* totals, int32_t* off, int W,
                          int nblk, int row0, int* s_mat, int* s_tot, int* s_wsum) {
  const int tid = threadIdx.x, n = W * nblk;
#pragma unroll 8
  for (int i = tid; i < n; i += kPlanBlock) s_mat[i] = ld_plan<COH>(&src[i]);
  __syncthreads();
  for (int c = tid; c < W; c += kPlanBlock) {
    int s = 0;
    for (int b = 0; b < nblk; ++b) s += s_mat[b * W + c];
    s_tot[c] = s;
    if (totals) totals[c] = s;
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_tot, W, s_wsum);
  for (int c = tid; c < W; c += kPlanBlock) {
    int run = row0 + s_tot[c];
    off[c] = run;
    for (int b = 0; b < nblk; ++b) {
      st_plan<COH>(&base[b * W + c], run);
      run += s_mat[b * W + c];
    }
  }
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
    int n = s_run[c];
    for (int q = 0; q < wv; ++q) n += __popcll(s_mask[q * W + c]);
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

    // An id outside [0, E) or repeated in the row is dropped (the first
    // occurrence of a repeat stays) and flags the routing as bad.
    int e[KMAX];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      int v = -1;
      if (live && j < k) {
        v = idx[at + j];
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
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (live && j < k) {
        const int r = e[j] >= 0 ? s_pre[wv * E + e[j]] + __popcll(s_mask[wv * E + e[j]] & below) : -1;
        st_plan<COH>(&w.lr[at + j], r);
      }
    }
    for (int i = tid; i < E; i += kPlanBlock)
      s_run[i] = s_pre[(kPlanWaves - 1) * E + i] + __popcll(s_mask[(kPlanWaves - 1) * E + i]);

    if (d.dedup) {
      __syncthreads();
      for (int i = tid; i < kPlanWaves * K; i += kPlanBlock) s_mask[i] = 0;
      // Key of the first slot of each distinct destination node: the
      // forwarder rank n*G + owner(t) % G, or with load-aware forwarders the
      // (owner, node) pair owner*N + n (its forwarder is chosen by the scan).
      // Later slots of the node point back to the first.
      const int owner = live ? split_part(t, d.tbase, d.trem) : 0;
      int nd[KMAX], key[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        nd[j] = e[j] >= 0 ? s_node[e[j]] : -1;
        key[j] = nd[j] < 0 ? -1 : d.load_aware ? owner * d.N + nd[j] : nd[j] * d.G + owner % d.G;
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
      for (int j = 0; j < KMAX; ++j) {
        if (live && j < k) {
          const int r =
              key[j] >= 0 ? s_pre[wv * K + key[j]] + __popcll(s_mask[wv * K + key[j]] & below) : -1;
          w.fkey[at + j] = key[j];
          w.flr[at + j] = r;
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
  if (tid == 0) st_plan<COH>(&w.tile_flags[tile], s_bad);
}

// Load-aware forwarders (FUSCO article, "load balancing and cross-node
// deduplication": forwarding follows the load and is spread evenly over a
// node's GPUs).  Keys are (owner s, node n) pairs; the load of a pair is its
// staging rows.  In each node the owners are ranked by load (more first, ties
// to the lower owner) and dealt to the node's G ranks in snake order.  Staging
// rows stay ordered by (forwarder, token); owners hold ascending token ranges,
// so inside a forwarder that is (owner, token).  Writes the forwarder table,
// stage_off and the (tile, pair) bases; returns D.  Needs R*N <= 1024 and
// nblk * R * N <= kScanLdsInts.
template <bool COH = false>
__device__ int scan_load_aware(const Dims& d, const Work& w, int* s_mat, int* s_tot, int* s_wsum) {
  __shared__ int s_load[MOE_MAX_EXPERTS];  // per pair
  __shared__ int s_fwd[MOE_MAX_EXPERTS];   // per pair
  const int tid = threadIdx.x, R = d.R, N = d.N, G = d.G, K = d.fkeys, nblk = d.nblk;
#pragma unroll 8
  for (int i = tid; i < K * nblk; i += kPlanBlock) s_mat[i] = ld_plan<COH>(&w.tile_fcounts[i]);
  __syncthreads();
  for (int c = tid; c < K; c += kPlanBlock) {
    int l = 0;
    for (int b = 0; b < nblk; ++b) l += s_mat[b * K + c];
    s_load[c] = l;
  }
  __syncthreads();
  for (int c = tid; c < K; c += kPlanBlock) {
    const int s = c / N, n = c % N, l = s_load[c];
    int rank = 0;
    for (int s2 = 0; s2 < R; ++s2) {
      const int l2 = s_load[s2 * N + n];
      rank += (l2 > l || (l2 == l && s2 < s)) ? 1 : 0;
    }
    const int lap = rank / G, pos = rank % G;
    const int f = n * G + ((lap & 1) ? G - 1 - pos : pos);
    s_fwd[c] = f;
    w.fwd[c] = f;
  }
  __syncthreads();
  for (int f = tid; f < R; f += kPlanBlock) {  // rows each forwarder stages
    const int n = f / G;
    int tot = 0;
    for (int s = 0; s < R; ++s) tot += s_fwd[s * N + n] == f ? s_load[s * N + n] : 0;
    s_tot[f] = tot;
  }
  __syncthreads();
  const int staged = block_exclusive_scan(s_tot, R, s_wsum);
  for (int f = tid; f <= R; f += kPlanBlock) w.stage_off[f] = f < R ? s_tot[f] : staged;
  for (int c = tid; c < K; c += kPlanBlock) {
    const int s = c / N, n = c % N, f = s_fwd[c];
    int run = s_tot[f];
    for (int s2 = 0; s2 < s; ++s2) run += s_fwd[s2 * N + n] == f ? s_load[s2 * N + n] : 0;
    for (int b = 0; b < nblk; ++b) {
      w.tile_fbase[b * K + c] = run;
      run += s_mat[b * K + c];
    }
  }
  __syncthreads();
  return staged;
}

// LDS of one band scan.
struct ScanLds {
  int* mat;   // [kScanLdsInts] count matrix of the band's tiles
  int* tot;   // [MOE_MAX_EXPERTS]
  int* wsum;  // [kPlanWaves]
};

// One band by the whole block: scans its [tiles x experts] count matrix (and,
// with dedup, which runs with one band only, the [tiles x staging keys] one)
// into base rows, the band's expert and rank offsets and its status.  The
// band's receive rows start at band * d.band * k.
template <bool DEDUP = true, bool COH = false>
__device__ __forceinline__ void scan_band(const Dims& d, const Work& w, int band,
                                          const ScanLds& L) {
  int* s_mat = L.mat;
  int* s_tot = L.tot;
  int* s_wsum = L.wsum;
  const int tid = threadIdx.x, E = d.E, R = d.R;
  const int t0 = band * d.tpb, nt = min(d.tpb, d.nblk - t0);
  const int row0 = band * d.band * d.k;
  const int rows = scan_tiles<COH>(w.tile_counts + (int64_t)t0 * E, w.tile_base + (int64_t)t0 * E,
                              w.counts + (int64_t)band * E, w.expert_off + (int64_t)band * (E + 1),
                              E, nt, row0, s_mat, s_tot, s_wsum);
  int32_t* roff = w.rank_off + (int64_t)band * (R + 1);
  for (int r = tid; r <= R; r += kPlanBlock) {
    const int first = r * d.ebase + min(r, d.erem);  // first expert of rank r
    roff[r] = row0 + (first < E ? s_tot[first] : rows);
  }
  int staged = 0;
  if (DEDUP && d.dedup) {
    __syncthreads();
    if (d.load_aware) {
      staged = scan_load_aware<COH>(d, w, s_mat, s_tot, s_wsum);
    } else {
      staged = scan_tiles<COH>(w.tile_fcounts, w.tile_fbase, nullptr, w.stage_off, R, d.nblk, 0,
                               s_mat, s_tot, s_wsum);
      for (int c = tid; c < R * d.N; c += kPlanBlock)
        w.fwd[c] = (c % d.N) * d.G + (c / d.N) % d.G;
    }
  }
  int bad = 0;
  for (int b = tid; b < nt; b += kPlanBlock) bad |= ld_plan<COH>(&w.tile_flags[t0 + b]);
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    w.band_status[band] = bad ? MOE_ERR_BAD_ROUTING : MOE_OK;
    if (DEDUP && d.dedup) w.ctrl[kCtrlStaged] = staged;
  }
}

}  // namespace
}  // namespace moe
