// Route plan on gfx950: per-expert histogram, exclusive scan and segment
// descriptors for the gather-send / scatter-recv shuffle (FUSCO article,
// "core innovation": the sender's reads are driven by segment descriptors).
//
// route_count  one block per tile of tokens (256 tokens per pass, 4 waves,
//              lane = token).  Each wave builds, for every expert, the 64-bit
//              ballot of its lanes routed to that expert: a lane holds k
//              experts, so the ballots are assembled in LDS with 64-bit OR
//              atomics (order-free, hence deterministic).  A slot's rank
//              inside the tile is the popcount of its expert's ballot below
//              the lane, plus the popcounts of the earlier waves' ballots and
//              of the earlier passes.  The tile's per-expert counts go to HBM.
// route_scan   one block loads the [tiles x experts] count matrix into LDS,
//              sums columns, scans the expert totals and writes every
//              (tile, expert) base row, the expert and rank offsets and the
//              status.  (Back-to-back kernels on one stream start with no gap
//              on this GPU, so the kernel boundary is the cheapest grid-wide
//              wait: cheaper than a last-arriving-block ticket with its
//              release / acquire fences.)
//
// With node deduplication the same is done a second time over the keys
// "forwarder rank of (token, node)" of the first slot of each distinct
// destination node of a token, which orders staging rows by (forwarder,
// token) (FUSCO article, "load balancing and cross-node deduplication": one
// copy per destination node through a forwarding GPU).
//
// A slot's receive row is then tile_base[tile][expert] + its in-tile rank:
// the stable (expert, token) order.  The data-movement kernels that run next
// finish slot_of / row_src (and stage_of / stage_src) on the fly; the
// per-token route_assign kernel does the same when a consumer needs the plan
// without a dispatch.
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
// of every (tile, column) (to base).  Leaves the offsets in s_tot; returns the
// grand total.  Needs W * nblk <= kScanLdsInts.
__device__ int scan_tiles(const int32_t* src, int32_t* base, int32_t* totals, int32_t* off, int W,
                          int nblk, int* s_mat, int* s_tot, int* s_wsum) {
  const int tid = threadIdx.x, n = W * nblk;
#pragma unroll 8
  for (int i = tid; i < n; i += kPlanBlock) s_mat[i] = src[i];
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
    int run = s_tot[c];
    off[c] = run;
    for (int b = 0; b < nblk; ++b) {
      base[b * W + c] = run;
      run += s_mat[b * W + c];
    }
  }
  if (tid == 0) off[W] = total;
  __syncthreads();
  return total;
}

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void route_count_kernel(Dims d,
                                                                 const int32_t* __restrict__ idx,
                                                                 Work w) {
  __shared__ unsigned long long s_mask[kPlanWaves * MOE_MAX_EXPERTS];  // per-wave ballots; 32 KiB
  __shared__ int s_run[MOE_MAX_EXPERTS];   // tile's slots per expert so far
  __shared__ int s_frun[MOE_MAX_EXPERTS];  // tile's staging rows per forwarder so far (R <= E)
  __shared__ int s_node[MOE_MAX_EXPERTS];  // destination node of each expert (dedup)
  __shared__ int s_bad;

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
    const int t = blockIdx.x * d.tile + pass * kPlanBlock + tid;
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
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (live && j < k) {
        int r = -1;
        if (e[j] >= 0) {
          r = s_run[e[j]] + __popcll(s_mask[wv * E + e[j]] & below);
          for (int w2 = 0; w2 < wv; ++w2) r += __popcll(s_mask[w2 * E + e[j]]);
        }
        w.lr[at + j] = r;
      }
    }
    __syncthreads();
    for (int i = tid; i < E; i += kPlanBlock)
      s_run[i] += __popcll(s_mask[i]) + __popcll(s_mask[E + i]) + __popcll(s_mask[2 * E + i]) +
                  __popcll(s_mask[3 * E + i]);

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
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (live && j < k) {
          int r = -1;
          if (key[j] >= 0) {
            r = s_frun[key[j]] + __popcll(s_mask[wv * K + key[j]] & below);
            for (int w2 = 0; w2 < wv; ++w2) r += __popcll(s_mask[w2 * K + key[j]]);
          }
          w.fkey[at + j] = key[j];
          w.flr[at + j] = r;
        }
      }
      __syncthreads();
      for (int i = tid; i < K; i += kPlanBlock)
        s_frun[i] += __popcll(s_mask[i]) + __popcll(s_mask[K + i]) + __popcll(s_mask[2 * K + i]) +
                     __popcll(s_mask[3 * K + i]);
    }
    __syncthreads();
  }

  for (int i = tid; i < E; i += kPlanBlock) w.tile_counts[blockIdx.x * E + i] = s_run[i];
  if (d.dedup)
    for (int i = tid; i < K; i += kPlanBlock) w.tile_fcounts[blockIdx.x * K + i] = s_frun[i];
  if (tid == 0) w.tile_flags[blockIdx.x] = s_bad;
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
__device__ int scan_load_aware(const Dims& d, const Work& w, int* s_mat, int* s_tot, int* s_wsum) {
  __shared__ int s_load[MOE_MAX_EXPERTS];  // per pair
  __shared__ int s_fwd[MOE_MAX_EXPERTS];   // per pair
  const int tid = threadIdx.x, R = d.R, N = d.N, G = d.G, K = d.fkeys, nblk = d.nblk;
#pragma unroll 8
  for (int i = tid; i < K * nblk; i += kPlanBlock) s_mat[i] = w.tile_fcounts[i];
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

// One block: scans the [tiles x experts] count matrix (and, with dedup, the
// [tiles x forwarders] one) into base rows, offsets and the status.
__global__ __launch_bounds__(kPlanBlock) void route_scan_kernel(Dims d, Work w) {
  __shared__ int s_mat[kScanLdsInts];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[kPlanWaves];
  const int tid = threadIdx.x, E = d.E, R = d.R;
  const int rows = scan_tiles(w.tile_counts, w.tile_base, w.counts, w.expert_off, E, d.nblk, s_mat,
                              s_tot, s_wsum);
  for (int r = tid; r <= R; r += kPlanBlock) {
    const int first = r * d.ebase + min(r, d.erem);  // first expert of rank r
    w.rank_off[r] = first < E ? s_tot[first] : rows;
  }
  int staged = 0;
  if (d.dedup) {
    __syncthreads();
    if (d.load_aware) {
      staged = scan_load_aware(d, w, s_mat, s_tot, s_wsum);
    } else {
      staged = scan_tiles(w.tile_fcounts, w.tile_fbase, nullptr, w.stage_off, R, d.nblk, s_mat,
                          s_tot, s_wsum);
      for (int c = tid; c < R * d.N; c += kPlanBlock)
        w.fwd[c] = (c % d.N) * d.G + (c / d.N) % d.G;
    }
  }
  int bad = 0;
  for (int b = tid; b < d.nblk; b += kPlanBlock) bad |= w.tile_flags[b];
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    w.ctrl[kCtrlStatus] = bad ? MOE_ERR_BAD_ROUTING : MOE_OK;
    w.ctrl[kCtrlStaged] = staged;
  }
}

// Finishes the plan one token per thread (slot_of, row_src; with dedup
// stage_of, stage_src) for consumers that run without a dispatch.
template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void route_assign_kernel(Dims d,
                                                                  const int32_t* __restrict__ idx,
                                                                  Work w) {
  const int t = blockIdx.x * kPlanBlock + threadIdx.x;
  if (t >= d.T) return;
  const int64_t at = (int64_t)t * d.k;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  int slot[KMAX];
  token_slots<KMAX>(d, w, idx, t, slot);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < d.k) {
      w.slot_of[at + j] = slot[j];
      if ((uint32_t)slot[j] < rows) w.row_src[slot[j]] = t;
    }
  }
  if (d.dedup) {
    int p[KMAX];
    uint32_t lead;
    token_stages<KMAX>(d, w, t, p, lead);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < d.k) {
        w.stage_of[at + j] = p[j];
        if (((lead >> j) & 1u) && (uint32_t)p[j] < (uint32_t)d.smax) w.stage_src[p[j]] = t;
      }
    }
  }
}

// Modelled link traffic for plan reads (not on the shuffle's path): rows,
// distinct tokens per destination rank, and distinct tokens per destination
// node, for every owner rank.  Counters must be zero on entry.
template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void traffic_kernel(Dims d, const int32_t* __restrict__ idx,
                                                             Work w) {
  const int t = blockIdx.x * kPlanBlock + threadIdx.x;
  if (t >= d.T) return;
  const int64_t at = (int64_t)t * d.k;
  const int s = split_part(t, d.tbase, d.trem);
  int dr[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    dr[j] = -1;
    if (j < d.k && w.slot_of[at + j] >= 0) dr[j] = split_part(idx[at + j], d.ebase, d.erem);
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (dr[j] < 0) continue;
    atomicAdd(&w.send_rows[s * d.R + dr[j]], 1);
    bool new_rank = true, new_node = true;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) {
      if (dr[jj] < 0) continue;
      new_rank = new_rank && dr[jj] != dr[j];
      new_node = new_node && dr[jj] / d.G != dr[j] / d.G;
    }
    if (new_rank) atomicAdd(&w.send_copies[s * d.R + dr[j]], 1);
    if (new_node) atomicAdd(&w.node_copies[s * d.N + dr[j] / d.G], 1);
  }
}

template <template <int> class Launch, typename... A>
hipError_t by_topk(int k, A... a) {
  if (k <= 2) return Launch<2>::run(a...);
  if (k <= 4) return Launch<4>::run(a...);
  if (k <= 8) return Launch<8>::run(a...);
  return Launch<16>::run(a...);
}

template <int KMAX>
struct CountLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
    hipLaunchKernelGGL(route_count_kernel<KMAX>, dim3(d.nblk), dim3(kPlanBlock), 0, s, d, idx, w);
    return hipGetLastError();
  }
};

template <int KMAX>
struct AssignLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
    const int blocks = (d.T + kPlanBlock - 1) / kPlanBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(route_assign_kernel<KMAX>, dim3(blocks), dim3(kPlanBlock), 0, s, d, idx, w);
    return hipGetLastError();
  }
};

template <int KMAX>
struct TrafficLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
    const int blocks = (d.T + kPlanBlock - 1) / kPlanBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(traffic_kernel<KMAX>, dim3(blocks), dim3(kPlanBlock), 0, s, d, idx, w);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_route_count(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  const hipError_t e = by_topk<CountLaunch>(d.k, d, idx, w, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kPlanBlock), 0, s, d, w);
  return hipGetLastError();
}

hipError_t launch_route_assign(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<AssignLaunch>(d.k, d, idx, w, s);
}

hipError_t launch_traffic(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<TrafficLaunch>(d.k, d, idx, w, s);
}

}  // namespace moe
