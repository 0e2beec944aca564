// Route plan on gfx950: per-expert histogram, exclusive scan and segment
// descriptors for the gather-send / scatter-recv shuffle (FUSCO article,
// "core innovation": the sender's reads are driven by segment descriptors).
//
// Two launches, no atomics, no grid-wide wait, deterministic:
//
//  route_count   one block per tile of tokens (256 tokens per pass, 4 waves,
//                lane = token).  Validates the tile's routing, and gives every
//                slot (t, j) its rank among the earlier slots of the tile that
//                name the same expert.  Ranks come from a wavefront
//                ballot-match: for slot position q the wave takes one ballot
//                per bit of the expert id, and every lane rebuilds from those
//                ballots the mask of lanes whose q-th expert equals its own;
//                OR-ing over q gives all lanes that name the expert, its
//                popcount below the lane is the in-wave rank, and the lowest
//                such lane publishes the wave's count in LDS.  Earlier waves'
//                counts (and earlier passes') are added from LDS.  Writes the
//                tile's per-expert counts and the in-tile ranks.
//
//  route_assign  one block per tile again.  Each block sums the tile counts
//                over all tiles and over the tiles before its own (at most 64
//                tiles, so one batch of loads per thread), scans the totals
//                into expert offsets in LDS, and turns every in-tile rank into
//                a receive row: row = expert_off[e] + rows of e in earlier
//                tiles + in-tile rank.  That is the stable (expert, token)
//                order.  Block 0 also publishes counts, offsets and status.
//
// With node deduplication the same machinery runs a second time over the keys
// "forwarder rank of (token, node)" for the first slot of each distinct node
// of a token, giving staging rows ordered by (forwarder, token) (FUSCO
// article, "load balancing and cross-node deduplication": one copy per
// destination node through a forwarding GPU).
//
// Expert -> rank and token -> owner use the contiguous ceil/floor split of
// TensorRT-LLM PR #13888 ("support non-divisible EP in MoE alltoall",
// performance commit message), with base and remainder hoisted into the
// kernel arguments and a single divide when the remainder is zero.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int split_part(int i, int base, int rem) {
  if (rem == 0) return i / base;
  const int cut = rem * (base + 1);
  return i < cut ? i / (base + 1) : rem + (i - cut) / base;
}

// For every j, m[j] = lanes holding v[j] (of the calling lane) in any of
// their k positions.  Values < 0 are absent and match nothing; the mask of
// an absent v[j] is meaningless.  Must be called by the whole wave.
template <int KMAX>
__device__ __forceinline__ void wave_match(const int (&v)[KMAX], int k, int nbits,
                                           uint64_t (&m)[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) m[j] = 0;
#pragma unroll
  for (int q = 0; q < KMAX; ++q) {
    if (q < k) {
      uint64_t acc[KMAX];
      const uint64_t present = __ballot(v[q] >= 0);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) acc[j] = present;
      for (int b = 0; b < nbits; ++b) {
        const uint64_t ones = __ballot((v[q] >> b) & 1);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) acc[j] &= ((v[j] >> b) & 1) ? ones : ~ones;
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) m[j] |= acc[j];
    }
  }
}

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

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void route_count_kernel(Dims d,
                                                                 const int32_t* __restrict__ idx,
                                                                 Work w) {
  __shared__ int s_wc[kPlanWaves * MOE_MAX_EXPERTS];   // per-wave expert counts
  __shared__ int s_run[MOE_MAX_EXPERTS];               // tile counts so far
  __shared__ int s_fwc[kPlanWaves * MOE_MAX_EXPERTS];  // per-wave forwarder counts (R <= E)
  __shared__ int s_frun[MOE_MAX_EXPERTS];
  __shared__ int s_bad;

  const int tid = threadIdx.x, wv = tid / kWave, lane = tid % kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  const int E = d.E, R = d.R, k = d.k;

  for (int i = tid; i < E; i += kPlanBlock) s_run[i] = 0;
  if (d.dedup)
    for (int i = tid; i < R; i += kPlanBlock) s_frun[i] = 0;
  if (tid == 0) s_bad = 0;

  for (int pass = 0; pass < d.passes; ++pass) {
    const int t = (blockIdx.x * d.passes + pass) * kPlanBlock + tid;
    const bool live = t < d.T;
    for (int i = tid; i < kPlanWaves * E; i += kPlanBlock) s_wc[i] = 0;
    if (d.dedup)
      for (int i = tid; i < kPlanWaves * R; i += kPlanBlock) s_fwc[i] = 0;

    // Load and validate: an id outside [0, E) or repeated in the row is
    // dropped (the first occurrence of a repeat stays).
    int e[KMAX];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      int v = -1;
      if (live && j < k) {
        v = idx[(int64_t)t * k + j];
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
    __syncthreads();  // LDS zeroed; previous pass finished with it

    uint64_t m[KMAX];
    wave_match<KMAX>(e, k, d.ebits, m);
    int lr[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      lr[j] = -1;
      if (e[j] >= 0) {
        lr[j] = __popcll(m[j] & below);
        if (lr[j] == 0) s_wc[wv * E + e[j]] = __popcll(m[j]);
      }
    }

    int f[KMAX], flr[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) f[j] = flr[j] = -1;
    if (d.dedup) {
      // Key of the first slot of each distinct destination node: the
      // forwarder rank n*G + owner(t) % G.
      const int g = live ? split_part(t, d.tbase, d.trem) % d.G : 0;
      int nd[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) nd[j] = e[j] >= 0 ? split_part(e[j], d.ebase, d.erem) / d.G : -1;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        bool first = nd[j] >= 0;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) first = first && nd[jj] != nd[j];
        if (first) f[j] = nd[j] * d.G + g;
      }
      wave_match<KMAX>(f, k, d.fbits, m);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (f[j] >= 0) {
          flr[j] = __popcll(m[j] & below);
          if (flr[j] == 0) s_fwc[wv * R + f[j]] = __popcll(m[j]);
        }
      }
    }
    if (bad) s_bad = 1;
    __syncthreads();

    if (live) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          int r = -1;
          if (e[j] >= 0) {
            r = s_run[e[j]] + lr[j];
            for (int w2 = 0; w2 < wv; ++w2) r += s_wc[w2 * E + e[j]];
          }
          w.slot_of[(int64_t)t * k + j] = r;
          if (d.dedup) {
            int u = -1;
            if (f[j] >= 0) {
              u = s_frun[f[j]] + flr[j];
              for (int w2 = 0; w2 < wv; ++w2) u += s_fwc[w2 * R + f[j]];
            }
            w.stage_of[(int64_t)t * k + j] = u;
          }
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < E; i += kPlanBlock)
      s_run[i] += s_wc[i] + s_wc[E + i] + s_wc[2 * E + i] + s_wc[3 * E + i];
    if (d.dedup)
      for (int i = tid; i < R; i += kPlanBlock)
        s_frun[i] += s_fwc[i] + s_fwc[R + i] + s_fwc[2 * R + i] + s_fwc[3 * R + i];
    __syncthreads();
  }

  for (int i = tid; i < E; i += kPlanBlock) w.tile_counts[blockIdx.x * E + i] = s_run[i];
  if (d.dedup)
    for (int i = tid; i < R; i += kPlanBlock) w.tile_fcounts[blockIdx.x * R + i] = s_frun[i];
  if (tid == 0) w.tile_flags[blockIdx.x] = s_bad;
}

// Sum column `col` of a [nblk, width] tile-major matrix over all tiles and
// over the tiles before `blk`.
__device__ __forceinline__ void column_sums(const int32_t* __restrict__ m, int width, int col,
                                            int nblk, int blk, int& total, int& before) {
  int tot = 0, pre = 0;
#pragma unroll 16
  for (int b = 0; b < nblk; ++b) {
    const int c = m[b * width + col];
    tot += c;
    pre += b < blk ? c : 0;
  }
  total = tot;
  before = pre;
}

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void route_assign_kernel(Dims d,
                                                                  const int32_t* __restrict__ idx,
                                                                  Work w) {
  __shared__ int s_off[MOE_MAX_EXPERTS];   // expert_off[e]
  __shared__ int s_pre[MOE_MAX_EXPERTS];   // rows of e in earlier tiles
  __shared__ int s_foff[MOE_MAX_EXPERTS];  // stage_off[f]
  __shared__ int s_fpre[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[kPlanWaves];
  __shared__ int s_bad;

  const int tid = threadIdx.x, blk = blockIdx.x;
  const int E = d.E, R = d.R, k = d.k;

  for (int e = tid; e < E; e += kPlanBlock)
    column_sums(w.tile_counts, E, e, d.nblk, blk, s_off[e], s_pre[e]);
  if (d.dedup)
    for (int f = tid; f < R; f += kPlanBlock)
      column_sums(w.tile_fcounts, R, f, d.nblk, blk, s_foff[f], s_fpre[f]);
  if (blk == 0 && tid == 0) {
    int bad = 0;
    for (int b = 0; b < d.nblk; ++b) bad |= w.tile_flags[b];
    s_bad = bad;
  }
  __syncthreads();

  if (blk == 0)
    for (int e = tid; e < E; e += kPlanBlock) w.counts[e] = s_off[e];
  __syncthreads();  // the scan rewrites s_off in place
  const int rows = block_exclusive_scan(s_off, E, s_wsum);
  int staged = 0;
  if (d.dedup) staged = block_exclusive_scan(s_foff, R, s_wsum);

  if (blk == 0) {
    for (int e = tid; e < E; e += kPlanBlock) w.expert_off[e] = s_off[e];
    for (int r = tid; r <= R; r += kPlanBlock) {
      const int first = r * d.ebase + min(r, d.erem);  // first expert of rank r
      w.rank_off[r] = first < E ? s_off[first] : rows;
      if (d.dedup) w.stage_off[r] = r < R ? s_foff[r] : staged;
    }
    if (tid == 0) {
      w.expert_off[E] = rows;
      w.ctrl[0] = s_bad ? MOE_ERR_BAD_ROUTING : MOE_OK;
      w.ctrl[1] = staged;
    }
  }

  for (int pass = 0; pass < d.passes; ++pass) {
    const int t = (blk * d.passes + pass) * kPlanBlock + tid;
    if (t >= d.T) continue;
    const int64_t at = (int64_t)t * k;
    int e[KMAX], lr[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      lr[j] = j < k ? w.slot_of[at + j] : -1;
      e[j] = lr[j] >= 0 ? idx[at + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        int row = -1;
        if (lr[j] >= 0) {
          row = s_off[e[j]] + s_pre[e[j]] + lr[j];
          if ((uint32_t)row < (uint32_t)(d.T * k)) w.row_src[row] = t;
        }
        w.slot_of[at + j] = row;
      }
    }
    if (d.dedup) {
      int nd[KMAX], p[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        nd[j] = e[j] >= 0 ? split_part(e[j], d.ebase, d.erem) / d.G : -1;
        p[j] = -1;
      }
      const int g = split_part(t, d.tbase, d.trem) % d.G;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          const int u = w.stage_of[at + j];  // in-tile rank, set on a node's first slot
          if (u >= 0) {
            const int f = nd[j] * d.G + g;
            p[j] = s_foff[f] + s_fpre[f] + u;
            if ((uint32_t)p[j] < (uint32_t)d.smax) w.stage_src[p[j]] = t;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          int q = p[j];
#pragma unroll
          for (int jj = 0; jj < j; ++jj)
            if (q < 0 && nd[j] >= 0 && nd[jj] == nd[j] && p[jj] >= 0) q = p[jj];
          w.stage_of[at + j] = q;
        }
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
    hipLaunchKernelGGL(route_assign_kernel<KMAX>, dim3(d.nblk), dim3(kPlanBlock), 0, s, d, idx, w);
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
  return by_topk<CountLaunch>(d.k, d, idx, w, s);
}

hipError_t launch_route_assign(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<AssignLaunch>(d.k, d, idx, w, s);
}

hipError_t launch_traffic(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<TrafficLaunch>(d.k, d, idx, w, s);
}

}  // namespace moe
