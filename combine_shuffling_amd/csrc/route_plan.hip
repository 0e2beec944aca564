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
// With node deduplication the same is done over the keys "forwarder rank of
// (token, node)" of the first slot of each distinct destination node of a
// token, which orders staging rows by (forwarder, token) (FUSCO article,
// "load balancing and cross-node deduplication": one copy per destination
// node through a forwarding GPU).  route_count counts both key sets in one
// pass; route_scan scans the staging keys in a block of their own, beside
// the expert keys' block.
//
// A slot's receive row is then tile_base[tile][expert] + its in-tile rank:
// the stable (expert, token) order.  The data-movement kernels that run next
// finish slot_of / row_src (and stage_of / stage_src) on the fly; the
// per-token route_assign kernel does the same when a consumer needs the plan
// without a dispatch.
#include <mutex>

#include "plan_body.h"

namespace moe {
namespace {

// Workspace of moe_route_plan_static: one copy on every GPU the library runs
// on, held until the process ends.  In host code `scratch` only stands in for
// the symbol; its device address comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void route_count_kernel(Dims d,
                                                                 const int32_t* __restrict__ idx,
                                                                 Work w) {
  __shared__ unsigned long long s_mask[kPlanWaves * MOE_MAX_EXPERTS];  // per-wave ballots; 32 KiB
  __shared__ int s_pre[kPlanWaves * MOE_MAX_EXPERTS];  // slots before each (wave, key); 16 KiB
  __shared__ int s_run[MOE_MAX_EXPERTS];   // tile's slots per expert so far
  __shared__ int s_frun[MOE_MAX_EXPERTS];  // tile's staging rows per key so far (fkeys <= 1024)
  __shared__ int s_node[MOE_MAX_EXPERTS];  // destination node of each expert (dedup)
  __shared__ int s_bad;
  count_tile<KMAX>(d, idx, w, blockIdx.x, CountLds{s_mask, s_pre, s_run, s_frun, s_node, &s_bad});
}

// One block of kScanBlock threads per band, and with node deduplication (one
// band) one more block for the staging keys (one per node with load-aware
// forwarders).  Each column of a count matrix
// is summed, and its tile bases written, by several threads (one run of
// consecutive tiles each).
__global__ __launch_bounds__(kScanBlock) void route_scan_kernel(Dims d, Work w) {
  __shared__ int s_mat[kScanLdsInts];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[kScanBlock / kWave];
  __shared__ int s_part[kScanBlock];
  const ScanLds L{s_mat, s_tot, s_wsum, s_part};
  if ((int)blockIdx.x < d.nbands) scan_band<false, kScanBlock>(d, w, blockIdx.x, L);
  else scan_stage_keys<false, kScanBlock>(d, w, blockIdx.x - d.nbands, L);
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

// Clears the three traffic matrices before traffic_kernel adds into them (a
// fill kernel rather than memset nodes, so that the sequence holds kernels
// only).
__global__ __launch_bounds__(kPlanBlock) void traffic_clear_kernel(Dims d, Work w) {
  const int i = blockIdx.x * kPlanBlock + threadIdx.x;
  if (i < d.R * d.R) {
    w.send_rows[i] = 0;
    w.send_copies[i] = 0;
  }
  if (i < d.R * d.N) w.node_copies[i] = 0;
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
    return launch(MOE_KERNEL_ROUTE_COUNT, route_count_kernel<KMAX>, dim3(d.nblk), dim3(kPlanBlock),
                  0, s, d, idx, w);
  }
};

template <int KMAX>
struct AssignLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
    const int blocks = (d.T + kPlanBlock - 1) / kPlanBlock;
    if (blocks == 0) return hipSuccess;
    return launch(MOE_KERNEL_ROUTE_ASSIGN, route_assign_kernel<KMAX>, dim3(blocks),
                  dim3(kPlanBlock), 0, s, d, idx, w);
  }
};

template <int KMAX>
struct TrafficLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
    const int blocks = (d.T + kPlanBlock - 1) / kPlanBlock;
    if (blocks == 0) return hipSuccess;
    return launch(MOE_KERNEL_TRAFFIC, traffic_kernel<KMAX>, dim3(blocks), dim3(kPlanBlock), 0, s, d,
                  idx, w);
  }
};

}  // namespace

hipError_t static_workspace(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_route_count(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<CountLaunch>(d.k, d, idx, w, s);
}

hipError_t launch_route_scan(const Dims& d, const Work& w, hipStream_t s) {
  const int stage_blocks = d.dedup ? (d.load_aware ? d.N : 1) : 0;
  return launch(MOE_KERNEL_ROUTE_SCAN, route_scan_kernel, dim3(d.nbands + stage_blocks),
                dim3(kScanBlock), 0, s, d, w);
}

hipError_t launch_route_assign(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  return by_topk<AssignLaunch>(d.k, d, idx, w, s);
}

// Clears the counters, then counts (no counting launch for an empty batch).
hipError_t launch_traffic(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s) {
  const int blocks = (d.R * d.R + kPlanBlock - 1) / kPlanBlock;
  const hipError_t e = launch(MOE_KERNEL_TRAFFIC_CLEAR, traffic_clear_kernel, dim3(blocks),
                              dim3(kPlanBlock), 0, s, d, w);
  if (e != hipSuccess) return e;
  return by_topk<TrafficLaunch>(d.k, d, idx, w, s);
}

}  // namespace moe
