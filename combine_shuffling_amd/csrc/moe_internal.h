// Internal declarations shared by the host API (moe_api.cpp) and the gfx950
// kernels (route_plan.hip, move.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe_shuffle.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kPlanBlock = 256;    // threads per route-plan block = tokens per pass
constexpr int kPlanWaves = kPlanBlock / kWave;
constexpr int kMaxPlanTiles = 64;  // route-plan tiles (blocks) at most
// Tile-count matrix the route-plan scan holds in LDS (128 KiB of gfx950's
// 160 KiB per workgroup).  More, smaller tiles shorten the count kernel: the
// [tiles x experts] matrix of the DeepSeek-V3-like workload takes 64
// one-pass tiles instead of 32 two-pass ones (route 27.4 -> 23.1 us), and
// its [tiles x (owner, node)] matrix of load-aware forwarders 64 one-pass
// tiles instead of 32 two-pass ones.
constexpr int kScanLdsInts = 32768;
// Threads of the route-plan scan block.
constexpr int kScanBlock = 1024;
// A band's matrix in the banded pipeline, whose dynamic LDS stays under the
// default 64 KiB limit.
constexpr int kBandScanLdsInts = 8192;
// Tile-count matrices up to this size are scanned in the gather (measured,
// one stream: olmoe 16 x 64 gains 2 us per step; qwen3's 32 x 128, with
// 16-wave gather blocks, 8 us; nondiv's 64 x 100 loses 14 us, as every
// gather block then redoes a 6400-entry scan).
constexpr int kFusedScanInts = 4096;

// ctrl words at the start of the workspace.
constexpr int kCtrlStaged = 1;     // D, staging rows used
constexpr int kCtrlWords = 64;

// Banded pipeline: counters in Work::pipe, each in a slot of its own
// (kPipeSlot ints, so polls of one counter do not contend with updates of
// another): the head slots, then three per band (count tiles done, scan
// done, gather tickets done).  All zero between launches: the last block of
// every launch clears them.
constexpr int kPipeSlot = 64;      // ints per counter slot (256 bytes)
constexpr int kPipeTicket = 0;     // next ticket to hand out
constexpr int kPipeExit = 1;       // blocks that have left the ticket loop
constexpr int kPipeStall = 2;      // set when a bounded wait gave up
constexpr int kPipeHead = 4;       // head slots
constexpr int kPipeMaxSteps = 256; // schedule steps (bands + stage lags) at most

// Per-launch kernel timing (moe_plan_timing): while a call on a plan whose
// timing is on runs on this thread, timer_take hands out the next event pair
// for a launch of kernel `id` (moe_kernel); false: launch untimed.
bool timer_take(int id, hipEvent_t* start, hipEvent_t* stop);

// Launches `kernel` on stream s; with a pair from timer_take, the pair is
// bound to the kernel's own start and end (hipExtLaunchKernel).
template <typename... P, typename... A>
hipError_t launch(int id, void (*kernel)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                  A... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  if (timer_take(id, &start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, start, stop, 0u, static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<P>(args)...);
  return hipGetLastError();
}

// Sizes and the hoisted constants of the two ceil/floor splits.  Passed by
// value to every kernel.
struct Dims {
  int32_t T, H, E, k, R, G, N;
  int32_t ebase, erem;    // experts: E / R, E % R
  int32_t tbase, trem;    // tokens:  T / R, T % R (owner ranks)
  int32_t passes;         // 256-token passes per plan tile
  int32_t tile;           // tokens per plan tile = 256 * passes
  int32_t nblk;           // plan tiles
  int32_t band;           // tokens per band (a multiple of tile; >= T with one band)
  int32_t nbands;         // bands, each routed as a batch of its own
  int32_t tpb;            // plan tiles per band
  int32_t fused_scan;     // the single-hop gather scans the tile counts itself (small plans)
  int32_t dedup;          // MOE_FLAG_NODE_DEDUP set
  int32_t load_aware;     // MOE_FLAG_LOAD_AWARE_FORWARDERS set
  int32_t fkeys;          // staging keys: forwarders (R), or (node, owner) pairs n * R + s (R * N)
  int32_t chunks;         // 16-byte chunks per row = H / 8
  int32_t segs;           // 64-chunk row segments per row = ceil(chunks / 64)
  int32_t smax;           // staging rows allocated (T * min(k, N) with dedup, else 0)
};

// Device pointers into the caller's workspace (int32 arrays).
struct Work {
  int32_t* ctrl;          // [kCtrlWords]
  int32_t* band_status;   // [nbands]    moe_status of each band's route
  int32_t* pipe;          // [(kPipeHead + 3 * nbands) * kPipeSlot] banded-pipeline counters
  int32_t* tile_flags;    // [nblk]      bad-routing flag per tile
  int32_t* tile_counts;   // [nblk * E]  rows per (tile, expert), tile-major
  int32_t* tile_base;     // [nblk * E]  first receive row of (tile, expert)
  int32_t* counts;        // [nbands * E]
  int32_t* expert_off;    // [nbands * (E + 1)]  global receive rows
  int32_t* rank_off;      // [nbands * (R + 1)]
  int32_t* lr;            // [T * k]     rank of slot (t, j) among its tile's slots of that expert; -1 dropped
  int32_t* slot_of;       // [T * k]     token slot -> receive row (-1: dropped)
  int32_t* row_src;       // [T * k]     receive row -> token
  int32_t* tile_fcounts;  // [nblk * fkeys] staging rows per (tile, key)                 (dedup)
  int32_t* tile_fbase;    // [nblk * fkeys] first staging row of (tile, key)              (dedup)
  int32_t* tile_ncounts;  // [nblk * N]  staging rows per (tile, node)        (load-aware forwarders)
  int32_t* fwd;           // [R * N]     forwarder of (owner s, node n) at s * N + n      (dedup)
  int32_t* stage_off;     // [R + 1]     first staging row of each forwarder               (dedup)
  int32_t* fkey;          // [T * k]     staging key of the node's first slot; -2-j on later
                          //             slots of the node (j = its first slot); -1 dropped (dedup)
  int32_t* flr;           // [T * k]     rank among the tile's staging rows of that forwarder (dedup)
  int32_t* stage_of;      // [T * k]     token slot -> staging row of its node             (dedup)
  int32_t* stage_src;     // [smax]      staging row -> token                              (dedup)
  int32_t* send_rows;     // [R * R]     modelled link traffic (filled on demand)
  int32_t* send_copies;   // [R * R]
  int32_t* node_copies;   // [R * N]
};

// The fp8 gather folds the scan in only up to 64 experts: its rows carry half
// the bytes, so the scan each block redoes weighs twice as much (qwen3 fp8
// dispatch 55 us with the separate scan, 63.5 us folded; olmoe 23.1 -> 17.8).
inline bool fp8_fused_scan(const Dims& d) { return d.fused_scan && d.E <= kWave; }

// Byte offsets of each Work array from the workspace base, and the total.
struct Layout {
  size_t ctrl, band_status, pipe, tile_flags, tile_counts, tile_base, counts, expert_off, rank_off, lr, slot_of,
      row_src, tile_fcounts, tile_fbase, tile_ncounts, fwd, stage_off, fkey, flr, stage_of, stage_src,
      send_rows, send_copies, node_copies, total;
};

Layout make_layout(const Dims& d);
Work bind_work(const Layout& l, void* base);

// The per-device static workspace of moe_route_plan_static (route_plan.hip):
// its device address on the current device, looked up once per device.
hipError_t static_workspace(void** out);

// Route plan (route_plan.hip).
// route_count, and route_scan (one block per band).
hipError_t launch_route_count(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);
hipError_t launch_route_scan(const Dims& d, const Work& w, hipStream_t s);
hipError_t launch_route_assign(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);
hipError_t launch_traffic(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);

// Data movement (move.hip).  gather and stage_a also finish the plan
// (slot_of, row_src, stage_of, stage_src) from the in-tile ranks.  With
// d.fused_scan the gather reads the raw tile counts and needs no route_scan.
hipError_t launch_gather(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                         const Work& w, hipStream_t s);
hipError_t launch_dedup_dispatch(const Dims& d, const int32_t* idx, const uint16_t* x,
                                 uint16_t* staging, uint16_t* recv, const Work& w, hipStream_t s);
// Tokens per chunk of a chunked call with node deduplication: 0 the dispatch,
// 1 the fp8 dispatch, 2 the hierarchical combine.
int64_t chunk_tokens(const Dims& d, int call);
hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* wts, void* out,
                          bool out_f32, const Work& w, hipStream_t s);
// Two-hop combine of a node-deduplicated plan: fp32 partial per staging row,
// then the sum over the token's nodes.  part: [smax, H] float32.
hipError_t launch_combine_hier(const Dims& d, const uint16_t* y,
                               const float* wts, float* part, void* out, bool out_f32,
                               const Work& w, hipStream_t s);
// Banded pipeline: route, dispatch and combine (identity expert) of every
// band in one persistent launch (pipeline.hip).  Work::pipe must be zero.
hipError_t launch_pipeline(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                           const float* wts, void* out, bool out_f32, const Work& w,
                           hipStream_t s);
// Zeroes the pipeline's counters in a workspace.
hipError_t launch_counters_clear(const Dims& d, const Work& w, hipStream_t s);
// fp8 payload (OCP E4M3 codes, one power-of-two scale per 128-element block).
hipError_t launch_gather_fp8(const Dims& d, const int32_t* idx, const uint16_t* x, uint8_t* recv8,
                             float* rscale, const Work& w, hipStream_t s);
// Node-deduplicated fp8 dispatch: stage_a_fp8 then stage_b_fp8.  Also
// finishes slot_of / row_src / stage_of / stage_src.
hipError_t launch_stage_fp8(const Dims& d, const int32_t* idx, const uint16_t* x,
                            uint8_t* stage8, float* sscale, uint8_t* recv8, float* rscale,
                            const Work& w, hipStream_t s);
hipError_t launch_combine_fp8(const Dims& d, const uint8_t* y8, const float* yscale,
                              const float* wts, void* out, bool out_f32, const Work& w,
                              hipStream_t s);

}  // namespace moe
