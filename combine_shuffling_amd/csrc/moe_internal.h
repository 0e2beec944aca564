// Internal declarations shared by the host API (moe_api.cpp) and the gfx950
// kernels (route_plan.hip, move.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe_shuffle.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kPlanBlock = 256;    // threads per route-plan block = tokens per pass
constexpr int kPlanWaves = kPlanBlock / kWave;
constexpr int kMaxPlanTiles = 64;  // route-plan tiles (blocks); tiles grow past 64*256 tokens
constexpr int kMoveBlock = 256;    // threads per data-movement block

// Sizes and the hoisted constants of the two ceil/floor splits.  Passed by
// value to every kernel.
struct Dims {
  int32_t T, H, E, k, R, G, N;
  int32_t ebase, erem;    // experts: E / R, E % R
  int32_t tbase, trem;    // tokens:  T / R, T % R (owner ranks)
  int32_t passes;         // 256-token passes per plan tile
  int32_t nblk;           // plan tiles
  int32_t ebits, fbits;   // bits that tell expert ids / forwarder ids apart
  int32_t dedup;          // MOE_FLAG_NODE_DEDUP set
  int32_t chunks;         // 16-byte chunks per row = H / 8
  int32_t smax;           // staging rows allocated (T * min(k, N) with dedup, else 0)
};

// Device pointers into the caller's workspace.  Sizes in int32 elements.
struct Work {
  int32_t* ctrl;          // [64]: [0] status of the last route, [1] D staging rows used
  int32_t* tile_flags;    // [nblk]      bad-routing flag per tile
  int32_t* tile_counts;   // [nblk * E]  rows per (tile, expert), tile-major
  int32_t* counts;        // [E]
  int32_t* expert_off;    // [E + 1]
  int32_t* rank_off;      // [R + 1]
  int32_t* slot_of;       // [T * k]     token slot -> receive row (-1: dropped)
  int32_t* row_src;       // [T * k]     receive row -> token
  int32_t* tile_fcounts;  // [nblk * R]  staging rows per (tile, forwarder)       (dedup)
  int32_t* stage_off;     // [R + 1]     first staging row of each forwarder       (dedup)
  int32_t* stage_of;      // [T * k]     token slot -> staging row of its node     (dedup)
  int32_t* stage_src;     // [Dmax]      staging row -> token                      (dedup)
  int32_t* send_rows;     // [R * R]     modelled link traffic (filled on demand)
  int32_t* send_copies;   // [R * R]
  int32_t* node_copies;   // [R * N]
};

// Byte offsets of each Work array from the workspace base, and the total.
struct Layout {
  size_t ctrl, tile_flags, tile_counts, counts, expert_off, rank_off, slot_of, row_src,
      tile_fcounts, stage_off, stage_of, stage_src, send_rows, send_copies, node_copies, total;
};

Layout make_layout(const Dims& d, int64_t staging_rows_max);
Work bind_work(const Layout& l, void* base);

// Route plan (route_plan.hip).
hipError_t launch_route_count(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);
hipError_t launch_route_assign(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);
hipError_t launch_traffic(const Dims& d, const int32_t* idx, const Work& w, hipStream_t s);

// Data movement (move.hip).
hipError_t launch_gather(const Dims& d, const uint16_t* x, uint16_t* recv, const Work& w,
                         hipStream_t s);
hipError_t launch_stage_a(const Dims& d, const uint16_t* x, uint16_t* staging, const Work& w,
                          int64_t staging_rows_max, hipStream_t s);
hipError_t launch_stage_b(const Dims& d, const uint16_t* staging, uint16_t* recv, const Work& w,
                          int64_t staging_rows_max, hipStream_t s);
hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* wts, void* out,
                          bool out_f32, const Work& w, hipStream_t s);

}  // namespace moe
