// Host side of the C ABI declared in include/moe_shuffle.h: argument checks,
// workspace layout, and the launch sequence of each call.  moe_plan_create
// makes no HIP call, so plans can be built and checked on a machine without
// a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"

namespace moe {
// Event pairs of moe_plan_timing and the kernel of each recorded launch.
struct LaunchTimer {
  std::vector<hipEvent_t> start, stop;
  std::vector<int32_t> ids;
  int used = 0;
};
}  // namespace moe

struct moe_plan {
  moe_config cfg;
  moe::Dims d;
  moe::Layout layout;
  int64_t staging_rows_max;
  // Bound by moe_route_plan.
  const int32_t* idx;
  void* ws;
  moe::Work work;
  bool routed;     // route_count has been launched for the bound routing
  bool scanned;    // route_scan has been launched for it (tile bases, offsets, status)
  bool assigned;   // slot_of / row_src (and stage_of / stage_src) are final
  moe::LaunchTimer* timer;  // per-launch timing, or null
};

namespace moe {
namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The timer of the plan whose call is running on this thread.
thread_local LaunchTimer* tl_timer = nullptr;

// Makes `plan`'s timer the active one for the lifetime of the scope (each
// API call that launches kernels opens one).
struct TimerScope {
  LaunchTimer* prev;
  explicit TimerScope(const moe_plan* plan) : prev(tl_timer) { tl_timer = plan->timer; }
  ~TimerScope() { tl_timer = prev; }
};

void destroy_events(LaunchTimer* t) {
  for (hipEvent_t e : t->start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->stop) (void)hipEventDestroy(e);
  t->start.clear();
  t->stop.clear();
  t->ids.clear();
  t->used = 0;
}

}  // namespace

bool timer_take(int id, hipEvent_t* start, hipEvent_t* stop) {
  LaunchTimer* t = tl_timer;
  if (t == nullptr || t->used >= (int)t->start.size()) return false;
  *start = t->start[t->used];
  *stop = t->stop[t->used];
  t->ids[t->used] = id;
  ++t->used;
  return true;
}

Layout make_layout(const Dims& d) {
  Layout l{};
  size_t at = 0;
  auto take = [&](size_t& field, int64_t ints) {
    field = at;
    at = align_up(at + (size_t)std::max<int64_t>(ints, 1) * sizeof(int32_t), 256);
  };
  const int64_t tk = (int64_t)d.T * d.k;
  const int64_t fk = d.dedup ? tk : 1;
  take(l.ctrl, kCtrlWords);
  take(l.band_status, d.nbands);
  take(l.pipe, (kPipeHead + 3 * (int64_t)d.nbands) * kPipeSlot);
  take(l.tile_flags, d.nblk);
  take(l.tile_counts, (int64_t)d.nblk * d.E);
  take(l.tile_base, (int64_t)d.nblk * d.E);
  take(l.counts, (int64_t)d.nbands * d.E);
  take(l.expert_off, (int64_t)d.nbands * (d.E + 1));
  take(l.rank_off, (int64_t)d.nbands * (d.R + 1));
  take(l.lr, tk);
  take(l.slot_of, tk);
  take(l.row_src, tk);
  take(l.tile_fcounts, d.dedup ? (int64_t)d.nblk * d.fkeys : 1);
  take(l.tile_fbase, d.dedup ? (int64_t)d.nblk * d.fkeys : 1);
  take(l.tile_ncounts, d.load_aware ? (int64_t)d.nblk * d.N : 1);
  take(l.fwd, d.dedup ? (int64_t)d.R * d.N : 1);
  take(l.stage_off, d.dedup ? d.R + 1 : 1);
  take(l.fkey, fk);
  take(l.flr, fk);
  take(l.stage_of, fk);
  take(l.stage_src, d.dedup ? d.smax : 1);
  take(l.send_rows, (int64_t)d.R * d.R);
  take(l.send_copies, (int64_t)d.R * d.R);
  take(l.node_copies, (int64_t)d.R * d.N);
  l.total = at;
  return l;
}

Work bind_work(const Layout& l, void* base) {
  char* b = static_cast<char*>(base);
  auto p = [&](size_t off) { return reinterpret_cast<int32_t*>(b + off); };
  Work w{};
  w.ctrl = p(l.ctrl);
  w.band_status = p(l.band_status);
  w.pipe = p(l.pipe);
  w.tile_flags = p(l.tile_flags);
  w.tile_counts = p(l.tile_counts);
  w.tile_base = p(l.tile_base);
  w.counts = p(l.counts);
  w.expert_off = p(l.expert_off);
  w.rank_off = p(l.rank_off);
  w.lr = p(l.lr);
  w.slot_of = p(l.slot_of);
  w.row_src = p(l.row_src);
  w.tile_fcounts = p(l.tile_fcounts);
  w.tile_fbase = p(l.tile_fbase);
  w.tile_ncounts = p(l.tile_ncounts);
  w.fwd = p(l.fwd);
  w.stage_off = p(l.stage_off);
  w.fkey = p(l.fkey);
  w.flr = p(l.flr);
  w.stage_of = p(l.stage_of);
  w.stage_src = p(l.stage_src);
  w.send_rows = p(l.send_rows);
  w.send_copies = p(l.send_copies);
  w.node_copies = p(l.node_copies);
  return w;
}

// Launches the plan's scan if the route left it to the gather (small plans).
moe_status ensure_scanned(moe_plan* plan, hipStream_t s) {
  if (plan->scanned) return MOE_OK;
  if (launch_route_scan(plan->d, plan->work, s) != hipSuccess) return MOE_ERR_HIP;
  plan->scanned = true;
  return MOE_OK;
}

// Makes slot_of / row_src (and the staging arrays) final when no dispatch
// has done it since the last route.
moe_status ensure_assigned(moe_plan* plan, hipStream_t s) {
  if (plan->assigned) return MOE_OK;
  if (ensure_scanned(plan, s) != MOE_OK) return MOE_ERR_HIP;
  if (launch_route_assign(plan->d, plan->idx, plan->work, s) != hipSuccess) return MOE_ERR_HIP;
  plan->assigned = true;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_EXPERTS_LT_RANKS: return "fewer experts than ranks: the split would leave ranks without experts";
    case MOE_ERR_BAD_ROUTING: return "routing names an expert outside [0, E) or repeats one in a row";
    case MOE_ERR_PLAN_NOT_ROUTED: return "plan has not been routed (call moe_route_plan first)";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_UNSUPPORTED: return "sizes beyond the library's limits";
    case MOE_ERR_PIPELINE_STALL: return "a banded-pipeline wait gave up; outputs are unspecified";
    case MOE_ERR_STATIC_WORKSPACE:
      return "the plan's workspace exceeds the static per-device workspace (MOE_STATIC_WORKSPACE_BYTES)";
  }
  return "unknown status";
}

moe_status moe_expert_partition(int32_t num_experts, int32_t num_ranks, int32_t* lo_out) {
  if (!lo_out || num_experts <= 0 || num_ranks <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (num_experts < num_ranks) return MOE_ERR_EXPERTS_LT_RANKS;
  const int32_t base = num_experts / num_ranks, rem = num_experts % num_ranks;
  for (int32_t d = 0; d <= num_ranks; ++d) lo_out[d] = d * base + std::min(d, rem);
  return MOE_OK;
}

moe_status moe_plan_create(const moe_config* cfg, moe_plan** out) {
  if (!cfg || !out) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config c = *cfg;
  if (c.num_tokens < 0 || c.hidden <= 0 || c.hidden % 8 || c.num_experts <= 0 || c.top_k <= 0 ||
      c.num_ranks <= 0 || c.ranks_per_node <= 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c.flags & ~(MOE_FLAG_NODE_DEDUP | MOE_FLAG_LOAD_AWARE_FORWARDERS))
    return MOE_ERR_INVALID_ARGUMENT;
  if (c.num_experts > MOE_MAX_EXPERTS || c.top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (c.top_k > c.num_experts) return MOE_ERR_INVALID_ARGUMENT;
  if (c.num_experts < c.num_ranks) return MOE_ERR_EXPERTS_LT_RANKS;
  if (c.num_ranks % c.ranks_per_node) return MOE_ERR_INVALID_ARGUMENT;
  const int32_t nodes = c.num_ranks / c.ranks_per_node;
  const bool dedup = (c.flags & MOE_FLAG_NODE_DEDUP) != 0;
  const bool load_aware = (c.flags & MOE_FLAG_LOAD_AWARE_FORWARDERS) != 0;
  if (dedup && nodes < 2) return MOE_ERR_INVALID_ARGUMENT;
  if (load_aware && !dedup) return MOE_ERR_INVALID_ARGUMENT;
  if (load_aware && (int64_t)c.num_ranks * nodes > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;

  if (c.band_tokens < 0 || c.band_tokens % moe::kPlanBlock) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t T = c.num_tokens, chunks = c.hidden / 8;
  const bool banded = c.band_tokens > 0 && c.band_tokens < T;
  if (banded && dedup) return MOE_ERR_UNSUPPORTED;
  const int64_t staging_max = dedup ? T * std::min<int64_t>(c.top_k, nodes) : 0;
  // Row and wave-item numbers are 32-bit; the last block of a launch numbers
  // a few wave-items past the end before it finds them dead, so keep 4096 clear.
  const int64_t lim = (int64_t)INT32_MAX - 4096;
  if (T * c.top_k >= lim || T * chunks >= lim || staging_max * chunks >= lim)
    return MOE_ERR_UNSUPPORTED;

  moe::Dims d{};
  d.T = (int32_t)T;
  d.H = c.hidden;
  d.E = c.num_experts;
  d.k = c.top_k;
  d.R = c.num_ranks;
  d.G = c.ranks_per_node;
  d.N = nodes;
  d.ebase = d.E / d.R;
  d.erem = d.E % d.R;
  d.tbase = d.T / d.R;
  d.trem = d.T % d.R;
  d.dedup = dedup ? 1 : 0;
  d.load_aware = load_aware ? 1 : 0;
  d.fkeys = load_aware ? d.R * d.N : d.R;
  const int64_t widest = std::max<int64_t>(d.E, dedup ? d.fkeys : 1);
  if (banded) {
    // One 256-token tile per pass; a band's tile-count matrix must fit the
    // scan's LDS, and the pipeline's schedule holds at most 192 bands.
    d.passes = 1;
    d.tile = moe::kPlanBlock;
    d.nblk = (int32_t)((T + d.tile - 1) / d.tile);
    d.band = c.band_tokens;
    d.tpb = d.band / d.tile;
    d.nbands = (int32_t)((T + d.band - 1) / d.band);
    if ((int64_t)d.tpb * d.E > moe::kBandScanLdsInts || d.nbands > 192) return MOE_ERR_UNSUPPORTED;
  } else {
    // At most kMaxPlanTiles tiles, and few enough that the scan kernel holds
    // the [tiles x experts] (and [tiles x staging keys]) count matrix in LDS.
    const int64_t max_tiles = std::min<int64_t>(moe::kMaxPlanTiles, moe::kScanLdsInts / widest);
    const int64_t per_tile_cap = (int64_t)moe::kPlanBlock * max_tiles;
    d.passes = (int32_t)std::max<int64_t>(1, (T + per_tile_cap - 1) / per_tile_cap);
    d.tile = moe::kPlanBlock * d.passes;
    d.nblk = (int32_t)std::max<int64_t>(1, (T + d.tile - 1) / d.tile);
    d.band = d.nblk * d.tile;
    d.tpb = d.nblk;
    d.nbands = 1;
  }
  // Small single-hop plans: the gather scans the tile counts itself.
  d.fused_scan = (!dedup && d.nbands == 1 &&
                  (int64_t)d.nblk * d.E <= moe::kFusedScanInts) ? 1 : 0;
  d.chunks = (int32_t)chunks;
  d.segs = (int32_t)((chunks + moe::kWave - 1) / moe::kWave);
  d.smax = (int32_t)staging_max;

  moe_plan* p = new (std::nothrow) moe_plan();
  if (!p) return MOE_ERR_UNSUPPORTED;
  p->cfg = c;
  p->d = d;
  p->staging_rows_max = staging_max;
  p->layout = moe::make_layout(d);
  p->idx = nullptr;
  p->ws = nullptr;
  p->routed = false;
  p->scanned = false;
  p->assigned = false;
  p->timer = nullptr;
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* plan) {
  if (plan && plan->timer) {
    moe::destroy_events(plan->timer);
    delete plan->timer;
  }
  delete plan;
}

const char* moe_kernel_name(int32_t kernel) {
  static const char* const names[MOE_KERNEL_COUNT] = {
      "route_count_kernel",   "route_scan_kernel",      "route_assign_kernel",
      "traffic_clear_kernel", "traffic_kernel",         "gather_kernel",
      "gather_scan_kernel",   "stage_a_kernel",         "stage_b_kernel",
      "combine_kernel",       "combine_part_kernel",    "combine_nodes_kernel",
      "gather_fp8_kernel",    "gather_fp8_scan_kernel", "stage_a_fp8_kernel",
      "stage_b_fp8_kernel",   "combine_fp8_kernel",     "pipeline_kernel",
      "counters_clear_kernel", "stage_ab_kernel",       "stage_ab_fp8_kernel",
      "combine_pn_kernel"};
  return kernel >= 0 && kernel < MOE_KERNEL_COUNT ? names[kernel] : "?";
}

moe_status moe_plan_timing(moe_plan* plan, int32_t capacity) {
  if (!plan || capacity < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->timer) {
    moe::destroy_events(plan->timer);
    if (capacity == 0) {
      delete plan->timer;
      plan->timer = nullptr;
      return MOE_OK;
    }
  } else {
    if (capacity == 0) return MOE_OK;
    plan->timer = new (std::nothrow) moe::LaunchTimer();
    if (!plan->timer) return MOE_ERR_UNSUPPORTED;
  }
  moe::LaunchTimer* t = plan->timer;
  for (int32_t i = 0; i < capacity; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return MOE_ERR_HIP;
    }
    t->start.push_back(a);
    t->stop.push_back(b);
  }
  t->ids.assign(capacity, -1);
  t->used = 0;
  return MOE_OK;
}

moe_status moe_plan_timing_read(moe_plan* plan, int32_t* kernel_ids, float* start_ms, float* ms,
                                int32_t cap, int32_t* count) {
  if (!plan || !plan->timer || !count || cap < 0 ||
      (cap > 0 && (!kernel_ids || !start_ms || !ms)))
    return MOE_ERR_INVALID_ARGUMENT;
  moe::LaunchTimer* t = plan->timer;
  const int n = t->used;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(t->stop[i]) != hipSuccess) return MOE_ERR_HIP;
    if (i < cap) {
      float e = 0.0f, st = 0.0f;
      if (hipEventElapsedTime(&e, t->start[i], t->stop[i]) != hipSuccess) return MOE_ERR_HIP;
      if (i > 0 && hipEventElapsedTime(&st, t->start[0], t->start[i]) != hipSuccess)
        return MOE_ERR_HIP;
      kernel_ids[i] = t->ids[i];
      start_ms[i] = st;
      ms[i] = e;
    }
  }
  *count = n;
  t->used = 0;
  return MOE_OK;
}

size_t moe_plan_workspace_bytes(const moe_plan* plan) { return plan ? plan->layout.total : 0; }

int64_t moe_plan_recv_rows(const moe_plan* plan) {
  return plan ? (int64_t)plan->d.T * plan->d.k : 0;
}

int64_t moe_plan_staging_rows_max(const moe_plan* plan) {
  return plan ? plan->staging_rows_max : 0;
}

int64_t moe_plan_bands(const moe_plan* plan) { return plan ? plan->d.nbands : 0; }

int64_t moe_plan_chunk_tokens(const moe_plan* plan, int32_t call) {
  if (!plan) return 0;
  if (!plan->d.dedup || call < 0 || call > 2) return plan->d.T;
  return moe::chunk_tokens(plan->d, call);
}

moe_status moe_route_plan(moe_plan* plan, const int32_t* topk_idx, void* workspace, void* stream) {
  if (!plan || !workspace || !moe::aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (plan->d.T > 0 && (!topk_idx || !moe::aligned(topk_idx, 4))) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  plan->routed = false;
  plan->assigned = false;
  plan->idx = topk_idx;
  plan->ws = workspace;
  plan->work = moe::bind_work(plan->layout, workspace);
  plan->scanned = false;
  if (moe::launch_route_count(plan->d, topk_idx, plan->work, s) != hipSuccess) return MOE_ERR_HIP;
  plan->routed = true;
  // Small single-hop plans leave the scan to the gather (and to whoever reads
  // the plan arrays before it).
  if (!plan->d.fused_scan && moe::ensure_scanned(plan, s) != MOE_OK) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_route_plan_static(moe_plan* plan, const int32_t* topk_idx, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->layout.total > (size_t)MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_STATIC_WORKSPACE;
  if (plan->d.T > 0 && (!topk_idx || !moe::aligned(topk_idx, 4))) return MOE_ERR_INVALID_ARGUMENT;
  void* ws = nullptr;
  if (moe::static_workspace(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_route_plan(plan, topk_idx, ws, stream);
}

moe_status moe_pipeline(moe_plan* plan, const int32_t* topk_idx, void* workspace,
                        const uint16_t* x, uint16_t* recv, const float* topk_w, void* out,
                        int32_t out_dtype, void* stream) {
  if (!plan || !workspace || !moe::aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (plan->d.dedup || plan->d.H % 64) return MOE_ERR_UNSUPPORTED;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.T > 0 &&
      (!topk_idx || !x || !recv || !topk_w || !out || !moe::aligned(topk_idx, 4) ||
       !moe::aligned(x, 16) || !moe::aligned(recv, 128) || !moe::aligned(topk_w, 4) ||
       !moe::aligned(out, 16)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.T == 0) return moe_route_plan(plan, topk_idx, workspace, stream);
  hipStream_t s = static_cast<hipStream_t>(stream);
  plan->routed = false;
  plan->assigned = false;
  plan->idx = topk_idx;
  plan->ws = workspace;
  plan->work = moe::bind_work(plan->layout, workspace);
  // Every launch zeroes the counters first (one small kernel): a caller's
  // workspace may hold anything, a reused allocation included.
  if (moe::launch_counters_clear(plan->d, plan->work, s) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_pipeline(plan->d, topk_idx, x, recv, topk_w, out, out_dtype == MOE_OUT_F32,
                           plan->work, s) != hipSuccess)
    return MOE_ERR_HIP;
  plan->routed = true;
  plan->scanned = true;
  plan->assigned = true;
  return MOE_OK;
}

moe_status moe_dispatch(moe_plan* plan, const uint16_t* x, uint16_t* recv, uint16_t* staging,
                        void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  if (plan->d.T == 0) return MOE_OK;
  if (!x || !recv || !moe::aligned(x, 16) || !moe::aligned(recv, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.dedup && (!staging || !moe::aligned(staging, 16))) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!plan->d.dedup) {
    if (moe::launch_gather(plan->d, plan->idx, x, recv, plan->work, s) != hipSuccess)
      return MOE_ERR_HIP;
    plan->assigned = true;
    return MOE_OK;
  }
  if (moe::ensure_scanned(plan, s) != MOE_OK) return MOE_ERR_HIP;
  plan->assigned = true;
  return moe::from_hip(
      moe::launch_dedup_dispatch(plan->d, plan->idx, x, staging, recv, plan->work, s));
}

moe_status moe_combine(moe_plan* plan, const uint16_t* y, const float* topk_w, void* out,
                       int32_t out_dtype, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.T == 0) return MOE_OK;
  if (!y || !topk_w || !out || !moe::aligned(y, 16) || !moe::aligned(topk_w, 4) ||
      !moe::aligned(out, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_status st = moe::ensure_assigned(plan, s);
  if (st != MOE_OK) return st;
  return moe::from_hip(
      moe::launch_combine(plan->d, y, topk_w, out, out_dtype == MOE_OUT_F32, plan->work, s));
}

moe_status moe_combine_hier(moe_plan* plan, const uint16_t* y, const float* topk_w,
                            float* partials, void* out, int32_t out_dtype, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  if (!plan->d.dedup) return MOE_ERR_INVALID_ARGUMENT;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.T == 0) return MOE_OK;
  if (!y || !topk_w || !partials || !out || !moe::aligned(y, 16) || !moe::aligned(topk_w, 4) ||
      !moe::aligned(partials, 16) || !moe::aligned(out, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_status st = moe::ensure_assigned(plan, s);
  if (st != MOE_OK) return st;
  return moe::from_hip(moe::launch_combine_hier(plan->d, y, topk_w, partials, out,
                                                out_dtype == MOE_OUT_F32, plan->work, s));
}

int64_t moe_plan_scale_blocks(const moe_plan* plan) {
  return plan ? ((int64_t)plan->d.H + 127) / 128 : 0;
}

moe_status moe_dispatch_fp8(moe_plan* plan, const uint16_t* x, uint8_t* recv8, float* recv_scale,
                            uint8_t* staging8, float* staging_scale, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  if (plan->d.T == 0) return MOE_OK;
  if (!x || !recv8 || !recv_scale || !moe::aligned(x, 16) || !moe::aligned(recv8, 16) ||
      !moe::aligned(recv_scale, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.dedup && (!staging8 || !staging_scale || !moe::aligned(staging8, 16) ||
                        !moe::aligned(staging_scale, 4)))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // small single-hop plans with up to 64 experts: the fp8 gather scans the
  // tile counts itself
  if (!moe::fp8_fused_scan(plan->d) && moe::ensure_scanned(plan, s) != MOE_OK) return MOE_ERR_HIP;
  const hipError_t e =
      plan->d.dedup ? moe::launch_stage_fp8(plan->d, plan->idx, x, staging8, staging_scale, recv8,
                                            recv_scale, plan->work, s)
                    : moe::launch_gather_fp8(plan->d, plan->idx, x, recv8, recv_scale, plan->work, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  plan->assigned = true;
  return MOE_OK;
}

moe_status moe_combine_fp8(moe_plan* plan, const uint8_t* y8, const float* y_scale,
                           const float* topk_w, void* out, int32_t out_dtype, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->d.T == 0) return MOE_OK;
  if (!y8 || !y_scale || !topk_w || !out || !moe::aligned(y8, 16) || !moe::aligned(y_scale, 4) ||
      !moe::aligned(topk_w, 4) || !moe::aligned(out, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_status st = moe::ensure_assigned(plan, s);
  if (st != MOE_OK) return st;
  return moe::from_hip(moe::launch_combine_fp8(plan->d, y8, y_scale, topk_w, out,
                                               out_dtype == MOE_OUT_F32, plan->work, s));
}

moe_status moe_plan_read(moe_plan* plan, int32_t item, void* host_dst, size_t bytes,
                         void* stream) {
  if (!plan || !host_dst) return MOE_ERR_INVALID_ARGUMENT;
  const moe::TimerScope timing(plan);
  if (!plan->routed) return MOE_ERR_PLAN_NOT_ROUTED;
  const moe::Dims& d = plan->d;
  const moe::Work w = plan->work;
  const int64_t tk = (int64_t)d.T * d.k;
  const int32_t* src = nullptr;
  int64_t n = 0;
  bool traffic = false;
  switch (item) {
    case MOE_ITEM_STATUS: src = w.band_status; n = 1; break;
    case MOE_ITEM_COUNTS: src = w.counts; n = (int64_t)d.nbands * d.E; break;
    case MOE_ITEM_EXPERT_OFFSETS: src = w.expert_off; n = (int64_t)d.nbands * (d.E + 1); break;
    case MOE_ITEM_RANK_OFFSETS: src = w.rank_off; n = (int64_t)d.nbands * (d.R + 1); break;
    case MOE_ITEM_SLOT_OF: src = w.slot_of; n = tk; break;
    case MOE_ITEM_ROW_SRC: src = w.row_src; n = tk; break;
    case MOE_ITEM_NUM_STAGED: src = w.ctrl + moe::kCtrlStaged; n = 1; break;
    case MOE_ITEM_STAGE_OFFSETS: src = w.stage_off; n = d.R + 1; break;
    case MOE_ITEM_STAGE_OF: src = w.stage_of; n = tk; break;
    case MOE_ITEM_STAGE_SRC: src = w.stage_src; n = plan->staging_rows_max; break;
    case MOE_ITEM_SEND_ROWS: src = w.send_rows; n = (int64_t)d.R * d.R; traffic = true; break;
    case MOE_ITEM_SEND_COPIES: src = w.send_copies; n = (int64_t)d.R * d.R; traffic = true; break;
    case MOE_ITEM_NODE_COPIES: src = w.node_copies; n = (int64_t)d.R * d.N; traffic = true; break;
    case MOE_ITEM_FORWARDERS: src = w.fwd; n = (int64_t)d.R * d.N; break;
    default: return MOE_ERR_INVALID_ARGUMENT;
  }
  const bool dedup_item = item == MOE_ITEM_NUM_STAGED || item == MOE_ITEM_STAGE_OFFSETS ||
                          item == MOE_ITEM_STAGE_OF || item == MOE_ITEM_STAGE_SRC ||
                          item == MOE_ITEM_FORWARDERS;
  if (dedup_item && !d.dedup) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = (size_t)n * sizeof(int32_t);
  if (bytes < need) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (moe::ensure_scanned(plan, s) != MOE_OK) return MOE_ERR_HIP;
  const bool per_slot = item == MOE_ITEM_SLOT_OF || item == MOE_ITEM_ROW_SRC ||
                        item == MOE_ITEM_STAGE_OF || item == MOE_ITEM_STAGE_SRC || traffic;
  if (per_slot) {
    const moe_status st = moe::ensure_assigned(plan, s);
    if (st != MOE_OK) return st;
  }
  if (traffic) {
    if (moe::launch_traffic(d, plan->idx, w, s) != hipSuccess) return MOE_ERR_HIP;
  }
  if (item == MOE_ITEM_STATUS) {
    // One status per band: report the first that is not MOE_OK.
    std::vector<int32_t> st(d.nbands, 0);
    if (hipMemcpyAsync(st.data(), w.band_status, st.size() * sizeof(int32_t),
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return MOE_ERR_HIP;
    int32_t worst = MOE_OK;
    for (int32_t v : st)
      if (v != MOE_OK && worst == MOE_OK) worst = v;
    std::memcpy(host_dst, &worst, sizeof worst);
    return MOE_OK;
  }
  if (need > 0) {
    if (hipMemcpyAsync(host_dst, src, need, hipMemcpyDeviceToHost, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return moe::from_hip(hipStreamSynchronize(s));
}

}  // extern "C"
