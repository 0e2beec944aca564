// Banded pipeline on gfx950: route plan, dispatch and combine of every band
// of tokens in one persistent launch.
//
// INC-MoE abstract: the tokens are cut into bands that flow through a
// dispatch -> expert -> combine pipeline inside a single persistent kernel,
// with thread blocks of different roles working on different bands at the
// same time and handing bands on through device-side synchronization.  Here
// the expert is the identity (combine reads the receive rows the dispatch
// wrote) and the dispatch of a band needs that band's route plan first, so a
// band passes four stages:
//
//   count    one ticket per plan tile of the band (route_count's body);
//   scan     one ticket per band (route_scan's body for that band);
//   gather   one ticket per block-chunk of the band's wave-items;
//   combine  one ticket per block-chunk of the band's wave-items.
//
// Tickets are handed out in one global order by an atomic counter, step by
// step: step s holds count(s), scan(s - Ls), gather(s - Ls - Lg) and
// combine(s - Ls - Lg - Lc).  A stage of band b depends only on the previous
// stage of the same band, and that stage's tickets all come earlier in the
// order, so the lowest unfinished ticket can always run: every wait ends,
// whether or not the whole grid is resident.  The lags make the waits rare:
// when combine(b) is handed out, roughly a grid's worth of other tickets has
// been handed out since gather(b).
//
// Hand-over.  The L2 is per XCD and not coherent across XCDs, and an
// agent-scope release / acquire fence writes back / invalidates a whole L2:
// paid per ticket, that costs more than the data movement.  So everything
// one block hands to another inside the launch is written with device-scope
// (sc1) stores, which go through to the coherence point: the plan arrays
// (in-tile ranks, tile counts and flags, tile bases, slot_of) and the
// receive rows.  Plan arrays are also read with device-scope loads.  The
// receive rows are read with plain loads: with 2H a multiple of 128 bytes and
// bands a multiple of 256 tokens, no cache line holds bytes of two bands, and
// a band's rows are read only by its combine, after its gather is complete,
// so no L1 or L2 can hold a stale copy.  A producer's waves wait for their
// stores to be acknowledged, the block meets at a barrier, and one thread
// adds 1 to the stage's counter for the band (device-scope atomic).  A
// consumer's first thread polls that counter until it reaches the stage's
// ticket count and the block meets at a barrier before touching the data.
// Each wait is bounded: after kSpinLimit polls it gives up, skips its work and
// flags a stall, which the launch's last block turns into
// MOE_ERR_PIPELINE_STALL for every band.  The last block to leave also clears
// the counters, so the next launch finds them at zero.
#include <algorithm>

#include "move_body.h"
#include "plan_body.h"

namespace moe {
namespace {

static_assert(kBlock == kPlanBlock, "pipeline roles share one block shape");

// Wave-items per wave of a gather / combine ticket (1, 2, 4 and 8 measured:
// 4 for both was best).
constexpr int kPipeGatherU = 4;
constexpr int kPipeCombineU = 4;
// Schedule lags, in steps, of the scan after the count and of the gather
// after the scan (the combine's lag is sized from the resident grid).
constexpr int kLagScan = 1;
constexpr int kLagGather = 1;
constexpr int kSpinLimit = 1 << 17;  // polls before a wait gives up

enum Role { kCount = 0, kScan = 1, kGather = 2, kCombine = 3, kRoles = 4 };

// Ticket schedule (host-computed, passed by value).
struct Sched {
  int total;                       // tickets
  int nsteps;
  int lag[kRoles];                 // step of (role, band b) = b + lag[role]
  int full[kRoles], last[kRoles];  // tickets of a role for a full band / the last band
  int step_start[kPipeMaxSteps + 1];
};

struct Ticket {
  int role, band, r;  // r: ticket index inside (role, band)
};

__device__ __forceinline__ Ticket decode(const Sched& S, int nbands, int tk) {
  int lo = 0, hi = S.nsteps;  // step_start[lo] <= tk < step_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (S.step_start[mid] <= tk) lo = mid;
    else hi = mid;
  }
  int r = tk - S.step_start[lo];
  Ticket t{kCombine, 0, 0};
#pragma unroll
  for (int role = 0; role < kRoles; ++role) {
    const int b = lo - S.lag[role];
    if (b < 0 || b >= nbands) continue;
    const int n = b == nbands - 1 ? S.last[role] : S.full[role];
    if (r < n) return Ticket{role, b, r};
    r -= n;
  }
  return t;  // not reached for tk < total
}

// Polls *p (device scope) until it reaches `need`; false on giving up.
__device__ __forceinline__ bool wait_for(int32_t* p, int need, int32_t* stall) {
  for (int spin = 0; spin < kSpinLimit; ++spin) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(stall, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

template <int KMAX, bool F32OUT>
__global__ __launch_bounds__(kBlock) void pipeline_kernel(Dims d, const int32_t* __restrict__ idx,
                                                          const u32x4* __restrict__ x,
                                                          u32x4* recv,
                                                          const float* __restrict__ wts,
                                                          void* __restrict__ out, Work w,
                                                          Sched S, int lds_count_run) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ int s_tk, s_ok, s_bad;
  const int tid = threadIdx.x;
  // Counter c lives at pipe[c * kPipeSlot].
  int32_t* pipe = w.pipe;
  int32_t* ticket = pipe + kPipeTicket * kPipeSlot;
  int32_t* exits = pipe + kPipeExit * kPipeSlot;
  int32_t* stall = pipe + kPipeStall * kPipeSlot;
  int32_t* count_done = pipe + kPipeHead * kPipeSlot;
  int32_t* scan_done = count_done + d.nbands * kPipeSlot;
  int32_t* gather_done = scan_done + d.nbands * kPipeSlot;

  // Count and scan share the dynamic LDS (never both in one ticket).
  int* s_ints = reinterpret_cast<int*>(s_dyn);
  const CountLds cl{reinterpret_cast<unsigned long long*>(s_dyn),
                    s_ints + lds_count_run - kPlanWaves * d.E, s_ints + lds_count_run, nullptr,
                    nullptr, &s_bad};
  const ScanLds sl{s_ints, s_ints + d.tpb * d.E, s_ints + d.tpb * d.E + d.E,
                   s_ints + d.tpb * d.E + d.E + kPlanWaves};

  // A block claims its next ticket once its work on the current one is
  // issued (thread 0 keeps the claim in a register): the atomic's round trip
  // then overlaps the wait for the ticket's stores, and no ticket waits in a
  // busy block while another block is free to take it (claimed at the start
  // of the current ticket instead, the last gathers of a band started only
  // when their blocks' previous tickets were done, and the band's combines
  // waited for them: olmoe 89.1 -> 83.5 us, qwen3 225.0 -> 211.5, nondiv
  // 358.2 -> 339.1).  A block works through its tickets in claim order, so
  // the lowest unfinished ticket is always the one its block is running.
  if (tid == 0) s_tk = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    __syncthreads();  // s_tk holds this ticket; the previous one is done with the LDS
    const int tk = s_tk;
    if (tk >= S.total) break;
    int next = 0;
    const Ticket t = decode(S, d.nbands, tk);

    bool ok = true;
    if (t.role != kCount) {
      int32_t* dep = (t.role == kScan ? count_done : t.role == kGather ? scan_done : gather_done) +
                     t.band * kPipeSlot;
      const int need = t.role == kScan ? (t.band == d.nbands - 1 ? S.last[kCount] : S.full[kCount])
                       : t.role == kGather ? 1
                       : (t.band == d.nbands - 1 ? S.last[kGather] : S.full[kGather]);
      if (tid == 0) s_ok = wait_for(dep, need, stall) ? 1 : 0;
      __syncthreads();
      ok = s_ok != 0;
    }

    const int t0 = t.band * d.band, t1 = min(t0 + d.band, d.T);
    if (ok) {
      switch (t.role) {
        case kCount: count_tile<KMAX, true>(d, idx, w, t.band * d.tpb + t.r, cl); break;
        case kScan: scan_band<true>(d, w, t.band, sl); break;
        case kGather:
          gather_chunk_lanes<KMAX, kPipeGatherU>(d, idx, x, recv, w, t.r, t0 * d.segs,
                                                 t1 * d.segs);
          break;
        default:
          combine_chunk_lanes<KMAX, kPipeCombineU, F32OUT>(d, recv, wts, w.slot_of, out, t.r,
                                                           t0 * d.segs, t1 * d.segs);
          break;
      }
    }
    if (tid == 0) next = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t.role != kCombine) {
      int32_t* done = (t.role == kCount ? count_done : t.role == kScan ? scan_done : gather_done) +
                      t.band * kPipeSlot;
      // This wave's device-scope stores have reached the coherence point.
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // everyone has read s_tk (and the LDS of this ticket)
    if (tid == 0) s_tk = next;
  }

  // Leave; the last block out reports a stall and clears the counters.
  if (tid == 0) {
    const int before = __hip_atomic_fetch_add(exits, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (before == (int)gridDim.x - 1) {
      if (__hip_atomic_load(stall, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT))
        for (int b = 0; b < d.nbands; ++b) w.band_status[b] = MOE_ERR_PIPELINE_STALL;
      for (int c = 0; c < kPipeHead + 3 * d.nbands; ++c) pipe[c * kPipeSlot] = 0;
    }
  }
}

__global__ void counters_clear_kernel(int32_t* pipe, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) pipe[i] = 0;
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Resident blocks of a kernel on the current device (occupancy x CUs).
template <typename K>
int resident_blocks(K kernel, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                   kBlock, lds) != hipSuccess)
    return 0;
  return per_cu * cus;
}

template <int KMAX>
struct PipelineLaunch {
  static hipError_t run(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                        const float* wts, void* out, bool out_f32, const Work& w, hipStream_t s) {
    // Dynamic LDS: count needs kPlanWaves * E ballots (64-bit), a
    // kPlanWaves * E prefix table and E running counts; scan needs the band's
    // tpb * E count matrix, E totals, kPlanWaves sums and kPlanBlock column parts.
    const int count_run = kPlanWaves * d.E * 3;  // in ints: ballots, then the prefix table
    const size_t count_bytes = sizeof(int) * ((size_t)count_run + d.E);
    const size_t scan_bytes = sizeof(int) * ((size_t)d.tpb * d.E + d.E + kPlanWaves + kPlanBlock);
    const size_t lds = (std::max(count_bytes, scan_bytes) + 15) / 16 * 16;
    auto kernel = out_f32 ? pipeline_kernel<KMAX, true> : pipeline_kernel<KMAX, false>;

    Sched S{};
    const int last_tokens = d.T - (d.nbands - 1) * d.band;
    const int gat = kWaves * kPipeGatherU, com = kWaves * kPipeCombineU;
    S.full[kCount] = d.tpb;
    S.last[kCount] = d.nblk - (d.nbands - 1) * d.tpb;
    S.full[kScan] = S.last[kScan] = 1;
    S.full[kGather] = ceil_div((int64_t)d.band * d.segs, gat);
    S.last[kGather] = ceil_div((int64_t)last_tokens * d.segs, gat);
    S.full[kCombine] = ceil_div((int64_t)d.band * d.segs, com);
    S.last[kCombine] = ceil_div((int64_t)last_tokens * d.segs, com);
    const int resident = resident_blocks(kernel, lds);
    if (resident <= 0) return hipErrorInvalidConfiguration;
    // Combine lag: about a grid's worth of tickets between gather(b) and combine(b).
    const int per_step = S.full[kCount] + 1 + S.full[kGather] + S.full[kCombine];
    const int lc = std::min(32, std::max(1, ceil_div(resident, per_step)));
    S.lag[kCount] = 0;
    S.lag[kScan] = kLagScan;
    S.lag[kGather] = S.lag[kScan] + kLagGather;
    S.lag[kCombine] = S.lag[kGather] + lc;
    S.nsteps = d.nbands + S.lag[kCombine];
    if (S.nsteps > kPipeMaxSteps) return hipErrorInvalidValue;
    int at = 0;
    for (int st = 0; st < S.nsteps; ++st) {
      S.step_start[st] = at;
      for (int role = 0; role < kRoles; ++role) {
        const int b = st - S.lag[role];
        if (b >= 0 && b < d.nbands) at += b == d.nbands - 1 ? S.last[role] : S.full[role];
      }
    }
    S.step_start[S.nsteps] = at;
    S.total = at;
    const int grid = std::min(S.total, resident);
    return launch(MOE_KERNEL_PIPELINE, kernel, dim3(grid), dim3(kBlock), (uint32_t)lds, s, d, idx,
                  reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(recv), wts, out, w, S,
                  count_run);
  }
};

template <template <int> class Launch, typename... A>
hipError_t by_topk(int k, A... a) {
  if (k <= 2) return Launch<2>::run(a...);
  if (k <= 4) return Launch<4>::run(a...);
  if (k <= 8) return Launch<8>::run(a...);
  return Launch<16>::run(a...);
}

}  // namespace

hipError_t launch_pipeline(const Dims& d, const int32_t* idx, const uint16_t* x, uint16_t* recv,
                           const float* wts, void* out, bool out_f32, const Work& w,
                           hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<PipelineLaunch>(d.k, d, idx, x, recv, wts, out, out_f32, w, s);
}

hipError_t launch_counters_clear(const Dims& d, const Work& w, hipStream_t s) {
  return launch(MOE_KERNEL_COUNTERS_CLEAR, counters_clear_kernel, dim3(1), dim3(kBlock), 0, s,
                w.pipe, (kPipeHead + 3 * d.nbands) * kPipeSlot);
}

}  // namespace moe
