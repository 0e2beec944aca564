// Device helpers shared by the route-plan and data-movement kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

// Part of element i under the contiguous ceil/floor split whose first `rem`
// parts hold base + 1 elements (TensorRT-LLM PR #13888, "support non-divisible
// EP in MoE alltoall", performance commit message: base and remainder are
// computed once per kernel, and a zero remainder takes a single divide).
__device__ __forceinline__ int split_part(int i, int base, int rem) {
  if (rem == 0) return i / base;
  const int cut = rem * (base + 1);
  return i < cut ? i / (base + 1) : rem + (i - cut) / base;
}

// Plan-array accesses.  COH = false: plain loads and stores (one kernel per
// step; the kernel boundary publishes everything).  COH = true: device-scope
// (sc1) accesses, for arrays one block writes and a block on another XCD
// reads inside the same launch (the banded pipeline): they go past the
// per-XCD L2 to the coherence point, so no cache-wide write-back or
// invalidate is needed to hand them over.
template <bool COH>
__device__ __forceinline__ int32_t ld_plan(const int32_t* p) {
  if constexpr (COH)
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

template <bool COH>
__device__ __forceinline__ void st_plan(int32_t* p, int32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Index of slot j of the token whose slots start at `at`: j itself for
// j < k, else slot 0 (an address inside the token's row, so the per-slot
// loads below need no branch and all of them issue before the first wait).
__device__ __forceinline__ int64_t slot_index(int64_t at, int j, int k) { return at + (j < k ? j : 0); }

// Receive row of every slot of token t: the row of (tile, expert) from the
// scan plus the slot's rank inside the tile; -1 for a dropped slot.  Two
// rounds of loads: ranks and expert ids, then the tile bases (branch-free,
// so each round issues together: the gather measured 26.9 -> 26.0 us on
// olmoe against per-slot loads).
template <int KMAX>
__device__ __forceinline__ void token_slots(const Dims& d, const Work& w,
                                            const int32_t* __restrict__ idx, int t,
                                            int (&slot)[KMAX]) {
  const int64_t at = (int64_t)t * d.k;
  int l[KMAX], e[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int64_t a = slot_index(at, j, d.k);
    l[j] = w.lr[a];
    e[j] = idx[a];
  }
  const int b = t / d.tile;
  int base[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) base[j] = w.tile_base[b * d.E + min(max(e[j], 0), d.E - 1)];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) slot[j] = (j < d.k && l[j] >= 0) ? base[j] + l[j] : -1;
}

// Staging row feeding every slot of token t (node deduplication): the first
// slot of a node owns the row (tile base of its forwarder plus its rank),
// later slots of the same node share it; -1 for a dropped slot.
// `lead` gets bit j set when slot j is the first slot of its node.
template <int KMAX>
__device__ __forceinline__ void token_stages(const Dims& d, const Work& w, int t,
                                             int (&p)[KMAX], uint32_t& lead) {
  const int64_t at = (int64_t)t * d.k;
  const int b = t / d.tile;
  int key[KMAX];
  lead = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    key[j] = j < d.k ? w.fkey[at + j] : -1;
    p[j] = key[j] >= 0 ? w.tile_fbase[b * d.fkeys + key[j]] + w.flr[at + j] : -1;
    if (key[j] >= 0) lead |= 1u << j;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
#pragma unroll
    for (int jj = 0; jj < j; ++jj)
      if (key[j] == -2 - jj) p[j] = p[jj];
}

// token_slots with the loads of one slot after another.  The staging kernel,
// which also resolves the token's staging rows, measured faster this way
// (DeepSeek-V3-like stage A 252 -> 224 us).
template <int KMAX>
__device__ __forceinline__ void token_slots_serial(const Dims& d, const Work& w,
                                                   const int32_t* __restrict__ idx, int t,
                                                   int (&slot)[KMAX]) {
  const int64_t at = (int64_t)t * d.k;
  const int b = t / d.tile;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    slot[j] = -1;
    if (j < d.k) {
      const int l = w.lr[at + j];
      if (l >= 0) slot[j] = w.tile_base[b * d.E + idx[at + j]] + l;
    }
  }
}

}  // namespace moe
