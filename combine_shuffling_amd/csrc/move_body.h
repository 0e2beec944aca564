// Device bodies of the single-hop data movement (gather, combine) and their
// helpers, shared by the one-kernel-per-step path (move.hip) and the banded
// pipeline (pipeline.hip).  The work unit and the method are described in
// move.hip.
#pragma once

#include "moe_device.h"

#ifndef MOE_GATHER_U
#define MOE_GATHER_U 1
#endif
#ifndef MOE_STAGE_U
#define MOE_STAGE_U 2
#endif
#ifndef MOE_COMBINE_U
// one wave-item per wave: more waves resident (measured in whole steps with
// x read from HBM, one stream: olmoe 59.2 -> 56.8 us, dsv3 1180 -> 1176 against 2)
#define MOE_COMBINE_U 1
#endif
#ifndef MOE_NT_LOAD
#define MOE_NT_LOAD 1
#endif
#ifndef MOE_COMBINE8_U
#define MOE_COMBINE8_U 1  // fp8 payload, one stream: qwen3 step 132.4 -> 122.4 us against 2
#endif
#ifndef MOE_NT_LOAD_X
#define MOE_NT_LOAD_X 0
#endif
#ifndef MOE_COMBINE_WAVES
// waves per block of the bf16 combine; best step, against 4-wave blocks:
// qwen3 205.2 -> 203.9 us, nondiv 339.1 -> 335.6, dsv3 1083.3 -> 1078.2,
// olmoe unchanged (2-wave blocks: olmoe 48.9 against 48.3, dsv3 1075)
#define MOE_COMBINE_WAVES 1
#endif
#ifndef MOE_COMBINE8_WAVES
// ... of the fp8 combine: 2-wave blocks made qwen3 fp8 118.1 us against 114.7
#define MOE_COMBINE8_WAVES 4
#endif
#ifndef MOE_MOVE_WAVES
#define MOE_MOVE_WAVES 4
#endif
#ifndef MOE_NT_STORE
#define MOE_NT_STORE 1
#endif

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = MOE_MOVE_WAVES;   // waves per block
constexpr int kBlock = kWaves * kWave;
constexpr int kGatherU = MOE_GATHER_U;    // wave-items per wave: gather
constexpr int kStageU = MOE_STAGE_U;      // wave-items per wave: stage_b (stage_a in move.hip)
constexpr int kCombineU = MOE_COMBINE_U;  // wave-items per wave: combine
constexpr int kCombine8U = MOE_COMBINE8_U; // wave-items per wave: combine of an fp8 payload
constexpr int kCombineWaves = MOE_COMBINE_WAVES;    // waves per block of the bf16 combine
constexpr int kCombine8Waves = MOE_COMBINE8_WAVES;  // ... of the fp8 combine
// Wave-items per launch at most: a grid is sized in work-items, a 32-bit count,
// so a batch of more wave-items is moved in several launches (2^24 items of
// at most 64 threads each).
constexpr int64_t kMaxLaunchItems = (int64_t)1 << 24;

// Rows are touched once per call: stream them past the caches (measured
// faster on gfx950 for both the row reads and the row writes).
template <typename V>
__device__ __forceinline__ void store_chunk(V* p, V v) {
#if MOE_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Rows that the next kernel of the step reads back (receive rows for the
// combine, staging rows for stage B) are written with plain stores when
// the whole buffer fits in half of the 256 MB MALL (AMD Infinity Cache), so
// the reader finds them there; half, so that two batches in flight both fit
// (OLMoE-like step, one stream: 63.6 -> 59.2 us).  Larger buffers would only
// evict each other and are streamed past the caches.
constexpr int64_t kKeepBytes = (int64_t)128 << 20;

__device__ __forceinline__ bool keep_rows(int64_t rows, int64_t row_bytes) {
  return rows * row_bytes <= kKeepBytes;
}

template <typename V>
__device__ __forceinline__ void store_row(V* p, V v, bool keep) {
  if (keep)
    *p = v;
  else
    store_chunk(p, v);
}

__device__ __forceinline__ u32x4 load_chunk(const u32x4* p) {
#if MOE_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Row store that another block reads in the same launch (the banded
// pipeline): a device-scope (sc1) 16-byte store, written through the per-XCD
// L2 to the coherence point, so the reader needs no cache maintenance.
template <bool COH>
__device__ __forceinline__ void store_row_chunk(u32x4* p, u32x4 v, bool keep) {
  if constexpr (COH)
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
  else
    store_row(p, v, keep);
}

// Token rows of x (dispatch source): plain loads measured faster here.
__device__ __forceinline__ u32x4 load_x_chunk(const u32x4* p) {
#if MOE_NT_LOAD_X
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Wave-item u of this wave: token t, chunk c of the lane, and whether the
// item exists / the lane's chunk is inside the row.
struct Item {
  int t, c;
  bool live, ok;
};

// Wave-items are numbered g = base + (blk * U + u) * W + wave (W waves a
// block); those at or past `limit` do not exist.  A kernel takes blk = its
// block index and its launch's range; the banded pipeline takes blk from its
// ticket and the band's range.
template <int U, int W = kWaves>
__device__ __forceinline__ Item wave_item(const Dims& d, int blk, int base, int limit, int u) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = __builtin_amdgcn_readfirstlane(base + (blk * U + u) * W + wave);
  Item it;
  it.live = g < limit;
  it.t = it.live ? g / d.segs : 0;
  const int seg = g - it.t * d.segs;
  it.c = seg * kWave + lane;
  it.ok = it.live && it.c < d.chunks;
  return it;
}


// Lane j (< k) writes the token's entry j of a per-slot plan array.
template <int KMAX>
__device__ __forceinline__ int lane_pick(const int (&v)[KMAX], int lane) {
  int r = -1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) r = lane == j ? v[j] : r;
  return r;
}

// Gather-send fused with scatter-recv for the wave-items of block-chunk blk.
template <int KMAX, int U, bool COH = false>
__device__ __forceinline__ void gather_chunk(const Dims& d, const int32_t* idx, const u32x4* x,
                                             u32x4* recv, const Work& w, int blk, int base,
                                             int limit) {
  const int lane = threadIdx.x % kWave;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const bool keep = keep_rows(rows, 2 * d.H);
  Item it[U];
  int slot[U][KMAX];
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, base, limit, u);
    if (it[u].live) {
      token_slots<KMAX, COH>(d, w, idx, it[u].t, slot[u]);
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) slot[u][j] = -1;
    }
    // after the slot loads (loading x first: nondiv gather 152.6 -> 158.8 us)
    if (it[u].ok) v[u] = load_x_chunk(&x[(int64_t)it[u].t * d.chunks + it[u].c]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // The first segment of a row publishes the token's slots.
    if (it[u].live && it[u].c == lane && lane < d.k) {
      const int s = lane_pick<KMAX>(slot[u], lane);
      st_plan<COH>(&w.slot_of[(int64_t)it[u].t * d.k + lane], s);
      if ((uint32_t)s < rows) w.row_src[s] = it[u].t;
    }
    if (it[u].ok) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if ((uint32_t)slot[u][j] < rows)
          store_row_chunk<COH>(&recv[(int64_t)slot[u][j] * d.chunks + it[u].c], v[u], keep);
    }
  }
}

// Wave-items [base, limit) of the batch (one launch of at most kMaxLaunchItems).
template <int KMAX, int U>
__global__ __launch_bounds__(kBlock) void gather_kernel(Dims d, const int32_t* __restrict__ idx,
                                                        const u32x4* __restrict__ x,
                                                        u32x4* __restrict__ recv, Work w, int base,
                                                        int limit) {
  gather_chunk<KMAX, U>(d, idx, x, recv, w, blockIdx.x, base, limit);
}

__device__ __forceinline__ void unpack_bf16(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(v[q] << 16);
    f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
  }
}

// float -> bf16 bits, round to nearest even; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Weighted combine for the wave-items of block-chunk blk (W waves a block).
template <int KMAX, int U, bool F32OUT, bool COH = false, int W = kWaves>
__device__ __forceinline__ void combine_chunk(const Dims& d, const u32x4* y, const float* wts,
                                              const int32_t* slot_of, void* out, int blk, int base,
                                              int limit) {
  const uint32_t rows = (uint32_t)(d.T * d.k);
  Item it[U];
  int slot[U][KMAX];
  float wj[U][KMAX];
  u32x4 v[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U, W>(d, blk, base, limit, u);
    const int64_t at = (int64_t)it[u].t * d.k;
    int sj[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {  // no branch between the loads: they issue together
      const int64_t a = slot_index(at, j, d.k);
      sj[j] = ld_plan<COH>(&slot_of[a]);
      wt[j] = wts[a];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool has = it[u].live && j < d.k;
      slot[u][j] = has && (uint32_t)sj[j] < rows ? sj[j] : -1;
      wj[u][j] = has ? wt[j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[u][j] >= 0 && it[u].ok) v[u][j] = load_chunk(&y[(int64_t)slot[u][j] * d.chunks + it[u].c]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!it[u].ok) continue;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (slot[u][j] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(v[u][j][q] << 16);
        const float hi = __uint_as_float(v[u][j][q] & 0xffff0000u);
        acc[2 * q] = __builtin_fmaf(wj[u][j], lo, acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wj[u][j], hi, acc[2 * q + 1]);
      }
    }
    const int64_t i = (int64_t)it[u].t * d.chunks + it[u].c;
    if constexpr (F32OUT) {
      f32x4* o = reinterpret_cast<f32x4*>(out) + i * 2;
      const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
      const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
      store_chunk(o, a);
      store_chunk(o + 1, b);
    } else {
      u32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
      store_chunk(reinterpret_cast<u32x4*>(out) + i, r);
    }
  }
}

// Wave-items [base, limit) of the batch (one launch of at most kMaxLaunchItems).
template <int KMAX, int U, bool F32OUT>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    Dims d, const u32x4* __restrict__ y, const float* __restrict__ wts,
    const int32_t* __restrict__ slot_of, void* __restrict__ out, int base, int limit) {
  combine_chunk<KMAX, U, F32OUT, false, kCombineWaves>(d, y, wts, slot_of, out, blockIdx.x, base,
                                                       limit);
}

}  // namespace
}  // namespace moe
