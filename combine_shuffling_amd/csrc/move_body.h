// Device bodies of the single-hop data movement (gather, combine) and their
// helpers, shared by the one-kernel-per-step path (move.hip) and the banded
// pipeline (pipeline.hip).  The work unit and the method are described in
// move.hip.
#pragma once

#include "moe_device.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;           // waves per block of the movement kernels
constexpr int kBlock = kWaves * kWave;
constexpr int kGatherU = 1;         // wave-items per wave: gather
constexpr int kStageU = 2;          // wave-items per wave: stage_b
// Wave-items per wave of the combine: one, so that more waves are resident
// (whole steps with x read from HBM, one stream: olmoe 59.2 -> 56.8 us,
// dsv3 1180 -> 1176 against two).
constexpr int kCombineU = 1;
// ... of the fp8 combine (one stream: qwen3 step 132.4 -> 122.4 us against two).
constexpr int kCombine8U = 1;
// Waves per block of the bf16 combine.  Timed alone after a cache flush,
// against 1-wave blocks: nondiv 160.0 -> 158.2 us, qwen3, dsv3 and olmoe
// level (4-wave blocks: nondiv 165.8, qwen3 104.6, dsv3 374.5).
constexpr int kCombineWaves = 2;
// ... of the fp8 combine: 2-wave blocks made qwen3 fp8 118.1 us against 114.7.
constexpr int kCombine8Waves = 4;
// Wave-items per launch at most: a grid is sized in work-items, a 32-bit count,
// so a batch of more wave-items is moved in several launches (2^24 items of
// at most 64 threads each).
constexpr int64_t kMaxLaunchItems = (int64_t)1 << 24;

// Rows are touched once per call: stream them past the caches (measured
// faster on gfx950 for both the row reads and the row writes).
template <typename V>
__device__ __forceinline__ void store_chunk(V* p, V v) {
  __builtin_nontemporal_store(v, p);
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
  return __builtin_nontemporal_load(p);
}

// Buffer descriptor of the `bytes` bytes at p, or of an empty range when
// `valid` is false: a buffer access outside the range is dropped (a store)
// or reads zero (a load), so an access through it needs no branch.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor, word 3 (gfx9 family)
constexpr int kCacheNt = 1 << 1;          // buffer cache policy: streaming (nt)
constexpr int kCacheSc1 = 1 << 4;         // buffer cache policy: device scope (sc1)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void* p, bool valid,
                                                             int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, valid ? bytes : 0,
                                           kBufferWord3);
}

// Row store that another block reads in the same launch (the banded
// pipeline): chunk at byte `off` of row `row` (wave-uniform) of a [rows,
// chunks] buffer when row < rows, a device-scope (sc1) store, written
// through the per-XCD L2 to the coherence point so that the reader needs no
// cache maintenance.  It is issued for every row and lane, through a
// descriptor of the row (scalar registers) with the lane's 32-bit offset:
// the descriptor's range discards a store that must not land.  Loads and
// stores share one counter of operations in flight on this GPU.  With the
// stores behind branches, or written as inline asm, or with a 64-bit
// address register per store in that kernel short of registers, the
// compiler waited for every operation in flight before each store (the
// previous store included): banded pipeline olmoe 100.9 -> 95.2 us, qwen3
// 273 -> 255, nondiv 460 -> 412 with this store and the lookups ahead of
// the row loads.  (The separate gather kernels keep plain branches and
// global stores: the same store there made nondiv's gather 147 -> 186 us.)
__device__ __forceinline__ void store_row_coherent(u32x4* base, int row, uint32_t rows,
                                                   int chunks, uint32_t off, u32x4 v) {
  const bool valid = (uint32_t)row < rows;
  const __amdgpu_buffer_rsrc_t r =
      row_buffer(base + (int64_t)(valid ? row : 0) * chunks, valid, chunks * (int)sizeof(u32x4));
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCacheSc1);
}

// Token rows of x (dispatch source): plain loads measured faster here.
__device__ __forceinline__ u32x4 load_x_chunk(const u32x4* p) { return *p; }

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
  const int seg = it.live ? g - it.t * d.segs : 0;  // a dead item: token 0, segment 0
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
template <int KMAX, int U>
__device__ __forceinline__ void gather_chunk(const Dims& d, const int32_t* idx, const u32x4* x,
                                             u32x4* recv, const Work& w, int blk, int base,
                                             int limit) {
  const int lane = threadIdx.x % kWave;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const bool keep = keep_rows(rows, 2 * d.H);
  // Every wave-item's slot lookups (scalar loads, with a counter of their
  // own), then every row load (x after the slot loads: nondiv gather 152.6 ->
  // 158.8 us the other way round).
  Item it[U];
  int slot[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, base, limit, u);
    if (it[u].live) {
      token_slots<KMAX>(d, w, idx, it[u].t, slot[u]);
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) slot[u][j] = -1;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (it[u].ok) v[u] = load_x_chunk(&x[(int64_t)it[u].t * d.chunks + it[u].c]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // The first segment of a row publishes the token's slots.
    if (it[u].live && it[u].c == lane && lane < d.k) {
      const int s = lane_pick<KMAX>(slot[u], lane);
      w.slot_of[(int64_t)it[u].t * d.k + lane] = s;
      if ((uint32_t)s < rows) w.row_src[s] = it[u].t;
    }
    if (it[u].ok) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if ((uint32_t)slot[u][j] < rows)
          store_row(&recv[(int64_t)slot[u][j] * d.chunks + it[u].c], v[u], keep);
    }
  }
}

// The gather of the banded pipeline, whose plan arrays are read with
// device-scope loads.  Those are vector loads, which complete in issue order
// and share one counter with the row loads and stores; a wave-uniform
// lookup result also has to land before it can move to a scalar register.
// So lane j (< k) of the wave looks up slot j of each wave-item, all items'
// lookups in two rounds (ranks and expert ids, then tile bases), and the
// slots are read out of the lanes (v_readlane) once they have all landed:
// two round trips a ticket, however many items.  Then every x load, then
// every row store, unconditional (store_row_coherent).
template <int KMAX, int U>
__device__ __forceinline__ void gather_chunk_lanes(const Dims& d, const int32_t* idx,
                                                   const u32x4* x, u32x4* recv, const Work& w,
                                                   int blk, int base, int limit) {
  const int lane = threadIdx.x % kWave;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  Item it[U];
  int l[U], e[U], slot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, base, limit, u);
    const bool has = it[u].live && lane < d.k;
    const int64_t a = has ? (int64_t)it[u].t * d.k + lane : 0;
    l[u] = ld_plan<true>(&w.lr[a]);
    e[u] = idx[a];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = it[u].t / d.tile;
    const int tb = ld_plan<true>(&w.tile_base[b * d.E + min(max(e[u], 0), d.E - 1)]);
    slot[u] = it[u].live && lane < d.k && l[u] >= 0 ? tb + l[u] : -1;
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = load_x_chunk(&x[it[u].ok ? (int64_t)it[u].t * d.chunks + it[u].c : 0]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t off = (uint32_t)it[u].c * (uint32_t)sizeof(u32x4);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      store_row_coherent(recv, __builtin_amdgcn_readlane(slot[u], j), rows, d.chunks, off, v[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // The first segment of a row publishes the token's slots.
    if (it[u].live && it[u].c == lane && lane < d.k) {
      st_plan<true>(&w.slot_of[(int64_t)it[u].t * d.k + lane], slot[u]);
      if ((uint32_t)slot[u] < rows) w.row_src[slot[u]] = it[u].t;
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
template <int KMAX, int U, bool F32OUT, int W = kWaves>
__device__ __forceinline__ void combine_chunk(const Dims& d, const u32x4* y, const float* wts,
                                              const int32_t* slot_of, void* out, int blk, int base,
                                              int limit) {
  const uint32_t rows = (uint32_t)(d.T * d.k);
  // Every wave-item's slots and weights, then every row load (the order
  // gather_chunk keeps, for the same reason).
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
      sj[j] = slot_of[a];
      wt[j] = wts[a];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool has = it[u].live && j < d.k;
      slot[u][j] = has && (uint32_t)sj[j] < rows ? sj[j] : -1;
      wj[u][j] = has ? wt[j] : 0.0f;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[u][j] >= 0 && it[u].ok)
        v[u][j] = load_chunk(&y[(int64_t)slot[u][j] * d.chunks + it[u].c]);
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

// The combine of the banded pipeline: slot_of is read with device-scope
// loads, so, as in gather_chunk_lanes, lane j (< k) looks up slot j and
// weight j of each wave-item, one round for all items, and the slots and
// weights are read out of the lanes.  The receive rows are read through a
// descriptor of the row (an empty one for a dropped slot; a lane past the
// row reads zero) and the outputs are written through one of the output
// row, so no load or store sits behind a branch.
template <int KMAX, int U, bool F32OUT>
__device__ __forceinline__ void combine_chunk_lanes(const Dims& d, const u32x4* y,
                                                    const float* wts, const int32_t* slot_of,
                                                    void* out, int blk, int base, int limit) {
  const int lane = threadIdx.x % kWave;
  const uint32_t rows = (uint32_t)(d.T * d.k);
  const int row_bytes = d.chunks * (int)sizeof(u32x4);
  Item it[U];
  int slot[U];
  float wt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    it[u] = wave_item<U>(d, blk, base, limit, u);
    const bool has = it[u].live && lane < d.k;
    const int64_t a = has ? (int64_t)it[u].t * d.k + lane : 0;
    slot[u] = ld_plan<true>(&slot_of[a]);
    wt[u] = wts[a];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool has = it[u].live && lane < d.k && (uint32_t)slot[u] < rows;
    slot[u] = has ? slot[u] : -1;
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int off = it[u].c * (int)sizeof(u32x4);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int s = __builtin_amdgcn_readlane(slot[u], j);
      const __amdgpu_buffer_rsrc_t r = row_buffer(y + (int64_t)(s >= 0 ? s : 0) * d.chunks,
                                                  s >= 0, row_bytes);
      v[u][j] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNt);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (__builtin_amdgcn_readlane(slot[u], j) < 0) continue;  // wave-uniform
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt[u]), j));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(v[u][j][q] << 16);
        const float hi = __uint_as_float(v[u][j][q] & 0xffff0000u);
        acc[2 * q] = __builtin_fmaf(wj, lo, acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wj, hi, acc[2 * q + 1]);
      }
    }
    const int64_t row = it[u].live ? it[u].t : 0;
    if constexpr (F32OUT) {
      const __amdgpu_buffer_rsrc_t r = row_buffer(reinterpret_cast<f32x4*>(out) + row * 2 * d.chunks,
                                                  it[u].live, 2 * row_bytes);
      const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
      const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), r, 2 * it[u].c * 16, 0,
                                             kCacheNt);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), r, 2 * it[u].c * 16 + 16,
                                             0, kCacheNt);
    } else {
      const __amdgpu_buffer_rsrc_t r =
          row_buffer(reinterpret_cast<u32x4*>(out) + row * d.chunks, it[u].live, row_bytes);
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
      __builtin_amdgcn_raw_buffer_store_b128(o, r, it[u].c * 16, 0, kCacheNt);
    }
  }
}

// Wave-items [base, limit) of the batch (one launch of at most kMaxLaunchItems).
template <int KMAX, int U, bool F32OUT>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    Dims d, const u32x4* __restrict__ y, const float* __restrict__ wts,
    const int32_t* __restrict__ slot_of, void* __restrict__ out, int base, int limit) {
  combine_chunk<KMAX, U, F32OUT, kCombineWaves>(d, y, wts, slot_of, out, blockIdx.x, base,
                                                       limit);
}

}  // namespace
}  // namespace moe
