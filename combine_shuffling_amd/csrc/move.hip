// Data movement on gfx950: dispatch (gather-send fused with scatter-recv),
// the two hops of node-deduplicated dispatch, and the weighted combine.
//
// All four kernels stream whole rows of 2H bytes as 16-byte chunks.  The work
// is the flat list of (row, chunk) items; 64 consecutive lanes cover 1 KiB of
// consecutive chunks, so every load and store instruction of a wave touches
// whole contiguous rows (coalesced, no LDS staging needed: source and
// destination rows are both contiguous).  Each thread handles U items spaced
// one block apart and issues all of their loads before any store, to keep
// enough bytes in flight to cover HBM latency.
//
//  gather   dispatch, single hop: each source row x[t] is read once and
//           written to its k receive rows (FUSCO article, "core innovation":
//           no pack buffer before the send, no reorder after the receive).
//  stage_a  deduplicated dispatch, hop 1: x[t] is read once and written once
//           per distinct destination node, to that node's forwarder staging
//           row (FUSCO article, "load balancing and cross-node
//           deduplication").
//  stage_b  hop 2, intra-node fan-out: each staging row is read once and
//           written to every receive row of its token on that node.
//  combine  out[t] = sum_j w[t,j] * y[slot_of[t,j]]: k row loads, one fp32
//           fused multiply-add per element and slot in ascending j starting
//           from 0, then round-to-nearest-even bf16 (or fp32) out (INC-MoE
//           abstract: combine back to each token's owner).
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherU = 4;   // items per thread, gather / stage kernels
constexpr int kCombineU = 2;  // items per thread, combine

__device__ __forceinline__ void store_row_chunk(u32x4* p, u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

template <int KMAX, int U>
__global__ __launch_bounds__(kMoveBlock) void gather_kernel(const u32x4* __restrict__ x,
                                                            u32x4* __restrict__ recv,
                                                            const int32_t* __restrict__ slot_of,
                                                            int k, int chunks, int items,
                                                            uint32_t rows) {
  const int first = blockIdx.x * (kMoveBlock * U) + threadIdx.x;
  int slot[U][KMAX];
  int col[U];
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = first + u * kMoveBlock;
    const bool ok = i < items;
    const int t = ok ? i / chunks : 0;
    col[u] = i - t * chunks;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) slot[u][j] = (ok && j < k) ? slot_of[t * k + j] : -1;
    if (ok) v[u] = x[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if ((uint32_t)slot[u][j] < rows)
        store_row_chunk(&recv[(int64_t)slot[u][j] * chunks + col[u]], v[u]);
}

// Hop 1: one write per distinct destination node (a node's first slot holds
// the staging row; later slots of the same node repeat it).
template <int KMAX, int U>
__global__ __launch_bounds__(kMoveBlock) void stage_a_kernel(const u32x4* __restrict__ x,
                                                             u32x4* __restrict__ staging,
                                                             const int32_t* __restrict__ stage_of,
                                                             int k, int chunks, int items,
                                                             uint32_t rows) {
  const int first = blockIdx.x * (kMoveBlock * U) + threadIdx.x;
  int row[U][KMAX];
  int col[U];
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = first + u * kMoveBlock;
    const bool ok = i < items;
    const int t = ok ? i / chunks : 0;
    col[u] = i - t * chunks;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) row[u][j] = (ok && j < k) ? stage_of[t * k + j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
      for (int jj = 0; jj < j; ++jj)
        if (row[u][jj] == row[u][j]) row[u][j] = -1;
    if (ok) v[u] = x[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if ((uint32_t)row[u][j] < rows)
        store_row_chunk(&staging[(int64_t)row[u][j] * chunks + col[u]], v[u]);
}

// Hop 2: staging row p (token stage_src[p]) goes to every slot of that token
// whose staging row is p.  Rows at or past D (ctrl[1]) are unused.
template <int KMAX, int U>
__global__ __launch_bounds__(kMoveBlock) void stage_b_kernel(const u32x4* __restrict__ staging,
                                                             u32x4* __restrict__ recv,
                                                             const int32_t* __restrict__ stage_src,
                                                             const int32_t* __restrict__ stage_of,
                                                             const int32_t* __restrict__ slot_of,
                                                             const int32_t* __restrict__ ctrl, int k,
                                                             int chunks, int items_max, int T,
                                                             uint32_t rows) {
  const int items = min(items_max, ctrl[1] * chunks);
  const int first = blockIdx.x * (kMoveBlock * U) + threadIdx.x;
  int dst[U][KMAX];
  int col[U];
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = first + u * kMoveBlock;
    const bool ok = i < items;
    const int p = ok ? i / chunks : 0;
    col[u] = i - p * chunks;
    int t = ok ? stage_src[p] : 0;
    const bool tok = ok && (uint32_t)t < (uint32_t)T;
    t = tok ? t : 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      dst[u][j] = -1;
      if (tok && j < k && stage_of[t * k + j] == p) dst[u][j] = slot_of[t * k + j];
    }
    if (ok) v[u] = staging[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if ((uint32_t)dst[u][j] < rows)
        store_row_chunk(&recv[(int64_t)dst[u][j] * chunks + col[u]], v[u]);
}

// float -> bf16 bits, round to nearest even; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int KMAX, int U, bool F32OUT>
__global__ __launch_bounds__(kMoveBlock) void combine_kernel(const u32x4* __restrict__ y,
                                                             const float* __restrict__ wts,
                                                             const int32_t* __restrict__ slot_of,
                                                             void* __restrict__ out, int k,
                                                             int chunks, int items, uint32_t rows) {
  const int first = blockIdx.x * (kMoveBlock * U) + threadIdx.x;
  int slot[U][KMAX];
  float wj[U][KMAX];
  u32x4 v[U][KMAX];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = first + u * kMoveBlock;
    const bool ok = i < items;
    const int t = ok ? i / chunks : 0;
    const int c = i - t * chunks;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      slot[u][j] = (ok && j < k) ? slot_of[t * k + j] : -1;
      if ((uint32_t)slot[u][j] >= rows) slot[u][j] = -1;
      wj[u][j] = (ok && j < k) ? wts[t * k + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[u][j] >= 0) v[u][j] = y[(int64_t)slot[u][j] * chunks + c];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = first + u * kMoveBlock;
    if (i >= items) continue;
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
    if constexpr (F32OUT) {
      f32x4* o = reinterpret_cast<f32x4*>(out) + (int64_t)i * 2;
      const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
      const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
      __builtin_nontemporal_store(a, o);
      __builtin_nontemporal_store(b, o + 1);
    } else {
      u32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
      store_row_chunk(reinterpret_cast<u32x4*>(out) + i, r);
    }
  }
}

inline int blocks_for(int64_t items, int per_thread) {
  const int64_t per_block = (int64_t)kMoveBlock * per_thread;
  return (int)((items + per_block - 1) / per_block);
}

template <template <int> class Launch, typename... A>
hipError_t by_topk(int k, A... a) {
  if (k <= 2) return Launch<2>::run(a...);
  if (k <= 4) return Launch<4>::run(a...);
  if (k <= 8) return Launch<8>::run(a...);
  return Launch<16>::run(a...);
}

template <int KMAX>
struct GatherLaunch {
  static hipError_t run(const Dims& d, const uint16_t* x, uint16_t* recv, const Work& w,
                        hipStream_t s) {
    const int items = d.T * d.chunks;
    hipLaunchKernelGGL((gather_kernel<KMAX, kGatherU>), dim3(blocks_for(items, kGatherU)),
                       dim3(kMoveBlock), 0, s, reinterpret_cast<const u32x4*>(x),
                       reinterpret_cast<u32x4*>(recv), w.slot_of, d.k, d.chunks, items,
                       (uint32_t)(d.T * d.k));
    return hipGetLastError();
  }
};

template <int KMAX>
struct StageALaunch {
  static hipError_t run(const Dims& d, const uint16_t* x, uint16_t* staging, const Work& w,
                        int64_t rows_max, hipStream_t s) {
    const int items = d.T * d.chunks;
    hipLaunchKernelGGL((stage_a_kernel<KMAX, kGatherU>), dim3(blocks_for(items, kGatherU)),
                       dim3(kMoveBlock), 0, s, reinterpret_cast<const u32x4*>(x),
                       reinterpret_cast<u32x4*>(staging), w.stage_of, d.k, d.chunks, items,
                       (uint32_t)rows_max);
    return hipGetLastError();
  }
};

template <int KMAX>
struct StageBLaunch {
  static hipError_t run(const Dims& d, const uint16_t* staging, uint16_t* recv, const Work& w,
                        int64_t rows_max, hipStream_t s) {
    const int items = (int)(rows_max * d.chunks);
    hipLaunchKernelGGL((stage_b_kernel<KMAX, kGatherU>), dim3(blocks_for(items, kGatherU)),
                       dim3(kMoveBlock), 0, s, reinterpret_cast<const u32x4*>(staging),
                       reinterpret_cast<u32x4*>(recv), w.stage_src, w.stage_of, w.slot_of, w.ctrl,
                       d.k, d.chunks, items, d.T, (uint32_t)(d.T * d.k));
    return hipGetLastError();
  }
};

template <int KMAX>
struct CombineLaunch {
  static hipError_t run(const Dims& d, const uint16_t* y, const float* wts, void* out, bool f32,
                        const Work& w, hipStream_t s) {
    const int items = d.T * d.chunks;
    const dim3 grid(blocks_for(items, kCombineU));
    if (f32)
      hipLaunchKernelGGL((combine_kernel<KMAX, kCombineU, true>), grid, dim3(kMoveBlock), 0, s,
                         reinterpret_cast<const u32x4*>(y), wts, w.slot_of, out, d.k, d.chunks,
                         items, (uint32_t)(d.T * d.k));
    else
      hipLaunchKernelGGL((combine_kernel<KMAX, kCombineU, false>), grid, dim3(kMoveBlock), 0, s,
                         reinterpret_cast<const u32x4*>(y), wts, w.slot_of, out, d.k, d.chunks,
                         items, (uint32_t)(d.T * d.k));
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_gather(const Dims& d, const uint16_t* x, uint16_t* recv, const Work& w,
                         hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<GatherLaunch>(d.k, d, x, recv, w, s);
}

hipError_t launch_stage_a(const Dims& d, const uint16_t* x, uint16_t* staging, const Work& w,
                          int64_t staging_rows_max, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<StageALaunch>(d.k, d, x, staging, w, staging_rows_max, s);
}

hipError_t launch_stage_b(const Dims& d, const uint16_t* staging, uint16_t* recv, const Work& w,
                          int64_t staging_rows_max, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<StageBLaunch>(d.k, d, staging, recv, w, staging_rows_max, s);
}

hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* wts, void* out,
                          bool out_f32, const Work& w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  return by_topk<CombineLaunch>(d.k, d, y, wts, out, out_f32, w, s);
}

}  // namespace moe
