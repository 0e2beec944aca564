/*
 * moe_shuffle.h -- C ABI of the MI355X (gfx950) MoE expert-parallel shuffle.
 *
 * What it computes.  Under expert parallelism the experts live on different
 * ranks, so every token must travel to the ranks that host the experts it was
 * routed to, and the experts' outputs must travel back (FUSCO article,
 * "pain points").  Dispatch moves tokens to the ranks hosting their selected
 * experts; combine returns the expert outputs to each token's owner (INC-MoE
 * abstract).  Here the R expert-parallel ranks are R virtual ranks, i.e.
 * partitions of one GPU's HBM, and every "send" is an HBM-to-HBM row copy.
 *
 *   moe_route_plan   top-k routing -> per-expert histogram -> exclusive scan ->
 *                    segment descriptors (FUSCO article, "core innovation":
 *                    gather-send is driven by segment descriptors);
 *   moe_dispatch     gather-send fused with scatter-recv: each source row is
 *                    read once and written straight into its final, expert-
 *                    contiguous receive row (same section).  With
 *                    MOE_FLAG_NODE_DEDUP the row first goes once to a
 *                    staging row per destination node (the node's forwarding
 *                    GPU), then fans out inside the node (FUSCO article,
 *                    "load balancing and cross-node deduplication");
 *   moe_combine      out[t] = sum_j w[t,j] * y[slot_of[t,j]], fp32 accumulate
 *                    in ascending j (INC-MoE abstract: combine back to the
 *                    owner).
 *
 * Expert-to-rank partition: contiguous ceil/floor split, the first E % R
 * ranks hold E / R + 1 experts (TensorRT-LLM PR #13888, "support non-
 * divisible EP in MoE alltoall", performance commit message: 256 experts over
 * 7 ranks -> base 36, remainder 4).  E < R is rejected (same PR, commit on
 * ranks left without experts).
 *
 * Layouts (all row-major, all device buffers 16-byte aligned):
 *   x        [T, H]      bf16 bit patterns (uint16), the tokens;
 *   topk_idx [T, k]      int32 expert ids, each in [0, E), distinct in a row;
 *   topk_w   [T, k]      float32 combine weights, applied as given;
 *   recv     [T*k, H]    bf16: rank d's rows are [rank_off[d], rank_off[d+1]),
 *                        expert e's rows [expert_off[e], expert_off[e+1]),
 *                        tokens ascending inside an expert;
 *   staging  [Dmax, H]   bf16, rows ordered by (forwarder rank, token); the
 *                        forwarder of (token t, node n) is rank
 *                        n*G + owner(t) % G (or the load-aware choice, see
 *                        MOE_FLAG_LOAD_AWARE_FORWARDERS), owner(t) being the
 *                        contiguous ceil/floor split of the T tokens over R;
 *   out      [T, H]      bf16 (round to nearest even) or float32.
 *
 * Ownership.  The caller owns every device buffer (inputs, outputs and the
 * workspace).  The library owns only the host-side plan object; it never
 * allocates device memory and never synchronises except in moe_plan_read.
 * moe_route_plan binds topk_idx and the workspace to the plan: both must stay
 * alive and unmodified by anyone else until the last moe_dispatch /
 * moe_combine / moe_plan_read using that routing has completed on the stream.
 * Every call is asynchronous on the given stream (a hipStream_t; NULL = the
 * null stream).  A plan is not thread-safe; calls on one workspace that
 * overlap in time (different streams without ordering) race.
 *
 * Bands.  With band_tokens = B > 0 and B < T the batch is cut into
 * nb = ceil(T / B) bands; band b holds tokens [b*B, min((b+1)*B, T)) and owns
 * receive rows [b*B*k, min((b+1)*B, T)*k), laid out inside like a whole
 * batch's receive buffer (INC-MoE abstract: tokens are partitioned into bands
 * that go through dispatch, expert and combine one after another).  Every
 * call works on banded plans; COUNTS, EXPERT_OFFSETS and RANK_OFFSETS then
 * hold one row per band (global receive rows), and moe_pipeline runs the
 * whole path band by band in one launch.  Limits: B * E <= 2^21 (a band's
 * tile-count matrix fits the scan's LDS), nb <= 192.
 *
 * Errors.  Host-detectable errors return before anything is launched.  Bad
 * routing (an id outside [0, E) or repeated in a row) is found on the device:
 * such slots are dropped (no row is written for them, they add nothing to the
 * combine, their slot_of entry is -1), every access stays in bounds, and
 * moe_plan_read(MOE_ITEM_STATUS) reports MOE_ERR_BAD_ROUTING.
 */
#ifndef MOE_SHUFFLE_H
#define MOE_SHUFFLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null, negative, misaligned or inconsistent arguments */
  MOE_ERR_EXPERTS_LT_RANKS = 2, /* E < R: the split would leave ranks without experts  */
  MOE_ERR_BAD_ROUTING = 3,      /* device found an id out of range or repeated in a row */
  MOE_ERR_PLAN_NOT_ROUTED = 4,  /* dispatch/combine/read before moe_route_plan          */
  MOE_ERR_HIP = 5,              /* a HIP runtime call or kernel launch failed           */
  MOE_ERR_UNSUPPORTED = 6,      /* sizes beyond the library's limits (below)            */
  MOE_ERR_PIPELINE_STALL = 7,   /* a banded-pipeline wait gave up (moe_pipeline)         */
  MOE_ERR_STATIC_WORKSPACE = 8  /* moe_route_plan_static: the plan's workspace is larger
                                   than MOE_STATIC_WORKSPACE_BYTES                        */
} moe_status;

/* Limits: E <= 1024, 1 <= k <= 16, k <= E, R <= E, R % G == 0, H % 8 == 0,
 * T*k, T*H/8 and (with node dedup) T*min(k,N)*H/8 each below 2^31 - 4096
 * (row indices are 32-bit, byte offsets 64-bit); beyond, MOE_ERR_UNSUPPORTED.
 * Batches of more than 2^24 wave-items (1 KiB row segments) are moved in
 * several launches, since a grid counts its work-items in 32 bits. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/* Node deduplication (one copy per (token, node), then intra-node fan-out).
 * Requires N = R / G > 1. */
#define MOE_FLAG_NODE_DEDUP 1u
/* With MOE_FLAG_NODE_DEDUP: choose each (owner rank s, node n)'s forwarder by
 * load instead of the static n*G + s % G (FUSCO article, "load balancing and
 * cross-node deduplication": forwarding follows the load and is spread evenly
 * over the node's GPUs; the rule is a reading).  In each node the owners are
 * ranked by the rows they stage for it (more first, ties to the lower owner)
 * and dealt to the node's G ranks in snake order 0..G-1, G-1..0, ...
 * Requires R * N <= MOE_MAX_EXPERTS. */
#define MOE_FLAG_LOAD_AWARE_FORWARDERS 2u

typedef struct moe_config {
  int64_t num_tokens;     /* T >= 0 (0 is an empty batch: every call is a no-op) */
  int32_t hidden;         /* H > 0, multiple of 8 (row = 2H bytes, 16-byte chunks) */
  int32_t num_experts;    /* E, 1..MOE_MAX_EXPERTS                                 */
  int32_t top_k;          /* k, 1..min(E, MOE_MAX_TOPK)                             */
  int32_t num_ranks;      /* R, 1..E                                               */
  int32_t ranks_per_node; /* G, divides R; N = R / G nodes                          */
  uint32_t flags;         /* MOE_FLAG_*                                             */
  int32_t band_tokens;    /* 0: one band.  Else a multiple of 256: the tokens are cut
                             into bands of band_tokens consecutive tokens (the last
                             may be shorter), each routed as a batch of its own (see
                             "Bands" below).  Not with MOE_FLAG_NODE_DEDUP.          */
} moe_config;

typedef struct moe_plan moe_plan; /* opaque, host-side */

/* What moe_plan_read copies out (all int32 unless noted). */
typedef enum moe_item {
  MOE_ITEM_STATUS = 0,         /* 1 value: moe_status of the last route (MOE_OK, MOE_ERR_BAD_ROUTING,
                                  or MOE_ERR_PIPELINE_STALL after a moe_pipeline that gave up) */
  MOE_ITEM_COUNTS = 1,         /* [nb*E]     rows per (band, expert)                           */
  MOE_ITEM_EXPERT_OFFSETS = 2, /* [nb*(E+1)] first receive row of each expert, per band         */
  MOE_ITEM_RANK_OFFSETS = 3,   /* [nb*(R+1)] first receive row of each rank, per band           */
  MOE_ITEM_SLOT_OF = 4,        /* [T*k]   receive row of token slot (t, j), -1 if dropped       */
  MOE_ITEM_ROW_SRC = 5,        /* [T*k]   source token of each receive row                     */
  MOE_ITEM_NUM_STAGED = 6,     /* 1 value: D, staging rows used (dedup only)                    */
  MOE_ITEM_STAGE_OFFSETS = 7,  /* [R+1]   first staging row of each forwarder (dedup only)      */
  MOE_ITEM_STAGE_OF = 8,       /* [T*k]   staging row feeding token slot (t, j) (dedup only)    */
  MOE_ITEM_STAGE_SRC = 9,      /* [Dmax]  source token of each staging row; first D valid       */
  MOE_ITEM_SEND_ROWS = 10,     /* [R*R]   rows rank s sends to rank d (modelled link traffic)   */
  MOE_ITEM_SEND_COPIES = 11,   /* [R*R]   distinct tokens rank s sends to rank d                */
  MOE_ITEM_NODE_COPIES = 12,   /* [R*N]   distinct tokens rank s sends to node n                */
  MOE_ITEM_FORWARDERS = 13     /* [R*N]   forwarder rank of (owner s, node n) (dedup only)      */
} moe_item;

typedef enum moe_out_dtype { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_out_dtype;

/* Ceil/floor contiguous expert partition on the host: writes lo[0..R] with
 * rank d holding experts [lo[d], lo[d+1]).  The device uses the same rule.
 * lo_out: host array of R+1 int32, owned by the caller.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null, E <= 0, R <= 0),
 *         MOE_ERR_EXPERTS_LT_RANKS (E < R). */
moe_status moe_expert_partition(int32_t num_experts, int32_t num_ranks, int32_t* lo_out);

/* Validates cfg and creates a plan.  Host only: makes no HIP call.
 * Errors: INVALID_ARGUMENT, EXPERTS_LT_RANKS, UNSUPPORTED; *out untouched then. */
moe_status moe_plan_create(const moe_config* cfg, moe_plan** out);
void moe_plan_destroy(moe_plan* plan); /* NULL is a no-op */

/* Device workspace the caller must provide to moe_route_plan (bytes, a
 * multiple of 256; the buffer itself must be 256-byte aligned). */
size_t moe_plan_workspace_bytes(const moe_plan* plan);
int64_t moe_plan_recv_rows(const moe_plan* plan);         /* T*k                          */
int64_t moe_plan_staging_rows_max(const moe_plan* plan);  /* T*min(k, N) with dedup, else 0 */
int64_t moe_plan_bands(const moe_plan* plan);             /* nb (1 without bands)          */
/* Tokens per chunk of the calls that run over chunks of consecutive tokens
 * with MOE_FLAG_NODE_DEDUP: the batch's tokens [c*n, min((c+1)*n, T)) form
 * chunk c.  call 0: moe_dispatch, 1: moe_dispatch_fp8, 2: moe_combine_hier.
 * T without dedup or for any other call. */
int64_t moe_plan_chunk_tokens(const moe_plan* plan, int32_t call);

/* Route plan: validates routing, builds the per-expert histogram, its
 * exclusive scan and the segment descriptors (and, with dedup, the per-
 * forwarder staging descriptors).  topk_idx: device [T, k] int32.
 * workspace: device, moe_plan_workspace_bytes(plan) bytes, contents need
 * no initialisation.  Asynchronous.  The slot arrays (slot_of, row_src and
 * the staging ones) are finished by the next moe_dispatch, or by the next
 * moe_combine / moe_plan_read if no dispatch comes first.
 * Errors: INVALID_ARGUMENT, HIP. */
moe_status moe_route_plan(moe_plan* plan, const int32_t* topk_idx, void* workspace, void* stream);

/* Route plan without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The same route plan as moe_route_plan, with the
 * workspace taken from a buffer the library holds on each GPU instead of a
 * caller buffer: a static device array of MOE_STATIC_WORKSPACE_BYTES, present
 * on every GPU the library runs on until the process ends.  Nothing is
 * allocated.  The plan stays bound to that buffer (as to a caller workspace)
 * until its next route, and the moe_dispatch / moe_combine / moe_plan_read
 * calls that follow use it.  Every plan routed this way on one GPU shares
 * that GPU's buffer, which keeps the last route's contents: a later
 * moe_route_plan_static on the same GPU replaces the descriptors of the plan
 * routed before it, so calls of two such plans that overlap in time race
 * (route each plan again, on the same stream, before using it).  The buffer
 * needs no initialisation.  Not for moe_pipeline.
 * Errors: INVALID_ARGUMENT, STATIC_WORKSPACE (moe_plan_workspace_bytes(plan) >
 * MOE_STATIC_WORKSPACE_BYTES; checked before any HIP call), HIP. */
#define MOE_STATIC_WORKSPACE_BYTES (32u << 20)
moe_status moe_route_plan_static(moe_plan* plan, const int32_t* topk_idx, void* stream);

/* Dispatch: recv[slot_of[t, j]] = x[t] for every valid slot.  x: device
 * [T, H] bf16; recv: device [T*k, H] bf16.  staging: device
 * [staging_rows_max, H] bf16 when the plan has MOE_FLAG_NODE_DEDUP, else
 * ignored (may be NULL); with it, the two hops run over chunks of
 * consecutive tokens (moe_plan_chunk_tokens), hop 1 of a chunk
 * before its hop 2, which shares a launch with hop 1 of the next chunk.
 * Asynchronous.
 * Errors: PLAN_NOT_ROUTED, INVALID_ARGUMENT, HIP. */
moe_status moe_dispatch(moe_plan* plan, const uint16_t* x, uint16_t* recv, uint16_t* staging,
                        void* stream);

/* Combine: out[t] = sum_{j=0..k-1} topk_w[t, j] * y[slot_of[t, j]], each term
 * a float32 fused multiply-add in ascending j starting from 0, then rounded
 * to bf16 (nearest even) or stored as float32.  y: device [T*k, H] bf16 in
 * the receive layout; topk_w: device [T, k] float32; out: device [T, H] of
 * out_dtype.  Asynchronous.  Errors: PLAN_NOT_ROUTED, INVALID_ARGUMENT, HIP. */
moe_status moe_combine(moe_plan* plan, const uint16_t* y, const float* topk_w, void* out,
                       int32_t out_dtype, void* stream);

/* Hierarchical combine for plans with MOE_FLAG_NODE_DEDUP: the return path
 * of the forwarding GPU (FUSCO article, "load balancing and cross-node
 * deduplication") with the reduction done where the data meets (INC-MoE
 * abstract, ReduceScatter combine).  Hop 1, at the forwarder: one float32
 * partial per staging row (token t, node n), the fused multiply-add chain of
 * topk_w[t, j] * y[slot_of[t, j]] over t's slots on n in ascending j; hop 2,
 * at the owner: out[t] = sum of t's partials in ascending node order, then
 * bf16 (nearest even) or float32.  partials: device [staging_rows_max, H]
 * float32 scratch owned by the caller (first D rows written).  Runs over
 * chunks of consecutive tokens, both hops of a chunk before the next (two
 * launches a chunk); asynchronous.  Errors: PLAN_NOT_ROUTED,
 * INVALID_ARGUMENT (not a dedup plan, bad pointers), HIP. */
moe_status moe_combine_hier(moe_plan* plan, const uint16_t* y, const float* topk_w,
                            float* partials, void* out, int32_t out_dtype, void* stream);

/* ---- fp8 payload ----------------------------------------------------------
 * Low-precision payload for dispatch and combine (TensorRT-LLM PR #13888,
 * opt-in gate commit message: an fp8 low-precision combine is among the
 * checked cases; the pages fix no format, so this is a reading).  Codes are
 * OCP E4M3 (bias 7, largest finite 448, no infinities).  Every row is cut
 * into blocks of 128 elements (the last may be shorter); each block carries
 * one float32 scale 2^e, the smallest power of two with amax(|block|) <=
 * 448 * 2^e (1 for an all-zero block, and for a block holding an infinity or
 * a NaN, whose codes are then unspecified), and code = E4M3(value / 2^e)
 * rounded to nearest even.
 * Layouts: codes [rows, H] uint8 (16-byte aligned), scales [rows, nb] float32
 * with nb = moe_plan_scale_blocks(plan) = ceil(H / 128). */
int64_t moe_plan_scale_blocks(const moe_plan* plan);

/* fp8 dispatch: each token row of x (bf16 [T, H]) is quantized once and its
 * codes and block scales are written to its receive rows: recv8 [T*k, H]
 * uint8, recv_scale [T*k, nb] float32.  With MOE_FLAG_NODE_DEDUP the codes
 * and scales go first to one staging row per (token, node) -- staging8
 * [staging_rows_max, H] uint8 and staging_scale [staging_rows_max, nb]
 * float32, caller-owned, first D rows written -- and are then fanned out
 * inside the node (the same hops as moe_dispatch); without it staging8 and
 * staging_scale are ignored (may be NULL).  The receive rows are the same
 * either way.  Asynchronous.  Errors: PLAN_NOT_ROUTED, INVALID_ARGUMENT, HIP. */
moe_status moe_dispatch_fp8(moe_plan* plan, const uint16_t* x, uint8_t* recv8, float* recv_scale,
                            uint8_t* staging8, float* staging_scale, void* stream);

/* fp8 combine: out[t] = sum_j topk_w[t, j] * decode(y8, y_scale)[slot_of[t, j]]
 * with the decode exact (code value times its block scale) and the same
 * float32 fused multiply-add chain and output rounding as moe_combine.
 * y8 [T*k, H] uint8 and y_scale [T*k, nb] float32 in the receive layout.
 * Asynchronous.  Errors: PLAN_NOT_ROUTED, INVALID_ARGUMENT, HIP. */
moe_status moe_combine_fp8(moe_plan* plan, const uint8_t* y8, const float* y_scale,
                           const float* topk_w, void* out, int32_t out_dtype, void* stream);

/* Banded pipeline: route plan, dispatch and combine of every band in ONE
 * persistent launch, with the identity as the expert (y = recv).  INC-MoE
 * abstract: bands pass a dispatch -> expert -> combine pipeline inside a
 * single persistent kernel, role-specialised thread blocks working on
 * different bands at once and handing them on with device-side
 * synchronisation.  Per band, in order: count (its plan tiles), scan (its
 * segment descriptors), gather (recv rows, as moe_dispatch), combine (out,
 * as moe_combine over recv).  Results equal moe_route_plan + moe_dispatch +
 * moe_combine(y = recv) on the same plan, bit for bit.
 * Arguments as for those calls; the routing and the workspace are bound to
 * the plan as by moe_route_plan, and the plan is routed afterwards.  Needs
 * H % 64 == 0 (rows of whole 128-byte lines) and recv 128-byte aligned, so
 * that no cache line holds bytes of two bands.  The workspace also holds the
 * pipeline's counters, which every moe_pipeline zeroes before its launch (one
 * small extra kernel on the stream), so the workspace's contents need no
 * initialisation here either.  Every wait inside the
 * launch is bounded; a wait that gives up makes moe_plan_read(STATUS) report
 * MOE_ERR_PIPELINE_STALL (the outputs are then unspecified).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (MOE_FLAG_NODE_DEDUP, H % 64 != 0), HIP. */
moe_status moe_pipeline(moe_plan* plan, const int32_t* topk_idx, void* workspace,
                        const uint16_t* x, uint16_t* recv, const float* topk_w, void* out,
                        int32_t out_dtype, void* stream);

/* ---- per-launch kernel timing ---------------------------------------------
 * For measuring the library's kernels where they run, in the caller's own
 * sequence of calls.  The kernels, as moe_plan_timing_read names them (each
 * id's name is the kernel's symbol, as profilers list it): */
typedef enum moe_kernel {
  MOE_KERNEL_ROUTE_COUNT = 0,     /* histogram, in-tile ranks (moe_route_plan)               */
  MOE_KERNEL_ROUTE_SCAN = 1,      /* exclusive scan -> segment descriptors                   */
  MOE_KERNEL_ROUTE_ASSIGN = 2,    /* slot arrays for a combine / read without a dispatch      */
  MOE_KERNEL_TRAFFIC_CLEAR = 3,   /* zeroes the link-traffic matrices (moe_plan_read)        */
  MOE_KERNEL_TRAFFIC = 4,         /* link-traffic matrices (moe_plan_read)                   */
  MOE_KERNEL_GATHER = 5,          /* single-hop dispatch                                     */
  MOE_KERNEL_GATHER_SCAN = 6,     /* single-hop dispatch with the scan folded in (small plans) */
  MOE_KERNEL_STAGE_A = 7,         /* deduplicated dispatch, hop 1 (one launch per chunk)      */
  MOE_KERNEL_STAGE_B = 8,         /* deduplicated dispatch, hop 2 (one launch per chunk)      */
  MOE_KERNEL_COMBINE = 9,         /* moe_combine                                             */
  MOE_KERNEL_COMBINE_PART = 10,   /* moe_combine_hier, hop 1                                 */
  MOE_KERNEL_COMBINE_NODES = 11,  /* moe_combine_hier, hop 2                                 */
  MOE_KERNEL_GATHER_FP8 = 12,     /* moe_dispatch_fp8, single hop                            */
  MOE_KERNEL_GATHER_FP8_SCAN = 13,/* ... with the scan folded in                             */
  MOE_KERNEL_STAGE_A_FP8 = 14,    /* moe_dispatch_fp8 with dedup, hop 1                      */
  MOE_KERNEL_STAGE_B_FP8 = 15,    /* moe_dispatch_fp8 with dedup, hop 2                      */
  MOE_KERNEL_COMBINE_FP8 = 16,    /* moe_combine_fp8                                         */
  MOE_KERNEL_PIPELINE = 17,       /* moe_pipeline                                            */
  MOE_KERNEL_COUNTERS_CLEAR = 18, /* moe_pipeline: zeroes the pipeline's counters            */
  MOE_KERNEL_STAGE_AB = 19,       /* deduplicated dispatch: hop 2 of chunk c with hop 1 of
                                     chunk c + 1 in one launch (one per chunk boundary)       */
  MOE_KERNEL_STAGE_AB_FP8 = 20,   /* the same for moe_dispatch_fp8                          */
  MOE_KERNEL_COMBINE_PN = 21,     /* moe_combine_hier: hop 2 of chunk c with hop 1 of c + 1  */
  MOE_KERNEL_COUNT = 22
} moe_kernel;

/* Symbol name of a moe_kernel id (static text; "?" outside the enum). */
const char* moe_kernel_name(int32_t kernel);

/* Starts (capacity > 0) or stops (capacity = 0) per-launch timing of the
 * kernels that calls on this plan launch.  capacity > 0 creates `capacity`
 * pairs of HIP events on the current device (the plan's earlier pairs are
 * destroyed) and clears the record; from then on each kernel launched by a
 * call on this plan, up to `capacity` launches, is launched with
 * hipExtLaunchKernel and a pair bound to the kernel's own start and end, so a
 * pair's elapsed time is that kernel's execution on the GPU, with no launch
 * gap in it.  Launches beyond `capacity` run untimed.  capacity = 0 destroys
 * the events.  The plan owns the events.  Host call; no kernel is launched.
 * Errors: INVALID_ARGUMENT (null plan, capacity < 0), HIP. */
moe_status moe_plan_timing(moe_plan* plan, int32_t capacity);

/* Waits for the timed launches recorded since moe_plan_timing or the last
 * read (each pair's end event) and writes, for the first min(*count, cap) of
 * them in launch order, to the caller's host arrays of cap entries:
 * kernel_ids (moe_kernel), start_ms (milliseconds from the first recorded
 * launch's start to this launch's start; launches on other streams may start
 * earlier, giving a negative offset) and ms (the launch's own duration).
 * Sets *count to the number recorded and clears the record (the event pairs
 * are reused).  Errors: INVALID_ARGUMENT (null arguments, timing not
 * started), HIP. */
moe_status moe_plan_timing_read(moe_plan* plan, int32_t* kernel_ids, float* start_ms, float* ms,
                                int32_t cap, int32_t* count);

/* Copies one plan item to host memory (synchronises the stream).  bytes must
 * be at least the item's size (see moe_item).  The traffic matrices
 * (SEND_ROWS, SEND_COPIES, NODE_COPIES) are computed on demand by a small
 * kernel from the workspace.  Errors: PLAN_NOT_ROUTED, INVALID_ARGUMENT, HIP. */
moe_status moe_plan_read(moe_plan* plan, int32_t item, void* host_dst, size_t bytes,
                         void* stream);

/* Static text for a status code. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SHUFFLE_H */
