/*
 * swr.h -- sharded weight reassembly on one MI355X (gfx950): C ABI.
 *
 * The method (weight_sharding, zdszero.github.io): every layer keeps its
 * replicated weights as N byte chunks of one flat buffer T; just before the
 * layer runs, the chunks are gathered back into a full-weight workspace slot
 * and the layer's GEMMs read the weights through zero-copy views of that slot.
 * Here the N chunks all live in one GPU's HBM and the gather is an on-device
 * copy kernel on a side stream.
 *
 * Conventions shared by every entry point
 *   - Weights are out_features x in_features, row-major, K (= in) contiguous
 *     (weight_sharding, section "core abstraction").
 *   - dtype SWR_BF16: 2-byte bfloat16 elements.  SWR_FP8_E4M3FN: 1-byte OCP
 *     E4M3FN codes whose value is decode(code) * row_scale[row]; the fp32
 *     row scales are replicated and live outside the flat buffer
 *     (weight_sharding, section "loading", quantised variants).
 *   - Activations X are bfloat16, row-major [M, in] with a leading dimension.
 *   - "Device pointer" arguments are HIP device addresses of the current
 *     device; pointer *arrays* (chunk lists, source lists, partial lists) are
 *     host arrays of device pointers, read during the call only.
 *   - The caller owns every buffer.  The library borrows device buffers until
 *     the work it enqueued on the given stream has finished, and never
 *     allocates device memory in any entry point below.
 *   - Every call checks all of its arguments before it enqueues anything:
 *     on error nothing has been enqueued, the call returns a negative status
 *     and swr_last_error() describes the problem.  No call falls back to a
 *     different algorithm or to the host.
 *   - Streams: any hipStream_t of the current device, or 0 for the null
 *     stream.  Kernels are enqueued asynchronously.
 */
#ifndef SWR_H
#define SWR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ types */

enum swr_dtype { SWR_BF16 = 0, SWR_FP8_E4M3FN = 1 };

enum swr_status {
  SWR_OK = 0,
  SWR_E_INVALID = -1,  /* bad argument value, null pointer, unknown dtype   */
  SWR_E_ALIGN = -2,    /* a pointer or size is not 16-byte aligned          */
  SWR_E_CAPACITY = -3, /* a destination or workspace is too small           */
  SWR_E_SHAPE = -4,    /* inconsistent or unsupported shapes                */
  SWR_E_HIP = -5,      /* the HIP runtime reported an error                 */
  SWR_E_SEQUENCE = -6  /* planner calls out of the documented order         */
};

#define SWR_MAX_CHUNKS 64   /* N, chunks per layer                           */
#define SWR_MAX_WEIGHTS 64  /* weights per layer                             */
#define SWR_MAX_GROUP 16    /* projections per swr_proj_forward_grouped call */
#define SWR_MAX_SUB 4       /* sub-blocks of a merged weight (row shards)    */
#define SWR_ITEM_ALIGN 16   /* every item starts on a 16-byte boundary       */

typedef struct swr_weight_desc {
  int64_t out_features;
  int64_t in_features;
  int32_t dtype;    /* enum swr_dtype */
  int32_t reserved; /* must be 0 */
} swr_weight_desc;

typedef struct swr_view_desc {
  int64_t offset;       /* o_j: byte offset of the item in T (multiple of 16) */
  int64_t nbytes;       /* s_j = out * in * element size                      */
  int64_t out_features;
  int64_t in_features;
  int32_t dtype;
  int32_t reserved;
} swr_view_desc;

typedef struct swr_layout {
  int64_t payload_bytes; /* end of the last item                           */
  int64_t total_bytes;   /* |T|: payload rounded up to a multiple of 16*N  */
  int64_t chunk_bytes;   /* C = |T| / N, a multiple of 16                  */
  int32_t n_weights;
  int32_t n_chunks;      /* N */
} swr_layout;

/* ------------------------------------------------------- flat layout (a1) */

/*
 * swr_plan_layer -- host only, no device work.
 * weight_sharding, section "one AllGather per layer: flat layout", steps 1-2:
 * the layer's weights are laid end to end in the given order; each item
 * starts at the first 16-byte boundary at or after the previous item's end
 * (offsets relative to the start of T); |T| is the payload rounded up to a
 * multiple of 16*N; C = |T| / N.  Bytes between items and after the payload
 * are padding.
 *   w[n_weights]         weights in packing order (1 <= n_weights <= 64,
 *                        out, in >= 1, dtype BF16 or FP8_E4M3FN, reserved 0)
 *   n_chunks             N, 1 <= N <= 64
 *   views_out[n_weights] receives (o_j, s_j, out_j, in_j, dtype_j)
 *   layout_out           receives payload, |T|, C, n_weights, N
 * Errors: SWR_E_INVALID for null pointers or out-of-range counts/dtypes,
 *         SWR_E_SHAPE for non-positive sizes or sizes that overflow int64.
 */
int swr_plan_layer(const swr_weight_desc* w, int32_t n_weights, int32_t n_chunks,
                   swr_view_desc* views_out, swr_layout* layout_out);

/* ------------------------------------------------------------- pack (a2) */

/*
 * swr_pack_layer -- enqueue on `stream`.
 * weight_sharding, section "flat layout", steps 1-2, and section "loading"
 * (the one-time re-layout into flat chunks): writes every byte of
 * T = [W_0 | pad | W_1 | pad | ... | pad] into the N chunk buffers, chunk i
 * receiving T[i*C, (i+1)*C).  Padding bytes are written as zero.
 *   layout, views     as returned by swr_plan_layer (views[layout->n_weights])
 *   src_dev[n]        device pointers to the full weights, row-major, each
 *                     16-byte aligned and s_j bytes long
 *   chunk_dev[N]      device pointers, each 16-byte aligned, >= C bytes
 * Errors: SWR_E_INVALID (null/inconsistent layout), SWR_E_ALIGN, SWR_E_HIP.
 */
int swr_pack_layer(const swr_layout* layout, const swr_view_desc* views,
                   const void* const* src_dev, void* const* chunk_dev, hipStream_t stream);

/* The row shards of one weight, as a tensor-parallel loader leaves them on
 * the N ranks (weight_sharding, loading section).  A merged weight (gate_up
 * = [gate rows; up rows]) is split per sub-block: rank r holds, for each
 * sub-block b in order, the rows [r*R_b/N, (r+1)*R_b/N) of that sub-block,
 * contiguous.  A weight whose rows do not divide by N stays whole. */
typedef struct {
  int32_t n_sub;                  /* sub-blocks, 1..SWR_MAX_SUB (ignored when replicated)   */
  int32_t replicated;             /* nonzero: not row-sharded; src[0] holds the whole weight */
  int64_t sub_rows[SWR_MAX_SUB];  /* rows of each sub-block; each a multiple of N, sum = out */
  const void* src[SWR_MAX_CHUNKS];/* device, 16-byte aligned: rank r's shard (r < N)          */
} swr_row_shards;

/*
 * swr_redistribute_row_shards -- enqueue on `stream`.
 * The one-time re-layout of weight_sharding's loading section: from each
 * weight's row shards, write the N flat chunks, byte for byte what
 * swr_pack_layer writes from the whole weights (padding zero).  Chunk i
 * takes its bytes from whichever rank shards hold the rows its byte window
 * covers, so a chunk may straddle weights and shards.
 *   layout, views  from swr_plan_layer (host memory)
 *   shards         host array of layout->n_weights descriptors, read before
 *                  the call returns
 *   chunk_dev      N device buffers of >= chunk_bytes, 16-byte aligned
 * One launch per weight.  Every argument is checked before the first launch.
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_SHAPE (rows not a multiple of N
 * for a sharded weight, sub-blocks not adding up), SWR_E_HIP.
 */
int swr_redistribute_row_shards(const swr_layout* layout, const swr_view_desc* views,
                                const swr_row_shards* shards, void* const* chunk_dev,
                                hipStream_t stream);

/* ------------------------------------------------------- reassembly (a3) */

/*
 * swr_reassemble_into_slot -- enqueue on `side`.
 * weight_sharding, section "flat layout" step 3 (one gather per layer gives
 * every rank the whole T) and section "lookahead and ping-pong slot" (the
 * gather waits on a gate event, its completion is an event the consumer
 * waits on).  On one GPU the gather is the copy
 *     slot[i*C, (i+1)*C) = chunk_dev[i]   for i = 0..N-1.
 *   chunk_dev[N]   device pointers, 16-byte aligned, C bytes each (N <= 64)
 *   chunk_bytes    C, a positive multiple of 16
 *   slot           device pointer, 16-byte aligned, slot_bytes >= N*C
 *   self_rank      the rank whose chunk is local (0 <= self_rank < N); it only
 *                  changes the transfer count below
 *   gate           if non-null, `side` waits for it before the copy
 *   ready          if non-null, recorded on `side` after the copy
 *   remote_bytes   if non-null, *remote_bytes += (N-1)*C, the bytes a rank
 *                  receives from its peers (weight_sharding, cost section)
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_CAPACITY (slot too small),
 *         SWR_E_HIP.
 */
int swr_reassemble_into_slot(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes,
                             void* slot, int64_t slot_bytes, int32_t self_rank, hipStream_t side,
                             hipEvent_t gate, hipEvent_t ready, int64_t* remote_bytes);

/*
 * swr_reassemble_into_slot_dma -- the same gather, arguments, checks and
 * events as swr_reassemble_into_slot, but the bytes move on the GPU's DMA
 * engines (one device-to-device copy per chunk, hipMemcpyDeviceToDeviceNoCU)
 * instead of a copy kernel.  weight_sharding, section on the NCCL policy /
 * copy engine: a copy-engine gather leaves every compute unit to the layer's
 * GEMMs.  On MI355X the DMA engines move far fewer bytes per second than the
 * copy kernel; the trade is measured, not assumed.
 * Errors: as swr_reassemble_into_slot.
 */
int swr_reassemble_into_slot_dma(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes,
                                 void* slot, int64_t slot_bytes, int32_t self_rank, hipStream_t side,
                                 hipEvent_t gate, hipEvent_t ready, int64_t* remote_bytes);

/* ------------------------------------------------------------ GEMMs (a5-a8) */

/*
 * swr_proj_forward -- enqueue on `stream`.
 * One projection through a view (weight_sharding, section "flat layout"
 * step 4: the GEMM sees the full W):
 *     Y[m, o] = s[o] * sum_k X[m, k] * W[o, k]
 * accumulated in fp32; the result is rounded once to bf16 (round to nearest
 * even) unless y_fp32 is set.
 *   W          device pointer, 16-byte aligned, [out_f, in_f] of `dtype`
 *   row_scale  device pointer to fp32 [out_f], 16-byte aligned; NULL means
 *              s = 1 (must be non-NULL for FP8 weights)
 *   X          device pointer, bf16 [M, ldx] (the first in_f columns of each
 *              row are read), 16-byte aligned, ldx >= in_f
 *   Y          device pointer, bf16 or fp32 [M, ldy], 16-byte aligned,
 *              ldy >= out_f; the first out_f columns of each row are written
 *   workspace  NULL, or a 256-byte aligned device buffer of workspace_bytes
 *              used for split-K partial sums; with NULL every row tile is
 *              reduced over the whole K by one workgroup.  A non-NULL
 *              workspace smaller than swr_proj_workspace_bytes() is an error.
 *   Shapes: any out_f, in_f >= 1 and M >= 0 (M == 0 enqueues nothing).  The
 *   matrix-core streaming kernel runs when in_f and ldx are multiples of 64
 *   and 8; other shapes (odd projections) run a plain one-output-per-thread
 *   kernel.
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_SHAPE, SWR_E_CAPACITY, SWR_E_HIP.
 */
int swr_proj_forward(const void* W, int32_t dtype, const float* row_scale, int64_t out_f,
                     int64_t in_f, const void* X, int64_t ldx, int64_t M, void* Y, int32_t y_fp32,
                     int64_t ldy, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Split-K scratch bytes swr_proj_forward can use for these sizes (0 when it
 * does not split K), or a negative status.  Host only. */
int64_t swr_proj_workspace_bytes(int64_t M, int64_t out_f, int64_t in_f, int32_t dtype);

/* One projection of a grouped call: a view of a reassembled slot with its own
 * activations and output.  Fields as the arguments of swr_proj_forward. */
typedef struct {
  const void* W;          /* device, [out_features, in_features] of dtype, 16-byte aligned */
  const float* row_scale; /* device fp32 [out_features] or NULL (s = 1; not for FP8)       */
  const void* X;          /* device bf16 [M, ldx], 16-byte aligned                          */
  void* Y;                /* device bf16 or fp32 [M, ldy], 16-byte aligned                  */
  int64_t out_features, in_features, ldx, ldy;
  int32_t dtype, y_fp32;
} swr_proj_desc;

/*
 * swr_proj_forward_grouped -- enqueue on `stream`.
 * The projections of one layer, all read through views of the same
 * reassembled slot (weight_sharding, section "flat layout" step 4, and the
 * section on targets: one gather per layer serves every projection in it).
 * Each descriptor computes exactly what swr_proj_forward computes for it.
 * When every projection has the same dtype and can use the staged
 * matrix-core kernel (M <= 64, K a multiple of 256, weights under 2 GiB,
 * aligned) or the tiled one (M > 64, K a multiple of 64, weights and X under
 * 2 GiB, aligned) they run as ONE launch over all their tiles, which removes
 * the per-launch ramp and tail that dominate small views and small shards;
 * otherwise they are enqueued one after another.
 *   descs      host array of n descriptors, 1 <= n <= SWR_MAX_GROUP; read
 *              before the call returns
 *   M          tokens, shared by all projections (M == 0 enqueues nothing)
 *   workspace  as for swr_proj_forward, of at least
 *              swr_proj_grouped_workspace_bytes(descs, n, M) bytes (0 when the
 *              projections run as one launch)
 * All descriptors are validated before anything is enqueued.
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_SHAPE, SWR_E_CAPACITY, SWR_E_HIP.
 */
int swr_proj_forward_grouped(const swr_proj_desc* descs, int32_t n, int64_t M, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);

/* Scratch bytes swr_proj_forward_grouped needs for these descriptors (0 when
 * they run as one launch), or a negative status.  Host only. */
int64_t swr_proj_grouped_workspace_bytes(const swr_proj_desc* descs, int32_t n, int64_t M);

/*
 * swr_mlp_forward -- enqueue on `stream`.
 * The shared-expert MLP (vLLM PR #50656 report, test code: gate_up holds the
 * gate rows then the up rows; the activation is SiLU of the gate half times
 * the up half):
 *     G = X @ W_gate_up^T * s_gu        fp32, [M, 2I]
 *     h = bf16( silu(G[:, :I]) * G[:, I:] ),  silu(z) = z / (1 + exp(-z))
 *     Y = bf16( (h @ W_down^T) * s_d )
 *   W_gate_up  [2I, H] of dtype, W_down [H, I] of dtype, 16-byte aligned
 *   s_gu, s_d  fp32 [2I] and [H] row scales (NULL means 1; required for FP8)
 *   X          bf16 [M, H] contiguous; Y bf16 [M, H] contiguous; both 16-byte
 *              aligned
 *   workspace  device buffer of at least swr_mlp_workspace_bytes(M, H, I,
 *              dtype) bytes, 256-byte aligned; it holds h and any split-K
 *              partial sums and is overwritten
 *   H, I       >= 1; the fused matrix-core path needs H, I multiples of 64
 *              (and I of 32), other sizes run the plain kernel
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_SHAPE, SWR_E_CAPACITY, SWR_E_HIP.
 */
int swr_mlp_forward(const void* W_gate_up, const float* s_gu, const void* W_down,
                    const float* s_d, int32_t dtype, int64_t H, int64_t I, const void* X,
                    int64_t M, void* Y, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream);

/*
 * swr_mlp_forward_partial -- enqueue on `stream`.
 * One tensor-parallel rank's share of the shared-expert MLP (vLLM PR #50656
 * report, the TP-sharded shared expert: each rank holds a slice of the
 * intermediate dimension -- its gate rows, the matching up rows, and the
 * matching columns of down -- and the ranks' outputs are summed by an
 * all-reduce).  Computes what swr_mlp_forward computes for the slice, but Y
 * is fp32 [M, H] and not rounded, so the partials of all ranks can be added
 * (swr_sum_partials, rank order) and rounded once:
 *     Y_r = (bf16(silu(G_r[:, :I_r]) * G_r[:, I_r:]) @ W_down_r^T) * s_d
 *   W_gate_up  [2 I_r, H]: the rank's gate rows then its up rows, contiguous
 *   W_down     [H, I_r]: the rank's columns of down, contiguous
 *   s_d        the full down row scales (they multiply every partial)
 *   Y          fp32 [M, H] contiguous, 16-byte aligned
 *   workspace  as for swr_mlp_forward with I = I_r
 * Errors: as swr_mlp_forward.
 */
int swr_mlp_forward_partial(const void* W_gate_up, const float* s_gu, const void* W_down,
                            const float* s_d, int32_t dtype, int64_t H, int64_t I, const void* X,
                            int64_t M, float* Y, void* workspace, int64_t workspace_bytes,
                            hipStream_t stream);

/* Workspace bytes swr_mlp_forward needs for these sizes (>= 0), or a negative
 * status for invalid sizes.  Host only. */
int64_t swr_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, int32_t dtype);

/* Bytes of the fixed device scratch of swr_mlp_forward_noalloc (16 MiB). */
#define SWR_NOALLOC_SCRATCH_BYTES (INT64_C(16) << 20)

/*
 * swr_mlp_forward_noalloc -- enqueue on `stream`.
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): computes exactly
 * what swr_mlp_forward computes, with the same kernels and the same bits,
 * but takes no workspace.  Its scratch (h and any split-K partial sums) is a
 * fixed array of SWR_NOALLOC_SCRATCH_BYTES in the library's device memory,
 * one per GPU, held until the process ends; the call itself allocates
 * nothing.  The first call on a device (with that device current) looks up
 * the array's address there.
 *   Arguments as swr_mlp_forward without workspace / workspace_bytes.
 *   Limit: swr_mlp_workspace_bytes(M, H, I, dtype) must not exceed
 *   SWR_NOALLOC_SCRATCH_BYTES (the shared-expert MLP, H = 6144, I = 14336,
 *   needs about 8 MB at 64 tokens); larger calls fail with SWR_E_CAPACITY
 *   before any HIP call.
 *   Concurrency: every call on one GPU uses that GPU's single array, which
 *   keeps the last call's contents; calls whose work overlaps on one GPU (two
 *   streams, two threads) race on it and must be ordered by the caller.
 * Errors: as swr_mlp_forward, plus SWR_E_CAPACITY for sizes beyond the
 * scratch.
 */
int swr_mlp_forward_noalloc(const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d,
                            int32_t dtype, int64_t H, int64_t I, const void* X, int64_t M, void* Y,
                            hipStream_t stream);

/*
 * FP8 activations (an option beyond the pages, which keep activations in
 * BF16; the weight_sharding page's FP8 variant quantises the weights only).
 *
 * swr_quantize_rows_e4m3 -- per-token quantisation of BF16 rows:
 *   S[m] = max_k |X[m, k]| / 448 in binary32 (1 for an all-zero row),
 *   Q[m, k] = the E4M3FN value nearest to the binary32 quotient X[m, k] / S[m],
 *   ties to the even code, magnitudes above 448 saturating to 448.
 * X: M x K BF16, row stride ldx elements (X 16-byte aligned, ldx % 8 == 0);
 * Q: M x K E4M3FN codes, row stride ldq bytes (Q 8-byte aligned, ldq % 8 ==
 * 0); S: M floats.  Finite inputs.  Enqueued on `stream`; caller-owned memory.
 * Errors: SWR_E_INVALID (null pointer), SWR_E_SHAPE (M < 0, K < 1, ld < K),
 * SWR_E_ALIGN, SWR_E_HIP.
 */
int swr_quantize_rows_e4m3(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q, int64_t ldq, float* S,
                           hipStream_t stream);

/*
 * swr_mlp_forward_fp8act -- the shared-expert MLP with FP8 weights and FP8
 * activations on the FP8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4):
 *   (q_x, s_x) = quantize(X);  G = (q_x @ W_gate_up^T) * s_x[m] * s_gu[o];
 *   h = bf16(silu(G[:, :I]) * G[:, I:]);  (q_h, s_h) = quantize(h);
 *   Y = bf16((q_h @ W_down^T) * s_h[m] * s_d[o]),
 * fp32 accumulation, quantize as in swr_quantize_rows_e4m3.  Weights and
 * layouts as swr_mlp_forward with dtype SWR_FP8_E4M3FN; H and I multiples of
 * 64; s_gu and s_d required.  The workspace (swr_mlp_fp8act_workspace_bytes,
 * 256-byte aligned) holds the codes and scales of X and h, and h.  Every M is
 * accepted; the tiled kernels suit prefill-sized M.
 * Errors: SWR_E_INVALID (null pointer), SWR_E_SHAPE (sizes, weights of 2 GiB
 * or more), SWR_E_ALIGN, SWR_E_CAPACITY (workspace), SWR_E_HIP.
 */
int swr_mlp_forward_fp8act(const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d, int64_t H,
                           int64_t I, const void* X, int64_t M, void* Y, void* workspace, int64_t workspace_bytes,
                           hipStream_t stream);
int64_t swr_mlp_fp8act_workspace_bytes(int64_t M, int64_t H, int64_t I);


/*
 * swr_sum_partials -- enqueue on `stream`.
 * Sharded-matrices notes (copecc.github.io), local matmul case 3: when the
 * contraction dimension is split, each shard yields a partial result and
 * the full result is their sum:
 *     out[i] = parts[0][i] + parts[1][i] + ... + parts[n-1][i]
 * added in fp32 in that fixed order, stored as fp32 or rounded to bf16.
 *   parts[n]   device pointers to fp32 arrays of `count` elements, 16-byte
 *              aligned (1 <= n <= 64)
 *   out        device pointer, fp32 or bf16 [count], 16-byte aligned
 * Errors: SWR_E_INVALID, SWR_E_ALIGN, SWR_E_HIP.
 */
int swr_sum_partials(const float* const* parts, int32_t n, int64_t count, void* out,
                     int32_t out_bf16, hipStream_t stream);

/* ------------------------------------------------------ scheduler (a9) */

/*
 * The lookahead / ping-pong planner (weight_sharding, sections "lookahead
 * and ping-pong slot", "implementation in SGLang" and "CUDA graph and the
 * draft model").  Per forward over layers [start, end):
 *     swr_planner_reset(p);                  records the forward-start event
 *     swr_planner_pre_dispatch(p, start);    side: gather(start) -> slot 0
 *     for l in [start, end):
 *         swr_planner_maybe_dispatch(p, l+1);  side: wait gate, gather(l+1)
 *                                              into slot (l+1-start) % 2,
 *                                              record ready(l+1); no-op if
 *                                              l+1 is outside [start, end)
 *         swr_planner_wait_ready_once(p, l, &slot);  compute waits ready(l)
 *                                              at most once per forward
 *         ... the layer's GEMMs on `compute`, reading views of *slot ...
 *         swr_planner_update_done_event(p, l);  records done(l) on compute
 * The gate of gather(l) is done(l-2), the last reader of the same slot, or
 * the forward-start event when l-2 < start.  At most two layers' full
 * weights exist at any time.  The planner owns its hipEvents; it borrows the
 * streams, slots and chunk buffers.  Calls are not thread-safe.
 */
typedef struct swr_planner swr_planner;

/* Trace op codes reported by swr_planner_trace (quadruples op, stream, layer, slot). */
enum swr_trace_op {
  SWR_OP_RECORD_START = 1, SWR_OP_WAIT_START = 2, SWR_OP_WAIT_DONE = 3, SWR_OP_COPY = 4,
  SWR_OP_RECORD_READY = 5, SWR_OP_WAIT_READY = 6, SWR_OP_RECORD_DONE = 7,
  SWR_OP_COPY_NEXT = 8, /* cyclic mode: the next forward's first layer */
  SWR_OP_RECORD_BEGIN = 9, /* gate SWR_GATE_BEGIN: compute stream begins layer l (after its ready wait) */
  SWR_OP_WAIT_BEGIN = 10,  /* side stream waits for that record before a gather */
  SWR_OP_RECORD_FREE = 11, /* dedicated first-layer prefetch: slot 0's last reader (layer l) is done */
  SWR_OP_WAIT_FREE = 12    /* the prefetch stream waits for that record before gathering the first layer */
};
enum swr_trace_stream { SWR_STREAM_COMPUTE = 0, SWR_STREAM_SIDE = 1, SWR_STREAM_PREFETCH = 2 };

/* start < end; slot_a, slot_b device pointers (16-byte aligned, slot_bytes
 * each).  compute and side are normally two streams; they may be the same
 * stream ("one queue"): the gathers then run between the layers' GEMMs in
 * queue order, the waits between the two roles are implied by that order and
 * are not enqueued, and the trace is unchanged.  Errors: SWR_E_INVALID,
 * SWR_E_ALIGN, SWR_E_HIP (event creation). */
int swr_planner_create(int32_t start, int32_t end, hipStream_t compute, hipStream_t side,
                       void* slot_a, void* slot_b, int64_t slot_bytes, swr_planner** out);

/* Register layer `layer`'s chunks (host array of N device pointers, C bytes
 * each).  N*C must fit in slot_bytes (else SWR_E_CAPACITY). */
int swr_planner_set_layer(swr_planner* p, int32_t layer, const void* const* chunk_dev,
                          int32_t n_chunks, int64_t chunk_bytes);

int swr_planner_reset(swr_planner* p);
/* SWR_E_SEQUENCE if reset() was not called, or `layer` != start. */
int swr_planner_pre_dispatch(swr_planner* p, int32_t layer);
/* No-op (SWR_OK) outside [start, end) (except layer == end in cyclic mode);
 * SWR_E_SEQUENCE if `layer` was already dispatched in this forward or layer-1
 * was not dispatched. */
int swr_planner_maybe_dispatch(swr_planner* p, int32_t layer);
/* Makes `compute` wait for ready(layer) the first time it is called for
 * `layer` in this forward; later calls only return the slot.  *slot_out gets
 * the slot base (views are slot + o_j).  SWR_E_SEQUENCE if `layer` was not
 * dispatched. */
int swr_planner_wait_ready_once(swr_planner* p, int32_t layer, void** slot_out);
/* SWR_E_SEQUENCE if wait_ready_once(layer) was not called first. */
int swr_planner_update_done_event(swr_planner* p, int32_t layer);
/* Gate of the planner's gathers (swr_planner_set_gate). */
#define SWR_GATE_DONE 0  /* gather(l+1) waits for done(l-1), as the pages (default)     */
#define SWR_GATE_BEGIN 1 /* gather(l+1) waits for the compute stream to begin layer l */
#define SWR_GATE_AFTER 2 /* gather(l+1) waits for done(l): no overlap                  */

/*
 * swr_planner_set_gate -- which compute-stream event gates each gather.
 * weight_sharding, lookahead and ping-pong section: the gather of layer l+1
 * may overwrite its slot once layer l-1, the slot's last reader, is done.
 *   SWR_GATE_DONE   the gather waits for done(l-1) (the pages' gate).
 *   SWR_GATE_BEGIN  the gather waits for an event recorded on the compute
 *                   stream right after that stream's wait for ready(l), i.e.
 *                   when layer l begins.  That point follows done(l-1) in
 *                   stream order and the gather of layer l precedes it on the
 *                   side stream, so the dependencies are the same; the gather
 *                   is enqueued by swr_planner_wait_ready_once(l) instead of
 *                   swr_planner_maybe_dispatch(l+1) (which then only marks it
 *                   pending), and on one GPU the layer's GEMM workgroups are
 *                   resident before the copy's many short workgroups arrive.
 * The trace then shows SWR_OP_RECORD_BEGIN / SWR_OP_WAIT_BEGIN in place of
 * SWR_OP_WAIT_DONE.
 *   SWR_GATE_AFTER  the gather of l+1 waits for done(l) and is enqueued by
 *                   swr_planner_update_done_event(l) (swr_planner_maybe_dispatch
 *                   only marks it pending): the same gathers, slots and events
 *                   with no overlap.  On one GPU the gather (2|T| bytes) and the
 *                   GEMMs (|T| bytes) draw on the same HBM, and a slot that the
 *                   GEMMs read right after it was written is partly still in the
 *                   last-level cache; this is the one-GPU schedule.  The trace
 *                   shows SWR_OP_WAIT_DONE of layer l before each gather.
 * Host only.
 * Errors: SWR_E_INVALID (null planner, unknown gate), SWR_E_SEQUENCE (a
 * gather is pending).
 */
int swr_planner_set_gate(swr_planner* p, int32_t gate);

/* Gather engines of the planner (swr_planner_set_copy_engine). */
#define SWR_ENGINE_KERNEL 0 /* swr_reassemble_into_slot (default)      */
#define SWR_ENGINE_DMA 1    /* swr_reassemble_into_slot_dma            */

/*
 * swr_planner_set_copy_engine -- which gather the planner enqueues from now
 * on: SWR_ENGINE_KERNEL (the copy kernel) or SWR_ENGINE_DMA (the DMA engines,
 * weight_sharding section on the NCCL policy / copy engine).  The launch/wait
 * sequence and the trace are the same for both.  Host only.
 * Errors: SWR_E_INVALID (null planner, unknown engine).
 */
int swr_planner_set_copy_engine(swr_planner* p, int32_t engine);

#define SWR_MAX_GATHER_LDS 65536

/*
 * swr_planner_set_gather_lds -- LDS, in bytes, that each workgroup of the
 * planner's copy-kernel gathers reserves and never touches (0, the default:
 * none).  It only limits how many copy workgroups share a CU.  On one GPU the
 * gather of layer l+1 and the GEMMs of layer l share the CUs and HBM, and the
 * copy's many short workgroups otherwise crowd out the GEMMs' long-lived ones;
 * the weight_sharding page's copy-engine gather exists so that the copy does
 * not take compute units from the GEMMs (NCCL policy / copy engine section),
 * and this is the compute-unit copy's way to yield them.  A reservation R
 * leaves floor(160 KB / R) copy workgroups per idle CU and
 * floor((160 KB - G) / R) beside compute workgroups holding G bytes of LDS.
 * The copy alone keeps its bandwidth with two workgroups per CU (R up to
 * 64 KB).  The DMA engine (SWR_ENGINE_DMA) ignores it.  Host only; applies to
 * gathers enqueued from now on.
 * Errors: SWR_E_INVALID (null planner, bytes outside [0, SWR_MAX_GATHER_LDS]).
 */
int swr_planner_set_gather_lds(swr_planner* p, int32_t bytes);

/* Cyclic mode, for a model that runs the same layers forward after forward.
 * The pages move the draft model's first-layer gather out of the loop so it
 * overlaps other work (weight_sharding, "CUDA graph and the draft model");
 * here maybe_dispatch(end) gathers the NEXT forward's first layer into slot 0,
 * gated by done(end - 2), the last reader of slot 0 when the layer count is
 * even.  The next forward's pre_dispatch(start) then enqueues nothing and its
 * wait_ready_once(start) waits for that gather.  The trace shows the early
 * gather as SWR_OP_COPY_NEXT.  SWR_E_INVALID for an odd number of layers. */
int swr_planner_set_cyclic(swr_planner* p, int32_t enabled);

/*
 * swr_planner_set_first_prefetch -- gather the first layer on a dedicated
 * stream, outside the forward (weight_sharding, "CUDA graph and the draft
 * model": the draft model's layer-0 gather runs outside the captured graph on
 * its own stream, overlapping the main model's last layers, and the graph
 * waits for it).  With a non-null `stream`:
 *   - swr_planner_pre_dispatch(start) enqueues nothing; the forward's first
 *     layer is the one swr_planner_prefetch_first gathered into slot 0;
 *   - swr_planner_wait_ready_once(start) makes the compute stream wait for
 *     that gather's ready event (while the compute stream is capturing, with
 *     hipEventWaitExternal, so the graph holds the wait as a node and every
 *     replay waits again);
 *   - swr_planner_update_done_event(l0), l0 the last layer of the forward
 *     that reads slot 0 (the last l with l - start even), records a "free"
 *     event (while capturing, as an event-record node added to the graph,
 *     which every replay records).
 * Call swr_planner_prefetch_first once before the first forward and once
 * after each forward (or each replay of a captured forward), outside any
 * capture.  Refused while a forward is in progress, with the compute stream,
 * and in cyclic mode (which gathers the first layer in the previous forward
 * instead).  NULL turns the mode off.  Host only.
 * Errors: SWR_E_INVALID, SWR_E_SEQUENCE.
 */
int swr_planner_set_first_prefetch(swr_planner* p, hipStream_t stream);

/*
 * swr_planner_prefetch_first -- enqueue on the dedicated stream: wait for the
 * latest "free" event (none before the first forward), gather layer start
 * into slot 0 (copy kernel or DMA engines, as swr_planner_set_copy_engine),
 * record ready(start).  The trace lists SWR_OP_WAIT_FREE, SWR_OP_COPY_NEXT and
 * SWR_OP_RECORD_READY on SWR_STREAM_PREFETCH.  Counts as a gather in
 * swr_planner_counters.
 * Errors: SWR_E_INVALID, SWR_E_SEQUENCE (no prefetch stream, no chunks for
 * the first layer), SWR_E_HIP.
 */
int swr_planner_prefetch_first(swr_planner* p);

/* Timing of the gathers and of the layers.  swr_planner_set_timing(p, capacity)
 * with capacity > 0 makes every later dispatch record two timing events on the
 * side stream around its copy (after the gate wait, before the ready record),
 * and every later layer two on the compute stream (the begin record after its
 * ready wait, and one after its done record), each in a ring of `capacity`
 * event pairs; 0 turns timing off.  Either way the
 * launch/wait sequence is the same.  swr_planner_gather_times writes the copy
 * durations (milliseconds) of the timed dispatches still in the ring, oldest
 * first, at most `cap` of them, and sets *n to the number written; every one
 * of those copies must have finished (else SWR_E_HIP). */
int swr_planner_set_timing(swr_planner* p, int32_t capacity);
/* With paused != 0, later dispatches and layers record no timing events (a
 * layer that already recorded its begin still records its end), so that a
 * caller can time a sample of its forwards; the rings keep their contents.
 * 0 resumes.  Has no effect while timing is off.  Errors: SWR_E_INVALID. */
int swr_planner_pause_timing(swr_planner* p, int32_t paused);
int swr_planner_gather_times(const swr_planner* p, float* ms, int32_t cap, int32_t* n);

/* The compute span of each timed layer, oldest first: from the begin record
 * (after the layer's ready wait, the last packet before its kernels) to the
 * record after its done event, in ms.  Timing is on while set_timing's
 * capacity is non-zero; the ring keeps the last `capacity` layers.  Host only;
 * synchronise the compute stream first.  Errors: SWR_E_INVALID, SWR_E_HIP. */
int swr_planner_layer_times(const swr_planner* p, float* ms, int32_t cap, int32_t* n);
/* Bytes received from peers so far (sum of (N-1)*C over gathers), and the
 * number of gathers issued, since creation. */
int swr_planner_counters(const swr_planner* p, int64_t* remote_bytes, int64_t* gathers);
/* Copies up to `cap` ops (4 int32 each: op, stream, layer, slot; -1 where
 * not applicable) recorded since the last reset into ops; *n = total count. */
int swr_planner_trace(const swr_planner* p, int32_t* ops, int32_t cap, int32_t* n);
void swr_planner_destroy(swr_planner* p);

/* ------------------------------------------------------------- errors */

/* Text of the last error on the calling thread ("" if none). */
const char* swr_last_error(void);

/* Library version string. */
const char* swr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWR_H */
