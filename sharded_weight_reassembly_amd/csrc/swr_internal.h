// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swr.h"

namespace swr {

// Native 16-byte vectors (usable with the nontemporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Records a printf-style message as the calling thread's last error and
// returns `code` so call sites can `return fail(...)`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_fail(hipError_t e, const char* what);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- copies
struct ChunkPtrs {
  const void* p[SWR_MAX_CHUNKS];
};
// One weight of the row-shard re-layout (see swr_redistribute_row_shards).
struct RedistArgs {
  const uint8_t* src[SWR_MAX_CHUNKS];  // rank shards (replicated: src[0] is the whole weight)
  void* chunk[SWR_MAX_CHUNKS];
  int64_t begin, end;                  // bytes of T written by this launch
  int64_t off, size, row_bytes;        // the weight's item
  int64_t sub_start[SWR_MAX_SUB + 1];  // first row of each sub-block in the weight
  int64_t sub_first[SWR_MAX_SUB];      // first row of each sub-block inside a rank shard
  int64_t chunk_bytes;
  int32_t n_sub, replicated, n;
};
hipError_t launch_redistribute(const RedistArgs& a, hipStream_t stream);

hipError_t launch_reassemble(const ChunkPtrs& chunks, int n_chunks, int64_t chunk_bytes, void* slot,
                             unsigned lds_bytes, hipStream_t stream);
// swr_reassemble_into_slot whose copy workgroups each reserve lds_bytes of
// LDS (the planner's gather, swr_planner_set_gather_lds).
int reassemble_reserving(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes, void* slot,
                         int64_t slot_bytes, int32_t self_rank, hipStream_t side, hipEvent_t gate, hipEvent_t ready,
                         int64_t* remote_bytes, unsigned lds_bytes);

struct PackPlan {
  const void* src[SWR_MAX_WEIGHTS];
  int64_t off[SWR_MAX_WEIGHTS];
  int64_t size[SWR_MAX_WEIGHTS];
  void* chunk[SWR_MAX_CHUNKS];
  int64_t chunk_bytes;
  int64_t total_bytes;
  int32_t n_weights;
  int32_t n_chunks;
};
hipError_t launch_pack(const PackPlan& plan, hipStream_t stream);

struct PartPtrs {
  const float* p[SWR_MAX_CHUNKS];
};
hipError_t launch_sum_partials(const PartPtrs& parts, int n, int64_t count, void* out, bool out_bf16,
                               hipStream_t stream);

// ---------------------------------------------------------------- GEMMs
enum OutMode { OUT_BF16 = 0, OUT_F32 = 1, OUT_SILU_BF16 = 2 };

// One weight-streaming GEMM  Y[m, o] = s[o] * sum_k X[m, k] W[o, k]  (or, in
// OUT_SILU_BF16 mode, h[m, j] = silu(G[m, j]) * G[m, I + j] with G the scaled
// product over 2I rows).  The plan fixes the kernel shape and split-K.
struct GemmProblem {
  const void* W;
  int dtype;
  const float* scale;  // may be null
  const void* X;       // bf16 (E4M3FN codes for launch_tile_fp8act)
  int64_t ldx;
  int64_t M;
  int64_t rows;  // output rows of W (2I in SILU mode)
  int64_t K;
  void* Y;
  int64_t ldy;
  int mode;
};

struct GemmPlan {
  int kind;      // 0 streaming MFMA, 1 generic, 2 LDS-staged MFMA (decode), 3 tiled MFMA (prefill),
                 // 6 LDS-staged with eight waves split along K in two row halves and X through
                 // LDS (decode, 17-64 tokens)
  int mt;        // 16-token blocks per workgroup (1, 2, 4)
  int rt;        // 16-row tiles per workgroup (kind 3: weight rows per tile, 128 or 256)
  int64_t rb;    // output rows per row block, a multiple of 4 up to the rt tiles' rows
                 // (gate rows in SILU mode); fewer masks the tiles' last rows
  int ksplit;    // workgroups along K
  int64_t kper;  // K elements per split (multiple of the stage length)
  int sk;        // staged kinds: K elements per stage (256, or 512 for one FP8 token block)
  int64_t partial_bytes;  // fp32 split-K scratch needed (0 if ksplit == 1)
};

GemmPlan plan_gemm(const GemmProblem& p, bool may_split = true);
bool plan_is_valid(const GemmProblem& p, const GemmPlan& plan);
// Enqueues the GEMM; `partial` must hold plan.partial_bytes bytes.
hipError_t launch_gemm(const GemmProblem& p, const GemmPlan& plan, float* partial, hipStream_t stream);

// Grouped projections (no SiLU mode): true when the n problems can run as one
// staged launch (same dtype and token count, M <= 64, K a multiple of 256,
// aligned); sets the token blocks and row tiles per workgroup.
constexpr int kMaxGroup = SWR_MAX_GROUP;
bool grouped_plan(const GemmProblem* ps, int n, int* mt, int* rt);
hipError_t launch_grouped(const GemmProblem* ps, int n, int mt, int rt, hipStream_t stream);

// The MLP behind swr_mlp_forward (y_fp32: swr_mlp_forward_partial): checks
// every argument, then enqueues the GEMMs with `workspace` as scratch.
int mlp_impl(const char* fn, const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d,
             int32_t dtype, int64_t H, int64_t I, const void* X, int64_t M, void* Y, bool y_fp32, void* workspace,
             int64_t workspace_bytes, hipStream_t stream);

// ---------------------------------------------------------------- FP8 activations
// Per-token E4M3FN codes and scales of BF16 rows (quant.hip).
hipError_t launch_quantize_rows(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q, int64_t ldq, float* S,
                                hipStream_t stream);
// The tiled GEMM with FP8 weights and FP8 activations: p.X holds E4M3FN codes
// (p.ldx bytes per token), xscale one fp32 scale per token; p.K % 64 == 0.
hipError_t launch_tile_fp8act(const GemmProblem& p, const float* xscale, hipStream_t stream);

}  // namespace swr
