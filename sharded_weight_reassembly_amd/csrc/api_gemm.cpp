// C ABI of the GEMM entry points: argument checks, plan selection and the
// workspace layout.  Every check happens before anything is enqueued.
#include "swr_internal.h"

using swr::aligned;
using swr::fail;

namespace {

constexpr int64_t kWorkspaceAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(int32_t d) { return d == SWR_BF16 || d == SWR_FP8_E4M3FN; }

// A 256-byte aligned stand-in pointer: plans made with it assume the fast
// (aligned) kernel, which needs the most scratch.
const void* kAlignedProbe = reinterpret_cast<const void*>(uintptr_t(1) << 20);

swr::GemmProblem mlp_gate_up(const void* W, const float* s, int32_t dtype, int64_t H, int64_t I, const void* X,
                             int64_t M, void* h) {
  swr::GemmProblem p{};
  p.W = W;
  p.dtype = dtype;
  p.scale = s;
  p.X = X;
  p.ldx = H;
  p.M = M;
  p.rows = 2 * I;
  p.K = H;
  p.Y = h;
  p.ldy = I;
  p.mode = swr::OUT_SILU_BF16;
  return p;
}

swr::GemmProblem mlp_down(const void* W, const float* s, int32_t dtype, int64_t H, int64_t I, const void* h,
                          int64_t M, void* Y) {
  swr::GemmProblem p{};
  p.W = W;
  p.dtype = dtype;
  p.scale = s;
  p.X = h;
  p.ldx = I;
  p.M = M;
  p.rows = H;
  p.K = I;
  p.Y = Y;
  p.ldy = H;
  p.mode = swr::OUT_BF16;
  return p;
}

int64_t h_bytes(int64_t M, int64_t I) { return round_up(M * I * 2, kWorkspaceAlign); }

int check_sizes(const char* fn, int64_t M, int64_t a, int64_t b) {
  const int64_t kLimit = INT64_C(1) << 40;
  if (M < 0 || a < 1 || b < 1 || M > kLimit || a > kLimit || b > kLimit || (M > 0 && a > kLimit / M) ||
      (M > 0 && b > kLimit / M) || a > kLimit / b)
    return fail(SWR_E_SHAPE, "%s: unsupported sizes M=%lld, %lld, %lld", fn, (long long)M, (long long)a, (long long)b);
  return SWR_OK;
}

}  // namespace

extern "C" int64_t swr_proj_workspace_bytes(int64_t M, int64_t out_f, int64_t in_f, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(SWR_E_INVALID, "swr_proj_workspace_bytes: unknown dtype %d", dtype);
  if (int rc = check_sizes("swr_proj_workspace_bytes", M, out_f, in_f)) return rc;
  swr::GemmProblem p{};
  p.W = kAlignedProbe;
  p.dtype = dtype;
  p.X = kAlignedProbe;
  p.ldx = round_up(in_f, 8);
  p.M = M;
  p.rows = out_f;
  p.K = in_f;
  p.mode = swr::OUT_BF16;
  swr::clear_error();
  return swr::plan_gemm(p).partial_bytes;
}

extern "C" int swr_proj_forward(const void* W, int32_t dtype, const float* row_scale, int64_t out_f, int64_t in_f,
                                const void* X, int64_t ldx, int64_t M, void* Y, int32_t y_fp32, int64_t ldy,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  const char* fn = "swr_proj_forward";
  if (!W || !X || !Y) return fail(SWR_E_INVALID, "%s: null pointer", fn);
  if (!valid_dtype(dtype)) return fail(SWR_E_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (dtype == SWR_FP8_E4M3FN && !row_scale) return fail(SWR_E_INVALID, "%s: FP8 weights need row scales", fn);
  if (int rc = check_sizes(fn, M, out_f, in_f)) return rc;
  if (ldx < in_f || ldy < out_f) return fail(SWR_E_SHAPE, "%s: ldx=%lld < in or ldy=%lld < out", fn,
                                             (long long)ldx, (long long)ldy);
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 16) || (row_scale && !aligned(row_scale, 16)))
    return fail(SWR_E_ALIGN, "%s: W, X, Y and row_scale must be 16-byte aligned", fn);
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
    return fail(SWR_E_INVALID, "%s: workspace_bytes=%lld with workspace=%p", fn, (long long)workspace_bytes, workspace);
  if (workspace && !aligned(workspace, kWorkspaceAlign))
    return fail(SWR_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  swr::GemmProblem p{};
  p.W = W;
  p.dtype = dtype;
  p.scale = row_scale;
  p.X = X;
  p.ldx = ldx;
  p.M = M;
  p.rows = out_f;
  p.K = in_f;
  p.Y = Y;
  p.ldy = ldy;
  p.mode = y_fp32 ? swr::OUT_F32 : swr::OUT_BF16;
  // no scratch given: a plan without K splits (no partial sums)
  const swr::GemmPlan plan = swr::plan_gemm(p, workspace != nullptr);
  if (plan.partial_bytes > workspace_bytes)
    return fail(SWR_E_CAPACITY, "%s: workspace holds %lld bytes, needs %lld", fn, (long long)workspace_bytes,
                (long long)plan.partial_bytes);
  if (M == 0) {
    swr::clear_error();
    return SWR_OK;
  }
  const hipError_t e = swr::launch_gemm(p, plan, static_cast<float*>(workspace), stream);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_proj_forward: launch");
  swr::clear_error();
  return SWR_OK;
}

namespace {

// Checks one grouped descriptor like swr_proj_forward checks its arguments.
int check_desc(const char* fn, const swr_proj_desc& d, int i, int64_t M) {
  if (!d.W || !d.X || !d.Y) return fail(SWR_E_INVALID, "%s: descriptor %d has a null pointer", fn, i);
  if (!valid_dtype(d.dtype)) return fail(SWR_E_INVALID, "%s: descriptor %d has unknown dtype %d", fn, i, d.dtype);
  if (d.dtype == SWR_FP8_E4M3FN && !d.row_scale)
    return fail(SWR_E_INVALID, "%s: descriptor %d: FP8 weights need row scales", fn, i);
  if (int rc = check_sizes(fn, M, d.out_features, d.in_features)) return rc;
  if (d.ldx < d.in_features || d.ldy < d.out_features)
    return fail(SWR_E_SHAPE, "%s: descriptor %d: ldx=%lld < in or ldy=%lld < out", fn, i, (long long)d.ldx,
                (long long)d.ldy);
  if (!aligned(d.W, 16) || !aligned(d.X, 16) || !aligned(d.Y, 16) || (d.row_scale && !aligned(d.row_scale, 16)))
    return fail(SWR_E_ALIGN, "%s: descriptor %d: W, X, Y and row_scale must be 16-byte aligned", fn, i);
  return SWR_OK;
}

swr::GemmProblem desc_problem(const swr_proj_desc& d, int64_t M) {
  swr::GemmProblem p{};
  p.W = d.W;
  p.dtype = d.dtype;
  p.scale = d.row_scale;
  p.X = d.X;
  p.ldx = d.ldx;
  p.M = M;
  p.rows = d.out_features;
  p.K = d.in_features;
  p.Y = d.Y;
  p.ldy = d.ldy;
  p.mode = d.y_fp32 ? swr::OUT_F32 : swr::OUT_BF16;
  return p;
}

// Validates the group; on success fills ps and returns the scratch the call
// needs (0 for one grouped launch), else a negative status.
int64_t plan_group(const char* fn, const swr_proj_desc* descs, int32_t n, int64_t M, swr::GemmProblem* ps,
                   bool* one_launch, int* mt, int* rt) {
  if (!descs) return fail(SWR_E_INVALID, "%s: null descriptor array", fn);
  if (n < 1 || n > SWR_MAX_GROUP) return fail(SWR_E_INVALID, "%s: n=%d outside [1, %d]", fn, n, SWR_MAX_GROUP);
  for (int i = 0; i < n; ++i) {
    if (int rc = check_desc(fn, descs[i], i, M)) return rc;
    ps[i] = desc_problem(descs[i], M);
  }
  *one_launch = swr::grouped_plan(ps, n, mt, rt);
  if (*one_launch) return 0;
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t b = swr::plan_gemm(ps[i]).partial_bytes;
    if (b > need) need = b;
  }
  return need;
}

}  // namespace

extern "C" int64_t swr_proj_grouped_workspace_bytes(const swr_proj_desc* descs, int32_t n, int64_t M) {
  swr::GemmProblem ps[SWR_MAX_GROUP];
  bool one = false;
  int mt = 0, rt = 0;
  const int64_t need = plan_group("swr_proj_grouped_workspace_bytes", descs, n, M, ps, &one, &mt, &rt);
  if (need >= 0) swr::clear_error();
  return need;
}

extern "C" int swr_proj_forward_grouped(const swr_proj_desc* descs, int32_t n, int64_t M, void* workspace,
                                        int64_t workspace_bytes, hipStream_t stream) {
  const char* fn = "swr_proj_forward_grouped";
  swr::GemmProblem ps[SWR_MAX_GROUP];
  bool one = false;
  int mt = 0, rt = 0;
  const int64_t need = plan_group(fn, descs, n, M, ps, &one, &mt, &rt);
  if (need < 0) return int(need);
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
    return fail(SWR_E_INVALID, "%s: workspace_bytes=%lld with workspace=%p", fn, (long long)workspace_bytes, workspace);
  if (workspace && !aligned(workspace, kWorkspaceAlign))
    return fail(SWR_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  // separate launches: each projection as swr_proj_forward would plan it
  swr::GemmPlan plans[SWR_MAX_GROUP];
  if (!one) {
    for (int i = 0; i < n; ++i) {
      plans[i] = swr::plan_gemm(ps[i], workspace != nullptr);
      if (plans[i].partial_bytes > workspace_bytes)
        return fail(SWR_E_CAPACITY, "%s: workspace holds %lld bytes, descriptor %d needs %lld", fn,
                    (long long)workspace_bytes, i, (long long)plans[i].partial_bytes);
    }
  }
  if (M == 0) {
    swr::clear_error();
    return SWR_OK;
  }
  if (one) {
    const hipError_t e = swr::launch_grouped(ps, n, mt, rt, stream);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_proj_forward_grouped: launch");
  } else {
    for (int i = 0; i < n; ++i) {
      const hipError_t e = swr::launch_gemm(ps[i], plans[i], static_cast<float*>(workspace), stream);
      if (e != hipSuccess) return swr::hip_fail(e, "swr_proj_forward_grouped: launch");
    }
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" int64_t swr_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(SWR_E_INVALID, "swr_mlp_workspace_bytes: unknown dtype %d", dtype);
  if (int rc = check_sizes("swr_mlp_workspace_bytes", M, H, 2 * I)) return rc;
  const int64_t pg =
      swr::plan_gemm(mlp_gate_up(kAlignedProbe, nullptr, dtype, H, I, kAlignedProbe, M, nullptr)).partial_bytes;
  const int64_t pd =
      swr::plan_gemm(mlp_down(kAlignedProbe, nullptr, dtype, H, I, kAlignedProbe, M, nullptr)).partial_bytes;
  swr::clear_error();
  return h_bytes(M, I) + round_up(pg > pd ? pg : pd, kWorkspaceAlign);
}

namespace swr {

// The MLP of swr_mlp_forward; with y_fp32 the down GEMM writes fp32 (no rounding).
int mlp_impl(const char* fn, const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d,
             int32_t dtype, int64_t H, int64_t I, const void* X, int64_t M, void* Y, bool y_fp32, void* workspace,
             int64_t workspace_bytes, hipStream_t stream) {
  if (!W_gate_up || !W_down || !X || !Y || !workspace) return fail(SWR_E_INVALID, "%s: null pointer", fn);
  if (!valid_dtype(dtype)) return fail(SWR_E_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (dtype == SWR_FP8_E4M3FN && (!s_gu || !s_d)) return fail(SWR_E_INVALID, "%s: FP8 weights need row scales", fn);
  if (int rc = check_sizes(fn, M, H, 2 * I)) return rc;
  if (!aligned(W_gate_up, 16) || !aligned(W_down, 16) || !aligned(X, 16) || !aligned(Y, 16) ||
      (s_gu && !aligned(s_gu, 16)) || (s_d && !aligned(s_d, 16)))
    return fail(SWR_E_ALIGN, "%s: weights, scales, X and Y must be 16-byte aligned", fn);
  if (!aligned(workspace, kWorkspaceAlign)) return fail(SWR_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  const int64_t need = swr_mlp_workspace_bytes(M, H, I, dtype);
  if (need < 0) return int(need);
  if (workspace_bytes < need)
    return fail(SWR_E_CAPACITY, "%s: workspace holds %lld bytes, needs %lld", fn, (long long)workspace_bytes,
                (long long)need);
  if (M == 0) {
    swr::clear_error();
    return SWR_OK;
  }
  void* h = workspace;
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + h_bytes(M, I));
  const swr::GemmProblem gu = mlp_gate_up(W_gate_up, s_gu, dtype, H, I, X, M, h);
  swr::GemmProblem dn = mlp_down(W_down, s_d, dtype, H, I, h, M, Y);
  if (y_fp32) dn.mode = swr::OUT_F32;
  const swr::GemmPlan pg = swr::plan_gemm(gu);
  const swr::GemmPlan pd = swr::plan_gemm(dn);
  hipError_t e = swr::launch_gemm(gu, pg, partial, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp: gate_up launch");
  e = swr::launch_gemm(dn, pd, partial, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp: down launch");
  swr::clear_error();
  return SWR_OK;
}

}  // namespace swr

using swr::mlp_impl;

extern "C" int swr_mlp_forward(const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d,
                               int32_t dtype, int64_t H, int64_t I, const void* X, int64_t M, void* Y,
                               void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return mlp_impl("swr_mlp_forward", W_gate_up, s_gu, W_down, s_d, dtype, H, I, X, M, Y, false, workspace,
                  workspace_bytes, stream);
}

extern "C" int swr_mlp_forward_partial(const void* W_gate_up, const float* s_gu, const void* W_down,
                                       const float* s_d, int32_t dtype, int64_t H, int64_t I, const void* X,
                                       int64_t M, float* Y, void* workspace, int64_t workspace_bytes,
                                       hipStream_t stream) {
  return mlp_impl("swr_mlp_forward_partial", W_gate_up, s_gu, W_down, s_d, dtype, H, I, X, M, Y, true, workspace,
                  workspace_bytes, stream);
}

// ---------------------------------------------------------------- FP8 activations

namespace {

// Workspace of swr_mlp_forward_fp8act: [q_x: M*H][s_x: M][h: M*I bf16][q_h: M*I][s_h: M], 256-byte sections.
struct Fp8ActSections {
  int64_t qx, sx, h, qh, sh, total;
};

Fp8ActSections fp8act_sections(int64_t M, int64_t H, int64_t I) {
  Fp8ActSections w{};
  w.qx = 0;
  w.sx = w.qx + round_up(M * H, kWorkspaceAlign);
  w.h = w.sx + round_up(M * 4, kWorkspaceAlign);
  w.qh = w.h + round_up(M * I * 2, kWorkspaceAlign);
  w.sh = w.qh + round_up(M * I, kWorkspaceAlign);
  w.total = w.sh + round_up(M * 4, kWorkspaceAlign);
  return w;
}

}  // namespace

extern "C" int64_t swr_mlp_fp8act_workspace_bytes(int64_t M, int64_t H, int64_t I) {
  if (int rc = check_sizes("swr_mlp_fp8act_workspace_bytes", M, H, 2 * I)) return rc;
  swr::clear_error();
  return fp8act_sections(M, H, I).total;
}

extern "C" int swr_mlp_forward_fp8act(const void* W_gate_up, const float* s_gu, const void* W_down, const float* s_d,
                                      int64_t H, int64_t I, const void* X, int64_t M, void* Y, void* workspace,
                                      int64_t workspace_bytes, hipStream_t stream) {
  const char* fn = "swr_mlp_forward_fp8act";
  if (!W_gate_up || !W_down || !X || !Y || !workspace || !s_gu || !s_d)
    return fail(SWR_E_INVALID, "%s: null pointer (FP8 weights need row scales)", fn);
  if (int rc = check_sizes(fn, M, H, 2 * I)) return rc;
  if (H % 64 != 0 || I % 64 != 0)
    return fail(SWR_E_SHAPE, "%s: H=%lld and I=%lld must be multiples of 64", fn, (long long)H, (long long)I);
  if (2 * I * H >= (INT64_C(1) << 31) || H * I >= (INT64_C(1) << 31) || H >= (INT64_C(1) << 22) ||
      I >= (INT64_C(1) << 22))
    return fail(SWR_E_SHAPE, "%s: weights of 2 GiB or more", fn);
  if (!aligned(W_gate_up, 16) || !aligned(W_down, 16) || !aligned(X, 16) || !aligned(Y, 16) || !aligned(s_gu, 16) ||
      !aligned(s_d, 16))
    return fail(SWR_E_ALIGN, "%s: weights, scales, X and Y must be 16-byte aligned", fn);
  if (!aligned(workspace, kWorkspaceAlign)) return fail(SWR_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  const Fp8ActSections w = fp8act_sections(M, H, I);
  if (workspace_bytes < w.total)
    return fail(SWR_E_CAPACITY, "%s: workspace holds %lld bytes, needs %lld", fn, (long long)workspace_bytes,
                (long long)w.total);
  if (M == 0) {
    swr::clear_error();
    return SWR_OK;
  }
  char* ws = static_cast<char*>(workspace);
  void* qx = ws + w.qx;
  float* sx = reinterpret_cast<float*>(ws + w.sx);
  void* h = ws + w.h;
  void* qh = ws + w.qh;
  float* sh = reinterpret_cast<float*>(ws + w.sh);
  hipError_t e = swr::launch_quantize_rows(X, H, M, H, qx, H, sx, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp fp8act: quantize X");
  const swr::GemmProblem gu = mlp_gate_up(W_gate_up, s_gu, SWR_FP8_E4M3FN, H, I, qx, M, h);
  e = swr::launch_tile_fp8act(gu, sx, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp fp8act: gate_up launch");
  e = swr::launch_quantize_rows(h, I, M, I, qh, I, sh, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp fp8act: quantize h");
  const swr::GemmProblem dn = mlp_down(W_down, s_d, SWR_FP8_E4M3FN, H, I, qh, M, Y);
  e = swr::launch_tile_fp8act(dn, sh, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "mlp fp8act: down launch");
  swr::clear_error();
  return SWR_OK;
}
