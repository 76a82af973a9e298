// C ABI of libfa2tiles.so (declared in include/fa.h).
//
// Every entry point validates all of its arguments on the host before the
// first HIP call, so a rejected call launches nothing and has no side
// effects.  No C++ exception crosses the boundary: launchers return
// hipError_t, which is mapped to FA_ERR_HIP.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "kernels.h"

using fa::BwdArgs;
using fa::FwdArgs;
using fa::MergeArgs;

namespace {

constexpr int kVersion = 200;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_dtype(int dtype) { return (dtype == FA_F32 || dtype == FA_F16 || dtype == FA_BF16) ? FA_OK : FA_ERR_DTYPE; }

// Tensors read or written as 16-byte vectors.
int check_tensors(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return FA_ERR_NULL;
  for (const void* p : ps)
    if (!aligned(p, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Optional fp32 per-row vectors (NULL allowed).
int check_opt_scalars(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned(p, 4)) return FA_ERR_ALIGN;
  return FA_OK;
}

// fp32 per-row vectors (LSE, Delta, l0, gl0, gq).
int check_scalars(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return FA_ERR_NULL;
  for (const void* p : ps)
    if (!aligned(p, 4)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Head dims: 16, 32, 64, 128, 256 (those the tutorial's Function accepts)
// for every entry point and dtype.
int check_attn_shape(int B, int H, int M, int N, int D) {
  if (B <= 0 || H <= 0 || M <= 0 || N <= 0 || D <= 0) return FA_ERR_SHAPE;
  // grid sizes and element offsets must stay representable
  const int64_t bh = (int64_t)B * H;
  if (bh > (1 << 24) || M > (1 << 24) || N > (1 << 24)) return FA_ERR_SHAPE;
  if (bh * (int64_t)(M > N ? M : N) * D > ((int64_t)1 << 46)) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int resolve_scale(float sm_scale, int D, float* out) {
  if (sm_scale == 0.0f) {
    *out = 1.0f / sqrtf((float)D);
    return FA_OK;
  }
  if (!isfinite(sm_scale) || sm_scale < 0.0f) return FA_ERR_UNSUPPORTED;
  *out = sm_scale;
  return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

#define FA_TRY(expr)            \
  do {                          \
    const int st_ = (expr);     \
    if (st_ != FA_OK) return st_; \
  } while (0)

int run_fwd(FwdArgs& a, hipStream_t s) {
  return hip_status(fa::fwd_generic(a.dtype, a.variant, a.D) ? fa::launch_attn_fwd_generic(a, s)
                                                              : fa::launch_attn_fwd(a, s));
}

// The whole backward.  MFMA path (16-bit, D in {16, 32, 64, 128}, and plain
// attention at D = 256): the dQ pass
// forms Delta itself and writes it for the dK/dV pass that follows (two
// launches); generic path: the Delta kernel, then the two passes.
int run_bwd(BwdArgs& a, const void* o, const float* dlse, float* delta, hipStream_t s) {
  if (fa::bwd_generic(a.dtype, a.variant, a.D)) {
    FA_TRY(hip_status(fa::launch_attn_delta(a.dtype, o, a.dout, dlse, delta, (int64_t)a.B * a.H * a.M, a.D, s)));
    a.delta = delta;
    FA_TRY(hip_status(fa::launch_attn_dkdv_generic(a, s)));
    return hip_status(fa::launch_attn_dq_generic(a, s));
  }
  a.o = o;
  a.dlse = dlse;
  a.delta_out = delta;
  FA_TRY(hip_status(fa::launch_attn_dq(a, s)));
  a.o = nullptr;
  a.dlse = nullptr;
  a.delta_out = nullptr;
  a.delta = delta;
  return hip_status(fa::launch_attn_dkdv(a, s));
}

// One pass of the backward (dK/dV or dQ) reading a given Delta.
int run_bwd_pass(BwdArgs& a, const float* delta, hipStream_t s, bool dkdv) {
  a.delta = delta;
  const bool gen = fa::bwd_generic(a.dtype, a.variant, a.D);
  if (dkdv) return hip_status(gen ? fa::launch_attn_dkdv_generic(a, s) : fa::launch_attn_dkdv(a, s));
  return hip_status(gen ? fa::launch_attn_dq_generic(a, s) : fa::launch_attn_dq(a, s));
}

size_t delta_bytes(int B, int H, int M) { return (size_t)B * H * M * sizeof(float); }

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is non-positive or too large";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype code";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is misaligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but unsupported arguments";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return kVersion; }

int fa_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int M,
           int N, int D, int causal, float sm_scale, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({q, k, v, o}));
  FA_TRY(check_scalars({lse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  FwdArgs a = {};
  a.dtype = dtype;
  a.variant = fa::PLAIN;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  return run_fwd(a, (hipStream_t)stream);
}

int fa_fwd_fp8(int out_dtype, const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H,
               int M, int N, int D, int causal, float sm_scale, void* stream) {
  if (out_dtype != FA_F16 && out_dtype != FA_BF16) return FA_ERR_DTYPE;
  FA_TRY(check_tensors({q, k, vt, o}));
  FA_TRY(check_scalars({lse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (N % 16 != 0) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  fa::Fp8Args a = {};
  a.out_dtype = out_dtype;
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  return hip_status(fa::launch_attn_fwd_fp8(a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_size(int B, int H, int M, int N, int D, int dtype) {
  (void)N;
  (void)D;
  (void)dtype;
  if (B <= 0 || H <= 0 || M <= 0) return 0;
  return delta_bytes(B, H, M);
}

// Validation and arguments of the whole backward, before the Delta buffer.
static int bwd_args(int dtype, int variant, const void* q, const void* k, const void* q2, const void* k2,
                    const void* v, const void* o, const void* dout, const float* lse, const float* dlse, void* dq,
                    void* dk, void* dq2, void* dk2, void* dv, int B, int H, int M, int N, int D, int causal,
                    float sm_scale, int w, BwdArgs* out) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({q, k, v, o, dout, dq, dk, dv}));
  if (variant == fa::PW) FA_TRY(check_tensors({q2, k2, dq2, dk2}));
  FA_TRY(check_scalars({lse}));
  FA_TRY(check_opt_scalars({dlse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  BwdArgs& a = *out;
  a = BwdArgs{};
  a.dtype = dtype;
  a.variant = variant;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q2 = q2;
  a.k2 = k2;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq2 = dq2;
  a.dk2 = dk2;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  a.w = w;
  return FA_OK;
}

static int bwd_common(int dtype, int variant, const void* q, const void* k, const void* q2, const void* k2,
                      const void* v, const void* o, const void* dout, const float* lse, const float* dlse,
                      void* dq, void* dk, void* dq2, void* dk2, void* dv, void* workspace, size_t workspace_bytes,
                      int B, int H, int M, int N, int D, int causal, float sm_scale, int w, void* stream) {
  BwdArgs a;
  FA_TRY(bwd_args(dtype, variant, q, k, q2, k2, v, o, dout, lse, dlse, dq, dk, dq2, dk2, dv, B, H, M, N, D, causal,
                  sm_scale, w, &a));
  if (!workspace || workspace_bytes < delta_bytes(B, H, M)) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return FA_ERR_ALIGN;
  return run_bwd(a, o, dlse, (float*)workspace, (hipStream_t)stream);
}

int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H,
           int M, int N, int D, int causal, float sm_scale, void* stream) {
  return bwd_common(dtype, fa::PLAIN, q, k, nullptr, nullptr, v, o, dout, lse, nullptr, dq, dk, nullptr, nullptr, dv,
                    workspace, workspace_bytes, B, H, M, N, D, causal, sm_scale, 0, stream);
}

int fa_bwd_dlse(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, const float* dlse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int M, int N, int D, int causal, float sm_scale,
                void* stream) {
  return bwd_common(dtype, fa::PLAIN, q, k, nullptr, nullptr, v, o, dout, lse, dlse, dq, dk, nullptr, nullptr, dv,
                    workspace, workspace_bytes, B, H, M, N, D, causal, sm_scale, 0, stream);
}

int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int M, int N, int D, int causal,
                   float sm_scale, void* stream) {
  BwdArgs a;
  FA_TRY(bwd_args(dtype, fa::PLAIN, q, k, nullptr, nullptr, v, o, dout, lse, nullptr, dq, dk, nullptr, nullptr, dv, B,
                  H, M, N, D, causal, sm_scale, 0, &a));
  const int64_t rows = (int64_t)B * H * M;
  if (rows > fa::kNoAllocDeltaRows) return FA_ERR_UNSUPPORTED;
  float* delta = nullptr;
  FA_TRY(hip_status(fa::noalloc_delta_scratch((size_t)rows, &delta)));
  return run_bwd(a, o, nullptr, delta, (hipStream_t)stream);
}

int fa_bwd_delta(int dtype, const void* o, const void* dout, const float* dlse, float* delta, int B, int H, int M,
                 int D, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({o, dout}));
  FA_TRY(check_scalars({delta}));
  FA_TRY(check_opt_scalars({dlse}));
  FA_TRY(check_attn_shape(B, H, M, M, D));
  return hip_status(
      fa::launch_attn_delta(dtype, o, dout, dlse, delta, (int64_t)B * H * M, D, (hipStream_t)stream));
}

static int bwd_pass(bool dkdv, int dtype, const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, void* dq, void* dk, void* dv, int B, int H, int M, int N,
                    int D, int causal, float sm_scale, void* stream) {
  FA_TRY(check_dtype(dtype));
  if (dkdv)
    FA_TRY(check_tensors({q, k, v, dout, dk, dv}));
  else
    FA_TRY(check_tensors({q, k, v, dout, dq}));
  FA_TRY(check_scalars({lse, delta}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  BwdArgs a = {};
  a.dtype = dtype;
  a.variant = fa::PLAIN;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  return run_bwd_pass(a, delta, (hipStream_t)stream, dkdv);
}

int fa_bwd_dkdv(int dtype, const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const float* delta, void* dk, void* dv, int B, int H, int M, int N, int D, int causal,
                float sm_scale, void* stream) {
  return bwd_pass(true, dtype, q, k, v, dout, lse, delta, nullptr, dk, dv, B, H, M, N, D, causal, sm_scale,
                  stream);
}

int fa_bwd_dq(int dtype, const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const float* delta, void* dq, int B, int H, int M, int N, int D, int causal, float sm_scale,
              void* stream) {
  return bwd_pass(false, dtype, q, k, v, dout, lse, delta, dq, nullptr, nullptr, B, H, M, N, D, causal, sm_scale,
                  stream);
}

int fa_bwd_dq_delta(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, const float* dlse, float* delta, void* dq, int B, int H, int M, int N, int D,
                    int causal, float sm_scale, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({q, k, v, o, dout, dq}));
  FA_TRY(check_scalars({lse, delta}));
  FA_TRY(check_opt_scalars({dlse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  BwdArgs a = {};
  a.dtype = dtype;
  a.variant = fa::PLAIN;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  hipStream_t s = (hipStream_t)stream;
  if (fa::bwd_generic(dtype, fa::PLAIN, D)) {
    FA_TRY(hip_status(fa::launch_attn_delta(dtype, o, dout, dlse, delta, (int64_t)B * H * M, D, s)));
    a.delta = delta;
    return hip_status(fa::launch_attn_dq_generic(a, s));
  }
  a.o = o;
  a.dlse = dlse;
  a.delta_out = delta;
  return hip_status(fa::launch_attn_dq(a, s));
}

int fa_fwd_jvp(int dtype, const void* q, const void* k, const void* v, const void* tq, const void* tk,
               const void* tv, void* o, float* lse, void* to, int B, int H, int M, int N, int D, int causal,
               float sm_scale, void* stream) {
  return fa_fwd_jvp_tlse(dtype, q, k, v, tq, tk, tv, o, lse, to, nullptr, B, H, M, N, D, causal, sm_scale, stream);
}

int fa_fwd_jvp_tlse(int dtype, const void* q, const void* k, const void* v, const void* tq, const void* tk,
                    const void* tv, void* o, float* lse, void* to, float* tlse, int B, int H, int M, int N, int D,
                    int causal, float sm_scale, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({q, k, v, tq, tk, tv, o, to}));
  FA_TRY(check_scalars({lse}));
  FA_TRY(check_opt_scalars({tlse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  FwdArgs a = {};
  a.dtype = dtype;
  a.variant = fa::JVP;
  a.q = q;
  a.k = k;
  a.v = v;
  a.tq = tq;
  a.tk = tk;
  a.tv = tv;
  a.o = o;
  a.lse = lse;
  a.to = to;
  a.tlse = tlse;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  return run_fwd(a, (hipStream_t)stream);
}

int pw_fwd(int dtype, const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* o,
           float* lse, int B, int H, int M, int N, int D, int causal, float sm_scale, int w, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_tensors({q1, k1, q2, k2, v, o}));
  FA_TRY(check_scalars({lse}));
  FA_TRY(check_attn_shape(B, H, M, N, D));
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  float scale;
  FA_TRY(resolve_scale(sm_scale, D, &scale));
  FwdArgs a = {};
  a.dtype = dtype;
  a.variant = fa::PW;
  a.q = q1;
  a.k = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.causal = causal;
  a.sm_scale = scale;
  a.w = w;
  return run_fwd(a, (hipStream_t)stream);
}

size_t pw_bwd_workspace_size(int B, int H, int M, int N, int D, int dtype) {
  return fa_bwd_workspace_size(B, H, M, N, D, dtype);
}

int pw_bwd(int dtype, const void* q1, const void* k1, const void* q2, const void* k2, const void* v, const void* o,
           const void* dout, const float* lse, void* dq1, void* dk1, void* dq2, void* dk2, void* dv,
           void* workspace, size_t workspace_bytes, int B, int H, int M, int N, int D, int causal, float sm_scale,
           int w, void* stream) {
  return bwd_common(dtype, fa::PW, q1, k1, q2, k2, v, o, dout, lse, nullptr, dq1, dk1, dq2, dk2, dv, workspace,
                    workspace_bytes, B, H, M, N, D, causal, sm_scale, w, stream);
}

int pw_bwd_dlse(int dtype, const void* q1, const void* k1, const void* q2, const void* k2, const void* v,
                const void* o, const void* dout, const float* lse, const float* dlse, void* dq1, void* dk1,
                void* dq2, void* dk2, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int M, int N,
                int D, int causal, float sm_scale, int w, void* stream) {
  return bwd_common(dtype, fa::PW, q1, k1, q2, k2, v, o, dout, lse, dlse, dq1, dk1, dq2, dk2, dv, workspace,
                    workspace_bytes, B, H, M, N, D, causal, sm_scale, w, stream);
}

static int check_merge(int dtype, int rows, int D, float eps) {
  FA_TRY(check_dtype(dtype));
  if (rows <= 0 || D <= 0) return FA_ERR_SHAPE;
  if ((int64_t)rows * D > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  if (D % 8 != 0) return FA_ERR_UNSUPPORTED;
  if (!isfinite(eps) || eps < 0.0f) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int resmerge_fwd(int dtype, const void* x, const void* q, const void* y0, const float* l0, void* y, float* lse,
                 int rows, int D, float eps, void* stream) {
  FA_TRY(check_tensors({x, q, y0, y}));
  FA_TRY(check_scalars({l0, lse}));
  FA_TRY(check_merge(dtype, rows, D, eps));
  MergeArgs a = {};
  a.dtype = dtype;
  a.x = x;
  a.q = q;
  a.y0 = y0;
  a.l0 = l0;
  a.y = y;
  a.lse = lse;
  a.rows = rows;
  a.D = D;
  a.eps = eps;
  return hip_status(fa::launch_merge_fwd(a, (hipStream_t)stream));
}

size_t resmerge_bwd_workspace_size(int rows, int D) {
  if (rows <= 0 || D <= 0) return 0;
  return (size_t)fa::merge_bwd_partial_rows(rows, D) * (size_t)D * sizeof(float);
}

int resmerge_bwd(int dtype, const void* x, const void* q, const void* y0, const float* l0, const void* gy,
                 const float* gl, void* gx, float* gq, void* gy0, float* gl0, void* workspace,
                 size_t workspace_bytes, int rows, int D, float eps, void* stream) {
  return resmerge_bwd_acc(dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, workspace, workspace_bytes, rows, D, eps, 0,
                          stream);
}

int resmerge_bwd_acc(int dtype, const void* x, const void* q, const void* y0, const float* l0, const void* gy,
                     const float* gl, void* gx, float* gq, void* gy0, float* gl0, void* workspace,
                     size_t workspace_bytes, int rows, int D, float eps, int accumulate, void* stream) {
  FA_TRY(check_tensors({x, q, y0, gy, gx, gy0}));
  FA_TRY(check_scalars({l0, gq, gl0}));
  if (gl && !aligned(gl, 4)) return FA_ERR_ALIGN;
  FA_TRY(check_merge(dtype, rows, D, eps));
  if (accumulate != 0 && accumulate != 1) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < resmerge_bwd_workspace_size(rows, D)) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  MergeArgs a = {};
  a.dtype = dtype;
  a.x = x;
  a.q = q;
  a.y0 = y0;
  a.l0 = l0;
  a.gy = gy;
  a.gl = gl;
  a.gx = gx;
  a.gq = gq;
  a.gy0 = gy0;
  a.gl0 = gl0;
  a.partial = (float*)workspace;
  a.rows = rows;
  a.D = D;
  a.eps = eps;
  a.accumulate = accumulate;
  return hip_status(fa::launch_merge_bwd(a, (hipStream_t)stream));
}

static int check_lse_merge(int dtype, int S, int rows, int D) {
  FA_TRY(check_dtype(dtype));
  if (S <= 0 || rows <= 0 || D <= 0) return FA_ERR_SHAPE;
  if (S > (1 << 16) || (int64_t)S * rows * D > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  if (D % 8 != 0 || D > 4096) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int lse_merge_fwd(int dtype, const void* ys, const float* lses, void* y, float* lse, int S, int rows, int D,
                  void* stream) {
  FA_TRY(check_tensors({ys, y}));
  FA_TRY(check_scalars({lses, lse}));
  FA_TRY(check_lse_merge(dtype, S, rows, D));
  fa::LseMergeArgs a = {};
  a.dtype = dtype;
  a.ys = ys;
  a.lses = lses;
  a.y = y;
  a.lse = lse;
  a.S = S;
  a.rows = rows;
  a.D = D;
  return hip_status(fa::launch_lse_merge_fwd(a, (hipStream_t)stream));
}

int lse_merge_bwd(int dtype, const void* ys, const float* lses, const void* gy, const float* gl, void* gys,
                  float* glses, int S, int rows, int D, void* stream) {
  FA_TRY(check_tensors({ys, gy, gys}));
  FA_TRY(check_scalars({lses, glses}));
  FA_TRY(check_opt_scalars({gl}));
  FA_TRY(check_lse_merge(dtype, S, rows, D));
  fa::LseMergeArgs a = {};
  a.dtype = dtype;
  a.ys = ys;
  a.lses = lses;
  a.gy = gy;
  a.gl = gl;
  a.gys = gys;
  a.glses = glses;
  a.S = S;
  a.rows = rows;
  a.D = D;
  return hip_status(fa::launch_lse_merge_bwd(a, (hipStream_t)stream));
}

}  // extern "C"
