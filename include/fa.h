/*
 * fa.h -- C ABI of libfa2tiles.so: FlashAttention-2-style tiled attention,
 * its backward, its fused forward-mode JVP, piecewise attention, and the
 * block-residual online-softmax merge, as hand-written HIP kernels for
 * AMD MI355X (gfx950).
 *
 * Common conventions (every entry point)
 * --------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or keeps a pointer after a call returns.  Outputs
 *   are overwritten, never accumulated into.
 * - Attention tensors are contiguous [B, H, S, D] (D fastest): q-like tensors
 *   have S = M rows (queries), k-like tensors S = N rows (keys).  LSE and the
 *   backward's Delta are contiguous fp32 [B, H, M].
 * - dtype selects the element type of every attention tensor (and of the
 *   merge's D-length row tensors): FA_F32, FA_F16 or FA_BF16.  Matrix
 *   products of fp16/bf16 inputs run on MFMA with fp32 accumulation; the
 *   probabilities P (and dS) are rounded to the input dtype before the
 *   products that consume them, as the FlagAttention kernels do.  FA_F32
 *   inputs are computed entirely in fp32 arithmetic.
 * - LSE is the natural-log log-sum-exp of the scaled scores of each query
 *   row (FlagAttention piecewise.py stores it this way; the Triton tutorial
 *   stores log2 -- same information, different unit).  A query row with no
 *   visible key gets O = 0 and LSE = -inf.
 * - causal is 0 or 1.  Causal masking is aligned bottom-right: query i sees
 *   key j iff j <= i + (N - M) (the P_SEQ offset of FlagAttention).
 * - sm_scale == 0 selects the default 1/sqrt(D) (the pages' "None"); any
 *   other value must be finite and > 0.
 * - stream is a hipStream_t passed as void*; NULL is the default stream.
 *   Launches are asynchronous; the caller synchronises.
 * - Every argument is validated on the host BEFORE any HIP call; if a check
 *   fails nothing is launched and the matching negative fa_status is
 *   returned.  A failed launch returns FA_ERR_HIP.  No C++ exception crosses
 *   this boundary.
 * - Alignment (FA_ERR_ALIGN otherwise): tensors of the call's dtype (q, k,
 *   v, o, dout, the gradients and tangents, the merge's row tensors and q)
 *   16 bytes; fp32 per-row vectors (lse, delta, l0, gl, gl0, gq) and the
 *   attention backward's workspace 4 bytes; the merge backward's workspace
 *   16 bytes.
 * - Supported attention shapes: B, H, M, N >= 1 (any lengths; the kernels
 *   mask the last partial tile); D in {16, 32, 64, 128, 256}, the head dims
 *   the tutorial's Function accepts, on every attention entry point and in
 *   every dtype (fa_fwd_fp8: D in {64, 128}).  16-bit D = 16, 32, 64, 128
 *   run on the matrix cores (D = 16 as zero-padded D = 32 tiles), as do the
 *   16-bit forward, backward and fused JVP at D = 256; fp32 and piecewise
 *   attention at D = 256 run a slower kernel without them.  Any other D
 *   gives FA_ERR_UNSUPPORTED.
 *
 * The seven entry points of the hot path (fa_fwd, fa_bwd, fa_fwd_jvp,
 * pw_fwd, pw_bwd, resmerge_fwd, resmerge_bwd) keep the pages' operations
 * and nothing more; options the pages do not have (a gradient reaching LSE,
 * the LSE tangent, accumulation into gx/gq) are separate entry points with
 * their own names (*_dlse, *_tlse, *_acc) and one extra argument each.
 *
 * Citations name the page and the function or passage whose computation the
 * entry point performs:
 *   [tutorial]  Birch-san's gist _06_fused_attention_blockptr_jvp.py (Triton
 *               fused-attention tutorial with JVP) and its comment thread;
 *   [piecewise] FlagAttention src/flag_attn/piecewise.py;
 *   [merge]     flash_attn_res 0.1.11, slop/backward_phase_2.txt.
 */
#ifndef FA2TILES_FA_H
#define FA2TILES_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  FA_ERR_SHAPE = -2,       /* a size is <= 0 or the sizes overflow         */
  FA_ERR_DTYPE = -3,       /* unknown dtype code                            */
  FA_ERR_ALIGN = -4,       /* a pointer is not aligned as required          */
  FA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required    */
  FA_ERR_UNSUPPORTED = -6, /* valid but unsupported (D, M/N granularity...)  */
  FA_ERR_HIP = -7          /* a HIP launch or runtime call failed           */
} fa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_strerror(int status);

/* Library ABI version (major*100 + minor). */
int fa_version(void);

/*
 * Attention forward [tutorial: _attn_fwd / _attn_fwd_inner; piecewise:
 * _fwd_kernel without the piecewise score selection].
 *   O   = softmax(sm_scale * Q K^T  (causally masked))  V      [B,H,M,D]
 *   lse = log sum_j exp(sm_scale * q_i . k_j)  over visible j  [B,H,M] fp32
 * One kernel; online softmax over K/V blocks; causal blocks beyond the
 * diagonal are skipped.
 */
int fa_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * FP8 attention forward [tutorial: _attn_fwd with FP8_OUTPUT inputs, the
 * float8 e5m2 path of its test and benchmark].  q [B,H,M,D], k [B,H,N,D]
 * and vt [B,H,D,N] (V transposed, keys contiguous, as the tutorial feeds an
 * fp8 V) hold OCP float8 e5m2 bytes; o [B,H,M,D] is written in out_dtype
 * (FA_F16 or FA_BF16; the tutorial writes fp8 and upcasts to compare),
 * lse [B,H,M] fp32 as fa_fwd.  Both products use fp8 matrix instructions
 * with fp32 accumulation; P is rounded to float8 e4m3 for P V (the tutorial
 * rounds it to e5m2).  D in {64, 128}; N a multiple of 16 (the V^t rows are
 * read in 16-key chunks); FA_ERR_UNSUPPORTED otherwise, FA_ERR_DTYPE for
 * another out_dtype.
 */
int fa_fwd_fp8(int out_dtype, const void* q, const void* k, const void* vt, void* o, float* lse,
               int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * Attention backward [tutorial: _attn_bwd_preprocess, _attn_bwd_dkdv,
 * _attn_bwd_dq, with the non-causal block range from the comment thread;
 * piecewise: _bwd_preprocess, _bwd_kv_kernel, _bwd_q_kernel].
 * Gradients dq, dk, dv of <dout, O> with (O, LSE) = fa_fwd(q, k, v); o
 * and lse must be the outputs of fa_fwd on the same inputs.  The steps:
 *   Delta_i = sum_d o_id dout_id                      (fa_bwd_delta)
 *   dK, dV  with K/V resident, looping over queries  (fa_bwd_dkdv)
 *   dQ      with Q resident, looping over keys       (fa_bwd_dq)
 * For fp16/bf16 fa_bwd makes two launches on `stream`: fa_bwd_dq_delta (the
 * dQ pass forming Delta as it loads each query row, and writing it to the
 * workspace), then fa_bwd_dkdv; for fp32, the three steps above in order.
 * workspace: device buffer of at least fa_bwd_workspace_size() bytes (it
 * holds Delta); it is scratch, its content on return is unspecified.
 */
size_t fa_bwd_workspace_size(int B, int H, int M, int N, int D, int dtype);
int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * fa_bwd with a gradient reaching the LSE output as well (not on the pages:
 * their backward takes dout only).  Gradients of <dout, O> + <dlse, LSE>;
 * dlse [B,H,M] fp32 is e.g. resmerge_bwd's gl0 when the attention output
 * feeds the merge as (y0, l0); NULL means zeros, i.e. exactly fa_bwd.  By
 * the chain rule dLSE_i/dS_ij = P_ij, so it enters as
 * dS = P (dP - (Delta - dlse)): Delta_i = sum_d o_id dout_id - dlse_i.
 * Arguments otherwise as fa_bwd (dlse is inserted after lse).
 */
int fa_bwd_dlse(int dtype, const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, const float* dlse, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes,
                int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and kernels, with Delta kept in a device array of the library
 * instead of a caller workspace.  Arguments as fa_bwd without workspace and
 * workspace_bytes.  B*H*M must not exceed 2^21 rows (the array holds 8 MiB of
 * fp32; FA_ERR_UNSUPPORTED beyond).  The first call on a device looks the
 * array's address up once (FA_ERR_HIP if that fails); no call allocates.
 * Each GPU has one such array, shared by every call on it: calls that overlap
 * on one GPU (different streams or host threads) race on it and give
 * undefined results.
 */
int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/* The steps of fa_bwd, exposed separately so each can be timed. */
/* delta [B,H,M] fp32 <- rowsum(o * dout) - dlse (dlse may be NULL)
 * [tutorial: _attn_bwd_preprocess] */
int fa_bwd_delta(int dtype, const void* o, const void* dout, const float* dlse, float* delta,
                 int B, int H, int M, int D, void* stream);
/* dk, dv [B,H,N,D] from q, k, v, dout, lse and delta  [tutorial: _attn_bwd_dkdv] */
int fa_bwd_dkdv(int dtype, const void* q, const void* k, const void* v, const void* dout,
                const float* lse, const float* delta, void* dk, void* dv,
                int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);
/* dq [B,H,M,D] from q, k, v, dout, lse and delta  [tutorial: _attn_bwd_dq] */
int fa_bwd_dq(int dtype, const void* q, const void* k, const void* v, const void* dout,
              const float* lse, const float* delta, void* dq,
              int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);
/* The preprocess and the dQ pass in one launch [tutorial: _attn_bwd_preprocess
 * and _attn_bwd_dq]: each query row's Delta is formed from o, dout and dlse
 * (NULL = zeros) as that row's operands are loaded, written to delta [B,H,M]
 * fp32 (bit-identical to fa_bwd_delta's) and used for dq.  fp32 runs
 * fa_bwd_delta then fa_bwd_dq.  Same argument rules as fa_bwd_dq. */
int fa_bwd_dq_delta(int dtype, const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, const float* dlse, float* delta, void* dq,
                    int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * Fused forward-mode JVP [tutorial: the ENABLE_JVP path of _attn_fwd_inner
 * and the tangent epilogue of _attn_fwd; method of Lu & Song, arXiv
 * 2410.11081].  Outputs o and lse exactly as fa_fwd, plus the tangent
 *   to = d/dt O(q + t*tq, k + t*tk, v + t*tv) at t = 0          [B,H,M,D]
 * computed in the same pass: with Sdot = sm_scale (tq K^T + Q tk^T),
 *   to = (P*Sdot) V - rowsum(P*Sdot) O + P tv.
 * tq is q-like, tk and tv are k-like.
 */
int fa_fwd_jvp(int dtype, const void* q, const void* k, const void* v,
               const void* tq, const void* tk, const void* tv,
               void* o, float* lse, void* to,
               int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * fa_fwd_jvp that also returns the tangent of lse (not on the pages: they
 * return tO only).  tlse [B,H,M] fp32 (may be NULL, which is exactly
 * fa_fwd_jvp) receives rowsum(P*Sdot), since dLSE_i/dS_ij = P_ij; 0 for a
 * row with no visible key.  Arguments otherwise as fa_fwd_jvp (tlse is
 * inserted after to).
 */
int fa_fwd_jvp_tlse(int dtype, const void* q, const void* k, const void* v,
                    const void* tq, const void* tk, const void* tv,
                    void* o, float* lse, void* to, float* tlse,
                    int B, int H, int M, int N, int D, int causal, float sm_scale, void* stream);

/*
 * Piecewise attention forward [piecewise: attention() and _fwd_kernel].
 * Score of (i, j): sm_scale * q1_i . k1_j if |i + (N - M) - j| <= w, else
 * sm_scale * q2_i . k2_j; then softmax, P V and lse as fa_fwd.  w may be
 * negative (every pair then uses q2, k2).  Blocks entirely inside or outside
 * the band compute one product; only blocks crossing it compute both.
 */
int pw_fwd(int dtype, const void* q1, const void* k1, const void* q2, const void* k2,
           const void* v, void* o, float* lse,
           int B, int H, int M, int N, int D, int causal, float sm_scale, int w, void* stream);

/*
 * Piecewise attention backward [piecewise: _bwd_preprocess, _bwd_kv_kernel,
 * _bwd_q_kernel].  dS is split by the same distance rule: the near part
 * yields dq1, dk1, the far part dq2, dk2; dv = P^T dout.  o and lse must come
 * from pw_fwd on the same inputs.  workspace as for fa_bwd
 * (pw_bwd_workspace_size() bytes, holds Delta).
 */
size_t pw_bwd_workspace_size(int B, int H, int M, int N, int D, int dtype);
int pw_bwd(int dtype, const void* q1, const void* k1, const void* q2, const void* k2,
           const void* v, const void* o, const void* dout, const float* lse,
           void* dq1, void* dk1, void* dq2, void* dk2, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int H, int M, int N, int D, int causal, float sm_scale, int w, void* stream);

/* pw_bwd with a gradient dlse [B,H,M] fp32 reaching the LSE output (may be
 * NULL: exactly pw_bwd), entering dS as in fa_bwd_dlse; dlse is inserted
 * after lse. */
int pw_bwd_dlse(int dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                const void* v, const void* o, const void* dout, const float* lse, const float* dlse,
                void* dq1, void* dk1, void* dq2, void* dk2, void* dv,
                void* workspace, size_t workspace_bytes,
                int B, int H, int M, int N, int D, int causal, float sm_scale, int w, void* stream);

/*
 * Block-residual two-way online-softmax merge, forward [merge:
 * reference_forward].  Per row r of x, y0 ([rows, D], dtype):
 *   rho = (mean(x^2) + eps)^-1/2;  l1 = rho * (x . q);  m = max(l0, l1)
 *   a = e^(l0-m) / Z, b = e^(l1-m) / Z, Z = e^(l0-m) + e^(l1-m)
 *   y = a*y0 + b*x   ([rows, D], dtype);   lse = m + log Z   ([rows] fp32)
 * q is the pseudo-query ([D], dtype); l0 is [rows] fp32 (may hold -inf).
 * D must be a multiple of 8; eps must be finite and >= 0.
 */
int resmerge_fwd(int dtype, const void* x, const void* q, const void* y0, const float* l0,
                 void* y, float* lse, int rows, int D, float eps, void* stream);

/*
 * Merge backward [merge: the phase-2 merge backward kernel and its
 * launcher].  VJP of resmerge_fwd for <gy, y> + <gl, lse>; gl == NULL means
 * zeros.  Outputs: gx, gy0 [rows, D] dtype; gl0 [rows] fp32; gq [D] fp32 =
 * sum over rows, reduced in a fixed order (no float atomics, so repeated
 * calls are bitwise identical).  Every output is overwritten.  workspace:
 * at least resmerge_bwd_workspace_size(rows, D) bytes of device scratch
 * (per-block partial sums of gq).
 */
size_t resmerge_bwd_workspace_size(int rows, int D);
int resmerge_bwd(int dtype, const void* x, const void* q, const void* y0, const float* l0,
                 const void* gy, const float* gl, void* gx, float* gq, void* gy0, float* gl0,
                 void* workspace, size_t workspace_bytes, int rows, int D, float eps, void* stream);

/*
 * resmerge_bwd with the page kernel's accumulate semantics as an option.
 * accumulate = 0: exactly resmerge_bwd.  accumulate = 1: the gradient is
 * added to what gx and gq hold (gx rounded once after the fp32 sum), as the
 * page's kernel adds into the caller's grad_intrablock_partial_sum and
 * grad_pseudo_query buffers; gy0 and gl0 are overwritten in both modes, as
 * on the page.  Other values: FA_ERR_UNSUPPORTED.  accumulate is inserted
 * after eps.
 */
int resmerge_bwd_acc(int dtype, const void* x, const void* q, const void* y0, const float* l0,
                     const void* gy, const float* gl, void* gx, float* gq, void* gy0, float* gl0,
                     void* workspace, size_t workspace_bytes, int rows, int D, float eps,
                     int accumulate, void* stream);

/*
 * N-way online-softmax merge of (y, lse) partials, forward [merge: the
 * two-way combine of reference_forward with both logits given, for S
 * inputs].  Combines attention outputs over disjoint key ranges (e.g. the
 * o/lse pairs of fa_fwd on key splits) into attention over all of them.
 * Per row r:
 *   lse = log sum_s exp(lses[s, r]),   y = sum_s exp(lses[s, r] - lse) ys[s, r]
 * ys [S, rows, D] dtype; lses [S, rows] fp32 (natural log, may hold -inf);
 * y [rows, D] dtype; lse [rows] fp32.  A row whose logits are all -inf
 * gets y = 0 and lse = -inf.  1 <= S <= 65536; D a multiple of 8, at most
 * 4096 (FA_ERR_UNSUPPORTED otherwise).
 */
int lse_merge_fwd(int dtype, const void* ys, const float* lses, void* y, float* lse,
                  int S, int rows, int D, void* stream);

/*
 * Its backward: the VJP of lse_merge_fwd for <gy, y> + <gl, lse> (gl may be
 * NULL: zeros).  With w_s = exp(lses[s] - lse):
 *   gys[s] = w_s gy   ([S, rows, D] dtype),
 *   glses[s] = w_s (gl + gy . (ys[s] - y))   ([S, rows] fp32).
 * Every output element is overwritten; no workspace.
 */
int lse_merge_bwd(int dtype, const void* ys, const float* lses, const void* gy, const float* gl,
                  void* gys, float* glses, int S, int rows, int D, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA2TILES_FA_H */
