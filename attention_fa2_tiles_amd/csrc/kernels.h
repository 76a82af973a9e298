// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Arguments here are already validated; every launcher returns hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum Variant : int { PLAIN = 0, JVP = 1, PW = 2 };

struct FwdArgs {
  int dtype;               // fa_dtype code
  int variant;             // PLAIN, JVP or PW
  const void* q;           // q   (PW: q1)
  const void* k;           // k   (PW: k1)
  const void* v;
  const void* q2;          // PW only
  const void* k2;          // PW only
  const void* tq;          // JVP only
  const void* tk;          // JVP only
  const void* tv;          // JVP only
  void* o;
  float* lse;
  void* to;                // JVP only
  float* tlse;             // JVP only, may be NULL
  int B, H, M, N, D;
  int causal;
  float sm_scale;          // resolved (> 0)
  int w;                   // PW only
};

struct BwdArgs {
  int dtype;
  int variant;             // PLAIN or PW
  const void* q;           // (PW: q1)
  const void* k;           // (PW: k1)
  const void* v;
  const void* q2;          // PW only
  const void* k2;          // PW only
  const void* dout;
  const float* lse;
  const float* delta;
  const void* o;           // dQ pass with Delta: o, dlse (may be NULL) and
  const float* dlse;       // the Delta output; NULL delta_out = read delta
  float* delta_out;
  void* dq;                // (PW: dq1)
  void* dk;                // (PW: dk1)
  void* dv;
  void* dq2;               // PW only
  void* dk2;               // PW only
  int B, H, M, N, D;
  int causal;
  float sm_scale;
  int w;
};

struct MergeArgs {
  int dtype;
  const void* x;
  const void* q;
  const void* y0;
  const float* l0;
  void* y;                 // fwd
  float* lse;              // fwd
  const void* gy;          // bwd
  const float* gl;         // bwd (may be null)
  void* gx;                // bwd
  float* gq;               // bwd
  void* gy0;               // bwd
  float* gl0;              // bwd
  float* partial;          // bwd workspace
  int rows, D;
  float eps;
  int accumulate;          // bwd: add gx, gq into the outputs instead of overwriting
};

struct LseMergeArgs {
  int dtype;
  const void* ys;          // [S, rows, D]
  const float* lses;       // [S, rows]
  void* y;                 // fwd [rows, D]
  float* lse;              // fwd [rows]
  const void* gy;          // bwd [rows, D]
  const float* gl;         // bwd [rows] (may be null)
  void* gys;               // bwd [S, rows, D]
  float* glses;            // bwd [S, rows]
  int S;
  int64_t rows;
  int D;
};

struct Fp8Args {
  int out_dtype;           // fa_dtype of o (fp16 or bf16)
  const void* q;           // [B, H, M, D] e5m2
  const void* k;           // [B, H, N, D] e5m2
  const void* vt;          // [B, H, D, N] e5m2
  void* o;                 // [B, H, M, D]
  float* lse;              // [B, H, M]
  int B, H, M, N, D;
  int causal;
  float sm_scale;          // resolved (> 0)
};

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_attn_fwd_fp8(const Fp8Args& a, hipStream_t s);
// delta = rowsum(o * dout) - dlse (dlse may be NULL: zeros)
hipError_t launch_attn_delta(int dtype, const void* o, const void* dout, const float* dlse, float* delta,
                             int64_t rows, int D, hipStream_t s);
hipError_t launch_attn_dkdv(const BwdArgs& a, hipStream_t s);
hipError_t launch_attn_dq(const BwdArgs& a, hipStream_t s);

// Generic (no MFMA) versions of the same operations: fp32 inputs, and the
// 16-bit head dims the MFMA kernels do not cover (16; 256 outside the plain
// forward).  Any dtype, D in {16, 32, 64, 128, 256}.
hipError_t launch_attn_fwd_generic(const FwdArgs& a, hipStream_t s);
hipError_t launch_attn_dkdv_generic(const BwdArgs& a, hipStream_t s);
hipError_t launch_attn_dq_generic(const BwdArgs& a, hipStream_t s);

// Whether a shape runs on the generic kernels rather than the MFMA ones.
inline bool fwd_generic(int dtype, int variant, int D) {
  return dtype == 0 || (D == 256 && variant == PW);
}
inline bool bwd_generic(int dtype, int variant, int D) {
  return dtype == 0 || (D == 256 && variant != PLAIN);
}

// The no-allocation backward's Delta rows live in a device array of this
// many floats (8 MiB), one copy per GPU; noalloc_delta_scratch returns the
// current device's copy (looked up once per device), or an error when rows
// exceeds it.
constexpr int64_t kNoAllocDeltaRows = (int64_t)1 << 21;
hipError_t noalloc_delta_scratch(size_t rows, float** out);

hipError_t launch_merge_fwd(const MergeArgs& a, hipStream_t s);
int merge_bwd_partial_rows(int rows, int D);   // number of gq partial vectors
hipError_t launch_merge_bwd(const MergeArgs& a, hipStream_t s);

hipError_t launch_lse_merge_fwd(const LseMergeArgs& a, hipStream_t s);
hipError_t launch_lse_merge_bwd(const LseMergeArgs& a, hipStream_t s);

}  // namespace fa
