// Launchers of the gfx950 kernels (host side). Each enqueues on `st` and
// returns the launch status; argument validation happens in api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// fmt: 0 NF4 (codes [N, K/2]), 1 INT8, 2 FP8 E4M3 (codes [N, K]); one fp32 per 64-block
hipError_t launch_quantize(int fmt, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                           uint32_t* nonfinite_blocks, hipStream_t st);
hipError_t launch_dequantize(int fmt, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                             hipStream_t st);
// launch_quantize with a per-device counter of non-finite blocks, read back
// into *nonfinite_out (synchronizes `st`; calls are serialized)
hipError_t quantize_counting(int fmt, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                             uint32_t* nonfinite_out, hipStream_t st);
// checkpoint-order codes (row-major; NF4 column 2c in the low nibble of byte c)
// and row-major block values -> the storage order of the GEMMs
hipError_t launch_pack_codes(int fmt, const uint8_t* src, const float* src_abs, int64_t N, int64_t K, uint8_t* codes,
                             float* absmax, hipStream_t st);

// Skinny rank-r products ------------------------------------------------------

// out[M, R] (bf16) = in[M, Kd] . [ad1; ad2]^T with fp32 accumulation: adapter
// rows j < r1 come from ad1 [r1, Kd] and go to out1 (row stride ld1), rows
// r1 <= j < r1 + r2 from ad2 [r2, Kd] to out2 (row stride ld2); r2 may be 0.
struct NtArgs {
  const uint16_t* in;
  int64_t M, Kd;
  const uint16_t* ad1;
  const uint16_t* ad2;
  int r1, r2;
  uint16_t* out1;
  uint16_t* out2;
  int64_t ld1, ld2;
  int ad_kr;  // 1: a single adapter ad1 stored [Kd, r1] (r1 = 16, 32, 64, 128 or 256, r2 == 0), e.g. B for G = dY.B
};
hipError_t launch_skinny_nt(const NtArgs& a, hipStream_t st);

// Reduction over M of P[M, R]^T . Q[M, Kd] (P row stride ldp, R = r1 + r2 <=
// kTnMaxR): rows j < r1 give s1 * (..) into out1, the others s2 * (..) into
// out2 (j counted from r1). Element (j, k) goes to out[j * ldo + k], or to
// out[k * ldo + j] when transposed; fp32, or bf16 (one rounding of the fp32
// sum) when out_bf16. launch_skinny_tn splits the rows
// over workgroups that write fp32 partials to `part`; launch_tn_reduce (next
// on the same stream), or the prologue of a backward GEMM launched next with
// them, adds them in split order and writes out1/out2.
constexpr int kTnMaxR = 128;
struct TnPlan {
  int splits;
  int col_tiles;
  int64_t rows;  // rows per split (multiple of 64)
};
TnPlan skinny_tn_plan(int64_t M, int64_t Kd, int R);
struct TnArgs {
  const uint16_t* P;
  int64_t ldp;
  int r1, r2;
  float s1, s2;
  void* out1;           // float, or bf16 bits when out_bf16
  void* out2;
  int64_t ldo1, ldo2;
  int transposed;
  int accumulate;       // 1: add the result to what out1/out2 hold (sums over batch tiles; fp32 only)
  int out_bf16;
  const uint16_t* Q;
  int64_t M, Kd;
  float* part;          // [splits, R, Kd]
  int64_t rows;         // set by the launchers from skinny_tn_plan
  int splits;
};
// Up to kTnMaxJobs independent reductions in one launch of each kernel
// (blockIdx.z selects the job; every job has its own `part`).
constexpr int kTnMaxJobs = 3;
struct TnJobs {
  TnArgs job[kTnMaxJobs];
  int n;
};
hipError_t launch_skinny_tn(TnJobs jobs, hipStream_t st);
hipError_t launch_tn_reduce(TnJobs jobs, hipStream_t st);
// The jobs of a skinny_tn launch that still need their partials reduced (more
// than one split), with `splits` set; the backward GEMM takes such a set and
// does the reduction itself (launch_gemm_bwd*, `red`).
TnJobs tn_reduce_jobs(const TnJobs& jobs);

// One launch before a backward: dst[C, R] = src[R, C]^T for each job (bf16).
constexpr int kMaxPrepJobs = 3;
struct TransposeJob {
  const uint16_t* src;
  uint16_t* dst;
  int64_t R, C;
};
struct PrepJobs {
  TransposeJob job[kMaxPrepJobs];
  int n;
};
hipError_t launch_prep(const PrepJobs& jobs, hipStream_t st);

// p[0..n) = 0 (a kernel, so the call stays capturable in a graph)
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st);
hipError_t launch_fill_zero_u16(uint16_t* p, int64_t n, hipStream_t st);

// dst[i] = bf16(src[i]) (round to nearest even) for up to kMaxCastJobs arrays in one launch
constexpr int kMaxCastJobs = 6;
struct CastJob {
  const float* src;
  uint16_t* dst;
  int64_t n;
};
struct CastJobs {
  CastJob job[kMaxCastJobs];
  int n;
};
hipError_t launch_cast_bf16(const CastJobs& jobs, hipStream_t st);

// Fused dequant GEMMs -------------------------------------------------------
struct WSrc {           // one frozen quantized weight [N, K] with its LoRA pair
  const uint8_t* codes;  // [N, K/2] (NF4) or [N, K] (INT8, FP8)
  const float* absmax;   // [N, K/64]: NF4 absmax, 8-bit scale
  const uint16_t* lora_i;  // fwd: B [N, r] ; bwd: A [r, K]
  const uint16_t* lora_j;  // fwd: Z [M, r] ; bwd: G [M, r] with row stride ldj
  int r;
  int64_t ldj;
  float s;
  int fmt;               // 0 NF4, 1 INT8, 2 FP8 (E4M3)
};

// The fused GEMMs, one set per weight format (gemm_fwd.hip and gemm_bwd.hip
// are compiled once per format into the namespaces f0, f1, f2).
#define QL_GEMM_LAUNCHERS                                                                                          \
  /* Y[M, N] = X . What^T + s . Z . B^T */                                                                         \
  hipError_t launch_gemm_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, uint16_t* Y,              \
                             hipStream_t st);                                                                      \
  /* the same with RoPE (heads of 128, rotate half) applied to the fp32 result before its bf16 rounding */          \
  hipError_t launch_gemm_fwd_rope(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, const int32_t* pos,  \
                                  const float* table, int64_t max_pos, uint16_t* Y, hipStream_t st);               \
  /* gate/up of the SwiGLU block in one pass: g, u [M, N], h = silu(g) * u */                                      \
  hipError_t launch_gemm_fwd_gateup(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc wg, WSrc wu,          \
                                    uint16_t* g, uint16_t* u, uint16_t* h, hipStream_t st);                        \
  /* dX[M, K] = dY0 . What0 + s0 . G0 . A0 (+ dY1 . What1 + s1 . G1 . A1 when dY1 != null); red (may be null): */ \
  /* reductions of the preceding skinny_tn (tn_reduce_jobs) done by the same launch */                              \
  hipError_t launch_gemm_bwd(const uint16_t* dY0, WSrc w0, const uint16_t* dY1, WSrc w1, int64_t M, int64_t K,     \
                             int64_t N, uint16_t* dX, const TnJobs* red, hipStream_t st);                          \
  /* dh = dY . What + s . G . A (never stored); dg = dh*u*sig(g)*(1+g*(1-sig(g))), du = dh*silu(g) */              \
  hipError_t launch_gemm_bwd_swiglu(const uint16_t* dY, WSrc w, int64_t M, int64_t K, int64_t N, const uint16_t* g, \
                                    const uint16_t* u, uint16_t* dg, uint16_t* du, const TnJobs* red,              \
                                    hipStream_t st);
namespace f0 { QL_GEMM_LAUNCHERS }
namespace f1 { QL_GEMM_LAUNCHERS }
namespace f2 { QL_GEMM_LAUNCHERS }
#undef QL_GEMM_LAUNCHERS

// Dispatch on the weight format (every weight of one call shares its format).
#define QL_BY_FMT(fmt, call) \
  ((fmt) == 0 ? f0::call : (fmt) == 1 ? f1::call : f2::call)
inline hipError_t launch_gemm_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, uint16_t* Y,
                                  hipStream_t st) {
  return QL_BY_FMT(w.fmt, launch_gemm_fwd(X, M, K, N, w, Y, st));
}
inline hipError_t launch_gemm_fwd_rope(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, const int32_t* pos,
                                       const float* table, int64_t max_pos, uint16_t* Y, hipStream_t st) {
  return QL_BY_FMT(w.fmt, launch_gemm_fwd_rope(X, M, K, N, w, pos, table, max_pos, Y, st));
}
inline hipError_t launch_gemm_fwd_gateup(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc wg, WSrc wu,
                                         uint16_t* g, uint16_t* u, uint16_t* h, hipStream_t st) {
  return QL_BY_FMT(wg.fmt, launch_gemm_fwd_gateup(X, M, K, N, wg, wu, g, u, h, st));
}
inline hipError_t launch_gemm_bwd(const uint16_t* dY0, WSrc w0, const uint16_t* dY1, WSrc w1, int64_t M, int64_t K,
                                  int64_t N, uint16_t* dX, const TnJobs* red, hipStream_t st) {
  return QL_BY_FMT(w0.fmt, launch_gemm_bwd(dY0, w0, dY1, w1, M, K, N, dX, red, st));
}
inline hipError_t launch_gemm_bwd_swiglu(const uint16_t* dY, WSrc w, int64_t M, int64_t K, int64_t N,
                                         const uint16_t* g, const uint16_t* u, uint16_t* dg, uint16_t* du,
                                         const TnJobs* red, hipStream_t st) {
  return QL_BY_FMT(w.fmt, launch_gemm_bwd_swiglu(dY, w, M, K, N, g, u, dg, du, red, st));
}
#undef QL_BY_FMT

// Small-batch path (batches of at most kSmallMaxM tokens, ranks up to
// kSmallMaxR): one workgroup per 32 x 32 output tile, its four waves splitting
// the reduction.
constexpr int64_t kSmallMaxM = 256;
constexpr int kSmallMaxR = 32;
struct SmallFwdArgs {       // Y = X . What^T + s . Z . B^T and Z = X . A^T
  const uint16_t* X;        // [M, K]
  const uint8_t* codes;     // frozen weight [N, K] (storage order of qlora.h)
  const float* absmax;
  const uint16_t* A;        // [r, K]
  const uint16_t* B;        // [N, r]
  int64_t M, K, N;
  int r;
  float s;
  uint16_t* Y;              // [M, N]
  uint16_t* Z;              // [M, r]
};
struct SmallBwdArgs {       // dX = dY . What + s . G . A and G = dY . B
  const uint16_t* dY;       // [M, N]
  const uint8_t* codes;
  const float* absmax;
  const uint16_t* A;
  const uint16_t* B;
  int64_t M, K, N;
  int r;
  float s;
  uint16_t* dX;             // [M, K] (may be null: G only)
  uint16_t* G;              // [M, r]
};
hipError_t launch_small_fwd(const SmallFwdArgs& a, int fmt, hipStream_t st);
hipError_t launch_small_bwd(const SmallBwdArgs& a, int fmt, hipStream_t st);

// LM head and chunked cross-entropy: Y [M, N] = X [M, K] . W [N, K]^T (bf16
// operands, W in the tiled order of launch_tile_nt, fp32 or bf16 output); per-row statistics of a logits chunk; counts
// and the final mean.
hipError_t launch_gemm_nt_bf16(const uint16_t* X, const uint16_t* W, int64_t M, int64_t K, int64_t N, void* Y,
                               bool out_f32, float* stats, hipStream_t st);
hipError_t launch_ce_count(const int32_t* tgt, int64_t M, int64_t V, int32_t* n_keep, hipStream_t st);
hipError_t launch_ce_rows(const float* logits, const float* stats, const int32_t* tgt, const int32_t* n_keep,
                          int64_t C, int64_t V, float* loss_rows, uint16_t* dz, hipStream_t st);
hipError_t launch_ce_total(const float* loss_rows, int64_t M, const int32_t* n_keep, float* loss, hipStream_t st);
// the weight operand of launch_gemm_nt_bf16 in its tiled order (W = src or src^T)
hipError_t launch_tile_nt(const uint16_t* src, int64_t R, int64_t C, bool transpose, uint16_t* dst, hipStream_t st);

// RMSNorm rows of x [M,H] with frozen weight w [H]: y bf16, rstd fp32 [M];
// backward: dx only.
hipError_t launch_rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, float eps, uint16_t* y,
                              float* rstd, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd, int64_t M,
                              int64_t H, uint16_t* dx, hipStream_t st);
// cos/sin table [max_pos][d/2][2] fp32 of the RoPE angles (fp64 angles and sin/cos)
hipError_t launch_rope_table(int d, double base, int64_t max_pos, float* table, hipStream_t st);
// In-place RoPE of q [M, hq*d] and k [M, hk*d] by pos [M]; inverse rotates back.
hipError_t launch_rope(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t M, int hq, int hk, int d, double base,
                       bool inverse, hipStream_t st);

}  // namespace qlora
