// Launchers of the gfx950 kernels (host side). Each enqueues on `st` and
// returns the launch status; argument validation happens in api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                           uint32_t* nonfinite_blocks, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                             hipStream_t st);

// out[M, r] (bf16) = in[M, Kd] . ad[r, Kd]^T ; fp32 accumulation.
// Up to two adapters: rows j < r1 come from ad1 (written to out1, width r1),
// rows r1 <= j < r1 + r2 from ad2 (written to out2, width r2); ad2 may be null.
hipError_t launch_skinny_nt(const uint16_t* in, int64_t M, int64_t Kd, const uint16_t* ad1, int r1, uint16_t* out1,
                            const uint16_t* ad2, int r2, uint16_t* out2, hipStream_t st);

// part[S, r, Kd] (fp32) = per-split partial of P[M, r]^T . Q[M, Kd]; returns S via *splits.
int skinny_tn_splits(int64_t M, int64_t Kd);
hipError_t launch_skinny_tn(const uint16_t* P, int r, const uint16_t* Q, int64_t M, int64_t Kd, float* part,
                            int splits, hipStream_t st);
// out = s * sum_S part ; transposed: out[k, j] (ld = r), else out[j, k] (ld = Kd)
hipError_t launch_reduce_splits(const float* part, int splits, int r, int64_t Kd, float s, float* out, bool transposed,
                                hipStream_t st);

// p[0..n) = 0 (a kernel, so the call stays capturable in a graph)
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st);

// dst[C, R] = src[R, C]^T for bf16 matrices
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, hipStream_t st);

// Fused dequant GEMMs -------------------------------------------------------
struct WSrc {           // one frozen 4-bit weight [N, K] with its LoRA pair
  const uint8_t* codes;  // [N, K/2]
  const float* absmax;   // [N, K/64]
  const uint16_t* lora_i;  // fwd: B [N, r] ; bwd: A^T [K, r]
  const uint16_t* lora_j;  // fwd: Z [M, r] ; bwd: G [M, r]
  int r;
  float s;
};

// Y[M, N] = X . What^T + s . Z . B^T
hipError_t launch_gemm_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, uint16_t* Y, hipStream_t st);
// gate/up of the SwiGLU block in one pass: g, u [M, N], h = silu(g) * u
hipError_t launch_gemm_fwd_gateup(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc wg, WSrc wu, uint16_t* g,
                                  uint16_t* u, uint16_t* h, hipStream_t st);
// dX[M, K] = sum_t dY_t . What_t + s_t . G_t . A_t over one or two (dY_t, W_t) pairs
// (the concatenated reduction of gate and up); each dY_t is [M, N].
hipError_t launch_gemm_bwd(const uint16_t* dY0, WSrc w0, const uint16_t* dY1, WSrc w1, int64_t M, int64_t K,
                           int64_t N, uint16_t* dX, hipStream_t st);
// down-projection backward with the SwiGLU backward in the epilogue:
// dh = dY . What + s . G . A (never stored); dg = dh*u*sig(g)*(1+g*(1-sig(g))), du = dh*silu(g)
hipError_t launch_gemm_bwd_swiglu(const uint16_t* dY, WSrc w, int64_t M, int64_t K, int64_t N, const uint16_t* g,
                                  const uint16_t* u, uint16_t* dg, uint16_t* du, hipStream_t st);

}  // namespace qlora
