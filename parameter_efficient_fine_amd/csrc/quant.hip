// 4-bit block quantization of a frozen weight and its inverse (gfx950).
//
// "Unsloth vs The Stack v2", quantized-base card: the base weight is frozen
// in 4 bits and only the adapter trains. Format: for row n and 64-column block
// b, absmax = max |W| over the block; x = W / absmax (IEEE fp32 division);
// code = number of NF4 thresholds strictly below x (a tie goes to the lower
// level); a block of zeros stores absmax 0 and code 7. Two codes per byte,
// even column in the low nibble. Dequantization is fp32(L[code] * absmax).
#include "common.hpp"
#include "internal.hpp"

namespace qlora {

// One wave per (row, block); lane e handles column 64*b + e.
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks, int64_t kb_per_row,
                                                  int64_t K, uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                  uint32_t* __restrict__ nonfinite) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  const int64_t n = blk / kb_per_row, b = blk - n * kb_per_row;
  const float w = W[n * K + b * kBlock + lane];
  const bool bad = !__builtin_isfinite(w);
  float a = __builtin_fabsf(w);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  int code = 7;
  if (a != 0.0f) {
    const float x = w / a;
    code = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) code += (x > nf4_threshold(j)) ? 1 : 0;
  }
  const int partner = __shfl_xor(code, 1);
  if ((lane & 1) == 0) codes[n * (K / 2) + b * (kBlock / 2) + (lane >> 1)] = (uint8_t)(code | (partner << 4));
  const unsigned long long anybad = __ballot(bad);
  if (lane == 0) {
    absmax[n * kb_per_row + b] = anybad ? __builtin_nanf("") : a;
    if (anybad && nonfinite) atomicAdd(nonfinite, 1u);
  }
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

// One thread per code byte -> two fp32 outputs.
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                                    int64_t nbytes, int64_t K, float* __restrict__ W_hat) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nbytes) return;
  const int64_t half = K / 2;
  const int64_t n = i / half, c = i - n * half;
  const float a = absmax[n * (K / kBlock) + (2 * c) / kBlock];
  const uint8_t byte = codes[i];
  float2 out;
  out.x = nf4_level(byte & 15) * a;
  out.y = nf4_level(byte >> 4) * a;
  reinterpret_cast<float2*>(W_hat)[i] = out;
}

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                           uint32_t* nonfinite_blocks, hipStream_t st) {
  if (nonfinite_blocks) {
    k_zero_u32<<<1, 64, 0, st>>>(nonfinite_blocks);
  }
  const int64_t kb = K / kBlock, nblocks = N * kb;
  if (nblocks == 0) return hipGetLastError();
  const int64_t grid = (nblocks + 3) / 4;
  k_quantize<<<(unsigned)grid, 256, 0, st>>>(W, nblocks, kb, K, codes, absmax, nonfinite_blocks);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                             hipStream_t st) {
  const int64_t nbytes = N * K / 2;
  if (nbytes == 0) return hipSuccess;
  k_dequantize<<<(unsigned)((nbytes + 255) / 256), 256, 0, st>>>(codes, absmax, nbytes, K, W_hat);
  return hipGetLastError();
}

}  // namespace qlora
