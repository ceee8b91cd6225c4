// Block quantization of a frozen weight and its inverse (gfx950): the 4-bit
// NF4 format and, further down, the 8-bit INT8 and FP8 (E4M3) formats.
//
// "Unsloth vs The Stack v2", quantized-base card: the base weight is frozen
// in 4 bits and only the adapter trains. Format: for row n and 64-column block
// b, absmax = max |W| over the block; x = W / absmax (IEEE fp32 division);
// code = number of NF4 thresholds strictly below x (a tie goes to the lower
// level); a block of zeros stores absmax 0 and code 7. Dequantization is
// fp32(L[code] * absmax). Two codes per byte: in each run of 8 columns
// 8j .. 8j+7 (4 bytes), byte b holds column 8j+b in its low nibble and column
// 8j+b+4 in its high nibble, the order the GEMMs' dequantizer reads.
// Storage order of rows and blocks (all formats): tile-major, see TileAddr in
// common.hpp.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace qlora {

// Sixteen lanes per (row, block), four blocks per wave: lane i of a group
// handles columns 64*b + 4i .. 4i+3 (one 16-byte load), so each lane works on
// four independent weights and a block's absmax takes four shuffle steps.
__device__ __forceinline__ float group16_max(float a) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  return a;
}

// Whether any lane of this lane's 16-lane group has `bad` set.
__device__ __forceinline__ bool group16_any(bool bad, int lane) {
  return ((__ballot(bad) >> (lane & 48)) & 0xFFFFull) != 0;
}

__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks, int64_t kb_per_row,
                                                  int64_t N, int64_t K, uint8_t* __restrict__ codes,
                                                  float* __restrict__ absmax, uint32_t* __restrict__ nonfinite) {
  const int lane = threadIdx.x & 63, i = lane & 15;
  const int64_t blk = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (blk >= nblocks) return;  // whole 16-lane groups leave together
  const int64_t n = blk / kb_per_row, b = blk - n * kb_per_row;
  const TileAddr ta(n, b, N, K);
  const f32x4 w = *reinterpret_cast<const f32x4*>(W + n * K + b * kBlock + 4 * i);
  bool bad = false;
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bad = bad || !__builtin_isfinite(w[e]);
    a = fmaxf(a, __builtin_fabsf(w[e]));
  }
  a = group16_max(a);
  uint32_t packed = 0;  // code of column 4i + e in byte e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int code = 7;
    if (a != 0.0f) {
      const float x = w[e] / a;
      code = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) code += (x > nf4_threshold(j)) ? 1 : 0;
    }
    packed |= (uint32_t)code << (8 * e);
  }
  // run of 8 columns = lanes 2m (low nibbles) and 2m + 1 (columns + 4: high nibbles)
  const uint32_t partner = __shfl_xor(packed, 1);
  if ((i & 1) == 0)
    *reinterpret_cast<uint32_t*>(codes + ta.code(kBlock / 2) + 4 * (i >> 1)) = packed | (partner << 4);
  const bool anybad = group16_any(bad, lane);
  if (i == 0) {
    absmax[ta.value()] = anybad ? __builtin_nanf("") : a;
    if (anybad && nonfinite) atomicAdd(nonfinite, 1u);
  }
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

// One thread per 4 code bytes (a run of 8 columns) -> 8 fp32 outputs (row-major W_hat).
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                                    int64_t nruns, int64_t N, int64_t K, float* __restrict__ W_hat) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nruns) return;
  const int64_t runs = K / 8;
  const int64_t n = i / runs, j = i - n * runs;
  const TileAddr ta(n, j / 8, N, K);
  const float a = absmax[ta.value()];
  const uint32_t x = *reinterpret_cast<const uint32_t*>(codes + ta.code(kBlock / 2) + 4 * (j % 8));
  f32x4 lo, hi;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    lo[b] = nf4_level((x >> (8 * b)) & 15) * a;
    hi[b] = nf4_level((x >> (8 * b + 4)) & 15) * a;
  }
  reinterpret_cast<f32x4*>(W_hat)[2 * i] = lo;
  reinterpret_cast<f32x4*>(W_hat)[2 * i + 1] = hi;
}

// ---------------------------------------------------------------------------
// 8-bit formats ("Rev vs unsloth", fused quantized-LoRA card: int8 and fp8
// base weights). Per row n and 64-column block b, with a = max |W|:
//   INT8: s = a / 127, q = clamp(rint(W / s), -127, 127), a two's-complement byte;
//   FP8:  s = a / 448, code = the OCP E4M3 value nearest to W / s (ties to the
//         even code, saturating at 448; sign bit = the sign of W / s);
// a block of zeros stores s = 0 and codes 0. The block's fp32 slot holds s.

// fp32 -> E4M3 with round to nearest even; |x| >= 448 saturates to 448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float ax = __builtin_fabsf(x);
  uint32_t mag;
  if (ax >= 448.0f) {
    mag = 0x7Eu;
  } else if (ax < 0.015625f) {           // below 2^-6: multiples of 2^-9 (codes 0..8)
    mag = (uint32_t)__builtin_rintf(ax * 512.0f);
  } else {                               // round the fp32 significand to 3 bits, rebias 127 -> 7
    const uint32_t b = __builtin_bit_cast(uint32_t, ax);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    mag = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    mag = mag > 0x7Eu ? 0x7Eu : mag;
  }
  return sign | mag;
}

// One wave per (row, block); lane e handles column 64*b + e.
template <int F>
__global__ __launch_bounds__(256) void k_quantize8(const float* __restrict__ W, int64_t nblocks, int64_t kb_per_row,
                                                   int64_t N, int64_t K, uint8_t* __restrict__ codes,
                                                   float* __restrict__ scale, uint32_t* __restrict__ nonfinite) {
  const int lane = threadIdx.x & 63, i = lane & 15;
  const int64_t blk = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (blk >= nblocks) return;  // whole 16-lane groups leave together
  const int64_t n = blk / kb_per_row, b = blk - n * kb_per_row;
  const TileAddr ta(n, b, N, K);
  const f32x4 w = *reinterpret_cast<const f32x4*>(W + n * K + b * kBlock + 4 * i);
  bool bad = false;
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bad = bad || !__builtin_isfinite(w[e]);
    a = fmaxf(a, __builtin_fabsf(w[e]));
  }
  a = group16_max(a);
  const float s = a / (F == kInt8 ? 127.0f : 448.0f);
  uint32_t packed = 0;  // code of column 4i + e in byte e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t code = 0;
    if (s != 0.0f) {
      const float x = w[e] / s;
      if constexpr (F == kInt8) {
        const float q = fminf(fmaxf(__builtin_rintf(x), -127.0f), 127.0f);
        code = (uint32_t)(int)q & 0xFFu;
      } else {
        code = e4m3_encode(x);
      }
    }
    packed |= code << (8 * e);
  }
  *reinterpret_cast<uint32_t*>(codes + ta.code(kBlock) + 4 * i) = packed;
  const bool anybad = group16_any(bad, lane);
  if (i == 0) {
    scale[ta.value()] = anybad ? __builtin_nanf("") : s;
    if (anybad && nonfinite) atomicAdd(nonfinite, 1u);
  }
}

// One thread per 4 codes -> 4 fp32 outputs, decoded as the GEMMs decode them.
template <int F>
__global__ __launch_bounds__(256) void k_dequantize8(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
                                                     int64_t nquads, int64_t N, int64_t K, float* __restrict__ W_hat) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nquads) return;
  const int64_t e0 = 4 * i, n = e0 / K, k = e0 - n * K;
  const TileAddr ta(n, k / kBlock, N, K);
  const WPrep<F> p = wprep<F>(scale[ta.value()]);
  const uint32_t x = *reinterpret_cast<const uint32_t*>(codes + ta.code(kBlock) + k % kBlock);
  reinterpret_cast<f32x4*>(W_hat)[i] = wdeq4_f32<F>(x, p);
}

// ---------------------------------------------------------------------------
// Checkpoint order -> this library's order. A 4-bit checkpoint stores codes
// row-major [N, K/2] with column 2c in the low and 2c+1 in the high nibble of
// byte c, and its fp32 absmax row-major [N, K/64]; the 8-bit formats store one
// byte per column, row-major [N, K]. One thread per 4 code bytes (NF4: a run
// of 8 columns, whose nibbles are re-paired column b with b+4; 8-bit: 4
// columns, copied); the first thread of each (row, block) moves its value.
template <int F>
__global__ __launch_bounds__(256) void k_pack_codes(const uint8_t* __restrict__ src, const float* __restrict__ src_abs,
                                                    int64_t nquads, int64_t N, int64_t K, uint8_t* __restrict__ codes,
                                                    float* __restrict__ absmax) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nquads) return;
  constexpr int64_t kBB = F == kNF4 ? kBlock / 2 : kBlock;  // code bytes per row and block
  const int64_t row_bytes = F == kNF4 ? K / 2 : K;
  const int64_t n = (4 * i) / row_bytes, byte = 4 * i - n * row_bytes;
  const int64_t b = byte / kBB;
  const TileAddr ta(n, b, N, K);
  uint32_t x = *reinterpret_cast<const uint32_t*>(src + 4 * i);
  if constexpr (F == kNF4) {
    uint32_t c[8];  // columns 8j .. 8j+7 of this run
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (x >> (4 * e)) & 15u;
    x = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) x |= (c[q] | (c[q + 4] << 4)) << (8 * q);
  }
  *reinterpret_cast<uint32_t*>(codes + ta.code(kBB) + byte % kBB) = x;
  if (byte % kBB == 0) absmax[ta.value()] = src_abs[n * (K / kBlock) + b];
}

hipError_t launch_pack_codes(int fmt, const uint8_t* src, const float* src_abs, int64_t N, int64_t K, uint8_t* codes,
                             float* absmax, hipStream_t st) {
  const int64_t nquads = N * (fmt == kNF4 ? K / 2 : K) / 4;
  if (nquads == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nquads + 255) / 256);
  if (fmt == kNF4)
    k_pack_codes<kNF4><<<grid, 256, 0, st>>>(src, src_abs, nquads, N, K, codes, absmax);
  else if (fmt == kInt8)
    k_pack_codes<kInt8><<<grid, 256, 0, st>>>(src, src_abs, nquads, N, K, codes, absmax);
  else
    k_pack_codes<kFp8><<<grid, 256, 0, st>>>(src, src_abs, nquads, N, K, codes, absmax);
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                           uint32_t* nonfinite_blocks, hipStream_t st) {
  if (nonfinite_blocks) {
    k_zero_u32<<<1, 64, 0, st>>>(nonfinite_blocks);
  }
  const int64_t kb = K / kBlock, nblocks = N * kb;
  if (nblocks == 0) return hipGetLastError();
  const unsigned grid = (unsigned)((nblocks + 15) / 16);  // 16 blocks per workgroup
  if (fmt == kNF4)
    k_quantize<<<grid, 256, 0, st>>>(W, nblocks, kb, N, K, codes, absmax, nonfinite_blocks);
  else if (fmt == kInt8)
    k_quantize8<kInt8><<<grid, 256, 0, st>>>(W, nblocks, kb, N, K, codes, absmax, nonfinite_blocks);
  else
    k_quantize8<kFp8><<<grid, 256, 0, st>>>(W, nblocks, kb, N, K, codes, absmax, nonfinite_blocks);
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                             hipStream_t st) {
  if (fmt == kNF4) {
    const int64_t nruns = N * K / 8;
    if (nruns == 0) return hipSuccess;
    k_dequantize<<<(unsigned)((nruns + 255) / 256), 256, 0, st>>>(codes, absmax, nruns, N, K, W_hat);
    return hipGetLastError();
  }
  const int64_t nquads = N * K / 4;
  if (nquads == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nquads + 255) / 256);
  if (fmt == kInt8)
    k_dequantize8<kInt8><<<grid, 256, 0, st>>>(codes, absmax, nquads, N, K, W_hat);
  else
    k_dequantize8<kFp8><<<grid, 256, 0, st>>>(codes, absmax, nquads, N, K, W_hat);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Synchronous quantization that reports non-finite blocks: a counter in device
// memory of this code object (one per GPU, its address looked up once per
// device), zeroed by the quantizer's launch and read back after it. Calls are
// serialized, since every call on a device shares its counter.

namespace {
__device__ uint32_t g_nonfinite_count;
std::mutex g_count_mu;
constexpr int kMaxDevices = 64;
uint32_t* g_count_ptr[kMaxDevices];
}  // namespace

hipError_t quantize_counting(int fmt, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                             uint32_t* nonfinite_out, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_count_mu);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_count_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_nonfinite_count));
    if (e != hipSuccess) return e;
    g_count_ptr[dev] = static_cast<uint32_t*>(p);
  }
  e = launch_quantize(fmt, W, N, K, codes, absmax, g_count_ptr[dev], st);
  if (e != hipSuccess) return e;
  uint32_t host = 0;
  e = hipMemcpyAsync(&host, g_count_ptr[dev], sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  *nonfinite_out = host;
  return e;
}

}  // namespace qlora
