// Device-side building blocks shared by the gfx950 kernels of the fused QLoRA
// layer: vector types, MFMA wrappers, bf16 packing, the NF4 codebook and the
// 4-bit -> bf16 dequantizer used inside the GEMM tiles.
//
// Method: "Rev vs unsloth", fused quantized-LoRA card (a frozen 4-bit weight
// and a LoRA adapter evaluated as one layer); "Unsloth vs The Stack v2",
// quantized-base card (4-bit frozen base). The 4-bit format -- 16 NormalFloat
// levels, one fp32 absmax per 64 consecutive elements of a weight row, two
// codes per byte -- is the plainest reading of the bitsandbytes 4-bit
// checkpoints the pages load. The byte order in memory is this library's own
// (TileAddr below; inside a row, runs of 8 columns as dequant8 reads them).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlock = 64;  // weight elements per absmax

// NormalFloat-4 levels (QLoRA paper's printed table) as fp32 bit patterns.
// Index = 4-bit code. Level 7 is the exact zero.
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu, 0xbdba7871u, 0x00000000u,
    0x3da2faffu, 0x3e24cae3u, 0x3e7c04ddu, 0x3ead033au, 0x3ee1a4b8u, 0x3f1007abu, 0x3f3913b3u, 0x3f800000u};

__host__ __device__ constexpr float nf4_level(int c) { return __builtin_bit_cast(float, kNF4Bits[c]); }

// Decision threshold between level j and j+1: the midpoint, formed in double
// precision and rounded once to fp32 (evaluated at compile time).
__host__ __device__ constexpr float nf4_threshold(int j) {
  return (float)(((double)nf4_level(j) + (double)nf4_level(j + 1)) * 0.5);
}

// ---------------------------------------------------------------------------
// bf16 helpers (bit patterns in uint16/uint32; conversion is round-to-nearest-even
// by v_cvt_pk_bf16_f32)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (gfx950). Operand layouts, for lane l of a wave64:
//   32x32x16: A row i = l%32, k = 8*(l/32)+e ; B col j = l%32, k = 8*(l/32)+e
//             C/D: col j = l%32, row i = 8*(v/4) + 4*(l/32) + v%4 (v = 0..15)
//   16x16x32: A row i = l%16, k = 8*(l/16)+e ; B col j = l%16, k = 8*(l/16)+e
//             C/D: col j = l%16, row i = 4*(l/16) + v (v = 0..3)

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// LDS transposed read (ds_read_b64_tr_b16). Within each 16-lane group, lane s
// supplies the address of 4 consecutive bf16; lane i receives element i%4 of
// the chunks supplied by lanes i/4, 4+i/4, 8+i/4, 12+i/4. When lane s points
// at row (s/4), columns 4*(s%4)..+3 of a row-major tile, lane i ends up with
// rows 0..3 of column i: the tile is read column-wise.
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// 4-bit -> bf16 dequantization inside the GEMM tiles.
//
// For one (row, 64-block) the 16 possible outputs bf16(fp32(L[c] * absmax))
// are formed once (16 multiplies, 8 packed conversions) and kept as two byte
// planes (low bytes and high bytes of the 16 bf16 values, 4 dwords each).
// A code then selects its two bytes with v_perm_b32: the low three bits pick
// a byte inside an 8-byte half-table, bit 3 picks the half.

struct Nf4Lut {
  uint32_t lo[4];
  uint32_t hi[4];
};

__device__ __forceinline__ Nf4Lut make_lut(float absmax) {
  uint32_t p[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) p[q] = pack_bf16x2(nf4_level(2 * q) * absmax, nf4_level(2 * q + 1) * absmax);
  Nf4Lut t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// (a & m) | c as one v_and_or_b32. That instruction has three operands and,
// on this architecture, no literal slot and a single scalar-register read, so
// the two constants are pinned to vector registers (the empty asm only names
// the register; the compiler hoists it out of loops).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  asm("" : "+v"(m));
  asm("" : "+v"(c));
  return (a & m) | c;
}

// x holds 8 codes in the device's dword order: byte b carries element b in its
// low nibble and element b + 4 in its high nibble. Returns the 8 bf16 values
// as 4 dwords in element order: out[q] = elem 2q | elem 2q+1 << 16.
// The low and the high nibbles each select 4 table entries at once (two
// 8-entry lookups on bits 0-2, one merge on bit 3), giving the low and the
// high bytes of 4 consecutive elements; one more select per output dword
// interleaves them.
__device__ __forceinline__ u32x4 dequant8(uint32_t x, const Nf4Lut& t) {
  const uint32_t xs = x >> 4;
  const uint32_t sa = x & 0x07070707u;   // elements 0..3, bits 0-2
  const uint32_t sb = xs & 0x07070707u;  // elements 4..7
  const uint32_t ha = and_or(x >> 1, 0x04040404u, 0x03020100u);   // byte i + 4*bit3
  const uint32_t hb = and_or(xs >> 1, 0x04040404u, 0x03020100u);
  const uint32_t loa = perm(perm(t.lo[3], t.lo[2], sa), perm(t.lo[1], t.lo[0], sa), ha);
  const uint32_t hia = perm(perm(t.hi[3], t.hi[2], sa), perm(t.hi[1], t.hi[0], sa), ha);
  const uint32_t lob = perm(perm(t.lo[3], t.lo[2], sb), perm(t.lo[1], t.lo[0], sb), hb);
  const uint32_t hib = perm(perm(t.hi[3], t.hi[2], sb), perm(t.hi[1], t.hi[0], sb), hb);
  u32x4 r;
  r[0] = perm(hia, loa, 0x05010400u);  // elem0 | elem1 << 16
  r[1] = perm(hia, loa, 0x07030602u);  // elem2 | elem3 << 16
  r[2] = perm(hib, lob, 0x05010400u);  // elem4 | elem5 << 16
  r[3] = perm(hib, lob, 0x07030602u);  // elem6 | elem7 << 16
  return r;
}

// ---------------------------------------------------------------------------
// Storage order of a quantized weight [N, K]: rows in groups of 64 (the last
// group may be shorter, nr rows); inside a group, the 64-column blocks one
// after the other, each block holding the group's nr rows in order. So the
// codes of one (64-row group, 64-column block) tile are contiguous (nr rows x
// 32 bytes for NF4, x 64 bytes for 8-bit) and so are its nr block values.
// A GEMM wave that needs one block of 32 or 64 consecutive rows then reads
// one contiguous run instead of one short piece per row.
struct TileAddr {
  int64_t group_row0, nr, b, r, K;
  __host__ __device__ TileAddr(int64_t n, int64_t blk, int64_t N, int64_t K_) {
    group_row0 = n - n % 64;
    nr = (N - group_row0) < 64 ? (N - group_row0) : 64;
    b = blk;
    r = n - group_row0;
    K = K_;
  }
  // byte offset of this row's codes in block b; bb = code bytes per row and block
  __host__ __device__ int64_t code(int64_t bb) const { return group_row0 * (K / 64) * bb + (b * nr + r) * bb; }
  // index of this row's value (absmax or scale) for block b
  __host__ __device__ int64_t value() const { return group_row0 * (K / 64) + b * nr + r; }
};

// ---------------------------------------------------------------------------
// Weight formats. Every format stores one fp32 per 64-element block of a
// weight row ("absmax" array): NF4 its absmax (levels span [-1, 1]), INT8 and
// FP8 their scale s (absmax / 127, absmax / 448). The dequantized weight is
// fp32(v * that value) for the code's exact value v, then bf16 for the MFMA.

enum WFmt { kNF4 = 0, kInt8 = 1, kFp8 = 2 };

// bytes of codes per weight element x 2 (NF4: 1, 8-bit: 2)
template <int F>
constexpr int kCodeHalfBytes = F == kNF4 ? 1 : 2;

// Per (row, block) state formed once from the block's fp32 value.
template <int F>
struct WPrep;
template <>
struct WPrep<kNF4> {
  Nf4Lut lut;
};
template <>
struct WPrep<kInt8> {
  float s, o;  // scale and -128 * scale
};
template <>
struct WPrep<kFp8> {
  float s;
};

template <int F>
__device__ __forceinline__ WPrep<F> wprep(float a) {
  if constexpr (F == kNF4) {
    return WPrep<kNF4>{make_lut(a)};
  } else if constexpr (F == kInt8) {
    return WPrep<kInt8>{a, -128.0f * a};
  } else {
    return WPrep<kFp8>{a};
  }
}

// Elements 8c .. 8c+7 of a run of codes held in 16-byte registers (NF4: 8
// codes per dword, byte b = element b | element b+4 << 4; 8-bit: 4 codes per
// dword, element e in byte e) -> 8 bf16 in element order, out[q] = elem 2q | elem 2q+1 << 16.
template <int F, int NV>
__device__ __forceinline__ u32x4 wdeq8(const u32x4 (&cw)[NV], int c, const WPrep<F>& p) {
  if constexpr (F == kNF4) {
    return dequant8(cw[c >> 2][c & 3], p.lut);
  } else if constexpr (F == kInt8) {
    // byte b ^ 0x80 = q + 128 as an unsigned byte; fma(q + 128, s, -128 s)
    // rounds the exact q * s once, i.e. equals fp32(q * s)
    float v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = 2 * c + h;
      const uint32_t x = cw[d >> 2][d & 3] ^ 0x80808080u;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * h + e] = __builtin_fmaf((float)((x >> (8 * e)) & 0xffu), p.s, p.o);
    }
    return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
  } else {
    // E4M3 bytes decoded exactly to fp32 by the hardware, then one multiply
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = 2 * c + h;
      const uint32_t x = cw[d >> 2][d & 3];
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, true);
      r[2 * h] = pack_bf16x2(lo[0] * p.s, lo[1] * p.s);
      r[2 * h + 1] = pack_bf16x2(hi[0] * p.s, hi[1] * p.s);
    }
    return r;
  }
}

// The same values in fp32 (for the dequantize entry point, which exposes the
// exact operand values): element e of 4 codes in dword x.
template <int F>
__device__ __forceinline__ f32x4 wdeq4_f32(uint32_t x, const WPrep<F>& p) {
  f32x4 v;
  if constexpr (F == kInt8) {
    const uint32_t y = x ^ 0x80808080u;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf((float)((y >> (8 * e)) & 0xffu), p.s, p.o);
  } else {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, true);
    v = f32x4{lo[0] * p.s, lo[1] * p.s, hi[0] * p.s, hi[1] * p.s};
  }
  return v;
}

// ---------------------------------------------------------------------------
// Buffer resources: loads and stores through a descriptor with a hardware
// range check. An offset at or beyond num_records reads zero and drops a
// store, which replaces data-dependent branches at tile edges.

constexpr int kOff = (int)0x80000000u;  // an offset beyond every buffer's num_records
// Cache policy of the GEMM epilogues' 16-byte result stores: non-temporal (the
// lines go out of the L2 first; no workgroup of the launch reads them back).
// Whole fwd+bwd steps measured 1% faster at the attention and decoder-layer shapes.
constexpr int kStoreNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// s_waitcnt immediate: wait until at most n vector-memory ops are outstanding
// (lgkm and exp counters not waited).
constexpr unsigned waitcnt_vm(int n) { return (unsigned)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8)); }

// Workgroup barrier that waits for this wave's LDS operations only, so global
// loads issued before it stay in flight (a full __syncthreads() would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// Operand and store helpers of the GEMM tiles

// 8 bf16 of row `row` (-1: none) of a bf16 matrix with row stride ld, columns
// c..c+7 (zero at and beyond r). ALIGNED (r and ld multiples of 8, base 16-byte
// aligned): one 16-byte load; otherwise eight 2-byte loads.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 rank8(__amdgpu_buffer_rsrc_t rs, int64_t row, int64_t ld, int r, int c) {
  if (ALIGNED) {
    const int off = (row >= 0 && c < r) ? (int)((row * ld + c) * 2) : kOff;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e0 = c + 2 * q, e1 = e0 + 1;
    const int o0 = (row >= 0 && e0 < r) ? (int)((row * ld + e0) * 2) : kOff;
    const int o1 = (row >= 0 && e1 < r) ? (int)((row * ld + e1) * 2) : kOff;
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, o0, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, o1, 0, 0);
    w[q] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// s * v (8 bf16) as a sum of two bf16 vectors hi + lo (|s*v - hi - lo| <= 2^-16 |s*v|;
// lo == 0 when s is a power of two), so that s can ride on an MFMA operand.
__device__ __forceinline__ void split_scaled(const u32x4 v, float s, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = bf16_lo(v[q]) * s, b = bf16_hi(v[q]) * s;
    const uint32_t hb = pack_bf16x2(a, b);
    hi[q] = hb;
    lo[q] = pack_bf16x2(a - bf16_lo(hb), b - bf16_hi(hb));
  }
}

// Whether any lane of the wave holds a nonzero low part (two fragments' worth):
// the MFMAs of the low parts change nothing when every one is zero.
__device__ __forceinline__ bool lo_any(const u32x4 a, const u32x4 b) {
  const uint32_t v = a[0] | a[1] | a[2] | a[3] | b[0] | b[1] | b[2] | b[3];
  return __builtin_amdgcn_ballot_w64(v != 0u) != 0;
}

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t rs, int off, const float (&v)[4]) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rs, off, 0, 0);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace qlora
