// Skinny rank-r products of the LoRA path (gfx950).
//
// "Unsloth vs PyTorch" video, 1:35-2:00: the adapters are skinny (rank 8 to
// 128) against 4096-wide weights, so the products are bracketed to keep every
// intermediate M x r (or r x K) and never form the N x K matrix B.A.
//   skinny_nt:  Z = X.A^T  and  G = dY.B          ([M,Kd] x [r,Kd]^T -> [M,r])
//   skinny_tn:  dA = s.G^T.X  and  dB^T = s.Z^T.dY  ([M,r]^T x [M,Kd] -> [r,Kd])
// Both read their big operand exactly once and are HBM-bound.
#include "common.hpp"
#include "internal.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// skinny_nt: 16 rows of `in` per workgroup, 4 waves interleaved over the
// 32-wide k steps, MFMA 16x16x32, partial sums combined through LDS.
// RP = adapter rows (r1 + r2) rounded up to 16.

template <int RP>
__global__ __launch_bounds__(256) void k_skinny_nt(const uint16_t* __restrict__ in, int64_t M, int64_t Kd,
                                                   const uint16_t* __restrict__ ad1, int r1,
                                                   uint16_t* __restrict__ out1, const uint16_t* __restrict__ ad2,
                                                   int r2, uint16_t* __restrict__ out2) {
  constexpr int NF = RP / 16;
  __shared__ float red[4][16][RP + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int R = r1 + r2;
  const int64_t row = m0 + (lane & 15);
  const bool row_ok = row < M;
  const int kofs = 8 * (lane >> 4);
  const int64_t nsteps = (Kd + 31) / 32;  // a ragged last step is masked per lane (Kd % 8 == 0)

  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // adapter row pointers for this lane's j within each 16-row fragment
  const uint16_t* adp[NF];
  bool ad_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int j = 16 * f + (lane & 15);
    ad_ok[f] = j < R;
    adp[f] = j < r1 ? ad1 + (int64_t)j * Kd : (j < R ? ad2 + (int64_t)(j - r1) * Kd : ad1);
  }
  const uint16_t* inp = in + (row_ok ? row : 0) * Kd;

  constexpr int U = 4;
  for (int64_t s0 = wave; s0 < nsteps; s0 += 4 * U) {
    u32x4 a[U];
    u32x4 b[U][NF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + 4 * u;
      const int64_t k = s * 32 + kofs;
      const bool ok = s < nsteps && k < Kd;
      a[u] = (ok && row_ok) ? *reinterpret_cast<const u32x4*>(inp + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int f = 0; f < NF; ++f)
        b[u][f] = (ok && ad_ok[f]) ? *reinterpret_cast<const u32x4*>(adp[f] + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = mfma16(a[u], b[u][f], acc[f]);
  }
  // C layout: col j = lane%16 (adapter row), row i = 4*(lane/16) + v (token row)
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][16 * f + (lane & 15)] = acc[f][v];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * R; idx += 256) {
    const int i = idx / R, j = idx - i * R;
    const int64_t m = m0 + i;
    if (m >= M) continue;
    const float v = (red[0][i][j] + red[1][i][j]) + (red[2][i][j] + red[3][i][j]);
    const uint16_t h = __builtin_bit_cast(uint16_t, (__bf16)v);
    if (j < r1)
      out1[m * r1 + j] = h;
    else
      out2[m * r2 + (j - r1)] = h;
  }
}

hipError_t launch_skinny_nt(const uint16_t* in, int64_t M, int64_t Kd, const uint16_t* ad1, int r1, uint16_t* out1,
                            const uint16_t* ad2, int r2, uint16_t* out2, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int R = r1 + (ad2 ? r2 : 0);
  if (!ad2) r2 = 0;
  const unsigned grid = (unsigned)((M + 15) / 16);
#define QL_NT(RPV) \
  k_skinny_nt<RPV><<<grid, 256, 0, st>>>(in, M, Kd, ad1, r1, out1, ad2, r2, out2)
  if (R <= 16)
    QL_NT(16);
  else if (R <= 32)
    QL_NT(32);
  else if (R <= 64)
    QL_NT(64);
  else if (R <= 128)
    QL_NT(128);
  else if (R <= 256)
    QL_NT(256);
  else
    return hipErrorInvalidValue;
#undef QL_NT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// skinny_tn: part[s, j, k] = sum over the rows m of split s of P[m, j] * Q[m, k].
// Workgroup = 256 columns of Q x one split of the rows; 4 waves x 64 columns.
// Both operands are staged row-major in LDS and read column-wise with
// ds_read_b64_tr_b16 so that each lane holds 8 consecutive rows (the reduction).

constexpr int kTnCols = 256;
constexpr int kTnRows = 32;  // rows of P/Q per step (one MFMA reduction)
constexpr int kTnQStride = kTnCols + 16;  // bf16 elements per LDS row (bank spread)

template <int RP>
__global__ __launch_bounds__(256) void k_skinny_tn(const uint16_t* __restrict__ P, int r,
                                                   const uint16_t* __restrict__ Q, int64_t M, int64_t Kd,
                                                   int64_t rows_per_split, float* __restrict__ part) {
  constexpr int NJ = RP / 16;
  constexpr int PS = RP + 16;  // P tile row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kTnRows * kTnQStride];
  __shared__ __attribute__((aligned(16))) uint16_t sP[kTnRows * PS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kTnCols;
  const int split = blockIdx.y;
  const int64_t mbeg = (int64_t)split * rows_per_split;
  const int64_t mend = mbeg + rows_per_split < M ? mbeg + rows_per_split : M;

  f32x4 acc[NJ][4];
#pragma unroll
  for (int a = 0; a < NJ; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, s = lane & 15;
  for (int64_t m0 = mbeg; m0 < mend; m0 += kTnRows) {
    // stage Q tile [32 rows x 256 cols]: 1024 chunks of 16 B, 4 per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = t + 256 * q;
      const int rr = c >> 5, cc = (c & 31) * 8;
      const int64_t m = m0 + rr, k = k0 + cc;
      u32x4 v = {0, 0, 0, 0};
      if (m < mend && k < Kd) v = *reinterpret_cast<const u32x4*>(Q + m * Kd + k);
      *reinterpret_cast<u32x4*>(&sQ[rr * kTnQStride + cc]) = v;
    }
    // stage P tile [32 rows x RP cols] (zero beyond r and beyond the split)
    for (int e = t; e < kTnRows * RP; e += 256) {
      const int rr = e / RP, j = e - rr * RP;
      const int64_t m = m0 + rr;
      sP[rr * PS + j] = (m < mend && j < r) ? P[m * r + j] : (uint16_t)0;
    }
    __syncthreads();
    // operands: lane (group g, index s) -> rows 8g..8g+7, column s of a 16-wide fragment
    u32x4 pa[NJ], qb[4];
#pragma unroll
    for (int a = 0; a < NJ; ++a) {
      const u32x2 lo = lds_read_tr(&sP[(8 * g + (s >> 2)) * PS + 16 * a + 4 * (s & 3)]);
      const u32x2 hi = lds_read_tr(&sP[(8 * g + 4 + (s >> 2)) * PS + 16 * a + 4 * (s & 3)]);
      pa[a] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int col = 64 * wave + 16 * b + 4 * (s & 3);
      const u32x2 lo = lds_read_tr(&sQ[(8 * g + (s >> 2)) * kTnQStride + col]);
      const u32x2 hi = lds_read_tr(&sQ[(8 * g + 4 + (s >> 2)) * kTnQStride + col]);
      qb[b] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int a = 0; a < NJ; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma16(pa[a], qb[b], acc[a][b]);
    __syncthreads();
  }
  // C layout: col (k) = lane%16, row (j) = 4*(lane/16) + v
  float* dst = part + (int64_t)split * r * Kd;
#pragma unroll
  for (int a = 0; a < NJ; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t k = k0 + 64 * wave + 16 * b + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * a + 4 * (lane >> 4) + v;
        if (j < r && k < Kd) dst[(int64_t)j * Kd + k] = acc[a][b][v];
      }
    }
}

int skinny_tn_splits(int64_t M, int64_t Kd) {
  // enough workgroups to cover the chip, with >= 256 rows per split
  const int64_t col_tiles = (Kd + kTnCols - 1) / kTnCols;
  int64_t splits = (1024 + col_tiles - 1) / col_tiles;
  const int64_t max_by_rows = (M + 255) / 256;
  if (splits > max_by_rows) splits = max_by_rows;
  if (splits < 1) splits = 1;
  if (splits > 256) splits = 256;
  return (int)splits;
}

hipError_t launch_skinny_tn(const uint16_t* P, int r, const uint16_t* Q, int64_t M, int64_t Kd, float* part,
                            int splits, hipStream_t st) {
  int64_t rows = (M + splits - 1) / splits;
  rows = (rows + kTnRows - 1) / kTnRows * kTnRows;
  dim3 grid((unsigned)((Kd + kTnCols - 1) / kTnCols), (unsigned)splits);
#define QL_TN(RPV) k_skinny_tn<RPV><<<grid, 256, 0, st>>>(P, r, Q, M, Kd, rows, part)
  if (r <= 16)
    QL_TN(16);
  else if (r <= 32)
    QL_TN(32);
  else if (r <= 64)
    QL_TN(64);
  else if (r <= 128)
    QL_TN(128);
  else if (r <= 256)
    QL_TN(256);
  else
    return hipErrorInvalidValue;
#undef QL_TN
  return hipGetLastError();
}

// out = s * sum_splits part, summed in split order (deterministic).
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, int splits, int r, int64_t Kd,
                                                       float s, float* __restrict__ out, int transposed) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)r * Kd;
  if (idx >= total) return;
  float acc = 0.f;
  for (int p = 0; p < splits; ++p) acc += part[(int64_t)p * total + idx];
  acc *= s;
  if (transposed) {
    const int64_t j = idx / Kd, k = idx - j * Kd;
    out[k * r + j] = acc;
  } else {
    out[idx] = acc;
  }
}

hipError_t launch_reduce_splits(const float* part, int splits, int r, int64_t Kd, float s, float* out, bool transposed,
                                hipStream_t st) {
  const int64_t total = (int64_t)r * Kd;
  if (total == 0) return hipSuccess;
  k_reduce_splits<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(part, splits, r, Kd, s, out, transposed ? 1 : 0);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_zero_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                        uint16_t* __restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * C) return;
  const int64_t c = idx / R, rr = idx - c * R;
  dst[idx] = src[rr * C + c];
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, hipStream_t st) {
  if (R * C == 0) return hipSuccess;
  k_transpose_bf16<<<(unsigned)((R * C + 255) / 256), 256, 0, st>>>(src, R, C, dst);
  return hipGetLastError();
}

}  // namespace qlora
