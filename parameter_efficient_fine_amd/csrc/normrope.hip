// RMSNorm and rotary position embeddings (RoPE) on gfx950: the steps on
// either side of the projections ("Unsloth" wiki entry, Theory: fused
// kernels for RMSNorm and RoPE; "Unsloth vs PyTorch" video, 2:11-2:22).
// Both are HBM-bound: one pass over the data, fp32 arithmetic, one bf16
// rounding per output element.
//
// RMSNorm: one wave per row, the row held in registers (8 bf16 per lane and
// chunk, up to 16 chunks: H <= 8192), the reduction by cross-lane shuffles;
// rows longer than that are streamed twice. The weight w is frozen, so the
// backward gives dx only.
//
// RoPE ("rotate half" pairing of element i with i + d/2): one workgroup per
// 4 tokens; the d/2 angles p * base^(-2i/d) and their cos/sin are formed once
// per token in fp64 into LDS and shared by all q and k heads; each thread then
// rotates 8 pairs of a head with two 16-byte loads and stores (in place).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace qlora {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4 u, float (&f)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_lo(u[q]);
    f[2 * q + 1] = bf16_hi(u[q]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 u;
#pragma unroll
  for (int q = 0; q < 4; ++q) u[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
  return u;
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, int off, const u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// NQ > 0: the row lives in registers (lane l holds chunks l + 64q, q < NQ).
// NQ == 0: any H, the row is read twice.
template <int NQ>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                     int64_t M, int64_t H, float eps, uint16_t* __restrict__ y,
                                                     float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves only
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row * H, H * 2);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + row * H, H * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, H * 2);
  const int64_t nch = H / 8;
  float ss = 0.f;
  if constexpr (NQ > 0) {
    u32x4 v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t c = lane + 64 * q;
      v[q] = ld16(rx, c < nch ? (int)(c * 16) : kOff);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float f[8];
      unpack8(v[q], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)H + eps);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t c = lane + 64 * q;
      const int off = c < nch ? (int)(c * 16) : kOff;
      float f[8], g[8];
      unpack8(v[q], f);
      unpack8(ld16(rw, off), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = g[e] * (f[e] * r);
      st16(ry, off, pack8(f));
    }
    if (lane == 0) rstd[row] = r;
  } else {
    for (int64_t c = lane; c < nch; c += 64) {
      float f[8];
      unpack8(ld16(rx, (int)(c * 16)), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)H + eps);
    for (int64_t c = lane; c < nch; c += 64) {
      float f[8], g[8];
      unpack8(ld16(rx, (int)(c * 16)), f);
      unpack8(ld16(rw, (int)(c * 16)), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = g[e] * (f[e] * r);
      st16(ry, (int)(c * 16), pack8(f));
    }
    if (lane == 0) rstd[row] = r;
  }
}

// dx = rstd * (g - n * mean(g * n)),  g = w * dy,  n = x * rstd
template <int NQ>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w, const float* __restrict__ rstd,
                                                     int64_t M, int64_t H, uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row * H, H * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dy + row * H, H * 2);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(dx + row * H, H * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, H * 2);
  const int64_t nch = H / 8;
  const float r = rstd[row];
  float dot = 0.f;
  if constexpr (NQ > 0) {
    u32x4 vx[NQ], vd[NQ], vw[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t c = lane + 64 * q;
      const int off = c < nch ? (int)(c * 16) : kOff;
      vx[q] = ld16(rx, off);
      vd[q] = ld16(rd, off);
      vw[q] = ld16(rw, off);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float fx[8], fd[8], fw[8];
      unpack8(vx[q], fx);
      unpack8(vd[q], fd);
      unpack8(vw[q], fw);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += (fw[e] * fd[e]) * (fx[e] * r);
    }
    const float mean = wave_sum(dot) / (float)H;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t c = lane + 64 * q;
      const int off = c < nch ? (int)(c * 16) : kOff;
      float fx[8], fd[8], fw[8];
      unpack8(vx[q], fx);
      unpack8(vd[q], fd);
      unpack8(vw[q], fw);
#pragma unroll
      for (int e = 0; e < 8; ++e) fx[e] = r * (fw[e] * fd[e] - (fx[e] * r) * mean);
      st16(ro, off, pack8(fx));
    }
  } else {
    for (int64_t c = lane; c < nch; c += 64) {
      float fx[8], fd[8], fw[8];
      unpack8(ld16(rx, (int)(c * 16)), fx);
      unpack8(ld16(rd, (int)(c * 16)), fd);
      unpack8(ld16(rw, (int)(c * 16)), fw);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += (fw[e] * fd[e]) * (fx[e] * r);
    }
    const float mean = wave_sum(dot) / (float)H;
    for (int64_t c = lane; c < nch; c += 64) {
      float fx[8], fd[8], fw[8];
      unpack8(ld16(rx, (int)(c * 16)), fx);
      unpack8(ld16(rd, (int)(c * 16)), fd);
      unpack8(ld16(rw, (int)(c * 16)), fw);
#pragma unroll
      for (int e = 0; e < 8; ++e) fx[e] = r * (fw[e] * fd[e] - (fx[e] * r) * mean);
      st16(ro, (int)(c * 16), pack8(fx));
    }
  }
}

constexpr int kRopeMaxHalf = 512;  // d/2 <= 512
constexpr int kRopeTok = 4;        // tokens per workgroup

// In-place rotation of the q heads [M, hq*d] and k heads [M, hk*d] of
// kRopeTok tokens by their positions; sign = -1 rotates back (the backward).
__global__ __launch_bounds__(256) void k_rope(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                              const int32_t* __restrict__ pos, int64_t M, int hq, int hk, int d,
                                              double base, float sign) {
  __shared__ float cs[kRopeTok][kRopeMaxHalf], sn[kRopeTok][kRopeMaxHalf];
  const int64_t m0 = (int64_t)blockIdx.x * kRopeTok;
  const int half = d / 2;
  for (int idx = threadIdx.x; idx < kRopeTok * half; idx += 256) {
    const int tk = idx / half, i = idx - tk * half;
    const double p = m0 + tk < M ? (double)pos[m0 + tk] : 0.0;
    const double a = p * pow(base, -2.0 * i / d);
    double s, c;
    sincos(a, &s, &c);
    cs[tk][i] = (float)c;
    sn[tk][i] = sign * (float)s;
  }
  __syncthreads();
  const int groups = half / 8;  // 8 pairs per work item
  const int per_tok = (hq + hk) * groups;
  const int64_t ntok = (M - m0) < kRopeTok ? (M - m0) : kRopeTok;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + m0 * (int64_t)hq * d, ntok * hq * d * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + m0 * (int64_t)hk * d, ntok * hk * d * 2);
  for (int it = threadIdx.x; it < kRopeTok * per_tok; it += 256) {
    const int tk = it / per_tok, rem = it - tk * per_tok;
    const int head = rem / groups, g = rem - head * groups;
    const bool isq = head < hq;
    const int hh = isq ? head : head - hq;
    // rows past M fall outside the resources: loads read zero, stores are dropped
    const int off_lo = ((tk * (isq ? hq : hk) + hh) * d + 8 * g) * 2, off_hi = off_lo + half * 2;
    const __amdgpu_buffer_rsrc_t r = isq ? rq : rk;
    float lo[8], hi[8];
    unpack8(ld16(r, off_lo), lo);
    unpack8(ld16(r, off_hi), hi);
    float olo[8], ohi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = cs[tk][8 * g + e], s = sn[tk][8 * g + e];
      olo[e] = lo[e] * c - hi[e] * s;
      ohi[e] = hi[e] * c + lo[e] * s;
    }
    st16(r, off_lo, pack8(olo));
    st16(r, off_hi, pack8(ohi));
  }
}

template <class F>
hipError_t by_chunks(int64_t H, F&& f) {
  const int64_t nq = (H / 8 + 63) / 64;
  if (nq <= 1) return f(std::integral_constant<int, 1>{});
  if (nq <= 2) return f(std::integral_constant<int, 2>{});
  if (nq <= 4) return f(std::integral_constant<int, 4>{});
  if (nq <= 8) return f(std::integral_constant<int, 8>{});
  if (nq <= 16) return f(std::integral_constant<int, 16>{});
  return f(std::integral_constant<int, 0>{});
}

}  // namespace

hipError_t launch_rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, float eps, uint16_t* y,
                              float* rstd, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const unsigned grid = (unsigned)((M + 3) / 4);
  return by_chunks(H, [&](auto nq) {
    k_rmsnorm_fwd<decltype(nq)::value><<<grid, 256, 0, st>>>(x, w, M, H, eps, y, rstd);
    return hipGetLastError();
  });
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd, int64_t M,
                              int64_t H, uint16_t* dx, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const unsigned grid = (unsigned)((M + 3) / 4);
  return by_chunks(H, [&](auto nq) {
    k_rmsnorm_bwd<decltype(nq)::value><<<grid, 256, 0, st>>>(dy, x, w, rstd, M, H, dx);
    return hipGetLastError();
  });
}

// cos/sin of every (position, frequency), formed as k_rope forms them (angle and
// sin/cos in fp64, rounded once to fp32): table[(p * d/2 + i) * 2 + 0 / 1] =
// cos / sin of p * base^(-2i/d). Read by the q/k projection GEMM's RoPE epilogue.
__global__ __launch_bounds__(256) void k_rope_table(int d, double base, int64_t n, float* __restrict__ table) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int half = d / 2;
  const int64_t p = idx / half;
  const int i = (int)(idx - p * half);
  const double a = (double)p * pow(base, -2.0 * i / d);
  double sv, cv;
  sincos(a, &sv, &cv);
  reinterpret_cast<f32x2*>(table)[idx] = f32x2{(float)cv, (float)sv};
}

hipError_t launch_rope_table(int d, double base, int64_t max_pos, float* table, hipStream_t st) {
  const int64_t n = max_pos * (d / 2);
  if (n == 0) return hipSuccess;
  k_rope_table<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(d, base, n, table);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t M, int hq, int hk, int d, double base,
                       bool inverse, hipStream_t st) {
  if (M == 0 || hq + hk == 0) return hipSuccess;
  k_rope<<<(unsigned)((M + kRopeTok - 1) / kRopeTok), 256, 0, st>>>(q, k, pos, M, hq, hk, d, base,
                                                                   inverse ? -1.f : 1.f);
  return hipGetLastError();
}

}  // namespace qlora
