// Fused 4-bit-dequant GEMMs of the QLoRA layer on gfx950 MFMA.
//
// "Rev vs unsloth", fused quantized-LoRA card: the quantized weight product
// and the LoRA term are one operation, with no dequantized copy of the weight
// in HBM. "Unsloth" wiki entry, Theory: hand-derived backward for the LoRA
// path; fused SwiGLU block with intermediates kept on chip.
//
//   forward  (NT):  Y  = X . What^T + s . Z . B^T        (Z = X.A^T from skinny_nt)
//   backward (NN):  dX = dY . What  + s . G . A          (G = dY.B  from skinny_nt)
//
// One workgroup = 4 waves (2 x 2) computing a 256 x 256 output tile with
// 32x32x16 bf16 MFMAs and fp32 accumulators (128 x 128 per wave). The MFMA
// "i" side is the weight dimension (the contiguous dimension of the output),
// the "j" side is tokens, so each lane owns 4 consecutive output columns.
// Each 64-wide reduction step:
//   * activations: 256 rows x 64 bf16 staged through LDS (double-buffered);
//   * weight: 4-bit codes + absmax loaded from HBM, dequantized by the VALU
//     into a bf16 LDS tile (one thread = one (row, 64-block) of codes);
//     forward reads it row-wise (ds_read_b128), backward column-wise with
//     ds_read_b64_tr_b16 because the reduction runs over the weight's rows.
// The rank-r term is added to the accumulators in the epilogue from the
// skinny tensors (Z or G) and the adapter (B or A^T): the N x K product B.A
// is never formed and no second output is written.
#include "common.hpp"
#include "internal.hpp"

namespace qlora {

enum GemmMode { kFwd = 0, kFwdGateUp = 1, kBwd = 2, kBwdSwiGLU = 3 };

struct GemmArgs {
  const uint16_t* act0;  // fwd: X [M,K]; bwd: dY [M,N] (gate part of the concat reduction)
  const uint16_t* act1;  // bwd concat: second dY [M,N]
  WSrc w0, w1;           // weight sources (gate/up, or the concatenated reduction)
  int64_t M, K, N;
  int nsrc;
  uint16_t* out0;  // Y | g | dX | dg
  uint16_t* out1;  // u | du
  uint16_t* out2;  // h
  const uint16_t* aux0;  // swiglu backward: saved g [M, N_down_in]
  const uint16_t* aux1;  // swiglu backward: saved u
};

constexpr int kBI = 256, kBJ = 256, kBR = 64;
constexpr int kXS = kBR + 8;         // LDS row stride (bf16) of activation and forward weight tiles
constexpr int kWSB = kBI + 16;       // LDS row stride of the backward weight tile
constexpr int kXElems = kBJ * kXS;
constexpr int kWElemsF = kBI * kXS;
constexpr int kWElemsB = kBR * kWSB;

constexpr size_t gemm_lds_bytes(int mode) {
  return (size_t)2 * 2 * (kXElems + (mode >= kBwd ? kWElemsB : kWElemsF));
}

// 8 bf16 of a rank-r row (zero beyond r) as one MFMA operand.
__device__ __forceinline__ u32x4 load_rank8(const uint16_t* row, int r, int c) {
  if ((r & 7) == 0) {
    if (c < r) return *reinterpret_cast<const u32x4*>(row + c);
    return u32x4{0, 0, 0, 0};
  }
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = (c + 2 * q < r) ? row[c + 2 * q] : 0u;
    const uint32_t hi = (c + 2 * q + 1 < r) ? row[c + 2 * q + 1] : 0u;
    w[q] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// s * (rows_i . rows_j^T) for one 32x32 fragment: lane's i row and j row pointers
// (null = outside the matrix).
__device__ __forceinline__ f32x16 lora_frag(const uint16_t* irow, const uint16_t* jrow, int r, int lane) {
  f32x16 t = {};
  const int c0 = 8 * (lane >> 5);
  for (int rr = 0; rr < r; rr += 16) {
    const u32x4 a = irow ? load_rank8(irow, r, rr + c0) : u32x4{0, 0, 0, 0};
    const u32x4 b = jrow ? load_rank8(jrow, r, rr + c0) : u32x4{0, 0, 0, 0};
    t = mfma32(a, b, t);
  }
  return t;
}

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void k_qgemm(GemmArgs p) {
  constexpr bool BW = MODE >= kBwd;
  constexpr int WE = BW ? kWElemsB : kWElemsF;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sW = smem;            // [2][WE]
  uint16_t* sX = smem + 2 * WE;   // [2][kXElems]

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t M = p.M, K = p.K, N = p.N;
  // i extent: fwd -> N (gate/up: 128 weight rows of each source per tile), bwd -> K
  const int64_t ipt = (MODE == kFwdGateUp) ? 128 : kBI;
  const int64_t iext = BW ? K : N;
  const int64_t nJ = (M + kBJ - 1) / kBJ;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * ipt, j0 = jt * kBJ;
  const int64_t ld_act = BW ? N : K;              // row length of the activation operand
  const int64_t red_len = BW ? N : K;             // reduction length per source
  const int steps_per_src = (int)((red_len + kBR - 1) / kBR);
  const int nsteps = steps_per_src * (BW ? p.nsrc : 1);

  // ---- per-thread staging registers
  u32x4 xr[8];
  u32x4 cr[2];
  float am;

  auto load_stage = [&](int step) {
    const int src = BW ? step / steps_per_src : 0;
    const int64_t r0 = (int64_t)(step - src * steps_per_src) * kBR;
    const uint16_t* act = (BW && src) ? p.act1 : p.act0;
    const WSrc& w = (src || (MODE == kFwdGateUp && ((t & 127) >= 64))) ? p.w1 : p.w0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = t + 256 * q;
      const int row = c >> 3, col = (c & 7) * 8;
      const int64_t m = j0 + row, rc = r0 + col;
      xr[q] = (m < M && rc < red_len) ? *reinterpret_cast<const u32x4*>(act + m * ld_act + rc) : u32x4{0, 0, 0, 0};
    }
    int64_t n, kb;
    bool ok;
    if (!BW) {
      n = (MODE == kFwdGateUp) ? i0 + 64 * (t >> 7) + (t & 63) : i0 + t;
      kb = r0 / kBlock;
      ok = n < N;
    } else {
      n = r0 + (t >> 2);
      kb = i0 / kBlock + (t & 3);
      ok = n < N && kb * kBlock < K;
    }
    if (ok) {
      const u32x4* cp = reinterpret_cast<const u32x4*>(w.codes + n * (K / 2) + kb * (kBlock / 2));
      cr[0] = cp[0];
      cr[1] = cp[1];
      am = w.absmax[n * (K / kBlock) + kb];
    } else {
      cr[0] = u32x4{0, 0, 0, 0};
      cr[1] = u32x4{0, 0, 0, 0};
      am = 0.f;
    }
  };

  auto store_stage = [&](int buf) {
    const Nf4Lut lut = make_lut(am);
    uint16_t* dstW = sW + buf * WE + (BW ? (t >> 2) * kWSB + (t & 3) * kBlock : t * kXS);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t codes8 = cr[q >> 2][q & 3];
      *reinterpret_cast<u32x4*>(dstW + 8 * q) = dequant8(codes8, lut);
    }
    uint16_t* dstX = sX + buf * kXElems;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = t + 256 * q;
      *reinterpret_cast<u32x4*>(dstX + (c >> 3) * kXS + (c & 7) * 8) = xr[q];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  auto compute = [&](int buf) {
    const uint16_t* bW = sW + buf * WE;
    const uint16_t* bX = sX + buf * kXElems;
#pragma unroll
    for (int ks = 0; ks < kBR / 16; ++ks) {
      u32x4 av[4], bv[4];
#pragma unroll
      for (int fj = 0; fj < 4; ++fj)
        bv[fj] = *reinterpret_cast<const u32x4*>(bX + (wj * 128 + 32 * fj + (lane & 31)) * kXS + 16 * ks +
                                                 8 * (lane >> 5));
      if (!BW) {
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
          av[fi] = *reinterpret_cast<const u32x4*>(bW + (wi * 128 + 32 * fi + (lane & 31)) * kXS + 16 * ks +
                                                   8 * (lane >> 5));
      } else {
        const int g = lane >> 4, s = lane & 15;
        const int rowb = 16 * ks + 8 * (g >> 1) + (s >> 2);
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
          const int col = wi * 128 + 32 * fi + 16 * (g & 1) + 4 * (s & 3);
          const u32x2 lo = lds_read_tr(bW + rowb * kWSB + col);
          const u32x2 hi = lds_read_tr(bW + (rowb + 4) * kWSB + col);
          av[fi] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj) acc[fi][fj] = mfma32(av[fi], bv[fj], acc[fi][fj]);
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) load_stage(step + 1);
    compute(cur);
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: rank-r term, activation, bf16 stores
  const int jl = lane & 31;
#pragma unroll
  for (int fj = 0; fj < 4; ++fj) {
    const int64_t m = j0 + wj * 128 + 32 * fj + jl;
    const bool m_ok = m < M;
    if (MODE == kFwd || MODE == kBwd || MODE == kBwdSwiGLU) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) {
        const int64_t ir = i0 + wi * 128 + 32 * fi + jl;  // this lane's i row for the operand load
        for (int src = 0; src < (MODE == kBwd ? p.nsrc : 1); ++src) {
          const WSrc& w = src ? p.w1 : p.w0;
          const f32x16 lt = lora_frag(ir < iext ? w.lora_i + ir * w.r : nullptr,
                                      m_ok ? w.lora_j + m * w.r : nullptr, w.r, lane);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[fi][fj][v] += w.s * lt[v];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t ic = i0 + wi * 128 + 32 * fi + 8 * q + 4 * (lane >> 5);  // first of 4 output columns
          if (!m_ok || ic >= iext) continue;
          float a4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) a4[e] = acc[fi][fj][4 * q + e];
          const int64_t o = m * iext + ic;
          if (MODE == kBwdSwiGLU) {
            const u32x2 gw = *reinterpret_cast<const u32x2*>(p.aux0 + o);
            const u32x2 uw = *reinterpret_cast<const u32x2*>(p.aux1 + o);
            float gv[4] = {bf16_lo(gw[0]), bf16_hi(gw[0]), bf16_lo(gw[1]), bf16_hi(gw[1])};
            float uv[4] = {bf16_lo(uw[0]), bf16_hi(uw[0]), bf16_lo(uw[1]), bf16_hi(uw[1])};
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = sigmoid_f(gv[e]);
              dg[e] = a4[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
              du[e] = a4[e] * gv[e] * sg;
            }
            *reinterpret_cast<u32x2*>(p.out0 + o) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
            *reinterpret_cast<u32x2*>(p.out1 + o) = u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
          } else {
            *reinterpret_cast<u32x2*>(p.out0 + o) = u32x2{pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3])};
          }
        }
      }
    } else {  // kFwdGateUp: fragments 0,1 = gate rows, 2,3 = up rows of the same 64 output columns
#pragma unroll
      for (int fi = 0; fi < 2; ++fi) {
        const int64_t ir = i0 + wi * 64 + 32 * fi + jl;
        const bool i_ok = ir < N;
        const f32x16 lg = lora_frag(i_ok ? p.w0.lora_i + ir * p.w0.r : nullptr,
                                    m_ok ? p.w0.lora_j + m * p.w0.r : nullptr, p.w0.r, lane);
        const f32x16 lu = lora_frag(i_ok ? p.w1.lora_i + ir * p.w1.r : nullptr,
                                    m_ok ? p.w1.lora_j + m * p.w1.r : nullptr, p.w1.r, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t ic = i0 + wi * 64 + 32 * fi + 8 * q + 4 * (lane >> 5);
          if (!m_ok || ic >= N) continue;
          float gv[4], uv[4], hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[e] = acc[fi][fj][4 * q + e] + p.w0.s * lg[4 * q + e];
            uv[e] = acc[fi + 2][fj][4 * q + e] + p.w1.s * lu[4 * q + e];
            hv[e] = gv[e] * sigmoid_f(gv[e]) * uv[e];
          }
          const int64_t o = m * N + ic;
          *reinterpret_cast<u32x2*>(p.out0 + o) = u32x2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
          *reinterpret_cast<u32x2*>(p.out1 + o) = u32x2{pack_bf16x2(uv[0], uv[1]), pack_bf16x2(uv[2], uv[3])};
          *reinterpret_cast<u32x2*>(p.out2 + o) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        }
      }
    }
  }
}

template <int MODE>
static hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st) {
  static bool attr_done = false;  // per process; the attribute is per function
  const size_t lds = gemm_lds_bytes(MODE);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)k_qgemm<MODE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t ipt = (MODE == kFwdGateUp) ? 128 : kBI;
  const int64_t iext = MODE >= kBwd ? a.K : a.N;
  const int64_t nI = (iext + ipt - 1) / ipt, nJ = (a.M + kBJ - 1) / kBJ;
  if (nI * nJ == 0) return hipSuccess;
  k_qgemm<MODE><<<(unsigned)(nI * nJ), 256, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, uint16_t* Y, hipStream_t st) {
  GemmArgs a{};
  a.act0 = X;
  a.w0 = w;
  a.w1 = w;
  a.M = M, a.K = K, a.N = N, a.nsrc = 1;
  a.out0 = Y;
  return launch_qgemm<kFwd>(a, st);
}

hipError_t launch_gemm_fwd_gateup(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc wg, WSrc wu, uint16_t* g,
                                  uint16_t* u, uint16_t* h, hipStream_t st) {
  GemmArgs a{};
  a.act0 = X;
  a.w0 = wg;
  a.w1 = wu;
  a.M = M, a.K = K, a.N = N, a.nsrc = 2;
  a.out0 = g, a.out1 = u, a.out2 = h;
  return launch_qgemm<kFwdGateUp>(a, st);
}

hipError_t launch_gemm_bwd(const uint16_t* dY0, WSrc w0, const uint16_t* dY1, WSrc w1, int64_t M, int64_t K,
                           int64_t N, uint16_t* dX, hipStream_t st) {
  GemmArgs a{};
  a.act0 = dY0;
  a.act1 = dY1 ? dY1 : dY0;
  a.w0 = w0;
  a.w1 = dY1 ? w1 : w0;
  a.M = M, a.K = K, a.N = N, a.nsrc = dY1 ? 2 : 1;
  a.out0 = dX;
  return launch_qgemm<kBwd>(a, st);
}

hipError_t launch_gemm_bwd_swiglu(const uint16_t* dY, WSrc w, int64_t M, int64_t K, int64_t N, const uint16_t* g,
                                  const uint16_t* u, uint16_t* dg, uint16_t* du, hipStream_t st) {
  GemmArgs a{};
  a.act0 = dY;
  a.act1 = dY;
  a.w0 = w;
  a.w1 = w;
  a.M = M, a.K = K, a.N = N, a.nsrc = 1;
  a.out0 = dg, a.out1 = du;
  a.aux0 = g, a.aux1 = u;
  return launch_qgemm<kBwdSwiGLU>(a, st);
}

}  // namespace qlora
