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

#ifndef QLORA_GEMM_WAVES
#define QLORA_GEMM_WAVES 8
#endif
constexpr int kBI = 256, kBJ = 256, kBR = 64;
constexpr int kXS = kBR + 8;         // LDS row stride (bf16) of activation and forward weight tiles
constexpr int kWSB = kBI + 32;       // LDS row stride of the backward weight tile: 16 banks mod 64, so
                                     // each half-wave of a transposed read touches 64 distinct banks
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

template <int MODE, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW / 4, NW / 4)))
void k_qgemm(GemmArgs p) {
  constexpr bool BW = MODE >= kBwd;
  constexpr int WE = BW ? kWElemsB : kWElemsF;
  constexpr int T = 64 * NW;          // threads
  constexpr int WJ = NW / 2;          // waves along j (tokens); 2 waves along i
  constexpr int TJ = kBJ / WJ;        // j extent of one wave
  constexpr int FJ = TJ / 32;         // 32x32 fragments along j per wave
  constexpr int XC = (kBJ * kBR / 8) / T;  // 16-byte activation chunks per thread per step
  constexpr int WC = 512 / T;         // 16-byte code chunks (32 weights) per thread per step
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sW = smem;            // [2][WE]
  uint16_t* sX = smem + 2 * WE;   // [2][kXElems]

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wi = wave / WJ, wj = wave % WJ;
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

  // This thread's weight block (row, 64-block) of the tile: 256 blocks per step,
  // each split into two 16-byte halves of codes.
  const int blk = (t * WC) >> 1;       // 0..255
  const int half0 = (t * WC) & 1;      // first half handled (0 when WC == 2)

  // ---- per-thread staging registers (two sets each, used alternately by even and odd steps).
  // Loads go to clamped, always-valid addresses; out-of-range data is masked
  // only where it is consumed, so no instruction waits on a load early.
  u32x4 xa[XC], xb[XC];    // activations two steps ahead
  u32x4 ca[WC], cb[WC];    // codes: the next step's (being dequantized) and the one after
  float aa, ab;            // absmax of those blocks
  uint32_t xoka, xokb;     // bit q: activation chunk q is inside the matrix
  bool coka, cokb;         // the weight block is inside the matrix

  auto load_x = [&](int step, u32x4 (&xr)[XC], uint32_t& xok) {
    const int src = BW ? step / steps_per_src : 0;
    const int64_t r0 = (int64_t)(step - src * steps_per_src) * kBR;
    const uint16_t* act = (BW && src) ? p.act1 : p.act0;
    xok = 0;
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int c = t + T * q;
      const int row = c >> 3, col = (c & 7) * 8;
      const int64_t m = j0 + row, rc = r0 + col;
      xok |= (m < M && rc < red_len) ? (1u << q) : 0u;
      xr[q] = *reinterpret_cast<const u32x4*>(act + (m < M ? m : M - 1) * ld_act + (rc < red_len ? rc : 0));
    }
  };

  auto load_codes = [&](int step, u32x4 (&cr)[WC], float& am, bool& cok) {
    const int src = BW ? step / steps_per_src : 0;
    const int64_t r0 = (int64_t)(step - src * steps_per_src) * kBR;
    const WSrc& w = (src || (MODE == kFwdGateUp && ((blk & 127) >= 64))) ? p.w1 : p.w0;
    int64_t n, kb;
    bool ok;
    if (!BW) {
      n = (MODE == kFwdGateUp) ? i0 + 64 * (blk >> 7) + (blk & 63) : i0 + blk;
      kb = r0 / kBlock;
      ok = n < N;
    } else {
      n = r0 + (blk >> 2);
      kb = i0 / kBlock + (blk & 3);
      ok = n < N && kb * kBlock < K;
    }
    cok = ok;
    const int64_t nn = ok ? n : 0, kk = ok ? kb : 0;
    am = w.absmax[nn * (K / kBlock) + kk];  // first: the LUT needs it before the codes
    const u32x4* cp = reinterpret_cast<const u32x4*>(w.codes + nn * (K / 2) + kk * (kBlock / 2)) + half0;
#pragma unroll
    for (int h = 0; h < WC; ++h) cr[h] = cp[h];
  };

  auto store_x = [&](int buf, const u32x4 (&xr)[XC], uint32_t xok) {
    uint16_t* dstX = sX + buf * kXElems;
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int c = t + T * q;
      *reinterpret_cast<u32x4*>(dstX + (c >> 3) * kXS + (c & 7) * 8) =
          ((xok >> q) & 1u) ? xr[q] : u32x4{0, 0, 0, 0};
    }
  };

  // piece q (8 weights) of codes cr -> bf16 in the weight tile of buffer buf
  // (a block outside the matrix has a zero LUT, so its codes do not matter)
  auto dequant_piece = [&](int buf, int q, const u32x4 (&cr)[WC], const Nf4Lut& lut) {
    uint16_t* dstW = sW + buf * WE + (BW ? (blk >> 2) * kWSB + (blk & 3) * kBlock : blk * kXS) + 32 * half0;
    *reinterpret_cast<u32x4*>(dstW + 8 * q) = dequant8(cr[q >> 2][q & 3], lut);
  };

  f32x16 acc[4][FJ];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < FJ; ++b) acc[a][b] = f32x16{};

  // MFMAs of one k-substep from LDS buffer buf
  auto compute_ks = [&](int buf, int ks) {
    const uint16_t* bW = sW + buf * WE;
    const uint16_t* bX = sX + buf * kXElems;
    u32x4 av[4], bv[FJ];
#pragma unroll
    for (int fj = 0; fj < FJ; ++fj)
      bv[fj] = *reinterpret_cast<const u32x4*>(bX + (wj * TJ + 32 * fj + (lane & 31)) * kXS + 16 * ks +
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
      for (int fj = 0; fj < FJ; ++fj) acc[fi][fj] = mfma32(av[fi], bv[fj], acc[fi][fj]);
  };

  // LDS-only workgroup barrier: the register-staged global loads of later
  // steps stay in flight across it (a full __syncthreads would wait for them).
  auto lds_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
    __builtin_amdgcn_s_barrier();
  };

  // One step: MFMAs of step s from buffer s&1 while the VALU dequantizes step
  // s+1's codes (loaded a step earlier) into the other buffer; loads for step
  // s+2 are issued first, and step s+1's activations (loaded a step earlier)
  // are written to LDS last.
  auto body = [&](int step, const u32x4 (&xcur)[XC], uint32_t xokcur, u32x4 (&xnext)[XC], uint32_t& xoknext,
                  const u32x4 (&ccur)[WC], float acur, bool cokcur, u32x4 (&cnext)[WC], float& anext,
                  bool& coknext) {
    const int cur = step & 1;
    const int s2 = step + 2 < nsteps ? step + 2 : nsteps - 1;
    // codes before activations: the next step waits for the codes (in-order
    // vmcnt) while this step's activation loads may still be in flight
    load_codes(s2, cnext, anext, coknext);
    load_x(s2, xnext, xoknext);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the step
    const Nf4Lut lut = make_lut(cokcur ? acur : 0.f);
#pragma unroll
    for (int ks = 0; ks < kBR / 16; ++ks) {
      compute_ks(cur, ks);
#pragma unroll
      for (int q = ks * WC; q < (ks + 1) * WC; ++q) dequant_piece(cur ^ 1, q, ccur, lut);
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation stores wait for their loads: keep them last
    store_x(cur ^ 1, xcur, xokcur);
    lds_barrier();
  };

  // Prologue: step 0 staged into buffer 0; step 1's activations and codes in registers.
  load_codes(0, cb, ab, cokb);
  load_x(0, xb, xokb);
  load_codes(nsteps > 1 ? 1 : 0, ca, aa, coka);
  load_x(nsteps > 1 ? 1 : 0, xa, xoka);
  {
    const Nf4Lut lut = make_lut(cokb ? ab : 0.f);
#pragma unroll
    for (int q = 0; q < 4 * WC; ++q) dequant_piece(0, q, cb, lut);
  }
  store_x(0, xb, xokb);
  __syncthreads();

  for (int step = 0; step < nsteps; step += 2) {
    body(step, xa, xoka, xb, xokb, ca, aa, coka, cb, ab, cokb);
    if (step + 1 < nsteps) body(step + 1, xb, xokb, xa, xoka, cb, ab, cokb, ca, aa, coka);
  }

  // ---- epilogue: rank-r term, activation, bf16 stores
  const int jl = lane & 31;
#pragma unroll
  for (int fj = 0; fj < FJ; ++fj) {
    const int64_t m = j0 + wj * TJ + 32 * fj + jl;
    const bool m_ok = m < M;
    if (MODE == kFwd || MODE == kBwd || MODE == kBwdSwiGLU) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) {
        const int64_t ir = i0 + wi * 128 + 32 * fi + jl;  // this lane's i row for the operand load
        for (int src = 0; src < (MODE == kBwd ? p.nsrc : 1); ++src) {
          const WSrc& w = src ? p.w1 : p.w0;
          const f32x16 lt = lora_frag(ir < iext ? w.lora_i + ir * w.r : nullptr,
                                      m_ok ? w.lora_j + m * w.ldj : nullptr, w.r, lane);
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
                                    m_ok ? p.w0.lora_j + m * p.w0.ldj : nullptr, p.w0.r, lane);
        const f32x16 lu = lora_frag(i_ok ? p.w1.lora_i + ir * p.w1.r : nullptr,
                                    m_ok ? p.w1.lora_j + m * p.w1.ldj : nullptr, p.w1.r, lane);
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

constexpr int kWaves = QLORA_GEMM_WAVES;

template <int MODE>
static hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st) {
  static bool attr_done = false;  // per process; the attribute is per function
  const size_t lds = gemm_lds_bytes(MODE);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)k_qgemm<MODE, kWaves>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t ipt = (MODE == kFwdGateUp) ? 128 : kBI;
  const int64_t iext = MODE >= kBwd ? a.K : a.N;
  const int64_t nI = (iext + ipt - 1) / ipt, nJ = (a.M + kBJ - 1) / kBJ;
  if (nI * nJ == 0) return hipSuccess;
  k_qgemm<MODE, kWaves><<<(unsigned)(nI * nJ), 64 * kWaves, lds, st>>>(a);
  return hipGetLastError();
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
