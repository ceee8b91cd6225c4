// Forward fused-dequant GEMM of the QLoRA layer on gfx950:
//   Y = X . What^T + s . Z . B^T          (Z = X.A^T from skinny_nt)
// and the SwiGLU gate/up variant: g, u, h = silu(g) * u in one pass.
//
// "Rev vs unsloth", fused quantized-LoRA card: the 4-bit weight product and
// the LoRA term are one operation with no dequantized weight in HBM.
//
// Design (one workgroup = 4 waves, 256 weight rows x 256 tokens, K in steps of 64):
//   * each wave owns 64 weight rows (two 32-row MFMA fragments) and all 256
//     tokens (eight fragments), so a weight row is used by exactly one wave:
//     its 4-bit codes are loaded from HBM and dequantized by the VALU straight
//     into MFMA A-operand registers -- the weight never touches LDS;
//   * within a 64-wide step, lane half h = lane/32 takes k in [32h, 32h+32) and
//     substep ks the 8 values 32h+8ks..+7 (a fixed permutation of the
//     reduction order, applied to both operands), so one 16-byte load of codes
//     per row feeds all four substeps and dequant8() yields operands directly;
//   * only the activation tile (256 x 64 bf16 = 32 KB) goes through LDS: it is
//     copied by buffer_load ... lds (no VGPR staging, no ds_write) into a ring
//     of four buffers, XOR-swizzled so the fragment reads are conflict-free;
//   * the loop is software-pipelined over 16-wide substeps: while 16 MFMAs run,
//     the next substep's fragments are read and dequantized; loads run two
//     steps ahead; instruction issue is interleaved with sched_group_barrier.
// Out-of-range rows and tokens are handled by the buffer range check (loads
// return zero, stores are dropped), so the kernel has no data-dependent branch
// and the 256 accumulators per lane stay in AGPRs.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

// This source is compiled once per weight format (QL_WFMT: 0 NF4, 1 INT8,
// 2 FP8); each object defines the launchers of its format's namespace.
#ifndef QL_WFMT
#define QL_WFMT 0
#endif
#if QL_WFMT == 0
#define QL_FMT_NS f0
#elif QL_WFMT == 1
#define QL_FMT_NS f1
#elif QL_WFMT == 2
#define QL_FMT_NS f2
#else
#error "QL_WFMT must be 0, 1 or 2"
#endif

namespace qlora {

namespace {

constexpr int kFmt = QL_WFMT;
constexpr int kNV = kFmt == kNF4 ? 1 : 2;   // 16-byte code loads per lane, row and step
constexpr int kCodeStepB = 16 * kNV;        // code bytes of a lane's 32 elements

constexpr int kTok = 256;       // tokens per workgroup
constexpr int kStep = 64;       // reduction step (one absmax block)
constexpr int kRowB = kStep * 2;           // bytes of one token row of the activation tile (dense)
constexpr int kBufB = kTok * kRowB;        // 32 KB per buffer
constexpr int kNBuf = 4;                   // activation ring: step s reads buffer s%4
constexpr size_t kLds = (size_t)kNBuf * kBufB;

struct FwdArgs {
  const uint16_t* X;  // [M, K]
  WSrc w0, w1;        // plain: w0 only; gate/up: w0 = gate, w1 = up
  int64_t M, K, N;
  uint16_t* out0;  // Y | g
  uint16_t* out1;  // u
  uint16_t* out2;  // h
};

// The epilogue is branch-free: loads and stores go through buffer resources
// (out-of-range lanes read zero or drop their store); divergent branches there
// would push the 256 accumulators out of AGPRs and spill the main loop.

template <int F, bool GATEUP, int RP, bool ALIGNED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void k_qgemm_fwd(FwdArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [kNBuf][256 rows][128 B], swizzled
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS bases stay scalar
  const int h = lane >> 5, jl = lane & 31;
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t ipt = GATEUP ? 128 : 256;  // output columns per workgroup
  const int64_t nJ = (M + kTok - 1) / kTok;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * ipt, j0 = jt * kTok;
  const int nsteps = (int)(K / kStep);
  const int64_t rows_here = (M - j0) < kTok ? (M - j0) : kTok;  // tokens of this tile that exist

  // This lane's two weight rows: fragment f covers rows nb[f] .. nb[f]+31, lane row nb[f] + jl.
  int64_t nb[2];
  nb[0] = GATEUP ? i0 + 32 * wave : i0 + 64 * wave;
  nb[1] = GATEUP ? nb[0] : nb[0] + 32;

  // ---- buffer resources; per-lane offsets are fixed, the step advances a scalar offset
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.X + j0 * K, rows_here * K * 2);
  // Codes and block values are stored tile-major (TileAddr): both fragments of
  // a wave lie in one 64-row group, whose block b holds its nr rows in order,
  // so a step's codes of the wave's rows are one contiguous run.
  constexpr int64_t kBB = kBlock * kCodeHalfBytes<F> / 2;  // code bytes per row and block
  const int64_t grp = nb[0] - nb[0] % 64;
  const int64_t nrw = (N - grp) < 64 ? ((N - grp) > 0 ? (N - grp) : 64) : 64;  // rows of the group
  __amdgpu_buffer_rsrc_t rC[2], rA[2];
  int offC[2], offA[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const bool second = GATEUP && f == 1;
    rC[f] = make_rsrc(second ? p.w1.codes : p.w0.codes, N * (K / kBlock) * kBB);
    rA[f] = make_rsrc(second ? p.w1.absmax : p.w0.absmax, N * (K / kBlock) * 4);
    const int64_t n = nb[f] + jl;
    offC[f] = n < N ? (int)(grp * (K / kBlock) * kBB + (n - grp) * kBB + kCodeStepB * h) : kOff;
    offA[f] = n < N ? (int)((grp * (K / kBlock) + (n - grp)) * 4) : kOff;
  }
  const int codes_per_step = (int)(nrw * kBB), values_per_step = (int)(nrw * 4);  // scalar strides
  // activation copy: wave w, instruction i fills tile rows 64w+8i .. +7; lane l writes
  // physical chunk l%8 of row 64w+8i+l/8, which holds logical chunk (l%8) ^ ((row>>1)&7)
  int offX[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    offX[i] = (int)((int64_t)row * K * 2 + 16 * c);
  }
  auto dma_x = [&](int step, int buf) {
    const int soff = step * kRowB;
    uint8_t* base = smem + buf * kBufB + (64 * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (__attribute__((address_space(3))) void*)(base + 8 * i * kRowB),
                                               16, offX[i], soff, 0, 0);
  };
  auto load_codes = [&](int step, u32x4 (&cr)[2][kNV], float (&am)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < kNV; ++v)
        cr[f][v] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rC[f], offC[f] + 16 * v, step * codes_per_step, 0));
#pragma unroll
    for (int f = 0; f < 2; ++f)
      am[f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rA[f], offA[f], step * values_per_step, 0));
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[f][j] = f32x16{};

  // ---- the rank-r term, accumulated first by MFMA: acc = (s.B rows) . (Z rows)^T.
  // (Adding it here rather than in the epilogue keeps every accumulator in AGPRs.)
  {
    const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(p.w0.lora_i, N * (int64_t)p.w0.r * 2);
    const __amdgpu_buffer_rsrc_t rZ0 = make_rsrc(p.w0.lora_j + j0 * p.w0.r, rows_here * p.w0.r * 2);
    const __amdgpu_buffer_rsrc_t rB1 = make_rsrc(p.w1.lora_i, N * (int64_t)p.w1.r * 2);
    const __amdgpu_buffer_rsrc_t rZ1 = make_rsrc(p.w1.lora_j + j0 * p.w1.r, rows_here * p.w1.r * 2);
    const int c0 = 8 * h;
#pragma unroll
    for (int rr = 0; rr < RP; rr += 16) {
      u32x4 bh[2], bl[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const bool second = GATEUP && f == 1;
        const int64_t ir = nb[f] + jl;
        const int rs = second ? p.w1.r : p.w0.r;
        const u32x4 bv = rank8<ALIGNED>(second ? rB1 : rB0, ir < N ? ir : -1, rs, rs, rr + c0);
        split_scaled(bv, second ? p.w1.s : p.w0.s, bh[f], bl[f]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t mr = 32 * j + jl;
        const int64_t zrow = mr < rows_here ? mr : -1;
        const u32x4 z0 = rank8<ALIGNED>(rZ0, zrow, p.w0.r, p.w0.r, rr + c0);
        const u32x4 z1 = GATEUP ? rank8<ALIGNED>(rZ1, zrow, p.w1.r, p.w1.r, rr + c0) : z0;
        acc[0][j] = mfma32(bh[0], z0, acc[0][j]);
        acc[0][j] = mfma32(bl[0], z0, acc[0][j]);
        acc[1][j] = mfma32(bh[1], z1, acc[1][j]);
        acc[1][j] = mfma32(bl[1], z1, acc[1][j]);
      }
    }
  }

  // ---- main loop, software-pipelined over 16-wide substeps.
  // While the 16 MFMAs of substep g run, the operands of substep g+1 are
  // prepared: activation fragments read from LDS, weight fragments
  // dequantized from codes already in registers. Step s reads LDS buffer s%4;
  // its activations were copied during step s-3 and published by the barrier
  // ending step s-2, so substep 0 of step s+1 can be read during step s.
  u32x4 cs0[2][kNV], cs1[2][kNV], cs2[2][kNV];  // codes of steps s, s+1, s+2 (rotating)
  float as0[2], as1[2], as2[2];
  WPrep<F> L0[2], L1[2], L2[2];  // per-block tables / scales, rotating with the codes
  u32x4 bv[2][8];                // activation fragments, alternating by substep
  u32x4 av[2][2];                // weight fragments, alternating by substep

  // per-lane byte offset of activation fragment chunk for substep ks (swizzled)
  int offB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) offB[ks] = jl * kRowB + 16 * ((4 * h + ks) ^ ((jl >> 1) & 7));
  auto read_b = [&](int buf, int ks, u32x4 (&dst)[8]) {
    const uint8_t* bx = smem + buf * kBufB + offB[ks];
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = *reinterpret_cast<const u32x4*>(bx + 32 * j * kRowB);
  };
  auto dequant_a = [&](const u32x4 (&cr)[2][kNV], int ks, const WPrep<F> (&lut)[2], u32x4 (&dst)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) dst[f] = wdeq8<F>(cr[f], ks, lut[f]);
  };
  auto luts = [&](const float (&am)[2], WPrep<F> (&lut)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) lut[f] = wprep<F>(am[f]);
  };
  auto mfmas = [&](const u32x4 (&a)[2], const u32x4 (&b)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[0][j] = mfma32(a[0], b[j], acc[0][j]);
      acc[1][j] = mfma32(a[1], b[j], acc[1][j]);
    }
  };
  // issue order inside a substep: 16 MFMAs, each followed by a slice of the
  // other work (LDS reads for the next substep, loads, dequant VALU)
  auto interleave = [&](auto nds_read, auto nvmem, auto nvalu) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < decltype(nds_read)::value) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < decltype(nvmem)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I12 = std::integral_constant<int, 12>;

  // Step s: VMEM issue order is fixed (4 code loads, then 8 activation copies)
  // so the wait before the closing barrier can be counted: the copies of step
  // s+2 (issued during step s-1) must have landed; 12 ops of step s may remain.
  auto body = [&](int s, const u32x4 (&cc)[2][kNV], const WPrep<F> (&lc)[2], const u32x4 (&cn)[2][kNV],
                  const float (&an)[2], WPrep<F> (&ln)[2], u32x4 (&cl)[2][kNV], float (&al)[2]) {
    const int b0 = s % kNBuf, b1 = (s + 1) % kNBuf, b3 = (s + 3) % kNBuf;
    const int s2 = s + 2 < nsteps ? s + 2 : nsteps - 1;
    const int s3 = s + 3 < nsteps ? s + 3 : nsteps - 1;
    // substep 0: codes of s+2 and activations of s+3 requested
    load_codes(s2, cl, al);
    dma_x(s3, b3);
    read_b(b0, 1, bv[1]);
    dequant_a(cc, 1, lc, av[1]);
    mfmas(av[0], bv[0]);
    interleave(I8{}, I12{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 1
    read_b(b0, 2, bv[0]);
    dequant_a(cc, 2, lc, av[0]);
    mfmas(av[1], bv[1]);
    interleave(I8{}, I0{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 2: also the LUTs of step s+1
    read_b(b0, 3, bv[1]);
    dequant_a(cc, 3, lc, av[1]);
    luts(an, ln);
    mfmas(av[0], bv[0]);
    interleave(I8{}, I0{}, I8{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 3: substep 0 of step s+1 prepared from buffer (s+1)%4
    read_b(b1, 0, bv[0]);
    dequant_a(cn, 0, ln, av[0]);
    mfmas(av[1], bv[1]);
    interleave(I8{}, I0{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(12));  // activation copies of step s+2 done
    __builtin_amdgcn_s_waitcnt(0xC07F);           // and this wave's LDS reads
    __builtin_amdgcn_s_barrier();
  };

  // Prologue: codes of steps 0, 1; activations of steps 0, 1, 2 copied (0 and 1 published).
  load_codes(0, cs0, as0);
  load_codes(nsteps > 1 ? 1 : 0, cs1, as1);
  dma_x(0, 0);
  dma_x(nsteps > 1 ? 1 : 0, 1);
  dma_x(nsteps > 2 ? 2 : nsteps - 1, 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
  __builtin_amdgcn_s_barrier();
  luts(as0, L0);
  read_b(0, 0, bv[0]);
  dequant_a(cs0, 0, L0, av[0]);
  // Whole triples in the loop (the code sets rotate with period 3) and the
  // last one or two steps after it: no conditional body inside the loop, so
  // the waits the compiler derives at the loop head are the steady-state ones.
  int s = 0;
  for (; s + 2 < nsteps; s += 3) {
    body(s, cs0, L0, cs1, as1, L1, cs2, as2);
    body(s + 1, cs1, L1, cs2, as2, L2, cs0, as0);
    body(s + 2, cs2, L2, cs0, as0, L0, cs1, as1);
  }
  if (s < nsteps) body(s, cs0, L0, cs1, as1, L1, cs2, as2);
  if (s + 1 < nsteps) body(s + 1, cs1, L1, cs2, as2, L2, cs0, as0);

  // ---- epilogue (no control flow): SwiGLU gate for gate/up, bf16 stores
  const __amdgpu_buffer_rsrc_t rO0 = make_rsrc(p.out0 + j0 * N, rows_here * N * 2);
  const __amdgpu_buffer_rsrc_t rO1 = make_rsrc(GATEUP ? p.out1 + j0 * N : p.out0, GATEUP ? rows_here * N * 2 : 0);
  const __amdgpu_buffer_rsrc_t rO2 = make_rsrc(GATEUP ? p.out2 + j0 * N : p.out0, GATEUP ? rows_here * N * 2 : 0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t mr = 32 * j + jl;  // token row within the tile
    const bool m_ok = mr < rows_here;
    if (!GATEUP) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t ic = nb[f] + 8 * q + 4 * h;
          const int off = (m_ok && ic < N) ? (int)((mr * N + ic) * 2) : kOff;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[f][j][4 * q + e];
          store4(rO0, off, v);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t ic = nb[0] + 8 * q + 4 * h;
        const int off = (m_ok && ic < N) ? (int)((mr * N + ic) * 2) : kOff;
        float gv[4], uv[4], hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[e] = acc[0][j][4 * q + e];
          uv[e] = acc[1][j][4 * q + e];
          hv[e] = gv[e] * sigmoid_f(gv[e]) * uv[e];
        }
        store4(rO0, off, gv);
        store4(rO1, off, uv);
        store4(rO2, off, hv);
      }
    }
  }
}

template <bool GATEUP, int RP, bool ALIGNED>
hipError_t launch_rp(const FwdArgs& a, hipStream_t st) {
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)k_qgemm_fwd<kFmt, GATEUP, RP, ALIGNED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t ipt = GATEUP ? 128 : 256;
  const int64_t nI = (a.N + ipt - 1) / ipt, nJ = (a.M + kTok - 1) / kTok;
  if (nI * nJ == 0) return hipSuccess;
  k_qgemm_fwd<kFmt, GATEUP, RP, ALIGNED><<<(unsigned)(nI * nJ), 256, kLds, st>>>(a);
  return hipGetLastError();
}

template <bool GATEUP, int RP>
hipError_t launch_al(const FwdArgs& a, hipStream_t st) {
  const bool aligned = (a.w0.r % 8 == 0) && (a.w1.r % 8 == 0);
  return aligned ? launch_rp<GATEUP, RP, true>(a, st) : launch_rp<GATEUP, RP, false>(a, st);
}

template <bool GATEUP>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  const int r = a.w0.r > a.w1.r ? a.w0.r : a.w1.r;
  if (r <= 16) return launch_al<GATEUP, 16>(a, st);
  if (r <= 32) return launch_al<GATEUP, 32>(a, st);
  if (r <= 64) return launch_al<GATEUP, 64>(a, st);
  if (r <= 128) return launch_al<GATEUP, 128>(a, st);
  if (r <= 256) return launch_al<GATEUP, 256>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

namespace QL_FMT_NS {

hipError_t launch_gemm_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, uint16_t* Y, hipStream_t st) {
  FwdArgs a{};
  a.X = X;
  a.w0 = a.w1 = w;
  a.M = M, a.K = K, a.N = N;
  a.out0 = Y;
  return launch<false>(a, st);
}

hipError_t launch_gemm_fwd_gateup(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc wg, WSrc wu, uint16_t* g,
                                  uint16_t* u, uint16_t* h, hipStream_t st) {
  FwdArgs a{};
  a.X = X;
  a.w0 = wg;
  a.w1 = wu;
  a.M = M, a.K = K, a.N = N;
  a.out0 = g, a.out1 = u, a.out2 = h;
  return launch<true>(a, st);
}

}  // namespace QL_FMT_NS

}  // namespace qlora
