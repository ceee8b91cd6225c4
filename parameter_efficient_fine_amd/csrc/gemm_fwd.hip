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
//     steps ahead; instruction issue is interleaved with sched_group_barrier;
//     a step's 8 activation copies (each needs its own LDS base in m0) go out
//     two per substep rather than all at once (forward GEMM -5% at the attn
//     shape: the burst left a gap of some 100 cycles between two MFMAs).
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
constexpr int64_t kCUs = 256;   // compute units of the chip (one workgroup each)
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
  const int32_t* pos;     // RoPE epilogue: token positions [M]
  const float* rope_tab;  // [max_pos][64][2] fp32 (cos, sin)
  int64_t max_pos;
};

constexpr int kRopeD = 128;  // head size of the RoPE epilogue (Llama-3)

// The tables of two weight rows held by the two halves of a wave (row 0 by
// lanes 0-31, row 1 by lanes 32-63, lane l and l+32 on the same pair): each
// lane builds the table of its own half's row, and v_permlane32_swap (the
// upper 32 lanes of its first operand exchanged with the lower 32 lanes of its
// second) hands every lane both: with both operands equal to the own table,
// the first result carries row 0's table in all 64 lanes, the second row 1's.
__device__ __forceinline__ void make_lut_pair(float absmax_own, Nf4Lut& t0, Nf4Lut& t1) {
  const Nf4Lut own = make_lut(absmax_own);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto lo = __builtin_amdgcn_permlane32_swap(own.lo[q], own.lo[q], false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(own.hi[q], own.hi[q], false, false);
    t0.lo[q] = lo[0], t1.lo[q] = lo[1];
    t0.hi[q] = hi[0], t1.hi[q] = hi[1];
  }
}

// The epilogue is branch-free: loads and stores go through buffer resources
// (out-of-range lanes read zero or drop their store); divergent branches there
// would push the 256 accumulators out of AGPRs and spill the main loop.

// EPI: 0 the plain product, 1 with the RoPE epilogue, 2 the plain product on
// 128-token tiles (TK tokens per workgroup), taken where 256-token tiles would
// leave CUs idle (launch_rp). Each output element sums the same products in the
// same order on either tile, so both give the same bits.
// (The body is a device function that the kernel below calls: with the tile
// size a template parameter of a kernel itself, the host compilation emitted
// no launch stubs for it.)
template <int F, bool GATEUP, int RP, bool ALIGNED, int EPI>
__device__ __forceinline__ void qgemm_fwd_body(FwdArgs p) {
  constexpr bool ROPE = EPI == 1;
  constexpr int TK = EPI == 2 ? 128 : kTok;
  static_assert(EPI != 2 || !GATEUP, "128-token tiles: plain product only");
  constexpr int NJ = TK / 32;          // token fragments per wave, activation copies per wave and step
  constexpr int kBuf = TK * kRowB;     // bytes of one ring buffer
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [kNBuf][TK rows][128 B], swizzled
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS bases stay scalar
  const int h = lane >> 5, jl = lane & 31;
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t ipt = GATEUP ? 128 : 256;  // output columns per workgroup
  const int64_t nJ = (M + TK - 1) / TK;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * ipt, j0 = jt * TK;
  const int nsteps = (int)(K / kStep);
  const int64_t rows_here = (M - j0) < TK ? (M - j0) : TK;  // tokens of this tile that exist

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
  // activation copy: wave w, instruction i fills tile rows (TK/4)w+8i .. +7; lane l writes
  // physical chunk l%8 of row (TK/4)w+8i+l/8, which holds logical chunk (l%8) ^ ((row>>1)&7)
  int offX[NJ];
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int row = (TK / 4) * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    offX[i] = (int)((int64_t)row * K * 2 + 16 * c);
  }
  auto dma_q = [&](int step, int buf, int q) {  // quarter q of the NJ copies
    const int soff = step * kRowB;
    uint8_t* base = smem + buf * kBuf + ((TK / 4) * wave) * kRowB;
#pragma unroll
    for (int i = q * (NJ / 4); i < (q + 1) * (NJ / 4); ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (__attribute__((address_space(3))) void*)(base + 8 * i * kRowB),
                                               16, offX[i], soff, 0, 0);
  };
  auto dma_x = [&](int step, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_q(step, buf, q);
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

  f32x16 acc[2][NJ];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = f32x16{};

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
      u32x4 z[NJ][2];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t mr = 32 * j + jl;
        const int64_t zrow = mr < rows_here ? mr : -1;
        z[j][0] = rank8<ALIGNED>(rZ0, zrow, p.w0.r, p.w0.r, rr + c0);
        z[j][1] = GATEUP ? rank8<ALIGNED>(rZ1, zrow, p.w1.r, p.w1.r, rr + c0) : z[j][0];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[0][j] = mfma32(bh[0], z[j][0], acc[0][j]);
        acc[1][j] = mfma32(bh[1], z[j][1], acc[1][j]);
      }
      // the low parts only where some lane has one (none when s is a power of two)
      if (lo_any(bl[0], bl[1])) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[0][j] = mfma32(bl[0], z[j][0], acc[0][j]);
          acc[1][j] = mfma32(bl[1], z[j][1], acc[1][j]);
        }
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
  u32x4 bv[2][NJ];               // activation fragments, alternating by substep
  u32x4 av[2][2];                // weight fragments, alternating by substep

  // per-lane byte offset of activation fragment chunk for substep ks (swizzled)
  int offB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) offB[ks] = jl * kRowB + 16 * ((4 * h + ks) ^ ((jl >> 1) & 7));
  auto read_b = [&](int buf, int ks, u32x4 (&dst)[NJ]) {
    const uint8_t* bx = smem + buf * kBuf + offB[ks];
#pragma unroll
    for (int j = 0; j < NJ; ++j) dst[j] = *reinterpret_cast<const u32x4*>(bx + 32 * j * kRowB);
  };
  auto dequant_a = [&](const u32x4 (&cr)[2][kNV], int ks, const WPrep<F> (&lut)[2], u32x4 (&dst)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) dst[f] = wdeq8<F>(cr[f], ks, lut[f]);
  };
  // NF4: lane half h builds the table of fragment h's row (lanes l and l+32 hold
  // the same two rows) and the halves exchange them
  auto luts = [&](const float (&am)[2], WPrep<F> (&lut)[2]) {
    if constexpr (F == kNF4) {
      make_lut_pair(h ? am[1] : am[0], lut[0].lut, lut[1].lut);
    } else {
#pragma unroll
      for (int f = 0; f < 2; ++f) lut[f] = wprep<F>(am[f]);
    }
  };
  auto mfmas = [&](const u32x4 (&a)[2], const u32x4 (&b)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[0][j] = mfma32(a[0], b[j], acc[0][j]);
      acc[1][j] = mfma32(a[1], b[j], acc[1][j]);
    }
  };
  // issue order inside a substep: its 2*NJ MFMAs, each followed by a slice of
  // the other work (the NJ LDS reads of the next substep first, loads, and the
  // dequant VALU spread at nvalu * 8/NJ ops per MFMA: the same per substep for
  // either tile)
  auto interleave = [&](auto nvmem, auto nvalu) {
#pragma unroll
    for (int i = 0; i < 2 * NJ; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < decltype(nvmem)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value * 8 / NJ, 0);
    }
  };
  constexpr int kCL = 2 * kNV + 2;  // code and block-value loads of a step
  using IC = std::integral_constant<int, kCL + NJ / 4>;
  using IQ = std::integral_constant<int, NJ / 4>;
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;

  // Step s: VMEM issue order is fixed (the code loads, then NJ activation
  // copies) so the wait before the closing barrier can be counted: the copies
  // of step s+2 (issued during step s-1) must have landed; the kCL + NJ ops of
  // step s may remain.
  auto body = [&](int s, const u32x4 (&cc)[2][kNV], const WPrep<F> (&lc)[2], const u32x4 (&cn)[2][kNV],
                  const float (&an)[2], WPrep<F> (&ln)[2], u32x4 (&cl)[2][kNV], float (&al)[2]) {
    const int b0 = s % kNBuf, b1 = (s + 1) % kNBuf, b3 = (s + 3) % kNBuf;
    const int s2 = s + 2 < nsteps ? s + 2 : nsteps - 1;
    const int s3 = s + 3 < nsteps ? s + 3 : nsteps - 1;
    // substep 0: codes of s+2 and two of the activation copies of s+3 requested
    load_codes(s2, cl, al);
    dma_q(s3, b3, 0);
    read_b(b0, 1, bv[1]);
    dequant_a(cc, 1, lc, av[1]);
    mfmas(av[0], bv[0]);
    interleave(IC{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 1
    dma_q(s3, b3, 1);
    read_b(b0, 2, bv[0]);
    dequant_a(cc, 2, lc, av[0]);
    mfmas(av[1], bv[1]);
    interleave(IQ{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 2: also the LUTs of step s+1
    dma_q(s3, b3, 2);
    read_b(b0, 3, bv[1]);
    dequant_a(cc, 3, lc, av[1]);
    luts(an, ln);
    mfmas(av[0], bv[0]);
    interleave(IQ{}, I6{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 3: substep 0 of step s+1 prepared from buffer (s+1)%4
    dma_q(s3, b3, 3);
    read_b(b1, 0, bv[0]);
    dequant_a(cn, 0, ln, av[0]);
    mfmas(av[1], bv[1]);
    interleave(IQ{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCL + NJ));  // activation copies of step s+2 done
    __builtin_amdgcn_s_waitcnt(0xC07F);           // and this wave's LDS reads
    __builtin_amdgcn_s_barrier();
  };

  // Prologue: codes of steps 0, 1; activations of steps 0, 1, 2 copied (0 and 1 published).
  load_codes(0, cs0, as0);
  load_codes(nsteps > 1 ? 1 : 0, cs1, as1);
  dma_x(0, 0);
  dma_x(nsteps > 1 ? 1 : 0, 1);
  dma_x(nsteps > 2 ? 2 : nsteps - 1, 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(NJ));
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

  // ---- RoPE epilogue ("Unsloth" wiki entry, Theory: fused RoPE kernel; rotate
  // half, heads of 128 output columns, so the workgroup's 256 columns are two
  // heads). The rotation pairs column i with i + 64 of the same head, which
  // another wave holds; so, 32 tokens at a time, the four waves park their fp32
  // results in LDS (free once the loop has ended) as a [32 token][256 column]
  // tile, and each lane then takes one token and 8 frequencies
  // (4g .. 4g+3 and 32+4g .. 32+4g+3) in both heads: it reads each (cos, sin)
  // it needs once, rotates (first half v c - w s, second half w c + v s) and
  // rounds once to bf16. Tile rows are 64 chunks of 16 bytes, chunk c of row t
  // stored at c ^ (t & 7) (conflict-free writes and reads); the (cos, sin) rows
  // come from the position table two fragments ahead.
  if constexpr (ROPE) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's trailing copies into the ring have landed
    __builtin_amdgcn_s_barrier();   // and every wave is done reading the ring
    // lane indices re-read through an empty asm: no prologue offsets stay alive
    // across the main loop for this epilogue
    int lne = lane, jle = jl, he = h;
    asm volatile("" : "+v"(lne), "+v"(jle), "+v"(he));
    float* const xb = reinterpret_cast<float*>(smem);  // [2 parity][32 rows][256 columns]
    const int L = 64 * wave + lne, tt = L >> 3, g = L & 7;  // reader: token row tt, frequency group g
    const int Ni = (int)N, rh = (int)rows_here, ci0 = (int)i0;
    const __amdgpu_buffer_rsrc_t rPos = make_rsrc(p.pos + j0, rows_here * 4);
    const __amdgpu_buffer_rsrc_t rTab = make_rsrc(p.rope_tab, p.max_pos * (kRopeD / 2) * 8);
    const __amdgpu_buffer_rsrc_t rY = make_rsrc(p.out0 + j0 * N, rows_here * N * 2);
    const int maxp = (int)p.max_pos;
    // (cos, sin) of frequencies 4g .. 4g+3 and 32+4g .. +3 at the position of token
    // row tt of fragment j (a position outside the table reads zeros)
    u32x4 tb[3][4];
    auto tload = [&](int j, u32x4 (&t)[4]) {
      const int pj = (int)__builtin_amdgcn_raw_buffer_load_b32(rPos, (32 * j + tt) * 4, 0, 0);
      const int base = (pj >= 0 && pj < maxp) ? (pj * (kRopeD / 2) + 4 * g) * 8 : kOff;
      const int b2 = base == kOff ? kOff : base + 32 * 8;
      t[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rTab, base, 0, 0));
      t[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rTab, base, 16, 0));
      t[2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rTab, b2, 0, 0));
      t[3] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rTab, b2, 16, 0));
    };
    tload(0, tb[0]);
    tload(1, tb[1]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) tload(j + 2, tb[(j + 2) % 3]);
      float* const tile = xb + (j & 1) * 32 * 256;
      // writer: token row jle, chunk 16 wave + 8f + 2q + he holds columns 64 wave + 32f + 8q + 4he .. +3
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (16 * wave + 8 * f + 2 * q + he) ^ (jle & 7);
          *reinterpret_cast<f32x4*>(tile + jle * 256 + 4 * c) =
              f32x4{acc[f][j][4 * q], acc[f][j][4 * q + 1], acc[f][j][4 * q + 2], acc[f][j][4 * q + 3]};
        }
      lds_barrier();
      // reader: quarter k = head (k >> 1), half (k & 1); chunks 16k + g (frequencies 4g ..)
      // and 16k + 8 + g (frequencies 32 + 4g ..)
      f32x4 v[4][2];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          v[k][u] = *reinterpret_cast<const f32x4*>(tile + tt * 256 + 4 * ((16 * k + 8 * u + g) ^ (tt & 7)));
      const u32x4(&t)[4] = tb[j % 3];
      const int mr = 32 * j + tt;
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4 t0 = __builtin_bit_cast(f32x4, t[2 * u]), t1 = __builtin_bit_cast(f32x4, t[2 * u + 1]);
          const float c[4] = {t0[0], t0[2], t1[0], t1[2]}, sn[4] = {t0[1], t0[3], t1[1], t1[3]};
          const f32x4 a = v[2 * hd][u], b = v[2 * hd + 1][u];  // first and second half of the head
          float lo[4], hi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = a[e] * c[e] - b[e] * sn[e];
            hi[e] = b[e] * c[e] + a[e] * sn[e];
          }
          const int icl = ci0 + 128 * hd + 32 * u + 4 * g, ich = icl + 64;
          store4(rY, (mr < rh && icl < Ni) ? (mr * Ni + icl) * 2 : kOff, lo);
          store4(rY, (mr < rh && ich < Ni) ? (mr * Ni + ich) * 2 : kOff, hi);
        }
    }
    return;
  }

  // ---- epilogue through LDS. The accumulator layout gives a lane 4 columns of
  // one token, so direct stores would write 8 bytes into each of 32 rows per
  // instruction. Instead each wave parks its results as bf16 in its own 32 KB
  // of the ring (idle once the loop has ended), token-major, and reads them
  // back in 16-byte row pieces: a store instruction then covers whole 128-byte
  // (plain: 64 columns) or 64-byte (gate/up: 32 columns) pieces of 8 or 16 rows.
  // Plain: rows of 128 bytes, 16-byte chunk c of token row t at c ^ (t & 7).
  // Gate/up: g and u, then h, as rows of 64 bytes, chunk c at c ^ ((t >> 2) & 3);
  // h = silu(g) * u from the fp32 accumulators.
  __builtin_amdgcn_s_waitcnt(0);  // this wave's trailing copies into the ring have landed
  __builtin_amdgcn_s_barrier();   // and every wave is done reading the ring
  int jle = jl, he = h, lne = lane;
  asm volatile("" : "+v"(jle), "+v"(he), "+v"(lne));  // no prologue values kept alive for this
  uint8_t* const reg = smem + wave * (TK * 128);
  const int rh = (int)rows_here;
  if constexpr (!GATEUP) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int t = 32 * j + jle;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2*>(reg + t * 128 + 16 * ((4 * f + q) ^ (t & 7)) + 8 * he) =
              u32x2{pack_bf16x2(acc[f][j][4 * q], acc[f][j][4 * q + 1]),
                    pack_bf16x2(acc[f][j][4 * q + 2], acc[f][j][4 * q + 3])};
    }
    lds_barrier();
    const __amdgpu_buffer_rsrc_t rY = make_rsrc(p.out0 + j0 * N, rows_here * N * 2);
    const int c = lne & 7, tq = lne >> 3;
    const int64_t col = i0 + 64 * wave + 8 * c;
#pragma unroll
    for (int u = 0; u < TK / 8; ++u) {
      const int t = 8 * u + tq;
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + t * 128 + 16 * (c ^ (t & 7)));
      const int off = (t < rh && col < N) ? (int)((t * N + col) * 2) : kOff;
      __builtin_amdgcn_raw_buffer_store_b128(v, rY, off, 0, kStoreNT);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rO0 = make_rsrc(p.out0 + j0 * N, rows_here * N * 2);
    const __amdgpu_buffer_rsrc_t rO1 = make_rsrc(p.out1 + j0 * N, rows_here * N * 2);
    const __amdgpu_buffer_rsrc_t rO2 = make_rsrc(p.out2 + j0 * N, rows_here * N * 2);
    const int c = lne & 3, tq = lne >> 2;
    const int64_t col = i0 + 32 * wave + 8 * c;
    auto put = [&](uint8_t* dst, int j, int q, const float (&v)[4]) {
      const int t = 32 * j + jle;
      *reinterpret_cast<u32x2*>(dst + t * 64 + 16 * (q ^ ((t >> 2) & 3)) + 8 * he) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    };
    auto drain = [&](const uint8_t* src, __amdgpu_buffer_rsrc_t rO) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int t = 16 * u + tq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + t * 64 + 16 * (c ^ ((t >> 2) & 3)));
        const int off = (t < rh && col < N) ? (int)((t * N + col) * 2) : kOff;
        __builtin_amdgcn_raw_buffer_store_b128(v, rO, off, 0, kStoreNT);
      }
    };
    // g into the first half, u into the second, h into the first again; every
    // wave touches only its own region, so the barriers only order its own LDS work
    uint8_t* const reg2 = reg + kTok * 64;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float gv[4] = {acc[0][j][4 * q], acc[0][j][4 * q + 1], acc[0][j][4 * q + 2], acc[0][j][4 * q + 3]};
        put(reg, j, q, gv);
      }
    lds_barrier();
    drain(reg, rO0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float uv[4] = {acc[1][j][4 * q], acc[1][j][4 * q + 1], acc[1][j][4 * q + 2], acc[1][j][4 * q + 3]};
        put(reg2, j, q, uv);
      }
    lds_barrier();
    drain(reg2, rO1);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[0][j][4 * q + e];
          hv[e] = g * sigmoid_f(g) * acc[1][j][4 * q + e];
        }
        put(reg, j, q, hv);
      }
    lds_barrier();
    drain(reg, rO2);
  }
}

template <int F, bool GATEUP, int RP, bool ALIGNED, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void k_qgemm_fwd(FwdArgs p) {
  qgemm_fwd_body<F, GATEUP, RP, ALIGNED, EPI>(p);
}

template <bool GATEUP, int RP, bool ALIGNED, bool ROPE>
hipError_t launch_rp(const FwdArgs& a, hipStream_t st) {
  // set once per kernel instance; a function-local static is initialised exactly
  // once even when several threads make their first call together
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_qgemm_fwd<kFmt, GATEUP, RP, ALIGNED, ROPE ? 1 : 0>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int64_t ipt = GATEUP ? 128 : 256;
  const int64_t nI = (a.N + ipt - 1) / ipt, nJ = (a.M + kTok - 1) / kTok;
  if (nI * nJ == 0) return hipSuccess;
  if constexpr (!GATEUP && !ROPE) {
    // 128-token tiles where 256-token ones leave CUs idle and the 128-token
    // grid still runs in one pass of one workgroup per CU (a decoded weight
    // then feeds half as many MFMAs, which only pays where CUs would idle)
    const int64_t nJ128 = (a.M + 127) / 128;
    if (a.M > 256 && nI * nJ < kCUs && nI * nJ128 <= kCUs) {
      constexpr size_t kLds128 = (size_t)kNBuf * 128 * kRowB;
      static const hipError_t attr128 = hipFuncSetAttribute(
          (const void*)k_qgemm_fwd<kFmt, false, RP, ALIGNED, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
          (int)kLds128);
      if (attr128 != hipSuccess) return attr128;
      k_qgemm_fwd<kFmt, false, RP, ALIGNED, 2><<<(unsigned)(nI * nJ128), 256, kLds128, st>>>(a);
      return hipGetLastError();
    }
  }
  k_qgemm_fwd<kFmt, GATEUP, RP, ALIGNED, ROPE ? 1 : 0><<<(unsigned)(nI * nJ), 256, kLds, st>>>(a);
  return hipGetLastError();
}

template <bool GATEUP, int RP, bool ROPE>
hipError_t launch_al(const FwdArgs& a, hipStream_t st) {
  const bool aligned = (a.w0.r % 8 == 0) && (a.w1.r % 8 == 0);
  return aligned ? launch_rp<GATEUP, RP, true, ROPE>(a, st) : launch_rp<GATEUP, RP, false, ROPE>(a, st);
}

template <bool GATEUP, bool ROPE = false>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  const int r = a.w0.r > a.w1.r ? a.w0.r : a.w1.r;
  if (r <= 16) return launch_al<GATEUP, 16, ROPE>(a, st);
  if (r <= 32) return launch_al<GATEUP, 32, ROPE>(a, st);
  if (r <= 64) return launch_al<GATEUP, 64, ROPE>(a, st);
  if (r <= 128) return launch_al<GATEUP, 128, ROPE>(a, st);
  if (r <= 256) return launch_al<GATEUP, 256, ROPE>(a, st);
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

hipError_t launch_gemm_fwd_rope(const uint16_t* X, int64_t M, int64_t K, int64_t N, WSrc w, const int32_t* pos,
                                const float* table, int64_t max_pos, uint16_t* Y, hipStream_t st) {
  if (N % kRopeD != 0) return hipErrorInvalidValue;
  FwdArgs a{};
  a.X = X;
  a.w0 = a.w1 = w;
  a.M = M, a.K = K, a.N = N;
  a.out0 = Y;
  a.pos = pos;
  a.rope_tab = table;
  a.max_pos = max_pos;
  return launch<false, true>(a, st);
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
