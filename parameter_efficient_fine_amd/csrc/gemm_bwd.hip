// Backward fused-dequant GEMM of the QLoRA layer on gfx950:
//   dX = dY . What + s . G . A                  (G = dY.B from skinny_nt)
// with two variants: a concatenated reduction over two (dY, W) pairs (the
// gate and up projections of the SwiGLU block feed one dX), and the SwiGLU
// backward applied to the down projection's product (dh never stored):
//   dg = dh * u * sig(g) * (1 + g * (1 - sig(g))),   du = dh * silu(g).
//
// "Unsloth" wiki entry, Theory: the hand-derived LoRA backward and the fused
// SwiGLU block; "Rev vs unsloth", fused quantized-LoRA card: no dequantized
// weight in HBM; "Unsloth vs PyTorch" video, 1:35-2:00: the rank-r term goes
// through the skinny G and A, never through the N x K product B.A.
//
// Design (one workgroup = 4 waves, 256 output columns x 256 tokens, the
// reduction over N in steps of 64):
//   * each wave owns 64 output columns -- one 64-column block of every weight
//     row -- and all 256 tokens (8 MFMA fragments), 256 fp32 accumulators per
//     lane in AGPRs;
//   * the reduction runs over weight rows, so a lane needs 8 consecutive rows
//     of one column: lane l dequantizes weight row n0 + l of the wave's block
//     (one NF4 table per lane and step), the wave writes its private 64 x 64
//     bf16 tile to LDS (XOR-swizzled, conflict-free) and reads it back
//     column-wise with ds_read_b64_tr_b16. The tile is private to the wave:
//     no barrier guards it;
//   * the dY tile (256 tokens x 64) is copied by buffer_load ... lds, double
//     buffered; codes run a step ahead;
//   * the compiler must assume a transposed LDS read may touch memory an
//     LDS copy is still writing, and waits for every copy in flight before
//     one. So all 16 transposed reads of a step are issued together, during
//     the previous step's last 16 MFMAs, right after that step's barrier (by
//     which the copies they would wait for have landed), and the next copies
//     are issued after them. During the MFMAs, the dY fragments of the next
//     substep are read (plain reads) and the next step's weight rows are
//     dequantized straight into the other tile buffer.
// Tile edges use the buffer range check: rows past N and columns past K read
// zero, tokens past M drop their stores.
//
// k_qgemm_bwd8 below is the same pipeline with 8 waves (two per SIMD), each
// holding 64 columns x 128 tokens; every product uses it except the
// two-source one at rank 256, the only one this 4-wave kernel runs.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "reduce.hpp"

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
constexpr int kNV = kFmt == kNF4 ? 2 : 4;  // 16-byte code loads per lane and step (64 elements)

constexpr int kTok = 256;                  // tokens per workgroup
constexpr int kStep = 64;                  // reduction rows per step
constexpr int kRowB = kStep * 2;           // bytes of one token row of the dY tile
constexpr int kBufB = kTok * kRowB;        // 32 KB per dY buffer
constexpr int kWRowB = 128;                // one weight row of a wave's tile (64 columns)
constexpr int kWBufB = kStep * kWRowB;     // 8 KB per wave and buffer
constexpr size_t kLds = 2 * (size_t)kBufB + 2 * 4 * (size_t)kWBufB;  // 128 KB: dY x2, weight tiles 4 waves x2

enum BwdMode { kPlain = 0, kConcat = 1, kSwiGLU = 2 };

struct BwdArgs {
  const uint16_t* dY[2];  // [M, N] per source
  WSrc w[2];              // lora_i = A [r, K], lora_j = G [M, r] (row stride ldj)
  int64_t M, K, N;        // dX [M, K]; reduction over N per source
  uint16_t* out0;         // dX | dg
  uint16_t* out1;         // du
  const uint16_t* g;      // SwiGLU: saved g, u [M, K]
  const uint16_t* u;
  TnJobs red;             // partial sums of the preceding skinny_tn to reduce (n = 0: none)
};

// Weight tile swizzle: 16-byte chunk q of row j is stored at chunk q ^ wsw(j),
// wsw(j) = the bits of j & 7 reordered (bit 0 -> 0, bit 1 -> 2, bit 2 -> 1).
// A 16-byte LDS write serves 8 lanes per cycle within a 128-byte bank window:
// the 8 rows a wave writes together (one chunk each) get 8 distinct chunk
// positions. The transposed reads take 4 consecutive rows x 4 chunks per
// 256-byte window: rows j and j + 2 differ in bit 2 of wsw, so they fall in
// opposite halves of the row.
__device__ __forceinline__ int wsw(int j) { return (j & 1) | (((j >> 1) & 1) << 2) | (((j >> 2) & 1) << 1); }

template <int F, int MODE, int RP, bool ALIGNED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void k_qgemm_bwd(BwdArgs p) {
  // launched only for the two-source product at rank 256, whose rank term does
  // not fit the 8-wave kernel's 256 registers per lane (launch_rp)
  static_assert(MODE != kSwiGLU, "the SwiGLU backward runs on the 8-wave kernel");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // dY [2], then weight tiles [2][4 waves]
  constexpr int NSRC = MODE == kConcat ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, jl = lane & 31;
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t nJ = (M + kTok - 1) / kTok;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * 256, j0 = jt * kTok;
  const int sps = (int)((N + kStep - 1) / kStep);  // steps per source
  const int nsteps = sps * NSRC;
  const bool ragged = (N % kStep) != 0;
  const int64_t rows_here = (M - j0) < kTok ? (M - j0) : kTok;
  const int64_t kc = i0 + 64 * wave;  // this wave's first output column (a 64-column block)
  const bool k_ok = kc < K;
  uint8_t* const wtile = smem + 2 * kBufB + wave * kWBufB;  // buffer b at + b * 4 * kWBufB

  // ---- dY copies (as the forward's activation copies). Lane l of instruction
  // i fills row 64w + 8i + l/8, physical chunk l%8 = logical chunk
  // (l%8) ^ ((row>>1)&7). In a ragged last step the chunks past N read nothing.
  int offY[8], offYl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    offY[i] = (int)((int64_t)row * N * 2 + 16 * c);
    offYl[i] = (int64_t)(sps - 1) * kStep + 8 * c < N ? offY[i] : kOff;
  }
  auto dma_y = [&](int step, int buf) {
    const int src = NSRC > 1 && step >= sps ? 1 : 0;
    const int sl = step - src * sps;
    const bool last = ragged && sl == sps - 1;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY[src ? NSRC - 1 : 0] + j0 * N, rows_here * N * 2);
    uint8_t* base = smem + buf * kBufB + (64 * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (__attribute__((address_space(3))) void*)(base + 8 * i * kRowB), 16,
                                               last ? offYl[i] : offY[i], sl * kRowB, 0, 0);
  };

  // ---- codes and block value of weight row n0 + lane, block kc/64. They are
  // stored tile-major (TileAddr): a step's 64 rows are one row group whose
  // block kc/64 holds their codes row after row, so the wave reads one
  // contiguous tile and lane l its l-th run. Per-lane offsets are
  // loop-invariant; each step gets buffer resources based at its tile and
  // sized to the rows that exist, so rows past N read zero (zero codes and
  // value give an all-zero table) with no per-step VGPR arithmetic next to
  // loads in flight.
  constexpr int kHB = kCodeHalfBytes<F>;  // 2 x bytes per code
  constexpr int64_t kBB = kBlock * kHB / 2;  // code bytes per row and block
  const int offC = k_ok ? (int)(lane * kBB) : kOff;
  const int offA = k_ok ? lane * 4 : kOff;
  auto load_codes = [&](int step, u32x4 (&cr)[kNV], float& am) {
    const int src = NSRC > 1 && step >= sps ? 1 : 0;
    const int64_t n0 = (int64_t)(step - src * sps) * kStep;
    const WSrc& w = p.w[src ? NSRC - 1 : 0];
    const int64_t nr = (N - n0) < kStep ? (N - n0) : kStep;  // rows of this group
    const int64_t jb = kc / kBlock;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(w.codes + n0 * (K / kBlock) * kBB + jb * nr * kBB, nr * kBB);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(w.absmax + n0 * (K / kBlock) + jb * nr, nr * 4);
#pragma unroll
    for (int v = 0; v < kNV; ++v)
      cr[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, offC, 16 * v, 0));
    am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, offA, 0, 0));
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[f][j] = f32x16{};

  // ---- the rank-r term first, by MFMA: acc += (s.A^T rows) . (G rows)^T.
  // A is read in place ([r, K]): a lane's 8 rank entries of column k are
  // strided by K (eight 2-byte loads, once per kernel).
#pragma unroll
  for (int src = 0; src < NSRC; ++src) {
    const WSrc& w = p.w[src];
    const __amdgpu_buffer_rsrc_t rA_ = make_rsrc(w.lora_i, K * (int64_t)w.r * 2);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(w.lora_j + j0 * w.ldj, rows_here * w.ldj * 2);
    const int c0 = 8 * h;
#pragma unroll
    for (int rr = 0; rr < RP; rr += 16) {
      u32x4 ah[2], al[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int64_t ir = kc + 32 * f + jl;
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e0 = rr + c0 + 2 * q, e1 = e0 + 1;
          const int o0 = (ir < K && e0 < w.r) ? (int)(((int64_t)e0 * K + ir) * 2) : kOff;
          const int o1 = (ir < K && e1 < w.r) ? (int)(((int64_t)e1 * K + ir) * 2) : kOff;
          wv[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA_, o0, 0, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA_, o1, 0, 0) << 16);
        }
        split_scaled(u32x4{wv[0], wv[1], wv[2], wv[3]}, w.s, ah[f], al[f]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t mr = 32 * j + jl;
        const u32x4 z = rank8<ALIGNED>(rG, mr < rows_here ? mr : -1, w.ldj, w.r, rr + c0);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          acc[f][j] = mfma32(ah[f], z, acc[f][j]);
          acc[f][j] = mfma32(al[f], z, acc[f][j]);
        }
      }
    }
  }

  // ---- operand reads.
  // B (dY): token 32j + jl, reduction rows 16ks + 8h .. +7 = chunk 2ks + h.
  int offB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) offB[ks] = jl * kRowB + 16 * ((2 * ks + h) ^ ((jl >> 1) & 7));
  u32x4 bv[2][8];
  auto read_b = [&](int buf, int ks, u32x4 (&dst)[8]) {
    const uint8_t* bx = smem + buf * kBufB + offB[ks];
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = *reinterpret_cast<const u32x4*>(bx + 32 * j * kRowB);
  };
  // A (weights): fragment f = columns 32f .. 32f+31 of the wave's block, column
  // 32f + l%32, rows 16ks + 8h .. +7, as two transposed reads (rows +0..3, +4..7).
  // Within a 16-lane group, lane s points at row (s>>2) (+4), columns 4(s&3)..+3
  // of a 16-column group; the swizzle only depends on the row mod 8.
  int offW[2][2];
  {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = 8 * (g >> 1) + (s >> 2) + 4 * hi;
        const int col = 32 * f + 16 * (g & 1) + 4 * (s & 3);
        offW[f][hi] = row * kWRowB + 16 * ((col >> 3) ^ wsw(row)) + 2 * (col & 7);
      }
  }
  u32x4 av[4][2];  // the whole step's weight operands
  auto read_a = [&](int wb, int ks) {
    const uint8_t* wt = wtile + wb * 4 * kWBufB;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const u32x2 lo = lds_read_tr(wt + offW[f][0] + ks * 16 * kWRowB);
      const u32x2 hi = lds_read_tr(wt + offW[f][1] + ks * 16 * kWRowB);
      av[ks][f] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // weight row n0 + lane of the next step: chunk q -> tile buffer wb
  const int wsl = wsw(lane);
  auto dequant_write = [&](int wb, const u32x4 (&cr)[kNV], const WPrep<F>& lut, int q0) {
    uint8_t* row = wtile + wb * 4 * kWBufB + lane * kWRowB;
#pragma unroll
    for (int q = q0; q < q0 + 2; ++q)
      *reinterpret_cast<u32x4*>(row + 16 * (q ^ wsl)) = wdeq8<F>(cr, q, lut);
  };
  auto mfmas = [&](const u32x4 (&a)[2], const u32x4 (&b)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[0][j] = mfma32(a[0], b[j], acc[0][j]);
      acc[1][j] = mfma32(a[1], b[j], acc[1][j]);
    }
  };
  // issue order inside a substep: 16 MFMAs, each followed by a slice of the
  // other work (LDS reads, global loads, VALU). The tile writes take the last
  // slots: each waits for a whole dequantization chain, and an early slot
  // would pull that chain in front of the MFMAs instead of between them.
  auto interleave = [&](auto nds_read, auto nds_write, auto nvmem, auto nvalu) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < decltype(nds_read)::value) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i >= 16 - decltype(nds_write)::value) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      if (i < decltype(nvmem)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;
  using I8 = std::integral_constant<int, 8>;
  using I12 = std::integral_constant<int, 12>;

  // Step s: dY from buffer s&1 and weights from tile buffer s&1, both read
  // ahead (entering the step, av holds all of its weight operands and bv[0]
  // its first dY fragments). During substeps 0-2 the codes of step s+1 (cc,
  // loaded during step s-1) are dequantized into tile buffer (s+1)&1 and the
  // codes of step s+2 are requested. Substep 3 starts with the step's only
  // barrier (the dY copies of step s+1 landed, every wave is done with dY
  // buffer s&1); its MFMAs then overlap the reads of step s+1's operands,
  // after which -- never before a transposed read -- the dY copies of step
  // s+2 go to buffer s&1.
  auto body = [&](int s, const u32x4 (&cc)[kNV], float ac, u32x4 (&cn)[kNV], float& an) {
    const int b0 = s & 1, b1 = b0 ^ 1;
    const int s2 = s + 2 < nsteps ? s + 2 : nsteps - 1;
    // substep 0 (also the table of step s+1's rows and the codes of step s+2)
    load_codes(s2, cn, an);
    const WPrep<F> lut = wprep<F>(ac);
    read_b(b0, 1, bv[1]);
    dequant_write(b1, cc, lut, 0);
    mfmas(av[0], bv[0]);
    interleave(I8{}, I2{}, I3{}, I6{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 1
    read_b(b0, 2, bv[0]);
    dequant_write(b1, cc, lut, 2);
    mfmas(av[1], bv[1]);
    interleave(I8{}, I2{}, I0{}, I4{});
    __builtin_amdgcn_sched_barrier(0);
    // substep 2
    read_b(b0, 3, bv[1]);
    dequant_write(b1, cc, lut, 4);
    dequant_write(b1, cc, lut, 6);
    mfmas(av[2], bv[0]);
    interleave(I8{}, I4{}, I0{}, I8{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's dY copies of step s+1 (and codes of s+2)
    __builtin_amdgcn_s_waitcnt(0xC07F);          // this wave's LDS reads and tile writes
    __builtin_amdgcn_s_barrier();
    // substep 3: MFMAs of step s while step s+1's operands are read
    mfmas(av[3], bv[1]);
    read_b(b1, 0, bv[0]);
    read_a(b1, 0);
    read_a(b1, 1);
    read_a(b1, 2);
    read_a(b1, 3);
    interleave(I12{}, I0{}, I0{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    dma_y(s2, b0);  // after every transposed read of the step
  };

  // Prologue: codes of steps 0 and 1; dY of steps 0 and 1; tile buffer 0 = step 0;
  // the operands of step 0 read.
  u32x4 cA[kNV], cB[kNV];
  float aA, aB;
  load_codes(0, cA, aA);
  load_codes(nsteps > 1 ? 1 : 0, cB, aB);
  dma_y(0, 0);
  dma_y(nsteps > 1 ? 1 : 0, 1);
  {
    const WPrep<F> lut0 = wprep<F>(aA);
#pragma unroll
    for (int q = 0; q < 8; q += 2) dequant_write(0, cA, lut0, q);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));  // dY copies of step 0
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  read_b(0, 0, bv[0]);
  read_a(0, 0);
  read_a(0, 1);
  read_a(0, 2);
  read_a(0, 3);
  for (int s = 0; s < nsteps; s += 2) {
    body(s, cB, aB, cA, aA);
    if (s + 1 < nsteps) body(s + 1, cA, aA, cB, aB);
  }

  // ---- epilogue (no control flow): bf16 stores
  const __amdgpu_buffer_rsrc_t rO0 = make_rsrc(p.out0 + j0 * K, rows_here * K * 2);
  int jle = jl, he = h;  // fresh copies: no prologue offsets kept alive across the loop
  asm volatile("" : "+v"(jle), "+v"(he));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t mr = 32 * j + jle;
    const bool m_ok = mr < rows_here;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t ic = kc + 32 * f + 8 * q + 4 * he;
        const int off = (m_ok && ic < K) ? (int)((mr * K + ic) * 2) : kOff;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[f][j][4 * q + e];
        store4(rO0, off, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Two waves per SIMD (8 waves, 512 lanes), same 256 x 256 output tile:
// wave w owns the 64-column block w & 3 and the 128 tokens 128 (w >> 2) ..,
// so waves w and w + 4 -- the pair on one SIMD -- share one weight tile per
// step; each dequantizes 32 of its 64 rows (lane l: row 32 (w >> 2) + l % 32,
// columns 32 (l / 32) ..) and both read the whole tile after the step's
// barrier. With two waves on a SIMD, one wave's MFMAs run while the other
// waits on its VALU chains, LDS reads or the barrier.
template <int F, int MODE, int RP, bool ALIGNED>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void k_qgemm_bwd8(BwdArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // dY [2], then weight tiles [2][4 blocks]
  constexpr int NSRC = MODE == kConcat ? 2 : 1;
  constexpr int kNVh = kNV / 2;  // 16-byte code loads per lane and step (32 elements)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cb = wave & 3, th = wave >> 2;  // column block, token half
  const int h = lane >> 5, jl = lane & 31;
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t nJ = (M + kTok - 1) / kTok;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * 256, j0 = jt * kTok;
  const int sps = (int)((N + kStep - 1) / kStep);  // steps per source
  const int nsteps = sps * NSRC;
  const bool ragged = (N % kStep) != 0;
  const int64_t rows_here = (M - j0) < kTok ? (M - j0) : kTok;
  const int64_t kc = i0 + 64 * cb;  // the block's first output column
  const bool k_ok = kc < K;
  uint8_t* const wtile = smem + 2 * kBufB + cb * kWBufB;  // buffer b at + b * 4 * kWBufB

  // ---- dY copies: wave w fills tile rows 32w .. 32w+31 (4 instructions of 8
  // rows), physical chunk l%8 = logical chunk (l%8) ^ ((row>>1)&7).
  int offY[4], offYl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    offY[i] = (int)((int64_t)row * N * 2 + 16 * c);
    offYl[i] = (int64_t)(sps - 1) * kStep + 8 * c < N ? offY[i] : kOff;
  }
  auto dma_y = [&](int step, int buf) {
    const int src = NSRC > 1 && step >= sps ? 1 : 0;
    const int sl = step - src * sps;
    const bool last = ragged && sl == sps - 1;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY[src ? NSRC - 1 : 0] + j0 * N, rows_here * N * 2);
    uint8_t* base = smem + buf * kBufB + (32 * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (__attribute__((address_space(3))) void*)(base + 8 * i * kRowB), 16,
                                               last ? offYl[i] : offY[i], sl * kRowB, 0, 0);
  };

  // ---- codes and block value of weight row n0 + 32th + l%32, half l/32 of block kc/64
  constexpr int kHB = kCodeHalfBytes<F>;
  constexpr int64_t kBB = kBlock * kHB / 2;
  const int wrow = 32 * th + jl;
  const int offC = k_ok ? (int)(wrow * kBB + 16 * kNVh * h) : kOff;
  const int offA = k_ok ? wrow * 4 : kOff;
  auto load_codes = [&](int step, u32x4 (&cr)[kNVh], float& am) {
    const int src = NSRC > 1 && step >= sps ? 1 : 0;
    const int64_t n0 = (int64_t)(step - src * sps) * kStep;
    const WSrc& w = p.w[src ? NSRC - 1 : 0];
    const int64_t nr = (N - n0) < kStep ? (N - n0) : kStep;
    const int64_t jb = kc / kBlock;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(w.codes + n0 * (K / kBlock) * kBB + jb * nr * kBB, nr * kBB);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(w.absmax + n0 * (K / kBlock) + jb * nr, nr * 4);
#pragma unroll
    for (int v = 0; v < kNVh; ++v)
      cr[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, offC, 16 * v, 0));
    am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, offA, 0, 0));
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[f][j] = f32x16{};

  // ---- the rank-r term first: acc += (s.A^T rows) . (G rows)^T
#pragma unroll
  for (int src = 0; src < NSRC; ++src) {
    const WSrc& w = p.w[src];
    const __amdgpu_buffer_rsrc_t rA_ = make_rsrc(w.lora_i, K * (int64_t)w.r * 2);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(w.lora_j + j0 * w.ldj, rows_here * w.ldj * 2);
    const int c0 = 8 * h;
#pragma unroll
    for (int rr = 0; rr < RP; rr += 16) {
      u32x4 ah[2], al[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int64_t ir = kc + 32 * f + jl;
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e0 = rr + c0 + 2 * q, e1 = e0 + 1;
          const int o0 = (ir < K && e0 < w.r) ? (int)(((int64_t)e0 * K + ir) * 2) : kOff;
          const int o1 = (ir < K && e1 < w.r) ? (int)(((int64_t)e1 * K + ir) * 2) : kOff;
          wv[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA_, o0, 0, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA_, o1, 0, 0) << 16);
        }
        split_scaled(u32x4{wv[0], wv[1], wv[2], wv[3]}, w.s, ah[f], al[f]);
      }
      u32x4 z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t mr = 128 * th + 32 * j + jl;
        z[j] = rank8<ALIGNED>(rG, mr < rows_here ? mr : -1, w.ldj, w.r, rr + c0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[f][j] = mfma32(ah[f], z[j], acc[f][j]);
      // the low parts only where some lane has one (none when s is a power of two)
      if (lo_any(al[0], al[1])) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[f][j] = mfma32(al[f], z[j], acc[f][j]);
      }
    }
  }

  // ---- operand reads: dY token 128th + 32j + jl, reduction rows 16ks + 8h .. +7
  int offB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) offB[ks] = (128 * th + jl) * kRowB + 16 * ((2 * ks + h) ^ ((jl >> 1) & 7));
  u32x4 bv[2][4];
  auto read_b = [&](int buf, int ks, u32x4 (&dst)[4]) {
    const uint8_t* bx = smem + buf * kBufB + offB[ks];
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = *reinterpret_cast<const u32x4*>(bx + 32 * j * kRowB);
  };
  int offW[2][2];
  {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = 8 * (g >> 1) + (s >> 2) + 4 * hi;
        const int col = 32 * f + 16 * (g & 1) + 4 * (s & 3);
        offW[f][hi] = row * kWRowB + 16 * ((col >> 3) ^ wsw(row)) + 2 * (col & 7);
      }
  }
  u32x4 av[4][2];
  auto read_a = [&](int wb, int ks) {
    const uint8_t* wt = wtile + wb * 4 * kWBufB;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const u32x2 lo = lds_read_tr(wt + offW[f][0] + ks * 16 * kWRowB);
      const u32x2 hi = lds_read_tr(wt + offW[f][1] + ks * 16 * kWRowB);
      av[ks][f] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // this lane's half row: logical chunks 4h .. 4h+3 of row wrow
  const int wsl = wsw(wrow);
  auto dequant_write = [&](int wb, const u32x4 (&cr)[kNVh], const WPrep<F>& lut, int q0, int q1) {
    uint8_t* row = wtile + wb * 4 * kWBufB + wrow * kWRowB;
#pragma unroll
    for (int q = q0; q < q1; ++q)
      *reinterpret_cast<u32x4*>(row + 16 * ((4 * h + q) ^ wsl)) = wdeq8<F>(cr, q, lut);
  };
  auto mfmas = [&](const u32x4 (&a)[2], const u32x4 (&b)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[0][j] = mfma32(a[0], b[j], acc[0][j]);
      acc[1][j] = mfma32(a[1], b[j], acc[1][j]);
    }
  };
  auto interleave = [&](auto nds_read, auto nds_write, auto nvmem, auto nvalu) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < decltype(nds_read)::value) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i >= 8 - decltype(nds_write)::value) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      if (i < decltype(nvmem)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I8 = std::integral_constant<int, 8>;

  // Step s, as in the 4-wave kernel: substeps 0-2 dequantize this wave's half
  // of step s+1's tile (codes loaded during step s-1) and request step s+2's
  // codes; substep 3 follows the barrier and reads step s+1's operands.
  auto body = [&](int s, const u32x4 (&cc)[kNVh], float ac, u32x4 (&cn)[kNVh], float& an) {
    const int b0 = s & 1, b1 = b0 ^ 1;
    const int s2 = s + 2 < nsteps ? s + 2 : nsteps - 1;
    load_codes(s2, cn, an);
    const WPrep<F> lut = wprep<F>(ac);
    read_b(b0, 1, bv[1]);
    dequant_write(b1, cc, lut, 0, 2);
    mfmas(av[0], bv[0]);
    interleave(I4{}, I2{}, I2{}, I8{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(b0, 2, bv[0]);
    dequant_write(b1, cc, lut, 2, 3);
    mfmas(av[1], bv[1]);
    interleave(I4{}, I1{}, I0{}, I5{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(b0, 3, bv[1]);
    dequant_write(b1, cc, lut, 3, 4);
    mfmas(av[2], bv[0]);
    interleave(I4{}, I1{}, I0{}, I5{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's dY copies of step s+1 (and codes of s+2)
    __builtin_amdgcn_s_waitcnt(0xC07F);          // this wave's LDS reads and tile writes
    __builtin_amdgcn_s_barrier();
    mfmas(av[3], bv[1]);
    read_b(b1, 0, bv[0]);
    read_a(b1, 0);
    read_a(b1, 1);
    read_a(b1, 2);
    read_a(b1, 3);
    interleave(I8{}, I0{}, I0{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    dma_y(s2, b0);  // after every transposed read of the step
  };

  // Prologue: codes of steps 0 and 1; dY of steps 0 and 1; tile buffer 0 = step 0;
  // the operands of step 0 read.
  u32x4 cA[kNVh], cB[kNVh];
  float aA, aB;
  load_codes(0, cA, aA);
  load_codes(nsteps > 1 ? 1 : 0, cB, aB);
  dma_y(0, 0);
  dma_y(nsteps > 1 ? 1 : 0, 1);
  // the reductions of the preceding skinny_tn, one contiguous slice per
  // workgroup, while this prologue's loads are in flight
  if (p.red.n > 0) tn_reduce_slice(p.red, blockIdx.x, gridDim.x, threadIdx.x, 512);
  {
    const WPrep<F> lut0 = wprep<F>(aA);
    dequant_write(0, cA, lut0, 0, 4);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  read_b(0, 0, bv[0]);
  read_a(0, 0);
  read_a(0, 1);
  read_a(0, 2);
  read_a(0, 3);
  for (int s = 0; s < nsteps; s += 2) {
    body(s, cB, aB, cA, aA);
    if (s + 1 < nsteps) body(s + 1, cA, aA, cB, aB);
  }

  // ---- epilogue: tokens 128th + 32j + jl
  const __amdgpu_buffer_rsrc_t rO0 = make_rsrc(p.out0 + j0 * K, rows_here * K * 2);
  const __amdgpu_buffer_rsrc_t rO1 = make_rsrc(MODE == kSwiGLU ? p.out1 + j0 * K : p.out0,
                                               MODE == kSwiGLU ? rows_here * K * 2 : 0);
  const __amdgpu_buffer_rsrc_t rGs = make_rsrc(MODE == kSwiGLU ? p.g + j0 * K : p.out0,
                                               MODE == kSwiGLU ? rows_here * K * 2 : 0);
  const __amdgpu_buffer_rsrc_t rUs = make_rsrc(MODE == kSwiGLU ? p.u + j0 * K : p.out0,
                                               MODE == kSwiGLU ? rows_here * K * 2 : 0);
  if constexpr (MODE == kSwiGLU) {
    // SwiGLU backward through LDS: dh (fp32) of 64 tokens x 64 columns per wave
    // and half, token-major rows of 256 bytes (16-byte chunk c of row t at
    // c ^ (t & 15)); each lane then takes 8 consecutive columns of one token:
    // 16-byte loads of g and u, 16-byte stores of dg and du. The g, u loads of
    // a half are issued before its dh is parked, so their latency is hidden.
    __builtin_amdgcn_s_waitcnt(0);  // this wave's trailing dY copies have landed
    __builtin_amdgcn_s_barrier();   // and every wave is done with the buffers
    int jle = jl, he = h, lne = lane;
    asm volatile("" : "+v"(jle), "+v"(he), "+v"(lne));
    uint8_t* const reg = smem + wave * (64 * 256);
    const int c8 = lne & 7, tq = lne >> 3, rh = (int)rows_here, Ki = (int)K;
    const int col = (int)kc + 8 * c8;
    u32x4 gq[8], uq[8];
    auto off_of = [&](int hf, int u) {
      const int mr = 128 * th + 64 * hf + 8 * u + tq;
      return (mr < rh && col < Ki) ? (mr * Ki + col) * 2 : kOff;
    };
    auto load_gu = [&](int hf) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        gq[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rGs, off_of(hf, u), 0, 0));
        uq[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rUs, off_of(hf, u), 0, 0));
      }
    };
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      load_gu(hf);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int t = 32 * jj + jle;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[f][2 * hf + jj];
            *reinterpret_cast<f32x4*>(reg + t * 256 + 16 * ((8 * f + 2 * q + he) ^ (t & 15))) =
                f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          }
      }
      lds_barrier();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = 8 * u + tq;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(reg + t * 256 + 16 * ((2 * c8) ^ (t & 15)));
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(reg + t * 256 + 16 * ((2 * c8 + 1) ^ (t & 15)));
        const float dh[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        float dg[8], du[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gv = (e & 1) ? bf16_hi(gq[u][e >> 1]) : bf16_lo(gq[u][e >> 1]);
          const float uv = (e & 1) ? bf16_hi(uq[u][e >> 1]) : bf16_lo(uq[u][e >> 1]);
          const float sg = sigmoid_f(gv);
          dg[e] = dh[e] * uv * sg * (1.0f + gv * (1.0f - sg));
          du[e] = dh[e] * gv * sg;
        }
        const int off = off_of(hf, u);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]), pack_bf16x2(dg[4], dg[5]),
                  pack_bf16x2(dg[6], dg[7])},
            rO0, off, 0, kStoreNT);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]), pack_bf16x2(du[4], du[5]),
                  pack_bf16x2(du[6], du[7])},
            rO1, off, 0, kStoreNT);
      }
      lds_barrier();  // the half's reads are done before the next half is parked
    }
    return;
  }
  // dX through LDS (as in the forward GEMM): each wave parks its 128 tokens x 64
  // columns as bf16 in its own 16 KB of the idle buffers, rows of 128 bytes with
  // 16-byte chunk c of token row t at c ^ (t & 7), and stores 16-byte row pieces,
  // so that one store instruction writes whole 128-byte pieces of 8 rows.
  __builtin_amdgcn_s_waitcnt(0);  // this wave's trailing dY copies have landed
  __builtin_amdgcn_s_barrier();   // and every wave is done with the buffers
  int jle = jl, he = h, lne = lane;
  asm volatile("" : "+v"(jle), "+v"(he), "+v"(lne));
  uint8_t* const reg = smem + wave * (128 * 128);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
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
  const int c = lne & 7, tq = lne >> 3, rh = (int)rows_here;
  const int64_t col = kc + 8 * c;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int t = 8 * u + tq, mr = 128 * th + t;
    const u32x4 v = *reinterpret_cast<const u32x4*>(reg + t * 128 + 16 * (c ^ (t & 7)));
    const int off = (mr < rh && col < K) ? (int)((mr * K + col) * 2) : kOff;
    __builtin_amdgcn_raw_buffer_store_b128(v, rO0, off, 0, kStoreNT);
  }
}

template <int MODE, int RP, bool ALIGNED>
hipError_t launch_rp(const BwdArgs& a, hipStream_t st) {
  // The 8-wave kernel (measured 3-7% faster than the 4-wave one for every
  // mode), except at rank 256 with two sources, whose rank term does not fit
  // its 256 registers per lane.
  constexpr bool k8 = !(MODE == kConcat && RP >= 256);
  const void* kfn;
  if constexpr (k8)
    kfn = (const void*)k_qgemm_bwd8<kFmt, MODE, RP, ALIGNED>;
  else
    kfn = (const void*)k_qgemm_bwd<kFmt, MODE, RP, ALIGNED>;
  // set once per kernel instance; a function-local static is initialised exactly
  // once even when several threads make their first call together
  static const hipError_t attr = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int64_t nI = (a.K + 255) / 256, nJ = (a.M + kTok - 1) / kTok;
  if (nI * nJ == 0) return a.red.n ? launch_tn_reduce(a.red, st) : hipSuccess;
  if constexpr (k8) {
    k_qgemm_bwd8<kFmt, MODE, RP, ALIGNED><<<(unsigned)(nI * nJ), 512, kLds, st>>>(a);
  } else {  // the 4-wave kernel leaves the reductions to their own launch
    k_qgemm_bwd<kFmt, MODE, RP, ALIGNED><<<(unsigned)(nI * nJ), 256, kLds, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.red.n) return e;
    return launch_tn_reduce(a.red, st);
  }
  return hipGetLastError();
}

bool rank_rows_aligned(const WSrc& w) {
  return w.r % 8 == 0 && w.ldj % 8 == 0 && (reinterpret_cast<uintptr_t>(w.lora_j) & 15) == 0;
}

template <int MODE, int RP>
hipError_t launch_al(const BwdArgs& a, hipStream_t st) {
  const bool aligned = rank_rows_aligned(a.w[0]) && rank_rows_aligned(a.w[1]);
  return aligned ? launch_rp<MODE, RP, true>(a, st) : launch_rp<MODE, RP, false>(a, st);
}

template <int MODE>
hipError_t launch(const BwdArgs& a, hipStream_t st) {
  const int r = a.w[0].r > a.w[1].r ? a.w[0].r : a.w[1].r;
  if (r <= 16) return launch_al<MODE, 16>(a, st);
  if (r <= 32) return launch_al<MODE, 32>(a, st);
  if (r <= 64) return launch_al<MODE, 64>(a, st);
  if (r <= 128) return launch_al<MODE, 128>(a, st);
  if (r <= 256) return launch_al<MODE, 256>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

namespace QL_FMT_NS {

hipError_t launch_gemm_bwd(const uint16_t* dY0, WSrc w0, const uint16_t* dY1, WSrc w1, int64_t M, int64_t K,
                           int64_t N, uint16_t* dX, const TnJobs* red, hipStream_t st) {
  BwdArgs a{};
  if (red) a.red = *red;
  a.dY[0] = dY0;
  a.dY[1] = dY1 ? dY1 : dY0;
  a.w[0] = w0;
  a.w[1] = dY1 ? w1 : w0;
  a.M = M, a.K = K, a.N = N;
  a.out0 = dX;
  return dY1 ? launch<kConcat>(a, st) : launch<kPlain>(a, st);
}

hipError_t launch_gemm_bwd_swiglu(const uint16_t* dY, WSrc w, int64_t M, int64_t K, int64_t N, const uint16_t* g,
                                  const uint16_t* u, uint16_t* dg, uint16_t* du, const TnJobs* red, hipStream_t st) {
  BwdArgs a{};
  if (red) a.red = *red;
  a.dY[0] = a.dY[1] = dY;
  a.w[0] = a.w[1] = w;
  a.M = M, a.K = K, a.N = N;
  a.out0 = dg, a.out1 = du;
  a.g = g, a.u = u;
  return launch<kSwiGLU>(a, st);
}

}  // namespace QL_FMT_NS

}  // namespace qlora
