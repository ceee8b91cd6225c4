// Small-batch path of the fused QLoRA layer (gfx950): batches of at most
// kSmallMaxM tokens and ranks up to 32. The 256 x 256 tiles of the main GEMMs
// give such a batch a handful of workgroups (two at 256 tokens x 512 outputs)
// and the rank-r steps cost a launch each, so here one workgroup computes a
// 32 x 32 output tile and does the rank-r products of its own tile alongside,
// which leaves three launches per forward + backward. The reduction is split
// over the workgroup's kKS waves (wave w takes 64-deep blocks w, w + kKS, ..,
// each wave prefetching its next block): a short reduction is then a few
// load round trips deep instead of one per block. The waves' fp32 partial
// products are added in wave order (fixed, so runs repeat bit for bit), and
// wave 0 finishes the tile:
//   forward  k_small_fwd: Y = X.What^T + s.Z.B^T and Z = X.A^T (Z formed by the
//            wave from the X fragments it loads anyway; the workgroups of the
//            first column tile write it out);
//   backward k_small_bwd: dX = dY.What + s.G.A with G = dY.B formed from the
//            dY fragments it loads anyway (the first column tile writes G);
//            then skinny_tn gives dB = s.dY^T.Z and dA = s.G^T.X in one split.
// Method: "Rev vs unsloth", fused quantized-LoRA card (4-bit weight and adapter
// as one layer, no dequantized weight in HBM); "Unsloth vs PyTorch" video,
// 1:35-2:00 (the rank-r products bracketed through the M x r tensors).
#include "common.hpp"
#include "internal.hpp"

namespace qlora {

namespace {

constexpr int kT = 32;   // tokens per workgroup, and output columns (fwd: weight rows; bwd: input features)
constexpr int kRS = 32;  // rank slots (r <= 32, zero past r)
constexpr int kKS = 4;   // waves per workgroup, splitting the reduction

// wave 0's a and b += the partial products that waves 1 .. kKS-1 left in part,
// in wave order. Every wave of the workgroup calls it; the other waves return
// false and are done.
__device__ __forceinline__ bool sum_waves(f32x16 (&part)[kKS - 1][2][64], int wave, int lane, f32x16& a,
                                          f32x16& b) {
  if (wave > 0) {
    part[wave - 1][0][lane] = a;
    part[wave - 1][1][lane] = b;
  }
  __syncthreads();
  if (wave > 0) return false;
#pragma unroll
  for (int w = 0; w < kKS - 1; ++w) {
    a += part[w][0][lane];
    b += part[w][1][lane];
  }
  return true;
}

// ---------------------------------------------------------------------------
// Forward. Lane l: weight row n0 + l%32 and input column half l/32 of each
// 16-wide substep (A operand of the 32x32x16 MFMA), token m0 + l%32 (B operand).
// Codes and block values are read from the tile-major storage: the 32 rows of
// a workgroup lie in one 64-row group, whose block b holds its nr rows' codes
// one after the other.
template <int F, bool ALIGNED>
__global__ __launch_bounds__(64 * kKS) void k_small_fwd(SmallFwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t zt[kT * kRS];  // Z tile [token][rank] bf16
  __shared__ f32x16 part[kKS - 1][2][64];                          // partial Y and Z products of waves 1..
  const int lane = threadIdx.x & 63, jl = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t nJ = (M + kT - 1) / kT;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t n0 = kT * it, m0 = kT * jt;
  const int64_t rows_here = (M - m0) < kT ? (M - m0) : kT;
  const int r = p.r;
  constexpr int64_t kBB = kBlock * kCodeHalfBytes<F> / 2;  // code bytes per row and block
  const int64_t grp = n0 - n0 % 64;
  const int64_t nr = (N - grp) < 64 ? (N - grp) : 64;  // rows of the 64-row group
  const int64_t nblk = K / kBlock;
  const int64_t n = n0 + jl;
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(p.codes + grp * nblk * kBB, nr * nblk * kBB);
  const __amdgpu_buffer_rsrc_t rAm = make_rsrc(p.absmax + grp * nblk, nr * nblk * 4);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.X + m0 * K, rows_here * K * 2);
  const __amdgpu_buffer_rsrc_t rLA = make_rsrc(p.A, (int64_t)r * K * 2);
  // per-lane offsets; the block advances by nr rows of codes / values
  const int offc = n < N ? (int)((n - grp) * kBB) : kOff;
  const int offa = n < N ? (int)((n - grp) * 4) : kOff;
  const int offx = (int)((jl * K + 8 * h) * 2);          // rows past the batch read zero
  const int offla = jl < r ? (int)((jl * K + 8 * h) * 2) : kOff;
  const int cstep = (int)(nr * kBB), astep = (int)(nr * 4);

  struct Blk {
    u32x4 c[4];  // codes of substep ks in c[ks] (NF4: one dword, 8-bit: two)
    u32x4 x[4], la[4];
    float am;
  };
  auto load = [&](int64_t b, Blk& t) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cb = 16 * ks + 8 * h;  // first column of this lane's 8 in the block
      if constexpr (F == kNF4) {
        t.c[ks] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rC, offc == kOff ? kOff : offc + 4 * (cb / 8),
                                                             (int)(b * cstep), 0), 0u, 0u, 0u};
      } else {
        const u32x2 v = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rC, offc == kOff ? kOff : offc + cb, (int)(b * cstep), 0));
        t.c[ks] = u32x4{v[0], v[1], 0u, 0u};
      }
      const int kk2 = (int)((b * kBlock + 16 * ks) * 2);
      t.x[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, offx, kk2, 0));
      t.la[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rLA, offla, kk2, 0));
    }
    t.am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rAm, offa, (int)(b * astep), 0));
  };

  f32x16 acc = f32x16{}, accz = f32x16{};
  Blk cur, nxt;
  if (wave < nblk) load(wave, cur);
  for (int64_t b = wave; b < nblk; b += kKS) {
    if (b + kKS < nblk) load(b + kKS, nxt);
    const WPrep<F> prep = wprep<F>(cur.am);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 cw[1] = {cur.c[ks]};
      acc = mfma32(wdeq8<F, 1>(cw, 0, prep), cur.x[ks], acc);  // D[weight row][token]
      accz = mfma32(cur.la[ks], cur.x[ks], accz);              // D[rank][token]
    }
    cur = nxt;
  }
  if (!sum_waves(part, wave, lane, acc, accz)) return;

  // wave 0 from here. Z in bf16 (lane: token jl, ranks 8q + 4h .. +3): the LDS
  // tile for the rank term (written and read back by this wave alone), and the
  // saved Z from the first column tile
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x2*>(&zt[jl * kRS + 8 * q + 4 * h]) =
        u32x2{pack_bf16x2(accz[4 * q], accz[4 * q + 1]), pack_bf16x2(accz[4 * q + 2], accz[4 * q + 3])};
  if (it == 0 && jl < rows_here) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rk = 8 * q + 4 * h + e;
        if (rk < r) p.Z[(m0 + jl) * r + rk] = zt[jl * kRS + rk];
      }
  }
  // rank term: acc += (s.B rows) . (Z rows)^T, s.B split hi + lo on the operand
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B, N * (int64_t)r * 2);
#pragma unroll
  for (int rr = 0; rr < kRS; rr += 16) {
    if (rr >= r) break;
    u32x4 bh, bl;
    split_scaled(rank8<ALIGNED>(rB, n < N ? n : -1, r, r, rr + 8 * h), p.s, bh, bl);
    const u32x4 z = *reinterpret_cast<const u32x4*>(&zt[jl * kRS + rr + 8 * h]);
    acc = mfma32(bh, z, acc);
    acc = mfma32(bl, z, acc);
  }
  // Y (lane: token jl, weight rows 8q + 4h .. +3)
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(p.Y + m0 * N, rows_here * N * 2);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t ic = n0 + 8 * q + 4 * h;
    const int off = (jl < rows_here && ic < N) ? (int)((jl * N + ic) * 2) : kOff;
    const float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    store4(rY, off, v);
  }
}

// ---------------------------------------------------------------------------
// Backward dX and G. Workgroup = input columns kc .. kc+31 x tokens m0 .. m0+31.
// Per 64-row step of the reduction over N: lane l dequantizes weight row n0 + l,
// columns kc .. kc+31 (one (row, block) table) into the LDS tile wt [64][32] and
// copies that row of B (ranks 0..31, zero past r) into bt [64][32]; both are read
// column-wise with ds_read_b64_tr_b16 (lane: column l%32, rows 8(l/32) .. +7 of
// the substep), which is the A operand of dX = What^T . dY^T and the B operand of
// G = dY . B. The dY fragment (token l%32, 8 rows) serves both products.
template <int F, bool ALIGNED>
__global__ __launch_bounds__(64 * kKS) void k_small_bwd(SmallBwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t wts[kKS][64 * kT];   // per wave: weight rows x 32 columns
  __shared__ __attribute__((aligned(16))) uint16_t bts[kKS][64 * kRS];  // per wave: B rows x 32 ranks
  __shared__ __attribute__((aligned(16))) uint16_t gt[kT * kRS];        // G [token][rank] bf16
  __shared__ f32x16 part[kKS - 1][2][64];                               // partial dX and G products of waves 1..
  const int lane = threadIdx.x & 63, jl = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t* const wt = wts[wave];  // private to the wave: its own writes and reads, in order, need no barrier
  uint16_t* const bt = bts[wave];
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t nJ = (M + kT - 1) / kT;
  const int64_t ik = blockIdx.x / nJ, jt = blockIdx.x - ik * nJ;
  const int64_t kc = kT * ik, m0 = kT * jt;
  const int64_t rows_here = (M - m0) < kT ? (M - m0) : kT;
  const int r = p.r;
  constexpr int64_t kBB = kBlock * kCodeHalfBytes<F> / 2;
  constexpr int kNVs = F == kNF4 ? 1 : 2;  // 16-byte code loads per lane and step (32 columns)
  const int64_t nblk = K / kBlock, jb = kc / kBlock;
  const int hoff = (int)(((kc % kBlock) / kT) * kBB / 2);  // this column half's bytes in the row's block
  const int nsteps = (int)((N + 63) / 64);
  const __amdgpu_buffer_rsrc_t rdY = make_rsrc(p.dY + m0 * N, rows_here * N * 2);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B, N * (int64_t)r * 2);
  // transposed-read address of lane (group g = l/16, s = l%16): row 8(g>>1) + (s>>2)
  // (+4 for the second half of the 8), column 16(g&1) + 4(s&3); rows advance by 16 per substep
  const int g = lane >> 4, sl = lane & 15;
  const int trow = 8 * (g >> 1) + (sl >> 2), tcol = 16 * (g & 1) + 4 * (sl & 3);

  struct Stp {
    u32x4 c[kNVs];
    float am;
    u32x4 brow[4];
    u32x4 dy[4];
  };
  auto load = [&](int st, Stp& t) {
    const int64_t n0 = 64 * (int64_t)st;
    const int64_t nr = (N - n0) < 64 ? (N - n0) : 64;  // rows of this 64-row group
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes + n0 * nblk * kBB + jb * nr * kBB, nr * kBB);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.absmax + n0 * nblk + jb * nr, nr * 4);
#pragma unroll
    for (int v = 0; v < kNVs; ++v)
      t.c[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(lane * kBB) + hoff, 16 * v, 0));
    t.am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, lane * 4, 0, 0));
    const int64_t nrow = n0 + lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) t.brow[c] = rank8<ALIGNED>(rB, nrow < N ? nrow : -1, r, r, 8 * c);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int64_t nc = n0 + 16 * ks + 8 * h;  // N % 8 == 0: a group of 8 is wholly in or out
      const int off = nc < N ? (int)((jl * N + nc) * 2) : kOff;
      t.dy[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdY, off, 0, 0));
    }
  };

  f32x16 acc = f32x16{}, accg = f32x16{};
  Stp cur, nxt;
  if (wave < nsteps) load(wave, cur);
  for (int st = wave; st < nsteps; st += kKS) {
    if (st + kKS < nsteps) load(st + kKS, nxt);
    const WPrep<F> prep = wprep<F>(cur.am);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<u32x4*>(&wt[lane * kT + 8 * c]) = wdeq8<F, kNVs>(cur.c, c, prep);
      *reinterpret_cast<u32x4*>(&bt[lane * kRS + 8 * c]) = cur.brow[c];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int o0 = (16 * ks + trow) * kT + tcol, o1 = o0 + 4 * kT;
      const u32x2 w0 = lds_read_tr(&wt[o0]), w1 = lds_read_tr(&wt[o1]);
      const u32x2 b0 = lds_read_tr(&bt[o0]), b1 = lds_read_tr(&bt[o1]);
      acc = mfma32(u32x4{w0[0], w0[1], w1[0], w1[1]}, cur.dy[ks], acc);   // D[input column][token]
      accg = mfma32(cur.dy[ks], u32x4{b0[0], b0[1], b1[0], b1[1]}, accg);  // D[token][rank]
    }
    cur = nxt;
  }
  if (!sum_waves(part, wave, lane, acc, accg)) return;

  // wave 0 from here. G in bf16 (lane: rank jl, tokens 8q + 4h .. +3) into gt
  // [token][rank], written and read back by this wave alone
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      gt[(8 * q + 4 * h + e) * kRS + jl] = __builtin_bit_cast(uint16_t, (__bf16)accg[4 * q + e]);
  if (ik == 0 && jl < rows_here) {  // G rows of this token tile: token jl, ranks 16h .. 16h+15
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rk = 16 * h + e;
      if (rk < r) p.G[(m0 + jl) * r + rk] = gt[jl * kRS + rk];
    }
  }
  // rank term: acc += (s.A^T rows) . (G rows)^T; A read in place, [r, K]
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, K * (int64_t)r * 2);
  const int64_t col = kc + jl;
#pragma unroll
  for (int rr = 0; rr < kRS; rr += 16) {
    if (rr >= r) break;
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e0 = rr + 8 * h + 2 * q, e1 = e0 + 1;
      const int o0 = e0 < r ? (int)(((int64_t)e0 * K + col) * 2) : kOff;
      const int o1 = e1 < r ? (int)(((int64_t)e1 * K + col) * 2) : kOff;
      wv[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA, o0, 0, 0) |
              ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA, o1, 0, 0) << 16);
    }
    u32x4 ah, al;
    split_scaled(u32x4{wv[0], wv[1], wv[2], wv[3]}, p.s, ah, al);
    const u32x4 gz = *reinterpret_cast<const u32x4*>(&gt[jl * kRS + rr + 8 * h]);
    acc = mfma32(ah, gz, acc);
    acc = mfma32(al, gz, acc);
  }
  // dX (lane: token jl, input columns 8q + 4h .. +3)
  const __amdgpu_buffer_rsrc_t rO = make_rsrc(p.dX ? p.dX + m0 * K : nullptr, p.dX ? rows_here * K * 2 : 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t ic = kc + 8 * q + 4 * h;
    const int off = jl < rows_here ? (int)((jl * K + ic) * 2) : kOff;
    const float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    store4(rO, off, v);
  }
}

}  // namespace

hipError_t launch_small_fwd(const SmallFwdArgs& a, int fmt, hipStream_t st) {
  if (a.r < 1 || a.r > kSmallMaxR || a.M < 1) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((a.N + kT - 1) / kT) * ((a.M + kT - 1) / kT));
  const bool al = a.r % 8 == 0;
#define QL_SF(FM)                                               \
  do {                                                          \
    if (al)                                                     \
      k_small_fwd<FM, true><<<grid, 64 * kKS, 0, st>>>(a);            \
    else                                                        \
      k_small_fwd<FM, false><<<grid, 64 * kKS, 0, st>>>(a);           \
  } while (0)
  if (fmt == kNF4)
    QL_SF(kNF4);
  else if (fmt == kInt8)
    QL_SF(kInt8);
  else
    QL_SF(kFp8);
#undef QL_SF
  return hipGetLastError();
}

hipError_t launch_small_bwd(const SmallBwdArgs& a, int fmt, hipStream_t st) {
  if (a.r < 1 || a.r > kSmallMaxR || a.M < 1) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((a.K + kT - 1) / kT) * ((a.M + kT - 1) / kT));
  const bool al = a.r % 8 == 0;
#define QL_SB(FM)                                               \
  do {                                                          \
    if (al)                                                     \
      k_small_bwd<FM, true><<<grid, 64 * kKS, 0, st>>>(a);            \
    else                                                        \
      k_small_bwd<FM, false><<<grid, 64 * kKS, 0, st>>>(a);           \
  } while (0)
  if (fmt == kNF4)
    QL_SB(kNF4);
  else if (fmt == kInt8)
    QL_SB(kInt8);
  else
    QL_SB(kFp8);
#undef QL_SB
  return hipGetLastError();
}

}  // namespace qlora
