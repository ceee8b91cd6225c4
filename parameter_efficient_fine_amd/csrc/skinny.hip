// Skinny rank-r products of the LoRA path (gfx950).
//
// "Unsloth vs PyTorch" video, 1:35-2:00: the adapters are skinny (rank 8 to
// 128) against 4096-wide weights, so the products are bracketed to keep every
// intermediate M x r (or r x K) and never form the N x K matrix B.A.
//   skinny_nt:  Z = X.A^T  and  G = dY.B            ([M,Kd] x [r,Kd]^T -> [M,r])
//   skinny_tn:  dA = s.G^T.X  and  dB^T = s.Z^T.dY  ([M,r]^T x [M,Kd] -> [r,Kd])
// Both read their big operand once and are HBM-bound; MFMA 16x16x32 does the
// arithmetic, and the kernels are built to keep many loads in flight.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "reduce.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// skinny_nt: 16*RF rows of `in` per workgroup (RF row fragments; RF > 1 when
// M is large enough to keep one workgroup per CU, so each adapter fragment
// loaded serves RF fragments of `in`). The waves interleave over the 32-wide
// k steps (wave w takes steps w, w + NW, ...) and issue U steps of loads at
// once. `in` is read through a buffer resource covering the workgroup's rows:
// a lane's row and k position form a loop-invariant VGPR offset, the step a
// scalar offset, and rows past M read zero -- the loop has no per-lane
// condition (a per-lane select there turns into divergent branches that
// serialize the loads). The steps a wave owns are done in batches of U, then
// U/2, .., 1 (binary remainder); a ragged last step (Kd % 32 != 0) is done
// apart with masks. Per-wave partial sums are combined by a fixed-order tree
// in LDS, one row fragment at a time. RP = r1 + r2 rounded up to 16.
//
// KT: the adapter is given as [Kd, R] (R = RP), the layout of B in G = dY.B,
// so no transposed copy is made. Each wave copies the adapter rows of a step
// (32 x R bf16, one contiguous run) into its own LDS slot with buffer_load ...
// lds and reads the MFMA operand column-wise with ds_read_b64_tr_b16.
// KA: a single adapter given as [R, Kd] (A in Z = X.A^T) goes through the same
// LDS slots, R rows of 64 bytes per step, and is read back row-wise. Otherwise
// (two stacked adapters) each lane loads its adapter row piece directly.

template <int RP, int RF>
struct NtShape {
  static constexpr int NF = RP / 16;            // 16-row adapter fragments
  static constexpr int NW = RP >= 256 ? 4 : 8;  // waves
  static constexpr int U0 = RP <= 32 ? 16 : (RP <= 64 ? 4 : (RP <= 128 ? 2 : 1));
  static constexpr int U = U0 / RF > 0 ? U0 / RF : 1;  // steps per batch
};

template <int RP, int RF, bool KT, bool KA>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NtShape<RP, RF>::NW, 64 * NtShape<RP, RF>::NW)))
void k_skinny_nt(NtArgs p) {
  constexpr bool KL = KT || KA;  // adapter steps staged in LDS
  constexpr int NF = NtShape<RP, RF>::NF, NW = NtShape<RP, RF>::NW;
  // KT: at most 16 KB of adapter slots per wave (8 KB from rank 128 on, next to the
  // larger reduction buffer)
  constexpr int kUK = (RP >= 128 ? 128 : 256) / RP > 0 ? (RP >= 128 ? 128 : 256) / RP : 1;
  constexpr int U = KL && NtShape<RP, RF>::U > kUK ? kUK : NtShape<RP, RF>::U;
  __shared__ float red[NW / 2][16][RP + 4];
  __shared__ __attribute__((aligned(16))) uint16_t kts[KL ? NW * U * 32 * RP : 8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = p.M, Kd = p.Kd;
  const int64_t m0 = (int64_t)blockIdx.x * 16 * RF;
  const int R = p.r1 + p.r2;
  const int64_t rows_here = (M - m0) < 16 * RF ? (M - m0) : 16 * RF;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.in + m0 * Kd, rows_here * Kd * 2);
  const int row = lane & 15, kofs = 8 * (lane >> 4);
  int voff[RF];
#pragma unroll
  for (int rf = 0; rf < RF; ++rf) voff[rf] = (int)(((16 * rf + row) * Kd + kofs) * 2);

  const uint16_t* adp[NF];  // this lane's adapter row, at its k offset
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int j = 16 * f + row;
    const int jc = j < R ? j : 0;
    adp[f] = (jc < p.r1 ? p.ad1 + (int64_t)jc * Kd : p.ad2 + (int64_t)(jc - p.r1) * Kd) + kofs;
  }
  // KT: adapter rows of step st = bytes [64 R st, 64 R (st + 1)) of ad1; lane l of
  // copy instruction i moves bytes 16 (64 i + l) of the run. Transposed reads:
  // in 16-lane group g, lane s points at row 8g + s/4 (+4), columns 16f + 4 (s%4)
  // of the 32 x RP slot; lane i then holds rows 8g .. 8g+7 of column 16f + i.
  // KA: a single adapter stored [R, Kd]; step st's block is R rows of 64 bytes at
  // column offset 64 st. Lane l of copy instruction i moves row 16i + l/4, bytes
  // 16 (l%4) of it, so the slot holds the block row-major (64 bytes per row) and
  // lane l then reads row 16f + l%16, bytes 16 (l/16): its MFMA operand. Rows past
  // R are out of range of the resource and read zero.
  const __amdgpu_buffer_rsrc_t rad =
      make_rsrc(p.ad1, KT ? Kd * RP * 2 : (KA ? (int64_t)p.r1 * Kd * 2 : 0));
  uint16_t* const kslot = kts + (KL ? wave * U * 32 * RP : 0);
  const int kd32 = (int)Kd;  // KA: row 16i + l/4 at byte (16i + l/4) Kd 2 + 16 (l%4)
  const int kaoff0 = (lane >> 2) * kd32 * 2 + 16 * (lane & 3);
  auto ka_read = [&](int u, u32x4 (&dst)[NF]) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(kslot + u * 32 * RP) + (lane & 15) * 64 + 16 * (lane >> 4);
#pragma unroll
    for (int f = 0; f < NF; ++f) dst[f] = *reinterpret_cast<const u32x4*>(base + f * 1024);
  };
  const int ktr = ((8 * (lane >> 4) + ((lane & 15) >> 2)) * RP + 4 * (lane & 3)) * 2;
  auto kt_copy = [&](int u, int64_t st) {  // KT and KA: step st's adapter block into slot u
#pragma unroll
    for (int i = 0; i < RP / 16; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rad, (__attribute__((address_space(3))) void*)(kslot + u * 32 * RP + i * 512), 16,
          KT ? (64 * i + lane) * 16 : kaoff0 + 32 * i * kd32, (int)(st * 64 * (KT ? RP : 1)), 0, 0);
  };
  auto kt_read = [&](int u, u32x4 (&dst)[NF]) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(kslot + u * 32 * RP) + ktr;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const u32x2 lo = lds_read_tr(base + 32 * f);
      const u32x2 hi = lds_read_tr(base + 32 * f + 8 * RP);
      dst[f] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };

  f32x4 acc[RF][NF];
#pragma unroll
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[rf][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // V full steps starting at this wave's step index i0: loads first, then MFMAs
  auto batch = [&](auto vtag, int64_t i0) {
    constexpr int V = decltype(vtag)::value;
    u32x4 a[V][RF], b[V][NF];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int64_t st = wave + NW * (i0 + u);
#pragma unroll
      for (int rf = 0; rf < RF; ++rf)
        a[u][rf] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, voff[rf], (int)(st * 64), 0));
      if constexpr (KT) {
        kt_copy(u, st);
      } else if constexpr (KA) {
        kt_copy(u, st);
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) b[u][f] = *reinterpret_cast<const u32x4*>(adp[f] + st * 32);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch goes out before the first MFMA waits
    if constexpr (KL) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's adapter copies (and activation loads)
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if constexpr (KT)
          kt_read(u, b[u]);
        else
          ka_read(u, b[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < V; ++u)
#pragma unroll
      for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[rf][f] = mfma16(a[u][rf], b[u][f], acc[rf][f]);
  };
  const int64_t nfull = Kd / 32;  // steps with all 32 columns in range
  const int64_t cnt = nfull > wave ? (nfull - wave + NW - 1) / NW : 0;
  int64_t i = 0;
  for (; i + U <= cnt; i += U) batch(std::integral_constant<int, U>{}, i);
  if constexpr (U >= 16) if (i + 8 <= cnt) { batch(std::integral_constant<int, 8>{}, i); i += 8; }
  if constexpr (U >= 8) if (i + 4 <= cnt) { batch(std::integral_constant<int, 4>{}, i); i += 4; }
  if constexpr (U >= 4) if (i + 2 <= cnt) { batch(std::integral_constant<int, 2>{}, i); i += 2; }
  if constexpr (U >= 2) if (i + 1 <= cnt) { batch(std::integral_constant<int, 1>{}, i); i += 1; }
  if (nfull * 32 < Kd && wave == nfull % NW) {  // ragged last step, masked per lane
    const int64_t k = nfull * 32 + kofs;
    const bool ok = k < Kd;
    u32x4 b[NF];
    if constexpr (KT) {  // adapter rows past Kd read zero (buffer range)
      kt_copy(0, nfull);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      kt_read(0, b);
    } else if constexpr (KA) {  // columns past Kd: masked below
      kt_copy(0, nfull);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      ka_read(0, b);
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f) b[f] = *reinterpret_cast<const u32x4*>(adp[f] + (ok ? nfull * 32 : 0));
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
      if (!ok) b[f] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
      u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, voff[rf], (int)(nfull * 64), 0));
      if (!ok) a = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[rf][f] = mfma16(a, b[f], acc[rf][f]);
    }
  }

  // per row fragment, a fixed-order tree over the waves: (w, w + h) pairs for
  // h = NW/2, NW/4, .., 1. C layout: col j = lane%16 (adapter row),
  // row i = 4*(lane/16) + v (token row)
#pragma unroll
  for (int rf = 0; rf < RF; ++rf) {
#pragma unroll
    for (int h = NW / 2; h >= 1; h >>= 1) {
      if (wave >= h && wave < 2 * h) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave - h][4 * (lane >> 4) + v][16 * f + row] = acc[rf][f][v];
      }
      __syncthreads();
      if (wave < h) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rf][f][v] += red[wave][4 * (lane >> 4) + v][16 * f + row];
      }
      __syncthreads();
    }
  }
  if (wave != 0) return;
#pragma unroll
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int j = 16 * f + row;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 16 * rf + 4 * (lane >> 4) + v;
        if (m >= M || j >= R) continue;
        const uint16_t hv = __builtin_bit_cast(uint16_t, (__bf16)acc[rf][f][v]);
        if (j < p.r1)
          p.out1[m * p.ld1 + j] = hv;
        else
          p.out2[m * p.ld2 + (j - p.r1)] = hv;
      }
    }
}

template <int RP, bool KT, bool KA = false>
hipError_t launch_nt_rf(const NtArgs& a, hipStream_t st) {
  // row fragments per workgroup: as many as still leave >= 256 workgroups
  // (at most 2 for RP = 256, whose accumulators would spill at 4)
  constexpr int kMaxRF = RP >= 256 ? 2 : 4;
  int rf = 1;
  while (rf < kMaxRF && (a.M + 32 * rf - 1) / (32 * rf) >= 256) rf *= 2;
  const unsigned grid = (unsigned)((a.M + 16 * rf - 1) / (16 * rf));
  if (rf == 1)
    k_skinny_nt<RP, 1, KT, KA><<<grid, 64 * NtShape<RP, 1>::NW, 0, st>>>(a);
  else if (rf == 2)
    k_skinny_nt<RP, 2, KT, KA><<<grid, 64 * NtShape<RP, 2>::NW, 0, st>>>(a);
  else if constexpr (kMaxRF >= 4)
    k_skinny_nt<RP, 4, KT, KA><<<grid, 64 * NtShape<RP, 4>::NW, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_skinny_nt(const NtArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int R = a.r1 + a.r2;
  if (a.ad_kr) {  // a single adapter stored [Kd, R]
    if (a.r2 != 0) return hipErrorInvalidValue;  // R = 16, 32, 64, 128 or 256 below
    if (R == 16) return launch_nt_rf<16, true>(a, st);
    if (R == 32) return launch_nt_rf<32, true>(a, st);
    if (R == 64) return launch_nt_rf<64, true>(a, st);
    if (R == 128) return launch_nt_rf<128, true>(a, st);
    if (R == 256) return launch_nt_rf<256, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.r2 == 0) {  // a single adapter stored [R, Kd]: its steps staged in LDS
    if (R <= 16) return launch_nt_rf<16, false, true>(a, st);
    if (R <= 32) return launch_nt_rf<32, false, true>(a, st);
    if (R <= 64) return launch_nt_rf<64, false, true>(a, st);
    if (R <= 128) return launch_nt_rf<128, false, true>(a, st);
    if (R <= 256) return launch_nt_rf<256, false, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (R <= 16) return launch_nt_rf<16, false>(a, st);
  if (R <= 32) return launch_nt_rf<32, false>(a, st);
  if (R <= 64) return launch_nt_rf<64, false>(a, st);
  if (R <= 128) return launch_nt_rf<128, false>(a, st);
  if (R <= 256) return launch_nt_rf<256, false>(a, st);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// skinny_tn: out = s * P[M, R]^T . Q[M, Kd], reduced over the M rows (R <= 128).
//
// Workgroup = 128 columns of Q (4 waves x 32) x one split of the rows. Rows
// go 64 at a time through LDS, where both operands are read column-wise with
// ds_read_b64_tr_b16 (each lane then holds 8 consecutive rows: the reduction
// dimension). Two register sets keep the next two 64-row tiles in flight while
// one is consumed. Each split stores an fp32 partial; k_tn_reduce then adds
// the partials in split order (deterministic), scales, and writes the result
// (or adds it to the output, when a batch is reduced tile by tile).

constexpr int kTnCols = 128;
constexpr int kTnRows = 64;
constexpr int kTnQS = kTnCols + 16;  // LDS row stride (bf16): 8 banks between rows

TnPlan skinny_tn_plan(int64_t M, int64_t Kd, int R) {
  TnPlan pl;
  if (M < 1) M = 1;  // an empty batch launches nothing; size as for one row
  pl.col_tiles = (int)((Kd + kTnCols - 1) / kTnCols);
  const int64_t RR = (R + 15) / 16 * 16;
  // ~1 workgroup per CU (against ~2: half the partials for the reduction to add,
  // attn step -0.7%; the rank-128 and SwiGLU steps unchanged)
  int64_t splits = (256 + pl.col_tiles - 1) / pl.col_tiles;
  const int64_t by_traffic = M / (8 * RR);                     // partials <= 1/4 of Q's bytes
  if (splits > by_traffic) splits = by_traffic;
  if (splits > 64) splits = 64;
  if (M <= kSmallMaxM) splits = 1;  // short batches: one split, written out directly (no reduce launch)
  if (splits < 1) splits = 1;
  int64_t rows = (M + splits - 1) / splits;
  rows = (rows + kTnRows - 1) / kTnRows * kTnRows;
  pl.rows = rows;
  pl.splits = (int)((M + rows - 1) / rows);
  return pl;
}

template <int RP, bool PV>
__global__ __launch_bounds__(256) void k_skinny_tn(TnJobs jobs) {
  const TnArgs& p = jobs.job[blockIdx.z];
  if ((int64_t)blockIdx.y * p.rows >= p.M || (int64_t)blockIdx.x * kTnCols >= p.Kd) return;  // past this job's grid
  constexpr int NJ = RP / 16;
  constexpr int PS = RP + 16;                             // P tile row stride (bf16)
  constexpr int QCH = kTnRows * kTnCols / 8 / 256;        // 16-byte Q chunks per thread
  constexpr int PTOT = kTnRows * RP / 8;                  // 16-byte P chunks per tile
  constexpr int PCH = (PTOT + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kTnRows * kTnQS];
  __shared__ __attribute__((aligned(16))) uint16_t sP[kTnRows * PS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t M = p.M, Kd = p.Kd;
  const int R = p.r1 + p.r2;
  const int64_t k0 = (int64_t)blockIdx.x * kTnCols;
  const int64_t mbeg = (int64_t)blockIdx.y * p.rows;
  const int64_t nrows = (M - mbeg) < p.rows ? (M - mbeg) : p.rows;  // >= 1 by the plan
  const int ntiles = (int)((nrows + kTnRows - 1) / kTnRows);

  // Loop-invariant per-lane offsets inside a 64-row tile; each tile gets its
  // own buffer resources (base at the tile's first row, size = the rows left),
  // so rows past the split read zero and a tile past the end costs nothing.
  const int qrow = t >> 4, qcol = (t & 15) * 8;  // Q chunk q: row qrow + 16q
  const bool q_ok = k0 + qcol < Kd;
  int qoff[QCH];
#pragma unroll
  for (int q = 0; q < QCH; ++q) qoff[q] = q_ok ? (int)(((qrow + 16 * q) * Kd + k0 + qcol) * 2) : kOff;
  // P chunk q of this thread: chunk c = (t + 256 q) mod PTOT (threads past PTOT
  // duplicate a chunk: same data, same LDS slot)
  int poff[PCH][4];
  int pslot[PCH];
#pragma unroll
  for (int q = 0; q < PCH; ++q) {
    const int c = (t + 256 * q) % PTOT;
    const int prow = c / (RP / 8), pj = (c % (RP / 8)) * 8;
    pslot[q] = prow * PS + pj;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = pj + (PV ? 0 : 2 * e);
      poff[q][e] = j0 < R ? (int)((prow * p.ldp + j0) * 2) : kOff;
    }
  }
  auto load = [&](int tile, u32x4(&qv)[QCH], u32x4(&pv)[PCH]) {
    const int64_t mt = (int64_t)tile * kTnRows;
    const int64_t left = nrows - mt > 0 ? nrows - mt : 0;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(p.Q + (mbeg + mt) * Kd, left * Kd * 2);
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(p.P + (mbeg + mt) * p.ldp, left * p.ldp * 2);
#pragma unroll
    for (int q = 0; q < QCH; ++q)
      qv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qoff[q], 0, 0));
#pragma unroll
    for (int q = 0; q < PCH; ++q) {
      if (PV) {
        pv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, poff[q][0], 0, 0));
      } else {  // element-wise (R or the row stride not a multiple of 8)
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o0 = poff[q][e], o1 = (pslot[q] % PS) + 2 * e + 1 < R ? o0 + 2 : kOff;
          w[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rP, o0, 0, 0) |
                 ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rP, o1, 0, 0) << 16);
        }
        pv[q] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  // The issue order of every tile's loads is pinned (sched barriers), so the
  // loop entry and the back edge present the same outstanding-load sequence
  // and the compiler's wait counts keep the other tile in flight.
  auto load_pinned = [&](int tile, u32x4(&qv)[QCH], u32x4(&pv)[PCH]) {
    __builtin_amdgcn_sched_barrier(0);
    load(tile, qv, pv);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto stage = [&](const u32x4(&qv)[QCH], const u32x4(&pv)[PCH]) {
#pragma unroll
    for (int q = 0; q < QCH; ++q) *reinterpret_cast<u32x4*>(&sQ[(qrow + 16 * q) * kTnQS + qcol]) = qv[q];
#pragma unroll
    for (int q = 0; q < PCH; ++q) *reinterpret_cast<u32x4*>(&sP[pslot[q]]) = pv[q];
  };

  f32x4 acc[NJ][2];
#pragma unroll
  for (int a = 0; a < NJ; ++a) acc[a][0] = acc[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g = lane >> 4, sl = lane & 15;
  auto compute = [&]() {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int rb = 32 * half + 8 * g + (sl >> 2);
      u32x4 qb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = 32 * wave + 16 * b + 4 * (sl & 3);
        const u32x2 lo = lds_read_tr(&sQ[rb * kTnQS + col]);
        const u32x2 hi = lds_read_tr(&sQ[(rb + 4) * kTnQS + col]);
        qb[b] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int a = 0; a < NJ; ++a) {
        const u32x2 lo = lds_read_tr(&sP[rb * PS + 16 * a + 4 * (sl & 3)]);
        const u32x2 hi = lds_read_tr(&sP[(rb + 4) * PS + 16 * a + 4 * (sl & 3)]);
        const u32x4 pa = u32x4{lo[0], lo[1], hi[0], hi[1]};
        acc[a][0] = mfma16(pa, qb[0], acc[a][0]);
        acc[a][1] = mfma16(pa, qb[1], acc[a][1]);
      }
    }
  };

  // Loads are issued unconditionally (a tile past the end reads nothing), so
  // the compiler's wait counts stay exact and two tiles stay in flight.
  u32x4 q0[QCH], p0[PCH], q1[QCH], p1[PCH];
  load_pinned(0, q0, p0);
  load_pinned(1, q1, p1);
  for (int tile = 0; tile < ntiles; tile += 2) {
    stage(q0, p0);
    lds_barrier();
    load_pinned(tile + 2, q0, p0);
    compute();
    lds_barrier();
    if (tile + 1 >= ntiles) break;
    stage(q1, p1);
    lds_barrier();
    load_pinned(tile + 3, q1, p1);
    compute();
    lds_barrier();
  }

  // One split: the result itself, as k_tn_reduce would write it from a single
  // partial (one multiply by s, then fp32 (accumulated or not) or bf16).
  if (p.splits == 1) {
#pragma unroll
    for (int a = 0; a < NJ; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t k = k0 + 32 * wave + 16 * b + sl;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = 16 * a + 4 * g + v;
          if (j >= R || k >= Kd) continue;
          const bool first = j < p.r1;
          const float val = acc[a][b][v] * (first ? p.s1 : p.s2);
          const int64_t jr = first ? j : j - p.r1, ldo = first ? p.ldo1 : p.ldo2;
          const int64_t idx = p.transposed ? k * ldo + jr : jr * ldo + k;
          void* out = first ? p.out1 : p.out2;
          if (p.out_bf16) {
            static_cast<uint16_t*>(out)[idx] = __builtin_bit_cast(uint16_t, (__bf16)val);
          } else {
            float* o = static_cast<float*>(out) + idx;
            *o = p.accumulate ? *o + val : val;
          }
        }
      }
    return;
  }
  // this split's partial. C layout: col (Q column) = lane%16, row (j) = 4*(lane/16) + v
  float* dst = p.part + (int64_t)blockIdx.y * R * Kd;
#pragma unroll
  for (int a = 0; a < NJ; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t k = k0 + 32 * wave + 16 * b + sl;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * a + 4 * g + v;
        if (j < R && k < Kd) dst[(int64_t)j * Kd + k] = acc[a][b][v];
      }
    }

}

// out = s * (sum of the split partials, added in split order): one float4 of
// outputs per thread with every split's load in flight at once. Not in
// skinny_tn itself: a launch boundary makes the partials of all workgroups
// visible (an in-kernel "last workgroup reduces" scheme needs device-scope
// release fences, which write back the whole L2 of an XCD and cost far more
// here). When a backward GEMM follows, it does this work in its prologue
// instead, and this kernel is launched only when none does.
__global__ __launch_bounds__(64) void k_tn_reduce(TnJobs jobs) {
  const TnArgs& p = jobs.job[blockIdx.z];
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (int64_t)(p.r1 + p.r2) * (p.Kd / 4)) return;
  tn_reduce_quad(p, idx);
}

hipError_t launch_skinny_tn(TnJobs jobs, hipStream_t st) {
  if (jobs.n < 1 || jobs.n > kTnMaxJobs) return hipErrorInvalidValue;
  int rmax = 0;
  bool pv = true;
  int64_t gx = 0, gy = 0;
  for (int i = 0; i < jobs.n; ++i) {
    TnArgs& a = jobs.job[i];
    const int R = a.r1 + a.r2;
    const TnPlan pl = skinny_tn_plan(a.M, a.Kd, R);
    a.rows = pl.rows;
    a.splits = pl.splits;
    rmax = R > rmax ? R : rmax;
    pv = pv && (a.ldp % 8 == 0) && (R % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.P) & 15) == 0);
    gx = pl.col_tiles > gx ? pl.col_tiles : gx;
    gy = pl.splits > gy ? pl.splits : gy;
  }
  dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)jobs.n);
#define QL_TN(RPV)                                         \
  do {                                                     \
    if (pv)                                                \
      k_skinny_tn<RPV, true><<<grid, 256, 0, st>>>(jobs);  \
    else                                                   \
      k_skinny_tn<RPV, false><<<grid, 256, 0, st>>>(jobs); \
  } while (0)
  if (rmax <= 16)
    QL_TN(16);
  else if (rmax <= 32)
    QL_TN(32);
  else if (rmax <= 64)
    QL_TN(64);
  else if (rmax <= kTnMaxR)
    QL_TN(128);
  else
    return hipErrorInvalidValue;
#undef QL_TN
  return hipGetLastError();
}

TnJobs tn_reduce_jobs(const TnJobs& jobs) {
  TnJobs multi{};  // the jobs with more than one split (one-split jobs wrote their result already)
  for (int i = 0; i < jobs.n && i < kTnMaxJobs; ++i) {
    TnArgs a = jobs.job[i];
    a.splits = skinny_tn_plan(a.M, a.Kd, a.r1 + a.r2).splits;
    if (a.splits > 1) multi.job[multi.n++] = a;
  }
  return multi;
}

hipError_t launch_tn_reduce(TnJobs jobs, hipStream_t st) {
  if (jobs.n < 1 || jobs.n > kTnMaxJobs) return hipErrorInvalidValue;
  jobs = tn_reduce_jobs(jobs);
  int64_t nmax = 0;
  for (int i = 0; i < jobs.n; ++i) {
    const int64_t n = (int64_t)(jobs.job[i].r1 + jobs.job[i].r2) * (jobs.job[i].Kd / 4);
    nmax = n > nmax ? n : nmax;
  }
  if (nmax == 0) return hipSuccess;
  k_tn_reduce<<<dim3((unsigned)((nmax + 63) / 64), 1, (unsigned)jobs.n), 64, 0, st>>>(jobs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Preparation of a backward call, one launch: the adapter transposes (B^T rows
// for G = dY.B, A^T rows for the rank-r term of dX).

__global__ __launch_bounds__(256) void k_prep(PrepJobs jobs) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kMaxPrepJobs; ++i) {
    if (i >= jobs.n) break;
    const TransposeJob& j = jobs.job[i];
    if (idx < j.R * j.C) {
      const int64_t c = idx / j.R, rr = idx - c * j.R;
      j.dst[idx] = j.src[rr * j.C + c];
    }
  }
}

hipError_t launch_prep(const PrepJobs& jobs, hipStream_t st) {
  int64_t work = 0;
  for (int i = 0; i < jobs.n; ++i) work = work > jobs.job[i].R * jobs.job[i].C ? work : jobs.job[i].R * jobs.job[i].C;
  if (work == 0) return hipSuccess;
  k_prep<<<(unsigned)((work + 255) / 256), 256, 0, st>>>(jobs);
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

__global__ __launch_bounds__(256) void k_fill_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_fill_zero_u16(uint16_t* p, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_zero_u16<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

// bf16 copies of fp32 arrays (blockIdx.y selects the array)
__global__ __launch_bounds__(256) void k_cast_bf16(CastJobs jobs) {
  const CastJob& j = jobs.job[blockIdx.y];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < j.n) j.dst[i] = __builtin_bit_cast(uint16_t, (__bf16)j.src[i]);
}

hipError_t launch_cast_bf16(const CastJobs& jobs, hipStream_t st) {
  if (jobs.n < 1 || jobs.n > kMaxCastJobs) return hipErrorInvalidValue;
  int64_t nmax = 0;
  for (int i = 0; i < jobs.n; ++i) nmax = jobs.job[i].n > nmax ? jobs.job[i].n : nmax;
  if (nmax == 0) return hipSuccess;
  k_cast_bf16<<<dim3((unsigned)((nmax + 255) / 256), (unsigned)jobs.n), 256, 0, st>>>(jobs);
  return hipGetLastError();
}

}  // namespace qlora
