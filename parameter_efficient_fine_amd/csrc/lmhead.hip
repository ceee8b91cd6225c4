// Chunked cross-entropy over the frozen language-model head on gfx950
// ("Unsloth" wiki entry, Theory: chunked cross-entropy that never forms the
// [B, T, V] logits; "Unsloth vs PyTorch" video, 3:06-3:51: the loss computed
// slice by slice, each slice dropped, the same gradient).
//
// Per chunk of C tokens (api.cpp drives the chunks):
//   logits [C, V] fp32 = h_c . W^T        k_gemm_nt<true>   (W [V, H] bf16, frozen),
//     with each row's (max, sum exp) over every 256-column tile
//   per row: lse, loss, dz = (softmax - onehot) / n   k_ce_rows (dz bf16 [C, V])
//   dh_c [C, H] bf16 = dz . W = dz . (W^T)^T   k_gemm_nt<false> on W^T [H, V]
// W and W^T are laid out once at set-up (qlora_lmhead_prepare, k_tile_nt):
// both products are then "X . W^T" GEMMs over tiled weights.
//
// k_gemm_nt is the forward QLoRA GEMM's skeleton with bf16 weights: one
// workgroup = 4 waves, 256 weight rows x 256 tokens, K in steps of 64; each
// wave owns 64 weight rows, loaded from HBM straight into MFMA A-operand
// registers one step ahead (rows are private to a wave); the activation tile
// goes through LDS by buffer_load ... lds into a ring of four buffers. The
// frozen head is stored pre-tiled (k_tile_nt, at set-up): the 64 x 64 block of
// a row group and step is 8 KB laid out in the order the wave's lanes read
// it, so every weight load is one contiguous 1 KB run.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace qlora {

namespace {

constexpr int kTok = 256;
constexpr int kStep = 64;
constexpr int kRowB = kStep * 2;
constexpr int kBufB = kTok * kRowB;  // 32 KB
constexpr int kNBuf = 4;
constexpr size_t kLds = (size_t)kNBuf * kBufB;

struct NtGemmArgs {
  const uint16_t* X;  // [M, K]
  const uint16_t* W;  // [N, K]
  int64_t M, K, N;
  void* Y;            // [M, N] fp32 or bf16
  float* stats;       // fp32 output only, may be null: [M, ceil(N / 256)] pairs (max, sum exp(z - max))
                      // of each row over each 256-column tile
};

template <bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void k_gemm_nt(NtGemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [kNBuf][256 rows][128 B], swizzled
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 5, jl = lane & 31;
  const int64_t M = p.M, K = p.K, N = p.N;
  const int64_t nJ = (M + kTok - 1) / kTok;
  const int64_t it = blockIdx.x / nJ, jt = blockIdx.x - it * nJ;
  const int64_t i0 = it * 256, j0 = jt * kTok;
  const int nsteps = (int)(K / kStep);
  const int64_t rows_here = (M - j0) < kTok ? (M - j0) : kTok;

  // weight rows of this lane: fragment f = rows i0 + 64 wave + 32 f + jl; lane
  // half h reads k in [32h, 32h + 32) of a step, substep ks the 8 values 32h + 8ks.
  // Tiled storage: block (row group g, step t) at (g K/64 + t) * 8 KB, inside it
  // the 16-byte piece of (f, ks, lane) at ((4 f + ks) * 64 + lane) * 16.
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, N * K * 2);
  const int64_t g = i0 / 64 + wave;
  int offW[2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
    offW[f] = 64 * g < N ? (int)(g * (K / 64) * 8192 + (4 * f * 64 + lane) * 16) : kOff;
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.X + j0 * K, rows_here * K * 2);
  int offX[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    offX[i] = (int)((int64_t)row * K * 2 + 16 * c);
  }
  auto dma_x = [&](int step, int buf) {
    uint8_t* base = smem + buf * kBufB + (64 * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (__attribute__((address_space(3))) void*)(base + 8 * i * kRowB),
                                               16, offX[i], step * kRowB, 0, 0);
  };
  auto load_w = [&](int step, u32x4 (&wr)[4][2]) {  // substep-major: substep 0 lands first
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int f = 0; f < 2; ++f)
        wr[ks][f] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, offW[f] + 1024 * ks, step * 8192, 0));
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[f][j] = f32x16{};

  int offB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) offB[ks] = jl * kRowB + 16 * ((4 * h + ks) ^ ((jl >> 1) & 7));
  u32x4 bv[2][8];
  auto read_b = [&](int buf, int ks, u32x4 (&dst)[8]) {
    const uint8_t* bx = smem + buf * kBufB + offB[ks];
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = *reinterpret_cast<const u32x4*>(bx + 32 * j * kRowB);
  };
  auto mfmas = [&](const u32x4 (&a)[2], const u32x4 (&b)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[0][j] = mfma32(a[0], b[j], acc[0][j]);
      acc[1][j] = mfma32(a[1], b[j], acc[1][j]);
    }
  };
  auto interleave = [&](auto nds_read, auto nvmem) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < decltype(nds_read)::value) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < decltype(nvmem)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I8 = std::integral_constant<int, 8>;

  // Step s: weights in wc (loaded during step s-1), activations from LDS
  // buffer s%4 (copied during step s-3, published by the barrier ending step
  // s-2). Meanwhile the weights of step s+1 and the activations of step s+3
  // are requested; substep 0 of step s+1 is read from buffer (s+1)%4 in the
  // last substep. VMEM issue order per step: 8 weight loads, 8 copies.
  auto body = [&](int s, const u32x4 (&wc)[4][2], u32x4 (&wn)[4][2]) {
    const int b0 = s % kNBuf, b1 = (s + 1) % kNBuf, b3 = (s + 3) % kNBuf;
    const int s1 = s + 1 < nsteps ? s + 1 : nsteps - 1;
    const int s3 = s + 3 < nsteps ? s + 3 : nsteps - 1;
    load_w(s1, wn);
    dma_x(s3, b3);
    read_b(b0, 1, bv[1]);
    mfmas(wc[0], bv[0]);
    interleave(I8{}, I8{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(b0, 2, bv[0]);
    mfmas(wc[1], bv[1]);
    interleave(I8{}, I8{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(b0, 3, bv[1]);
    mfmas(wc[2], bv[0]);
    interleave(I8{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(b1, 0, bv[0]);
    mfmas(wc[3], bv[1]);
    interleave(I8{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));  // the copies of step s+2 have landed
    __builtin_amdgcn_s_waitcnt(0xC07F);           // and this wave's LDS reads
    __builtin_amdgcn_s_barrier();
  };

  // Prologue in the order a step issues its loads: weights of step 0 stand in
  // for "weights of the next step", then the copies of steps 0, 1, 2.
  u32x4 wa[4][2], wb[4][2];
  load_w(0, wa);
  __builtin_amdgcn_sched_barrier(0);
  dma_x(0, 0);
  dma_x(nsteps > 1 ? 1 : 0, 1);
  dma_x(nsteps > 2 ? 2 : nsteps - 1, 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));  // copies of steps 0 and 1
  __builtin_amdgcn_s_barrier();
  read_b(0, 0, bv[0]);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    body(s, wa, wb);
    body(s + 1, wb, wa);
  }
  if (s < nsteps) body(s, wa, wb);

  // ---- epilogue through LDS (the activation ring is idle now): each wave parks
  // its 64 columns token-major, 16-byte chunk c of token row t at c ^ (t & 15)
  // (fp32, 256-byte rows, two passes of 128 tokens) or c ^ (t & 7) (bf16,
  // 128-byte rows, one pass), and every store then writes whole row pieces.
  constexpr int kOutB = OUT_F32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rO = make_rsrc((uint8_t*)p.Y + j0 * N * kOutB, rows_here * N * kOutB);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's trailing copies into the ring have landed
  __builtin_amdgcn_s_barrier();   // and every wave is done reading the ring
  {
    int jle = jl, he = h, lne = lane;
    asm volatile("" : "+v"(jle), "+v"(he), "+v"(lne));
    const int rh = (int)rows_here;
    if constexpr (OUT_F32) {
      uint8_t* const reg = smem + wave * (128 * 256);
      const int c = lne & 15, tq = lne >> 4;
      const int64_t col = i0 + 64 * wave + 4 * c;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = 32 * jj + jle;
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16& a = acc[f][4 * pass + jj];
              *reinterpret_cast<f32x4*>(reg + t * 256 + 16 * ((8 * f + 2 * q + he) ^ (t & 15))) =
                  f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            }
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int t = 4 * u + tq, mr = 128 * pass + t;
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + t * 256 + 16 * (c ^ (t & 15)));
          const int off = (mr < rh && col < N) ? (int)((mr * N + col) * 4) : kOff;
          __builtin_amdgcn_raw_buffer_store_b128(v, rO, off, 0, kStoreNT);
        }
        lds_barrier();
      }
    } else {
      uint8_t* const reg = smem + wave * (256 * 128);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
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
      const int c = lne & 7, tq = lne >> 3;
      const int64_t col = i0 + 64 * wave + 8 * c;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int t = 8 * u + tq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + t * 128 + 16 * (c ^ (t & 7)));
        const int off = (t < rh && col < N) ? (int)((t * N + col) * 2) : kOff;
        __builtin_amdgcn_raw_buffer_store_b128(v, rO, off, 0, kStoreNT);
      }
    }
  }

  // ---- row statistics of this 256-column tile (logits only): each lane pair
  // (l, l ^ 32) holds a token's 64 columns of the wave; the 4 waves' partials
  // are combined in wave order through LDS (the activation ring is free now).
  if constexpr (OUT_F32) {
    if (p.stats == nullptr) return;
    float* const red = reinterpret_cast<float*>(smem);  // [4 waves][256 tokens][2]
    lds_barrier();  // every wave is past its last operand read
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float mx = -__builtin_inff(), sm = 0.f;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t ic = i0 + 64 * wave + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
          if (ic < N) mx = fmaxf(mx, acc[f][j][v]);
        }
      // exp(z - max) as the hardware 2^x of (z - max) log2(e): one transcendental
      // op per logit instead of the libm sequence (the sum is a statistic; its
      // relative error stays at the fp32 rounding level)
      const float ml = mx == -__builtin_inff() ? 0.f : mx * 1.44269504088896341f;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t ic = i0 + 64 * wave + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
          if (ic < N) sm += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[f][j][v], 1.44269504088896341f, -ml));
        }
      const float mp = __shfl_xor(mx, 32), sp = __shfl_xor(sm, 32);
      const float mm = fmaxf(mx, mp);
      const float a = mx == -__builtin_inff() ? 0.f : sm * expf(mx - mm);
      const float b = mp == -__builtin_inff() ? 0.f : sp * expf(mp - mm);
      if (h == 0) {
        red[(wave * 256 + 32 * j + jl) * 2] = mm;
        red[(wave * 256 + 32 * j + jl) * 2 + 1] = a + b;
      }
    }
    lds_barrier();
    const int64_t row = t;  // one token row per thread
    float mx = -__builtin_inff(), sm = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float m2 = red[(w * 256 + t) * 2], s2 = red[(w * 256 + t) * 2 + 1];
      const float mm = fmaxf(mx, m2);
      const float a = mx == -__builtin_inff() ? 0.f : sm * expf(mx - mm);
      const float b = m2 == -__builtin_inff() ? 0.f : s2 * expf(m2 - mm);
      mx = mm;
      sm = a + b;
    }
    const int64_t ntiles = (N + 255) / 256;
    if (row < rows_here) {
      p.stats[((j0 + row) * ntiles + it) * 2] = mx;
      p.stats[((j0 + row) * ntiles + it) * 2 + 1] = sm;
    }
  }
}

// Row statistics and gradient of the cross-entropy, one workgroup per row of
// the chunk: lse = max + log(sum exp(z - max)) (fp32), from the logits GEMM's
// per-tile pairs (max, sum exp) combined in tile order; loss_m = lse - z[t]
// for kept rows (t >= 0), dz = (exp(z - lse) - [v == t]) / n in bf16 (0 on
// ignored rows): one pass over the row's logits.
__global__ __launch_bounds__(256) void k_ce_rows(const float* __restrict__ logits, const float* __restrict__ stats,
                                                 int64_t ntiles, const int32_t* __restrict__ tgt,
                                                 const int32_t* __restrict__ n_keep, int64_t V,
                                                 float* __restrict__ loss_rows, uint16_t* __restrict__ dz) {
  __shared__ float red_m[256], red_s[256];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const float* z = logits + m * V;
  const int t = tgt[m];
  const int64_t nq = V / 4;
  float mx = -__builtin_inff(), sm = 0.f;
  for (int64_t q = tid; q < ntiles; q += 256) {
    const float m2 = stats[(m * ntiles + q) * 2], s2 = stats[(m * ntiles + q) * 2 + 1];
    const float mm = fmaxf(mx, m2);
    const float a = mx == -__builtin_inff() ? 0.f : sm * expf(mx - mm);
    const float b = m2 == -__builtin_inff() ? 0.f : s2 * expf(m2 - mm);
    mx = mm;
    sm = a + b;
  }
  red_m[tid] = mx;
  red_s[tid] = sm;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {  // fixed-order tree
    if (tid < w) {
      const float m1 = red_m[tid], m2 = red_m[tid + w];
      const float mm = fmaxf(m1, m2);
      const float s1 = m1 == -__builtin_inff() ? 0.f : red_s[tid] * expf(m1 - mm);
      const float s2 = m2 == -__builtin_inff() ? 0.f : red_s[tid + w] * expf(m2 - mm);
      red_m[tid] = mm;
      red_s[tid] = s1 + s2;
    }
    __syncthreads();
  }
  const float lse = red_m[0] + logf(red_s[0]);
  const int n = *n_keep;
  const bool keep = t >= 0 && t < V;
  const float inv_n = (keep && n > 0) ? 1.0f / (float)n : 0.0f;
  if (tid == 0) loss_rows[m] = keep ? lse - z[t] : 0.0f;
  uint16_t* d = dz + m * V;
  auto grad4 = [&](int64_t q, const f32x4& v) {
    float g[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = (expf(v[e] - lse) - ((int64_t)4 * q + e == t ? 1.0f : 0.0f)) * inv_n;
    *reinterpret_cast<u32x2*>(d + 4 * q) = u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
  };
  // four loads in flight per thread, then the ragged rest one by one
  int64_t q = tid;
  for (; q + 3 * 256 < nq; q += 4 * 256) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = reinterpret_cast<const f32x4*>(z)[q + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u) grad4(q + 256 * u, v[u]);
  }
  for (; q < nq; q += 256) grad4(q, reinterpret_cast<const f32x4*>(z)[q]);
}

// Number of kept targets (t >= 0 and t < V), one workgroup, fixed order.
__global__ __launch_bounds__(256) void k_ce_count(const int32_t* __restrict__ tgt, int64_t M, int64_t V,
                                                  int32_t* __restrict__ n_keep) {
  __shared__ int red[256];
  int c = 0;
  for (int64_t m = threadIdx.x; m < M; m += 256) c += (tgt[m] >= 0 && tgt[m] < V) ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_keep = red[0];
}

// loss = sum of the per-row losses / n, one workgroup, fixed order.
__global__ __launch_bounds__(256) void k_ce_total(const float* __restrict__ loss_rows, int64_t M,
                                                  const int32_t* __restrict__ n_keep, float* __restrict__ loss) {
  __shared__ float red[256];
  float a = 0.f;
  for (int64_t m = threadIdx.x; m < M; m += 256) a += loss_rows[m];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = *n_keep;
    *loss = n > 0 ? red[0] / (float)n : 0.0f;
  }
}

// The weight operand of k_gemm_nt in its tiled order: dst holds W [N, K]
// (W = src [R, C] when !transpose, W = src^T when transpose) as blocks of
// 64 rows x 64 columns, block (g, t) at (g K/64 + t) * 8 KB, and inside a
// block the 8 consecutive values k = 64t + 32h + 8ks .. +7 of row
// n = 64g + 32f + jl at ((4 f + ks) * 64 + jl + 32 h) * 16 bytes.
// One thread per 16-byte piece. N % 64 == 0, K % 64 == 0.
__global__ __launch_bounds__(256) void k_tile_nt(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                 bool transpose, uint16_t* __restrict__ dst) {
  const int64_t N = transpose ? C : R, K = transpose ? R : C;
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (piece >= N * K / 8) return;
  const int64_t blk = piece / 512, in = piece - blk * 512;
  const int64_t g = blk / (K / 64), t = blk - g * (K / 64);
  const int fks = (int)(in / 64), lane = (int)(in % 64);
  const int f = fks / 4, ks = fks % 4, jl = lane % 32, h = lane / 32;
  const int64_t n = 64 * g + 32 * f + jl, k = 64 * t + 32 * h + 8 * ks;
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = transpose ? src[(k + e) * C + n] : src[n * C + k + e];
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = (uint32_t)v[2 * q] | ((uint32_t)v[2 * q + 1] << 16);
  reinterpret_cast<u32x4*>(dst)[piece] = out;
}

template <bool OUT_F32>
hipError_t launch_nt(const NtGemmArgs& a, hipStream_t st) {
  // set once per kernel instance; a function-local static is initialised exactly
  // once even when several threads make their first call together
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_gemm_nt<OUT_F32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int64_t nI = (a.N + 255) / 256, nJ = (a.M + kTok - 1) / kTok;
  if (nI * nJ == 0) return hipSuccess;
  k_gemm_nt<OUT_F32><<<(unsigned)(nI * nJ), 256, kLds, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt_bf16(const uint16_t* X, const uint16_t* W, int64_t M, int64_t K, int64_t N, void* Y,
                               bool out_f32, float* stats, hipStream_t st) {
  NtGemmArgs a{X, W, M, K, N, Y, out_f32 ? stats : nullptr};
  return out_f32 ? launch_nt<true>(a, st) : launch_nt<false>(a, st);
}

hipError_t launch_ce_count(const int32_t* tgt, int64_t M, int64_t V, int32_t* n_keep, hipStream_t st) {
  k_ce_count<<<1, 256, 0, st>>>(tgt, M, V, n_keep);
  return hipGetLastError();
}

hipError_t launch_ce_rows(const float* logits, const float* stats, const int32_t* tgt, const int32_t* n_keep,
                          int64_t C, int64_t V, float* loss_rows, uint16_t* dz, hipStream_t st) {
  if (C == 0) return hipSuccess;
  k_ce_rows<<<(unsigned)C, 256, 0, st>>>(logits, stats, (V + 255) / 256, tgt, n_keep, V, loss_rows, dz);
  return hipGetLastError();
}

hipError_t launch_ce_total(const float* loss_rows, int64_t M, const int32_t* n_keep, float* loss, hipStream_t st) {
  k_ce_total<<<1, 256, 0, st>>>(loss_rows, M, n_keep, loss);
  return hipGetLastError();
}

hipError_t launch_tile_nt(const uint16_t* src, int64_t R, int64_t C, bool transpose, uint16_t* dst, hipStream_t st) {
  const int64_t pieces = R * C / 8;
  if (pieces == 0) return hipSuccess;
  k_tile_nt<<<(unsigned)((pieces + 255) / 256), 256, 0, st>>>(src, R, C, transpose, dst);
  return hipGetLastError();
}

}  // namespace qlora
