// The split-order sum of skinny_tn's fp32 partials, shared by k_tn_reduce and
// by the backward GEMM, which does this work in its prologue when it is
// launched right after skinny_tn (the launch boundary makes the partials
// visible, so no separate reduce launch is needed).
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace qlora {

// Output quad idx of one job (row j = idx / (Kd / 4), columns 4 (idx % (Kd / 4))
// .. +3): the partials of splits 0, 1, .. added in that order, scaled by the
// row's s, rounded once to bf16 or stored (or added) as fp32. WIDE: loads go
// out 16 splits at a time (else 4 at a time, for callers with other values
// live); the order of the additions is the same either way.
template <bool WIDE = true>
__device__ __forceinline__ void tn_reduce_quad(const TnArgs& p, int64_t idx) {
  const int64_t Kd = p.Kd, kq = Kd / 4;
  const int j = (int)(idx / kq);
  const int64_t k = 4 * (idx - j * kq);
  const float* src = p.part + (int64_t)j * Kd + k;
  const int64_t sstride = (int64_t)(p.r1 + p.r2) * Kd;
  f32x4 sum = *reinterpret_cast<const f32x4*>(src);
  int sp = 1;
  for (; WIDE && sp + 16 <= p.splits; sp += 16) {
    f32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const f32x4*>(src + (int64_t)(sp + i) * sstride);
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += v[i];
  }
  for (; sp + 4 <= p.splits; sp += 4) {
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const f32x4*>(src + (int64_t)(sp + i) * sstride);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += v[i];
  }
  for (; sp < p.splits; ++sp) sum += *reinterpret_cast<const f32x4*>(src + (int64_t)sp * sstride);
  const bool first = j < p.r1;
  const float s = first ? p.s1 : p.s2;
  void* out = first ? p.out1 : p.out2;
  const int64_t jr = first ? j : j - p.r1;
  const int64_t ldo = first ? p.ldo1 : p.ldo2;
  sum *= s;
  if (p.out_bf16) {  // one rounding of the fp32 sum (no accumulation in bf16)
    uint16_t* ob = static_cast<uint16_t*>(out);
    if (p.transposed) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ob[(k + c) * ldo + jr] = __builtin_bit_cast(uint16_t, (__bf16)sum[c]);
    } else {
      *reinterpret_cast<u32x2*>(ob + jr * ldo + k) = u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
    }
    return;
  }
  float* of = static_cast<float*>(out);
  if (p.transposed) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float* o = of + (k + c) * ldo + jr;
      *o = p.accumulate ? *o + sum[c] : sum[c];
    }
  } else {
    f32x4* o = reinterpret_cast<f32x4*>(of + jr * ldo + k);
    *o = p.accumulate ? *o + sum : sum;
  }
}

// Output quads of all jobs: job z owns (r1 + r2) * Kd / 4 of them, after those of jobs < z.
__device__ __forceinline__ int64_t tn_reduce_quads(const TnJobs& jobs) {
  int64_t t = 0;
  for (int z = 0; z < jobs.n; ++z) t += (int64_t)(jobs.job[z].r1 + jobs.job[z].r2) * (jobs.job[z].Kd / 4);
  return t;
}

// Workgroup `wg` of `nwg` takes one contiguous slice of all jobs' quads; its
// threads (nthr of them, this one `tid`) walk the slice, 4 splits in flight each.
__device__ __forceinline__ void tn_reduce_slice(const TnJobs& jobs, int64_t wg, int64_t nwg, int tid, int nthr) {
  const int64_t total = tn_reduce_quads(jobs);
  const int64_t chunk = (total + nwg - 1) / nwg;
  const int64_t g0 = wg * chunk, g1 = (g0 + chunk) < total ? (g0 + chunk) : total;
  for (int64_t g = g0 + tid; g < g1; g += nthr) {
    int64_t base = 0;
    int z = 0;
    for (; z + 1 < jobs.n; ++z) {
      const int64_t n = (int64_t)(jobs.job[z].r1 + jobs.job[z].r2) * (jobs.job[z].Kd / 4);
      if (g < base + n) break;
      base += n;
    }
    tn_reduce_quad<false>(jobs.job[z], g - base);
  }
}

}  // namespace qlora
