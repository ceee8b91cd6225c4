// C ABI of the fused QLoRA layer: argument checks, workspace carving and the
// kernel sequence of each call on the caller's stream. The math of each step
// is stated in include/qlora.h; the kernels live in quant.hip, skinny.hip,
// gemm_fwd.hip and gemm_bwd.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>
#include <cstdio>
#include <cstring>

#include "../../include/qlora.h"
#include "internal.hpp"

using namespace qlora;

namespace {

thread_local char g_err[256] = "";

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return QLORA_EHIP;
}

#define QL_CHECK(expr)                                  \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return hip_fail(e_, #expr);   \
  } while (0)

// ---- optional launch timing (measurement support; see qlora_profile_begin)
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> recs;
  size_t next = 0;
  int64_t dropped = 0;
} g_prof;

template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& f) {
  if (!g_prof.on) return f();
  if (g_prof.next + 2 > g_prof.pool.size()) {
    ++g_prof.dropped;
    return f();
  }
  hipEvent_t a = g_prof.pool[g_prof.next++], b = g_prof.pool[g_prof.next++];
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  if (e == hipSuccess) g_prof.recs.push_back({name, a, b});
  return e;
}

#define QL_LAUNCH(name, st, expr) QL_CHECK(timed(name, st, [&]() { return (expr); }))

// Size limits keeping every buffer offset the kernels form within 32 bits.
constexpr int64_t kMaxDim = int64_t(1) << 21;
constexpr int64_t kMaxWeight = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool layer_ok(const qlora_layer* L) {
  if (!L || !L->codes || !L->absmax || !L->A || !L->B) return false;
  if (L->K <= 0 || L->K % 64 != 0 || L->N <= 0 || L->N % 8 != 0) return false;
  if (L->r < 1 || L->r > 256) return false;
  if (L->format < QLORA_FMT_NF4 || L->format > QLORA_FMT_FP8) return false;
  if (L->grad_dtype != QLORA_GRAD_BF16 && L->grad_dtype != QLORA_GRAD_F32) return false;
  // code bytes of the weight stay below 2^30 for every format
  if (L->K > kMaxDim || L->N > kMaxDim || L->N * L->K > (L->format == QLORA_FMT_NF4 ? kMaxWeight : kMaxWeight / 2))
    return false;
  if (!aligned16(L->codes) || !aligned16(L->absmax) || !aligned16(L->A) || !aligned16(L->B)) return false;
  return true;
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

bool grads_bf16(const qlora_layer* L) { return L->grad_dtype == QLORA_GRAD_BF16; }

// zero [n] gradient values of the layer's gradient type
hipError_t zero_grad(void* p, int64_t n, bool bf16, hipStream_t st) {
  return bf16 ? launch_fill_zero_u16(static_cast<uint16_t*>(p), n, st)
              : launch_fill_zero_f32(static_cast<float*>(p), n, st);
}

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t cap, used = 0;
  bool ok = true;
  template <class T>
  T* take(size_t count) {
    const size_t b = up256(count * sizeof(T));
    if (used + b > cap) {
      ok = false;
      return nullptr;
    }
    T* p = reinterpret_cast<T*>(base + used);
    used += b;
    return p;
  }
};

// The skinny_tn launches behind one reduction with adapter widths (r1, r2):
// one launch when r1 + r2 fits a launch, else chunks of each part.
template <class F>
void tn_chunks(int r1, int r2, F&& f) {
  if (r1 + r2 <= kTnMaxR) {
    f(0, r1, r2);
    return;
  }
  for (int c = 0; c < r1; c += kTnMaxR) f(c, std::min(kTnMaxR, r1 - c), 0);
  for (int c = 0; c < r2; c += kTnMaxR) f(r1 + c, std::min(kTnMaxR, r2 - c), 0);
}

// fp32 partials of one reduction launch (256-byte multiple, in floats)
size_t tn_part_floats(int64_t M, int64_t Kd, int R) {
  const TnPlan pl = skinny_tn_plan(M, Kd, R);
  return up256((size_t)pl.splits * (size_t)R * (size_t)Kd * sizeof(float)) / sizeof(float);
}

// Workspace of the reductions of a call: every reduction (chunk) has partials
// of its own, so independent reductions can share a launch.
struct BwdLayout {
  size_t part = 0;  // floats
  void add(int64_t M, int64_t Kd, int r1, int r2 = 0) {
    tn_chunks(r1, r2, [&](int, int a, int b) { part += tn_part_floats(M, Kd, a + b); });
  }
};

BwdLayout bwd_layout(int64_t M, int64_t K, int64_t N, int64_t r) {
  BwdLayout l;
  l.add(M, N, (int)r);  // dB
  l.add(M, K, (int)r);  // dA
  return l;
}

size_t bwd_ws(int64_t M, int64_t K, int64_t N, int64_t r) {
  const BwdLayout l = bwd_layout(M, K, N, r);
  return up256(r * N * 2) + up256(M * r * 2) + up256(l.part * 4);
}

// The SwiGLU block's backward reductions, in launch order: the down projection's
// part, then the gate and up projections' part.
BwdLayout mlp_bwd_down_layout(int64_t M, int64_t H, int64_t I, int64_t r) {
  BwdLayout l;
  l.add(M, H, (int)r);            // dB_down
  l.add(M, I, (int)r);            // dA_down
  return l;
}

BwdLayout mlp_bwd_gu_layout(int64_t M, int64_t H, int64_t I, int64_t r) {
  BwdLayout l;
  l.add(M, I, (int)r);            // dB_gate
  l.add(M, I, (int)r);            // dB_up
  l.add(M, H, (int)r, (int)r);    // dA_gate, dA_up
  return l;
}

BwdLayout mlp_bwd_layout(int64_t M, int64_t H, int64_t I, int64_t r) {
  BwdLayout l;
  l.part = mlp_bwd_down_layout(M, H, I, r).part + mlp_bwd_gu_layout(M, H, I, r).part;
  return l;
}

size_t mlp_bwd_ws(int64_t M, int64_t H, int64_t I, int64_t r) {
  const BwdLayout l = mlp_bwd_layout(M, H, I, r);
  return 2 * up256((size_t)M * I * 2) + up256(M * r * 2) + up256(M * 2 * r * 2) + up256(r * H * 2) +
         2 * up256(r * I * 2) + up256(l.part * 4);
}

// Token-tiled SwiGLU block: per-tile intermediates only (tile T = min(tile, M)).
// A tile's last GEMM (the forward's down projection, the backward's dX: T
// tokens by H columns in 256 x 256 tiles) runs on a second stream beside the
// next tile's work when it launches fewer workgroups than the chip has CUs;
// the buffers it reads then alternate between two copies.
constexpr int64_t kChipCUs = 256;
bool tiles_overlap(int64_t M, int64_t T, int64_t H) {
  return M > T && ((T + 255) / 256) * ((H + 255) / 256) < kChipCUs;
}

size_t mlp_fwd_tiled_ws(int64_t M, int64_t H, int64_t I, int64_t tile) {
  const int64_t T = std::min(tile, M);
  return (tiles_overlap(M, T, H) ? 4 : 3) * up256((size_t)T * I * 2);  // g, u, h of one tile (h twice)
}

// Reduction partials of the tiled backward: the down part's and the gate/up
// part's in regions of their own (the two parts of a tile run on different
// streams). The split count of a reduction is not monotone in its row count
// (rows per split are rounded to 64), so a ragged last tile can need more
// partials than a full one: each region is sized for the larger.
struct TiledPart {
  size_t down = 0, gu = 0;  // floats
};

TiledPart mlp_tiled_part(int64_t M, int64_t H, int64_t I, int64_t r, int64_t tile) {
  const int64_t T = std::min(tile, M);
  TiledPart p;
  p.down = mlp_bwd_down_layout(T, H, I, r).part;
  p.gu = mlp_bwd_gu_layout(T, H, I, r).part;
  if (T > 0) {
    const int64_t last = M - ((M - 1) / T) * T;
    p.down = std::max(p.down, mlp_bwd_down_layout(last, H, I, r).part);
    p.gu = std::max(p.gu, mlp_bwd_gu_layout(last, H, I, r).part);
  }
  return p;
}

// fp32 sums of the six adapter gradients over the tiles (used for bf16 gradients,
// which are rounded once after the last tile): dA_g, dA_u [r, H], dA_d [r, I],
// dB_g, dB_u [I, r], dB_d [H, r]
size_t mlp_grad_acc_bytes(int64_t H, int64_t I, int64_t r) {
  return 2 * up256(r * H * 4) + up256(r * I * 4) + 2 * up256(I * r * 4) + up256(H * r * 4);
}

size_t mlp_bwd_tiled_ws(int64_t M, int64_t H, int64_t I, int64_t r, int64_t tile) {
  const int64_t T = std::min(tile, M);
  const TiledPart tp = mlp_tiled_part(M, H, I, r, tile);
  // g, u, h, dg, du of one tile (dg and du twice when the tiles overlap)
  return (tiles_overlap(M, T, H) ? 7 : 5) * up256((size_t)T * I * 2) + up256(T * r * 2) + up256(T * 2 * r * 2) +
         up256(r * H * 2) + 2 * up256(r * I * 2) + up256((tp.down + tp.gu) * 4) + mlp_grad_acc_bytes(H, I, r);
}

// Batches of at most kSmallMaxM tokens (ranks up to kSmallMaxR) take the
// small-batch kernels: one workgroup per 32 x 32 output tile, the rank-r products
// of the tile formed alongside, one-split reductions written out directly.
bool small_batch(const qlora_layer* L, int64_t M) { return M <= kSmallMaxM && L->r <= kSmallMaxR; }

WSrc wsrc(const qlora_layer* L, const uint16_t* lora_i, const uint16_t* lora_j, int64_t ldj = 0) {
  WSrc w;
  w.codes = L->codes;
  w.absmax = L->absmax;
  w.lora_i = lora_i;
  w.lora_j = lora_j;
  w.r = (int)L->r;
  w.ldj = ldj ? ldj : L->r;
  w.s = L->s;
  w.fmt = L->format;
  return w;
}

NtArgs nt1(const uint16_t* in, int64_t M, int64_t Kd, const uint16_t* ad, int r, uint16_t* out, int64_t ld) {
  NtArgs a{};
  a.in = in;
  a.M = M;
  a.Kd = Kd;
  a.ad1 = ad;
  a.ad2 = ad;
  a.r1 = r;
  a.r2 = 0;
  a.out1 = out;
  a.out2 = out;
  a.ld1 = ld;
  a.ld2 = ld;
  return a;
}

// G = in . B for B stored [Kd, r] (the layer's layout): read in place for the
// ranks skinny_nt's [Kd, r] form is built for (16, 32, 64, 128, 256), else from
// the transposed copy Bt [r, Kd] (made by the prep kernel).
bool b_in_place(int64_t r) { return r == 16 || r == 32 || r == 64 || r == 128 || r == 256; }
NtArgs ntB(const uint16_t* in, int64_t M, int64_t Kd, const uint16_t* B, const uint16_t* Bt, int r, uint16_t* out,
           int64_t ld) {
  NtArgs a = nt1(in, M, Kd, b_in_place(r) ? B : Bt, r, out, ld);
  a.ad_kr = b_in_place(r) ? 1 : 0;
  return a;
}

// Collects independent reductions (out = s * P^T . Q) and issues them as one
// skinny_tn launch per batch of kTnMaxJobs, each job with its own slice of the
// partial buffer; the split partials are then added by one tn_reduce launch,
// or, for the last batch, by the backward GEMM launched next (flush(&red)).
struct TnCall {
  float* part;
  const float* part_end;  // end of the partial region carved for this call
  hipStream_t st;
  int accumulate = 0;  // add to the outputs instead of overwriting them (fp32 outputs)
  bool out_bf16 = false;  // outputs are bf16 (rounded once from the fp32 sums)
  TnJobs jobs{};
  int rc = QLORA_OK;
  // out = s * P^T . Q (P [M, r] with row stride ldp, Q [M, Kd]); transposed -> [Kd, r]
  void one(const uint16_t* P, int64_t ldp, int r, float s, const uint16_t* Q, int64_t M, int64_t Kd, void* out,
           bool transposed) {
    two(P, ldp, r, s, out, 0, 0.f, nullptr, Q, M, Kd, transposed);
  }
  // rows j < r1 of P^T . Q into out1 (scale s1), rows r1 <= j < r1 + r2 into out2 (scale s2)
  void two(const uint16_t* P, int64_t ldp, int r1, float s1, void* out1, int r2, float s2, void* out2,
           const uint16_t* Q, int64_t M, int64_t Kd, bool transposed) {
    const size_t es = out_bf16 ? 2 : 4;  // bytes per output element
    tn_chunks(r1, r2, [&](int c0, int a1, int a2) {
      // chunk columns [c0, c0 + a1 + a2) of P; a2 > 0 only for the single job covering both parts
      const bool in2 = c0 >= r1;
      TnArgs a{};
      a.P = P + c0;
      a.ldp = ldp;
      a.r1 = a1;
      a.r2 = a2;
      a.s1 = in2 ? s2 : s1;
      a.s2 = s2;
      const int64_t jo = in2 ? c0 - r1 : c0;  // first output row of the chunk
      char* o1 = static_cast<char*>(in2 ? out2 : out1);
      a.out1 = o1 + es * (transposed ? jo : jo * Kd);
      a.ldo1 = transposed ? (in2 ? r2 : r1) : Kd;
      a.out2 = out2 ? out2 : out1;
      a.ldo2 = transposed ? r2 : Kd;
      a.transposed = transposed ? 1 : 0;
      a.accumulate = accumulate;
      a.out_bf16 = out_bf16 ? 1 : 0;
      a.Q = Q;
      a.M = M;
      a.Kd = Kd;
      a.part = part;
      part += tn_part_floats(M, Kd, a1 + a2);
      if (part > part_end && rc == QLORA_OK) {  // never write past the carved region
        snprintf(g_err, sizeof(g_err), "reduction partials exceed the workspace");
        rc = QLORA_EWORKSPACE;
      }
      if (jobs.n == kTnMaxJobs) flush();
      jobs.job[jobs.n++] = a;
    });
  }
  // defer != null: launch skinny_tn only and hand the reductions it leaves
  // (one-split jobs are written out by skinny_tn itself) to the caller, which
  // passes them to the backward GEMM it launches next on the same stream.
  int flush(TnJobs* defer = nullptr) {
    if (defer) defer->n = 0;
    if (jobs.n == 0 || rc != QLORA_OK) return rc;
    const TnJobs red = tn_reduce_jobs(jobs);
    hipError_t e = timed("skinny_tn", st, [&]() { return launch_skinny_tn(jobs, st); });
    if (e == hipSuccess && red.n) {
      if (defer)
        *defer = red;
      else
        e = timed("tn_reduce", st, [&]() { return launch_tn_reduce(jobs, st); });
    }
    if (e != hipSuccess) rc = hip_fail(e, "skinny_tn");
    jobs.n = 0;
    return rc;
  }
};

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument (shape, null or misaligned pointer)";
    case QLORA_EUNSUPPORTED: return "unsupported";
    case QLORA_EWORKSPACE: return "workspace missing or too small";
    case QLORA_ENONFINITE: return "the weight holds Inf or NaN";
    case QLORA_EHIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

const char* qlora_last_error(void) { return g_err; }

int qlora_quantize(int format, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                   uint32_t* nonfinite_blocks, void* stream) {
  if (format < QLORA_FMT_NF4 || format > QLORA_FMT_FP8) return QLORA_EINVAL;
  if (N < 0 || K < 0 || K % 64 != 0) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!W || !codes || !absmax || !aligned16(W) || !aligned16(codes)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (nonfinite_blocks) {
    QL_LAUNCH("quantize", st, launch_quantize(format, W, N, K, codes, absmax, nonfinite_blocks, st));
    return QLORA_OK;
  }
  uint32_t bad = 0;
  QL_CHECK(quantize_counting(format, W, N, K, codes, absmax, &bad, st));
  return bad ? QLORA_ENONFINITE : QLORA_OK;
}

int qlora_pack_codes(int format, const uint8_t* src_codes, const float* src_absmax, int64_t N, int64_t K,
                     uint8_t* codes, float* absmax, void* stream) {
  if (format < QLORA_FMT_NF4 || format > QLORA_FMT_FP8) return QLORA_EINVAL;
  if (N < 0 || K < 0 || K % 64 != 0 || K > kMaxDim || N > kMaxDim) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!src_codes || !src_absmax || !codes || !absmax) return QLORA_EINVAL;
  if (!aligned16(src_codes) || !aligned16(src_absmax) || !aligned16(codes) || !aligned16(absmax)) return QLORA_EINVAL;
  const size_t cb = (size_t)N * (format == QLORA_FMT_NF4 ? K / 2 : K), ab = (size_t)N * (K / 64) * 4;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  if (overlap(src_codes, cb, codes, cb) || overlap(src_absmax, ab, absmax, ab) || overlap(src_codes, cb, absmax, ab) ||
      overlap(src_absmax, ab, codes, cb))
    return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("pack_codes", st, launch_pack_codes(format, src_codes, src_absmax, N, K, codes, absmax, st));
  return QLORA_OK;
}

int qlora_dequantize(int format, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                     void* stream) {
  if (format < QLORA_FMT_NF4 || format > QLORA_FMT_FP8) return QLORA_EINVAL;
  if (N < 0 || K < 0 || K % 64 != 0) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!codes || !absmax || !W_hat || !aligned16(W_hat) || (format != QLORA_FMT_NF4 && !aligned16(codes)))
    return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("dequantize", st, launch_dequantize(format, codes, absmax, N, K, W_hat, st));
  return QLORA_OK;
}

size_t qlora_workspace_size(int op, int64_t M, int64_t K, int64_t N, int64_t r) {
  if (M < 0 || K < 0 || N < 0 || r < 1) return 0;
  switch (op) {
    case QLORA_OP_FORWARD: return 0;
    case QLORA_OP_BACKWARD: return bwd_ws(M, K, N, r);
    case QLORA_OP_MLP_FORWARD: return 0;
    case QLORA_OP_MLP_BACKWARD: return mlp_bwd_ws(M, K, N, r);
    default: return 0;
  }
}

int qlora_forward(const qlora_layer* L, const uint16_t* X, int64_t M, uint16_t* Y, uint16_t* Z_save, void* ws,
                  size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!layer_ok(L) || M < 0) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !Z_save || !aligned16(X) || !aligned16(Y) || !aligned16(Z_save)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int r = (int)L->r;
  if (small_batch(L, M)) {
    const SmallFwdArgs a{X, L->codes, L->absmax, L->A, L->B, M, L->K, L->N, r, L->s, Y, Z_save};
    QL_LAUNCH("small_fwd", st, launch_small_fwd(a, L->format, st));
    return QLORA_OK;
  }
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(nt1(X, M, L->K, L->A, r, Z_save, r), st));
  QL_LAUNCH("gemm_fwd", st, launch_gemm_fwd(X, M, L->K, L->N, wsrc(L, L->B, Z_save), Y, st));
  return QLORA_OK;
}

int qlora_rope_table(int d, float base, int64_t max_pos, float* table, void* stream) {
  if (d < 16 || d > 1024 || d % 16 != 0 || !(base > 1.f) || max_pos < 0 || max_pos > kMaxDim) return QLORA_EINVAL;
  if (max_pos == 0) return QLORA_OK;
  if (!table || !aligned16(table)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("rope_table", st, launch_rope_table(d, (double)base, max_pos, table, st));
  return QLORA_OK;
}

int qlora_forward_rope(const qlora_layer* L, const uint16_t* X, int64_t M, const int32_t* pos, const float* table,
                       int64_t max_pos, int d, uint16_t* Y, uint16_t* Z_save, void* stream) {
  if (!layer_ok(L) || M < 0 || d != 128 || L->N % d != 0 || max_pos < 1 || max_pos > kMaxDim) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !Z_save || !pos || !table || !aligned16(X) || !aligned16(Y) || !aligned16(Z_save) ||
      !aligned16(table))
    return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int r = (int)L->r;
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(nt1(X, M, L->K, L->A, r, Z_save, r), st));
  QL_LAUNCH("gemm_fwd_rope", st,
            launch_gemm_fwd_rope(X, M, L->K, L->N, wsrc(L, L->B, Z_save), pos, table, max_pos, Y, st));
  return QLORA_OK;
}

int qlora_backward(const qlora_layer* L, const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save, int64_t M,
                   uint16_t* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  if (!layer_ok(L) || M < 0) return QLORA_EINVAL;
  if (!dA || !dB || !aligned16(dA) || !aligned16(dB)) return QLORA_EINVAL;
  const int64_t K = L->K, N = L->N;
  const int r = (int)L->r;
  hipStream_t st = (hipStream_t)stream;
  if (M > 0) {
    if (!dY || !X || !Z_save || !aligned16(dY) || !aligned16(X) || !aligned16(Z_save)) return QLORA_EINVAL;
    if (dX && !aligned16(dX)) return QLORA_EINVAL;
  }
  const size_t need = bwd_ws(M, K, N, r);
  if (!ws || ws_bytes < need) return QLORA_EWORKSPACE;
  const BwdLayout lay = bwd_layout(M, K, N, r);
  Carve c{(char*)ws, ws_bytes};
  uint16_t* Bt = c.take<uint16_t>((size_t)r * N);
  uint16_t* G = c.take<uint16_t>((size_t)M * r);
  float* part = c.take<float>(lay.part);
  if (!c.ok) return QLORA_EWORKSPACE;
  const bool gb = grads_bf16(L);
  if (M == 0) {  // empty batch: gradients are zero
    QL_LAUNCH("fill_zero", st, zero_grad(dA, (int64_t)r * K, gb, st));
    QL_LAUNCH("fill_zero", st, zero_grad(dB, (int64_t)N * r, gb, st));
    return QLORA_OK;
  }
  if (small_batch(L, M) && dX) {
    // dX and G in one launch, then dB and dA (one split each, written directly)
    const SmallBwdArgs a{dY, L->codes, L->absmax, L->A, L->B, M, K, N, r, L->s, dX, G};
    QL_LAUNCH("small_bwd", st, launch_small_bwd(a, L->format, st));
    TnCall tn{part, part + lay.part, st};
    tn.out_bf16 = gb;
    tn.one(Z_save, r, r, L->s, dY, M, N, dB, true);
    tn.one(G, r, r, L->s, X, M, K, dA, false);
    return tn.flush();
  }
  if (!b_in_place(r)) {
    PrepJobs pj{};
    pj.job[0] = {L->B, Bt, N, r};  // B [N, r] -> B^T [r, N]
    pj.n = 1;
    QL_LAUNCH("prep", st, launch_prep(pj, st));
  }
  // G = dY.B ; dB = s.dY^T.Z (written transposed from Z^T.dY) and dA = s.G^T.X in one pair of launches ; dX
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(ntB(dY, M, N, L->B, Bt, r, G, r), st));
  TnCall tn{part, part + lay.part, st};
  tn.out_bf16 = gb;
  tn.one(Z_save, r, r, L->s, dY, M, N, dB, true);
  tn.one(G, r, r, L->s, X, M, K, dA, false);
  TnJobs red{};  // reduced by the backward GEMM when there is one
  if (int rc = tn.flush(dX ? &red : nullptr)) return rc;
  if (dX) QL_LAUNCH("gemm_bwd", st, launch_gemm_bwd(dY, wsrc(L, L->A, G), nullptr, WSrc{}, M, K, N, dX, &red, st));
  return QLORA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward without a caller workspace, for callers that cannot allocate device
// memory. Its workspace is this file-scope array: each GPU the library runs on
// holds its own copy for the life of the process. Host code never uses the
// array's name as a device address: the address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];

// this device's copy of `scratch` (looked up on first use)
int scratch_for_current_device(void** out) {
  int dev = 0;
  QL_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices) {
    snprintf(g_err, sizeof(g_err), "device %d: no scratch slot", dev);
    return QLORA_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    QL_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}
}  // namespace

extern "C" {

int qlora_backward_noalloc(const qlora_layer* L, const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save,
                           int64_t M, uint16_t* dX, void* dA, void* dB, void* stream) {
  if (!layer_ok(L) || M < 0) return QLORA_EINVAL;
  const size_t need = bwd_ws(M, L->K, L->N, L->r);
  if (need > (size_t)QLORA_NOALLOC_SCRATCH_BYTES) {
    snprintf(g_err, sizeof(g_err), "qlora_backward_noalloc: needs %zu bytes of scratch, the limit is %zu", need,
             (size_t)QLORA_NOALLOC_SCRATCH_BYTES);
    return QLORA_EWORKSPACE;
  }
  void* ws = nullptr;
  if (int rc = scratch_for_current_device(&ws)) return rc;
  // every scratch byte the backward reads is written earlier in the same call
  // (G, the B^T copy, the reduction partials), so nothing needs clearing
  return qlora_backward(L, dY, X, Z_save, M, dX, dA, dB, ws, (size_t)QLORA_NOALLOC_SCRATCH_BYTES, stream);
}

static bool mlp_shapes_ok(const qlora_layer* g, const qlora_layer* u, const qlora_layer* d) {
  if (!layer_ok(g) || !layer_ok(u) || !layer_ok(d)) return false;
  if (g->K != u->K || g->N != u->N || d->K != g->N || d->N != g->K) return false;
  if (g->r != u->r || g->r != d->r) return false;
  if (g->format != u->format || g->format != d->format) return false;
  if (g->grad_dtype != u->grad_dtype || g->grad_dtype != d->grad_dtype) return false;
  return true;
}

}  // extern "C"

namespace {

// Z_g, Z_u = X.A_g^T, X.A_u^T (row stride r each)
int mlp_zgu(const qlora_layer* gate, const qlora_layer* up, const uint16_t* X, int64_t M, uint16_t* Zg, uint16_t* Zu,
            hipStream_t st) {
  const int64_t H = gate->K;
  const int r = (int)gate->r;
  if (2 * r <= 256) {
    NtArgs a = nt1(X, M, H, gate->A, r, Zg, r);
    a.ad2 = up->A;
    a.r2 = r;
    a.out2 = Zu;
    QL_LAUNCH("skinny_nt", st, launch_skinny_nt(a, st));
  } else {
    QL_LAUNCH("skinny_nt", st, launch_skinny_nt(nt1(X, M, H, gate->A, r, Zg, r), st));
    QL_LAUNCH("skinny_nt", st, launch_skinny_nt(nt1(X, M, H, up->A, r, Zu, r), st));
  }
  return QLORA_OK;
}

// SwiGLU block forward over M tokens, first part: Z_g, Z_u, then g, u, h and Z_d.
int mlp_fwd_gu(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* X,
               int64_t M, uint16_t* g, uint16_t* u, uint16_t* h, uint16_t* Zg, uint16_t* Zu, uint16_t* Zd,
               hipStream_t st) {
  const int64_t H = gate->K, I = gate->N;
  const int r = (int)gate->r;
  if (int rc = mlp_zgu(gate, up, X, M, Zg, Zu, st)) return rc;
  QL_LAUNCH("gemm_fwd_gateup", st,
            launch_gemm_fwd_gateup(X, M, H, I, wsrc(gate, gate->B, Zg), wsrc(up, up->B, Zu), g, u, h, st));
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(nt1(h, M, I, down->A, r, Zd, r), st));
  return QLORA_OK;
}

// second part: Y = h.W_d^T + s.Z_d.B_d^T
int mlp_fwd_down(const qlora_layer* down, const uint16_t* h, int64_t M, uint16_t* Y, const uint16_t* Zd,
                 hipStream_t st) {
  QL_LAUNCH("gemm_fwd", st, launch_gemm_fwd(h, M, down->K, down->N, wsrc(down, down->B, Zd), Y, st));
  return QLORA_OK;
}

int mlp_fwd_body(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* X,
                 int64_t M, uint16_t* Y, uint16_t* g, uint16_t* u, uint16_t* h, uint16_t* Zg, uint16_t* Zu,
                 uint16_t* Zd, hipStream_t st) {
  if (int rc = mlp_fwd_gu(gate, up, down, X, M, g, u, h, Zg, Zu, Zd, st)) return rc;
  return mlp_fwd_down(down, h, M, Y, Zd, st);
}

struct MlpBwdWs {
  uint16_t *dg, *du, *Gd, *Ggu, *Btd, *Btg, *Btu;
  float* part;
  size_t part_floats;
};

MlpBwdWs carve_mlp_bwd(Carve& c, int64_t M, int64_t H, int64_t I, int64_t r, size_t part_floats) {
  MlpBwdWs w;
  w.dg = c.take<uint16_t>((size_t)M * I);
  w.du = c.take<uint16_t>((size_t)M * I);
  w.Gd = c.take<uint16_t>((size_t)M * r);
  w.Ggu = c.take<uint16_t>((size_t)M * 2 * r);  // row m: G_gate[m, :] then G_up[m, :]
  w.Btd = c.take<uint16_t>((size_t)r * H);
  w.Btg = c.take<uint16_t>((size_t)r * I);
  w.Btu = c.take<uint16_t>((size_t)r * I);
  w.part = c.take<float>(part_floats);
  w.part_floats = part_floats;
  return w;
}

int mlp_zero_grads(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, void* const dA[3],
                   void* const dB[3], hipStream_t st) {
  const qlora_layer* Ls[3] = {gate, up, down};
  for (int i = 0; i < 3; ++i) {
    QL_LAUNCH("fill_zero", st, zero_grad(dA[i], Ls[i]->r * Ls[i]->K, grads_bf16(Ls[i]), st));
    QL_LAUNCH("fill_zero", st, zero_grad(dB[i], Ls[i]->N * Ls[i]->r, grads_bf16(Ls[i]), st));
  }
  return QLORA_OK;
}

int mlp_prep(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const MlpBwdWs& w,
             hipStream_t st) {
  const int64_t H = gate->K, I = gate->N, r = gate->r;
  if (b_in_place(r)) return QLORA_OK;  // the G products read B in place
  PrepJobs pj{};
  pj.job[0] = {down->B, w.Btd, H, r};
  pj.job[1] = {gate->B, w.Btg, I, r};
  pj.job[2] = {up->B, w.Btu, I, r};
  pj.n = 3;
  QL_LAUNCH("prep", st, launch_prep(pj, st));
  return QLORA_OK;
}

// SwiGLU block backward over M tokens, after mlp_prep, in two parts. accumulate
// = 1 adds the adapter gradients to dA/dB (later tiles of a batch); each part's
// reduction partials go to [part, part_end).
// Down projection: G_d = dY.B_d ; dB_d = s.dY^T.Z_d and dA_d = s.G_d^T.h ; dh -> (dg, du)
// in the GEMM epilogue.
int mlp_bwd_down(const qlora_layer* down, const uint16_t* dY, const uint16_t* g, const uint16_t* u,
                 const uint16_t* h, const uint16_t* Zd, int64_t M, void* dA_d, void* dB_d, const MlpBwdWs& w,
                 float* part, const float* part_end, int accumulate, bool out_bf16, hipStream_t st) {
  const int64_t H = down->N, I = down->K;
  const int r = (int)down->r;
  TnCall tn{part, part_end, st, accumulate};
  tn.out_bf16 = out_bf16;
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(ntB(dY, M, H, down->B, w.Btd, r, w.Gd, r), st));
  tn.one(Zd, r, r, down->s, dY, M, H, dB_d, true);
  tn.one(w.Gd, r, r, down->s, h, M, I, dA_d, false);
  TnJobs red{};  // reduced by the backward GEMM launched next
  if (int rc = tn.flush(&red)) return rc;
  QL_LAUNCH("gemm_bwd_swiglu", st,
            launch_gemm_bwd_swiglu(dY, wsrc(down, down->A, w.Gd), M, I, H, g, u, w.dg, w.du, &red, st));
  return QLORA_OK;
}

// Gate and up, after the down part: G = d(g|u).B ; dB = s.d(g|u)^T.Z ;
// dA_g = s_g.G_g^T.X and dA_u = s_u.G_u^T.X (one pass over X when 2r fits a
// launch) ; dX = dg.W_g + du.W_u + s.G_g.A_g + s.G_u.A_u, one GEMM over the
// concatenated reduction.
int mlp_bwd_gu(const qlora_layer* gate, const qlora_layer* up, const uint16_t* X, const uint16_t* Zg,
               const uint16_t* Zu, int64_t M, uint16_t* dX, void* const dA[3], void* const dB[3], const MlpBwdWs& w,
               float* part, const float* part_end, int accumulate, bool out_bf16, hipStream_t st) {
  const int64_t H = gate->K, I = gate->N;
  const int r = (int)gate->r;
  uint16_t* Gg = w.Ggu;
  uint16_t* Gu = w.Ggu + r;
  TnCall tn{part, part_end, st, accumulate};
  tn.out_bf16 = out_bf16;
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(ntB(w.dg, M, I, gate->B, w.Btg, r, Gg, 2 * r), st));
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(ntB(w.du, M, I, up->B, w.Btu, r, Gu, 2 * r), st));
  tn.one(Zg, r, r, gate->s, w.dg, M, I, dB[0], true);
  tn.one(Zu, r, r, up->s, w.du, M, I, dB[1], true);
  tn.two(w.Ggu, 2 * r, r, gate->s, dA[0], r, up->s, dA[1], X, M, H, false);
  TnJobs red{};
  if (int rc = tn.flush(dX ? &red : nullptr)) return rc;
  if (dX)
    QL_LAUNCH("gemm_bwd", st,
              launch_gemm_bwd(w.dg, wsrc(gate, gate->A, Gg, 2 * r), w.du, wsrc(up, up->A, Gu, 2 * r), M, H, I, dX,
                              &red, st));
  return QLORA_OK;
}

int mlp_bwd_body(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* dY,
                 const uint16_t* X, const uint16_t* g, const uint16_t* u, const uint16_t* h, const uint16_t* Zg,
                 const uint16_t* Zu, const uint16_t* Zd, int64_t M, uint16_t* dX, void* const dA[3],
                 void* const dB[3], const MlpBwdWs& w, bool out_bf16, hipStream_t st) {
  float* const mid = w.part + mlp_bwd_down_layout(M, gate->K, gate->N, gate->r).part;
  if (int rc = mlp_bwd_down(down, dY, g, u, h, Zd, M, dA[2], dB[2], w, w.part, mid, 0, out_bf16, st)) return rc;
  return mlp_bwd_gu(gate, up, X, Zg, Zu, M, dX, dA, dB, w, mid, w.part + w.part_floats, 0, out_bf16, st);
}

// ---- a second stream per device for the token-tiled SwiGLU block: a tile's
// last GEMM (at 1024 tokens, 64 workgroups of 256 x 256 outputs) runs beside
// the next tile's work instead of leaving most CUs idle. Created on first use
// with the device current, at the default priority and non-blocking (no
// implicit ordering with the null stream); kept until the process ends.
std::mutex g_aux_mu;
constexpr int kAuxDevices = 64;
hipStream_t g_aux[kAuxDevices];

int aux_stream_for_current_device(hipStream_t* out) {
  int dev = 0;
  QL_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kAuxDevices) {
    snprintf(g_err, sizeof(g_err), "device %d: no second-stream slot", dev);
    return QLORA_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_aux_mu);
  if (!g_aux[dev]) QL_CHECK(hipStreamCreateWithFlags(&g_aux[dev], hipStreamNonBlocking));
  *out = g_aux[dev];
  return QLORA_OK;
}

// Fork and join between the caller's stream and the second stream, for tiles
// whose buffers alternate between two copies: tile t's work on the second
// stream reads copy t % 2, and the caller's stream waits for that work to end
// before it writes the copy again (tile t + 2). The destructor joins, so that no
// return leaves work of the call behind on the second stream.
struct TileOverlap {
  hipStream_t st, aux = nullptr;
  hipEvent_t ev = nullptr, done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  bool forked = false;
  explicit TileOverlap(hipStream_t s) : st(s) {}
  TileOverlap(const TileOverlap&) = delete;
  TileOverlap& operator=(const TileOverlap&) = delete;
  ~TileOverlap() {
    (void)join();
    for (hipEvent_t e : {ev, done[0], done[1]})
      if (e) (void)hipEventDestroy(e);
  }
  int init() {
    if (int rc = aux_stream_for_current_device(&aux)) return rc;
    QL_CHECK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    QL_CHECK(hipEventCreateWithFlags(&done[0], hipEventDisableTiming));
    QL_CHECK(hipEventCreateWithFlags(&done[1], hipEventDisableTiming));
    return QLORA_OK;
  }
  // before the caller's stream writes copy b again
  int reclaim(int b) {
    if (pending[b]) {
      QL_CHECK(hipStreamWaitEvent(st, done[b], 0));
      pending[b] = false;
    }
    return QLORA_OK;
  }
  // what is enqueued next on the second stream starts after all that is enqueued on the caller's
  int fork() {
    QL_CHECK(hipEventRecord(ev, st));
    QL_CHECK(hipStreamWaitEvent(aux, ev, 0));
    forked = true;
    return QLORA_OK;
  }
  // the second stream is done with copy b once what is enqueued on it so far has run
  int release(int b) {
    QL_CHECK(hipEventRecord(done[b], aux));
    pending[b] = true;
    return QLORA_OK;
  }
  // the caller's stream waits for all of the call's work on the second stream
  int join() {
    if (!forked) return QLORA_OK;
    forked = false;
    pending[0] = pending[1] = false;
    QL_CHECK(hipEventRecord(ev, aux));
    QL_CHECK(hipStreamWaitEvent(st, ev, 0));
    return QLORA_OK;
  }
};

bool mlp_grads_ok(void* const dA[3], void* const dB[3]) {
  if (!dA || !dB) return false;
  for (int i = 0; i < 3; ++i)
    if (!dA[i] || !dB[i] || !aligned16(dA[i]) || !aligned16(dB[i])) return false;
  return true;
}

}  // namespace

extern "C" {

int swiglu_mlp_forward(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* X,
                       int64_t M, uint16_t* Y, uint16_t* g_save, uint16_t* u_save, uint16_t* h_save,
                       uint16_t* Z_save, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!mlp_shapes_ok(gate, up, down) || M < 0) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !g_save || !u_save || !h_save || !Z_save) return QLORA_EINVAL;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(g_save) || !aligned16(u_save) || !aligned16(h_save) ||
      !aligned16(Z_save))
    return QLORA_EINVAL;
  const size_t Mr = (size_t)M * gate->r;
  return mlp_fwd_body(gate, up, down, X, M, Y, g_save, u_save, h_save, Z_save, Z_save + Mr, Z_save + 2 * Mr,
                      (hipStream_t)stream);
}

int swiglu_mlp_backward(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* dY,
                        const uint16_t* X, const uint16_t* g_save, const uint16_t* u_save, const uint16_t* h_save,
                        const uint16_t* Z_save, int64_t M, uint16_t* dX, void* const dA[3], void* const dB[3],
                        void* ws, size_t ws_bytes, void* stream) {
  if (!mlp_shapes_ok(gate, up, down) || M < 0 || !mlp_grads_ok(dA, dB)) return QLORA_EINVAL;
  const int64_t H = gate->K, I = gate->N, r = gate->r;
  hipStream_t st = (hipStream_t)stream;
  if (M > 0) {
    if (!dY || !X || !g_save || !u_save || !h_save || !Z_save) return QLORA_EINVAL;
    if (!aligned16(dY) || !aligned16(X) || !aligned16(g_save) || !aligned16(u_save) || !aligned16(h_save) ||
        !aligned16(Z_save) || (dX && !aligned16(dX)))
      return QLORA_EINVAL;
  }
  if (!ws || ws_bytes < mlp_bwd_ws(M, H, I, r)) return QLORA_EWORKSPACE;
  Carve c{(char*)ws, ws_bytes};
  const MlpBwdWs w = carve_mlp_bwd(c, M, H, I, r, mlp_bwd_layout(M, H, I, r).part);
  if (!c.ok) return QLORA_EWORKSPACE;
  if (M == 0) return mlp_zero_grads(gate, up, down, dA, dB, st);
  if (int rc = mlp_prep(gate, up, down, w, st)) return rc;
  const size_t Mr = (size_t)M * r;
  return mlp_bwd_body(gate, up, down, dY, X, g_save, u_save, h_save, Z_save, Z_save + Mr, Z_save + 2 * Mr, M, dX,
                      dA, dB, w, grads_bf16(gate), st);
}

size_t swiglu_mlp_tiled_workspace_size(int backward, int64_t M, int64_t H, int64_t I, int64_t r, int64_t tile) {
  if (M < 0 || H < 0 || I < 0 || r < 1 || tile < 1) return 0;
  return backward ? mlp_bwd_tiled_ws(M, H, I, r, tile) : mlp_fwd_tiled_ws(M, H, I, tile);
}

int swiglu_mlp_forward_tiled(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                             const uint16_t* X, int64_t M, int64_t tile, uint16_t* Y, uint16_t* Z_save, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!mlp_shapes_ok(gate, up, down) || M < 0 || tile < 1) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !Z_save || !aligned16(X) || !aligned16(Y) || !aligned16(Z_save)) return QLORA_EINVAL;
  const int64_t H = gate->K, I = gate->N, r = gate->r;
  const int64_t T = std::min(tile, M);
  if (!ws || ws_bytes < mlp_fwd_tiled_ws(M, H, I, tile)) return QLORA_EWORKSPACE;
  Carve c{(char*)ws, ws_bytes};
  const bool two = tiles_overlap(M, T, H);  // the down projection's GEMM on the second stream
  uint16_t* g = c.take<uint16_t>((size_t)T * I);
  uint16_t* u = c.take<uint16_t>((size_t)T * I);
  uint16_t* hb[2];
  hb[0] = c.take<uint16_t>((size_t)T * I);
  hb[1] = two ? c.take<uint16_t>((size_t)T * I) : hb[0];
  if (!c.ok) return QLORA_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  TileOverlap ov(st);
  if (two)
    if (int rc = ov.init()) return rc;
  const size_t Mr = (size_t)M * r;
  for (int64_t t0 = 0, t = 0; t0 < M; t0 += T, ++t) {
    const int64_t Mt = std::min(T, M - t0);
    const int b = (int)(t & 1);
    uint16_t* Zt = Z_save + (size_t)t0 * r;
    if (int rc = ov.reclaim(b)) return rc;
    if (int rc = mlp_fwd_gu(gate, up, down, X + t0 * H, Mt, g, u, hb[b], Zt, Zt + Mr, Zt + 2 * Mr, st)) return rc;
    if (!two) {
      if (int rc = mlp_fwd_down(down, hb[b], Mt, Y + t0 * H, Zt + 2 * Mr, st)) return rc;
      continue;
    }
    // Y rows of this tile on the second stream, beside the next tile's Z, g, u, h
    if (int rc = ov.fork()) return rc;
    if (int rc = mlp_fwd_down(down, hb[b], Mt, Y + t0 * H, Zt + 2 * Mr, ov.aux)) return rc;
    if (int rc = ov.release(b)) return rc;
  }
  return ov.join();
}

int swiglu_mlp_backward_tiled(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                              const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save, int64_t M, int64_t tile,
                              uint16_t* dX, void* const dA[3], void* const dB[3], void* ws, size_t ws_bytes,
                              void* stream) {
  if (!mlp_shapes_ok(gate, up, down) || M < 0 || tile < 1 || !mlp_grads_ok(dA, dB)) return QLORA_EINVAL;
  const int64_t H = gate->K, I = gate->N, r = gate->r;
  hipStream_t st = (hipStream_t)stream;
  if (M > 0) {
    if (!dY || !X || !Z_save || !aligned16(dY) || !aligned16(X) || !aligned16(Z_save) || (dX && !aligned16(dX)))
      return QLORA_EINVAL;
  }
  const int64_t T = std::min(tile, M);
  if (!ws || ws_bytes < mlp_bwd_tiled_ws(M, H, I, r, tile)) return QLORA_EWORKSPACE;
  Carve c{(char*)ws, ws_bytes};
  const bool two = tiles_overlap(M, T, H);  // each tile's gate/up part on the second stream
  uint16_t* g = c.take<uint16_t>((size_t)T * I);
  uint16_t* u = c.take<uint16_t>((size_t)T * I);
  uint16_t* h = c.take<uint16_t>((size_t)T * I);
  const TiledPart tp = mlp_tiled_part(M, H, I, r, tile);
  MlpBwdWs wb[2];
  wb[0] = carve_mlp_bwd(c, T, H, I, r, tp.down + tp.gu);
  wb[1] = wb[0];
  if (two) {  // a second dg, du: the gate/up part of tile t reads copy t % 2
    wb[1].dg = c.take<uint16_t>((size_t)T * I);
    wb[1].du = c.take<uint16_t>((size_t)T * I);
  }
  const MlpBwdWs& w = wb[0];
  float* const part_gu = w.part + tp.down;  // the down part's region, then the gate/up part's
  // bf16 gradients: the tiles add into fp32 sums, rounded once at the end
  const bool gb = grads_bf16(gate);
  const qlora_layer* Ls[3] = {gate, up, down};
  void* accA[3];
  void* accB[3];
  for (int i = 0; i < 3; ++i) {
    accA[i] = c.take<float>((size_t)Ls[i]->r * Ls[i]->K);
    accB[i] = c.take<float>((size_t)Ls[i]->N * Ls[i]->r);
  }
  if (!c.ok) return QLORA_EWORKSPACE;
  if (M == 0) return mlp_zero_grads(gate, up, down, dA, dB, st);
  if (int rc = mlp_prep(gate, up, down, w, st)) return rc;
  void* const* oA = gb ? accA : dA;
  void* const* oB = gb ? accB : dB;
  TileOverlap ov(st);
  if (two)
    if (int rc = ov.init()) return rc;
  const size_t Mr = (size_t)M * r;
  for (int64_t t0 = 0, t = 0; t0 < M; t0 += T, ++t) {
    const int64_t Mt = std::min(T, M - t0);
    const int b = (int)(t & 1);
    const int acc = t0 > 0 ? 1 : 0;
    const uint16_t* Xt = X + t0 * H;
    const uint16_t* Zt = Z_save + (size_t)t0 * r;
    if (int rc = ov.reclaim(b)) return rc;
    // recompute the tile's g, u, h (bitwise what the forward produced: same kernels, same inputs)
    QL_LAUNCH("gemm_fwd_gateup", st,
              launch_gemm_fwd_gateup(Xt, Mt, H, I, wsrc(gate, gate->B, Zt), wsrc(up, up->B, Zt + Mr), g, u, h, st));
    if (int rc = mlp_bwd_down(down, dY + t0 * H, g, u, h, Zt + 2 * Mr, Mt, oA[2], oB[2], wb[b], w.part, part_gu, acc,
                              false, st))
      return rc;
    // the gate and up projections' gradients and dX rows: on the second stream
    // beside the next tile's recompute and down part (each gradient still adds
    // its tiles in order, on one stream)
    hipStream_t sg = st;
    if (two) {
      if (int rc = ov.fork()) return rc;
      sg = ov.aux;
    }
    if (int rc = mlp_bwd_gu(gate, up, Xt, Zt, Zt + Mr, Mt, dX ? dX + t0 * H : nullptr, oA, oB, wb[b], part_gu,
                            part_gu + tp.gu, acc, false, sg))
      return rc;
    if (two)
      if (int rc = ov.release(b)) return rc;
  }
  if (int rc = ov.join()) return rc;
  if (gb) {
    CastJobs cj{};
    for (int i = 0; i < 3; ++i) {
      cj.job[cj.n++] = {static_cast<const float*>(accA[i]), static_cast<uint16_t*>(dA[i]), Ls[i]->r * Ls[i]->K};
      cj.job[cj.n++] = {static_cast<const float*>(accB[i]), static_cast<uint16_t*>(dB[i]), Ls[i]->N * Ls[i]->r};
    }
    QL_LAUNCH("cast_bf16", st, launch_cast_bf16(cj, st));
  }
  return QLORA_OK;
}

int qlora_rmsnorm_forward(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, float eps, uint16_t* y,
                          float* rstd, void* stream) {
  if (M < 0 || H <= 0 || H % 8 != 0 || H > kMaxDim || !(eps >= 0.f)) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!x || !w || !y || !rstd || !aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(rstd))
    return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("rmsnorm_fwd", st, launch_rmsnorm_fwd(x, w, M, H, eps, y, rstd, st));
  return QLORA_OK;
}

int qlora_rmsnorm_backward(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd, int64_t M,
                           int64_t H, uint16_t* dx, void* stream) {
  if (M < 0 || H <= 0 || H % 8 != 0 || H > kMaxDim) return QLORA_EINVAL;
  if (M == 0) return QLORA_OK;
  if (!dy || !x || !w || !rstd || !dx || !aligned16(dy) || !aligned16(x) || !aligned16(w) || !aligned16(rstd) ||
      !aligned16(dx))
    return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("rmsnorm_bwd", st, launch_rmsnorm_bwd(dy, x, w, rstd, M, H, dx, st));
  return QLORA_OK;
}

static int rope_call(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t M, int hq, int hk, int d, float base,
                     bool inverse, void* stream) {
  if (M < 0 || hq < 0 || hk < 0 || d < 16 || d > 1024 || d % 16 != 0 || !(base > 1.f)) return QLORA_EINVAL;
  if ((int64_t)(hq > hk ? hq : hk) * d > kMaxDim) return QLORA_EINVAL;
  if (M == 0 || hq + hk == 0) return QLORA_OK;
  if (!pos || (hq && (!q || !aligned16(q))) || (hk && (!k || !aligned16(k)))) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH(inverse ? "rope_bwd" : "rope_fwd", st, launch_rope(q, k, pos, M, hq, hk, d, (double)base, inverse, st));
  return QLORA_OK;
}

int qlora_rope_forward(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t M, int hq, int hk, int d, float base,
                       void* stream) {
  return rope_call(q, k, pos, M, hq, hk, d, base, false, stream);
}

int qlora_rope_backward(uint16_t* dq, uint16_t* dk, const int32_t* pos, int64_t M, int hq, int hk, int d, float base,
                        void* stream) {
  return rope_call(dq, dk, pos, M, hq, hk, d, base, true, stream);
}

int qlora_lmhead_prepare(const uint16_t* W, int64_t V, int64_t H, uint16_t* Wp, uint16_t* Wtp, void* stream) {
  if (V <= 0 || H <= 0 || V % 64 != 0 || H % 64 != 0 || V > kMaxDim || H > kMaxDim || H * V > kMaxWeight / 2)
    return QLORA_EINVAL;
  if (!W || !Wp || !Wtp || !aligned16(W) || !aligned16(Wp) || !aligned16(Wtp)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("tile", st, launch_tile_nt(W, V, H, false, Wp, st));   // logits: rows v, reduction over h
  QL_LAUNCH("tile", st, launch_tile_nt(W, V, H, true, Wtp, st));   // dh: rows h, reduction over v
  return QLORA_OK;
}

static bool ce_shapes_ok(int64_t M, int64_t H, int64_t V, int64_t chunk) {
  if (M < 0 || chunk < 1 || H <= 0 || V <= 0 || H % 64 != 0 || V % 64 != 0) return false;
  return H <= kMaxDim && V <= kMaxDim && H * V <= kMaxWeight / 2;
}

static size_t ce_ws(int64_t M, int64_t V, int64_t chunk) {
  const int64_t C = std::min(chunk, M);
  return up256((size_t)C * V * 4) + up256((size_t)C * V * 2) + up256((size_t)C * ((V + 255) / 256) * 8) + 256;
}

size_t qlora_ce_workspace_size(int64_t M, int64_t V, int64_t chunk) {
  if (M < 0 || V <= 0 || chunk < 1) return 0;
  return ce_ws(M, V, chunk);
}

int qlora_chunked_ce(const uint16_t* h, const uint16_t* Wp, const uint16_t* Wtp, const int32_t* targets, int64_t M,
                     int64_t H, int64_t V, int64_t chunk, float* loss, float* loss_rows, uint16_t* dh, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!ce_shapes_ok(M, H, V, chunk)) return QLORA_EINVAL;
  if (!loss) return QLORA_EINVAL;
  if (M > 0 && (!h || !Wp || !Wtp || !targets || !loss_rows || !dh || !aligned16(h) || !aligned16(Wp) ||
                !aligned16(Wtp) || !aligned16(dh)))
    return QLORA_EINVAL;
  if (!ws || ws_bytes < ce_ws(M, V, chunk)) return QLORA_EWORKSPACE;
  const int64_t C = std::min(chunk, M);
  Carve c{(char*)ws, ws_bytes};
  float* logits = c.take<float>((size_t)C * V);
  uint16_t* dz = c.take<uint16_t>((size_t)C * V);
  float* stats = c.take<float>((size_t)C * ((V + 255) / 256) * 2);
  int32_t* n_keep = c.take<int32_t>(64);
  if (!c.ok) return QLORA_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("ce_count", st, launch_ce_count(targets, M, V, n_keep, st));
  for (int64_t r0 = 0; r0 < M; r0 += C) {
    const int64_t Mc = std::min(C, M - r0);
    // logits of the chunk (fp32), their row statistics and gradient, then dh = dz . W
    QL_LAUNCH("gemm_nt", st, launch_gemm_nt_bf16(h + r0 * H, Wp, Mc, H, V, logits, true, stats, st));
    QL_LAUNCH("ce_rows", st, launch_ce_rows(logits, stats, targets + r0, n_keep, Mc, V, loss_rows + r0, dz, st));
    QL_LAUNCH("gemm_nt", st, launch_gemm_nt_bf16(dz, Wtp, Mc, V, H, dh + r0 * H, false, nullptr, st));
  }
  QL_LAUNCH("ce_total", st, launch_ce_total(loss_rows, M, n_keep, loss, st));
  return QLORA_OK;
}

int qlora_profile_begin(int max_launches) {
  if (max_launches < 1) return QLORA_EINVAL;
  while ((int)g_prof.pool.size() < 2 * max_launches) {
    hipEvent_t e;
    QL_CHECK(hipEventCreate(&e));
    g_prof.pool.push_back(e);
  }
  g_prof.recs.clear();
  g_prof.recs.reserve((size_t)max_launches);  // no host allocation while recording
  g_prof.next = 0;
  g_prof.dropped = 0;
  g_prof.on = true;
  return QLORA_OK;
}

int qlora_profile_end(qlora_kernel_time* out, int max_entries, int* n_entries) {
  g_prof.on = false;
  int n = 0;
  for (const ProfRec& rec : g_prof.recs) {
    QL_CHECK(hipEventSynchronize(rec.b));
    float ms = 0.f;
    QL_CHECK(hipEventElapsedTime(&ms, rec.a, rec.b));
    int i = 0;
    for (; i < n; ++i)
      if (strncmp(out[i].name, rec.name, sizeof(out[i].name)) == 0) break;
    if (i == n) {
      if (n >= max_entries) continue;
      memset(&out[n], 0, sizeof(out[n]));
      strncpy(out[n].name, rec.name, sizeof(out[n].name) - 1);
      ++n;
    }
    out[i].launches += 1;
    out[i].total_ms += ms;
  }
  if (n_entries) *n_entries = n;
  g_prof.recs.clear();
  g_prof.next = 0;
  return g_prof.dropped ? QLORA_EUNSUPPORTED : QLORA_OK;
}

}  // extern "C"
