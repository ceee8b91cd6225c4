// C ABI of the fused QLoRA layer: argument checks, workspace carving and the
// kernel sequence of each call on the caller's stream. The math of each step
// is stated in include/qlora.h; the kernels live in quant.hip, skinny.hip and
// gemm.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool layer_ok(const qlora_layer* L) {
  if (!L || !L->codes || !L->absmax || !L->A || !L->B) return false;
  if (L->K <= 0 || L->K % 64 != 0 || L->N <= 0 || L->N % 8 != 0) return false;
  if (L->r < 1 || L->r > 256) return false;
  if (!aligned16(L->codes) || !aligned16(L->absmax) || !aligned16(L->A) || !aligned16(L->B)) return false;
  return true;
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

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

size_t tn_part_bytes(int64_t M, int64_t Kd, int64_t r) {
  return up256((size_t)skinny_tn_splits(M, Kd) * (size_t)r * (size_t)Kd * sizeof(float));
}

size_t bwd_ws(int64_t M, int64_t K, int64_t N, int64_t r) {
  const size_t part = std::max(tn_part_bytes(M, N, r), tn_part_bytes(M, K, r));
  return up256(r * N * 2) + up256(K * r * 2) + up256(M * r * 2) + part;
}

size_t mlp_bwd_ws(int64_t M, int64_t H, int64_t I, int64_t r) {
  size_t part = std::max(tn_part_bytes(M, H, r), tn_part_bytes(M, I, r));
  return 2 * up256((size_t)M * I * 2) + 3 * up256(M * r * 2) + up256(r * H * 2) + 2 * up256(r * I * 2) +
         up256(I * r * 2) + 2 * up256(H * r * 2) + part;
}

WSrc wsrc(const qlora_layer* L, const uint16_t* lora_i, const uint16_t* lora_j) {
  WSrc w;
  w.codes = L->codes;
  w.absmax = L->absmax;
  w.lora_i = lora_i;
  w.lora_j = lora_j;
  w.r = (int)L->r;
  w.s = L->s;
  return w;
}

// dOut = s * P^T . Q reduced over M (P [M,r], Q [M,Kd]); transposed -> [Kd, r]
int tn_reduce(const uint16_t* P, int r, const uint16_t* Q, int64_t M, int64_t Kd, float s, float* out,
              bool transposed, float* part, hipStream_t st) {
  const int splits = skinny_tn_splits(M, Kd);
  QL_LAUNCH("skinny_tn", st, launch_skinny_tn(P, r, Q, M, Kd, part, splits, st));
  QL_LAUNCH("reduce_splits", st, launch_reduce_splits(part, splits, r, Kd, s, out, transposed, st));
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument (shape, null or misaligned pointer)";
    case QLORA_EUNSUPPORTED: return "unsupported";
    case QLORA_EWORKSPACE: return "workspace missing or too small";
    case QLORA_EHIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

const char* qlora_last_error(void) { return g_err; }

int qlora_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax, uint32_t* nonfinite_blocks,
                   void* stream) {
  if (N < 0 || K < 0 || K % 64 != 0) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!W || !codes || !absmax || !aligned16(W) || !aligned16(codes)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("quantize", st, launch_quantize(W, N, K, codes, absmax, nonfinite_blocks, st));
  return QLORA_OK;
}

int qlora_dequantize(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat, void* stream) {
  if (N < 0 || K < 0 || K % 64 != 0) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!codes || !absmax || !W_hat || !aligned16(W_hat)) return QLORA_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  QL_LAUNCH("dequantize", st, launch_dequantize(codes, absmax, N, K, W_hat, st));
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
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(X, M, L->K, L->A, r, Z_save, nullptr, 0, nullptr, st));
  QL_LAUNCH("gemm_fwd", st, launch_gemm_fwd(X, M, L->K, L->N, wsrc(L, L->B, Z_save), Y, st));
  return QLORA_OK;
}

int qlora_backward(const qlora_layer* L, const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save, int64_t M,
                   uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (!layer_ok(L) || M < 0) return QLORA_EINVAL;
  if (!dA || !dB) return QLORA_EINVAL;
  const int64_t K = L->K, N = L->N;
  const int r = (int)L->r;
  hipStream_t st = (hipStream_t)stream;
  if (M > 0) {
    if (!dY || !X || !Z_save || !aligned16(dY) || !aligned16(X) || !aligned16(Z_save)) return QLORA_EINVAL;
    if (dX && !aligned16(dX)) return QLORA_EINVAL;
  }
  const size_t need = bwd_ws(M, K, N, r);
  if (!ws || ws_bytes < need) return QLORA_EWORKSPACE;
  Carve c{(char*)ws, ws_bytes};
  uint16_t* Bt = c.take<uint16_t>((size_t)r * N);
  uint16_t* At = c.take<uint16_t>((size_t)K * r);
  uint16_t* G = c.take<uint16_t>((size_t)M * r);
  float* part = c.take<float>((size_t)std::max(tn_part_bytes(M, N, r), tn_part_bytes(M, K, r)) / sizeof(float));
  if (!c.ok) return QLORA_EWORKSPACE;
  if (M == 0) {  // empty batch: gradients are zero
    QL_LAUNCH("fill_zero_f32", st, launch_fill_zero_f32(dA, (int64_t)r * K, st));
    QL_LAUNCH("fill_zero_f32", st, launch_fill_zero_f32(dB, (int64_t)N * r, st));
    return QLORA_OK;
  }
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(L->B, N, r, Bt, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(L->A, r, K, At, st));
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(dY, M, N, Bt, r, G, nullptr, 0, nullptr, st));
  int rc = tn_reduce(Z_save, r, dY, M, N, L->s, dB, true, part, st);
  if (rc) return rc;
  if (dX) QL_LAUNCH("gemm_bwd", st, launch_gemm_bwd(dY, wsrc(L, At, G), nullptr, WSrc{}, M, K, N, dX, st));
  return tn_reduce(G, r, X, M, K, L->s, dA, false, part, st);
}

static bool mlp_shapes_ok(const qlora_layer* g, const qlora_layer* u, const qlora_layer* d) {
  if (!layer_ok(g) || !layer_ok(u) || !layer_ok(d)) return false;
  if (g->K != u->K || g->N != u->N || d->K != g->N || d->N != g->K) return false;
  if (g->r != u->r || g->r != d->r) return false;
  return true;
}

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
  hipStream_t st = (hipStream_t)stream;
  const int64_t H = gate->K, I = gate->N;
  const int r = (int)gate->r;
  uint16_t* Zg = Z_save;
  uint16_t* Zu = Z_save + (size_t)M * r;
  uint16_t* Zd = Z_save + 2 * (size_t)M * r;
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(X, M, H, gate->A, r, Zg, up->A, r, Zu, st));
  QL_LAUNCH("gemm_fwd_gateup", st, launch_gemm_fwd_gateup(X, M, H, I, wsrc(gate, gate->B, Zg), wsrc(up, up->B, Zu), g_save, u_save, h_save,
                                  st));
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(h_save, M, I, down->A, r, Zd, nullptr, 0, nullptr, st));
  QL_LAUNCH("gemm_fwd", st, launch_gemm_fwd(h_save, M, I, H, wsrc(down, down->B, Zd), Y, st));
  return QLORA_OK;
}

int swiglu_mlp_backward(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down, const uint16_t* dY,
                        const uint16_t* X, const uint16_t* g_save, const uint16_t* u_save, const uint16_t* h_save,
                        const uint16_t* Z_save, int64_t M, uint16_t* dX, float* const dA[3], float* const dB[3],
                        void* ws, size_t ws_bytes, void* stream) {
  if (!mlp_shapes_ok(gate, up, down) || M < 0 || !dA || !dB) return QLORA_EINVAL;
  for (int i = 0; i < 3; ++i)
    if (!dA[i] || !dB[i]) return QLORA_EINVAL;
  const int64_t H = gate->K, I = gate->N;
  const int r = (int)gate->r;
  hipStream_t st = (hipStream_t)stream;
  if (M > 0) {
    if (!dY || !X || !g_save || !u_save || !h_save || !Z_save) return QLORA_EINVAL;
    if (!aligned16(dY) || !aligned16(X) || !aligned16(g_save) || !aligned16(u_save) || !aligned16(h_save) ||
        !aligned16(Z_save) || (dX && !aligned16(dX)))
      return QLORA_EINVAL;
  }
  const size_t need = mlp_bwd_ws(M, H, I, r);
  if (!ws || ws_bytes < need) return QLORA_EWORKSPACE;
  Carve c{(char*)ws, ws_bytes};
  uint16_t* dg = c.take<uint16_t>((size_t)M * I);
  uint16_t* du = c.take<uint16_t>((size_t)M * I);
  uint16_t* Gd = c.take<uint16_t>((size_t)M * r);
  uint16_t* Gg = c.take<uint16_t>((size_t)M * r);
  uint16_t* Gu = c.take<uint16_t>((size_t)M * r);
  uint16_t* Btd = c.take<uint16_t>((size_t)r * H);
  uint16_t* Btg = c.take<uint16_t>((size_t)r * I);
  uint16_t* Btu = c.take<uint16_t>((size_t)r * I);
  uint16_t* Atd = c.take<uint16_t>((size_t)I * r);
  uint16_t* Atg = c.take<uint16_t>((size_t)H * r);
  uint16_t* Atu = c.take<uint16_t>((size_t)H * r);
  float* part = c.take<float>(std::max(tn_part_bytes(M, H, r), tn_part_bytes(M, I, r)) / sizeof(float));
  if (!c.ok) return QLORA_EWORKSPACE;
  if (M == 0) {
    const qlora_layer* Ls[3] = {gate, up, down};
    for (int i = 0; i < 3; ++i) {
      QL_LAUNCH("fill_zero_f32", st, launch_fill_zero_f32(dA[i], (int64_t)r * Ls[i]->K, st));
      QL_LAUNCH("fill_zero_f32", st, launch_fill_zero_f32(dB[i], (int64_t)Ls[i]->N * r, st));
    }
    return QLORA_OK;
  }
  const uint16_t* Zg = Z_save;
  const uint16_t* Zu = Z_save + (size_t)M * r;
  const uint16_t* Zd = Z_save + 2 * (size_t)M * r;
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(down->B, H, r, Btd, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(gate->B, I, r, Btg, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(up->B, I, r, Btu, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(down->A, r, I, Atd, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(gate->A, r, H, Atg, st));
  QL_LAUNCH("transpose_bf16", st, launch_transpose_bf16(up->A, r, H, Atu, st));
  // down projection: G_d = dY.B_d ; dB_d = s.dY^T.Z_d ; dh -> (dg, du) in the GEMM epilogue ; dA_d = s.G_d^T.h
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(dY, M, H, Btd, r, Gd, nullptr, 0, nullptr, st));
  int rc = tn_reduce(Zd, r, dY, M, H, down->s, dB[2], true, part, st);
  if (rc) return rc;
  QL_LAUNCH("gemm_bwd_swiglu", st, launch_gemm_bwd_swiglu(dY, wsrc(down, Atd, Gd), M, I, H, g_save, u_save, dg, du, st));
  rc = tn_reduce(Gd, r, h_save, M, I, down->s, dA[2], false, part, st);
  if (rc) return rc;
  // gate and up: G = d(g|u).B ; dB = s.d(g|u)^T.Z
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(dg, M, I, Btg, r, Gg, nullptr, 0, nullptr, st));
  QL_LAUNCH("skinny_nt", st, launch_skinny_nt(du, M, I, Btu, r, Gu, nullptr, 0, nullptr, st));
  rc = tn_reduce(Zg, r, dg, M, I, gate->s, dB[0], true, part, st);
  if (rc) return rc;
  rc = tn_reduce(Zu, r, du, M, I, up->s, dB[1], true, part, st);
  if (rc) return rc;
  // dX = dg.W_g + du.W_u + s.G_g.A_g + s.G_u.A_u : one GEMM over the concatenated reduction
  if (dX) QL_LAUNCH("gemm_bwd", st, launch_gemm_bwd(dg, wsrc(gate, Atg, Gg), du, wsrc(up, Atu, Gu), M, H, I, dX, st));
  rc = tn_reduce(Gg, r, X, M, H, gate->s, dA[0], false, part, st);
  if (rc) return rc;
  return tn_reduce(Gu, r, X, M, H, up->s, dA[1], false, part, st);
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
