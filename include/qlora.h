/*
 * qlora.h -- C ABI of the MI355X (gfx950) fused QLoRA linear layer.
 *
 * What is computed (sources are the pages' titles and passages):
 *   A frozen weight W [N,K] is stored in 4 bits and a trainable rank-r LoRA
 *   pair (A [r,K], B [N,r]) sits on it ("Rev vs unsloth", fused quantized-LoRA
 *   card; "Unsloth vs The Stack v2", quantized-base card: 4-bit weights stay
 *   frozen, only the adapters train). With s = lora_alpha / r:
 *       Y  = X.W^T + s.(X.A^T).B^T
 *       dX = dY.W + s.(dY.B).A
 *       dB = s.dY^T.(X.A^T)         dA = s.(dY.B)^T.X        (no dW: W is frozen)
 *   These are the hand-derived LoRA gradients of the "Unsloth" wiki entry
 *   (Theory) and of the "Unsloth vs PyTorch" video (0:43-1:24); every product
 *   is bracketed through the skinny M x r tensors so the N x K matrix B.A is
 *   never formed (same video, 1:35-2:00). The SwiGLU block of the wiki entry
 *   (Theory: fused SwiGLU) is g = lin_gate(X), u = lin_up(X),
 *   h = silu(g)*u, Y = lin_down(h), LoRA on all three projections.
 *
 * 4-bit format (the pages say only "4-bit" bitsandbytes checkpoints; this is
 * the NF4 reading): per row n and 64-column block b, absmax = max |W|,
 * code = nearest of the 16 NormalFloat-4 levels to W/absmax (fp32 division;
 * ties to the lower level), two codes per byte (byte order below);
 * dequantized weight What = fp32(L[code] * absmax). A block of zeros has
 * absmax 0 and code 7 (the exact zero level).
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned. bf16 tensors are passed as uint16_t bit
 *     patterns. The library allocates no device memory; scratch space comes
 *     from the caller's workspace (size from qlora_workspace_size).
 *   - Shapes: K % 64 == 0, N % 8 == 0, 1 <= r <= 256, K and N <= 2^21,
 *     N*K <= 2^31 (2^30 for the 8-bit formats), M >= 0 (M == 0 is a no-op; a backward then writes zero
 *     gradients). Anything else returns QLORA_EINVAL before any launch.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t, 0 = the
 *     null stream) and returns without synchronising. (The token-tiled SwiGLU
 *     calls also run part of their work on a second stream of the library's,
 *     ordered against `stream` by events.) Launch failures return
 *     QLORA_EHIP; qlora_last_error() gives the HIP error text.
 *   - Calls are re-entrant; concurrent calls must not share output or
 *     workspace buffers.
 *   - Matrix products accumulate in fp32. Y, dX, Z, g, u, h are rounded once
 *     to bf16 (round to nearest even). dA and dB are summed in fp32 and
 *     written in the layer's grad_dtype: bf16 (rounded once, the default and
 *     the adapters' parameter type) or fp32.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_EINVAL = -1,       /* bad shape, null pointer, misalignment */
  QLORA_EUNSUPPORTED = -2, /* valid request this build does not handle */
  QLORA_EWORKSPACE = -3,   /* workspace missing or smaller than qlora_workspace_size */
  QLORA_EHIP = -4,         /* a HIP launch failed; see qlora_last_error() */
  QLORA_ENONFINITE = -5    /* qlora_quantize (synchronous form): W holds Inf or NaN */
} qlora_status;

/* Formats of the frozen weight ("Rev vs unsloth", fused quantized-LoRA card:
 * int4, int8 and fp8 base weights; "Unsloth vs The Stack v2": 4-bit and
 * 8-bit). All keep one fp32 per 64-element block of a weight row (the
 * `absmax` array):
 *   QLORA_FMT_NF4   codes [N, K/2], 4-bit NormalFloat levels (below); the block
 *                   value is its absmax.
 *   QLORA_FMT_INT8  codes [N, K], two's-complement q in [-127, 127]; the block
 *                   value is s = absmax / 127, q = rint(W / s) (half to even).
 *   QLORA_FMT_FP8   codes [N, K], OCP E4M3 bytes (bias 7, max 448); the block
 *                   value is s = absmax / 448, code = nearest E4M3 value to
 *                   W / s (ties to the even code), saturating at 448.
 * A block of zeros stores 0 and zero codes (NF4: code 7). The dequantized
 * weight is fp32(v * block value) for the code's exact value v.
 * Storage order (codes and block values alike): rows in groups of 64 (the
 * last group may hold fewer, nr, rows); within a group, its 64-column blocks
 * one after the other, each holding the group's nr rows in order. Row n's
 * codes for block b therefore start at byte
 *   g*K/64*bb + (b*nr + r)*bb      (g = n - n%64, r = n%64, bb = 32 or 64)
 * and its block value sits at index g*K/64 + b*nr + r; the sizes are those of
 * the row-major arrays. (The GEMMs then read a whole tile of a row group as
 * one contiguous run.) Inside a row's 32 NF4 bytes of a block, each run of 8
 * columns 8j .. 8j+7 takes 4 bytes, byte b holding column 8j+b in its low
 * nibble and column 8j+b+4 in its high nibble (the order the GEMMs decode
 * fastest); the 8-bit formats keep one byte per column in column order.
 * qlora_quantize writes this order, every call reads it; qlora_pack_codes
 * converts codes and block values from the row-major checkpoint order. */
typedef enum { QLORA_FMT_NF4 = 0, QLORA_FMT_INT8 = 1, QLORA_FMT_FP8 = 2 } qlora_format;

/* Type of the adapter gradients dA, dB written by the backward calls. */
typedef enum { QLORA_GRAD_BF16 = 0, QLORA_GRAD_F32 = 1 } qlora_grad_dtype;

typedef enum {
  QLORA_OP_FORWARD = 0,
  QLORA_OP_BACKWARD = 1,
  QLORA_OP_MLP_FORWARD = 2,
  QLORA_OP_MLP_BACKWARD = 3
} qlora_op;

/* One LoRA-adapted quantized projection: out = in . What^T + s . (in . A^T) . B^T. */
typedef struct {
  const uint8_t* codes;  /* NF4: [N, K/2] bytes, two 4-bit codes per byte; INT8, FP8: [N, K];
                            in the storage order described with qlora_format */
  const float* absmax;   /* [N, K/64] fp32 value of each 64-column block (see qlora_format) */
  const uint16_t* A;     /* [r, K]    bf16 LoRA down projection */
  const uint16_t* B;     /* [N, r]    bf16 LoRA up projection */
  int64_t K;             /* input features */
  int64_t N;             /* output features */
  int64_t r;             /* LoRA rank */
  float s;               /* lora_alpha / r */
  int32_t format;        /* qlora_format of codes/absmax */
  int32_t grad_dtype;    /* qlora_grad_dtype of dA, dB (0: bf16) */
} qlora_layer;

/* Quantize W [N,K] fp32 to codes and absmax [N,K/64] in `format` (qlora_format).
 * A block holding Inf/NaN gets absmax = NaN and unspecified codes, and is
 * counted:
 *   - nonfinite_blocks != NULL (device uint32): the count is written there and
 *     the call stays asynchronous, like every other call;
 *   - nonfinite_blocks == NULL: the library counts in a device word of its own
 *     (one per GPU), synchronizes `stream` (whose device must be the current
 *     one) and returns QLORA_ENONFINITE if any block was non-finite. Such calls
 *     are serialized inside the library.
 * Setup-time call. */
int qlora_quantize(int format, const float* W, int64_t N, int64_t K, uint8_t* codes, float* absmax,
                   uint32_t* nonfinite_blocks, void* stream);

/* Take codes and block values in the row-major order of a pre-quantized
 * checkpoint ("Unsloth" wiki entry, API; "Unsloth -- the speed layer" lesson:
 * 4-bit bitsandbytes checkpoints loaded as they are) and write this library's
 * storage order (described with qlora_format). Source: NF4 codes [N, K/2],
 * column 2c in the low nibble and 2c+1 in the high nibble of byte c; INT8/FP8
 * codes [N, K], one byte per column; block values src_absmax [N, K/64] fp32.
 * Destinations have the same sizes and must not overlap the sources. All
 * pointers 16-byte aligned; K % 64 == 0. */
int qlora_pack_codes(int format, const uint8_t* src_codes, const float* src_absmax, int64_t N, int64_t K,
                     uint8_t* codes, float* absmax, void* stream);

/* What [N,K] fp32 = fp32(v(code) * absmax), decoded as the GEMMs decode it.
 * Exposes the exact operand values for testing. */
int qlora_dequantize(int format, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, float* W_hat,
                     void* stream);

/* Workspace bytes needed by `op` (qlora_op) for M tokens. For the MLP ops,
 * K is the model width and N the intermediate width. */
size_t qlora_workspace_size(int op, int64_t M, int64_t K, int64_t N, int64_t r);

/* Forward of one projection. X [M,K] bf16 -> Y [M,N] bf16 and Z_save = X.A^T
 * [M,r] bf16 (kept for the backward). Needs no workspace (ws may be NULL). */
int qlora_forward(const qlora_layer* L, const uint16_t* X, int64_t M, uint16_t* Y, uint16_t* Z_save,
                  void* ws, size_t ws_bytes, void* stream);

/* Backward of one projection for upstream dY [M,N]. Writes dX [M,K] bf16
 * (dX may be NULL to skip it), dA [r,K] and dB [N,r] in L->grad_dtype.
 * X and Z_save are the forward's input and saved tensor. */
int qlora_backward(const qlora_layer* L, const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save,
                   int64_t M, uint16_t* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream);

/* qlora_backward for callers that cannot allocate device memory (code under
 * graph capture, serving loops, harnesses that forbid it): the same kernels
 * and results, with the workspace taken from a scratch array inside the
 * library (QLORA_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends)
 * instead of a caller buffer. The call allocates nothing. A backward whose
 * workspace (qlora_workspace_size(QLORA_OP_BACKWARD, ...)) exceeds the limit
 * returns QLORA_EWORKSPACE (qlora_last_error() gives both sizes). Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams or threads) race and must be serialized by the caller. The current
 * device must be the stream's device. */
#define QLORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int qlora_backward_noalloc(const qlora_layer* L, const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save,
                           int64_t M, uint16_t* dX, void* dA, void* dB, void* stream);

/* SwiGLU MLP forward: g = lin_gate(X), u = lin_up(X), h = silu(g)*u,
 * Y = lin_down(h). gate/up: K = H (model width), N = I; down: K = I, N = H.
 * Saves g, u, h [M,I] bf16 and Z_save [3][M][r] (gate, up, down) for the
 * backward. All three layers must share r, format and grad_dtype. Needs no
 * workspace. */
int swiglu_mlp_forward(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                       const uint16_t* X, int64_t M, uint16_t* Y, uint16_t* g_save, uint16_t* u_save,
                       uint16_t* h_save, uint16_t* Z_save, void* ws, size_t ws_bytes, void* stream);

/* SwiGLU MLP backward for upstream dY [M,H]. dA[i], dB[i] (i = 0 gate,
 * 1 up, 2 down) receive [r,K_i] and [N_i,r] in the layers' grad_dtype;
 * dX [M,H] bf16 may be NULL. */
int swiglu_mlp_backward(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                        const uint16_t* dY, const uint16_t* X, const uint16_t* g_save, const uint16_t* u_save,
                        const uint16_t* h_save, const uint16_t* Z_save, int64_t M, uint16_t* dX,
                        void* const dA[3], void* const dB[3], void* ws, size_t ws_bytes, void* stream);

/* Token-tiled SwiGLU block ("Unsloth vs PyTorch" video, 4:25-4:36: tiled
 * feed-forward layers for long context). The batch is cut into tiles of
 * `tile` tokens (the last one ragged), and only one tile's intermediates exist
 * at a time:
 *   forward  - per tile, g, u, h are formed in the workspace and dropped after
 *              the tile's Y rows; nothing of size M x I is saved. Z_save
 *              [3][M][r] (gate, up, down) is written as by swiglu_mlp_forward.
 *   backward - per tile, g, u, h are recomputed from X and Z_save (the same
 *              kernels on the same inputs: bitwise the forward's values), then
 *              the block's backward runs on the tile; dX rows are written per
 *              tile and dA/dB are summed over the tiles in tile order.
 * Y, Z_save and dX equal swiglu_mlp_forward/backward's bit for bit (every
 * token's row is computed the same way); dA and dB differ only by the fp32
 * summation order across tiles (identical when tile >= M); bf16 gradients
 * are summed over the tiles in fp32 and rounded once at the end. The workspace
 * scales with min(tile, M), not M: size from
 * swiglu_mlp_tiled_workspace_size(backward = 0 or 1, M, H, I, r, tile).
 * tile >= 1 (a multiple of 256 keeps every GEMM tile full).
 * With more than one tile, when a tile's last GEMM would leave CUs idle
 * (ceil(tile/256) * ceil(H/256) < 256 workgroups), the last part of each tile
 * runs on a second stream beside the next tile's work on `stream`: the
 * forward's down projection GEMM, and the backward's gate and up part (their
 * G products, reductions and the dX GEMM). The second stream is kept by the library, one per device,
 * created on first use. Events order it against `stream`, and every such part
 * is done before work enqueued on `stream` after the call starts. Results are
 * those of a single-stream run: the same kernels run on the same inputs, and
 * each gradient adds its tiles in order on one stream. The buffers that the
 * second stream reads (h; dg and du) are held twice in the workspace. Calls
 * from several threads on one device share that stream, so their second-stream
 * parts run one after another. The calls can be captured in a HIP graph once
 * that stream exists (after one such call on the device): it joins the
 * capture through the events. */
size_t swiglu_mlp_tiled_workspace_size(int backward, int64_t M, int64_t H, int64_t I, int64_t r, int64_t tile);
int swiglu_mlp_forward_tiled(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                             const uint16_t* X, int64_t M, int64_t tile, uint16_t* Y, uint16_t* Z_save, void* ws,
                             size_t ws_bytes, void* stream);
int swiglu_mlp_backward_tiled(const qlora_layer* gate, const qlora_layer* up, const qlora_layer* down,
                              const uint16_t* dY, const uint16_t* X, const uint16_t* Z_save, int64_t M, int64_t tile,
                              uint16_t* dX, void* const dA[3], void* const dB[3], void* ws, size_t ws_bytes,
                              void* stream);

/* RMSNorm before the projections ("Unsloth" wiki entry, Theory: fused RMSNorm
 * kernel; no formula on the pages, the Llama definition is taken): per row of
 * x [M,H] bf16, rstd = 1/sqrt(mean(x^2) + eps) (fp32, saved [M]) and
 * y = bf16(w * (x * rstd)) with the frozen bf16 weight w [H]. H % 8 == 0,
 * eps >= 0. One pass over x. */
int qlora_rmsnorm_forward(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, float eps, uint16_t* y,
                          float* rstd, void* stream);

/* Backward of the RMSNorm for upstream dy [M,H]: dx = rstd * (g - n * mean(g * n))
 * with g = w * dy and n = x * rstd (rstd from the forward). w is frozen with the
 * base model, so no weight gradient is formed. dx may not alias dy or x. */
int qlora_rmsnorm_backward(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd, int64_t M,
                           int64_t H, uint16_t* dx, void* stream);

/* Rotary position embeddings after the q and k projections ("Unsloth" wiki
 * entry, Theory: fused RoPE kernel; "Unsloth vs PyTorch" video, 2:11-2:22),
 * in place on q [M, hq*d] and k [M, hk*d] bf16 (hq or hk may be 0; q or k is
 * then ignored). Token m has position pos[m] (int32, device) and each head
 * vector is rotated pairwise, element i with element i + d/2 ("rotate half"):
 *   a = pos * base^(-2i/d),  v[i] <- v[i] cos a - v[i+d/2] sin a,
 *                            v[i+d/2] <- v[i+d/2] cos a + v[i] sin a.
 * The angles and their cos/sin are formed in fp64, the rotation in fp32,
 * one bf16 rounding. 16 <= d <= 1024, d % 16 == 0, base > 1.
 * qlora_rope_backward applies the inverse rotation to the gradients dq, dk. */
int qlora_rope_forward(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t M, int hq, int hk, int d, float base,
                       void* stream);
int qlora_rope_backward(uint16_t* dq, uint16_t* dk, const int32_t* pos, int64_t M, int hq, int hk, int d, float base,
                        void* stream);

/* cos/sin table of the RoPE angles for positions 0 .. max_pos-1:
 * table[(p*d/2 + i)*2 + 0] = cos(p * base^(-2i/d)), [.. + 1] = sin(..), fp32
 * values of the fp64 angles and sin/cos (as qlora_rope_forward forms them).
 * [max_pos][d/2][2] floats; built once and shared by every layer.
 * 16 <= d <= 1024, d % 16 == 0, base > 1, max_pos <= 2^21. */
int qlora_rope_table(int d, float base, int64_t max_pos, float* table, void* stream);

/* Forward of a q or k projection with RoPE fused into its GEMM ("Unsloth"
 * wiki entry, Theory: fused RoPE kernel; "Unsloth vs PyTorch" video,
 * 2:11-2:22): Y = rope(X.W^T + s.(X.A^T).B^T) by pos [M] (int32), heads of
 * d = 128 output columns (N % 128 == 0), rotate-half pairing as in
 * qlora_rope_forward, applied to the fp32 GEMM result before its one bf16
 * rounding; Z_save = X.A^T as in qlora_forward. `table` is qlora_rope_table's
 * for this d and base, covering every position (0 <= pos < max_pos; a position
 * outside it gives zeros in its row, no fault). The backward is
 * qlora_rope_backward on dY (in place) followed by qlora_backward. */
int qlora_forward_rope(const qlora_layer* L, const uint16_t* X, int64_t M, const int32_t* pos, const float* table,
                       int64_t max_pos, int d, uint16_t* Y, uint16_t* Z_save, void* stream);

/* Cross-entropy over the frozen language-model head, chunked over tokens so
 * that the [M, V] logits never exist ("Unsloth" wiki entry, Theory: chunked
 * cross-entropy; "Unsloth vs PyTorch" video, 3:06-3:51). For h [M,H] (bf16,
 * the final hidden states), W [V,H] (bf16 head) and targets [M] (int32;
 * t < 0 or t >= V ignores the row):
 *   z = h . W^T, lse_m = log sum_v exp z[m,v], loss_m = lse_m - z[m,t_m],
 *   loss = sum over kept rows / n (n = kept rows; 0 if none),
 *   dh = dz . W with dz = (softmax(z) - onehot(t)) / n on kept rows, 0 elsewhere.
 * Per chunk of `chunk` tokens the logits are formed in fp32 in the workspace
 * (with each row's max and sum of exp over every 256-column tile, so the row
 * statistics take no extra pass over the logits), turned into dz (bf16) and
 * multiplied back; the
 * workspace holds one chunk (qlora_ce_workspace_size), so memory follows the
 * chunk, not M. W is frozen: no weight gradient. qlora_lmhead_prepare lays
 * W out once for the two products: Wp (for z = h . W^T) and Wtp (for dh =
 * dz . W), each V*H bf16 values in 64 x 64 blocks ordered as the GEMM's lanes
 * read them (block (g, t) of the product's weight [N, K] -- W itself or W^T --
 * at (g*K/64 + t)*4096 values; in it, the values k = 64t + 32hh + 8ks .. +7 of
 * row n = 64g + 32f + j at ((4f + ks)*64 + j + 32hh)*8 values). loss (1
 * float), loss_rows [M] (0 on ignored rows) and dh [M,H] are device outputs.
 * H % 64 == 0, V % 64 == 0, H, V <= 2^21, H*V <= 2^30. */
int qlora_lmhead_prepare(const uint16_t* W, int64_t V, int64_t H, uint16_t* Wp, uint16_t* Wtp, void* stream);
size_t qlora_ce_workspace_size(int64_t M, int64_t V, int64_t chunk);
int qlora_chunked_ce(const uint16_t* h, const uint16_t* Wp, const uint16_t* Wtp, const int32_t* targets, int64_t M,
                     int64_t H, int64_t V, int64_t chunk, float* loss, float* loss_rows, uint16_t* dh, void* ws,
                     size_t ws_bytes, void* stream);

/* Measurement support (off the hot path; not thread-safe).
 * qlora_profile_begin creates, once, a pool of 2*max_launches hipEvents and
 * from then on brackets each kernel launch made by this library with an event
 * pair recorded on that launch's stream. qlora_profile_end waits for those
 * events, stops recording and writes one entry per kernel class (launch count
 * and summed event time). It returns QLORA_EUNSUPPORTED if more launches were
 * made than the pool could hold (those were not timed). No call allocates
 * anything while recording. */
typedef struct {
  char name[32];
  int64_t launches;
  double total_ms;
} qlora_kernel_time;
int qlora_profile_begin(int max_launches);
int qlora_profile_end(qlora_kernel_time* out, int max_entries, int* n_entries);

/* Short text for a status code; for QLORA_EHIP, the last HIP error seen by this thread. */
const char* qlora_status_string(int status);
const char* qlora_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_H */
