/*
 * gdpa.h - C ABI of the MI355X (gfx950) Generalized Dot Product Attention library.
 *
 * GDPA is dot-product attention whose softmax is replaced by a pointwise
 * activation (GDPA README, page "gdpa/README.md", intro).  There is no row
 * normaliser, so for every sequence b, query head h and its KV head
 * g = h / (Hq / Hkv):
 *
 *     S = scale * Q_bh K_bg^T        P = M .* act(S)        O_bh = P V_bg
 *
 * and, given dO, the backward products
 *
 *     dP = dO V^T   dS = M .* act'(S) .* dP   dQ = scale dS K
 *     dK = scale sum_{h in g} dS^T Q          dV = sum_{h in g} P^T dO.
 *
 * M is the attention mask (README "Features": causal, non-causal, sliding
 * window); masked pairs contribute exactly zero.  Jagged batches follow the
 * cu_seqlens/max_seqlen convention of the README's "CUTE-DSL" usage example
 * (flash_attn_varlen_func).  Head configurations MHA/GQA/MQA and the
 * activation list come from "Features"; FP8 (E4M3) is forward-only there.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains them; they must stay valid until the
 *    work queued on `stream` completes.
 *  - Layouts are row-major with the head dimension fastest:
 *      fixed length:  q [B, Lq, Hq, D], o/dO [B, Lq, Hq, Dv],
 *                     k [B, Lk, Hkv, D], v [B, Lk, Hkv, Dv]
 *      jagged:        q [total_q, Hq, D], o/dO [total_q, Hq, Dv],
 *                     k [total_k, Hkv, D], v [total_k, Hkv, Dv]
 *    with D = head_dim (Q and K) and Dv = head_dim_v (V and O); dq/dk/dv
 *    have the layouts of q/k/v.
 *    cu_seqlens_{q,k}: device int32 [B+1], cu[0] = 0, non-decreasing,
 *    cu[B] = total.  Zero-length sequences are allowed.
 *  - Element types: inputs bf16 or fp16; or 8- and 4-bit q/k with bf16 v
 *    (and dO): FP8 E4M3 codes with fp32 per-tensor descales (gdpa_fwd,
 *    gdpa_varlen_fwd), MXFP8 or MXFP4 codes with E8M0 block scales
 *    (gdpa_varlen_fwd_mxfp8, gdpa_varlen_fwd_mxfp4), and for the backward of
 *    all three gdpa_varlen_bwd_lowp.  Outputs fp32, bf16 or fp16 (fp32 is the
 *    mode whose accuracy the tests bound most tightly).
 *  - Outputs are overwritten, never accumulated into.  Query rows with no
 *    allowed key get O = 0 and dQ = 0; keys no query attends get dK = dV = 0.
 *    dK/dV are summed over the query heads of each KV group.
 *  - All work is queued on `stream` (a hipStream_t; NULL = default stream) and
 *    the call returns without synchronising.
 *  - Errors are returned as gdpa_status_t, never thrown.  Argument checks run
 *    on the host before any HIP call.  Invalid device data (e.g. a
 *    non-monotone cu_seqlens or a length above max_seqlen) is undefined
 *    behaviour, unless the environment variable GDPA_DEBUG_CHECKS is set to a
 *    value other than 0 at the call: jagged calls then copy cu_seqlens_q/k to
 *    the host (synchronising `stream`) and return GDPA_ERR_INVALID_ARG, with
 *    nothing queued, if cu[0] != 0, cu[B] != total, an entry decreases or a
 *    length exceeds max_seqlen.
 *  - Results are bitwise deterministic for a given input and launch.
 */
#ifndef GDPA_H_
#define GDPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDPA_ABI_VERSION 3  /* 2: head_dim_v after head_dim in the four entry points;
                               3: backward workspace queries take the dQ storage type
                               (and the jagged one total_q), fixed-length backward
                               calls need a workspace, GDPA_ERR_DEVICE_WAIT */

typedef enum {
  GDPA_OK = 0,
  GDPA_ERR_INVALID_ARG = 1,          /* null pointer, bad size, Hq % Hkv != 0, bad enum */
  GDPA_ERR_UNSUPPORTED = 2,          /* valid but not implemented (head dim, dtype combination) */
  GDPA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the *_workspace_size() query */
  GDPA_ERR_HIP = 4,                  /* a HIP runtime call or kernel launch failed */
  GDPA_ERR_DEVICE_WAIT = 5           /* debug mode only (GDPA_DEBUG_CHECKS): a wait of the
                                        ordered dQ reduction gave up; gradients are invalid */
} gdpa_status_t;

/* Activation replacing softmax (README "Features": custom activations).
 * GELU_TANH, FAST_GELU and FAST_GELU_BF16 all compute the tanh approximation
 * of GELU; SILU and FAST_SILU both compute x*sigmoid(x).  act_param is the
 * LeakyReLU negative slope and is ignored otherwise. */
typedef enum {
  GDPA_ACT_IDENTITY = 0,
  GDPA_ACT_GELU = 1,
  GDPA_ACT_GELU_TANH = 2,
  GDPA_ACT_FAST_GELU = 3,
  GDPA_ACT_FAST_GELU_BF16 = 4,
  GDPA_ACT_RELU = 5,
  GDPA_ACT_RELU2 = 6,
  GDPA_ACT_LEAKY_RELU = 7,
  GDPA_ACT_SILU = 8,
  GDPA_ACT_FAST_SILU = 9,
  GDPA_ACT_HARDSWISH = 10
} gdpa_act_t;

/* Mask (README "Features": causal, non-causal, sliding window).  Causal masks
 * align bottom-right: query i of a sequence with Lq queries and Lk keys may
 * see key j iff j <= i + Lk - Lq.  SLIDING_WINDOW allows
 * i' - window_left <= j <= i' + window_right with i' = i + Lk - Lq, where a
 * negative window side is unbounded.  For NONE and CAUSAL the window
 * arguments are ignored. */
typedef enum {
  GDPA_MASK_NONE = 0,
  GDPA_MASK_CAUSAL = 1,
  GDPA_MASK_SLIDING_WINDOW = 2
} gdpa_mask_t;

typedef enum {
  GDPA_DTYPE_BF16 = 0,
  GDPA_DTYPE_FP16 = 1,      /* IEEE binary16 */
  GDPA_DTYPE_FP8_E4M3 = 2,  /* OCP E4M3 codes, forward q/k only */
  GDPA_DTYPE_FP32 = 3,      /* outputs only */
  GDPA_DTYPE_MXFP8_E4M3 = 4, /* OCP MXFP8: E4M3 codes + E8M0 scales; gdpa_varlen_fwd_mxfp8 only */
  GDPA_DTYPE_MXFP4_E2M1 = 5  /* OCP MXFP4: E2M1 pairs + E8M0 scales; gdpa_varlen_fwd_mxfp4 only */
} gdpa_dtype_t;

/* ------------------------------------------------------------------ forward
 * O = M .* act(scale * q_descale * k_descale * Q K^T) V per (sequence, head).
 *   q, k, v, o     : device tensors in the layouts above.
 *   head_dim, head_dim_v : head dims of Q/K and of V/O: (64, 64), (96, 96),
 *                    (128, 128), or (192, 128) (the README's "(192, 128)"; 16-bit
 *                    inputs only).  Other pairs, and FP8 q/k at (192, 128),
 *                    return GDPA_ERR_UNSUPPORTED before anything is queued.
 *   scale          : multiplies Q K^T inside the activation (FA softmax_scale).
 *   qk_dtype, v_dtype : BF16 and BF16, FP16 and FP16, or FP8_E4M3 (q and k
 *                    codes) and BF16.  P is rounded to v's type for P V, so
 *                    other pairings return GDPA_ERR_UNSUPPORTED.  With FP16,
 *                    |act(scale q.k)| must stay below 65504 * scale (P is
 *                    kept unscaled in fp16; ReLU^2 scores above ~256 overflow).
 *   out_dtype      : GDPA_DTYPE_FP32, GDPA_DTYPE_BF16 or GDPA_DTYPE_FP16.
 *   q_descale, k_descale : per-tensor fp32 factors of FP8 codes (ignored for bf16).
 *   workspace      : device scratch of at least gdpa_*_workspace_size() bytes
 *                    (may be NULL when that size is 0); contents are clobbered.
 */
gdpa_status_t gdpa_fwd(const void* q, const void* k, const void* v, void* o,
                       int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                       int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v,
                       float scale, int32_t mask, int32_t window_left, int32_t window_right,
                       int32_t act, float act_param,
                       int32_t qk_dtype, int32_t v_dtype, int32_t out_dtype,
                       float q_descale, float k_descale,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Jagged forward.  max_seqlen_q/k are host upper bounds of the per-sequence
 * lengths (used to size the launch; no device->host copy is made);
 * total_q/total_k are the packed token counts (cu[B]); a total above batch x
 * max_seqlen returns GDPA_ERR_INVALID_ARG. */
gdpa_status_t gdpa_varlen_fwd(const void* q, const void* k, const void* v, void* o,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int64_t total_q, int64_t total_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v,
                              float scale, int32_t mask, int32_t window_left, int32_t window_right,
                              int32_t act, float act_param,
                              int32_t qk_dtype, int32_t v_dtype, int32_t out_dtype,
                              float q_descale, float k_descale,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Jagged forward with MXFP8 Q and K (the README's "Features" list MXFP8 among
 * its coming datatypes; the format is the OCP Microscaling Formats
 * specification's MXFP8 E4M3).  q [total_q, Hq, D] and k [total_k, Hkv, D]
 * hold E4M3 codes; q_scale [total_q, Hq, D/32] and k_scale [total_k, Hkv, D/32]
 * hold the E8M0 scale of each block of 32 consecutive head-dim elements
 * (value 2^(byte - 127); 255 is NaN), so element d of a row stands for
 * e4m3(code) * 2^(scale[d / 32] - 127).  v is bf16 [total_k, Hkv, D], o as in
 * gdpa_varlen_fwd.  head_dim is 64 or 128 (else GDPA_ERR_UNSUPPORTED); the
 * other arguments, the workspace and the errors are those of gdpa_varlen_fwd
 * (q_scale / k_scale NULL with work to do: GDPA_ERR_INVALID_ARG).  Both score
 * operands enter gfx950's block-scaled MFMA with their scales. */
gdpa_status_t gdpa_varlen_fwd_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                    const void* v, void* o,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int64_t total_q, int64_t total_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                    int32_t act, float act_param, int32_t out_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Jagged forward with MXFP4 Q and K (README "Features": "MXFP4 and MXFP8
 * forward & backward (coming soon)"; the format is the OCP Microscaling
 * Formats specification's MXFP4: FP4 E2M1 elements — 1 sign, 2 exponent bits
 * with bias 1, 1 mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 — with
 * one E8M0 scale per block of 32).  q [total_q, Hq, D / 2] and
 * k [total_k, Hkv, D / 2] bytes each hold two elements of a row: element 2 i
 * in the low nibble of byte i, element 2 i + 1 in the high nibble (the
 * specification leaves the packing open).  q_scale / k_scale, v, o, the head
 * dims (64 or 128), the other arguments, the workspace and the errors are
 * those of gdpa_varlen_fwd_mxfp8.  Both score operands enter gfx950's
 * block-scaled MFMA in its FP4 form with their scales. */
gdpa_status_t gdpa_varlen_fwd_mxfp4(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                    const void* v, void* o,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int64_t total_q, int64_t total_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                    int32_t act, float act_param, int32_t out_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- backward
 * Gradients of L = sum(O .* dO) for the forward above.  in_dtype (q, k, v and
 * dout) is GDPA_DTYPE_BF16 or GDPA_DTYPE_FP16; P and dS are rounded to it for
 * the products (an FP8 in_dtype returns GDPA_ERR_UNSUPPORTED here: 8- and
 * 4-bit Q/K take gdpa_varlen_bwd_lowp).  dq has q's layout, dk/dv have k's layout;
 * all three are written in grad_dtype (GDPA_DTYPE_FP32, GDPA_DTYPE_BF16 or
 * GDPA_DTYPE_FP16).  Head dims as in the forward: (64, 64), (96, 96),
 * (128, 128) or (192, 128) (dv then has v's 128 columns; dq and dk q's and
 * k's 192).
 * dQ sums the partial products of all key blocks in a fixed order, so results
 * are bitwise reproducible (an fp32 reduction inside the workspace, or inside
 * dq itself when grad_dtype is FP32: dq is then written more than once
 * during the call).
 * Partial gradients: dq == NULL skips dQ; dk == dv == NULL skips dK and dV
 * (e.g. frozen keys/values).  dk and dv must be both NULL or both non-NULL,
 * and at least one gradient must be requested (else GDPA_ERR_INVALID_ARG).
 * The workspace (gdpa_*bwd_workspace_size with this grad_dtype) is required
 * by every backward call that has work to do; it is cleared and written on
 * the device by the call itself. */
gdpa_status_t gdpa_bwd(const void* q, const void* k, const void* v, const void* dout,
                       void* dq, void* dk, void* dv,
                       int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                       int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v,
                       float scale, int32_t mask, int32_t window_left, int32_t window_right,
                       int32_t act, float act_param,
                       int32_t in_dtype, int32_t grad_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

gdpa_status_t gdpa_varlen_bwd(const void* q, const void* k, const void* v, const void* dout,
                              void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int64_t total_q, int64_t total_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v,
                              float scale, int32_t mask, int32_t window_left, int32_t window_right,
                              int32_t act, float act_param,
                              int32_t in_dtype, int32_t grad_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Jagged backward from 8- or 4-bit Q and K: the gradients of the forwards
 * above with FP8 (gdpa_varlen_fwd with GDPA_DTYPE_FP8_E4M3 q/k), MXFP8
 * (gdpa_varlen_fwd_mxfp8) or MXFP4 (gdpa_varlen_fwd_mxfp4) inputs.  The README
 * lists FP8 as forward-only and "MXFP4 and MXFP8 forward & backward (coming
 * soon)"; reading: the gradients of L = sum(O .* dO) with respect to the
 * values the codes stand for (code x per-tensor descale for FP8, code x
 * 2^(scale - 127) per block of 32 for the MX formats).
 *   q, q_scale, k, k_scale : as in the forward of qk_dtype (GDPA_DTYPE_FP8_E4M3
 *                    with q_scale = k_scale = NULL and the descales; the MX
 *                    dtypes with their scale arrays, descales ignored)
 *   v, dout        : bf16 [total_k, Hkv, D] and [total_q, Hq, D]
 *   dq, dk, dv     : as in gdpa_varlen_bwd (dq, dk with D columns, in
 *                    grad_dtype; NULL to skip as there)
 *   head_dim       : D of Q, K, V and O; the head dims of the format's
 *                    forward (FP8 64, 96, 128; MX 64, 128), else
 *                    GDPA_ERR_UNSUPPORTED
 * The codes are first decoded on the device into bf16 copies in the
 * workspace (the values are exact in bf16: E4M3 and E2M1 values, times a
 * power of two for the MX formats, unless a block scale takes them outside
 * bf16's normal range), then the 16-bit backward runs on them with the FP8
 * descales folded into the scalar factors of S, dQ and dK.  Workspace:
 * gdpa_varlen_bwd_lowp_workspace_size (the 16-bit backward's plus the two
 * copies).  Errors as in gdpa_varlen_bwd; every check runs before the first
 * launch. */
gdpa_status_t gdpa_varlen_bwd_lowp(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                   const void* v, const void* dout, void* dq, void* dk, void* dv,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int64_t total_q, int64_t total_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                   int32_t act, float act_param,
                                   int32_t qk_dtype, float q_descale, float k_descale, int32_t grad_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free jagged backward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as gdpa_varlen_bwd, without
 * the workspace: the call uses a scratch array of
 * GDPA_NOALLOC_SCRATCH_BYTES that the library keeps in every GPU's memory
 * for the life of the process, and allocates nothing.  A call whose
 * workspace query (gdpa_varlen_bwd_workspace_size) exceeds that size returns
 * GDPA_ERR_WORKSPACE_TOO_SMALL before launching anything (an fp32 gradient
 * never needs more than the sequence order, the queue state and one turn
 * counter per (64-row query tile, query head)).  All calls on one GPU share
 * its array and every call clears on the device what it needs cleared:
 * calls that can overlap on one GPU (different streams, or threads without
 * ordering) race and must be ordered by the caller. */
#define GDPA_NOALLOC_SCRATCH_BYTES (8u << 20)
gdpa_status_t gdpa_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* dout,
                                      void* dq, void* dk, void* dv,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int64_t total_q, int64_t total_k,
                                      int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                      int32_t head_dim_v,
                                      float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                      int32_t act, float act_param,
                                      int32_t in_dtype, int32_t grad_dtype, void* stream);

/* Workspace each call needs, in bytes (0 = none; pass NULL then).  Arguments
 * mirror the shape arguments of the matching entry point.
 * Forward: jagged calls of 1..4096 sequences need 4 bytes per sequence plus
 * 32, rounded up to 256: the call first builds there, on the device, the
 * order in which sequences are processed (costliest first: the most 64 x 64
 * (query, key) blocks holding a pair the mask allows) and the counters of
 * the work queues its kernels draw items from (see the README's load-balanced
 * scheduling of jagged batches).  Fixed-length calls and larger batches need
 * none.
 * Backward: the sequence order (jagged calls of up to 4096 sequences), 17
 * words of work-queue state and a failed-wait flag, one int32 turn counter
 * per (64-row query tile, query head) of the ordered dQ reduction, and, when
 * grad_dtype is 16-bit and dQ is reduced over several key blocks inside the
 * dK/dV pass (max seqlen_k > 128 with GDPA_BWD_DQ=fused set), an fp32 dQ
 * accumulator of total_q * num_heads_q * head_dim values; each part rounded
 * up to 256 bytes.  The queries read GDPA_BWD_DQ as the calls do.
 * A query whose answer would pass 2^60 bytes returns SIZE_MAX (no call can
 * be given that much).
 * A call given less than its query returns GDPA_ERR_WORKSPACE_TOO_SMALL before
 * launching anything.  The workspace is caller-owned and only used on the
 * call's stream; calls that share one must be ordered on one stream. */
size_t gdpa_fwd_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                               int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim);
size_t gdpa_varlen_fwd_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim);
size_t gdpa_bwd_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                               int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               int32_t grad_dtype);
size_t gdpa_varlen_bwd_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int64_t total_q, int32_t num_heads_q, int32_t num_heads_kv,
                                      int32_t head_dim, int32_t grad_dtype);
/* gdpa_varlen_bwd_lowp: the 16-bit backward's workspace (as
 * gdpa_varlen_bwd_workspace_size), then bf16 copies of Q and K
 * (total_q * num_heads_q + total_k * num_heads_kv rows of head_dim values),
 * each part rounded up to 256 bytes; SIZE_MAX past 2^60. */
size_t gdpa_varlen_bwd_lowp_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                           int64_t total_q, int64_t total_k, int32_t num_heads_q,
                                           int32_t num_heads_kv, int32_t head_dim, int32_t qk_dtype,
                                           int32_t grad_dtype);

/* Human-readable name of a status code (static storage; never NULL). */
const char* gdpa_status_string(gdpa_status_t status);

/* Returns GDPA_ABI_VERSION of the loaded library. */
int32_t gdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDPA_H_ */
