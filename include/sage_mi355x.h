/*
 * sage_mi355x.h -- C ABI of libsage_mi355x.so: the SageAttention2-style quantised
 * softmax attention forward ("sage2") for AMD Instinct MI355X (gfx950).
 *
 * The operation is the dense, non-causal attention O = softmax(Q K^T * sm_scale) V
 * of a video diffusion transformer block, B sequences of N packed tokens, H heads
 * of D = 128 channels.  The pages this follows are benchmark artefacts that name
 * its stages and shapes but print no arithmetic:
 *   - "gb10-sampling-component-profile-1344x768-124f-seed440420.json",
 *     attention_internal_p50_milliseconds.sage2: qk_quantize, v_quantize,
 *     attention_forward, framework_and_k_smoothing_estimate (sage_quantize_qk,
 *     sage_quantize_v and sage_attn_fwd are those stages; the K smoothing
 *     statistic is computed inside sage_quantize_qk);
 *   - "gb10-sage2-p0-interleave-softmax-latency.json", q_shape [1, 37810, 56, 128]
 *     and scheduler (64-key tiles, cta_k = 64; 32-query warps, warp_q = 32);
 *   - "gb10-sage-strided-nhd-summary-1344x768-124f-seed440420.json", dataflow:
 *     Q/K/V are read as strided views of the QKV projection output with no
 *     materialising copy, and the output is written token-major for out_proj;
 *     next_targets on the profile page asks for exactly such a dense kernel.
 * The arithmetic is SageAttention2's: INT8 Q and K with per-block fp32 scales
 * amax / 127 and round-to-nearest-even, K smoothed by its per-head token mean,
 * OCP FP8 E4M3 V with per-channel scales amax / 448, an fp32 online softmax over
 * 64-key tiles, and P rounded to E4M3 (as 448 * p) for the FP8 P.V product.
 *
 * Around that path: sage_attn_fwd_bf16 (the unquantised path), sage_attn_fwd_int8qk
 * (INT8 Q K^T with an unquantised P.V), sage_quantize_qkv (both quantisers in one
 * call), sage_qk_norm_rope and sage_quantize_qkv_rope (the RMSNorm + RoPE step
 * before quantisation, in place or fused), and sage_attn_fwd_mx / sage_mx_quantize
 * (the output as OCP MX blocks for the projection after attention).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers; `stream` is a hipStream_t passed as
 *     void* (NULL = the default stream).  Every call only enqueues work on
 *     `stream`: the library never synchronises, allocates, frees or caches
 *     device memory, holds no mutable global state and is re-entrant.  The
 *     caller owns every buffer and keeps it alive until the work completes.
 *     The one exception is sage_quantize_qkv_noalloc, whose scratch is a device
 *     array of the library's own, shared by all its calls on a GPU.
 *   - bf16 inputs are [B, N, H, D] views with unit d-stride and element strides
 *     (stride_b, stride_n, stride_h).  Contiguous HND, contiguous NHD and the
 *     strided views of a packed [B, N, 3*H*D] projection buffer are all such views.
 *   - Only D == SAGE_HEAD_DIM is supported.
 *   - Code and scale buffers use Npad = sage_npad(N) = round_up(N, SAGE_N_ALIGN)
 *     tokens; entries for tokens N..Npad-1 are written as zero.
 *   - Errors: arguments are validated on the host before anything is enqueued
 *     and a non-zero sage_status is returned (nothing is launched).  A failed
 *     launch returns SAGE_ERR_HIP: the status is that of the call's own kernel
 *     launches (hipLaunchKernel's return values, the first failing one stops
 *     the call); the thread's last-error state left by the caller's earlier HIP
 *     calls is neither reported nor cleared.  There is no fallback path.  NaN
 *     or infinite inputs are outside the contract and are not checked.
 */
#ifndef SAGE_MI355X_H
#define SAGE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_HEAD_DIM 128 /* channels per head */
#define SAGE_Q_BLOCK 32   /* tokens per Q scale */
#define SAGE_K_BLOCK 64   /* tokens per K scale (= keys per softmax tile) */
#define SAGE_P_TILE 64    /* keys per online-softmax step; P is rounded per tile */
#define SAGE_N_ALIGN 256  /* code buffers hold round_up(N, 256) tokens */
#define SAGE_MX_E4M3 0    /* MXFP8: E4M3 elements, one byte each */
#define SAGE_MX_E2M1 1    /* MXFP4: E2M1 elements, two per byte */

typedef enum {
    SAGE_OK = 0,
    SAGE_ERR_NULL = 1,      /* a required pointer is NULL */
    SAGE_ERR_SHAPE = 2,     /* B, N, H < 1, D != 128, B or H > 65535, or
                               B * H * Npad > 2^29 - 1 (launch sizes) */
    SAGE_ERR_STRIDE = 3,    /* strides let tokens or heads overlap */
    SAGE_ERR_ALIGN = 4,     /* a pointer or stride breaks 16-byte alignment */
    SAGE_ERR_WORKSPACE = 5, /* workspace too small */
    SAGE_ERR_HIP = 6,       /* the HIP runtime reported an error */
    SAGE_ERR_VALUE = 7      /* sm_scale or eps not finite and positive, or an unknown format */
} sage_status;

/* A [B, N, H, D] bf16 view: element (b, n, h, d) is at
 * data + b*stride_b + n*stride_n + h*stride_h + d (strides in elements).
 * data must be 16-byte aligned and all strides multiples of 8 (so every
 * 128-channel head row is 16-byte aligned); strides may not be negative.
 * Input views are only read and may overlap (e.g. a broadcast head). */
typedef struct {
    const void *data;
    int64_t stride_b, stride_n, stride_h;
} sage_bf16_in;

typedef struct {
    void *data;
    int64_t stride_b, stride_n, stride_h;
} sage_bf16_out;

/* An output view: as above, 8-byte aligned, strides multiples of 4; the
 * (b, n, h) rows of D elements must be disjoint (else SAGE_ERR_STRIDE). */

/* round_up(N, SAGE_N_ALIGN); 0 for N < 1. */
int64_t sage_npad(int N);

/* Bytes of device workspace sage_quantize_qk needs: ceil(N/64)*B*H*D doubles
 * (per-64-token fp64 partial sums of K). */
size_t sage_qk_workspace_bytes(int B, int N, int H, int D);

/* Bytes of device workspace sage_quantize_v needs: ceil(N/256)*B*H*D floats
 * (per-256-token partial channel maxima of |V|) plus B*H*D floats. */
size_t sage_v_workspace_bytes(int B, int N, int H, int D);

/* qk_quantize with K smoothing (profile page, attention_internal_p50_milliseconds
 * .sage2: qk_quantize and framework_and_k_smoothing_estimate).
 *   k_mean [B, H, D] fp32: the token mean of K per (b, h, d), summed in fp64 over
 *     64-token chunks in ascending token order, the chunk sums in ascending
 *     order, divided by N in fp64, rounded once to fp32.
 *   q_codes [B, H, Npad, D] int8, q_scale [B, H, Npad/32] fp32: per (b, h, block
 *     of 32 tokens) scale = amax/127 (IEEE fp32 division) and code =
 *     clamp(rne(x / scale), -127, 127) with x / scale an IEEE fp32 division;
 *     a block whose amax is 0 has scale 0 and zero codes.
 *   k_codes [B, H, Npad, D] int8, k_scale [B, H, Npad/64] fp32: the same on
 *     x = fp32(k) - k_mean[b, h, d] (one fp32 subtraction) with 64-token blocks.
 *   workspace: >= sage_qk_workspace_bytes(B, N, H, D) bytes, 8-byte aligned;
 *     contents on entry are ignored.
 * Codes, scales and k_mean are bit-exactly defined by the above (no tolerance).
 * q_codes/k_codes 16-byte aligned; scales and k_mean 4-byte aligned. */
int sage_quantize_qk(const sage_bf16_in *q, const sage_bf16_in *k, int B, int N, int H, int D,
                     int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale,
                     float *k_mean, void *workspace, size_t workspace_bytes, void *stream);

/* v_quantize (profile page, attention_internal_p50_milliseconds.sage2.v_quantize).
 *   v_scale [B, H, D] fp32: sv = amax / 448 over all N tokens of the channel
 *     (IEEE fp32 division; 0 when amax is 0).
 *   v_codes: OCP E4M3FN codes of v / sv (IEEE fp32 division; round to nearest
 *     even, saturating at +-448, sign of zero kept; 0x00 where sv is 0), stored
 *     tile-major as the FP8 P.V operand: byte
 *         (((b*H + h)*(Npad/64) + t)*128 + d)*64 + p
 *     holds the code of token 64*t + kappa(p), channel d, where for p = 32*u + j
 *     (u in {0, 1}, j in 0..31)
 *         kappa(p) = 32*(j/16) + 8*((j%16)/4) + 4*u + (j%4).
 *     Tokens N..Npad-1 hold 0x00.  v_codes 16-byte aligned.
 *   workspace: >= sage_v_workspace_bytes(B, N, H, D) bytes, 4-byte aligned. */
int sage_quantize_v(const sage_bf16_in *v, int B, int N, int H, int D,
                    uint8_t *v_codes, float *v_scale, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Bytes of device workspace sage_quantize_qkv needs: ceil(N/64)*B*H*D doubles
 * (K-mean chunk partials) plus ceil(N/64)*B*H*D floats (per-64-token channel
 * maxima of |V|) plus B*H*D floats. */
size_t sage_qkv_workspace_bytes(int B, int N, int H, int D);

/* sage_quantize_qk and sage_quantize_v in one call: the same outputs, bit for
 * bit, from three passes over the inputs instead of six (one pass gathers the K
 * smoothing statistic, the V channel maxima and the Q codes; the last writes the
 * K and V codes).  This folds the profile page's
 * framework_and_k_smoothing_estimate into the quantisation passes.  Arguments,
 * layouts and alignment as the two calls; workspace >=
 * sage_qkv_workspace_bytes(B, N, H, D) bytes, 8-byte aligned. */
int sage_quantize_qkv(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N, int H,
                      int D, int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale,
                      float *k_mean, uint8_t *v_codes, float *v_scale, void *workspace,
                      size_t workspace_bytes, void *stream);

/* sage_quantize_qkv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same three kernels and the same outputs, bit for bit, with no workspace
 * argument.  Their scratch (sage_qkv_workspace_bytes(B, N, H, D) bytes) lives in
 * a device array owned by the library, of sage_qkv_noalloc_max_bytes() = 64 MiB:
 * each GPU it is called on holds its own copy from the first call until the
 * process ends.  The call allocates and frees nothing; the first call on a
 * device looks the array's address up (hipGetSymbolAddress) with that device
 * current.  Every call on one GPU shares its copy and leaves its own contents
 * there, so calls that overlap on one GPU (different streams, or host threads)
 * race: serialise them.  Each call writes every scratch entry it reads, so
 * nothing has to be cleared between calls.  Sizes whose scratch exceeds 64 MiB
 * (sage_qkv_workspace_bytes > sage_qkv_noalloc_max_bytes(), i.e. about
 * B * H * ceil(N/64) > 43690; one block-24 sequence, N = 37810, H = 56, needs
 * 50.9 MB, two do not fit) return SAGE_ERR_WORKSPACE before anything is
 * enqueued.  Other arguments and errors as sage_quantize_qkv. */
size_t sage_qkv_noalloc_max_bytes(void);
int sage_quantize_qkv_noalloc(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N,
                              int H, int D, int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale,
                              float *k_mean, uint8_t *v_codes, float *v_scale, void *stream);

/* The step before quantisation: RMSNorm and rotary position embedding of Q and K
 * in place on their strided views (strided page, dataflow.qk_transform; profile
 * page, representative_block_24_p50_milliseconds.sage2.rms_rope).  For every
 * (b, n, h) row x of D channels:
 *   r   = 1 / sqrt(ss / D + eps), ss = sum_d x_d^2
 *   y_d = (x_d * r) * gamma[d]                       (gamma_q for Q, gamma_k for K)
 *   (y_2i, y_2i+1) <- (y_2i c - y_2i+1 s,  y_2i s + y_2i+1 c),  (c, s) = rope[n][i]
 *   x <- bf16(y), round to nearest even.
 * ss is the exact sum of the squares of the bf16 inputs rounded once to fp32
 * (nearest even; +inf beyond the fp32 range), so no summation order enters; the
 * rest is fp32 arithmetic, every product and sum rounded (no fused multiply-add),
 * IEEE sqrt and division.  The result is bit-exactly defined by this.
 *   q, k: [B, N, H, D] views written in place: 16-byte aligned, strides
 *     multiples of 8, distinct (b, n, h) rows (else SAGE_ERR_STRIDE); Q and K
 *     must not share elements (not checked).
 *   gamma_q, gamma_k: [D] fp32; rope: [N, D/2, 2] fp32 (cos, sin) pairs, the
 *     same for every batch and head; all 16-byte aligned, device memory.
 *   eps: finite and > 0 (else SAGE_ERR_VALUE). */
int sage_qk_norm_rope(const sage_bf16_out *q, const sage_bf16_out *k, int B, int N, int H, int D,
                      const float *gamma_q, const float *gamma_k, const float *rope, float eps, void *stream);

/* Bytes of device workspace sage_quantize_qkv_rope needs:
 * sage_qkv_workspace_bytes(B, N, H, D) plus B*H*Npad floats (the norm factor r of
 * every K row, computed by the first pass and reused by the last). */
size_t sage_qkv_rope_workspace_bytes(int B, int N, int H, int D);

/* sage_qk_norm_rope fused into sage_quantize_qkv: the codes, scales and k_mean
 * that sage_qk_norm_rope followed by sage_quantize_qkv produce, bit for bit, with
 * Q and K read once less and not written (the transformed Q and K are not
 * materialised; q and k are only read).  Arguments as the two calls, except the
 * workspace: >= sage_qkv_rope_workspace_bytes(B, N, H, D) bytes, 8-byte aligned
 * (else SAGE_ERR_WORKSPACE / SAGE_ERR_ALIGN). */
int sage_quantize_qkv_rope(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N, int H,
                           int D, const float *gamma_q, const float *gamma_k, const float *rope, float eps,
                           int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale, float *k_mean,
                           uint8_t *v_codes, float *v_scale, void *workspace, size_t workspace_bytes,
                           void *stream);

/* attention_forward (profile page, attention_internal_p50_milliseconds.sage2
 * .attention_forward; latency page, the whole artefact): from the buffers the two
 * calls above wrote, for every query i < N of every (b, h):
 *   a_ij = sum_d qc_id * kc_jd (exact int32)
 *   s_ij = a_ij * q_scale[i/32] * k_scale[j/64] * sm_scale (fp32)
 *   for 64-key tiles in ascending order (the last one partial, keys >= N absent):
 *     m  <- max(m, max_j s_ij);  rescale l and acc by exp(m_old - m)
 *     p_ij = exp(s_ij - m);  l += p_ij (fp32, before rounding)
 *     acc_d += E4M3(448 * p_ij) * E4M3^-1(vc_jd)   (FP8 MFMA, fp32 accumulate)
 *   out[b, i, h, d] = bf16_rne(acc_d * v_scale[d] / (448 * l)).
 * Results match that definition within floating-point tolerance (fp32 exp and
 * accumulation order).  Rows >= N are not written.  out must be 8-byte aligned
 * with stride_n, stride_h multiples of 4 (token-major [B, N, H*D] is the
 * intended layout: stride_b = N*H*D, stride_n = H*D, stride_h = D).
 * sm_scale must be finite and > 0 (1/sqrt(128) for the softmax). */
int sage_attn_fwd(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes,
                  const float *k_scale, const uint8_t *v_codes, const float *v_scale,
                  int B, int N, int H, int D, float sm_scale, const sage_bf16_out *out,
                  void *stream);

/* The unquantised comparison path: the same softmax(Q K^T * sm_scale) V straight
 * from the strided bf16 views, BF16 MFMA for Q K^T and P.V (P rounded to bf16),
 * fp32 online softmax over 64-key tiles.  Output as sage_attn_fwd.  K and V
 * token rows must not overlap: 128 <= stride_n <= 2^23 (else SAGE_ERR_STRIDE). */
int sage_attn_fwd_bf16(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v,
                       int B, int N, int H, int D, float sm_scale, const sage_bf16_out *out,
                       void *stream);

/* INT8 Q K^T with an unquantised P.V: the precision split the profile page runs
 * as "sol_int8_qk" (sampling_stage_step_2_seconds.sol_int8_qk_tau_1_3_exact_
 * conditioning_kv: Q and K quantised, V not), here dense and non-causal.  Scores
 * come from the codes and scales sage_quantize_qk wrote, exactly as in
 * sage_attn_fwd; then for every query i < N of every (b, h):
 *   for 64-key tiles in ascending order (the last one partial, keys >= N absent):
 *     m  <- max(m, max_j s_ij);  rescale l and acc by exp(m_old - m)
 *     p_ij = exp(s_ij - m);  l += p_ij (fp32)
 *     acc_d += bf16_rne(p_ij) * v[b, j, h, d]   (BF16 MFMA, fp32 accumulate)
 *   out[b, i, h, d] = bf16_rne(acc_d / l).
 * v is the bf16 [B, N, H, D] view (as for sage_attn_fwd_bf16: 16-byte aligned,
 * strides multiples of 8, 128 <= stride_n <= 2^23 so token rows do not overlap).
 * No V quantisation pass is needed.  Output and errors as sage_attn_fwd. */
int sage_attn_fwd_int8qk(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes,
                         const float *k_scale, const sage_bf16_in *v, int B, int N, int H, int D,
                         float sm_scale, const sage_bf16_out *out, void *stream);

/* OCP microscaling (MX) output for the projection after attention: the profile
 * page's next_targets lists a fused low-precision projection epilogue (the
 * pages' projections run in NVFP4, sage2_block_share_estimates.nvfp4_projections);
 * MI355X's native block-scaled formats are OCP MX, which its MFMAs consume
 * directly.  Blocks are 32 consecutive channels of the token-major [B, N, H*D]
 * row (32 | D, so a block lies in one head).  Per block (OCP Microscaling
 * Formats v1.0): amax = max |x_i|; X = floor(log2 amax) - emax (8 for E4M3, 2 for
 * E2M1), clamped to [-127, 127], and -127 when amax is 0; scale byte = X + 127
 * (E8M0); element i = the round-to-nearest-even, saturating E4M3 (max 448) or
 * E2M1 (max 6) encoding of x_i / 2^X, sign of zero kept.
 *   codes: [B, N, H*D] bytes (SAGE_MX_E4M3) or [B, N, H*D/2] (SAGE_MX_E2M1,
 *     element 2i in the low nibble of byte i), token-major, contiguous;
 *   scales: [B, N, H*D/32] E8M0 bytes.
 * Codes and scales are bit-exactly defined by the input values.
 *
 * sage_mx_quantize: the MX blocks of a bf16 [B, N, H, D] view (16-byte aligned,
 * strides multiples of 8).  codes 16-byte aligned (whole blocks are stored with
 * 16-byte stores), scales any alignment.  fmt not one of the two formats gives
 * SAGE_ERR_VALUE. */
int sage_mx_quantize(const sage_bf16_in *x, int B, int N, int H, int D, int fmt, uint8_t *codes,
                     uint8_t *scales, void *stream);

/* sage_attn_fwd with the output written as MX blocks instead of bf16: the
 * blocks of exactly the bf16 values sage_attn_fwd would write (so the result
 * equals sage_mx_quantize of that output, byte for byte).  Arguments as
 * sage_attn_fwd; codes and scales laid out as for sage_mx_quantize, codes 4-byte
 * aligned; rows >= N are not written. */
int sage_attn_fwd_mx(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes,
                     const float *k_scale, const uint8_t *v_codes, const float *v_scale,
                     int B, int N, int H, int D, float sm_scale, int fmt, uint8_t *codes,
                     uint8_t *scales, void *stream);

/* A static, human-readable name for a sage_status value. */
const char *sage_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_MI355X_H */
