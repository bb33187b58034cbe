/*
 * saq.h - C ABI of the joint-sequence QKNorm + 3D RoPE -> block selection ->
 * block-sparse attention layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the per-layer self-attention of a video+audio diffusion
 * transformer over one joint token sequence (Sol Engine "H3 on device" page:
 * intro, which says this attention dominates the profile; lossless-kernels
 * fusion table, row "fused QKNorm + RoPE"; Sol-Attn paragraph, which computes
 * only the attention blocks a per-step selection keeps).
 *
 * Conventions shared by every call:
 *  - Tensors q, k, v, o are bf16, shape [B, S, H, D], contiguous (D fastest),
 *    in device memory owned by the caller, 16-byte aligned.
 *  - Block masks are uint8 [B, H, nB, nB] with nB = ceil(S / block); block i
 *    holds tokens [i*block, min((i+1)*block, S)), so the last block may be
 *    partial.
 *  - Supported: D in {64, 128}; block in {64, 128}; 1 <= S; nB <= 4096;
 *    1 <= B, H; B*S*H*D < 2^31.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous on that stream; the library allocates nothing,
 *    keeps no state between calls and is safe to call from several threads.
 *  - Every argument is validated on the host before any launch; a call that
 *    returns non-zero has launched nothing. Validation covers sizes, ranges,
 *    alignment and overlap, not where a pointer lives: every buffer must be
 *    device memory of the current device (hipMalloc or torch's allocator), and
 *    a host pointer is undefined behaviour that typically faults the kernel.
 *    Device-side faults surface at the caller's next synchronisation, as for
 *    any HIP launch.
 *  - Return value: SAQ_OK (0) or a negative SAQ_ERR_* code; nothing crosses
 *    the ABI as an exception. saq_status_string() names the code and
 *    saq_last_hip_error() returns the HIP error of the calling thread's last
 *    SAQ_ERR_HIP.
 */
#ifndef SAQ_H
#define SAQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum saq_status {
    SAQ_OK = 0,
    SAQ_ERR_NULL = -1,         /* a required pointer is NULL */
    SAQ_ERR_SHAPE = -2,        /* a size is <= 0, inconsistent, or too large */
    SAQ_ERR_UNSUPPORTED = -3,  /* D or block outside the supported set */
    SAQ_ERR_ALIGN = -4,        /* a tensor pointer is not 16-byte aligned */
    SAQ_ERR_RANGE = -5,        /* keep_ratio, eps, base or scale out of range */
    SAQ_ERR_WORKSPACE = -6,    /* workspace too small or NULL */
    SAQ_ERR_HIP = -7,          /* a HIP call failed; see saq_last_hip_error() */
    SAQ_ERR_NO_DEVICE = -8,    /* no HIP device is visible */
    SAQ_ERR_ALIAS = -9         /* an output overlaps an input it must not */
};

/*
 * Fused QKNorm + 3D multimodal RoPE, in place on q and k.
 * (Sol Engine "H3 on device" page, fusion table, row "fused QKNorm + RoPE":
 * the fused kernel replaces two read/write passes over Q and K.)
 *
 * For every (b, s, h) row x of q (weight w_q) and of k (weight w_k):
 *   x_hat[d] = x[d] / sqrt(mean_d(x^2) + eps) * w[d]
 * then head_dim is split into contiguous sections of widths (dt, dh, dw) for
 * the axes (t, h, w); in the section of axis a, each adjacent pair
 * (2i, 2i+1) is rotated by theta = pos_thw[s][a] * rope_base^(-2i/d_a):
 *   (x0, x1) <- (x0 cos theta - x1 sin theta, x0 sin theta + x1 cos theta).
 * The norm and rotation run in fp32 (angles in fp64), the result is rounded
 * to bf16 (nearest-even) and written back in place.
 *
 *   q, k     bf16 [B,S,H,D], read and overwritten. Any finite values: a row
 *            whose fp32 sum of squares would overflow (entries beyond about
 *            2^60) is normalised through a pass scaled by 2^-68.
 *   pos_thw  int32 [S,3] device array of (t, h, w) positions, shared by all
 *            batch entries; any values are allowed.
 *   w_q, w_k fp32 [D] device arrays.
 *   dt+dh+dw must equal D, each even and >= 0 (multiples of 8 for speed are
 *   not required). rope_base > 1, eps > 0, both finite.
 * q and k must not overlap.
 */
int saq_qknorm_rope(void* q, void* k, const int32_t* pos_thw, const float* w_q, const float* w_k,
                    int32_t B, int32_t S, int32_t H, int32_t D, int32_t dt, int32_t dh, int32_t dw,
                    double rope_base, double eps, void* stream);

/*
 * Out-of-place form of saq_qknorm_rope: reads q_in, k_in and writes q_out,
 * k_out (same shapes). Each output may equal its own input (then it is the
 * in-place call) but must not partially overlap any other tensor.
 */
int saq_qknorm_rope_out(const void* q_in, const void* k_in, void* q_out, void* k_out,
                        const int32_t* pos_thw, const float* w_q, const float* w_k,
                        int32_t B, int32_t S, int32_t H, int32_t D, int32_t dt, int32_t dh, int32_t dw,
                        double rope_base, double eps, void* stream);

/*
 * Number of key blocks kept per query block:
 *   k = clamp(ceil(keep_ratio * nB - 1e-6), 1, nB),
 * evaluated in fp64 (the 1e-6 guard keeps rounding error from raising k).
 * Returns SAQ_ERR_RANGE for keep_ratio outside (0, 1] or NaN, SAQ_ERR_SHAPE
 * for nB < 1. Pure host function.
 */
int32_t saq_kept_blocks(double keep_ratio, int32_t nB);

/* Bytes of device workspace saq_select_blocks needs for these sizes, or 0 if
 * the sizes are invalid. Pure host function. */
size_t saq_select_blocks_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block);

/*
 * Training-free dynamic block selection (Sol-Attn paragraph of the Sol Engine
 * "H3 on device" page: only the (query block, key block) tiles the selection
 * keeps are computed; KOCPC article on Sol-H3, "Specific outcomes": the
 * selection is made dynamically at inference time). The pages do not give the
 * rule; this call implements the following one, per (b, h):
 *   1. p_i = mean of the rows of block i (fp64; exact sums of bf16 values),
 *      for q and k separately;
 *   2. s_ij = sum_d pq_i[d] * pk_j[d] in fp64, d ascending, each product and
 *      each sum rounded separately (no fused multiply-add);
 *   3. row i keeps block i plus the k-1 largest s_ij over j != i, with
 *      k = saq_kept_blocks(keep_ratio, nB); ties go to the lower j and -0.0
 *      equals +0.0.
 * Output: block_mask [B,H,nB,nB] uint8 with exactly k ones per row and a one
 * on the diagonal. Bit-for-bit deterministic. Inputs must be finite.
 * The block sums of step 1 are exact, hence independent of summation order
 * (and equal between this call and saq_qknorm_rope_pool), when every value
 * satisfies |x| < 16 and is 0 or >= 2^-35 in magnitude. QKNorm output with
 * weights of magnitude < 1.4 meets the upper bound for D <= 128 (|x_hat| <=
 * sqrt(D) * max|w|); the lower one fails only for values that tiny. Outside
 * that range the result is still deterministic, but the two selection paths
 * may round the means differently.
 *
 *   q, k       bf16 [B,S,H,D]: the post-prologue tensors attention consumes.
 *   workspace  device buffer of at least
 *              saq_select_blocks_workspace_bytes(B,S,H,D,block) bytes,
 *              256-byte aligned; its contents are scratch.
 */
int saq_select_blocks(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D,
                      int32_t block, double keep_ratio, uint8_t* block_mask, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * saq_select_blocks for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same selection, the same mask bit for bit, with the workspace taken from
 * a scratch array the library holds in device memory, one copy per GPU, from
 * the library's load until the process ends. Sizes whose workspace
 * (saq_select_blocks_workspace_bytes) exceeds SAQ_NOALLOC_SCRATCH_BYTES are
 * rejected with SAQ_ERR_WORKSPACE before any HIP call; the full 127,040-token,
 * 40-head layer at block 128 needs 123 MB and fits. The call allocates
 * nothing. Every call on one GPU uses that GPU's one array, so calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller; successive calls on one stream are safe. Arguments
 * and other errors as saq_select_blocks; the first call on a device may also
 * return SAQ_ERR_HIP if the array's address cannot be obtained.
 */
#define SAQ_NOALLOC_SCRATCH_BYTES (128u << 20)
int saq_select_blocks_noalloc(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D,
                              int32_t block, double keep_ratio, uint8_t* block_mask, void* stream);

/*
 * Block-sparse flash attention (Sol-Attn paragraph of the Sol Engine "H3 on
 * device" page: attention computed only on the kept blocks, with an online
 * softmax). For each (b, h, query block i), over the kept key blocks j in
 * ascending order:
 *   o_t = sum_{u in kept tokens} softmax_u(q_t . k_u * scale) v_u,
 * non-causal, every valid token of a kept block taking part. QK^T and PV run
 * on bf16 MFMA with fp32 accumulation; softmax statistics are fp32; the
 * result is rounded to bf16. A query block with no kept key block gets
 * o = 0. Any 0/1 mask is accepted (a non-zero byte counts as 1).
 *
 *   softmax_scale  > 0, or <= 0 to mean 1/sqrt(D); must be finite.
 *   o              bf16 [B,S,H,D]; must not overlap q, k, v or block_mask.
 *   q, k, v        finite, and small enough that the fp32 accumulations stay
 *                  finite: the scores q.k * scale, and sums of up to S products
 *                  of v with weights <= 2^8. |q|, |k| <= 2^55 and |v| <= 2^90
 *                  suffice (D <= 128, S <= 2^20); beyond that o is undefined.
 *                  Outputs of saq_qknorm_rope with weights |w| <= 2^40 are.
 */
int saq_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                          int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                          float softmax_scale, void* o, void* stream);

/*
 * Fused QKNorm + 3D RoPE + block pooling (the first step of selection folded
 * into the prologue's single pass over Q and K; Sol Engine "H3 on device" page,
 * fusion table "fused QKNorm + RoPE", and its Sol-Attn paragraph on avoiding a
 * separate routing stage). Computes exactly what saq_qknorm_rope_out computes
 * into q_out/k_out (same bits), and also writes the per-block fp64 means of the
 * bf16 q_out and k_out into the head of `workspace`, as saq_select_blocks would
 * compute them (bit-identical: the sums of bf16 values are exact in fp64).
 * Follow with saq_select_blocks_pooled on the same workspace.
 *
 *   block      64 or 128; workspace >= saq_select_blocks_workspace_bytes(...),
 *              256-byte aligned.
 *   Extra limit: H*D <= 8192 (SAQ_ERR_UNSUPPORTED otherwise).
 * Aliasing rules as saq_qknorm_rope_out; the workspace must not overlap any
 * tensor.
 */
int saq_qknorm_rope_pool(const void* q_in, const void* k_in, void* q_out, void* k_out, const int32_t* pos_thw,
                         const float* w_q, const float* w_k, int32_t B, int32_t S, int32_t H, int32_t D,
                         int32_t dt, int32_t dh, int32_t dw, double rope_base, double eps, int32_t block,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block selection from the pooled vectors saq_qknorm_rope_pool left in
 * `workspace` (scores + top-k + diagonal, the same rule and bit-identical result
 * as saq_select_blocks on the tensors that call wrote).
 */
int saq_select_blocks_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, double keep_ratio,
                             uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cross-step mask reuse, measured (Sol Engine "H3 on device" page, cross-step
 * cache paragraph: consecutive denoising steps are nearly identical through the
 * middle of the schedule, and a cheap change detector decides what to recompute).
 *
 * saq_mask_overlap: for two masks [B,H,nB,nB] (non-zero byte = kept), writes
 * counts[2*(b*H+h)] = #(kept in both), counts[2*(b*H+h)+1] = #(kept in a).
 * counts: device int64 [2*B*H], 8-byte aligned; masks 16-byte aligned;
 * B*H <= 65535. Exact integers.
 *
 * saq_pooled_change: the change detector on the pooled block means that
 * saq_qknorm_rope_pool leaves in a selection workspace. With P = all 2*B*H*nB*D
 * pooled values, writes out[0] = sum (P_cur - P_prev)^2 and
 * out[1] = sum P_prev^2 in fp64 (fixed reduction order: identical bits on every
 * run); the relative change is sqrt(out[0] / out[1]). out: device double array
 * of at least saq_pooled_change_out_len() entries (the rest is scratch).
 */
int saq_mask_overlap(const uint8_t* mask_a, const uint8_t* mask_b, int32_t B, int32_t H, int32_t nB,
                     int64_t* counts, void* stream);
size_t saq_pooled_change_out_len(void);
int saq_pooled_change(const void* workspace_prev, const void* workspace_cur, int32_t B, int32_t S, int32_t H,
                      int32_t D, int32_t block, double* out, size_t out_len, void* stream);

/*
 * Gated block selection for a step loop: the mask of an earlier step is kept
 * while the pooled block means it was selected from have barely moved, in the
 * manner of the cross-step cache on the same page (one threshold on a cheap
 * relative-change signal). The decision is taken on the device, so the call
 * needs no host round trip and the stream stays asynchronous.
 *
 * Inputs: `workspace` as left by saq_qknorm_rope_pool for the current step
 * (the current pooled means P_cur); `pooled_ref`, a caller-owned device buffer
 * of saq_pooled_bytes(...) bytes (16-byte aligned) holding the pooled means P_ref
 * the mask in `block_mask` was selected from; `state`, a device double array of
 * saq_reuse_state_len() entries (8-byte aligned).
 *
 * Steps, in stream order:
 *   1. state[0] = sum (P_cur - P_ref)^2, state[1] = sum P_ref^2 (fp64, fixed
 *      reduction order, as saq_pooled_change);
 *   2. the mask is kept iff force == 0 and state[0] <= (threshold*threshold) *
 *      state[1] (fp64, evaluated in that order); state[2] = 0.0 if kept,
 *      1.0 if recomputed;
 *   3. if recomputed: block_mask = saq_select_blocks_pooled(...) on `workspace`
 *      (bit-identical), then pooled_ref = P_cur; if kept, block_mask and
 *      pooled_ref are left untouched.
 * The rest of `state` is scratch. On the first step of a loop pass force = 1
 * (pooled_ref may then hold anything finite, or anything at all: it only feeds
 * state[0..1]). threshold: finite and >= 0 (SAQ_ERR_RANGE otherwise); 0 keeps
 * the mask only when the pooled means are unchanged. No buffer may overlap
 * another (SAQ_ERR_ALIAS).
 */
size_t saq_pooled_bytes(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block);
size_t saq_reuse_state_len(void);
int saq_select_blocks_reuse(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, double keep_ratio,
                            double threshold, int32_t force, uint8_t* block_mask, void* workspace,
                            size_t workspace_bytes, void* pooled_ref, size_t pooled_ref_bytes, double* state,
                            size_t state_len, void* stream);

/*
 * INT8 / FP8 block codecs: the two ends of the multi-GPU attention exchange,
 * whose inputs travel as INT8 and outputs as FP8 (KOCPC article on Sol-H3,
 * "Technical Composition"). Encode a bf16 tensor [B,S,H,D] into one byte per
 * element (same layout) plus one fp32 scale per (batch, token block, head)
 * tile, scales laid out [B,H,nB]; decode back to bf16.
 *
 * A tile is tokens [i*block, min((i+1)*block, S)) of one head over all D
 * channels. With amax = max |x| over the tile and Q = 127 (INT8) or 448 (FP8):
 * inv = Q / amax and s = amax / Q (correctly rounded fp32 divisions); each x
 * becomes round-to-nearest-even of the fp32 product x * inv, as an integer
 * clamped to [-127, 127] (INT8) or as the nearest OCP E4M3 value (FP8: bias 7,
 * no infinities, largest finite 448; the tile's amax maps to +-Q, so nothing
 * overflows). A tile with amax < 2^-100 stores s = 0 and zero codes. Decoding:
 * bf16 round-to-nearest-even of the fp32 product value(code) * s.
 *
 *   x, y      bf16 [B,S,H,D], 16-byte aligned; finite values (others undefined)
 *   codes     1 byte per element, [B,S,H,D], 8-byte aligned
 *   scales    fp32 [B,H,nB], 4-byte aligned (written by quantize, read by dequantize)
 *   D and block in {64, 128}. No buffer may overlap another (SAQ_ERR_ALIAS).
 */
int saq_quantize_int8(const void* x, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int8_t* codes,
                      float* scales, void* stream);
int saq_dequantize_int8(const int8_t* codes, const float* scales, int32_t B, int32_t S, int32_t H, int32_t D,
                        int32_t block, void* y, void* stream);
int saq_quantize_fp8(const void* x, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, uint8_t* codes,
                     float* scales, void* stream);
int saq_dequantize_fp8(const uint8_t* codes, const float* scales, int32_t B, int32_t S, int32_t H, int32_t D,
                       int32_t block, void* y, void* stream);

/*
 * Block-sparse attention with the block selection folded into the attention
 * pass: no separate routing stage and no mask in memory (the Sol-Attn
 * paragraph of the "H3 on device" page describes the selection as part of the
 * online-softmax pass; its rule is not given, so the rule is the one of
 * saq_select_blocks). Each workgroup scores its query block against every key
 * block from the pooled means that saq_qknorm_rope_pool left in `workspace`,
 * keeps the diagonal and the k-1 best (k = saq_kept_blocks(keep_ratio, nB)),
 * and attends over them. The mask and the output are bit-identical to
 * saq_select_blocks_pooled followed by saq_block_sparse_attn.
 *
 *   workspace       as written by saq_qknorm_rope_pool for these q, k (only its
 *                   pooled part, 2*B*H*nB*D doubles, is read); 256-byte aligned
 *   block_mask_out  optional uint8 [B,H,nB,nB]: the rows chosen (null: not written)
 *   D = block = 128 only (SAQ_ERR_UNSUPPORTED otherwise); other arguments,
 *   layouts and aliasing rules as saq_block_sparse_attn.
 */
int saq_block_sparse_attn_select(const void* q, const void* k, const void* v, const void* workspace,
                                 size_t workspace_bytes, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                                 double keep_ratio, float softmax_scale, void* o, uint8_t* block_mask_out,
                                 void* stream);

/* Static, NUL-terminated name of a status code. */
const char* saq_status_string(int status);

/* The hipError_t of the calling thread's most recent SAQ_ERR_HIP (0 if none). */
int saq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SAQ_H */
