// C ABI of the layer (declared in include/saq.h): host-side validation, then
// launches on the caller's stream. Validation never calls HIP, so an invalid
// call returns its status before anything touches the device.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/saq.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

int check_dims(int32_t B, int32_t S, int32_t H, int32_t D) {
    if (B < 1 || S < 1 || H < 1 || D < 1) return SAQ_ERR_SHAPE;
    if (D != 64 && D != 128) return SAQ_ERR_UNSUPPORTED;
    // B*S*H*D < 2^31, checked factor by factor so that no product can overflow
    const int64_t lim = (int64_t)1 << 31;
    int64_t n = (int64_t)B * S;
    if (n >= lim) return SAQ_ERR_SHAPE;
    n *= H;
    if (n >= lim) return SAQ_ERR_SHAPE;
    n *= D;
    if (n >= lim) return SAQ_ERR_SHAPE;
    return SAQ_OK;
}

int check_block(int32_t S, int32_t block) {
    if (block != 64 && block != 128) return SAQ_ERR_UNSUPPORTED;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    if (nB > saq::kMaxBlocks) return SAQ_ERR_SHAPE;
    return SAQ_OK;
}

int device_ready() {
    int count = 0;
    const hipError_t err = hipGetDeviceCount(&count);
    if (err != hipSuccess || count < 1) {
        g_last_hip_error = (int)err;
        return SAQ_ERR_NO_DEVICE;
    }
    return SAQ_OK;
}

int finish(hipError_t err) {
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return SAQ_ERR_HIP;
    }
    return SAQ_OK;
}

int validate_prologue(const void* q_in, const void* k_in, const void* q_out, const void* k_out,
                      const int32_t* pos_thw, const float* w_q, const float* w_k, int32_t B, int32_t S,
                      int32_t H, int32_t D, int32_t dt, int32_t dh, int32_t dw, double base, double eps) {
    if (!q_in || !k_in || !q_out || !k_out || !pos_thw || !w_q || !w_k) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    if (dt < 0 || dh < 0 || dw < 0 || (int64_t)dt + dh + dw != D || (dt | dh | dw) & 1) return SAQ_ERR_SHAPE;
    if (!(base > 1.0) || !isfinite(base) || !(eps > 0.0) || !isfinite(eps)) return SAQ_ERR_RANGE;
    if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out)) return SAQ_ERR_ALIGN;
    const size_t bytes = (size_t)B * S * H * D * 2;
    // each output may be its own input (in place) but no other overlap is allowed
    if (overlaps(q_in, bytes, k_in, bytes) || overlaps(q_out, bytes, k_out, bytes) ||
        overlaps(q_out, bytes, k_in, bytes) || overlaps(k_out, bytes, q_in, bytes))
        return SAQ_ERR_ALIAS;
    if ((q_out != q_in && overlaps(q_out, bytes, q_in, bytes)) ||
        (k_out != k_in && overlaps(k_out, bytes, k_in, bytes)))
        return SAQ_ERR_ALIAS;
    return SAQ_OK;
}

saq::RopeTable make_rope_table(int32_t dt, int32_t dh, int32_t dw, double base) {
    saq::RopeTable t;
    memset(&t, 0, sizeof(t));
    const int32_t widths[3] = {dt, dh, dw};
    int p = 0;
    for (int a = 0; a < 3; ++a)
        for (int i = 0; i < widths[a] / 2; ++i) t.inv_freq[p++] = pow(base, -2.0 * i / widths[a]);
    t.pair_end_t = dt / 2;
    t.pair_end_h = (dt + dh) / 2;
    return t;
}

}  // namespace

extern "C" {

int saq_qknorm_rope_out(const void* q_in, const void* k_in, void* q_out, void* k_out, const int32_t* pos_thw,
                        const float* w_q, const float* w_k, int32_t B, int32_t S, int32_t H, int32_t D,
                        int32_t dt, int32_t dh, int32_t dw, double rope_base, double eps, void* stream) {
    int st = validate_prologue(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, D, dt, dh, dw, rope_base, eps);
    if (st) return st;
    if ((int64_t)B * S >= ((int64_t)1 << 31)) return SAQ_ERR_SHAPE;
    st = device_ready();
    if (st) return st;
    const saq::RopeTable table = make_rope_table(dt, dh, dw, rope_base);
    return finish(saq::launch_qknorm_rope(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, D, table,
                                          (float)eps, (hipStream_t)stream));
}

int saq_qknorm_rope(void* q, void* k, const int32_t* pos_thw, const float* w_q, const float* w_k, int32_t B,
                    int32_t S, int32_t H, int32_t D, int32_t dt, int32_t dh, int32_t dw, double rope_base,
                    double eps, void* stream) {
    return saq_qknorm_rope_out(q, k, q, k, pos_thw, w_q, w_k, B, S, H, D, dt, dh, dw, rope_base, eps, stream);
}

int saq_qknorm_rope_pool(const void* q_in, const void* k_in, void* q_out, void* k_out, const int32_t* pos_thw,
                         const float* w_q, const float* w_k, int32_t B, int32_t S, int32_t H, int32_t D,
                         int32_t dt, int32_t dh, int32_t dw, double rope_base, double eps, int32_t block,
                         void* workspace, size_t workspace_bytes, void* stream) {
    int st = validate_prologue(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, D, dt, dh, dw, rope_base, eps);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    if ((int64_t)H * D > saq::kMaxRowElems) return SAQ_ERR_UNSUPPORTED;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    if ((int64_t)B * nB >= ((int64_t)1 << 31)) return SAQ_ERR_SHAPE;
    const size_t need = saq::select_workspace_bytes(B, H, nB, D);
    if (!workspace || workspace_bytes < need) return SAQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return SAQ_ERR_ALIGN;
    const size_t bytes = (size_t)B * S * H * D * 2;
    if (overlaps(workspace, need, q_in, bytes) || overlaps(workspace, need, k_in, bytes) ||
        overlaps(workspace, need, q_out, bytes) || overlaps(workspace, need, k_out, bytes))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    const saq::RopeTable table = make_rope_table(dt, dh, dw, rope_base);
    return finish(saq::launch_qknorm_rope_pool(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, D, table,
                                               (float)eps, block, (double*)workspace, (hipStream_t)stream));
}

int saq_select_blocks_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, double keep_ratio,
                             uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_mask) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    const int32_t nB = (S + block - 1) / block;
    const int32_t kept = saq_kept_blocks(keep_ratio, nB);
    if (kept < 0) return kept;
    const size_t need = saq::select_workspace_bytes(B, H, nB, D);
    if (!workspace || workspace_bytes < need) return SAQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return SAQ_ERR_ALIGN;
    if (overlaps(workspace, need, block_mask, (size_t)B * H * nB * nB)) return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    return finish(saq::launch_select_from_pooled(B, S, H, D, block, kept, block_mask, workspace,
                                                 (hipStream_t)stream));
}

int saq_mask_overlap(const uint8_t* mask_a, const uint8_t* mask_b, int32_t B, int32_t H, int32_t nB,
                     int64_t* counts, void* stream) {
    if (!mask_a || !mask_b || !counts) return SAQ_ERR_NULL;
    if (B < 1 || H < 1 || nB < 1 || nB > saq::kMaxBlocks || (int64_t)B * H > 65535) return SAQ_ERR_SHAPE;
    if (((uintptr_t)counts & 7u) != 0 || !aligned16(mask_a) || !aligned16(mask_b)) return SAQ_ERR_ALIGN;
    const size_t mbytes = (size_t)B * H * nB * nB;
    if (overlaps(counts, (size_t)B * H * 16, mask_a, mbytes) || overlaps(counts, (size_t)B * H * 16, mask_b, mbytes))
        return SAQ_ERR_ALIAS;
    const int st = device_ready();
    if (st) return st;
    return finish(saq::launch_mask_overlap(mask_a, mask_b, B, H, nB, counts, (hipStream_t)stream));
}

size_t saq_pooled_change_out_len(void) { return 2 + 2 * (size_t)saq::kChangeGroups; }

int saq_pooled_change(const void* workspace_prev, const void* workspace_cur, int32_t B, int32_t S, int32_t H,
                      int32_t D, int32_t block, double* out, size_t out_len, void* stream) {
    if (!workspace_prev || !workspace_cur || !out) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    if (out_len < saq_pooled_change_out_len()) return SAQ_ERR_WORKSPACE;
    if (((uintptr_t)out & 7u) != 0 || ((uintptr_t)workspace_prev & 255u) != 0 || ((uintptr_t)workspace_cur & 255u) != 0)
        return SAQ_ERR_ALIGN;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    const int64_t n = 2 * (int64_t)B * H * nB * D;
    if (overlaps(out, out_len * 8, workspace_prev, (size_t)n * 8) || overlaps(out, out_len * 8, workspace_cur, (size_t)n * 8))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    return finish(saq::launch_pooled_change((const double*)workspace_prev, (const double*)workspace_cur, n, out,
                                            (hipStream_t)stream));
}

size_t saq_pooled_bytes(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block) {
    if (check_dims(B, S, H, D) || check_block(S, block)) return 0;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    return (size_t)2 * B * H * nB * D * sizeof(double);
}

size_t saq_reuse_state_len(void) { return (size_t)saq::kReuseStateLen; }

int saq_select_blocks_reuse(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, double keep_ratio,
                            double threshold, int32_t force, uint8_t* block_mask, void* workspace,
                            size_t workspace_bytes, void* pooled_ref, size_t pooled_ref_bytes, double* state,
                            size_t state_len, void* stream) {
    if (!block_mask || !workspace || !pooled_ref || !state) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    const int32_t nB = (S + block - 1) / block;
    const int32_t kept = saq_kept_blocks(keep_ratio, nB);
    if (kept < 0) return kept;
    if (!(threshold >= 0.0) || !isfinite(threshold)) return SAQ_ERR_RANGE;
    const size_t need = saq::select_workspace_bytes(B, H, nB, D);
    const size_t pooled = saq_pooled_bytes(B, S, H, D, block);
    if (workspace_bytes < need || pooled_ref_bytes < pooled || state_len < saq_reuse_state_len())
        return SAQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0 || ((uintptr_t)pooled_ref & 15u) != 0 || ((uintptr_t)state & 7u) != 0)
        return SAQ_ERR_ALIGN;
    const size_t mbytes = (size_t)B * H * nB * nB;
    const size_t sbytes = state_len * sizeof(double);
    if (overlaps(workspace, need, block_mask, mbytes) || overlaps(pooled_ref, pooled, workspace, need) ||
        overlaps(pooled_ref, pooled, block_mask, mbytes) || overlaps(state, sbytes, workspace, need) ||
        overlaps(state, sbytes, pooled_ref, pooled) || overlaps(state, sbytes, block_mask, mbytes))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    return finish(saq::launch_select_reuse(B, S, H, D, block, kept, workspace, (double*)pooled_ref, threshold,
                                           force != 0 ? 1 : 0, block_mask, state, (hipStream_t)stream));
}

static int validate_codec(const void* bf, const void* codes, const float* scales, int32_t B, int32_t S, int32_t H,
                          int32_t D, int32_t block) {
    if (!bf || !codes || !scales) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    if ((int64_t)B * nB * H >= ((int64_t)1 << 31)) return SAQ_ERR_SHAPE;
    if (!aligned16(bf) || ((uintptr_t)codes & 7u) != 0 || ((uintptr_t)scales & 3u) != 0) return SAQ_ERR_ALIGN;
    const size_t n = (size_t)B * S * H * D;
    const size_t sbytes = (size_t)B * H * nB * sizeof(float);
    if (overlaps(bf, n * 2, codes, n) || overlaps(bf, n * 2, scales, sbytes) || overlaps(codes, n, scales, sbytes))
        return SAQ_ERR_ALIAS;
    return device_ready();
}

static int quantize_entry(bool fp8, const void* x, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                          void* codes, float* scales, void* stream) {
    const int st = validate_codec(x, codes, scales, B, S, H, D, block);
    if (st) return st;
    return finish(saq::launch_quantize(fp8, x, codes, scales, B, S, H, D, block, (hipStream_t)stream));
}

static int dequantize_entry(bool fp8, const void* codes, const float* scales, int32_t B, int32_t S, int32_t H,
                            int32_t D, int32_t block, void* y, void* stream) {
    const int st = validate_codec(y, codes, scales, B, S, H, D, block);
    if (st) return st;
    return finish(saq::launch_dequantize(fp8, codes, scales, y, B, S, H, D, block, (hipStream_t)stream));
}

int saq_quantize_int8(const void* x, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int8_t* codes,
                      float* scales, void* stream) {
    return quantize_entry(false, x, B, S, H, D, block, codes, scales, stream);
}

int saq_dequantize_int8(const int8_t* codes, const float* scales, int32_t B, int32_t S, int32_t H, int32_t D,
                        int32_t block, void* y, void* stream) {
    return dequantize_entry(false, codes, scales, B, S, H, D, block, y, stream);
}

int saq_quantize_fp8(const void* x, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, uint8_t* codes,
                     float* scales, void* stream) {
    return quantize_entry(true, x, B, S, H, D, block, codes, scales, stream);
}

int saq_dequantize_fp8(const uint8_t* codes, const float* scales, int32_t B, int32_t S, int32_t H, int32_t D,
                       int32_t block, void* y, void* stream) {
    return dequantize_entry(true, codes, scales, B, S, H, D, block, y, stream);
}

int32_t saq_kept_blocks(double keep_ratio, int32_t nB) {
    if (nB < 1) return SAQ_ERR_SHAPE;
    if (!(keep_ratio > 0.0 && keep_ratio <= 1.0)) return SAQ_ERR_RANGE;
    double kk = ceil(keep_ratio * (double)nB - 1e-6);
    if (kk < 1.0) kk = 1.0;
    if (kk > (double)nB) kk = (double)nB;
    return (int32_t)kk;
}

size_t saq_select_blocks_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block) {
    if (check_dims(B, S, H, D) || check_block(S, block)) return 0;
    const int64_t nB = ((int64_t)S + block - 1) / block;
    return saq::select_workspace_bytes(B, H, nB, D);
}

int saq_select_blocks(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                      double keep_ratio, uint8_t* block_mask, void* workspace, size_t workspace_bytes,
                      void* stream) {
    if (!q || !k || !block_mask) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    const int32_t nB = (S + block - 1) / block;
    const int32_t kept = saq_kept_blocks(keep_ratio, nB);
    if (kept < 0) return kept;
    if (!aligned16(q) || !aligned16(k)) return SAQ_ERR_ALIGN;
    const size_t need = saq::select_workspace_bytes(B, H, nB, D);
    if (!workspace || workspace_bytes < need) return SAQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return SAQ_ERR_ALIGN;
    const size_t bytes = (size_t)B * S * H * D * 2;
    const size_t mbytes = (size_t)B * H * nB * nB;
    if (overlaps(block_mask, mbytes, q, bytes) || overlaps(block_mask, mbytes, k, bytes) ||
        overlaps(workspace, need, q, bytes) || overlaps(workspace, need, k, bytes) ||
        overlaps(workspace, need, block_mask, mbytes))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    return finish(saq::launch_select_blocks(q, k, B, S, H, D, block, kept, block_mask, workspace,
                                            (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Block selection without a caller workspace (saq_select_blocks_noalloc): its
// scratch is this file-scope device array. Each GPU the library runs on holds
// its own copy from the module's load until the process ends; the host learns
// that copy's address once per device with hipGetSymbolAddress (the array's
// name is not a device address in host code) and passes only that address to
// the kernels.
namespace {

static __device__ __align__(256) uint8_t scratch[SAQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first call on that device.
int scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return SAQ_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SAQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || p == nullptr) {
            g_last_hip_error = (int)err;
            return SAQ_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SAQ_OK;
}

}  // namespace

extern "C" {

int saq_select_blocks_noalloc(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D,
                              int32_t block, double keep_ratio, uint8_t* block_mask, void* stream) {
    if (!q || !k || !block_mask) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    const int32_t nB = (S + block - 1) / block;
    const int32_t kept = saq_kept_blocks(keep_ratio, nB);
    if (kept < 0) return kept;
    if (!aligned16(q) || !aligned16(k)) return SAQ_ERR_ALIGN;
    if (saq::select_workspace_bytes(B, H, nB, D) > (size_t)SAQ_NOALLOC_SCRATCH_BYTES) return SAQ_ERR_WORKSPACE;
    const size_t bytes = (size_t)B * S * H * D * 2;
    const size_t mbytes = (size_t)B * H * nB * nB;
    if (overlaps(block_mask, mbytes, q, bytes) || overlaps(block_mask, mbytes, k, bytes)) return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st) return st;
    return finish(saq::launch_select_blocks(q, k, B, S, H, D, block, kept, block_mask, ws, (hipStream_t)stream));
}

int saq_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* block_mask, int32_t B,
                          int32_t S, int32_t H, int32_t D, int32_t block, float softmax_scale, void* o,
                          void* stream) {
    if (!q || !k || !v || !block_mask || !o) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    if (!isfinite(softmax_scale)) return SAQ_ERR_RANGE;
    if ((int64_t)B * H * ((S + block - 1) / block) >= ((int64_t)1 << 31)) return SAQ_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SAQ_ERR_ALIGN;
    const int32_t nB = (S + block - 1) / block;
    const size_t bytes = (size_t)B * S * H * D * 2;
    const size_t mbytes = (size_t)B * H * nB * nB;
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes) ||
        overlaps(o, bytes, block_mask, mbytes))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    return finish(saq::launch_block_sparse_attn(q, k, v, block_mask, B, S, H, D, block, scale, o,
                                                (hipStream_t)stream));
}

int saq_block_sparse_attn_select(const void* q, const void* k, const void* v, const void* workspace,
                                 size_t workspace_bytes, int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                                 double keep_ratio, float softmax_scale, void* o, uint8_t* block_mask_out,
                                 void* stream) {
    if (!q || !k || !v || !workspace || !o) return SAQ_ERR_NULL;
    int st = check_dims(B, S, H, D);
    if (st) return st;
    st = check_block(S, block);
    if (st) return st;
    if (D != 128 || block != 128) return SAQ_ERR_UNSUPPORTED;
    if (!isfinite(softmax_scale)) return SAQ_ERR_RANGE;
    const int32_t nB = (S + block - 1) / block;
    const int32_t kept = saq_kept_blocks(keep_ratio, nB);
    if (kept < 0) return kept;
    if ((int64_t)B * H * nB >= ((int64_t)1 << 31)) return SAQ_ERR_SHAPE;
    const size_t pooled = (size_t)2 * B * H * nB * D * sizeof(double);
    if (workspace_bytes < pooled) return SAQ_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SAQ_ERR_ALIGN;
    if (((uintptr_t)workspace & 255u) != 0) return SAQ_ERR_ALIGN;
    const size_t bytes = (size_t)B * S * H * D * 2;
    const size_t mbytes = (size_t)B * H * nB * nB;
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes) ||
        overlaps(o, bytes, workspace, pooled))
        return SAQ_ERR_ALIAS;
    if (block_mask_out &&
        (overlaps(block_mask_out, mbytes, o, bytes) || overlaps(block_mask_out, mbytes, workspace, pooled) ||
         overlaps(block_mask_out, mbytes, q, bytes) || overlaps(block_mask_out, mbytes, k, bytes) ||
         overlaps(block_mask_out, mbytes, v, bytes)))
        return SAQ_ERR_ALIAS;
    st = device_ready();
    if (st) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    return finish(saq::launch_block_sparse_attn_select(q, k, v, (const double*)workspace, B, S, H, kept, scale, o,
                                                       block_mask_out, (hipStream_t)stream));
}

const char* saq_status_string(int status) {
    switch (status) {
        case SAQ_OK: return "ok";
        case SAQ_ERR_NULL: return "null pointer argument";
        case SAQ_ERR_SHAPE: return "invalid or too large shape";
        case SAQ_ERR_UNSUPPORTED: return "unsupported head_dim or block size (supported: 64, 128)";
        case SAQ_ERR_ALIGN: return "tensor pointer not 16-byte aligned (workspace: 256-byte)";
        case SAQ_ERR_RANGE: return "argument out of range (keep_ratio, eps, rope_base or softmax_scale)";
        case SAQ_ERR_WORKSPACE: return "workspace missing or too small";
        case SAQ_ERR_HIP: return "HIP call failed";
        case SAQ_ERR_NO_DEVICE: return "no HIP device visible";
        case SAQ_ERR_ALIAS: return "output overlaps an input";
        default: return "unknown status";
    }
}

int saq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
