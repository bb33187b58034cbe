// Host-side driver for the C ABI's argument validation, built with the address
// and undefined-behaviour sanitizers on the host code (tests/test_capi_sanitized.py).
// Every call below must be rejected on the host, or (valid arguments, no GPU
// visible) report SAQ_ERR_NO_DEVICE, without any sanitizer report. Pointers are
// never dereferenced: validation runs before any HIP call.
#include <stdint.h>
#include <stdio.h>

#include <limits>

#include "saq.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
    if (got != want) {
        printf("FAIL %s: got %d want %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    const uintptr_t F = 0x10000;                       // 16-byte aligned, never dereferenced
    void* const p1 = (void*)(F * 1);
    void* const p2 = (void*)(F * 2);
    void* const p3 = (void*)(F * 3);
    const int32_t* pos = (const int32_t*)(F * 4);
    const float* w = (const float*)(F * 5);
    const int32_t big = std::numeric_limits<int32_t>::max();

    // prologue
    expect(saq_qknorm_rope(nullptr, p2, pos, w, w, 1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6, nullptr), SAQ_ERR_NULL, "rope null");
    expect(saq_qknorm_rope(p1, p2, pos, w, w, big, big, big, 64, 16, 24, 24, 1e4, 1e-6, nullptr), SAQ_ERR_SHAPE, "rope huge");
    expect(saq_qknorm_rope(p1, p2, pos, w, w, -1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6, nullptr), SAQ_ERR_SHAPE, "rope neg");
    expect(saq_qknorm_rope(p1, p2, pos, w, w, 1, 16, 2, 96, 32, 32, 32, 1e4, 1e-6, nullptr), SAQ_ERR_UNSUPPORTED, "rope D");
    expect(saq_qknorm_rope(p1, p2, pos, w, w, 1, 16, 2, 64, 16, 24, 24, 1.0, 1e-6, nullptr), SAQ_ERR_RANGE, "rope base");
    expect(saq_qknorm_rope(p1, (void*)(F * 2 + 8), pos, w, w, 1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6, nullptr), SAQ_ERR_ALIGN, "rope align");
    expect(saq_qknorm_rope((void*)(1ull << 26), (void*)(2ull << 26), pos, w, w, 1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6,
                           nullptr), SAQ_ERR_NO_DEVICE, "rope valid");
    expect(saq_qknorm_rope_pool(p1, p2, p3, (void*)(F * 6), pos, w, w, 1, 16, 65, 128, 32, 48, 48, 1e4, 1e-6, 64,
                                (void*)(1 << 28), 8, nullptr), SAQ_ERR_ALIAS, "pool overlap");

    // selection
    expect((int)saq_select_blocks_workspace_bytes(big, big, big, 128, 128), 0, "ws huge");
    expect(saq_kept_blocks(0.5, big), (int32_t)((big + 1ll) / 2), "kept big");
    expect(saq_kept_blocks(-0.0, 10), SAQ_ERR_RANGE, "kept -0");
    expect(saq_select_blocks(p1, p2, 1, big, 2, 64, 64, 0.5, (uint8_t*)p3, (void*)(1 << 24), 1 << 20, nullptr),
           SAQ_ERR_SHAPE, "select huge S");
    expect(saq_select_blocks((void*)(1ull << 26), (void*)(2ull << 26), 1, 1024, 2, 64, 64, 0.5, (uint8_t*)(3ull << 26),
                             (void*)(1 << 24), 1 << 20, nullptr),
           SAQ_ERR_NO_DEVICE, "select valid");
    expect(saq_select_blocks_pooled(1, 1024, 2, 64, 64, 0.5, (uint8_t*)p3, (void*)(1 << 24), 16, nullptr),
           SAQ_ERR_WORKSPACE, "pooled small ws");
    expect(saq_mask_overlap((const uint8_t*)p1, (const uint8_t*)p2, big, big, 4096, (int64_t*)(1 << 24), nullptr),
           SAQ_ERR_SHAPE, "overlap huge");
    expect(saq_pooled_change(p1, p2, 1, 1024, 2, 64, 64, (double*)(1 << 24), 1, nullptr), SAQ_ERR_WORKSPACE,
           "change small out");
    expect(saq_select_blocks_reuse(1, 1024, 2, 64, 64, 0.5, 1e308 * 10, 0, (uint8_t*)p3, (void*)(1 << 24), 1 << 20,
                                   (void*)(1 << 25), 1 << 20, (double*)(1 << 26), saq_reuse_state_len(), nullptr),
           SAQ_ERR_RANGE, "reuse inf threshold");

    // attention
    expect(saq_block_sparse_attn(p1, p2, p3, (const uint8_t*)(F * 4), 1, big, big, 128, 128, 0.f, (void*)(1 << 24),
                                 nullptr), SAQ_ERR_SHAPE, "attn huge");
    expect(saq_block_sparse_attn((void*)(1ull << 26), (void*)(2ull << 26), (void*)(3ull << 26),
                                 (const uint8_t*)(4ull << 26), 1, 1024, 2, 64, 64, 0.f, (void*)(5ull << 26), nullptr),
           SAQ_ERR_NO_DEVICE, "attn valid");
    expect(saq_block_sparse_attn_select(p1, p2, p3, (void*)(1 << 24), 1 << 20, 1, 1024, 2, 64, 64, 0.5, 0.f,
                                        (void*)(1 << 25), nullptr, nullptr), SAQ_ERR_UNSUPPORTED, "attn select D");

    // codecs
    expect(saq_quantize_int8(p1, big, big, big, 128, 128, (int8_t*)(1 << 24), (float*)(1 << 25), nullptr),
           SAQ_ERR_SHAPE, "quant huge");
    expect(saq_dequantize_fp8((const uint8_t*)(1ull << 26), (const float*)(2ull << 26), 1, 1024, 2, 64, 64,
                              (void*)(3ull << 26), nullptr),
           SAQ_ERR_NO_DEVICE, "dequant valid");

    for (int st = -12; st <= 2; ++st)
        if (saq_status_string(st) == nullptr) {
            printf("FAIL status string %d\n", st);
            ++failures;
        }
    printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
