// A C++ client of the C ABI (include/saq.h) that uses nothing but the HIP
// runtime for memory: it reads one layer's inputs from a file, runs the layer
// through the named calls (qknorm_rope_out -> select_blocks ->
// block_sparse_attn) and through the fused-pooling calls (qknorm_rope_pool ->
// select_blocks_pooled -> block_sparse_attn) on its own stream, and writes
// every output back to a file. Test infrastructure: tests/test_gpu_cabi.py
// compares the outputs with the Python binding's and with the oracle.
//
// Input file (little-endian): int32 B, S, H, D, dt, dh, dw, block; float64
// keep_ratio, base, eps; then q, k, v (bf16 bits, B*S*H*D each), pos_thw
// (int32, S*3), w_q, w_k (float32, D each).
// Output file: q_hat, k_hat (split path), mask, o (split path), q_hat, k_hat,
// mask, o (fused path), in that order, as raw bytes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "saq.h"

#define HIP_OK(x)                                                                              \
    do {                                                                                       \
        hipError_t e_ = (x);                                                                   \
        if (e_ != hipSuccess) {                                                                \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                                          \
        }                                                                                      \
    } while (0)
#define SAQ_OK_(x)                                                                             \
    do {                                                                                       \
        int s_ = (x);                                                                          \
        if (s_ != SAQ_OK) {                                                                    \
            std::fprintf(stderr, "%s failed: %s\n", #x, saq_status_string(s_));               \
            return 3;                                                                          \
        }                                                                                      \
    } while (0)

template <typename T>
static bool read_vec(FILE* f, std::vector<T>& v, size_t n) {
    v.resize(n);
    return std::fread(v.data(), sizeof(T), n, f) == n;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
        return 1;
    }
    FILE* fin = std::fopen(argv[1], "rb");
    if (!fin) return 1;
    int32_t hdr[8];
    double fl[3];
    if (std::fread(hdr, sizeof(int32_t), 8, fin) != 8 || std::fread(fl, sizeof(double), 3, fin) != 3) return 1;
    const int32_t B = hdr[0], S = hdr[1], H = hdr[2], D = hdr[3], dt = hdr[4], dh = hdr[5], dw = hdr[6],
                  block = hdr[7];
    const double keep = fl[0], base = fl[1], eps = fl[2];
    if (B < 1 || S < 1 || H < 1 || D < 1 || block < 1) return 1;
    const size_t n = (size_t)B * S * H * D;
    const int32_t nB = (S + block - 1) / block;
    const size_t nm = (size_t)B * H * nB * nB;
    std::vector<uint16_t> q, k, v;
    std::vector<int32_t> pos;
    std::vector<float> wq, wk;
    if (!read_vec(fin, q, n) || !read_vec(fin, k, n) || !read_vec(fin, v, n) || !read_vec(fin, pos, (size_t)S * 3) ||
        !read_vec(fin, wq, (size_t)D) || !read_vec(fin, wk, (size_t)D))
        return 1;
    std::fclose(fin);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *dq, *dk, *dv, *dqh, *dkh, *do1, *do2, *dqf, *dkf, *dws, *dws2;
    uint8_t *dm1, *dm2;
    int32_t* dpos;
    float *dwq, *dwk;
    const size_t bytes = n * 2;
    const size_t ws_bytes = saq_select_blocks_workspace_bytes(B, S, H, D, block);
    if (ws_bytes == 0) return 4;
    for (void** p : {&dq, &dk, &dv, &dqh, &dkh, &do1, &do2, &dqf, &dkf}) HIP_OK(hipMalloc(p, bytes));
    HIP_OK(hipMalloc(&dws, ws_bytes));
    HIP_OK(hipMalloc(&dws2, ws_bytes));
    HIP_OK(hipMalloc(&dm1, nm));
    HIP_OK(hipMalloc(&dm2, nm));
    HIP_OK(hipMalloc(&dpos, (size_t)S * 3 * sizeof(int32_t)));
    HIP_OK(hipMalloc(&dwq, (size_t)D * sizeof(float)));
    HIP_OK(hipMalloc(&dwk, (size_t)D * sizeof(float)));
    HIP_OK(hipMemcpy(dq, q.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, k.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, v.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dpos, pos.data(), (size_t)S * 3 * sizeof(int32_t), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dwq, wq.data(), (size_t)D * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dwk, wk.data(), (size_t)D * sizeof(float), hipMemcpyHostToDevice));

    // the named calls
    SAQ_OK_(saq_qknorm_rope_out(dq, dk, dqh, dkh, dpos, dwq, dwk, B, S, H, D, dt, dh, dw, base, eps, stream));
    SAQ_OK_(saq_select_blocks(dqh, dkh, B, S, H, D, block, keep, dm1, dws, ws_bytes, stream));
    SAQ_OK_(saq_block_sparse_attn(dqh, dkh, dv, dm1, B, S, H, D, block, 0.0f, do1, stream));
    // pooling fused into the prologue
    SAQ_OK_(saq_qknorm_rope_pool(dq, dk, dqf, dkf, dpos, dwq, dwk, B, S, H, D, dt, dh, dw, base, eps, block, dws2,
                                 ws_bytes, stream));
    SAQ_OK_(saq_select_blocks_pooled(B, S, H, D, block, keep, dm2, dws2, ws_bytes, stream));
    SAQ_OK_(saq_block_sparse_attn(dqf, dkf, dv, dm2, B, S, H, D, block, 0.0f, do2, stream));
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<uint8_t> out(bytes);
    std::vector<uint8_t> mout(nm);
    FILE* fo = std::fopen(argv[2], "wb");
    if (!fo) return 1;
    for (int pass = 0; pass < 2; ++pass) {
        void* srcs[3] = {pass ? dqf : dqh, pass ? dkf : dkh, nullptr};
        for (int t = 0; t < 2; ++t) {
            HIP_OK(hipMemcpy(out.data(), srcs[t], bytes, hipMemcpyDeviceToHost));
            std::fwrite(out.data(), 1, bytes, fo);
        }
        HIP_OK(hipMemcpy(mout.data(), pass ? dm2 : dm1, nm, hipMemcpyDeviceToHost));
        std::fwrite(mout.data(), 1, nm, fo);
        HIP_OK(hipMemcpy(out.data(), pass ? do2 : do1, bytes, hipMemcpyDeviceToHost));
        std::fwrite(out.data(), 1, bytes, fo);
    }
    std::fclose(fo);
    for (void* p : {dq, dk, dv, dqh, dkh, do1, do2, dqf, dkf, dws, dws2}) HIP_OK(hipFree(p));
    HIP_OK(hipFree(dm1));
    HIP_OK(hipFree(dm2));
    HIP_OK(hipFree(dpos));
    HIP_OK(hipFree(dwq));
    HIP_OK(hipFree(dwk));
    HIP_OK(hipStreamDestroy(stream));
    std::printf("layer_client ok: B=%d S=%d H=%d D=%d block=%d keep=%.3f\n", B, S, H, D, block, keep);
    return 0;
}
