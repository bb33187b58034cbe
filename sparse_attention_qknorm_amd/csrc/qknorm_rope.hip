// Fused QKNorm + 3D multimodal RoPE for gfx950.
//
// Sol Engine "H3 on device" page, lossless-kernels fusion table, row "fused
// QKNorm + RoPE": one pass over Q and K replaces the separate norm and rotary
// passes and the 3D position indexing. Per (token, head) row x:
//   x_hat = x / sqrt(mean(x^2) + eps) * w, then each adjacent pair (2i, 2i+1)
//   of section a in (t, h, w) turns by pos_a * base^(-2i/d_a).
//
// Design: one workgroup per token (b, s). The token's Q and K rows (H*D bf16
// each) are contiguous in [B,S,H,D], so the workgroup streams 2*H*D*2 bytes
// with 16-byte loads and stores and touches nothing else but pos_thw[s] and
// the two weight vectors. The D/2 rotation angles of the token are computed
// once in fp64 (sincos of pos * inv_freq) into LDS and reused by all heads of
// Q and K. A row of D elements is D/8 lanes; its sum of squares is reduced with
// lane shuffles inside that lane group. The pass is HBM-bound: 8*D bytes per
// (token, head) for the read and write of q and k.
#include "common.h"
#include "kernels.h"

namespace saq {

namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;   // 16-byte chunks kept in flight per thread

template <int D>
__global__ __launch_bounds__(kThreads) void qknorm_rope_kernel(
    const uint4* q_in, const uint4* k_in, uint4* q_out, uint4* k_out,
    const int32_t* __restrict__ pos_thw, const float* __restrict__ w_q, const float* __restrict__ w_k,
    int32_t S, int32_t H, RopeTable table, float eps) {
    constexpr int kLanesPerRow = D / 8;
    constexpr int kPairs = D / 2;
    __shared__ float2 cs[kPairs];

    const int64_t token = blockIdx.x;             // b * S + s
    const int32_t s = (int32_t)(token % S);
    const int tid = threadIdx.x;

    if (tid < kPairs) {
        const int axis = tid < table.pair_end_t ? 0 : (tid < table.pair_end_h ? 1 : 2);
        const double theta = (double)pos_thw[(int64_t)s * 3 + axis] * table.inv_freq[tid];
        double sn, cn;
        sincos(theta, &sn, &cn);
        cs[tid] = make_float2((float)cn, (float)sn);
    }
    __syncthreads();

    // Every chunk a thread visits has the same position inside its row.
    const int lane_in_row = tid % kLanesPerRow;
    float2 rot[4];
    float wq[8], wk[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) rot[p] = cs[lane_in_row * 4 + p];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        wq[e] = w_q[lane_in_row * 8 + e];
        wk[e] = w_k[lane_in_row * 8 + e];
    }

    const int chunks_per_tensor = H * kLanesPerRow;
    const int total = 2 * chunks_per_tensor;
    const int64_t base = token * (int64_t)chunks_per_tensor;

    for (int c0 = tid; c0 < total; c0 += kThreads * kBatch) {
        uint4 raw[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int c = c0 + j * kThreads;
            if (c < total) {
                raw[j] = c < chunks_per_tensor ? q_in[base + c] : k_in[base + c - chunks_per_tensor];
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int c = c0 + j * kThreads;
            // Whole rows are in or out together (total and the stride are multiples of a row).
            if (c < total) {
                const bool is_q = c < chunks_per_tensor;
                const uint32_t w32[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bf16_bits_to_f32(w32[e] & 0xffffu);
                    x[2 * e + 1] = bf16_bits_to_f32(w32[e] >> 16);
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
                for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kLanesPerRow);
                const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
                uint32_t outw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float y0 = x[2 * p] * rinv * (is_q ? wq[2 * p] : wk[2 * p]);
                    const float y1 = x[2 * p + 1] * rinv * (is_q ? wq[2 * p + 1] : wk[2 * p + 1]);
                    const float r0 = y0 * rot[p].x - y1 * rot[p].y;
                    const float r1 = y0 * rot[p].y + y1 * rot[p].x;
                    outw[p] = f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16);
                }
                const uint4 o = make_uint4(outw[0], outw[1], outw[2], outw[3]);
                if (is_q) q_out[base + c] = o;
                else k_out[base + c - chunks_per_tensor] = o;
            }
        }
    }
}

}  // namespace

hipError_t launch_qknorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                              const int32_t* pos_thw, const float* w_q, const float* w_k,
                              int32_t B, int32_t S, int32_t H, int32_t D, const RopeTable& table,
                              float eps, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)B * S));
    const dim3 block(kThreads);
    if (D == 128) {
        hipLaunchKernelGGL((qknorm_rope_kernel<128>), grid, block, 0, stream, (const uint4*)q_in,
                           (const uint4*)k_in, (uint4*)q_out, (uint4*)k_out, pos_thw, w_q, w_k, S, H, table, eps);
    } else {
        hipLaunchKernelGGL((qknorm_rope_kernel<64>), grid, block, 0, stream, (const uint4*)q_in,
                           (const uint4*)k_in, (uint4*)q_out, (uint4*)k_out, pos_thw, w_q, w_k, S, H, table, eps);
    }
    return hipGetLastError();
}

}  // namespace saq

namespace saq {

namespace {

// ---------------------------------------------------------------------------
// Fused form with block pooling. One workgroup per (b, block of `block` tokens)
// covering every head: one thread per 16-byte chunk position (head, 8
// channels) of a token row, H*D/8 of them (rounded up to whole wavefronts),
// each handling that position of both q and k for the whole block. The
// workgroup walks the block's tokens one at a time, applies QKNorm + RoPE
// exactly as the per-token kernel above (same arithmetic, same bits), writes
// the bf16 results, and accumulates the rounded bf16 values it wrote in fp64.
// Sums of bf16 values with |x| < 16 are exact in fp64, so the means equal those
// of the separate pooling pass bit for bit, and the pass saves that pass's
// re-read of q-hat and k-hat. Each token's rotation angles are computed once
// (fp64 sincos, staged in LDS kTokChunk tokens at a time) for all heads of q
// and k. Measured at the full shape: one token per step and whole rows per
// workgroup beat splitting the heads over workgroups or keeping more tokens in
// flight per thread.
constexpr int kPoolMaxThreads = 1024;                          // H*D <= 8192

template <int D>
__global__ __launch_bounds__(kPoolMaxThreads) void qknorm_rope_pool_kernel(
    const uint4* q_in, const uint4* k_in, uint4* q_out, uint4* k_out, const int32_t* __restrict__ pos_thw,
    const float* __restrict__ w_q, const float* __restrict__ w_k, int32_t S, int32_t H, RopeTable table, float eps,
    int32_t block, int32_t nB, double* __restrict__ pooled) {
    constexpr int kLanesPerRow = D / 8;
    constexpr int kPairs = D / 2;
    constexpr int kTokChunk = 32;                              // tokens whose angles are staged at once
    __shared__ float2 cs[kTokChunk][kPairs];

    const int T = (int)blockDim.x;
    const int64_t bi = blockIdx.x;                             // b * nB + i
    const int i = (int)(bi % nB);
    const int64_t b = bi / nB;
    const int t0 = i * block;
    const int t1 = min(t0 + block, S);
    const int tid = threadIdx.x;
    const int P = H * kLanesPerRow;                            // chunk positions per token row
    const bool active = tid < P;                               // whole rows in or out together
    const int lane_in_row = tid % kLanesPerRow;
    float wq[8], wk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        wq[e] = w_q[lane_in_row * 8 + e];
        wk[e] = w_k[lane_in_row * 8 + e];
    }
    double acc[2][8];                                          // [tensor][channel]
#pragma unroll
    for (int ten = 0; ten < 2; ++ten)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[ten][e] = 0.0;

    for (int tc = t0; tc < t1; tc += kTokChunk) {
        const int nt = min(kTokChunk, t1 - tc);
        __syncthreads();                                       // previous chunk's angles consumed
        for (int wi = tid; wi < nt * kPairs; wi += T) {
            const int tt = wi / kPairs, p = wi % kPairs;
            const int axis = p < table.pair_end_t ? 0 : (p < table.pair_end_h ? 1 : 2);
            const double theta = (double)pos_thw[(int64_t)(tc + tt) * 3 + axis] * table.inv_freq[p];
            double sn, cn;
            sincos(theta, &sn, &cn);
            cs[tt][p] = make_float2((float)cn, (float)sn);
        }
        __syncthreads();
        if (!active) continue;
        for (int ts = 0; ts < nt; ++ts) {
            const int64_t at = (b * S + tc + ts) * (int64_t)P + tid;
            const uint4 raw[2] = {q_in[at], k_in[at]};
            float2 rot[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) rot[p] = cs[ts][lane_in_row * 4 + p];
#pragma unroll
            for (int ten = 0; ten < 2; ++ten) {
                const uint32_t w32[4] = {raw[ten].x, raw[ten].y, raw[ten].z, raw[ten].w};
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bf16_bits_to_f32(w32[e] & 0xffffu);
                    x[2 * e + 1] = bf16_bits_to_f32(w32[e] >> 16);
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
                for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kLanesPerRow);
                const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
                uint32_t outw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float y0 = x[2 * p] * rinv * (ten == 0 ? wq[2 * p] : wk[2 * p]);
                    const float y1 = x[2 * p + 1] * rinv * (ten == 0 ? wq[2 * p + 1] : wk[2 * p + 1]);
                    const uint32_t h0 = f32_to_bf16_bits(y0 * rot[p].x - y1 * rot[p].y);
                    const uint32_t h1 = f32_to_bf16_bits(y0 * rot[p].y + y1 * rot[p].x);
                    outw[p] = h0 | (h1 << 16);
                    acc[ten][2 * p] += (double)bf16_bits_to_f32(h0);
                    acc[ten][2 * p + 1] += (double)bf16_bits_to_f32(h1);
                }
                const uint4 o = make_uint4(outw[0], outw[1], outw[2], outw[3]);
                if (ten == 0) q_out[at] = o;
                else k_out[at] = o;
            }
        }
    }
    if (!active) return;
    const int64_t Bsz = gridDim.x / nB;
    const int h = tid / kLanesPerRow;
#pragma unroll
    for (int ten = 0; ten < 2; ++ten) {
        double* out = pooled + ((((int64_t)ten * Bsz + b) * H + h) * nB + i) * (int64_t)D + lane_in_row * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = acc[ten][e] / (double)(t1 - t0);
    }
}

template <int D>
void launch_pool_d(const void* q_in, const void* k_in, void* q_out, void* k_out, const int32_t* pos_thw,
                   const float* w_q, const float* w_k, int32_t B, int32_t S, int32_t H, const RopeTable& table,
                   float eps, int32_t block, int32_t nB, double* pooled, hipStream_t stream) {
    const int P = H * (D / 8);                                 // <= kMaxRowElems / 8 = 1024
    const int T = ((P + kWave - 1) / kWave) * kWave;
    hipLaunchKernelGGL((qknorm_rope_pool_kernel<D>), dim3((unsigned)((int64_t)B * nB)), dim3(T), 0, stream,
                       (const uint4*)q_in, (const uint4*)k_in, (uint4*)q_out, (uint4*)k_out, pos_thw, w_q, w_k, S,
                       H, table, eps, block, nB, pooled);
}

}  // namespace

hipError_t launch_qknorm_rope_pool(const void* q_in, const void* k_in, void* q_out, void* k_out,
                                   const int32_t* pos_thw, const float* w_q, const float* w_k, int32_t B,
                                   int32_t S, int32_t H, int32_t D, const RopeTable& table, float eps,
                                   int32_t block, double* pooled, hipStream_t stream) {
    const int32_t nB = (S + block - 1) / block;
    if (D == 128)
        launch_pool_d<128>(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, table, eps, block, nB, pooled, stream);
    else
        launch_pool_d<64>(q_in, k_in, q_out, k_out, pos_thw, w_q, w_k, B, S, H, table, eps, block, nB, pooled, stream);
    return hipGetLastError();
}

}  // namespace saq
