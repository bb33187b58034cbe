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
#include "stream_io.h"

namespace saq {

namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;   // 16-byte chunks kept in flight per thread

// Sum over the kLanesPerRow (8 or 16) adjacent lanes holding one row, with DPP
// lane exchanges (no LDS): swap neighbours, swap pairs, mirror the halves of
// each 8-lane group, then (16 lanes) mirror the two 8-lane groups. Each step
// adds two equal-shaped partial sums, so every lane ends with the same bits.
template <int kLanesPerRow>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(kLanesPerRow == 8 || kLanesPerRow == 16, "row of 8 or 16 lanes");
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    if constexpr (kLanesPerRow == 16)
        v = v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// QKNorm + RoPE of one 16-byte chunk (8 channels) of a (token, head) row, the
// row spread over kLanesPerRow adjacent lanes. Both prologue kernels call this
// one routine, with contraction into FMA switched off and every FMA written
// out, so they produce the same bits. The reciprocal square root is the
// hardware's (within 1 fp32 ulp; the result is rounded to bf16). With kAcc,
// the rounded bf16 outputs are also added to acc in fp64 (exact for these
// values).
template <bool kAcc, int kLanesPerRow>
__device__ __forceinline__ uint4 norm_rope_chunk(const uint4 raw, const float (&w)[8], const float2 (&rot)[4],
                                                 float eps, float inv_d, double (&acc)[8]) {
#pragma clang fp contract(off)
    const uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_bits_to_f32(w32[e] & 0xffffu);
        x[2 * e + 1] = __uint_as_float(w32[e] & 0xffff0000u);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = row_sum<kLanesPerRow>(ss);
    float rinv = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_d, eps));
    if (__builtin_isinf(ss)) {
        // A row with entries beyond about 2^60 overflows the fp32 sum of squares. Every lane of the row
        // takes this branch (they hold the same sum). Redo the sum on x * 2^-68, exact and finite for
        // every finite bf16 x, and scale back: rsqrt(sum(x^2)/D) = rsqrt(sum((x 2^-68)^2)/D) * 2^-68.
        // eps * 2^-136 would be lost against any such mean square, so it is left out.
        float ss2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xs = x[e] * 0x1p-68f;
            ss2 = __builtin_fmaf(xs, xs, ss2);
        }
        ss2 = row_sum<kLanesPerRow>(ss2);
        rinv = __builtin_amdgcn_rsqf(ss2 * inv_d) * 0x1p-68f;
    }
    uint32_t outw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float y0 = x[2 * p] * rinv * w[2 * p];
        const float y1 = x[2 * p + 1] * rinv * w[2 * p + 1];
        const uint32_t h0 = f32_to_bf16_bits(__builtin_fmaf(y0, rot[p].x, -(y1 * rot[p].y)));
        const uint32_t h1 = f32_to_bf16_bits(__builtin_fmaf(y0, rot[p].y, y1 * rot[p].x));
        outw[p] = h0 | (h1 << 16);
        if constexpr (kAcc) {
            acc[2 * p] += (double)bf16_bits_to_f32(h0);
            acc[2 * p + 1] += (double)bf16_bits_to_f32(h1);
        }
    }
    return make_uint4(outw[0], outw[1], outw[2], outw[3]);
}

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
                raw[j] = c < chunks_per_tensor ? load_once(&q_in[base + c]) : load_once(&k_in[base + c - chunks_per_tensor]);
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int c = c0 + j * kThreads;
            // Whole rows are in or out together (total and the stride are multiples of a row).
            if (c < total) {
                const bool is_q = c < chunks_per_tensor;
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = is_q ? wq[e] : wk[e];
                double unused[8];
                const uint4 o = norm_rope_chunk<false, kLanesPerRow>(raw[j], w, rot, eps, 1.0f / D, unused);
                if (is_q) store_once(&q_out[base + c], o);
                else store_once(&k_out[base + c - chunks_per_tensor], o);
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
// workgroup walks the block's tokens, applies QKNorm + RoPE exactly as the
// per-token kernel above (same arithmetic, same bits), writes the bf16
// results, and accumulates the rounded bf16 values it wrote in fp64. Sums of
// bf16 values with |x| < 16 are exact in fp64, so the means equal those of the
// separate pooling pass bit for bit, and the pass saves that pass's re-read of
// q-hat and k-hat. The walk is software-pipelined: the loads of the next
// kDepth tokens are in flight while a token is processed, across the chunk
// boundaries too, and the rotation angles (fp64 sincos, computed once per token
// for all heads of q and k) are staged in two LDS buffers of kTokChunk tokens,
// the next chunk's computed while the current one is used.
constexpr int kPoolMaxThreads = 1024;                          // H*D <= 8192


// kDepth: tokens in flight ahead of the one processed; kMaxThreads bounds the
// workgroup (and so the registers available per thread).
template <int D, int kMaxThreads, int kDepth>
__global__ __launch_bounds__(kMaxThreads) void qknorm_rope_pool_kernel(
    const uint4* q_in, const uint4* k_in, uint4* q_out, uint4* k_out, const int32_t* __restrict__ pos_thw,
    const float* __restrict__ w_q, const float* __restrict__ w_k, int32_t S, int32_t H, RopeTable table, float eps,
    int32_t block, int32_t nB, double* __restrict__ pooled) {
    constexpr int kLanesPerRow = D / 8;
    constexpr int kPairs = D / 2;
    constexpr int kTokChunk = 16;                              // tokens whose angles are staged at once
    __shared__ float2 cs[2][kTokChunk][kPairs];

    const int T = (int)blockDim.x;
    const int64_t bi = blockIdx.x;                             // b * nB + i
    const int i = (int)(bi % nB);
    const int64_t b = bi / nB;
    const int t0 = i * block;
    const int t1 = min(t0 + block, S);
    const int n = t1 - t0;
    const int tid = threadIdx.x;
    const int P = H * kLanesPerRow;                            // chunk positions per token row
    const bool active = tid < P;                               // whole rows in or out together
    const int lane_in_row = tid % kLanesPerRow;

    auto stage_angles = [&](int c) {                           // chunk c of the block into buffer c % 2
        const int tc = t0 + c * kTokChunk;
        const int nt = min(kTokChunk, t1 - tc);
        for (int wi = tid; wi < nt * kPairs; wi += T) {
            const int tt = wi / kPairs, p = wi % kPairs;
            const int axis = p < table.pair_end_t ? 0 : (p < table.pair_end_h ? 1 : 2);
            const double theta = (double)pos_thw[(int64_t)(tc + tt) * 3 + axis] * table.inv_freq[p];
            double sn, cn;
            sincos(theta, &sn, &cn);
            cs[c & 1][tt][p] = make_float2((float)cn, (float)sn);
        }
    };

    float wq[8], wk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        wq[e] = w_q[lane_in_row * 8 + e];
        wk[e] = w_k[lane_in_row * 8 + e];
    }
    double accq[8], acck[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) accq[e] = acck[e] = 0.0;

    const int64_t row0 = (b * S + t0) * (int64_t)P + tid;       // position tid of token t0
    uint4 rq[kDepth], rk[kDepth];                               // the next kDepth tokens, oldest first
    if (active) {
#pragma unroll
        for (int a = 0; a < kDepth; ++a)
            if (a < n) {
                rq[a] = load_once(&q_in[row0 + (int64_t)a * P]);
                rk[a] = load_once(&k_in[row0 + (int64_t)a * P]);
            }
    }
    const uint4* qsrc = q_in + row0 + (int64_t)kDepth * P;     // token t + kDepth
    const uint4* ksrc = k_in + row0 + (int64_t)kDepth * P;
    uint4* qdst = q_out + row0;                                // token t
    uint4* kdst = k_out + row0;
    stage_angles(0);
    for (int t = 0; t < n; ++t) {
        const int tt = t % kTokChunk;
        if (tt == 0) {
            __syncthreads();                                   // this chunk staged; the other buffer free
            if (t + kTokChunk < n) stage_angles(t / kTokChunk + 1);
        }
        if (active) {
            const uint4 cq = rq[0], ck = rk[0];
#pragma unroll
            for (int a = 0; a + 1 < kDepth; ++a) {
                rq[a] = rq[a + 1];
                rk[a] = rk[a + 1];
            }
            if (t + kDepth < n) {
                rq[kDepth - 1] = load_once(qsrc);
                rk[kDepth - 1] = load_once(ksrc);
            }
            qsrc += P;
            ksrc += P;
            float2 rot[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) rot[p] = cs[(t / kTokChunk) & 1][tt][lane_in_row * 4 + p];
            store_once(qdst, norm_rope_chunk<true, kLanesPerRow>(cq, wq, rot, eps, 1.0f / D, accq));
            store_once(kdst, norm_rope_chunk<true, kLanesPerRow>(ck, wk, rot, eps, 1.0f / D, acck));
            qdst += P;
            kdst += P;
        }
    }
    if (!active) return;
    const int64_t Bsz = gridDim.x / nB;
    const int h = tid / kLanesPerRow;
    double* outq = pooled + (((int64_t)0 * Bsz + b) * H + h) * nB * (int64_t)D + (int64_t)i * D + lane_in_row * 8;
    double* outk = pooled + (((int64_t)1 * Bsz + b) * H + h) * nB * (int64_t)D + (int64_t)i * D + lane_in_row * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        outq[e] = accq[e] / (double)n;
        outk[e] = acck[e] / (double)n;
    }
}

template <int D>
void launch_pool_d(const void* q_in, const void* k_in, void* q_out, void* k_out, const int32_t* pos_thw,
                   const float* w_q, const float* w_k, int32_t B, int32_t S, int32_t H, const RopeTable& table,
                   float eps, int32_t block, int32_t nB, double* pooled, hipStream_t stream) {
    const int P = H * (D / 8);                                 // <= kMaxRowElems / 8 = 1024
    const int T = ((P + kWave - 1) / kWave) * kWave;
    const dim3 grid((unsigned)((int64_t)B * nB));
    if (T <= 768)       // up to 12 wavefronts: room for three tokens in flight
        hipLaunchKernelGGL((qknorm_rope_pool_kernel<D, 768, 3>), grid, dim3(T), 0, stream, (const uint4*)q_in,
                           (const uint4*)k_in, (uint4*)q_out, (uint4*)k_out, pos_thw, w_q, w_k, S, H, table, eps,
                           block, nB, pooled);
    else
        hipLaunchKernelGGL((qknorm_rope_pool_kernel<D, kPoolMaxThreads, 1>), grid, dim3(T), 0, stream,
                           (const uint4*)q_in, (const uint4*)k_in, (uint4*)q_out, (uint4*)k_out, pos_thw, w_q, w_k,
                           S, H, table, eps, block, nB, pooled);
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
