// Training-free dynamic block selection for gfx950.
//
// The Sol-Attn paragraph of the Sol Engine "H3 on device" page says only the
// (query block, key block) tiles a per-step selection keeps are computed, and
// the KOCPC article on Sol-H3 ("Specific outcomes of key optimizations") says
// the selection is decided dynamically during inference. The rule implemented
// here (the pages do not give one), per (b, h):
//   p_i  = mean of the q-hat (k-hat) rows of block i, fp64;
//   s_ij = sum_d pq_i[d] * pk_j[d], fp64, d ascending, no fused multiply-add;
//   row i keeps i and the k-1 largest s_ij (j != i), ties to the lower j.
//
// Three kernels:
//  1. pool:   one workgroup per (tensor, b, block, head); 16-byte loads of the
//             block's rows, fp64 sums. The inputs are bf16 with |x| < 16 and,
//             when non-zero, |x| >= 2^-35, so every partial sum is exact in
//             fp64 and the result does not depend on the reduction order.
//             HBM-bound: 4*D bytes per (token, head).
//  2. scores: per (b, h) a tiled nB x nB product of the pooled vectors in fp64
//             vector ALU (128x128 tile per workgroup, 8x8 per thread, pooled
//             vectors staged in LDS by 16-wide d slices). Contraction into FMA
//             is switched off so every product and sum rounds on its own, in
//             the same order as the definition. The scores leave as uint64
//             keys whose unsigned order is the fp64 order (-0.0 -> +0.0).
//  3. topk:   one wavefront per query-block row; the row's keys sit in
//             registers; a bitwise search over the key value, counting with
//             wave ballots, finds the (k-1)-th largest key T (32 steps on the
//             upper halves, 32 more only when keys tie there); keys > T are
//             kept, and keys == T are kept in ascending j until k-1 are kept.
#include "common.h"
#include "kernels.h"

namespace saq {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- pooling

template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                        double* __restrict__ pooled, int32_t S, int32_t H,
                                                        int32_t block, int32_t nB) {
    constexpr int kLanesPerRow = D / 8;                 // 16-byte chunks per row
    constexpr int kRowsPerPass = kThreads / kLanesPerRow;
    __shared__ double part[kRowsPerPass][D + 1];

    // blockIdx.x = ((tensor * B + b) * nB + i) * H + h
    int64_t id = blockIdx.x;
    const int h = (int)(id % H);
    id /= H;
    const int i = (int)(id % nB);
    id /= nB;
    const int64_t tb = id;                              // tensor * B + b
    const int64_t Bsz = gridDim.x / ((int64_t)nB * H * 2);
    const int tensor = (int)(tb / Bsz);
    const int64_t b = tb % Bsz;
    const uint4* x = tensor == 0 ? q : k;

    const int lane = threadIdx.x % kLanesPerRow;
    const int row0 = threadIdx.x / kLanesPerRow;
    const int t0 = i * block;
    const int t1 = min(t0 + block, S);

    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int t = t0 + row0; t < t1; t += kRowsPerPass) {
        const uint4 raw = x[((b * S + t) * H + h) * kLanesPerRow + lane];
        const uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16_bits_to_f32(w32[e] & 0xffffu);
            acc[2 * e + 1] += (double)bf16_bits_to_f32(w32[e] >> 16);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[row0][lane * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        double sum = 0.0;
        for (int r = 0; r < kRowsPerPass; ++r) sum += part[r][threadIdx.x];
        pooled[(((int64_t)tensor * Bsz + b) * H + h) * (int64_t)nB * D + (int64_t)i * D + threadIdx.x] =
            sum / (double)(t1 - t0);
    }
}

// ---------------------------------------------------------------- scores

__device__ __forceinline__ uint64_t order_key(double s) {
    uint64_t u = __double_as_longlong(s);
    if (u == 0x8000000000000000ull) u = 0;                      // -0.0 ranks as +0.0
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// 128 x 128 tiles, 8 x 8 scores per thread (rows ty + 16r, columns tx + 16s, so a
// wavefront's column reads are 16 consecutive doubles and its row reads are
// broadcasts), d staged 16 at a time into LDS rows padded to 129 doubles (the
// transposing writes then spread over the banks) while the next 16 are loaded
// into registers. Each score is sum over d ascending of the rounded products,
// each partial sum rounded: the canonical order of the selection rule.
constexpr int kTile2 = 128;
constexpr int kSlice2 = 16;
constexpr int kPad2 = kTile2 + 1;

template <int D>
__global__ __launch_bounds__(kThreads) void scores128_kernel(const double* __restrict__ pq,
                                                             const double* __restrict__ pk,
                                                             uint64_t* __restrict__ keys, int32_t nB, int32_t tiles,
                                                             const double* __restrict__ gate) {
#pragma clang fp contract(off)
    __shared__ double sq[kSlice2][kPad2];
    __shared__ double sk[kSlice2][kPad2];
    if (gate != nullptr && *gate == 0.0) return;        // the mask of an earlier step is kept

    const int64_t bh = blockIdx.x / ((int64_t)tiles * tiles);
    const int tile = (int)(blockIdx.x % ((int64_t)tiles * tiles));
    const int ti = tile / tiles;
    const int tj = tile % tiles;
    const double* a = pq + bh * (int64_t)nB * D;
    const double* c = pk + bh * (int64_t)nB * D;

    const int tx = threadIdx.x % 16;
    const int ty = threadIdx.x / 16;
    double acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[r][s] = 0.0;

    // staging: element e = threadIdx.x + kThreads * m of a slice is (row e / kSlice2, d e % kSlice2); the
    // next slice is loaded into registers while the current one is multiplied
    constexpr int kPer = kSlice2 * kTile2 / kThreads;
    double nq[kPer], nk[kPer];
    auto fetch = [&](int d0) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int e = threadIdx.x + kThreads * m;
            const int row = e / kSlice2;
            const int dd = e % kSlice2;
            const int gi = ti * kTile2 + row;
            const int gj = tj * kTile2 + row;
            nq[m] = gi < nB ? a[(int64_t)gi * D + d0 + dd] : 0.0;
            nk[m] = gj < nB ? c[(int64_t)gj * D + d0 + dd] : 0.0;
        }
    };
    fetch(0);
    for (int d0 = 0; d0 < D; d0 += kSlice2) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int e = threadIdx.x + kThreads * m;
            sq[e % kSlice2][e / kSlice2] = nq[m];
            sk[e % kSlice2][e / kSlice2] = nk[m];
        }
        __syncthreads();
        if (d0 + kSlice2 < D) fetch(d0 + kSlice2);
#pragma unroll 2
        for (int dd = 0; dd < kSlice2; ++dd) {
            double x[8], y[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) x[r] = sq[dd][ty + 16 * r];
#pragma unroll
            for (int s = 0; s < 8; ++s) y[s] = sk[dd][tx + 16 * s];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const double prod = x[r] * y[s];
                    acc[r][s] = acc[r][s] + prod;
                }
        }
        __syncthreads();
    }
    uint64_t* out = keys + bh * (int64_t)nB * nB;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int gi = ti * kTile2 + ty + 16 * r;
        if (gi >= nB) continue;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int gj = tj * kTile2 + tx + 16 * s;
            if (gj < nB) out[(int64_t)gi * nB + gj] = order_key(acc[r][s]);
        }
    }
}

// ---------------------------------------------------------------- top-k

__device__ __forceinline__ int wave_count(bool p) {
    return __popcll(__ballot(p));
}

template <int R>   // keys per lane: nB <= 64 * R
__global__ __launch_bounds__(kThreads) void topk_kernel(const uint64_t* __restrict__ keys, uint8_t* __restrict__ mask,
                                                        int32_t nB, int64_t rows, int32_t kept,
                                                        const double* __restrict__ gate) {
    if (gate != nullptr && *gate == 0.0) return;
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    if (row >= rows) return;                              // whole wave leaves together
    const int i = (int)(row % nB);
    const uint64_t* kr = keys + row * nB;
    uint8_t* mr = mask + row * nB;

    uint64_t key[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = lane + kWave * r;
        valid[r] = j < nB && j != i;
        key[r] = j < nB ? kr[j] : 0;
    }
    const int need = kept - 1;                            // blocks chosen besides the diagonal

    uint64_t T = ~0ull;                                   // need == 0: nothing passes key > T
    int eq_take = 0;
    if (need > 0) {
        // The search runs on the upper 32 bits first. When every key whose upper half equals the
        // threshold's is kept anyway (the common case: distinct scores rarely agree in their top
        // 32 bits), the selection is already decided; otherwise the search goes on through the
        // lower 32 bits exactly as a 64-step search would.
        uint32_t T32 = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T32 | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) cnt += wave_count(valid[r] && (uint32_t)(key[r] >> 32) >= cand);
            if (cnt >= need) T32 = cand;
        }
        int gt32 = 0, eq32 = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t hi = (uint32_t)(key[r] >> 32);
            gt32 += wave_count(valid[r] && hi > T32);
            eq32 += wave_count(valid[r] && hi == T32);
        }
        if (T32 != 0 && need - gt32 == eq32) {
            T = ((uint64_t)T32 << 32) - 1ull;             // keys > T: exactly those with upper half >= T32
        } else {
            T = (uint64_t)T32 << 32;
            for (int bit = 31; bit >= 0; --bit) {
                const uint64_t cand = T | (1ull << bit);
                int cnt = 0;
#pragma unroll
                for (int r = 0; r < R; ++r) cnt += wave_count(valid[r] && key[r] >= cand);
                if (cnt >= need) T = cand;
            }
            int gt = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) gt += wave_count(valid[r] && key[r] > T);
            eq_take = need - gt;
        }
    }
    const uint64_t below = (1ull << lane) - 1ull;         // lanes with a lower j in this group
    int taken = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = lane + kWave * r;
        const uint64_t eq = __ballot(valid[r] && key[r] == T);
        const int before = taken + __popcll(eq & below);
        const bool sel = valid[r] && (key[r] > T || (key[r] == T && before < eq_take));
        taken += __popcll(eq);
        if (j < nB) mr[j] = (uint8_t)((sel || j == i) ? 1 : 0);
    }
}

template <int R>
void launch_topk(const uint64_t* keys, uint8_t* mask, int32_t nB, int64_t rows, int32_t kept, const double* gate,
                 hipStream_t stream) {
    const int64_t waves_per_wg = kThreads / kWave;
    const dim3 grid((unsigned)((rows + waves_per_wg - 1) / waves_per_wg));
    hipLaunchKernelGGL((topk_kernel<R>), grid, dim3(kThreads), 0, stream, keys, mask, nB, rows, kept, gate);
}

}  // namespace

size_t select_workspace_bytes(int64_t B, int64_t H, int64_t nB, int64_t D) {
    const size_t pooled = (size_t)2 * B * H * nB * D * sizeof(double);
    const size_t keys = (size_t)B * H * nB * nB * sizeof(uint64_t);
    return ((pooled + 255) / 256) * 256 + keys;
}

hipError_t launch_select_from_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                                     uint8_t* mask, void* workspace, hipStream_t stream, const double* gate) {
    const int32_t nB = (S + block - 1) / block;
    const double* pq = (const double*)workspace;
    const double* pk = pq + (size_t)B * H * nB * D;
    const size_t pooled_bytes = ((size_t)2 * B * H * nB * D * sizeof(double) + 255) / 256 * 256;
    uint64_t* keys = (uint64_t*)((char*)workspace + pooled_bytes);

    const int32_t tiles = (nB + kTile2 - 1) / kTile2;
    const dim3 score_grid((unsigned)((int64_t)B * H * tiles * tiles));
    if (D == 128) {
        hipLaunchKernelGGL((scores128_kernel<128>), score_grid, dim3(kThreads), 0, stream, pq, pk, keys, nB, tiles,
                           gate);
    } else {
        hipLaunchKernelGGL((scores128_kernel<64>), score_grid, dim3(kThreads), 0, stream, pq, pk, keys, nB, tiles,
                           gate);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int64_t rows = (int64_t)B * H * nB;
    if (nB <= 64) launch_topk<1>(keys, mask, nB, rows, kept, gate, stream);
    else if (nB <= 256) launch_topk<4>(keys, mask, nB, rows, kept, gate, stream);
    else if (nB <= 1024) launch_topk<16>(keys, mask, nB, rows, kept, gate, stream);
    else launch_topk<64>(keys, mask, nB, rows, kept, gate, stream);
    return hipGetLastError();
}

hipError_t launch_select_blocks(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D,
                                int32_t block, int32_t kept, uint8_t* mask, void* workspace,
                                hipStream_t stream) {
    const int32_t nB = (S + block - 1) / block;
    double* pooled = (double*)workspace;
    const dim3 pool_grid((unsigned)((int64_t)2 * B * nB * H));
    if (D == 128) {
        hipLaunchKernelGGL((pool_kernel<128>), pool_grid, dim3(kThreads), 0, stream, (const uint4*)q,
                           (const uint4*)k, pooled, S, H, block, nB);
    } else {
        hipLaunchKernelGGL((pool_kernel<64>), pool_grid, dim3(kThreads), 0, stream, (const uint4*)q,
                           (const uint4*)k, pooled, S, H, block, nB);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_select_from_pooled(B, S, H, D, block, kept, mask, workspace, stream);
}

}  // namespace saq
