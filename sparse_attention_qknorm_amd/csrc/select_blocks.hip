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
// Kernels:
//  1. pool:   one workgroup per (tensor, b, block, head); 16-byte loads of the
//             block's rows, fp64 sums. The inputs are bf16 with |x| < 16 and,
//             when non-zero, |x| >= 2^-35, so every partial sum is exact in
//             fp64 and the result does not depend on the reduction order.
//             HBM-bound: 4*D bytes per (token, head).
//  2. nB <= 1024 (every shape of the layer up to 131,072 tokens at block 128):
//     transpose: the pooled k means go to [b,h][d][nBpad] (zeros past nB), so
//             a wavefront reading one d of 256 consecutive key blocks reads
//             2 KB of contiguous memory.
//     select_fused: one workgroup per (b, h, strip of 16/32/64 query rows)
//             computes the strip's scores against every key block in fp64
//             vector ALU (16 rows x 4 keys per thread; query means broadcast
//             from LDS, key means straight from the transposed copy), keeps
//             the upper 32 bits of each score's order key in LDS, and then
//             each wavefront selects its rows there: a bitwise search over the
//             32-bit keys, counting with wave ballots, finds the upper half T
//             of the (k-1)-th largest key; keys above T are kept; when keys
//             sharing T must be split, only those scores are recomputed in
//             full (same canonical order) and the search goes on over their
//             lower 32 bits, ties going to the lower j. The mask row is
//             written straight from the ballots; nothing of size nB^2 goes
//             through memory except the mask itself.
//  3. nB > 1024 (up to 4096):
//     scores: per (b, h) a tiled nB x nB product of the pooled vectors in fp64
//             vector ALU (128x128 tile per workgroup, 8x8 per thread, pooled
//             vectors staged in LDS by 16-wide d slices). The scores leave as
//             uint64 keys whose unsigned order is the fp64 order.
//     topk:   one wavefront per query-block row; the row's keys sit in
//             registers; the same bitwise search (32 steps on the upper halves,
//             32 more only when keys tie there).
// Contraction into FMA is switched off in every score loop, so each product and
// each sum rounds on its own, in the order of the definition, and every path
// produces the same scores bit for bit.
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

// ---------------------------------------------------------------- fused scores + top-k (nB <= 1024)

constexpr int kFusedMaxBlocks = 1024;

__host__ __device__ constexpr int fused_pad(int nB) { return nB <= 256 ? 256 : nB <= 512 ? 512 : 1024; }

// pk [bh][nB][D] -> pkT [bh][D][nBpad], zeros for j >= nB. 32 x 32 tiles of doubles through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void transpose_pk_kernel(const double* __restrict__ pk,
                                                                double* __restrict__ pkT, int32_t nB,
                                                                int32_t nBpad, const double* __restrict__ gate) {
    __shared__ double tile[32][33];
    if (gate != nullptr && *gate == 0.0) return;
    constexpr int kDTiles = D / 32;
    const int jtiles = nBpad / 32;
    const int64_t bh = blockIdx.x / ((int64_t)jtiles * kDTiles);
    const int rem = (int)(blockIdx.x % ((int64_t)jtiles * kDTiles));
    const int j0 = (rem / kDTiles) * 32;
    const int d0 = (rem % kDTiles) * 32;
    const int tx = threadIdx.x % 32;
    const int ty = threadIdx.x / 32;
    const double* src = pk + bh * (int64_t)nB * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = j0 + ty + 8 * r;
        tile[ty + 8 * r][tx] = j < nB ? src[(int64_t)j * D + d0 + tx] : 0.0;
    }
    __syncthreads();
    double* dst = pkT + bh * (int64_t)D * nBpad;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(int64_t)(d0 + ty + 8 * r) * nBpad + j0 + tx] = tile[tx][ty + 8 * r];
}

// Exact fp64 score of (query mean x in LDS, key mean y in memory) in the canonical order.
template <int D>
__device__ __forceinline__ double canonical_score(const double* x, const double* __restrict__ y) {
#pragma clang fp contract(off)
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
        const double prod = x[d] * y[d];
        s = s + prod;
    }
    return s;
}

// Workgroup of 4 wavefronts; WR row groups of 16 query rows x (4 / WR) key groups of 256 key blocks.
// Lane l of a wavefront holds 16 rows x key blocks 256*kg + 4l .. 4l+3.
template <int D, int WR>
__global__ __launch_bounds__(kThreads, WR == 1 ? 2 : 1) void select_fused_kernel(const double* __restrict__ pq,
                                                                   const double* __restrict__ pk,
                                                                   const double* __restrict__ pkT,
                                                                   uint8_t* __restrict__ mask, int32_t nB,
                                                                   int32_t kept, const double* __restrict__ gate) {
#pragma clang fp contract(off)
    constexpr int WK = 4 / WR;
    constexpr int kRows = 16 * WR;
    constexpr int kPad = 256 * WK;                       // key columns held (nBpad)
    constexpr int kM = kPad / kWave;                     // keys per lane in the selection
    __shared__ __attribute__((aligned(16))) double xq[kRows * D];
    __shared__ __attribute__((aligned(16))) uint32_t keys[kRows * kPad];
    if (gate != nullptr && *gate == 0.0) return;        // the mask of an earlier step is kept

    const int strips = (nB + kRows - 1) / kRows;
    const int64_t bh = blockIdx.x / strips;
    const int i0 = (int)(blockIdx.x % strips) * kRows;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;

    // the strip's query means (zeros past nB)
    {
        const double2* src = (const double2*)(pq + (bh * nB + i0) * (int64_t)D);
        double2* dst = (double2*)xq;
        const int valid = min(kRows, nB - i0) * D / 2;
        for (int e = tid; e < kRows * D / 2; e += kThreads) dst[e] = e < valid ? src[e] : make_double2(0.0, 0.0);
    }
    __syncthreads();

    // ---- scores: 16 rows x 4 key blocks per lane, d ascending, no FMA
    {
        const int rg = wave / WK;
        const int kg = wave % WK;
        const int jb = 256 * kg + 4 * lane;
        const double* yp = pkT + bh * (int64_t)D * kPad + jb;
        const double* xr = xq + 16 * rg * D;
        double acc[16][4];
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] = 0.0;
        double2 ya[2][2], yb[2][2];                      // [d of the pair][key pair]
        auto load_y = [&](int d, double2 (&y)[2][2]) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                y[u][0] = *(const double2*)(yp + (int64_t)(d + u) * kPad);
                y[u][1] = *(const double2*)(yp + (int64_t)(d + u) * kPad + 2);
            }
        };
        auto fma_free = [&](int d, const double2 (&y)[2][2]) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const double2 x = *(const double2*)(xr + r * D + d);    // LDS broadcast: x[r][d], x[r][d+1]
                const double yv0[4] = {y[0][0].x, y[0][0].y, y[0][1].x, y[0][1].y};
                const double yv1[4] = {y[1][0].x, y[1][0].y, y[1][1].x, y[1][1].y};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double p0 = x.x * yv0[e];
                    acc[r][e] = acc[r][e] + p0;
                    const double p1 = x.y * yv1[e];
                    acc[r][e] = acc[r][e] + p1;
                }
            }
        };
        load_y(0, ya);
        for (int d = 0; d < D; d += 4) {
            load_y(d + 2, yb);
            fma_free(d, ya);
            if (d + 4 < D) load_y(d + 4, ya);
            fma_free(d + 2, yb);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            uint4 w;
            w.x = (uint32_t)(order_key(acc[r][0]) >> 32);
            w.y = (uint32_t)(order_key(acc[r][1]) >> 32);
            w.z = (uint32_t)(order_key(acc[r][2]) >> 32);
            w.w = (uint32_t)(order_key(acc[r][3]) >> 32);
            *(uint4*)(keys + (16 * rg + r) * kPad + jb) = w;
        }
    }
    __syncthreads();

    // ---- selection: wavefront w takes rows w, w+4, ...
    const uint64_t below = (1ull << lane) - 1ull;
    const int need = kept - 1;                           // blocks chosen besides the diagonal
    for (int r = wave; r < kRows; r += 4) {
        const int i = i0 + r;
        if (i >= nB) break;
        // valid keys are >= 2^20 (finite scores); 0 marks j >= nB and the diagonal
        uint32_t key[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const int j = lane + kWave * m;
            key[m] = (j < nB && j != i) ? keys[r * kPad + j] : 0u;
        }
        uint32_t T = 0xffffffffu;                        // need == 0: nothing passes key >= T + 1
        bool all_eq = true;                              // every key equal to T is kept
        uint32_t tied = 0;                               // bit m: key[m] == T and must be split
        uint32_t lo[kM];
        uint32_t Tlo = 0;
        int eq_take = 0;
        if (need > 0) {
            T = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int cnt = 0;
#pragma unroll
                for (int m = 0; m < kM; ++m) cnt += __popcll(__ballot(key[m] >= cand));
                if (cnt >= need) T = cand;
            }
            int gt = 0, eq = 0;
#pragma unroll
            for (int m = 0; m < kM; ++m) {
                gt += __popcll(__ballot(key[m] > T));
                eq += __popcll(__ballot(key[m] == T));
            }
            const int take = need - gt;                  // 1 <= take <= eq
            if (take < eq) {
                // split the keys whose upper halves equal T by their full fp64 scores
                all_eq = false;
                const double* pkh = pk + bh * (int64_t)nB * D;
#pragma unroll
                for (int m = 0; m < kM; ++m) {
                    lo[m] = 0;
                    if (key[m] == T) {
                        tied |= 1u << m;
                        lo[m] = (uint32_t)order_key(canonical_score<D>(xq + r * D, pkh + (int64_t)(lane + kWave * m) * D));
                    }
                }
                // largest Tlo with #(tied keys with lo >= Tlo) >= take (Tlo = 0 always qualifies)
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t cand = Tlo | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int m = 0; m < kM; ++m) cnt += __popcll(__ballot(((tied >> m) & 1u) && lo[m] >= cand));
                    if (cnt >= take) Tlo = cand;
                }
                int gt_lo = 0;
#pragma unroll
                for (int m = 0; m < kM; ++m) gt_lo += __popcll(__ballot(((tied >> m) & 1u) && lo[m] > Tlo));
                eq_take = take - gt_lo;
            }
        }
        uint8_t* mrow = mask + (bh * nB + i) * (int64_t)nB;
        int taken = 0;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const int j = lane + kWave * m;
            bool sel;
            if (all_eq) {
                sel = key[m] != 0u && key[m] >= T && need > 0;
            } else {
                const bool t = (tied >> m) & 1u;
                const uint64_t eqb = __ballot(t && lo[m] == Tlo);
                const int before = taken + __popcll(eqb & below);
                taken += __popcll(eqb);
                sel = key[m] > T || (t && (lo[m] > Tlo || (lo[m] == Tlo && before < eq_take)));
            }
            if (j < nB) mrow[j] = (uint8_t)((sel || j == i) ? 1 : 0);
        }
    }
}

template <int D>
hipError_t launch_fused(const double* pq, const double* pk, double* pkT, uint8_t* mask, int32_t B, int32_t H,
                        int32_t nB, int32_t kept, const double* gate, hipStream_t stream) {
    const int nBpad = fused_pad(nB);
    const int64_t BH = (int64_t)B * H;
    hipLaunchKernelGGL((transpose_pk_kernel<D>), dim3((unsigned)(BH * (nBpad / 32) * (D / 32))), dim3(kThreads), 0,
                       stream, pk, pkT, nB, nBpad, gate);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int WR = 1024 / nBpad;
    const int64_t strips = (nB + 16 * WR - 1) / (16 * WR);
    const dim3 grid((unsigned)(BH * strips));
    if (WR == 1)
        hipLaunchKernelGGL((select_fused_kernel<D, 1>), grid, dim3(kThreads), 0, stream, pq, pk, pkT, mask, nB, kept,
                           gate);
    else if (WR == 2)
        hipLaunchKernelGGL((select_fused_kernel<D, 2>), grid, dim3(kThreads), 0, stream, pq, pk, pkT, mask, nB, kept,
                           gate);
    else
        hipLaunchKernelGGL((select_fused_kernel<D, 4>), grid, dim3(kThreads), 0, stream, pq, pk, pkT, mask, nB, kept,
                           gate);
    return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(int64_t B, int64_t H, int64_t nB, int64_t D) {
    const size_t pooled = ((size_t)2 * B * H * nB * D * sizeof(double) + 255) / 256 * 256;
    // nB <= 1024: the transposed pooled k means [B,H][D][nBpad]; beyond: the uint64 score keys [B,H,nB,nB]
    const size_t tail = nB <= kFusedMaxBlocks ? (size_t)B * H * D * fused_pad((int)nB) * sizeof(double)
                                              : (size_t)B * H * nB * nB * sizeof(uint64_t);
    return pooled + tail;
}

hipError_t launch_select_from_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                                     uint8_t* mask, void* workspace, hipStream_t stream, const double* gate) {
    const int32_t nB = (S + block - 1) / block;
    const double* pq = (const double*)workspace;
    const double* pk = pq + (size_t)B * H * nB * D;
    const size_t pooled_bytes = ((size_t)2 * B * H * nB * D * sizeof(double) + 255) / 256 * 256;
    void* tail = (char*)workspace + pooled_bytes;

    if (nB <= kFusedMaxBlocks) {
        return D == 128 ? launch_fused<128>(pq, pk, (double*)tail, mask, B, H, nB, kept, gate, stream)
                        : launch_fused<64>(pq, pk, (double*)tail, mask, B, H, nB, kept, gate, stream);
    }
    uint64_t* keys = (uint64_t*)tail;
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
    if (nB <= 2048) launch_topk<32>(keys, mask, nB, rows, kept, gate, stream);
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
