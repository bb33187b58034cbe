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
//     limbs:  each pooled vector, scaled by a power of two, is split into four
//             int8 limbs (exact to 2^-30 of its scale) plus its exponent.
//     select_filtered: one workgroup per (b, h, strip of 32-128 query rows).
//             Exact integer MFMAs over the limbs give every score of the strip
//             to within a proven bound; they are kept as 32-bit fixed-point keys
//             in LDS. Each wavefront then selects its rows there: a bitwise
//             search (wave ballots) finds the threshold key to within 16
//             units; keys clear of the threshold by more than the bound are
//             decided by it, and only the few keys inside that band get their
//             canonical fp64 scores computed, which decide them exactly (ties
//             to the lower j). The mask row is written from the ballots;
//             nothing of size nB^2 goes through memory except the mask itself.
//  3. nB > 1024 (up to 4096):
//     scores: per (b, h) a tiled nB x nB product of the pooled vectors in fp64
//             vector ALU (128x128 tile per workgroup, 8x8 per thread, pooled
//             vectors staged in LDS by 16-wide d slices). The scores leave as
//             uint64 keys whose unsigned order is the fp64 order.
//     topk:   one wavefront per query-block row; the row's keys sit in
//             registers; a bitwise search with wave ballots (32 steps on the
//             upper halves, 32 more only when keys tie there).
// Contraction into FMA is switched off in every score loop, so each product and
// each sum rounds on its own, in the order of the definition, and every path
// produces the same scores bit for bit.
#include "common.h"
#include "kernels.h"
#include "stream_io.h"

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
        const uint4 raw = load_once(&x[((b * S + t) * H + h) * kLanesPerRow + lane]);
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

// ---------------------------------------------------------------- filtered selection (nB <= 1024)

constexpr int kFusedMaxBlocks = 1024;

__host__ __device__ constexpr int fused_pad(int nB) { return nB <= 256 ? 256 : nB <= 512 ? 512 : 1024; }

typedef int int32x4 __attribute__((ext_vector_type(4)));

constexpr int kLimbs = 4;
constexpr int kNoExp = -4096;             // exponent recorded for an all-zero vector
constexpr int kKeyFracBits = 27;          // approximate key = floor(score * 2^27) + 2^31
constexpr int kSearchLowBit = 4;          // the threshold search resolves key bits 31..4
// Twice the bound on |approximate - exact| score, in key units, rounded up (the bound is
// derived above select_filtered_kernel): 2 * 1.75 * 2^-23 * 2^27 = 56.
constexpr uint32_t kBand = 56;
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
// 16-row query tiles per wavefront in the score phase. Two would halve the key-limb reads but
// need 128 KB of keys per workgroup, one workgroup per CU: measured slower (0.26 vs 0.20 ms).
constexpr int kSelU = 1;

// pooled [2][BH][nB][D] fp64 -> limbs [2][BH][4][D/16][nBpad][16] int8 (16-byte pieces of the
// vectors, piece-major so that 16 consecutive blocks' pieces are 256 contiguous bytes, the shape
// of one MFMA operand load; zeros for j >= nB) and, for the k means, exponents [BH][nBpad].
// A vector x with max |x_d| = f 2^F (f in [1/2, 1)) is scaled to x~ = x 2^-(F+2), so |x~_d| < 1/4,
// and written as x~ = a1 2^-8 + a2 2^-15 + a3 2^-22 + a4 2^-29 + r: each a_n rounds what is left
// to the nearest integer (|a_n| <= 64) and |r| <= 2^-30. Every step is exact in fp64.
template <int D>
__global__ __launch_bounds__(kThreads) void limbs_kernel(const double* __restrict__ pooled, int8_t* __restrict__ limbs,
                                                         int32_t* __restrict__ kexp, int64_t BH, int32_t nB,
                                                         int32_t nBpad, const double* __restrict__ gate) {
    constexpr int kPer = 16;                             // elements per thread
    constexpr int kTpr = D / kPer;                       // threads per vector
    constexpr int kRowsPerWg = kThreads / kTpr;
    if (gate != nullptr && *gate == 0.0) return;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + threadIdx.x / kTpr;   // (tensor * BH + bh) * nBpad + j
    const int part = threadIdx.x % kTpr;
    const int64_t tbh = row / nBpad;
    const int j = (int)(row % nBpad);

    double x[kPer];
    if (j < nB) {
        const double2* src = (const double2*)(pooled + (tbh * nB + j) * (int64_t)D + part * kPer);
#pragma unroll
        for (int e = 0; e < kPer / 2; ++e) {
            const double2 v = src[e];
            x[2 * e] = v.x;
            x[2 * e + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kPer; ++e) x[e] = 0.0;
    }
    double mx = 0.0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) mx = fmax(mx, fabs(x[e]));
#pragma unroll
    for (int o = 1; o < kTpr; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o));
    int F = kNoExp;
    if (mx > 0.0) (void)frexp(mx, &F);
    const int up = mx > 0.0 ? 6 - F : 0;                 // y = x~ * 2^8 = x * 2^(6-F)

    uint32_t w[kLimbs][kPer / 4];
#pragma unroll
    for (int n = 0; n < kLimbs; ++n)
#pragma unroll
        for (int c = 0; c < kPer / 4; ++c) w[n][c] = 0u;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        double y = ldexp(x[e], up);
        const double a1 = rint(y);
        y = (y - a1) * 128.0;
        const double a2 = rint(y);
        y = (y - a2) * 128.0;
        const double a3 = rint(y);
        y = (y - a3) * 128.0;
        const double a4 = rint(y);
        const int sh = 8 * (e % 4);
        w[0][e / 4] |= ((uint32_t)(int)a1 & 0xffu) << sh;
        w[1][e / 4] |= ((uint32_t)(int)a2 & 0xffu) << sh;
        w[2][e / 4] |= ((uint32_t)(int)a3 & 0xffu) << sh;
        w[3][e / 4] |= ((uint32_t)(int)a4 & 0xffu) << sh;
    }
#pragma unroll
    for (int n = 0; n < kLimbs; ++n) {
        int8_t* dst = limbs + (((tbh * kLimbs + n) * kTpr + part) * nBpad + j) * (int64_t)kPer;
        *(uint4*)dst = make_uint4(w[n][0], w[n][1], w[n][2], w[n][3]);
    }
    if (tbh >= BH && part == 0) kexp[(tbh - BH) * nBpad + j] = F;
}

// Exact fp64 score in the canonical order, both means in LDS.
template <int D>
__device__ __forceinline__ double canonical_score_lds(const double* x, const double* y) {
#pragma clang fp contract(off)
    double s = 0.0;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
        const double prod = x[d] * y[d];
        s = s + prod;
    }
    return s;
}

// The same score with the key mean (block j of pk) in memory, as a plain call, for the rare wide
// bands; the address is formed here so that no per-slot pointer stays live in the caller.
template <int D>
__device__ __noinline__ double canonical_score_call(const double* x, const double* __restrict__ pk, int j) {
#pragma clang fp contract(off)
    const double* y = pk + (int64_t)j * D;
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
        const double prod = x[d] * y[d];
        s = s + prod;
    }
    return s;
}

// wavefront-wide reductions of the device library (DPP lane exchanges)
extern "C" __device__ int32_t __ockl_wfred_max_i32(int32_t);
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// One workgroup of 8 wavefronts per (b, h, strip of 16 * 8/KG query rows); nBpad = 128 * KG.
//
// Approximate scores. With the limbs above, P_nm = sum_d a_n[d] b_m[d] is an exact integer
// (v_mfma_i32_16x16x64_i8), and so is t 2^37 = sum over n + m <= 5 of P_nm 2^(7 (5 - n - m)):
// ten products, grouped by n + m into four int32 accumulators. Against x~ . y~, t leaves out the
// products with n + m >= 6 and the remainders r: per d at most 3 * 64 * 64 * 2^-44 +
// 2 * 64 * 64 * 2^-51 + 64 * 64 * 2^-58 + 2 * 2^-30 / 4 + 2^-60 < 1.5 * 2^-30, so
// |t - x~ . y~| < 1.5 * 2^-23 over 128 d. In the head's frame (each key's t times 2^(F_j - Fmax),
// Fmax the largest key exponent of the head: a power of two <= 1, so every row keeps its order)
// the key floor(t 2^(F_j - Fmax + 27)) + 2^31, an integer shift of t 2^37, is off the exact
// canonical fp64 score in the same frame (whose own rounding is below 128 * 2^-53 * 8 = 2^-43) by
// less than 1.5 * 2^-23 + 2^-26 (two key units) + 2^-43 < 1.75 * 2^-23: at most kBand / 2 units.
//
// Selection per row. A bitwise search with wave ballots, started below the bits all the row's keys
// share and narrowed to one key per lane once at most 64 keys remain in play, puts the (k-1)-th
// largest key K* in [T, T + 15]; the (k-1)-th largest exact score then lies within kBand / 2 of
// K*. Keys above T + 15 + kBand are therefore strictly above it (kept), keys below T - kBand
// strictly below it (dropped), whatever the ties. The keys left in the band number at least the
// picks still owed; when they number more, only their canonical fp64 scores are computed and the
// owed picks go to the largest, ties to the lower j (-0.0 equal to +0.0).
template <int D, int KG>
__global__ __launch_bounds__(kSelThreads, kSelU == 1 ? 4 : 2) void select_filtered_kernel(
    const double* __restrict__ pq, const double* __restrict__ pk, const int8_t* __restrict__ limbs,
    const int32_t* __restrict__ kexp, uint8_t* __restrict__ mask, int32_t nB, int32_t kept, int64_t BH,
    const double* __restrict__ gate) {
    constexpr int kPad = 128 * KG;                       // key columns held
    constexpr int kRows = 16 * kSelU * (kSelWaves / KG); // query rows per workgroup
    constexpr int kChunks = D / 64;
    constexpr int kParts = D / 16;                       // 16-byte pieces of a limb vector
    constexpr int kM = kPad / kWave;                     // keys per lane in the selection
    constexpr int kTiles = 8;                            // 16-key tiles per wavefront
    __shared__ __attribute__((aligned(16))) uint32_t keys[kRows * kPad];   // 64 KB: two workgroups per CU
    __shared__ __attribute__((aligned(16))) double xrow[kSelWaves][D];
    __shared__ uint32_t slot[kSelWaves][kWave];
    __shared__ int pick_s[kSelWaves][kWave];
    __shared__ int fmax_w[kSelWaves];
    if (gate != nullptr && *gate == 0.0) return;         // the mask of an earlier step is kept

    // Hardware deals workgroup ids round-robin over the 8 XCDs: XCD x takes heads x, x + 8, ... one
    // after another, all strips of a head together, so the head's key limbs (512 KB) are read from
    // that XCD's L2 by every strip.
    const int strips = (nB + kRows - 1) / kRows;
    const int64_t seq = blockIdx.x / kNumXcd;           // position in the XCD's sequence
    const int64_t bh = (seq / strips) * kNumXcd + blockIdx.x % kNumXcd;
    if (bh >= BH) return;
    const int i0 = (int)(seq % strips) * kRows;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int32_t* ke = kexp + bh * kPad;

    // ---- approximate keys: wavefront = kSelU 16-row query tiles x 128 key blocks
    {
        const int p = wave / KG;
        const int kg = wave % KG;
        const int lr = lane % 16;
        const int lg = lane / 16;
        const int8_t* ql = limbs + bh * kLimbs * (int64_t)kPad * D;
        const int8_t* kl = limbs + (BH + bh) * kLimbs * (int64_t)kPad * D;
        // operand loads first; the exponent reduction runs while they are in flight
        int32x4 qa[kSelU][kLimbs][kChunks];
#pragma unroll
        for (int u = 0; u < kSelU; ++u)
#pragma unroll
            for (int a = 0; a < kLimbs; ++a)
#pragma unroll
                for (int c = 0; c < kChunks; ++c)
                    qa[u][a][c] = *(const int32x4*)(ql + (size_t)(a * kParts + 4 * c) * kPad * 16 +
                                                    (uint32_t)((lg * kPad + i0 + 16 * (kSelU * p + u) + lr) * 16));
        // a tile's key limbs and exponent are loaded together, one tile ahead of their use
        // (uniform bases per limb piece plus one 32-bit lane offset, so the loads take scalar bases)
        auto load_k = [&](int t, int32x4 (&kb)[kLimbs][kChunks], int& f) {
            const int j = 128 * kg + 16 * t + lr;
            const uint32_t off = (uint32_t)((lg * kPad + j) * 16);
#pragma unroll
            for (int a = 0; a < kLimbs; ++a)
#pragma unroll
                for (int c = 0; c < kChunks; ++c)
                    kb[a][c] = *(const int32x4*)(kl + (size_t)(a * kParts + 4 * c) * kPad * 16 + off);
            f = ke[j];
        };
        int32x4 kb0[kLimbs][kChunks], kb1[kLimbs][kChunks];
        int f0, f1;
        load_k(0, kb0, f0);

        // the head's largest key exponent
        {
            int f = kNoExp;
            for (int j = tid; j < nB; j += kSelThreads) f = max(f, ke[j]);
            f = __ockl_wfred_max_i32(f);
            if (lane == 0) fmax_w[wave] = f;
        }
        __syncthreads();
        int fmax = fmax_w[0];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) fmax = max(fmax, fmax_w[w]);

        auto tile = [&](int t, const int32x4 (&kb)[kLimbs][kChunks], int fj) {
            int32x4 g[kSelU][kLimbs];                    // g[.][n]: limb pairs with index sum n (0-based)
#pragma unroll
            for (int u = 0; u < kSelU; ++u)
#pragma unroll
                for (int n = 0; n < kLimbs; ++n) g[u][n] = int32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
#pragma unroll
                for (int u = 0; u < kSelU; ++u)
#pragma unroll
                    for (int n = 0; n < kLimbs; ++n)
#pragma unroll
                        for (int a = 0; a <= n; ++a)
                            g[u][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[u][a][c], kb[n - a][c], g[u][n], 0, 0, 0);
            // output element r of lane l: row 4 * (l / 16) + r of the tile, key column l % 16
            const int j = 128 * kg + 16 * t + lr;
            const int shift = min(fmax - fj + 10, 63);    // t 2^37 -> t 2^(27 + F_j - Fmax); >= 10
#pragma unroll
            for (int u = 0; u < kSelU; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t t37 = ((int64_t)g[u][0][r] << 21) + ((int64_t)g[u][1][r] << 14) +
                                        ((int64_t)g[u][2][r] << 7) + (int64_t)g[u][3][r];
                    const int row = 16 * (kSelU * p + u) + 4 * lg + r;
                    keys[row * kPad + j] = (uint32_t)(int32_t)(t37 >> shift) ^ 0x80000000u;
                }
        };
#pragma unroll 1
        for (int t = 0; t < kTiles; t += 2) {
            load_k(t + 1, kb1, f1);
            tile(t, kb0, f0);
            if (t + 2 < kTiles) load_k(t + 2, kb0, f0);
            tile(t + 1, kb1, f1);
        }
    }
    __syncthreads();

    // ---- selection: wavefront w takes rows w, w + 8, ...
    const uint64_t below = (1ull << lane) - 1ull;
    const int need = kept - 1;                           // blocks chosen besides the diagonal
    for (int r = wave; r < kRows; r += kSelWaves) {
        const int i = i0 + r;
        if (i >= nB) break;
        // valid keys lie within 2^30 + 1 of 2^31 (|t| < 8); 0 marks j >= nB and the diagonal
        uint32_t key[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const int j = lane + kWave * m;
            const uint32_t v = keys[r * kPad + j];
            key[m] = (j < nB && j != i) ? v : 0u;
        }
        uint32_t pick = 0;                               // bit m: key block lane + 64 m is kept
        if (need > 0) {
            // bits shared by every valid key of the row
            uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
            for (int m = 0; m < kM; ++m) {
                kmax = max(kmax, key[m]);
                kmin = min(kmin, key[m] != 0u ? key[m] : 0xffffffffu);
            }
            kmax = __ockl_wfred_max_u32(kmax);
            kmin = __ockl_wfred_min_u32(kmin);
            // invariant: K* lies in [T, T + 2^(bit+1)); cT keys are >= T, cU keys >= T + 2^(bit+1)
            int bit = 31 - __clz((int)(kmin ^ kmax));     // -1 when all keys are equal
            uint32_t T = bit >= 31 ? 0u : bit < 0 ? kmin : (kmin & ~((2u << bit) - 1u));
            int cT = nB - 1, cU = 0;
            for (; bit >= kSearchLowBit && cT - cU > kWave; --bit) {
                const uint32_t cand = T | (1u << bit);
                uint64_t bl[kM];
#pragma unroll
                for (int m = 0; m < kM; ++m) bl[m] = __ballot(key[m] >= cand);
                int cnt = 0;
#pragma unroll
                for (int m = 0; m < kM; ++m) cnt += __popcll(bl[m]);
                if (cnt >= need) {
                    T = cand;
                    cT = cnt;
                } else {
                    cU = cnt;
                }
            }
            if (bit >= kSearchLowBit) {
                // at most 64 keys in [T, T + 2^(bit+1)): one per lane for the remaining bits
                const uint32_t width = bit >= 31 ? 0xffffffffu : (2u << bit) - 1u;
                int base = 0;
#pragma unroll
                for (int m = 0; m < kM; ++m) {
                    const bool in = key[m] != 0u && key[m] >= T && key[m] - T <= width;
                    const uint64_t bits = __ballot(in);
                    const int at = base + __popcll(bits & below);
                    if (in && at < kWave) slot[wave][at] = key[m];
                    base += __popcll(bits);
                }
                wave_sync_lds();
                const uint32_t ck = lane < base ? slot[wave][lane] : 0u;
                wave_sync_lds();
                const int above = cU;                    // keys above the gathered range
                for (; bit >= kSearchLowBit; --bit) {
                    const uint32_t cand = T | (1u << bit);
                    if (above + __popcll(__ballot(ck >= cand)) >= need) T = cand;
                }
            }
            const uint32_t hi = T + ((1u << kSearchLowBit) - 1u) + kBand;
            const uint32_t lo = T - kBand;
            uint32_t band = 0;
            int n_in = 0, n_band = 0;
#pragma unroll
            for (int m = 0; m < kM; ++m) {
                const bool in = key[m] > hi;
                const bool b = key[m] != 0u && key[m] >= lo && key[m] <= hi;
                pick |= (uint32_t)in << m;
                band |= (uint32_t)b << m;
                n_in += __popcll(__ballot(in));
                n_band += __popcll(__ballot(b));
            }
            const int take = need - n_in;                // 1 <= take <= n_band
            if (take == n_band) {
                pick |= band;
            } else {
                const double* xg = pq + (bh * nB + i) * (int64_t)D;     // the row's query mean
                const double* pkh = pk + bh * nB * (int64_t)D;
                if (n_band <= kWave) {
                    // gather the band's key blocks into one slot per lane, score them exactly, rank
                    int base = 0;
#pragma unroll
                    for (int m = 0; m < kM; ++m) {
                        const bool b = (band >> m) & 1u;
                        const uint64_t bits = __ballot(b);
                        const int at = base + __popcll(bits & below);
                        if (b && at < kWave) slot[wave][at] = (uint32_t)(lane + kWave * m);
                        base += __popcll(bits);
                    }
                    wave_sync_lds();
                    const int jj = lane < n_band ? (int)slot[wave][lane] : 0;
                    // The query mean goes to xrow, the band's key means kStage at a time to this row's
                    // key region (its keys are in registers by now); every load of a round is issued
                    // before the first store, then lane e scores band entry e from LDS.
                    constexpr int kStage = kPad * 4 / (D * 8);
                    double* ybuf = (double*)&keys[r * kPad];
                    const bool xl = 2 * lane < D;
                    double2 xv = make_double2(0.0, 0.0);
                    if (xl) xv = *(const double2*)(xg + 2 * lane);
                    uint64_t ek = 0;
                    for (int g0 = 0; g0 < n_band; g0 += kStage) {
                        const int cnt = min(kStage, n_band - g0);
                        double2 yv[kStage];
#pragma unroll
                        for (int s2 = 0; s2 < kStage; ++s2) {
                            const int js = __shfl(jj, min(g0 + s2, n_band - 1));    // past the band: a repeat
                            yv[s2] = xl ? *(const double2*)(pkh + (int64_t)js * D + 2 * lane) : make_double2(0.0, 0.0);
                        }
                        if (g0 == 0 && xl) *(double2*)&xrow[wave][2 * lane] = xv;
#pragma unroll
                        for (int s2 = 0; s2 < kStage; ++s2)
                            if (s2 < cnt && xl) *(double2*)&ybuf[s2 * D + 2 * lane] = yv[s2];
                        wave_sync_lds();
                        if (lane >= g0 && lane < g0 + cnt)
                            ek = order_key(canonical_score_lds<D>(xrow[wave], ybuf + (lane - g0) * D));
                        wave_sync_lds();
                    }
                    int rank = 0;
                    for (int e = 0; e < n_band; ++e) {
                        const uint32_t elo = __shfl((uint32_t)ek, e);
                        const uint32_t ehi = __shfl((uint32_t)(ek >> 32), e);
                        const int ej = __shfl(jj, e);
                        const uint64_t other = ((uint64_t)ehi << 32) | elo;
                        rank += (other > ek || (other == ek && ej < jj)) ? 1 : 0;
                    }
                    pick_s[wave][lane] = (lane < n_band && rank < take) ? 1 : 0;
                    wave_sync_lds();
                    base = 0;
#pragma unroll
                    for (int m = 0; m < kM; ++m) {
                        const bool b = (band >> m) & 1u;
                        const uint64_t bits = __ballot(b);
                        const int at = base + __popcll(bits & below);
                        if (b && at < kWave) pick |= (uint32_t)(pick_s[wave][at] != 0) << m;
                        base += __popcll(bits);
                    }
                } else {
                    // a wide band (many equal or nearly equal scores): exact keys for the whole band,
                    // a 64-bit bitwise search over them, ties to the lower j
                    for (int d = 2 * lane; d < D; d += 2 * kWave) *(double2*)&xrow[wave][d] = *(const double2*)(xg + d);
                    wave_sync_lds();
                    uint64_t ek[kM];
#pragma unroll
                    for (int m = 0; m < kM; ++m)
                        ek[m] = ((band >> m) & 1u)
                                    ? order_key(canonical_score_call<D>(xrow[wave], pkh, lane + kWave * m))
                                    : 0ull;
                    uint64_t T64 = 0;
                    for (int b64 = 63; b64 >= 0; --b64) {
                        const uint64_t cand = T64 | (1ull << b64);
                        int cnt = 0;
#pragma unroll
                        for (int m = 0; m < kM; ++m) cnt += __popcll(__ballot(((band >> m) & 1u) && ek[m] >= cand));
                        if (cnt >= take) T64 = cand;
                    }
                    int gt = 0;
#pragma unroll
                    for (int m = 0; m < kM; ++m) gt += __popcll(__ballot(((band >> m) & 1u) && ek[m] > T64));
                    const int eq_take = take - gt;
                    int taken = 0;
#pragma unroll
                    for (int m = 0; m < kM; ++m) {
                        const bool b = (band >> m) & 1u;
                        const uint64_t eqb = __ballot(b && ek[m] == T64);
                        const int before = taken + __popcll(eqb & below);
                        taken += __popcll(eqb);
                        if (b && (ek[m] > T64 || (ek[m] == T64 && before < eq_take))) pick |= 1u << m;
                    }
                }
                wave_sync_lds();
            }
        }
        uint8_t* mrow = mask + (bh * nB + i) * (int64_t)nB;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const int j = lane + kWave * m;
            if (j < nB) mrow[j] = (uint8_t)((((pick >> m) & 1u) != 0u || j == i) ? 1 : 0);
        }
    }
}

template <int D, int KG>
void launch_filtered_kg(const double* pq, const double* pk, const int8_t* limbs, const int32_t* kexp,
                        uint8_t* mask, int64_t BH, int32_t nB, int32_t kept, const double* gate,
                        hipStream_t stream) {
    constexpr int kRows = 16 * kSelU * (kSelWaves / KG);
    const int64_t strips = (nB + kRows - 1) / kRows;
    const int64_t groups = (BH + kNumXcd - 1) / kNumXcd * kNumXcd * strips;
    hipLaunchKernelGGL((select_filtered_kernel<D, KG>), dim3((unsigned)groups), dim3(kSelThreads), 0, stream,
                       pq, pk, limbs, kexp, mask, nB, kept, BH, gate);
}

template <int D>
hipError_t launch_filtered(const double* pq, void* tail, uint8_t* mask, int32_t B, int32_t H, int32_t nB,
                           int32_t kept, const double* gate, hipStream_t stream) {
    const int nBpad = fused_pad(nB);
    const int64_t BH = (int64_t)B * H;
    const double* pk = pq + BH * nB * D;
    int8_t* limbs = (int8_t*)tail;
    int32_t* kexp = (int32_t*)(limbs + (size_t)2 * BH * kLimbs * nBpad * D);
    constexpr int kRowsPerWg = kThreads / (D / 16);      // divides nBpad
    hipLaunchKernelGGL((limbs_kernel<D>), dim3((unsigned)(2 * BH * nBpad / kRowsPerWg)), dim3(kThreads), 0, stream,
                       pq, limbs, kexp, BH, nB, nBpad, gate);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (nBpad == 256) launch_filtered_kg<D, 2>(pq, pk, limbs, kexp, mask, BH, nB, kept, gate, stream);
    else if (nBpad == 512) launch_filtered_kg<D, 4>(pq, pk, limbs, kexp, mask, BH, nB, kept, gate, stream);
    else launch_filtered_kg<D, 8>(pq, pk, limbs, kexp, mask, BH, nB, kept, gate, stream);
    return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(int64_t B, int64_t H, int64_t nB, int64_t D) {
    const size_t pooled = ((size_t)2 * B * H * nB * D * sizeof(double) + 255) / 256 * 256;
    // nB <= 1024: int8 limbs [2][B,H][4][nBpad][D] + k exponents [B,H][nBpad] int32; beyond: the
    // uint64 score keys [B,H,nB,nB]
    const size_t tail = nB <= kFusedMaxBlocks
                            ? (size_t)B * H * fused_pad((int)nB) * ((size_t)2 * kLimbs * D + sizeof(int32_t))
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
        return D == 128 ? launch_filtered<128>(pq, tail, mask, B, H, nB, kept, gate, stream)
                        : launch_filtered<64>(pq, tail, mask, B, H, nB, kept, gate, stream);
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
