// Block-sparse flash attention for gfx950 (bf16 MFMA, fp32 online softmax).
//
// Sol-Attn paragraph of the Sol Engine "H3 on device" page: attention over the
// joint video+audio sequence computes only the (query block, key block) tiles
// that the selection keeps, inside an online-softmax pass.
//
// One workgroup per (b, h, query block i); BLOCK/32 wavefronts, each owning 32
// query rows. For every kept key block j (ascending):
//   S^T = K_j Q_i^T    v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q^T held in
//                      registers for the whole loop;
//   online softmax     each lane holds one query row (lane % 32) and half of the
//                      keys of every 32-key tile, so row maxima and sums are
//                      lane-local plus one exchange with lane ^ 32;
//   O^T += V_j^T P^T   A = V^T from LDS, B = P^T re-packed from the S^T
//                      accumulators without any data movement: the key order
//                      inside a 16-key MFMA step is permuted to match the
//                      accumulator layout, and V is staged in LDS with four
//                      consecutive keys interleaved per d ([key/4][d][4]) so
//                      each lane reads its keys with 8-byte loads.
// O^T accumulates with each lane holding its own query row, so the rescale by
// exp2(m_old - m_new) and the final 1/l are lane-local. Keys past S score -inf
// (and K/V rows past S are staged as zeros); rows past S are not stored.
// Workgroups are renumbered so every XCD (own L2) works through adjacent query
// blocks of the same head, whose kept key blocks overlap.
#include "common.h"
#include "kernels.h"

namespace saq {

namespace {

template <int BLOCK, int D>
struct AttnShape {
    static constexpr int kWaves = BLOCK / 32;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kKeyTiles = BLOCK / 32;        // 32-key tiles of S^T
    static constexpr int kDSteps = D / 16;              // k-steps of the QK^T product
    static constexpr int kDTiles = D / 32;              // 32-wide d tiles of O^T
    static constexpr int kKeySteps = BLOCK / 16;        // k-steps of the PV product
    static constexpr int kKPitch = D + 8;               // bf16 elements per staged K row (16 B pad)
    static constexpr int kVPitch = D * 4;               // bf16 elements per staged group of 4 keys
    static constexpr int kKChunks = BLOCK * D / 8;      // 16-byte chunks of a K tile
    static constexpr int kVUnits = (BLOCK / 4) * (D / 2);  // (4 keys x 2 d) units of a V tile
    static constexpr int kKPerThread = kKChunks / kThreads;
    static constexpr int kVPerThread = kVUnits / kThreads;
    static_assert(kThreads == BLOCK * 2, "launch bound of the kernel");
    static_assert(kKChunks % kThreads == 0 && kVUnits % kThreads == 0, "tile split");
};

template <int BLOCK, int D>
__global__ __launch_bounds__(BLOCK * 2) void block_sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint8_t* __restrict__ mask, uint16_t* __restrict__ o, int32_t S, int32_t H, int32_t nB,
    int64_t n_items, float scale_log2) {
    using Sh = AttnShape<BLOCK, D>;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BLOCK * Sh::kKPitch];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[(BLOCK / 4) * Sh::kVPitch];
    __shared__ uint16_t kept[kMaxBlocks];
    __shared__ int n_kept_s;

    const int64_t item = xcd_contiguous_index(blockIdx.x, n_items);
    const int i = (int)(item % nB);
    const int64_t bh = item / nB;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int g = lane / 32;

    // ---- compact the mask row into an ascending list of kept key blocks (wave 0)
    if (wave == 0) {
        const uint8_t* mrow = mask + item * (int64_t)nB;
        int count = 0;
        for (int j0 = 0; j0 < nB; j0 += kWave) {
            const int j = j0 + lane;
            const bool keep = j < nB && mrow[j] != 0;
            const uint64_t bits = __ballot(keep);
            if (keep) kept[count + __popcll(bits & ((1ull << lane) - 1ull))] = (uint16_t)j;
            count += __popcll(bits);
        }
        if (lane == 0) n_kept_s = count;
    }

    const int64_t row_stride = (int64_t)H * D;          // elements between consecutive tokens
    const int64_t head_off = b * (int64_t)S * row_stride + (int64_t)h * D;

    // ---- Q^T as the B operand: lane holds query row (32*wave + l32), d = 16*step + 8*g + [0..7]
    bf16x8 qb[Sh::kDSteps];
    {
        const int qrow = i * BLOCK + wave * 32 + l32;
        if (qrow < S) {
            const uint16_t* src = q + head_off + (int64_t)qrow * row_stride + 8 * g;
#pragma unroll
            for (int st = 0; st < Sh::kDSteps; ++st) qb[st] = *(const bf16x8*)(src + 16 * st);
        } else {
#pragma unroll
            for (int st = 0; st < Sh::kDSteps; ++st) qb[st] = (bf16x8){};
        }
    }

    f32x16 oacc[Sh::kDTiles];
#pragma unroll
    for (int t = 0; t < Sh::kDTiles; ++t) oacc[t] = (f32x16){};
    float m_run = -INFINITY;   // running max of the scaled (log2-domain) scores of this lane's row
    float l_run = 0.f;         // this lane's share of the row's softmax denominator

    __syncthreads();
    const int n_kept = n_kept_s;

    uint4 kreg[Sh::kKPerThread];
    uint32_t vreg[Sh::kVPerThread][4];

    auto load_tile = [&](int j) {
        const int key0 = j * BLOCK;
#pragma unroll
        for (int n = 0; n < Sh::kKPerThread; ++n) {
            const int c = tid + n * Sh::kThreads;
            const int r = c / (D / 8);
            const int ch = c % (D / 8);
            const int key = key0 + r;
            kreg[n] = key < S ? *(const uint4*)(k + head_off + (int64_t)key * row_stride + 8 * ch)
                              : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < Sh::kVPerThread; ++n) {
            const int u = tid + n * Sh::kThreads;
            const int dp = u % (D / 2);
            const int g4 = u / (D / 2);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 4 * g4 + r;
                vreg[n][r] = key < S ? *(const uint32_t*)(v + head_off + (int64_t)key * row_stride + 2 * dp) : 0u;
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int n = 0; n < Sh::kKPerThread; ++n) {
            const int c = tid + n * Sh::kThreads;
            const int r = c / (D / 8);
            const int ch = c % (D / 8);
            *(uint4*)(k_lds + r * Sh::kKPitch + 8 * ch) = kreg[n];
        }
#pragma unroll
        for (int n = 0; n < Sh::kVPerThread; ++n) {
            const int u = tid + n * Sh::kThreads;
            const int dp = u % (D / 2);
            const int g4 = u / (D / 2);
            const uint32_t* w = vreg[n];
            uint4 packed;
            packed.x = (w[0] & 0xffffu) | (w[1] << 16);            // d = 2dp, keys 0,1
            packed.y = (w[2] & 0xffffu) | (w[3] << 16);            // d = 2dp, keys 2,3
            packed.z = (w[0] >> 16) | (w[1] & 0xffff0000u);        // d = 2dp+1, keys 0,1
            packed.w = (w[2] >> 16) | (w[3] & 0xffff0000u);        // d = 2dp+1, keys 2,3
            *(uint4*)(v_lds + g4 * Sh::kVPitch + (2 * dp) * 4) = packed;
        }
    };

    if (n_kept > 0) load_tile(kept[0]);

    for (int n = 0; n < n_kept; ++n) {
        const int j = kept[n];
        __syncthreads();                       // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (n + 1 < n_kept) load_tile(kept[n + 1]);   // next tile's global loads overlap this tile's math

        // ---- S^T tile: rows = keys, cols = this wave's 32 query rows
        f32x16 sacc[Sh::kKeyTiles];
#pragma unroll
        for (int kt = 0; kt < Sh::kKeyTiles; ++kt) {
            sacc[kt] = (f32x16){};
            const uint16_t* krow = k_lds + (kt * 32 + l32) * Sh::kKPitch + 8 * g;
#pragma unroll
            for (int st = 0; st < Sh::kDSteps; ++st) {
                const bf16x8 a = *(const bf16x8*)(krow + 16 * st);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[st], sacc[kt], 0, 0, 0);
            }
        }

        // ---- online softmax (log2 domain); acc v of tile kt holds key 32kt + 8(v/4) + 4g + v%4
        const int key0 = j * BLOCK;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < Sh::kKeyTiles; ++kt)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int key = key0 + kt * 32 + 8 * (vv / 4) + 4 * g + (vv % 4);
                const float sv = key < S ? sacc[kt][vv] * scale_log2 : -INFINITY;
                sacc[kt][vv] = sv;
                mx = fmaxf(mx, sv);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);              // finite: every kept block has a valid key
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pb[Sh::kKeySteps];
#pragma unroll
        for (int ks = 0; ks < Sh::kKeySteps; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = exp2f(sacc[ks / 2][8 * (ks % 2) + e] - m_new);
                psum += p;
                pb[ks][e] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int t = 0; t < Sh::kDTiles; ++t) oacc[t] *= alpha;

        // ---- O^T += V^T P^T; k-index 8g + e of step ks is key 16ks + 8(e/4) + 4g + e%4
#pragma unroll
        for (int t = 0; t < Sh::kDTiles; ++t) {
            const int d = t * 32 + l32;
#pragma unroll
            for (int ks = 0; ks < Sh::kKeySteps; ++ks) {
                const uint16_t* vp = v_lds + (4 * ks + g) * Sh::kVPitch + d * 4;
                const bf16x4 lo = *(const bf16x4*)vp;
                const bf16x4 hi = *(const bf16x4*)(vp + 2 * Sh::kVPitch);
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[t], 0, 0, 0);
            }
        }
    }

    // ---- normalise and store: lane holds row l32 and d = 32t + 8(v/4) + 4g + v%4
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int qrow = i * BLOCK + wave * 32 + l32;
    if (qrow < S) {
        uint16_t* dst = o + head_off + (int64_t)qrow * row_stride;
#pragma unroll
        for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                uint2 w;
                w.x = f32_to_bf16_bits(oacc[t][4 * m + 0] * inv) | (f32_to_bf16_bits(oacc[t][4 * m + 1] * inv) << 16);
                w.y = f32_to_bf16_bits(oacc[t][4 * m + 2] * inv) | (f32_to_bf16_bits(oacc[t][4 * m + 3] * inv) << 16);
                *(uint2*)(dst + t * 32 + 8 * m + 4 * g) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// Production shape (block 128, head_dim 128): direct-to-LDS staging.
//
// K and V tiles (128 keys x 256 B) go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: no registers, asynchronous, and rows past S
// read as zeros through the buffer's range check. Each 16-byte chunk c of LDS
// row r sits at chunk position c ^ swz(r), an XOR swizzle under which both the
// 16-byte K reads (16 rows, one chunk) and the transposed V reads (4 rows x 4
// chunks) hit all 64 banks once.
//
// QK^T: lane (l32, g) reads K row pi(l32), pi swapping bits 2 and 3 of the row
// index, so accumulator v of 32-key tile kt holds key
// 32kt + 16(v/8) + 8g + 4((v/4)%2) + v%4: for 16-key step s = 2kt + a the
// registers 8a..8a+7 are exactly keys 16s + 8g + 0..7, the B operand of the PV
// MFMA in natural key order.
// PV: V^T is read with ds_read_b64_tr_b16. Within each 16-lane group, lane j
// supplies the 8 bytes at row kappa0 + j/4, columns d0 + 4(j%4); lane i then
// receives V[kappa0 + e][d0 + i] for e = 0..3. Two such reads give a lane its
// 8 keys for one d.
// Softmax in the log2 domain with a lazily updated maximum: the running max
// used in the exponent only moves (and O is only rescaled) when a tile's max
// exceeds it by more than 8, so p <= 2^8 and the rescale is almost never paid.
// Row sums use v_dot2 on the bf16 P, the same values the PV product consumes.
// Operand reads from LDS run one MFMA step ahead of the MFMAs that use them (the
// next d-step's K fragments, the next key step's V^T fragments), with the order
// pinned by scheduling-group barriers; the transposed-V read addresses are
// precomputed per lane (eight base offsets, the key step only adds 16 rows).
// Three workgroup barriers per tile: K_n landed; after QK^T, V_n landed and K_n
// released (the K_{n+1} copy is issued there, and softmax runs straight into
// PV without a barrier between them); after PV, V_n released (V_{n+1} issued).
// Folding the V wait into the post-QK^T barrier instead of a fourth barrier
// before PV was measured 4% faster with the same output bits. The QK^T MFMAs run
// at raised wavefront priority (s_setprio 1, back to 0 before the barrier): 0.9%
// faster; raising it in PV or softmax as well was slower.
namespace d128 {

constexpr int kBlock = 128;
constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kBlock * kRowBytes;               // 32 KB
constexpr int kLoadsPerWave = kTileBytes / 1024 / (kThreads / kWave);   // 8 x 1 KB per wave per tile
constexpr float kLazyRescale = 8.0f;                         // log2 units
constexpr int kXcdPeriod = 16;                               // query-block deal over the XCDs: runs of
constexpr int kXcdRun = 2;                                   // kXcdRun blocks, period kXcdPeriod = 8 runs

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// s_waitcnt with vmcnt <= n and the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The tile loop. The two LDS tiles come in as separate __restrict__ pointers:
// once inlined, the compiler's wait-count pass can then tell the K and V
// direct-to-LDS copies apart, so reading V does not wait for the K prefetch of
// the next tile.
__device__ __forceinline__ void tile_loop(uint8_t* __restrict__ k_lds, uint8_t* __restrict__ v_lds,
                                          const uint16_t* __restrict__ kept, int n_kept,
                                          const __amdgpu_buffer_rsrc_t& rk, const __amdgpu_buffer_rsrc_t& rv,
                                          uint32_t row_bytes_g, const bf16x8 (&qb)[kD / 16], int32_t S,
                                          float scale_log2, f32x16 (&oacc)[kD / 32], float& l_run) {
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int g = lane / 32;
    const int grp = lane / 16;
    const int jl = lane % 16;

    // staging: load n of this wave fills LDS bytes [C*1024, C*1024+1024), C = 8*wave + n,
    // i.e. rows 4C .. 4C+3; lane -> row 4C + lane/16 (row mod 16 = 4(n%4) + lane/16), chunk
    // position lane%16, which holds global chunk (lane%16) ^ swz(row)
    const uint32_t stage_row = (uint32_t)(4 * kLoadsPerWave * wave + lane / 16) * row_bytes_g;
    uint32_t stage_chunk[4];
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) stage_chunk[n4] = (uint32_t)(((lane % 16) ^ (((lane / 16) << 2) | n4)) * 16);
    auto issue_k = [&](int j) {
        const uint32_t tile_off = (uint32_t)j * (uint32_t)kBlock * row_bytes_g;
#pragma unroll
        for (int n = 0; n < kLoadsPerWave; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_void*)(k_lds + (kLoadsPerWave * wave + n) * 1024), 16,
                (int)(stage_row + stage_chunk[n % 4] + tile_off + (uint32_t)(4 * n) * row_bytes_g), 0, 0, 0);
    };
    auto issue_v = [&](int j) {
        const uint32_t tile_off = (uint32_t)j * (uint32_t)kBlock * row_bytes_g;
#pragma unroll
        for (int n = 0; n < kLoadsPerWave; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (lds_void*)(v_lds + (kLoadsPerWave * wave + n) * 1024), 16,
                (int)(stage_row + stage_chunk[n % 4] + tile_off + (uint32_t)(4 * n) * row_bytes_g), 0, 0, 0);
    };

    const int krow = swap_bits23(l32);                 // K row this lane feeds as A-operand row l32
    const int kfr = swz(krow);
    // byte offsets of this lane's transposed V reads: row 16s + 8g + 4hh + jl/4 and chunk 4t + .. of a tile;
    // the swizzle of those rows does not depend on s, so s only adds 16 rows (4096 bytes)
    uint32_t voff[2][kD / 32];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int t = 0; t < kD / 32; ++t) {
            const int r = 8 * g + 4 * hh + jl / 4;
            const int c = 4 * t + 2 * (grp % 2) + (jl % 4) / 2;
            voff[hh][t] = (uint32_t)(r * kRowBytes + ((c ^ swz(r)) * 16) + 8 * (jl % 2));
        }
    float m_used = -INFINITY;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    if (n_kept > 0) {
        issue_k(kept[0]);
        issue_v(kept[0]);
    }
    for (int n = 0; n < n_kept; ++n) {
        const int j = kept[n];
        const bool more = n + 1 < n_kept;
        wait_vmcnt<kLoadsPerWave>();                  // K_n landed (V_n may still be in flight)
        __syncthreads();

        f32x16 sacc[kBlock / 32];
#pragma unroll
        for (int kt = 0; kt < kBlock / 32; ++kt) sacc[kt] = (f32x16){};
        __builtin_amdgcn_s_setprio(1);                // QK^T issues ahead of the SIMD's other wavefront
        const uint8_t* krow_p = k_lds + krow * kRowBytes;
        // the next d-step's four K fragments are read while this step's four MFMAs run
        bf16x8 ka[2][kBlock / 32];
#pragma unroll
        for (int kt = 0; kt < kBlock / 32; ++kt)
            ka[0][kt] = *(const bf16x8*)(krow_p + kt * 32 * kRowBytes + ((0 + g) ^ kfr) * 16);
#pragma unroll
        for (int st = 0; st < kD / 16; ++st) {
            if (st + 1 < kD / 16) {
                const int c = (2 * (st + 1) + g) ^ kfr;
#pragma unroll
                for (int kt = 0; kt < kBlock / 32; ++kt)
                    ka[(st + 1) & 1][kt] = *(const bf16x8*)(krow_p + kt * 32 * kRowBytes + c * 16);
            }
#pragma unroll
            for (int kt = 0; kt < kBlock / 32; ++kt)      // four independent accumulators in turn
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1][kt], qb[st], sacc[kt], 0, 0, 0);
        }
        // pin the order: the first step's reads, then per step the next step's 4 reads before its 4 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < kD / 16; ++st) {
            if (st + 1 < kD / 16) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        wait_vmcnt<0>();                               // V_n landed
        __syncthreads();                               // ... and every wave is done with K_n
        if (more) issue_k(kept[n + 1]);

        // ---- softmax
        if ((j + 1) * kBlock > S) {                    // ragged last block: keys past S take no part
#pragma unroll
            for (int kt = 0; kt < kBlock / 32; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int key = j * kBlock + 32 * kt + 16 * (vv / 8) + 8 * g + 4 * ((vv / 4) % 2) + vv % 4;
                    if (key >= S) sacc[kt][vv] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < kBlock / 32; ++kt)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) mx = fmaxf(mx, sacc[kt][vv]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * scale_log2;
        const bool grow = mt > m_used + kLazyRescale;
        if (__ballot(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_used - mt) : 1.0f;
            m_used = grow ? mt : m_used;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < kD / 32; ++t) oacc[t] *= alpha;
        }
        bf16x8 pb[kBlock / 16];
#pragma unroll
        for (int s = 0; s < kBlock / 16; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pb[s][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[s / 2][8 * (s % 2) + e], scale_log2, -m_used));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 t2 = {pb[s][2 * e], pb[s][2 * e + 1]};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(t2, ones, l_run, false);
            }
        }

        // ---- O^T += V^T P^T
        // the next key step's four V^T fragments are read while this step's four MFMAs run
        bf16x4 va[2][kD / 32][2];
#pragma unroll
        for (int t = 0; t < kD / 32; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                va[0][t][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(v_lds + voff[hh][t]));
#pragma unroll
        for (int s = 0; s < kBlock / 16; ++s) {
            if (s + 1 < kBlock / 16) {
#pragma unroll
                for (int t = 0; t < kD / 32; ++t)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        va[(s + 1) & 1][t][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (lds_bf16x4*)(v_lds + voff[hh][t] + 16 * (s + 1) * kRowBytes));
            }
#pragma unroll
            for (int t = 0; t < kD / 32; ++t) {              // four independent accumulators in turn
                const bf16x8 a = __builtin_shufflevector(va[s & 1][t][0], va[s & 1][t][1], 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], oacc[t], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
        for (int s = 0; s < kBlock / 16; ++s) {
            if (s + 1 < kBlock / 16) __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
        }
        __syncthreads();                               // every wave is done with V_n
        if (more) issue_v(kept[n + 1]);
    }
}

// In-kernel block selection (the selection folded into the attention pass):
// the pooled fp64 block means of q-hat and k-hat, the number of kept blocks per
// row, and an optional mask to write the chosen row into.
struct SelectArgs {
    const double* pq;        // [B][H][nB][D]
    const double* pk;        // [B][H][nB][D]
    int32_t kept;            // k: kept key blocks per query block, the diagonal included
    uint8_t* mask_out;       // [B][H][nB][nB] or null
};

__device__ __forceinline__ uint64_t score_order_key(double s) {
    uint64_t u = __double_as_longlong(s);
    if (u == 0x8000000000000000ull) u = 0;                      // -0.0 ranks as +0.0
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Selects the kept key blocks of query block i of head bh into kept[0 .. n): the
// diagonal plus the k-1 largest scores s_ij = sum_d pq_i[d] * pk_j[d] over j != i
// (fp64, d ascending, each product and sum rounded: the selection's canonical
// order), ties to the lower j; the same rule, order and result as the separate
// score and top-k kernels. keys: kMaxBlocks uint64 of LDS scratch. The caller
// synchronises the workgroup before reading kept / n_kept.
__device__ __forceinline__ void select_row(const SelectArgs& a, int64_t bh, int i, int nB, uint64_t* keys,
                                           uint16_t* kept, int* n_kept) {
#pragma clang fp contract(off)
    const double* pqi = a.pq + (bh * nB + i) * kD;
    const double* pkh = a.pk + bh * nB * (int64_t)kD;
    for (int j = threadIdx.x; j < nB; j += kThreads) {
        const double2* pkj = (const double2*)(pkh + (int64_t)j * kD);
        double s = 0.0;
#pragma unroll 8
        for (int d2 = 0; d2 < kD / 2; ++d2) {
            const double2 y = pkj[d2];
            const double p0 = pqi[2 * d2] * y.x;
            s = s + p0;
            const double p1 = pqi[2 * d2 + 1] * y.y;
            s = s + p1;
        }
        keys[j] = score_order_key(s);
    }
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    const int need = a.kept - 1;                        // blocks chosen besides the diagonal
    uint64_t T = ~0ull;                                 // need == 0: nothing passes key > T
    int eq_take = 0;
    if (need > 0) {
        // largest T with #(valid keys >= T) >= need, bit by bit from the top
        T = 0;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t cand = T | (1ull << bit);
            int cnt = 0;
            for (int j0 = 0; j0 < nB; j0 += kWave) {
                const int j = j0 + lane;
                cnt += __popcll(__ballot(j < nB && j != i && keys[j] >= cand));
            }
            if (cnt >= need) T = cand;
        }
        int gt = 0;
        for (int j0 = 0; j0 < nB; j0 += kWave) {
            const int j = j0 + lane;
            gt += __popcll(__ballot(j < nB && j != i && keys[j] > T));
        }
        eq_take = need - gt;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    uint8_t* mrow = a.mask_out ? a.mask_out + (bh * nB + i) * (int64_t)nB : nullptr;
    int taken = 0, count = 0;
    for (int j0 = 0; j0 < nB; j0 += kWave) {
        const int j = j0 + lane;
        const bool valid = j < nB && j != i;
        const uint64_t key = j < nB ? keys[j] : 0;
        const uint64_t eq = __ballot(valid && key == T);
        const int before = taken + __popcll(eq & below);
        const bool chosen = valid && (key > T || (key == T && before < eq_take));
        taken += __popcll(eq);
        const bool keep = chosen || j == i;
        if (mrow && j < nB) mrow[j] = keep ? 1 : 0;
        const uint64_t bits = __ballot(keep);
        if (keep) kept[count + __popcll(bits & below)] = (uint16_t)j;
        count += __popcll(bits);
    }
    if (lane == 0) *n_kept = count;
}

template <bool kSelect>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint8_t* __restrict__ mask, uint16_t* __restrict__ o, int32_t S, int32_t H, int32_t nB,
    int64_t n_items, float scale_log2, uint32_t head_bytes, SelectArgs sel) {
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds[kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds[kTileBytes];
    __shared__ uint16_t kept[kMaxBlocks];
    __shared__ int n_kept_s;

    // Hardware deals workgroup ids round-robin over the 8 XCDs. All XCDs work on one
    // (b, h) at a time, so that head's K and V stay resident in the memory-side cache.
    // Within it, XCD x takes the query blocks i with (i mod kXcdPeriod) / kXcdRun == x in
    // ascending order: runs of two adjacent blocks dealt round-robin. Measured against
    // giving each XCD one contiguous range of the head, this is 1.5% faster at the full
    // layer with bit-identical outputs (a replay of the kept lists through a 4 MB LRU per
    // XCD puts the L2 hit rate at 56-59% against 42-48%).
    const int per = (nB + kXcdPeriod - 1) / kXcdPeriod * kXcdRun;
    const int64_t slot = blockIdx.x / kNumXcd;
    const int run = (int)(slot % per);
    const int i = (run / kXcdRun) * kXcdPeriod + (int)(blockIdx.x % kNumXcd) * kXcdRun + run % kXcdRun;
    if (i >= nB) return;                               // ragged split: whole workgroup leaves
    const int64_t bh = slot / per;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int64_t item = bh * nB + i;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int g = lane / 32;

    if constexpr (kSelect) {
        // the K tile's LDS is free until the tile loop: it holds the row's score keys
        select_row(sel, bh, i, nB, (uint64_t*)k_lds, kept, &n_kept_s);
    } else if (wave == 0) {
        const uint8_t* mrow = mask + item * (int64_t)nB;
        int count = 0;
        for (int j0 = 0; j0 < nB; j0 += kWave) {
            const int j = j0 + lane;
            const bool keep = j < nB && mrow[j] != 0;
            const uint64_t bits = __ballot(keep);
            if (keep) kept[count + __popcll(bits & ((1ull << lane) - 1ull))] = (uint16_t)j;
            count += __popcll(bits);
        }
        if (lane == 0) n_kept_s = count;
    }

    const int64_t row_stride = (int64_t)H * kD;                 // elements
    const uint32_t row_bytes_g = (uint32_t)(row_stride * 2);    // bytes between tokens
    const int64_t head_off = b * (int64_t)S * row_stride + (int64_t)h * kD;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + head_off), (short)0,
                                                                         (int)head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + head_off), (short)0,
                                                                         (int)head_bytes, 0x00020000);

    // Q^T as the B operand: row 32*wave + l32 of the block, d = 16*st + 8g + [0..7]
    bf16x8 qb[kD / 16];
    const int qrow = i * kBlock + wave * 32 + l32;
    if (qrow < S) {
        const uint16_t* src = q + head_off + (int64_t)qrow * row_stride + 8 * g;
#pragma unroll
        for (int st = 0; st < kD / 16; ++st) qb[st] = *(const bf16x8*)(src + 16 * st);
    } else {
#pragma unroll
        for (int st = 0; st < kD / 16; ++st) qb[st] = (bf16x8){};
    }

    f32x16 oacc[kD / 32];
#pragma unroll
    for (int t = 0; t < kD / 32; ++t) oacc[t] = (f32x16){};
    float l_run = 0.f;

    __syncthreads();
    tile_loop(k_lds, v_lds, kept, n_kept_s, rk, rv, row_bytes_g, qb, S, scale_log2, oacc, l_run);

    // ---- normalise and store: lane holds row l32 and d = 32t + 8(v/4) + 4g + v%4
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < S) {
        uint16_t* dst = o + head_off + (int64_t)qrow * row_stride;
#pragma unroll
        for (int t = 0; t < kD / 32; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                uint2 w;
                w.x = f32_to_bf16_bits(oacc[t][4 * m + 0] * inv) | (f32_to_bf16_bits(oacc[t][4 * m + 1] * inv) << 16);
                w.y = f32_to_bf16_bits(oacc[t][4 * m + 2] * inv) | (f32_to_bf16_bits(oacc[t][4 * m + 3] * inv) << 16);
                *(uint2*)(dst + t * 32 + 8 * m + 4 * g) = w;
            }
    }
}

template <bool kSelect>
hipError_t launch_t(const void* q, const void* k, const void* v, const uint8_t* mask, int32_t B, int32_t S, int32_t H,
                    float scale, void* o, const SelectArgs& sel, hipStream_t stream) {
    const int32_t nB = (S + kBlock - 1) / kBlock;
    const int64_t n_items = (int64_t)B * H * nB;
    const int per = (nB + kXcdPeriod - 1) / kXcdPeriod * kXcdRun;
    const int64_t n_groups = (int64_t)B * H * per * kNumXcd;
    const float scale_log2 = scale * 1.4426950408889634f;
    // bytes of one head's rows within one batch entry, up to the end of row S-1
    const uint64_t head_bytes = ((uint64_t)(S - 1) * H * kD + kD) * 2;
    hipLaunchKernelGGL(attn_kernel<kSelect>, dim3((unsigned)n_groups), dim3(kThreads), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, mask, (uint16_t*)o, S, H, nB,
                       n_items, scale_log2, (uint32_t)head_bytes, sel);
    return hipGetLastError();
}

hipError_t launch(const void* q, const void* k, const void* v, const uint8_t* mask, int32_t B, int32_t S, int32_t H,
                  float scale, void* o, hipStream_t stream) {
    return launch_t<false>(q, k, v, mask, B, S, H, scale, o, SelectArgs{nullptr, nullptr, 0, nullptr}, stream);
}

}  // namespace d128

template <int BLOCK, int D>
hipError_t launch_impl(const void* q, const void* k, const void* v, const uint8_t* mask, int32_t B, int32_t S,
                       int32_t H, float scale, void* o, hipStream_t stream) {
    using Sh = AttnShape<BLOCK, D>;
    const int32_t nB = (S + BLOCK - 1) / BLOCK;
    const int64_t n_items = (int64_t)B * H * nB;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((block_sparse_attn_kernel<BLOCK, D>), dim3((unsigned)n_items), dim3(Sh::kThreads), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, mask, (uint16_t*)o, S, H, nB,
                       n_items, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_sparse_attn_select(const void* q, const void* k, const void* v, const double* pooled,
                                           int32_t B, int32_t S, int32_t H, int32_t kept, float scale, void* o,
                                           uint8_t* mask_out, hipStream_t stream) {
    const int64_t nB = (S + d128::kBlock - 1) / d128::kBlock;
    const d128::SelectArgs sel{pooled, pooled + (int64_t)B * H * nB * d128::kD, kept, mask_out};
    return d128::launch_t<true>(q, k, v, nullptr, B, S, H, scale, o, sel, stream);
}

hipError_t launch_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* mask,
                                    int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                                    float scale, void* o, hipStream_t stream) {
    if (block == 128 && D == 128) return d128::launch(q, k, v, mask, B, S, H, scale, o, stream);
    if (block == 128 && D == 64) return launch_impl<128, 64>(q, k, v, mask, B, S, H, scale, o, stream);
    if (block == 64 && D == 128) return launch_impl<64, 128>(q, k, v, mask, B, S, H, scale, o, stream);
    return launch_impl<64, 64>(q, k, v, mask, B, S, H, scale, o, stream);
}

}  // namespace saq
