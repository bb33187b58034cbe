// Cross-step reuse of the block mask, and the measurements that gate it.
//
// Consecutive denoising steps produce very similar activations through most of
// the schedule (Sol Engine "H3 on device" page, cross-step cache paragraph: a
// cheap change detector on the first block's residual decides whether the rest
// is recomputed). Here the same idea gates the block selection: the pooled
// q-hat/k-hat block means fully determine the mask, so their relative change
// between two steps is the detector, and the mask overlap between steps measures
// what reuse would cost.
//
//  * mask_overlap: per (b, h), the number of (i, j) kept in both masks and the
//    number kept in the first (integer counts, exact).
//  * pooled_change: sum of squared differences of two pooled-vector sets and the
//    sum of squares of the first, in fp64, reduced in a fixed order (per-thread
//    strided sums, a fixed tree per workgroup, then one workgroup over the
//    per-workgroup partials), so the result is the same bits on every run.
//  * select_reuse: the gated selection. The change of the current pooled
//    vectors against those the mask in use was selected from decides on the
//    device whether the score and top-k kernels run (they read the decision and
//    return at once when the mask is kept), so a step loop needs no host
//    round trip; on a recompute the current pooled vectors become the new
//    reference.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace saq {

namespace {

constexpr int kThreads = 256;

constexpr int kOverlapSplit = 16;     // workgroups per (b, h) for the overlap counts

// high bit of each byte set iff that byte is non-zero
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
    return (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
}

__global__ void zero_counts_kernel(int64_t* __restrict__ counts, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) counts[e] = 0;
}

// grid (kOverlapSplit, B*H): workgroup g of head bh counts bytes [g*n/G, (g+1)*n/G) of that head's nB x nB
// bytes, 16 at a time where the address allows it, and adds its integer totals atomically (exact, so the
// result does not depend on the order).
__global__ __launch_bounds__(kThreads) void mask_overlap_kernel(const uint8_t* __restrict__ a,
                                                                const uint8_t* __restrict__ b, int64_t n_per_head,
                                                                int64_t* __restrict__ counts) {
    __shared__ int64_t red[2][kThreads / kWave];
    const int64_t bh = blockIdx.y;
    const int64_t lo = bh * n_per_head + n_per_head * blockIdx.x / kOverlapSplit;
    const int64_t hi = bh * n_per_head + n_per_head * (blockIdx.x + 1) / kOverlapSplit;
    int64_t both = 0, na = 0;
    // bytes up to the first 16-byte boundary (a and b share their alignment: same offsets, 16-aligned bases)
    const int64_t vlo = min(hi, (lo + 15) & ~(int64_t)15);
    const int64_t vhi = max(vlo, hi & ~(int64_t)15);
    for (int64_t e = lo + threadIdx.x; e < vlo; e += kThreads) {
        const bool x = a[e] != 0, y = b[e] != 0;
        na += x;
        both += x && y;
    }
    const uint4* a4 = (const uint4*)(a + vlo);
    const uint4* b4 = (const uint4*)(b + vlo);
    const int64_t n4 = (vhi - vlo) / 16;
    for (int64_t e = threadIdx.x; e < n4; e += kThreads) {
        const uint4 x = a4[e], y = b4[e];
        const uint32_t ax[4] = {x.x, x.y, x.z, x.w};
        const uint32_t by[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t nx = nonzero_bytes(ax[k]);
            na += __popc(nx);
            both += __popc(nx & nonzero_bytes(by[k]));
        }
    }
    for (int64_t e = vhi + threadIdx.x; e < hi; e += kThreads) {
        const bool x = a[e] != 0, y = b[e] != 0;
        na += x;
        both += x && y;
    }
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        both += __shfl_xor(both, off);
        na += __shfl_xor(na, off);
    }
    if (threadIdx.x % kWave == 0) {
        red[0][threadIdx.x / kWave] = both;
        red[1][threadIdx.x / kWave] = na;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t s0 = 0, s1 = 0;
        for (int w = 0; w < kThreads / kWave; ++w) {
            s0 += red[0][w];
            s1 += red[1][w];
        }
        atomicAdd((unsigned long long*)&counts[2 * bh], (unsigned long long)s0);
        atomicAdd((unsigned long long*)&counts[2 * bh + 1], (unsigned long long)s1);
    }
}

// fixed-order tree sum of one double per thread over a workgroup
__device__ double block_sum_fixed(double v, double* sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int s = kThreads / 2; s >= 1; s >>= 1) {
        if (threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + s];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void pooled_change_partial_kernel(const double* __restrict__ prev,
                                                                         const double* __restrict__ cur, int64_t n,
                                                                         double* __restrict__ partial) {
#pragma clang fp contract(off)
    __shared__ double sh[kThreads];
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    double d2 = 0.0, p2 = 0.0;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
        const double x = prev[e], y = cur[e];
        const double d = y - x;
        d2 = d2 + d * d;
        p2 = p2 + x * x;
    }
    const double sd = block_sum_fixed(d2, sh);
    const double sp = block_sum_fixed(p2, sh);
    if (threadIdx.x == 0) {
        partial[2 * blockIdx.x] = sd;
        partial[2 * blockIdx.x + 1] = sp;
    }
}

__global__ __launch_bounds__(kThreads) void pooled_change_final_kernel(const double* __restrict__ partial,
                                                                       int32_t groups, double* __restrict__ out) {
#pragma clang fp contract(off)
    __shared__ double sh[kThreads];
    double d2 = 0.0, p2 = 0.0;
    for (int g = threadIdx.x; g < groups; g += kThreads) {
        d2 = d2 + partial[2 * g];
        p2 = p2 + partial[2 * g + 1];
    }
    const double sd = block_sum_fixed(d2, sh);
    const double sp = block_sum_fixed(p2, sh);
    if (threadIdx.x == 0) {
        out[0] = sd;
        out[1] = sp;
    }
}

// state[2] = 1.0 (recompute) unless the relative change is at most the threshold:
// reuse iff d2 <= (threshold * threshold) * p2, evaluated in this order in fp64
__global__ void reuse_decide_kernel(double* __restrict__ state, double threshold, int32_t force) {
#pragma clang fp contract(off)
    if (threadIdx.x != 0) return;
    const double t2 = threshold * threshold;
    const double bound = t2 * state[1];
    const bool reuse = force == 0 && state[0] <= bound;
    state[2] = reuse ? 0.0 : 1.0;
}

// ref <- cur over the pooled vectors, when the gate says the mask was recomputed
__global__ __launch_bounds__(kThreads) void copy_if_kernel(const double2* __restrict__ src, double2* __restrict__ dst,
                                                           int64_t n2, const double* __restrict__ gate) {
    if (*gate == 0.0) return;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n2; e += stride) dst[e] = src[e];
}

}  // namespace

hipError_t launch_mask_overlap(const uint8_t* a, const uint8_t* b, int32_t B, int32_t H, int32_t nB, int64_t* counts,
                               hipStream_t stream) {
    const int64_t n = 2 * (int64_t)B * H;
    hipLaunchKernelGGL(zero_counts_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                       counts, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(mask_overlap_kernel, dim3(kOverlapSplit, (unsigned)((int64_t)B * H)), dim3(kThreads), 0, stream,
                       a, b, (int64_t)nB * nB, counts);
    return hipGetLastError();
}

hipError_t launch_pooled_change(const double* prev, const double* cur, int64_t n, double* out, hipStream_t stream) {
    double* partial = out + 2;
    hipLaunchKernelGGL(pooled_change_partial_kernel, dim3(kChangeGroups), dim3(kThreads), 0, stream, prev, cur, n,
                       partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(pooled_change_final_kernel, dim3(1), dim3(kThreads), 0, stream, (const double*)partial,
                       (int32_t)kChangeGroups, out);
    return hipGetLastError();
}

hipError_t launch_select_reuse(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                               void* workspace_cur, double* pooled_ref, double threshold, int32_t force,
                               uint8_t* mask, double* state, hipStream_t stream) {
    const int64_t nB = (S + block - 1) / block;
    const int64_t n = 2 * (int64_t)B * H * nB * D;             // pooled q then k
    const double* cur = (const double*)workspace_cur;
    // state[0..1] and the partials at state[4..]: the change of cur against ref
    const double* prev = pooled_ref;
    double* partial = state + 4;
    hipLaunchKernelGGL(pooled_change_partial_kernel, dim3(kChangeGroups), dim3(kThreads), 0, stream, prev, cur, n,
                       partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(pooled_change_final_kernel, dim3(1), dim3(kThreads), 0, stream, (const double*)partial,
                       (int32_t)kChangeGroups, state);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(reuse_decide_kernel, dim3(1), dim3(kWave), 0, stream, state, threshold, force);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const double* gate = state + 2;
    err = launch_select_from_pooled(B, S, H, D, block, kept, mask, workspace_cur, stream, gate);
    if (err != hipSuccess) return err;
    const int64_t n2 = n / 2;                                  // D is even
    const int64_t groups = std::min<int64_t>(2048, (n2 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(copy_if_kernel, dim3((unsigned)std::max<int64_t>(1, groups)), dim3(kThreads), 0, stream,
                       (const double2*)cur, (double2*)pooled_ref, n2, gate);
    return hipGetLastError();
}

}  // namespace saq
