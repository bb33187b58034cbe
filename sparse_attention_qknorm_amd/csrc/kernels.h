// Host-side launchers of the gfx950 kernels (internal to the library; the
// public interface is the C ABI in include/saq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace saq {

constexpr int kMaxPairs = 64;      // D <= 128
constexpr int kMaxBlocks = 4096;   // nB limit of the selection and attention kernels

// Per-pair rotary frequencies, passed by value in the kernel arguments.
struct RopeTable {
    double inv_freq[kMaxPairs];    // pair p of its section: base^(-2i/d_a)
    int32_t pair_end_t;            // pairs [0, pair_end_t) rotate with t
    int32_t pair_end_h;            // pairs [pair_end_t, pair_end_h) with h, the rest with w
};

hipError_t launch_qknorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                              const int32_t* pos_thw, const float* w_q, const float* w_k,
                              int32_t B, int32_t S, int32_t H, int32_t D, const RopeTable& table,
                              float eps, hipStream_t stream);

// Workspace layout of the selection: pooled fp64 vectors of q then k
// [2][B][H][nB][D], then the uint64 score keys [B][H][nB][nB].
size_t select_workspace_bytes(int64_t B, int64_t H, int64_t nB, int64_t D);

hipError_t launch_select_blocks(const void* q, const void* k, int32_t B, int32_t S, int32_t H, int32_t D,
                                int32_t block, int32_t kept, uint8_t* mask, void* workspace,
                                hipStream_t stream);

hipError_t launch_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* mask,
                                    int32_t B, int32_t S, int32_t H, int32_t D, int32_t block,
                                    float scale, void* o, hipStream_t stream);

}  // namespace saq

namespace saq {

// Fused prologue + pooling: also writes the per-block fp64 means of the bf16
// q-hat and k-hat into `pooled` ([2][B][H][nB][D], the head of the selection
// workspace). Supports H*D <= kMaxRowElems.
constexpr int kMaxRowElems = 8192;

hipError_t launch_qknorm_rope_pool(const void* q_in, const void* k_in, void* q_out, void* k_out,
                                   const int32_t* pos_thw, const float* w_q, const float* w_k, int32_t B,
                                   int32_t S, int32_t H, int32_t D, const RopeTable& table, float eps,
                                   int32_t block, double* pooled, hipStream_t stream);

// Selection from pooled vectors already in the workspace (scores + top-k only).
hipError_t launch_select_from_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                                     uint8_t* mask, void* workspace, hipStream_t stream);

}  // namespace saq
