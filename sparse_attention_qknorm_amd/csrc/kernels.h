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
// [2][B][H][nB][D] (padded to 256 bytes), then for nB <= 1024 the int8 limbs
// of both [2][B][H][4][D/16][nBpad][16] (nBpad = 256, 512 or 1024) and the k vectors'
// exponents [B][H][nBpad] (int32), for larger nB the uint64 score keys
// [B][H][nB][nB].
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
// With a gate, both kernels read *gate on the device and do nothing when it is 0.0.
hipError_t launch_select_from_pooled(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                                     uint8_t* mask, void* workspace, hipStream_t stream,
                                     const double* gate = nullptr);

}  // namespace saq

namespace saq {

// Cross-step reuse measurements (step_reuse.hip).
constexpr int kChangeGroups = 512;   // workgroups of the first pooled-change stage

hipError_t launch_mask_overlap(const uint8_t* a, const uint8_t* b, int32_t B, int32_t H, int32_t nB, int64_t* counts,
                               hipStream_t stream);

// out: [2 + 2*kChangeGroups] doubles; out[0] = sum (cur-prev)^2, out[1] = sum prev^2
hipError_t launch_pooled_change(const double* prev, const double* cur, int64_t n, double* out, hipStream_t stream);

// Gated selection. state: [kReuseStateLen] doubles; state[0..1] as out[0..1] of
// launch_pooled_change between ref and cur, state[2] = 1.0 if the mask is
// recomputed, 0.0 if the previous one is kept; the rest is scratch. On
// recompute, cur's pooled vectors are also copied into ref.
constexpr int kReuseStateLen = 4 + 2 * kChangeGroups;
hipError_t launch_select_reuse(int32_t B, int32_t S, int32_t H, int32_t D, int32_t block, int32_t kept,
                               void* workspace_cur, double* pooled_ref, double threshold, int32_t force,
                               uint8_t* mask, double* state, hipStream_t stream);

}  // namespace saq

namespace saq {

// INT8 / FP8 (OCP E4M3) block codecs (codecs.hip): codes [B,S,H,D] (1 byte each), scales fp32 [B,H,nB].
hipError_t launch_quantize(bool fp8, const void* x, void* codes, float* scales, int32_t B, int32_t S, int32_t H,
                           int32_t D, int32_t block, hipStream_t stream);
hipError_t launch_dequantize(bool fp8, const void* codes, const float* scales, void* y, int32_t B, int32_t S,
                             int32_t H, int32_t D, int32_t block, hipStream_t stream);

}  // namespace saq

namespace saq {

// Attention with the block selection folded in (block 128, head_dim 128 only):
// each workgroup selects its query block's kept key blocks from the pooled means
// (pooled = the head of a workspace written by launch_qknorm_rope_pool) with the
// selection's rule, optionally writes that mask row, and attends over them.
hipError_t launch_block_sparse_attn_select(const void* q, const void* k, const void* v, const double* pooled,
                                           int32_t B, int32_t S, int32_t H, int32_t kept, float scale, void* o,
                                           uint8_t* mask_out, hipStream_t stream);

}  // namespace saq
