"""Plain, slow, fp64 CPU oracle for the joint-sequence attention layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check of the package entry
file and the bench's CPU-baseline leg use it. It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants) and imports nothing
from it; both sides are fed the same seeded inputs from a generator module
that holds none of the method's arithmetic.

What it computes, in the order of the layer:

1. QKNorm (``qknorm``): RMS normalisation of every (token, head) row of Q and
   K over head_dim, scaled by a learned per-channel weight. The pages name the
   operation only as one half of the fused "QKNorm + RoPE" kernel (Sol Engine
   "H3 on device" page, fusion table of the lossless-kernels section); the row
   axis, the weight shape and the place of epsilon are this oracle's reading.
2. 3D multimodal RoPE (``rope_3d``): the "3D MM-RoPE" of the same fusion-table
   row, read as three contiguous head_dim sections (t, h, w), each a 1-D rotary
   embedding of adjacent pairs with frequencies base^(-2i/d_a).
3. Block selection (``pool_blocks``, ``block_scores``, ``select_topk``,
   ``select_blocks``): per (batch, head), mean-pool q and k over each block of
   tokens, score every (query block, key block) pair by the dot product of the
   pooled vectors, and keep the top-k key blocks of each query block plus the
   diagonal. The pages say only that selection is dynamic, per step,
   training- and calibration-free and decides which attention blocks are
   computed (Sol-Attn paragraph of the "H3 on device" page; KOCPC article on
   Sol-H3, "Specific outcomes of key optimizations"); the rule is the build's.
4. Block-sparse attention (``block_sparse_attention``): non-causal softmax
   attention of each query block over the tokens of its kept key blocks only.
5. Cross-step reuse measurements (``mask_overlap``, ``pooled_change``): the
   overlap of two steps' masks and the relative change of their pooled block
   means, the detector that gates reusing a mask (cross-step cache paragraph of
   the "H3 on device" page).
6. INT8 / FP8 block codecs (``oracle.codecs``): per-(token block, head) scaled
   quantise/dequantise of the attention exchange's inputs (INT8) and outputs
   (OCP E4M3), the transfer formats of multi-GPU Sol-Attn (KOCPC article on
   Sol-H3, "Technical Composition").

Every function is pinned by CPU tests to something other than itself: closed
forms, invariants, library routines (complex multiplication, logspace,
math.fsum, exact rationals, torch's float64 scaled_dot_product_attention) and
brute force on tiny inputs. The conventions the pages leave open (row axis of
the norm, epsilon placement, RoPE pair layout and frequency schedule, the
selection rule itself) are readings: the tests pin the oracle to each reading's
closed forms, not to the method, whose exact form the pages do not give.
"""
from .prologue import qknorm, rope_inv_freq, rope_3d, qknorm_rope
from .selection import (num_kept_blocks, pool_blocks, block_scores, select_topk,
                        select_blocks, block_token_range)
from .attention import block_sparse_attention, block_sparse_attention_rows, dense_attention
from . import codecs
from .step_reuse import mask_overlap, pooled_change, relative_change, keeps_mask, reuse_schedule

__all__ = [
    "qknorm", "rope_inv_freq", "rope_3d", "qknorm_rope",
    "num_kept_blocks", "pool_blocks", "block_scores", "select_topk", "select_blocks",
    "block_token_range", "block_sparse_attention", "block_sparse_attention_rows", "dense_attention",
    "mask_overlap", "pooled_change", "relative_change", "keeps_mask", "reuse_schedule", "codecs",
]
