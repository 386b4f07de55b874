"""quant_verify_gemv_amd: the Q4_K batched speculative-verify step on MI355X.

The hot path (activation staging, Q4_K dequant + MFMA skinny GEMM, split-K
combine, row argmax, greedy accept, draft block proposals, chains of
dependent products in one launch, target probability rows for the
stochastic verify) runs in HIP kernels inside libkq.so,
behind the C ABI of include/kq.h. This package is the thin Python binding.
"""
from .lib import (CHAIN_ERROR_OFFSET, DRAFT_VERIFY_LENGTHS, FORMATS, LAYOUT_Q5K_TILED16,  # noqa: F401
                  LAYOUT_Q6K_TILED16, LAYOUT_ROWS, LAYOUT_TILED16,
                  MAX_GROUP, Chain, ChainPhase, ChainPlan, KQError, chain_encode, chain_table_bytes,
                  draft_block_argmax, draft_block_argmax_staged, gemv_chain, gemv_rows, gemv_staged, gemv_staged_group, softmax_rows, softmax_workspace_bytes,
                  speculative_decide, speculative_decide_mt, speculative_first_reject, speculative_resample,
                  gather_rows, MT19937,
                  group_scratch_bytes, launch_geometry, load, new_group_scratch,
                  new_scratch, scratch_bytes, stage_rows, staged_bytes, status_string, stream_probe, tile_weights,
                  tiled_bytes, verify, verify_staged, verify_tree_staged, workspace_bytes)

QK = 256
BLOCK_BYTES = 144
MAX_ROWS = 16
