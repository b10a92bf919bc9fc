"""One MSA decode step over preallocated device buffers.

Plumbing only: it owns the torch tensors the C ABI writes into and issues the
calls in order -- insert (optional), index score + max-pool, selection,
sparse attention, or for NVFP4 caches the two fused launches (insert + index,
selection + attention) -- on one stream, with no host synchronisation, so the step
can be captured into a HIP graph.
"""
from __future__ import annotations

import torch

from . import (MSA_DIM_MAJOR, MSA_F32, MSA_FP8_E4M3, MSA_HALF_ROWS, MSA_MAX_ROWS, MSA_NVFP4, MSA_TOKEN_MAJOR,
               Batch, Cache,
               msa_block_maxpool_topk, msa_workspace_bytes, msa_index_score, msa_insert_index_score,
               msa_kv_insert, msa_select_decode, msa_sparse_decode)

GROUPS = 4
HEADS = 32


def make_caches(dtype, num_pages: int, tensor_scale: float, device="cuda"):
    """(k, v, idx) page pools in the layouts the kernels read.  dtype: MSA_NVFP4, MSA_FP8_E4M3 or
    MSA_F32 (True / False stand for NVFP4 / F32)."""
    dt = (MSA_NVFP4 if dtype else MSA_F32) if isinstance(dtype, bool) else dtype
    k = Cache.empty(dt, MSA_TOKEN_MAJOR, GROUPS, num_pages, tensor_scale, device)
    v = Cache.empty(dt, MSA_TOKEN_MAJOR if dt == MSA_F32 else MSA_DIM_MAJOR, GROUPS, num_pages, tensor_scale, device)
    idx = Cache.empty(dt, MSA_HALF_ROWS if dt == MSA_FP8_E4M3 else MSA_TOKEN_MAJOR, 1, num_pages, tensor_scale, device)
    return k, v, idx


class MsaDecoder:
    def __init__(self, batch: Batch, k_cache: Cache, v_cache: Cache, idx_cache: Cache, topk: int = 16,
                 device="cuda"):
        self.batch, self.k, self.v, self.idx, self.topk = batch, k_cache, v_cache, idx_cache, topk
        B, R, P = batch.B, batch.R, batch.max_pages
        self.q_dtype = MSA_F32 if k_cache.dtype == MSA_F32 else MSA_FP8_E4M3
        self.block_scores = torch.empty((B, R, GROUPS, P), dtype=torch.float32, device=device)
        self.sel = torch.empty((B, R, GROUPS, topk), dtype=torch.int32, device=device)
        self.cnt = torch.empty((B, R, GROUPS), dtype=torch.int32, device=device)
        self.out = torch.empty((B, R, HEADS, 128), dtype=torch.float32, device=device)
        nbytes = msa_workspace_bytes(batch, topk)
        self.workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)

    def insert(self, k, v, idx_k, slots, stream=None):
        msa_kv_insert(k, v, idx_k, slots, self.k, self.v, self.idx, stream)

    def index(self, q_idx, q_scale=1.0, token_scores=None, stream=None):
        msa_index_score(self.batch, q_idx, self.q_dtype, q_scale, self.idx, self.block_scores, token_scores, stream)

    def insert_index(self, k, v, idx_k, q_idx, q_scale=1.0, token_scores=None, stream=None):
        """Steps 0+1+2 in one launch (NVFP4 caches): k, v [B*R][4][128] and idx_k [B*R][128] are the rows of
        positions L_b - R .. L_b - 1, request-major."""
        msa_insert_index_score(self.batch, k, v, idx_k, q_idx, self.q_dtype, q_scale, self.k, self.v, self.idx,
                               self.block_scores, token_scores, stream)

    def select(self, stream=None):
        msa_block_maxpool_topk(self.batch, self.block_scores, 0, self.topk, self.sel, self.cnt, stream)

    def attend(self, q, q_scale, sm_scale, stream=None):
        msa_sparse_decode(self.batch, q, self.q_dtype, q_scale, sm_scale, self.k, self.v, self.sel, self.cnt,
                          self.topk, self.out, self.workspace, stream)

    def select_attend(self, q, q_scale, sm_scale, stream=None):
        """Steps 3+4 in one launch (NVFP4 caches)."""
        msa_select_decode(self.batch, self.block_scores, self.topk, q, self.q_dtype, q_scale, sm_scale, self.k,
                          self.v, self.sel, self.cnt, self.out, self.workspace, stream)

    def step(self, q_idx, q, q_scale, sm_scale, new_tokens=None, stream=None, fused=True):
        """new_tokens: optional (k [n][4][128], v [n][4][128], idx [n][128], slots [n]) FP32 rows to insert first.
        fused (NVFP4 or FP8 caches): insert + index in one launch and selection + attention in another; the new rows
        must then be those of positions L_b - R .. L_b - 1, request-major (their slots follow from the block
        table and are not read)."""
        quant = self.k.dtype != MSA_F32
        if fused and quant and new_tokens is not None and self.batch.R <= MSA_MAX_ROWS:
            k, v, i, _ = new_tokens
            self.insert_index(k, v, i, q_idx, q_scale, None, stream)
        else:
            if new_tokens is not None:
                k, v, i, s = new_tokens
                self.insert(k, v, i, s, stream)
            self.index(q_idx, q_scale, None, stream)
        if fused and quant:
            self.select_attend(q, q_scale, sm_scale, stream)
        else:
            self.select(stream)
            self.attend(q, q_scale, sm_scale, stream)
        return self.out
