"""Buffer allocation and call sequencing for one drop layer.

Plumbing only: allocates the outputs and workspaces the C ABI asks for with
torch, then calls the library in the order of the path (select, compact,
metadata, scatter-back).  No arithmetic of the method happens here.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (SelectParams, compact, compact_workspace_bytes, make_params, max_blocks,
               scatter_back, select_blocks, select_blocks_profiled, select_workspace_bytes,
               update_metadata)


def _empty(n, dtype, device):
    return torch.empty(max(int(n), 1), dtype=dtype, device=device)


@dataclass
class SelectBuffers:
    params: SelectParams
    num_reqs: int
    max_tokens: int
    block_scores: torch.Tensor
    block_offsets: torch.Tensor
    keep_block: torch.Tensor
    keep_mask: torch.Tensor
    kept: torch.Tensor
    workspace: torch.Tensor

    @staticmethod
    def allocate(params: SelectParams, num_reqs: int, max_tokens: int, device="cuda"):
        mb = max_blocks(params.block_size, num_reqs, max_tokens)
        ws = select_workspace_bytes(params, num_reqs, max_tokens)
        return SelectBuffers(
            params, num_reqs, max_tokens,
            block_scores=_empty(mb, torch.float32, device),
            block_offsets=_empty(num_reqs + 1, torch.int32, device),
            keep_block=_empty(mb, torch.uint8, device),
            keep_mask=_empty(max_tokens, torch.uint8, device),
            kept=_empty(num_reqs, torch.int32, device),
            workspace=_empty(ws, torch.uint8, device),
        )

    def run(self, q, k, cu_seqlens, scores_in=None, stream=None, score_events=None):
        """score_events: optional (begin, end) hipEvent_t handles recorded around
        the score kernel (the instrumentation entry point)."""
        qs = q.stride(0) if q is not None else 0
        ks = k.stride(0) if k is not None else 0
        if score_events is not None:
            return select_blocks_profiled(self.params, q, qs, k, ks, cu_seqlens, self.num_reqs,
                                          self.max_tokens, scores_in, self.block_scores, self.block_offsets,
                                          self.keep_block, self.keep_mask, self.kept, self.workspace,
                                          score_events[0], score_events[1], stream=stream)
        return select_blocks(self.params, q, qs, k, ks, cu_seqlens, self.num_reqs, self.max_tokens,
                             scores_in, self.block_scores, self.block_offsets, self.keep_block,
                             self.keep_mask, self.kept, self.workspace, stream=stream)


@dataclass
class CompactBuffers:
    num_reqs: int
    max_tokens: int
    index_out: torch.Tensor
    cu_out: torch.Tensor
    workspace: torch.Tensor

    @staticmethod
    def allocate(num_reqs: int, max_tokens: int, device="cuda"):
        return CompactBuffers(
            num_reqs, max_tokens,
            index_out=_empty(max_tokens, torch.int32, device),
            cu_out=_empty(num_reqs + 1, torch.int32, device),
            workspace=_empty(compact_workspace_bytes(num_reqs, max_tokens), torch.uint8, device),
        )

    def run(self, keep_mask, cu_seqlens, src, dst, index_in=None, stream=None):
        rb = [t[0].numel() * t.element_size() if t.dim() > 1 else t.element_size() for t in src]
        return compact(keep_mask, cu_seqlens, self.num_reqs, self.max_tokens, src, dst, rb, index_in,
                       self.index_out, self.cu_out, self.workspace, stream=stream)


@dataclass
class MetadataBuffers:
    num_reqs: int
    num_layers: int
    max_drops: int
    seq_lens: torch.Tensor
    num_actual_tokens: torch.Tensor
    drop_count: torch.Tensor
    drop_layer: torch.Tensor
    drop_len: torch.Tensor
    seqused_base: torch.Tensor

    @staticmethod
    def allocate(seq_lens, num_layers: int, max_drops: int, device="cuda"):
        sl = torch.as_tensor(seq_lens, dtype=torch.int32).to(device)
        R = sl.numel()
        return MetadataBuffers(
            R, num_layers, max_drops,
            seq_lens=sl.clone(),
            num_actual_tokens=torch.zeros(1, dtype=torch.int32, device=device),
            drop_count=torch.zeros(max(R, 1), dtype=torch.int32, device=device),
            drop_layer=torch.full((max(R * max_drops, 1),), -1, dtype=torch.int32, device=device),
            drop_len=torch.full((max(R * max_drops, 1),), -1, dtype=torch.int32, device=device),
            seqused_base=sl.repeat(num_layers).contiguous() if R else _empty(1, torch.int32, device),
        )

    def run(self, layer, cu_old, cu_new, stream=None):
        return update_metadata(layer, self.num_layers, self.num_reqs, cu_old, cu_new, self.seq_lens,
                               self.num_actual_tokens, self.drop_count, self.drop_layer, self.drop_len,
                               self.max_drops, self.seqused_base, stream=stream)


def run_scatter_back(compacted, index_map, cu_out, num_reqs, max_tokens, full, stream=None):
    rb = compacted[0].numel() * compacted.element_size()
    return scatter_back(compacted, rb, index_map, cu_out, num_reqs, max_tokens, full, full.shape[0],
                        stream=stream)


__all__ = ["SelectBuffers", "CompactBuffers", "MetadataBuffers", "run_scatter_back", "make_params"]
