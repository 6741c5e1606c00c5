"""Convenience wrapper: owns a plan plus the caller-side device buffers
(plan image and workspace, allocated through torch) and calls the C ABI."""
from __future__ import annotations

import torch

from . import deft as D


class TreeAttention:
    """Plan a tree once, then run tree attention over paged KV.

    query_lens (optional): multi-token query nodes, the leading tokens of its
    own node each query sees.

    desc: a deft_attn_desc (see deft.make_desc).  Device buffers are torch
    tensors on `device`; the plan image is uploaded on `stream`.
    chunk_tokens 0 takes the library's rule (deft_plan_auto_chunk_tokens) for
    the tree plan; the chosen size is kept in self.chunk_tokens.

    single_dispatch (default True): a call is one launch
    (deft_tree_attention_fused: partial and merge work-groups in one grid,
    handing rows over through tickets in the plan's device image), so calls
    on one runner must not overlap; False runs the partial kernel and the
    merge kernel (deft_tree_attention).  Both give the same bits.
    """

    def __init__(self, parents, seg_lens, query_nodes, chunk_tokens: int, desc, device="cuda",
                 stream=None, query_centric: bool = False, node_chunks: bool = False,
                 query_lens=None, single_dispatch: bool = True):
        self.desc = desc
        self.single_dispatch = single_dispatch
        if chunk_tokens == 0:
            if query_centric or node_chunks:
                raise ValueError("the chunk-size rule is for the tree plan")
            chunk_tokens = D.deft_plan_auto_chunk_tokens(parents, seg_lens, query_nodes, desc,
                                                         query_lens=query_lens)
        self.chunk_tokens = chunk_tokens
        if query_lens is not None:
            if query_centric or node_chunks:
                raise ValueError("query_lens is supported by the tree plan only")
            self.plan = D.deft_plan_create_multi_token(parents, seg_lens, query_nodes, query_lens,
                                                       chunk_tokens)
        else:
            create = (D.deft_plan_create_query_centric if query_centric else
                      D.deft_plan_create_node_chunks if node_chunks else D.deft_plan_create)
            self.plan = create(parents, seg_lens, query_nodes, chunk_tokens)
        plan_bytes, ws_bytes = D.deft_plan_device_bytes(self.plan, desc)
        self.plan_bytes, self.workspace_bytes = plan_bytes, ws_bytes
        self.dev_plan = torch.empty(max(plan_bytes, 256), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device)
        D.deft_plan_upload(self.plan, desc, self.dev_plan, stream)

    def view(self) -> dict:
        return D.deft_plan_export(self.plan)

    def __call__(self, q, k_cache, v_cache, block_table, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        run = D.deft_tree_attention_fused if self.single_dispatch else D.deft_tree_attention
        run(q, k_cache, v_cache, block_table, self.plan, out, self.desc, self.workspace, stream)
        return out

    def partials(self, q, k_cache, v_cache, block_table, partial_format=D.DEFT_PARTIAL_F32, stream=None):
        """Per-slot (O, m, l) from the partial kernel alone, as device tensors
        (O fp32 unnormalised, or bf16 divided by l)."""
        s = self.plan_view_counts()
        hq, d = self.desc.num_q_heads, self.desc.head_dim
        odt = torch.bfloat16 if partial_format == D.DEFT_PARTIAL_BF16_NORM else torch.float32
        po = torch.empty((s, hq, d), dtype=odt, device=q.device)
        pm = torch.empty((s, hq), dtype=torch.float32, device=q.device)
        pl = torch.empty((s, hq), dtype=torch.float32, device=q.device)
        D.deft_partial_attention(q, k_cache, v_cache, block_table, self.plan, self.desc, po, pm, pl,
                                 partial_format, stream)
        return po, pm, pl

    def plan_view_counts(self) -> int:
        return int(D.deft_plan_export(self.plan)["num_slots"])
