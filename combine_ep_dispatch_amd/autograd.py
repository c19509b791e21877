"""Autograd wrappers over the C ABI, shaped after the forward/backward pairs
the NeMo AutoModel fused_a2a page documents (HybridEPDispatch: dispatch
forward, combine-of-gradients backward; HybridEPCombine: combine forward,
redispatch backward).

Marshalling only: every step runs in libepx's HIP kernels.

    d = EpDispatcher(cfg, device)            # owns layout, workspace, buffers
    recv = d.dispatch(x, topk_ids)           # [R, H] bf16, differentiable in x
    y = d.combine(expert_out, probs)         # [T, H] bf16, differentiable in
                                             # expert_out and probs
    y.backward(grad)                         # -> x.grad, expert_out.grad, probs.grad

dispatch() builds the layout (the "handle") in the same call as the
dispatch and keeps it for the combine and both backward passes; rows past a segment's used rows are left as the
buffers held them (zero for the buffers allocated here).  Every routing
gets a layout of its own, and each forward node keeps the layout it ran
with, so routing the next batch before this one's backward is safe.  The
routing is not differentiable; probs is, through the router-probability
gradient.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import (EpConfig, Layout, ep_combine, ep_combine_bwd, ep_combine_bwd_probs, ep_dispatch,
               ep_dispatch_bwd, ep_dispatch_layout, ep_dispatch_with_layout, ep_query, workspace_for)

__all__ = ["EpDispatcher"]


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, cfg, layout, topk_ids=None, workspace=None):
        # with topk_ids, the layout is built in the same call (one kernel for
        # decode-sized batches)
        recv = torch.zeros(cfg.recv_rows, cfg.hidden, dtype=torch.bfloat16, device=x.device)
        if topk_ids is None:
            ep_dispatch(cfg, layout, x.contiguous().view(-1), recv.view(-1))
        else:
            ep_dispatch_with_layout(cfg, topk_ids, workspace, layout, x.contiguous().view(-1), recv.view(-1))
        ctx.cfg, ctx.layout = cfg, layout
        return recv

    @staticmethod
    def backward(ctx, grad_recv):
        cfg = ctx.cfg
        gx = torch.empty(cfg.num_tokens, cfg.hidden, dtype=torch.bfloat16, device=grad_recv.device)
        ep_dispatch_bwd(cfg, ctx.layout, grad_recv.to(torch.bfloat16).contiguous().view(-1), gx.view(-1))
        return gx, None, None, None, None


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, expert_out, probs, cfg, layout):
        y = torch.empty(cfg.num_tokens, cfg.hidden, dtype=torch.bfloat16, device=expert_out.device)
        eo = expert_out.contiguous()
        p = None if probs is None else probs.contiguous().float()
        ep_combine(cfg, layout, eo.view(-1), None if p is None else p.view(-1), y.view(-1))
        ctx.cfg, ctx.layout = cfg, layout
        ctx.has_probs = probs is not None
        ctx.save_for_backward(eo, p if p is not None else torch.empty(0, device=eo.device))
        return y

    @staticmethod
    def backward(ctx, grad_y):
        cfg, layout = ctx.cfg, ctx.layout
        eo, p = ctx.saved_tensors
        gy = grad_y.to(torch.bfloat16).contiguous()
        g_out = torch.zeros(cfg.recv_rows, cfg.hidden, dtype=torch.bfloat16, device=gy.device)
        ep_combine_bwd(cfg, layout, gy.view(-1), p.view(-1) if ctx.has_probs else None, g_out.view(-1))
        g_probs = None
        if ctx.has_probs and ctx.needs_input_grad[1]:
            g_probs = torch.empty(cfg.num_tokens, cfg.top_k, dtype=torch.float32, device=gy.device)
            ep_combine_bwd_probs(cfg, layout, gy.view(-1), eo.view(-1), g_probs.view(-1))
        return g_out, g_probs, None, None


class EpDispatcher:
    """Dispatch / combine with autograd for one configuration on one device."""

    def __init__(self, cfg: EpConfig, device, recv_rows: Optional[int] = None):
        q = ep_query(cfg)
        cfg.recv_rows = q.min_recv_rows if recv_rows is None else recv_rows
        self.cfg = cfg
        self.device = torch.device(device)
        self.layout = Layout.empty(cfg, self.device)
        self.workspace = workspace_for(cfg, self.device)

    def route(self, topk_ids: torch.Tensor) -> Layout:
        """Build a new layout (counts, offsets, token_row, expert_ids, src_info,
        flags) for these ids; later dispatch/combine calls use it.  Nodes
        already recorded keep the layout they ran with."""
        layout = Layout.empty(self.cfg, self.device)
        ep_dispatch_layout(self.cfg, topk_ids.to(torch.int32).contiguous().view(-1), self.workspace, layout)
        self.layout = layout
        return layout

    def dispatch(self, x: torch.Tensor, topk_ids: Optional[torch.Tensor] = None) -> torch.Tensor:
        """[T, H] bf16 -> [R, H] bf16 receive rows.  With topk_ids, routes in
        the same call (ep_dispatch_with_layout) into a new layout that later
        calls use, as route() would."""
        if topk_ids is None:
            return _Dispatch.apply(x, self.cfg, self.layout)
        layout = Layout.empty(self.cfg, self.device)
        ids = topk_ids.to(torch.int32).contiguous().view(-1)
        recv = _Dispatch.apply(x, self.cfg, layout, ids, self.workspace)
        self.layout = layout
        return recv

    def combine(self, expert_out: torch.Tensor, probs: Optional[torch.Tensor]) -> torch.Tensor:
        """[R, H] bf16 expert outputs -> [T, H] bf16, weighted by probs [T, K] (or 1)."""
        return _Combine.apply(expert_out, probs, self.cfg, self.layout)

    def tokens_per_expert(self) -> torch.Tensor:
        """Routed rows per group [S, G] (the shared group included)."""
        return self.layout.counts
