"""MoE expert-parallel token dispatch and combine for one MI355X's share.

Thin Python binding over libepx.so (C ABI in include/epx.h): the functions
below only check tensor shapes, dtypes and devices and pass raw pointers and
the current HIP stream; every step runs in the library's HIP kernels.  There
is no CPU fallback: a missing library raises.

Typical use (all tensors on one GPU, bf16 payloads as torch.bfloat16)::

    cfg = EpConfig(num_tokens=T, hidden=H, num_experts=E, num_segments=S,
                   top_k=K, align=128)
    cfg.recv_rows = ep_query(cfg).min_recv_rows
    lay = Layout.empty(cfg, device)
    ws = workspace_for(cfg, device)
    ep_dispatch_layout(cfg, topk_ids, ws, lay)
    ep_dispatch(cfg, lay, x, recv)
    ...
    ep_combine(cfg, lay, expert_out, probs, y)
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import (EP_FLAG_BAD_ID, EP_FLAG_DROPPED, EP_FLAG_INTERNAL, EP_FLAG_MAP_OVERFLOW,  # noqa: F401
                   EP_NOALLOC_SCRATCH_BYTES, EP_ZERO_PAD_ROWS, EP_LAYOUT_LOOKBACK, EP_LAYOUT_DIRECT,
                   EP_LAYOUT_BARRIER, EP_LAYOUT_COUNT, EpCfg, EpLayout)

__all__ = [
    "EpConfig", "Layout", "QueryResult", "ep_query", "workspace_for", "ep_dispatch_layout",
    "ep_dispatch_layout_noalloc", "EP_NOALLOC_SCRATCH_BYTES", "ep_combine_nvfp4", "ep_dispatch_with_layout",
    "ep_dispatch_nvfp4_with_layout", "ep_dispatch_fp8_with_layout",
    "ep_dispatch", "ep_dispatch_nvfp4", "ep_dispatch_fp8", "ep_combine", "ep_dispatch_bwd", "ep_combine_bwd",
    "ep_combine_bwd_probs", "ep_indices_to_multihot", "ep_multihot_to_indices", "assert_no_overflow", "EpError", "abi_version", "EP_ZERO_PAD_ROWS", "EP_LAYOUT_LOOKBACK", "EP_LAYOUT_DIRECT", "EP_LAYOUT_BARRIER", "EP_LAYOUT_COUNT", "EP_FLAG_DROPPED",
    "EP_FLAG_BAD_ID", "EP_FLAG_INTERNAL",
]


class EpError(RuntimeError):
    """A nonzero status from libepx."""


@dataclasses.dataclass
class EpConfig:
    """Mirror of ep_cfg_t (see include/epx.h for the meaning of every field)."""

    num_tokens: int
    hidden: int
    num_experts: int
    num_segments: int
    top_k: int
    align: int = 1
    seg_capacity: int = 0
    shared_expert: int = 0
    src_segment: int = 0
    recv_rows: int = 0
    flags: int = 0

    @property
    def kp(self) -> int:
        return self.top_k + self.shared_expert

    @property
    def groups_per_segment(self) -> int:
        return self.num_experts // self.num_segments + self.shared_expert

    def to_c(self) -> EpCfg:
        return EpCfg(self.num_tokens, self.hidden, self.num_experts, self.num_segments, self.top_k,
                     self.align, self.seg_capacity, self.shared_expert, self.src_segment, 0,
                     self.recv_rows, self.flags, 0)


class QueryResult(NamedTuple):
    min_recv_rows: int
    workspace_bytes: int
    groups_per_segment: int


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _lib.lib().ep_strerror(status).decode()
        raise EpError(f"{what}: {msg} (status {status})")


def abi_version() -> int:
    return int(_lib.lib().ep_abi_version())


def ep_query(cfg: EpConfig) -> QueryResult:
    rows, ws, g = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    c = cfg.to_c()
    _check(_lib.lib().ep_query(ctypes.byref(c), ctypes.byref(rows), ctypes.byref(ws), ctypes.byref(g)),
           "ep_query")
    return QueryResult(rows.value, ws.value, g.value)


def workspace_for(cfg: EpConfig, device) -> torch.Tensor:
    """A zero-filled uint8 device tensor large enough for ep_dispatch_layout's
    workspace.  Keep passing the same tensor to later layout calls: each call
    leaves it ready for the next (it must only be zero before its first use)."""
    return torch.zeros(ep_query(cfg).workspace_bytes, dtype=torch.uint8, device=device)


@dataclasses.dataclass
class Layout:
    """The dispatch handle: int32 device tensors written by ep_dispatch_layout."""

    counts: torch.Tensor          # [S, G]
    seg_base: torch.Tensor        # [S + 1]
    row_offsets: torch.Tensor     # [S, G + 1]
    scales_offsets: torch.Tensor  # [S, G + 1]
    token_row: torch.Tensor       # [T, K']
    expert_ids: torch.Tensor      # [R]
    src_info: torch.Tensor        # [R, 2]
    flags: torch.Tensor           # [1]

    @staticmethod
    def empty(cfg: EpConfig, device) -> "Layout":
        S, G, R = cfg.num_segments, cfg.groups_per_segment, cfg.recv_rows
        i32 = dict(dtype=torch.int32, device=device)
        return Layout(torch.empty(S, G, **i32), torch.empty(S + 1, **i32),
                      torch.empty(S, G + 1, **i32), torch.empty(S, G + 1, **i32),
                      torch.empty(cfg.num_tokens, cfg.kp, **i32), torch.empty(R, **i32),
                      torch.empty(R, 2, **i32), torch.empty(1, **i32))

    def check(self, cfg: EpConfig, device) -> None:
        S, G, R = cfg.num_segments, cfg.groups_per_segment, cfg.recv_rows
        want = {"counts": S * G, "seg_base": S + 1, "row_offsets": S * (G + 1),
                "scales_offsets": S * (G + 1), "token_row": cfg.num_tokens * cfg.kp,
                "expert_ids": R, "src_info": 2 * R, "flags": 1}
        for name, n in want.items():
            _tensor(getattr(self, name), f"layout.{name}", torch.int32, n, device)

    def to_c(self) -> EpLayout:
        return EpLayout(*(getattr(self, f).data_ptr() for f in
                          ("counts", "seg_base", "row_offsets", "scales_offsets", "token_row",
                           "expert_ids", "src_info", "flags")))


def _tensor(t: Optional[torch.Tensor], name: str, dtype, numel: int, device=None) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _stream(stream, device) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ep_dispatch_layout(cfg: EpConfig, topk_ids: torch.Tensor, workspace: torch.Tensor, layout: Layout,
                       stream=None) -> None:
    dev = topk_ids.device
    _tensor(topk_ids, "topk_ids", torch.int32, cfg.num_tokens * cfg.top_k)
    _tensor(workspace, "workspace", torch.uint8, workspace.numel(), dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_layout(ctypes.byref(c), topk_ids.data_ptr(), workspace.data_ptr(),
                                         workspace.numel(), ctypes.byref(L), _stream(stream, dev)),
           "ep_dispatch_layout")


def ep_dispatch_layout_noalloc(cfg: EpConfig, topk_ids: torch.Tensor, layout: Layout, stream=None) -> None:
    """ep_dispatch_layout with the library's built-in scratch instead of a
    workspace: allocates nothing.  Calls that may overlap on one GPU race."""
    dev = topk_ids.device
    _tensor(topk_ids, "topk_ids", torch.int32, cfg.num_tokens * cfg.top_k)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_layout_noalloc(ctypes.byref(c), topk_ids.data_ptr(), ctypes.byref(L),
                                                 _stream(stream, dev)), "ep_dispatch_layout_noalloc")


def ep_dispatch(cfg: EpConfig, layout: Layout, x: torch.Tensor, recv: torch.Tensor, stream=None) -> None:
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(recv, "recv", torch.bfloat16, R * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch(ctypes.byref(c), ctypes.byref(L), x.data_ptr(), recv.data_ptr(),
                                  _stream(stream, dev)), "ep_dispatch")


def ep_dispatch_with_layout(cfg: EpConfig, topk_ids: torch.Tensor, workspace: torch.Tensor, layout: Layout,
                            x: torch.Tensor, recv: torch.Tensor, stream=None) -> None:
    """ep_dispatch_layout then ep_dispatch in one call (one kernel for
    decode-sized batches of up to 512 routed slots)."""
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(topk_ids, "topk_ids", torch.int32, T * cfg.top_k, dev)
    _tensor(workspace, "workspace", torch.uint8, workspace.numel(), dev)
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(recv, "recv", torch.bfloat16, R * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_with_layout(ctypes.byref(c), topk_ids.data_ptr(), workspace.data_ptr(),
                                              workspace.numel(), ctypes.byref(L), x.data_ptr(), recv.data_ptr(),
                                              _stream(stream, dev)), "ep_dispatch_with_layout")


def ep_dispatch_nvfp4_with_layout(cfg: EpConfig, topk_ids: torch.Tensor, workspace: torch.Tensor, layout: Layout,
                                  x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, rowscale: torch.Tensor,
                                  stream=None) -> None:
    """ep_dispatch_layout then ep_dispatch_nvfp4 in one call (one kernel for
    decode-sized batches of up to 512 routed slots)."""
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(topk_ids, "topk_ids", torch.int32, T * cfg.top_k, dev)
    _tensor(workspace, "workspace", torch.uint8, workspace.numel(), dev)
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(codes, "codes", torch.uint8, R * (H // 2), dev)
    _tensor(scales, "scales", torch.uint8, R * (H // 16), dev)
    _tensor(rowscale, "rowscale", torch.bfloat16, R, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_nvfp4_with_layout(ctypes.byref(c), topk_ids.data_ptr(), workspace.data_ptr(),
                                                    workspace.numel(), ctypes.byref(L), x.data_ptr(),
                                                    codes.data_ptr(), scales.data_ptr(), rowscale.data_ptr(),
                                                    _stream(stream, dev)), "ep_dispatch_nvfp4_with_layout")


def ep_dispatch_fp8_with_layout(cfg: EpConfig, topk_ids: torch.Tensor, workspace: torch.Tensor, layout: Layout,
                                x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """ep_dispatch_layout then ep_dispatch_fp8 in one call (one kernel for
    decode-sized batches of up to 512 routed slots)."""
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(topk_ids, "topk_ids", torch.int32, T * cfg.top_k, dev)
    _tensor(workspace, "workspace", torch.uint8, workspace.numel(), dev)
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(codes, "codes", torch.uint8, R * H, dev)
    _tensor(scales, "scales", torch.float32, R * (H // 128), dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_fp8_with_layout(ctypes.byref(c), topk_ids.data_ptr(), workspace.data_ptr(),
                                                  workspace.numel(), ctypes.byref(L), x.data_ptr(), codes.data_ptr(),
                                                  scales.data_ptr(), _stream(stream, dev)),
           "ep_dispatch_fp8_with_layout")


def ep_dispatch_nvfp4(cfg: EpConfig, layout: Layout, x: torch.Tensor, codes: torch.Tensor,
                      scales: torch.Tensor, rowscale: torch.Tensor, stream=None) -> None:
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(codes, "codes", torch.uint8, R * (H // 2), dev)
    _tensor(scales, "scales", torch.uint8, R * (H // 16), dev)
    _tensor(rowscale, "rowscale", torch.bfloat16, R, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_nvfp4(ctypes.byref(c), ctypes.byref(L), x.data_ptr(), codes.data_ptr(),
                                        scales.data_ptr(), rowscale.data_ptr(), _stream(stream, dev)),
           "ep_dispatch_nvfp4")


def ep_dispatch_fp8(cfg: EpConfig, layout: Layout, x: torch.Tensor, codes: torch.Tensor,
                    scales: torch.Tensor, stream=None) -> None:
    """FP8 dispatch: codes uint8 [R, H] (E4M3), scales float32 [R, H/128]."""
    dev = x.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(x, "x", torch.bfloat16, T * H)
    _tensor(codes, "codes", torch.uint8, R * H, dev)
    _tensor(scales, "scales", torch.float32, R * (H // 128), dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_fp8(ctypes.byref(c), ctypes.byref(L), x.data_ptr(), codes.data_ptr(),
                                      scales.data_ptr(), _stream(stream, dev)), "ep_dispatch_fp8")


def ep_combine(cfg: EpConfig, layout: Layout, expert_out: torch.Tensor, probs: Optional[torch.Tensor],
               y: torch.Tensor, stream=None) -> None:
    dev = expert_out.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(expert_out, "expert_out", torch.bfloat16, R * H)
    if probs is not None:
        _tensor(probs, "probs", torch.float32, T * cfg.top_k, dev)
    _tensor(y, "y", torch.bfloat16, T * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_combine(ctypes.byref(c), ctypes.byref(L), expert_out.data_ptr(),
                                 None if probs is None else probs.data_ptr(), y.data_ptr(),
                                 _stream(stream, dev)), "ep_combine")


def ep_combine_nvfp4(cfg: EpConfig, layout: Layout, codes: torch.Tensor, scales: torch.Tensor,
                     rowscale: torch.Tensor, probs: Optional[torch.Tensor], y: torch.Tensor, stream=None) -> None:
    """Combine over NVFP4 expert-output rows: codes uint8 [R, H/2], E4M3
    scales uint8 [R, H/16], rowscale bf16 [R] -> y bf16 [T, H]."""
    dev = codes.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(codes, "codes", torch.uint8, R * (H // 2))
    _tensor(scales, "scales", torch.uint8, R * (H // 16), dev)
    _tensor(rowscale, "rowscale", torch.bfloat16, R, dev)
    if probs is not None:
        _tensor(probs, "probs", torch.float32, T * cfg.top_k, dev)
    _tensor(y, "y", torch.bfloat16, T * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_combine_nvfp4(ctypes.byref(c), ctypes.byref(L), codes.data_ptr(), scales.data_ptr(),
                                       rowscale.data_ptr(), None if probs is None else probs.data_ptr(),
                                       y.data_ptr(), _stream(stream, dev)), "ep_combine_nvfp4")


def ep_dispatch_bwd(cfg: EpConfig, layout: Layout, grad_recv: torch.Tensor, grad_x: torch.Tensor,
                    stream=None) -> None:
    dev = grad_recv.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(grad_recv, "grad_recv", torch.bfloat16, R * H)
    _tensor(grad_x, "grad_x", torch.bfloat16, T * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_dispatch_bwd(ctypes.byref(c), ctypes.byref(L), grad_recv.data_ptr(),
                                      grad_x.data_ptr(), _stream(stream, dev)), "ep_dispatch_bwd")


def ep_combine_bwd(cfg: EpConfig, layout: Layout, grad_y: torch.Tensor, probs: Optional[torch.Tensor],
                   grad_expert_out: torch.Tensor, stream=None) -> None:
    dev = grad_y.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(grad_y, "grad_y", torch.bfloat16, T * H)
    if probs is not None:
        _tensor(probs, "probs", torch.float32, T * cfg.top_k, dev)
    _tensor(grad_expert_out, "grad_expert_out", torch.bfloat16, R * H, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_combine_bwd(ctypes.byref(c), ctypes.byref(L), grad_y.data_ptr(),
                                     None if probs is None else probs.data_ptr(),
                                     grad_expert_out.data_ptr(), _stream(stream, dev)), "ep_combine_bwd")


def ep_combine_bwd_probs(cfg: EpConfig, layout: Layout, grad_y: torch.Tensor, expert_out: torch.Tensor,
                         grad_probs: torch.Tensor, stream=None) -> None:
    """grad_probs[t, k] = <grad_y[t], expert_out[token_row[t, k]]> (fp32, [T, K])."""
    dev = grad_y.device
    T, H, R = cfg.num_tokens, cfg.hidden, cfg.recv_rows
    _tensor(grad_y, "grad_y", torch.bfloat16, T * H)
    _tensor(expert_out, "expert_out", torch.bfloat16, R * H, dev)
    _tensor(grad_probs, "grad_probs", torch.float32, T * cfg.top_k, dev)
    layout.check(cfg, dev)
    c, L = cfg.to_c(), layout.to_c()
    _check(_lib.lib().ep_combine_bwd_probs(ctypes.byref(c), ctypes.byref(L), grad_y.data_ptr(),
                                           expert_out.data_ptr(), grad_probs.data_ptr(),
                                           _stream(stream, dev)), "ep_combine_bwd_probs")


def ep_indices_to_multihot(cfg: EpConfig, topk_ids: torch.Tensor, probs: Optional[torch.Tensor],
                           routing_map: torch.Tensor, dense_probs: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    """Compact top-k -> routing_map uint8 [T, E] (+ dense_probs float32 [T, E])."""
    dev = topk_ids.device
    T, E, K = cfg.num_tokens, cfg.num_experts, cfg.top_k
    _tensor(topk_ids, "topk_ids", torch.int32, T * K)
    _tensor(routing_map, "routing_map", torch.uint8, T * E, dev)
    if dense_probs is not None:
        _tensor(dense_probs, "dense_probs", torch.float32, T * E, dev)
        _tensor(probs, "probs", torch.float32, T * K, dev)
    c = cfg.to_c()
    _check(_lib.lib().ep_indices_to_multihot(
        ctypes.byref(c), topk_ids.data_ptr(), None if probs is None else probs.data_ptr(),
        routing_map.data_ptr(), None if dense_probs is None else dense_probs.data_ptr(),
        _stream(stream, dev)), "ep_indices_to_multihot")


def ep_multihot_to_indices(cfg: EpConfig, routing_map: torch.Tensor, dense_probs: Optional[torch.Tensor],
                           topk_ids: torch.Tensor, probs: Optional[torch.Tensor] = None,
                           flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """routing_map uint8 [T, E] (+ dense_probs) -> compact top-k ids [T, K] (+ probs)."""
    dev = routing_map.device
    T, E, K = cfg.num_tokens, cfg.num_experts, cfg.top_k
    _tensor(routing_map, "routing_map", torch.uint8, T * E)
    _tensor(topk_ids, "topk_ids", torch.int32, T * K, dev)
    if probs is not None:
        _tensor(probs, "probs", torch.float32, T * K, dev)
        _tensor(dense_probs, "dense_probs", torch.float32, T * E, dev)
    if flags is not None:
        _tensor(flags, "flags", torch.int32, 1, dev)
    c = cfg.to_c()
    _check(_lib.lib().ep_multihot_to_indices(
        ctypes.byref(c), routing_map.data_ptr(), None if dense_probs is None else dense_probs.data_ptr(),
        topk_ids.data_ptr(), None if probs is None else probs.data_ptr(),
        None if flags is None else flags.data_ptr(), _stream(stream, dev)), "ep_multihot_to_indices")


def assert_no_overflow(layout: Layout, capacity: Optional[int] = None) -> None:
    """Read the device flags word (a host sync) and raise if any slot was dropped
    or an id was invalid (NeMo AutoModel token_dispatcher page,
    _assert_no_hybridep_overflow: fail loudly instead of training on dropped
    tokens)."""
    f = int(layout.flags.item())
    if f & EP_FLAG_DROPPED:
        cap = f" (capacity {capacity} rows per segment)" if capacity is not None else ""
        raise EpError(f"dispatch dropped slots at segment capacity{cap}")
    if f & EP_FLAG_BAD_ID:
        raise EpError("dispatch saw expert ids outside [-1, num_experts)")
    if f & EP_FLAG_INTERNAL:
        raise EpError("dispatch layout scan did not complete")
