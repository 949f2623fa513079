"""Device buffers for one MoE layer configuration, and a forward call.

Plumbing only: torch allocates the caller-owned buffers the C ABI expects
(outputs, routing and dispatch results, workspace), and ``MoELayer.forward``
hands them to ``moe_forward``.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib


def torch_dtype(cfg: _lib.MoeConfig):
    return torch.bfloat16 if cfg.dtype == _lib.MOE_BF16 else torch.float32


@dataclass
class ForwardBuffers:
    out: torch.Tensor             # [T, d]
    topk_ids: torch.Tensor        # [T, k] int32
    topk_w: torch.Tensor          # [T, k] float32
    expert_counts: torch.Tensor   # [E] int32
    expert_offsets: torch.Tensor  # [E+1] int32
    perm: torch.Tensor            # [T*k] int32
    inv_perm: torch.Tensor        # [T*k] int32
    ws: torch.Tensor              # uint8 workspace
    expert_order: Optional[torch.Tensor] = None  # [T, E] uint8 (rerouting forward only)

    @staticmethod
    def allocate(cfg: _lib.MoeConfig, device="cuda", reroute: bool = False) -> "ForwardBuffers":
        T, d, E, k = cfg.num_tokens, cfg.hidden_size, cfg.num_experts, cfg.num_experts_per_tok
        i32 = dict(dtype=torch.int32, device=device)
        op = _lib.MOE_OP_FORWARD_REROUTE if reroute else _lib.MOE_OP_FORWARD
        return ForwardBuffers(
            out=torch.empty((T, d), dtype=torch_dtype(cfg), device=device),
            topk_ids=torch.empty((T, k), **i32),
            topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
            expert_counts=torch.empty(E, **i32),
            expert_offsets=torch.empty(E + 1, **i32),
            perm=torch.empty(T * k, **i32),
            inv_perm=torch.empty(T * k, **i32),
            ws=torch.empty(max(1, _lib.moe_workspace_size(cfg, op)), dtype=torch.uint8, device=device),
            expert_order=torch.empty((T, E), dtype=torch.uint8, device=device) if reroute else None,
        )

    def _dispatch_op(self) -> int:
        return _lib.MOE_OP_DISPATCH_REROUTE if self.expert_order is not None else _lib.MOE_OP_DISPATCH

    def scratch_view(self, cfg: _lib.MoeConfig, name: str) -> torch.Tensor:
        """The router ("route") or dispatcher ("dispatch") scratch inside the forward workspace."""
        a = lambda b: (b + 255) // 256 * 256  # noqa: E731
        r = _lib.moe_workspace_size(cfg, _lib.MOE_OP_ROUTE)
        d = _lib.moe_workspace_size(cfg, self._dispatch_op())
        if name == "route":
            return self.ws[:max(r, 1)]
        return self.ws[a(r):a(r) + max(d, 1)]

    def workspace_view(self, cfg: _lib.MoeConfig, name: str) -> torch.Tensor:
        """Xp, H or Yp as a tensor view into the forward workspace (the layout moe_forward uses:
        router scratch, dispatch scratch, then Xp, H, Yp, each 256-byte aligned)."""
        T, d, F, k = cfg.num_tokens, cfg.hidden_size, cfg.intermediate_size, cfg.num_experts_per_tok
        es = 2 if cfg.dtype == _lib.MOE_BF16 else 4
        a = lambda b: (b + 255) // 256 * 256  # noqa: E731
        disp = a(_lib.moe_workspace_size(cfg, _lib.MOE_OP_ROUTE)) + a(_lib.moe_workspace_size(cfg, self._dispatch_op()))
        xp = a(T * k * d * es)
        h = a(T * k * F * es)
        start, cols = {"Xp": (disp, d), "H": (disp + xp, F), "Yp": (disp + xp + h, d)}[name]
        n = T * k * cols * es
        return self.ws[start:start + n].view(torch_dtype(cfg)).view(T * k, cols)


class MoELayer:
    """Weights of one layer resident on the GPU, plus its forward buffers.
    ``reroute``: over-capacity pairs move to their token's next-best expert
    with room instead of being dropped (``moe_forward_reroute``)."""

    def __init__(self, cfg: _lib.MoeConfig, Wg: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor,
                 gate_bias: Optional[torch.Tensor] = None, device="cuda", reroute: bool = False):
        self.cfg = cfg
        self.reroute = reroute
        self.Wg, self.W1, self.W2, self.gate_bias = Wg, W1, W2, gate_bias
        self.buf = ForwardBuffers.allocate(cfg, device, reroute)

    def forward(self, X: torch.Tensor, stream=None) -> torch.Tensor:
        b = self.buf
        if self.reroute:
            _lib.moe_forward_reroute(self.cfg, X, self.Wg, self.gate_bias, self.W1, self.W2, b.out, b.topk_ids,
                                     b.topk_w, b.expert_order, b.expert_counts, b.expert_offsets, b.perm, b.inv_perm,
                                     b.ws, stream=stream)
        else:
            _lib.moe_forward(self.cfg, X, self.Wg, self.gate_bias, self.W1, self.W2, b.out, b.topk_ids, b.topk_w,
                             b.expert_counts, b.expert_offsets, b.perm, b.inv_perm, b.ws, stream=stream)
        return b.out
