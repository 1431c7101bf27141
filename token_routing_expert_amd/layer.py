"""One MoE layer forward on one GPU, as a chain of libmoe355 calls.

The step order is the forward pass of "Expert parallelism"
(zerotofrontier.app), section "Expert parallelism", with the cross-GPU
exchanges removed: route (1), send counts and permute (2), grouped expert
products (5), unpermute and weight (7).  All device buffers are allocated
once here, so ``forward()`` launches kernels only.
"""
from __future__ import annotations

import numpy as np

from . import (moe_grouped_down, moe_grouped_gate_up, moe_grouped_gate_up_gather,
               moe_grouped_swiglu, moe_permute, moe_permute_workspace_bytes, moe_route_topk,
               moe_router_bias_update, moe_router_logits, moe_send_counts, moe_unpermute_combine)
from .inputs import MoeConfig


def to_device(a: np.ndarray, device="cuda"):
    """Host array to a device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    """Device tensor to a host array; bf16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class MoeLayer:
    """Device-resident inputs, weights and every intermediate buffer of one layer.

    fused_gather=True skips the packed copy X[order]: the permute computes
    indices only and the first expert product reads the token rows through
    order itself (moe_grouped_gate_up_gather).  Both paths give the same bits.

    w_router [E, d] (optional) puts the router product in front of the route:
    each forward computes the logits from x.  bias [E] fp32 (optional)
    selects on logits + bias (auxiliary-loss-free balancing); with
    bias_lr != 0 every forward ends with the bias update from that batch's
    per-expert counts, so the next forward routes with the new bias.
    """

    def __init__(self, cfg: MoeConfig, x, w13, w2, logits=None, sh_w13=None, sh_w2=None,
                 topk_ids=None, topk_w=None, device="cuda", fused_gather=False, w_router=None,
                 bias=None, bias_lr=0.0):
        import torch
        self.cfg = cfg
        self.fused_gather = fused_gather
        dev = torch.device(device)
        self.device = dev
        self.x = x if isinstance(x, torch.Tensor) else to_device(x, dev)
        self.w13 = w13 if isinstance(w13, torch.Tensor) else to_device(w13, dev)
        self.w2 = w2 if isinstance(w2, torch.Tensor) else to_device(w2, dev)
        act = self.x.dtype
        T, k, E, d, ffn = cfg.T, cfg.k, cfg.E, cfg.d, cfg.ffn
        M = T * k
        i32 = torch.int32
        if cfg.gating == "given":
            self.logits = None
            self.topk_ids = topk_ids if isinstance(topk_ids, torch.Tensor) else to_device(topk_ids, dev)
            self.topk_w = topk_w if isinstance(topk_w, torch.Tensor) else to_device(topk_w, dev)
        else:
            if w_router is not None:
                self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
            else:
                self.logits = logits if isinstance(logits, torch.Tensor) else to_device(logits, dev)
            self.topk_ids = torch.empty((T, k), dtype=i32, device=dev)
            self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.w_router = None if w_router is None else (
            w_router if isinstance(w_router, torch.Tensor) else to_device(w_router, dev))
        self.bias = None if bias is None else (
            bias if isinstance(bias, torch.Tensor) else to_device(bias, dev))
        self.bias_lr = float(bias_lr)
        self.send_counts = torch.empty((cfg.n_ep, cfg.n_ep), dtype=i32, device=dev) if cfg.n_ep else None
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.order = torch.empty(M, dtype=i32, device=dev)
        self.inv = torch.empty(M, dtype=i32, device=dev)
        self.x_perm = None if fused_gather else torch.empty((M, d), dtype=act, device=dev)
        self.workspace = torch.empty(max(16, moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8,
                                     device=dev)
        self.h = torch.empty((M, ffn), dtype=act, device=dev)
        self.y_perm = torch.empty((M, d), dtype=act, device=dev)
        self.y = torch.empty((T, d), dtype=act, device=dev)
        if cfg.shared:
            self.sh_w13 = sh_w13 if isinstance(sh_w13, torch.Tensor) else to_device(sh_w13, dev)
            self.sh_w2 = sh_w2 if isinstance(sh_w2, torch.Tensor) else to_device(sh_w2, dev)
            self.sh_offsets = torch.tensor([0, T], dtype=i32, device=dev)
            self.sh_h = torch.empty((T, ffn), dtype=act, device=dev)
            self.y_sh = torch.empty((T, d), dtype=act, device=dev)
        else:
            self.y_sh = None

    def router(self, stream=None):
        """The router product logits = x w_router^T (a no-op without w_router)."""
        if self.w_router is not None:
            moe_router_logits(self.x, self.w_router, self.logits, stream=stream)

    def route(self, stream=None):
        c = self.cfg
        if c.gating != "given":
            moe_route_topk(self.logits, c.k, c.gating, c.renormalize, c.n_groups, c.topk_groups,
                           self.topk_ids, self.topk_w, stream=stream, bias=self.bias)
        if c.n_ep:
            moe_send_counts(self.topk_ids, c.E, c.n_ep, self.send_counts, stream=stream)

    def permute(self, stream=None):
        moe_permute(self.x, self.topk_ids, self.cfg.E, self.counts, self.offsets, self.order,
                    self.inv, self.x_perm, self.workspace, stream=stream,
                    rows=not self.fused_gather)

    def experts_routed(self, stream=None):
        if self.fused_gather:
            self.gate_up(stream)
            self.down(stream)
        else:
            moe_grouped_swiglu(self.x_perm, self.offsets, self.w13, self.w2, self.h, self.y_perm,
                               stream=stream)

    def gate_up(self, stream=None):
        """The routed experts' first product alone (the same launch experts_routed makes)."""
        if self.fused_gather:
            moe_grouped_gate_up_gather(self.x, self.order, self.cfg.k, self.offsets, self.w13,
                                       self.h, stream=stream)
        else:
            moe_grouped_gate_up(self.x_perm, self.offsets, self.w13, self.h, stream=stream)

    def down(self, stream=None):
        """The routed experts' second product alone."""
        moe_grouped_down(self.h, self.offsets, self.w2, self.y_perm, stream=stream)

    def experts_shared(self, stream=None):
        if self.cfg.shared:
            moe_grouped_swiglu(self.x, self.sh_offsets, self.sh_w13, self.sh_w2, self.sh_h,
                               self.y_sh, stream=stream)

    def experts(self, stream=None):
        self.experts_routed(stream)
        self.experts_shared(stream)

    def combine(self, stream=None):
        moe_unpermute_combine(self.y_perm, self.inv, self.topk_w, self.y_sh, self.y, stream=stream)

    def bias_update(self, stream=None):
        """bias += bias_lr (mean load - load) from this batch's counts (a no-op
        without a bias or with bias_lr = 0)."""
        if self.bias is not None and self.bias_lr != 0.0:
            moe_router_bias_update(self.counts, self.bias, self.bias_lr, stream=stream)

    def forward(self, stream=None):
        self.router(stream)
        self.route(stream)
        self.permute(stream)
        self.experts(stream)
        self.combine(stream)
        self.bias_update(stream)
        return self.y
