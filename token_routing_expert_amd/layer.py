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


def _upload_into(dst, a):
    """Copy a host array (or device tensor) into the device tensor dst."""
    import torch
    if isinstance(a, torch.Tensor):
        dst.copy_(a)
        return
    a = np.ascontiguousarray(a)
    src = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    dst.copy_(src)


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

    merge_shared puts the always-active shared expert into the routed launches
    as group E (fused-gather path only): its T rows follow the T k packed rows,
    gathered through order entries t k, and its matrices sit after the routed
    experts' in one weight tensor each.  The outputs are the same bits either
    way; at DeepSeek-V3 decode shape the step time is too (the shared expert's
    88 MB stream costs the same inside the routed launches as in its own), so
    the default is off.

    w_router [E, d] (optional) puts the router product in front of the route:
    each forward computes the logits from x.  bias [E] fp32 (optional)
    selects on logits + bias (auxiliary-loss-free balancing); with
    bias_lr != 0 every forward ends with the bias update from that batch's
    per-expert counts, so the next forward routes with the new bias.
    """

    def __init__(self, cfg: MoeConfig, x, w13, w2, logits=None, sh_w13=None, sh_w2=None,
                 topk_ids=None, topk_w=None, device="cuda", fused_gather=False, w_router=None,
                 bias=None, bias_lr=0.0, merge_shared=False):
        import torch
        self.cfg = cfg
        self.fused_gather = fused_gather
        if merge_shared and not (fused_gather and cfg.shared):
            raise ValueError("merge_shared needs the fused-gather path and a shared expert")
        self.merge_shared = bool(merge_shared)
        dev = torch.device(device)
        self.device = dev
        self.x = x if isinstance(x, torch.Tensor) else to_device(x, dev)
        act = self.x.dtype
        T, k, E, d, ffn = cfg.T, cfg.k, cfg.E, cfg.d, cfg.ffn
        M = T * k
        i32 = torch.int32
        if self.merge_shared:
            # Routed experts 0 .. E-1, then the shared expert as group E.
            self.w13_all = torch.empty((E + 1, 2, ffn, d), dtype=act, device=dev)
            self.w2_all = torch.empty((E + 1, d, ffn), dtype=act, device=dev)
            _upload_into(self.w13_all[:E], w13)
            _upload_into(self.w2_all[:E], w2)
            _upload_into(self.w13_all[E:], sh_w13)
            _upload_into(self.w2_all[E:], sh_w2)
            self.w13, self.w2 = self.w13_all[:E], self.w2_all[:E]
        else:
            self.w13 = w13 if isinstance(w13, torch.Tensor) else to_device(w13, dev)
            self.w2 = w2 if isinstance(w2, torch.Tensor) else to_device(w2, dev)
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
        self.inv = torch.empty(M, dtype=i32, device=dev)
        self.x_perm = None if fused_gather else torch.empty((M, d), dtype=act, device=dev)
        self.workspace = torch.empty(max(16, moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8,
                                     device=dev)
        self.y = torch.empty((T, d), dtype=act, device=dev)
        if self.merge_shared:
            # The permute writes the first M (E + 1) entries; the shared group's
            # entries are fixed: order[M + t] = t k, offsets[E + 1] = M + T.
            R = M + T
            self.order_all = torch.empty(R, dtype=i32, device=dev)
            self.order_all[M:] = torch.arange(T, dtype=i32, device=dev) * k
            self.offsets_all = torch.empty(E + 2, dtype=i32, device=dev)
            self.offsets_all[E + 1] = R
            self.order, self.offsets = self.order_all[:M], self.offsets_all[:E + 1]
            self.h = torch.empty((R, ffn), dtype=act, device=dev)
            self.y_perm_all = torch.empty((R, d), dtype=act, device=dev)
            self.y_perm, self.y_sh = self.y_perm_all[:M], self.y_perm_all[M:]
        else:
            self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
            self.order = torch.empty(M, dtype=i32, device=dev)
            self.h = torch.empty((M, ffn), dtype=act, device=dev)
            self.y_perm = torch.empty((M, d), dtype=act, device=dev)
        if self.merge_shared:
            self.sh_w13, self.sh_w2 = self.w13_all[E:], self.w2_all[E:]
        elif cfg.shared:
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
        if self.merge_shared:
            moe_grouped_gate_up_gather(self.x, self.order_all, self.cfg.k, self.offsets_all,
                                       self.w13_all, self.h, stream=stream)
        elif self.fused_gather:
            moe_grouped_gate_up_gather(self.x, self.order, self.cfg.k, self.offsets, self.w13,
                                       self.h, stream=stream)
        else:
            moe_grouped_gate_up(self.x_perm, self.offsets, self.w13, self.h, stream=stream)

    def down(self, stream=None):
        """The routed experts' second product alone."""
        if self.merge_shared:
            moe_grouped_down(self.h, self.offsets_all, self.w2_all, self.y_perm_all, stream=stream)
        else:
            moe_grouped_down(self.h, self.offsets, self.w2, self.y_perm, stream=stream)

    def experts_shared(self, stream=None):
        """The shared expert's own launches (with merge_shared its rows are
        part of the routed launches and this does nothing)."""
        if self.cfg.shared and not self.merge_shared:
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
