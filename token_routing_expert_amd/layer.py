"""One MoE layer forward on one GPU, as a chain of libmoe355 calls.

The step order is the forward pass of "Expert parallelism"
(zerotofrontier.app), section "Expert parallelism", with the cross-GPU
exchanges removed: route (1), send counts and permute (2), grouped expert
products (5), unpermute and weight (7).  All device buffers are allocated
once here, so ``forward()`` launches kernels only.
"""
from __future__ import annotations

import numpy as np

from . import (MoeError, moe_combine_backward, moe_gate_backward, moe_grouped_down,
               moe_expert_capacity, moe_expert_loop_swiglu, moe_permute_capacity,
               moe_permute_capacity_workspace_bytes,
               moe_router_backward,
               moe_grouped_down_backward, moe_grouped_gate_up, moe_grouped_gate_up_backward,
               moe_grouped_gate_up_gather, moe_grouped_gate_up_save, moe_grouped_swiglu,
               moe_grouped_weight_grad, moe_permute, moe_permute_workspace_bytes, moe_route_topk,
               moe_router_bias_update, moe_router_logits, moe_send_counts, moe_unpermute_combine,
               moe_dense_swiglu, moe_dense_swiglu_workspace_bytes)
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

    capacity_factor (a number) runs the experts the second of the three ways
    "Expert parallelism", section "Token permutation and grouped GEMMs", sets
    out: every expert's block padded (or cut) to cap = ceil(CF T k / E) rows
    and one batched product over the E blocks; an expert's assignments past
    its cap are dropped and add nothing to the combine.  The permute then
    writes block-padded order and inv (moe_permute_capacity), the products run
    over E cap rows, and the combine skips dropped slots.

    expert_loop=True runs them the first way: one product pair per expert
    (moe_expert_loop_swiglu), on the packed rows X[order], with the segment
    sizes copied to the host in every step.

    train=True keeps what the backward needs: the first product also stores
    the pre-activations gu, and ``backward(dy)`` then returns the gradients
    of the layer (bf16 or fp32; with a router product bf16).  The packed
    rows X[order] are kept too (the
    permute writes them even on the fused-gather path; not with
    merge_shared): the first product's weight gradient reads them as
    contiguous rows.  The backward is the forward's steps in
    reverse ("Expert parallelism", section "How many bytes move"): the
    combine's gradient goes out to the expert rows, through the two products
    (input and weight gradients), and back into the tokens.
    """

    def __init__(self, cfg: MoeConfig, x, w13, w2, logits=None, sh_w13=None, sh_w2=None,
                 topk_ids=None, topk_w=None, device="cuda", fused_gather=False, w_router=None,
                 bias=None, bias_lr=0.0, merge_shared=False, train=False, capacity_factor=None,
                 expert_loop=False):
        import torch
        self.cfg = cfg
        self.train = bool(train)
        self.fused_gather = fused_gather
        self.capacity_factor = capacity_factor
        self.expert_loop = bool(expert_loop)
        if (capacity_factor is not None or expert_loop) and (train or merge_shared):
            raise ValueError("capacity_factor / expert_loop: forward only, shared expert not merged")
        if capacity_factor is not None and expert_loop:
            raise ValueError("capacity_factor and expert_loop are two different forms")
        if expert_loop and fused_gather:
            raise ValueError("expert_loop runs on the packed rows (fused_gather=False)")
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
        # Rows of the expert products: M packed rows, or E cap block rows.
        self.cap = None if capacity_factor is None else moe_expert_capacity(M, E, capacity_factor)
        R = M if self.cap is None else E * self.cap
        self.rows = R
        keep_rows = not fused_gather or (self.train and not merge_shared)
        self.x_perm = torch.empty((R, d), dtype=act, device=dev) if keep_rows else None
        ws = moe_permute_workspace_bytes(T, k, E) if self.cap is None else \
            moe_permute_capacity_workspace_bytes(T, k, E)
        self.workspace = torch.empty(max(16, ws), dtype=torch.uint8, device=dev)
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
            self.order = torch.empty(R, dtype=i32, device=dev)
            self.h = torch.empty((R, ffn), dtype=act, device=dev)
            self.y_perm = torch.empty((R, d), dtype=act, device=dev)
        if self.merge_shared:
            self.sh_w13, self.sh_w2 = self.w13_all[E:], self.w2_all[E:]
        elif cfg.shared:
            self.sh_w13 = sh_w13 if isinstance(sh_w13, torch.Tensor) else to_device(sh_w13, dev)
            self.sh_w2 = sh_w2 if isinstance(sh_w2, torch.Tensor) else to_device(sh_w2, dev)
            self.sh_offsets = torch.tensor([0, T], dtype=i32, device=dev)
            self.sh_h = torch.empty((T, ffn), dtype=act, device=dev)
            self.y_sh = torch.empty((T, d), dtype=act, device=dev)
            # A shared expert over few tokens (decode) splits its reductions
            # over many workgroups (moe_dense_swiglu) instead of tiling by
            # output columns alone, which leaves most CUs idle.
            self.sh_dense = act == torch.bfloat16 and 0 < T <= 256 and d % 64 == 0 and ffn % 64 == 0
            if self.sh_dense:
                self.sh_ws = torch.empty(moe_dense_swiglu_workspace_bytes(T, d, ffn), dtype=torch.uint8,
                                         device=dev)
        else:
            self.y_sh = None
        if self.train:
            if act != torch.bfloat16 and self.w_router is not None:
                raise MoeError("train=True with a router product needs bf16")
            self.gu = torch.empty((self.h.shape[0], 2 * ffn), dtype=act, device=dev)
            if cfg.shared and not self.merge_shared:
                self.sh_gu = torch.empty((T, 2 * ffn), dtype=act, device=dev)
        self._grads = None

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
        if self.cap is not None:
            moe_permute_capacity(self.x, self.topk_ids, self.cfg.E, self.cap, self.counts,
                                 self.offsets, self.order, self.inv, self.x_perm, self.workspace,
                                 stream=stream, rows=self.x_perm is not None)
            return
        moe_permute(self.x, self.topk_ids, self.cfg.E, self.counts, self.offsets, self.order,
                    self.inv, self.x_perm, self.workspace, stream=stream,
                    rows=self.x_perm is not None)

    def experts_routed(self, stream=None):
        if self.expert_loop:
            moe_expert_loop_swiglu(self.x_perm, self.offsets, self.w13, self.w2, self.h, self.y_perm,
                                   stream=stream)
            return
        if self.fused_gather or self.train:
            self.gate_up(stream)
            self.down(stream)
        else:
            moe_grouped_swiglu(self.x_perm, self.offsets, self.w13, self.w2, self.h, self.y_perm,
                               stream=stream)

    def gate_up(self, stream=None):
        """The routed experts' first product alone (the same launch experts_routed makes)."""
        if self.expert_loop:
            # The loop form's launches come in pairs per expert: both products
            # run here, down() has nothing left to do.
            self.experts_routed(stream)
            return
        if self.train:
            if self.merge_shared:
                moe_grouped_gate_up_save(self.x, self.offsets_all, self.w13_all, self.h, self.gu,
                                         order=self.order_all, k=self.cfg.k, stream=stream)
            elif self.fused_gather:
                moe_grouped_gate_up_save(self.x, self.offsets, self.w13, self.h, self.gu,
                                         order=self.order, k=self.cfg.k, stream=stream)
            else:
                moe_grouped_gate_up_save(self.x_perm, self.offsets, self.w13, self.h, self.gu,
                                         stream=stream)
        elif self.merge_shared:
            moe_grouped_gate_up_gather(self.x, self.order_all, self.cfg.k, self.offsets_all,
                                       self.w13_all, self.h, stream=stream)
        elif self.fused_gather:
            moe_grouped_gate_up_gather(self.x, self.order, self.cfg.k, self.offsets, self.w13,
                                       self.h, stream=stream)
        else:
            moe_grouped_gate_up(self.x_perm, self.offsets, self.w13, self.h, stream=stream)

    def down(self, stream=None):
        """The routed experts' second product alone."""
        if self.expert_loop:
            return
        if self.merge_shared:
            moe_grouped_down(self.h, self.offsets_all, self.w2_all, self.y_perm_all, stream=stream)
        else:
            moe_grouped_down(self.h, self.offsets, self.w2, self.y_perm, stream=stream)

    def experts_shared(self, stream=None):
        """The shared expert's own launches (with merge_shared its rows are
        part of the routed launches and this does nothing)."""
        if self.cfg.shared and not self.merge_shared:
            if self.sh_dense:
                moe_dense_swiglu(self.x, self.sh_w13, self.sh_w2, h=self.sh_h,
                                 gu=self.sh_gu if self.train else None, y=self.y_sh,
                                 workspace=self.sh_ws, stream=stream)
            elif self.train:
                moe_grouped_gate_up_save(self.x, self.sh_offsets, self.sh_w13, self.sh_h,
                                         self.sh_gu, stream=stream)
                moe_grouped_down(self.sh_h, self.sh_offsets, self.sh_w2, self.y_sh, stream=stream)
            else:
                moe_grouped_swiglu(self.x, self.sh_offsets, self.sh_w13, self.sh_w2, self.sh_h,
                                   self.y_sh, stream=stream)

    def experts(self, stream=None):
        self.experts_routed(stream)
        self.experts_shared(stream)

    def combine(self, stream=None):
        moe_unpermute_combine(self.y_perm, self.inv, self.topk_w, self.y_sh, self.y, stream=stream,
                              rows=self.rows if self.cap is not None else None)

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

    # ------------------------------------------------------------------
    # Backward (train=True)
    # ------------------------------------------------------------------

    def _grad_buffers(self):
        """Every buffer of the backward, allocated on its first call."""
        if self._grads is not None:
            return self._grads
        import torch
        c, dev, act = self.cfg, self.device, self.x.dtype
        T, k, E, d, ffn = c.T, c.k, c.E, c.d, c.ffn
        M = T * k
        R = self.h.shape[0]             # M, or M + T with the shared expert merged
        G = E + 1 if self.merge_shared else E
        b = {
            "dy_perm": torch.empty((R, d), dtype=act, device=dev),
            "dgu": torch.empty((R, 2 * ffn), dtype=act, device=dev),
            "dx_perm": torch.empty((R, d), dtype=act, device=dev),
            "dx": torch.empty((T, d), dtype=act, device=dev),
            "dw13": torch.empty((G, 2, ffn, d), dtype=act, device=dev),
            "dw2": torch.empty((G, d, ffn), dtype=act, device=dev),
        }
        if c.gating != "given":
            b["dgate"] = torch.empty((T, k), dtype=torch.float32, device=dev)
            b["dlogits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
        if self.w_router is not None:
            from . import moe_router_backward_workspace_bytes
            b["dw_router"] = torch.empty((E, d), dtype=act, device=dev)
            b["router_ws"] = torch.empty(max(16, moe_router_backward_workspace_bytes(T, E)),
                                         dtype=torch.uint8, device=dev)
        if c.shared and not self.merge_shared:
            b["sh_dgu"] = torch.empty((T, 2 * ffn), dtype=act, device=dev)
            b["dx_sh"] = torch.empty((T, d), dtype=act, device=dev)
            b["dsh_w13"] = torch.empty((1, 2, ffn, d), dtype=act, device=dev)
            b["dsh_w2"] = torch.empty((1, d, ffn), dtype=act, device=dev)
        self._grads = b
        return b

    # The backward's steps, in order (BACKWARD_STAGES); backward() runs them
    # all.  Each takes the output gradient dy [T, d].
    BACKWARD_STAGES = ("bwd_combine", "bwd_down", "bwd_gate_up", "bwd_wgrad_down",
                       "bwd_wgrad_gate_up", "bwd_shared", "bwd_dx", "bwd_gates", "bwd_router")

    def _bwd_views(self):
        merged = self.merge_shared
        return (self.offsets_all if merged else self.offsets, self.w13_all if merged else self.w13,
                self.w2_all if merged else self.w2, self.order_all if merged else self.order)

    def bwd_combine(self, dy, stream=None):
        """The combine's backward: the gradient goes out to the expert rows
        (scaled by the gates), the gate gradients come back."""
        b, M = self._grad_buffers(), self.cfg.T * self.cfg.k
        merged = self.merge_shared
        moe_combine_backward(dy, self.inv, self.topk_w, self.y_perm if "dgate" in b else None,
                             b["dy_perm"][:M] if merged else b["dy_perm"], b.get("dgate"),
                             b["dy_perm"][M:] if merged else None, stream=stream,
                             want_dgate="dgate" in b)

    def bwd_down(self, dy, stream=None):
        """Second product's input gradient and the SwiGLU backward: dgu."""
        b = self._grad_buffers()
        offsets, _, w2, _ = self._bwd_views()
        moe_grouped_down_backward(b["dy_perm"], offsets, w2, self.gu, b["dgu"], stream=stream)

    def bwd_gate_up(self, dy, stream=None):
        """First product's input gradient: the packed rows' dx_perm."""
        b = self._grad_buffers()
        offsets, w13, _, _ = self._bwd_views()
        moe_grouped_gate_up_backward(b["dgu"], offsets, w13, b["dx_perm"], stream=stream)

    def bwd_wgrad_down(self, dy, stream=None):
        """Weight gradient of the second product: dW_down,e = dy_perm^T h."""
        b = self._grad_buffers()
        offsets, _, _, _ = self._bwd_views()
        moe_grouped_weight_grad(b["dy_perm"], self.h, offsets, b["dw2"], stream=stream)

    def bwd_wgrad_gate_up(self, dy, stream=None):
        """Weight gradient of the first product: dW13,e = dgu^T x rows."""
        b, c = self._grad_buffers(), self.cfg
        offsets, _, _, order = self._bwd_views()
        if self.x_perm is not None and not self.merge_shared:
            moe_grouped_weight_grad(b["dgu"], self.x_perm, offsets, b["dw13"], stream=stream)
        else:
            moe_grouped_weight_grad(b["dgu"], self.x, offsets, b["dw13"], b_order=order, b_k=c.k,
                                    stream=stream)

    def bwd_shared(self, dy, stream=None):
        """The shared expert's own backward launches (merged: nothing to do)."""
        c, b = self.cfg, self._grad_buffers()
        if not c.shared or self.merge_shared:
            return
        moe_grouped_down_backward(dy, self.sh_offsets, self.sh_w2, self.sh_gu, b["sh_dgu"],
                                  stream=stream)
        moe_grouped_gate_up_backward(b["sh_dgu"], self.sh_offsets, self.sh_w13, b["dx_sh"],
                                     stream=stream)
        moe_grouped_weight_grad(dy, self.sh_h, self.sh_offsets, b["dsh_w2"], stream=stream)
        moe_grouped_weight_grad(b["sh_dgu"], self.x, self.sh_offsets, b["dsh_w13"], stream=stream)

    def bwd_dx(self, dy, stream=None):
        """The dispatch's gradient combined back into the tokens (+ shared)."""
        c, b, M = self.cfg, self._grad_buffers(), self.cfg.T * self.cfg.k
        if self.merge_shared:
            rows, dx_sh = b["dx_perm"][:M], b["dx_perm"][M:]
        else:
            rows, dx_sh = b["dx_perm"], b["dx_sh"] if c.shared else None
        moe_unpermute_combine(rows, self.inv, None, dx_sh, b["dx"], stream=stream, k=c.k)

    def bwd_gates(self, dy, stream=None):
        """The gates' backward to the logits (nothing when the gates are given)."""
        c, b = self.cfg, self._grad_buffers()
        if "dgate" in b:
            moe_gate_backward(self.logits, self.topk_ids, self.topk_w, b["dgate"], c.gating,
                              c.renormalize, b["dlogits"], stream=stream)

    def bwd_router(self, dy, stream=None):
        """The router product's backward: dx += dlogits w_router, dw_router
        (nothing without a router)."""
        if self.w_router is None:
            return
        b = self._grad_buffers()
        moe_router_backward(b["dlogits"], self.x, self.w_router, b["dx"], b["dw_router"],
                            b["router_ws"], stream=stream)

    def backward(self, dy, stream=None):
        """Gradients of the layer at its last forward, for the output gradient
        dy [T, d].  Returns a dict of device tensors: dx, dw13, dw2, and when
        present dgate and dlogits (through the gates), dsh_w13, dsh_w2 (shared
        expert), dw_router (router product; dx then includes its part).  The
        buffers are reused by the next call."""
        if not self.train:
            raise MoeError("backward() needs a layer built with train=True")
        for name in self.BACKWARD_STAGES:
            getattr(self, name)(dy, stream)
        c, b = self.cfg, self._grad_buffers()
        out = {"dx": b["dx"]}
        if self.merge_shared:
            out.update(dw13=b["dw13"][:c.E], dw2=b["dw2"][:c.E], dsh_w13=b["dw13"][c.E:],
                       dsh_w2=b["dw2"][c.E:])
        else:
            out.update(dw13=b["dw13"], dw2=b["dw2"])
            if c.shared:
                out.update(dsh_w13=b["dsh_w13"], dsh_w2=b["dsh_w2"])
        if "dgate" in b:
            out.update(dlogits=b["dlogits"], dgate=b["dgate"])
        if "dw_router" in b:
            out["dw_router"] = b["dw_router"]
        return out
