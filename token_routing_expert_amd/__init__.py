"""Python binding of libmoe355: argument marshalling only.

Each function has the name of the C entry point it calls (include/moe355.h),
takes torch CUDA tensors, passes their device pointers and the current HIP
stream, and raises ``MoeError`` on a non-zero status.  Every step of the path
runs in the library's HIP kernels; PyTorch only supplies device memory (output
tensors are allocated with ``torch.empty`` when not given) and the stream.
There is no fallback: if libmoe355.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe355.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1

# Every symbol include/moe355.h declares.
EXPORTS = ("moe_status_string", "moe_route_topk", "moe_route_topk_biased", "moe_router_logits",
           "moe_router_bias_update", "moe_sigmoid_pinned", "moe_send_counts",
           "moe_permute_workspace_bytes", "moe_permute", "moe_grouped_swiglu",
           "moe_grouped_gate_up", "moe_grouped_gate_up_gather", "moe_grouped_down",
           "moe_unpermute_combine", "moe_grouped_gate_up_save", "moe_combine_backward",
           "moe_gate_backward", "moe_grouped_down_backward", "moe_grouped_gate_up_backward",
           "moe_grouped_weight_grad", "moe_router_backward_workspace_bytes",
           "moe_router_backward", "moe_dense_swiglu_workspace_bytes", "moe_dense_swiglu",
           "moe_unpermute_combine_rows", "moe_expert_capacity",
           "moe_permute_capacity_workspace_bytes", "moe_permute_capacity", "moe_expert_loop_swiglu",
           "moe_permute_noalloc")


class MoeError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe355.so and declare the C signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise MoeError(f"{path} is not built; run `python -m token_routing_expert_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route_topk.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.moe_route_topk_biased.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.moe_router_logits.argtypes = [P, i32, i32, i32, P, i32, P, P]
    lib.moe_router_bias_update.argtypes = [P, i32, ctypes.c_float, P, P]
    lib.moe_sigmoid_pinned.argtypes = [P, P, i64, P]
    lib.moe_send_counts.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.moe_permute_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_permute_workspace_bytes.restype = sz
    lib.moe_permute.argtypes = [P, i32, i32, i32, P, i32, i32, P, P, P, P, P, P, sz, P]
    lib.moe_grouped_swiglu.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P, P, P]
    lib.moe_grouped_gate_up.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P]
    lib.moe_grouped_gate_up_gather.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, i32, P, P, P]
    lib.moe_grouped_down.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P]
    lib.moe_unpermute_combine.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P]
    lib.moe_grouped_gate_up_save.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, i32, P, P, P, P]
    lib.moe_combine_backward.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P]
    lib.moe_gate_backward.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, P]
    lib.moe_grouped_down_backward.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P, P]
    lib.moe_grouped_gate_up_backward.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P]
    lib.moe_grouped_weight_grad.argtypes = [P, P, i32, i32, i32, i32, P, i32, P, i32, i32, P, P]
    lib.moe_router_backward_workspace_bytes.argtypes = [i32, i32]
    lib.moe_router_backward_workspace_bytes.restype = sz
    lib.moe_router_backward.argtypes = [P, P, i32, i32, i32, P, i32, P, P, P, sz, P]
    lib.moe_dense_swiglu_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_dense_swiglu_workspace_bytes.restype = sz
    lib.moe_dense_swiglu.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, sz, P]
    lib.moe_unpermute_combine_rows.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P]
    lib.moe_expert_capacity.argtypes = [i64, i32, ctypes.c_double]
    lib.moe_expert_capacity.restype = i64
    lib.moe_permute_capacity_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_permute_capacity_workspace_bytes.restype = sz
    lib.moe_permute_capacity.argtypes = [P, i32, i32, i32, P, i32, i32, i32, P, P, P, P, P, P, sz, P]
    lib.moe_expert_loop_swiglu.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, P, P, P, P]
    lib.moe_permute_noalloc.argtypes = [P, i32, i32, i32, P, i32, i32, P, P, P, P, P, P]
    for name in ("moe_route_topk", "moe_route_topk_biased", "moe_router_logits",
                 "moe_router_bias_update", "moe_sigmoid_pinned", "moe_send_counts", "moe_permute",
                 "moe_grouped_swiglu", "moe_grouped_gate_up", "moe_grouped_gate_up_gather",
                 "moe_grouped_down", "moe_unpermute_combine", "moe_grouped_gate_up_save",
                 "moe_combine_backward", "moe_gate_backward", "moe_grouped_down_backward",
                 "moe_grouped_gate_up_backward", "moe_grouped_weight_grad", "moe_router_backward",
                 "moe_dense_swiglu", "moe_unpermute_combine_rows", "moe_permute_capacity",
                 "moe_expert_loop_swiglu", "moe_permute_noalloc"):
        getattr(lib, name).restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().moe_status_string(rc).decode()
        raise MoeError(f"{what}: {msg}")


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, name, dtypes):
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise MoeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _shape(t, shape, name, what):
    """Raise unless t (an output buffer the kernels write from the sizes they
    are given) has exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(f"{what}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _dtype_code(t) -> int:
    torch = _torch()
    return MOE_BF16 if t.dtype == torch.bfloat16 else MOE_F32


def _act_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def moe_sigmoid_pinned(x, y=None, stream=None):
    torch = _torch()
    _dev(x, "x", (torch.float32,))
    y = torch.empty_like(x) if y is None else _dev(y, "y", (torch.float32,))
    _check(load_library().moe_sigmoid_pinned(_ptr(x), _ptr(y), x.numel(), _stream(stream)),
           "moe_sigmoid_pinned")
    return y


def moe_route_topk(logits, k, gating="softmax", renormalize=True, n_groups=1, topk_groups=1,
                   topk_ids=None, topk_w=None, stream=None, bias=None):
    """Top-k ids [T,k] int32 and gates [T,k] fp32 from fp32 logits [T,E].

    bias [E] fp32 (optional) selects through moe_route_topk_biased: the
    choice on logits + bias, the gates on the logits."""
    torch = _torch()
    _dev(logits, "logits", (torch.float32,))
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,))
    _shape(topk_ids, (T, k), "topk_ids", "moe_route_topk")
    _shape(topk_w, (T, k), "topk_w", "moe_route_topk")
    g = MOE_SOFTMAX if gating == "softmax" else MOE_SIGMOID if gating == "sigmoid" else -1
    lib = load_library()
    if bias is None:
        _check(lib.moe_route_topk(_ptr(logits), T, E, k, g, int(bool(renormalize)), n_groups,
                                  topk_groups, _ptr(topk_ids), _ptr(topk_w), _stream(stream)),
               "moe_route_topk")
    else:
        _dev(bias, "bias", (torch.float32,))
        if bias.numel() != E:
            raise MoeError("moe_route_topk_biased: bias must have one entry per expert")
        _check(lib.moe_route_topk_biased(_ptr(logits), _ptr(bias), T, E, k, g,
                                         int(bool(renormalize)), n_groups, topk_groups,
                                         _ptr(topk_ids), _ptr(topk_w), _stream(stream)),
               "moe_route_topk_biased")
    return topk_ids, topk_w


def moe_router_logits(x, w_router, logits=None, stream=None):
    """logits [T,E] fp32 = x [T,d] . w_router [E,d]^T (fp32 accumulation)."""
    torch = _torch()
    _dev(x, "x", _act_dtypes())
    _dev(w_router, "w_router", (x.dtype,))
    T, d = x.shape
    E, d2 = w_router.shape
    if d2 != d:
        raise MoeError("moe_router_logits: w_router must be [E, d]")
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if logits is None else logits
    _dev(logits, "logits", (torch.float32,))
    _shape(logits, (T, E), "logits", "moe_router_logits")
    _check(load_library().moe_router_logits(_ptr(x), _dtype_code(x), T, d, _ptr(w_router), E,
                                            _ptr(logits), _stream(stream)), "moe_router_logits")
    return logits


def moe_router_bias_update(counts, bias, lr, stream=None):
    """bias [E] += lr (mean(counts) - counts), in place (fp32, one rounding per operation)."""
    torch = _torch()
    _dev(counts, "counts", (torch.int32,))
    _dev(bias, "bias", (torch.float32,))
    if counts.numel() != bias.numel():
        raise MoeError("moe_router_bias_update: counts and bias must have E entries each")
    _check(load_library().moe_router_bias_update(_ptr(counts), counts.numel(), float(lr),
                                                 _ptr(bias), _stream(stream)),
           "moe_router_bias_update")
    return bias


def moe_send_counts(topk_ids, E, n_ep, send_counts=None, stream=None):
    """Send-count matrix [n_ep, n_ep] int32 (row = source rank)."""
    torch = _torch()
    _dev(topk_ids, "topk_ids", (torch.int32,))
    T, k = topk_ids.shape
    if send_counts is None:
        send_counts = torch.empty((n_ep, n_ep), dtype=torch.int32, device=topk_ids.device)
    _dev(send_counts, "send_counts", (torch.int32,))
    _shape(send_counts, (n_ep, n_ep), "send_counts", "moe_send_counts")
    _check(load_library().moe_send_counts(_ptr(topk_ids), T, k, E, n_ep, _ptr(send_counts),
                                          _stream(stream)), "moe_send_counts")
    return send_counts


def moe_permute_workspace_bytes(T, k, E) -> int:
    return int(load_library().moe_permute_workspace_bytes(T, k, E))


def moe_permute(x, topk_ids, E, counts=None, offsets=None, order=None, inv=None, x_perm=None,
                workspace=None, stream=None, rows=True):
    """Returns (counts [E], offsets [E+1], order [Tk], inv [Tk], x_perm [Tk, d]).

    rows=False is the index-only mode: x only gives T and d, no row is copied
    and x_perm is returned as None.
    """
    torch = _torch()
    _dev(x, "x", _act_dtypes())
    _dev(topk_ids, "topk_ids", (torch.int32,))
    T, d = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    M = T * k
    i32 = torch.int32
    counts = torch.empty(E, dtype=i32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=i32, device=dev) if offsets is None else offsets
    order = torch.empty(M, dtype=i32, device=dev) if order is None else order
    inv = torch.empty(M, dtype=i32, device=dev) if inv is None else inv
    if rows:
        x_perm = torch.empty((M, d), dtype=x.dtype, device=dev) if x_perm is None else x_perm
    elif x_perm is not None:
        raise MoeError("moe_permute: x_perm given in index-only mode")
    nbytes = moe_permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    for name, t, n in (("counts", counts, E), ("offsets", offsets, E + 1), ("order", order, M),
                       ("inv", inv, M)):
        _dev(t, name, (i32,))
        _shape(t, (n,), name, "moe_permute")
    if rows:
        _dev(x_perm, "x_perm", (x.dtype,))
        _shape(x_perm, (M, d), "x_perm", "moe_permute")
    _check(load_library().moe_permute(
        _ptr(x) if rows else None, _dtype_code(x), T, d, _ptr(topk_ids), k, E, _ptr(counts),
        _ptr(offsets), _ptr(order), _ptr(inv), _ptr(x_perm), _ptr(workspace), workspace.numel(),
        _stream(stream)), "moe_permute")
    return counts, offsets, order, inv, x_perm


def moe_permute_noalloc(x, topk_ids, E, counts, offsets, order, inv, x_perm=None, stream=None):
    """moe_permute without a workspace: the library's own device scratch holds
    the histograms, so the call allocates nothing (every output must be
    given; x_perm None is the index-only mode).  Returns the outputs."""
    torch = _torch()
    _dev(x, "x", _act_dtypes())
    _dev(topk_ids, "topk_ids", (torch.int32,))
    T, d = x.shape
    k = topk_ids.shape[1]
    M = T * k
    for name, t, n in (("counts", counts, E), ("offsets", offsets, E + 1), ("order", order, M),
                       ("inv", inv, M)):
        _dev(t, name, (torch.int32,))
        _shape(t, (n,), name, "moe_permute_noalloc")
    if x_perm is not None:
        _dev(x_perm, "x_perm", (x.dtype,))
        _shape(x_perm, (M, d), "x_perm", "moe_permute_noalloc")
    rows = x_perm is not None
    _check(load_library().moe_permute_noalloc(
        _ptr(x) if rows else None, _dtype_code(x), T, d, _ptr(topk_ids), k, E, _ptr(counts),
        _ptr(offsets), _ptr(order), _ptr(inv), _ptr(x_perm), _stream(stream)), "moe_permute_noalloc")
    return counts, offsets, order, inv, x_perm


def moe_grouped_swiglu(a, offsets, w13, w2, h=None, y=None, stream=None):
    """y [M, d] = per-segment SwiGLU experts of the packed rows a [M, d]; h is scratch."""
    torch = _torch()
    _dev(a, "a", _act_dtypes())
    _dev(offsets, "offsets", (torch.int32,))
    _dev(w13, "w13", (a.dtype,))
    _dev(w2, "w2", (a.dtype,))
    M, d = a.shape
    G, two, ffn, d2 = w13.shape
    if two != 2 or d2 != d or tuple(w2.shape) != (G, d, ffn) or offsets.numel() != G + 1:
        raise MoeError("moe_grouped_swiglu: inconsistent shapes")
    h = torch.empty((M, ffn), dtype=a.dtype, device=a.device) if h is None else h
    y = torch.empty((M, d), dtype=a.dtype, device=a.device) if y is None else y
    _dev(h, "h", (a.dtype,))
    _dev(y, "y", (a.dtype,))
    _shape(h, (M, ffn), "h", "moe_grouped_swiglu")
    _shape(y, (M, d), "y", "moe_grouped_swiglu")
    _check(load_library().moe_grouped_swiglu(_ptr(a), _dtype_code(a), M, d, ffn, _ptr(offsets),
                                             G, _ptr(w13), _ptr(w2), _ptr(h), _ptr(y),
                                             _stream(stream)), "moe_grouped_swiglu")
    return y


def moe_dense_swiglu_workspace_bytes(M, d, ffn) -> int:
    return int(load_library().moe_dense_swiglu_workspace_bytes(M, d, ffn))


def moe_dense_swiglu(x, w13, w2, h=None, gu=None, y=None, workspace=None, stream=None):
    """One expert's SwiGLU MLP on few rows (at most 256) with split reductions:
    x [M, d], w13 [2, ffn, d] (or [1, 2, ffn, d]), w2 [d, ffn] (or [1, d, ffn]);
    returns y [M, d].  gu, when given, receives the pre-activations [M, 2 ffn]."""
    torch = _torch()
    _dev(x, "x", (torch.bfloat16,))
    w13 = w13[0] if w13.dim() == 4 else w13
    w2 = w2[0] if w2.dim() == 3 else w2
    _dev(w13, "w13", (x.dtype,))
    _dev(w2, "w2", (x.dtype,))
    M, d = x.shape
    two, ffn, d2 = w13.shape
    if two != 2 or d2 != d or tuple(w2.shape) != (d, ffn):
        raise MoeError("moe_dense_swiglu: inconsistent shapes")
    h = torch.empty((M, ffn), dtype=x.dtype, device=x.device) if h is None else h
    y = torch.empty((M, d), dtype=x.dtype, device=x.device) if y is None else y
    _dev(h, "h", (x.dtype,))
    _dev(y, "y", (x.dtype,))
    _shape(h, (M, ffn), "h", "moe_dense_swiglu")
    _shape(y, (M, d), "y", "moe_dense_swiglu")
    if gu is not None:
        _dev(gu, "gu", (x.dtype,))
        _shape(gu, (M, 2 * ffn), "gu", "moe_dense_swiglu")
    nbytes = moe_dense_swiglu_workspace_bytes(M, d, ffn)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", (torch.uint8,))
    _check(load_library().moe_dense_swiglu(
        _ptr(x), _dtype_code(x), M, d, ffn, _ptr(w13), _ptr(w2), _ptr(h),
        _ptr(gu) if gu is not None else None, _ptr(y), _ptr(workspace), workspace.numel(),
        _stream(stream)), "moe_dense_swiglu")
    return y


def _expert_shapes(name, a, offsets, w13=None, w2=None):
    torch = _torch()
    _dev(a, "a", _act_dtypes())
    _dev(offsets, "offsets", (torch.int32,))
    for wname, w in (("w13", w13), ("w2", w2)):
        if w is not None:
            _dev(w, wname, (a.dtype,))
    G = offsets.numel() - 1
    if w13 is not None and (w13.dim() != 4 or w13.shape[0] != G or w13.shape[1] != 2):
        raise MoeError(f"{name}: w13 must be [G, 2, ffn, d] with G = offsets.numel() - 1")
    if w2 is not None and (w2.dim() != 3 or w2.shape[0] != G):
        raise MoeError(f"{name}: w2 must be [G, d, ffn] with G = offsets.numel() - 1")
    return G


def moe_grouped_gate_up(a, offsets, w13, h=None, stream=None):
    """h [M, ffn] = SiLU(a W_gate^T) * (a W_up^T) per expert segment of the packed rows a [M, d]."""
    G = _expert_shapes("moe_grouped_gate_up", a, offsets, w13=w13)
    M, d = a.shape
    ffn = w13.shape[2]
    if w13.shape[3] != d:
        raise MoeError("moe_grouped_gate_up: inconsistent shapes")
    h = _torch().empty((M, ffn), dtype=a.dtype, device=a.device) if h is None else h
    _dev(h, "h", (a.dtype,))
    _shape(h, (M, ffn), "h", "moe_grouped_gate_up")
    _check(load_library().moe_grouped_gate_up(_ptr(a), _dtype_code(a), M, d, ffn, _ptr(offsets),
                                              G, _ptr(w13), _ptr(h), _stream(stream)),
           "moe_grouped_gate_up")
    return h


def moe_grouped_gate_up_gather(x, order, k, offsets, w13, h=None, stream=None):
    """moe_grouped_gate_up on the rows x[order // k] without materialising them.

    x [T, d] in token order, order [M] (moe_permute's order, M = T k, possibly
    followed by entries t k that repeat token t); returns h [M, ffn].
    """
    torch = _torch()
    G = _expert_shapes("moe_grouped_gate_up_gather", x, offsets, w13=w13)
    _dev(order, "order", (torch.int32,))
    T, d = x.shape
    M = order.numel()
    ffn = w13.shape[2]
    if w13.shape[3] != d:
        raise MoeError("moe_grouped_gate_up_gather: inconsistent shapes")
    h = torch.empty((M, ffn), dtype=x.dtype, device=x.device) if h is None else h
    _dev(h, "h", (x.dtype,))
    _shape(h, (M, ffn), "h", "moe_grouped_gate_up_gather")
    _check(load_library().moe_grouped_gate_up_gather(
        _ptr(x), _dtype_code(x), T, k, M, d, ffn, _ptr(order), _ptr(offsets), G, _ptr(w13),
        _ptr(h), _stream(stream)), "moe_grouped_gate_up_gather")
    return h


def moe_grouped_down(h, offsets, w2, y=None, stream=None):
    """y [M, d] = h W_down^T per expert segment of h [M, ffn]."""
    G = _expert_shapes("moe_grouped_down", h, offsets, w2=w2)
    M, ffn = h.shape
    d = w2.shape[1]
    if w2.shape[2] != ffn:
        raise MoeError("moe_grouped_down: inconsistent shapes")
    y = _torch().empty((M, d), dtype=h.dtype, device=h.device) if y is None else y
    _dev(y, "y", (h.dtype,))
    _shape(y, (M, d), "y", "moe_grouped_down")
    _check(load_library().moe_grouped_down(_ptr(h), _dtype_code(h), M, ffn, d, _ptr(offsets), G,
                                           _ptr(w2), _ptr(y), _stream(stream)), "moe_grouped_down")
    return y


def moe_unpermute_combine(y_perm, inv, topk_w, y_shared=None, y=None, stream=None, k=None,
                          rows=None):
    """y [T, d] = sum_j topk_w[t,j] y_perm[inv[t k + j]] (+ y_shared[t]).

    topk_w None (then k is required): every gate is 1, the sum of a token's
    k rows -- the permute's backward.  rows (optional): y_perm holds this
    many rows (moe_unpermute_combine_rows; inv entries outside [0, rows),
    such as a dropped assignment's -1, add nothing)."""
    torch = _torch()
    _dev(y_perm, "y_perm", _act_dtypes())
    _dev(inv, "inv", (torch.int32,))
    if topk_w is None:
        if not k or inv.numel() % k:
            raise MoeError("moe_unpermute_combine: k must divide inv's length when topk_w is None")
        T = inv.numel() // k
    else:
        _dev(topk_w, "topk_w", (torch.float32,))
        T, k = topk_w.shape
    d = y_perm.shape[1]
    if rows is not None:
        if rows < 0 or y_perm.shape[0] < rows or inv.numel() != T * k:
            raise MoeError("moe_unpermute_combine: inv must have T k entries and y_perm `rows` rows")
    elif y_perm.shape[0] < T * k or inv.numel() != T * k:
        raise MoeError("moe_unpermute_combine: inv must have T k entries and y_perm at least T k rows")
    if y_shared is not None:
        _dev(y_shared, "y_shared", (y_perm.dtype,))
        _shape(y_shared, (T, d), "y_shared", "moe_unpermute_combine")
    y = torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device) if y is None else y
    _dev(y, "y", (y_perm.dtype,))
    _shape(y, (T, d), "y", "moe_unpermute_combine")
    lib = load_library()
    if rows is None:
        _check(lib.moe_unpermute_combine(_ptr(y_perm), _dtype_code(y_perm), T, k, d, _ptr(inv),
                                         _ptr(topk_w), _ptr(y_shared), _ptr(y), _stream(stream)),
               "moe_unpermute_combine")
    else:
        _check(lib.moe_unpermute_combine_rows(_ptr(y_perm), int(rows), _dtype_code(y_perm), T, k, d,
                                              _ptr(inv), _ptr(topk_w), _ptr(y_shared), _ptr(y),
                                              _stream(stream)), "moe_unpermute_combine_rows")
    return y


# --------------------------------------------------------------------------
# The two other ways to run the expert products: padded to a capacity and
# batched, or one product per expert in a loop.
# --------------------------------------------------------------------------

def moe_expert_capacity(M, E, cf) -> int:
    """cap = ceil(cf M / E) rows per expert block (host function)."""
    cap = int(load_library().moe_expert_capacity(int(M), int(E), float(cf)))
    if cap < 0:
        raise MoeError("moe_expert_capacity: E < 1, M < 0 or cf <= 0")
    return cap


def moe_permute_capacity_workspace_bytes(T, k, E) -> int:
    return int(load_library().moe_permute_capacity_workspace_bytes(T, k, E))


def moe_permute_capacity(x, topk_ids, E, cap, counts=None, offsets=None, order=None, inv=None,
                         x_cap=None, workspace=None, stream=None, rows=True):
    """Pad to capacity: returns (counts [E] before the cap, offsets [E+1] = e cap,
    order [E cap] (-1: padding slot), inv [T k] (-1: dropped), x_cap [E cap, d]
    or None in index-only mode (rows=False))."""
    torch = _torch()
    _dev(x, "x", _act_dtypes())
    _dev(topk_ids, "topk_ids", (torch.int32,))
    T, d = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise MoeError("moe_permute_capacity: topk_ids must have one row per token of x")
    dev, i32 = x.device, torch.int32
    S = E * cap
    counts = torch.empty(E, dtype=i32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=i32, device=dev) if offsets is None else offsets
    order = torch.empty(S, dtype=i32, device=dev) if order is None else order
    inv = torch.empty(T * k, dtype=i32, device=dev) if inv is None else inv
    for name, t, n in (("counts", counts, E), ("offsets", offsets, E + 1), ("order", order, S),
                       ("inv", inv, T * k)):
        _dev(t, name, (i32,))
        _shape(t, (n,), name, "moe_permute_capacity")
    if rows:
        x_cap = torch.empty((S, d), dtype=x.dtype, device=dev) if x_cap is None else x_cap
        _dev(x_cap, "x_cap", (x.dtype,))
        _shape(x_cap, (S, d), "x_cap", "moe_permute_capacity")
    elif x_cap is not None:
        raise MoeError("moe_permute_capacity: x_cap given in index-only mode")
    nbytes = moe_permute_capacity_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check(load_library().moe_permute_capacity(
        _ptr(x) if rows else None, _dtype_code(x), T, d, _ptr(topk_ids), k, E, int(cap),
        _ptr(counts), _ptr(offsets), _ptr(order), _ptr(inv), _ptr(x_cap), _ptr(workspace),
        workspace.numel(), _stream(stream)), "moe_permute_capacity")
    return counts, offsets, order, inv, x_cap


def moe_expert_loop_swiglu(a, offsets, w13, w2, h=None, y=None, offsets_host=None, stream=None):
    """moe_grouped_swiglu as a loop of one product pair per expert.  The loop
    needs the segment sizes on the host: offsets_host (an int32 array of
    G + 1 entries) or, when None, a copy of offsets made here (a device-to-host
    synchronisation)."""
    import numpy as np
    torch = _torch()
    G = _expert_shapes("moe_expert_loop_swiglu", a, offsets, w13=w13, w2=w2)
    M, d = a.shape
    ffn = w13.shape[2]
    if w13.shape[3] != d or tuple(w2.shape) != (G, d, ffn):
        raise MoeError("moe_expert_loop_swiglu: inconsistent shapes")
    if offsets_host is None:
        offsets_host = offsets.cpu().numpy()
    oh = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    if oh.shape != (G + 1,):
        raise MoeError("moe_expert_loop_swiglu: offsets_host must have G + 1 entries")
    h = torch.empty((M, ffn), dtype=a.dtype, device=a.device) if h is None else h
    y = torch.empty((M, d), dtype=a.dtype, device=a.device) if y is None else y
    _dev(h, "h", (a.dtype,))
    _dev(y, "y", (a.dtype,))
    _shape(h, (M, ffn), "h", "moe_expert_loop_swiglu")
    _shape(y, (M, d), "y", "moe_expert_loop_swiglu")
    _check(load_library().moe_expert_loop_swiglu(
        _ptr(a), _dtype_code(a), M, d, ffn, _ptr(offsets), oh.ctypes.data_as(ctypes.c_void_p), G,
        _ptr(w13), _ptr(w2), _ptr(h), _ptr(y), _stream(stream)), "moe_expert_loop_swiglu")
    return y


# --------------------------------------------------------------------------
# Training: the forward product that keeps the pre-activations, and the
# backward pass.
# --------------------------------------------------------------------------

def moe_grouped_gate_up_save(x, offsets, w13, h=None, gu=None, order=None, k=1, stream=None):
    """h [M, ffn] as moe_grouped_gate_up(_gather), plus the pre-activations
    gu [M, 2 ffn] (gate columns, then up columns) for the backward.  With
    order, row p is x[order[p] // k] (M = order.numel()); else x is [M, d]."""
    torch = _torch()
    G = _expert_shapes("moe_grouped_gate_up_save", x, offsets, w13=w13)
    T, d = x.shape
    if order is not None:
        _dev(order, "order", (torch.int32,))
        M = order.numel()
    else:
        M = T
    ffn = w13.shape[2]
    if w13.shape[3] != d:
        raise MoeError("moe_grouped_gate_up_save: inconsistent shapes")
    h = torch.empty((M, ffn), dtype=x.dtype, device=x.device) if h is None else h
    gu = torch.empty((M, 2 * ffn), dtype=x.dtype, device=x.device) if gu is None else gu
    _dev(h, "h", (x.dtype,))
    _dev(gu, "gu", (x.dtype,))
    _shape(h, (M, ffn), "h", "moe_grouped_gate_up_save")
    _shape(gu, (M, 2 * ffn), "gu", "moe_grouped_gate_up_save")
    _check(load_library().moe_grouped_gate_up_save(
        _ptr(x), _dtype_code(x), T, k, M, d, ffn, _ptr(order), _ptr(offsets), G, _ptr(w13),
        _ptr(h), _ptr(gu), _stream(stream)), "moe_grouped_gate_up_save")
    return h, gu


def moe_combine_backward(dy, inv, topk_w, y_perm=None, dy_perm=None, dgate=None, dy_shared=None,
                         stream=None, want_dgate=True):
    """The combine's backward: dy_perm [M, d] (row inv[t k + j] = w[t,j] dy[t])
    and, with y_perm, dgate [T, k] (dgate[t,j] = dy[t] . y_perm[inv[t k + j]]).
    dy_shared [T, d] (optional) receives a copy of dy (the shared expert's
    gradient rows).  Returns (dy_perm, dgate or None)."""
    torch = _torch()
    _dev(dy, "dy", _act_dtypes())
    _dev(inv, "inv", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,))
    T, k = topk_w.shape
    d = dy.shape[1]
    dev = dy.device
    dy_perm = torch.empty((T * k, d), dtype=dy.dtype, device=dev) if dy_perm is None else dy_perm
    _dev(dy_perm, "dy_perm", (dy.dtype,))
    _shape(dy, (T, d), "dy", "moe_combine_backward")
    _shape(dy_perm, (T * k, d), "dy_perm", "moe_combine_backward")
    if inv.numel() != T * k:
        raise MoeError("moe_combine_backward: inv must have T k entries")
    if want_dgate and y_perm is not None:
        _dev(y_perm, "y_perm", (dy.dtype,))
        if y_perm.shape[0] < T * k or y_perm.shape[1] != d:
            raise MoeError("moe_combine_backward: y_perm must have at least T k rows of d")
        dgate = torch.empty((T, k), dtype=torch.float32, device=dev) if dgate is None else dgate
        _dev(dgate, "dgate", (torch.float32,))
        _shape(dgate, (T, k), "dgate", "moe_combine_backward")
    else:
        y_perm, dgate = None, None
    if dy_shared is not None:
        _dev(dy_shared, "dy_shared", (dy.dtype,))
        _shape(dy_shared, (T, d), "dy_shared", "moe_combine_backward")
    _check(load_library().moe_combine_backward(
        _ptr(dy), _dtype_code(dy), T, k, d, _ptr(inv), _ptr(topk_w), _ptr(y_perm), _ptr(dy_perm),
        _ptr(dgate), _ptr(dy_shared), _stream(stream)), "moe_combine_backward")
    return dy_perm, dgate


def moe_gate_backward(logits, topk_ids, topk_w, dgate, gating="softmax", renormalize=True,
                      dlogits=None, stream=None):
    """dlogits [T, E] fp32 from the gate gradients dgate [T, k]."""
    torch = _torch()
    _dev(logits, "logits", (torch.float32,))
    _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,))
    _dev(dgate, "dgate", (torch.float32,))
    T, E = logits.shape
    k = topk_ids.shape[1]
    dlogits = torch.empty((T, E), dtype=torch.float32, device=logits.device) if dlogits is None \
        else dlogits
    _dev(dlogits, "dlogits", (torch.float32,))
    _shape(dlogits, (T, E), "dlogits", "moe_gate_backward")
    _shape(topk_ids, (T, k), "topk_ids", "moe_gate_backward")
    _shape(topk_w, (T, k), "topk_w", "moe_gate_backward")
    _shape(dgate, (T, k), "dgate", "moe_gate_backward")
    g = MOE_SOFTMAX if gating == "softmax" else MOE_SIGMOID if gating == "sigmoid" else -1
    _check(load_library().moe_gate_backward(_ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                            _ptr(dgate), T, E, k, g, int(bool(renormalize)),
                                            _ptr(dlogits), _stream(stream)), "moe_gate_backward")
    return dlogits


def moe_grouped_down_backward(dy_perm, offsets, w2, gu, dgu=None, stream=None):
    """dgu [M, 2 ffn]: dh = dy_perm W_down,e per segment, then the SwiGLU
    backward at the saved pre-activations gu (gate columns, then up)."""
    G = _expert_shapes("moe_grouped_down_backward", dy_perm, offsets, w2=w2)
    M, d = dy_perm.shape
    ffn = w2.shape[2]
    if w2.shape[1] != d or tuple(gu.shape) != (M, 2 * ffn):
        raise MoeError("moe_grouped_down_backward: inconsistent shapes")
    _dev(gu, "gu", (dy_perm.dtype,))
    dgu = _torch().empty((M, 2 * ffn), dtype=dy_perm.dtype, device=dy_perm.device) if dgu is None \
        else dgu
    _dev(dgu, "dgu", (dy_perm.dtype,))
    _shape(dgu, (M, 2 * ffn), "dgu", "moe_grouped_down_backward")
    _check(load_library().moe_grouped_down_backward(
        _ptr(dy_perm), _dtype_code(dy_perm), M, d, ffn, _ptr(offsets), G, _ptr(w2), _ptr(gu),
        _ptr(dgu), _stream(stream)), "moe_grouped_down_backward")
    return dgu


def moe_grouped_gate_up_backward(dgu, offsets, w13, dx_perm=None, stream=None):
    """dx_perm [M, d] = dgu [M, 2 ffn] W13,e per segment (W13,e as [2 ffn, d])."""
    G = _expert_shapes("moe_grouped_gate_up_backward", dgu, offsets, w13=w13)
    M = dgu.shape[0]
    ffn, d = w13.shape[2], w13.shape[3]
    if dgu.shape[1] != 2 * ffn:
        raise MoeError("moe_grouped_gate_up_backward: inconsistent shapes")
    dx_perm = _torch().empty((M, d), dtype=dgu.dtype, device=dgu.device) if dx_perm is None \
        else dx_perm
    _dev(dx_perm, "dx_perm", (dgu.dtype,))
    _shape(dx_perm, (M, d), "dx_perm", "moe_grouped_gate_up_backward")
    _check(load_library().moe_grouped_gate_up_backward(
        _ptr(dgu), _dtype_code(dgu), M, d, ffn, _ptr(offsets), G, _ptr(w13), _ptr(dx_perm),
        _stream(stream)), "moe_grouped_gate_up_backward")
    return dx_perm


def moe_grouped_weight_grad(a, b, offsets, out=None, b_order=None, b_k=1, stream=None):
    """out [G, m, n]: out[e] = a[seg e]^T b[rows of seg e] for a [M, m] and
    b [*, n]; with b_order, row p of b is b[b_order[p] // b_k]."""
    torch = _torch()
    _dev(a, "a", _act_dtypes())
    _dev(b, "b", (a.dtype,))
    _dev(offsets, "offsets", (torch.int32,))
    G = offsets.numel() - 1
    M, m = a.shape
    b_rows, n = b.shape
    if b_order is not None:
        _dev(b_order, "b_order", (torch.int32,))
        if b_order.numel() != M:
            raise MoeError("moe_grouped_weight_grad: b_order must have one entry per row of a")
    elif b_rows != M:
        raise MoeError("moe_grouped_weight_grad: a and b must have the same rows")
    out = torch.empty((G, m, n), dtype=a.dtype, device=a.device) if out is None else out
    _dev(out, "out", (a.dtype,))
    if out.numel() != G * m * n:
        raise MoeError("moe_grouped_weight_grad: out must hold [G, m, n]")
    _check(load_library().moe_grouped_weight_grad(
        _ptr(a), _ptr(b), _dtype_code(a), M, m, n, _ptr(offsets), G, _ptr(b_order), b_k, b_rows,
        _ptr(out), _stream(stream)), "moe_grouped_weight_grad")
    return out


def moe_router_backward_workspace_bytes(T, E) -> int:
    return int(load_library().moe_router_backward_workspace_bytes(T, E))


def moe_router_backward(dlogits, x, w_router, dx=None, dw_router=None, workspace=None,
                        stream=None):
    """The router product's backward: dx [T, d] += dlogits w_router (when dx
    is given) and dw_router [E, d] = dlogits^T x (allocated when None).
    Returns dw_router."""
    torch = _torch()
    _dev(dlogits, "dlogits", (torch.float32,))
    _dev(x, "x", _act_dtypes())
    _dev(w_router, "w_router", (x.dtype,))
    T, d = x.shape
    E = w_router.shape[0]
    if tuple(dlogits.shape) != (T, E) or w_router.shape[1] != d:
        raise MoeError("moe_router_backward: inconsistent shapes")
    if dx is not None:
        _dev(dx, "dx", (x.dtype,))
        _shape(dx, (T, d), "dx", "moe_router_backward")
    dw_router = torch.empty((E, d), dtype=x.dtype, device=x.device) if dw_router is None \
        else dw_router
    _dev(dw_router, "dw_router", (x.dtype,))
    _shape(dw_router, (E, d), "dw_router", "moe_router_backward")
    nbytes = moe_router_backward_workspace_bytes(T, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(load_library().moe_router_backward(
        _ptr(dlogits), _ptr(x), _dtype_code(x), T, d, _ptr(w_router), E, _ptr(dx), _ptr(dw_router),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_router_backward")
    return dw_router
