"""CPU oracle for the MoE layer (forward and backward) -- TEST INFRASTRUCTURE ONLY.

The product (the HIP library and its Python binding) never imports this
package.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  The arithmetic lives in ``oracle.c`` (plain C
loops, fp64 accumulation); this module builds it with gcc and wraps each
function for numpy arrays.  It shares no code with the HIP path.

Each wrapper names the page passage its C function follows; see oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle355.so")
# Another build of oracle.c to load instead (the tests' sanitizer run sets it).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

F32, BF16, F64 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle355.so (gcc, OpenMP, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_sigmoid_pinned.argtypes = [ctypes.c_float]
    lib.orc_sigmoid_pinned.restype = ctypes.c_float
    lib.orc_sigmoid_pinned_array.argtypes = [P, P, i64]
    lib.orc_route.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P]
    lib.orc_route.restype = i32
    lib.orc_send_counts.argtypes = [P, i32, i32, i32, i32, P]
    lib.orc_send_counts.restype = i32
    lib.orc_permute_index.argtypes = [P, i64, i32, P, P, P, P]
    lib.orc_permute_index.restype = i32
    lib.orc_gather_rows.argtypes = [P, i64, P, i64, i32, P]
    lib.orc_expert_capacity.argtypes = [i64, i32, f64]
    lib.orc_expert_capacity.restype = i64
    lib.orc_permute_capacity.argtypes = [P, i64, i32, i64, P, P, P]
    lib.orc_permute_capacity.restype = i32
    lib.orc_expert_swiglu_rows.argtypes = [P, i32, i64, i32, i32, P, P, P, P]
    lib.orc_combine.argtypes = [P, i32, i64, i32, i32, P, P, P, i32, P]
    lib.orc_alltoall_bytes.argtypes = [i64, i32, i64, i32, f64, f64, i32]
    lib.orc_alltoall_bytes.restype = f64
    lib.orc_router_logits.argtypes = [P, i32, i64, i32, P, i32, P]
    lib.orc_bias_update.argtypes = [P, i32, ctypes.c_float, P]
    lib.orc_bias_update.restype = i32
    lib.orc_combine_backward.argtypes = [P, i32, i64, i32, i32, P, P, P, i32, P, P]
    lib.orc_expert_swiglu_backward_rows.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P, P,
                                                    P, P, P]
    lib.orc_down_backward_rows.argtypes = [P, i64, i32, i32, P, P, i32, P, P]
    lib.orc_gate_up_backward_rows.argtypes = [P, i64, i32, i32, P, P, i32, P]
    lib.orc_weight_grad.argtypes = [P, i64, i32, P, i32, P, i32, P, i32, P]
    lib.orc_gate_backward.argtypes = [P, i32, i32, i32, P, i32, i32, P, P]
    lib.orc_gate_backward.restype = i32
    lib.orc_router_backward.argtypes = [P, i32, i64, i32, P, i32, P, P, P]
    lib.orc_num_threads.restype = i32
    lib.orc_set_num_threads.argtypes = [i32]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing only)."""
    _load().orc_set_num_threads(int(n))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def sigmoid_pinned(x: np.ndarray) -> np.ndarray:
    """The pinned fp32 sigmoid used for group scores (oracle.c, orc_sigmoid_pinned)."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    _load().orc_sigmoid_pinned_array(_ptr(x), _ptr(y), x.size)
    return y


def route(logits: np.ndarray, k: int, gating: str = "softmax", renormalize: int = 1,
          n_groups: int = 1, topk_groups: int = 1, bias=None):
    """O1: top-k ids [T,k] int32 and gates [T,k] fp32 (oracle.c, orc_route).

    bias [E] fp32 (optional): selection on logits + bias, gates from the
    unbiased logits (auxiliary-loss-free balancing)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    g = SOFTMAX if gating == "softmax" else SIGMOID
    b = None if bias is None else _c(bias, np.float32)
    if b is not None and b.shape != (E,):
        raise ValueError("bias must have one entry per expert")
    rc = _load().orc_route(_ptr(logits), None if b is None else _ptr(b), T, E, k, g,
                           int(renormalize), n_groups, topk_groups, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("orc_route: arguments outside the contract")
    return ids, w


def router_logits(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """O0: logits [T,E] fp32 = x [T,d] . wg [E,d]^T, fp64 sums (oracle.c, orc_router_logits).
    bf16 operands are uint16 bit patterns."""
    x = _c(x)
    wg = _c(wg)
    if x.dtype != wg.dtype or x.ndim != 2 or wg.ndim != 2 or x.shape[1] != wg.shape[1]:
        raise ValueError("router_logits: x [T,d] and wg [E,d] of one dtype")
    T, d = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), np.float32)
    _load().orc_router_logits(_ptr(x), _dtype_code(x), T, d, _ptr(wg), E, _ptr(out))
    return out


def bias_update(bias: np.ndarray, counts: np.ndarray, lr: float) -> np.ndarray:
    """Auxiliary-loss-free bias step: returns bias + lr (avg - counts) in fp32
    (oracle.c, orc_bias_update)."""
    b = np.array(bias, np.float32, copy=True)
    c = _c(counts, np.int32)
    if b.shape != c.shape or b.ndim != 1:
        raise ValueError("bias_update: bias and counts of shape [E]")
    if _load().orc_bias_update(_ptr(c), c.size, float(np.float32(lr)), _ptr(b)) != 0:
        raise ValueError("orc_bias_update: arguments outside the contract")
    return b


def send_counts(ids: np.ndarray, E: int, n_ep: int) -> np.ndarray:
    """O2: send-count matrix S [n_ep, n_ep], row = source rank (oracle.c, orc_send_counts)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    S = np.empty((n_ep, n_ep), np.int32)
    if _load().orc_send_counts(_ptr(ids), T, k, E, n_ep, _ptr(S)) != 0:
        raise ValueError("orc_send_counts: arguments outside the contract")
    return S


def permute_index(ids: np.ndarray, E: int):
    """O3: counts [E], offsets [E+1], order [M], inv [M] (oracle.c, orc_permute_index)."""
    flat = _c(ids, np.int32).reshape(-1)
    M = flat.size
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    order = np.empty(M, np.int32)
    inv = np.empty(M, np.int32)
    if _load().orc_permute_index(_ptr(flat), M, E, _ptr(counts), _ptr(offsets), _ptr(order),
                                 _ptr(inv)) != 0:
        raise ValueError("orc_permute_index: expert id out of range")
    return counts, offsets, order, inv


def expert_capacity(M: int, E: int, cf: float) -> int:
    """N2: cap = ceil(CF M / E), the rows of every expert's block in the
    padded batched form (oracle.c, orc_expert_capacity)."""
    cap = _load().orc_expert_capacity(M, E, float(cf))
    if cap < 0:
        raise ValueError("orc_expert_capacity: arguments outside the contract")
    return int(cap)


def permute_capacity(ids: np.ndarray, E: int, cap: int):
    """N2: counts [E] (before the cap), slot_of [M] (slot e cap + r, or -1 when
    dropped), assign_of [E cap] (assignment, or -1 for a padding slot)
    (oracle.c, orc_permute_capacity)."""
    flat = _c(ids, np.int32).reshape(-1)
    M = flat.size
    counts = np.empty(E, np.int32)
    slot_of = np.empty(M, np.int32)
    assign_of = np.empty(E * cap, np.int32)
    if _load().orc_permute_capacity(_ptr(flat), M, E, cap, _ptr(counts), _ptr(slot_of),
                                    _ptr(assign_of)) != 0:
        raise ValueError("orc_permute_capacity: expert id out of range or cap < 0")
    return counts, slot_of, assign_of


def gather_rows_padded(x: np.ndarray, assign_of: np.ndarray, k: int) -> np.ndarray:
    """The padded batch: slot s holds token assign_of[s] // k bit for bit, a
    padding slot (assign_of = -1) holds zeros."""
    out = np.zeros((assign_of.size,) + x.shape[1:], x.dtype)
    live = assign_of >= 0
    out[live] = gather_rows(x, assign_of[live], k)
    return out


def gather_rows(x: np.ndarray, order: np.ndarray, k: int) -> np.ndarray:
    """X[order] with packed row p = token order[p] // k, bit for bit (oracle.c, orc_gather_rows)."""
    x = _c(x)
    order = _c(order, np.int32)
    out = np.empty((order.size,) + x.shape[1:], x.dtype)
    row_bytes = x.strides[0] if x.shape[0] else x.itemsize * int(np.prod(x.shape[1:]))
    _load().orc_gather_rows(_ptr(x), row_bytes, _ptr(order), order.size, k, _ptr(out))
    return out


def expert_swiglu_rows(xrows: np.ndarray, expert_of_row: np.ndarray, w13: np.ndarray,
                       w2: np.ndarray) -> np.ndarray:
    """O4: y[r] = W_down,e (SiLU(W_gate,e x_r) * W_up,e x_r) in fp64 (oracle.c)."""
    xrows = _c(xrows)
    w13 = _c(w13)
    w2 = _c(w2)
    dt = _dtype_code(xrows)
    if _dtype_code(w13) != dt or _dtype_code(w2) != dt:
        raise TypeError("rows and weights must share a dtype")
    R, d = xrows.shape
    G, two, ffn, d2 = w13.shape
    assert two == 2 and d2 == d and w2.shape == (G, d, ffn)
    e = _c(expert_of_row, np.int32).reshape(-1)
    assert e.size == R and (R == 0 or (e.min() >= 0 and e.max() < G))
    y = np.empty((R, d), np.float64)
    _load().orc_expert_swiglu_rows(_ptr(xrows), dt, R, d, ffn, _ptr(e), _ptr(w13), _ptr(w2), _ptr(y))
    return y


def combine(y_perm: np.ndarray, inv: np.ndarray, w: np.ndarray, y_shared=None) -> np.ndarray:
    """O5: y[t] = sum_j w[t,j] y_perm[inv[t k + j]] (+ y_shared[t]) in fp64 (oracle.c)."""
    y_perm = _c(y_perm)
    w = _c(w, np.float32)
    T, k = w.shape
    d = y_perm.shape[1]
    inv = _c(inv, np.int32).reshape(-1)
    assert inv.size == T * k
    y = np.empty((T, d), np.float64)
    if y_shared is not None:
        y_shared = _c(y_shared)
        assert y_shared.shape == (T, d)
        sh_ptr, sh_dt = _ptr(y_shared), _dtype_code(y_shared)
    else:
        sh_ptr, sh_dt = None, 0
    _load().orc_combine(_ptr(y_perm), _dtype_code(y_perm), T, k, d, _ptr(inv), _ptr(w), sh_ptr,
                        sh_dt, _ptr(y))
    return y


def alltoall_bytes(T_loc: int, k: int, d: int, n_ep: int, s_disp: float, s_comb: float,
                   training: bool = False) -> float:
    """Dispatch + combine bytes one GPU sends per layer (oracle.c, orc_alltoall_bytes)."""
    return _load().orc_alltoall_bytes(T_loc, k, d, n_ep, s_disp, s_comb, int(training))


# --------------------------------------------------------------------------
# Compositions of O1..O5 (step order of the forward pass in "Expert parallelism").
# --------------------------------------------------------------------------

def layer_tokens(x, ids, w, w13, w2, tokens, sh_w13=None, sh_w2=None):
    """The plain definition for selected tokens: y[t] = sum_j w[t,j] f_{ids[t,j]}(x[t])
    (+ f_shared(x[t])), evaluated with O4 and O5 in fp64.  Returns [len(tokens), d]."""
    tokens = np.asarray(tokens, np.int64)
    k = ids.shape[1]
    xs = _c(x[tokens])
    rows = np.repeat(xs, k, axis=0)
    y_rows = expert_swiglu_rows(rows, ids[tokens].reshape(-1), w13, w2)
    y_sh = None
    if sh_w13 is not None:
        y_sh = expert_swiglu_rows(xs, np.zeros(len(tokens), np.int32), sh_w13, sh_w2)
    inv = np.arange(len(tokens) * k, dtype=np.int32)
    return combine(y_rows, inv, w[tokens], y_sh)


def layer_tokens_capacity(x, ids, w, slot_of, w13, w2, tokens, sh_w13=None, sh_w2=None):
    """The padded batched form's output for selected tokens: the plain
    definition with every dropped assignment (slot_of = -1) left out,
    y[t] = sum over kept j of w[t,j] f_{ids[t,j]}(x[t]) (+ f_shared(x[t])),
    evaluated with O4 and O5 in fp64.  Returns [len(tokens), d]."""
    tokens = np.asarray(tokens, np.int64)
    k = ids.shape[1]
    kept = (np.asarray(slot_of).reshape(-1, k)[tokens] >= 0).reshape(-1)
    xs = _c(x[tokens])
    rows = np.repeat(xs, k, axis=0)[kept]
    y_rows = expert_swiglu_rows(rows, ids[tokens].reshape(-1)[kept], w13, w2)
    y_sh = None
    if sh_w13 is not None:
        y_sh = expert_swiglu_rows(xs, np.zeros(len(tokens), np.int32), sh_w13, sh_w2)
    inv = np.full(len(tokens) * k, -1, np.int32)
    inv[kept] = np.arange(int(kept.sum()), dtype=np.int32)
    return combine(y_rows, inv, w[tokens], y_sh)


# --------------------------------------------------------------------------
# Backward pass (oracle.c, functions B0..B5): the chain rule applied to the
# forward definition; "Expert parallelism", section "How many bytes move",
# gives its shape (the combine's gradient is dispatched, the dispatch's
# gradient combined).
# --------------------------------------------------------------------------

def combine_backward(dy: np.ndarray, inv: np.ndarray, w: np.ndarray, y_perm: np.ndarray):
    """B5: dy_perm [T k, d] (row inv[t k + j] = w[t,j] dy[t]) and dw [T,k]
    (dw[t,j] = dy[t] . y_perm[inv[t k + j]]), fp64 (oracle.c)."""
    dy = _c(dy)
    y_perm = _c(y_perm)
    w = _c(w, np.float32)
    T, k = w.shape
    d = dy.shape[1]
    inv = _c(inv, np.int32).reshape(-1)
    assert inv.size == T * k and dy.shape == (T, d) and y_perm.shape[1] == d
    dy_perm = np.empty((T * k, d), np.float64)
    dw = np.empty((T, k), np.float64)
    _load().orc_combine_backward(_ptr(dy), _dtype_code(dy), T, k, d, _ptr(inv), _ptr(w),
                                 _ptr(y_perm), _dtype_code(y_perm), _ptr(dy_perm), _ptr(dw))
    return dy_perm, dw


def expert_swiglu_backward_rows(xrows: np.ndarray, expert_of_row: np.ndarray, w13: np.ndarray,
                                w2: np.ndarray, dyrows: np.ndarray, want_dx: bool = True,
                                want_dw: bool = True, want_act: bool = False):
    """B4: (dx [R,d], dw13 [G,2,ffn,d], dw2 [G,d,ffn]) in fp64 for rows x_r of
    experts expert_of_row[r] with output gradients dyrows (oracle.c).  With
    want_act also (gu, dgu), each [R, 2 ffn]: the pre-activations (g, u) and
    their gradients (dg, du).  An output not asked for is None."""
    xrows = _c(xrows)
    w13 = _c(w13)
    w2 = _c(w2)
    dt = _dtype_code(xrows)
    if _dtype_code(w13) != dt or _dtype_code(w2) != dt:
        raise TypeError("rows and weights must share a dtype")
    R, d = xrows.shape
    G, two, ffn, d2 = w13.shape
    assert two == 2 and d2 == d and w2.shape == (G, d, ffn)
    e = _c(expert_of_row, np.int32).reshape(-1)
    assert e.size == R and (R == 0 or (e.min() >= 0 and e.max() < G))
    dyrows = _c(dyrows, np.float64)
    assert dyrows.shape == (R, d)
    dx = np.empty((R, d), np.float64) if want_dx else None
    dw13 = np.empty((G, 2, ffn, d), np.float64) if want_dw else None
    dw2 = np.empty((G, d, ffn), np.float64) if want_dw else None
    gu = np.empty((R, 2 * ffn), np.float64) if want_act else None
    dgu = np.empty((R, 2 * ffn), np.float64) if want_act else None
    opt = lambda a: None if a is None else _ptr(a)
    _load().orc_expert_swiglu_backward_rows(
        _ptr(xrows), dt, R, d, ffn, _ptr(e), G, _ptr(w13), _ptr(w2), _ptr(dyrows), opt(dx), opt(gu),
        opt(dgu), opt(dw13), opt(dw2))
    if want_act:
        return dx, dw13, dw2, gu, dgu
    return dx, dw13, dw2


def expert_backward_dense(xrows, w13e, w2e, dyrows):
    """One expert's backward by the chain rule, with fp64 matrix products as
    its steps (for whole weight-gradient matrices at full size, where the
    plain loops of orc_expert_swiglu_backward_rows would take hours):
        g = X Wg^T, u = X Wu^T, h = SiLU(g) u           (forward, kept)
        dh = dY Wd,  dWd = dY^T h
        dg = dh u SiLU'(g), du = dh SiLU(g),  SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g)
        dW13 = (dg^T X, du^T X),  dX = dg Wg + du Wu.
    xrows [R, d], w13e [2, ffn, d], w2e [d, ffn], dyrows [R, d] (bf16 bits or
    floats).  Returns (dx [R, d], dw13 [2, ffn, d], dw2 [d, ffn]) in fp64."""
    X, W13, W2, dY = _f64(xrows), _f64(w13e), _f64(w2e), _f64(dyrows)
    g, u = X @ W13[0].T, X @ W13[1].T
    s = 1.0 / (1.0 + np.exp(-g))
    silu = g * s
    h = silu * u
    dh = dY @ W2
    dw2 = dY.T @ h
    dg = dh * u * (s * (1.0 + g * (1.0 - s)))
    du = dh * silu
    dw13 = np.stack([dg.T @ X, du.T @ X])
    dx = dg @ W13[0] + du @ W13[1]
    return dx, dw13, dw2


def _f64(a):
    a = np.asarray(a)
    return _c(bf16_bits_to_f64(a) if a.dtype == np.uint16 else a, np.float64)


def down_backward_rows(dyrows, expert_of_row, w2, gu):
    """B4a: dgu [R, 2 ffn] from dy rows, w2 [G, d, ffn] and given
    pre-activations gu [R, 2 ffn] (bf16 bit patterns are widened exactly)."""
    dy = _f64(dyrows)
    gu = _f64(gu)
    w2 = _c(w2)
    R, d = dy.shape
    ffn = w2.shape[2]
    e = _c(expert_of_row, np.int32).reshape(-1)
    assert gu.shape == (R, 2 * ffn) and e.size == R
    out = np.empty((R, 2 * ffn), np.float64)
    _load().orc_down_backward_rows(_ptr(dy), R, d, ffn, _ptr(e), _ptr(w2), _dtype_code(w2),
                                   _ptr(gu), _ptr(out))
    return out


def gate_up_backward_rows(dgu, expert_of_row, w13):
    """B4b: dx [R, d] from given dgu [R, 2 ffn] and w13 [G, 2, ffn, d]."""
    dgu = _f64(dgu)
    w13 = _c(w13)
    R = dgu.shape[0]
    ffn, d = w13.shape[2], w13.shape[3]
    e = _c(expert_of_row, np.int32).reshape(-1)
    assert dgu.shape == (R, 2 * ffn) and e.size == R
    out = np.empty((R, d), np.float64)
    _load().orc_gate_up_backward_rows(_ptr(dgu), R, d, ffn, _ptr(e), _ptr(w13), _dtype_code(w13),
                                      _ptr(out))
    return out


def weight_grad(a, b, offsets, b_order=None, b_k=1):
    """B4c: c [G, m, n], c[e] = sum over segment e's rows of a[r]^T b[src(r)]."""
    a = _f64(a)
    b = _f64(b)
    offsets = _c(offsets, np.int32)
    G = offsets.size - 1
    R, m = a.shape
    n = b.shape[1]
    order = None if b_order is None else _c(b_order, np.int32)
    out = np.empty((G, m, n), np.float64)
    _load().orc_weight_grad(_ptr(a), R, m, _ptr(b), n, _ptr(offsets), G,
                            None if order is None else _ptr(order), int(b_k), _ptr(out))
    return out


def gate_backward(logits: np.ndarray, ids: np.ndarray, dw: np.ndarray, gating: str = "softmax",
                  renormalize: int = 1) -> np.ndarray:
    """B1: dlogits [T,E] fp64 from the gate gradients dw [T,k] (oracle.c)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    dw = _c(dw, np.float64)
    assert ids.shape == (T, k) and dw.shape == (T, k)
    out = np.empty((T, E), np.float64)
    g = SOFTMAX if gating == "softmax" else SIGMOID
    if _load().orc_gate_backward(_ptr(logits), T, E, k, _ptr(ids), g, int(renormalize), _ptr(dw),
                                 _ptr(out)) != 0:
        raise ValueError("orc_gate_backward: arguments outside the contract")
    return out


def router_backward(x: np.ndarray, wg: np.ndarray, dlogits: np.ndarray, want_dx: bool = True,
                    want_dwg: bool = True):
    """B0: dx = dlogits wg [T,d] and dwg = dlogits^T x [E,d], fp64 (oracle.c)."""
    x = _c(x)
    wg = _c(wg)
    if x.dtype != wg.dtype:
        raise TypeError("x and wg must share a dtype")
    T, d = x.shape
    E = wg.shape[0]
    dl = _c(dlogits, np.float64)
    assert dl.shape == (T, E) and wg.shape == (E, d)
    dx = np.empty((T, d), np.float64) if want_dx else None
    dwg = np.empty((E, d), np.float64) if want_dwg else None
    _load().orc_router_backward(_ptr(x), _dtype_code(x), T, d, _ptr(wg), E, _ptr(dl),
                                None if dx is None else _ptr(dx), None if dwg is None else _ptr(dwg))
    return dx, dwg


def layer_backward(x, logits, ids, w, w13, w2, dy, gating="softmax", renormalize=1,
                   sh_w13=None, sh_w2=None, wg=None):
    """The whole layer's backward for all T tokens, composed from B0..B5 in
    the reverse order of the forward steps.  ids, w are the forward's route
    (logits may be None when the gates were given).  Returns a dict of fp64
    gradients: dx [T,d], dw13, dw2, dgate [T,k], and when present dlogits
    [T,E], dsh_w13, dsh_w2, dwg [E,d]."""
    T, k = ids.shape
    d = x.shape[1]
    xs = _c(x)
    rows = np.repeat(xs, k, axis=0)                        # row a = t k + j holds x[t]
    expert = _c(ids, np.int32).reshape(-1)
    y_rows = expert_swiglu_rows(rows, expert, w13, w2)    # the forward's y_perm, token-major
    ident = np.arange(T * k, dtype=np.int32)
    dy_rows, dgate = combine_backward(dy, ident, w, y_rows)
    dx_rows, dw13, dw2 = expert_swiglu_backward_rows(rows, expert, w13, w2, dy_rows)
    dx = dx_rows.reshape(T, k, d).sum(axis=1)              # the permute's gradient: a token's rows summed
    out = {"dw13": dw13, "dw2": dw2, "dgate": dgate}
    if sh_w13 is not None:
        dx_sh, out["dsh_w13"], out["dsh_w2"] = expert_swiglu_backward_rows(
            xs, np.zeros(T, np.int32), sh_w13, sh_w2, _c(dy).astype(np.float64)
            if _dtype_code(_c(dy)) != BF16 else bf16_bits_to_f64(dy))
        dx = dx + dx_sh
    if logits is not None:
        out["dlogits"] = gate_backward(logits, ids, dgate, gating, renormalize)
        if wg is not None:
            dxr, out["dwg"] = router_backward(xs, wg, out["dlogits"])
            dx = dx + dxr
    out["dx"] = dx
    return out


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) widened exactly to fp64."""
    a = np.ascontiguousarray(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
