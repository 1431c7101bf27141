"""Pins of the oracle's backward pass (oracle.c, B0..B5).  CPU only.

The pages fix the backward's shape ("Expert parallelism", section "How many
bytes move": the combine's gradient is dispatched and the dispatch's
gradient combined) and its cost (section "A worked example at DeepSeek-V3's
shape": twice the forward's products); its values follow from the forward
definition by the chain rule.  The oracle writes those derivatives out by
hand; these tests pin them to two things that do not share that derivation:

  * reverse-mode autodiff (torch, fp64, CPU) of the layer written in its
    dense-masked form, y[t] = sum_e m[t,e] f_e(x[t]) (+ f_shared(x[t])),
    with m the gate where e is chosen and 0 elsewhere -- every expert
    evaluated on every token, no permutation at all;
  * central finite differences of the oracle's own forward (pinned in
    test_oracle_pins.py) in fp64;

plus the invariants the gate maps impose on their gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from token_routing_expert_amd import inputs


def _problem(seed, T=6, E=4, k=2, d=16, ffn=8, shared=True, dtype=np.float64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(dtype)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w13 = (0.3 * rng.standard_normal((E, 2, ffn, d))).astype(dtype)
    w2 = (0.3 * rng.standard_normal((E, d, ffn))).astype(dtype)
    sh13 = (0.3 * rng.standard_normal((1, 2, ffn, d))).astype(dtype) if shared else None
    sh2 = (0.3 * rng.standard_normal((1, d, ffn))).astype(dtype) if shared else None
    dy = rng.standard_normal((T, d)).astype(dtype)
    return x, logits, w13, w2, sh13, sh2, dy, k


def _mlp(xt, w13e, w2e):
    g = xt @ w13e[0].T
    u = xt @ w13e[1].T
    return (torch.nn.functional.silu(g) * u) @ w2e.T


def _gates(lt, ids_t, gating, renorm):
    """Gates of one token from its logits with torch's library maps."""
    if gating == "softmax":
        return torch.softmax(lt[ids_t], 0) if renorm else torch.softmax(lt, 0)[ids_t]
    s = torch.sigmoid(lt[ids_t])
    return s / s.sum() if renorm else s


def _autograd(x, logits, w13, w2, sh13, sh2, dy, ids, gating, renorm, wg=None):
    T, E = logits.shape
    f64 = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    X, W13, W2 = f64(x), f64(w13), f64(w2)
    leaves = {"dx": X, "dw13": W13, "dw2": W2}
    if wg is not None:
        WG = f64(wg)
        L = X @ WG.T
        leaves["dwg"] = WG
    else:
        L = f64(logits)
        leaves["dlogits"] = L
    if sh13 is not None:
        SH13, SH2 = f64(sh13), f64(sh2)
        leaves["dsh_w13"], leaves["dsh_w2"] = SH13, SH2
    ys = []
    for t in range(T):
        it = torch.tensor(ids[t], dtype=torch.long)
        gate = _gates(L[t], it, gating, renorm)
        m = torch.zeros(E, dtype=torch.float64).index_put((it,), gate)
        yt = sum(m[e] * _mlp(X[t], W13[e], W2[e]) for e in range(E))
        if sh13 is not None:
            yt = yt + _mlp(X[t], SH13[0], SH2[0])
        ys.append(yt)
    Y = torch.stack(ys)
    (Y * torch.tensor(np.asarray(dy, np.float64))).sum().backward()
    return {name: t.grad.numpy() for name, t in leaves.items()}


def _close(a, b, rel):
    scale = max(np.abs(b).max(), 1e-30)
    assert np.abs(a - b).max() <= rel * scale, f"max err {np.abs(a - b).max() / scale:.3g}"


@pytest.mark.parametrize("gating,renorm", [("softmax", 1), ("softmax", 0), ("sigmoid", 1),
                                           ("sigmoid", 0)])
@pytest.mark.parametrize("shared", [False, True])
def test_backward_matches_autodiff_of_dense_form(gating, renorm, shared):
    x, logits, w13, w2, sh13, sh2, dy, k = _problem(7 + renorm, shared=shared)
    ids, w = oracle.route(logits, k, gating, renorm)
    got = oracle.layer_backward(x, logits, ids, w, w13, w2, dy, gating, renorm, sh13, sh2)
    ref = _autograd(x, logits, w13, w2, sh13, sh2, dy, ids, gating, renorm)
    # The oracle's gates are rounded once to fp32 (O1), so dy_perm = w dy
    # carries a relative error of about 6e-8; everything else is fp64.
    for name, r in ref.items():
        _close(got[name], r, 1e-6)


def test_backward_with_router_matches_autodiff():
    x, logits, w13, w2, sh13, sh2, dy, k = _problem(11, E=8, k=3)
    wg = 0.5 * np.random.default_rng(3).standard_normal((8, x.shape[1]))
    lg = oracle.router_logits(x, wg)                      # fp32, the route's precision
    ids, w = oracle.route(lg, k, "sigmoid", 1)
    got = oracle.layer_backward(x, lg, ids, w, w13, w2, dy, "sigmoid", 1, sh13, sh2, wg=wg)
    ref = _autograd(x, lg, w13, w2, sh13, sh2, dy, ids, "sigmoid", 1, wg=wg)
    # The oracle takes the gates and their derivative at the fp32 logits;
    # autodiff at the fp64 product x wg^T.  They differ by fp32 rounding.
    for name in ("dx", "dw13", "dw2", "dwg", "dsh_w13", "dsh_w2"):
        _close(got[name], ref[name], 2e-6)


def _loss(x, ids, w, w13, w2, dy):
    y = oracle.layer_tokens(x, ids, w, w13, w2, np.arange(x.shape[0]))
    return float((y * dy).sum())


@pytest.mark.parametrize("seed", [1, 2])
def test_backward_matches_finite_differences(seed):
    x, logits, w13, w2, _, _, dy, k = _problem(seed, shared=False)
    ids, w = oracle.route(logits, k, "softmax", 1)
    got = oracle.layer_backward(x, None, ids, w, w13, w2, dy)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for name, arr in (("dx", x), ("dw13", w13), ("dw2", w2)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            a_hi, a_lo = arr.copy(), arr.copy()
            a_hi[idx] += eps
            a_lo[idx] -= eps
            args = {"dx": (x, w13, w2), "dw13": (x, w13, w2), "dw2": (x, w13, w2)}[name]
            hi = [a_hi if a is arr else a for a in args]
            lo = [a_lo if a is arr else a for a in args]
            fd = (_loss(hi[0], ids, w, hi[1], hi[2], dy) - _loss(lo[0], ids, w, lo[1], lo[2], dy)) / (2 * eps)
            assert abs(fd - got[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, got[name][idx])


def test_gate_gradient_invariants():
    """Each gate map is invariant along one direction of the logits, so its
    gradient is orthogonal to it: softmax over the chosen (or all) logits
    ignores a common shift; s_j / sum s_i ignores a common scale of the s."""
    rng = np.random.default_rng(5)
    T, E, k = 64, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k))
    for gating, renorm in (("softmax", 1), ("softmax", 0), ("sigmoid", 1), ("sigmoid", 0)):
        ids, _ = oracle.route(logits, k, gating, renorm)
        dl = oracle.gate_backward(logits, ids, dw, gating, renorm)
        chosen = np.zeros((T, E), bool)
        np.put_along_axis(chosen, ids.astype(np.int64), True, axis=1)
        if not (gating == "softmax" and renorm == 0):
            assert np.all(dl[~chosen] == 0.0)
        if gating == "softmax":
            np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
        elif renorm:
            s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
            # sum_i dl_i / (1 - s_i) = sum_i s_i ds_i = 0 over the chosen
            np.testing.assert_allclose(np.where(chosen, dl / (1 - s), 0).sum(axis=1), 0.0, atol=1e-12)


def test_gate_gradient_brute_force_single_token():
    """For one token and sigmoid not renormalised, the gate is s(l_j) itself;
    its derivative is s (1 - s), checked against a central difference."""
    l = np.array([[0.3, -1.2, 2.0, 0.1]], np.float32)
    ids, _ = oracle.route(l, 2, "sigmoid", 0)
    dw = np.array([[1.0, 1.0]])
    dl = oracle.gate_backward(l, ids, dw, "sigmoid", 0)
    for j in range(2):
        e = ids[0, j]
        z = float(l[0, e])
        fd = (1 / (1 + np.exp(-(z + 1e-6))) - 1 / (1 + np.exp(-(z - 1e-6)))) / 2e-6
        assert abs(dl[0, e] - fd) < 1e-8


def test_bf16_operands_widen_exactly():
    """bf16 bit patterns and their exact fp64 values give the same gradients."""
    x, logits, w13, w2, sh13, sh2, dy, k = _problem(4, dtype=np.float32)
    to_bf16 = lambda a: (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xb, w13b, w2b, s13b, s2b, dyb = map(to_bf16, (x, w13, w2, sh13, sh2, dy))
    ids, w = oracle.route(logits, k, "softmax", 1)
    a = oracle.layer_backward(xb, logits, ids, w, w13b, w2b, dyb, "softmax", 1, s13b, s2b)
    f = oracle.bf16_bits_to_f64
    b = oracle.layer_backward(f(xb), logits, ids, w, f(w13b), f(w2b), f(dyb), "softmax", 1, f(s13b),
                              f(s2b))
    for name in a:
        np.testing.assert_allclose(a[name], b[name], rtol=1e-12, atol=1e-14)


def test_combine_backward_packed_positions():
    """dy_perm lands at the packed positions inv (a permutation) and dw pairs
    each slot with its own packed row."""
    rng = np.random.default_rng(9)
    T, k, d, E = 5, 3, 8, 4
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, order, inv = oracle.permute_index(ids, E)
    w = rng.random((T, k)).astype(np.float32)
    dy = rng.standard_normal((T, d))
    y_perm = rng.standard_normal((T * k, d))
    dy_perm, dw = oracle.combine_backward(dy, inv, w, y_perm)
    for p in range(T * k):
        t, j = divmod(int(order[p]), k)
        np.testing.assert_array_equal(dy_perm[p], np.float64(w[t, j]) * dy[t])
        assert abs(dw[t, j] - float(np.dot(dy[t], y_perm[p]))) < 1e-12


def test_preactivations_and_their_gradients_match_autodiff():
    """B4's optional outputs: the pre-activations (g, u) of each row and their
    gradients (dg, du), against torch's evaluation and reverse-mode autodiff
    of one SwiGLU MLP per expert."""
    rng = np.random.default_rng(12)
    R, G, d, ffn = 9, 3, 16, 8
    x = rng.standard_normal((R, d))
    e = rng.integers(0, G, R).astype(np.int32)
    w13 = 0.3 * rng.standard_normal((G, 2, ffn, d))
    w2 = 0.3 * rng.standard_normal((G, d, ffn))
    dy = rng.standard_normal((R, d))
    _, _, _, gu, dgu = oracle.expert_swiglu_backward_rows(x, e, w13, w2, dy, want_act=True)
    for r in range(R):
        X = torch.tensor(x[r])
        g = (torch.tensor(w13[e[r], 0]) @ X).requires_grad_(True)
        u = (torch.tensor(w13[e[r], 1]) @ X).requires_grad_(True)
        y = torch.tensor(w2[e[r]]) @ (torch.nn.functional.silu(g) * u)
        (y * torch.tensor(dy[r])).sum().backward()
        np.testing.assert_allclose(gu[r], np.concatenate([g.detach().numpy(), u.detach().numpy()]),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dgu[r], np.concatenate([g.grad.numpy(), u.grad.numpy()]),
                                   rtol=1e-10, atol=1e-12)


def test_backward_stages_compose_to_the_whole():
    """B4a, B4b and B4c fed B4's own intermediates reproduce B4's outputs, so
    they carry B4's autodiff pin; B4c with an order reads the gathered rows."""
    rng = np.random.default_rng(13)
    R, G, d, ffn, k = 11, 3, 16, 8, 2
    x = rng.standard_normal((R, d))
    e = np.sort(rng.integers(0, G, R)).astype(np.int32)
    offsets = np.searchsorted(e, np.arange(G + 1)).astype(np.int32)
    w13 = 0.3 * rng.standard_normal((G, 2, ffn, d))
    w2 = 0.3 * rng.standard_normal((G, d, ffn))
    dy = rng.standard_normal((R, d))
    dx, dw13, dw2, gu, dgu = oracle.expert_swiglu_backward_rows(x, e, w13, w2, dy, want_act=True)
    np.testing.assert_allclose(oracle.down_backward_rows(dy, e, w2, gu), dgu, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.gate_up_backward_rows(dgu, e, w13), dx, rtol=1e-13, atol=1e-13)
    g, u = gu[:, :ffn], gu[:, ffn:]
    h = g / (1 + np.exp(-g)) * u
    np.testing.assert_allclose(oracle.weight_grad(dy, h, offsets), dw2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.weight_grad(dgu, x, offsets).reshape(G, 2, ffn, d), dw13,
                               rtol=1e-12, atol=1e-12)
    # The gathered form: row r of b is xt[order[r] // k].
    T = 7
    xt = rng.standard_normal((T, d))
    order = rng.integers(0, T * k, R).astype(np.int32)
    np.testing.assert_array_equal(oracle.weight_grad(dgu, xt, offsets, order, k),
                                  oracle.weight_grad(dgu, xt[order // k], offsets))


@pytest.mark.parametrize("R,d,ffn,dtype", [(37, 24, 16, "f32"), (5, 64, 32, "bf16"), (1, 8, 8, "f32")])
def test_dense_expert_backward_matches_autodiff(R, d, ffn, dtype):
    """expert_backward_dense (fp64 matrix products as the chain rule's steps)
    against torch's fp64 autodiff of one expert's SwiGLU MLP, dY-weighted."""
    cfg = inputs.MoeConfig("t", 3, T=R, E=1, k=1, d=d, ffn=ffn, dtype=dtype, gating="softmax",
                           w_std=0.3)
    x = inputs.gen_x(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg)
    dy = np.random.default_rng(R + d).standard_normal((R, d))
    dx, dw13, dw2 = oracle.expert_backward_dense(x, w13[0], w2[0], dy)
    f = oracle.bf16_bits_to_f64 if dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    X = torch.tensor(f(x), requires_grad=True)
    W13 = torch.tensor(f(w13)[0], requires_grad=True)
    W2 = torch.tensor(f(w2)[0], requires_grad=True)
    (_mlp(X, W13, W2) * torch.tensor(dy)).sum().backward()
    _close(dx, X.grad.numpy(), 1e-12)
    _close(dw13, W13.grad.numpy(), 1e-12)
    _close(dw2, W2.grad.numpy(), 1e-12)
    # and the oracle's plain loops agree with it
    dx_c, dw13_c, dw2_c = oracle.expert_swiglu_backward_rows(x, np.zeros(R, np.int32), w13, w2, dy)
    _close(dx, dx_c, 1e-12)
    _close(dw13, np.asarray(dw13_c).reshape(dw13.shape), 1e-12)
    _close(dw2, np.asarray(dw2_c).reshape(dw2.shape), 1e-12)
