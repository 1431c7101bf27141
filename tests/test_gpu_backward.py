"""GPU parity of the backward pass (and of the forward product that keeps the
pre-activations) against the CPU oracle's backward (oracle.c, B0..B5), on
seeded inputs that span several 128 x 128 tiles and K slices with ragged
segment tails, empty experts and a single-row expert.

Bars: bf16 outputs within 2e-2 of the row's largest oracle magnitude; fp32
outputs per-row relative 1e-4; copies bit for bit.  The stage tests feed the
oracle's step the very values the GPU step read (a row of a weight gradient
is one output row of dW_e there).  The chain and layer tests compare with
the oracle computed from x alone, where the GPU's bf16 pre-activations
enter: weight gradients are then compared per matrix (see
test_expert_backward_chain).
"""
import numpy as np
import pytest

import oracle
from token_routing_expert_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_expert_amd as m
    m.load_library()
    return m


def dev(a):
    from token_routing_expert_amd.layer import to_device
    return to_device(a)


def host(t):
    from token_routing_expert_amd.layer import to_host
    return to_host(t)


def f64(a):
    a = np.asarray(a)
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def to_bf16(a):
    return inputs.f32_to_bf16_bits(np.asarray(a, np.float32))


def rows_close(gpu, ref, rel, what=""):
    """Per row: max |gpu - ref| <= rel * max |ref| (an all-zero row: exact)."""
    gpu = f64(gpu).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    err = np.abs(gpu - ref).max(axis=1)
    scale = np.abs(ref).max(axis=1)
    bad = err > rel * scale
    worst = float(np.max(err / np.maximum(scale, 1e-300))) if err.size else 0.0
    assert not bad.any(), f"{what}: {bad.sum()} rows off; worst rel {worst:.3g}"
    return worst


def gate_grad_close(gpu, ref, w, dgate, rel, what="dlogits"):
    """The logits' gradient takes differences of the gate gradients (e.g.
    softmax: w_j (dgate_j - sum_i w_i dgate_i)), so its rounding error scales
    with the operands, not with the (possibly cancelling) result: per token,
    |gpu - ref| <= rel * max_j |w_j| * sum_j |dgate_j|, which bounds every
    term of the formula in all four gate modes."""
    scale = np.abs(w).max(axis=1) * np.abs(dgate).sum(axis=1)
    err = np.abs(f64(gpu) - ref).max(axis=1)
    assert np.all(err <= rel * scale), f"{what}: worst {np.max(err / np.maximum(scale, 1e-300)):.3g}"
    return float(np.max(err / np.maximum(scale, 1e-300)))


def _segments_problem(seed, d, ffn, sizes, dt="bf16"):
    G, M = len(sizes), sum(sizes)
    cfg = inputs.MoeConfig("t", seed, T=max(M, 1), E=G, k=1, d=d, ffn=ffn, dtype=dt,
                           gating="softmax", w_std=0.05)
    x = inputs.gen_x(cfg)[:M]
    w13, w2 = inputs.gen_expert_weights(cfg)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    expert = np.repeat(np.arange(G, dtype=np.int32), sizes)
    dy = np.random.default_rng(seed + 7).standard_normal((M, d)).astype(np.float32)
    return x, w13, w2, offsets, expert, to_bf16(dy) if dt == "bf16" else dy


BWD_CASES = [
    # d, ffn, segment sizes: several tiles and slices, ragged tails, empty
    # and one-row experts, a segment longer than the 64-row K slice many
    # times over (the weight gradient's reduction)
    (256, 256, [1, 0, 5, 300, 128, 127, 64, 31]),
    (384, 640, [700]),
    (128, 128, [0, 0, 3]),
    (512, 256, [250, 0, 321, 97, 640, 1]),
    (256, 384, [65, 129, 0, 2]),
    # the ping-pong tiles (more rows per expert, N a multiple of 256): the
    # medium family above, the large one here, with ragged tails
    (256, 512, [300, 0, 1000, 97]),
    (512, 768, [200, 333, 260, 250]),
    # experts of 6 and 7 row tiles of 256: the tile order's blocks of 4
    # m-tiles, the last one partial
    (256, 256, [1300, 2, 1537, 257]),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("gather", [False, True])
def test_gate_up_save(lib, dt, gather):
    """h is the same bits as moe_grouped_gate_up(_gather); gu matches the
    oracle's pre-activations."""
    d, ffn, sizes = 256, 384, [100, 0, 333, 17, 1]
    x, w13, w2, offsets, expert, _ = _segments_problem(3, d, ffn, sizes, dt)
    M = len(expert)
    if gather:
        k = 2
        rng = np.random.default_rng(5)
        T = (M + k - 1) // k + 3
        order = rng.integers(0, T * k, M).astype(np.int32)
        xt = inputs.gen_x(inputs.MoeConfig("t", 9, T=T, E=1, k=1, d=d, ffn=ffn, dtype=dt,
                                           gating="softmax"))
        rows = oracle.gather_rows(xt, order, k)
        h, gu = lib.moe_grouped_gate_up_save(dev(xt), dev(offsets), dev(w13), order=dev(order), k=k)
        h_ref = lib.moe_grouped_gate_up_gather(dev(xt), dev(order), k, dev(offsets), dev(w13))
    else:
        rows = x
        h, gu = lib.moe_grouped_gate_up_save(dev(x), dev(offsets), dev(w13))
        h_ref = lib.moe_grouped_gate_up(dev(x), dev(offsets), dev(w13))
    torch.cuda.synchronize()
    assert np.array_equal(host(h).view(np.uint8), host(h_ref).view(np.uint8))
    _, _, _, gu_o, _ = oracle.expert_swiglu_backward_rows(rows, expert, w13, w2,
                                                         np.zeros((M, d)), want_dx=False,
                                                         want_dw=False, want_act=True)
    rows_close(host(gu), gu_o, 1e-4 if dt == "f32" else 2e-2, "gu")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,k,E,d", [(300, 2, 8, 256), (129, 8, 32, 512), (64, 1, 4, 128),
                                     (50, 6, 16, 136)])
def test_combine_backward(lib, dt, T, k, E, d):
    rng = np.random.default_rng(T + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, order, inv = oracle.permute_index(ids, E)
    w = rng.random((T, k)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    y_perm = rng.standard_normal((T * k, d)).astype(np.float32)
    if dt == "bf16":
        dy, y_perm = to_bf16(dy), to_bf16(y_perm)
    dy_sh = torch.empty((T, d), dtype=dev(dy).dtype, device="cuda")
    dy_perm, dgate = lib.moe_combine_backward(dev(dy), dev(inv), dev(w), dev(y_perm),
                                              dy_shared=dy_sh)
    torch.cuda.synchronize()
    ref_perm, ref_gate = oracle.combine_backward(dy, inv, w, y_perm)
    # One rounding of an exact product: within half an output ulp.
    rows_close(host(dy_perm), ref_perm, 2.0 ** -8 if dt == "bf16" else 2.0 ** -23, "dy_perm")
    # fp32 dot products of d terms: |err| <= d u sum |terms| (u = 2^-24).
    terms = np.abs(f64(dy))[:, None, :] * np.abs(f64(y_perm)[inv.reshape(T, k)])
    bound = d * 2.0 ** -24 * terms.sum(axis=2)
    assert np.all(np.abs(host(dgate) - ref_gate) <= bound + 1e-30)
    assert np.array_equal(host(dy_sh).view(np.uint8), np.ascontiguousarray(dy).view(np.uint8))


def test_combine_backward_without_gate_gradient(lib):
    T, k, E, d = 40, 2, 4, 64
    rng = np.random.default_rng(1)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, _, inv = oracle.permute_index(ids, E)
    w = rng.random((T, k)).astype(np.float32)
    dy = to_bf16(rng.standard_normal((T, d)))
    dy_perm, dgate = lib.moe_combine_backward(dev(dy), dev(inv), dev(w), want_dgate=False)
    torch.cuda.synchronize()
    assert dgate is None
    ref, _ = oracle.combine_backward(dy, inv, w, np.zeros((T * k, d), np.float32))
    rows_close(host(dy_perm), ref, 2.0 ** -8, "dy_perm")


@pytest.mark.parametrize("T,E,k,gating,renorm,ng,tg", [
    (1024, 8, 2, "softmax", 1, 1, 1), (333, 8, 2, "softmax", 0, 1, 1),
    (512, 256, 8, "sigmoid", 1, 8, 4), (200, 256, 8, "sigmoid", 1, 1, 1),
    (100, 64, 6, "sigmoid", 0, 1, 1), (77, 1000, 16, "softmax", 0, 1, 1)])
def test_gate_backward(lib, T, E, k, gating, renorm, ng, tg):
    rng = np.random.default_rng(E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(logits, k, gating, renorm, ng, tg)
    dgate = rng.standard_normal((T, k)).astype(np.float32)
    dl = lib.moe_gate_backward(dev(logits), dev(ids), dev(w), dev(dgate), gating, renorm)
    torch.cuda.synchronize()
    ref = oracle.gate_backward(logits, ids, dgate, gating, renorm)
    gate_grad_close(host(dl), ref, w, dgate, 1e-4)
    if not (gating == "softmax" and not renorm):
        chosen = np.zeros((T, E), bool)
        np.put_along_axis(chosen, ids.astype(np.int64), True, axis=1)
        assert np.all(host(dl)[~chosen] == 0.0)


def blocks_close(gpu, ref, rel, what=""):
    """Per matrix block (leading index): max |gpu - ref| <= rel * max |ref|."""
    return rows_close(np.asarray(gpu).reshape(ref.shape[0], -1), ref.reshape(ref.shape[0], -1),
                      rel, what)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", BWD_CASES)
def test_expert_backward_stages(lib, case, dt):
    """Each backward product against the oracle's step (B4a, B4b, B4c) fed
    the very inputs the GPU step read: the pre-activations, dgu and h that
    the GPU produced, the same dy and weights (fp32: the 4-wave tiles)."""
    d, ffn, sizes = case
    bar = 1e-4 if dt == "f32" else 2e-2
    x, w13, w2, offsets, expert, dy = _segments_problem(11, d, ffn, sizes, dt)
    G = len(sizes)
    xd, w13d, w2d, offd = dev(x), dev(w13), dev(w2), dev(offsets)
    h, gu = lib.moe_grouped_gate_up_save(xd, offd, w13d)
    dgu = lib.moe_grouped_down_backward(dev(dy), offd, w2d, gu)
    dx = lib.moe_grouped_gate_up_backward(dgu, offd, w13d)
    dw2 = lib.moe_grouped_weight_grad(dev(dy), h, offd)
    dw13 = lib.moe_grouped_weight_grad(dgu, xd, offd)
    torch.cuda.synchronize()
    gu_h, dgu_h, h_h = host(gu), host(dgu), host(h)
    worst = {
        "dgu": rows_close(dgu_h, oracle.down_backward_rows(dy, expert, w2, gu_h), bar, "dgu"),
        "dx": rows_close(host(dx), oracle.gate_up_backward_rows(dgu_h, expert, w13), bar, "dx"),
        "dw2": rows_close(host(dw2).reshape(-1, ffn),
                          oracle.weight_grad(dy, h_h, offsets).reshape(-1, ffn), bar, "dw2"),
        "dw13": rows_close(host(dw13).reshape(-1, d),
                           oracle.weight_grad(dgu_h, x, offsets).reshape(-1, d), bar, "dw13")}
    print(dt, case[:2], {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
    empty = [e for e, n in enumerate(sizes) if n == 0]
    assert all(np.all(host(dw2)[e] == 0) and np.all(host(dw13)[e] == 0) for e in empty)
    assert dw13.shape == (G, 2 * ffn, d)


@pytest.mark.parametrize("case", BWD_CASES)
def test_expert_backward_chain(lib, case):
    """The same chain against B4 computed from x alone (exact pre-activations,
    no rounding between the steps).  The GPU keeps g and u in bf16 (as it
    keeps h), so the error of dg scales with |dh u|, not with |dg|: where
    SiLU'(g) is near its zero the element's relative error is large.  Rows
    of dx and dgu, and each weight-gradient matrix as a whole, stay within
    the bar; a weight-gradient row of an expert with one or two rows can be
    a single such element times x, so the weight gradients are compared per
    matrix (dW_down,e, dW_gate,e, dW_up,e)."""
    d, ffn, sizes = case
    x, w13, w2, offsets, expert, dy = _segments_problem(11, d, ffn, sizes)
    G = len(sizes)
    xd, w13d, w2d, offd = dev(x), dev(w13), dev(w2), dev(offsets)
    h, gu = lib.moe_grouped_gate_up_save(xd, offd, w13d)
    dgu = lib.moe_grouped_down_backward(dev(dy), offd, w2d, gu)
    dx = lib.moe_grouped_gate_up_backward(dgu, offd, w13d)
    dw2 = lib.moe_grouped_weight_grad(dev(dy), h, offd)
    dw13 = lib.moe_grouped_weight_grad(dgu, xd, offd)
    torch.cuda.synchronize()
    dx_o, dw13_o, dw2_o, _, dgu_o = oracle.expert_swiglu_backward_rows(
        x, expert, w13, w2, f64(dy), want_act=True)
    rows_close(host(dgu), dgu_o, 2e-2, "dgu")
    rows_close(host(dx), dx_o, 2e-2, "dx")
    blocks_close(host(dw2), dw2_o, 2e-2, "dw2")
    blocks_close(host(dw13).reshape(G * 2, ffn, d), dw13_o.reshape(G * 2, ffn, d), 2e-2, "dw13")


def test_weight_grad_gather_is_bit_identical_to_packed_rows(lib):
    """Reading B's rows through order gives the same bits as the packed copy."""
    T, k, E, d, m = 500, 2, 6, 256, 256
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, offsets, order, _ = oracle.permute_index(ids, E)
    x = to_bf16(rng.standard_normal((T, d)))
    a = to_bf16(rng.standard_normal((T * k, m)))
    packed = oracle.gather_rows(x, order, k)
    g1 = lib.moe_grouped_weight_grad(dev(a), dev(x), dev(offsets), b_order=dev(order), b_k=k)
    g2 = lib.moe_grouped_weight_grad(dev(a), dev(packed), dev(offsets))
    torch.cuda.synchronize()
    assert np.array_equal(host(g1).view(np.uint8), host(g2).view(np.uint8))


def test_weight_grad_of_no_rows_is_zero(lib):
    """M = 0 still writes every expert's gradient (all zero)."""
    out = torch.full((3, 128, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    a = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    offsets = torch.zeros(4, dtype=torch.int32, device="cuda")
    lib.moe_grouped_weight_grad(a, b, offsets, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("m,n", [(128, 256), (256, 512)])
def test_weight_grad_of_empty_segments_is_zero_on_both_kernels(lib, m, n):
    """Experts with no rows get zero gradients on the 4-wave tiles (m = 128)
    and on the ping-pong tiles (m, n multiples of 256), next to experts that
    have rows."""
    sizes = [0, 70, 0, 300, 0]
    M = sum(sizes)
    rng = np.random.default_rng(17)
    a = to_bf16(rng.standard_normal((M, m)))
    b = to_bf16(rng.standard_normal((M, n)))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    out = torch.full((len(sizes), m, n), 3.0, dtype=torch.bfloat16, device="cuda")
    lib.moe_grouped_weight_grad(dev(a), dev(b), dev(offsets), out)
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle.weight_grad(a, b, offsets)
    for e, k in enumerate(sizes):
        if k == 0:
            assert np.all(got[e] == 0)
        else:
            rows_close(got[e], ref[e], 2e-2, f"dW[{e}]")


def test_unit_gate_combine_sums_rows(lib):
    """moe_unpermute_combine with no gates is the permute's backward: each
    token gets the sum of its k rows (plus the shared row)."""
    T, k, E, d = 77, 3, 5, 64
    rng = np.random.default_rng(8)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, _, inv = oracle.permute_index(ids, E)
    rows = to_bf16(rng.standard_normal((T * k, d)))
    sh = to_bf16(rng.standard_normal((T, d)))
    y = lib.moe_unpermute_combine(dev(rows), dev(inv), None, dev(sh), k=k)
    torch.cuda.synchronize()
    ref = oracle.combine(rows, inv, np.ones((T, k), np.float32), sh)
    rows_close(host(y), ref, 2.0 ** -8, "dx")


def test_layer_backward_small_fp32(lib):
    """The small fp32 layer (1,024 tokens, 8 experts, top-2 softmax) trained:
    every gradient within the fp32 bar of 1e-4 per row (weight gradients per
    output row) of the oracle's fp64 backward."""
    from token_routing_expert_amd.layer import MoeLayer
    cfg = inputs.CONFIGS["small_fp32"]
    x, logits = inputs.gen_x(cfg), inputs.gen_logits(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg)
    dy = np.random.default_rng(8).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    layer = MoeLayer(cfg, x, w13, w2, logits=logits, device="cuda", fused_gather=True, train=True)
    layer.forward()
    g = layer.backward(dev(dy))
    torch.cuda.synchronize()
    ids, w = oracle.route(logits, cfg.k, cfg.gating, cfg.renormalize)
    ref = oracle.layer_backward(x, logits, ids, w, w13, w2, dy, cfg.gating, cfg.renormalize)
    worst = {"dx": rows_close(host(g["dx"]), ref["dx"], 1e-4, "dx"),
             "dw13": rows_close(host(g["dw13"]).reshape(-1, cfg.d), ref["dw13"].reshape(-1, cfg.d),
                                1e-4, "dw13"),
             "dw2": rows_close(host(g["dw2"]).reshape(-1, cfg.ffn), ref["dw2"].reshape(-1, cfg.ffn),
                               1e-4, "dw2"),
             "dlogits": gate_grad_close(host(g["dlogits"]), ref["dlogits"], w,
                                        host(g["dgate"]).astype(np.float64), 1e-4)}
    print("small_fp32", {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)


LAYER_CASES = [
    # name, T, E, k, d, ffn, gating, renorm, groups, shared, merge, fused
    ("small_bf16", 1024, 8, 2, 256, 512, "softmax", 1, (1, 1), False, False, True),
    ("grouped_shared", 512, 32, 4, 256, 256, "sigmoid", 1, (4, 2), True, False, True),
    ("merged_shared", 384, 16, 2, 256, 384, "sigmoid", 1, (1, 1), True, True, True),
    # T <= 256: the shared expert runs on the split-reduction kernel, which
    # also writes the pre-activations its backward reads.
    ("dense_shared", 128, 32, 4, 256, 256, "sigmoid", 1, (4, 2), True, False, True),
    ("packed_rows", 300, 8, 2, 384, 256, "softmax", 0, (1, 1), False, False, False),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_backward_matches_oracle(lib, case):
    from token_routing_expert_amd.layer import MoeLayer
    name, T, E, k, d, ffn, gating, renorm, (ng, tg), shared, merge, fused = case
    cfg = inputs.MoeConfig(name, 21, T=T, E=E, k=k, d=d, ffn=ffn, dtype="bf16", gating=gating,
                           renormalize=renorm, n_groups=ng, topk_groups=tg, shared=int(shared),
                           w_std=0.05)
    x, logits = inputs.gen_x(cfg), inputs.gen_logits(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg)
    sh13, sh2 = inputs.gen_expert_weights(cfg, shared=True) if shared else (None, None)
    dy = to_bf16(np.random.default_rng(3).standard_normal((T, d)))
    layer = MoeLayer(cfg, x, w13, w2, logits=logits, sh_w13=sh13, sh_w2=sh2, device="cuda",
                     fused_gather=fused, merge_shared=merge, train=True)
    if shared and not merge:
        assert layer.sh_dense == (T <= 256)
    layer.forward()
    g = layer.backward(dev(dy))
    torch.cuda.synchronize()
    ids, w = oracle.route(logits, k, gating, renorm, ng, tg)
    assert np.array_equal(host(layer.topk_ids), ids)
    ref = oracle.layer_backward(x, logits, ids, w, w13, w2, dy, gating, renorm, sh13, sh2)
    # Weight gradients per matrix (see test_expert_backward_chain).
    worst = {"dx": rows_close(host(g["dx"]), ref["dx"], 2e-2, "dx"),
             "dw13": blocks_close(host(g["dw13"]).reshape(-1, ffn, d), ref["dw13"].reshape(-1, ffn, d),
                                  2e-2, "dw13"),
             "dw2": blocks_close(host(g["dw2"]), ref["dw2"], 2e-2, "dw2")}
    # The gate gradient is a dot product of dy with the expert output, which
    # the forward keeps in bf16; its error scales with sum_m |dy y|, not with
    # the (cancelling) sum itself.  The logits' gradient is then checked on
    # the GPU's gate gradient: it takes differences of the gate gradients
    # (softmax: w_j (dgate_j - sum_i w_i dgate_i)), which cancel as well.
    dgate = host(g["dgate"]).astype(np.float64)
    y_rows = oracle.expert_swiglu_rows(np.repeat(x, k, axis=0), ids.reshape(-1), w13, w2)
    absdot = (np.abs(f64(dy))[:, None, :] * np.abs(y_rows.reshape(T, k, d))).sum(axis=2)
    assert np.all(np.abs(dgate - ref["dgate"]) <= 2e-2 * absdot), "dgate"
    worst["dgate"] = float(np.max(np.abs(dgate - ref["dgate"]) / absdot))
    worst["dlogits"] = gate_grad_close(host(g["dlogits"]),
                                       oracle.gate_backward(logits, ids, dgate, gating, renorm), w,
                                       dgate, 1e-4)
    if shared:
        worst["dsh_w13"] = blocks_close(host(g["dsh_w13"]).reshape(-1, ffn, d),
                                        ref["dsh_w13"].reshape(-1, ffn, d), 2e-2, "dsh_w13")
        worst["dsh_w2"] = blocks_close(host(g["dsh_w2"]), ref["dsh_w2"], 2e-2, "dsh_w2")
    print(name, {k_: f"{v:.2e}" for k_, v in worst.items()}, flush=True)


def test_router_backward(lib):
    """dx += dlogits w_router and dw_router = dlogits^T x against the oracle's
    B0 (the GPU rounds dlogits to bf16 once, inside the 2e-2 bar)."""
    T, E, d = 700, 256, 512
    rng = np.random.default_rng(31)
    dl = (1e-2 * rng.standard_normal((T, E))).astype(np.float32)
    x = to_bf16(rng.standard_normal((T, d)))
    wr = to_bf16(rng.standard_normal((E, d)) / np.sqrt(d))
    dx0 = to_bf16(rng.standard_normal((T, d)))
    dx = dev(dx0)
    dwr = lib.moe_router_backward(dev(dl), dev(x), dev(wr), dx)
    torch.cuda.synchronize()
    ref_dx, ref_dw = oracle.router_backward(x, wr, dl)
    rows_close(host(dx), ref_dx + f64(dx0), 2e-2, "dx")
    rows_close(host(dwr), ref_dw, 2e-2, "dw_router")
    for T_, E_, d_ in ((50, 256, 512), (700, 8, 512), (700, 256, 384)):
        with pytest.raises(lib.MoeError):
            lib.moe_router_backward(torch.zeros((T_, E_), device="cuda"),
                                    torch.zeros((T_, d_), dtype=torch.bfloat16, device="cuda"),
                                    torch.zeros((E_, d_), dtype=torch.bfloat16, device="cuda"))


def test_layer_backward_with_router(lib):
    """A training step with the router product in front: dx includes the
    router's part, dw_router its weight gradient; the oracle takes the GPU's
    logits (the route is bit-exact on them) and the same router weights."""
    from token_routing_expert_amd.layer import MoeLayer
    cfg = inputs.MoeConfig("router_train", 23, T=512, E=256, k=8, d=256, ffn=256, dtype="bf16",
                           gating="sigmoid", renormalize=1, n_groups=8, topk_groups=4, w_std=0.05)
    x = inputs.gen_x(cfg)
    w13, w2 = inputs.gen_expert_weights(cfg)
    wr = inputs.gen_router_weights(cfg)
    dy = to_bf16(np.random.default_rng(4).standard_normal((cfg.T, cfg.d)))
    layer = MoeLayer(cfg, x, w13, w2, device="cuda", fused_gather=True, w_router=wr, train=True)
    layer.forward()
    g = layer.backward(dev(dy))
    torch.cuda.synchronize()
    logits = host(layer.logits)
    ids, w = oracle.route(logits, cfg.k, cfg.gating, 1, 8, 4)
    assert np.array_equal(host(layer.topk_ids), ids)
    ref = oracle.layer_backward(x, logits, ids, w, w13, w2, dy, "sigmoid", 1, wg=wr)
    worst = {"dx": rows_close(host(g["dx"]), ref["dx"], 2e-2, "dx"),
             "dw_router": rows_close(host(g["dw_router"]), ref["dwg"], 2e-2, "dw_router"),
             "dw13": blocks_close(host(g["dw13"]).reshape(-1, cfg.ffn, cfg.d),
                                  ref["dw13"].reshape(-1, cfg.ffn, cfg.d), 2e-2, "dw13")}
    print("router_train", {k_: f"{v:.2e}" for k_, v in worst.items()}, flush=True)


def test_training_step_graph_replays_bitwise(lib):
    """Forward + backward captured in one HIP graph (no call allocates,
    synchronises or writes with a memset once the buffers exist) replays to
    the eager step's bits, with eager work between the replays."""
    from token_routing_expert_amd.layer import MoeLayer
    cfg = inputs.MoeConfig("graph_train", 25, T=512, E=256, k=8, d=256, ffn=256, dtype="bf16",
                           gating="sigmoid", renormalize=1, n_groups=8, topk_groups=4, shared=True,
                           w_std=0.05)
    w13, w2 = inputs.gen_expert_weights(cfg)
    sh = inputs.gen_expert_weights(cfg, shared=True)
    L = MoeLayer(cfg, inputs.gen_x(cfg), w13, w2, sh_w13=sh[0], sh_w2=sh[1], device="cuda",
                 fused_gather=True, w_router=inputs.gen_router_weights(cfg), train=True)
    dy = dev(to_bf16(np.random.default_rng(6).standard_normal((cfg.T, cfg.d))))

    def step():
        L.forward()
        return L.backward(dy)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for v in out.values():
            v.zero_()                # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, ref[k]), (i, k)
