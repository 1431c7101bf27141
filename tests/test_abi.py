"""The C-ABI library loads and exports every entry point include/moe355.h
declares; host-side argument validation rejects bad calls before any launch.
CPU only: nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

import token_routing_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe355.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe355.so not built (run __graft_entry__.build())")
    return moe.load_library()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3):
        s = lib.moe_status_string(code).decode()
        assert s.startswith("MOE_")
    assert lib.moe_status_string(7).decode() == "unknown moe_status"


def test_workspace_bytes(lib):
    assert lib.moe_permute_workspace_bytes(8192, 8, 256) == 32 * 256 * 4     # 2048-row chunks
    assert lib.moe_permute_workspace_bytes(1, 1, 4) == 4 * 4
    assert lib.moe_permute_workspace_bytes(0, 8, 256) == 16
    big = lib.moe_permute_workspace_bytes(1 << 22, 8, 1024)
    assert big <= 1024 * 1024 * 4                                           # at most 1024 chunks


INVALID, UNSUPPORTED = -1, -2
NULL = None


def test_route_validation(lib):
    f = lib.moe_route_topk
    assert f(NULL, -1, 8, 2, 0, 1, 1, 1, NULL, NULL, NULL) == INVALID        # T < 0
    assert f(NULL, 4, 8, 9, 0, 1, 1, 1, NULL, NULL, NULL) == INVALID         # k > E
    assert f(NULL, 4, 8, 0, 0, 1, 1, 1, NULL, NULL, NULL) == INVALID         # k < 1
    assert f(NULL, 4, 8, 2, 0, 1, 3, 1, NULL, NULL, NULL) == INVALID         # E % n_groups
    assert f(NULL, 4, 8, 2, 1, 1, 4, 5, NULL, NULL, NULL) == INVALID         # topk_groups > n_groups
    assert f(NULL, 4, 8, 2, 1, 1, 8, 1, NULL, NULL, NULL) == INVALID         # group of one expert
    assert f(NULL, 4, 8, 8, 1, 1, 4, 1, NULL, NULL, NULL) == INVALID         # kept groups too few
    assert f(NULL, 4, 8, 2, 5, 1, 1, 1, NULL, NULL, NULL) == INVALID         # bad gating
    assert f(NULL, 4, 2048, 2, 0, 1, 1, 1, NULL, NULL, NULL) == UNSUPPORTED  # E > 1024
    assert f(NULL, 4, 64, 17, 0, 1, 1, 1, NULL, NULL, NULL) == UNSUPPORTED   # k > 16
    assert f(NULL, 4, 8, 2, 0, 1, 1, 1, NULL, NULL, NULL) == INVALID         # null pointers
    assert f(NULL, 0, 8, 2, 0, 1, 1, 1, NULL, NULL, NULL) == 0               # T = 0: no-op


def test_send_counts_validation(lib):
    f = lib.moe_send_counts
    assert f(NULL, 6, 2, 4, 4, NULL, NULL) == INVALID                        # T % n_ep
    assert f(NULL, 8, 2, 6, 4, NULL, NULL) == INVALID                        # E % n_ep
    assert f(NULL, 8, 2, 8, 0, NULL, NULL) == INVALID
    assert f(NULL, 4096, 1, 2048, 2048, NULL, NULL) == UNSUPPORTED
    assert f(NULL, 8, 2, 8, 4, NULL, NULL) == INVALID                        # null pointers


def test_permute_validation(lib):
    f = lib.moe_permute
    a = ctypes.c_void_p(16)     # a well-aligned non-null value; never dereferenced on error paths
    b = ctypes.c_void_p(24)     # misaligned
    ws = lib.moe_permute_workspace_bytes(4, 2, 8)
    assert f(a, 1, 4, 12, a, 2, 8, a, a, a, a, a, a, ws, NULL) == UNSUPPORTED   # d % 8
    assert f(a, 1, 4, 16, a, 2, 2000, a, a, a, a, a, a, ws, NULL) == UNSUPPORTED  # E > 1024
    assert f(a, 1, 4, 16, a, 2, 8, a, a, a, a, a, a, ws - 1, NULL) == INVALID   # workspace
    assert f(b, 1, 4, 16, a, 2, 8, a, a, a, a, a, a, ws, NULL) == INVALID       # misaligned x
    assert f(a, 1, 4, 16, NULL, 2, 8, a, a, a, a, a, a, ws, NULL) == INVALID    # null ids
    assert f(a, 7, 4, 16, a, 2, 8, a, a, a, a, a, a, ws, NULL) == INVALID       # dtype
    assert f(a, 1, -1, 16, a, 2, 8, a, a, a, a, a, a, ws, NULL) == INVALID


def test_grouped_swiglu_validation(lib):
    f = lib.moe_grouped_swiglu
    a = ctypes.c_void_p(16)
    assert f(a, 1, 64, 96, 256, a, 4, a, a, a, a, NULL) == UNSUPPORTED      # d % 128
    assert f(a, 1, 64, 128, 200, a, 4, a, a, a, a, NULL) == UNSUPPORTED     # ffn % 128
    assert f(a, 1, 64, 128, 256, a, 5000, a, a, a, a, NULL) == UNSUPPORTED  # G > 4096
    assert f(a, 1, 64, 128, 256, a, 0, a, a, a, a, NULL) == INVALID         # G < 1
    assert f(a, 1, 64, 128, 256, NULL, 4, a, a, a, a, NULL) == INVALID      # null offsets
    assert f(ctypes.c_void_p(8), 1, 64, 128, 256, a, 4, a, a, a, a, NULL) == INVALID
    assert f(a, 1, 0, 128, 256, NULL, 4, NULL, NULL, NULL, NULL, NULL) == 0  # M = 0: no-op


def test_grouped_halves_validation(lib):
    a = ctypes.c_void_p(16)
    for f, args in ((lib.moe_grouped_gate_up, lambda M, d, ffn, off, G, p: (a, 1, M, d, ffn, off, G, a, p, NULL)),
                    (lib.moe_grouped_down, lambda M, d, ffn, off, G, p: (a, 1, M, ffn, d, off, G, a, p, NULL))):
        assert f(*args(64, 96, 256, a, 4, a)) == UNSUPPORTED       # d % 128
        assert f(*args(64, 128, 200, a, 4, a)) == UNSUPPORTED      # ffn % 128
        assert f(*args(64, 128, 256, a, 5000, a)) == UNSUPPORTED   # G > 4096
        assert f(*args(64, 128, 256, a, 0, a)) == INVALID          # G < 1
        assert f(*args(64, 128, 256, NULL, 4, a)) == INVALID       # null offsets
        assert f(*args(64, 128, 256, a, 4, NULL)) == INVALID       # null output
        assert f(*args(64, 128, 256, a, 4, ctypes.c_void_p(24))) == INVALID   # misaligned output
        assert f(*args(0, 128, 256, NULL, 4, NULL)) == 0           # M = 0: no-op


def test_gate_up_gather_validation(lib):
    f = lib.moe_grouped_gate_up_gather
    a = ctypes.c_void_p(16)
    #       x  dt T  k  M   d    ffn  order off G  w13 h  stream
    assert f(a, 1, 8, 0, 16, 128, 256, a, a, 4, a, a, NULL) == INVALID          # k < 1
    assert f(a, 1, 8, 2, -1, 128, 256, a, a, 4, a, a, NULL) == INVALID          # M < 0
    assert f(a, 1, 8, 2, 16, 96, 256, a, a, 4, a, a, NULL) == UNSUPPORTED       # d % 128
    assert f(a, 1, 8, 2, 16, 128, 256, NULL, a, 4, a, a, NULL) == INVALID       # null order
    assert f(a, 1, 8, 2, 16, 128, 256, a, a, 4, a, ctypes.c_void_p(24), NULL) == INVALID
    assert f(a, 1, 1 << 20, 2, 16, 4096, 256, a, a, 4, a, a, NULL) == UNSUPPORTED  # x >= 4 GiB
    assert f(NULL, 1, 8, 2, 0, 128, 256, NULL, NULL, 4, NULL, NULL, NULL) == 0    # M = 0: no-op


def test_permute_index_only_validation(lib):
    f = lib.moe_permute
    a = ctypes.c_void_p(16)
    ws = lib.moe_permute_workspace_bytes(8, 2, 4)
    #       x     dt T  d   ids k  E  counts off order inv x_perm ws  bytes
    assert f(a, 1, 8, 16, a, 2, 4, a, a, a, a, NULL, a, ws, NULL) == INVALID   # x without x_perm
    assert f(NULL, 1, 8, 16, a, 2, 4, a, a, a, a, a, a, ws, NULL) == INVALID   # x_perm without x


def test_router_validation(lib):
    a = ctypes.c_void_p(16)
    f = lib.moe_router_logits
    #       x  dt T  d    w  E  logits stream
    assert f(a, 1, 4, 96, a, 8, a, NULL) == UNSUPPORTED      # 192-byte rows
    assert f(a, 1, 4, 128, a, 0, a, NULL) == INVALID         # E < 1
    assert f(a, 1, 4, 128, NULL, 8, a, NULL) == INVALID      # null weights
    assert f(a, 1, 4, 128, ctypes.c_void_p(24), 8, a, NULL) == INVALID   # misaligned
    assert f(NULL, 1, 0, 128, NULL, 8, NULL, NULL) == 0      # T = 0: no-op
    g = lib.moe_router_bias_update
    assert g(a, 0, ctypes.c_float(1.0), a, NULL) == INVALID
    assert g(a, 2000, ctypes.c_float(1.0), a, NULL) == UNSUPPORTED
    assert g(NULL, 4, ctypes.c_float(1.0), a, NULL) == INVALID
    h = lib.moe_route_topk_biased
    #       logits bias T  E  k  gating renorm ng tg ids w  stream
    assert h(a, NULL, 4, 8, 2, 0, 1, 1, 1, a, a, NULL) == INVALID   # null bias
    assert h(a, a, 4, 8, 9, 0, 1, 1, 1, a, a, NULL) == INVALID      # k > E
    assert h(NULL, NULL, 0, 8, 2, 0, 1, 1, 1, NULL, NULL, NULL) == 0


def test_combine_validation(lib):
    f = lib.moe_unpermute_combine
    a = ctypes.c_void_p(16)
    assert f(a, 1, 4, 2, 12, a, a, NULL, a, NULL) == UNSUPPORTED            # d % 8
    assert f(a, 1, 4, 65, 16, a, a, NULL, a, NULL) == UNSUPPORTED           # k > 64
    assert f(a, 1, 4, 0, 16, a, a, NULL, a, NULL) == INVALID
    assert f(a, 1, 4, 2, 16, NULL, a, NULL, a, NULL) == INVALID
    assert f(a, 1, 4, 2, 16, a, a, ctypes.c_void_p(40), a, NULL) == INVALID  # misaligned shared
    assert f(a, 1, 0, 2, 16, NULL, NULL, NULL, NULL, NULL) == 0


def test_backward_validation(lib):
    a = ctypes.c_void_p(16)
    mis = ctypes.c_void_p(24)
    f = lib.moe_grouped_gate_up_save
    #       x  dt T  k  M   d    ffn  order off G  w13 h  gu    stream
    assert f(a, 1, 8, 2, 16, 128, 256, a, a, 4, a, a, NULL, NULL) == INVALID      # null gu
    assert f(a, 1, 8, 2, 16, 128, 256, a, a, 4, a, a, mis, NULL) == INVALID       # misaligned gu
    assert f(a, 1, 8, 2, 16, 96, 256, a, a, 4, a, a, a, NULL) == UNSUPPORTED      # d % 128
    assert f(NULL, 1, 8, 2, 0, 128, 256, NULL, NULL, 4, NULL, NULL, NULL, NULL) == 0
    f = lib.moe_combine_backward
    #       dy dt T  k  d   inv w  y_perm dy_perm dgate dy_sh stream
    assert f(a, 1, 4, 2, 16, a, a, a, a, NULL, NULL, NULL) == INVALID       # y_perm without dgate
    assert f(a, 1, 4, 2, 16, a, a, NULL, a, a, NULL, NULL) == INVALID       # dgate without y_perm
    assert f(a, 1, 4, 2, 12, a, a, a, a, a, NULL, NULL) == UNSUPPORTED      # d % 8
    assert f(a, 1, 4, 65, 16, a, a, a, a, a, NULL, NULL) == UNSUPPORTED     # k > 64
    assert f(a, 1, 4, 2, 16, a, NULL, a, a, a, NULL, NULL) == INVALID       # null gates
    assert f(a, 1, 4, 2, 16, a, a, a, mis, a, NULL, NULL) == INVALID        # misaligned dy_perm
    assert f(NULL, 1, 0, 2, 16, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 0
    f = lib.moe_gate_backward
    #       logits ids w  dgate T  E  k  gating renorm dl stream
    assert f(a, a, a, a, 4, 8, 9, 0, 1, a, NULL) == INVALID                 # k > E
    assert f(a, a, a, a, 4, 8, 2, 7, 1, a, NULL) == INVALID                 # gating
    assert f(a, a, a, NULL, 4, 8, 2, 0, 1, a, NULL) == INVALID              # null dgate
    assert f(a, a, a, a, 4, 5000, 2, 0, 1, a, NULL) == UNSUPPORTED          # E > 4096
    assert f(NULL, NULL, NULL, NULL, 0, 8, 2, 0, 1, NULL, NULL) == 0
    for g in (lib.moe_grouped_down_backward, lib.moe_grouped_gate_up_backward):
        extra = (a,) if g is lib.moe_grouped_down_backward else ()
        #          a  dt M   d    ffn  off G  w  [gu] out stream
        assert g(a, 7, 64, 128, 256, a, 4, a, *extra, a, NULL) == INVALID       # dtype
        assert g(a, 1, 64, 96, 256, a, 4, a, *extra, a, NULL) == UNSUPPORTED    # d % 128
        assert g(a, 1, 64, 128, 200, a, 4, a, *extra, a, NULL) == UNSUPPORTED   # ffn % 128
        assert g(a, 1, 64, 128, 256, a, 0, a, *extra, a, NULL) == INVALID       # G < 1
        assert g(a, 1, 64, 128, 256, NULL, 4, a, *extra, a, NULL) == INVALID    # null offsets
        assert g(a, 1, 64, 128, 256, a, 4, a, *extra, mis, NULL) == INVALID     # misaligned out
        assert g(a, 1, 0, 128, 256, NULL, 4, NULL, *((NULL,) if extra else ()), NULL, NULL) == 0
    g = lib.moe_grouped_weight_grad
    #       a  b  dt M   m    n    off G  order bk brows c  stream
    assert g(a, a, 7, 64, 128, 256, a, 4, NULL, 1, 0, a, NULL) == INVALID       # dtype
    assert g(a, a, 1, 64, 96, 256, a, 4, NULL, 1, 0, a, NULL) == UNSUPPORTED    # m % 128
    assert g(a, a, 1, 64, 128, 256, a, 4, NULL, 0, 0, a, NULL) == INVALID       # b_k < 1
    assert g(a, a, 1, 64, 128, 256, a, 4, a, 2, 0, a, NULL) == INVALID          # b_rows < 1
    assert g(a, a, 1, 64, 128, 256, NULL, 4, NULL, 1, 0, a, NULL) == INVALID    # null offsets
    assert g(a, mis, 1, 64, 128, 256, a, 4, NULL, 1, 0, a, NULL) == INVALID     # misaligned b


def test_router_backward_validation(lib):
    a = ctypes.c_void_p(16)
    ws = lib.moe_router_backward_workspace_bytes(512, 256)
    assert ws >= 512 * 256 * 2
    f = lib.moe_router_backward
    #       dl x  dt T    d    wr E    dx dw ws bytes stream
    assert f(a, a, 0, 512, 512, a, 256, a, a, a, ws, NULL) == UNSUPPORTED    # fp32
    assert f(a, a, 1, 512, 512, a, 8, a, a, a, ws, NULL) == UNSUPPORTED      # E % 256
    assert f(a, a, 1, 50, 512, a, 256, a, a, a, ws, NULL) == UNSUPPORTED     # T < 96
    assert f(a, a, 1, 512, 512, a, 256, a, a, a, ws - 1, NULL) == INVALID    # small workspace
    assert f(a, a, 1, 512, 512, NULL, 256, a, a, a, ws, NULL) == INVALID     # null weights
    assert f(a, a, 1, 512, 512, a, 256, NULL, NULL, NULL, 0, NULL) == 0      # nothing asked


def test_dense_swiglu_validation(lib):
    a = ctypes.c_void_p(16)
    ws = lib.moe_dense_swiglu_workspace_bytes(128, 7168, 2048)
    # gate/up split 8 ways: 8 x 128 x 4096 fp32 partial sums
    assert ws == 8 * 128 * 4096 * 4
    f = lib.moe_dense_swiglu
    #       x  dt M    d    ffn w13 w2 h gu    y  ws bytes stream
    assert f(a, 0, 128, 256, 128, a, a, a, NULL, a, a, ws, NULL) == UNSUPPORTED   # fp32
    assert f(a, 1, 257, 256, 128, a, a, a, NULL, a, a, ws, NULL) == UNSUPPORTED   # M > 256
    assert f(a, 1, 128, 200, 128, a, a, a, NULL, a, a, ws, NULL) == UNSUPPORTED   # d % 64
    assert f(a, 1, -1, 256, 128, a, a, a, NULL, a, a, ws, NULL) == INVALID
    small = lib.moe_dense_swiglu_workspace_bytes(128, 256, 128)
    assert f(a, 1, 128, 256, 128, a, a, a, NULL, a, a, small - 1, NULL) == INVALID
    assert f(a, 1, 128, 256, 128, a, NULL, a, NULL, a, a, small, NULL) == INVALID  # null w2
    assert f(a, 1, 128, 256, 128, a, a, a, ctypes.c_void_p(8), a, a, small, NULL) == INVALID  # gu alignment
    assert f(NULL, 1, 0, 256, 128, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 0   # no rows


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(moe.MoeError):
        moe.load_library(str(tmp_path / "missing.so"))


def test_capacity_host_function(lib):
    """moe_expert_capacity against the oracle's independent ceil(cf M / E)."""
    import oracle
    lib.moe_expert_capacity.restype = ctypes.c_int64
    lib.moe_expert_capacity.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_double]
    for M in (0, 1, 12, 2048, 32768, 65536, 999_999):
        for E in (1, 3, 4, 8, 256, 1024):
            for cf in (0.01, 0.5, 1.0, 1.1, 1.25, 2.0, 7.3):
                assert lib.moe_expert_capacity(M, E, cf) == oracle.expert_capacity(M, E, cf)
    assert lib.moe_expert_capacity(10, 0, 1.0) == -1
    assert lib.moe_expert_capacity(10, 4, 0.0) == -1
    assert lib.moe_expert_capacity(-1, 4, 1.0) == -1


def test_permute_capacity_validation(lib):
    f = lib.moe_permute_capacity
    P = ctypes.c_void_p
    fake = P(4096)   # never dereferenced: every call below fails its host checks
    ws = lib.moe_permute_capacity_workspace_bytes(64, 2, 8)
    assert ws == lib.moe_permute_workspace_bytes(64, 2, 8) + 9 * 4
    args = lambda T=64, k=2, E=8, cap=16, wsb=ws: (fake, 1, T, 64, fake, k, E, cap, fake, fake, fake,
                                                   fake, fake, fake, wsb, NULL)
    assert f(*args(T=-1)) == INVALID
    assert f(*args(k=0)) == INVALID
    assert f(*args(cap=-1)) == INVALID
    assert f(*args(E=2048)) == UNSUPPORTED
    assert f(*args(E=1024, cap=1 << 21)) == UNSUPPORTED     # E cap >= 2^31
    assert f(*args(wsb=ws - 4)) == INVALID                  # workspace too small
    assert f(fake, 1, 64, 64, fake, 2, 8, 16, NULL, fake, fake, fake, fake, fake, ws, NULL) == INVALID
    # exactly one of x, x_cap given
    assert f(fake, 1, 64, 64, fake, 2, 8, 16, fake, fake, fake, fake, NULL, fake, ws, NULL) == INVALID


def test_combine_rows_and_loop_validation(lib):
    P = ctypes.c_void_p
    fake = P(4096)
    lib.moe_unpermute_combine_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, P, P, P, P, P]
    g = lib.moe_unpermute_combine_rows
    assert g(fake, -1, 1, 4, 2, 64, fake, fake, NULL, fake, NULL) == INVALID   # rows < 0
    assert g(NULL, 8, 1, 4, 2, 64, fake, fake, NULL, fake, NULL) == INVALID    # rows > 0, no y_perm
    assert g(fake, 8, 1, 0, 2, 64, fake, fake, NULL, fake, NULL) == 0          # T = 0: no-op
    h = lib.moe_expert_loop_swiglu
    bad = (ctypes.c_int32 * 3)(0, 6, 4)
    out_of_range = (ctypes.c_int32 * 3)(0, 4, 9)
    assert h(fake, 1, 8, 128, 128, fake, NULL, 2, fake, fake, fake, fake, NULL) == INVALID
    assert h(fake, 1, 8, 128, 128, fake, bad, 2, fake, fake, fake, fake, NULL) == INVALID
    assert h(fake, 1, 8, 128, 128, fake, out_of_range, 2, fake, fake, fake, fake, NULL) == INVALID
    assert h(fake, 1, 8, 96, 128, fake, bad, 2, fake, fake, fake, fake, NULL) == UNSUPPORTED  # d % 128
