"""The Python binding's own argument checks (host side, before any call into
the library): non-device tensors, wrong dtypes and inconsistent shapes raise
MoeError.  CPU only: every case is rejected before a kernel could launch."""
import pytest

import token_routing_expert_amd as moe

torch = pytest.importorskip("torch")


def cpu(*shape, dtype=None):
    return torch.zeros(shape, dtype=dtype or torch.float32)


def test_host_tensors_are_rejected():
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_route_topk(cpu(4, 8), 2)
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_router_logits(cpu(4, 128), cpu(8, 128))
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_permute(cpu(4, 16), cpu(4, 2, dtype=torch.int32), 4)
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_grouped_swiglu(cpu(4, 128), cpu(2, dtype=torch.int32), cpu(1, 2, 128, 128),
                               cpu(1, 128, 128))
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_unpermute_combine(cpu(8, 16), cpu(8, dtype=torch.int32), cpu(4, 2))
    with pytest.raises(moe.MoeError, match="device tensor"):
        moe.moe_router_bias_update(cpu(4, dtype=torch.int32), cpu(4), 0.1)


def test_wrong_dtypes_are_rejected():
    # dtype checks run before the device check only where the tensor is on a
    # device; on the host the device check fires first, with the same class
    with pytest.raises(moe.MoeError):
        moe.moe_route_topk(cpu(4, 8, dtype=torch.float64), 2)
    with pytest.raises(moe.MoeError):
        moe.moe_sigmoid_pinned(cpu(4, dtype=torch.int32))


def test_library_loads_without_a_gpu():
    lib = moe.load_library()
    assert lib.moe_status_string(-2).decode()
