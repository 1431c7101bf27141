"""moe_permute_noalloc (the permute for callers that cannot allocate: its
histograms live in a library-owned device array) against moe_permute with a
caller workspace: two calls in a row, the second on a smaller input, every
output bit for bit, and neither call changing the memory torch or the device
report as allocated."""
import gc

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_expert_amd as m
    m.load_library()
    return m


def _case(T, k, E, d, seed):
    r = np.random.default_rng(seed)
    p = np.r_[0.4, np.full(E - 1, 0.6 / (E - 1))]
    ids = np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(r.standard_normal((T, d), dtype=np.float32)).to("cuda").to(torch.bfloat16)
    return torch.from_numpy(ids).to("cuda"), x


def _outputs(T, k, E, d):
    i32 = torch.int32
    return (torch.full((E,), -7, dtype=i32, device="cuda"),
            torch.full((E + 1,), -7, dtype=i32, device="cuda"),
            torch.full((T * k,), -7, dtype=i32, device="cuda"),
            torch.full((T * k,), -7, dtype=i32, device="cuda"),
            torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("rows", [True, False])
def test_noalloc_permute_matches_workspace_permute(lib, rows):
    # First call: DeepSeek-V3 prefill's shape of the index work (8192 tokens,
    # top-8 of 256); second: a smaller batch with other experts and rows.
    for T, k, E, d, seed in ((8192, 8, 256, 256, 1), (1000, 2, 64, 512, 2)):
        ids, x = _case(T, k, E, d, seed)
        want = lib.moe_permute(x, ids, E, rows=rows)
        got_bufs = _outputs(T, k, E, d)
        if not rows:
            got_bufs = got_bufs[:4] + (None,)
        torch.cuda.synchronize()
        gc.collect()
        before = torch.cuda.memory_allocated()
        free_before = torch.cuda.mem_get_info()[0]
        got = lib.moe_permute_noalloc(x, ids, E, *got_bufs)
        torch.cuda.synchronize()
        # No growth (garbage collected during the call may only shrink them).
        assert torch.cuda.memory_allocated() <= before
        assert torch.cuda.mem_get_info()[0] >= free_before
        for name, a, b in zip(("counts", "offsets", "order", "inv", "x_perm"), got, want):
            if b is None:
                assert a is None
                continue
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (T, name)


def test_noalloc_permute_rejects_oversized_workspace(lib):
    """E = 1024 with T k = 2^19 + 2048 needs more than the 1 MiB array: the
    call is refused before any launch."""
    T, k, E = (1 << 19) + 2048, 1, 1024
    i32 = torch.int32
    ids = torch.zeros((T, k), dtype=i32, device="cuda")
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device="cuda")
    assert lib.moe_permute_workspace_bytes(T, k, E) > (1 << 20)
    outs = (torch.empty(E, dtype=i32, device="cuda"), torch.empty(E + 1, dtype=i32, device="cuda"),
            torch.empty(T * k, dtype=i32, device="cuda"), torch.empty(T * k, dtype=i32, device="cuda"))
    with pytest.raises(lib.MoeError, match="UNSUPPORTED|unsupported"):
        lib.moe_permute_noalloc(x, ids, E, *outs)
