"""The allocation-free format search (fp4_search_format_static, on the library's static
scratch) against the workspace entry point (fp4_search_format): records and packed codes
bit-exact, on two calls in a row on the same GPU, the second on a smaller input (the
scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

F = pytest.importorskip("bit_floating_point_amd")


def _tensors(T, numel, seed):
    """Seeded heavy-tailed weights: 0.02 N(0,1), with 5% of the entries from a Student-t(4)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    z = torch.randn((T, numel), generator=g, device="cuda")
    chi = sum(torch.randn((T, numel), generator=g, device="cuda") ** 2 for _ in range(4))
    t4 = torch.randn((T, numel), generator=g, device="cuda") / torch.sqrt(chi / 4)
    sel = torch.rand((T, numel), generator=g, device="cuda") < 0.05
    return (torch.where(sel, t4, z) * 0.02).contiguous()


def test_search_static_scratch_matches_workspace_entry_point():
    assert torch.cuda.is_available(), "needs a GPU"
    lib = F._lib.lib()
    # 32 tensors of 4M values need 9.8 MB of the 16 MiB scratch; then a smaller call
    for T, numel, seed in ((32, 4096 * 1024, 11), (5, 33280, 12)):
        print("static search", T, numel, "scratch bytes", lib.fp4_search_workspace_size(T, numel, 3, 100), flush=True)
        w = _tensors(T, numel, seed)
        ref_res, ref_packed = F.fp4_search_format(w)
        res = torch.full_like(ref_res, 0xAB)
        packed = torch.full_like(ref_packed, 0xAB)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        F.fp4_search_format_static(w, results=res, packed=packed)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(res, ref_res)
        assert torch.equal(packed, ref_packed)
        recs = F.search_results_host(res)
        assert all((r.e, r.m) in ((1, 2), (2, 1), (3, 0)) for r in recs)
    # a size past the scratch is refused on the host
    with pytest.raises(F.FP4Error) as ei:
        F.fp4_search_format_static(torch.empty((64, 1 << 24), dtype=torch.float32, device="cuda"))
    assert ei.value.status == F._lib.FP4_ERR_WORKSPACE
