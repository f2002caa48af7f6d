"""The allocation-free permute (mc2_moe_permute_noalloc, for callers that
cannot allocate device memory) against mc2_moe_permute with a caller
workspace, through the C ABI: every output bit-exact, on two calls in a row
(the second smaller, so it runs over what the first left in the library's
scratch array)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import to_dev
from oracle import moe as om

pytestmark = pytest.mark.gpu


def _outputs(T, K, E, H, dtype):
    return dict(permuted=torch.full((T * K, H), -3, dtype=torch.int16, device="cuda").view(dtype),
                sorted_idx=torch.full((T * K,), -5, dtype=torch.int32, device="cuda"),
                unpermute_idx=torch.full((T * K,), -5, dtype=torch.int32, device="cuda"),
                expert_offsets=torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_permute_matches_workspace_permute(order):
    cases = [(32768, 8, 128, 256, 71), (700, 4, 32, 136, 72)]
    for T, K, E, H, seed in cases:
        d = wl.moe_inputs(seed=seed, tokens=T, hidden=H, num_experts=E, topk=K,
                          local_experts=min(E, 16), inter=64)
        sel = d["sel"].copy()
        if T < 1000:
            sel[5, 1] = E  # an invalid id: left out by both
        x, s = to_dev(d["x"], "bf16"), to_dev(sel)
        err_a = torch.zeros(1, dtype=torch.int32, device="cuda")
        err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
        a = _outputs(T, K, E, H, torch.bfloat16)
        b = _outputs(T, K, E, H, torch.bfloat16)
        ws = torch.empty(mc2.mc2_moe_permute_workspace_size(T, K, E), dtype=torch.uint8,
                         device="cuda")
        mc2.mc2_moe_permute(x, s, E, workspace=ws, dev_err=err_a, **a)
        mc2.mc2_moe_permute_noalloc(x, s, E, dev_err=err_b, **b)
        torch.cuda.synchronize()
        assert err_a.item() == err_b.item()
        for key in ("sorted_idx", "unpermute_idx", "expert_offsets"):
            assert torch.equal(a[key], b[key]), key
        assert torch.equal(a["permuted"].view(torch.int16), b["permuted"].view(torch.int16))
        ref = om.permute(np.zeros((T, 1), np.uint16), sel, E)
        np.testing.assert_array_equal(b["sorted_idx"].cpu().numpy(), ref["sorted_idx"])
        np.testing.assert_array_equal(b["unpermute_idx"].cpu().numpy(), ref["unpermute_idx"])
