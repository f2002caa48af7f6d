"""K split of a thin last round (stream-K for the tail): with a workspace, the
tiles of a last dispatch round that is at most half full run as two K halves
on two workgroups, which exchange fp32 / int32 partials.

What the tests pin:
  - int8: the raw int32 accumulator is bit-exact against the oracle and equal
    to the unsplit schedule (integer sums do not depend on the split);
  - 16-bit: every element against the oracle, on ragged rows, a ragged last
    column tile, K tails, both x2 layouts and a K loop over two shards;
  - both exchange policies (the first half waits for a running partner, or
    never waits and hands the whole tile over) give the same bits: each
    element is the same two fp32 halves added once;
  - ready flags still rise once per segment, counters and the workspace's
    control words are zero after every call, and a second call in a row
    (control words reused) gives the same bits.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import assert_tol, to_dev, to_f64
from oracle import gemm as og

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="the K split is switched off in the library: its first device runs "
                            "faulted on the partial stores (a scalar base address read too soon "
                            "after v_readfirstlane wrote it); the fix has not run on the device"),
]

POLICIES = (mc2.MC2_SPLIT_PAIR, mc2.MC2_SPLIT_ALONE)


@pytest.fixture
def ws():
    w = torch.zeros(mc2.mc2_split_workspace_size(), dtype=torch.uint8, device="cuda")
    yield w
    mc2.mc2_set_split_policy(mc2.MC2_SPLIT_PAIR)


def _ctl_zero(w):
    torch.cuda.synchronize()
    return int(w[:4096].count_nonzero().item()) == 0


def _flags(G):
    return (torch.zeros(G, dtype=torch.int32, device="cuda"),
            torch.zeros(G, dtype=torch.int32, device="cuda"))


def _t(dtype):
    return "bf16" if dtype == wl.BF16 else None


@pytest.mark.parametrize("x2_trans", [True, False])
def test_int8_split_accumulator_bit_exact(ws, x2_trans):
    """W = 4 chunks of 256 rows, k = 2048 (16 stages of 128), n = 1024: the 16
    tiles fill a sixteenth of the CUs, so every tile is split. The int32
    accumulator equals the oracle and the unsplit schedule under both
    policies, twice in a row; the bf16 dequantised output equals the unsplit
    one bit for bit."""
    W = 4
    d = wl.gemm_inputs(71, W * 256, 2048, 1024, wl.I8, x2_trans=x2_trans, quant=True)
    x1, x2 = to_dev(d["x1"]), to_dev(d["x2"])
    ref = og.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype="i8", out_dtype="i32",
                   x2_trans=x2_trans)
    base = mc2.mc2_mm_rs_local(x1, x2, W, 1, x2_trans=x2_trans, out_dtype=torch.int32,
                               split=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_f64(base), ref)
    for pol in POLICIES:
        mc2.mc2_set_split_policy(pol)
        for _ in range(2):
            out = mc2.mc2_mm_rs_local(x1, x2, W, 1, x2_trans=x2_trans, out_dtype=torch.int32,
                                      workspace=ws)
            assert _ctl_zero(ws), f"control words left set (policy {pol})"
            assert torch.equal(out, base), f"policy {pol}"
    s1, s2 = to_dev(d["x1_scale"]), to_dev(d["x2_scale"])
    q0 = mc2.mc2_mm_rs_local(x1, x2, W, 1, x2_trans=x2_trans, x1_scale=s1, x2_scale=s2,
                             split=False)
    q1 = mc2.mc2_mm_rs_local(x1, x2, W, 1, x2_trans=x2_trans, x1_scale=s1, x2_scale=s2,
                             workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F16])
@pytest.mark.parametrize("x2_trans", [True, False])
@pytest.mark.parametrize("k", [1088, 1096])
def test_float_split_ragged_every_element(ws, dtype, x2_trans, k):
    """W = 4 chunks of 500 rows (each chunk's second tile row holds 244 rows:
    its lower row half is ragged), n = 1400 (a last column tile of 120), k =
    1088 (17 stages: halves of 8 and 9) or 1096 (a K tail in the last stage).
    48 tiles, all split. Every element against the oracle; both policies give
    the same bits; flags raised, counters and control words zero."""
    W = 4
    d = wl.gemm_inputs(72, W * 500, k, 1400, dtype, std=1.0, x2_trans=x2_trans)
    x1, x2 = to_dev(d["x1"], _t(dtype)), to_dev(d["x2"], _t(dtype))
    ref = og.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype=dtype, x2_trans=x2_trans)
    flags, cnt = _flags(W)
    outs = []
    for epoch, pol in enumerate(POLICIES, start=1):
        mc2.mc2_set_split_policy(pol)
        out = mc2.mc2_mm_rs_local(x1, x2, W, 2, x2_trans=x2_trans, ready_flags=flags,
                                  flag_counters=cnt, epoch=epoch, workspace=ws)
        assert _ctl_zero(ws)
        assert flags.cpu().tolist() == [epoch] * W and cnt.cpu().tolist() == [0] * W
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    assert_tol(to_f64(outs[0]), ref, f"split {dtype} k={k}")
    ag = mc2.mc2_ag_mm_local(x1, x2, W, 3, x2_trans=x2_trans, workspace=ws)
    assert _ctl_zero(ws)
    assert_tol(to_f64(ag), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype=dtype,
                                    x2_trans=x2_trans), "ag_mm split")


def test_split_tail_after_full_rounds(ws):
    """The C2 chunk shape at k = 1024 (16 stages): 384 tiles, one full round
    of 256 and a last round of 128 split tiles (the last chunks in due order).
    Sampled rows of every chunk (the first and last, and random ones) on 96
    columns against the oracle; both policies give the same bits; flags."""
    W, mc, k, n = 8, 1024, 1024, 3072
    d = wl.gemm_inputs(73, W * mc, k, n, wl.BF16, std=1.0, x2_trans=True)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    flags, cnt = _flags(W)
    outs = []
    for epoch, pol in enumerate(POLICIES, start=3):
        mc2.mc2_set_split_policy(pol)
        out = mc2.mc2_ag_mm_local(x1, x2, W, 5, x2_trans=True, ready_flags=flags,
                                  flag_counters=cnt, epoch=epoch, workspace=ws)
        assert _ctl_zero(ws)
        assert flags.cpu().tolist() == [epoch] * W and cnt.cpu().tolist() == [0] * W
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([
        np.arange(W) * mc, np.arange(W) * mc + mc - 1, rng.choice(W * mc, 96, replace=False)]))
    cols = np.sort(rng.choice(n, 96, replace=False))
    ref = og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16", x2_trans=True, rows=rows,
                   cols=cols)
    assert_tol(to_f64(outs[0])[np.ix_(rows, cols)], ref, "C2 shape, split tail")


def test_simulated_reduce_scatter_split_at_the_shard_boundary(ws):
    """nsim = W = 2 partials of k = 512 (8 stages each): the K loop of 16
    stages splits where the second shard begins, so each half sums one
    partial. With a bias (added once per partial)."""
    W = 2
    d = wl.gemm_inputs(74, W * 512, 512, 1024, wl.BF16, std=1.0, nsim=W, bias=True)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    bias = to_dev(d["bias"], "bf16")
    out = mc2.mc2_mm_rs_local(x1, x2, W, 0, bias=bias, workspace=ws)
    assert _ctl_zero(ws)
    ref = og.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype="bf16", nsim=W, bias=d["bias"])
    assert_tol(to_f64(out), ref, "simulated RS, split")


def test_inflags_consumer_with_split_tail(ws):
    """AllGatherMatmul consumer side with every input flag raised, on a shape
    whose tiles are all split: no timeout reported, flags, parity."""
    W = 4
    d = wl.gemm_inputs(75, W * 500, 1088, 1400, wl.BF16, std=1.0)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    inf = torch.full((W,), 3, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags, cnt = _flags(W)
    out = mc2.mc2_ag_mm_local_inflags(x1, x2, W, 1, inf, 3, ready_flags=flags,
                                      flag_counters=cnt, epoch=8, dev_err=err, workspace=ws)
    assert _ctl_zero(ws)
    assert err.item() == 0
    assert flags.cpu().tolist() == [8] * W and cnt.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"),
               "inflags, split")
