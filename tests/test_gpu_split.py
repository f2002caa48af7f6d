"""Finer split granularity: every chunk cut into comm_turn pieces, each with
its own ready flag (and input flag on the AllGatherMatmul consumer side),
through the C ABI. Values never depend on the split."""
import time

import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import assert_tol, to_dev, to_f64
from oracle import gemm as og
from test_gpu_gemm import _hip

pytestmark = pytest.mark.gpu


def _piece_edges(m, W, turn):
    """First and last row of every piece, in the oracle's split."""
    rows = []
    for c in range(W):
        for j in range(max(turn, 1)):
            p = og.sub_chunk_rows(m, W, c, turn, j)
            rows += [p.start, p.stop - 1]
    return np.unique(np.array(rows))


def _flags(G):
    return (torch.zeros(G, dtype=torch.int32, device="cuda"),
            torch.zeros(G, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("turn", [1, 2, 3, 7])
def test_rs_pieces_same_values_and_flags(turn):
    """W=4 chunks of 600 rows (pieces of unequal size for 7), ragged n: the
    result is bit-identical to the unsplit call, every segment's flag is
    raised, the counters return to zero, twice in a row."""
    W, mc = 4, 600
    d = wl.gemm_inputs(61, W * mc, 512, 392, wl.BF16, std=1.0)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    base = mc2.mc2_mm_rs_local(x1, x2, W, 1)
    G = W * max(turn, 1)
    flags, cnt = _flags(G)
    for epoch in (1, 2):
        out = mc2.mc2_mm_rs_local(x1, x2, W, 1, ready_flags=flags, flag_counters=cnt,
                                  epoch=epoch, comm_turn=turn)
        torch.cuda.synchronize()
        assert torch.equal(out, base)
        assert flags.cpu().tolist() == [epoch] * G and cnt.cpu().tolist() == [0] * G
    rows = _piece_edges(W * mc, W, turn)
    ref = og.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype="bf16", rows=rows)
    assert_tol(to_f64(out)[rows], ref, f"comm_turn {turn}")


@pytest.mark.parametrize("turn", [3, 4])
def test_ag_pieces_with_half_tile_tail(turn):
    """The C2 chunk shape (8 x 1024 rows, n = 3072) at k = 256, cut into 3
    pieces (342/341/341 rows: the lower half of every second tile row holds no
    rows) or 4 (256 rows each). The last dispatch round runs as half tiles in
    both cases."""
    W, mc, k, n = 8, 1024, 256, 3072
    d = wl.gemm_inputs(62, W * mc, k, n, wl.BF16, std=1.0)
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    base = mc2.mc2_ag_mm_local(x, w, W, 5)
    G = W * turn
    flags, cnt = _flags(G)
    out = mc2.mc2_ag_mm_local(x, w, W, 5, ready_flags=flags, flag_counters=cnt, epoch=7,
                              comm_turn=turn)
    torch.cuda.synchronize()
    assert torch.equal(out, base)
    assert flags.cpu().tolist() == [7] * G and cnt.cpu().tolist() == [0] * G
    rows = _piece_edges(W * mc, W, turn)
    cols = np.sort(np.random.default_rng(3).choice(n, 64, replace=False))
    ref = og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16", rows=rows, cols=cols)
    assert_tol(to_f64(out)[np.ix_(rows, cols)], ref, f"comm_turn {turn}")


def test_ag_inflags_per_piece_raised_later():
    """Input flags per piece: the six remote segments (3 chunks x 2 pieces) are
    raised 3 ms apart in reverse order by stream writes while the kernel runs;
    the kernel waits for each and the result is exact."""
    W, rank, S = 4, 1, 2
    d = wl.gemm_inputs(63, W * 130, 512, 264, wl.BF16, std=1.0)
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    inf = torch.zeros(W * S, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags, cnt = _flags(W * S)
    hip = _hip()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    out = mc2.mc2_ag_mm_local_inflags(x, w, W, rank, inf, 5, spin_limit=400000, dev_err=err,
                                      ready_flags=flags, flag_counters=cnt, epoch=2, comm_turn=S)
    t1.record()
    # compute order of the remote segments: (2,0) (2,1) (3,0) (3,1) (0,0) (0,1); raise reversed
    for c, j in reversed([(2, 0), (2, 1), (3, 0), (3, 1), (0, 0), (0, 1)]):
        time.sleep(0.003)
        assert hip.hipStreamWriteValue32(side.cuda_stream, inf.data_ptr() + 4 * (c * S + j), 5, 0) == 0
    torch.cuda.synchronize()
    assert err.item() == 0
    assert t0.elapsed_time(t1) > 12.0, "the kernel did not wait for the flags"
    assert flags.cpu().tolist() == [2] * (W * S) and cnt.cpu().tolist() == [0] * (W * S)
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "pieces")


def test_ag_inflags_one_piece_missing_times_out():
    """One remote piece never arrives: with a small spin limit its tiles give
    up, MC2_DEVERR_TIMEOUT is set, the call ends, every counter is back to
    zero, and the next call with all flags present is exact."""
    W, S = 4, 3
    d = wl.gemm_inputs(64, W * 130, 512, 264, wl.BF16, std=1.0)
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    inf = torch.full((W * S,), 9, dtype=torch.int32, device="cuda")
    inf[2 * S + 1] = 0  # piece 1 of chunk 2
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags, cnt = _flags(W * S)
    mc2.mc2_ag_mm_local_inflags(x, w, W, 0, inf, 9, spin_limit=64, ready_flags=flags,
                                flag_counters=cnt, epoch=1, dev_err=err, comm_turn=S)
    torch.cuda.synchronize()
    assert err.item() == mc2.MC2_DEVERR_TIMEOUT
    assert cnt.cpu().tolist() == [0] * (W * S) and flags.cpu().tolist() == [1] * (W * S)
    inf[2 * S + 1] = 9
    err.zero_()
    out = mc2.mc2_ag_mm_local_inflags(x, w, W, 0, inf, 9, spin_limit=64, ready_flags=flags,
                                      flag_counters=cnt, epoch=2, dev_err=err, comm_turn=S)
    torch.cuda.synchronize()
    assert err.item() == 0 and flags.cpu().tolist() == [2] * (W * S)
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "after")


def test_c5b_pieces_full_size_sampled():
    """The simulated W=8 reduce-scatter at full size with 4 pieces per chunk,
    in the launch configuration the benchmark times."""
    _, b = wl.c5_inputs()
    W, S = 8, 4
    x1, x2 = to_dev(b["x1"], "bf16"), to_dev(b["x2"], "bf16")
    flags, cnt = _flags(W * S)
    out = mc2.mc2_mm_rs_local(x1, x2, W, 0, ready_flags=flags, flag_counters=cnt, epoch=1,
                              comm_turn=S)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [1] * (W * S) and cnt.cpu().tolist() == [0] * (W * S)
    rows = _piece_edges(16384, W, S)
    cols = np.sort(np.random.default_rng(4).choice(8192, 32, replace=False))
    ref = og.mm_rs(b["x1"], b["x2"], world_size=W, in_dtype="bf16", nsim=W, rows=rows, cols=cols)
    assert_tol(to_f64(out)[np.ix_(rows, cols)], ref, "C5b pieces")


def test_ready_flags_in_host_pinned_memory():
    """Ready flags for a host-side consumer: the segment flags land in
    host-pinned memory, where the host reads them without a device copy."""
    W, S = 4, 2
    d = wl.gemm_inputs(65, W * 256, 512, 264, wl.BF16, std=1.0)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    hf = torch.zeros(W * S, dtype=torch.int32, pin_memory=True)
    cnt = torch.zeros(W * S, dtype=torch.int32, device="cuda")
    out = mc2.mc2_mm_rs_local(x1, x2, W, 3, ready_flags=hf, flag_counters=cnt, epoch=11,
                              comm_turn=S)
    torch.cuda.synchronize()
    assert hf.tolist() == [11] * (W * S) and cnt.cpu().tolist() == [0] * (W * S)
    assert torch.equal(out, mc2.mc2_mm_rs_local(x1, x2, W, 3))
