"""Parity of the rank-chunked GEMM (MatmulReduceScatter / AllGatherMatmul
compute share) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import DEQUANT_RTOL, assert_rel, assert_tol, to_dev, to_f64, torch_dtype
from oracle import gemm as og

pytestmark = pytest.mark.gpu


def _run_rs(d, W, rank, out_dtype=None, bias=None, flags=None, epoch=0):
    t = wl.BF16 if d["dtype"] == wl.BF16 else d["dtype"]
    x1 = to_dev(d["x1"], t)
    x2 = to_dev(d["x2"], t)
    kw = {}
    if "x1_scale" in d and out_dtype != "i32":
        kw = dict(x1_scale=to_dev(d["x1_scale"]), x2_scale=to_dev(d["x2_scale"]))
    if bias is not None:
        kw["bias"] = to_dev(bias, "bf16" if bias.dtype == np.uint16 else None)
    if flags is not None:
        kw.update(ready_flags=flags[0], flag_counters=flags[1], epoch=epoch)
    out = mc2.mc2_mm_rs_local(x1, x2, W, rank, x2_trans=d["x2_trans"],
                              out_dtype=torch_dtype(out_dtype) if out_dtype else None, **kw)
    torch.cuda.synchronize()
    return out


def _oracle_rs(d, W, out_dtype=None, bias=None, rows=None, cols=None):
    kw = {}
    if "x1_scale" in d and out_dtype != "i32":
        kw = dict(x1_scale=d["x1_scale"], x2_scale=d["x2_scale"])
    return og.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype=d["dtype"], nsim=d["nsim"],
                    x2_trans=d["x2_trans"], bias=bias, out_dtype=out_dtype, rows=rows,
                    cols=cols, **kw)


def test_c1_simulated_w2_reduce_scatter_fp16():
    """Config 1: two fp16 partials (128,512)x(512,64) summed into two 64-row chunks."""
    d = wl.c1_inputs()
    for rank in (0, 1):
        out = _run_rs(d, 2, rank)
        ref = _oracle_rs(d, 2)
        assert_tol(to_f64(out), ref, f"C1 rank {rank}")
        for c in range(2):
            rows = og.chunk_rows(128, 2, c)
            assert_tol(to_f64(out)[rows], ref[rows], f"C1 chunk {c}")


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("x2_trans", [False, True])
@pytest.mark.parametrize("nsim", [1, 4])
def test_rs_ragged_tiles(dtype, x2_trans, nsim):
    """Chunks of 200 rows (a ragged 128-row tile), k = 776 (a K tail inside each
    shard), n = 392 (a ragged column tile); N(0,1) values so the relative term
    of the gate bites."""
    W = 4
    d = wl.gemm_inputs(21, W * 200, 776, 392, dtype, std=1.0, nsim=nsim, x2_trans=x2_trans)
    out = _run_rs(d, W, 3)
    assert_tol(to_f64(out), _oracle_rs(d, W), f"rs {dtype} trans={x2_trans} nsim={nsim}")
    out32 = _run_rs(d, W, 1, out_dtype="f32")
    ref32 = _oracle_rs(d, W, out_dtype="f32")
    assert_tol(to_f64(out32), ref32, "fp32 out", rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("nsim", [1, 2])
def test_rs_bias_added_per_partial(nsim):
    W = 2
    d = wl.gemm_inputs(22, 256, 512, 136, wl.BF16, std=1.0, nsim=nsim, bias=True)
    out = _run_rs(d, W, 0, bias=d["bias"])
    assert_tol(to_f64(out), _oracle_rs(d, W, bias=d["bias"]), "bias")


@pytest.mark.parametrize("x2_trans", [False, True])
def test_int8_raw_accumulator_bit_exact(x2_trans):
    d = wl.gemm_inputs(23, 4 * 130, 1040, 272, wl.I8, x2_trans=x2_trans)
    out = _run_rs(d, 4, 0, out_dtype="i32")
    np.testing.assert_array_equal(to_f64(out), _oracle_rs(d, 4, out_dtype="i32"))


def test_int8_extreme_values_bit_exact():
    """All entries +-127 with k = 65520: |acc| ~ 1.06e9 stays exact in int32."""
    k, m, n = 65520, 128, 256
    x1 = np.full((m, k), 127, np.int8)
    x2 = np.full((k, n), -127, np.int8)
    x2[:, 1::2] = 127
    d = {"x1": x1, "x2": x2, "dtype": wl.I8, "nsim": 1, "x2_trans": False}
    out = _run_rs(d, 1, 0, out_dtype="i32")
    np.testing.assert_array_equal(to_f64(out), _oracle_rs(d, 1, out_dtype="i32"))


@pytest.mark.parametrize("x2_trans", [False, True])
def test_int8_dequant_fp32_and_bf16(x2_trans):
    d = wl.gemm_inputs(24, 4 * 130, 1040, 272, wl.I8, x2_trans=x2_trans, quant=True)
    out32 = _run_rs(d, 4, 2, out_dtype="f32")
    assert_rel(to_f64(out32), _oracle_rs(d, 4, out_dtype="f32"), DEQUANT_RTOL, "dequant fp32")
    for od in ("bf16", "f16"):
        out = _run_rs(d, 4, 2, out_dtype=od)
        assert_tol(to_f64(out), _oracle_rs(d, 4, out_dtype=od), f"dequant {od}")


def test_int8_bias_extension():
    d = wl.gemm_inputs(25, 256, 512, 64, wl.I8, quant=True, bias=True)
    out = _run_rs(d, 2, 0, out_dtype="f32", bias=d["bias"])
    ref = og.mm_rs(d["x1"], d["x2"], world_size=2, in_dtype="i8", bias=d["bias"],
                   bias_dtype="bf16", x1_scale=d["x1_scale"], x2_scale=d["x2_scale"],
                   out_dtype="f32")
    assert_rel(to_f64(out), ref, DEQUANT_RTOL, "int8 bias")


@pytest.mark.parametrize("rank", [0, 3])
@pytest.mark.parametrize("x2_trans", [False, True])
def test_ag_mm_with_flags(rank, x2_trans):
    W = 8
    d = wl.gemm_inputs(26, W * 100, 512, 264, wl.BF16, std=1.0, x2_trans=x2_trans)
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    counters = torch.zeros(W, dtype=torch.int32, device="cuda")
    x = to_dev(d["x1"], "bf16")
    w = to_dev(d["x2"], "bf16")
    for epoch in (7, 8):
        out = mc2.mc2_ag_mm_local(x, w, W, rank, x2_trans=x2_trans, ready_flags=flags,
                                  flag_counters=counters, epoch=epoch)
        torch.cuda.synchronize()
        assert flags.cpu().tolist() == [epoch] * W
        assert counters.cpu().tolist() == [0] * W
    ref = og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16", x2_trans=x2_trans)
    assert_tol(to_f64(out), ref, "ag_mm")


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F16])
def test_rs_longest_k_and_most_chunks(dtype):
    """K = 65528 (the largest multiple of 8 below 65535) over W = 32 chunks of 8
    rows each, n = 8: one tile per chunk, 1024 K stages, with flags."""
    W = 32
    d = wl.gemm_inputs(92, W * 8, 65528, 8, dtype, std=1.0)
    t = "bf16" if dtype == wl.BF16 else None
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, dtype=torch.int32, device="cuda")
    out = mc2.mc2_mm_rs_local(to_dev(d["x1"], t), to_dev(d["x2"], t), W, 31, ready_flags=flags,
                              flag_counters=cnt, epoch=6)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [6] * W and cnt.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), _oracle_rs(d, W), f"k=65528 {dtype}")


def test_ag_mm_smallest_shapes():
    """k = 8 and n = 8 (one 16-byte piece each), one row per chunk."""
    W = 8
    d = wl.gemm_inputs(93, W, 8, 8, wl.BF16, std=1.0)
    out = mc2.mc2_ag_mm_local(to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16"), W, 3)
    torch.cuda.synchronize()
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "k=n=8")


def test_rs_flags_reset_between_calls():
    W = 4
    d = wl.gemm_inputs(27, W * 256, 512, 512, wl.BF16, std=1.0)
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    counters = torch.zeros(W, dtype=torch.int32, device="cuda")
    for epoch in (1, 2, 3):
        _run_rs(d, W, 1, flags=(flags, counters), epoch=epoch)
        assert flags.cpu().tolist() == [epoch] * W
        assert counters.cpu().tolist() == [0] * W


def test_last_round_as_half_tiles():
    """More 256-row tiles than CUs, with a last round under half full: those
    tiles run as two 128-row halves. Chunks of 1000 rows (the last 256-row tile
    is ragged and its second half partial) and n = 8696 (a ragged column
    tile); ready flags on, both chunk orders."""
    W = 2
    d = wl.gemm_inputs(28, W * 1000, 256, 8696, wl.BF16, std=1.0)
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    counters = torch.zeros(W, dtype=torch.int32, device="cuda")
    ref = _oracle_rs(d, W)
    for rank in (0, 1):
        out = _run_rs(d, W, rank, flags=(flags, counters), epoch=rank + 5)
        assert flags.cpu().tolist() == [rank + 5] * W
        assert counters.cpu().tolist() == [0] * W
        assert_tol(to_f64(out), ref, f"rs rank {rank}")
    out = mc2.mc2_ag_mm_local(to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16"), W, 1,
                              ready_flags=flags, flag_counters=counters, epoch=9)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [9] * W
    assert counters.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "ag_mm")


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_ragged_chunks_columns_and_k(dtype):
    """W = 8 chunks of 1000 rows (ragged 256-row tiles), n = 1400 (a last
    column tile of 120 columns), k = 776 (a K tail): every element against the
    oracle, with ready flags, in reduce-scatter and AllGatherMatmul order and
    in both x2 layouts; then the simulated W = 2 reduce-scatter of two shards
    of k = 392."""
    W = 8
    t = "bf16" if dtype == wl.BF16 else None
    d = wl.gemm_inputs(29, W * 1000, 776, 1400, dtype, std=1.0)
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    counters = torch.zeros(W, dtype=torch.int32, device="cuda")
    ref = _oracle_rs(d, W)
    out = _run_rs(d, W, 3, flags=(flags, counters), epoch=4)
    assert flags.cpu().tolist() == [4] * W
    assert counters.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), ref, f"rs {dtype}")
    dn = wl.x2_as_nk(d)
    out = _run_rs(dn, W, 3, flags=(flags, counters), epoch=5)
    assert flags.cpu().tolist() == [5] * W
    assert_tol(to_f64(out), ref, f"rs {dtype} x2 (n, k)")
    out = mc2.mc2_ag_mm_local(to_dev(d["x1"], t), to_dev(d["x2"], t), W, 5,
                              ready_flags=flags, flag_counters=counters, epoch=6)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [6] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype=dtype), "ag_mm")
    d2 = wl.gemm_inputs(30, 8000, 392, 1400, dtype, std=1.0, nsim=2)
    assert_tol(to_f64(_run_rs(d2, 2, 0)), _oracle_rs(d2, 2), f"sim rs {dtype}")


def test_bias_pieces_and_inflags_on_ragged_chunks():
    """Other paths on the same ragged launch shapes: bias with the test-only
    fp32 output; comm_turn 3 pieces with their own flags, bit-identical to the
    unsplit call (W = 2 chunks of 3000 rows, pieces of 1000); input flags,
    all present."""
    W = 8
    d = wl.gemm_inputs(31, W * 1000, 392, 1400, wl.BF16, std=1.0, bias=True)
    out = _run_rs(d, W, 2, out_dtype="f32", bias=d["bias"])
    assert_tol(to_f64(out), _oracle_rs(d, W, out_dtype="f32", bias=d["bias"]), "bias f32",
               rtol=1e-4, atol=1e-3)
    d2 = wl.gemm_inputs(32, 6000, 392, 1400, wl.BF16, std=1.0)
    x1, x2 = to_dev(d2["x1"], "bf16"), to_dev(d2["x2"], "bf16")
    base = mc2.mc2_mm_rs_local(x1, x2, 2, 1)
    flags = torch.zeros(6, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(6, dtype=torch.int32, device="cuda")
    out = mc2.mc2_mm_rs_local(x1, x2, 2, 1, ready_flags=flags, flag_counters=cnt, epoch=7,
                              comm_turn=3)
    torch.cuda.synchronize()
    assert torch.equal(out, base)
    assert flags.cpu().tolist() == [7] * 6 and cnt.cpu().tolist() == [0] * 6
    assert_tol(to_f64(base), _oracle_rs(d2, 2), "unsplit")
    inf = torch.full((W,), 5, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, dtype=torch.int32, device="cuda")
    out = mc2.mc2_ag_mm_local_inflags(to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16"), W, 6,
                                      inf, 5, ready_flags=flags, flag_counters=cnt, epoch=9,
                                      dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert flags.cpu().tolist() == [9] * W and cnt.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "inflags")


# ------------------------------------------------- AllGatherMatmul input flags

def _hip():
    """The HIP runtime this process already uses (the one torch loaded)."""
    import ctypes as C
    path = next(line.split()[-1] for line in open("/proc/self/maps")
                if "libamdhip64.so" in line)
    lib = C.CDLL(path)
    lib.hipStreamWriteValue32.restype = C.c_int
    lib.hipStreamWriteValue32.argtypes = [C.c_void_p, C.c_void_p, C.c_uint32, C.c_uint]
    return lib


def test_ag_mm_inflags_all_present():
    W = 4
    d = wl.gemm_inputs(41, W * 130, 512, 264, wl.BF16, std=1.0)
    inf = torch.full((W,), 77, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, dtype=torch.int32, device="cuda")
    out = mc2.mc2_ag_mm_local_inflags(to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16"), W, 2,
                                      inf, 77, ready_flags=flags, flag_counters=cnt, epoch=3,
                                      dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert flags.cpu().tolist() == [3] * W and cnt.cpu().tolist() == [0] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "inflags")


def test_ag_mm_inflags_raised_later_by_another_agent():
    """The input flags of the three remote chunks are raised one by one, 3 ms
    apart and in reverse order, by stream writes (executed by the command
    processor, not by this kernel) while the kernel runs: the kernel's tiles
    wait for them, and the result is exact."""
    import time
    W, rank = 4, 1
    d = wl.gemm_inputs(42, W * 130, 512, 264, wl.BF16, std=1.0)
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    inf = torch.zeros(W, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hip = _hip()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    out = mc2.mc2_ag_mm_local_inflags(x, w, W, rank, inf, 5, spin_limit=200000, dev_err=err)
    t1.record()
    for c in (0, 3, 2):  # remote chunks, reverse of the compute order 2, 3, 0
        time.sleep(0.003)
        assert hip.hipStreamWriteValue32(side.cuda_stream, inf.data_ptr() + 4 * c, 5, 0) == 0
    torch.cuda.synchronize()
    assert err.item() == 0
    assert t0.elapsed_time(t1) > 6.0, "the kernel did not wait for the flags"
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "late flags")


def test_ag_mm_inflags_timeout_reported_and_state_kept():
    """A flag that never arrives: with a small spin limit every tile of that
    chunk gives up, MC2_DEVERR_TIMEOUT is set, the kernel ends normally, and
    the ready-flag counters are left consistent for the next call."""
    W = 4
    d = wl.gemm_inputs(43, W * 130, 512, 264, wl.BF16, std=1.0)
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    inf = torch.tensor([9, 9, 0, 9], dtype=torch.int32, device="cuda")  # chunk 2 never ready
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, dtype=torch.int32, device="cuda")
    mc2.mc2_ag_mm_local_inflags(x, w, W, 0, inf, 9, spin_limit=64, ready_flags=flags,
                                flag_counters=cnt, epoch=1, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == mc2.MC2_DEVERR_TIMEOUT
    assert cnt.cpu().tolist() == [0] * W and flags.cpu().tolist() == [1] * W
    inf[2] = 9
    err.zero_()
    out = mc2.mc2_ag_mm_local_inflags(x, w, W, 0, inf, 9, spin_limit=64, ready_flags=flags,
                                      flag_counters=cnt, epoch=2, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0 and flags.cpu().tolist() == [2] * W
    assert_tol(to_f64(out), og.ag_mm(d["x1"], d["x2"], world_size=W, in_dtype="bf16"), "after")
