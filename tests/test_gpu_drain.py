"""A ready flag releases its segment: a consumer that copies each segment out
as soon as its flag reads the call's epoch gets exactly the bytes the call
finally leaves in `out`.

The fused operators hand each finished chunk to the communication engine
while later chunks are still being computed (torch_npu.npu_mm_reduce_scatter_base
API doc, "功能说明"; "NPU Training Operators - MC2": the compute/communication
split and its pipeline inside the fused operator). On this GPU the hand-off
point is the per-segment ready flag, and the consumer stands in for that
engine: a second stream that waits on each flag in due order
(hipStreamWaitValue32, executed by the runtime, not by the producer kernel)
and then copies the segment's rows into a side buffer.

Before every call the output is filled with a sentinel that changes with the
epoch, and so is the side buffer: a copy taken before the segment's bytes had
landed, or released by a stale flag, shows the sentinel (or the previous
call's bytes) and fails the bitwise comparison. The flags live in host-pinned
memory so that the host can always release a waiting consumer: a flag that
never rises fails the test after a bounded wait instead of hanging it.
"""
import functools
import time

import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import to_dev
from oracle import gemm as og

pytestmark = pytest.mark.gpu

WAIT_EQ = 1  # hipStreamWaitValueEq
TIMEOUT_S = 10.0


@functools.lru_cache(maxsize=1)
def _hip():
    """The HIP runtime this process already uses (the one torch loaded)."""
    import ctypes as C
    path = next(line.split()[-1] for line in open("/proc/self/maps")
                if "libamdhip64.so" in line)
    lib = C.CDLL(path)
    lib.hipStreamWaitValue32.restype = C.c_int
    lib.hipStreamWaitValue32.argtypes = [C.c_void_p, C.c_void_p, C.c_uint32, C.c_uint,
                                         C.c_uint32]
    return lib


# Workloads in the launch configuration the benchmark times. Each entry gives
# (rows of out, world size, kind, ranks, producer(out, flags, counters,
# epoch, comm_turn)).
@functools.lru_cache(maxsize=1)
def _c1():
    d = wl.c1_inputs()
    x1, x2 = to_dev(d["x1"]), to_dev(d["x2"])

    def run(out, fl, cn, e, S, rank):
        mc2.mc2_mm_rs_local(x1, x2, 2, rank, out=out, ready_flags=fl, flag_counters=cn,
                            epoch=e, comm_turn=S)
    return (128, 64), torch.float16, 2, "rs", run


@functools.lru_cache(maxsize=1)
def _c2():
    d = wl.x2_as_nk(wl.c2_inputs())
    x, w = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")

    def run(out, fl, cn, e, S, rank):
        mc2.mc2_ag_mm_local(x, w, 8, rank, x2_trans=True, out=out, ready_flags=fl,
                            flag_counters=cn, epoch=e, comm_turn=S)
    return (8192, 3072), torch.bfloat16, 8, "ag", run


@functools.lru_cache(maxsize=1)
def _c3():
    d = wl.x2_as_nk(wl.c3_inputs())
    x1, x2 = to_dev(d["x1"]), to_dev(d["x2"])
    s1, s2 = to_dev(d["x1_scale"]), to_dev(d["x2_scale"])

    def run(out, fl, cn, e, S, rank):
        mc2.mc2_mm_rs_local(x1, x2, 4, rank, x2_trans=True, x1_scale=s1, x2_scale=s2, out=out,
                            ready_flags=fl, flag_counters=cn, epoch=e, comm_turn=S)
    return (4096, 2048), torch.bfloat16, 4, "rs", run


@functools.lru_cache(maxsize=1)
def _c5b():
    _, b = wl.c5_inputs()
    b = wl.x2_as_nk(b)
    x1, x2 = to_dev(b["x1"], "bf16"), to_dev(b["x2"], "bf16")

    def run(out, fl, cn, e, S, rank):
        mc2.mc2_mm_rs_local(x1, x2, 8, rank, x2_trans=True, out=out, ready_flags=fl,
                            flag_counters=cn, epoch=e, comm_turn=S)
    return (16384, 8192), torch.bfloat16, 8, "rs", run


WORKLOADS = {"c1": _c1, "c2": _c2, "c3": _c3, "c5b": _c5b}
# shares whose tiles take more than one dispatch round on 256 compute units
MULTI_ROUND = ("c2", "c5b")


def _sentinel(epoch, salt):
    """A 16-bit NaN pattern that differs between epochs and buffers."""
    return 0x7F81 + ((epoch * 7 + salt) % 0x70)


def _drained_call(name, rank, S, epoch, state):
    """One producer call with a concurrent drain. Returns (out, side, info)."""
    shape, dtype, W, kind, run = WORKLOADS[name]()
    m = shape[0]
    G = W * S
    hip = _hip()
    if "out" not in state:
        state["out"] = torch.empty(shape, dtype=dtype, device="cuda")
        state["side"] = torch.empty(shape, dtype=dtype, device="cuda")
        state["cnt"] = torch.zeros(64, dtype=torch.int32, device="cuda")
        state["prod"] = torch.cuda.Stream()
        state["drain"] = torch.cuda.Stream()
    out, side, cnt = state["out"], state["side"], state["cnt"]
    prod, drain = state["prod"], state["drain"]
    flags = torch.zeros(G, dtype=torch.int32, pin_memory=True)
    go = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    order = og.segment_order(W, rank, kind, S)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    p_start, p_end = ev(), ev()
    d_done = [ev() for _ in order]
    fv = flags.numpy()
    seen = np.full(G, np.nan)
    try:
        with torch.cuda.stream(prod):
            out.view(torch.int16).fill_(_sentinel(epoch, 1))
            # the producer starts only once the drain is fully enqueued behind it
            assert hip.hipStreamWaitValue32(prod.cuda_stream, go.data_ptr(), 1, WAIT_EQ,
                                            0xFFFFFFFF) == 0
            p_start.record()
            run(out, flags, cnt, epoch, S, rank)
            p_end.record()
        with torch.cuda.stream(drain):
            side.view(torch.int16).fill_(_sentinel(epoch, 2))
            for i, (c, j) in enumerate(order):
                g = c * S + j
                rows = og.sub_chunk_rows(m, W, c, S, j)
                assert hip.hipStreamWaitValue32(drain.cuda_stream, flags.data_ptr() + 4 * g,
                                                epoch, WAIT_EQ, 0xFFFFFFFF) == 0
                side[rows].copy_(out[rows])
                d_done[i].record()
        # host view of the flags: the time each segment's flag is first seen
        go[0] = 1
        t0 = time.perf_counter()
        while True:
            now = time.perf_counter() - t0
            seen[(fv == epoch) & np.isnan(seen)] = now
            if not np.isnan(seen).any() and d_done[-1].query() and p_end.query():
                break
            if now > TIMEOUT_S:
                raise AssertionError(
                    f"{name} rank {rank} comm_turn {S} epoch {epoch}: segments "
                    f"{np.flatnonzero(np.isnan(seen)).tolist()} did not raise their flag "
                    f"within {TIMEOUT_S} s")
        flags_seen = fv.copy()
    finally:
        # release every waiter (the producer's start gate and the drain's
        # flags) so that nothing stays blocked, whatever happened above
        go[0] = 1
        if np.isnan(seen).any():
            fv[:] = epoch
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    info = {
        "order": order,
        "seen": seen,
        "flags": flags_seen,
        "counters": cnt[:G].cpu().tolist(),
        "producer_ms": p_start.elapsed_time(p_end),
        "drain_ms": [p_start.elapsed_time(e) for e in d_done],
    }
    return out, side, info


CASES = [("c1", r, S) for r in (0, 1) for S in (1, 4)] + \
        [(n, r, S) for n in ("c2", "c3", "c5b") for r in (0, 3) for S in (1, 4)]


@pytest.fixture(scope="module")
def state():
    return {}


@pytest.mark.parametrize("name,rank,S", CASES)
def test_drained_segments_equal_final_output(name, rank, S, state):
    st = state.setdefault(name, {})
    for epoch in (3 + 2 * rank + S, 40 + 2 * rank + S):
        out, side, info = _drained_call(name, rank, S, epoch, st)
        G = len(info["order"])
        assert info["flags"].tolist() == [epoch] * G
        assert info["counters"] == [0] * G
        # every byte the drain copied equals what the call finally left in out
        a, b = side.view(torch.int16), out.view(torch.int16)
        if not torch.equal(a, b):
            bad = (a != b).any(dim=1).nonzero().flatten()
            raise AssertionError(f"{name} rank {rank} comm_turn {S} epoch {epoch}: drained "
                                 f"rows differ from the final output, first rows "
                                 f"{bad[:8].tolist()} of {bad.numel()}")
        # and no row of out still holds the sentinel
        assert not (b == _sentinel(epoch, 1)).all(dim=1).any()
        # the drain runs in due order, so its first copy is of the first
        # segment due. Where the segments span more than one dispatch round,
        # the host also sees the first segment due raised before the last one
        # (in one round all segments complete together, in any order).
        assert all(x <= y for x, y in zip(info["drain_ms"], info["drain_ms"][1:]))
        if name in MULTI_ROUND:
            (c0, j0), (c1, j1) = info["order"][0], info["order"][-1]
            assert info["seen"][c0 * S + j0] <= info["seen"][c1 * S + j1], info["seen"]


@pytest.mark.parametrize("rank", [0, 3])
def test_drain_overlaps_the_producer(rank, state):
    """On the largest share (eight dispatch rounds), the first segment due is
    copied out while the producer is still computing: the flag releases the
    segment mid-kernel, not at the kernel's end."""
    st = state.setdefault("c5b", {})
    _, _, info = _drained_call("c5b", rank, 1, 90 + rank, st)
    assert info["drain_ms"][0] < info["producer_ms"], (info["drain_ms"], info["producer_ms"])
