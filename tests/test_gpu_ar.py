"""Parity of the MatmulAllReduce local share and of its combining step
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import ATOL, RTOL, assert_tol, to_dev, to_f64, torch_dtype
from oracle import gemm as og
from oracle import numerics

pytestmark = pytest.mark.gpu

MODES = (mc2.MC2_AR_ONE_ROUNDING, mc2.MC2_AR_RANK_ROUNDED, mc2.MC2_AR_HOP_ROUNDED)


def _assert_combined(gpu, ref, parts, rounding, what):
    """Partials rounded before the combine: a partial whose exact value lies
    near a rounding boundary may round to the neighbouring value on one side
    and not the other (fp32 versus exact accumulation), and the sum carries
    that difference in full even where the partials cancel. So the bound
    scales with the magnitudes the roundings act on: the single-rounding
    tolerance of every partial, plus (hop rounding) one of every running
    sum, plus that of the result."""
    P = np.asarray(parts, np.float64)
    scale = np.abs(P).sum(axis=0)
    if rounding == mc2.MC2_AR_HOP_ROUNDED:
        scale = scale + np.abs(np.cumsum(P, axis=0)[1:]).sum(axis=0)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bound = RTOL * (np.abs(ref) + scale) + (2 * P.shape[0] + 1) * ATOL
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside the combined bound; "
                           f"worst gpu={gpu[bad][0]!r} ref={ref[bad][0]!r}")
    # the bound is wide only where partials cancel; elsewhere the results agree
    assert np.mean(err <= RTOL * np.abs(ref) + ATOL) >= 0.999, what
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    assert float(np.sqrt(np.mean(err ** 2))) <= 0.02 * rms_ref + 1e-6, what


def _partials(d, W, dtype, rows=None, cols=None):
    """The oracle's per-rank partials, each one product rounded to dtype."""
    return np.stack([og.mm_rs(np.asarray(d["x1"])[w], np.asarray(d["x2"])[w], world_size=1,
                              in_dtype=dtype, x2_trans=d["x2_trans"], bias=d.get("bias"),
                              rows=rows, cols=cols) for w in range(W)])


def _stored_partials(rng, W, elems, dtype):
    """Finite partials spread over many binades (wide enough for bf16 that an
    fp32 sum of two is often inexact; into the subnormals for fp16), with some
    signed zeros, in storage format."""
    lo, hi = (-60, 60) if dtype == wl.BF16 else (-16, 10)
    v = rng.standard_normal((W, elems)) * np.exp2(rng.integers(lo, hi, (W, elems)))
    z = rng.random((W, elems))
    v[z < 0.03] = 0.0
    v[z < 0.01] = -0.0
    if dtype == wl.BF16:
        return wl.encode_bf16(v.astype(np.float32))
    return v.astype(np.float16)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F16])
@pytest.mark.parametrize("W", [1, 2, 3, 8, 32])
def test_ar_sum_bit_exact(dtype, W):
    """The combining step sums in fp64 in rank order and rounds once per
    rounding point, as the oracle does: identical bits."""
    rng = np.random.default_rng(100 + W)
    parts = _stored_partials(rng, W, 8 * 1000, dtype)
    dev = to_dev(parts, "bf16" if dtype == wl.BF16 else None)
    for mode in (mc2.MC2_AR_RANK_ROUNDED, mc2.MC2_AR_HOP_ROUNDED):
        out = mc2.mc2_ar_sum_local(dev, mode)
        torch.cuda.synchronize()
        ref = og.ar_sum(parts, dtype=dtype, rounding=mode)
        got = to_f64(out)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("x2_trans", [False, True])
def test_mm_ar_modes_ragged(dtype, x2_trans):
    """W = 4 partials of a (333, 776) @ (776, 392) product (ragged tiles, a K
    tail, rows not divisible by W), with bias, in every rounding mode."""
    W = 4
    d = wl.gemm_inputs(51, 333, 776, 392, dtype, std=1.0, nsim=W, x2_trans=x2_trans, bias=True)
    t = "bf16" if dtype == wl.BF16 else None
    x1, x2, b = to_dev(d["x1"], t), to_dev(d["x2"], t), to_dev(d["bias"], t)
    parts = _partials(d, W, dtype)
    ws = torch.empty(mc2.mc2_mm_ar_workspace_size(333, 392, W, torch_dtype(dtype),
                                                  mc2.MC2_AR_HOP_ROUNDED),
                     dtype=torch.uint8, device="cuda")
    for mode in MODES:
        out = mc2.mc2_mm_ar_local(x1, x2, W, rounding=mode, x2_trans=x2_trans, bias=b,
                                  workspace=ws)
        torch.cuda.synchronize()
        ref = og.mm_ar(d["x1"], d["x2"], world_size=W, in_dtype=dtype, x2_trans=x2_trans,
                       bias=d["bias"], rounding=mode)
        if mode == mc2.MC2_AR_ONE_ROUNDING:
            assert_tol(to_f64(out), ref, f"mode {mode}")
            continue
        # each rank's rounded partial, as left in the workspace: one rounding each
        got = to_f64(ws[: W * 333 * 392 * 2].view(torch_dtype(dtype)).view(W, 333, 392))
        for w in range(W):
            assert_tol(got[w], parts[w], f"mode {mode} partial {w}")
        _assert_combined(to_f64(out), ref, parts, mode, f"mode {mode}")


def test_mm_ar_one_rounding_is_the_simulated_sum():
    """With one rounding, every rank's result is the simulated reduce-scatter's
    full matrix: the same kernel arithmetic, so identical bits."""
    W = 4
    d = wl.gemm_inputs(52, 4 * 96, 512, 136, wl.BF16, std=1.0, nsim=W)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    ar = mc2.mc2_mm_ar_local(x1, x2, W, rounding=mc2.MC2_AR_ONE_ROUNDING)
    rs = mc2.mc2_mm_rs_local(x1, x2, W, 0)
    torch.cuda.synchronize()
    assert torch.equal(ar, rs)


def test_mm_ar_precision_risk_on_gpu():
    """The precision risk the pages warn of, measured on the GPU results: the
    mean error against the exact sum grows with every rounding of partials."""
    W = 8
    d = wl.gemm_inputs(53, 256, 512, 256, wl.BF16, std=1.0, nsim=W)
    x1, x2 = to_dev(d["x1"], "bf16"), to_dev(d["x2"], "bf16")
    exact = sum(numerics.decode(d["x1"][w], "bf16") @ numerics.decode(d["x2"][w], "bf16")
                for w in range(W))
    err = []
    for mode in MODES:
        out = mc2.mc2_mm_ar_local(x1, x2, W, rounding=mode)
        torch.cuda.synchronize()
        err.append(float(np.mean(np.abs(to_f64(out) - exact))))
    assert err[0] < err[1] < err[2], err


def test_mm_ar_full_size_sampled():
    """The simulated W=8 workload (8 partials of (16384, 1024) @ (1024, 8192))
    combined with per-rank and per-hop rounding, sampled."""
    _, b = wl.c5_inputs()
    W = 8
    x1, x2 = to_dev(b["x1"], "bf16"), to_dev(b["x2"], "bf16")
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(16384, 24, replace=False))
    cols = np.sort(rng.choice(8192, 32, replace=False))
    ws = torch.empty(mc2.mc2_mm_ar_workspace_size(16384, 8192, W, torch.bfloat16,
                                                  mc2.MC2_AR_HOP_ROUNDED),
                     dtype=torch.uint8, device="cuda")
    parts = _partials(b, W, "bf16", rows, cols)
    for mode in (mc2.MC2_AR_RANK_ROUNDED, mc2.MC2_AR_HOP_ROUNDED):
        out = mc2.mc2_mm_ar_local(x1, x2, W, rounding=mode, workspace=ws)
        torch.cuda.synchronize()
        ref = og.mm_ar(b["x1"], b["x2"], world_size=W, in_dtype="bf16", rounding=mode,
                       rows=rows, cols=cols)
        _assert_combined(to_f64(out)[np.ix_(rows, cols)], ref, parts, mode, f"mode {mode}")
