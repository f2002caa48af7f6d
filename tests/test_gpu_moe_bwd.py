"""Parity of the backward of the MoE dispatch / combine pair (fc2 and fc1
input and weight gradients, SwiGLU backward) against the CPU oracle, through
the C ABI."""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import assert_tol, to_dev, to_f64
from oracle import moe as om
from oracle import numerics as on

pytestmark = pytest.mark.gpu


def _dec(b):
    return on.decode(b, "bf16")


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _assert_wgrad(got, ref, P, Q, sizes, what):
    """fp32 weight gradients: every entry of group g is a sum of K_g exact
    bf16 x bf16 products accumulated in fp32, so |gpu - exact| stays within
    (K_g + 2) * 2^-24 * sum_k |p_k q_k| (accumulation plus the final rounding)."""
    off = 0
    for g, cnt in enumerate(int(c) for c in sizes):
        S = np.abs(P[off:off + cnt]).T @ np.abs(Q[off:off + cnt])
        bound = (cnt + 2) * 2.0 ** -24 * S
        err = np.abs(np.asarray(got[g], np.float64) - ref[g])
        bad = err > bound
        assert not bad.any(), (f"{what} group {g}: {int(bad.sum())} entries outside the fp32 "
                               f"accumulation bound, worst {err[bad].max()}")
        if cnt == 0:
            assert not np.asarray(got[g]).any(), f"{what}: empty group {g} not zero"
        off += cnt


def _small_case():
    E, El, rank = 8, 4, 1
    send_counts = np.array([5, 3, 0, 9, 300, 0, 1, 77], dtype=np.int32)
    recv = send_counts[4:8].copy()
    start, n = 17, 378
    H, I = 264, 136
    d = wl.moe_inputs(seed=71, tokens=16, hidden=H, num_experts=E, topk=2, local_experts=El,
                      inter=I, w_std=0.05)
    b = wl.moe_backward_inputs(72, 400, H, I)
    return dict(E=E, El=El, rank=rank, send_counts=send_counts, recv=recv, start=start, n=n,
                H=H, I=I, w1=d["w1"], w2=d["w2"], **b)


@pytest.mark.parametrize("act", ["none", "swiglu"])
def test_combine_backward_small_ragged(act):
    """ep_rank 1 of 2, local groups of 300, 0, 1 and 77 rows, H = 264 and
    I = 136 (ragged tiles in both): the fc2 input gradient (or, fused, the
    SwiGLU input gradient) and dW2, with the rows past the groups untouched."""
    c = _small_case()
    n, I, H = c["n"], c["I"], c["H"]
    h_rows = n + 3
    cols = 2 * I if act == "swiglu" else I
    dgrad = torch.full((h_rows, cols), 7.0, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mc2.mc2_gmm_combine_backward(
        to_dev(c["dy"], "bf16"), to_dev(c["recv"]), to_dev(c["send_counts"]), to_dev(c["w2"], "bf16"),
        to_dev(c["h"][:h_rows], "bf16"), ep_rank=c["rank"], num_experts=c["E"],
        act=mc2.MC2_ACT_SWIGLU if act == "swiglu" else mc2.MC2_ACT_NONE,
        g_saved=to_dev(c["g"][:h_rows], "bf16") if act == "swiglu" else None,
        dgrad_out=dgrad, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref, ref_dw2 = om.combine_backward(c["dy"], c["recv"], c["send_counts"], ep_rank=1,
                                       local_experts=4, w2=c["w2"], h=c["h"][:h_rows],
                                       g_saved=c["g"][:h_rows], act=act)
    got = to_f64(dgrad)
    assert_tol(got[:n], ref, f"dgrad {act}")
    assert (got[n:] == 7.0).all()
    # the weight gradient, from a second call that returns it
    _, dw2 = mc2.mc2_gmm_combine_backward(
        to_dev(c["dy"], "bf16"), to_dev(c["recv"]), to_dev(c["send_counts"]), to_dev(c["w2"], "bf16"),
        to_dev(c["h"][:h_rows], "bf16"), ep_rank=c["rank"], num_experts=c["E"])
    torch.cuda.synchronize()
    _assert_wgrad(dw2.cpu().numpy(), ref_dw2, _dec(c["h"][:n]), _dec(c["dy"][17:17 + n]), c["recv"],
                  "dW2")


def test_dispatch_backward_small_ragged():
    """The fc1 input gradient lands in exactly this rank's send rows of dx_buf;
    dW1 over the send rows of each local group."""
    c = _small_case()
    n, H, I = c["n"], c["H"], c["I"]
    rest = wl.combine_standins(73, 400, H)
    dx = to_dev(rest, "bf16")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, dw1 = mc2.mc2_gmm_dispatch_backward(
        to_dev(c["dg"][:n + 5], "bf16"), to_dev(c["recv"]), to_dev(c["send_counts"]),
        to_dev(c["w1"], "bf16"), to_dev(c["send"], "bf16"), dx, ep_rank=1, num_experts=8, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref_dx, ref_dw1 = om.dispatch_backward(c["dg"][:n + 5], c["recv"], c["send_counts"], ep_rank=1,
                                           local_experts=4, w1=c["w1"], send_buf=c["send"],
                                           dx_buf=_dec(rest))
    got = to_f64(dx)
    assert_tol(got[17:17 + n], ref_dx[17:17 + n], "dX")
    np.testing.assert_array_equal(_bits(dx)[:17], rest[:17])
    np.testing.assert_array_equal(_bits(dx)[17 + n:], rest[17 + n:])
    _assert_wgrad(dw1.cpu().numpy(), ref_dw1, _dec(c["send"][17:17 + n]), _dec(c["dg"][:n]),
                  c["recv"], "dW1")


def test_backward_count_mismatch_reported_nothing_written():
    c = _small_case()
    bad = c["recv"].copy()
    bad[2] += 1
    I, H = c["I"], c["H"]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dgrad = torch.full((400, I), 3.0, dtype=torch.bfloat16, device="cuda")
    dw2 = torch.full((4, I, H), 5.0, dtype=torch.float32, device="cuda")
    mc2.mc2_gmm_combine_backward(
        to_dev(c["dy"], "bf16"), to_dev(bad), to_dev(c["send_counts"]), to_dev(c["w2"], "bf16"),
        to_dev(c["h"], "bf16"), ep_rank=1, num_experts=8, dgrad_out=dgrad, dw2_out=dw2,
        dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & mc2.MC2_DEVERR_COUNTS
    assert (dgrad.float() == 3.0).all() and (dw2 == 5.0).all()


def _sub_groups(rows, gstart):
    """Sizes of the groups that the sorted local rows `rows` fall in."""
    g = np.searchsorted(gstart, rows, side="right") - 1
    return np.bincount(g, minlength=len(gstart) - 1)


def test_c4_backward_full_size_sampled():
    """The C4 shapes (32768 tokens, top-8 of 128 experts, local experts 0-15,
    H = 2048, I = 768) with the counts of its router, in the launch
    configuration the benchmark times; sampled rows and columns against the
    oracle."""
    d = wl.c4_inputs()
    counts = om.histc(d["sel"], d["E"]).astype(np.int32)
    recv = counts[:16].copy()
    n = int(recv.sum())
    H, I = d["H"], d["I"]
    b = wl.moe_backward_inputs(1006, n, H, I)
    dev = {k: to_dev(v, "bf16") for k, v in b.items()}
    w1, w2 = to_dev(d["w1"], "bf16"), to_dev(d["w2"], "bf16")
    rc, sc = to_dev(recv), to_dev(counts)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dG, dw2 = mc2.mc2_gmm_combine_backward(dev["dy"], rc, sc, w2, dev["h"], ep_rank=0,
                                           num_experts=128, act=mc2.MC2_ACT_SWIGLU,
                                           g_saved=dev["g"], dev_err=err)
    dx = torch.zeros((n, H), dtype=torch.bfloat16, device="cuda")
    _, dw1 = mc2.mc2_gmm_dispatch_backward(dev["dg"], rc, sc, w1, dev["send"], dx, ep_rank=0,
                                           num_experts=128, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    rng = np.random.default_rng(8)
    gstart = np.concatenate([[0], np.cumsum(recv)])
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), gstart[1:-1],
                                     gstart[1:-1] - 1]))
    rows = rows[(rows >= 0) & (rows < n)]
    sizes = _sub_groups(rows, gstart)
    W1, W2 = _dec(d["w1"]), _dec(d["w2"])
    dA, _ = om.gmm_backward(np.zeros((len(rows), I)), sizes, W2, _dec(b["dy"][rows]))
    ref = on.round_to(om.swiglu_backward(_dec(b["g"][rows]), dA), "bf16")
    assert_tol(to_f64(dG[torch.as_tensor(rows, device="cuda")]), ref, "C4 dG rows")
    ref, _ = om.gmm_backward(np.zeros((len(rows), H)), sizes, W1, _dec(b["dg"][rows]))
    assert_tol(to_f64(dx[torch.as_tensor(rows, device="cuda")]), on.round_to(ref, "bf16"),
               "C4 dX rows")
    J = np.sort(rng.choice(H, 24, replace=False))
    _, ref = om.gmm_backward(_dec(b["h"]), recv, W2[:, :, J], _dec(b["dy"])[:, J])
    _assert_wgrad(dw2.cpu().numpy()[:, :, J], ref, _dec(b["h"]), _dec(b["dy"])[:, J], recv, "C4 dW2")
    J2 = np.sort(rng.choice(2 * I, 24, replace=False))
    _, ref = om.gmm_backward(_dec(b["send"]), recv, W1[:, :, J2], _dec(b["dg"])[:, J2])
    _assert_wgrad(dw1.cpu().numpy()[:, :, J2], ref, _dec(b["send"]), _dec(b["dg"])[:, J2], recv,
                  "C4 dW1")


def test_weight_gradient_split_groups_deterministic():
    """Groups of 5000 and 9000 rows (2 and 3 slices of 4096 rows, partial tiles
    summed in slice order) plus an empty one: the whole dW1 and dW2 against
    the oracle, and a second call gives the same bits, with workspaces whose
    every byte is 0xff (the tile counters are cleared by the call itself)."""
    H, I = 264, 136
    send_counts = np.array([5000, 0, 9000], dtype=np.int32)
    recv = send_counts.copy()
    n = int(recv.sum())
    d = wl.moe_inputs(seed=74, tokens=16, hidden=H, num_experts=3, topk=1, local_experts=3,
                      inter=I, w_std=0.05)
    b = wl.moe_backward_inputs(75, n, H, I)
    dev = {k: to_dev(v, "bf16") for k, v in b.items()}
    rc, sc = to_dev(recv), to_dev(send_counts)
    w1, w2 = to_dev(d["w1"], "bf16"), to_dev(d["w2"], "bf16")
    dx = torch.zeros((n, H), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    dirty = lambda m, nn: torch.full((mc2.mc2_gmm_backward_workspace_size(n, 3, m, nn),), 0xFF,
                                     dtype=torch.uint8, device="cuda")
    for call in range(2):
        _, dw2 = mc2.mc2_gmm_combine_backward(dev["dy"], rc, sc, w2, dev["h"], ep_rank=0,
                                              num_experts=3, dev_err=err,
                                              workspace=dirty(I, H) if call else None)
        _, dw1 = mc2.mc2_gmm_dispatch_backward(dev["dg"], rc, sc, w1, dev["send"], dx, ep_rank=0,
                                               num_experts=3, dev_err=err,
                                               workspace=dirty(H, 2 * I) if call else None)
        torch.cuda.synchronize()
        outs.append((dw1.cpu().numpy(), dw2.cpu().numpy()))
    assert err.item() == 0
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    _, ref_dw2 = om.combine_backward(b["dy"], recv, send_counts, ep_rank=0, local_experts=3,
                                     w2=d["w2"], h=b["h"], act="none")
    _assert_wgrad(outs[0][1], ref_dw2, _dec(b["h"]), _dec(b["dy"]), recv, "split dW2")
    _, ref_dw1 = om.dispatch_backward(b["dg"], recv, send_counts, ep_rank=0, local_experts=3,
                                      w1=d["w1"], send_buf=b["send"], dx_buf=np.zeros((n, H)))
    _assert_wgrad(outs[0][0], ref_dw1, _dec(b["send"]), _dec(b["dg"]), recv, "split dW1")


def test_weight_gradient_long_ragged_groups_ragged_tiles():
    """40011 rows in ragged groups (17001 and 22943 rows: several 4096-row
    slices each, the last ending inside a K stage; groups of 3 and 64 rows)
    with H = 264 (a 256-wide tile plus an 8-wide one, for the rows of dW1 and
    the columns of dW2) and I = 136: both operands are read in place, k-major,
    with the clamped last 16-byte piece at the ragged edges. The whole dW1 and
    dW2 against the oracle."""
    H, I = 264, 136
    send_counts = np.array([17001, 3, 0, 64, 22943], dtype=np.int32)
    recv = send_counts.copy()
    n = int(recv.sum())
    d = wl.moe_inputs(seed=76, tokens=16, hidden=H, num_experts=5, topk=1, local_experts=5,
                      inter=I, w_std=0.05)
    b = wl.moe_backward_inputs(77, n, H, I)
    dev = {k: to_dev(v, "bf16") for k, v in b.items()}
    rc, sc = to_dev(recv), to_dev(send_counts)
    w1, w2 = to_dev(d["w1"], "bf16"), to_dev(d["w2"], "bf16")
    dx = torch.zeros((n, H), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, dw2 = mc2.mc2_gmm_combine_backward(dev["dy"], rc, sc, w2, dev["h"], ep_rank=0,
                                          num_experts=5, dev_err=err)
    _, dw1 = mc2.mc2_gmm_dispatch_backward(dev["dg"], rc, sc, w1, dev["send"], dx, ep_rank=0,
                                           num_experts=5, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    _, ref_dw2 = om.combine_backward(b["dy"], recv, send_counts, ep_rank=0, local_experts=5,
                                     w2=d["w2"], h=b["h"], act="none")
    _assert_wgrad(dw2.cpu().numpy(), ref_dw2, _dec(b["h"]), _dec(b["dy"]), recv, "many-item dW2")
    ref_dx, ref_dw1 = om.dispatch_backward(b["dg"], recv, send_counts, ep_rank=0,
                                           local_experts=5, w1=d["w1"], send_buf=b["send"],
                                           dx_buf=np.zeros((n, H)))
    _assert_wgrad(dw1.cpu().numpy(), ref_dw1, _dec(b["send"]), _dec(b["dg"]), recv, "many-item dW1")
    # the input gradient too, every row: its 159 row tiles by 2 column tiles
    # leave a last round of 62 tiles on 256 CUs, run as 128-row halves
    assert_tol(to_f64(dx), ref_dx, "many-item dX")


def test_swiglu_combine_backward_half_tile_last_round():
    """The fused SwiGLU backward in the last dispatch round of the grouped
    kernel: groups of 5000, 300, 3 and 10900 rows give 66 row tiles by 4
    column tiles (I = 1024), 264 tiles on 256 CUs, so the last 8 run as
    128-row halves; they are the last row tiles of the 10900-row group, whose
    final tile holds 148 rows (its upper half is not empty). H = 200 puts a
    tail in K. Every element of dG against the oracle."""
    H, I = 200, 1024
    send_counts = np.array([5000, 300, 3, 10900], dtype=np.int32)
    recv = send_counts.copy()
    n = int(recv.sum())
    d = wl.moe_inputs(seed=78, tokens=16, hidden=H, num_experts=4, topk=1, local_experts=4,
                      inter=I, w_std=0.05)
    b = wl.moe_backward_inputs(79, n, H, I)
    dgrad = torch.full((n, 2 * I), 7.0, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mc2.mc2_gmm_combine_backward(to_dev(b["dy"], "bf16"), to_dev(recv), to_dev(send_counts),
                                 to_dev(d["w2"], "bf16"), to_dev(b["h"], "bf16"), ep_rank=0,
                                 num_experts=4, act=mc2.MC2_ACT_SWIGLU,
                                 g_saved=to_dev(b["g"], "bf16"), dgrad_out=dgrad, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref, _ = om.combine_backward(b["dy"], recv, send_counts, ep_rank=0, local_experts=4,
                                 w2=d["w2"], h=b["h"], g_saved=b["g"], act="swiglu")
    assert_tol(to_f64(dgrad), ref, "SwiGLU dG with a half-tile last round")


def test_backward_no_local_rows():
    """Every local expert receives no rows: the weight gradients are exact
    zeros and no input-gradient row is written."""
    H, I = 64, 32
    send_counts = np.array([7, 5, 0, 0], dtype=np.int32)  # experts 2, 3 are rank 1's
    recv = send_counts[2:4].copy()
    d = wl.moe_inputs(seed=76, tokens=8, hidden=H, num_experts=4, topk=1, local_experts=2,
                      inter=I)
    b = wl.moe_backward_inputs(77, 12, H, I)
    rc, sc = to_dev(recv), to_dev(send_counts)
    dgrad = torch.full((4, 2 * I), 9.0, dtype=torch.bfloat16, device="cuda")
    dx = torch.full((12, H), 9.0, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, dw2 = mc2.mc2_gmm_combine_backward(to_dev(b["dy"], "bf16"), rc, sc, to_dev(d["w2"], "bf16"),
                                          to_dev(b["h"][:4], "bf16"), ep_rank=1, num_experts=4,
                                          act=mc2.MC2_ACT_SWIGLU, g_saved=to_dev(b["g"][:4], "bf16"),
                                          dgrad_out=dgrad, dev_err=err)
    _, dw1 = mc2.mc2_gmm_dispatch_backward(to_dev(b["dg"][:4], "bf16"), rc, sc,
                                           to_dev(d["w1"], "bf16"), to_dev(b["send"], "bf16"), dx,
                                           ep_rank=1, num_experts=4, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert not dw2.any() and not dw1.any()
    assert (dgrad.float() == 9.0).all() and (dx.float() == 9.0).all()
