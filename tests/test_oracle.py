"""Pins for the CPU oracle: it is checked against what the pages and the
mathematics fix, never against itself.

Each test names the plausible mistake it would catch.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import gemm, moe, numerics
from conftest import GOLDEN

def bf16_bits(vals):
    """Exact small values -> bf16 bits via torch (independent of the oracle)."""
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- numerics

def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    got = numerics.decode(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1 + 2 ** -7
    assert got[3] == 0.0 and math.copysign(1, got[4]) == -1 and math.isinf(got[5])


def test_round_hand_cases():
    """Ties to even, subnormal spacing and overflow (a wrong significand width
    or a round-half-up rule fails here)."""
    with open(os.path.join(GOLDEN, "rounding_hand.txt"), encoding="utf-8") as f:
        n = 0
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fmt, val, _, want = line.split()
            v = float.fromhex(val) if "0x" in val else float(val)
            w = float("inf") if want == "inf" else (float.fromhex(want) if "0x" in want else float(want))
            assert numerics.round_to(np.array([v]), fmt)[0] == w, line
            n += 1
    assert n >= 8


def test_round_bf16_matches_torch_cast():
    """float32 values are rounded once either way, so the float64 -> bf16
    rounding must agree with torch's float32 -> bf16 cast bit for bit."""
    rng = np.random.default_rng(0)
    parts = [rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
             (rng.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16 | 0x8000).view(np.float32),  # ties
             (rng.integers(0, 2 ** 23, 5000).astype(np.uint32)).view(np.float32)]  # subnormals
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.concatenate(parts)
        x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.round_to(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        (rng.integers(-2048, 2048, 3000) + 0.5) * 2.0 ** rng.integers(-25, 5, 3000)])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    got = numerics.round_to(x, "f16")
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------- GEMM

def _brute_mm(A, B):
    m, k = A.shape
    n = B.shape[1]
    C = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            s = 0.0
            for t in range(k):
                s += A[i, t] * B[t, j]
            C[i, j] = s
    return C


def test_mm_rs_hand_example(golden):
    """Hand-worked W=2 reduce-scatter: catches a dropped partial, a bias added
    once instead of per partial, or swapped chunks."""
    g = golden("mm_rs_w2_hand.txt")
    x1 = np.stack([g["x1_0"], g["x1_1"]]).astype(np.float16)
    x2 = np.stack([g["x2_0"], g["x2_1"]]).astype(np.float16)
    out = gemm.mm_rs(x1, x2, world_size=2, in_dtype="f16", nsim=2)
    np.testing.assert_array_equal(out, g["out_nobias"])
    outb = gemm.mm_rs(x1, x2, world_size=2, in_dtype="f16", nsim=2,
                      bias=g["bias"].astype(np.float16))
    np.testing.assert_array_equal(outb, g["out_bias"])
    np.testing.assert_array_equal(outb[gemm.chunk_rows(4, 2, 0)], g["chunk0_bias"])
    np.testing.assert_array_equal(outb[gemm.chunk_rows(4, 2, 1)], g["chunk1_bias"])
    # x2 handed over transposed gives the same product
    x2t = np.ascontiguousarray(np.swapaxes(x2, 1, 2))
    np.testing.assert_array_equal(
        gemm.mm_rs(x1, x2t, world_size=2, in_dtype="f16", nsim=2, x2_trans=True), out)


def test_mm_brute_force_nonsquare():
    """Triple loop on a non-square shape: a transposed operand or a wrong
    index fails (m, k, n all different)."""
    d = wl.gemm_inputs(5, 6, 7, 5, wl.BF16, std=1.0, nsim=1, bias=True)
    A = numerics.decode(d["x1"], "bf16")
    B = numerics.decode(d["x2"], "bf16")
    b = numerics.decode(d["bias"], "bf16")
    want = numerics.round_to(_brute_mm(A, B) + b[None, :], "bf16")
    got = gemm.mm_rs(d["x1"], d["x2"], world_size=2, in_dtype="bf16", bias=d["bias"])
    np.testing.assert_array_equal(got, want)
    got_ag = gemm.ag_mm(d["x1"], d["x2"], world_size=3, in_dtype="bf16", bias=d["bias"])
    np.testing.assert_array_equal(got_ag, want)


def test_chunks_concatenate_to_full_matmul():
    d = wl.gemm_inputs(6, 64, 32, 24, wl.BF16, std=1.0)
    full = gemm.mm_rs(d["x1"], d["x2"], world_size=1, in_dtype="bf16", out_dtype="f32")
    W = 4
    parts = [gemm.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype="bf16", out_dtype="f32",
                        rows=np.arange(64)[gemm.chunk_rows(64, W, c)]) for c in range(W)]
    np.testing.assert_array_equal(np.concatenate(parts), full)
    # row/col restriction equals slicing of the full result
    rows, cols = np.array([3, 17, 40]), np.array([0, 5, 23])
    np.testing.assert_array_equal(
        gemm.mm_rs(d["x1"], d["x2"], world_size=W, in_dtype="bf16", rows=rows, cols=cols),
        numerics.round_to(full, "bf16")[np.ix_(rows, cols)])


def test_sim_rs_equals_concatenated_k():
    """sum_w x1_w @ x2_w == [x1_0 | x1_1 | ...] @ [x2_0 ; x2_1 ; ...]."""
    d = wl.gemm_inputs(7, 16, 24, 8, wl.F16, nsim=3)
    got = gemm.mm_rs(d["x1"], d["x2"], world_size=2, in_dtype="f16", nsim=3, out_dtype="f32")
    A = np.concatenate([d["x1"][w] for w in range(3)], axis=1).astype(np.float64)
    B = np.concatenate([d["x2"][w] for w in range(3)], axis=0).astype(np.float64)
    np.testing.assert_allclose(got, A @ B, rtol=1e-13, atol=1e-12)


def test_int8_exact_against_integer_matmul():
    """The float64 route must equal numpy's integer matmul bit for bit."""
    d = wl.gemm_inputs(8, 96, 1024, 80, wl.I8)
    acc = gemm.mm_rs(d["x1"], d["x2"], world_size=4, in_dtype="i8", out_dtype="i32")
    want = d["x1"].astype(np.int64) @ d["x2"].astype(np.int64)
    assert acc.dtype == np.int64
    np.testing.assert_array_equal(acc, want)
    # extreme values: all +-127 at the largest k the API accepts stays exact
    k = 65534
    x1 = np.full((1, k), 127, np.int8)
    x2 = np.full((k, 1), -127, np.int8)
    assert gemm.mm_rs(x1, x2, world_size=1, in_dtype="i8", out_dtype="i32")[0, 0] == -127 * 127 * k


def test_quant_hand_example(golden):
    """Hand-worked dequant: catches a scale applied by the wrong index or
    bias added after scaling."""
    g = golden("mm_quant_hand.txt")
    x1, x2 = g["x1"].astype(np.int8), g["x2"].astype(np.int8)
    s1, s2 = g["x1_scale"].astype(np.float32), g["x2_scale"].astype(np.float32)
    np.testing.assert_array_equal(
        gemm.mm_rs(x1, x2, world_size=2, in_dtype="i8", out_dtype="i32"), g["acc"])
    np.testing.assert_array_equal(
        gemm.mm_rs(x1, x2, world_size=2, in_dtype="i8", x1_scale=s1, x2_scale=s2), g["out_nobias"])
    np.testing.assert_array_equal(
        gemm.mm_rs(x1, x2, world_size=2, in_dtype="i8", x1_scale=s1, x2_scale=s2,
                   bias=bf16_bits(g["bias"]), bias_dtype="bf16", out_dtype="f32"), g["out_bias"])


def test_quant_unit_and_pow2_scales_closed_form():
    d = wl.gemm_inputs(9, 32, 256, 16, wl.I8)
    acc = d["x1"].astype(np.int64) @ d["x2"].astype(np.int64)
    ones = np.ones(32, np.float32), np.ones(16, np.float32)
    np.testing.assert_array_equal(
        gemm.mm_rs(d["x1"], d["x2"], world_size=1, in_dtype="i8", x1_scale=ones[0],
                   x2_scale=ones[1], out_dtype="f32"), acc)
    s1 = np.ldexp(np.ones(32), -(np.arange(32) % 7)).astype(np.float32)
    s2 = np.ldexp(np.ones(16), (np.arange(16) % 3) - 1).astype(np.float32)
    got = gemm.mm_rs(d["x1"], d["x2"], world_size=1, in_dtype="i8", x1_scale=s1,
                     x2_scale=s2, out_dtype="f32")
    want = acc * s1[:, None].astype(np.float64) * s2[None, :].astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_quant_brute_force_random_scales():
    d = wl.gemm_inputs(10, 5, 9, 4, wl.I8, quant=True)
    got = gemm.mm_rs(d["x1"], d["x2"], world_size=1, in_dtype="i8",
                     x1_scale=d["x1_scale"], x2_scale=d["x2_scale"], out_dtype="f32")
    for i in range(5):
        for j in range(4):
            acc = sum(int(d["x1"][i, t]) * int(d["x2"][t, j]) for t in range(9))
            want = (float(d["x1_scale"][i]) * float(d["x2_scale"][j])) * acc
            assert got[i, j] == pytest.approx(want, rel=1e-15)


def test_chunk_order():
    assert gemm.chunk_order(4, 1, "ag") == [1, 2, 3, 0]
    assert gemm.chunk_order(4, 1, "rs") == [2, 3, 0, 1]
    assert gemm.chunk_order(8, 0, "ag") == list(range(8))
    assert sorted(gemm.chunk_order(8, 5, "rs")) == list(range(8))
    assert gemm.chunk_order(8, 5, "rs")[-1] == 5


def test_chunk_rows_requires_divisible_m():
    with pytest.raises(ValueError):
        gemm.chunk_rows(10, 4, 0)
    assert gemm.chunk_rows(128, 2, 1) == slice(64, 128)


def test_sub_chunk_rows_hand_worked():
    # m = 20, W = 2: chunk 1 is rows 10..19; three pieces of 4, 3, 3 rows
    got = [gemm.sub_chunk_rows(20, 2, 1, 3, j) for j in range(3)]
    assert got == [slice(10, 14), slice(14, 17), slice(17, 20)]
    # the default split and a split of one keep the chunk whole
    assert gemm.sub_chunk_rows(20, 2, 0, 0, 0) == slice(0, 10)
    assert gemm.sub_chunk_rows(20, 2, 0, 1, 0) == slice(0, 10)
    # an even split: 4 pieces of 256 rows of a 1024-row chunk
    assert gemm.sub_chunk_rows(8192, 8, 3, 4, 2) == slice(3 * 1024 + 512, 3 * 1024 + 768)


@pytest.mark.parametrize("m,W,s", [(64, 4, 3), (96, 2, 7), (40, 8, 5), (1024, 1, 9)])
def test_sub_chunks_partition_each_chunk(m, W, s):
    for c in range(W):
        pieces = [gemm.sub_chunk_rows(m, W, c, s, j) for j in range(s)]
        rows = np.concatenate([np.arange(p.start, p.stop) for p in pieces])
        np.testing.assert_array_equal(rows, np.arange(m)[gemm.chunk_rows(m, W, c)])
        sizes = [p.stop - p.start for p in pieces]
        assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
        assert sizes == sorted(sizes, reverse=True)


def test_sub_chunk_rows_rejects_empty_pieces():
    with pytest.raises(ValueError):
        gemm.sub_chunk_rows(16, 4, 0, 5, 0)
    with pytest.raises(ValueError):
        gemm.sub_chunk_rows(16, 4, 0, 2, 2)


def test_segment_order():
    assert gemm.segment_order(2, 1, "rs", 2) == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert gemm.segment_order(4, 1, "ag", 0) == [(1, 0), (2, 0), (3, 0), (0, 0)]
    order = gemm.segment_order(8, 5, "rs", 3)
    assert sorted(c * 3 + j for c, j in order) == list(range(24))
    assert order[-3:] == [(5, 0), (5, 1), (5, 2)]


# ----------------------------------------------------------------- MoE

def test_histc_against_torch_histc_and_bincount():
    d = wl.moe_inputs(seed=11, tokens=512, hidden=8, num_experts=64, topk=4,
                      local_experts=4, inter=4)
    counts = moe.histc(d["sel"], 64)
    th = torch.histc(torch.from_numpy(d["sel"]).float().reshape(-1), bins=64, min=0, max=64)
    np.testing.assert_array_equal(counts, th.numpy().astype(np.int64))
    np.testing.assert_array_equal(counts, np.bincount(d["sel"].reshape(-1), minlength=64))
    assert counts.sum() == 512 * 4


def test_histc_ignores_invalid_ids():
    sel = np.array([[0, 5], [-1, 2], [3, 3]], np.int32)
    np.testing.assert_array_equal(moe.histc(sel, 4), [1, 0, 1, 2])


def test_permute_hand_example(golden):
    g = golden("moe_permute_hand.txt")
    sel = g["sel"].astype(np.int32)
    x = np.arange(3 * 4, dtype=np.uint16).reshape(3, 4)
    p = moe.permute(x, sel, 3)
    np.testing.assert_array_equal(moe.histc(sel, 3), g["counts"])
    np.testing.assert_array_equal(p["sorted_idx"], g["sorted_idx"])
    np.testing.assert_array_equal(p["unpermute_idx"], g["unpermute_idx"])
    np.testing.assert_array_equal(p["offsets"], g["offsets"])
    np.testing.assert_array_equal(p["permuted"], x[g["permuted_token"].astype(int)])
    out = moe.unpermute(g["y_full"], p["unpermute_idx"], g["probs"].astype(np.float32), 3, 2)
    np.testing.assert_array_equal(out, g["out"])


def _brute_permute(sel, E):
    flat = sel.reshape(-1)
    order = []
    for e in range(E):
        for s in range(flat.size):
            if flat[s] == e:
                order.append(s)
    return np.array(order, dtype=np.int64)


def test_permute_brute_force_and_properties():
    d = wl.moe_inputs(seed=12, tokens=300, hidden=16, num_experts=16, topk=3,
                      local_experts=4, inter=4)
    sel = d["sel"].copy()
    sel[7, 1] = 16      # invalid ids are left out
    sel[100, 0] = -3
    p = moe.permute(d["x"], sel, 16)
    order = _brute_permute(sel, 16)
    n = p["n_valid"]
    assert n == 300 * 3 - 2 == order.size
    np.testing.assert_array_equal(p["sorted_idx"][:n], order)
    assert np.all(p["sorted_idx"][n:] == -1)
    # unpermute_idx is the inverse permutation
    np.testing.assert_array_equal(p["unpermute_idx"][p["sorted_idx"][:n]], np.arange(n))
    assert p["unpermute_idx"][7 * 3 + 1] == -1 and p["unpermute_idx"][100 * 3] == -1
    # segments: sizes equal counts and each segment is ascending in slot order
    counts = moe.histc(sel, 16)
    np.testing.assert_array_equal(np.diff(p["offsets"]), counts)
    for e in range(16):
        seg = p["sorted_idx"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(sel.reshape(-1)[seg] == e)
    np.testing.assert_array_equal(p["permuted"], d["x"][order // 3])


def test_permute_unpermute_identity_top1():
    """top-1, probs = 1, no GMM: unpermute(permute(x)) == x bit for bit."""
    rng = np.random.default_rng(13)
    T, H, E = 200, 24, 8
    x = wl.encode_bf16(rng.standard_normal((T, H), dtype=np.float32))
    sel = rng.integers(0, E, (T, 1)).astype(np.int32)
    p = moe.permute(x, sel, E)
    y = numerics.decode(p["permuted"], "bf16")
    out = moe.unpermute(y, p["unpermute_idx"], np.ones((T, 1), np.float32), T, 1)
    np.testing.assert_array_equal(out, numerics.decode(x, "bf16"))


def test_permute_unpermute_identity_top8_eighths():
    """top-8 with probs = 1/8: the sum of eight x/8 terms is exact, so out == x."""
    rng = np.random.default_rng(14)
    T, H, E, K = 64, 16, 32, 8
    x = wl.encode_bf16(rng.standard_normal((T, H), dtype=np.float32))
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    p = moe.permute(x, sel, E)
    out = moe.unpermute(numerics.decode(p["permuted"], "bf16"), p["unpermute_idx"],
                        np.full((T, K), 0.125, np.float32), T, K)
    np.testing.assert_array_equal(out, numerics.decode(x, "bf16"))


def test_swiglu_closed_forms():
    a = np.array([[0.0, 3.0], [40.0, 2.0], [-40.0, 5.0], [1.0, 1.0]])
    h = moe.swiglu(a)[:, 0]
    assert h[0] == 0.0
    assert h[1] == pytest.approx(80.0, rel=1e-15)
    assert abs(h[2]) < 1e-15
    assert h[3] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # gate and up are not interchangeable
    assert moe.swiglu(np.array([[2.0, 3.0]]))[0, 0] != moe.swiglu(np.array([[3.0, 2.0]]))[0, 0]


def test_gmm_swiglu_hand_example(golden):
    g = golden("gmm_swiglu_hand.txt")
    rows = bf16_bits(g["rows"])
    w1 = bf16_bits(np.stack([g["w1_0"], g["w1_1"]]))
    h = moe.gmm(rows, g["group_sizes"].astype(int), w1, act="swiglu")
    np.testing.assert_array_equal(h[:, 0], g["h_bf16"].reshape(-1))
    np.testing.assert_allclose(moe.swiglu(numerics.decode(rows, "bf16")[:1] @ numerics.decode(w1[0], "bf16"))[:, 0],
                               g["h_exact"].reshape(-1)[:1], rtol=1e-15)


def test_gmm_single_group_is_plain_matmul():
    d = wl.moe_inputs(seed=15, tokens=40, hidden=32, num_experts=4, topk=2,
                      local_experts=1, inter=8)
    rows = d["x"][:37]
    got = moe.gmm(rows, [37], d["w1"], act="none")
    want = numerics.round_to(numerics.decode(rows, "bf16") @ numerics.decode(d["w1"][0], "bf16"), "bf16")
    np.testing.assert_array_equal(got, want)


def test_gmm_brute_force_ragged_and_empty_groups():
    d = wl.moe_inputs(seed=16, tokens=40, hidden=6, num_experts=4, topk=2,
                      local_experts=4, inter=3)
    sizes = [5, 0, 9, 1]
    rows = d["x"][:15]
    got = moe.gmm(rows, sizes, d["w1"], act="swiglu")
    R = numerics.decode(rows, "bf16")
    Wt = numerics.decode(d["w1"], "bf16")
    off = 0
    for g, cnt in enumerate(sizes):
        for r in range(off, off + cnt):
            a = _brute_mm(R[r:r + 1], Wt[g])[0]
            want = [a[j] / (1 + math.exp(-a[j])) * a[3 + j] for j in range(3)]
            np.testing.assert_array_equal(got[r], numerics.round_to(np.array(want), "bf16"))
        off += cnt


def test_swiglu_backward_closed_forms():
    """At gate 0: s = 1/2, silu = 0, silu' = 1/2. Large gate: silu' -> 1 and
    silu -> g. Very negative gate: both vanish. Catches a dropped term of
    silu' or swapped gate / up columns."""
    dh = np.array([[2.0, -3.0]])
    got = moe.swiglu_backward(np.array([[0.0, 0.0, 5.0, 7.0]]), dh)
    np.testing.assert_array_equal(got, [[5.0, -10.5, 0.0, 0.0]])
    got = moe.swiglu_backward(np.array([[40.0, 3.0]]), np.array([[1.5]]))
    np.testing.assert_allclose(got, [[4.5, 60.0]], rtol=1e-12)
    got = moe.swiglu_backward(np.array([[-60.0, 3.0]]), np.array([[1.5]]))
    assert np.all(np.abs(got) < 1e-20)
    # g = 1: silu' = s (1 + (1 - s)) with s = 1 / (1 + e^-1)
    s = 1.0 / (1.0 + math.exp(-1.0))
    got = moe.swiglu_backward(np.array([[1.0, 2.0]]), np.array([[1.0]]))
    np.testing.assert_allclose(got, [[2.0 * s * (2.0 - s), s]], rtol=1e-15)


def _leaf(a):
    return torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)


def test_gmm_backward_matches_autograd():
    """dX = dY W^T and dW = X^T dY per group against torch autograd in float64,
    ragged and empty groups, non-square K x N (a transposed operand fails)."""
    rng = np.random.default_rng(5)
    sizes, K, N = [3, 0, 5, 1], 6, 4
    X = rng.standard_normal((9, K))
    W = rng.standard_normal((4, K, N))
    dY = rng.standard_normal((9, N))
    dX, dW = moe.gmm_backward(X, sizes, W, dY)
    Xt, Wt = _leaf(X), _leaf(W)
    outs, off = [], 0
    for g, c in enumerate(sizes):
        outs.append(Xt[off:off + c] @ Wt[g])
        off += c
    (torch.cat(outs) * torch.tensor(dY)).sum().backward()
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert not dW[1].any()


def test_moe_backward_chain_matches_autograd():
    """The combine and dispatch backward on ep_rank 1 of 2 (E = 4, E_l = 2),
    with bf16-stored inputs: each stage equals torch autograd of the forward
    stage it inverts (fc2 on the stored h, SwiGLU on the stored
    pre-activation, fc1 on the send rows), and only this rank's rows of the
    input-gradient buffer change."""
    rng = np.random.default_rng(6)
    send_counts = np.array([2, 3, 4, 5])
    recv = send_counts[2:4]
    H, I, n = 16, 8, 9
    bf = lambda shape, sd=1.0: wl.encode_bf16((rng.standard_normal(shape) * sd).astype(np.float32))
    send_buf, dy_buf = bf((14, H)), bf((14, H))
    w1, w2 = bf((2, H, 2 * I), 0.3), bf((2, I, H), 0.3)
    g_saved, h = bf((n, 2 * I), 2.0), bf((n, I))
    dec = lambda b: numerics.decode(b, "bf16")

    dgrad, dW2 = moe.combine_backward(dy_buf, recv, send_counts, ep_rank=1, local_experts=2,
                                      w2=w2, h=h, g_saved=g_saved, act="swiglu", dtype=None)
    hl, w2l, gl = _leaf(dec(h)), _leaf(dec(w2)), _leaf(dec(g_saved))
    dY = torch.tensor(dec(dy_buf)[5:14])
    y = torch.cat([hl[:4] @ w2l[0], hl[4:] @ w2l[1]])
    (y * dY).sum().backward()
    np.testing.assert_allclose(dW2, w2l.grad.numpy(), rtol=1e-12, atol=1e-12)
    act = torch.nn.functional.silu(gl[:, :I]) * gl[:, I:]
    (act * hl.grad).sum().backward()
    np.testing.assert_allclose(dgrad, gl.grad.numpy(), rtol=1e-12, atol=1e-12)

    dg = bf((n, 2 * I))
    rest = rng.standard_normal((14, H))
    dx, dW1 = moe.dispatch_backward(dg, recv, send_counts, ep_rank=1, local_experts=2, w1=w1,
                                    send_buf=send_buf, dx_buf=rest, dtype=None)
    xl, w1l = _leaf(dec(send_buf)[5:14]), _leaf(dec(w1))
    a = torch.cat([xl[:4] @ w1l[0], xl[4:] @ w1l[1]])
    (a * torch.tensor(dec(dg))).sum().backward()
    np.testing.assert_allclose(dW1, w1l.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx[5:14], xl.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dx[:5], rest[:5])

    # the plain fc2 backward (no SwiGLU) is the fc2 input gradient itself
    dA, _ = moe.combine_backward(dy_buf, recv, send_counts, ep_rank=1, local_experts=2, w2=w2,
                                 h=h, act="none", dtype=None)
    np.testing.assert_allclose(dA, hl.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_dispatch_combine_slice_for_nonzero_rank():
    """ep_rank = 1 of 2 (E = 4, E_l = 2): the local rows start after experts
    0 and 1, and the combine writes exactly those rows."""
    rng = np.random.default_rng(17)
    send_counts = np.array([3, 1, 2, 4])
    H, I = 4, 2
    send_buf = wl.encode_bf16(rng.standard_normal((10, H), dtype=np.float32))
    w1 = wl.encode_bf16(rng.standard_normal((2, H, 2 * I), dtype=np.float32))
    w2 = wl.encode_bf16(rng.standard_normal((2, I, H), dtype=np.float32))
    recv = send_counts[2:4]
    h = moe.dispatch(send_buf, send_counts, recv, ep_rank=1, local_experts=2, w1=w1)
    assert h.shape == (6, I)
    np.testing.assert_array_equal(h, moe.gmm(send_buf[4:10], [2, 4], w1, act="swiglu"))
    base = np.full((10, H), 7.0)
    y = moe.combine(h, recv, send_counts, ep_rank=1, local_experts=2, w2=w2, combine_buf=base)
    assert np.all(y[:4] == 7.0)
    Wt = numerics.decode(w2, "bf16")
    np.testing.assert_array_equal(y[4:6], numerics.round_to(h[:2] @ Wt[0], "bf16"))
    np.testing.assert_array_equal(y[6:10], numerics.round_to(h[2:6] @ Wt[1], "bf16"))
    with pytest.raises(ValueError):
        moe.dispatch(send_buf, send_counts, np.array([2, 3]), ep_rank=1, local_experts=2, w1=w1)


def test_moe_local_chain_small():
    """The chain's pieces compose: every token's output is the probability
    weighted sum of its local experts' fc2 rows, others contribute zero."""
    d = wl.moe_inputs(seed=18, tokens=96, hidden=16, num_experts=8, topk=2,
                      local_experts=2, inter=8)
    r = moe.moe_local(d["x"], d["sel"], d["probs"], d["w1"], d["w2"], num_experts=8,
                      ep_rank=0, local_experts=2)
    X = numerics.decode(d["x"], "bf16")
    W1 = numerics.decode(d["w1"], "bf16")
    W2 = numerics.decode(d["w2"], "bf16")
    for t in range(96):
        acc = np.zeros(16)
        for k in range(2):
            e = d["sel"][t, k]
            if e < 2:
                a = X[t] @ W1[e]
                h = numerics.round_to(a[:8] / (1 + np.exp(-a[:8])) * a[8:], "bf16")
                acc += float(d["probs"][t, k]) * numerics.round_to(h @ W2[e], "bf16")
        np.testing.assert_array_equal(r["out"][t], numerics.round_to(acc, "bf16"))


def test_router_shapes_ties_and_ranges():
    logits = np.zeros((2, 4), np.float32)
    sel, probs = wl.router(logits, np.zeros(4, np.float32), 2)
    np.testing.assert_array_equal(sel, [[0, 1], [0, 1]])
    np.testing.assert_allclose(probs, 0.25)
    d = wl.moe_inputs(seed=19, tokens=64, hidden=4, num_experts=16, topk=4,
                      local_experts=2, inter=2)
    assert d["sel"].min() >= 0 and d["sel"].max() < 16
    assert all(len(set(r)) == 4 for r in d["sel"].tolist())


def test_per_token_outputs_match_the_chain():
    """Two formulations of the same path agree: per token directly, and
    through histc -> permute -> grouped fc1/fc2 -> unpermute."""
    d = wl.moe_inputs(seed=20, tokens=64, hidden=16, num_experts=8, topk=3,
                      local_experts=4, inter=8)
    r = moe.moe_local(d["x"], d["sel"], d["probs"], d["w1"], d["w2"], num_experts=8,
                      ep_rank=1, local_experts=4)
    toks = np.arange(64)
    np.testing.assert_array_equal(
        moe.token_outputs(d["x"], d["sel"], d["probs"], d["w1"], d["w2"], toks, ep_rank=1,
                          local_experts=4), r["out"])
    start, n = moe.local_slice(r["counts"], 1, 4)
    slots = r["permute"]["sorted_idx"][start:start + n]
    h, y = moe.expert_ffn_rows(d["x"][slots // 3], d["sel"].reshape(-1)[slots] - 4, d["w1"], d["w2"])
    np.testing.assert_array_equal(h, r["h"])
    np.testing.assert_array_equal(y, r["y_full"][start:start + n])


# ---------------------------------------------------------------- MatmulAllReduce

def _bf(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_ar_sum_rank_rounded_is_the_correctly_rounded_exact_sum():
    """W = 32 bf16 partials (8-bit significands) within 10 binades: their exact
    sum needs at most 8 + 10 + 5 bits, so math.fsum (computed without the
    oracle) gives it exactly, it is exact in float32 too, and torch's
    float32 -> bf16 cast is then its one correct rounding. The rank-rounded
    combine must equal it. Catches a dropped partial, a wrong rounding and a
    per-hop rounding."""
    rng = np.random.default_rng(21)
    W, n = 32, 500
    # sign * m * 2^(e - 7) with m in [128, 256): exponents e in [-5, 5)
    m = rng.integers(128, 256, (W, n)).astype(np.float64)
    e = rng.integers(-5, 5, (W, n))
    vals = (rng.choice([-1.0, 1.0], (W, n)) * m * np.exp2(e - 7)).astype(np.float32)
    parts = bf16_bits(vals)
    got = gemm.ar_sum(parts, dtype="bf16", rounding=gemm.AR_RANK_ROUNDED)
    dec = torch.from_numpy(parts.view(np.int16)).view(torch.bfloat16).double().numpy()
    exact = np.array([math.fsum(dec[:, j]) for j in range(n)])
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, want)
    # and the hop-rounded combine is not the same function
    hop = gemm.ar_sum(parts, dtype="bf16", rounding=gemm.AR_HOP_ROUNDED)
    assert not np.array_equal(hop, want)


def test_mm_ar_rounding_modes_hand_worked_bf16():
    """bf16 spacing at 1 is 2**-7. Rank 0's partial 1 + 2**-8 sits exactly half
    way between 1 and 1 + 2**-7 and rounds (ties to even) to 1; rank 1's partial
    2**-8 is exact. The exact sum 1 + 2**-7 is a bf16 value: one rounding keeps
    it, rounding each rank's partial first loses it."""
    x1 = np.stack([_bf([[1.0, 2.0 ** -8]]), _bf([[2.0 ** -8, 0.0]])])
    x2 = np.stack([_bf([[1.0], [1.0]])] * 2)
    got = [gemm.mm_ar(x1, x2, world_size=2, in_dtype="bf16", rounding=r)[0, 0] for r in range(3)]
    assert got == [1.0 + 2.0 ** -7, 1.0, 1.0]


def test_mm_ar_hop_rounding_differs_from_rank_rounding():
    """Partials 1, 2**-8, 2**-8 are all bf16 values. Summed exactly they give
    1 + 2**-7 (a bf16 value); a running sum rounded after each addition stays
    at 1 (1 + 2**-8 is a tie that rounds to even twice)."""
    x1 = np.stack([_bf([[1.0]]), _bf([[2.0 ** -8]]), _bf([[2.0 ** -8]])])
    x2 = np.stack([_bf([[1.0]])] * 3)
    got = [gemm.mm_ar(x1, x2, world_size=3, in_dtype="bf16", rounding=r)[0, 0] for r in range(3)]
    assert got == [1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7, 1.0]


def test_mm_ar_rounding_modes_hand_worked_f16():
    """fp16 spacing at 1 is 2**-10: the same tie one binade of precision down."""
    x1 = np.stack([np.array([[1.0, 2.0 ** -11]], np.float16),
                   np.array([[2.0 ** -11, 0.0]], np.float16)])
    x2 = np.stack([np.ones((2, 1), np.float16)] * 2)
    got = [gemm.mm_ar(x1, x2, world_size=2, in_dtype="f16", rounding=r)[0, 0] for r in range(3)]
    assert got == [1.0 + 2.0 ** -10, 1.0, 1.0]


def test_ar_sum_small_integers_exact_and_w1_identity():
    parts = _bf([[3.0, -7.0], [5.0, 2.0], [-2.0, 4.0]])
    for r in (gemm.AR_RANK_ROUNDED, gemm.AR_HOP_ROUNDED):
        np.testing.assert_array_equal(gemm.ar_sum(parts, dtype="bf16", rounding=r), [6.0, -1.0])
    rng = np.random.default_rng(5)
    one = _bf(rng.standard_normal((1, 64)).astype(np.float32))
    for r in (gemm.AR_RANK_ROUNDED, gemm.AR_HOP_ROUNDED):
        np.testing.assert_array_equal(gemm.ar_sum(one, dtype="bf16", rounding=r),
                                      numerics.decode(one[0], "bf16"))


def test_mm_ar_precision_risk_grows_with_roundings():
    """The precision risk of rounding partials before the all-reduce: on N(0,1)
    data with W = 8 the mean error against the exact sum grows from one
    rounding to per-rank rounding to per-hop rounding."""
    rng = np.random.default_rng(6)
    W, m, k, n = 8, 32, 64, 48
    x1 = _bf(rng.standard_normal((W, m, k)).astype(np.float32))
    x2 = _bf(rng.standard_normal((W, k, n)).astype(np.float32))
    exact = sum(numerics.decode(x1[w], "bf16") @ numerics.decode(x2[w], "bf16") for w in range(W))
    err = [np.mean(np.abs(gemm.mm_ar(x1, x2, world_size=W, in_dtype="bf16", rounding=r) - exact))
           for r in range(3)]
    assert err[0] < err[1] < err[2]
