"""Parity of the MoE expert-parallel local path (histc, permute, grouped fc1 +
SwiGLU, grouped fc2, unpermute) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import assert_tol, to_dev, to_f64
from oracle import moe as om
from oracle import numerics as on

pytestmark = pytest.mark.gpu


def _small(seed=31, T=700, H=264, E=32, K=4, E_l=8, I=136):
    return wl.moe_inputs(seed=seed, tokens=T, hidden=H, num_experts=E, topk=K,
                         local_experts=E_l, inter=I)


def _err():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def test_histc_bit_exact_and_invalid_ids():
    d = _small()
    sel = d["sel"].copy()
    counts = mc2.mc2_moe_histc(to_dev(sel), 32)
    np.testing.assert_array_equal(counts.cpu().numpy(), om.histc(sel, 32))
    sel[3, 1] = 32
    sel[9, 0] = -1
    err = _err()
    counts = mc2.mc2_moe_histc(to_dev(sel), 32, dev_err=err)
    np.testing.assert_array_equal(counts.cpu().numpy(), om.histc(sel, 32))
    assert err.item() & mc2.MC2_DEVERR_EXPERT_ID


@pytest.mark.parametrize("n,E,offset", [
    (3 * 4096 + 77, 128, 0),    # whole 4096-id chunks (16-byte loads), then a ragged chunk
    (3 * 4096 + 77, 128, 1),    # ids not 16-byte aligned: element loads throughout
    (1029 * 4096 + 3, 128, 0),  # more chunks than blocks: blocks take a second chunk
    (8192, 1024, 0), (4096, 1, 0), (1, 5, 0), (4095, 3, 3)])
def test_histc_chunks_alignment_and_grid_stride(n, E, offset):
    sel = wl.expert_ids(77 + n % 1000, n, E)
    base = torch.zeros(n + offset, dtype=torch.int32, device="cuda")
    dsel = base[offset:]
    dsel.copy_(torch.from_numpy(sel))
    err = _err()
    counts = mc2.mc2_moe_histc(dsel, E, dev_err=err)
    np.testing.assert_array_equal(counts.cpu().numpy(), om.histc(sel, E))
    assert err.item() == 0  # lanes past the end are never reported as invalid ids
    # invalid ids in the first (whole) chunk and in the last one
    bad = sel.copy()
    for pos, v in ((0, E), (5, -1), (4000, 2**31 - 1), (n - 1, -2**31), (n // 2, E + 1)):
        bad[min(pos, n - 1)] = v
    dsel.copy_(torch.from_numpy(bad))
    counts = mc2.mc2_moe_histc(dsel, E, counts=counts, dev_err=err)
    np.testing.assert_array_equal(counts.cpu().numpy(), om.histc(bad, E))
    assert err.item() & mc2.MC2_DEVERR_EXPERT_ID


@pytest.mark.parametrize("T,K,E", [(700, 4, 32), (33, 8, 128), (5, 1, 3), (64, 64, 1024),
                                   (129, 3, 17)])
def test_permute_bit_exact(T, K, E):
    rng = np.random.default_rng(T * 1000 + K)
    H = 136
    x = wl.encode_bf16(rng.standard_normal((T, H), dtype=np.float32))
    sel = np.stack([rng.permutation(E)[:K] if K <= E else rng.integers(0, E, K)
                    for _ in range(T)]).astype(np.int32)
    perm, sidx, uidx, offs = mc2.mc2_moe_permute(to_dev(x, "bf16"), to_dev(sel), E)
    torch.cuda.synchronize()
    ref = om.permute(x, sel, E)
    n = ref["n_valid"]
    np.testing.assert_array_equal(sidx.cpu().numpy(), ref["sorted_idx"])
    np.testing.assert_array_equal(uidx.cpu().numpy(), ref["unpermute_idx"])
    np.testing.assert_array_equal(offs.cpu().numpy(), ref["offsets"])
    got = perm.view(torch.int16).cpu().numpy().view(np.uint16)[:n]
    np.testing.assert_array_equal(got, ref["permuted"])


def test_permute_invalid_ids_left_out():
    d = _small(seed=32)
    sel = d["sel"].copy()
    sel[0, 0] = 32
    sel[17, 2] = -4
    err = _err()
    perm, sidx, uidx, offs = mc2.mc2_moe_permute(to_dev(d["x"], "bf16"), to_dev(sel), 32,
                                                 dev_err=err)
    torch.cuda.synchronize()
    ref = om.permute(d["x"], sel, 32)
    assert err.item() & mc2.MC2_DEVERR_EXPERT_ID
    np.testing.assert_array_equal(sidx.cpu().numpy(), ref["sorted_idx"])
    np.testing.assert_array_equal(uidx.cpu().numpy(), ref["unpermute_idx"])
    np.testing.assert_array_equal(offs.cpu().numpy(), ref["offsets"])


def test_top1_permute_unpermute_identity_on_gpu():
    rng = np.random.default_rng(33)
    T, H, E = 1000, 512, 16
    x = wl.encode_bf16(rng.standard_normal((T, H), dtype=np.float32))
    sel = rng.integers(0, E, (T, 1)).astype(np.int32)
    perm, _, uidx, _ = mc2.mc2_moe_permute(to_dev(x, "bf16"), to_dev(sel), E)
    out = mc2.mc2_moe_unpermute(perm, uidx, torch.ones((T, 1), device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_unpermute_parity_with_standins():
    rng = np.random.default_rng(34)
    T, K, H = 300, 8, 264
    y = wl.combine_standins(35, T * K, H, std=1.0)
    idx = rng.permutation(T * K).astype(np.int32)
    idx[5] = -1
    probs = rng.uniform(0, 1, (T, K)).astype(np.float32)
    out = mc2.mc2_moe_unpermute(to_dev(y, "bf16"), to_dev(idx), to_dev(probs))
    ref = om.unpermute(on.decode(y, "bf16"), idx, probs, T, K)
    assert_tol(to_f64(out), ref, "unpermute")


@pytest.mark.parametrize("T,K,H", [(37, 13, 2312), (50, 64, 72), (9, 9, 4096)])
def test_unpermute_slot_groups_and_column_passes(T, K, H):
    """More than 8 slots per token (several groups of 8, the last one ragged)
    and rows of more than 2048 columns (several column passes, the last one
    ragged), with slots that hold no row."""
    rng = np.random.default_rng(T * K + H)
    y = wl.combine_standins(37, T * K, H, std=1.0)
    idx = rng.permutation(T * K).astype(np.int32)
    idx[rng.choice(T * K, size=max(1, T * K // 10), replace=False)] = -1
    probs = rng.uniform(0, 1, (T, K)).astype(np.float32)
    err = _err()
    out = mc2.mc2_moe_unpermute(to_dev(y, "bf16"), to_dev(idx), to_dev(probs), dev_err=err)
    ref = om.unpermute(on.decode(y, "bf16"), idx, probs, T, K)
    assert_tol(to_f64(out), ref, "unpermute")
    assert err.item() == 0


def test_unpermute_out_of_range_index_flagged():
    T, K, H = 4, 2, 8
    y = wl.combine_standins(36, 8, H)
    idx = np.array([0, 1, 2, 3, 4, 99, 6, 7], np.int32)
    err = _err()
    out = mc2.mc2_moe_unpermute(to_dev(y, "bf16"), to_dev(idx), torch.ones((T, K), device="cuda"),
                                dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & mc2.MC2_DEVERR_INDEX
    idx_ok = idx.copy()
    idx_ok[5] = -1
    ref = om.unpermute(on.decode(y, "bf16"), idx_ok, np.ones((T, K), np.float32), T, K)
    np.testing.assert_array_equal(to_f64(out), ref)


def _gmm_inputs(seed, sizes, H, I, E, E_l, ep_rank):
    rng = np.random.default_rng(seed)
    send_counts = rng.integers(0, 40, E).astype(np.int32)
    send_counts[ep_rank * E_l:(ep_rank + 1) * E_l] = sizes
    rows = int(send_counts.sum())
    send = wl.encode_bf16(rng.standard_normal((rows, H), dtype=np.float32))
    w1 = wl.encode_bf16(rng.standard_normal((E_l, H, 2 * I), dtype=np.float32) * 0.1)
    w2 = wl.encode_bf16(rng.standard_normal((E_l, I, H), dtype=np.float32) * 0.1)
    return send_counts, send, w1, w2


@pytest.mark.parametrize("ep_rank", [0, 2])
@pytest.mark.parametrize("act", ["swiglu", "none"])
def test_gmm_dispatch_ragged_and_empty_groups(ep_rank, act):
    E, E_l, H, I = 16, 4, 200, 136
    sizes = np.array([130, 0, 1, 257], np.int32)
    sc, send, w1, _ = _gmm_inputs(37 + ep_rank, sizes, H, I, E, E_l, ep_rank)
    recv = sc[ep_rank * E_l:(ep_rank + 1) * E_l].copy()
    a = mc2.MC2_ACT_SWIGLU if act == "swiglu" else mc2.MC2_ACT_NONE
    h = mc2.mc2_gmm_dispatch(to_dev(send, "bf16"), to_dev(sc), to_dev(recv), to_dev(w1, "bf16"),
                             ep_rank=ep_rank, num_experts=E, act=a)
    ref = om.dispatch(send, sc, recv, ep_rank=ep_rank, local_experts=E_l, w1=w1, act=act)
    assert_tol(to_f64(h)[:ref.shape[0]], ref, f"dispatch {act}")


def test_gmm_combine_writes_only_local_rows():
    E, E_l, H, I, ep_rank = 16, 4, 264, 136, 1
    sizes = np.array([64, 0, 190, 3], np.int32)
    sc, send, _, w2 = _gmm_inputs(41, sizes, H, I, E, E_l, ep_rank)
    recv = sizes.copy()
    rng = np.random.default_rng(42)
    h = wl.encode_bf16(rng.standard_normal((int(sizes.sum()), I), dtype=np.float32))
    base = wl.combine_standins(43, send.shape[0], H)
    buf = to_dev(base, "bf16")
    mc2.mc2_gmm_combine(to_dev(h, "bf16"), to_dev(recv), to_dev(sc), to_dev(w2, "bf16"), buf,
                        ep_rank=ep_rank, num_experts=E)
    ref = om.combine(on.decode(h, "bf16"), recv, sc, ep_rank=ep_rank, local_experts=E_l, w2=w2,
                     combine_buf=on.decode(base, "bf16"))
    got = to_f64(buf)
    start, n = om.local_slice(sc, ep_rank, E_l)
    np.testing.assert_array_equal(np.delete(got, np.s_[start:start + n], 0),
                                  np.delete(ref, np.s_[start:start + n], 0))
    assert_tol(got[start:start + n], ref[start:start + n], "combine")


def test_gmm_count_mismatch_sets_error_and_writes_nothing():
    E, E_l, H, I = 8, 2, 64, 32
    sizes = np.array([5, 7], np.int32)
    sc, send, w1, _ = _gmm_inputs(44, sizes, H, I, E, E_l, 0)
    bad = np.array([5, 6], np.int32)
    err = _err()
    h = torch.full((send.shape[0], I), 3.0, dtype=torch.bfloat16, device="cuda")
    mc2.mc2_gmm_dispatch(to_dev(send, "bf16"), to_dev(sc), to_dev(bad), to_dev(w1, "bf16"),
                         ep_rank=0, num_experts=E, h_out=h, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & mc2.MC2_DEVERR_COUNTS
    assert bool((h.float() == 3.0).all())


def _gpu_chain(d, ep_rank=0, rest=None):
    T, K, E, E_l = d["T"], d["K"], d["E"], d["E_l"]
    x = to_dev(d["x"], "bf16")
    sel = to_dev(d["sel"])
    err = _err()
    counts = mc2.mc2_moe_histc(sel, E, dev_err=err)
    perm, sidx, uidx, offs = mc2.mc2_moe_permute(x, sel, E, dev_err=err)
    recv = counts[ep_rank * E_l:(ep_rank + 1) * E_l].contiguous()
    h = mc2.mc2_gmm_dispatch(perm, counts, recv, to_dev(d["w1"], "bf16"), ep_rank=ep_rank,
                             num_experts=E, dev_err=err)
    buf = (torch.zeros((T * K, d["H"]), dtype=torch.bfloat16, device="cuda") if rest is None
           else to_dev(rest, "bf16"))
    mc2.mc2_gmm_combine(h, recv, counts, to_dev(d["w2"], "bf16"), buf, ep_rank=ep_rank,
                        num_experts=E, dev_err=err)
    out = mc2.mc2_moe_unpermute(buf, uidx, to_dev(d["probs"]), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    return {"counts": counts, "perm": perm, "sidx": sidx, "uidx": uidx, "h": h, "buf": buf,
            "out": out}


@pytest.mark.parametrize("standins", [False, True])
def test_moe_chain_small(standins):
    d = _small(seed=45, T=900, H=256, E=32, K=4, E_l=8, I=128)
    d["w1"] = wl.encode_bf16(on.decode(d["w1"], "bf16").astype(np.float32) * 5)
    rest = wl.combine_standins(46, 900 * 4, 256, std=0.05) if standins else None
    g = _gpu_chain(d, rest=rest)
    r = om.moe_local(d["x"], d["sel"], d["probs"], d["w1"], d["w2"], num_experts=32, ep_rank=0,
                     local_experts=8,
                     combine_rest=None if rest is None else on.decode(rest, "bf16"))
    np.testing.assert_array_equal(g["counts"].cpu().numpy(), r["counts"])
    np.testing.assert_array_equal(g["uidx"].cpu().numpy(), r["permute"]["unpermute_idx"])
    nloc = int(r["counts"][:8].sum())
    assert_tol(to_f64(g["h"])[:nloc], r["h"], "fc1+swiglu")
    assert_tol(to_f64(g["buf"]), r["y_full"], "fc2 combine buffer")
    assert_tol(to_f64(g["out"]), r["out"], "unpermute out")
