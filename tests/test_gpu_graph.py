"""The MoE local chain and the chunked GEMM with ready flags, captured in a HIP
graph (torch.cuda.CUDAGraph) on the caller's stream. No entry point
allocates, synchronizes or records a memset, so every replay must give the
eager result bit for bit. Each replay is checked, with the program's own
eager work (new inputs copied in, buffers cleared) and a synchronization
between replays."""
import pytest
import torch

import workloads as wl
from gemm_collective_core_amd import mc2
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

T, H, E, K, E_L, I = 900, 256, 32, 4, 8, 128


def _capture(fn):
    """fn() captured into a graph after a warm-up call on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_moe_chain_graph_replays_bit_exact():
    seeds = (51, 52, 53)
    inputs = [wl.moe_inputs(seed=s, tokens=T, hidden=H, num_experts=E, topk=K,
                            local_experts=E_L, inter=I) for s in seeds]
    d0 = inputs[0]
    x = to_dev(d0["x"], "bf16")
    sel = to_dev(d0["sel"])
    probs = to_dev(d0["probs"])
    w1, w2 = to_dev(d0["w1"], "bf16"), to_dev(d0["w2"], "bf16")
    dev = x.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    recv = counts[:E_L]
    perm = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
    sidx = torch.empty(T * K, dtype=torch.int32, device=dev)
    uidx = torch.empty(T * K, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws = torch.empty(mc2.mc2_moe_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev)
    h = torch.empty((T * K, I), dtype=torch.bfloat16, device=dev)
    buf = torch.zeros((T * K, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def chain():
        mc2.mc2_moe_histc(sel, E, counts=counts, dev_err=err)
        mc2.mc2_moe_permute(x, sel, E, permuted=perm, sorted_idx=sidx, unpermute_idx=uidx,
                            expert_offsets=offs, workspace=ws, dev_err=err)
        mc2.mc2_gmm_dispatch(perm, counts, recv, w1, ep_rank=0, num_experts=E, h_out=h,
                             dev_err=err)
        mc2.mc2_gmm_combine(h, recv, counts, w2, buf, ep_rank=0, num_experts=E, dev_err=err)
        mc2.mc2_moe_unpermute(buf, uidx, probs, out=out, dev_err=err)

    def load(d):
        # eager work between runs: new routing, tokens and weights; the
        # combine buffer and the error word cleared
        sel.copy_(torch.from_numpy(d["sel"]))
        probs.copy_(torch.from_numpy(d["probs"]))
        x.copy_(to_dev(d["x"], "bf16"))
        w1.copy_(to_dev(d["w1"], "bf16"))
        w2.copy_(to_dev(d["w2"], "bf16"))
        buf.zero_()
        err.zero_()

    def snapshot():
        nloc = int(counts[:E_L].sum().item())
        return {"counts": counts.clone(), "offs": offs.clone(), "sidx": sidx.clone(),
                "uidx": uidx.clone(), "perm": perm[:int(offs[E].item())].clone(),
                "h": h[:nloc].clone(), "buf": buf.clone(), "out": out.clone()}

    eager = []
    for d in inputs:
        load(d)
        chain()
        torch.cuda.synchronize()
        assert err.item() == 0
        eager.append(snapshot())
    g = _capture(chain)
    # every seed twice, in an order that never repeats the previous inputs
    for i in (0, 1, 2, 1, 0, 2):
        load(inputs[i])
        g.replay()
        torch.cuda.synchronize()
        assert err.item() == 0, f"replay of seed {seeds[i]}"
        got = snapshot()
        for name, ref in eager[i].items():
            a, b = got[name], ref
            assert a.shape == b.shape, (name, seeds[i])
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                (name, seeds[i])


@pytest.mark.parametrize("op", ["mm_rs", "ag_mm"])
def test_chunked_gemm_with_flags_graph_replays(op):
    """The chunked GEMM with ready flags: each replay raises every flag to the
    captured epoch (cleared eagerly before it), leaves the counters at zero and
    writes the eager output bit for bit."""
    W = 4
    nsim = W if op == "mm_rs" else 1
    ds = [wl.gemm_inputs(s, W * 200, 776, 392, wl.BF16, std=1.0, nsim=nsim) for s in (61, 62)]
    x1 = to_dev(ds[0]["x1"], "bf16")
    x2 = to_dev(ds[0]["x2"], "bf16")
    m = W * 200
    out = torch.empty((m, 392), dtype=torch.bfloat16, device="cuda")
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, dtype=torch.int32, device="cuda")
    epoch = 11

    def run():
        if op == "mm_rs":
            mc2.mc2_mm_rs_local(x1, x2, W, 1, out=out, ready_flags=flags, flag_counters=cnt,
                                epoch=epoch)
        else:
            mc2.mc2_ag_mm_local(x1, x2, W, 1, out=out, ready_flags=flags, flag_counters=cnt,
                                epoch=epoch)

    def load(d):
        x1.copy_(to_dev(d["x1"], "bf16"))
        x2.copy_(to_dev(d["x2"], "bf16"))
        out.fill_(0)
        flags.zero_()

    eager = []
    for d in ds:
        load(d)
        run()
        torch.cuda.synchronize()
        eager.append(out.clone())
    g = _capture(run)
    for i in (0, 1, 0, 1):
        load(ds[i])
        g.replay()
        torch.cuda.synchronize()
        assert flags.cpu().tolist() == [epoch] * W
        assert cnt.cpu().tolist() == [0] * W
        assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), i
