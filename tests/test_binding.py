"""The Python binding rejects tensors whose shape or dtype does not match what
the kernels index, before anything reaches the library (the C ABI sees only
pointers and sizes). These run on the CPU: metadata is checked before the
device, so CPU tensors with a wrong shape fail on the shape, and CPU tensors
with every shape right fail only on the device check."""
import pytest
import torch

from gemm_collective_core_amd import mc2

bf, f16, i8, i32, f32 = torch.bfloat16, torch.float16, torch.int8, torch.int32, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


ON_GPU = "must be on the GPU"


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_mm_rs_local_checks():
    x1, x2 = z(256, 512), z(512, 64)
    _raises(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0), ON_GPU)
    _raises(lambda: mc2.mc2_mm_rs_local(x1, z(512, 64, dtype=f16), 2, 0), "x2 must be")
    _raises(lambda: mc2.mc2_mm_rs_local(x1, z(500, 64), 2, 0), "k mismatch")
    _raises(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0, bias=z(63)), "bias must have shape")
    _raises(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0, bias=z(64, dtype=f16)), "bias must be")
    _raises(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0, out=z(256, 65)), "out must have shape")
    _raises(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0, out=z(256, 64, dtype=f16)), "out must be")
    q1, q2 = z(256, 512, dtype=i8), z(512, 64, dtype=i8)
    _raises(lambda: mc2.mc2_mm_rs_local(q1, q2, 2, 0, x1_scale=z(255, dtype=f32),
                                        x2_scale=z(64, dtype=f32)), "x1_scale must hold 256")
    _raises(lambda: mc2.mc2_mm_rs_local(q1, q2, 2, 0, x1_scale=z(256, dtype=f32),
                                        x2_scale=z(64)), "x2_scale must be")
    _raises(lambda: mc2.mc2_mm_rs_local(q1, q2, 2, 0, x1_scale=z(256, dtype=f32),
                                        x2_scale=z(64, dtype=f32), bias=z(64, dtype=f16)),
            "bias must be")
    _raises(lambda: mc2.mc2_mm_rs_local(q1, q2, 2, 0, x1_scale=z(256, dtype=f32),
                                        x2_scale=z(64, dtype=f32)), ON_GPU)


def test_ag_mm_local_checks():
    x, w = z(8 * 16, 512), z(64, 512)
    _raises(lambda: mc2.mc2_ag_mm_local(x, w, 8, 0, x2_trans=True), ON_GPU)
    _raises(lambda: mc2.mc2_ag_mm_local(x, w, 8, 0), "k mismatch")
    _raises(lambda: mc2.mc2_ag_mm_local(x, z(64, 512, dtype=f16), 8, 0, x2_trans=True), "x2 must be")
    _raises(lambda: mc2.mc2_ag_mm_local(x, w, 8, 0, x2_trans=True, out=z(128, 32)),
            "out must have shape")
    _raises(lambda: mc2.mc2_ag_mm_local(x, w, 8, 0, x2_trans=True, out=z(128, 64, dtype=f16)),
            "out must be")
    _raises(lambda: mc2.mc2_ag_mm_local(x, w, 8, 0, x2_trans=True, bias=z(128)),
            "bias must have shape")
    _raises(lambda: mc2.mc2_ag_mm_local(z(128, 512, dtype=i8), w, 8, 0, x2_trans=True),
            "x_gathered must be one of")
    inf = z(8, dtype=i32)
    _raises(lambda: mc2.mc2_ag_mm_local_inflags(x, w, 8, 0, inf, 1, x2_trans=True,
                                                out=z(128, 63)), "out must have shape")
    _raises(lambda: mc2.mc2_ag_mm_local_inflags(x, w, 8, 0, inf, 1, x2_trans=True,
                                                dev_err=z(1, dtype=f32)), "dev_err must be")


def test_mm_ar_and_ar_sum_checks():
    x1, x2 = z(4, 100, 512), z(4, 512, 64)
    _raises(lambda: mc2.mc2_mm_ar_local(x1, x2, 4, out=z(100, 63)), "out must have shape")
    _raises(lambda: mc2.mc2_mm_ar_local(x1, z(4, 512, 64, dtype=f16), 4), "x2 must be")
    _raises(lambda: mc2.mc2_mm_ar_local(x1, x2, 4, bias=z(65)), "bias must have shape")
    _raises(lambda: mc2.mc2_mm_ar_local(x1, x2, 4, workspace=z(64, dtype=f32)),
            "workspace must be")
    _raises(lambda: mc2.mc2_ar_sum_local(z(4, 64), 1, out=z(63)), "out must have shape")
    _raises(lambda: mc2.mc2_ar_sum_local(z(4, 64, dtype=f32), 1), "partials must be one of")


def test_moe_histc_permute_unpermute_checks():
    T, K, E, H = 10, 4, 16, 64
    x, sel = z(T, H), z(T, K, dtype=i32)
    _raises(lambda: mc2.mc2_moe_histc(sel, E, counts=z(E - 1, dtype=i32)), "counts must hold")
    _raises(lambda: mc2.mc2_moe_histc(z(T, K, dtype=torch.int64), E), "sel must be")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, permuted=z(T * K, H + 8)),
            "permuted must have shape")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, permuted=z(T * K, H, dtype=f16)),
            "permuted must be")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, sorted_idx=z(T * K - 1, dtype=i32)),
            "sorted_idx must hold")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, unpermute_idx=z(T * K, dtype=torch.int64)),
            "unpermute_idx must be")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, expert_offsets=z(E, dtype=i32)),
            "expert_offsets must hold")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E, workspace=z(64, dtype=f32)),
            "workspace must be")
    _raises(lambda: mc2.mc2_moe_permute(x, sel, E), ON_GPU)
    y, idx, probs = z(T * K, H), z(T * K, dtype=i32), z(T, K, dtype=f32)
    _raises(lambda: mc2.mc2_moe_unpermute(y, idx, probs), ON_GPU)
    _raises(lambda: mc2.mc2_moe_unpermute(y, idx, z(T, K)), "probs must be")
    _raises(lambda: mc2.mc2_moe_unpermute(y, z(T * K - 1, dtype=i32), probs),
            "unpermute_idx must hold")
    _raises(lambda: mc2.mc2_moe_unpermute(y, idx, probs, out=z(T, H - 8)), "out must have shape")
    _raises(lambda: mc2.mc2_moe_unpermute(z(T * K, H, dtype=f16), idx, probs), "y_full must be")


def test_moe_noalloc_permute_checks():
    T, K, E, H = 10, 4, 16, 64
    x, sel = z(T, H), z(T, K, dtype=i32)
    outs = dict(permuted=z(T * K, H), sorted_idx=z(T * K, dtype=i32),
                unpermute_idx=z(T * K, dtype=i32), expert_offsets=z(E + 1, dtype=i32))
    _raises(lambda: mc2.mc2_moe_permute_noalloc(x, sel, E, **outs), ON_GPU)
    bad = dict(outs, expert_offsets=z(E, dtype=i32))
    _raises(lambda: mc2.mc2_moe_permute_noalloc(x, sel, E, **bad), "expert_offsets must hold")
    bad = dict(outs, permuted=None)
    _raises(lambda: mc2.mc2_moe_permute_noalloc(x, sel, E, **bad), "every output")


def test_gmm_checks():
    E, El, H, I = 16, 4, 64, 32
    sc, rc = z(E, dtype=i32), z(El, dtype=i32)
    send, w1, w2 = z(100, H), z(El, H, 2 * I), z(El, I, H)
    kw = dict(ep_rank=0, num_experts=E)
    _raises(lambda: mc2.mc2_gmm_dispatch(send, sc, rc, w1, **kw), ON_GPU)
    _raises(lambda: mc2.mc2_gmm_dispatch(send, z(E - 1, dtype=i32), rc, w1, **kw),
            "send_counts must hold")
    _raises(lambda: mc2.mc2_gmm_dispatch(send, sc, z(El, dtype=torch.int64), w1, **kw),
            "recv_counts must be")
    _raises(lambda: mc2.mc2_gmm_dispatch(z(100, H + 8), sc, rc, w1, **kw), "send_buf must have")
    _raises(lambda: mc2.mc2_gmm_dispatch(send, sc, rc, w1, h_out=z(100, 2 * I), **kw),
            "h_out must have shape")
    _raises(lambda: mc2.mc2_gmm_dispatch(send, sc, rc, z(El, H, 2 * I, dtype=f16), **kw),
            "w1 must be")
    h, buf = z(100, I), z(100, H)
    _raises(lambda: mc2.mc2_gmm_combine(h, rc, sc, w2, buf, **kw), ON_GPU)
    _raises(lambda: mc2.mc2_gmm_combine(z(100, I + 8), rc, sc, w2, buf, **kw), "h must have")
    _raises(lambda: mc2.mc2_gmm_combine(h, rc, sc, w2, z(100, H, dtype=f16), **kw),
            "combine_buf must be")


def test_gmm_backward_checks():
    E, El, H, I = 16, 4, 64, 32
    sc, rc = z(E, dtype=i32), z(El, dtype=i32)
    w1, w2 = z(El, H, 2 * I), z(El, I, H)
    dy, h, g = z(100, H), z(100, I), z(100, 2 * I)
    kw = dict(ep_rank=0, num_experts=E)
    _raises(lambda: mc2.mc2_gmm_combine_backward(dy, rc, sc, w2, h, **kw), ON_GPU)
    _raises(lambda: mc2.mc2_gmm_combine_backward(dy, rc, sc, w2, h, act=mc2.MC2_ACT_SWIGLU,
                                                 g_saved=z(100, I), **kw), "g_saved must have")
    _raises(lambda: mc2.mc2_gmm_combine_backward(dy, rc, sc, w2, h, dgrad_out=z(100, 2 * I),
                                                 **kw), "dgrad_out must have")
    _raises(lambda: mc2.mc2_gmm_combine_backward(dy, rc, sc, w2, h, dw2_out=z(El, I, H), **kw),
            "dw2_out must be")
    _raises(lambda: mc2.mc2_gmm_combine_backward(z(100, H - 8), rc, sc, w2, h, **kw),
            "dy_buf must have")
    dg, send, dx = z(100, 2 * I), z(100, H), z(100, H)
    _raises(lambda: mc2.mc2_gmm_dispatch_backward(dg, rc, sc, w1, send, dx, **kw), ON_GPU)
    _raises(lambda: mc2.mc2_gmm_dispatch_backward(z(100, I), rc, sc, w1, send, dx, **kw),
            "dg must have")
    _raises(lambda: mc2.mc2_gmm_dispatch_backward(dg, rc, sc, w1, send, z(100, H + 8), **kw),
            "dx_buf must have")
    _raises(lambda: mc2.mc2_gmm_dispatch_backward(dg, rc, sc, w1, send, dx,
                                                  dw1_out=z(El, H, I, dtype=f32), **kw),
            "dw1_out must have")
