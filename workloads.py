"""Seeded synthetic inputs for the MC2 compute core.

This module is the single source of inputs for both the HIP path and the CPU
oracle. It draws random numbers and encodes them into the storage formats the
kernels read (bf16 as uint16 bit patterns, fp16, int8, fp32, int32). It holds
none of the arithmetic of the operators themselves: no matmul, no chunking, no
counting, no permutation.

The workloads follow the shapes of the operators described in the pages:

* ``torch_npu.npu_mm_reduce_scatter_base`` API doc, "调用示例" (single-op
  example): x1 (128, 512) and x2 (512, 64) in fp16, values ``torch.randn``.
* CANN hccl issue 158 (AllGather vs AllGather+MatMul latency on Atlas A2): the
  all-gather matmul with hidden size 3072.
* "NPU Training Operators - MC2", section "执行路径" (execution path): the MoE
  expert-parallel dispatch/combine with router outputs ``selected_experts``
  and ``routing_weights``.

Every draw uses ``numpy.random.default_rng(seed)`` in the order documented on
each function. Floating-point values are drawn in float32 and then encoded with
round-to-nearest-even into the storage dtype.
"""
from __future__ import annotations

import numpy as np

# Storage dtype names shared by tests and bench.
BF16 = "bf16"
F16 = "f16"
I8 = "i8"
F32 = "f32"
I32 = "i32"


def encode_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite draws, so NaN handling is not needed here.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 draws into the storage dtype."""
    if dtype == BF16:
        return encode_bf16(a)
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16)
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"cannot encode float draws as {dtype}")


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return encode(a, dtype)


def int8_uniform(rng, shape):
    """Symmetric uniform integers in [-127, 127] (the value -128 is never drawn)."""
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def scales_uniform(rng, shape, lo=1e-3, hi=1e-2):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


# --------------------------------------------------------------------------
# Dense chunked GEMM workloads
# --------------------------------------------------------------------------

def gemm_inputs(seed, m, k, n, dtype, *, std=1.0, nsim=1, x2_trans=False,
                bias=False, quant=False):
    """Generic chunked-GEMM inputs.

    Draw order: for w in range(nsim): x1_w (m, k), then x2_w ((k, n), or
    (n, k) when ``x2_trans``); then bias (n) if requested; then x1_scale
    (nsim, m) and x2_scale (nsim, n) when ``quant``.

    Returns a dict with x1 of shape (nsim, m, k) (or (m, k) when nsim == 1),
    x2 stacked the same way, and optional bias / x1_scale / x2_scale.
    """
    rng = np.random.default_rng(seed)
    x1s, x2s = [], []
    for _ in range(nsim):
        if dtype == I8:
            x1s.append(int8_uniform(rng, (m, k)))
            x2s.append(int8_uniform(rng, (n, k) if x2_trans else (k, n)))
        else:
            x1s.append(_normal(rng, (m, k), std, dtype))
            x2s.append(_normal(rng, (n, k) if x2_trans else (k, n), std, dtype))
    out = {
        "x1": np.stack(x1s) if nsim > 1 else x1s[0],
        "x2": np.stack(x2s) if nsim > 1 else x2s[0],
        "dtype": dtype, "m": m, "k": k, "n": n, "nsim": nsim,
        "x2_trans": x2_trans,
    }
    if bias:
        bdt = BF16 if dtype == I8 else dtype
        out["bias"] = _normal(rng, (n,), std, bdt)
        out["bias_dtype"] = bdt
    if quant:
        s1 = scales_uniform(rng, (nsim, m))
        s2 = scales_uniform(rng, (nsim, n))
        out["x1_scale"] = s1 if nsim > 1 else s1[0]
        out["x2_scale"] = s2 if nsim > 1 else s2[0]
    return out


def c1_inputs(seed=1001):
    """Simulated W=2 MatmulReduceScatter, fp16: per rank x1 (128,512) and
    x2 (512,64), N(0,1), no bias. Draws: x1_0, x2_0, x1_1, x2_1."""
    return gemm_inputs(seed, 128, 512, 64, F16, std=1.0, nsim=2)


def c2_inputs(seed=1002, m_c=1024, world_size=8, k=3072, n=3072):
    """AllGatherMatmul local share, bf16: gathered x (W*m_c, k) then weight
    (k, n), both N(0, 0.02) (0.02 read as the standard deviation)."""
    return gemm_inputs(seed, world_size * m_c, k, n, BF16, std=0.02)


def c3_inputs(seed=1003, m=4096, k=8192, n=2048):
    """Quantized MatmulReduceScatter local GEMM, int8: x1 (m,k), x2 (k,n)
    uniform in [-127,127]; then x1_scale (m) and x2_scale (n) uniform in
    [1e-3, 1e-2]."""
    return gemm_inputs(seed, m, k, n, I8, quant=True)


def c5a_inputs(seed=1005, m_c=2048, world_size=8, k=8192, n=3584):
    """Large AllGatherMatmul local share: x (W*m_c, k), weight (k, n),
    N(0, 0.02), bf16. Drawn first from seed 1005."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (world_size * m_c, k), 0.02, BF16)
    w = _normal(rng, (k, n), 0.02, BF16)
    return {"x1": x, "x2": w, "dtype": BF16, "m": world_size * m_c, "k": k,
            "n": n, "nsim": 1, "x2_trans": False}, rng


def c5_inputs(seed=1005, m=16384, k_a=8192, n_a=3584, world_size=8,
              k_b=1024, n_b=8192):
    """Config 5: (a) the large AllGatherMatmul share, then (b) a simulated
    W=8 MatmulReduceScatter with x1 stacked (W, m, k_b) and x2 stacked
    (W, k_b, n_b), all N(0, 0.02), bf16, from one generator in that order."""
    a, rng = c5a_inputs(seed, m // world_size, world_size, k_a, n_a)
    x1 = _normal(rng, (world_size, m, k_b), 0.02, BF16)
    x2 = _normal(rng, (world_size, k_b, n_b), 0.02, BF16)
    b = {"x1": x1, "x2": x2, "dtype": BF16, "m": m, "k": k_b, "n": n_b,
         "nsim": world_size, "x2_trans": False}
    return a, b


def x2_as_nk(d):
    """The same GEMM inputs with x2 held as (n, k) (stacked (nsim, n, k)) and
    flagged x2_trans: the layout of a Linear weight that is passed to the
    operator transposed. Same values, only the storage order changes."""
    out = dict(d)
    x2 = np.asarray(d["x2"])
    out["x2"] = np.ascontiguousarray(np.swapaxes(x2, -1, -2))
    out["x2_trans"] = True
    return out


# --------------------------------------------------------------------------
# MoE expert-parallel workloads
# --------------------------------------------------------------------------

def router(logits: np.ndarray, expert_bias: np.ndarray, topk: int):
    """Synthetic router that produces the method's inputs.

    z = logits + expert_bias, p = softmax(z) over experts in float64, the
    top-k experts by p (ties go to the lower expert id), and the selected p
    values as routing weights (not renormalised), stored as float32.
    The router itself is outside the operators; it only shapes the ids.
    """
    z = logits.astype(np.float64) + expert_bias.astype(np.float64)[None, :]
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    sel = order.astype(np.int32)
    probs = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return np.ascontiguousarray(sel), np.ascontiguousarray(probs)


def expert_ids(seed, n, num_experts):
    """n expert ids, int32, drawn independently from a skewed distribution:
    p(e) proportional to exp(b_e) with b N(0, 0.5) (the router's expert bias
    without the per-token logits). Draw order: b (E), then the n ids."""
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(size=(num_experts,)) * 0.5
    p = np.exp(b - b.max())
    p /= p.sum()
    return rng.choice(num_experts, size=n, p=p).astype(np.int32)


def moe_inputs(seed=1004, tokens=32768, hidden=2048, num_experts=128, topk=8,
               local_experts=16, inter=768, x_std=1.0, w_std=0.02):
    """MoE EP local share, bf16.

    Draw order: logits (T, E) N(0,1); expert bias (E) N(0, 0.5); x (T, H)
    N(0, x_std); fc1 weight (E_l, H, 2I) N(0, w_std); fc2 weight (E_l, I, H)
    N(0, w_std). Router as in :func:`router`.
    """
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(size=(tokens, num_experts), dtype=np.float32)
    ebias = rng.standard_normal(size=(num_experts,), dtype=np.float32) * np.float32(0.5)
    sel, probs = router(logits, ebias, topk)
    x = _normal(rng, (tokens, hidden), x_std, BF16)
    w1 = _normal(rng, (local_experts, hidden, 2 * inter), w_std, BF16)
    w2 = _normal(rng, (local_experts, inter, hidden), w_std, BF16)
    return {"sel": sel, "probs": probs, "x": x, "w1": w1, "w2": w2,
            "T": tokens, "H": hidden, "E": num_experts, "K": topk,
            "E_l": local_experts, "I": inter}


def c4_inputs(seed=1004):
    """MoE EP local share: 32768 tokens, H=2048, top-8 of 128 experts, local
    experts 0-15, fc1 (16,2048,1536), fc2 (16,768,2048)."""
    return moe_inputs(seed)


def moe_backward_inputs(seed, rows, hidden, inter, std=1.0):
    """Stand-ins for the tensors the backward of the MoE local path reads,
    for `rows` local rows, bf16, all N(0, std). Draw order: dy (rows, H), the
    output gradient in the combine buffer's rows; g (rows, 2I), the stored fc1
    pre-activation; h (rows, I), the stored fc2 input; dg (rows, 2I), the fc1
    output gradient; send (rows, H), the send-buffer rows of the local
    experts."""
    rng = np.random.default_rng(seed)
    return {"dy": _normal(rng, (rows, hidden), std, BF16),
            "g": _normal(rng, (rows, 2 * inter), std, BF16),
            "h": _normal(rng, (rows, inter), std, BF16),
            "dg": _normal(rng, (rows, 2 * inter), std, BF16),
            "send": _normal(rng, (rows, hidden), std, BF16)}


def combine_standins(seed, rows, hidden, std=0.05):
    """Stand-in rows for the part of the combine buffer that other ranks
    would return (N(0, 0.05), bf16)."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (rows, hidden), std, BF16)
