"""Oracle for the rank-chunked GEMM: MatmulReduceScatter and AllGatherMatmul.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module. It shares no code with the HIP path.

Sources (page title, section):

* ``torch_npu.npu_mm_reduce_scatter_base`` API doc, "功能说明" (function
  description): the basic formula (garbled on the page; read as
  ``output = reducescatter(x1 @ x2 + bias)``) and the quantized formula
  ``output = reducescatter((x1_scale * x2_scale) * (x1 @ x2 + bias))``.
* same page, "参数说明" (arguments): x1 (m, k), x2 (k, n) or transposed,
  m divisible by world_size, bias of size n, x1_scale (m, 1) per token,
  x2_scale (1, n) per channel, output_dtype bf16 (default) or fp16.
* same page, "返回值说明" (return value): the output dtype follows the input in
  the basic case and ``output_dtype`` in the quantized case.
* CANN hccl issue 158: ``npu_all_gather_base_mm(x1, x2, hcom, world_size)``
  computes ``allgather(x1) @ x2``.
* "NPU Training Operators - MC2", "底层 API 对照" and the MindSpeed-LLM
  description it quotes: ``npu_mm_all_reduce_base`` fuses the TP matmul with
  all_reduce, every rank ending with the sum of the W partials; same page,
  "风险": MC2 may cost precision on some models. The mc2_all_reduce article
  ("先搞懂AllReduce为什么慢"): ``full_out = all_reduce(x @ weights_shard)``.

Arithmetic is float64; the int8 products are integers whose partial sums stay
below 2**53 for every k the API accepts (k < 65535, |value| <= 127), so the
float64 matmul gives the exact integer result. The output is rounded once.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode, round_to

MAX_EXACT = 2.0 ** 53


def chunk_rows(m: int, world_size: int, c: int) -> slice:
    """Rows of destination chunk ``c``: the reduce-scatter hands rank c the
    c-th of ``world_size`` equal row blocks of the (m, n) result."""
    if m % world_size:
        raise ValueError("m must be divisible by world_size")
    mc = m // world_size
    return slice(c * mc, (c + 1) * mc)


def chunk_order(world_size: int, rank: int, kind: str) -> list[int]:
    """Order in which a rank computes its chunks.

    AllGatherMatmul starts with its own chunk (the only chunk it has before any
    data arrives) and walks (rank + i) mod W. MatmulReduceScatter walks
    (rank + 1 + i) mod W so that its own chunk, which it keeps, comes last and
    the first finished chunk can be sent at once. Values do not depend on it.
    """
    if kind == "ag":
        return [(rank + i) % world_size for i in range(world_size)]
    if kind == "rs":
        return [(rank + 1 + i) % world_size for i in range(world_size)]
    raise ValueError(kind)


def sub_chunk_rows(m: int, world_size: int, c: int, comm_turn: int, j: int) -> slice:
    """Rows of piece ``j`` of destination chunk ``c`` when the chunk is split
    ``comm_turn`` ways ([RS] "参数说明": comm_turn is the split granularity of
    the exchange between ranks, 0 meaning the default split).

    0 (the default) and 1 keep the chunk whole. s > 1 cuts its m_c rows into s
    contiguous pieces in row order whose sizes differ by at most one, the
    longer ones first: q = m_c // s rows each, plus one for the first m_c % s
    pieces. Every piece must be non-empty, so s <= m_c.
    """
    rows = chunk_rows(m, world_size, c)
    s = max(comm_turn, 1)
    mc = rows.stop - rows.start
    if s > mc:
        raise ValueError("more pieces than rows in a chunk")
    if not 0 <= j < s:
        raise ValueError("piece index out of range")
    q, r = divmod(mc, s)
    start = rows.start + j * q + min(j, r)
    return slice(start, start + q + (1 if j < r else 0))


def segment_order(world_size: int, rank: int, kind: str, comm_turn: int) -> list[tuple[int, int]]:
    """Order of the (chunk, piece) segments: the chunks in ``chunk_order``, the
    pieces of each chunk in row order. Segment (c, j) owns ready flag
    c * max(comm_turn, 1) + j."""
    s = max(comm_turn, 1)
    return [(c, j) for c in chunk_order(world_size, rank, kind) for j in range(s)]


def _stack(a, nsim):
    a = np.asarray(a)
    return a[None] if (nsim == 1 and a.ndim == 2) else a


def mm_rs(x1, x2, *, world_size, in_dtype, nsim=1, x2_trans=False, bias=None,
          bias_dtype=None, x1_scale=None, x2_scale=None, out_dtype=None,
          rows=None, cols=None):
    """MatmulReduceScatter, as the (m, n) matrix of all W destination chunks.

    ``nsim`` stacked operands x1 (nsim, m, k), x2 (nsim, k, n) stand for the
    partials of ``nsim`` ranks; the reduce-scatter sums them, so

    * basic:  P = sum_w (x1_w @ x2_w + bias)
    * quant:  P = sum_w (x1_scale_w[i] * x2_scale_w[j]) * (x1_w @ x2_w + bias)

    and chunk c of the result is ``P[chunk_rows(m, W, c)]``. The literal
    formula adds the bias inside each partial. ``out_dtype`` "bf16"/"f16"
    rounds once; "f32" returns the unrounded value; "i32" (int8 without scales
    only) returns the exact integer accumulator. ``rows``/``cols`` restrict the
    computation to those output rows and columns.
    """
    A = _stack(x1, nsim)
    B = _stack(x2, nsim)
    if A.shape[0] != nsim or B.shape[0] != nsim:
        raise ValueError("stacked operands must have nsim leading entries")
    m = A.shape[1]
    if m % world_size:
        raise ValueError("m must be divisible by world_size")
    quant = in_dtype == "i8"
    if out_dtype is None:
        out_dtype = "bf16" if quant else in_dtype
    if rows is not None:
        A = A[:, rows, :]
    if x2_trans:
        B = np.swapaxes(B, 1, 2)  # (nsim, k, n) view of the (n, k) storage
    if cols is not None:
        B = B[:, :, cols]
    Af = decode(A, in_dtype)
    Bf = decode(B, in_dtype)
    if Af.shape[2] != Bf.shape[1]:
        raise ValueError("k mismatch")
    k = Af.shape[2]
    bvec = None
    if bias is not None:
        bvec = decode(bias, bias_dtype or ("bf16" if quant else in_dtype))
        if cols is not None:
            bvec = bvec[cols]
    if quant:
        if k * 127 * 127 >= MAX_EXACT:
            raise ValueError("int8 accumulator would not be exact in float64")
        accs = [Af[w] @ Bf[w] for w in range(nsim)]
        if out_dtype == "i32":
            if nsim != 1 or bias is not None:
                raise ValueError("raw accumulator output is for one partial without bias")
            return accs[0].astype(np.int64)
        s1 = np.asarray(x1_scale, dtype=np.float32).reshape(nsim, -1).astype(np.float64)
        s2 = np.asarray(x2_scale, dtype=np.float32).reshape(nsim, -1).astype(np.float64)
        if rows is not None:
            s1 = s1[:, rows]
        if cols is not None:
            s2 = s2[:, cols]
        P = np.zeros_like(accs[0])
        for w in range(nsim):
            inner = accs[w] + (bvec[None, :] if bvec is not None else 0.0)
            P += (s1[w][:, None] * s2[w][None, :]) * inner
    else:
        P = np.zeros((Af.shape[1], Bf.shape[2]))
        for w in range(nsim):
            P += Af[w] @ Bf[w] + (bvec[None, :] if bvec is not None else 0.0)
    return round_to(P, out_dtype)


def ag_mm(x_gathered, x2, *, world_size, in_dtype, x2_trans=False, bias=None,
          rows=None, cols=None):
    """AllGatherMatmul local share: ``allgather(x1) @ x2 (+ bias)``.

    ``x_gathered`` (W * m_c, k) holds the W gathered chunks in rank order;
    output chunk c (rows of rank c's input) is ``out[chunk_rows(...)]``. The
    result has the input dtype.
    """
    X = np.asarray(x_gathered)
    if X.shape[0] % world_size:
        raise ValueError("gathered rows must be W * m_c")
    if rows is not None:
        X = X[rows]
    B = np.asarray(x2)
    if x2_trans:
        B = B.T
    if cols is not None:
        B = B[:, cols]
    P = decode(X, in_dtype) @ decode(B, in_dtype)
    if bias is not None:
        bv = decode(bias, in_dtype)
        P = P + (bv[cols] if cols is not None else bv)[None, :]
    return round_to(P, in_dtype)


AR_ONE_ROUNDING, AR_RANK_ROUNDED, AR_HOP_ROUNDED = 0, 1, 2


def ar_sum(partials, *, dtype, rounding):
    """The all-reduce sum of W partials already in ``dtype`` storage, (W, ...)
    -> (...), rounded to ``dtype``.

    * AR_RANK_ROUNDED: the W stored partials summed exactly (float64, rank
      order) and rounded once;
    * AR_HOP_ROUNDED: a running sum rounded to ``dtype`` after every addition,
      in rank order: s = p_0, s = round(s + p_w) for w = 1 .. W-1 (a ring
      reduction carried out in the storage dtype).
    """
    P = decode(np.asarray(partials), dtype)
    if rounding == AR_RANK_ROUNDED:
        s = np.zeros(P.shape[1:])
        for w in range(P.shape[0]):
            s = s + P[w]
        return round_to(s, dtype)
    if rounding == AR_HOP_ROUNDED:
        s = P[0].copy()
        for w in range(1, P.shape[0]):
            s = round_to(s + P[w], dtype)
        return s
    raise ValueError(rounding)


def mm_ar(x1, x2, *, world_size, in_dtype, x2_trans=False, bias=None, rounding=AR_ONE_ROUNDING,
          rows=None, cols=None):
    """MatmulAllReduce local share: every rank ends with the full (m, n)
    ``P = sum_w (x1_w @ x2_w + bias)`` of the W partials, x1 (W, m, k) and x2
    (W, k, n) (or (W, n, k) with ``x2_trans``) stacked as in ``mm_rs``.

    * AR_ONE_ROUNDING: the sum rounded once (one accumulator over all W
      partials, as the fused kernel keeps it);
    * AR_RANK_ROUNDED / AR_HOP_ROUNDED: each rank's partial is first rounded to
      ``in_dtype`` (what a rank sends), then combined by ``ar_sum``.
    """
    # every rank keeps all rows: no row chunking (world_size only counts partials)
    if rounding == AR_ONE_ROUNDING:
        return mm_rs(x1, x2, world_size=1, in_dtype=in_dtype, nsim=world_size,
                     x2_trans=x2_trans, bias=bias, rows=rows, cols=cols)
    parts = [mm_rs(np.asarray(x1)[w], np.asarray(x2)[w], world_size=1, in_dtype=in_dtype,
                   x2_trans=x2_trans, bias=bias, rows=rows, cols=cols)
             for w in range(world_size)]
    # round_to returns float64 values on the dtype's grid; ar_sum reads storage
    stored = np.stack(parts)
    if in_dtype == "bf16":
        stored = (stored.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        stored = stored.astype(np.float16)
    return ar_sum(stored, dtype=in_dtype, rounding=rounding)
