"""Oracle for the MoE expert-parallel local path (dispatch / combine pair).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module. It shares no code with the HIP path.

Source: "NPU Training Operators - MC2", section "执行路径" (execution path of
``ep_mc2_forward``): token counts by ``torch.histc(selected_experts, bins=E,
min=0, max=E)``; ``send_counts`` = local counts and ``recv_counts`` = the
columns of this rank's experts in the gathered counts; ``permute(hidden,
selected_experts)``; AllToAllv + GroupedMatmul(fc1); SwiGLU; GroupedMatmul(fc2)
+ AllToAllv with the counts swapped; ``unpermute(h, unpermute_indices,
probs=routing_weights)``. Section "迁移检查" (pre-migration checks): the local
expert range starts at ``ep_rank * num_local_experts`` and ids must lie in
[0, num_experts).

Readings where the page is silent (each listed with the design notes):

* ids outside [0, E) are invalid: counts ignore them, permute leaves them out
  (their unpermute index is -1) and unpermute skips them;
* the order inside one expert's segment is the flat slot order t*K + k
  (a stable sort), which fixes every index bit-exactly;
* ``gate_up_proj`` holds the gate in columns [0, I) and the up projection in
  columns [I, 2I); SwiGLU(g, u) = silu(g) * u with silu(g) = g / (1 + e^-g),
  applied to the unrounded fc1 product; the fc1 and fc2 outputs are stored as
  bf16;
* with a single source rank the received rows of local expert g are the send
  buffer's rows of expert ep_rank * E_l + g, and the combine writes its result
  back over those same rows.

Backward (same page, "PR 改动": the two autograd Functions wrap the fused
operator in forward and backward; "验证项": the fc1 / fc2 gradients are
compared against the plain alltoall path). The page gives no formulas; the
gradients are those of the forward above, with these readings:

* the combine's input gradient comes back in the combine buffer's layout (the
  rows the send buffer used), and the dispatch's input gradient goes out in
  the send buffer's layout, as the reverse AllToAllv would move them;
* SwiGLU's backward uses the fc1 pre-activation as the forward stored it
  (bf16) and the unrounded fc2 input gradient; the gradients handed between
  stages (fc2 input, fc1 output, fc1 input) are stored as bf16;
* weight gradients are kept in float (fp32 on the device) and not rounded to
  bf16.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode, round_to


def histc(sel, num_experts: int) -> np.ndarray:
    """counts[e] = number of (t, k) slots routed to expert e, 0 <= e < E."""
    flat = np.asarray(sel).reshape(-1)
    return np.array([np.count_nonzero(flat == e) for e in range(num_experts)],
                    dtype=np.int64)


def permute(x, sel, num_experts: int):
    """Sort the T*K routed slots by expert, stably.

    Returns ``permuted`` (rows of x in slot order, only the first n_valid rows
    defined, as the stored bit patterns), ``sorted_idx`` (T*K: the flat slot
    t*K+k at each position, -1 past n_valid), ``unpermute_idx`` (T*K: the
    position of each slot, -1 for invalid ids) and ``offsets`` (E+1: start of
    each expert's segment, offsets[E] = n_valid).
    """
    sel = np.asarray(sel)
    T, K = sel.shape
    flat = sel.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < num_experts)
    keys = np.where(valid, flat, num_experts)
    order = np.argsort(keys, kind="stable")
    n_valid = int(valid.sum())
    sorted_idx = np.full(T * K, -1, dtype=np.int64)
    sorted_idx[:n_valid] = order[:n_valid]
    unpermute_idx = np.full(T * K, -1, dtype=np.int64)
    unpermute_idx[order[:n_valid]] = np.arange(n_valid)
    counts = histc(sel, num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    x = np.asarray(x)
    permuted = x[order[:n_valid] // K]
    return {"permuted": permuted, "sorted_idx": sorted_idx,
            "unpermute_idx": unpermute_idx, "offsets": offsets,
            "n_valid": n_valid}


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu(a: np.ndarray) -> np.ndarray:
    """(rows, 2I) -> (rows, I): silu(gate) * up with gate = a[:, :I]."""
    inter = a.shape[1] // 2
    with np.errstate(over="ignore"):
        return silu(a[:, :inter]) * a[:, inter:]


def gmm(rows, group_sizes, weights, *, act="none", dtype="bf16"):
    """Grouped matmul: group g takes the next group_sizes[g] rows and
    multiplies them by weights[g] (K, N); with ``act='swiglu'`` SwiGLU is
    applied to the float64 product. Output rounded to ``dtype`` once."""
    R = decode(rows, dtype)
    Wt = decode(weights, dtype)
    sizes = [int(s) for s in group_sizes]
    n_out = Wt.shape[2] // 2 if act == "swiglu" else Wt.shape[2]
    out = np.zeros((sum(sizes), n_out))
    off = 0
    for g, cnt in enumerate(sizes):
        a = R[off:off + cnt] @ Wt[g]
        out[off:off + cnt] = swiglu(a) if act == "swiglu" else a
        off += cnt
    return round_to(out, dtype)


def local_slice(send_counts, ep_rank: int, local_experts: int):
    """Rows of the send buffer that hold this rank's experts."""
    sc = np.asarray(send_counts, dtype=np.int64)
    start = int(sc[:ep_rank * local_experts].sum())
    n = int(sc[ep_rank * local_experts:(ep_rank + 1) * local_experts].sum())
    return start, n


def check_counts(send_counts, recv_counts, ep_rank, local_experts):
    """With one source rank, recv_counts must equal the send counts of this
    rank's experts (the shape check of the validation table)."""
    sc = np.asarray(send_counts, dtype=np.int64)
    rc = np.asarray(recv_counts, dtype=np.int64)
    mine = sc[ep_rank * local_experts:(ep_rank + 1) * local_experts]
    if rc.shape != mine.shape or not np.array_equal(rc, mine):
        raise ValueError("recv_counts disagree with send_counts")


def dispatch(send_buf, send_counts, recv_counts, *, ep_rank, local_experts,
             w1, act="swiglu"):
    """GroupedMatmul (fc1) over the rows received for the local experts."""
    check_counts(send_counts, recv_counts, ep_rank, local_experts)
    start, n = local_slice(send_counts, ep_rank, local_experts)
    rows = np.asarray(send_buf)[start:start + n]
    return gmm(rows, recv_counts, w1, act=act)


def combine(h_values, recv_counts, send_counts, *, ep_rank, local_experts, w2,
            combine_buf):
    """GroupedMatmul (fc2); the result goes back over this rank's rows of the
    combine buffer (float64 values). ``h_values`` are the bf16 fc1 outputs."""
    check_counts(send_counts, recv_counts, ep_rank, local_experts)
    start, n = local_slice(send_counts, ep_rank, local_experts)
    Wt = decode(w2, "bf16")
    out = np.array(combine_buf, dtype=np.float64, copy=True)
    off = 0
    for g, cnt in enumerate(np.asarray(recv_counts, dtype=np.int64)):
        cnt = int(cnt)
        out[start + off:start + off + cnt] = round_to(h_values[off:off + cnt] @ Wt[g], "bf16")
        off += cnt
    return out


def unpermute(y_full, unpermute_idx, probs, T: int, K: int):
    """out[t] = sum over k of probs[t, k] * y_full[unpermute_idx[t*K + k]],
    slots with index -1 skipped; rounded to bf16."""
    Y = np.asarray(y_full, dtype=np.float64)
    idx = np.asarray(unpermute_idx, dtype=np.int64).reshape(T, K)
    P = np.asarray(probs, dtype=np.float32).astype(np.float64).reshape(T, K)
    out = np.zeros((T, Y.shape[1]))
    for k in range(K):
        ok = idx[:, k] >= 0
        out[ok] += P[ok, k][:, None] * Y[idx[ok, k]]
    return round_to(out, "bf16")


def expert_ffn_rows(x_rows, experts, w1, w2):
    """fc1 + SwiGLU and fc2 for single rows: row i goes through local expert
    experts[i]. Returns (h, y) as float64 values of the bf16 results."""
    X = decode(x_rows, "bf16")
    experts = [int(e) for e in experts]
    W1 = {e: decode(np.asarray(w1)[e], "bf16") for e in set(experts)}
    W2 = {e: decode(np.asarray(w2)[e], "bf16") for e in set(experts)}
    h = np.stack([round_to(swiglu((X[i] @ W1[e])[None, :])[0], "bf16")
                  for i, e in enumerate(experts)])
    y = np.stack([round_to(h[i] @ W2[e], "bf16") for i, e in enumerate(experts)])
    return h, y


def token_outputs(x, sel, probs, w1, w2, tokens, *, ep_rank, local_experts):
    """Unpermuted output of the given tokens when only this rank's experts
    contribute: out[t] = bf16(sum_k probs[t,k] * y(x[t], sel[t,k])) over the
    slots routed to a local expert, k ascending (y as in
    :func:`expert_ffn_rows`)."""
    sel = np.asarray(sel)
    x = np.asarray(x)
    first = ep_rank * local_experts
    rows, exps, owner, wts = [], [], [], []
    for i, t in enumerate(tokens):
        for k in range(sel.shape[1]):
            e = int(sel[t, k]) - first
            if 0 <= e < local_experts:
                rows.append(t)
                exps.append(e)
                owner.append(i)
                wts.append(float(np.float32(probs[t, k])))
    acc = np.zeros((len(tokens), x.shape[1]))
    if rows:
        _, y = expert_ffn_rows(x[rows], exps, w1, w2)
        for j in range(len(rows)):
            acc[owner[j]] += wts[j] * y[j]
    return round_to(acc, "bf16")


def moe_local(x, sel, probs, w1, w2, *, num_experts, ep_rank, local_experts,
              combine_rest=None):
    """The whole local path: histc -> permute -> fc1+SwiGLU -> fc2 ->
    unpermute. ``combine_rest`` holds the float64 values of the combine-buffer
    rows that other ranks would return (zeros when None)."""
    sel = np.asarray(sel)
    T, K = sel.shape
    counts = histc(sel, num_experts)
    p = permute(x, sel, num_experts)
    recv = counts[ep_rank * local_experts:(ep_rank + 1) * local_experts]
    h = dispatch(p["permuted"], counts, recv, ep_rank=ep_rank,
                 local_experts=local_experts, w1=w1, act="swiglu")
    H = np.asarray(x).shape[1]
    buf = np.zeros((T * K, H)) if combine_rest is None else np.asarray(combine_rest, dtype=np.float64)
    y_full = combine(h, recv, counts, ep_rank=ep_rank, local_experts=local_experts,
                     w2=w2, combine_buf=buf)
    out = unpermute(y_full, p["unpermute_idx"], probs, T, K)
    return {"counts": counts, "permute": p, "h": h, "y_full": y_full, "out": out}


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def swiglu_backward(a, dh):
    """Gradient of SwiGLU at the pre-activation ``a`` (rows, 2I), for the
    output gradient ``dh`` (rows, I): (rows, 2I) holding
    dh * up * silu'(gate) in the gate columns and dh * silu(gate) in the up
    columns, where silu'(g) = s * (1 + g * (1 - s)) with s = 1 / (1 + e^-g)."""
    a = np.asarray(a, dtype=np.float64)
    inter = a.shape[1] // 2
    gate, up = a[:, :inter], a[:, inter:]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-gate))
    return np.concatenate([dh * up * (s * (1.0 + gate * (1.0 - s))), dh * (gate * s)], axis=1)


def gmm_backward(rows, group_sizes, weights, dy):
    """Gradients of the grouped matmul Y_g = X_g @ W_g for the output gradient
    ``dy``: dX_g = dY_g @ W_g^T and dW_g = X_g^T @ dY_g, group after group,
    in float64 (unrounded). ``rows``, ``weights`` and ``dy`` are float64
    values. Returns (dX (rows, K), dW (G, K, N))."""
    X = np.asarray(rows, dtype=np.float64)
    Wt = np.asarray(weights, dtype=np.float64)
    D = np.asarray(dy, dtype=np.float64)
    dX = np.zeros((X.shape[0], Wt.shape[1]))
    dW = np.zeros(Wt.shape)
    off = 0
    for g, cnt in enumerate(int(c) for c in group_sizes):
        dX[off:off + cnt] = D[off:off + cnt] @ Wt[g].T
        dW[g] = X[off:off + cnt].T @ D[off:off + cnt]
        off += cnt
    return dX, dW


def combine_backward(dy_buf, recv_counts, send_counts, *, ep_rank, local_experts, w2, h,
                     g_saved=None, act="none", dtype="bf16"):
    """Backward of the combine segment (GroupedMatmul fc2 -> AllToAllv).

    ``dy_buf`` holds the output gradient in the combine buffer's layout
    (bf16); this rank's rows are those ``combine`` wrote. ``h`` holds the fc2
    inputs (bf16, group after group from row 0). Returns (dgrad, dW2):
    dW2[g] = h_g^T @ dY_g (float64) and dgrad, the gradient of the fc2 input
    (act 'none') or, with act 'swiglu', of the fc1 pre-activation
    ``g_saved`` (bf16, rows x 2I) through SwiGLU. dgrad is rounded to
    ``dtype`` (None: unrounded)."""
    check_counts(send_counts, recv_counts, ep_rank, local_experts)
    start, n = local_slice(send_counts, ep_rank, local_experts)
    dY = decode(np.asarray(dy_buf)[start:start + n], "bf16")
    Hv = decode(np.asarray(h)[:n], "bf16")
    dA, dW2 = gmm_backward(Hv, recv_counts, decode(w2, "bf16"), dY)
    if act == "swiglu":
        dA = swiglu_backward(decode(np.asarray(g_saved)[:n], "bf16"), dA)
    elif act != "none":
        raise ValueError(act)
    return (round_to(dA, dtype) if dtype else dA), dW2


def dispatch_backward(dg, recv_counts, send_counts, *, ep_rank, local_experts, w1, send_buf,
                      dx_buf, dtype="bf16"):
    """Backward of the dispatch segment (AllToAllv -> GroupedMatmul fc1).

    ``dg`` holds the gradient of the fc1 output (bf16, group after group from
    row 0). Returns (dx, dW1): dW1[g] = R_g^T @ dG_g (float64) over this
    rank's rows R of ``send_buf``, and dx, a float64 copy of ``dx_buf`` whose
    rows of this rank (the send buffer's) hold dG_g @ W1_g^T rounded to
    ``dtype`` (None: unrounded)."""
    check_counts(send_counts, recv_counts, ep_rank, local_experts)
    start, n = local_slice(send_counts, ep_rank, local_experts)
    R = decode(np.asarray(send_buf)[start:start + n], "bf16")
    dX, dW1 = gmm_backward(R, recv_counts, decode(w1, "bf16"), decode(np.asarray(dg)[:n], "bf16"))
    out = np.array(dx_buf, dtype=np.float64, copy=True)
    out[start:start + n] = round_to(dX, dtype) if dtype else dX
    return out, dW1
