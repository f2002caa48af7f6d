"""Thin Python binding over the C ABI of ``include/mc2.h``.

Every function has the name of the C entry point it calls and only marshals
arguments: it checks that tensors live on the GPU with the expected dtype and
layout, passes their data pointers and the current HIP stream, and raises
:class:`Mc2Error` on a nonzero status. All computation runs in the HIP
library; there is no other code path.
"""
from __future__ import annotations

import torch

from . import _lib

MC2_F16, MC2_BF16, MC2_I8, MC2_F32, MC2_I32 = 0, 1, 2, 3, 4
MC2_ACT_NONE, MC2_ACT_SWIGLU = 0, 1
MC2_AR_ONE_ROUNDING, MC2_AR_RANK_ROUNDED, MC2_AR_HOP_ROUNDED = 0, 1, 2
MC2_DEVERR_EXPERT_ID, MC2_DEVERR_COUNTS, MC2_DEVERR_INDEX, MC2_DEVERR_TIMEOUT = 1, 2, 4, 8

_CODES = {torch.float16: MC2_F16, torch.bfloat16: MC2_BF16, torch.int8: MC2_I8,
          torch.float32: MC2_F32, torch.int32: MC2_I32}
_TORCH = {v: k for k, v in _CODES.items()}


class Mc2Error(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.load().mc2_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise Mc2Error(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
    return next(t for t in ts if t is not None).device


def _want(t, name, *, shape=None, dtype=None, dtypes=None, numel=None):
    """Rejects a tensor whose metadata does not match what the kernel will
    index: the C library only sees pointers and sizes, so a wrong shape or
    dtype here would make a kernel read or write past the buffer. None
    passes (optional arguments)."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")


_FLOAT16 = (torch.float16, torch.bfloat16)
_ERR = dict(dtype=torch.int32, numel=1)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    return _CODES[dt]


def mc2_version() -> str:
    return _lib.load().mc2_version().decode()


MC2_SPLIT_PAIR = 0
MC2_SPLIT_ALONE = 1

# K-split workspaces handed out by the binding, one per (device, stream): the
# library leaves their control words zero after every call, and calls on one
# stream never overlap.
_split_ws = {}


def mc2_split_workspace_size() -> int:
    return int(_lib.load().mc2_split_workspace_size())


def mc2_set_split_policy(policy: int) -> None:
    _check("mc2_set_split_policy", _lib.load().mc2_set_split_policy(int(policy)))


def _split_workspace(dev, split, workspace):
    """(pointer, bytes) of the K-split workspace: the caller's, none
    (split=False), or the binding's own for this device and stream."""
    if not split:
        return None, 0
    if workspace is not None:
        _want(workspace, "workspace", dtype=torch.uint8)
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        return workspace.data_ptr(), workspace.numel()
    key = (dev.index, _stream(dev))
    ws = _split_ws.get(key)
    if ws is None:
        ws = torch.zeros(mc2_split_workspace_size(), dtype=torch.uint8, device=dev)
        _split_ws[key] = ws
    return ws.data_ptr(), ws.numel()


def _check_flags(world_size, comm_turn, ready_flags, flag_counters):
    """Flag arrays hold one uint32 per segment: world_size * max(comm_turn, 1).
    The counters live on the GPU; the ready flags on the GPU or in host-pinned
    memory (for a host-side consumer)."""
    segs = world_size * max(int(comm_turn), 1)
    for a in (ready_flags, flag_counters):
        if a is not None and (a.dtype not in (torch.int32, torch.uint32) or a.numel() < segs
                              or not a.is_contiguous()):
            raise ValueError(f"flag arrays must hold {segs} int32 (world_size * max(comm_turn, 1))")
    if flag_counters is not None and not flag_counters.is_cuda:
        raise ValueError("flag_counters must be on the GPU")
    if ready_flags is not None and not (ready_flags.is_cuda or ready_flags.is_pinned()):
        raise ValueError("ready_flags must be GPU or host-pinned memory")


def mc2_mm_rs_local(x1, x2, world_size, rank, *, x2_trans=False, bias=None, x1_scale=None,
                    x2_scale=None, out_dtype=None, out=None, ready_flags=None,
                    flag_counters=None, epoch=0, comm_turn=0, split=True, workspace=None):
    """MatmulReduceScatter compute share; x1 (m, k) or stacked (nsim, m, k),
    x2 (k, n) / (n, k) or stacked. Returns out (m, n). split=False runs a thin
    last round as half tiles instead of K halves; workspace: a uint8 GPU
    tensor for the K split (zeroed before its first use), else the binding's
    own for this stream."""
    if x1.dim() not in (2, 3):
        raise ValueError("x1 must be (m, k) or stacked (nsim, m, k)")
    _want(x1, "x1", dtypes=(torch.float16, torch.bfloat16, torch.int8))
    _want(x2, "x2", dtype=x1.dtype)
    nsim = 1 if x1.dim() == 2 else x1.shape[0]
    m, k = x1.shape[-2], x1.shape[-1]
    n = x2.shape[-2] if x2_trans else x2.shape[-1]
    if x2.dim() != x1.dim() or (x2.dim() == 3 and x2.shape[0] != nsim):
        raise ValueError("x1 and x2 must be stacked alike")
    if (x2.shape[-1] if x2_trans else x2.shape[-2]) != k:
        raise ValueError("k mismatch between x1 and x2")
    quant = x1.dtype == torch.int8
    _want(bias, "bias", shape=(n,), dtype=torch.bfloat16 if quant else x1.dtype)
    _want(x1_scale, "x1_scale", dtype=torch.float32, numel=m)
    _want(x2_scale, "x2_scale", dtype=torch.float32, numel=n)
    if out_dtype is None:
        out_dtype = torch.bfloat16 if quant else x1.dtype
    _want(out, "out", shape=(m, n), dtype=out_dtype)
    dev = _dev(x1, x2, bias, x1_scale, x2_scale, out, flag_counters)
    _check_flags(world_size, comm_turn, ready_flags, flag_counters)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    ws, ws_bytes = _split_workspace(dev, split, workspace)
    st = _lib.load().mc2_mm_rs_local(
        x1.data_ptr(), x2.data_ptr(), m, k, n, world_size, rank, nsim, int(bool(x2_trans)),
        _CODES[x1.dtype], _ptr(bias), _ptr(x1_scale), _ptr(x2_scale), _CODES[out_dtype],
        out.data_ptr(), _ptr(ready_flags), _ptr(flag_counters), epoch, comm_turn, ws, ws_bytes,
        _stream(dev))
    _check("mc2_mm_rs_local", st)
    return out


def _check_ag(x_gathered, x2, world_size, x2_trans, bias, out):
    """Shapes of an AllGatherMatmul call: returns (W * m_c, k, n)."""
    if x_gathered.dim() != 2 or x2.dim() != 2:
        raise ValueError("x_gathered and x2 must be matrices")
    _want(x_gathered, "x_gathered", dtypes=_FLOAT16)
    _want(x2, "x2", dtype=x_gathered.dtype)
    M, k = x_gathered.shape
    if M % world_size:
        raise ValueError("rows of x_gathered must be world_size * m_c")
    n = x2.shape[0] if x2_trans else x2.shape[1]
    if (x2.shape[1] if x2_trans else x2.shape[0]) != k:
        raise ValueError("k mismatch between x_gathered and x2")
    _want(bias, "bias", shape=(n,), dtype=x_gathered.dtype)
    _want(out, "out", shape=(M, n), dtype=x_gathered.dtype)
    return M, k, n


def mc2_ag_mm_local(x_gathered, x2, world_size, rank, *, x2_trans=False, bias=None, out=None,
                    ready_flags=None, flag_counters=None, epoch=0, comm_turn=0, split=True,
                    workspace=None):
    """AllGatherMatmul compute share; x_gathered (W*m_c, k). Returns out.
    split / workspace as for mc2_mm_rs_local."""
    M, k, n = _check_ag(x_gathered, x2, world_size, x2_trans, bias, out)
    dev = _dev(x_gathered, x2, bias, out, flag_counters)
    _check_flags(world_size, comm_turn, ready_flags, flag_counters)
    if out is None:
        out = torch.empty((M, n), dtype=x_gathered.dtype, device=dev)
    ws, ws_bytes = _split_workspace(dev, split, workspace)
    st = _lib.load().mc2_ag_mm_local(
        x_gathered.data_ptr(), x2.data_ptr(), M // world_size, k, n, world_size, rank,
        int(bool(x2_trans)), _CODES[x_gathered.dtype], _ptr(bias), out.data_ptr(),
        _ptr(ready_flags), _ptr(flag_counters), epoch, comm_turn, ws, ws_bytes, _stream(dev))
    _check("mc2_ag_mm_local", st)
    return out


def mc2_ag_mm_local_inflags(x_gathered, x2, world_size, rank, in_flags, in_epoch, *,
                            spin_limit=1 << 24, x2_trans=False, bias=None, out=None,
                            ready_flags=None, flag_counters=None, epoch=0, dev_err=None,
                            comm_turn=0, split=True, workspace=None):
    """mc2_ag_mm_local whose tiles wait until in_flags[g] == in_epoch before
    reading segment g of a gathered chunk other than the own one. in_flags:
    world_size * max(comm_turn, 1) int32 on the GPU or in host-pinned memory."""
    M, k, n = _check_ag(x_gathered, x2, world_size, x2_trans, bias, out)
    _want(dev_err, "dev_err", **_ERR)
    segs = world_size * max(int(comm_turn), 1)
    if in_flags.dtype not in (torch.int32, torch.uint32) or in_flags.numel() != segs:
        raise ValueError(f"in_flags must hold {segs} int32")
    _check_flags(world_size, comm_turn, ready_flags, flag_counters)
    if not in_flags.is_cuda and not in_flags.is_pinned():
        raise ValueError("in_flags must be GPU or host-pinned memory")
    dev = _dev(x_gathered, x2, bias, out, flag_counters, dev_err)
    if out is None:
        out = torch.empty((M, n), dtype=x_gathered.dtype, device=dev)
    ws, ws_bytes = _split_workspace(dev, split, workspace)
    st = _lib.load().mc2_ag_mm_local_inflags(
        x_gathered.data_ptr(), x2.data_ptr(), M // world_size, k, n, world_size, rank,
        int(bool(x2_trans)), _CODES[x_gathered.dtype], _ptr(bias), out.data_ptr(),
        _ptr(ready_flags), _ptr(flag_counters), epoch, comm_turn, in_flags.data_ptr(), in_epoch,
        spin_limit, _ptr(dev_err), ws, ws_bytes, _stream(dev))
    _check("mc2_ag_mm_local_inflags", st)
    return out


def mc2_mm_ar_workspace_size(m, n, world_size, in_dtype, rounding) -> int:
    code = _CODES[in_dtype] if isinstance(in_dtype, torch.dtype) else int(in_dtype)
    return int(_lib.load().mc2_mm_ar_workspace_size(m, n, world_size, code, rounding))


def mc2_mm_ar_local(x1, x2, world_size, *, rounding=MC2_AR_ONE_ROUNDING, x2_trans=False,
                    bias=None, out=None, workspace=None):
    """MatmulAllReduce local share: the full (m, n) sum of the W stacked
    partials x1 (W, m, k) @ x2 (W, k, n) (or (W, n, k) with x2_trans), combined
    under `rounding`. A workspace is allocated when the mode needs one and
    none is given."""
    if x1.dim() != 3 or x2.dim() != 3 or x1.shape[0] != world_size or x2.shape[0] != world_size:
        raise ValueError("x1 and x2 must be stacked (world_size, ., .)")
    _want(x1, "x1", dtypes=_FLOAT16)
    _want(x2, "x2", dtype=x1.dtype)
    _, m, k = x1.shape
    n = x2.shape[1] if x2_trans else x2.shape[2]
    if (x2.shape[2] if x2_trans else x2.shape[1]) != k:
        raise ValueError("k mismatch between x1 and x2")
    _want(bias, "bias", shape=(n,), dtype=x1.dtype)
    _want(out, "out", shape=(m, n), dtype=x1.dtype)
    _want(workspace, "workspace", dtype=torch.uint8)
    dev = _dev(x1, x2, bias, out, workspace)
    if out is None:
        out = torch.empty((m, n), dtype=x1.dtype, device=dev)
    need = mc2_mm_ar_workspace_size(m, n, world_size, x1.dtype, rounding)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().mc2_mm_ar_local(
        x1.data_ptr(), x2.data_ptr(), m, k, n, world_size, int(bool(x2_trans)), _CODES[x1.dtype],
        _ptr(bias), rounding, out.data_ptr(), _ptr(workspace), ws_bytes, _stream(dev))
    _check("mc2_mm_ar_local", st)
    return out


def mc2_ar_sum_local(partials, rounding, *, out=None):
    """The all-reduce combining step: partials (W, ...) -> out (...)."""
    _want(partials, "partials", dtypes=_FLOAT16)
    _want(out, "out", shape=partials.shape[1:], dtype=partials.dtype)
    dev = _dev(partials, out)
    W = partials.shape[0]
    if out is None:
        out = torch.empty(partials.shape[1:], dtype=partials.dtype, device=dev)
    st = _lib.load().mc2_ar_sum_local(partials.data_ptr(), W, out.numel(), _CODES[partials.dtype],
                                      rounding, out.data_ptr(), _stream(dev))
    _check("mc2_ar_sum_local", st)
    return out


def mc2_moe_histc(sel, num_experts, *, counts=None, dev_err=None):
    _want(sel, "sel", dtype=torch.int32)
    _want(counts, "counts", dtype=torch.int32, numel=num_experts)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(sel, counts, dev_err)
    if counts is None:
        counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    st = _lib.load().mc2_moe_histc(sel.data_ptr(), sel.numel(), num_experts, counts.data_ptr(),
                                   _ptr(dev_err), _stream(dev))
    _check("mc2_moe_histc", st)
    return counts


def mc2_moe_permute_workspace_size(T, K, num_experts) -> int:
    return int(_lib.load().mc2_moe_permute_workspace_size(T, K, num_experts))


def _check_permute(x, sel, num_experts, permuted, sorted_idx, unpermute_idx, expert_offsets,
                   dev_err):
    if x.dim() != 2 or sel.dim() != 2:
        raise ValueError("x must be (T, H) and sel (T, K)")
    T, H = x.shape
    K = sel.shape[1]
    if sel.dtype != torch.int32 or sel.shape[0] != T:
        raise ValueError("sel must be int32 (T, K)")
    if x.element_size() != 2:
        raise ValueError("x must hold 16-bit elements")
    _want(permuted, "permuted", shape=(T * K, H), dtype=x.dtype)
    _want(sorted_idx, "sorted_idx", dtype=torch.int32, numel=T * K)
    _want(unpermute_idx, "unpermute_idx", dtype=torch.int32, numel=T * K)
    _want(expert_offsets, "expert_offsets", dtype=torch.int32, numel=num_experts + 1)
    _want(dev_err, "dev_err", **_ERR)
    return T, H, K


def mc2_moe_permute(x, sel, num_experts, *, permuted=None, sorted_idx=None, unpermute_idx=None,
                    expert_offsets=None, workspace=None, dev_err=None):
    """Returns (permuted, sorted_idx, unpermute_idx, expert_offsets)."""
    T, H, K = _check_permute(x, sel, num_experts, permuted, sorted_idx, unpermute_idx,
                             expert_offsets, dev_err)
    _want(workspace, "workspace", dtype=torch.uint8)
    dev = _dev(x, sel, permuted, sorted_idx, unpermute_idx, expert_offsets, workspace, dev_err)
    if permuted is None:
        permuted = torch.empty((T * K, H), dtype=x.dtype, device=dev)
    if sorted_idx is None:
        sorted_idx = torch.empty(T * K, dtype=torch.int32, device=dev)
    if unpermute_idx is None:
        unpermute_idx = torch.empty(T * K, dtype=torch.int32, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    ws = mc2_moe_permute_workspace_size(T, K, num_experts)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
    st = _lib.load().mc2_moe_permute(
        x.data_ptr(), T, H, sel.data_ptr(), K, num_experts, permuted.data_ptr(),
        sorted_idx.data_ptr(), unpermute_idx.data_ptr(), expert_offsets.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _ptr(dev_err),
        _stream(dev))
    _check("mc2_moe_permute", st)
    return permuted, sorted_idx, unpermute_idx, expert_offsets


MC2_PERMUTE_SCRATCH_BYTES = 4 << 20


def mc2_moe_permute_noalloc(x, sel, num_experts, *, permuted, sorted_idx, unpermute_idx,
                            expert_offsets, dev_err=None):
    """mc2_moe_permute with the library's own per-device counting workspace:
    the C call allocates nothing, so every output must be passed in. Calls
    that overlap on one device share that workspace and must be ordered."""
    if any(t is None for t in (permuted, sorted_idx, unpermute_idx, expert_offsets)):
        raise ValueError("every output must be passed in")
    T, H, K = _check_permute(x, sel, num_experts, permuted, sorted_idx, unpermute_idx,
                             expert_offsets, dev_err)
    dev = _dev(x, sel, permuted, sorted_idx, unpermute_idx, expert_offsets, dev_err)
    st = _lib.load().mc2_moe_permute_noalloc(
        x.data_ptr(), T, H, sel.data_ptr(), K, num_experts, permuted.data_ptr(),
        sorted_idx.data_ptr(), unpermute_idx.data_ptr(), expert_offsets.data_ptr(),
        _ptr(dev_err), _stream(dev))
    _check("mc2_moe_permute_noalloc", st)
    return permuted, sorted_idx, unpermute_idx, expert_offsets


def _check_counts(send_counts, recv_counts, num_experts, world_size_src, local_experts):
    _want(send_counts, "send_counts", dtype=torch.int32, numel=num_experts)
    _want(recv_counts, "recv_counts", dtype=torch.int32, numel=world_size_src * local_experts)


def mc2_gmm_dispatch(send_buf, send_counts, recv_counts, w1, *, ep_rank, num_experts,
                     world_size_src=1, act=MC2_ACT_SWIGLU, h_out=None, dev_err=None):
    """Grouped fc1 (+ SwiGLU) over the rows of the local experts. h_out must
    hold at least as many rows as the local experts receive; by default it has
    as many rows as send_buf."""
    if w1.dim() != 3 or send_buf.dim() != 2:
        raise ValueError("w1 must be (E_l, H, I2) and send_buf (rows, H)")
    E_l, H, I2 = w1.shape
    n_out = I2 // 2 if act == MC2_ACT_SWIGLU else I2
    _check_counts(send_counts, recv_counts, num_experts, world_size_src, E_l)
    _want(w1, "w1", dtype=torch.bfloat16)
    _want(send_buf, "send_buf", shape=(send_buf.shape[0], H), dtype=torch.bfloat16)
    if h_out is not None:
        _want(h_out, "h_out", shape=(h_out.shape[0], n_out), dtype=torch.bfloat16)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(send_buf, send_counts, recv_counts, w1, h_out, dev_err)
    if h_out is None:
        h_out = torch.empty((send_buf.shape[0], n_out), dtype=torch.bfloat16, device=dev)
    st = _lib.load().mc2_gmm_dispatch(
        send_buf.data_ptr(), send_buf.shape[0], send_counts.data_ptr(), recv_counts.data_ptr(),
        world_size_src, ep_rank, num_experts, E_l, w1.data_ptr(), H, I2, act, h_out.data_ptr(),
        h_out.shape[0], _ptr(dev_err), _stream(dev))
    _check("mc2_gmm_dispatch", st)
    return h_out


def mc2_gmm_combine(h, recv_counts, send_counts, w2, combine_buf, *, ep_rank, num_experts,
                    world_size_src=1, dev_err=None):
    """Grouped fc2 written back over the local experts' rows of combine_buf."""
    if w2.dim() != 3 or h.dim() != 2 or combine_buf.dim() != 2:
        raise ValueError("w2 must be (E_l, I, H), h (rows, I) and combine_buf (rows, H)")
    E_l, I, H = w2.shape
    _check_counts(send_counts, recv_counts, num_experts, world_size_src, E_l)
    _want(w2, "w2", dtype=torch.bfloat16)
    _want(h, "h", shape=(h.shape[0], I), dtype=torch.bfloat16)
    _want(combine_buf, "combine_buf", shape=(combine_buf.shape[0], H), dtype=torch.bfloat16)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(h, recv_counts, send_counts, w2, combine_buf, dev_err)
    st = _lib.load().mc2_gmm_combine(
        h.data_ptr(), h.shape[0], recv_counts.data_ptr(), send_counts.data_ptr(), world_size_src,
        ep_rank, num_experts, E_l, w2.data_ptr(), I, H, combine_buf.data_ptr(),
        combine_buf.shape[0], _ptr(dev_err), _stream(dev))
    _check("mc2_gmm_combine", st)
    return combine_buf


def mc2_gmm_backward_workspace_size(rows, local_experts, M, N) -> int:
    return int(_lib.load().mc2_gmm_backward_workspace_size(rows, local_experts, M, N))


def _workspace(nbytes, workspace, dev):
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    return workspace


def mc2_gmm_combine_backward(dy_buf, recv_counts, send_counts, w2, h, *, ep_rank, num_experts,
                             act=MC2_ACT_NONE, g_saved=None, world_size_src=1, dgrad_out=None,
                             dw2_out=None, workspace=None, dev_err=None):
    """Backward of the grouped fc2: returns (dgrad, dW2). dgrad is the fc2
    input gradient (rows of h, I), or with act=MC2_ACT_SWIGLU the gradient of
    the saved fc1 pre-activation g_saved (rows, 2I); dW2 (E_l, I, H) fp32."""
    if w2.dim() != 3 or h.dim() != 2 or dy_buf.dim() != 2:
        raise ValueError("w2 must be (E_l, I, H), h (rows, I) and dy_buf (rows, H)")
    E_l, I, H = w2.shape
    cols = 2 * I if act == MC2_ACT_SWIGLU else I
    _check_counts(send_counts, recv_counts, num_experts, world_size_src, E_l)
    _want(w2, "w2", dtype=torch.bfloat16)
    _want(dy_buf, "dy_buf", shape=(dy_buf.shape[0], H), dtype=torch.bfloat16)
    _want(h, "h", shape=(h.shape[0], I), dtype=torch.bfloat16)
    _want(g_saved, "g_saved", shape=(h.shape[0], 2 * I), dtype=torch.bfloat16)
    _want(dgrad_out, "dgrad_out", shape=(h.shape[0], cols), dtype=torch.bfloat16)
    _want(dw2_out, "dw2_out", shape=(E_l, I, H), dtype=torch.float32)
    _want(workspace, "workspace", dtype=torch.uint8)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(dy_buf, recv_counts, send_counts, w2, h, g_saved, dgrad_out, dw2_out, workspace,
               dev_err)
    if dgrad_out is None:
        dgrad_out = torch.empty((h.shape[0], cols), dtype=torch.bfloat16, device=dev)
    if dw2_out is None:
        dw2_out = torch.empty((E_l, I, H), dtype=torch.float32, device=dev)
    need = mc2_gmm_backward_workspace_size(h.shape[0], E_l, I, H)
    workspace = _workspace(need, workspace, dev)
    st = _lib.load().mc2_gmm_combine_backward(
        dy_buf.data_ptr(), dy_buf.shape[0], recv_counts.data_ptr(), send_counts.data_ptr(),
        world_size_src, ep_rank, num_experts, E_l, w2.data_ptr(), I, H, h.data_ptr(), h.shape[0],
        _ptr(g_saved), act, dgrad_out.data_ptr(), dw2_out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(dev_err), _stream(dev))
    _check("mc2_gmm_combine_backward", st)
    return dgrad_out, dw2_out


def mc2_gmm_dispatch_backward(dg, recv_counts, send_counts, w1, send_buf, dx_buf, *, ep_rank,
                              num_experts, world_size_src=1, dw1_out=None, workspace=None,
                              dev_err=None):
    """Backward of the grouped fc1: the input gradient goes into the local
    experts' rows of dx_buf (send-buffer layout); returns (dx_buf, dW1) with
    dW1 (E_l, H, I2) fp32."""
    if w1.dim() != 3 or dg.dim() != 2 or send_buf.dim() != 2 or dx_buf.dim() != 2:
        raise ValueError("w1 must be (E_l, H, I2); dg, send_buf and dx_buf matrices")
    E_l, H, I2 = w1.shape
    _check_counts(send_counts, recv_counts, num_experts, world_size_src, E_l)
    _want(w1, "w1", dtype=torch.bfloat16)
    _want(dg, "dg", shape=(dg.shape[0], I2), dtype=torch.bfloat16)
    _want(send_buf, "send_buf", shape=(send_buf.shape[0], H), dtype=torch.bfloat16)
    _want(dx_buf, "dx_buf", shape=(dx_buf.shape[0], H), dtype=torch.bfloat16)
    _want(dw1_out, "dw1_out", shape=(E_l, H, I2), dtype=torch.float32)
    _want(workspace, "workspace", dtype=torch.uint8)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(dg, recv_counts, send_counts, w1, send_buf, dx_buf, dw1_out, workspace, dev_err)
    if dw1_out is None:
        dw1_out = torch.empty((E_l, H, I2), dtype=torch.float32, device=dev)
    need = mc2_gmm_backward_workspace_size(send_buf.shape[0], E_l, H, I2)
    workspace = _workspace(need, workspace, dev)
    st = _lib.load().mc2_gmm_dispatch_backward(
        dg.data_ptr(), dg.shape[0], recv_counts.data_ptr(), send_counts.data_ptr(), world_size_src,
        ep_rank, num_experts, E_l, w1.data_ptr(), H, I2, send_buf.data_ptr(), send_buf.shape[0],
        dx_buf.data_ptr(), dx_buf.shape[0], dw1_out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(dev_err), _stream(dev))
    _check("mc2_gmm_dispatch_backward", st)
    return dx_buf, dw1_out


def mc2_moe_unpermute(y_full, unpermute_idx, probs, *, out=None, dev_err=None):
    if probs.dim() != 2 or y_full.dim() != 2:
        raise ValueError("probs must be (T, K) and y_full (rows, H)")
    T, K = probs.shape
    H = y_full.shape[1]
    _want(y_full, "y_full", dtype=torch.bfloat16)
    _want(probs, "probs", dtype=torch.float32)
    _want(unpermute_idx, "unpermute_idx", dtype=torch.int32, numel=T * K)
    _want(out, "out", shape=(T, H), dtype=torch.bfloat16)
    _want(dev_err, "dev_err", **_ERR)
    dev = _dev(y_full, unpermute_idx, probs, out, dev_err)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    st = _lib.load().mc2_moe_unpermute(
        y_full.data_ptr(), y_full.shape[0], unpermute_idx.data_ptr(), probs.data_ptr(), T, K, H,
        out.data_ptr(), _ptr(dev_err), _stream(dev))
    _check("mc2_moe_unpermute", st)
    return out
