"""Planted mistakes in the oracle (CPU only): each plausible slip must make at
least one pin fail. The mistakes are planted by monkeypatching the oracle in
this process; the oracle's source is never changed."""
import numpy as np
import pytest

import test_oracle as pins
from conftest import load_golden
from oracle import gemm, moe, numerics


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_bias_added_once_is_caught(monkeypatch):
    real = gemm.mm_rs

    def once(x1, x2, **kw):
        b = kw.pop("bias", None)
        out = real(x1, x2, **{**kw, "out_dtype": "f32"})
        if b is not None:
            out = out + numerics.decode(b, kw["in_dtype"])[None, :]
        return numerics.round_to(out, kw.get("out_dtype") or kw["in_dtype"])
    monkeypatch.setattr(gemm, "mm_rs", once)
    _fails(pins.test_mm_rs_hand_example, load_golden)


def test_transposed_operand_is_caught(monkeypatch):
    real = gemm.ag_mm
    monkeypatch.setattr(gemm, "ag_mm", lambda x, w, **kw: real(x, np.ascontiguousarray(np.asarray(w)[::-1]), **kw))
    _fails(pins.test_mm_brute_force_nonsquare)


def test_round_half_up_is_caught(monkeypatch):
    def half_up(x, dtype):
        x = np.asarray(x, np.float64)
        if dtype == "f32":
            return x
        p, emin, fmax = numerics._FORMATS[dtype]
        _, e = np.frexp(x)
        ulp = np.ldexp(1.0, np.maximum(e, emin) - p)
        q = np.floor(x / ulp + 0.5) * ulp
        return np.where(np.abs(q) > fmax, np.copysign(np.inf, x), q)
    monkeypatch.setattr(numerics, "round_to", half_up)
    _fails(pins.test_round_hand_cases)


def test_swapped_scale_index_is_caught(monkeypatch):
    real = gemm.mm_rs

    def swapped(x1, x2, **kw):
        if kw.get("x1_scale") is not None and kw.get("x2_scale") is not None:
            s1, s2 = kw["x1_scale"], kw["x2_scale"]
            if np.size(s1) == np.size(s2):
                kw = {**kw, "x1_scale": s2, "x2_scale": s1}
        return real(x1, x2, **kw)
    monkeypatch.setattr(gemm, "mm_rs", swapped)
    _fails(pins.test_quant_hand_example, load_golden)


def test_unstable_segment_order_is_caught(monkeypatch):
    real = moe.permute

    def reversed_segments(x, sel, E):
        p = real(x, sel, E)
        s = p["sorted_idx"].copy()
        for e in range(E):
            a, b = p["offsets"][e], p["offsets"][e + 1]
            s[a:b] = s[a:b][::-1]
        p["sorted_idx"] = s
        return p
    monkeypatch.setattr(moe, "permute", reversed_segments)
    _fails(pins.test_permute_brute_force_and_properties)


def test_swapped_gate_up_is_caught(monkeypatch):
    monkeypatch.setattr(moe, "swiglu", lambda a: moe.silu(a[:, a.shape[1] // 2:]) * a[:, :a.shape[1] // 2])
    _fails(pins.test_gmm_swiglu_hand_example, load_golden)


def test_unpermute_with_wrong_index_is_caught(monkeypatch):
    real = moe.unpermute

    def wrong(y, idx, probs, T, K):
        return real(y, np.argsort(np.asarray(idx)), probs, T, K)
    monkeypatch.setattr(moe, "unpermute", wrong)
    _fails(pins.test_permute_hand_example, load_golden)


def test_dropped_partial_is_caught(monkeypatch):
    real = gemm.mm_rs

    def first_only(x1, x2, **kw):
        if kw.get("nsim", 1) > 1:
            kw = {**kw, "nsim": 1}
            x1, x2 = np.asarray(x1)[0], np.asarray(x2)[0]
        return real(x1, x2, **kw)
    monkeypatch.setattr(gemm, "mm_rs", first_only)
    _fails(pins.test_sim_rs_equals_concatenated_k)


def test_histc_off_by_one_is_caught(monkeypatch):
    real = moe.histc
    monkeypatch.setattr(moe, "histc", lambda sel, E: np.roll(real(sel, E), 1))
    _fails(pins.test_histc_against_torch_histc_and_bincount)


def test_longer_pieces_last_is_caught(monkeypatch):
    real = gemm.sub_chunk_rows

    def longer_last(m, W, c, s, j):
        # the remainder rows given to the last pieces instead of the first
        k = max(s, 1)
        mirrored = real(m, W, c, s, k - 1 - j)
        rows = gemm.chunk_rows(m, W, c)
        return slice(rows.start + rows.stop - mirrored.stop, rows.start + rows.stop - mirrored.start)
    monkeypatch.setattr(gemm, "sub_chunk_rows", longer_last)
    _fails(pins.test_sub_chunk_rows_hand_worked)


def test_piece_start_off_by_one_is_caught(monkeypatch):
    real = gemm.sub_chunk_rows

    def shifted(m, W, c, s, j):
        r = real(m, W, c, s, j)
        return slice(r.start + (1 if j else 0), r.stop)
    monkeypatch.setattr(gemm, "sub_chunk_rows", shifted)
    _fails(pins.test_sub_chunks_partition_each_chunk, 64, 4, 3)


def test_pieces_before_chunks_is_caught(monkeypatch):
    def piece_major(W, rank, kind, s):
        return [(c, j) for j in range(max(s, 1)) for c in gemm.chunk_order(W, rank, kind)]
    monkeypatch.setattr(gemm, "segment_order", piece_major)
    _fails(pins.test_segment_order)


def test_dsilu_without_curvature_term_is_caught(monkeypatch):
    def flat(a, dh):
        a = np.asarray(a, dtype=np.float64)
        inter = a.shape[1] // 2
        g, u = a[:, :inter], a[:, inter:]
        s = 1.0 / (1.0 + np.exp(-g))
        return np.concatenate([dh * u * s, dh * g * s], axis=1)
    monkeypatch.setattr(moe, "swiglu_backward", flat)
    _fails(pins.test_swiglu_backward_closed_forms)


def test_weight_used_untransposed_in_dgrad_is_caught(monkeypatch):
    real = moe.gmm_backward

    def no_transpose(rows, sizes, weights, dy):
        dX, dW = real(rows, sizes, weights, dy)
        Wt = np.asarray(weights, dtype=np.float64)
        D = np.asarray(dy, dtype=np.float64)
        off = 0
        for g, c in enumerate(int(x) for x in sizes):
            k = min(Wt.shape[1], Wt.shape[2])
            dX[off:off + c, :k] = D[off:off + c, :k] @ Wt[g][:k, :k]
            off += c
        return dX, dW
    monkeypatch.setattr(moe, "gmm_backward", no_transpose)
    _fails(pins.test_gmm_backward_matches_autograd)


def test_combine_backward_reading_rows_from_zero_is_caught(monkeypatch):
    real = moe.local_slice
    monkeypatch.setattr(moe, "local_slice", lambda sc, r, el: (0, real(sc, r, el)[1]))
    _fails(pins.test_moe_backward_chain_matches_autograd)
