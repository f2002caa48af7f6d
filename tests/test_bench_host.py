"""Host-side pieces of the benchmark: the record that ties the committed HBM
traffic figure to the headline kernel's code."""
import json
import os

import bench


def _patched_hash(monkeypatch, tmp_path, edit):
    """Hash of the headline kernel's sources after `edit` of copies of them."""
    root = tmp_path / "repo"
    for f in bench.KERNEL_SOURCES:
        dst = root / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        with open(os.path.join(bench.ROOT, f), encoding="utf-8") as fh:
            dst.write_text(edit(f, fh.read()), encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_source_hash()


def test_hash_ignores_comments_and_blank_space(monkeypatch, tmp_path):
    base = _patched_hash(monkeypatch, tmp_path / "a", lambda f, t: t)
    first = bench.KERNEL_SOURCES[0]
    commented = _patched_hash(
        monkeypatch, tmp_path / "b",
        lambda f, t: ("// a new comment\n/* and a\n block */\n" + t.replace("\n", "\n\n")) if f == first else t)
    assert commented == base


def test_hash_follows_code(monkeypatch, tmp_path):
    base = _patched_hash(monkeypatch, tmp_path / "a", lambda f, t: t)
    first = bench.KERNEL_SOURCES[0]
    changed = _patched_hash(monkeypatch, tmp_path / "b",
                            lambda f, t: t + "\nconstexpr int kExtra = 1;\n" if f == first else t)
    assert changed != base


def test_traffic_record_is_consistent():
    """The committed record's totals are the scaled counters it lists, and
    the read scale taken from the plain device copy agrees with the one from
    the one-tile GEMM whose operands pass once through the loads into LDS."""
    with open(os.path.join(bench.ROOT, bench.TRAFFIC_FILE), encoding="utf-8") as f:
        rec = json.load(f)
    fetch = rec["fetch_size_kib_per_dispatch"]
    write = rec["write_size_kib_per_dispatch"]
    assert abs(fetch["mean"] - (fetch["c5a_ag_mm"] + fetch["c5b_sim_rs"]) / 2) < 1e-6 * fetch["mean"]
    rd = fetch["mean"] * 1024 * rec["fetch_scale"]
    wr = write["mean"] * 1024 * rec["write_scale"]
    assert abs(rd - rec["hbm_read_bytes_per_launch"]) < 1e-6 * rd
    assert abs(wr - rec["hbm_write_bytes_per_launch"]) < 1e-6 * wr
    assert abs(rd + wr - rec["traffic_bytes_per_launch"]) < 1e-6 * (rd + wr)
    lds = rec["calibration_lds_gemm"]
    assert abs(lds["fetch_scale"] / rec["fetch_scale"] - 1) < 0.01
    assert rec["launch"] == bench.HEADLINE_LAUNCH
    # every launch writes its output exactly once
    out_bytes = 2 * (bench.C5A[0] * bench.C5A[2] + bench.C5B[0] * bench.C5B[2]) / 2
    assert abs(wr / out_bytes - 1) < 0.01
