import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def load_golden(name):
    """Parse a hand-worked fixture: ``key = rows`` with rows split by ';'."""
    import numpy as np
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            rows = [[float(v) for v in r.split()] for r in val.split(";")]
            out[key] = np.array(rows if len(rows) > 1 else rows[0], dtype=np.float64)
    return out


@pytest.fixture
def golden():
    return load_golden


def device_asm(src, out, extra_inc=()):
    """gfx950 assembly of one HIP source, compiled with the library's flags."""
    import subprocess
    from gemm_collective_core_amd import build
    flags = [f for f in build.HIPCC_FLAGS if f != "-shared"]
    cmd = [build.hipcc(), *flags, "-I", os.path.join(build.ROOT, "include"),
           *[f"-I{d}" for d in extra_inc], "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out, encoding="utf-8") as f:
        return f.read()


@pytest.fixture(scope="session")
def library_asm(tmp_path_factory):
    """{source path: assembly} of every library source, compiled once for the
    static checks of the compiled kernels."""
    from concurrent.futures import ThreadPoolExecutor
    from gemm_collective_core_amd import build
    d = tmp_path_factory.mktemp("asm")
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        texts = list(ex.map(lambda s: device_asm(s, str(d / (os.path.basename(s) + ".s"))), srcs))
    return dict(zip(srcs, texts))
