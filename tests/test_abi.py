"""The C ABI without a GPU: the library loads, exports every entry point that
include/mc2.h declares, and rejects invalid arguments on the host before any
launch (these calls fail validation, so no device work is ever enqueued)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT
from gemm_collective_core_amd import _lib

HEADER = os.path.join(ROOT, "include", "mc2.h")
FAKE = 0x1000  # a non-NULL, 16-byte aligned address that is never dereferenced

MC2_OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUP, ERR_HIP, ERR_WS, ERR_ALIGN = range(8)
F16, BF16, I8, F32, I32 = range(5)


def declared():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(mc2_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmc2.so is not built: run `python -m gemm_collective_core_amd.build`")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.mc2_version().decode().startswith("mc2-gfx950")
    for s in range(8):
        assert lib.mc2_status_string(s).decode().startswith("MC2_")
    assert b"unknown" in lib.mc2_status_string(99)


def rs(lib, **over):
    a = dict(x1=FAKE, x2=FAKE, m=128, k=512, n=64, W=2, rank=0, nsim=1, trans=0, dt=F16,
             bias=None, s1=None, s2=None, odt=F16, out=FAKE, flags=None, cnt=None, epoch=0,
             turn=0)
    a.update(over)
    return lib.mc2_mm_rs_local(a["x1"], a["x2"], a["m"], a["k"], a["n"], a["W"], a["rank"],
                               a["nsim"], a["trans"], a["dt"], a["bias"], a["s1"], a["s2"],
                               a["odt"], a["out"], a["flags"], a["cnt"], a["epoch"], a["turn"],
                               a.get("ws"), a.get("ws_bytes", 0), None)


@pytest.mark.parametrize("over,code", [
    (dict(x1=None), ERR_NULL),
    (dict(out=None), ERR_NULL),
    (dict(m=129), ERR_SHAPE),             # m % world_size
    (dict(k=255), ERR_SHAPE),             # k >= 256
    (dict(k=65535), ERR_SHAPE),           # k < 65535
    (dict(W=3), ERR_SHAPE),               # world sizes 1, 2, 4, 8, 16, 32
    (dict(W=64, m=128), ERR_SHAPE),
    (dict(rank=2), ERR_SHAPE),
    (dict(nsim=3), ERR_SHAPE),
    (dict(dt=F32), ERR_DTYPE),
    (dict(odt=BF16), ERR_DTYPE),          # basic case: output dtype = input dtype
    (dict(s1=FAKE, s2=FAKE), ERR_DTYPE),  # scales only for int8
    (dict(dt=I8, odt=BF16), ERR_NULL),    # int8 needs both scales
    (dict(dt=I8, odt=I32, s1=FAKE), ERR_DTYPE),
    (dict(dt=I8, odt=F16, s1=FAKE, s2=FAKE, nsim=2), ERR_UNSUP),
    (dict(dt=I8, odt=I8), ERR_DTYPE),
    (dict(k=516), ERR_ALIGN),             # k % 8 for 16-bit inputs
    (dict(n=68), ERR_ALIGN),
    (dict(dt=I8, odt=I32, n=72), ERR_ALIGN),
    (dict(x1=FAKE + 8), ERR_ALIGN),
    (dict(flags=FAKE), ERR_NULL),         # flags need counters
    (dict(flags=FAKE, cnt=FAKE, epoch=0), ERR_SHAPE),
    (dict(turn=-1), ERR_SHAPE),           # comm_turn >= 0
    (dict(turn=65), ERR_SHAPE),           # at most m / W pieces (64 rows per chunk)
    (dict(ws=FAKE + 8, ws_bytes=1 << 20), ERR_ALIGN),  # the K-split workspace
])
def test_mm_rs_rejects(lib, over, code):
    assert rs(lib, **over) == code


def test_ag_mm_rejects(lib):
    f = lib.mc2_ag_mm_local
    tail = (None, None, 0, 0, None, 0, None)
    assert f(None, FAKE, 16, 512, 64, 8, 0, 0, BF16, None, FAKE, *tail) == ERR_NULL
    assert f(FAKE, FAKE, 16, 512, 64, 8, 8, 0, BF16, None, FAKE, *tail) == ERR_SHAPE
    assert f(FAKE, FAKE, 16, 512, 64, 8, 0, 0, I8, None, FAKE, *tail) == ERR_DTYPE
    assert f(FAKE, FAKE, 16, 500, 64, 8, 0, 0, BF16, None, FAKE, *tail) == ERR_ALIGN
    assert f(FAKE, FAKE, 0, 512, 64, 8, 0, 0, BF16, None, FAKE, *tail) == ERR_SHAPE
    assert f(FAKE, FAKE, 16, 512, 64, 8, 0, 0, BF16, None, FAKE, None, None, 0, 17, None, 0,
             None) == ERR_SHAPE
    assert f(FAKE, FAKE, 16, 512, 64, 8, 0, 0, BF16, None, FAKE, None, None, 0, -1, None, 0,
             None) == ERR_SHAPE
    assert f(FAKE, FAKE, 16, 512, 64, 8, 0, 0, BF16, None, FAKE, None, None, 0, 0, FAKE + 4,
             1 << 20, None) == ERR_ALIGN


def test_split_workspace_size_and_policy(lib):
    """The K-split workspace: 4096 bytes of control words, then two 128 KiB
    partial slots per pair of workgroups (half the CUs; 256 where no GPU is
    visible). The policy setter takes the two documented values only."""
    ws = lib.mc2_split_workspace_size()
    assert ws > 4096 and (ws - 4096) % (2 * 128 * 1024) == 0
    assert ws - 4096 <= 256 * 2 * 128 * 1024
    assert lib.mc2_set_split_policy(2) == ERR_SHAPE
    assert lib.mc2_set_split_policy(-1) == ERR_SHAPE
    assert lib.mc2_set_split_policy(1) == MC2_OK
    assert lib.mc2_set_split_policy(0) == MC2_OK


def test_moe_entry_points_reject(lib):
    assert lib.mc2_moe_histc(FAKE, 10, 0, FAKE, None, None) == ERR_SHAPE
    assert lib.mc2_moe_histc(FAKE, 10, 1025, FAKE, None, None) == ERR_SHAPE
    assert lib.mc2_moe_histc(None, 10, 8, FAKE, None, None) == ERR_NULL
    ws = lib.mc2_moe_permute_workspace_size(32768, 8, 128)
    assert ws >= 128 * (32768 // 32) * 4
    P = lib.mc2_moe_permute
    assert P(FAKE, 100, 64, FAKE, 8, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, None) == ERR_WS
    assert P(FAKE, 100, 60, FAKE, 8, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None, None) == ERR_ALIGN
    assert P(FAKE, 100, 64, FAKE, 65, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None, None) == ERR_SHAPE
    assert P(FAKE, 100, 64, FAKE, 8, 16, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None, None) == ERR_NULL
    D = lib.mc2_gmm_dispatch
    assert D(FAKE, 100, FAKE, FAKE, 2, 0, 16, 4, FAKE, 64, 64, 1, FAKE, 100, None, None) == ERR_UNSUP
    assert D(FAKE, 100, FAKE, FAKE, 1, 4, 16, 4, FAKE, 64, 64, 1, FAKE, 100, None, None) == ERR_SHAPE
    assert D(FAKE, 100, FAKE, FAKE, 1, 0, 16, 5, FAKE, 64, 64, 1, FAKE, 100, None, None) == ERR_SHAPE
    assert D(FAKE, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 64, 72, 1, FAKE, 100, None, None) == ERR_ALIGN
    assert D(FAKE, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 64, 64, 2, FAKE, 100, None, None) == ERR_SHAPE
    Cb = lib.mc2_gmm_combine
    assert Cb(FAKE, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 60, 64, FAKE, 100, None, None) == ERR_ALIGN
    assert Cb(None, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 64, 64, FAKE, 100, None, None) == ERR_NULL
    U = lib.mc2_moe_unpermute
    assert U(FAKE, 10, FAKE, FAKE, 4, 0, 64, FAKE, None, None) == ERR_SHAPE
    assert U(FAKE, 10, FAKE, FAKE, 4, 2, 4, FAKE, None, None) == ERR_SHAPE
    assert U(FAKE, 10, FAKE, FAKE, 4, 2, 68, FAKE, None, None) == ERR_ALIGN


def test_noalloc_permute_rejects_sizes_beyond_its_scratch(lib):
    """The allocation-free permute checks the size against its fixed scratch
    array before looking the array up or launching anything."""
    T, K, E = 1 << 20, 8, 128
    assert lib.mc2_moe_permute_workspace_size(T, K, E) > (4 << 20)
    assert lib.mc2_moe_permute_workspace_size(131072, 8, 128) <= (4 << 20)
    P = lib.mc2_moe_permute_noalloc
    assert P(FAKE, T, 64, FAKE, K, E, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_WS
    assert P(FAKE, 100, 64, FAKE, 65, 16, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert P(FAKE, 100, 64, FAKE, 8, 16, FAKE, None, FAKE, FAKE, None, None) == ERR_NULL


def test_ag_mm_inflags_validates(lib):
    f = lib.mc2_ag_mm_local_inflags
    base = (FAKE, FAKE, 100, 512, 264, 8, 0, 0, BF16, None, FAKE, None, None, 0, 0)
    nows = (None, 0, None)
    assert f(*base, None, 1, 100, None, *nows) == ERR_NULL      # in_flags required
    assert f(*base, FAKE, 0, 100, None, *nows) == ERR_SHAPE     # in_epoch != 0
    assert f(*base, FAKE, 1, 0, None, *nows) == ERR_SHAPE       # spin_limit >= 1
    assert f(None, *base[1:], FAKE, 1, 100, None, *nows) == ERR_NULL
    assert f(*base[:8], I8, *base[9:], FAKE, 1, 100, None, *nows) == ERR_DTYPE
    assert f(*base[:14], 101, FAKE, 1, 100, None, *nows) == ERR_SHAPE   # comm_turn <= m_c
    assert f(*base, FAKE, 1, 100, None, FAKE + 8, 1 << 20, None) == ERR_ALIGN


def test_mm_ar_validates(lib):
    f = lib.mc2_mm_ar_local
    assert lib.mc2_mm_ar_workspace_size(100, 64, 4, BF16, 0) == 0
    assert lib.mc2_mm_ar_workspace_size(100, 64, 4, BF16, 1) == 4 * 100 * 64 * 2
    assert lib.mc2_mm_ar_workspace_size(100, 64, 3, BF16, 1) == 0   # world sizes 1, 2, 4, ...
    assert lib.mc2_mm_ar_workspace_size(100, 64, 4, I8, 2) == 0
    base = (FAKE, FAKE, 100, 512, 64, 4, 0, BF16, None)
    assert f(*base, 1, FAKE, None, 0, None) == ERR_NULL            # the mode needs a workspace
    assert f(*base, 1, FAKE, FAKE, 16, None) == ERR_WS             # too small
    assert f(*base, 1, FAKE, FAKE + 8, 1 << 20, None) == ERR_ALIGN
    assert f(*base, 3, FAKE, None, 0, None) == ERR_SHAPE           # unknown mode
    assert f(FAKE, FAKE, 100, 512, 64, 3, 0, BF16, None, 0, FAKE, None, 0, None) == ERR_SHAPE
    assert f(FAKE, FAKE, 100, 512, 64, 4, 0, I8, None, 0, FAKE, None, 0, None) == ERR_DTYPE
    assert f(FAKE, FAKE, 100, 516, 64, 4, 0, BF16, None, 0, FAKE, None, 0, None) == ERR_ALIGN
    g = lib.mc2_ar_sum_local
    assert g(FAKE, 4, 1024, BF16, 0, FAKE, None) == ERR_SHAPE       # the sum step needs mode 1 or 2
    assert g(FAKE, 33, 1024, BF16, 1, FAKE, None) == ERR_SHAPE
    assert g(FAKE, 4, 1020, BF16, 1, FAKE, None) == ERR_ALIGN
    assert g(FAKE, 4, 1024, F32, 1, FAKE, None) == ERR_DTYPE


def test_gmm_backward_validates(lib):
    # tile counters (3 x 8 tiles x 16 experts, 256-byte aligned), no split slots below 2048 rows
    ws = lib.mc2_gmm_backward_workspace_size(1000, 16, 768, 2048)
    assert ws == (3 * 8 * 16 * 4 + 255) // 256 * 256
    # then 2 * rows / 4096 slots of 256 x 256 fp32 partial tiles per tile of an expert
    big = lib.mc2_gmm_backward_workspace_size(40000, 16, 768, 2048)
    assert big == 1536 + (2 * 40000 // 4096) * 24 * 256 * 256 * 4
    assert lib.mc2_gmm_backward_workspace_size(1000, 0, 768, 64) == 0
    Cb = lib.mc2_gmm_combine_backward
    base = (FAKE, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 64, 128, FAKE, 100)
    assert Cb(*base, None, 1, FAKE, FAKE, FAKE, 1 << 24, None, None) == ERR_NULL     # SwiGLU needs g_saved
    assert Cb(*base, None, 0, FAKE, FAKE, None, 0, None, None) == ERR_NULL          # workspace
    assert Cb(*base, None, 0, FAKE, FAKE, FAKE, 16, None, None) == ERR_WS
    assert Cb(*base, None, 2, FAKE, FAKE, FAKE, 1 << 24, None, None) == ERR_SHAPE    # unknown act
    assert Cb(*base[:4], 2, *base[5:], None, 0, FAKE, FAKE, FAKE, 1 << 24, None, None) == ERR_UNSUP
    assert Cb(*base[:9], 60, *base[10:], None, 0, FAKE, FAKE, FAKE, 1 << 24, None, None) == ERR_ALIGN
    Db = lib.mc2_gmm_dispatch_backward
    dbase = (FAKE, 100, FAKE, FAKE, 1, 0, 16, 4, FAKE, 64, 128, FAKE, 100, FAKE, 100, FAKE)
    assert Db(*dbase, FAKE, 16, None, None) == ERR_WS
    assert Db(*dbase, FAKE + 8, 1 << 24, None, None) == ERR_ALIGN
    assert Db(*dbase[:15], None, FAKE, 1 << 24, None, None) == ERR_NULL
    assert Db(*dbase[:5], 4, *dbase[6:], FAKE, 1 << 24, None, None) == ERR_SHAPE     # ep_rank < E / E_l


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """The ABI is a C ABI: the header compiles as C99 and a C program links
    against the built library and calls it (entry points that need no GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text(
        '#include <stdio.h>\n#include "mc2.h"\n'
        'int main(void) {\n'
        '  printf("%s|%s|%d\\n", mc2_version(), mc2_status_string(MC2_ERR_SHAPE),\n'
        '         mc2_mm_rs_local(0, 0, 1, 1, 1, 1, 0, 1, 0, MC2_BF16, 0, 0, 0, MC2_BF16, 0, 0, 0,\n'
        '                         0, 0, 0, 0, 0));\n'
        '  return 0;\n}\n')
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "use"
    cmd = [gcc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER),
           "-I", "/opt/rocm/include", str(src), "-o", str(exe), "-L", libdir, "-lmc2",
           "-Wl,-rpath," + libdir]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    version, status, code = out.stdout.strip().split("|")
    assert version.startswith("mc2-gfx950") and status.startswith("MC2_")
    assert int(code) == 1  # MC2_ERR_NULL: x1 is NULL
