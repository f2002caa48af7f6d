"""The scalar-register wait-state check (sgpr_hazard.py): the checker on small
listings, then on every kernel of the library as built and on the chunked
GEMM with its K split compiled in (whose partial stores are assembly with a
scalar base address), and on a planted kernel with the pattern that made the
split's first device runs fault: a store reading v_readfirstlane's result
with no wait states in between must be reported."""
import os
import re
import shutil

import pytest

import sgpr_hazard as sh
from conftest import device_asm as _device_asm


def _h(body):
    return sh.check_function(body.splitlines())


def test_readfirstlane_then_store_is_flagged():
    h = _h("\tv_readfirstlane_b32 s4, v1\n\tv_readfirstlane_b32 s5, v2\n"
           "\tglobal_store_dwordx4 v0, a[0:3], s[4:5] sc1\n")
    assert len(h) == 1 and h[0].startswith("v_readfirstlane_b32 s4") and "sc1" in h[0]


def test_five_wait_states_are_enough():
    assert _h("\tv_readfirstlane_b32 s4, v1\n\tv_readfirstlane_b32 s5, v2\n"
              "\ts_nop 4\n\tglobal_store_dwordx4 v0, a[0:3], s[4:5] sc1\n") == []
    # s5 has 5 wait states (the nop), s4 one more
    assert _h("\tv_readfirstlane_b32 s5, v2\n\ts_nop 3\n"
              "\tglobal_store_dwordx4 v0, a[0:3], s[4:5] sc1\n") != []
    assert _h("\tv_readfirstlane_b32 s5, v2\n" + "\ts_mov_b32 s9, 0\n" * 5 +
              "\tglobal_load_dwordx4 v[0:3], v0, s[4:5]\n") == []


def test_resource_and_offset_operands_and_carry_out():
    assert _h("\tv_readlane_b32 s10, v1, 0\n\tbuffer_load_dword v2, v3, s[8:11], 0 offen\n") != []
    assert _h("\tv_cmp_gt_u32_e64 s[12:13], v1, v2\n"
              "\tbuffer_store_dword v2, v3, s[8:11], s12 offen\n") != []
    assert _h("\tv_add_co_u32_e64 v4, s[6:7], v1, v2\n"
              "\tglobal_load_dword v5, v0, s[6:7]\n") != []
    # a vector destination, a vcc destination, or an unrelated register: clean
    assert _h("\tv_add_co_u32_e32 v4, vcc, v1, v2\n\tv_cmp_gt_u32_e32 vcc, v1, v2\n"
              "\tv_readfirstlane_b32 s20, v1\n\tglobal_load_dword v5, v0, s[6:7]\n") == []


def test_function_boundaries():
    text = ("_Z1fv:\n\tv_readfirstlane_b32 s4, v1\n\ts_endpgm\n.Lfunc_end0:\n"
            "_Z1gv:\n\tglobal_load_dword v5, v0, s[4:5]\n\ts_endpgm\n.Lfunc_end1:\n")
    assert sh.check_assembly(text) == {}
    text = "_Z1fv:\n.LBB0_1:\n\tv_readfirstlane_b32 s4, v1\n.LBB0_2:\n" \
           "\tglobal_load_dword v5, v0, s[4:5]\n\ts_endpgm\n.Lfunc_end0:\n"
    assert list(sh.check_assembly(text)) == ["_Z1fv"]


_HIPCC = shutil.which("hipcc") is not None or os.path.exists("/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not _HIPCC, reason="hipcc is needed to compile the kernels")
def test_library_kernels_wait_before_scalar_operands(library_asm):
    srcs, texts = list(library_asm), list(library_asm.values())
    found = {}
    for src, text in zip(srcs, texts):
        assert text.count(".Lfunc_end") > 0
        for fn, h in sh.check_assembly(text).items():
            found[f"{os.path.basename(src)}: {fn}"] = h[:3]
    assert not found, found


@pytest.mark.skipif(not _HIPCC, reason="hipcc is needed to compile the kernels")
def test_k_split_kernels_pass(tmp_path):
    """The chunked GEMM compiled with the K split switched on (a copy of the
    source with the switch flipped), so that its partial stores (device-scope
    global stores from the accumulation registers, with a scalar base
    address) are in the listing."""
    from gemm_collective_core_amd import build
    src = open(os.path.join(build.CSRC, "mc2_gemm.hip"), encoding="utf-8").read()
    flag = "constexpr bool kSplitEnabled = false;"
    assert src.count(flag) == 1
    copy = tmp_path / "mc2_gemm_split.hip"
    copy.write_text(src.replace(flag, "constexpr bool kSplitEnabled = true;"), encoding="utf-8")
    text = _device_asm(str(copy), str(tmp_path / "split.s"), extra_inc=(build.CSRC,))
    stores = re.findall(r"global_store_dwordx4 v\d+, a\[\d+:\d+\], s\[\d+:\d+\] sc1", text)
    assert len(stores) >= 64, len(stores)
    assert sh.check_assembly(text) == {}


_PLANT = r"""
#include <hip/hip_runtime.h>
#include <stdint.h>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ void plant(const uint64_t* bases, u32x4 v) {
  // a per-lane load, made scalar: v_readfirstlane writes the scalar registers
  const uint64_t bv = bases[threadIdx.x];
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv >> 32));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile(NOPS "global_store_dwordx4 %0, %1, %2"
               :: "v"(threadIdx.x * 16u), "v"(v), "s"(sb) : "memory");
}
"""


@pytest.mark.skipif(not _HIPCC, reason="hipcc is needed to compile the kernels")
@pytest.mark.parametrize("nops,bad", [("", True), ("s_nop 4\\n\\t", False)])
def test_planted_store_after_readfirstlane(tmp_path, nops, bad):
    """The pattern of the split's first device faults, compiled (never run):
    an assembly store whose scalar address comes straight from
    v_readfirstlane is reported without the 5 wait states, and passes with
    them."""
    f = tmp_path / "plant.hip"
    f.write_text(_PLANT.replace("NOPS", '"' + nops + '"'), encoding="utf-8")
    text = _device_asm(str(f), str(tmp_path / "plant.s"))
    assert "v_readfirstlane_b32" in text and "global_store_dwordx4" in text
    assert bool(sh.check_assembly(text)) == bad
