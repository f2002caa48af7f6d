"""The compiled kernels never touch a VGPR while an inline-asm LDS read into it
is still in flight (see lds_hazard.py for the model), and the checker itself
flags the pattern that once produced wrong results: the compiler copying one
dword of an asm operand read straight after issuing it."""
import os
import shutil

import pytest

import lds_hazard as lh

FN = "_Zkernel:\n"


def _hazards(body: str):
    return lh.check_assembly(FN + body + "\n.Lfunc_end0:\n").get("_Zkernel", [])


def test_copy_before_wait_is_flagged():
    h = _hazards("\tds_read_b128 v[34:37], v3\n\tv_mov_b32_e32 v99, v37\n"
                 "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    assert len(h) == 1 and "v_mov_b32_e32 v99, v37" in h[0]


def test_copy_after_wait_is_clean():
    assert _hazards("\tds_read_b128 v[34:37], v3\n\ts_waitcnt lgkmcnt(0)\n"
                    "\tv_mov_b32_e32 v99, v37\n\ts_endpgm") == []


def test_wait_count_retires_the_oldest_reads():
    body = ("\tds_read_b128 v[0:3], v40\n\tds_read_b128 v[4:7], v41\n"
            "\ts_waitcnt lgkmcnt(1)\n\tv_mov_b32_e32 v50, v3\n"   # first read done
            "\tv_mov_b32_e32 v51, v7\n"                            # second still in flight
            "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    h = _hazards(body)
    assert len(h) == 1 and "v51, v7" in h[0]


def test_write_of_an_in_flight_destination_is_flagged():
    h = _hazards("\tds_read_b64_tr_b16 v[10:11], v2\n\tv_add_u32_e32 v11, 1, v12\n"
                 "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    assert len(h) == 1


def test_read_skipped_on_one_path_is_not_reported_at_the_join():
    body = ("\ts_cbranch_scc1 .LBB0_2\n"
            "\tds_read_b128 v[0:3], v40\n"
            ".LBB0_2:\n"
            "\tv_mov_b32_e32 v50, v0\n"
            "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    assert _hazards(body) == []


def test_read_on_every_path_is_reported_after_the_branch():
    body = ("\tds_read_b128 v[0:3], v40\n"
            "\ts_cbranch_scc1 .LBB0_2\n"
            "\tv_add_u32_e32 v60, 1, v61\n"
            ".LBB0_2:\n"
            "\tv_mov_b32_e32 v50, v1\n"
            "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    h = _hazards(body)
    assert len(h) == 1 and "v50, v1" in h[0]


def test_in_order_overwrite_by_a_later_read_is_allowed():
    assert _hazards("\tds_read_b128 v[0:3], v40\n\tds_read_b128 v[0:3], v41\n"
                    "\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32_e32 v50, v0\n\ts_endpgm") == []


def test_read_carried_over_a_loop_back_edge():
    # issued at the end of an iteration, consumed after a wait in the next one;
    # a copy on the latch before the wait is a hazard
    body = ("\ts_waitcnt lgkmcnt(0)\n"
            ".LBB0_1:\n"
            "\ts_waitcnt lgkmcnt(0)\n"
            "\tv_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], v[8:11]\n"
            "\tds_read_b128 v[0:3], v40\n"
            "\tv_mov_b32_e32 v20, v2\n"
            "\ts_cbranch_scc1 .LBB0_1\n"
            "\ts_waitcnt lgkmcnt(0)\n\ts_endpgm")
    h = _hazards(body)
    assert len(h) == 1 and "v20, v2" in h[0]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to compile the kernels")
def test_compiled_kernels_have_no_in_flight_lds_access(library_asm):
    """Every kernel of the library, compiled for gfx950 as the build compiles
    it."""
    srcs, texts = list(library_asm), list(library_asm.values())
    found = {}
    nfun = 0
    for src, text in zip(srcs, texts):
        nfun += text.count(".Lfunc_end")
        for fn, h in lh.check_assembly(text).items():
            found[f"{os.path.basename(src)}: {fn}"] = h[:3]
    assert nfun >= 90, nfun  # the kernels were compiled and parsed
    assert not found, found
