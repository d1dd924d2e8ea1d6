"""Every HIP kernel, compiled for gfx950 as the library is, must not touch a
register that an outstanding LDS read is still filling (see lds_waits)."""
import os
import subprocess

import pytest

from lds_waits import kernel_bodies, violations
from split_kv_attention_amd import build

KERNEL_SOURCES = [f for f in sorted(os.listdir(build.CSRC)) if f.endswith(".hip")]


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_register_use_before_its_lds_read_lands(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [build.hipcc(), *build.HIP_FLAGS, "-S", "--cuda-device-only", os.path.join(build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    bodies = kernel_bodies(out.read_text())
    assert bodies, "no kernels found in the assembly"
    bad = {name: v for name, v in ((n, violations(b)) for n, b in bodies.items()) if v}
    assert not bad, "\n".join(f"{n}:\n  " + "\n  ".join(v[:5]) for n, v in bad.items())


def test_the_check_flags_a_copy_before_the_wait():
    """A planted mistake: a register copied before its lgkmcnt wait."""
    lines = [
        "ds_read_b128 v[0:3], v92 offset:96",
        "v_accvgpr_write_b32 a112, v0",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v5, v1",
    ]
    v = violations(lines)
    assert len(v) == 1 and "a112" in v[0]
    ok = ["ds_read_b128 v[0:3], v92", "ds_read_b128 v[4:7], v93", "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v9, v0"]
    assert violations(ok) == []
    late = ["ds_read_b128 v[0:3], v92", "ds_read_b128 v[4:7], v93", "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v9, v4"]
    assert len(violations(late)) == 1


def test_the_check_follows_branches_and_loops():
    """Planted mistakes that a straight walk would miss: a use on the taken
    side of a branch whose fall-through side waits, and a read at the end of
    a loop body used at its head through the back edge."""
    branch = [
        "ds_read_b128 v[0:3], v92",
        "s_cbranch_scc1 .LBB0_2",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v5, v0",
        "s_branch .LBB0_3",
        ".LBB0_2:",
        "v_mov_b32_e32 v6, v1",
        ".LBB0_3:",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v7, v2",
    ]
    v = violations(branch)
    assert len(v) == 1 and "v6" in v[0], v
    loop = [
        "s_mov_b32 s0, 0",
        ".LBB1_1:",
        "v_add_f32_e32 v8, v8, v4",
        "ds_read_b128 v[4:7], v93",
        "s_add_i32 s0, s0, 1",
        "s_cmp_lt_i32 s0, 8",
        "s_cbranch_scc1 .LBB1_1",
        "s_waitcnt lgkmcnt(0)",
    ]
    v = violations(loop)
    assert len(v) == 1 and "v4" in v[0], v
    loop_ok = loop[:4] + ["s_waitcnt lgkmcnt(0)"] + loop[4:]
    assert violations(loop_ok) == []
