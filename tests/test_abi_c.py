"""include/flce.h from C: a C99 program (tests/abi_c_check.c) compiles with -pedantic
-Werror, links against the built library and gets the same host-side answers as the
Python binding (no GPU is used)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "chunked_lm_head_amd")


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("abi_c") / "abi_c_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_c_check.c"),
                    "-L", LIBDIR, "-lflce", f"-Wl,-rpath,{LIBDIR}", "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return dict(line.split(" ", 1) for line in out.strip().splitlines())


def test_c_caller_matches_the_binding(c_output):
    from chunked_lm_head_amd import flce

    assert int(c_output["workspace"]) == flce.workspace_bytes(16384, 4096, 151936, 256)
    status, row_block = c_output["plan"].split()
    assert int(status) == 0
    assert int(row_block) == flce.describe_plan(16384, 4096, 151936, 256)["row_block"]
    assert int(c_output["distill"]) == flce.distill_workspace_bytes(16384, 4096, 5120, 151936,
                                                                     256)
    assert int(c_output["policy"]) == flce.policy_workspace_bytes(32768, 4096, 128000, 256, 4)
    assert int(c_output["chunk_rows"]) == flce.chunk_rows_for(8192)
    st, mb, cr = (int(v) for v in c_output["tune"].split())
    t = flce.tune(4, 8192, 4096, 128000, 8 << 30)
    assert st == 0 and (mb, cr) == (t["mini_batches"], t["chunk_rows"])
    assert int(c_output["bad_shape"]) == 4          # D not a multiple of 8
    assert c_output["status"] == "workspace too small"
    assert "multiple of 8" in c_output["bad_shape_error"]
    assert c_output["kernel"] == "bwd_grad ?"
    assert int(c_output["timing_off"]) == 1         # FLCE_ERR_ARG: NULL outputs
    assert "NULL" in c_output["last_error"]
    assert int(c_output["forward_scratch"]) == 16 << 20
