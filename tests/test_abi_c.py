"""The ABI from plain C: tests/abi_client.c is compiled as C99 with warnings as
errors against include/sketchssm.h and include/sketchssm_measure.h, linked to the built library and run on the
host (planner and status codes only, no GPU needed)."""
import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "rank_state_read_amd")


@pytest.mark.timeout(120)
def test_c_client(tmp_path, golden_dir):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libsketchssm.so")):
        pytest.fail("libsketchssm.so is not built")
    exe = tmp_path / "abi_client"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_client.c"),
           "-L", LIBDIR, "-lsketchssm", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, _, rest = line.partition(" ")
        out[key] = rest
    with open(os.path.join(golden_dir, "plan_small.json")) as f:
        g = json.load(f)
    ints = lambda s: [int(x) for x in s.split()]  # noqa: E731
    for key in ("frame_index", "frame_row_off", "z_row_off", "bucket", "order"):
        assert ints(out[key]) == g[key], key
    assert list(zip(ints(out["frame_group"]), ints(out["frame_rank"]))) == [tuple(f) for f in g["frames"]]
    assert int(out["z_elems"]) == 4 * 80 * sum(g["rank"])
    assert int(out["frame_elems"]) == 128 * sum(r for _, r in g["frames"])
    assert int(out["null_out"]) == 1      # SKSSM_EINVAL
    assert int(out["bad_V"]) == 2         # SKSSM_ESHAPE
    assert int(out["ordered_status"]) == 0
    o = list(g["order"])
    dense = [h for h in o if g["rank"][h] == 0]
    sk = [h for h in o if g["rank"][h] > 0]
    assert ints(out["ordered"]) == dense + sk[::-1]
    assert int(out["ordered_dense_late"]) == 2   # a dense head after a sketch head
    assert int(out["flush_null_plan"]) == 1
    assert int(out["probe_null"]) == 1    # SKSSM_EINVAL
    assert "aligned" in out["status_text"]
