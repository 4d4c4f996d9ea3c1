"""Host logic of the backward's one-launch schedule over packed runs (CPU only).

tests/native/check_run_tables.cpp is compiled against the library's headers and linked with the
built libtokengate.so, so it exercises the shipped plan_runs / make_tables and the work-group
decode unit_of: every (run, block, batch row x kv head) unit of random packed batches comes from
exactly one work-group of one launch, blocks stay in range, launches split at the run and range
limits, and units go out longest first.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "learned_token_pruning_gatescore_amd")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def test_run_tables_cover_every_unit_once(tmp_path):
    import learned_token_pruning_gatescore_amd as tg

    lib = tg.library_path()
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "check_run_tables")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(PKG, "csrc"), os.path.join(ROOT, "tests", "native", "check_run_tables.cpp"),
           "-L", os.path.dirname(lib), "-ltokengate", f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
