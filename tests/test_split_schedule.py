"""Host logic of the split decode schedule (no GPU): builds tests/split_sched_check.cpp against
the library's schedule source with hipcc and runs it (see that file for what it checks)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_split_schedule_covers_every_step_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_sched_check")
    cmd = [hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "split_sched_check.cpp"),
           os.path.join(ROOT, "tenant_serving_bitdelta_amd", "csrc", "split_sched.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().startswith("ok"), r.stdout[-4000:]


def test_split_schedule_under_host_sanitizers(tmp_path):
    """The same checks with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
    planner's tables, the piece map and the schedule cache)."""
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_sched_check_san")
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "split_sched_check.cpp"),
           os.path.join(ROOT, "tenant_serving_bitdelta_amd", "csrc", "split_sched.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower() and "not found" in r.stderr:
        pytest.skip("sanitizer runtime not available")
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip().startswith("ok"), (r.stdout + r.stderr)[-4000:]
