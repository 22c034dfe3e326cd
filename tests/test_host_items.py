"""Host logic: the bf16 step's list of workgroups (XCD ranges, split row groups).

tests/host/items_check.cpp compiles the host library's source into one program with its
checks (every tile exactly once, split halves adjacent inside one XCD range, the remap a
bijection, the split-count rule) and is linked with the built kernel object; no GPU call
is made."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KOBJ = os.path.join(ROOT, "partial_state_reuse_amd", "_build", "dita_kernels.o")


def test_workgroup_list(tmp_path):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    if not os.path.exists(KOBJ):
        pytest.skip("kernel object not built (partial_state_reuse_amd/build.py)")
    src = os.path.join(ROOT, "tests", "host", "items_check.cpp")
    obj, exe = str(tmp_path / "items_check.o"), str(tmp_path / "items_check")
    inc = ["-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "partial_state_reuse_amd", "csrc")]
    subprocess.run([HIPCC, "-std=c++17", "-O1", "-c", src, "-o", obj] + inc, check=True,
                   capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", obj, KOBJ, "-o", exe], check=True,
                   capture_output=True)
    env = dict(os.environ)
    env.pop("DITA_SPLITS_PER_XCD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
