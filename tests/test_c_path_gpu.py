"""The path driven from a plain C99 program (tests/c/path_from_c.c): device
buffers from the HIP runtime's C API, one caller-created stream; the flat path
(ep_get_layout -> ep_dispatch -> ep_combine) and the two-level one
(ep_hierarchical_dispatch -> ep_combine on chunked rows, ep_combine_two_level)
and the several-source one (ep_source_layout -> ep_source_dispatch_fused)
through libep.so, every output compared bit for bit with the CPU oracle inside
the same program."""
import os
import shutil
import subprocess

import pytest
import torch

import oracle
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_path_from_c(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    ep.lib()
    oracle.build(force=False)
    libdir = os.path.dirname(ep.LIB_PATH)
    odir = os.path.join(ROOT, "oracle")
    exe = str(tmp_path / "path_from_c")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "c", "path_from_c.c"),
           f"-L{libdir}", "-l:libep.so", f"-L{odir}", "-l:liboracle.so", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{odir}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "path ok" in r.stdout
