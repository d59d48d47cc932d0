"""The C ABI from a plain C program, without Python or torch in between:
tests/c_abi_consumer.c is compiled with gcc against include/attn.h and the
in-tree libattn.so (a second or so; no GPU code is built) and run as a
child process on the GPU.  It checks attn_fwd against a closed form (Q = 0:
each output row is the mean of the V rows it sees, LSE = ln of their count),
the ABI version and a rejected call."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "exact_attention_forward_06_amd")


def test_c_consumer_closed_form(tmp_path):
    gcc = shutil.which("gcc")
    assert gcc, "gcc not found"
    assert os.path.exists(os.path.join(LIB_DIR, "libattn.so")), "libattn.so is not built"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "c_abi_consumer")
    cmd = [gcc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_abi_consumer.c"),
           f"-L{rocm}/lib", "-lamdhip64", f"-L{LIB_DIR}", "-l:libattn.so",
           f"-Wl,-rpath,{LIB_DIR}:{rocm}/lib", "-lm", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stdout + b.stderr
    print("running the C consumer", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
