"""The host layer of the C ABI (argument checks, planning, the block-table
check) under AddressSanitizer: libmla is rebuilt with its host code
instrumented (device code as usual) and tests/test_abi.py runs against it in a
child process with the clang ASan runtime preloaded.  Every call there returns
before any launch, so this runs without a GPU.  Any out-of-bounds or
use-after-free access in the host code aborts the child with an ASan report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_host_code_is_clean_under_asan():
    from mla_latent_kv_23_amd import build as Bu
    lib = Bu.build_asan()
    env = dict(os.environ, MLA_LIBRARY=lib, LD_PRELOAD=Bu.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    # the child also checks that it really loaded the instrumented build
    probe = ("import mla_latent_kv_23_amd as M; M.load_library(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libmla_asan.so' in maps and 'libclang_rt.asan' in maps, 'ASan build not loaded'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
