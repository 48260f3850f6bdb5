"""Host-side contracts of the entry points (no GPU): the bench refuses more
than one GPU with a message, and the binding fails loudly (no fallback of
any kind) when the HIP library is absent."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no bench line is printed


def test_binding_fails_loudly_without_the_library(tmp_path):
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from gated_deltanet_recurrence_frame_amd import binding as gb\n"
        "gb.LIB_PATH = %r\n"
        "try:\n"
        "    gb.lib()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(1)\n" % (ROOT, str(tmp_path / "missing" / "libgdn.so")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout
