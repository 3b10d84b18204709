"""The host-only C++ of the library under the compiler's sanitizers (CPU).

* The NF4 host codec (csrc/nf4_host.cpp, the load-time quantizer of the
  frozen base) with AddressSanitizer and UndefinedBehaviorSanitizer, and its
  multithreaded path with ThreadSanitizer: tests/codec_host_check.cpp
  quantizes, checks, dequantizes and requantizes seeded weights of several
  lengths (exact round trip).
* The slot scheduler (csrc/sched.h) driven by the discrete-event simulation
  of tests/sched_sim.cpp, with AddressSanitizer and UndefinedBehaviorSanitizer.

The device-side runtime needs a GPU; its ordering is covered by the
simulation here and by the fault-injection and serialized-run tests on the
GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CODEC = os.path.join(ROOT, "layer_streamed_nf4_double_amd", "csrc", "nf4_host.cpp")
GXX = shutil.which("g++")
pytestmark = pytest.mark.skipif(GXX is None, reason="g++ not available")


def _build(tmp_path, name, srcs, san):
    exe = str(tmp_path / name)
    cmd = [GXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", f"-fsanitize={san}",
           "-pthread"] + srcs + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_host_codec_under_sanitizers(tmp_path, san):
    out = _run(_build(tmp_path, "codec", [os.path.join(ROOT, "tests", "codec_host_check.cpp"), CODEC],
                      san))
    assert out.startswith("ok "), out


def test_scheduler_simulation_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "sched", [os.path.join(ROOT, "tests", "sched_sim.cpp")], "address,undefined")
    for scen, L, n in [("sft", 8, 2), ("sfth", 8, 3), ("dpo", 5, 2), ("dpoh", 32, 4)]:
        out = _run(exe, scen, L, n, 3, 7)
        assert out.startswith("loads "), out
