"""The work-claim protocol of the forward, dQ and dK/dV kernels on the host
(CPU only): tests/sanitize/claim_driver.cpp runs claim_next (plan.h, the
function the kernels call with HIP atomics) from many threads with
std::atomic counters, under ThreadSanitizer, over grids of 0 to 20,000 items
with their spare workgroups, slow and fast "XCDs" and stale counter reads.
Every item must be claimed exactly once and every other workgroup must come
away empty; a control run with a planted double claim must be caught."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_masked_attention_amd", "csrc")


def _build(tmp):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = os.path.join(tmp, "claim_driver")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
                    "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "claim_driver.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def test_every_item_is_claimed_exactly_once():
    with tempfile.TemporaryDirectory(prefix="bdattn_claim_") as tmp:
        exe = _build(tmp)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                           env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
        word, cases, steals = r.stdout.split()
        assert word == "ok" and int(cases) == 117
        assert int(steals) > 0  # workgroups did take items from other queues
        c = subprocess.run([exe, "control"], capture_output=True, text=True, timeout=300)
        assert c.returncode == 0 and c.stdout.strip().endswith("caught"), c.stdout + c.stderr
