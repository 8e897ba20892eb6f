"""Host sanitizers over the C ABI (no GPU): the library's host code (argument checks,
workspace layout, routing plans, the partition planner) built with AddressSanitizer and
UndefinedBehaviorSanitizer, exercised by the ABI and caller-policy host suites, which
must pass with no report. A self-check first shows that the instrumented build does
report a host over-read, so a clean run means something."""
import os
import shutil
import subprocess
import sys

import pytest

from block_sparse_attention_02_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc is needed to build the sanitized library")


def _stale():
    if not os.path.exists(build.SAN_LIB):
        return True
    t = os.path.getmtime(build.SAN_LIB)
    srcs = build._sources() + [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)
                               if f.endswith(".h")]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_env():
    if _stale():
        build.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update(H3ATTN_LIB=build.SAN_LIB, LD_PRELOAD=build.san_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("H3ATTN_FORCE_FAIL", None)
    return env


def test_sanitizer_reports_a_planted_host_overread(san_env):
    """attn_router_plan told n = 200 over a 100-byte host array reads past it: ASan must
    stop the process with a heap-buffer-overflow report."""
    code = ("import numpy as np\n"
            "from block_sparse_attention_02_amd import api\n"
            "assert api.LIB_PATH.endswith('libh3attn_san.so')\n"
            "seg = np.zeros(100, dtype=np.uint8)\n"
            "api.lib().attn_router_plan(api._np_ptr(seg), 200, 0, 64, 0.5, None, None, None, "
            "None)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


def test_abi_and_policy_suites_pass_under_sanitizers(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "tests/test_policy.py"], cwd=ROOT, env=san_env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out
