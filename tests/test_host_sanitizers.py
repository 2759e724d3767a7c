"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): a copy of librlmoe built with both sanitizers on its host side runs
the expert-cache and C-ABI host tests in a child process that preloads the
ASan runtime.  A canary first checks that the instrumentation is live: a
table buffer one entry short must be reported as a heap overflow."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from quantized_routed_expert_rl_amd import build_sanitized as S  # noqa: E402

pytestmark = pytest.mark.skipif(
    shutil.which(S.B.HIPCC) is None and not os.path.exists(S.B.HIPCC) or S.asan_runtime() is None,
    reason="needs hipcc and clang's ASan runtime")


@pytest.fixture(scope="module")
def sanitized_env():
    lib = S.build()
    env = dict(os.environ)
    env.update(RLMOE_LIB=lib, LD_PRELOAD=S.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _run(env, args, timeout=600):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


CANARY = """
import ctypes as C, numpy as np
from quantized_routed_expert_rl_amd import binding as B
c = B.lib.rl_cache_create(4, 2, 8)
short = np.zeros(2 * 8 - 1, np.int32)           # one entry short of [2 x 8]
B.lib.rl_cache_table(c, short.ctypes.data)
print("no report")
"""


def test_sanitizer_reports_a_host_overflow(sanitized_env):
    r = _run(sanitized_env, ["-c", CANARY])
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]


def test_host_tests_clean_under_sanitizers(sanitized_env):
    r = _run(sanitized_env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_cache.py",
                             "tests/test_abi_host.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
