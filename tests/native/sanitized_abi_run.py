"""Run by tests/test_sanitizers.py in a child process whose environment
preloads the clang AddressSanitizer runtime: the C ABI library built with the
host side instrumented (-fsanitize=address,undefined on the host pass only),
driven through every argument check and size query of tests/test_abi_host.py.
No GPU is touched.  Exits non-zero on the first sanitizer report."""
import inspect
import os
import sys

ROOT = sys.argv[1]
SO = sys.argv[2]
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

from fp4_routed_expert_amd import _lib  # noqa: E402

_lib.SO_PATH = SO
import test_abi_host  # noqa: E402

test_abi_host.L = _lib.lib()
n = 0
for name in sorted(dir(test_abi_host)):
    fn = getattr(test_abi_host, name)
    if name.startswith("test_") and not inspect.signature(fn).parameters:   # fixture-free checks
        fn()
        n += 1
print(f"sanitized ABI run ok: {n} host checks")
