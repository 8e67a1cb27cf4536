"""The host builder, the forest accessors and host packing under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host-only entry points are compiled by g++ with both sanitizers into a
library of their own (prefix_shared_tree_packed_amd.build.build_host_sanitized;
no HIP code is in it), and the host parity suites run against it in a child
Python with libasan preloaded: the builder against the oracle on the worked
examples, brute-force cases and every workload, the C-ABI argument checks,
and FFD / Karmarkar-Karp against the oracle.  Any sanitizer report aborts the
child (halt_on_error), which fails this test.  Leak checking is off: the
interpreter itself never frees some of its memory.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# tests of device entry points need the full library (and a GPU for the
# metadata upload), so they stay out of the sanitized run, as does the
# export check of every declared symbol; the two largest workloads (long,
# long_control) are left to the unsanitized suite to keep the run short
HOST_ONLY = ("not device_entry_points and not meta_create and not forest_meta "
             "and not exports_every and not long")


def test_host_suites_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from prefix_shared_tree_packed_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), asan
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=asan,
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        PST_LIBRARY=lib,
    )
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", HOST_ONLY,
           "tests/test_builder_parity.py", "tests/test_capi.py", "tests/test_packing_parity.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-40:])
    assert r.returncode == 0, f"sanitized host suites failed ({r.returncode}):\n{tail}"
    assert " passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
