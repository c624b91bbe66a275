"""Build the host scheduler (csrc/pa_sched.cpp) on its own with the host
compiler, and run the scheduler parity tests in a child Python process bound
to that build instead of libpa.so.  Used by the sanitizer and hash-collision
tests (CPU only)."""

import os
import shutil
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_07_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CXX = shutil.which("g++")


def build(out_path, flags=(), extra_sources=(), shared=True):
    cmd = [CXX, "-O1", "-g", "-std=c++17", "-fPIC", *flags, f"-I{INCLUDE}", f"-I{CSRC}",
           os.path.join(CSRC, "pa_sched.cpp"), *extra_sources, "-o", str(out_path)]
    if shared:
        cmd.insert(1, "-shared")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(out_path)


CHILD = textwrap.dedent("""
    import ctypes, sys, types
    sys.path.insert(0, {root!r})
    sys.path.insert(0, {tests!r})
    # a stand-in package whose `lib` is the scheduler build under test: the
    # scheduler wrapper (paged_kv_attention_07_amd/sched.py) binds to it
    pkg = types.ModuleType("paged_kv_attention_07_amd")
    pkg.__path__ = [{pkgdir!r}]
    pkg.lib = ctypes.CDLL({lib!r})
    class PAError(RuntimeError):
        def __init__(self, fn, status):
            self.status = status
            super().__init__(f"{{fn}}: status {{status}}")
    pkg.PAError = PAError
    sys.modules["paged_kv_attention_07_amd"] = pkg
    {prelude}
    import pytest
    sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-o", "addopts=",
                          {test!r}]))
""")


def run_parity_child(lib, cwd, env=None, prelude=""):
    """Run tests/test_sched_parity.py against the scheduler build `lib`;
    `prelude` (Python source) runs first, after the stand-in package."""
    script = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"),
                          pkgdir=os.path.join(ROOT, "paged_kv_attention_07_amd"), lib=lib,
                          test=os.path.join(ROOT, "tests", "test_sched_parity.py"),
                          prelude=textwrap.dedent(prelude).strip())
    return subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                          env=env if env is not None else dict(os.environ), cwd=str(cwd),
                          timeout=600)
