#!/usr/bin/env python3
"""The CPU test tier under AddressSanitizer and UBSan.

Builds the host code of liblinattn (argument validation, the chunk plan, the stamp, the
launch code), the fp64 oracle and the input generator with -fsanitize=address,undefined
(clang for all three, so that one sanitizer runtime serves the whole process; the library's
device code is unchanged), then runs ``pytest tests -m "not gpu"`` with that runtime
preloaded and LA_SANITIZE=1, which makes the three loaders pick the sanitized builds.
Exits with pytest's status; any sanitizer report aborts the run.

    python tests/sanitize_host.py [extra pytest arguments]
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main() -> int:
    env = dict(os.environ, LA_SANITIZE="1")
    build = ("import sys; sys.path.insert(0, %r); import importlib.util, os; "
             "import synth, oracle; synth.build(); oracle.build(); "
             "spec = importlib.util.spec_from_file_location('b', os.path.join(%r, "
             "'causal_linear_attention_tiled_amd', '_build.py')); m = importlib.util.module_from_spec(spec); "
             "spec.loader.exec_module(m); m.build(verbose=True, sanitize=True)") % (ROOT, ROOT)
    subprocess.run([sys.executable, "-c", build], env=env, check=True)
    rt = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
