"""CPU test runs against sanitized builds (AddressSanitizer + UndefinedBehaviorSanitizer).

    python tests/sanitize.py [-j N]

1. The C oracle (``oracle/sa_oracle.c``) is built by gcc with
   ``-fsanitize=address,undefined -fno-sanitize-recover=all`` into
   ``_build_san/libsa_oracle_san.so``, and the CPU tests that call it run
   with gcc's ASan runtime preloaded (``--oracle-lib``).
2. libsketchattn is built with the same sanitizers on its host code only
   (hipcc, each flag behind ``-Xarch_host``; the device code is unchanged)
   into ``_build_san/libsketchattn_hostsan.so``, and the ABI tests (argument
   checks, workspace sizes, offset rules, tuning, exported symbols) run with
   clang's ASan runtime preloaded (``--sa-lib``).

Before each run a canary proves that the instrumentation is live: the same
library is called once, in a child process, with a host buffer shorter than
the sizes passed with it (the mistake is planted in the call, on the CPU),
and ASan must report the overflow.

Both runs use ``detect_leaks=0`` (the Python interpreter itself is not
instrumented and keeps its allocations to the end) and ``halt_on_error=1``,
so the first report fails the run. Exit status: 0 when both runs pass.
CPU only: nothing here touches a GPU, and these builds are never loaded by
GPU tests.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

OUT = os.path.join(ROOT, "_build_san")
SAN = ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g")
# hipcc: every sanitizer flag applies to the host compilation alone.
HOST_ONLY = [f for flag in SAN for f in ("-Xarch_host", flag)]

ORACLE_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_mutants.py", "tests/test_backward_oracle.py",
                "tests/test_refine_oracle.py", "tests/test_stca_oracle.py"]
ABI_TESTS = ["tests/test_abi.py"]


def _gcc_asan() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _clang_asan() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise SystemExit("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _env(preload: str) -> dict:
    return dict(os.environ, LD_PRELOAD=preload,
                ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


# Three rows of X where the call says four: the oracle's projection reads
# past the end of X.
ORACLE_CANARY = """
import ctypes, numpy as np, oracle
lib = oracle.load({path!r})
X = np.ones((3, 4), np.float32); W = np.ones((4, 2), np.float32); out = np.zeros((4, 2))
lib.sao_project(X.ctypes.data, W.ctypes.data, 0, 4, 2, 4, None, 0, 2, out.ctypes.data)
"""
# Three offsets where the call says B = 8 users (nine entries).
ABI_CANARY = """
import ctypes, numpy as np, sketch_attention_flashsa_amd as sa
lib = sa.load_library({path!r})
cu = np.zeros(3, np.int32); bad = ctypes.c_int32()
lib.sa_check_offsets_host(cu.ctypes.data, 8, 0, ctypes.byref(bad))
"""


def _canary(preload: str, code: str, path: str) -> bool:
    r = subprocess.run([sys.executable, "-c", code.format(path=path)], cwd=ROOT, env=_env(preload),
                       capture_output=True, text=True)
    caught = r.returncode != 0 and "AddressSanitizer: heap-buffer-overflow" in r.stderr
    print(f"canary ({os.path.basename(path)}): {'reported' if caught else 'NOT reported'}", flush=True)
    return caught


def _pytest(preload: str, tests: list[str], extra: list[str]) -> int:
    env = _env(preload)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *extra, *tests]
    print("+", f"LD_PRELOAD={preload}", " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    args = ap.parse_args()
    os.makedirs(OUT, exist_ok=True)

    import oracle
    oracle_lib = oracle.build(extra_flags=("-fsanitize=address,undefined", *SAN[2:]),
                              out=os.path.join(OUT, "libsa_oracle_san.so"))
    if not _canary(_gcc_asan(), ORACLE_CANARY, oracle_lib):
        return 2
    rc = _pytest(_gcc_asan(), ORACLE_TESTS, [f"--oracle-lib={oracle_lib}"])
    if rc != 0:
        print(f"oracle tests under ASan/UBSan failed (exit {rc})")
        return rc

    from sketch_attention_flashsa_amd import build as sab
    lib = sab.build(jobs=args.j, extra=HOST_ONLY, out_dir=OUT, lib=os.path.join(OUT, "libsketchattn_hostsan.so"))
    if not _canary(_clang_asan(), ABI_CANARY, lib):
        return 2
    rc = _pytest(_clang_asan(), ABI_TESTS, [f"--sa-lib={lib}"])
    if rc != 0:
        print(f"ABI tests under host ASan/UBSan failed (exit {rc})")
        return rc
    print("sanitizer runs passed")
    return 0


if __name__ == "__main__":
    sys.exit(main())
