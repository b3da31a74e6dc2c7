"""AddressSanitizer runs on the CPU (no GPU needed):

1. the host code of libmaxsim.so (the C-ABI argument checks, workspace and layout
   arithmetic, the one-shot workspace cache's lookup) built with ASan in its host pass
   only, device code unchanged, then tests/test_abi.py and tests/test_binding_host.py
   run against it with clang's ASan runtime preloaded;
2. the oracle's C built with gcc's ASan, then the oracle's pin suites run against it
   with gcc's ASan runtime preloaded.

    python tests/asan/run_asan.py [out_dir]

Exit status 0 when both runs pass with no ASan report.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from late_interaction_reranking_amd import build as libbuild  # noqa: E402

ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, env=env, capture_output=True, text=True)
    sys.stdout.write(r.stdout[-4000:])
    sys.stderr.write(r.stderr[-4000:])
    return r.returncode, r.stdout + r.stderr


def main() -> int:
    out = sys.argv[1] if len(sys.argv) > 1 else tempfile.mkdtemp(prefix="maxsim_asan_")
    os.makedirs(out, exist_ok=True)
    hipcc = libbuild._hipcc()
    # 1. libmaxsim with the host pass sanitised: the host unit rebuilt, the kernel units reused.
    libbuild.build()
    host_o = os.path.join(out, "host_asan.o")
    rc, _ = run([hipcc, *libbuild.HIPCC_FLAGS, *libbuild.NO_NAN_DEVICE, *ASAN_HOST, "-c",
                 os.path.join(libbuild.CSRC, "maxsim_host.hip"), "-o", host_o])
    if rc:
        return rc
    objs = [o for _, _, o in libbuild.units() if not o.endswith("host.o")] + [host_o]
    lib = os.path.join(out, "libmaxsim_asan.so")
    rc, _ = run([hipcc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", *ASAN_HOST,
                 "-Xarch_host", "-shared-libsan", "-o", lib, *objs])
    if rc:
        return rc
    clang_rt = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                              text=True).stdout.strip()
    env = dict(os.environ, MAXSIM_LIBRARY=lib, LD_PRELOAD=clang_rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    rc1, text1 = run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                      os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_binding_host.py")],
                     env=env)
    # 2. the oracle with gcc's ASan
    import oracle

    olib = os.path.join(out, "liboracle_asan.so")
    rc, _ = run(["gcc", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-fopenmp",
                 "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", olib, oracle.SOURCE, "-lm"])
    if rc:
        return rc
    gcc_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, MAXSIM_ORACLE_LIBRARY=olib, LD_PRELOAD=gcc_rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    pins = [os.path.join(ROOT, "tests", f) for f in ("test_oracle.py", "test_oracle_golden.py", "test_oracle_pairs.py",
                                                      "test_oracle_fp8.py", "test_oracle_topk.py")]
    rc2, text2 = run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *pins], env=env)
    bad = [t for t in (text1, text2) if "AddressSanitizer" in t]
    print(f"\nASan host C-ABI run: rc {rc1}; oracle run: rc {rc2}; ASan reports: {len(bad)}")
    return 0 if rc1 == 0 and rc2 == 0 and not bad else 1


if __name__ == "__main__":
    sys.exit(main())
