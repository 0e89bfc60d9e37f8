"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Built here with the sanitizers on the host side only (the device code of
the .hip sources is compiled as usual):
  * the C ABI library: argument checks, workspace sizing, schedule choice
    and the launch plans (hipcc, each -fsanitize after -Xarch_host);
  * the C oracle (clang, without OpenMP).
The host tests (not gpu) then run against both builds in a child process
with clang's sanitizer runtime preloaded; any report ends it with a non-zero
status.  A planted out-of-bounds read and a planted oversized shift, built
the same way, must end their process with a report, which shows the
sanitizers are live in that set-up.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang"
RT = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
OUT = os.path.join(ROOT, "bit_weight_gemm_amd", "_build_asan")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not RT or not os.path.exists(CLANG),
                                reason="clang's sanitizer runtime is not installed")


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s)
                                          for s in sources)


def _sanitized_library() -> str:
    from bit_weight_gemm_amd import build as hb
    lib = os.path.join(OUT, "libbiloco_hip_asan.so")
    srcs = [os.path.join(hb.CSRC, s) for s in hb.SOURCES]
    hdrs = [os.path.join(hb.CSRC, h) for h in hb.HEADERS]
    if _newer(lib, srcs + hdrs):
        return lib
    os.makedirs(OUT, exist_ok=True)
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [hb.HIPCC] + hb.COMMON + host_san + ["-g", "-x", "hip", "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        objs.append(obj)
    for p, src in zip(procs, srcs):
        out = p.communicate()[0]
        assert p.returncode == 0, f"{src}:\n{out.decode()[-3000:]}"
    subprocess.check_call([hb.HIPCC, f"--offload-arch={hb.ARCH}", "-shared", "-fPIC", "-o",
                           lib] + objs)
    return lib


def _sanitized_c(src, name) -> str:
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, name)
    if not _newer(lib, [src]):
        subprocess.check_call([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c11"] + SAN +
                              ["-o", lib, src, "-lm"])
    return lib


def _env(**extra):
    env = dict(os.environ, LD_PRELOAD=RT[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(extra)
    return env


def test_planted_faults_are_reported():
    src = os.path.join(OUT, "planted.c")
    os.makedirs(OUT, exist_ok=True)
    with open(src, "w") as f:
        f.write(textwrap.dedent("""
            #include <stdlib.h>
            int planted_oob(int i) { int *a = malloc(4 * sizeof(int)); a[0] = 1;
                                     int v = a[i]; free(a); return v; }
            int planted_shift(int s) { return 1 << s; }
        """))
    lib = _sanitized_c(src, "libplanted.so")
    for call, report in (("planted_oob(5)", "heap-buffer-overflow"),
                         ("planted_shift(40)", "shift exponent")):
        code = f"import ctypes; L = ctypes.CDLL({lib!r}); print(L.{call})"
        p = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True,
                           text=True, timeout=120)
        assert p.returncode != 0 and report in p.stderr, (call, p.stderr[-2000:])
    # the same process with in-bounds arguments runs clean
    code = f"import ctypes; L = ctypes.CDLL({lib!r}); print(L.planted_oob(0), L.planted_shift(3))"
    p = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 0 and p.stdout.split() == ["1", "8"], p.stderr[-2000:]


def test_host_suite_under_sanitizers():
    lib = _sanitized_library()
    orc = _sanitized_c(os.path.join(ROOT, "oracle", "biloco_oracle.c"), "liboracle_biloco_asan.so")
    env = _env(BILOCO_HIP_LIB=lib, BILOCO_ORACLE_LIB=orc)
    # the child loads the sanitized builds, not the product ones
    code = ("import sys; sys.path.insert(0, %r); from bit_weight_gemm_amd import binding as B; "
            "import oracle; B.lib(); print(B.LIB_PATH); print(oracle.build())" % ROOT)
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0 and p.stdout.split() == [lib, orc], p.stdout + p.stderr[-2000:]
    tests = sorted(set(glob.glob(os.path.join(ROOT, "tests", "test_*.py"))) -
                   {os.path.abspath(__file__)})
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + tests
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, tail
    assert "Sanitizer" not in p.stderr, tail
    assert " passed" in p.stdout, tail
