"""The oracle and the C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The oracle's pins and the host ABI tests run in a child process against sanitizer
builds of the same sources, with the sanitizer runtime preloaded and any report fatal:
  * the oracle: gcc, the build of oracle/build.py with sanitize=True (oracle/liboracle_san.so),
    picked up through H3DIT_ORACLE_LIB;
  * the HIP library: its host code instrumented by clang (each -fsanitize= passed with
    -Xarch_host, so the gfx950 code is built as usual and never runs here), picked up through
    H3DIT_LIB; the host tests exercise the argument and workspace checks that run before any
    launch.
A planted heap overflow in a throwaway library shows that the harness reports."""
import glob
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def child(args, preload, env, timeout=600):
    full = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **env)
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=full, capture_output=True, text=True,
                          timeout=timeout)


MAPPED = ("import sys, ctypes; sys.path.insert(0, {root!r}); import {mod} as m; m.{load}; "
          "maps = open('/proc/self/maps').read(); "
          "assert {lib!r} in maps, 'sanitizer build not mapped'; "
          "assert {rt!r} in maps, 'sanitizer runtime not mapped'; print('mapped')")


def test_harness_reports_a_planted_overflow(tmp_path):
    rt = gcc_asan()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int poke(int n) { int *a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", *oracle_build.SAN_FLAGS, "-fPIC", "-shared", "-o", str(lib), str(src)], check=True)
    r = child(["-c", f"import ctypes; ctypes.CDLL({str(lib)!r}).poke(4)"], rt, {}, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_sanitizers():
    rt = gcc_asan()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle_build.build(sanitize=True)
    env = {"H3DIT_ORACLE_LIB": lib, "OMP_NUM_THREADS": "4"}
    r = child(["-c", MAPPED.format(root=ROOT, mod="oracle", load="lib()", lib="liboracle_san.so", rt="libasan")],
              rt, env, timeout=120)
    assert r.returncode == 0 and "mapped" in r.stdout, r.stdout + r.stderr
    r = child(["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p", "no:cacheprovider"], rt, env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def hip_file_flags():
    """Per-source flags of the library build (loaded from build.py's file, so that the package,
    which maps the library on import, is not imported here)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "h3dit_build", os.path.join(ROOT, "audio_diffusion_transformer_dit_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.FILE_FLAGS


def build_host_sanitized(out_dir):
    """The HIP library with host code under ASan + UBSan (device code as usual)."""
    file_flags = hip_file_flags()
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    srcs = sorted(glob.glob(os.path.join(ROOT, "audio_diffusion_transformer_dit_amd", "csrc", "*.hip")))
    procs, objs = [], []
    for s in srcs:
        obj = os.path.join(out_dir, os.path.basename(s) + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fvisibility=hidden", "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), *file_flags.get(os.path.basename(s), []), *san, "-c", s,
             "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-3000:]
    lib = os.path.join(out_dir, "libh3dit.so")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs]
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"):
        link += ["-Xarch_host", flag]
    subprocess.run(link, check=True, capture_output=True)
    return lib


def test_host_abi_under_sanitizers(tmp_path):
    rt = clang_asan()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    lib = build_host_sanitized(str(tmp_path))
    env = {"H3DIT_LIB": lib}
    r = child(["-c", MAPPED.format(root=ROOT, mod="audio_diffusion_transformer_dit_amd", load="lib()",
                                   lib=lib, rt="libclang_rt.asan")], rt, env, timeout=120)
    assert r.returncode == 0 and "mapped" in r.stdout, r.stdout + r.stderr
    r = child(["-m", "pytest", "tests/test_abi_host.py", "-q", "-x", "-p", "no:cacheprovider"], rt, env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
