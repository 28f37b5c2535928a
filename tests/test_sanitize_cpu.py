"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): api.hip and noalloc.hip are rebuilt with the sanitizers on their
host pass only (-Xarch_host), linked with the other kernels' objects, and a
small C++ driver (tests/sanitize/abi_errors.cpp) calls every entry point with
arguments it must reject, and the size queries, without a device."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "hierarchical_sparse_attention_summaries_amd")
CSRC = os.path.join(PKG, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"   # the host compiler behind hipcc (same sanitizer runtime)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# the host-code sources the sanitizers check; the others are kernels plus launch stubs
CHECKED = ("api.hip", "noalloc.hip")


def _build_flags():
    import importlib.util
    spec = importlib.util.spec_from_file_location("hga_build_script_san",
                                                  os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.FLAGS, mod.sources()


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="no hipcc")
def test_host_code_under_asan_and_ubsan(tmp_path):
    flags, srcs = _build_flags()
    objs = []
    for src in srcs:
        name = os.path.basename(src)
        obj = str(tmp_path / (name + ".o"))
        extra = SAN if name in CHECKED else []
        prebuilt = os.path.join(ROOT, "_build", name + ".o")
        if not extra and os.path.exists(prebuilt) and \
                os.path.getmtime(prebuilt) >= os.path.getmtime(src):
            objs.append(prebuilt)       # a kernel object the last build() made
            continue
        _run([HIPCC, *flags, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_errors.o")
    # the driver is plain host C++ (no HIP): the host compiler alone
    _run([CLANGXX, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(ROOT, "tests", "sanitize", "abi_errors.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_errors")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
