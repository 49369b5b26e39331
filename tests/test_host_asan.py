"""The library's host code under AddressSanitizer (CPU only).

ds_rows.hip (argument checks, ragged tables, overlap tests, staging) is
compiled again with AddressSanitizer on its host side and linked with the
other objects of the normal build; the C-ABI tests and the binding's checks
then run against that library in a child process with the sanitizer's
runtime preloaded.  Any invalid host memory access aborts the child.
"""
import os
import shlex
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "scale_invariant_row_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
OTHERS = ["inst_l2.o", "inst_slerp.o", "inst_rownorm.o", "inst_l2_bwd.o", "inst_rownorm_bwd.o",
          "inst_act.o", "inst_qk.o", "inst_rescale.o", "inst_rms.o", "inst_rms_bwd.o",
          "inst_colblock.o"]


def asan_runtime():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    for cmd in ([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],):
        try:
            p = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            path = p.stdout.strip()
            if os.path.isabs(path) and os.path.exists(path):
                return hipcc, path
        except OSError:
            pass
    base = "/opt/rocm/llvm/lib/clang"
    if os.path.isdir(base):
        for v in sorted(os.listdir(base), reverse=True):
            path = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(path):
                return hipcc, path
    return hipcc, None


def test_host_abi_under_address_sanitizer(tmp_path):
    hipcc, runtime = asan_runtime()
    objs = [os.path.join(BUILD, o) for o in OTHERS]
    if not os.path.exists(hipcc) or runtime is None or not all(map(os.path.exists, objs)):
        pytest.skip("needs hipcc, the sanitizer runtime and a built library (_build objects)")
    obj = str(tmp_path / "ds_rows_asan.o")
    lib = str(tmp_path / "libdsrows_asan.so")
    flags = ("--offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -ffp-contract=off "
             "-Xclang -target-feature -Xclang -packed-fp32-ops "
             "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    cc = subprocess.run([hipcc, *shlex.split(flags), *inc, "-c", os.path.join(CSRC, "ds_rows.hip"),
                         "-o", obj], capture_output=True, text=True, timeout=600)
    assert cc.returncode == 0, cc.stdout + cc.stderr
    link = shlex.split("--offload-arch=gfx950 -shared -Xarch_host -fsanitize=address")
    ld = subprocess.run([hipcc, *link, "-o", lib, obj, *objs], capture_output=True, text=True,
                        timeout=600)
    assert ld.returncode == 0, ld.stdout + ld.stderr
    env = dict(os.environ, LD_PRELOAD=runtime, DS_ROWS_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1")
    probe = ("import sys; sys.path.insert(0, %r); from scale_invariant_row_amd import binding; "
             "binding.lib(); print(binding.LIB_PATH); "
             "print(any('asan' in l for l in open('/proc/self/maps')))" % ROOT)
    p = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0, p.stderr
    assert p.stdout.split() == [lib, "True"], p.stdout
    t = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"),
                        os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = t.stdout + t.stderr
    assert t.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
