"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

* The oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined and
  its pin tests run against that build.
* The library's host code (api.cpp: argument validation and dispatch;
  pack_host.cpp: the host packer) is rebuilt with the sanitizers on the host
  side only (device code is never instrumented), linked with the library's
  ordinary device objects, and the C-ABI tests run against that build.

Each run happens in a child process that preloads the matching sanitizer
runtime; any report aborts the child (-fno-sanitize-recover=all), so the
test passes only on a clean run.  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_bit_e2m1_amd", "csrc")
ORACLE_TESTS = ["tests/test_oracle_codec.py", "tests/test_oracle_pack.py", "tests/test_oracle_gather.py",
                "tests/test_oracle_rmsnorm.py"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _child(code, preload, tmp_path):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = f"detect_leaks=0:abort_on_error=0:log_path={tmp_path}/asan"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:log_path={tmp_path}/ubsan"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = ""
    for f in sorted(os.listdir(tmp_path)):
        if f.startswith(("asan", "ubsan")):
            with open(os.path.join(tmp_path, f)) as fh:
                reports += fh.read()
    assert r.returncode == 0 and not reports, f"rc={r.returncode}\n{reports}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fno-fast-math", "-fPIC", "-shared", "-pthread", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    rt = " ".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                  for n in ("libasan.so", "libubsan.so"))
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            f"import oracle; oracle._LIB = {lib!r}\n"
            "assert oracle.lib()._name == oracle._LIB\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', *{ORACLE_TESTS!r}]))\n")
    out = _child(code, rt, tmp_path)
    assert " passed" in out


def test_host_library_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    build = os.path.join(ROOT, "_build")
    dev = sorted(os.path.join(build, f) for f in os.listdir(build) if f.endswith(".hip.o")) \
        if os.path.isdir(build) else []
    if len(dev) < len([f for f in os.listdir(CSRC) if f.endswith(".hip")]):
        from block_scaled_bit_e2m1_amd import build as b
        b.build()
        dev = sorted(os.path.join(build, f) for f in os.listdir(build) if f.endswith(".hip.o"))
    host = []
    for name in ("api", "pack_host"):
        obj = str(tmp_path / f"{name}.o")
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
        for flag in SAN:
            cmd += ["-Xarch_host", flag]
        cmd += ["-x", "hip", "-c", os.path.join(CSRC, f"{name}.cpp"), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        host.append(obj)
    lib = str(tmp_path / "libbsq_san.so")
    subprocess.run([clang, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", *host, *dev,
                    "-o", lib, "-L/opt/rocm/lib", "-lamdhip64", "-lpthread", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True)
    rt = subprocess.check_output([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "from block_scaled_bit_e2m1_amd import bsq\n"
            f"bsq.LIB_PATH = {lib!r}\n"
            "assert bsq.lib()._name == bsq.LIB_PATH\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))\n")
    out = _child(code, rt, tmp_path)
    assert " passed" in out
