"""Host sanitizers (CPU only): AddressSanitizer and UndefinedBehaviorSanitizer
over the oracle and over the library's host code.

- The oracle (oracle/thrift_oracle.c) is rebuilt with both sanitizers and
  its pin suites run against that build.
- The library's sources are rebuilt with both sanitizers on the host side
  only (device code as usual) and the ABI tests run against that build:
  every call there fails argument validation, so the host paths that check
  arguments, size workspaces and prepare launches are what runs.

Each suite runs in a subprocess with the sanitizer runtime preloaded into
the interpreter; any report ends it with a failure.  Nothing here touches a
GPU.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_select.py", "tests/test_oracle_attention.py",
        "tests/test_oracle_decode.py", "tests/test_oracle_select_head.py", "tests/test_oracle_backward.py",
        "tests/test_oracle_fp8.py"]
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _reports(prefix):
    """Text of the sanitizer logs written under prefix.<pid>."""
    out = []
    for p in glob.glob(prefix + ".*"):
        with open(p) as f:
            out.append(f.read())
    return "\n".join(out)


def _run(cmd, env, log_prefix):
    env = dict(os.environ, **env)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={log_prefix}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:log_path={log_prefix}"
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    rep = _reports(log_prefix)
    assert r.returncode == 0 and not rep, f"sanitizer run failed (rc {r.returncode}):\n{rep[-3000:]}\n" \
                                          f"{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math"] + SAN + ["-I", os.path.join(ROOT, "oracle"), "-o", lib,
                                               os.path.join(ROOT, "oracle", "thrift_oracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + PINS,
         {"THRIFT_ORACLE_LIB": lib, "LD_PRELOAD": asan}, str(tmp_path / "oracle_san"))


def test_library_host_code_under_asan_ubsan(tmp_path):
    from fp16_attention_amd import build

    # sanitizers on the host compilation only: -Xarch_host before each flag
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    objs = [str(tmp_path / s.replace(".hip", ".o")) for s in build.SOURCES]

    def compile_one(so):
        src, obj = so
        cmd = [build.HIPCC] + build.FLAGS + build.EXTRA.get(src, []) + host_san + \
              ["-c", os.path.join(build.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)

    with cf.ThreadPoolExecutor(max_workers=len(objs)) as ex:
        list(ex.map(compile_one, zip(build.SOURCES, objs)))
    lib = str(tmp_path / "libthrift_san.so")
    subprocess.run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-o", lib] + objs, check=True, capture_output=True)
    clang = os.path.join(os.path.dirname(build.HIPCC), "..", "llvm", "bin", "clang")
    asan = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.fail(f"the compiler's ASan runtime is missing: {asan}")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import fp16_attention_amd._lib as L\n"
            "L.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n" % (ROOT, lib))
    _run([sys.executable, "-c", code], {"LD_PRELOAD": asan}, str(tmp_path / "lib_san"))
