"""Build the gfx950 HIP library libthrift.so in-tree (and the test-only
arithmetic probes, tests/libarith_probe.so).

Each HIP source is compiled for gfx950 only, in parallel, then linked into
one shared library next to this file.  Packed fp32 instructions are turned
off (-packed-fp32-ops): fp32 code stays on the scalar-per-lane VALU forms.
The backward's kernels ask for the VGPR form of the matrix instructions:
their products feed VALU work directly, and with results in accumulation
registers the compiler copied every one of them back per tile.  The forward
source is built without NaN semantics (-fno-honor-nans): its inputs are
finite, masked scores are -inf and never NaN, and with NaNs honoured every
maximum of matrix-instruction results is preceded by a canonicalising
self-maximum (five VALU instructions of the MX tile's 219).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libthrift.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["select.hip", "quantize.hip", "attention.hip", "backward.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]
EXTRA = {"backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"], "attention.hip": ["-fno-honor-nans"]}


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))


PROBE_SRC = os.path.join(ROOT, "tests", "arith_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "libarith_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The arithmetic probes of the tests (not part of the library)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-shared", "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on arith_probe.hip:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
