"""Build libwq.so in place: the HIP kernels and the host C++ in one shared library, for gfx950 only.

Run ``python -m weight_only_quantized_dequant_amd.build`` (or call ``build()``). It always
recompiles: every source to an object (in parallel), then one link. The result lands next to
this file, so it travels with the source tree.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwq.so")
# the plain-read probe that bench.py times beside the linears (measurement only, not libwq)
PROBE_SRC = os.path.join(CSRC, "probe", "read_floor.hip")
PROBE_LIB = os.path.join(HERE, "libwq_probe.so")
ARCH = "gfx950"

# Flags of one translation unit only. The prefill kernel keeps its MFMA accumulators in VGPRs:
# in AGPRs its loop copied all of them every iteration and needed over 256 registers per lane.
EXTRA_FLAGS = {"wq_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; libwq needs ROCm to build")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that line is noise
    noise = "is not a recognized feature for this target"
    return r.returncode, [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]


def build(verbose=False):
    """Compile csrc/*.hip and csrc/*.cpp into libwq.so, and csrc/probe/read_floor.hip into
    libwq_probe.so. Returns the path of libwq.so."""
    names = [f for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    common = [hipcc(), "--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC",
              # packed fp32 VALU ops stay off: the compiler must not form v_pk_{add,mul,fma}_f32
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-result", "-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="wqbuild") as tmpdir:
        objs = [os.path.join(tmpdir, n + ".o") for n in names]
        jobs = [common + EXTRA_FLAGS.get(n, []) + ["-c", os.path.join(CSRC, n), "-o", o] for n, o in zip(names, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), 4)) as ex:
            results = list(ex.map(_run, jobs))
        msgs = [l for _, m in results for l in m]
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("libwq build failed:\n" + "\n".join(msgs))
        tmp = LIB + ".tmp%d" % os.getpid()
        rc, m = _run([hipcc(), "--offload-arch=%s" % ARCH, "-fPIC", "-shared", *objs, "-o", tmp, "-lpthread"])
        msgs += m
        if rc != 0:
            raise RuntimeError("libwq link failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    rc, m = _run(common + ["-shared", PROBE_SRC, "-o", tmp])
    if rc != 0:
        raise RuntimeError("libwq_probe build failed:\n" + "\n".join(m))
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
