"""Build libhysparse.so (gfx950 only) in-tree from csrc/ with hipcc.

Each source compiles to an object under _build/ (in parallel), then one shared library is linked
next to this file.  Always recompiles: it is the "does it build" check.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
SO = os.path.join(HERE, "libhysparse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -fno-honor-nans: no kernel produces or tests for NaN (masked scores are -inf, never NaN), and
# without it every fmaxf operand straight from an MFMA is first re-canonicalized by an extra
# v_max_f32.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + HIP_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return src, obj, r.returncode, msg


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    objs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, msg in ex.map(_compile, srcs):
            if msg.strip() and (verbose or rc):
                print(msg, file=sys.stderr)
            if rc:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
            objs.append(obj)
    tmp = SO + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError("link of libhysparse.so failed")
    os.replace(tmp, SO)
    return SO


PROBES_SRC = os.path.join(HERE, "probes", "ceilings.hip")
PROBES_SO = os.path.join(HERE, "libhs_probes.so")


def build_probes():
    """The benchmark's measurement kernels (HBM read ceilings), a library of their own."""
    tmp = PROBES_SO + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + ["-shared", "-o", tmp, PROBES_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError("build of libhs_probes.so failed")
    os.replace(tmp, PROBES_SO)
    return PROBES_SO


if __name__ == "__main__":
    print(build(verbose=True))
