"""Builds libb2b.so (HIP for gfx950 only) in-tree, compiling the translation
units in parallel.  Usage: python -m chip_fusion_amd.build [-j N] [--remarks]"""
import argparse
import concurrent.futures
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libb2b.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # no hand-written packed-fp32 VALU ops: keep the compiler from emitting them too
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def library_path():
    return LIB


def _code_only(text):
    """Source text without comments and with whitespace collapsed: what the
    compiler sees, so that an edited comment does not count as a new kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# sources with no cascade kernel in them: planning, validation and launch
# code, and the measurement instruments (matrix-core loop, copy and stream)
NON_CASCADE_SOURCES = ("api.hip", "plan.cpp", "plan.hpp", "microbench.hip")


def source_digest():
    """sha256 over the code (comments and layout aside) of the sources the
    cascade kernels are built from (kernel headers and instance lists), used
    to tell whether stored profiler counters still describe those kernels."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".hpp")) and os.path.basename(f) not in NON_CASCADE_SOURCES:
            h.update(os.path.basename(f).encode())
            h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def _scratch_kernels(log):
    """(kernel, bytes per lane) for every kernel of a resource-usage report that
    spills to scratch memory."""
    out, name = [], None
    for line in log.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) and name and "kernel" in name:
            out.append((name, int(m.group(1))))
    return out


def _compile(src, remarks):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-x", "hip", "-c", src, "-o", obj,
                             "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    # every kernel keeps its working set in registers and LDS
    spills = _scratch_kernels(r.stderr)
    if spills:
        raise RuntimeError(f"{os.path.basename(src)}: kernels using scratch memory: {spills}")
    return obj, r.stderr if remarks else ""


def build(jobs=None, remarks=False, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    plan_src = os.path.join(CSRC, "plan.cpp")
    jobs = jobs or min(16, os.cpu_count() or 1)
    logs = {}
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        futs = {ex.submit(_compile, s, remarks): s for s in srcs}
        plan_obj = os.path.join(BUILD, "plan.cpp.o")
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-c", plan_src, "-o", plan_obj])
        objs = [plan_obj]
        for f in concurrent.futures.as_completed(futs):
            obj, log = f.result()
            objs.append(obj)
            logs[futs[f]] = log
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + sorted(objs)
                          + ["-L/opt/rocm/lib", "-lamdhip64"])
    os.replace(tmp, LIB)
    if verbose or remarks:
        for s, log in sorted(logs.items()):
            if log.strip():
                sys.stderr.write(f"== {os.path.basename(s)}\n{log}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("--remarks", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.remarks))
