"""In-tree build of the gfx950 library (libmoe_hip.so) and the input generator (libsynth.so)."""
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_hip.so")
SYNTH_SRC = os.path.join(PKG, "synth", "synth.c")
SYNTH_LIB = os.path.join(PKG, "synth", "libsynth.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from emitting packed fp32 arithmetic (host pass warns: harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_synth(verbose=False):
    tmp = SYNTH_LIB + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
          "-o", tmp, SYNTH_SRC, "-lm"], verbose)
    os.replace(tmp, SYNTH_LIB)


def build_hip(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs, procs = [], []
    for s in srcs:
        o = os.path.join(BUILD_DIR, os.path.basename(s) + ".o")
        cmd = [HIPCC, *HIP_FLAGS, "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), s))
        objs.append(o)
    failed = []
    for p, s in procs:
        _, err = p.communicate()
        lines = [ln for ln in (err or "").splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(s)
            print("\n".join(lines))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    # every kernel the library launches must be defined in it (a template whose
    # host-side instantiation is dropped shows up only as an undefined symbol)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "_ZN3moe" in ln]
    if nm.returncode == 0 and missing:
        raise RuntimeError(f"libmoe_hip.so would leave library symbols undefined: {missing[:3]}")
    os.replace(tmp, LIB)


def build_all(verbose=False):
    build_synth(verbose)
    build_hip(verbose)
