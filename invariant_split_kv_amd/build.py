"""Build libisk.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python invariant_split_kv_amd/build.py [-v]   (or call build()).
Run it by path: importing the package loads the library it builds.
Always recompiles; objects go to _build/ at the repository root.
"""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libisk.so")

SOURCES = ["plan.cpp", "api.cpp", "gqa_split.hip", "mla_split.hip", "mla_split_h32.hip", "mla_h128.hip", "combine.hip",
           "rmsnorm.hip", "linear.hip", "hbm_probe.hip", "audit.hip", "noalloc.hip"]
GEN_DIR = os.path.join(BUILD_DIR, "gen")
ARCH = "gfx950"
# Packed fp32 instructions stay disabled (the compiler would otherwise form
# v_pk_* ops from scalar float code).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-I", GEN_DIR,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-fvisibility=hidden"]


# Extra flags per source.  mla_split_h32.hip keeps its output block in AGPRs
# that only its inline asm touches, so the compiler must not place MFMA
# results or VGPR spills in AGPRs there; it also owns all the LDS it uses
# (no private arrays moved into LDS behind its back).
EXTRA_FLAGS = {
    "mla_split_h32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-spill-vgpr-to-agpr=0",
                          "-mllvm", "-disable-promote-alloca-to-lds"],
    "mla_h128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-spill-vgpr-to-agpr=0",
                     "-mllvm", "-disable-promote-alloca-to-lds"],
}

# Sources whose inline asm owns registers the compiler must never touch: all
# AGPRs (the output accumulator), v231 (an asm scratch register) and
# v232..v255 (the LDS operand ring).
ASM_OWNED = ["mla_split_h32.hip"]
# mla_h128.hip keeps its output block in AGPRs between its inline-asm blocks;
# the compiler's own code may use any VGPR but no AGPR.
AGPR_OWNED = ["mla_h128.hip"]


def check_agpr_ownership(asm_text: str) -> list:
    """Instructions outside inline-asm blocks that name an AGPR (must be none)."""
    bad, in_asm = [], False
    agpr = re.compile(r"(?<![\w.])a(\d+|\[)")
    for n, line in enumerate(asm_text.splitlines(), 1):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and s and not s.startswith((";", ".")) and not s.endswith(":"):
            parts = s.split(";")[0].split(None, 1)
            if len(parts) == 2 and agpr.search(parts[1]):
                bad.append((n, s))
    return bad


def check_register_ownership(asm_text: str) -> list:
    """Instructions outside inline-asm blocks that name an AGPR or one of
    v231..v255 (must be none)."""
    bad, in_asm = [], False
    agpr = re.compile(r"(?<![\w.])a(\d+|\[)")
    ring = re.compile(r"(?<![\w.])v(23[1-9]|24\d|25[0-5])\b")
    rng = re.compile(r"v\[(\d+):(\d+)\]")
    for n, line in enumerate(asm_text.splitlines(), 1):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and s and not s.startswith((";", ".")) and not s.endswith(":"):
            parts = s.split(";")[0].split(None, 1)
            if len(parts) == 2:
                ops = parts[1]
                if agpr.search(ops) or ring.search(ops) or any(int(m.group(2)) >= 231 for m in rng.finditer(ops)):
                    bad.append((n, s))
    return bad


def check_no_scalar_loads_in_tile_loop(asm_text: str) -> list:
    """Scalar memory loads inside an inner loop (loop depth >= 2: the tile
    loop inside the segment loop).  The hand-counted LDS waits in the tile
    loop of mla_split_h32.hip are correct only while in-order LDS operations
    are the only traffic on that counter; a scalar load completes out of
    order and would break them."""
    bad, depth = [], 0
    label = re.compile(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)")
    for n, line in enumerate(asm_text.splitlines(), 1):
        s = line.strip()
        if label.match(s) or s.startswith("; =>"):
            m = re.search(r"Depth=(\d+)", s)
            if label.match(s):
                depth = int(m.group(1)) if m else 0
            elif m:
                depth = int(m.group(1))
        elif re.match(r"^(s_load|s_buffer_load)", s) and depth >= 2:
            bad.append((n, s))
        elif re.match(r"^\w+:$", s) and not s.startswith("."):
            depth = 0   # a new function
    return bad


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libisk.so; returns the library path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    # generated tile loop of the dense 128-head MLA kernel
    sys.path.insert(0, CSRC)
    try:
        import gen_mla_h128
        import check_mla_h128
    finally:
        sys.path.pop(0)
    errors = check_mla_h128.check_all()
    if errors:
        raise RuntimeError("generated MLA tile loop fails its schedule check:\n  " + "\n  ".join(errors[:10]))
    gen_mla_h128.write_header(os.path.join(GEN_DIR, "mla_h128_seg.inc"))
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    while procs:
        _wait(procs.pop(0), verbose)
    for src in ASM_OWNED:
        asm = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".device.s")
        _run([hipcc, *FLAGS, *EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-S", os.path.join(CSRC, src),
              "-o", asm], verbose)
        with open(asm) as f:
            text = f.read()
        bad = check_register_ownership(text)
        if bad:
            raise RuntimeError(f"{src}: compiler-generated code uses registers owned by inline asm: {bad[:5]}")
        bad = check_no_scalar_loads_in_tile_loop(text)
        if bad:
            raise RuntimeError(f"{src}: scalar loads inside the tile loop: {bad[:5]}")
    for src in AGPR_OWNED:
        asm = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".device.s")
        _run([hipcc, *FLAGS, *EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-S", os.path.join(CSRC, src),
              "-o", asm], verbose)
        with open(asm) as f:
            bad = check_agpr_ownership(f.read())
        if bad:
            raise RuntimeError(f"{src}: compiler-generated code uses AGPRs owned by inline asm: {bad[:5]}")
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def _wait(item, verbose):
    cmd, p = item
    out, _ = p.communicate()
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
