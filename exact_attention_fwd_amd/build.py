"""Build the gfx950 HIP library ``libfa.so`` in-tree with hipcc.

    python -m exact_attention_fwd_amd.build        # or build() from Python

Every .hip file under csrc/ is compiled for gfx950 only and linked into one
shared library next to this file.  No JIT cache is used: the built library
lives in the package directory, so it travels with the source tree.

The build fails if any kernel spills vector registers to scratch.  Besides
the cost of scratch traffic in the hot loops, a spilling build of the dK/dV
kernel was miscompiled: a spilled 16-byte MFMA operand was reloaded as 12
bytes into accumulation registers whose fourth register was never written
(its copy was kept in another register that the reload on that path did
not read back), which produced NaN gradients.  Keeping every kernel free of
spills keeps that code path out of the compiler entirely.

It also fails if the device assembly of any kernel places an inline-asm
matrix instruction closer to a dependent instruction than the wait states
gfx950 requires (asm_lint): the compiler pads only the instructions it emits
itself.  Each source is compiled a second time with -S for that check, with
the same flags, in parallel with the object build.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libfa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # never emit packed fp32 VALU ops (v_pk_fma/add/mul_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # per-kernel register / LDS / spill report, parsed by _check_resources()
    "-Rpass-analysis=kernel-resource-usage",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every kernel source and link libfa.so; returns its path."""
    cc = hipcc()
    srcs = sources()
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs, asms, procs = [], [], []
        asm_flags = [f for f in HIPCC_FLAGS if not f.startswith("-Rpass")]
        for src in srcs:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            asm = os.path.join(tmp, os.path.basename(src) + ".s")
            for cmd, check in (([cc, *HIPCC_FLAGS, "-I", INCLUDE, "-c", src, "-o", obj], True),
                               ([cc, *asm_flags, "-I", INCLUDE, "--cuda-device-only", "-S", src, "-o", asm], False)):
                if verbose:
                    print(" ".join(cmd), flush=True)
                procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), check))
                if len(procs) >= jobs:
                    _wait(procs.pop(0), verbose)
            objs.append(obj)
            asms.append(asm)
        for p in procs:
            _wait(p, verbose)
        _lint(asms, verbose)
        out_tmp = LIB_PATH + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp,
                "-Wl,-rpath,/opt/rocm/lib"]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def kernel_resources(text: str):
    """Parse the kernel-resource-usage remarks: {kernel: {field: value}}."""
    out, name = {}, None
    for ln in text.splitlines():
        if "remark:" not in ln:
            continue
        body = ln.split("remark:", 1)[1].split(" [-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            name = val
            out[name] = {}
        elif name is not None and val:
            out[name][key] = val
    return out


def _check_resources(src, text):
    res = kernel_resources(text)
    bad = {k: v for k, v in res.items() if int(v.get("VGPRs Spill", "0")) > 0}
    if bad:
        lines = [f"  {k}: {v.get('VGPRs Spill')} VGPRs spilled" for k, v in bad.items()]
        raise RuntimeError(f"{os.path.basename(src)}: kernels spill vector registers (refused):\n" + "\n".join(lines))
    return res


def _lint(asms, verbose):
    from . import asm_lint
    found = []
    for path in asms:
        with open(path) as f:
            found.extend(asm_lint.check(f.read()))
    if found:
        shown = "\n".join(str(x) for x in found[:20])
        raise RuntimeError(f"inline-asm matrix instructions closer than gfx950's wait states "
                           f"({len(found)} pairs, refused):\n{shown}")
    if verbose:
        print(f"asm lint: {len(asms)} sources, no inline-asm wait-state violations", flush=True)


def _wait(item, verbose):
    src, p, check = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
    # (the remarks' source excerpts are the lines starting with "<n> |" or "|")
    lines = [ln for ln in text.splitlines()
             if "packed-fp32-ops" not in ln and "remark:" not in ln and not re.match(r"\s*(\d+\s*)?\|", ln)]
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(lines))
    if not check:
        return
    res = _check_resources(src, text)
    if verbose:
        if lines:
            print("\n".join(lines), flush=True)
        for k, v in res.items():
            print(f"  {k[:90]}: VGPR {v.get('VGPRs')} AGPR {v.get('AGPRs')} LDS {v.get('LDS Size [bytes/block]')} "
                  f"occupancy {v.get('Occupancy [waves/SIMD]')}", flush=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
