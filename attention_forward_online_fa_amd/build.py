"""Ahead-of-time build of libfa.so for gfx950 with hipcc.

The library is built in-tree (next to this file) so that it travels with the
source tree; nothing is JIT-compiled at run time.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
# Hash of the sources and flags a library was built from, written beside it.
HASH_PATH = LIB_PATH + ".srchash"
SOURCES = [os.path.join(CSRC, "fa_fwd.hip"), os.path.join(CSRC, "fa_api.cpp"),
           os.path.join(CSRC, "fa_bwd.hip"), os.path.join(CSRC, "fa_bwd_f32.hip"),
           os.path.join(CSRC, "fa_bwd_api.cpp"),
           os.path.join(CSRC, "fa_noalloc.hip")]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source compiler flags on top of HIP_FLAGS (by file name).
# fa_bwd_f32.hip: VGPR-form MFMAs (the fp32 D = 128 backward kernels run one
# wavefront per SIMD, where the default AGPR form costs register moves).
FILE_FLAGS: dict = {"fa_bwd_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_files() -> list:
    """Every file the library is compiled from: the sources, the internal
    headers under csrc/ and the public header."""
    hdrs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    return [*SOURCES, *hdrs, os.path.join(INCLUDE, "fa.h")]


def source_hash() -> str:
    """sha256 over the compiler flags and every file of source_files()."""
    h = hashlib.sha256(" ".join(HIP_FLAGS).encode() + repr(sorted(FILE_FLAGS.items())).encode())
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def built_hash():
    """The source hash recorded when the library on disk was built, or None."""
    try:
        with open(HASH_PATH) as fh:
            return fh.read().strip()
    except OSError:
        return None


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Kernels allowed to use private (scratch) memory. Every other kernel must keep
# all its state in registers and LDS; scratch traffic would dominate its time.
SCRATCH_ALLOWED = ("fwd_f32_kernelILi256E",)


def parse_resource_usage(remarks: str) -> dict:
    """Per-kernel {name: {"vgpr":, "agpr":, "scratch":, "vgpr_spill":, "lds":}} from
    hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split(" [-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in body:
            k, v = body.rsplit(":", 1)
            if k.strip() in keys:
                try:
                    out[cur][keys[k.strip()]] = int(v.strip())
                except ValueError:
                    pass
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into libfa.so (always recompiles) and record the
    source hash beside it. Returns the path.

    Fails if a kernel outside SCRATCH_ALLOWED uses scratch memory."""
    digest = source_hash()
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cc = hipcc()
    objdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        def compile_one(src):
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [cc, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
                   "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC, "-c", src,
                   "-o", obj]
            return cmd, obj, subprocess.run(cmd, capture_output=True, text=True)

        jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, SOURCES))
        remarks = ""
        for cmd, _, res in results:
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd)}")
            remarks += res.stderr
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _ in results],
                "-o", tmp]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError(f"link failed with status {res.returncode}: {' '.join(link)}")
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    usage = parse_resource_usage(remarks)
    bad = [k for k, u in usage.items()
           if u.get("scratch", 0) > 0 and not any(a in k for a in SCRATCH_ALLOWED)]
    if verbose:
        for k, u in sorted(usage.items()):
            sys.stderr.write(f"{k}: {u}\n")
    if bad:
        os.remove(tmp)
        raise RuntimeError(f"kernels use scratch memory: {bad}")
    os.replace(tmp, LIB_PATH)
    with open(HASH_PATH + ".tmp", "w") as fh:
        fh.write(digest + "\n")
    os.replace(HASH_PATH + ".tmp", HASH_PATH)
    return LIB_PATH


def ensure_built() -> str:
    """Build if no library exists yet; otherwise check that the library on
    disk was built from the current sources and raise if it was not (a stale
    library is never loaded silently)."""
    if not os.path.exists(LIB_PATH):
        build()
        return LIB_PATH
    have, want = built_hash(), source_hash()
    if have != want:
        raise RuntimeError(
            f"{LIB_PATH} does not match the sources (recorded source hash {have}, current "
            f"{want}): rebuild it with `python -m attention_forward_online_fa_amd.build`")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
