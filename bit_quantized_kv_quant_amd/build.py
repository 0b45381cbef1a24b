"""Build libminikv.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_quantized_kv_quant_amd.build

Every .hip file under csrc/ is compiled for gfx950 and linked into
bit_quantized_kv_quant_amd/libminikv.so.  Flags: packed-fp32 instructions are
disabled (-packed-fp32-ops), fp32 divide / sqrt stay correctly rounded, and the
quantiser is compiled without multiply-add contraction so its codes match an
IEEE evaluation bit for bit.
"""

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libminikv.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
]
PER_FILE = {
    # no fused multiply-add where the rule rounds; finite inputs (min / max need no NaN quieting)
    "quant_pack.hip": ["-ffp-contract=off", "-fno-honor-nans"],
    # MFMA results in ordinary VGPRs: the decode kernel reads every result at once
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def source_hash():
    """Build id of the library: the first 16 hex digits of a sha256 over every
    kernel, header and public-header source (name and bytes, in name order)."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h"))]
    files += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    for path in sorted(files, key=os.path.basename):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return "sha256:" + h.hexdigest()[:16]


def build(verbose=False, extra_flags=(), out=None):
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    lib_path = out or LIB
    tmp = tempfile.mkdtemp(prefix="minikv_build_")
    try:
        procs, objs = [], []
        build_id = f'-DMINIKV_BUILD_ID="{source_hash()}"'
        for src in sources():
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *COMMON, build_id, *extra_flags, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            log = p.communicate()[0].decode(errors="replace")
            if p.returncode != 0:
                failed.append((src, log))
            elif verbose and log.strip():
                print(log)
        if failed:
            msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = lib_path + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
        os.replace(tmp_lib, lib_path)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return lib_path


def ensure_built():
    """Build the library only when none is there (a fresh checkout: the built
    binary is not version-controlled).  A library built from other sources is
    left alone; loading it then raises, so stale code is never run silently."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
