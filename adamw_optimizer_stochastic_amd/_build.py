"""Build step: compiles the HIP sources into the in-tree shared library.

Three translation units (csrc/adamw_sr.hip: the AdamW step, the generator and
the conversions; csrc/gemm_sr.hip: the GEMM; csrc/random.hip: uniform/normal
draws and dropout; all include csrc/device.hpp, csrc/status.hpp and
include/adamw_sr.h) -> libadamw_sr.so, for gfx950 only. Flags that matter
for the arithmetic:
  -ffp-contract=off                          no fused multiply-adds (the
                                             sources also say so by pragma)
  -fhip-fp32-correctly-rounded-divide-sqrt   '/' and sqrt correctly rounded
  no -ffast-math, no denormal flushing       subnormals kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed f32 instructions
The library is written to a temporary name and renamed into place, so a
process that has the old library mapped is not disturbed.
"""

import os
import shutil
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SOURCES = [os.path.join(PKG_DIR, "csrc", "adamw_sr.hip"),
           os.path.join(PKG_DIR, "csrc", "gemm_sr.hip"),
           os.path.join(PKG_DIR, "csrc", "random.hip")]
DEPENDS = SOURCES + [os.path.join(PKG_DIR, "csrc", "device.hpp"),
                     os.path.join(PKG_DIR, "csrc", "status.hpp"),
                     os.path.join(ROOT, "include", "adamw_sr.h")]
LIB_NAME = "libadamw_sr.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-command-line-argument",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libadamw_sr.so)")
    return path


def build(out_path=LIB_PATH, extra_flags=(), verbose=False):
    """Compile the library. Always compiles (no up-to-date check): each
    source to an object in parallel, then one link."""
    out_dir = os.path.dirname(out_path)
    fd, tmp = tempfile.mkstemp(prefix=".libadamw_sr.", suffix=".so.tmp", dir=out_dir)
    os.close(fd)
    objdir = tempfile.mkdtemp(prefix=".libadamw_sr_obj.", dir=out_dir)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    noise = "packed-fp32-ops"  # the host pass does not know the feature
    try:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [hipcc(), *compile_flags, *extra_flags, "-I", os.path.join(ROOT, "include"),
                   "-c", src, "-o", obj]
            jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                    stderr=subprocess.STDOUT, text=True)))
        msgs = []
        failed = []
        for cmd, obj, proc in jobs:
            out = proc.communicate()[0]
            msgs += [ln for ln in out.splitlines() if noise not in ln]
            if proc.returncode != 0:
                failed.append(" ".join(cmd))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed) + "\n" + "\n".join(msgs))
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra_flags,
                *(obj for _, obj, _ in jobs), "-o", tmp]
        res = subprocess.run(link, capture_output=True, text=True)
        msgs += [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(link) + "\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(objdir, ignore_errors=True)
    return out_path


def is_built():
    return os.path.exists(LIB_PATH)


if __name__ == "__main__":
    print(build(verbose=True))
