"""Builds ``libmp.so`` (every ``csrc/*.hip`` source) in-tree for gfx950.

Each translation unit is compiled with ``hipcc --offload-arch=gfx950`` in
parallel into ``_build/`` at the repository root, then linked into
``megatron_tensor_transformer_02_amd/libmp.so``.  Packed fp32 instructions
are disabled (``-packed-fp32-ops``) for every GPU object.

``build(sanitize=True)`` builds a test-only variant whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer instrumentation (each
``-fsanitize=`` flag is passed for the host compilation only; the device code
is built as usual and is never run from it) into
``_build/asan/libmp_asan.so``, for exercising the argument validation layer
on the CPU under the sanitizers' runtime.
"""

import concurrent.futures as cf
import glob
import json
import re
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmp.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-unknown-warning-option",
    # The compiler's per-kernel register / scratch / occupancy remarks,
    # collected into kernel_resources.json beside the objects.
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK_NAME = re.compile(r"remark: Function Name: (\S+)")
_REMARK_FIELD = re.compile(r"remark:\s+(.+?):\s+(\S+) \[-Rpass-analysis=kernel-resource-usage\]")


def _resources(stderr):
    """{kernel symbol: {field: value}} from the resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = _REMARK_NAME.search(line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = _REMARK_FIELD.search(line)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1).strip()] = int(v) if v.lstrip("-").isdigit() else v
    return out


def _without_remarks(stderr):
    """The compiler's messages other than the resource remarks (and their
    source excerpts)."""
    keep, skip = [], 0
    for line in stderr.splitlines():
        if "[-Rpass-analysis=kernel-resource-usage]" in line:
            skip = 2  # the source line and caret the first remark of a kernel quotes
            continue
        if skip and (line.startswith(" ") or not line.strip()):
            skip -= 1
            continue
        skip = 0
        keep.append(line)
    return "\n".join(keep)


SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libmp_asan.so")


def _compile(src, extra, out_dir=BUILD):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj, res.stderr


def build(verbose=False, extra=(), jobs=None, sanitize=False):
    """Compile and link libmp.so (or, with ``sanitize``, the host-sanitized
    test build); returns its path.  Always rebuilds."""
    out_dir = ASAN_DIR if sanitize else BUILD
    lib = ASAN_LIB if sanitize else LIB
    extra = list(extra) + (SANITIZE_FLAGS + ["-O1"] if sanitize else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, out_dir), srcs))
    objs, resources = [], {}
    for obj, err in results:
        objs.append(obj)
        resources.update(_resources(err))
        msgs = _without_remarks(err)
        if verbose and msgs.strip():
            sys.stderr.write(msgs + "\n")
    with open(os.path.join(out_dir, "kernel_resources.json"), "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libasan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def asan_runtime():
    """Path of the compiler's AddressSanitizer runtime (to preload into a
    process that loads the sanitized build)."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return res.stdout.strip()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
