"""Build liblongflow.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m decode_attention_kv_05_amd.build

The library is written next to this file so it travels with the source tree.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblongflow.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# Read-bandwidth probes used by the benchmark only (not part of the library).
PROBE_PATH = os.path.join(HERE, "libhbm_probe.so")
PROBE_SOURCE = os.path.join(CSRC, "hbm_probe.hip")
SOURCES = [os.path.join(CSRC, n) for n in ("longflow_api.cpp", "longflow_kernels.hip", "evict_topk.hip",
                                            "stack_api.cpp", "stack_kernels.hip")]
ARCH = "gfx950"


# Sources each kernel family's code depends on (the host API and the shared
# headers count for every family).
_COMMON = ["longflow_api.cpp", "layout.h", "launch.h"]
_FAMILIES = {"decode": ["longflow_kernels.hip"], "topk": ["evict_topk.hip"],
             "stack": ["longflow_kernels.hip", "stack_api.cpp", "stack_kernels.hip", "stack_launch.h"]}
_HEADERS = {"decode": ["longflow.h"], "topk": ["longflow.h"], "stack": ["longflow.h", "longflow_stack.h"]}


# Code-generation flags; part of the whole library's source hash.
CODEGEN_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HASH_TAG = b"lf-source-hash:"


def source_hash(family=None):
    """Short hash of the sources of one kernel family ("decode", "topk",
    "stack"), or of the whole library (every source, header and the
    code-generation flags) when family is None; identifies a build."""
    import hashlib
    if family is None:
        names = _COMMON + sorted({n for v in _FAMILIES.values() for n in v})
        headers = sorted({n for v in _HEADERS.values() for n in v})
    else:
        names = _COMMON + _FAMILIES[family]
        headers = _HEADERS[family]
    h = hashlib.sha256()
    for path in sorted([os.path.join(CSRC, n) for n in names] + [os.path.join(INCLUDE, n) for n in headers]):
        with open(path, "rb") as f:
            h.update(f.read())
    if family is None:
        h.update(" ".join(CODEGEN_FLAGS).encode())
    return h.hexdigest()[:16]


def built_hash(path=LIB_PATH):
    """The source hash recorded in a built library (read from the file, not
    loaded), or None."""
    try:
        with open(path, "rb") as f:
            data = f.read()
    except OSError:
        return None
    at = data.find(HASH_TAG)
    if at < 0:
        return None
    return data[at + len(HASH_TAG):at + len(HASH_TAG) + 16].decode("ascii", "replace")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out_path):
    return [
        hipcc(), *CODEGEN_FLAGS, f'-DLF_SOURCE_HASH="{source_hash()}"',
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out_path,
    ]


def build_probe():
    """Compile the benchmark's read probes (libhbm_probe.so)."""
    tmp = PROBE_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), *CODEGEN_FLAGS, "-Wall", PROBE_SOURCE, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def build(verbose=False):
    """Compile the library (always) and return its path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def ensure_built():
    """Path of the built library, building it when it is absent or was built
    from other sources than the current ones (and the probe library when it
    is absent or older than its source)."""
    if built_hash() != source_hash():
        build()
    if not os.path.exists(PROBE_PATH) or os.path.getmtime(PROBE_PATH) < os.path.getmtime(PROBE_SOURCE):
        build_probe()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe())
