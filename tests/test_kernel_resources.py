"""Register use of every kernel, as the compiler reports it for gfx950: no
kernel keeps anything in scratch memory (register spills or private arrays
the compiler could not place in registers).  Scratch accesses go to memory
on every use; one private array in the group-of-4, d = 64 decode kernel
(a select between two array elements) once doubled that kernel's step time.
CPU only: the kernels are compiled, not run."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_kv_05_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _usage(source, tmp_path):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", CSRC, "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, source),
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    rows, cur = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (.*?) \[-Rpass", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = val
            rows[cur] = {}
        elif cur is not None:
            rows[cur][key] = val
    return rows


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("source", ["longflow_kernels.hip", "evict_topk.hip", "stack_kernels.hip"])
def test_no_kernel_uses_scratch(source, tmp_path):
    rows = _usage(source, tmp_path)
    kernels = {f: r for f, r in rows.items() if "kernel" in f}
    assert kernels, "no kernels reported"
    bad = {f: (r.get("ScratchSize [bytes/lane]"), r.get("VGPRs Spill")) for f, r in kernels.items()
           if r.get("ScratchSize [bytes/lane]", "0") != "0" or r.get("VGPRs Spill", "0") != "0"}
    assert not bad, bad
