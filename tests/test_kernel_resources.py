"""Every kernel compiles for gfx950 with no scratch memory and no spilled vector registers
(CPU only).  Scalar registers spilled into vector-register lanes cost no memory traffic, only a
lane read where the value is used: up to 96 are allowed.  The decode kernels spill kernel
arguments and loop-invariant addresses there (the most in the one-head-per-group instances); a
build without the code that raised the count from 64 timed within 1% of them.  The decode
instances that hand out an item list's last items by a counter (bf16 caches, launched only for a
few long requests) may spill up to 112: with that code the long context in 512-token partitions decodes
in 225 us against 247 us without it.

A register array indexed by a per-lane value, or too many live values, makes the compiler
place data in scratch memory: each access is then a memory round trip behind a full wait,
which once cost the quantized prefill a quarter of its rate.  The compiler's resource
remarks are read for every kernel instance."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_408_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _remarks(src, tmp):
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "-c",
           os.path.join(CSRC, src), "-o", os.path.join(tmp, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


def test_no_scratch_no_spills(tmp_path):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(2) as ex:
        found = list(ex.map(lambda s: _remarks(s, str(tmp_path)), ["pagedkv.hip", "prefill.hip"]))
    kernels = {**found[0], **found[1]}
    assert any("decode_mfma_kernel" in k for k in kernels) and any("prefill_kernel" in k for k in kernels)
    def sgpr_limit(name):   # decode_mfma_kernel<..., NW, true>: the counter-fed item list
        return 112 if re.search(r"decode_mfma_kernelILi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELb1E", name) else 96
    bad = {k: v for k, v in kernels.items()
           if v.get("ScratchSize [bytes/lane]", 0) or v.get("VGPRs Spill", 0) or v.get("SGPRs Spill", 0) > sgpr_limit(k)}
    assert not bad, f"{len(bad)} kernels with scratch or spills, e.g. {list(bad.items())[:3]}"
