"""Register budget of every kernel, read from the compiler's resource remarks
(CPU only: hipcc cross-compiles for gfx950 without a GPU).

Every kernel must run without scratch: a spill in the decode kernel's
shared-group path once made such batches four times slower while every
parity test still passed. The bf16 decode kernels must also stay within the
168 VGPRs that three waves per SIMD leave each wave."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from paged_kv_cache_429_amd import build

FILES = ["decode.hip", "prefill.hip", "kvops.hip"]


def _remarks(src, tmp):
    cmd = [build.hipcc()] + build._flags() + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                               os.path.join(build.CSRC, src), "-o", os.path.join(tmp, src + ".o")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    kernels, cur = {}, None
    for line in r.stdout.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: \s*(VGPRs|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(len(FILES)) as ex:
            parts = list(ex.map(lambda f: _remarks(f, tmp), FILES))
    return dict(zip(FILES, parts))


def test_every_kernel_reported(resources):
    for f, ks in resources.items():
        assert ks, f
        for name, r in ks.items():
            assert "VGPRs" in r and "ScratchSize" in r, (f, name, r)
    decode = resources["decode.hip"]
    assert sum("decode_kernel" in k for k in decode) == 10  # d 64 / 128 x five formats


def test_no_kernel_spills(resources):
    spilled = {k: r["ScratchSize"] for ks in resources.values() for k, r in ks.items() if r["ScratchSize"]}
    assert not spilled, spilled


def test_bf16_decode_fits_three_waves_per_simd(resources):
    # decode_kernel<D, 1>: bf16 pools (format code 1)
    bf16 = {k: r["VGPRs"] for k, r in resources["decode.hip"].items() if re.search(r"decode_kernelILi\d+ELi1E", k)}
    assert len(bf16) == 2
    assert all(v <= 168 for v in bf16.values()), bf16
