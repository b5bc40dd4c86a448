"""CPU check of the generated gfx950 code: every library source, compiled for the device with
the build's own flags (CFLAGS plus its per-source options), assembles to code that contains no
packed fp32 VALU instruction (the build's target feature keeps them out) and no scalar-cache
memory write (scalar stores, scalar atomics, or a write-back or discard of the scalar data
cache): all device memory writes go through vector memory instructions."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_attention_gather_amd import build as B

PACKED_F32 = re.compile(r"^\s*v_pk_[a-z0-9_]*_f32\b", re.M)
SCALAR_WRITE = re.compile(r"^\s*s_(store|buffer_store|scratch_store|atomic|buffer_atomic|"
                          r"dcache_wb|dcache_discard)", re.M)
MNEMONIC = re.compile(r"^\s*([vs]_[a-z0-9_]+)", re.M)


def _asm(src, extra, out):
    cmd = [B.hipcc(), *B.CFLAGS, *B.SOURCE_FLAGS.get(src, []), *extra, "--offload-device-only",
           "-S", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    assert "not a recognized feature" not in r.stdout, r.stdout
    with open(out) as fh:
        return fh.read()


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    jobs = [(s, [], str(d / (s + ".s"))) for s in B.SOURCES]
    jobs.append(("attn.hip", ["-DBSA_TRACE"], str(d / "attn_trace.s")))
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        texts = list(ex.map(lambda j: _asm(*j), jobs))
    return {os.path.basename(j[2]): t for j, t in zip(jobs, texts)}


def test_every_kernel_source_compiles_to_real_code(device_asm):
    for name, text in device_asm.items():
        if name == "api.hip.s":                      # host-side entry points only
            continue
        assert len(MNEMONIC.findall(text)) > 100, name


def test_no_packed_fp32_instructions(device_asm):
    for name, text in device_asm.items():
        hits = PACKED_F32.findall(text)
        assert not hits, (name, hits[:5])


def test_no_scalar_cache_writes(device_asm):
    for name, text in device_asm.items():
        hits = SCALAR_WRITE.findall(text)
        assert not hits, (name, hits[:5])


def test_attention_uses_the_matrix_cores(device_asm):
    assert "v_mfma_f32_32x32x16_bf16" in device_asm["attn.hip.s"]
    assert "v_mfma_scale_f32_32x32x64_f8f6f4" in device_asm["attn_fp8.hip.s"]
