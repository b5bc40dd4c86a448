"""bench.py's host logic (CPU only, no GPU touched): the one-GPU guard, argument checks, the
recorded HBM traffic figures (each belongs to exactly one attention source, mode and workload)
and the host description of the CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("args,msg", [(["--reuse", "0"], "--reuse"),
                                      (["--tile", "4,4"], "--tile"),
                                      (["--tile", "4,0,8"], "--tile"),
                                      (["--tile", "a,b,c"], "--tile")])
def test_bad_arguments_stop_before_any_work(args, msg):
    r = _run(*args)
    assert r.returncode != 0 and msg in r.stderr


def test_parse_tile():
    assert bench.parse_tile("") is None
    assert bench.parse_tile("8,4,4") == (8, 4, 4)


def test_traffic_figures_belong_to_one_kernel_mode_and_workload():
    """A recorded FETCH/WRITE figure is reported only for the attention source (and its
    compiler options), mode and workload it was measured on; any other source gives null."""
    keys = set()
    for t in bench.ATTN_TRAFFIC:
        key = (t["mode"], t["config"])
        assert key not in keys
        keys.add(key)
        got = bench.attn_traffic(t["config"], t["mode"])
        if bench.src_sha256(t["src"]) == t["sha256"]:
            want = int(round((t["fetch_kib"] * bench.FETCH_SCALE
                              + t["write_kib"] * bench.WRITE_SCALE) * 1024))
            assert got == want
        else:
            assert got is None                                  # taken on another kernel
    assert bench.attn_traffic("small", "bf16") is None            # never measured
    assert bench.attn_traffic("wan720p", "fp8-rne") is None


def test_traffic_lookup_rejects_a_changed_source(monkeypatch):
    t = dict(bench.ATTN_TRAFFIC[0])
    monkeypatch.setattr(bench, "ATTN_TRAFFIC", [dict(t, sha256=bench.src_sha256(t["src"])),
                                                dict(t, config="tiny", sha256="0" * 64)])
    assert bench.attn_traffic(t["config"], t["mode"]) is not None
    assert bench.attn_traffic("tiny", t["mode"]) is None


def test_kernel_key_covers_headers_and_compiler_options(tmp_path, monkeypatch):
    """A figure belongs to the kernel as compiled: its source, the library headers it includes
    and its per-source compiler options.  Changing a shared header changes the key of exactly the
    sources that include it; dropping the options changes the key of exactly the sources that
    have them."""
    import shutil
    from block_sparse_attention_gather_amd import build as B
    for src, flags in B.SOURCE_FLAGS.items():
        assert src in B.SOURCES and flags
    for src in ("attn.hip", "attn_fp8.hip"):
        assert {"attn_common.h", "plan.h"} <= set(bench.local_headers(src))
    before = {s: bench.src_sha256(s) for s in B.SOURCES}
    root = tmp_path / "r"
    csrc = root / "block_sparse_attention_gather_amd" / "csrc"
    shutil.copytree(B.CSRC, csrc)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert {s: bench.src_sha256(s) for s in B.SOURCES} == before    # same text, same keys
    with open(csrc / "attn_common.h", "a") as fh:
        fh.write("\n// changed\n")
    after = {s: bench.src_sha256(s) for s in B.SOURCES}
    for s in B.SOURCES:
        assert (after[s] != before[s]) == ("attn_common.h" in bench.local_headers(s)), s
    flagged = set(B.SOURCE_FLAGS)
    monkeypatch.setattr(B, "SOURCE_FLAGS", {})
    plain = {s: bench.src_sha256(s) for s in B.SOURCES}
    for s in B.SOURCES:
        assert (plain[s] != after[s]) == (s in flagged), s


def test_host_info_describes_the_cpu():
    h = bench.host_info()
    assert h["os_cpu_count"] == os.cpu_count()
    assert 1 <= h["affinity_cpus"] <= os.cpu_count()
    assert h["physical_cores"] is None or 1 <= h["physical_cores"] <= os.cpu_count()
    assert isinstance(h["blas"], list)


def test_default_workload_is_the_largest_video_layer():
    import argparse
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert isinstance(a, argparse.Namespace)
    assert a.config == "hunyuan720p" and a.gpus == 1 and a.cpu_stride == 0
