"""bench.py's host logic (CPU only, no GPU touched): the one-GPU guard, argument checks, and
the recorded HBM traffic figures, which belong to exactly one attention source and mode."""
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


def test_traffic_figures_match_the_current_kernel_sources():
    """The recorded FETCH/WRITE figures are reported only for the attention source and mode
    they were measured on; both figures in the table belong to the sources as they are now."""
    for mode, t in bench.ATTN_TRAFFIC.items():
        assert bench.src_sha256(t["src"]) == t["sha256"], (mode, "re-take the counters")
        got = bench.attn_traffic(t["config"], mode)
        want = int(round((t["fetch_kib"] * bench.FETCH_SCALE
                          + t["write_kib"] * bench.WRITE_SCALE) * 1024))
        assert got == want
        assert bench.attn_traffic("wan720p", mode) is None       # another workload
    assert bench.attn_traffic("wan480p", "fp8-rne") is None       # never measured


def test_kernel_key_covers_per_source_compiler_options():
    """A per-source compiler option is part of the kernel the traffic figures belong to: the key
    of a source with options differs from the plain sha256 of the file, and every option set
    names a source the build compiles."""
    import hashlib
    from block_sparse_attention_gather_amd import build as B
    for src, flags in B.SOURCE_FLAGS.items():
        assert src in B.SOURCES and flags
        with open(os.path.join(B.CSRC, src), "rb") as fh:
            plain = hashlib.sha256(fh.read()).hexdigest()
        assert bench.src_sha256(src) != plain
    for src in B.SOURCES:
        if src not in B.SOURCE_FLAGS:
            with open(os.path.join(B.CSRC, src), "rb") as fh:
                assert bench.src_sha256(src) == hashlib.sha256(fh.read()).hexdigest()
