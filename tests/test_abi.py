"""The C ABI without a GPU: header hygiene, exported symbols, host-side validation."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_gather_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", txt)))


def test_header_compiles_as_c99_and_cxx(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "bsa.h"\nint main(void){bsa_grid g={1,1,1,1,1,1,64};'
                   'return bsa_num_blocks(&g) == 1 ? 0 : 1;}\n')
    for cc, extra in (("gcc", ["-std=c99"]), ("g++", ["-std=c++11", "-x", "c++"])):
        r = subprocess.run([cc, *extra, "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                            "-I", os.path.dirname(HEADER), str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 20, names
    lib = ctypes.CDLL(bsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    r = subprocess.run(["nm", "-D", "--defined-only", bsa.LIB_PATH], capture_output=True,
                       text=True)
    exported = set(re.findall(r"\bT (bsa_\w+)", r.stdout))
    assert set(names) <= exported
    assert exported <= set(names), exported - set(names)     # nothing undeclared leaks
    # no C++ symbol of the implementation is exported either
    assert not re.search(r"\bT _Z", r.stdout), re.findall(r"\bT (_Z\w+)", r.stdout)[:5]


def test_trace_library_adds_only_the_trace_reader():
    """libbsa_trace.so (the -DBSA_TRACE debug build) exports the same ABI plus
    bsa_trace_read; the product library does not contain it."""
    assert os.path.exists(bsa.TRACE_LIB_PATH)
    r = subprocess.run(["nm", "-D", "--defined-only", bsa.TRACE_LIB_PATH], capture_output=True,
                       text=True)
    exported = set(re.findall(r"\bT (bsa_\w+)", r.stdout))
    assert exported == set(_declared()) | {"bsa_trace_read"}
    assert not hasattr(ctypes.CDLL(bsa.LIB_PATH), "bsa_trace_read")


def test_version_and_geometry_helpers():
    assert "gfx950" in bsa.version()
    L = bsa.lib()
    for (T, H, W, tile, B), (nb, npad) in [((2, 16, 16, (4, 4, 4), 64), (8, 512)),
                                            ((21, 30, 52, (4, 4, 8), 128), (256, 32768)),
                                            ((33, 45, 80, (4, 4, 8), 128), (929, 118912)),
                                            ((1, 1, 1, (4, 4, 8), 128), (1, 128))]:
        g = bsa.Grid(T, H, W, tile, B)._c()
        assert L.bsa_num_blocks(ctypes.byref(g)) == nb
        assert L.bsa_padded_len(ctypes.byref(g)) == npad
    bad = bsa.Grid(0, 16, 16, (4, 4, 4), 64)._c()
    assert L.bsa_num_blocks(ctypes.byref(bad)) == 0


FAKE = 0x7f0000000000            # never dereferenced: validation fails before any launch


def _route(**kw):
    L = bsa.lib()
    g = kw.pop("grid", bsa.Grid(2, 16, 16, (4, 4, 4), 64))._c()
    s = bsa._Shape(*kw.pop("shape", (1, 2, 64)))
    args = dict(q=FAKE, k=FAKE, top_p=0.9, k_floor=2, scale=0.125, row_ptr=FAKE, col=FAKE,
                nnz=FAKE, scores=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    st = L.bsa_score_and_route(args["q"], args["k"], ctypes.byref(s), ctypes.byref(g),
                               args["top_p"], args["k_floor"], args["scale"], args["row_ptr"],
                               args["col"], args["nnz"], args["scores"], args["ws"],
                               args["ws_bytes"], None)
    return st, L.bsa_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), -1, "non-NULL"),
    (dict(nnz=None), -1, "non-NULL"),
    (dict(top_p=1.5), -1, "top_p"),
    (dict(top_p=-0.1), -1, "top_p"),
    (dict(top_p=float("nan")), -1, "top_p"),
    (dict(k_floor=0), -1, "k_floor"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(shape=(1, 2, 96)), -2, "head_dim"),
    (dict(grid=bsa.Grid(2, 16, 16, (4, 4, 4), 32)), -2, "block"),
    (dict(shape=(1, 3000, 64)), -2, "batch*heads"),
    (dict(ws=None), -3, "workspace"),
    (dict(ws_bytes=16), -3, "workspace"),
    (dict(ws=FAKE + 8), -3, "aligned"),
    (dict(q=FAKE + 2), -1, "aligned"),
    (dict(grid=bsa.Grid(2, 0, 16, (4, 4, 4), 64)), -1, "grid"),
])
def test_route_validation(kw, status, msg):
    st, err = _route(**kw)
    assert st == status, (st, err)
    assert msg in err


def test_reorder_validation():
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(1, 2, 64)
    assert L.bsa_reorder(None, FAKE, ctypes.byref(s), ctypes.byref(g), 0, None) == -1
    s_bad = bsa._Shape(1, 2, 12)
    assert L.bsa_reorder(FAKE, FAKE + (1 << 24), ctypes.byref(s_bad), ctypes.byref(g), 0,
                         None) == -2
    # overlapping buffers
    assert L.bsa_reorder(FAKE, FAKE + 64, ctypes.byref(s), ctypes.byref(g), 0, None) == -1
    assert "overlap" in L.bsa_last_error().decode()
    assert L.bsa_reorder(FAKE, FAKE, None, ctypes.byref(g), 0, None) == -1


def test_reorder_pool_validation():
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(1, 2, 64)
    far = FAKE + (1 << 28)
    dst = FAKE + (1 << 24)
    assert L.bsa_reorder_pool(FAKE, None, None, None, None, ctypes.byref(s), ctypes.byref(g),
                              None) == -1
    assert "no output" in L.bsa_last_error().decode()
    s96 = bsa._Shape(1, 2, 96)                       # the pooled path is built for 64 and 128
    assert L.bsa_reorder_pool(FAKE, dst, far, None, None, ctypes.byref(s96), ctypes.byref(g),
                              None) == -2
    assert L.bsa_reorder_pool(FAKE, dst, FAKE + 4, None, None, ctypes.byref(s),
                              ctypes.byref(g), None) == -1        # pooled overlaps src
    assert L.bsa_reorder_pool(FAKE, dst, far + 4, None, None, ctypes.byref(s), ctypes.byref(g),
                              None) == -1                         # pooled misaligned
    assert "aligned" in L.bsa_last_error().decode()
    # E4M3 outputs: both or neither, and only for head_dim 128 / block 128
    assert L.bsa_reorder_pool(FAKE, dst, far, far + (1 << 24), None, ctypes.byref(s),
                              ctypes.byref(g), None) == -1
    assert L.bsa_reorder_pool(FAKE, dst, far, far + (1 << 24), far + (1 << 25), ctypes.byref(s),
                              ctypes.byref(g), None) == -2
    assert L.bsa_reorder_quantize_v(FAKE, None, dst, far, ctypes.byref(s), ctypes.byref(g),
                                    None) == -2
    s128 = bsa._Shape(1, 2, 128)
    g128 = bsa.Grid(2, 16, 16, (4, 4, 8), 128)._c()
    assert L.bsa_reorder_quantize_v(FAKE, None, None, far, ctypes.byref(s128),
                                    ctypes.byref(g128), None) == -1
    assert L.bsa_reorder_quantize_v(FAKE, None, FAKE + 64, far, ctypes.byref(s128),
                                    ctypes.byref(g128), None) == -1      # v8 overlaps src


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), -1, "non-NULL"),
    (dict(top_p=1.5), -1, "top_p"),
    (dict(k_floor=0), -1, "k_floor"),
    (dict(shape=(1, 2, 96)), -2, "head_dim"),
    (dict(ws_bytes=16), -3, "workspace"),
    (dict(q=FAKE + 8), -1, "aligned"),
])
def test_route_pooled_validation(kw, status, msg):
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(*kw.pop("shape", (1, 2, 64)))
    a = dict(q=FAKE, k=FAKE, top_p=0.9, k_floor=2, ws_bytes=1 << 30)
    a.update(kw)
    st = L.bsa_route_pooled(a["q"], a["k"], ctypes.byref(s), ctypes.byref(g), a["top_p"],
                            a["k_floor"], 0.125, FAKE, FAKE, FAKE, None, FAKE, a["ws_bytes"],
                            None)
    assert st == status, (st, L.bsa_last_error())
    assert msg in L.bsa_last_error().decode()


def test_stripe_validation():
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(1, 2, 64)
    ok = (ctypes.c_int32 * 12)(1, 0, 2, 1, 0, 3, 2, 1, 2, 3, -1, 3)
    bad = (ctypes.c_int32 * 12)(1, 0, 2, 1, 0, 3, 3, 0, 2, 1, 0, 1)      # head 1: Tw > Ts
    assert L.bsa_stripe_mask(bad, ctypes.byref(s), ctypes.byref(g), FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == -1
    assert "head 1" in L.bsa_last_error().decode()
    assert L.bsa_stripe_mask(None, ctypes.byref(s), ctypes.byref(g), FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == -1
    assert L.bsa_stripe_mask(ok, ctypes.byref(s), ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, 16,
                             None) == -3
    s96 = bsa._Shape(1, 2, 96)
    assert L.bsa_stripe_mask(ok, ctypes.byref(s96), ctypes.byref(g), FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == -2
    n = L.bsa_stripe_workspace_bytes(ctypes.byref(s), ctypes.byref(g))
    assert n > 0 and n % 256 == 0


def test_hilbert_order_validation():
    L = bsa.lib()
    g = bsa.Grid(21, 30, 52, (4, 4, 8), 128)._c()
    n = L.bsa_hilbert_order_workspace_bytes(ctypes.byref(g))
    assert n >= 2 * 64 ** 3 * 4 and n % 256 == 0              # cube of side 64
    assert L.bsa_hilbert_order(ctypes.byref(g), None, FAKE, n, None) == -1
    assert L.bsa_hilbert_order(ctypes.byref(g), FAKE + 2, FAKE, n, None) == -1
    assert L.bsa_hilbert_order(ctypes.byref(g), FAKE, FAKE, 16, None) == -3
    big = bsa.Grid(2, 300, 16, (4, 4, 8), 128)._c()
    assert L.bsa_hilbert_order(ctypes.byref(big), FAKE, FAKE, 1 << 40, None) == -2
    # a misaligned order table in a grid is rejected by every call
    bad = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    bad.order = FAKE + 2
    assert L.bsa_num_blocks(ctypes.byref(bad)) == 0


def test_attn_validation_before_device_query():
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(1, 2, 64)
    st = L.bsa_sparse_attn_fwd(FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(s), ctypes.byref(g),
                               0.125, FAKE, None, FAKE, 1 << 30, None)
    assert st == -1
    s96 = bsa._Shape(1, 2, 96)
    st = L.bsa_sparse_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s96),
                               ctypes.byref(g), 0.125, FAKE, None, FAKE, 1 << 30, None)
    assert st == -2
    st = L.bsa_sparse_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(g),
                               float("nan"), FAKE, None, FAKE, 1 << 30, None)
    assert st == -1


def test_noalloc_attn_validation_before_device_query():
    """bsa_sparse_attn_fwd_noalloc checks its arguments like bsa_sparse_attn_fwd before it
    looks at the device or its static scratch."""
    L = bsa.lib()
    g = bsa.Grid(2, 16, 16, (4, 4, 4), 64)._c()
    s = bsa._Shape(1, 2, 64)
    st = L.bsa_sparse_attn_fwd_noalloc(FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(s),
                                       ctypes.byref(g), 0.125, FAKE, None, None)
    assert st == -1 and b"non-NULL" in L.bsa_last_error()
    s96 = bsa._Shape(1, 2, 96)
    assert L.bsa_sparse_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s96),
                                         ctypes.byref(g), 0.125, FAKE, None, None) == -2
    assert L.bsa_sparse_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s),
                                         ctypes.byref(g), -1.0, FAKE, None, None) == -1
    assert L.bsa_sparse_attn_fwd_noalloc(FAKE + 8, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s),
                                         ctypes.byref(g), 0.125, FAKE, None, None) == -1


def test_route_workspace_size_is_host_computable():
    L = bsa.lib()
    for cfg, D in (((21, 30, 52, (4, 4, 8), 128), 128), ((2, 16, 16, (4, 4, 4), 64), 64)):
        g = bsa.Grid(*cfg)._c()
        s = bsa._Shape(1, 40, D)
        n = L.bsa_route_workspace_bytes(ctypes.byref(s), ctypes.byref(g))
        nb = L.bsa_num_blocks(ctypes.byref(g))
        assert n >= 2 * 40 * nb * D * 8          # pooled Q and K in fp64
        assert n % 256 == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 512, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        bsa.reorder(x, bsa.Grid(2, 16, 16, (4, 4, 4), 64))
