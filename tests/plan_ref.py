"""ctypes access to the library's sequential host planner (block_sparse_attention_gather_amd/
csrc/plan_host.h), compiled from tests/plan_driver.cpp with the host C++ compiler."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_attention_gather_amd", "csrc")
KNQ = 8
_lib = None


def lib():
    global _lib
    if _lib is None:
        out = os.path.join(tempfile.mkdtemp(prefix="planref"), "libplanref.so")
        subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Werror",
                        "-I", CSRC, os.path.join(HERE, "plan_driver.cpp"), "-o", out],
                       check=True, capture_output=True, text=True)
        L = ctypes.CDLL(out)
        P = ctypes.c_void_p
        L.plan_ref.restype = ctypes.c_longlong
        L.plan_ref.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                               P, P, P, P, ctypes.c_longlong]
        L.queue_group_ref.restype = ctypes.c_int
        L.queue_group_ref.argtypes = [ctypes.c_longlong]
        L.layout_ref.restype = None
        L.layout_ref.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, P]
        _lib = L
    return _lib


def queue_group(head_kv_bytes):
    """XCDs sharing a queue (head mode) for heads of head_kv_bytes of K and V."""
    return int(lib().queue_group_ref(head_kv_bytes))


def plan(row_ptr, n_blk, nbh, target, group=1):
    """-> dict(Kc, qstart, qlen, head_rank, slot_base, items [n, 4] int32)"""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    assert rp.shape == (nbh * n_blk + 1,)
    cap = nbh * n_blk + target
    hdr = np.zeros(1 + 2 * KNQ, np.int32)
    rank = np.zeros(nbh, np.int32)
    sbase = np.zeros(nbh, np.int32)
    items = np.zeros((cap, 4), np.int32)
    n = lib().plan_ref(rp.ctypes.data, n_blk, nbh, target, group, hdr.ctypes.data,
                       rank.ctypes.data, sbase.ctypes.data, items.ctypes.data, cap)
    assert n >= 0
    return dict(Kc=int(hdr[0]), qstart=hdr[1:1 + KNQ].copy(), qlen=hdr[1 + KNQ:].copy(),
                head_rank=rank, slot_base=sbase, items=items[:n].copy())


def layout(bh, n_blk, B, D, slots):
    out = np.zeros(10, np.int64)
    lib().layout_ref(bh, n_blk, B, D, slots, out.ctypes.data)
    keys = ["hdr", "head_seg", "head_slot_base", "items", "done", "part_o", "part_ml", "total",
            "max_items", "max_slots"]
    return {k: int(v) for k, v in zip(keys, out)}
