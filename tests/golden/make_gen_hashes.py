"""Record SHA-256 digests of the generator's bf16 bytes (input determinism, not expected
outputs): whole tiny and small workloads, two heads of each full-size layer.
Run from the repo root:  python tests/golden/make_gen_hashes.py"""
import hashlib
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from workloads import CONFIGS, gen_qkv  # noqa: E402

# Two heads of each full-size layer; the second of each is one whose bytes used to change
# with the CPU and BLAS build.
HEAD_PINS = {"wan480p": (0, 39), "wan720p": (0, 8), "hunyuan720p": (0, 12)}

out = {}
for name in ("tiny", "small"):
    h = hashlib.sha256()
    for a in gen_qkv(CONFIGS[name]):
        h.update(np.ascontiguousarray(a).tobytes())
    out[name] = h.hexdigest()
for name, heads in HEAD_PINS.items():
    h = hashlib.sha256()
    for a in gen_qkv(CONFIGS[name], heads=list(heads)):
        h.update(np.ascontiguousarray(a).tobytes())
    out["%s:heads=%s" % (name, ",".join(map(str, heads)))] = h.hexdigest()
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "gen_sha256.json"), "w") as fh:
    json.dump(out, fh, indent=1)
print(out)
