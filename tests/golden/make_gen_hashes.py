"""Record SHA-256 digests of the generator's bf16 bytes (input determinism, not expected
outputs).  Run from the repo root:  python tests/golden/make_gen_hashes.py"""
import hashlib
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from workloads import CONFIGS, gen_qkv  # noqa: E402

out = {}
for name in ("tiny", "small"):
    h = hashlib.sha256()
    for a in gen_qkv(CONFIGS[name]):
        h.update(np.ascontiguousarray(a).tobytes())
    out[name] = h.hexdigest()
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "gen_sha256.json"), "w") as fh:
    json.dump(out, fh, indent=1)
print(out)
