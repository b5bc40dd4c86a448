"""The seeded input generator: determinism, head subsets, bf16 rounding (CPU only)."""
import hashlib
import json
import os
from fractions import Fraction

import numpy as np

from workloads import CONFIGS, gen_qkv, bf16_bits_from_f64, f64_from_bf16_bits
from workloads.gen import load_gains


def _sha(arrs):
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic_bytes(golden_dir):
    with open(os.path.join(golden_dir, "gen_sha256.json")) as fh:
        want = json.load(fh)
    for name in ("tiny", "small"):
        assert _sha(gen_qkv(CONFIGS[name])) == want[name], name
        assert _sha(gen_qkv(CONFIGS[name], threads=1)) == want[name], name


def test_full_layer_heads_deterministic(golden_dir):
    """Two heads of each full-size layer, byte for byte (the field uses no BLAS and no
    vectorised math routine, so these bytes are the same on any CPU and thread count)."""
    with open(os.path.join(golden_dir, "gen_sha256.json")) as fh:
        want = json.load(fh)
    keys = [k for k in want if ":heads=" in k]
    assert len(keys) == 3
    for key in keys:
        name, heads = key.split(":heads=")
        heads = [int(x) for x in heads.split(",")]
        assert _sha(gen_qkv(CONFIGS[name], heads=heads)) == want[key], key


def test_head_subset_matches_full():
    cfg = CONFIGS["small"]
    full = gen_qkv(cfg)
    part = gen_qkv(cfg, heads=[5, 2])
    for f, p in zip(full, part):
        assert np.array_equal(f[:, :, [5, 2]], p)


def _rne_bf16_exact(x: float) -> float:
    """Reference rounding with exact rationals: nearest value with 8 significant bits,
    ties to an even last bit."""
    if x == 0:
        return 0.0
    f = Fraction(x)
    sgn = -1 if f < 0 else 1
    f = abs(f)
    e = 0
    while f >= 256:
        f /= 2
        e += 1
    while f < 128:
        f *= 2
        e -= 1
    lo = int(f)
    rem = f - lo
    m = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2) else 0)
    return sgn * float(Fraction(m) * Fraction(2) ** e)


def test_bf16_round_to_nearest_even():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(400) * 10.0 ** rng.integers(-8, 8, 400),
                         [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 255.5, 0.0,
                          1 + 2 ** -8 + 2 ** -40]])
    got = f64_from_bf16_bits(bf16_bits_from_f64(xs))
    for x, g in zip(xs, got):
        assert g == _rne_bf16_exact(float(x)), x


def test_gains_frozen_for_every_config():
    for name, cfg in CONFIGS.items():
        g = load_gains(cfg)
        assert g.shape == (cfg.heads,) and np.all(g > 0)
    assert load_gains(CONFIGS["wan720p"]).std() > 0.3       # heads differ in concentration
