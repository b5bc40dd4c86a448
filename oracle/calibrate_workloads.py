"""Freeze the per-head Q gains g_h of the synthetic workloads (writes workloads/gains.json).

TEST INFRASTRUCTURE ONLY.  The gain is the one knob that sets how concentrated the block
scores are, hence the block sparsity the Top-p router reaches.  For each workload with a
sparsity target this script bisects log g on the oracle's own routing rule, applied to the
pooled fp64 Q/K of the generator (before bf16 rounding, which moves block means by ~1e-3
relative and the sparsity by far less than the +-0.02 band).  Q is linear in g (the stripe
term included), so the block scores of gain g are exactly g times those of gain 1.

Run:  python -m oracle.calibrate_workloads [config ...]
"""
from __future__ import annotations

import json
import math
import sys

import numpy as np

from workloads import gen as G
from . import bsa_oracle as O


def pooled_scores_gain1(cfg: G.Config, head: int) -> np.ndarray:
    """Block scores of one head at gain 1: [n_blk, n_blk]."""
    q, k, _ = G.gen_head_f64(cfg, head, 1.0)
    pi = O.tile_perm(cfg.T, cfg.H, cfg.W, cfg.tile)
    Npad = O.padded_len(cfg.N, cfg.block)
    qt = np.zeros((1, 1, Npad, cfg.head_dim))
    kt = np.zeros((1, 1, Npad, cfg.head_dim))
    qt[0, 0, pi] = q
    kt[0, 0, pi] = k
    qb = O.pool(qt, cfg.N, cfg.block)
    kb = O.pool(kt, cfg.N, cfg.block)
    return O.block_scores(qb, kb, 1.0 / math.sqrt(cfg.head_dim))[0, 0]


def counts(s: np.ndarray, top_p: float, k_floor: int) -> np.ndarray:
    """Per-row kept-block counts under the oracle's Top-p/Top-k rule (vectorised over rows;
    counts do not depend on how equal scores are ordered)."""
    n = s.shape[-1]
    srt = -np.sort(-s, axis=-1)
    e = np.exp(srt - srt[:, :1])
    cum = np.cumsum(e / e.sum(axis=-1, keepdims=True), axis=-1)
    reach = cum >= top_p
    k_p = np.where(reach.any(axis=-1), reach.argmax(axis=-1) + 1, n)
    return np.minimum(n, np.maximum(k_p, k_floor))


def sparsity(s_list, g, cfg) -> float:
    tot = sum(counts(g * s, cfg.top_p, cfg.k_floor).sum() for s in s_list)
    rows = sum(s.shape[0] for s in s_list)
    return 1.0 - tot / (rows * s_list[0].shape[1])


def bisect_gain(s_list, cfg, target, lo=0.05, hi=200.0, iters=50) -> float:
    llo, lhi = math.log(lo), math.log(hi)
    for _ in range(iters):
        mid = 0.5 * (llo + lhi)
        if sparsity(s_list, math.exp(mid), cfg) < target:
            llo = mid
        else:
            lhi = mid
    return math.exp(0.5 * (llo + lhi))


def calibrate(name: str) -> dict:
    cfg = G.get_config(name)
    if name in ("tiny", "small"):
        return {"gains": [1.0] * cfg.heads, "note": "gain 1, no sparsity target"}
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        S = list(ex.map(lambda h: pooled_scores_gain1(cfg, h), range(cfg.heads)))
    if name == "wan720p":
        # head sparsities 0.30 + 0.60 k/39, assigned to heads by a seeded shuffle
        perm = np.random.Generator(np.random.PCG64(cfg.seed + 1000)).permutation(cfg.heads)
        targets = [0.30 + 0.60 * int(perm[h]) / (cfg.heads - 1) for h in range(cfg.heads)]
        gains = [bisect_gain([S[h]], cfg, targets[h]) for h in range(cfg.heads)]
        real = [sparsity([S[h]], gains[h], cfg) for h in range(cfg.heads)]
        return {"gains": gains, "targets": targets, "fp64_sparsity": real,
                "overall_fp64_sparsity": float(np.mean(real))}
    g = bisect_gain(S, cfg, 0.60)
    return {"gains": [g] * cfg.heads, "target": 0.60,
            "fp64_sparsity": sparsity(S, g, cfg)}


def main(argv):
    names = argv or ["tiny", "small", "wan480p", "wan720p", "hunyuan720p"]
    try:
        with open(G.GAINS_PATH) as fh:
            table = json.load(fh)
    except FileNotFoundError:
        table = {}
    for name in names:
        table[name] = calibrate(name)
        print(name, {k: (v if not isinstance(v, list) else v[:4]) for k, v in table[name].items()},
              flush=True)
        with open(G.GAINS_PATH, "w") as fh:
            json.dump(table, fh, indent=1)


if __name__ == "__main__":
    main(sys.argv[1:])
