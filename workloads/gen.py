"""Synthetic Q/K/V of the shapes the pages' video DiTs produce (Wan 2.1 480p/720p,
HunyuanVideo 720p latent grids), drawn from a seeded smooth positional field plus noise.

Recipe (one head at a time, each head from its own counter-derived PCG64 stream so that a
single head can be regenerated without the others):

* token n of the T x H x W latent grid sits at integer coordinates c_n = (t, h, w), raster
  order n = (t*H + h)*W + w;
* per head: a frequency scale s_h (fixed, or s0 * 2**U(-1, 1) when heads must differ), then a
  shared Q/K random-Fourier field with 8 frequencies omega_m ~ N(0, s_h^2 I_3), phases
  phi_m ~ U[0, 2 pi) and a D x 16 mixing matrix A ~ N(0, 1):
  f_n = A [cos(omega . c_n + phi), sin(omega . c_n + phi)] / sqrt(8)  (unit variance/channel),
  then an independent field f_V for V, then noise eps_Q, eps_K, eps_V ~ N(0, 1), each [N, D];
* Q = g_h (0.7 f + 0.3 eps_Q),  K = 0.7 f + 0.3 eps_K,  V = 0.7 f_V + 0.3 eps_V;
  Q and K share f, so q.k peaks at zero displacement: local, video-like attention;
* the optional periodic stripe term (HunyuanVideo-shaped workload) adds beta*u_n to channels
  0..15 of K and g_h*beta*u_n to Q, u_n = [cos, sin](2 pi f h / H), [cos, sin](2 pi f w / W)
  for f = 1..4, beta = 0.7 sqrt(D / 8) (the stripe peak equals the field peak); the term has
  no t, so it repeats every frame, and it repeats every W raster positions;
* all arithmetic in fp64, then one round-to-nearest-even to bf16; layout [1, N, heads, D];
* the cosines and sines come from per-axis tables of the C library's scalar cos/sin joined by
  the angle-addition formulas, and the products with A are elementwise sums in a fixed order,
  so the bytes are the same on every machine and for any thread count (no BLAS, no vectorised
  math routines).

The gain g_h is the single sparsity knob (the softmax scale is fixed by the method).  Frozen
per-config gains live in gains.json next to this file; they are produced once by a
calibration script that belongs to the oracle and are read here as plain numbers.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
GAINS_PATH = os.path.join(_HERE, "gains.json")


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    block: int
    tile: tuple            # (tile_t, tile_h, tile_w); product == block
    top_p: float
    k_floor: int
    seed: int
    sigma0: float = 0.15   # rad per token
    per_head_sigma: bool = True
    stripes: bool = False
    sparsity_target: str = ""
    batch: int = 1

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


CONFIGS = {
    "tiny": Config("tiny", 2, 16, 16, heads=2, head_dim=64, block=64, tile=(4, 4, 4),
                   top_p=0.9, k_floor=2, seed=1, per_head_sigma=False,
                   sparsity_target="none (gain 1)"),
    "small": Config("small", 5, 16, 24, heads=8, head_dim=64, block=64, tile=(4, 4, 4),
                    top_p=0.95, k_floor=4, seed=2, sparsity_target="none (gain 1)"),
    "wan480p": Config("wan480p", 21, 30, 52, heads=40, head_dim=128, block=128,
                      tile=(4, 4, 8), top_p=0.9, k_floor=8, seed=3,
                      sparsity_target="overall block sparsity 0.60 +- 0.02"),
    "wan720p": Config("wan720p", 21, 45, 80, heads=40, head_dim=128, block=128,
                      tile=(4, 4, 8), top_p=0.85, k_floor=8, seed=4,
                      sparsity_target="per-head sparsity 0.30 + 0.60 k/39, shuffled"),
    "hunyuan720p": Config("hunyuan720p", 33, 45, 80, heads=24, head_dim=128, block=128,
                          tile=(4, 4, 8), top_p=0.9, k_floor=16, seed=5, stripes=True,
                          sparsity_target="overall block sparsity 0.60 +- 0.02"),
}

ORDER = ["tiny", "small", "wan480p", "wan720p", "hunyuan720p"]


def get_config(name: str) -> Config:
    return CONFIGS[name]


def load_gains(cfg: Config) -> np.ndarray:
    """Per-head Q gains g_h for a config (1.0 where nothing is frozen yet)."""
    if os.path.exists(GAINS_PATH):
        with open(GAINS_PATH) as fh:
            table = json.load(fh)
        ent = table.get(cfg.name)
        if ent is not None:
            g = np.asarray(ent["gains"], dtype=np.float64)
            assert g.shape == (cfg.heads,), (cfg.name, g.shape)
            return g
    return np.ones(cfg.heads, dtype=np.float64)


# ---------------------------------------------------------------------------------------
# bf16 helpers (plain encodings, shared by both sides as input plumbing)
# ---------------------------------------------------------------------------------------
def bf16_bits_from_f64(x) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, round-half-to-even) -> uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                   # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)         # np.rint rounds half to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def f64_from_bf16_bits(u) -> np.ndarray:
    """Exact bf16 -> fp64 widening of uint16 bit patterns."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------
# generator
# ---------------------------------------------------------------------------------------
def _axis_index(cfg: Config):
    """Integer (t, h, w) of every raster token, each [N]."""
    n = np.arange(cfg.N, dtype=np.int64)
    return n // (cfg.H * cfg.W), (n // cfg.W) % cfg.H, n % cfg.W


def _head_rng(cfg: Config, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(cfg.seed,
                                                                      spawn_key=(head,))))


def _phasor(step: float, count: int, phase: float = 0.0):
    """cos and sin of step*i + phase for i < count, from the C library's scalar routines."""
    args = [step * i + phase for i in range(count)]
    return (np.array([math.cos(a) for a in args]), np.array([math.sin(a) for a in args]))


def _field(rng: np.random.Generator, cfg: Config, sigma: float, D: int) -> np.ndarray:
    """A [cos(omega . c_n + phi), sin(omega . c_n + phi)] / sqrt(8) over the raster grid.

    Built so that every value is a fixed sequence of single IEEE operations: per axis the
    scalar cos/sin of that axis' term (the phase rides on t), joined by the angle-addition
    formulas, and the mixing by A as 16 elementwise products summed in index order.  No BLAS
    call and no vectorised transcendental routine is involved, so the bytes do not depend on
    the CPU, the BLAS build or the number of threads."""
    omega = rng.normal(0.0, sigma, size=(8, 3))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=8)
    A = rng.standard_normal((D, 16))
    N = cfg.N
    z = np.empty((N, 16))
    for m in range(8):
        ct, st = _phasor(float(omega[m, 0]), cfg.T, float(phi[m]))
        ch, sh = _phasor(float(omega[m, 1]), cfg.H)
        cw, sw = _phasor(float(omega[m, 2]), cfg.W)
        c2 = ct[:, None] * ch[None, :] - st[:, None] * sh[None, :]          # [T, H]
        s2 = ct[:, None] * sh[None, :] + st[:, None] * ch[None, :]
        c3 = c2[:, :, None] * cw[None, None, :] - s2[:, :, None] * sw[None, None, :]
        s3 = c2[:, :, None] * sw[None, None, :] + s2[:, :, None] * cw[None, None, :]
        z[:, m] = c3.reshape(N)
        z[:, 8 + m] = s3.reshape(N)
    f = np.zeros((N, D))
    R = 2048                                       # rows per pass: the partial sums stay in cache
    tmp = np.empty((R, D))
    for r0 in range(0, N, R):
        r1 = min(N, r0 + R)
        fr, tr = f[r0:r1], tmp[:r1 - r0]
        for j in range(16):
            np.multiply(z[r0:r1, j:j + 1], A[None, :, j], out=tr)
            np.add(fr, tr, out=fr)
    f /= math.sqrt(8.0)
    return f


def _stripe_basis(cfg: Config) -> np.ndarray:
    _, hh, ww = _axis_index(cfg)
    cols = []
    for f in range(1, 5):
        ch, sh = _phasor(2 * math.pi * f / cfg.H, cfg.H)
        cw, sw = _phasor(2 * math.pi * f / cfg.W, cfg.W)
        cols += [ch[hh], sh[hh], cw[ww], sw[ww]]
    return np.stack(cols, axis=1)                                   # [N, 16]


def head_sigma(cfg: Config, rng: np.random.Generator) -> float:
    u = rng.uniform(-1.0, 1.0)            # always drawn, so the stream layout is fixed
    return cfg.sigma0 * (2.0 ** u) if cfg.per_head_sigma else cfg.sigma0


def _components(cfg: Config, rng: np.random.Generator, sigma: float):
    """The random parts of one head, in stream order: Q/K field, V field, noise of Q, K, V."""
    D = cfg.head_dim
    f = _field(rng, cfg, sigma, D)
    fv = _field(rng, cfg, sigma, D)
    eq = rng.standard_normal((cfg.N, D))
    ek = rng.standard_normal((cfg.N, D))
    ev = rng.standard_normal((cfg.N, D))
    return f, fv, eq, ek, ev


def _compose(cfg: Config, comps, gain: float, stripe):
    f, fv, eq, ek, ev = comps
    D = cfg.head_dim
    q = gain * (0.7 * f + 0.3 * eq)
    k = 0.7 * f + 0.3 * ek
    v = 0.7 * fv + 0.3 * ev
    if cfg.stripes:
        u = _stripe_basis(cfg) if stripe is None else stripe
        beta = 0.7 * math.sqrt(D / 8.0)
        q[:, :16] += gain * beta * u
        k[:, :16] += beta * u
    return q, k, v


def gen_head_f64(cfg: Config, head: int, gain: float = 1.0, stripe=None):
    """One head's (Q, K, V) in fp64, [N, D] each, before the bf16 rounding."""
    rng = _head_rng(cfg, head)
    s = head_sigma(cfg, rng)
    return _compose(cfg, _components(cfg, rng, s), gain, stripe)


def gen_qkv(cfg: Config, heads: Optional[Sequence[int]] = None,
            gains: Optional[np.ndarray] = None, threads: int = 0):
    """bf16 bit patterns (uint16) of Q, K, V, each [1, N, len(heads), D] (raster layout).

    `heads` selects a subset (default all); any subset reproduces exactly the same bytes as
    the full tensor restricted to those heads."""
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    gains = load_gains(cfg) if gains is None else np.asarray(gains, dtype=np.float64)
    N, D = cfg.N, cfg.head_dim
    stripe = _stripe_basis(cfg) if cfg.stripes else None
    out = [np.empty((1, N, len(heads), D), dtype=np.uint16) for _ in range(3)]

    def one(slot_head):
        slot, hd = slot_head
        qkv = gen_head_f64(cfg, hd, float(gains[hd]), stripe)
        for t in range(3):
            out[t][0, :, slot, :] = bf16_bits_from_f64(qkv[t])

    jobs = list(enumerate(heads))
    nthr = threads or min(8, os.cpu_count() or 1, len(jobs))
    if nthr > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out[0], out[1], out[2]


# ---------------------------------------------------------------------------------------
# denoising-step drift (for mask reuse across steps)
# ---------------------------------------------------------------------------------------
def gen_qkv_steps(cfg: Config, steps: Sequence[int], drift: float,
                  heads: Optional[Sequence[int]] = None, gains: Optional[np.ndarray] = None,
                  threads: int = 0):
    """Q, K, V of a layer at several denoising steps whose activations drift smoothly.

    Per head, the random parts at step s are cos(s*drift) x_a + sin(s*drift) x_b, where x_a
    are exactly the parts gen_qkv draws and x_b an independent draw of the same recipe (same
    frequency scale, its own stream); the stripe term and the gain stay fixed.  Every step has
    the distribution of the base workload, step 0 is byte-identical to gen_qkv, and two steps
    d apart have correlation cos(d*drift) in every random part.  Angles |s*drift| are limited
    to pi/2 (independent draws): past it the rotation turns towards -x_a, and since q.k is
    unchanged when Q and K both change sign, the masks of step 0 would come back.  Returns one
    (q, k, v) triple of bf16 bit arrays [1, N, len(heads), D] per entry of `steps`."""
    steps = list(steps)
    if any(abs(st * drift) > math.pi / 2 for st in steps):
        raise ValueError("step * drift must stay within [-pi/2, pi/2]")
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    gains = load_gains(cfg) if gains is None else np.asarray(gains, dtype=np.float64)
    N, D = cfg.N, cfg.head_dim
    stripe = _stripe_basis(cfg) if cfg.stripes else None
    out = [[np.empty((1, N, len(heads), D), dtype=np.uint16) for _ in range(3)] for _ in steps]

    def one(slot_head):
        slot, hd = slot_head
        rng = _head_rng(cfg, hd)
        sig = head_sigma(cfg, rng)
        xa = _components(cfg, rng, sig)
        rng_b = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
            cfg.seed, spawn_key=(hd, 1))))
        head_sigma(cfg, rng_b)                 # same stream layout; the scale is x_a's
        xb = _components(cfg, rng_b, sig)
        for si, st in enumerate(steps):
            th = st * drift
            if th == 0.0:
                comps = xa
            else:
                c, sn = math.cos(th), math.sin(th)
                comps = tuple(c * a + sn * b for a, b in zip(xa, xb))
            qkv = _compose(cfg, comps, float(gains[hd]), stripe)
            for t in range(3):
                out[si][t][0, :, slot, :] = bf16_bits_from_f64(qkv[t])

    jobs = list(enumerate(heads))
    nthr = threads or min(8, os.cpu_count() or 1, len(jobs))
    if nthr > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return [tuple(o) for o in out]

