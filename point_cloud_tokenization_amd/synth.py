"""Seeded synthetic pulse batches for tests and benchmarks.

The pages measure on real IceCube events that are not available here, so these
generators stand in for them with the same shapes and structure: a CSR batch
of events, coords [N,4] float32 (x, y, z, t), features [N,C] float32 with a
positive charge column, and int64 offsets [B+1].  This module holds no step of
the tokenizer; it only draws inputs.  All arithmetic is float64, rounded once
to float32.  numpy's PCG64 generator makes every batch a pure function of its
seed.

Workloads (sizes follow the shapes the pages describe: coords [N,4] with time
in the fourth column and six point features by default, num_patches = 128 --
README of felixyu7/neptune, "Usage" and "Parameters"):

  tiny_uniform          4 events, n = 50, 200, 1000, 3000, coords U[-1,1]^4,
                        P = 128, Voronoi, plain mean pool
  icecube_b64_voronoi   64 IceCube-shaped events, n ~ LogNormal(median 100,
                        sigma 1) clipped to [5, 5000], P = 128, Voronoi,
                        charge-weighted pool
  icecube_b64_knn16     same events, kNN mode with k = 16
  icecube_b256_lloyd3   256 such events, C = 16, three Lloyd rounds
  icecube_highE_b512    512 events, n ~ LogNormal(median 2000, sigma 1.2)
                        clipped to [100, 200000], P = 256

IceCube-shaped geometry: 86 strings on a triangular lattice with 125 m
spacing (the 85 lattice sites strictly inside r = 625 m plus the site at
(625 m, 0), which is first by angle among the six sites at r = 625 m), 60
sensors per string 17 m apart centred on z = 0.  Each event: a track vertex
uniform in the instrumented cylinder, a direction uniform on the sphere; each
pulse picks a sensor uniformly with replacement, and its time is the signed
distance along the track divided by c plus an Exponential(50 ns) delay.
x, y, z are standardized by /500 m and t by /3000 ns.  Features are standard
normal with column 5 replaced by a LogNormal(0, 1) charge.
"""
from __future__ import annotations

import math

import numpy as np

C_LIGHT_M_PER_NS = 0.299792458
CHARGE_COL = 5

WORKLOADS = {
    "tiny_uniform": dict(kind="uniform", ns=(50, 200, 1000, 3000), P=128, C=6, mode=0, k=16,
                         L=0, weighted=False, cfg=0),
    "icecube_b64_voronoi": dict(kind="icecube", B=64, median=100.0, sigma=1.0, lo=5, hi=5000,
                                P=128, C=6, mode=0, k=16, L=0, weighted=True, cfg=1),
    "icecube_b64_knn16": dict(kind="icecube", B=64, median=100.0, sigma=1.0, lo=5, hi=5000,
                              P=128, C=6, mode=1, k=16, L=0, weighted=True, cfg=2),
    "icecube_b256_lloyd3": dict(kind="icecube", B=256, median=100.0, sigma=1.0, lo=5, hi=5000,
                                P=128, C=16, mode=0, k=16, L=3, weighted=True, cfg=3),
    "icecube_highE_b512": dict(kind="icecube", B=512, median=2000.0, sigma=1.2, lo=100,
                               hi=200000, P=256, C=6, mode=0, k=16, L=0, weighted=True, cfg=4),
}
WORKLOAD_ORDER = list(WORKLOADS)


def timing_seed(name: str) -> int:
    return 1000 + WORKLOADS[name]["cfg"]


def parity_seed(name: str, r: int) -> int:
    return 1000 + WORKLOADS[name]["cfg"] + 10 * r


_GEOM = None


def icecube_geometry() -> np.ndarray:
    """[5160, 3] float64 sensor positions in metres."""
    global _GEOM
    if _GEOM is None:
        sites = []
        for i in range(-12, 13):
            for j in range(-12, 13):
                norm = i * i + i * j + j * j  # (r / 125 m)^2, exact integer
                x = 125.0 * (i + 0.5 * j)
                y = 125.0 * j * math.sqrt(3.0) / 2.0
                ang = math.atan2(y, x)
                if ang < 0.0:
                    ang += 2.0 * math.pi
                sites.append((norm, ang, x, y))
        sites.sort(key=lambda s: (s[0], s[1]))
        strings = np.array([(s[2], s[3]) for s in sites[:86]], dtype=np.float64)
        z = -501.5 + 17.0 * np.arange(60, dtype=np.float64)
        xy = np.repeat(strings, 60, axis=0)
        zz = np.tile(z, 86)
        _GEOM = np.column_stack([xy, zz])
    return _GEOM


def _features(rng, N, C):
    f = rng.standard_normal((N, C))
    if C > CHARGE_COL:
        f[:, CHARGE_COL] = np.exp(rng.standard_normal(N))
    return f


def _pack(ns, coords, feats):
    offsets = np.zeros(len(ns) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(ns, dtype=np.int64))
    return dict(coords=np.ascontiguousarray(coords, dtype=np.float32),
                features=np.ascontiguousarray(feats, dtype=np.float32),
                offsets=offsets)


def icecube_sizes(rng, B, median, sigma, lo, hi):
    n = np.rint(np.exp(math.log(median) + sigma * rng.standard_normal(B)))
    return np.clip(n, lo, hi).astype(np.int64)


def icecube_events(ns, seed, C=6):
    """IceCube-shaped events of the given sizes."""
    rng = np.random.default_rng(seed)
    ns = np.asarray(ns, dtype=np.int64)
    B = ns.size
    N = int(ns.sum())
    geom = icecube_geometry()
    r = 625.0 * np.sqrt(rng.random(B))
    phi = 2.0 * math.pi * rng.random(B)
    vz = rng.uniform(-501.5, 501.5, B)
    vtx = np.column_stack([r * np.cos(phi), r * np.sin(phi), vz])
    cth = rng.uniform(-1.0, 1.0, B)
    sth = np.sqrt(1.0 - cth * cth)
    ph2 = 2.0 * math.pi * rng.random(B)
    u = np.column_stack([sth * np.cos(ph2), sth * np.sin(ph2), cth])
    ev = np.repeat(np.arange(B), ns)
    dom = geom[rng.integers(0, geom.shape[0], N)]
    along = np.einsum("ij,ij->i", dom - vtx[ev], u[ev])
    t = along / C_LIGHT_M_PER_NS + rng.exponential(50.0, N)
    coords = np.column_stack([dom / 500.0, t / 3000.0])
    return _pack(ns, coords, _features(rng, N, C))


def uniform_events(ns, seed, C=6, lo=-1.0, hi=1.0):
    """coords i.i.d. uniform in [lo, hi]^4."""
    rng = np.random.default_rng(seed)
    N = int(np.sum(ns))
    coords = rng.uniform(lo, hi, (N, 4))
    return _pack(ns, coords, _features(rng, N, C))


def grid_events(ns, seed, C=6, side=3):
    """Tie-rich clouds: coords drawn from the integer grid {0..side-1}^4, so
    many pulses coincide and many distances are exactly equal."""
    rng = np.random.default_rng(seed)
    N = int(np.sum(ns))
    coords = rng.integers(0, side, (N, 4)).astype(np.float64)
    return _pack(ns, coords, _features(rng, N, C))


def identical_events(ns, seed, C=6):
    """Every pulse of an event at the same position (a random point per event)."""
    rng = np.random.default_rng(seed)
    ns = np.asarray(ns, dtype=np.int64)
    pts = rng.uniform(-1.0, 1.0, (ns.size, 4))
    coords = np.repeat(pts, ns, axis=0)
    return _pack(ns, coords, _features(rng, int(ns.sum()), C))


def seed_copies_events(ns, seed, C=6, strides=None):
    """Clouds where most pulses are exact copies of pulse 0 (the default FPS
    seed) and every stride-th pulse (positions stride-1, 2*stride-1, ...)
    lies on a far shell of radius 2..3.  After the first selection every
    copy has distance 0, so when the stride equals the number of pulses a
    lane holds, every lane's second-farthest distance is 0 while its
    farthest is large: many more candidates than a candidate list holds,
    and, once the far pulses are used up, the all-zero case."""
    rng = np.random.default_rng(seed)
    ns = np.asarray(ns, dtype=np.int64)
    strides = np.ones_like(ns) if strides is None else np.asarray(strides, dtype=np.int64)
    parts = []
    for n, st in zip(ns, strides):
        base = rng.uniform(-1.0, 1.0, 4)
        c = np.repeat(base[None, :], n, axis=0)
        far = np.arange(n) % st == st - 1
        far[0] = False
        k = int(far.sum())
        d = rng.standard_normal((k, 4))
        d /= np.linalg.norm(d, axis=1, keepdims=True)
        c[far] = base + d * rng.uniform(2.0, 3.0, (k, 1))
        parts.append(c)
    coords = np.concatenate(parts) if parts else np.zeros((0, 4))
    return _pack(ns, coords, _features(rng, int(ns.sum()), C))


def make_batch(name: str, seed: int | None = None) -> dict:
    """A batch of the named workload: coords, features, offsets and the
    tokenizer parameters (P, mode, k, L, weighted, charge_col)."""
    w = WORKLOADS[name]
    if seed is None:
        seed = timing_seed(name)
    if w["kind"] == "uniform":
        batch = uniform_events(w["ns"], seed, C=w["C"])
    else:
        rng = np.random.default_rng(seed ^ 0x5EED)
        ns = icecube_sizes(rng, w["B"], w["median"], w["sigma"], w["lo"], w["hi"])
        batch = icecube_events(ns, seed, C=w["C"])
    batch.update(workload=name, seed=seed, P=w["P"], mode=w["mode"], k=w["k"], L=w["L"],
                 weighted=w["weighted"], charge_col=CHARGE_COL)
    return batch
