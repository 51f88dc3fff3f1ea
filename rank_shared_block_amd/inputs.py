"""Seeded synthetic inputs for the reconstructed-linear workloads.

This module serves both the GPU path (tests, bench) and the CPU oracle (tests,
the bench's CPU baseline).  It holds none of the method's arithmetic: only
random draws, the rounding of each draw to the storage dtype, and the shapes of
the workloads.  Everything is returned as numpy float32 arrays whose values are
exactly representable in the requested dtype ("bf16" or "f32"); the rounded
arrays are the ground truth that both sides consume.

Recipe (one independent stream per tensor):

* generator: ``numpy.random.default_rng(SeedSequence([seed, workload, layer_or_band,
  family, tensor]))``, seed 0 by default;
* ``W0 ~ N(0, std = 1/sqrt(in_dim))`` (one per band and family; a band holds
  ``L / G`` consecutive layers), ``s ~ U(0.9, 1.1)``, ``U, V ~ N(0, std = 0.02)``
  (``V`` drawn directly in its transposed ``[r, in_dim]`` layout),
  ``x ~ N(0, 1)``;
* normals are float32 ziggurat draws scaled by the float32 std; uniforms are
  float64 draws cast to float32; each value is then rounded once, to nearest
  with ties to even, onto the bf16 grid when the dtype is bf16.

Projection shapes are ``(in_dim, out_dim)`` as in the model configs: the
Gemma-3-1B-shaped decoder (hidden 1152) and a larger decoder (hidden 5376).
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

FAMILIES = ("q", "k", "v", "o", "gate", "up", "down")
FAMILY_ID = {f: i for i, f in enumerate(FAMILIES)}
TENSOR_ID = {"W0": 0, "s": 1, "U": 2, "Vt": 3, "x": 4, "omega": 5, "W": 6}

# (in_dim, out_dim) per family
GEMMA_1B = {"q": (1152, 1024), "k": (1152, 256), "v": (1152, 256), "o": (1024, 1152),
            "gate": (1152, 6912), "up": (1152, 6912), "down": (6912, 1152)}
LARGE_DECODER = {"q": (5376, 4096), "k": (5376, 2048), "v": (5376, 2048), "o": (4096, 5376),
                 "gate": (5376, 21504), "up": (5376, 21504), "down": (21504, 5376)}

# Workload ids used in the seed path (stable; never renumber).
WORKLOAD_ID = {"single_f32": 1, "gemma_decode": 2, "gemma_prefill": 3,
               "large_decoder": 4, "materialize_fp4": 5, "decompose": 6, "test": 9}

# One decoder layer = four dispatches: fused QKV, o, fused gate/up, down.
LAYER_DISPATCHES = (("qkv", ("q", "k", "v")), ("o", ("o",)),
                    ("gateup", ("gate", "up")), ("down", ("down",)))


def round_to_bf16(a):
    """Round float32 values to the nearest bfloat16 (ties to even), in place-safe
    float32 storage.  Inputs must be finite."""
    a = np.ascontiguousarray(a, dtype=np.float32).copy()
    u = a.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def _rng(seed, key):
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(k) for k in key]))


def _finish(a, dtype):
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")


def normal(key, shape, std, dtype, seed=0):
    a = _rng(seed, key).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return _finish(a, dtype)


def uniform(key, shape, lo, hi, dtype, seed=0):
    a = _rng(seed, key).uniform(lo, hi, size=shape).astype(np.float32)
    return _finish(a, dtype)


def bundle(workload, layer, family, in_dim, out_dim, r, dtype, band=None,
           variant="normal", seed=0, draw_w0=True):
    """One projection's theta bundle: dict with W0 [N,K], s [N], U [N,r], Vt [r,K].

    ``band`` selects the shared W0 (default: one band per layer).  Variants:
    ``normal``; ``r0`` (rank 0, empty U/Vt); ``passthrough`` (s = 1, U = Vt = 0,
    W0 = the drawn weight, i.e. the layer's own weight); ``s0`` (s = 0, only the
    low-rank term remains; a stress case for the U/V path).  ``draw_w0=False``
    leaves W0 as None (a caller that already holds the band's identical draw).
    """
    wid, fid = WORKLOAD_ID[workload], FAMILY_ID.get(family, family)
    K, N = in_dim, out_dim
    b = layer if band is None else band
    W0 = normal((wid, 1000 + b, fid, TENSOR_ID["W0"]), (N, K), 1.0 / np.sqrt(K), dtype, seed) if draw_w0 else None
    if variant == "r0":
        r = 0
    s = uniform((wid, layer, fid, TENSOR_ID["s"]), (N,), 0.9, 1.1, dtype, seed)
    U = normal((wid, layer, fid, TENSOR_ID["U"]), (N, r), 0.02, dtype, seed)
    Vt = normal((wid, layer, fid, TENSOR_ID["Vt"]), (r, K), 0.02, dtype, seed)
    if variant == "passthrough":
        if W0 is None:
            raise ValueError("passthrough needs the drawn W0")
        s = np.ones((N,), np.float32)
        U = np.zeros((N, r), np.float32)
        Vt = np.zeros((r, K), np.float32)
    elif variant == "s0":
        s = np.zeros((N,), np.float32)
    elif variant not in ("normal", "r0"):
        raise ValueError(f"unknown variant {variant!r}")
    return {"W0": W0, "s": s, "U": U, "Vt": Vt}


def activations(workload, tag, M, K, dtype, seed=0):
    """x ~ N(0, 1), [M, K]; ``tag`` separates the inputs of different dispatches."""
    return normal((WORKLOAD_ID[workload], 50000 + int(tag), 0, TENSOR_ID["x"]),
                  (M, K), 1.0, dtype, seed)


def layer_bundles(workload, shapes, layers, r, dtype, num_bands=None, seed=0,
                  families=FAMILIES, threads=None):
    """Bundles for ``layers`` decoder layers: {layer: {family: bundle}}.

    With ``num_bands`` = G the W0 of layer l is band floor(l * G / L)'s (all
    layers of a band share the identical array object).  Draws run on a thread
    pool (numpy releases the GIL inside its bulk fills).
    """
    L = layers
    G = L if num_bands is None else num_bands
    band = [(l * G) // L for l in range(L)]
    threads = threads or min(16, os.cpu_count() or 1)
    first = {}                             # the first layer of each band draws its W0
    for l in range(L):
        first.setdefault(band[l], l)
    jobs = [(l, f) for l in range(L) for f in families]

    def one(job):
        l, f = job
        K, N = shapes[f]
        return job, bundle(workload, l, f, K, N, r, dtype, band=band[l], seed=seed,
                           draw_w0=first[band[l]] == l)

    with ThreadPoolExecutor(threads) as ex:
        done = dict(ex.map(one, jobs))
    out = {l: {} for l in range(L)}
    for (l, f), bd in done.items():
        if bd["W0"] is None:               # the same draw as the band's first layer: share it
            bd["W0"] = done[(first[band[l]], f)]["W0"]
        out[l][f] = bd
    return out


def gaussian_probe(workload, tag, l, K, seed=0):
    """The randomized SVD's Gaussian test matrix, [l, K] float64 ~ N(0, 1):
    each row one probe (drawn here so that both sides use the same one)."""
    return _rng(seed, (WORKLOAD_ID[workload], 70000 + int(tag), 0, TENSOR_ID["omega"])).standard_normal((l, K))


def trained_weight(workload, layer, family, in_dim, out_dim, dtype, band=None, waves=4, seed=0):
    """A synthetic stand-in for a trained projection weight [out_dim, in_dim]
    (no checkpoint is used): the band's shared draw W0 ~ N(0, 1/in_dim) with a
    row scale a ~ U(0.8, 1.2) drawn per layer, plus a smooth perturbation of
    low rank -- ``waves`` cosine waves over the (row, column) index grid, each
    of rank 2, amplitudes 0.2/sqrt(in_dim) down to 0.05/sqrt(in_dim),
    frequencies and phases drawn per layer -- plus noise ~ N(0, (0.01/sqrt(in_dim))^2).
    Rounded once to ``dtype``.  Layers of one band share the W0 draw, so the
    band mean of their weights is close to it."""
    wid, fid = WORKLOAD_ID[workload], FAMILY_ID.get(family, family)
    K, N = in_dim, out_dim
    b = layer if band is None else band
    base = _rng(seed, (wid, 1000 + b, fid, TENSOR_ID["W0"])).standard_normal((N, K), dtype=np.float32)
    g = _rng(seed, (wid, layer, fid, TENSOR_ID["W"]))
    a = g.uniform(0.8, 1.2, size=(N, 1))
    sd = 1.0 / np.sqrt(K)
    w = base.astype(np.float64) * (a * sd)
    n = np.arange(N, dtype=np.float64)[:, None] / N
    k = np.arange(K, dtype=np.float64)[None, :] / K
    for i in range(waves):
        amp = sd * (0.2 - 0.15 * i / max(1, waves - 1))
        fn, fk = g.uniform(0.5, 6.0, size=2)
        ph = g.uniform(0.0, 2.0 * np.pi)
        w += amp * np.cos(2.0 * np.pi * (fn * n + fk * k) + ph)
    w += g.standard_normal((N, K)) * (0.01 * sd)
    return _finish(w.astype(np.float32), dtype)
