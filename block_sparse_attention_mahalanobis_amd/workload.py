"""Seeded synthetic inputs for the Spark-Attn layer.

This module only draws random numbers.  It holds none of the method's
arithmetic (no moments, no whitening, no scores, no softmax), so both the
HIP path and the fp64 oracle can be fed from it without sharing any of the
computation they are compared on.

The real workload -- MiniMax-H3 layer activations on VBench prompts at
1344x768, 240 frames ("Spark-H3" page, Benchmark Results section) -- is not
available, so clustered Gaussian mixtures of the same shapes stand in for it:

* ``tiny``      fp32, H=1, N=1024, d=64, block 64, top-4 of 16 key blocks.
                4-component mixture, labels i.i.d. uniform; q, k and v all
                come from the mixture (means ~ N(0, 4I), std 0.5 times a
                per-component diag U(0.5, 2) scaling).
* ``draft``     bf16, latent grid 16x24x42 = 16,128 tokens, H=24, d=128,
                block 128, ratio 0.1.  64 components whose labels are the
                nearest of 64 seed points drawn uniformly in the (t, h, w)
                box (a Voronoi tessellation, so labels are smooth in space
                and time); q and k share labels but have separate means and
                scalings; v ~ N(0, 1).
* ``full768``   the same generator on the 61x48x84 = 245,952-token grid of a
                768p, 240-frame clip, H=40.
* ``sweep``     the ``draft`` shape with ratio in {0.1, 0.2, 0.3, 1.0}, on
                clustered q/k (``iid=False``) or on i.i.d. N(0, 1) q/k
                (``iid=True``), the latter standing in for early denoising
                steps where the spatio-temporal prior is weak.
* ``ref2va``    ``full768`` plus two 48x84 reference frames (8,064 tokens,
                254,016 in all) from a separate 8-component mixture; the
                anchor averages the 245,952 video queries only; ratio 0.2.

Every draw uses ``numpy.random.Generator(PCG64)``; each (head, tensor) pair
gets its own child ``SeedSequence`` spawned from the config seed, so any
single head can be regenerated alone.  Token order is raster (t, h, w).
bf16 workloads are rounded to bf16 (round to nearest even) here, once, and
returned as float32 arrays holding exactly bf16-representable values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_workload", "make_head", "round_to_bf16",
           "blocks_for", "topk_for"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str             # "f32" or "bf16"
    H: int
    d: int
    block: int
    ratio: float
    grid: Optional[tuple]  # (T, Hh, W) of the video latent, or None
    n_components: int
    iid: bool = False      # q, k i.i.d. N(0,1) instead of the mixture
    ref_grid: Optional[tuple] = None   # (T, Hh, W) of appended reference frames
    ref_components: int = 0
    N_flat: int = 0        # token count when there is no grid (tiny)

    @property
    def n_video(self) -> int:
        if self.grid is None:
            return self.N_flat
        return int(np.prod(self.grid))

    @property
    def N(self) -> int:
        n = self.n_video
        if self.ref_grid is not None:
            n += int(np.prod(self.ref_grid))
        return n

    @property
    def n_anchor(self) -> int:
        # the anchor averages the video queries only
        return self.n_video

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, "f32", 1, 64, 64, 0.25, None, 4, N_flat=1024),
    "draft": Workload("draft", 2, "bf16", 24, 128, 128, 0.1, (16, 24, 42), 64),
    "full768": Workload("full768", 3, "bf16", 40, 128, 128, 0.1, (61, 48, 84), 64),
    "sweep": Workload("sweep", 4, "bf16", 24, 128, 128, 0.1, (16, 24, 42), 64),
    "ref2va": Workload("ref2va", 5, "bf16", 40, 128, 128, 0.2, (61, 48, 84), 64,
                       ref_grid=(2, 48, 84), ref_components=8),
}


def blocks_for(N: int, block: int) -> int:
    """Number of token blocks, the last one possibly short."""
    return -(-N // block)


def topk_for(ratio: float, n_blocks: int) -> int:
    """Key blocks kept per query block for a density ratio: the smallest
    count that covers the ratio, clamped to [1, n_blocks]."""
    return int(min(n_blocks, max(1, math.ceil(ratio * n_blocks - 1e-9))))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); the result
    is float32 holding bf16-representable values.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = r.astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def _voronoi_labels(rng: np.random.Generator, grid: tuple, n_seeds: int) -> np.ndarray:
    """Label of the nearest of ``n_seeds`` uniform seed points, for every
    integer point of the grid in raster order (ties -> lower seed)."""
    T, Hh, W = grid
    seeds = rng.uniform(0.0, 1.0, size=(n_seeds, 3)) * np.array([T, Hh, W], dtype=np.float64)
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    pts = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.float64)
    best = np.full(pts.shape[0], np.inf)
    lab = np.zeros(pts.shape[0], dtype=np.int64)
    for s in range(n_seeds):
        dist = ((pts - seeds[s]) ** 2).sum(axis=1)
        better = dist < best
        best[better] = dist[better]
        lab[better] = s
    return lab


def _mixture(rng: np.random.Generator, labels: np.ndarray, n_comp: int, d: int) -> np.ndarray:
    """x = mu_z + 0.5 * D_z * eps with mu ~ N(0, 4I), D = diag U(0.5, 2)."""
    mu = rng.standard_normal((n_comp, d)) * 2.0
    scale = rng.uniform(0.5, 2.0, size=(n_comp, d)) * 0.5
    eps = rng.standard_normal((labels.shape[0], d), dtype=np.float32)
    return (mu[labels].astype(np.float32) + scale[labels].astype(np.float32) * eps)


def make_head(w: Workload, h: int) -> tuple:
    """q, k, v of head ``h`` as float32 arrays [N, d]."""
    root = np.random.SeedSequence([w.seed, 0x5A7C])
    head_ss = root.spawn(w.H)[h]
    s_lab, s_q, s_k, s_v, s_ref = head_ss.spawn(5)
    d = w.d
    n_vid = w.n_video
    if w.grid is None:
        labels = np.random.Generator(np.random.PCG64(s_lab)).integers(0, w.n_components, n_vid)
    else:
        labels = _voronoi_labels(np.random.Generator(np.random.PCG64(s_lab)), w.grid, w.n_components)
    gq = np.random.Generator(np.random.PCG64(s_q))
    gk = np.random.Generator(np.random.PCG64(s_k))
    gv = np.random.Generator(np.random.PCG64(s_v))
    if w.iid:
        q = gq.standard_normal((n_vid, d), dtype=np.float32)
        k = gk.standard_normal((n_vid, d), dtype=np.float32)
    else:
        q = _mixture(gq, labels, w.n_components, d)
        k = _mixture(gk, labels, w.n_components, d)
    if w.grid is None:
        v = _mixture(gv, labels, w.n_components, d)
    else:
        v = gv.standard_normal((n_vid, d), dtype=np.float32)
    if w.ref_grid is not None:
        gr = np.random.Generator(np.random.PCG64(s_ref))
        rlab = _voronoi_labels(gr, w.ref_grid, w.ref_components)
        rq = _mixture(gr, rlab, w.ref_components, d)
        rk = _mixture(gr, rlab, w.ref_components, d)
        rv = gr.standard_normal((rlab.shape[0], d), dtype=np.float32)
        q = np.concatenate([q, rq])
        k = np.concatenate([k, rk])
        v = np.concatenate([v, rv])
    out = []
    for x in (q, k, v):
        x = np.ascontiguousarray(x, dtype=np.float32)
        if w.dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return tuple(out)


def make_workload(w: Workload, heads: Optional[Sequence[int]] = None, threads: int = 8) -> tuple:
    """q, k, v as float32 arrays [len(heads), N, d] (all heads by default)."""
    heads = list(range(w.H)) if heads is None else list(heads)
    N, d = w.N, w.d
    q = np.empty((len(heads), N, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def one(i):
        q[i], k[i], v[i] = make_head(w, heads[i])

    with ThreadPoolExecutor(max(1, min(threads, len(heads)))) as ex:
        list(ex.map(one, range(len(heads))))
    return q, k, v
