"""Oracle for the data-independent comparison path (TurboQuant-style): a
randomized Walsh-Hadamard rotation followed by a fixed Lloyd-Max codebook.
fp64 throughout unless stated. Test infrastructure only.

Source: "Technisch Overzicht: Ablatie, Statistische Inferentie en Validatie
voor KV-Cache Compressie" (gist.science, Dutch summary), "Experimentele
Opstelling" (TurboQuant: a randomized Walsh-Hadamard transform spreads each
token's energy evenly, then a data-independent Beta Lloyd-Max codebook) and
"Regime-specifieke prestaties" (the rotation makes heavy-tailed marginals close
to Gaussian).

Every function is pinned by tests/test_oracle_rht.py; none is "parity
unpinned".
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

from . import codec

RHT_BITS = 3


def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (natural
    / Sylvester order): butterflies (a, b) -> (a + b, a - b) at spans 1, 2, 4..."""
    v = np.array(v, dtype=np.float64, copy=True)
    d = v.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        for start in range(0, d, 2 * h):
            a = v[..., start:start + h].copy()
            b = v[..., start + h:start + 2 * h].copy()
            v[..., start:start + h] = a + b
            v[..., start + h:start + 2 * h] = a - b
        h *= 2
    return v


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = H (D x) / sqrt(d): the seeded +-1 diagonal D first, then the FWHT.
    READING: orthonormal scaling 1/sqrt(d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return fwht(x * np.asarray(signs, dtype=np.float64)) / math.sqrt(d)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse of `rotate`: x = D H y / sqrt(d) (H is symmetric, H H = d I)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    return fwht(y) / math.sqrt(d) * np.asarray(signs, dtype=np.float64)


def lloyd_max(samples: np.ndarray, levels: int = 1 << RHT_BITS, tol: float = 1e-12,
              max_iter: int = 10000):
    """Lloyd's algorithm on training samples. READING (the pages name a Beta
    Lloyd-Max codebook but fix no procedure): start from the sample quantiles
    (k + 1/2)/L; alternate thresholds = midpoints of neighbouring centroids and
    centroids = mean of the samples in each cell (a sample equal to a threshold
    belongs to the upper cell); stop when no centroid moves by `tol` or more.
    Returns (centroids fp64, iterations)."""
    y = np.asarray(samples, dtype=np.float64)
    c = np.quantile(y, (np.arange(levels) + 0.5) / levels)
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        cell = (y[:, None] >= t[None, :]).sum(axis=1)
        sums = np.bincount(cell, weights=y, minlength=levels)
        cnts = np.bincount(cell, minlength=levels)
        new = np.where(cnts > 0, sums / np.maximum(cnts, 1), c)
        moved = float(np.max(np.abs(new - c)))
        c = new
        if moved < tol:
            return c, it
    return c, max_iter


def codebook_fp32(centroids: np.ndarray) -> np.ndarray:
    """The stored codebook: centroids rounded to fp32."""
    return np.asarray(centroids, dtype=np.float64).astype(np.float32)


def codebook_thresholds(cb32: np.ndarray) -> np.ndarray:
    """Decision thresholds: fl32 of the midpoints of neighbouring fp32
    centroids (the midpoint is exact in fp64)."""
    c = np.asarray(cb32, dtype=np.float32).astype(np.float64)
    return (0.5 * (c[:-1] + c[1:])).astype(np.float32)


def make_state(signs: np.ndarray, cb32: np.ndarray) -> Dict:
    signs = np.asarray(signs, dtype=np.int8)
    d = signs.shape[0]
    bits = np.full(d, RHT_BITS, dtype=np.uint8)
    return {"xform": codec.XFORM_RHT, "signs": signs,
            "codebook": np.asarray(cb32, dtype=np.float32),
            "thresholds": codebook_thresholds(cb32), "bits": bits,
            "total_bits": int(bits.astype(np.int64).sum())}


def encode_kv(state: Dict, x: np.ndarray):
    """Per token: norm nu = |x|, y = H D (x / nu) / sqrt(d), 3-bit codes from
    the codebook thresholds (count of thresholds <= fl32(y)), F1 packing with
    3 bits on every channel. READING: nu is stored per token as fp32 so that
    the codebook stays data-independent; nu = 0 gives y = 0.
    Returns (packed bytes, norms fp32)."""
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    u = np.where(nu[:, None] > 0, x / np.where(nu > 0, nu, 1.0)[:, None], 0.0)
    y = rotate(u, state["signs"])
    thr = state["thresholds"]
    q = np.stack([codec.quantize_channel(y[:, j], thr) for j in range(y.shape[1])], axis=1)
    return codec.pack(q, state["bits"]), nu.astype(np.float32)


def reconstruct_exact(state: Dict, packed: np.ndarray, norms: np.ndarray, n: int) -> np.ndarray:
    """x_hat = nu D H y_hat / sqrt(d) with y_hat the codebook values, fp64."""
    q = codec.unpack(packed, state["bits"], n)
    yhat = state["codebook"].astype(np.float64)[q]
    nu = np.asarray(norms, dtype=np.float32).astype(np.float64)[:n]   # one norm per token of the n
    return unrotate(yhat, state["signs"]) * nu[:, None]


def decode_kv(state: Dict, packed: np.ndarray, norms: np.ndarray, n: int, dtype: str) -> np.ndarray:
    return codec.round_to(reconstruct_exact(state, packed, norms, n), dtype)


def attend_compressed(k_state: Dict, v_state: Dict, k_packed: np.ndarray, k_norms: np.ndarray,
                      v_packed: np.ndarray, v_norms: np.ndarray, n: int, q: np.ndarray,
                      scale=None) -> np.ndarray:
    """One decode step over a Walsh-Hadamard (TurboQuant-style) cache, the
    decode-time side of the SQ versus TQ comparison (ablation summary,
    "Regime-Specifieke Prestaties en Kalibratiesensitiviteit" and "Opslag vs.
    Kwaliteit"): keys and values are the exact fp64 reconstructions
    nu D H y_hat / sqrt(d), then the same softmax attention as the eigen
    cache. Returns fp32 [g][d]."""
    khat = reconstruct_exact(k_state, k_packed, k_norms, n)
    vhat = reconstruct_exact(v_state, v_packed, v_norms, n)
    return codec.softmax_attention(q, khat, vhat, scale)

