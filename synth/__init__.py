"""Seeded synthetic inputs for the KV-cache codec.

This module is shared by the tests, the benchmark and the smoke check. It holds
no step of the codec itself: it only draws K/V token streams, decode-step
queries, random sign vectors and codebook training samples, with the shapes and
value distributions of the workloads below. Both the CPU oracle and the GPU
path receive the same arrays from here.

Value distributions follow the pages' description of the cache statistics:

* SPECTRA technical summary (gist.science, "Metodologia", observation 1): in
  the raw channel basis the KV channels are strongly correlated, and in the
  basis of the cache's own Gram matrix the energy concentrates in a few
  channels. Modelled as a power-law spectrum ``lambda_i = i**-alpha`` behind a
  random orthogonal rotation, plus a few raw-basis outlier channels.
* Ablation summary (gist.science/nl, "Regime-specifieke prestaties"):
  heavy-tailed data, modelled as Student-t(3) entries behind a random rotation.

Seeds: ``np.random.default_rng([cfg, layer, batch, head, kind, purpose])`` with
kind K=0 / V=1 and purpose 0 rotation, 1 samples, 2 outlier channels,
3 queries, 4 random signs, 5 codebook training samples, 6 per-layer decay,
7 the Gaussian matrix of the 1-bit residual sketch.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "rng_for", "haar_orthogonal", "spiked_gaussian",
    "student_t_rotated", "stream", "queries", "random_signs",
    "sphere_coordinate_samples", "layer_alpha", "to_bf16_values",
    "bf16_bits", "bf16_bits_to_f32",
]

D = 128
KIND_K, KIND_V = 0, 1
P_ROT, P_SAMPLES, P_OUTLIER, P_QUERY, P_SIGNS, P_LLOYD, P_ALPHA, P_SKETCH = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distribution and codec budgets."""
    cfg: int
    name: str
    layers: int
    batch: int
    kv_heads: int
    group: int               # query heads per KV head (GQA group size)
    n_tokens: int
    dtype: str               # "f32" or "bf16"
    data: str                # "spiked" or "student_t"
    alpha: Optional[float]   # spectrum decay; None -> per layer U(0.8, 1.5)
    n_outliers: int
    outlier_scale: float
    n_calib: Optional[int]
    budgets: Tuple[float, ...]
    share_over_batch: bool = False

    @property
    def n_streams(self) -> int:
        return self.layers * self.batch * self.kv_heads * 2


def _n_out(frac: float) -> int:
    # "1% / 2% outlier channels" of a 128-wide head, rounded up.
    return int(math.ceil(frac * D - 1e-9))


WORKLOADS = {
    1: Workload(1, "tiny codec, 1 layer x 1 KV head, 4096 fp32 tokens",
                1, 1, 1, 4, 4096, "f32", "spiked", 1.0, 4, 20.0, 1024, (2.0,)),
    2: Workload(2, "Llama-3.1-8B-shaped layer, 8 KV heads, GQA 4, 32768 bf16 tokens",
                1, 1, 8, 4, 32768, "bf16", "spiked", 1.2, _n_out(0.01), 20.0, 2048,
                (4.0, 2.0, 1.33)),
    3: Workload(3, "Student-t(3) rotated K/V on the Llama layer shape (RHT path)",
                1, 1, 8, 4, 32768, "bf16", "student_t", None, 0, 1.0, None, (3.0,)),
    4: Workload(4, "Llama-3.1-8B-shaped cache, 32 layers x 8 KV heads, 131072 bf16 tokens",
                32, 1, 8, 4, 131072, "bf16", "spiked", None, _n_out(0.01), 20.0, 2048,
                (2.0,)),
    5: Workload(5, "Qwen2.5-7B-shaped batched decode, 28 layers x 4 KV heads x batch 16",
                28, 16, 4, 7, 32768, "bf16", "spiked", 1.0, _n_out(0.02), 30.0, 2048,
                (1.33,), share_over_batch=True),
}


def rng_for(cfg: int, layer: int, batch: int, head: int, kind: int, purpose: int):
    return np.random.default_rng([cfg, layer, batch, head, kind, purpose])


def haar_orthogonal(rng, d: int = D) -> np.ndarray:
    """Random orthogonal matrix, Haar-distributed (QR of a Gaussian matrix with
    the signs of diag(R) moved into Q, Mezzadri 2007)."""
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def layer_alpha(w: Workload, layer: int) -> float:
    if w.alpha is not None:
        return float(w.alpha)
    return float(rng_for(w.cfg, layer, 0, 0, 0, P_ALPHA).uniform(0.8, 1.5))


def spiked_gaussian(n: int, alpha: float, q: np.ndarray, n_out: int, scale: float,
                    rng_z, rng_out) -> np.ndarray:
    """x = (z * sqrt(lambda)) Q^T with lambda_i = i^-alpha, then n_out raw
    channels multiplied by `scale`. fp64."""
    lam = np.arange(1, D + 1, dtype=np.float64) ** (-alpha)
    z = rng_z.standard_normal((n, D))
    x = (z * np.sqrt(lam)[None, :]) @ q.T
    if n_out > 0:
        idx = rng_out.permutation(D)[:n_out]
        x[:, idx] *= scale
    return x


def student_t_rotated(n: int, q: np.ndarray, rng_z, nu: float = 3.0) -> np.ndarray:
    t = rng_z.standard_t(nu, size=(n, D))
    return t @ q.T


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (RNE); returned as the exact values in fp32."""
    return bf16_bits_to_f32(bf16_bits(np.asarray(x, dtype=np.float32)))


def stream(w: Workload, layer: int, batch: int, head: int, kind: int,
           n: Optional[int] = None) -> np.ndarray:
    """One K or V stream, [n][128], as fp32 values exactly representable in the
    workload's dtype (bf16 values are returned widened to fp32)."""
    n = w.n_tokens if n is None else n
    b_shared = 0 if w.share_over_batch else batch
    q = haar_orthogonal(rng_for(w.cfg, layer, b_shared, head, kind, P_ROT))
    rng_z = rng_for(w.cfg, layer, batch, head, kind, P_SAMPLES)
    if w.data == "spiked":
        x = spiked_gaussian(n, layer_alpha(w, layer), q, w.n_outliers, w.outlier_scale,
                            rng_z, rng_for(w.cfg, layer, b_shared, head, kind, P_OUTLIER))
    else:
        x = student_t_rotated(n, q, rng_z)
    x32 = x.astype(np.float32)
    return to_bf16_values(x32) if w.dtype == "bf16" else x32


def queries(w: Workload, layer: int, batch: int, head: int) -> np.ndarray:
    """Decode-step queries of the `group` query heads that share KV head
    `head`: N(0, I) fp32, [group][128]."""
    rng = rng_for(w.cfg, layer, batch, head, 0, P_QUERY)
    return rng.standard_normal((w.group, D)).astype(np.float32)


def random_signs(cfg: int, layer: int, batch: int, head: int, kind: int) -> np.ndarray:
    """Seeded +-1 diagonal of the randomized Walsh-Hadamard transform, int8."""
    rng = rng_for(cfg, layer, batch, head, kind, P_SIGNS)
    return (rng.integers(0, 2, size=D) * 2 - 1).astype(np.int8)


def sketch_matrix(cfg: int, layer: int, batch: int, head: int, kind: int, m: int = D) -> np.ndarray:
    """Seeded Gaussian matrix S [m][128] (iid N(0, 1), fp32) of the 1-bit
    Johnson-Lindenstrauss residual sketch of one stream."""
    rng = rng_for(cfg, layer, batch, head, kind, P_SKETCH)
    return rng.standard_normal((m, D)).astype(np.float32)


def sphere_coordinate_samples(n: int = 1_000_000, d: int = D, seed_cfg: int = 3) -> np.ndarray:
    """Samples of one coordinate of a uniform point on the unit sphere S^(d-1):
    y = 2 Beta((d-1)/2, (d-1)/2) - 1. These train the data-independent
    codebook of the Walsh-Hadamard path."""
    rng = rng_for(seed_cfg, 0, 0, 0, 0, P_LLOYD)
    a = (d - 1) / 2.0
    return 2.0 * rng.beta(a, a, size=n) - 1.0
