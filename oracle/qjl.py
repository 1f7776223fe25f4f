"""Oracle of the 1-bit Johnson-Lindenstrauss residual sketch on the key
path of the Walsh-Hadamard cache (TQ-QKV in the ablation summary,
"Experimentele Opstelling" and "Belangrijkste Bijdragen" 1; the Jensen
amplification of its score noise in "Statistische Validatie en Jensen's
Ongelijkheid"). Test infrastructure only: the tests, the smoke check and the
CPU baseline of the benchmark use it; the library never does.

The eigen cache gets SpectralQuant's selective sketch (ablation summary,
"Experimentele Opstelling": SpectralQuant restricts its QJL sketch to the
leading effective dimensions). READING: it covers the quantization residual of the
water-filled channels, r_j = c_j - c_hat_j for the kept channels with a
positive step, in the latent basis (0 for dropped channels); the query is
taken to the same basis, so the estimate of (U^T q) . r is
sqrt(pi/2) / m ||r|| (S U^T q) . z.

READINGs (the pages give no parameters): m = 128 sketch bits per token;
S [m][d] iid N(0, 1), seeded per stream and passed in; the sketch of key k
is z = sign(S r) of the residual r = k - K_hat (K_hat the exact
reconstruction of its codes), sign(0) = +1, stored as one bit per row
(1 = non-negative) in the F1 layout with 1-bit channels; ||r|| is kept as
fp32; the score estimate of q . r is sqrt(pi/2) / m ||r|| (S q) . z, the
standard unbiased estimator for Gaussian S, added to q . K_hat before the
softmax. Values get no sketch (the pages drop V-path sketches).
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

from . import codec, rht

SKETCH_BITS = 128


def sketch_bits_vector(m: int = SKETCH_BITS) -> np.ndarray:
    return np.ones(m, dtype=np.uint8)


def sketch_encode(k_state: Dict, x: np.ndarray, k_packed: np.ndarray, k_norms: np.ndarray,
                  S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Sketch of the keys x [n][d] whose Walsh-Hadamard codes and norms are
    given: (packed sign bits, ||r|| fp32 [n])."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    S = np.asarray(S, dtype=np.float32).astype(np.float64)
    r = x - rht.reconstruct_exact(k_state, k_packed, k_norms, n)
    proj = r @ S.T                                   # [n][m]
    z = (proj >= 0.0).astype(np.int64)
    return codec.pack(z, sketch_bits_vector(S.shape[0])), np.sqrt(np.sum(r * r, axis=1)).astype(np.float32)


def score_correction(q: np.ndarray, sketch: np.ndarray, rnorm: np.ndarray, S: np.ndarray, n: int) -> np.ndarray:
    """Estimates of q_h . r_t, [g][n]: sqrt(pi/2) / m ||r_t|| (S q_h) . z_t."""
    S = np.asarray(S, dtype=np.float32).astype(np.float64)
    m = S.shape[0]
    z = 2.0 * codec.unpack(sketch, sketch_bits_vector(m), n).astype(np.float64) - 1.0   # [n][m]
    sq = np.asarray(q, dtype=np.float64) @ S.T                                       # [g][m]
    rn = np.asarray(rnorm, dtype=np.float32).astype(np.float64)[:n]
    return math.sqrt(math.pi / 2.0) / m * (sq @ z.T) * rn[None, :]


def attend_compressed(k_state: Dict, v_state: Dict, k_packed: np.ndarray, k_norms: np.ndarray,
                      sketch: np.ndarray, rnorm: np.ndarray, S: np.ndarray, v_packed: np.ndarray,
                      v_norms: np.ndarray, n: int, q: np.ndarray, scale=None) -> np.ndarray:
    """Decode-step attention over a Walsh-Hadamard cache whose keys carry the
    residual sketch: scores q . K_hat_t plus the sketch estimate of q . r_t,
    then the shared softmax core over the exact reconstructions. fp32 [g][d]."""
    khat = rht.reconstruct_exact(k_state, k_packed, k_norms, n)
    vhat = rht.reconstruct_exact(v_state, v_packed, v_norms, n)
    extra = score_correction(q, sketch, rnorm, S, n)
    return codec.softmax_attention(q, khat, vhat, scale, extra)


# ------------------------------------------------------- eigen cache (selective)
def latent_residual(state: Dict, x: np.ndarray) -> np.ndarray:
    """r_j = c_j - c_hat_j on the kept channels with a positive step, 0
    elsewhere, [n][d] fp64 (c = x U, c_hat the dequantized codes)."""
    c = codec.project(state, x)
    chat = codec.dequantize(state, codec.quantize(state, c))
    keep = (np.asarray(state["bits"]) > 0) & (np.asarray(state["steps"]) > 0)
    return np.where(keep[None, :], c - chat, 0.0)


def sketch_encode_eigen(state: Dict, x: np.ndarray, S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Selective sketch of keys x [n][d] on the eigen cache: (packed sign bits
    of S r, ||r|| fp32 [n])."""
    r = latent_residual(state, x)
    S = np.asarray(S, dtype=np.float32).astype(np.float64)
    z = (r @ S.T >= 0.0).astype(np.int64)
    return codec.pack(z, sketch_bits_vector(S.shape[0])), np.sqrt(np.sum(r * r, axis=1)).astype(np.float32)


def attend_compressed_eigen(k_state: Dict, v_state: Dict, k_packed: np.ndarray, sketch: np.ndarray,
                            rnorm: np.ndarray, S: np.ndarray, v_packed: np.ndarray, n: int, q: np.ndarray,
                            scale=None) -> np.ndarray:
    """Decode-step attention over an eigen cache whose keys carry the selective
    sketch: q . K_hat_t plus sqrt(pi/2)/m ||r_t|| (S U^T q) . z_t. fp32 [g][d]."""
    khat = codec.reconstruct_exact(k_state, k_packed, n)
    vhat = codec.reconstruct_exact(v_state, v_packed, n)
    qt = np.asarray(q, dtype=np.float64) @ k_state["U"]          # U^T q, [g][d]
    extra = score_correction(qt, sketch, rnorm, S, n)
    return codec.softmax_attention(q, khat, vhat, scale, extra)

