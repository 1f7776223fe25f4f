"""Oracle for the data-adaptive (eigenbasis) path: calibrate, encode, decode,
decode-step attention. fp64 throughout unless stated. Test infrastructure only.

Every function below is pinned by tests/test_oracle_codec.py; none is
"parity unpinned". Readings of the pages are marked READING.
"""
from __future__ import annotations

import functools
import math
from typing import Dict, List, Optional

import numpy as np
from scipy import optimize, special

MAX_BITS = 8
XFORM_EIGEN, XFORM_IDENTITY, XFORM_RHT = 0, 1, 2


# ---------------------------------------------------------------- calibration
def second_moment(x: np.ndarray, n_calib: int) -> np.ndarray:
    """Uncentred second moment of the first `n_calib` tokens, (1/n) X^T X.

    SPECTRA summary, "Metodologia" observations 1 and 3: the basis comes from
    the Gram matrix of the activations, G = E[h^T h] (no mean removed). The
    Dutch summary ("Experimentele Opstelling", SpectralQuant) calibrates it per
    head on representative tokens. READING: the representative tokens are the
    first n_calib tokens of the stream; K and V are calibrated separately.
    """
    x = np.asarray(x, dtype=np.float64)
    if not (0 < n_calib <= x.shape[0]):
        raise ValueError("n_calib must be in [1, n]")
    xc = x[:n_calib]
    return (xc.T @ xc) / float(n_calib)


def sign_fix(u: np.ndarray) -> np.ndarray:
    """Make each column's largest-magnitude entry positive (lowest row index on
    a magnitude tie). The pages fix no sign; READING: this rule, so that two
    implementations produce the same basis and hence the same codes."""
    u = np.array(u, dtype=np.float64, copy=True)
    for j in range(u.shape[1]):
        k = int(np.argmax(np.abs(u[:, j])))
        if u[k, j] < 0:
            u[:, j] = -u[:, j]
    return u


def eigenbasis(sigma: np.ndarray):
    """Energy-ordered orthonormal basis of the second moment: sigma = U diag(lam) U^T,
    lam descending (ties keep LAPACK's order), columns sign-fixed.

    SPECTRA summary, "Metodologia" observation 1 (rotated channels become
    uncorrelated and the energy concentrates) and "La Pipeline" step 1
    (orthogonal coordinates ordered by variance). The G-weighted SVD of W_K/W_V
    in step 1 gives the same basis when K = h W (checked in the tests)."""
    w, v = np.linalg.eigh(np.asarray(sigma, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    return sign_fix(v[:, order]), np.array(w[order], dtype=np.float64)


def identity_basis(sigma: np.ndarray):
    """Plain-KV (Dutch summary, "Systematische Ablatie": scalar quantization
    without rotation): U = I and lam = diag(sigma) in raw channel order.
    READING: channels are not re-sorted."""
    sigma = np.asarray(sigma, dtype=np.float64)
    return np.eye(sigma.shape[0]), np.array(np.diag(sigma), dtype=np.float64)


def total_bits_for(avg_bits: float, d: int) -> int:
    """Bits per token record for an average budget: floor(avg * d + 0.5)."""
    return int(math.floor(avg_bits * d + 0.5))


def water_fill(lam: np.ndarray, total_bits: int, max_bits: int = MAX_BITS) -> np.ndarray:
    """Integer reverse water-filling.

    SPECTRA summary, "La Pipeline" step 2: bits follow the marginal variances of
    the latent coordinates; high-variance channels get more, low-variance ones
    fewer, down to zero. READING: the Gaussian rate-distortion model
    D_j(b) = lam_j 4^-b, integerised greedily: each of the `total_bits` bits
    goes to the channel with the largest lam_j * 2^(-2 b_j) among channels
    below `max_bits` (lowest index on ties; lam <= 0 counts as 0).
    """
    lam = np.asarray(lam, dtype=np.float64)
    d = lam.shape[0]
    if total_bits < 0 or total_bits > max_bits * d:
        raise ValueError("budget out of range")
    lam_pos = np.where(lam > 0.0, lam, 0.0)
    b = np.zeros(d, dtype=np.int64)
    for _ in range(total_bits):
        gain = np.where(b < max_bits, lam_pos * np.ldexp(1.0, -2 * b), -1.0)
        j = int(np.argmax(gain))
        b[j] += 1
    return b.astype(np.uint8)


# ------------------------------------------------------------ scalar quantizer
def _phi(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.exp(-0.5 * np.where(np.isfinite(x), x, 0.0) ** 2) / math.sqrt(2.0 * math.pi)
    return np.where(np.isfinite(x), out, 0.0)


def _xphi(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.isfinite(x), x, 0.0) * _phi(x)


def _upper_cells(delta: float, levels: int):
    """Cells of the non-negative half of an even-level midrise quantizer:
    [i*delta, (i+1)*delta) with level (i + 1/2) delta; the last one is open."""
    half = levels // 2
    i = np.arange(half, dtype=np.float64)
    a = i * delta
    b = np.where(i < half - 1, (i + 1.0) * delta, np.inf)
    y = (i + 0.5) * delta
    p = special.ndtr(-a) - special.ndtr(-b)       # P(a <= X < b), upper-tail form
    return a, b, y, p, i + 0.5


def uniform_gaussian_mse(delta: float, levels: int) -> float:
    """MSE of the midrise uniform quantizer with `levels` levels and step
    `delta` on N(0, 1), from the exact Gaussian integrals (both halves)."""
    a, b, y, p, _ = _upper_cells(delta, levels)
    # int_a^b (x - y)^2 phi = P - [x phi]_a^b - 2y [phi]_a^b ... written out:
    mse_half = p - (_xphi(b) - _xphi(a)) + 2.0 * y * (_phi(b) - _phi(a)) + y * y * p
    return float(2.0 * np.sum(mse_half))


def _uniform_mse_slope(delta: float, levels: int) -> float:
    # d/d(delta) of the MSE; the moving cell edges contribute nothing because
    # each edge is the midpoint of its two levels.
    a, b, y, p, m = _upper_cells(delta, levels)
    first = _phi(a) - _phi(b)            # int_a^b x phi
    return float(-4.0 * np.sum(m * (first - m * delta * p)))


@functools.lru_cache(maxsize=None)
def delta_star(bits: int) -> float:
    """MSE-optimal step of the 2^bits-level midrise uniform quantizer for a
    unit Gaussian (root of the MSE slope, found by Brent's method).

    READING: "scalar-quantized" with bits from water-filling; each kept channel
    is quantized independently per token (SPECTRA summary, "La Pipeline" step
    3), with no per-token scale, by the uniform quantizer that is optimal for a
    Gaussian of the channel's variance."""
    if not (1 <= bits <= MAX_BITS):
        raise ValueError("bits must be in 1..8")
    levels = 1 << bits
    return float(optimize.brentq(_uniform_mse_slope, 1e-6, 4.0, args=(levels,),
                                 xtol=1e-300, rtol=8.9e-16, maxiter=500))


@functools.lru_cache(maxsize=None)
def quantizer_mse(bits: int) -> float:
    """eps(b): distortion of a unit-variance Gaussian channel at b bits, the
    MSE of the 2^b-level quantizer with step delta*(b); eps(0) = 1 (the channel
    is dropped and its whole variance is lost)."""
    if bits == 0:
        return 1.0
    return uniform_gaussian_mse(delta_star(bits), 1 << bits)


ALLOC_VARIANTS = ("greedy", "operational", "grouped", "floor", "gap")


def allocate_bits(lam: np.ndarray, total_bits: int, variant: str = "greedy", param: float = 0.0,
                  max_bits: int = MAX_BITS) -> np.ndarray:
    """Bit allocation variants, all calibrate-time choices that feed the same
    quantizer and format.

    greedy      the default reverse water-filling (`water_fill`).
    operational greedy on the quantizer's actual distortion: each bit goes
                to argmax lam_j (eps(b_j) - eps(b_j + 1)) (SPECTRA summary,
                "La Pipeline" step 2: bits follow the marginal variances;
                READING: the rate-distortion model replaced by the uniform
                quantizer's own MSE curve).
    grouped     adjacent channels share one width (SPECTRA summary, "La
                Pipeline" step 2, "Raggruppamento"): READING: groups of
                G = param channels [kG, (k+1)G); greedy over groups on the
                group variance sum Lam_k 4^-b_k, G bits per step, while at
                least G bits remain (sum of bits = G floor(B / G)).
    floor       a fixed floor of f = param bits on every channel (the
                ablation summary's "tail floor", "Opslag vs. Kwaliteit"),
                the rest of the budget by the default greedy.
    gap         spectral-gap pruning of the effective dimension (ablation
                summary, "Regime-Specifieke Prestaties en
                Kalibratiesensitiviteit", d_eff): READING: d_eff = 1 + the
                first j with lam_j >= r lam_{j+1} (r = param; d if none, and
                a positive lam_j followed by lam_{j+1} <= 0 counts as a gap);
                channels from d_eff on get 0 bits, the first d_eff channels
                share the budget by the default greedy (at most max_bits
                each, so the sum is min(B, max_bits d_eff)).
    Ties go to the lowest index; lam <= 0 counts as 0."""
    lam = np.asarray(lam, dtype=np.float64)
    d = lam.shape[0]
    if total_bits < 0 or total_bits > max_bits * d:
        raise ValueError("budget out of range")
    lam_pos = np.where(lam > 0.0, lam, 0.0)
    if variant == "greedy":
        return water_fill(lam, total_bits, max_bits)
    if variant == "operational":
        b = np.zeros(d, dtype=np.int64)
        for _ in range(total_bits):
            gain = np.array([lam_pos[j] * (quantizer_mse(int(b[j])) - quantizer_mse(int(b[j]) + 1))
                             if b[j] < max_bits else -1.0 for j in range(d)])
            b[int(np.argmax(gain))] += 1
        return b.astype(np.uint8)
    if variant == "grouped":
        G = int(param)
        if G < 1 or d % G:
            raise ValueError("group size must divide d")
        lam_g = lam_pos.reshape(d // G, G).sum(axis=1)
        bg = np.zeros(d // G, dtype=np.int64)
        left = total_bits
        while left >= G:
            gain = np.where(bg < max_bits, lam_g * np.ldexp(1.0, -2 * bg), -1.0)
            if gain.max() < 0:
                break
            bg[int(np.argmax(gain))] += 1
            left -= G
        return np.repeat(bg, G).astype(np.uint8)
    if variant == "floor":
        f = int(param)
        if f < 0 or f > max_bits or f * d > total_bits:
            raise ValueError("floor out of range")
        b = np.full(d, f, dtype=np.int64)
        for _ in range(total_bits - f * d):
            gain = np.where(b < max_bits, lam_pos * np.ldexp(1.0, -2 * b), -1.0)
            b[int(np.argmax(gain))] += 1
        return b.astype(np.uint8)
    if variant == "gap":
        r = float(param)
        if not r > 1.0:
            raise ValueError("gap ratio must exceed 1")
        d_eff = d
        for j in range(d - 1):
            if lam_pos[j] > 0 and (lam_pos[j + 1] <= 0 or lam_pos[j] >= r * lam_pos[j + 1]):
                d_eff = j + 1
                break
        b = np.zeros(d, dtype=np.int64)
        b[:d_eff] = water_fill(lam[:d_eff], min(total_bits, max_bits * d_eff), max_bits)
        return b.astype(np.uint8)
    raise ValueError(f"unknown variant {variant}")


def channel_offsets(bits: np.ndarray) -> np.ndarray:
    """Bit offset of each channel inside a token record (prefix sum)."""
    bits = np.asarray(bits, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(bits)[:-1]]).astype(np.int64)


def quantizer_steps(lam: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Step per channel: sqrt(lam_j) * delta_star(b_j); 0 for dropped channels."""
    lam = np.asarray(lam, dtype=np.float64)
    steps = np.zeros(lam.shape[0], dtype=np.float64)
    for j, b in enumerate(np.asarray(bits)):
        if b > 0:
            steps[j] = math.sqrt(max(float(lam[j]), 0.0)) * delta_star(int(b))
    return steps


def thresholds(step: float, bits: int) -> np.ndarray:
    """Decision thresholds t_k = fl32((k - L/2) * step), k = 1..L-1, L = 2^bits
    (product in fp64, then rounded to fp32)."""
    levels = 1 << int(bits)
    k = np.arange(1, levels, dtype=np.float64)
    return ((k - levels / 2.0) * float(step)).astype(np.float32)


def quantize_channel(c: np.ndarray, thr: np.ndarray) -> np.ndarray:
    """Code = number of thresholds t with t <= fl32(c) (IEEE comparisons).

    READING: the quantizer sees the coefficient rounded to fp32; a value equal
    to a threshold goes to the upper cell; NaN gives code 0 and +-Inf the
    outer codes; values beyond the outer levels clamp to them."""
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    thr = np.asarray(thr, dtype=np.float32)
    return (c32[:, None] >= thr[None, :]).sum(axis=1).astype(np.int64)


def dequantize_channel(q: np.ndarray, step: float, bits: int) -> np.ndarray:
    """Reconstruction level (q - (L-1)/2) * step of a midrise code."""
    levels = 1 << int(bits)
    return (np.asarray(q, dtype=np.float64) - (levels - 1) / 2.0) * float(step)


# ------------------------------------------------------------------- format F1
def packed_bytes(total_bits: int, n: int) -> int:
    """Stream length: ceil(n * B / 8) bytes rounded up to a multiple of 16."""
    nbytes = (n * total_bits + 7) // 8
    return (nbytes + 15) // 16 * 16


def pack(codes: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Format F1. READING (the pages only say the cache is append-only with
    tokens quantized one at a time, SPECTRA summary "La Pipeline" steps 2-3):
    token t's record holds stream bits [t*B, (t+1)*B); inside it, kept channels
    in ascending index j take bits [o_j, o_j + b_j), least significant code bit
    first; stream bit i is bit (i & 7) of byte (i >> 3). Padding bits are 0."""
    codes = np.asarray(codes, dtype=np.int64)
    bits = np.asarray(bits, dtype=np.int64)
    n = codes.shape[0]
    total = int(bits.sum())
    offs = channel_offsets(bits)
    bitmat = np.zeros((n, max(total, 1)), dtype=np.uint8)
    for j in range(bits.shape[0]):
        for k in range(int(bits[j])):
            bitmat[:, offs[j] + k] = (codes[:, j] >> k) & 1
    flat = bitmat[:, :total].reshape(-1)
    nbytes = packed_bytes(total, n)
    padded = np.zeros(nbytes * 8, dtype=np.uint8)
    padded[: flat.shape[0]] = flat
    groups = padded.reshape(-1, 8).astype(np.uint16)
    weights = (1 << np.arange(8, dtype=np.uint16))
    return (groups * weights[None, :]).sum(axis=1).astype(np.uint8)


def append_pack(packed_old: np.ndarray, n_old: int, codes_new: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Append-only cache (SPECTRA summary, "La Pipeline" steps 2-3: each new
    token is quantized on arrival and its record appended): the stream of
    n_old tokens followed by the records of codes_new [m][d], as F1 bytes of
    n_old + m tokens. Written bit by bit from the F1 layout (record r of the
    new tokens starts at stream bit (n_old + r) * B), independently of `pack`:
    the old stream's first n_old * B bits are kept, every later bit is the
    new records' or 0."""
    codes_new = np.asarray(codes_new, dtype=np.int64)
    bits = [int(b) for b in np.asarray(bits)]
    total = sum(bits)
    m = codes_new.shape[0]
    out = np.zeros(packed_bytes(total, n_old + m), dtype=np.uint8)
    old = np.asarray(packed_old, dtype=np.uint8)
    for i in range(n_old * total):
        if (int(old[i >> 3]) >> (i & 7)) & 1:
            out[i >> 3] |= np.uint8(1 << (i & 7))
    for r in range(m):
        pos = (n_old + r) * total
        for j, b in enumerate(bits):
            for k in range(b):
                if (int(codes_new[r, j]) >> k) & 1:
                    out[pos >> 3] |= np.uint8(1 << (pos & 7))
                pos += 1
    return out


def unpack(packed: np.ndarray, bits: np.ndarray, n: int) -> np.ndarray:
    """Inverse of `pack`: codes [n][d] (0 in dropped channels)."""
    packed = np.asarray(packed, dtype=np.uint8)
    bits = np.asarray(bits, dtype=np.int64)
    total = int(bits.sum())
    offs = channel_offsets(bits)
    allbits = ((packed[:, None] >> np.arange(8, dtype=np.uint8)[None, :]) & 1).reshape(-1)
    bitmat = allbits[: n * total].reshape(n, total) if total > 0 else np.zeros((n, 0), np.uint8)
    codes = np.zeros((n, bits.shape[0]), dtype=np.int64)
    for j in range(bits.shape[0]):
        for k in range(int(bits[j])):
            codes[:, j] |= bitmat[:, offs[j] + k].astype(np.int64) << k
    return codes


# ------------------------------------------------------------------- rounding
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (8 significant bits, ties to even, fp32
    exponent range), returned as fp64. One rounding step."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.round(x / quantum) * quantum


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------- the codec
def make_state(u: np.ndarray, lam: np.ndarray, bits: np.ndarray,
               xform: int = XFORM_EIGEN, steps: Optional[np.ndarray] = None) -> Dict:
    """Per-stream codec state: basis, variances, widths, steps, thresholds."""
    bits = np.asarray(bits, dtype=np.uint8)
    if bits.max(initial=0) > MAX_BITS:
        raise ValueError("bit width above 8")
    steps = quantizer_steps(lam, bits) if steps is None else np.asarray(steps, np.float64)
    thr: List[np.ndarray] = [thresholds(steps[j], int(bits[j])) if bits[j] > 0
                             else np.zeros(0, np.float32) for j in range(bits.shape[0])]
    return {"xform": xform, "U": np.asarray(u, np.float64), "lam": np.asarray(lam, np.float64),
            "bits": bits, "total_bits": int(bits.astype(np.int64).sum()),
            "offsets": channel_offsets(bits), "steps": steps, "thresholds": thr}


def calibrate_head(x: np.ndarray, n_calib: int, avg_bits: float,
                   bits: Optional[np.ndarray] = None, xform: int = XFORM_EIGEN) -> Dict:
    """Second moment -> basis -> bit allocation -> quantizer (one stream).
    `bits` given: an explicit allocation (e.g. uniform, SQU-KV) that must sum
    to floor(avg_bits * d + 0.5)."""
    sigma = second_moment(x, n_calib)
    if xform == XFORM_EIGEN:
        u, lam = eigenbasis(sigma)
    elif xform == XFORM_IDENTITY:
        u, lam = identity_basis(sigma)
    else:
        raise ValueError("use oracle.rht for the Walsh-Hadamard path")
    d = sigma.shape[0]
    budget = total_bits_for(avg_bits, d)
    if bits is None:
        bits = water_fill(lam, budget)
    elif int(np.sum(bits)) != budget:
        raise ValueError("bit vector does not match the budget")
    st = make_state(u, lam, bits, xform)
    st["sigma"] = sigma
    return st


def project(state: Dict, x: np.ndarray) -> np.ndarray:
    """Latent coefficients c = x U (SPECTRA summary, "La Pipeline" step 3:
    tokens are projected down into the latent basis). fp64."""
    return np.asarray(x, dtype=np.float64) @ state["U"]


def quantize(state: Dict, c: np.ndarray) -> np.ndarray:
    """Codes of all kept channels, [n][d] (0 in dropped channels)."""
    c = np.asarray(c, dtype=np.float64)
    q = np.zeros(c.shape, dtype=np.int64)
    for j, b in enumerate(state["bits"]):
        if b > 0:
            q[:, j] = quantize_channel(c[:, j], state["thresholds"][j])
    return q


def quantize_pack(state: Dict, c: np.ndarray) -> np.ndarray:
    return pack(quantize(state, c), state["bits"])


def encode_kv(state: Dict, x: np.ndarray) -> np.ndarray:
    """Project, quantize and pack a stream of tokens; returns F1 bytes."""
    return quantize_pack(state, project(state, x))


def dequantize(state: Dict, q: np.ndarray) -> np.ndarray:
    """Latent reconstruction; dropped channels are 0 (SPECTRA summary,
    "Metodologia" observation 2: a 0-bit channel is discarded)."""
    q = np.asarray(q)
    chat = np.zeros(q.shape, dtype=np.float64)
    for j, b in enumerate(state["bits"]):
        if b > 0:
            chat[:, j] = dequantize_channel(q[:, j], state["steps"][j], int(b))
    return chat


def reconstruct_exact(state: Dict, packed: np.ndarray, n: int) -> np.ndarray:
    """x_hat = c_hat U^T in fp64 (SPECTRA summary, "La Pipeline" step 3: full
    keys and values are rebuilt on the fly)."""
    return dequantize(state, unpack(packed, state["bits"], n)) @ state["U"].T


def decode_kv(state: Dict, packed: np.ndarray, n: int, dtype: str) -> np.ndarray:
    """Unpack, dequantize, inverse-rotate, round to the stream dtype."""
    return round_to(reconstruct_exact(state, packed, n), dtype)


def rel_mse(x: np.ndarray, xhat: np.ndarray) -> float:
    """relMSE = sum |x - x_hat|^2 / sum |x|^2 (Dutch summary, "Experimentele
    Opstelling", metrics)."""
    x = np.asarray(x, dtype=np.float64)
    e = x - np.asarray(xhat, dtype=np.float64)
    return float(np.sum(e * e) / np.sum(x * x))


def attend_compressed(k_state: Dict, v_state: Dict, k_packed: np.ndarray,
                      v_packed: np.ndarray, n: int, q: np.ndarray,
                      scale: Optional[float] = None) -> np.ndarray:
    """One decode step of softmax attention over the compressed cache.

    Keys and values are the exact (fp64) reconstructions of the packed streams
    (SPECTRA summary, "La Pipeline" step 3: K/V rebuilt for standard
    attention). s = q K^T * scale, softmax over all n tokens, o = p V.
    READING: scale 1/sqrt(d), no mask, no positional rotation. Returns fp32
    [g][d] for the g query heads of this KV head."""
    khat = reconstruct_exact(k_state, k_packed, n)
    vhat = reconstruct_exact(v_state, v_packed, n)
    return softmax_attention(q, khat, vhat, scale)


def softmax_attention(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray,
                      scale: Optional[float] = None, extra: Optional[np.ndarray] = None) -> np.ndarray:
    """Standard attention of g query heads over n reconstructed keys and
    values, fp64: s = (q K^T + extra) * scale, softmax over the n tokens,
    o = p V; `extra` [g][n] is an optional additive estimate of the part of
    q . k the reconstruction misses. READING: scale 1/sqrt(d), no mask, no
    positional rotation. fp32 [g][d]."""
    q = np.asarray(q, dtype=np.float64)
    d = khat.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    s = q @ khat.T
    if extra is not None:
        s = s + extra
    s = s * scale                                  # [g][n]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return (p @ vhat).astype(np.float32)
