"""Pins of the Walsh-Hadamard / Lloyd-Max oracle: textbook Hadamard matrix,
orthogonality, Lloyd fixed-point conditions, the exact sphere-coordinate
density and Max (1960)'s Gaussian 8-level table."""
import math

import numpy as np
import pytest
from scipy import integrate, linalg, stats

import synth
from oracle import codec, rht
from conftest import read_golden

D = 128


def check_fwht_is_sylvester_hadamard():
    v = np.random.default_rng(30).standard_normal((5, D))
    assert np.allclose(rht.fwht(v), v @ linalg.hadamard(D).T, rtol=0, atol=1e-12)
    h = rht.fwht(np.eye(D))
    assert np.array_equal(h, linalg.hadamard(D).astype(np.float64))
    assert np.array_equal(h @ h, D * np.eye(D))


def test_fwht_is_sylvester_hadamard():
    check_fwht_is_sylvester_hadamard()


def check_rotation_orthonormal_and_inverse():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((50, D))
    s = synth.random_signs(3, 0, 0, 0, 0)
    y = rht.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(rht.unrotate(y, s), x, rtol=0, atol=1e-12)
    # D first, then H: rotate(e_i) = s_i * (column i of H) / sqrt(d)
    e = np.zeros((1, D)); e[0, 5] = 1.0
    assert np.allclose(rht.rotate(e, s)[0], s[5] * linalg.hadamard(D)[:, 5] / math.sqrt(D))


def test_rotation_orthonormal_and_inverse():
    check_rotation_orthonormal_and_inverse()


@pytest.fixture(scope="module")
def lloyd():
    y = synth.sphere_coordinate_samples()
    c, it = rht.lloyd_max(y)
    return y, c, it


def check_lloyd_fixed_point(y, c):
    t = 0.5 * (c[:-1] + c[1:])
    cell = (y[:, None] >= t[None, :]).sum(axis=1)
    for k in range(c.shape[0]):
        assert abs(y[cell == k].mean() - c[k]) <= 1e-11


def test_lloyd_fixed_point(lloyd):
    y, c, it = lloyd
    assert it < 10000
    check_lloyd_fixed_point(y, c)
    assert np.all(np.diff(c) > 0)


def _exact_density_lloyd(levels=8):
    beta = stats.beta((D - 1) / 2, (D - 1) / 2)
    cdf = lambda t: beta.cdf((t + 1) / 2)
    mom = lambda lo, hi: integrate.quad(lambda t: t * beta.pdf((t + 1) / 2) / 2, lo, hi,
                                        epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    c = np.linspace(-0.2, 0.2, levels)
    for _ in range(3000):
        t = np.concatenate([[-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
        new = np.array([mom(t[k], t[k + 1]) / (cdf(t[k + 1]) - cdf(t[k])) for k in range(levels)])
        done = np.abs(new - c).max() < 1e-13
        c = new
        if done:
            break
    return c


def test_lloyd_matches_exact_density(lloyd):
    """Sample Lloyd vs Lloyd on the exact density (1 - y^2)^((d-3)/2).
    Tolerance 2e-3: the shift of the whole codebook is a nearly flat direction
    of the sample MSE, so sampling noise of 1e6 draws moves it by ~1e-3."""
    _, c, _ = lloyd
    ce = _exact_density_lloyd()
    assert np.abs(c - ce).max() <= 2e-3
    assert np.abs(ce + ce[::-1]).max() <= 1e-10          # exact density: symmetric
    assert np.abs(c + c[::-1]).max() <= 4e-3             # samples: symmetric within noise


def test_lloyd_approaches_gaussian_max1960(lloyd):
    """sqrt(d) * codebook -> 8-level Gaussian Lloyd-Max as d grows; at d=128
    the O(1/d) gap is below 0.03."""
    _, c, _ = lloyd
    ce = _exact_density_lloyd() * math.sqrt(D)
    rows = dict(read_golden("max1960_gaussian.txt"))
    g_out = np.array([float(v) for v in rows["lloyd8_outputs"]])
    assert np.abs(ce[4:] - g_out).max() <= 0.03
    assert np.abs(c[4:] * math.sqrt(D) - g_out).max() <= 0.05


def test_codebook_thresholds_fp32_midpoints():
    cb = np.array([-0.2, -0.1, -0.05, -0.01, 0.02, 0.06, 0.11, 0.19], np.float32)
    t = rht.codebook_thresholds(cb)
    assert t.dtype == np.float32
    for k in range(7):
        exact = (float(cb[k]) + float(cb[k + 1])) / 2
        assert abs(float(t[k]) - exact) <= abs(exact) * 2 ** -24


def test_rht_encode_decode(lloyd):
    _, c, _ = lloyd
    w = synth.WORKLOADS[3]
    x = synth.stream(w, 0, 0, 0, 0, n=2000)
    st = rht.make_state(synth.random_signs(3, 0, 0, 0, 0), rht.codebook_fp32(c))
    packed, norms = rht.encode_kv(st, x)
    assert packed.shape[0] == codec.packed_bytes(384, 2000)
    assert np.array_equal(norms, np.linalg.norm(x.astype(np.float64), axis=1).astype(np.float32))
    q = codec.unpack(packed, st["bits"], 2000)
    # codes are the codebook cells of the rotated, normalised token
    y = rht.rotate(x / np.linalg.norm(x, axis=1, keepdims=True), st["signs"])
    y32 = y.astype(np.float32)
    lo = np.concatenate([[-np.inf], st["thresholds"]]).astype(np.float64)
    hi = np.concatenate([st["thresholds"], [np.inf]]).astype(np.float64)
    assert np.all(lo[q] <= y32) and np.all(y32 < hi[q])
    xhat = rht.decode_kv(st, packed, norms, 2000, "bf16")
    r = codec.rel_mse(x, xhat)
    assert 0.02 < r < 0.05                        # ~ d * MSE of the 8-level codebook
    # zero token: norm 0, reconstruction 0
    z = np.zeros((3, D)); z[1] = x[0]
    p0, n0 = rht.encode_kv(st, z)
    assert n0[0] == 0 and np.all(rht.decode_kv(st, p0, n0, 3, "f32")[0] == 0)


def test_tq_beats_sq_on_heavy_tails(lloyd):
    """Soft reproduction of the Dutch summary ("Regime-specifieke prestaties"):
    on Student-t data the data-independent path wins at equal bits."""
    _, c, _ = lloyd
    w = synth.WORKLOADS[3]
    x = synth.stream(w, 0, 0, 1, 0, n=8192)
    st = rht.make_state(synth.random_signs(3, 0, 0, 1, 0), rht.codebook_fp32(c))
    p, nrm = rht.encode_kv(st, x)
    r_tq = codec.rel_mse(x, rht.decode_kv(st, p, nrm, 8192, "bf16"))
    sq = codec.calibrate_head(x, 2048, 3.0)
    r_sq = codec.rel_mse(x, codec.decode_kv(sq, codec.encode_kv(sq, x), 8192, "bf16"))
    assert r_tq < r_sq


# ------------------------------------------- attention over the Walsh-Hadamard cache
def _rht_pair(n=19, seed=33):
    rng = np.random.default_rng(seed)
    cb = rht.codebook_fp32(np.sort(rng.uniform(-0.25, 0.25, 8)))
    ks = rht.make_state(np.where(rng.random(D) < 0.5, -1, 1), cb)
    vs = rht.make_state(np.where(rng.random(D) < 0.5, -1, 1), cb)
    k = rng.standard_t(3, (n, D))
    v = rng.standard_t(3, (n, D))
    kp, kn = rht.encode_kv(ks, k)
    vp, vn = rht.encode_kv(vs, v)
    return ks, vs, kp, kn, vp, vn, k, v


def test_rht_attention_matches_plain_loops():
    """Against a plain-loop softmax attention of the exact reconstructions,
    written out independently of the oracle's vectorised core."""
    ks, vs, kp, kn, vp, vn, k, _ = _rht_pair()
    n = k.shape[0]
    q = np.random.default_rng(34).standard_normal((3, D))
    got = rht.attend_compressed(ks, vs, kp, kn, vp, vn, n, q)
    khat = rht.reconstruct_exact(ks, kp, kn, n)
    vhat = rht.reconstruct_exact(vs, vp, vn, n)
    for h in range(3):
        s = [sum(q[h, i] * khat[t, i] for i in range(D)) / math.sqrt(D) for t in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        want = [sum(e[t] * vhat[t, i] for t in range(n)) / z for i in range(D)]
        assert np.allclose(got[h], want, rtol=1e-6, atol=1e-6)


def test_rht_attention_special_cases():
    ks, vs, kp, kn, vp, vn, k, v = _rht_pair()
    q = np.random.default_rng(35).standard_normal((2, D))
    one = rht.attend_compressed(ks, vs, kp, kn, vp, vn, 1, q)
    v1 = rht.reconstruct_exact(vs, vp, vn, 1)[0]
    assert np.allclose(one, np.tile(v1, (2, 1)), rtol=1e-6, atol=1e-7)
    # identical keys: uniform weights -> mean of V_hat
    kp2, kn2 = rht.encode_kv(ks, np.tile(k[:1], (k.shape[0], 1)))
    o = rht.attend_compressed(ks, vs, kp2, kn2, vp, vn, k.shape[0], q)
    assert np.allclose(o, rht.reconstruct_exact(vs, vp, vn, k.shape[0]).mean(axis=0)[None, :], rtol=1e-6,
                       atol=1e-6)


def test_rht_latent_identity():
    """q . K_hat_t = nu_t / sqrt(d) * (y_hat_t . H D q): scores can be taken in
    the rotated basis (the form the GPU uses), with H from scipy."""
    ks, vs, kp, kn, vp, vn, k, _ = _rht_pair()
    n = k.shape[0]
    q = np.random.default_rng(36).standard_normal(D)
    khat = rht.reconstruct_exact(ks, kp, kn, n)
    yhat = ks["codebook"].astype(np.float64)[codec.unpack(kp, ks["bits"], n)]
    qt = linalg.hadamard(D) @ (ks["signs"] * q)
    lhs = khat @ q
    rhs = kn.astype(np.float64) / math.sqrt(D) * (yhat @ qt)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
