"""Pins of the eigenbasis-path oracle against things other than itself:
closed forms, brute force on tiny inputs, textbook identities, published
tables and hand-computed format vectors. The check_* helpers are reused by
test_oracle_mutations.py, which plants mistakes in the oracle and expects
these checks to fail."""
import itertools
import math

import numpy as np
import pytest
from scipy import integrate, linalg, special

import synth
from oracle import codec
from conftest import read_golden


# ------------------------------------------------------------------ helpers
def spd_from_spectrum(lam, seed):
    q = synth.haar_orthogonal(np.random.default_rng(seed), len(lam))
    return (q * np.asarray(lam)[None, :]) @ q.T


def gaussian_stream(n, lam, seed):
    rng = np.random.default_rng(seed)
    q = synth.haar_orthogonal(rng, len(lam))
    return (rng.standard_normal((n, len(lam))) * np.sqrt(lam)[None, :]) @ q.T


# --------------------------------------------------------------- O1 moment
def check_second_moment_bruteforce():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3))
    n_c = 5
    s = codec.second_moment(x, n_c)
    for a in range(3):
        for b in range(3):
            acc = 0.0
            for t in range(n_c):
                acc += float(x[t, a]) * float(x[t, b])
            assert abs(s[a, b] - acc / n_c) <= 1e-14 * max(1.0, abs(acc))


def test_second_moment_bruteforce():
    check_second_moment_bruteforce()


def test_second_moment_uncentred_and_psd():
    x = np.ones((4, 2)) * np.array([[3.0, -1.0]])       # constant tokens: mean != 0
    s = codec.second_moment(x, 4)
    assert np.allclose(s, [[9.0, -3.0], [-3.0, 1.0]], atol=0, rtol=1e-15)
    s2 = codec.second_moment(np.random.default_rng(2).standard_normal((50, 6)), 40)
    assert np.allclose(s2, s2.T, atol=0, rtol=0)
    assert np.linalg.eigvalsh(s2).min() > -1e-12


# ----------------------------------------------------------------- O2 basis
def check_eigenbasis_tridiagonal_closed_form():
    m = 12
    t = 2 * np.eye(m) - np.eye(m, k=1) - np.eye(m, k=-1)
    u, lam = codec.eigenbasis(t)
    k = np.arange(1, m + 1)
    lam_exact = np.sort(2 - 2 * np.cos(k * np.pi / (m + 1)))[::-1]
    assert np.allclose(lam, lam_exact, atol=1e-13, rtol=0)
    for col in range(m):
        # eigenvalue lam_exact[col] = 2 - 2 cos(kk pi/(m+1))
        kk = m - col
        v = np.sin(np.arange(1, m + 1) * kk * np.pi / (m + 1))
        v /= np.linalg.norm(v)
        assert min(np.abs(u[:, col] - v).max(), np.abs(u[:, col] + v).max()) < 1e-12


def test_eigenbasis_tridiagonal_closed_form():
    check_eigenbasis_tridiagonal_closed_form()


def check_eigenbasis_invariants(sigma):
    u, lam = codec.eigenbasis(sigma)
    d = sigma.shape[0]
    assert np.abs(u.T @ u - np.eye(d)).max() <= 1e-12
    rot = u.T @ sigma @ u
    off = rot - np.diag(np.diag(rot))
    assert np.abs(off).max() <= 1e-12 * lam[0]
    assert np.allclose(np.diag(rot), lam, rtol=1e-12, atol=1e-14 * lam[0])
    assert np.all(np.diff(lam) <= 0)
    for j in range(d):
        k = int(np.argmax(np.abs(u[:, j])))
        assert u[k, j] > 0


def test_eigenbasis_invariants_cfg1_stream():
    w = synth.WORKLOADS[1]
    x = synth.stream(w, 0, 0, 0, 0)
    check_eigenbasis_invariants(codec.second_moment(x, w.n_calib))


def test_eigenbasis_diagonal_is_permutation():
    vals = np.array([0.3, 5.0, 1.0, 2.5, 0.01])
    u, lam = codec.eigenbasis(np.diag(vals))
    assert np.array_equal(lam, np.sort(vals)[::-1])
    perm = np.argsort(-vals)
    assert np.array_equal(u, np.eye(5)[:, perm])


def check_gsvd_identity():
    """SPECTRA summary, "La Pipeline" step 1: whitening W by G^(1/2) gives the
    same basis. K = h W, G = h^T h / n: eig(K^T K / n) = right singular vectors
    of L_G^T W (G = L_G L_G^T), with lam = sigma^2."""
    rng = np.random.default_rng(3)
    n, big_d, d = 400, 24, 8
    h = rng.standard_normal((n, big_d)) @ rng.standard_normal((big_d, big_d))
    w = rng.standard_normal((big_d, d))
    g = h.T @ h / n
    lg = np.linalg.cholesky(g)
    _, sv, vt = np.linalg.svd(lg.T @ w, full_matrices=False)
    u, lam = codec.eigenbasis(codec.second_moment(h @ w, n))
    assert np.allclose(lam, sv ** 2, rtol=1e-10, atol=0)
    for j in range(d):
        v = vt[j]
        assert min(np.abs(u[:, j] - v).max(), np.abs(u[:, j] + v).max()) < 1e-9


def test_gsvd_identity():
    check_gsvd_identity()


def check_sign_rule_hand():
    u = codec.sign_fix(np.array([[0.6, -0.8], [-0.8, -0.6]]))
    assert np.array_equal(u, np.array([[-0.6, 0.8], [0.8, 0.6]]))
    assert np.array_equal(codec.sign_fix(u), u)
    tie = codec.sign_fix(np.array([[-0.5], [0.5], [0.1]]))   # tie -> lowest row wins
    assert tie[0, 0] == 0.5 and tie[1, 0] == -0.5
    # sign flips do not change U diag(lam) U^T
    s = spd_from_spectrum([3.0, 2.0, 1.0, 0.5], 22)
    uu, lam = codec.eigenbasis(s)
    assert np.allclose((uu * lam[None, :]) @ uu.T, s, rtol=0, atol=1e-13)


def test_sign_rule_idempotent_and_tie():
    check_sign_rule_hand()


def test_identity_basis():
    s = spd_from_spectrum([4.0, 1.0, 0.5], 9)
    u, lam = codec.identity_basis(s)
    assert np.array_equal(u, np.eye(3)) and np.array_equal(lam, np.diag(s))


# ------------------------------------------------------------- O5 allocation
def compositions(total, parts, cap):
    if parts == 1:
        if total <= cap:
            yield (total,)
        return
    for first in range(min(total, cap) + 1):
        for rest in compositions(total - first, parts - 1, cap):
            yield (first,) + rest


def check_water_fill_bruteforce(budgets=(4, 8, 12, 16)):
    rng = np.random.default_rng(4)
    lam = np.sort(rng.lognormal(0.0, 2.0, size=8))[::-1]
    for b_tot in budgets:
        allc = np.array(list(compositions(b_tot, 8, 8)), dtype=np.int64)
        obj = (lam[None, :] * np.ldexp(1.0, -2 * allc)).sum(axis=1)
        best = obj.min()
        b = codec.water_fill(lam, b_tot).astype(np.int64)
        assert b.sum() == b_tot
        got = float((lam * np.ldexp(1.0, -2 * b)).sum())
        assert got <= best * (1 + 1e-14)
        winners = allc[np.abs(obj - best) <= 1e-14 * best]
        assert any(np.array_equal(b, wv) for wv in winners)


def test_water_fill_bruteforce_d8():
    check_water_fill_bruteforce((4, 8, 12, 16, 24))


def test_water_fill_properties():
    rng = np.random.default_rng(5)
    lam = np.sort(rng.lognormal(0, 3, 128))[::-1]
    for b_tot in (0, 1, 170, 256, 512, 1024):
        b = codec.water_fill(lam, b_tot).astype(np.int64)
        assert b.sum() == b_tot and b.min() >= 0 and b.max() <= 8
        assert np.all(np.diff(b) <= 0)          # adjacent equal-width runs
    assert np.all(codec.water_fill(lam, 1024) == 8)
    with pytest.raises(ValueError):
        codec.water_fill(lam, 1025)
    # ties -> lowest index
    assert list(codec.water_fill(np.ones(4), 3)) == [1, 1, 1, 0]


def test_water_fill_above_continuous_bound():
    """Continuous reverse water-filling sum_j min(theta, lam_j) at the same
    rate is a lower bound of the integer greedy's distortion."""
    rng = np.random.default_rng(6)
    lam = np.sort(rng.lognormal(0, 2, 64))[::-1]
    for b_tot in (16, 64, 128, 200):
        def rate(theta):
            return np.sum(np.maximum(0.0, 0.5 * np.log2(lam / theta)))
        lo, hi = 1e-30, lam[0]
        for _ in range(300):
            mid = math.sqrt(lo * hi)
            lo, hi = (mid, hi) if rate(mid) > b_tot else (lo, mid)
        d_cont = np.sum(np.minimum(hi, lam))
        b = codec.water_fill(lam, b_tot).astype(np.int64)
        d_greedy = np.sum(lam * np.ldexp(1.0, -2 * b))
        assert d_greedy >= d_cont * (1 - 1e-9)


def test_total_bits_rounding():
    assert codec.total_bits_for(1.33, 128) == 170
    assert codec.total_bits_for(2.0, 128) == 256
    assert codec.total_bits_for(4.0, 128) == 512


# ------------------------------------------------------------ O6 quantizer
def check_delta_star_closed_form():
    assert abs(codec.delta_star(1) - 2 * math.sqrt(2 / math.pi)) <= 1e-14
    assert abs(codec.uniform_gaussian_mse(codec.delta_star(1), 2) - (1 - 2 / math.pi)) <= 1e-14


def test_delta_star_closed_form():
    check_delta_star_closed_form()


def check_delta_star_max1960():
    for key, vals in read_golden("max1960_gaussian.txt"):
        if key != "uniform":
            continue
        levels, step, mse = int(vals[0]), float(vals[1]), float(vals[2])
        b = levels.bit_length() - 1
        assert abs(codec.delta_star(b) - step) <= 0.6e-4 * max(1.0, step) + 0.5e-3 * step
        assert abs(codec.uniform_gaussian_mse(codec.delta_star(b), levels) - mse) <= 0.6e-3 * mse


def test_delta_star_max1960():
    check_delta_star_max1960()


def _mse_quadrature(delta, levels):
    """Independent route: adaptive quadrature of (x - Q(x))^2 phi(x)."""
    tot = 0.0
    edges = [-np.inf] + [(k - levels / 2) * delta for k in range(1, levels)] + [np.inf]
    for k in range(levels):
        y = (k - (levels - 1) / 2) * delta
        f = lambda x, y=y: (x - y) ** 2 * math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
        tot += integrate.quad(f, edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-12, limit=200)[0]
    return tot


def check_delta_star_stationary():
    for b in (2, 3, 5, 8):
        levels = 1 << b
        ds = codec.delta_star(b)
        for delta in (0.7 * ds, ds, 1.3 * ds):
            assert abs(codec.uniform_gaussian_mse(delta, levels) - _mse_quadrature(delta, levels)) \
                <= 1e-10 * _mse_quadrature(delta, levels)
        m0 = _mse_quadrature(ds, levels)
        for h in (1e-3, -1e-3):
            assert _mse_quadrature(ds * (1 + h), levels) > m0


def test_delta_star_stationary():
    check_delta_star_stationary()


def test_delta_star_mse_convex_decreasing():
    eps = [codec.uniform_gaussian_mse(codec.delta_star(b), 1 << b) for b in range(1, 9)]
    assert all(eps[i + 1] < eps[i] for i in range(7))
    assert all(eps[i] - eps[i + 1] > eps[i + 1] - eps[i + 2] for i in range(6))


def check_quantize_bruteforce():
    """Code = index of the nearest reconstruction level over all L levels
    (brute-force argmin; an exact tie goes to the upper level), except where
    the value sits within fp32 rounding of a midpoint."""
    rng = np.random.default_rng(7)
    for b in range(1, 9):
        levels = 1 << b
        step = float(rng.uniform(0.05, 3.0))
        thr = codec.thresholds(step, b)
        c = rng.standard_normal(3000) * step * levels / 3
        q = codec.quantize_channel(c, thr)
        c32 = c.astype(np.float32).astype(np.float64)
        lv = (np.arange(levels) - (levels - 1) / 2) * step
        checked = 0
        for i in range(c.shape[0]):
            dist = np.abs(c32[i] - lv)
            order = np.argsort(dist, kind="stable")
            if dist[order[1]] - dist[order[0]] <= 1e-6 * step:
                continue
            assert q[i] == order[0]
            checked += 1
        assert checked > 2900
        # a value exactly on threshold k (1-based) takes code k (upper cell)
        qt = codec.quantize_channel(thr.astype(np.float64), thr)
        assert np.array_equal(qt, np.arange(1, levels))


def test_quantize_bruteforce():
    check_quantize_bruteforce()


def check_quantize_error_bound():
    rng = np.random.default_rng(8)
    for b in range(1, 9):
        levels = 1 << b
        step = codec.delta_star(b)
        thr = codec.thresholds(step, b)
        c = rng.standard_normal(20000)
        q = codec.quantize_channel(c, thr)
        chat = codec.dequantize_channel(q, step, b)
        gran = np.abs(c) <= levels * step / 2
        err = np.abs(c - chat)
        assert err[gran].max() <= step / 2 * (1 + 1e-6) + 1e-7
        over = ~gran
        assert np.all((q[over] == 0) | (q[over] == levels - 1))
        assert np.allclose(err[over], np.abs(c[over]) - (levels - 1) * step / 2, rtol=1e-9)


def test_quantize_error_bound():
    check_quantize_error_bound()


def test_quantize_special_values():
    thr = codec.thresholds(0.5, 3)
    q = codec.quantize_channel(np.array([np.nan, np.inf, -np.inf, 1e30, -1e30]), thr)
    assert list(q) == [0, 7, 0, 7, 0]


def test_overload_rate_closed_form():
    rng = np.random.default_rng(10)
    for b in (1, 2, 3):
        levels = 1 << b
        step = codec.delta_star(b)
        c = rng.standard_normal(400000)
        q = codec.quantize_channel(c, codec.thresholds(step, b))
        over = np.mean(np.abs(c) > levels * step / 2)
        pred = 2 * special.ndtr(-levels * step / 2)
        assert abs(over - pred) <= 5 * math.sqrt(pred * (1 - pred) / c.size) + 1e-12
        assert q.min() >= 0 and q.max() <= levels - 1


# ----------------------------------------------------------------- O9 format
def _hand_cases():
    cases, cur = [], None
    for key, vals in read_golden("f1_hand_vectors.txt"):
        if key == "case":
            cur = {"bits": None, "codes": [], "bytes": None}
            cases.append(cur)
        elif key == "bits":
            cur["bits"] = np.array([int(v) for v in vals], np.uint8)
        elif key == "codes":
            cur["codes"].append([int(v) for v in vals])
        elif key == "bytes":
            cur["bytes"] = np.array([int(v) for v in vals], np.uint8)
    return cases


def check_pack_hand_vectors():
    for c in _hand_cases():
        codes = np.array(c["codes"], np.int64)
        got = codec.pack(codes, c["bits"])
        assert np.array_equal(got, c["bytes"]), (got, c["bytes"])
        assert np.array_equal(codec.unpack(got, c["bits"], codes.shape[0]), codes)


def test_pack_hand_vectors():
    check_pack_hand_vectors()


def _bigint_pack(codes, bits):
    """Independent packer: one Python integer holding the whole stream."""
    total = int(np.sum(bits))
    acc, pos = 0, 0
    for t in range(codes.shape[0]):
        for j in range(len(bits)):
            if bits[j]:
                acc |= int(codes[t, j]) << pos
                pos += int(bits[j])
    assert pos == total * codes.shape[0]
    nbytes = codec.packed_bytes(total, codes.shape[0])
    return np.frombuffer(acc.to_bytes(nbytes, "little"), dtype=np.uint8)


def check_pack_bigint():
    rng = np.random.default_rng(11)
    for trial in range(20):
        d = int(rng.integers(1, 17))
        bits = rng.integers(0, 9, size=d).astype(np.uint8)
        n = int(rng.integers(0, 9))
        codes = np.zeros((n, d), np.int64)
        for j in range(d):
            codes[:, j] = rng.integers(0, 1 << int(bits[j]), size=n)
        p = codec.pack(codes, bits)
        assert np.array_equal(p, _bigint_pack(codes, bits))
        assert p.shape[0] % 16 == 0
        assert np.array_equal(codec.unpack(p, bits, n), codes)


def test_pack_bigint_and_roundtrip():
    check_pack_bigint()


def test_pack_prefix_invariant():
    """Append-only cache (SPECTRA summary, "La Pipeline" steps 2-3): encoding
    n tokens then m more gives the same stream as encoding n+m at once."""
    rng = np.random.default_rng(12)
    bits = np.array([7, 5, 3, 3, 2, 1, 1, 0], np.uint8)     # B = 22, unaligned
    codes = np.stack([rng.integers(0, 1 << int(b), 37) for b in bits], axis=1)
    full = codec.pack(codes, bits)
    for m in (1, 5, 16, 36):
        part = codec.pack(codes[:m], bits)
        nb = m * 22 // 8
        assert np.array_equal(part[:nb], full[:nb])
        rem = (m * 22) % 8
        if rem:
            mask = (1 << rem) - 1
            assert (int(part[nb]) & mask) == (int(full[nb]) & mask)
            assert int(part[nb]) >> rem == 0


def test_append_pack_equals_pack_of_all():
    """Appending records to a stream gives the stream of all tokens (F1 is
    append-only), for record lengths on and off byte and word boundaries,
    appends of one token and of many, and old streams whose padding is dirty
    past the last record only where F1 allows none (it must stay ignored)."""
    rng = np.random.default_rng(21)
    for bits in (np.array([7, 5, 3, 3, 2, 1, 1, 0], np.uint8),      # B = 22
                 np.array([4] * 8, np.uint8),                      # B = 32, word aligned
                 np.array([3, 3, 2, 1, 0, 0, 0, 0], np.uint8)):    # B = 9
        n = 41
        codes = np.stack([rng.integers(0, 1 << int(b), n) for b in bits], axis=1)
        full = codec.pack(codes, bits)
        for n_old in (0, 1, 5, 16, 40):
            old = codec.pack(codes[:n_old], bits)
            got = codec.append_pack(old, n_old, codes[n_old:], bits)
            assert np.array_equal(got, full), (int(bits.sum()), n_old)
        # one token at a time
        cur = codec.pack(codes[:0], bits)
        for t in range(n):
            cur = codec.append_pack(cur, t, codes[t:t + 1], bits)
        assert np.array_equal(cur, full)
        # bits of the old stream past its records are not carried over
        old = codec.pack(codes[:3], bits).copy()
        nb = old.shape[0]
        tail_bit = 3 * int(bits.sum())
        if tail_bit < nb * 8:
            old[tail_bit >> 3] |= np.uint8(0xFF << (tail_bit & 7) & 0xFF)
            old[(tail_bit >> 3) + 1:] = 0xFF
        assert np.array_equal(codec.append_pack(old, 3, codes[3:], bits), full)


# -------------------------------------------------------------- O8 rounding# -------------------------------------------------------------- O8 rounding
def test_round_to_bf16():
    # agrees with the generator's bit-level fp32 -> bf16 RNE on fp32 inputs
    x = np.random.default_rng(13).standard_normal(20000).astype(np.float32) * 37
    assert np.array_equal(codec.round_to_bf16(x.astype(np.float64)),
                          synth.to_bf16_values(x).astype(np.float64))
    # exact ties go to even; fp64 inputs are rounded once (not via fp32)
    assert codec.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert codec.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert codec.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    assert codec.round_to_bf16(np.array([-0.0, 0.0]))[1] == 0.0


# ------------------------------------------------ O8 reconstruction identities
def check_parseval_and_dropped_energy():
    lam = np.arange(1, 33, dtype=np.float64) ** -1.5
    x = gaussian_stream(3000, lam, 14)
    st = codec.calibrate_head(x, 1000, 1.0)
    assert (st["bits"] == 0).any()
    c = codec.project(st, x)
    q = codec.quantize(st, c)
    chat = codec.dequantize(st, q)
    packed = codec.pack(q, st["bits"])
    xhat = codec.reconstruct_exact(st, packed, x.shape[0])
    lhs = np.sum((x - xhat) ** 2, axis=1)
    rhs = np.sum((c - chat) ** 2, axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-14)
    drop = st["bits"] == 0
    assert np.array_equal(chat[:, drop], np.zeros_like(chat[:, drop]))
    e_drop = np.sum((c - chat)[:, drop] ** 2)
    assert abs(e_drop - np.sum(c[:, drop] ** 2)) <= 1e-12 * np.sum(c[:, drop] ** 2)


def test_parseval_and_dropped_energy():
    check_parseval_and_dropped_energy()


def test_predicted_relmse():
    """relMSE ~ sum lam_j eps(b_j) / sum lam_j for Gaussian coefficients."""
    lam = np.arange(1, 129, dtype=np.float64) ** -1.0
    x = gaussian_stream(20000, lam, 15)
    st = codec.calibrate_head(x, 4096, 2.0)
    xhat = codec.reconstruct_exact(st, codec.encode_kv(st, x), x.shape[0])
    measured = codec.rel_mse(x, xhat)
    eps = np.array([1.0] + [codec.uniform_gaussian_mse(codec.delta_star(b), 1 << b)
                            for b in range(1, 9)])
    pred = np.sum(st["lam"] * eps[st["bits"]]) / np.sum(st["lam"])
    assert abs(measured - pred) <= 0.1 * pred


def test_water_filling_beats_uniform_on_spiked():
    w = synth.WORKLOADS[1]
    x = synth.stream(w, 0, 0, 0, 0)
    st_w = codec.calibrate_head(x, w.n_calib, 2.0)
    st_u = codec.calibrate_head(x, w.n_calib, 2.0, bits=np.full(128, 2, np.uint8))
    rw = codec.rel_mse(x, codec.decode_kv(st_w, codec.encode_kv(st_w, x), x.shape[0], "f32"))
    ru = codec.rel_mse(x, codec.decode_kv(st_u, codec.encode_kv(st_u, x), x.shape[0], "f32"))
    assert rw < ru


def test_identity_path_exact_projection():
    x = np.random.default_rng(16).standard_normal((64, 16))
    st = codec.calibrate_head(x, 64, 3.0, xform=codec.XFORM_IDENTITY)
    assert np.array_equal(codec.project(st, x), x)
    # iid unit-variance Gaussian channel, uniform 3 bits: relMSE -> eps(3)
    xx = np.random.default_rng(17).standard_normal((100000, 4))
    st = codec.calibrate_head(xx, 100000, 3.0, bits=np.full(4, 3, np.uint8),
                              xform=codec.XFORM_IDENTITY)
    r = codec.rel_mse(xx, codec.reconstruct_exact(st, codec.encode_kv(st, xx), xx.shape[0]))
    assert abs(r - codec.uniform_gaussian_mse(codec.delta_star(3), 8)) < 0.03 * r


# ---------------------------------------------------------------- O10 attention
def _attend_loops(khat, vhat, q, scale):
    g, n, d = q.shape[0], khat.shape[0], khat.shape[1]
    out = np.zeros((g, d))
    for h in range(g):
        s = [scale * sum(q[h, i] * khat[t, i] for i in range(d)) for t in range(n)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        for i in range(d):
            out[h, i] = sum(e[t] * vhat[t, i] for t in range(n)) / z
    return out


def _small_pair(n=23, d=8, seed=18, avg=3.0):
    lam = np.arange(1, d + 1, dtype=np.float64) ** -1.0
    k = gaussian_stream(n, lam, seed)
    v = gaussian_stream(n, lam * 2, seed + 1)
    ks = codec.calibrate_head(k, n, avg)
    vs = codec.calibrate_head(v, n, avg)
    return k, v, ks, vs, codec.encode_kv(ks, k), codec.encode_kv(vs, v)


def check_attention_loops():
    k, v, ks, vs, kp, vp = _small_pair()
    n, d = k.shape
    q = np.random.default_rng(19).standard_normal((3, d)).astype(np.float32).astype(np.float64)
    out = codec.attend_compressed(ks, vs, kp, vp, n, q)
    ref = _attend_loops(codec.reconstruct_exact(ks, kp, n), codec.reconstruct_exact(vs, vp, n),
                        q, 1 / math.sqrt(d))
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_attention_matches_loops():
    check_attention_loops()


def test_attention_special_cases():
    k, v, ks, vs, kp, vp = _small_pair()
    q = np.random.default_rng(20).standard_normal((2, 8))
    one = codec.attend_compressed(ks, vs, kp[:16], vp[:16], 1, q)
    v1 = codec.reconstruct_exact(vs, vp, 1)[0]
    assert np.allclose(one, np.tile(v1, (2, 1)), rtol=1e-6, atol=1e-7)
    # identical keys: uniform weights -> mean of V_hat
    kk = np.tile(k[:1], (23, 1))
    kp2 = codec.encode_kv(ks, kk)
    o = codec.attend_compressed(ks, vs, kp2, vp, 23, q)
    assert np.allclose(o, codec.reconstruct_exact(vs, vp, 23).mean(axis=0)[None, :], rtol=1e-6, atol=1e-7)


def test_latent_identity():
    k, v, ks, vs, kp, vp = _small_pair()
    q = np.random.default_rng(21).standard_normal(8)
    chat = codec.dequantize(ks, codec.unpack(kp, ks["bits"], 23))
    assert np.allclose((ks["U"].T @ q) @ chat.T, q @ (chat @ ks["U"].T).T, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- G5 self-checks
def test_self_checks_on_cfg2_head():
    w = synth.WORKLOADS[2]
    x = synth.stream(w, 0, 0, 3, 1, n=6000)
    sigma = codec.second_moment(x, w.n_calib)
    check_eigenbasis_invariants(sigma)
    for avg in w.budgets:
        st = codec.calibrate_head(x, w.n_calib, avg)
        assert int(st["bits"].astype(int).sum()) == codec.total_bits_for(avg, 128)
        assert np.all(np.diff(st["bits"].astype(int)) <= 0)


# ------------------------------------------------ allocation variants (next row)
def _compositions(total, parts, cap):
    if parts == 1:
        if total <= cap:
            yield (total,)
        return
    for first in range(min(total, cap) + 1):
        for rest in _compositions(total - first, parts - 1, cap):
            yield (first,) + rest


def test_quantizer_mse_decreasing_convex_and_closed_form():
    """eps(1) = 1 - 2/pi (levels +-sqrt(2/pi)); eps decreasing and convex in b,
    which is what makes the marginal greedy optimal."""
    eps = [codec.quantizer_mse(b) for b in range(9)]
    assert abs(eps[1] - (1 - 2 / math.pi)) < 1e-12
    assert all(eps[b + 1] < eps[b] for b in range(8))
    assert all(eps[b] - eps[b + 1] > eps[b + 1] - eps[b + 2] for b in range(7))


def test_operational_allocation_is_optimal_by_brute_force():
    rng = np.random.default_rng(60)
    for trial in range(4):
        lam = np.sort(rng.exponential(1.0, 5))[::-1] * (1 + trial)
        for B in (3, 7, 12):
            got = codec.allocate_bits(lam, B, "operational")
            assert got.sum() == B
            cost = lambda b: sum(lam[j] * codec.quantizer_mse(int(b[j])) for j in range(5))
            best = min(cost(c) for c in _compositions(B, 5, 8))
            assert cost(got) <= best * (1 + 1e-12)


def test_grouped_allocation_is_optimal_by_brute_force():
    rng = np.random.default_rng(61)
    lam = np.sort(rng.exponential(1.0, 8))[::-1]
    G = 2
    lam_g = lam.reshape(4, 2).sum(axis=1)
    for B in (4, 9, 12, 17):
        got = codec.allocate_bits(lam, B, "grouped", G)
        assert got.sum() == G * (B // G)
        assert np.all(got.reshape(4, 2)[:, 0] == got.reshape(4, 2)[:, 1])     # one width per group
        cost = lambda bg: sum(lam_g[k] * 4.0 ** -int(bg[k]) for k in range(4))
        best = min(cost(c) for c in _compositions(B // G, 4, 8))
        assert cost(got.reshape(4, 2)[:, 0]) <= best * (1 + 1e-12)
    # a group's variance is the sum over its channels, not its largest one
    got = codec.allocate_bits(np.array([1.0, 0.0, 0.6, 0.6]), 2, "grouped", 2)
    assert np.array_equal(got, [0, 0, 1, 1])


def test_floor_and_gap_allocations():
    lam = np.arange(1, 129, dtype=np.float64) ** -1.2
    f = codec.allocate_bits(lam, 300, "floor", 1)
    assert f.sum() == 300 and f.min() >= 1
    # the floor shifts the problem: the rest is the default greedy with 7-bit caps
    assert np.array_equal(f - 1, codec.water_fill(lam, 300 - 128, 7))
    # a planted spectral gap after channel 10 (ratio 1e4): nothing past it
    lam2 = np.concatenate([np.linspace(2.0, 1.0, 10), np.full(118, 1e-4)])
    g = codec.allocate_bits(lam2, 64, "gap", 100.0)
    assert g[10:].sum() == 0 and g.sum() == 64
    assert np.array_equal(g[:10], codec.water_fill(lam2[:10], 64))
    # budget beyond the kept channels' capacity is not spent
    assert codec.allocate_bits(lam2, 200, "gap", 100.0).sum() == 80
    # no gap above the ratio: the default
    assert np.array_equal(codec.allocate_bits(lam, 256, "gap", 100.0), codec.water_fill(lam, 256))
