"""Pins of the 1-bit Johnson-Lindenstrauss residual sketch oracle: the
estimator is unbiased with the closed-form variance of a Gaussian sketch,
its zero-mean score noise is amplified by exp as Jensen's inequality says
(E[exp(e)] = exp(var/2) for Gaussian e), a zero residual gives no
correction, and on real codes the corrected scores average to the true ones."""
import math

import numpy as np

import synth
from oracle import codec, qjl, rht

D = 128


def _estimates(q, r, trials, m=qjl.SKETCH_BITS, seed=80):
    rng = np.random.default_rng(seed)
    est = np.empty(trials)
    rn = float(np.sqrt(r @ r))
    for t in range(trials):
        S = rng.standard_normal((m, D))
        z = np.where(S @ r >= 0, 1.0, -1.0)
        est[t] = math.sqrt(math.pi / 2) / m * rn * float((S @ q) @ z)
    return est


def test_estimator_unbiased_with_closed_form_variance():
    rng = np.random.default_rng(81)
    q = rng.standard_normal(D)
    r = 0.3 * rng.standard_normal(D)
    est = _estimates(q, r, 4000)
    rn = math.sqrt(r @ r)
    var = rn * rn / qjl.SKETCH_BITS * (math.pi / 2 * (q @ q) - (q @ r / rn) ** 2)
    se = math.sqrt(var / est.size)
    assert abs(est.mean() - q @ r) < 4 * se
    assert abs(est.var() / var - 1) < 0.1


def test_jensen_amplification_of_score_noise():
    """The estimator's error e is zero-mean and near-Gaussian, so the softmax
    weight exp(s + e) is inflated on average by exp(var(e)/2)."""
    rng = np.random.default_rng(82)
    q = 0.5 * rng.standard_normal(D)
    r = 0.2 * rng.standard_normal(D)
    e = _estimates(q, r, 6000, seed=83) - q @ r
    assert abs(e.mean()) < 4 * e.std() / math.sqrt(e.size)
    ratio = np.exp(e).mean() / math.exp(e.var() / 2)
    assert abs(ratio - 1) < 0.03
    assert np.exp(e).mean() > 1.0


def _rht_case(n=64, seed=84):
    rng = np.random.default_rng(seed)
    cb = rht.codebook_fp32(rht.lloyd_max(synth.sphere_coordinate_samples(20000))[0])
    st = rht.make_state(np.where(rng.random(D) < 0.5, -1, 1), cb)
    x = rng.standard_t(3, (n, D))
    kp, kn = rht.encode_kv(st, x)
    S = rng.standard_normal((qjl.SKETCH_BITS, D)).astype(np.float32)
    return st, x, kp, kn, S


def test_zero_residual_gives_no_correction():
    st, x, kp, kn, S = _rht_case(n=5)
    exact = rht.reconstruct_exact(st, kp, kn, 5)         # keys equal to their reconstruction
    sk, rn = qjl.sketch_encode(st, exact, kp, kn, S)
    assert np.all(rn == 0)
    assert np.all(qjl.score_correction(np.ones((2, D)), sk, rn, S, 5) == 0)


def test_sketch_estimate_is_unbiased_on_real_codes():
    """On real codes the corrected score is an unbiased estimate of q . k:
    averaged over independent sketch matrices it converges to the true score,
    while any single sketch adds variance (at m = d about pi/2 times the
    uncorrected error, which is the noise the pages' Jensen analysis is about)."""
    st, x, kp, kn, _ = _rht_case()
    n = x.shape[0]
    q = np.random.default_rng(85).standard_normal((8, D))
    true = q @ x.T
    base = q @ rht.reconstruct_exact(st, kp, kn, n).T
    rng = np.random.default_rng(86)
    acc = np.zeros_like(base)
    T = 400
    for _ in range(T):
        S = rng.standard_normal((qjl.SKETCH_BITS, D)).astype(np.float32)
        sk, rn = qjl.sketch_encode(st, x, kp, kn, S)
        acc += base + qjl.score_correction(q, sk, rn, S, n)
    err_base = np.mean((base - true) ** 2)
    assert np.mean((acc / T - true) ** 2) < 0.015 * err_base


def test_sketch_bits_layout():
    """One bit per sketch row, F1 layout with 1-bit channels: bit t*m + i is
    row i of token t's sign (1 = non-negative)."""
    st, x, kp, kn, S = _rht_case(n=3)
    sk, _ = qjl.sketch_encode(st, x, kp, kn, S)
    r = x - rht.reconstruct_exact(st, kp, kn, 3)
    bits = np.unpackbits(sk, bitorder="little")[: 3 * qjl.SKETCH_BITS].reshape(3, -1)
    assert np.array_equal(bits, (r @ S.astype(np.float64).T >= 0).astype(np.uint8))
    assert sk.shape[0] == codec.packed_bytes(qjl.SKETCH_BITS, 3)


# ----------------------------------------------------- selective sketch, eigen cache
def _eigen_case(n=48, avg=1.33, seed=87):
    w = synth.WORKLOADS[2]
    x = synth.stream(w, 0, 0, 1, 0, n=2048)
    st = codec.calibrate_head(x, 2048, avg)
    S = np.random.default_rng(seed).standard_normal((qjl.SKETCH_BITS, D)).astype(np.float32)
    return st, x[:n], S


def test_latent_residual_identity():
    """q . k - q . K_hat = (U^T q) . (c - c_hat) exactly; the selective
    residual leaves out only the dropped channels' coefficients."""
    st, x, _ = _eigen_case()
    n = x.shape[0]
    q = np.random.default_rng(88).standard_normal(D)
    kp = codec.encode_kv(st, x)
    miss = x @ q - codec.reconstruct_exact(st, kp, n) @ q
    r = qjl.latent_residual(st, x)
    c = codec.project(st, x)
    dropped = np.asarray(st["bits"]) == 0
    assert dropped.any()                                  # 1.33 bits drops channels
    rest = c[:, dropped] @ (st["U"].T @ q)[dropped]
    assert np.allclose(miss, r @ (st["U"].T @ q) + rest, rtol=0, atol=1e-9 * np.abs(miss).max())
    assert np.all(r[:, dropped] == 0)


def test_selective_sketch_unbiased():
    """Over independent sketches the corrected score converges to
    q . K_hat + (U^T q) . r (the dropped channels stay uncorrected)."""
    st, x, _ = _eigen_case()
    n = x.shape[0]
    q = np.random.default_rng(89).standard_normal((4, D))
    kp = codec.encode_kv(st, x)
    base = q @ codec.reconstruct_exact(st, kp, n).T
    target = base + (q @ st["U"]) @ qjl.latent_residual(st, x).T
    rng = np.random.default_rng(90)
    acc = np.zeros_like(base)
    T = 300
    for _ in range(T):
        S = rng.standard_normal((qjl.SKETCH_BITS, D)).astype(np.float32)
        sk, rn = qjl.sketch_encode_eigen(st, x, S)
        acc += base + qjl.score_correction(q @ st["U"], sk, rn, S, n)
    assert np.mean((acc / T - target) ** 2) < 0.02 * np.mean((base - target) ** 2)


# ------------------------------------------- sketch-corrected attention (the extra term)
def _attention_loops(q, K, V, scale):
    """Textbook softmax attention written out token by token, fp64."""
    g, n = q.shape[0], K.shape[0]
    out = np.zeros((g, V.shape[1]))
    for h in range(g):
        s = [scale * float(np.dot(q[h], K[t])) for t in range(n)]
        mx = max(s)
        w = [math.exp(v - mx) for v in s]
        tot = sum(w)
        for t in range(n):
            out[h] += (w[t] / tot) * V[t]
    return out


def test_extra_term_enters_before_the_scale():
    """`extra` is an additive estimate of the part of q . k the reconstruction
    misses: with extra = q . (k - K_hat) exactly, attention over K_hat equals
    attention over the true keys; extra = 0 changes nothing."""
    rng = np.random.default_rng(91)
    d, n, g = 16, 9, 3
    k = rng.standard_normal((n, d)) * 2.0
    khat = k + 0.3 * rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal((g, d))
    exact = q @ (k - khat).T
    want = _attention_loops(q, k, v, 1.0 / math.sqrt(d))
    got = codec.softmax_attention(q, khat, v, extra=exact)
    assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max()
    assert np.array_equal(codec.softmax_attention(q, khat, v, extra=np.zeros((g, n))),
                          codec.softmax_attention(q, khat, v))
    # the correction is not negligible here
    assert np.abs(codec.softmax_attention(q, khat, v) - want).max() > 1e-2


# With m sign rows the estimate of q_h . r_t has standard deviation
# sigma_ht = |r_t| sqrt((pi/2 |q_h|^2 - (q_h . r_t / |r_t|)^2) / m) (the closed
# form pinned above). If every score moves by at most D (here 5 sigma times the
# softmax scale), output i moves by at most D R_i / 2, R_i the range of value
# channel i over the tokens: d/dl softmax(s + l e) . v_i = Cov(e, v_i) under the
# tilted weights, and |Cov| <= (range of e / 2)(range of v_i / 2) (Popoviciu).
SKETCH_ROWS = 400_000


def _convergence_bound(q, r, vhat, m, scale):
    rn2 = np.sum(r * r, axis=1)
    qn2 = np.sum(q * q, axis=1)
    sig = np.sqrt(rn2[None, :] * (math.pi / 2) * qn2[:, None] / m)
    delta = 5.0 * float(sig.max()) * scale
    return delta * (vhat.max(axis=0) - vhat.min(axis=0)) / 2.0


def _small_rht_caches(seed, d=16, n=10):
    rng = np.random.default_rng(seed)
    cb = rht.codebook_fp32(np.sort(rng.standard_normal(8)) / math.sqrt(d))
    kst = rht.make_state(np.where(rng.random(d) < 0.5, -1, 1), cb)
    vst = rht.make_state(np.where(rng.random(d) < 0.5, -1, 1), cb)
    k = rng.standard_t(3, (n, d))
    v = rng.standard_normal((n, d))
    kp, kn = rht.encode_kv(kst, k)
    vp, vn = rht.encode_kv(vst, v)
    S = rng.standard_normal((SKETCH_ROWS, d)).astype(np.float32)
    q = rng.standard_normal((3, d))
    return kst, vst, k, kp, kn, vp, vn, S, q


def check_sketch_attention_converges_rht(seed=92):
    """Walsh-Hadamard keys with their residual sketch: with 400k sign rows the
    corrected attention is attention over the unquantized keys, within the
    sampling bound; without the correction it is not."""
    kst, vst, k, kp, kn, vp, vn, S, q = _small_rht_caches(seed)
    d, n = k.shape[1], k.shape[0]
    sk, rn = qjl.sketch_encode(kst, k, kp, kn, S)
    got = qjl.attend_compressed(kst, vst, kp, kn, sk, rn, S, vp, vn, n, q)
    khat = rht.reconstruct_exact(kst, kp, kn, n)
    vhat = rht.reconstruct_exact(vst, vp, vn, n)
    scale = 1.0 / math.sqrt(d)
    want = _attention_loops(q, k, vhat, scale)
    bound = _convergence_bound(q, k - khat, vhat, SKETCH_ROWS, scale)
    assert np.all(np.abs(got - want) <= bound[None, :] + 1e-6), (np.abs(got - want).max(), bound.max())
    plain = _attention_loops(q, khat, vhat, scale)
    assert np.abs(plain - want).max() > 1.5 * bound.max()


def test_sketch_attention_converges_rht():
    check_sketch_attention_converges_rht()


def _small_eigen_caches(seed, avg, d=16, n=10):
    rng = np.random.default_rng(seed)
    lam = np.arange(1, d + 1, dtype=np.float64) ** -1.2
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    Q = Q * np.sign(np.diag(R))[None, :]
    calib = (rng.standard_normal((512, d)) * np.sqrt(lam)) @ Q.T
    kst = codec.calibrate_head(calib, 512, avg)
    vst = codec.calibrate_head((rng.standard_normal((512, d)) * np.sqrt(lam)) @ Q.T, 512, avg)
    k = (rng.standard_normal((n, d)) * np.sqrt(lam)) @ Q.T
    v = rng.standard_normal((n, d)) * 0.5
    S = rng.standard_normal((SKETCH_ROWS, d)).astype(np.float32)
    q = rng.standard_normal((3, d)) * 3.0
    return kst, vst, k, v, S, q


def check_sketch_attention_converges_eigen(avg, seed=93):
    """Eigen keys with the selective sketch: the corrected attention converges
    to attention over the keys with only their dropped channels missing,
    x - sum_{j dropped} c_j u_j (all keys exactly when no channel is dropped)."""
    kst, vst, k, v, S, q = _small_eigen_caches(seed, avg)
    d, n = k.shape[1], k.shape[0]
    kp, vp = codec.encode_kv(kst, k), codec.encode_kv(vst, v)
    sk, rn = qjl.sketch_encode_eigen(kst, k, S)
    got = qjl.attend_compressed_eigen(kst, vst, kp, sk, rn, S, vp, n, q)
    U = kst["U"]
    dropped = np.asarray(kst["bits"]) == 0
    k_target = k - (k @ U[:, dropped]) @ U[:, dropped].T
    khat = codec.reconstruct_exact(kst, kp, n)
    vhat = codec.reconstruct_exact(vst, vp, n)
    scale = 1.0 / math.sqrt(d)
    want = _attention_loops(q, k_target, vhat, scale)
    # the sketch sees the latent residual, whose norm is that of k_target - K_hat
    bound = _convergence_bound(q, k_target - khat, vhat, SKETCH_ROWS, scale)
    assert np.all(np.abs(got - want) <= bound[None, :] + 1e-6), (np.abs(got - want).max(), bound.max())
    plain = _attention_loops(q, khat, vhat, scale)
    assert np.abs(plain - want).max() > 1.5 * bound.max()
    return dropped.any()


def test_sketch_attention_converges_eigen_all_kept():
    assert not check_sketch_attention_converges_eigen(3.0)


def test_sketch_attention_converges_eigen_with_dropped_channels():
    assert check_sketch_attention_converges_eigen(0.75)
