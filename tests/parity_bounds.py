"""Per-difference checks for GPU codes and sketch bits against the oracle.

A GPU code may differ from the oracle's only where the projection error of
the GPU's arithmetic can move the coefficient across a decision threshold.
These helpers derive that error from the arithmetic and check every differing
entry against it, besides the fraction and the one-level rule.

Eigen / identity encode. The kernel forms y_j = sum_i x_i B_ij + L/2 with
B = U / step held as a bf16 pair (B_hi + B_lo): each of hi and lo keeps 8
significant bits, so |B - B_hi - B_lo| <= 2^-16 |B|; fp32 tokens are split the
same way (|x - x_hi - x_lo| <= 2^-16 |x|). The products are exact in fp32 and
summed in fp32 over at most 3 x 128 terms plus L/2, each addition within
2^-24 of its running sum, so |y_gpu - y| <= 2^-16 * 3 * sum_i |x_i| |B_ij|
+ 384 * 2^-24 * (sum_i |x_i B_ij| + L/2). In coefficient units (times the
step) that is below 2^-14 sum_i |x_i| |U_ij| + 2^-15 L step_j. The oracle
compares fl32(c) with fl32 thresholds, which adds 2^-24 (|c| + |t|). When
the GPU also calibrated the state, its basis and steps differ from the
oracle's by at most basis_err (absolute, per entry) and step_rel (relative):
the coefficient moves by at most basis_err sum_i |x_i| and the threshold by
step_rel |t|.
"""
import numpy as np


def projection_eps(x, U, steps, bits, basis_err=0.0, step_rel=0.0):
    """Bound on |c_gpu - c| in coefficient units, [n][d]."""
    ax = np.abs(np.asarray(x, np.float64))
    eps = 2.0 ** -14 * (ax @ np.abs(np.asarray(U, np.float64)))
    levels = np.where(np.asarray(bits) > 0, 1 << np.asarray(bits, np.int64), 0).astype(np.float64)
    eps = eps + 2.0 ** -15 * (levels * np.abs(np.asarray(steps, np.float64)))[None, :]
    if basis_err:
        eps = eps + basis_err * ax.sum(axis=1, keepdims=True)
    return eps, step_rel


def assert_code_diffs_at_boundaries(q_gpu, q_or, c, st, eps, step_rel=0.0, max_frac=1e-4):
    """q_gpu, q_or: codes [n][d]; c: the oracle's fp64 coefficients [n][d];
    st: the oracle state (bits, steps); eps from projection_eps. At most
    max_frac of kept codes differ, each by one level, and each differing
    coefficient lies within its bound of the threshold between the two codes,
    (k - L/2) step with k the larger code."""
    q_gpu = np.asarray(q_gpu, np.int64)
    q_or = np.asarray(q_or, np.int64)
    bits = np.asarray(st["bits"], np.int64)
    kept = bits > 0
    diff = q_gpu != q_or
    n_kept = max(1, q_or.shape[0] * int(kept.sum()))
    assert diff.sum() / n_kept <= max_frac, diff.sum() / n_kept
    if not diff.any():
        return
    assert np.abs(q_gpu - q_or)[diff].max() == 1
    t_idx, j_idx = np.nonzero(diff)
    k = np.maximum(q_gpu, q_or)[diff].astype(np.float64)
    L = (1 << bits[j_idx]).astype(np.float64)
    step = np.asarray(st["steps"], np.float64)[j_idx]
    thr = (k - L / 2.0) * step
    cc = np.asarray(c, np.float64)[t_idx, j_idx]
    e = np.broadcast_to(eps, c.shape)[t_idx, j_idx]
    allowed = e + 2.0 ** -24 * (np.abs(cc) + np.abs(thr)) + step_rel * np.abs(thr)
    far = np.abs(cc - thr) > allowed
    assert not far.any(), (f"{int(far.sum())} of {int(diff.sum())} differing codes are not at a threshold; "
                           f"worst |c - t| / bound = {float((np.abs(cc - thr) / allowed).max()):.3g}")


def rht_rotation_eps(x):
    """Walsh-Hadamard encode: the kernel forms H D x either from exact bf16
    products (entries +-1) summed in fp32 on the matrix cores (128 terms: error
    <= 128 * 2^-24 sum |x|) or by seven fp32 butterfly stages (each output's
    error <= 7 * 2^-24 sum |x|, inside the same bound), the
    norm |x| in fp32 (relative error <= 2^-18, one sum of squares and a square
    root) and compares against thresholds scaled by |x| sqrt(d) in fp32. In units
    of y = H D x / (|x| sqrt(d)) the bound per token is
    2^-17 sum_i |x_i| / (|x| sqrt(d)) + 2^-17 max(|y|, |t|)."""
    x = np.asarray(x, np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    d = x.shape[1]
    return np.where(nu > 0, 2.0 ** -17 * np.abs(x).sum(axis=1) / np.where(nu > 0, nu, 1.0) / np.sqrt(d), 0.0)


def assert_rht_code_diffs_at_boundaries(q_gpu, q_or, y, thresholds, eps_tok, max_frac=1e-4):
    """Walsh-Hadamard codes: y the oracle's rotated unit coordinates [n][d],
    thresholds the fp32 codebook thresholds (code k starts at thresholds[k-1])."""
    q_gpu = np.asarray(q_gpu, np.int64)
    q_or = np.asarray(q_or, np.int64)
    diff = q_gpu != q_or
    assert diff.mean() <= max_frac, diff.mean()
    if not diff.any():
        return
    assert np.abs(q_gpu - q_or)[diff].max() == 1
    t_idx, j_idx = np.nonzero(diff)
    k = np.maximum(q_gpu, q_or)[diff]
    thr = np.asarray(thresholds, np.float32).astype(np.float64)[k - 1]
    yy = np.asarray(y, np.float64)[t_idx, j_idx]
    allowed = eps_tok[t_idx] + 2.0 ** -17 * np.maximum(np.abs(yy), np.abs(thr)) + 2.0 ** -24
    far = np.abs(yy - thr) > allowed
    assert not far.any(), (f"{int(far.sum())} of {int(diff.sum())} differing codes are not at a threshold; "
                           f"worst |y - t| / bound = {float((np.abs(yy - thr) / allowed).max()):.3g}")


def assert_sign_diffs_small(z_gpu, z_or, proj, eps, max_frac):
    """Sketch signs: z = [S r >= 0] per row. A GPU sign may differ only where
    the oracle's S r lies within eps of 0 (eps [n][m], the error bound of the
    GPU's S r), and at most max_frac of the bits may differ."""
    diff = np.asarray(z_gpu) != np.asarray(z_or)
    assert diff.mean() <= max_frac, diff.mean()
    if not diff.any():
        return
    far = np.abs(np.asarray(proj, np.float64))[diff] > np.broadcast_to(eps, diff.shape)[diff]
    assert not far.any(), f"{int(far.sum())} of {int(diff.sum())} differing sign bits are not near 0"


def check_eigen_codes(q_gpu, st, x, gpu_state=None, max_frac=1e-4):
    """End-to-end check of GPU codes for tokens x [n][d] against the oracle
    state st: the oracle's codes of x, every difference at a threshold. With
    gpu_state (a state the GPU calibrated), its basis and steps enter the
    bound as measured differences from the oracle's."""
    from oracle import codec
    c = codec.project(st, x)
    q_or = codec.quantize(st, c)
    basis_err, step_rel = 0.0, 0.0
    if gpu_state is not None:
        basis_err = float(np.abs(gpu_state.basis() - st["U"]).max())
        s_o = np.asarray(st["steps"], np.float64)
        s_g = np.asarray(gpu_state.steps, np.float64)
        step_rel = float(np.max(np.abs(s_g - s_o) / np.where(s_o > 0, s_o, 1.0)))
    eps, step_rel = projection_eps(x, st["U"], st["steps"], st["bits"], basis_err, step_rel)
    assert_code_diffs_at_boundaries(q_gpu, q_or, c, st, eps, step_rel, max_frac)
    return q_or


def decode_w16(st, dtype):
    """Whether the library may decode this state in one fp16 pass: bf16
    output, at most 2 bits per value, largest kept step in [2^-7, 2^20] (the
    library's rule; in a batch every state must meet it, so a state that meets
    it may also go through the bf16 pair)."""
    bits = np.asarray(st["bits"])
    steps = np.asarray(st["steps"], np.float64)[bits > 0]
    smax = float(steps.max()) if steps.size else 0.0
    return dtype == "bf16" and int(bits.sum()) <= 2 * bits.shape[0] and (smax == 0.0 or 2.0 ** -7 <= smax <= 2.0 ** 20)


def decode_arith(st, dtype):
    """Bound on the GPU decode's error before the output rounding, per output
    dim. bf16 pair: each W_ij = U_ij step_j is held to 2^-17 relative and the
    exact integer codes are summed in fp32: 2^-15 sum_j |U_ij| step_j (L_j - 1).
    One fp16 pass: W_ij 2^e rounded to fp16 with its largest entry in
    [2^13, 2^14), so 2^-11 relative or 2^-25 absolute in the scaled units
    (below 2^-38 of the largest |W| after scaling back), against a bias of the
    same fp16 entries: the error is sum_j dW_ij (q_j - (L_j - 1)/2) <=
    2^-11 sum_j |W_ij| (L_j - 1)/2 + 2^-38 max|W| sum_j (L_j - 1)/2, plus the
    fp32 sums (2^-16 of the same magnitude)."""
    bits = np.asarray(st["bits"])
    levels_m1 = np.where(bits > 0, (1 << bits.astype(np.int64)) - 1, 0).astype(np.float64)
    mag = np.abs(np.asarray(st["U"], np.float64)) @ (np.asarray(st["steps"], np.float64) * levels_m1)
    if decode_w16(st, dtype):
        wmax = float((np.abs(np.asarray(st["U"], np.float64)) * np.asarray(st["steps"], np.float64)[None, :]).max())
        return (2.0 ** -12 + 2.0 ** -16) * mag + 2.0 ** -39 * wmax * levels_m1.sum()
    return 2.0 ** -15 * mag
