"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that at least one pin catches each of them. This is the evidence that
the pins constrain the oracle and do not merely restate it."""
import math

import numpy as np
import pytest

import test_oracle_codec as tc
import test_oracle_rht as tr
from oracle import codec, rht

_orig = {name: getattr(codec, name) for name in
         ("sign_fix", "eigenbasis", "water_fill", "thresholds", "dequantize_channel",
          "pack", "unpack", "reconstruct_exact", "attend_compressed", "second_moment",
          "delta_star", "_uniform_mse_slope", "quantize_channel", "uniform_gaussian_mse")}


def _fails(check, *args):
    try:
        check(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _sign_fix_smallest(u):
    u = np.array(u, dtype=np.float64, copy=True)
    for j in range(u.shape[1]):
        k = int(np.argmin(np.abs(u[:, j])))
        if u[k, j] < 0:
            u[:, j] = -u[:, j]
    return u


def _eig_ascending(sigma):
    w, v = np.linalg.eigh(sigma)
    return codec.sign_fix(v), w


def _eig_transposed(sigma):
    u, lam = _orig["eigenbasis"](sigma)
    return u.T.copy(), lam


def _water_fill_half_rate(lam, total_bits, max_bits=8):
    lam = np.asarray(lam, np.float64)
    b = np.zeros(lam.shape[0], np.int64)
    for _ in range(total_bits):
        gain = np.where(b < max_bits, np.maximum(lam, 0) * np.ldexp(1.0, -b), -1.0)
        b[int(np.argmax(gain))] += 1
    return b.astype(np.uint8)


def _thresholds_shifted(step, bits):
    levels = 1 << int(bits)
    k = np.arange(1, levels, dtype=np.float64)
    return ((k - levels / 2.0 + 0.5) * float(step)).astype(np.float32)


def _dequant_no_offset(q, step, bits):
    return np.asarray(q, np.float64) * float(step)


def _pack_msb_first(codes, bits):
    codes = np.asarray(codes, np.int64)
    rev = np.zeros_like(codes)
    for j, b in enumerate(np.asarray(bits)):
        for k in range(int(b)):
            rev[:, j] |= ((codes[:, j] >> k) & 1) << (int(b) - 1 - k)
    return _orig["pack"](rev, bits)


def _reconstruct_wrong_side(state, packed, n):
    return codec.dequantize(state, codec.unpack(packed, state["bits"], n)) @ state["U"]


def _attend_no_scale(k_state, v_state, k_packed, v_packed, n, q, scale=None):
    return _orig["attend_compressed"](k_state, v_state, k_packed, v_packed, n, q, scale=1.0)


def _moment_centred(x, n_calib):
    xc = np.asarray(x, np.float64)[:n_calib]
    xc = xc - xc.mean(axis=0)
    return xc.T @ xc / n_calib


def _slope_dropped_factor(delta, levels):
    a, b, y, p, m = codec._upper_cells(delta, levels)
    return float(-4.0 * np.sum((codec._phi(a) - codec._phi(b)) - m * delta * p))


def _quantize_ties_down(c, thr):
    c32 = np.asarray(c, np.float64).astype(np.float32)
    return (c32[:, None] > np.asarray(thr, np.float32)[None, :]).sum(axis=1).astype(np.int64)


def _mse_dropped_term(delta, levels):
    a, b, y, p, _ = codec._upper_cells(delta, levels)
    mse_half = p - (codec._xphi(b) - codec._xphi(a)) + y * y * p
    return float(2.0 * np.sum(mse_half))


MUTANTS = [
    ("sign_fix", _sign_fix_smallest, [tc.check_sign_rule_hand]),
    ("eigenbasis", _eig_ascending, [tc.check_eigenbasis_tridiagonal_closed_form]),
    ("eigenbasis", _eig_transposed, [tc.check_gsvd_identity]),
    ("water_fill", _water_fill_half_rate, [tc.check_water_fill_bruteforce]),
    ("thresholds", _thresholds_shifted, [tc.check_quantize_bruteforce]),
    ("dequantize_channel", _dequant_no_offset, [tc.check_quantize_error_bound]),
    ("pack", _pack_msb_first, [tc.check_pack_hand_vectors]),
    ("reconstruct_exact", _reconstruct_wrong_side, [tc.check_parseval_and_dropped_energy]),
    ("attend_compressed", _attend_no_scale, [tc.check_attention_loops]),
    ("second_moment", _moment_centred, [tc.check_gsvd_identity]),
    ("_uniform_mse_slope", _slope_dropped_factor,
     [tc.check_delta_star_closed_form, tc.check_delta_star_max1960, tc.check_delta_star_stationary]),
    ("quantize_channel", _quantize_ties_down, [tc.check_quantize_bruteforce]),
    ("uniform_gaussian_mse", _mse_dropped_term, [tc.check_delta_star_stationary]),
]


@pytest.mark.parametrize("name,mutant,checks", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, mutant, checks):
    for check in checks:
        assert not _fails(check), f"{check.__name__} fails on the unmodified oracle"
    monkeypatch.setattr(codec, name, mutant)
    codec.delta_star.cache_clear()
    try:
        assert any(_fails(check) for check in checks), f"mutant {mutant.__name__} not caught"
    finally:
        monkeypatch.undo()
        codec.delta_star.cache_clear()


def _fwht_swapped(v):
    v = np.array(v, dtype=np.float64, copy=True)
    d = v.shape[-1]
    h = 1
    while h < d:
        for start in range(0, d, 2 * h):
            a = v[..., start:start + h].copy()
            b = v[..., start + h:start + 2 * h].copy()
            v[..., start:start + h] = a - b
            v[..., start + h:start + 2 * h] = a + b
        h *= 2
    return v


def _rotate_h_then_d(x, signs):
    x = np.asarray(x, np.float64)
    return rht.fwht(x) * np.asarray(signs, np.float64) / math.sqrt(x.shape[-1])


@pytest.mark.parametrize("name,mutant,check", [
    ("fwht", _fwht_swapped, tr.check_fwht_is_sylvester_hadamard),
    ("rotate", _rotate_h_then_d, tr.check_rotation_orthonormal_and_inverse),
])
def test_rht_mutant_is_caught(monkeypatch, name, mutant, check):
    assert not _fails(check)
    monkeypatch.setattr(rht, name, mutant)
    assert _fails(check)


# ------------------------------------------------------------ later rows
import test_oracle_qjl as tq  # noqa: E402
from oracle import qjl  # noqa: E402


def _append_one_bit_late(packed_old, n_old, codes_new, bits):
    full = _orig_append(packed_old, n_old, codes_new, bits)
    out = np.zeros_like(full)
    allbits = np.unpackbits(full, bitorder="little")
    shifted = np.concatenate([[0], allbits[:-1]])
    keep = n_old * int(np.asarray(bits, np.int64).sum())
    shifted[:keep] = allbits[:keep]
    return np.packbits(shifted, bitorder="little")[: out.shape[0]]


_orig_append = codec.append_pack
_orig_alloc = codec.allocate_bits


def _alloc_operational_as_rd(lam, total_bits, variant="greedy", param=0.0, max_bits=8):
    if variant == "operational":
        return codec.water_fill(lam, total_bits, max_bits)
    return _orig_alloc(lam, total_bits, variant, param, max_bits)


def _alloc_grouped_by_max(lam, total_bits, variant="greedy", param=0.0, max_bits=8):
    if variant == "grouped":
        G = int(param)
        lam_g = np.repeat(np.asarray(lam, np.float64).reshape(-1, G).max(axis=1), G)
        return _orig_alloc(lam_g, total_bits, variant, param, max_bits)
    return _orig_alloc(lam, total_bits, variant, param, max_bits)


_orig_corr = qjl.score_correction


def _corr_no_sqrt_pi_2(q, sketch, rnorm, S, n):
    return _orig_corr(q, sketch, rnorm, S, n) / math.sqrt(math.pi / 2.0)


def _check_append():
    tc.test_append_pack_equals_pack_of_all()


def _check_qjl_unbiased():
    tq.test_sketch_estimate_is_unbiased_on_real_codes()


_orig_softmax = codec.softmax_attention


def _softmax_extra_after_scale(q, khat, vhat, scale=None, extra=None):
    d = khat.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if extra is None:
        return _orig_softmax(q, khat, vhat, scale)
    return _orig_softmax(q, khat, vhat, scale, np.asarray(extra) / sc)


def _softmax_extra_negated(q, khat, vhat, scale=None, extra=None):
    return _orig_softmax(q, khat, vhat, scale, None if extra is None else -np.asarray(extra))


def _attend_eigen_raw_query(k_state, v_state, k_packed, sketch, rnorm, S, v_packed, n, q, scale=None):
    khat = codec.reconstruct_exact(k_state, k_packed, n)
    vhat = codec.reconstruct_exact(v_state, v_packed, n)
    extra = qjl.score_correction(np.asarray(q, np.float64), sketch, rnorm, S, n)
    return codec.softmax_attention(q, khat, vhat, scale, extra)


def _check_sketch_attention():
    tq.check_sketch_attention_converges_rht()
    tq.check_sketch_attention_converges_eigen(0.75)


@pytest.mark.parametrize("module,name,mutant,check", [
    (codec, "append_pack", _append_one_bit_late, _check_append),
    (codec, "allocate_bits", _alloc_operational_as_rd, tc.test_operational_allocation_is_optimal_by_brute_force),
    (codec, "allocate_bits", _alloc_grouped_by_max, tc.test_grouped_allocation_is_optimal_by_brute_force),
    (qjl, "score_correction", _corr_no_sqrt_pi_2, _check_qjl_unbiased),
    (codec, "softmax_attention", _softmax_extra_after_scale, _check_sketch_attention),
    (codec, "softmax_attention", _softmax_extra_negated, _check_sketch_attention),
    (qjl, "attend_compressed_eigen", _attend_eigen_raw_query, _check_sketch_attention),
], ids=["append_one_bit_late", "operational_as_rd", "grouped_by_max", "qjl_no_sqrt_pi_2",
        "extra_after_scale", "extra_negated", "eigen_sketch_raw_query"])
def test_later_row_mutant_is_caught(monkeypatch, module, name, mutant, check):
    assert not _fails(check)
    monkeypatch.setattr(module, name, mutant)
    assert _fails(check)
