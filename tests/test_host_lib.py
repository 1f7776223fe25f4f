"""CPU tests of libstc's host side: the library loads without a GPU, exports
every symbol include/stc.h declares, its host math agrees with the oracle
(independent code), and invalid arguments are rejected with the right status
before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import codec, rht

stc = pytest.importorskip("spectral_transform_codec_amd")
from spectral_transform_codec_amd import _abi  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "stc.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(stc_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = _abi.lib()
    names = _declared_symbols()
    assert len(names) >= 20
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(_abi.SIGNATURES), set(names) ^ set(_abi.SIGNATURES)


def test_debug_build_exports_every_declared_symbol():
    """The debug build (device index checks) has the same C ABI and says so;
    the release build has no checks and reports no flags."""
    D = _abi.load(_abi.DEBUG_LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(D, name), name
    assert D.stc_debug_build() == 1
    L = _abi.lib()
    assert L.stc_debug_build() == 0
    f = ctypes.c_uint32(7)
    assert L.stc_debug_flags(ctypes.byref(f), None) == _abi.STC_OK and f.value == 0
    assert L.stc_debug_flags(None, None) == _abi.STC_EINVAL


def test_sizes():
    assert stc.state_bytes() == 512 * 1024
    for b, n in [(170, 4096), (256, 1), (384, 32768), (13, 7), (0, 5)]:
        assert stc.packed_bytes(b, n) == codec.packed_bytes(b, n)
    assert stc.total_bits(1.33) == 170 and stc.total_bits(2.0) == 256


def test_delta_star_matches_oracle():
    for b in range(1, 9):
        assert abs(stc.delta_star(b) - codec.delta_star(b)) <= 1e-12 * codec.delta_star(b)
    assert np.isnan(stc.delta_star(0)) and np.isnan(stc.delta_star(9))


def test_water_fill_matches_oracle():
    rng = np.random.default_rng(40)
    for trial in range(30):
        d = int(rng.integers(1, 129))
        lam = rng.lognormal(0, 2, d)
        if trial % 3 == 0:
            lam[rng.integers(0, d, 3)] = 0.0
            lam[rng.integers(0, d, 2)] = -1e-12
        if trial % 5 == 0:
            lam = np.round(lam, 1)      # ties
        b_tot = int(rng.integers(0, 8 * d + 1))
        assert np.array_equal(stc.water_fill(lam, b_tot), codec.water_fill(lam, b_tot))
    with pytest.raises(stc.StcError):
        stc.water_fill(np.ones(4), 33)


def test_eigh_matches_oracle():
    for cfg, n_c in ((1, 1024), (2, 2048), (5, 2048)):
        w = synth.WORKLOADS[cfg]
        x = synth.stream(w, 0, 0, 1, 1, n=n_c)
        s = codec.second_moment(x, n_c)
        u, lam = stc.eigh(s)
        uo, lo = codec.eigenbasis(s)
        assert np.abs(lam - lo).max() <= 1e-12 * lo[0]
        assert np.abs(u - uo).max() <= 1e-8
        assert np.abs(u.T @ u - np.eye(128)).max() <= 1e-12


def test_eigh_closed_form():
    m = 16
    t = 2 * np.eye(m) - np.eye(m, k=1) - np.eye(m, k=-1)
    u, lam = stc.eigh(t)
    k = np.arange(1, m + 1)
    assert np.allclose(lam, np.sort(2 - 2 * np.cos(k * np.pi / (m + 1)))[::-1], atol=1e-13, rtol=0)


def test_lloyd_matches_oracle():
    y = synth.sphere_coordinate_samples(200000)
    c1, it1 = stc.lloyd_max(y)
    c2, it2 = rht.lloyd_max(y)
    assert abs(it1 - it2) <= 1
    assert np.abs(c1 - c2).max() <= 1e-12


# ------------------------------------------------ argument validation (no GPU)
def _status(call, *args):
    return int(getattr(_abi.lib(), call)(*args))


def test_invalid_arguments_rejected_before_device_work():
    L = _abi.lib()
    info = _abi.HeadInfo()
    lam = np.ones(128)
    bits = np.full(128, 2, np.uint8)
    P = ctypes.POINTER
    lam_p = lam.ctypes.data_as(P(ctypes.c_double))
    bits_p = bits.ctypes.data_as(P(ctypes.c_uint8))
    fake = ctypes.c_void_p(4096)           # aligned, never dereferenced on these paths
    # unsupported head dim
    assert L.stc_state_init(64, 1, None, lam_p, bits_p, None, ctypes.byref(info), fake, None) == _abi.STC_EUNSUPPORTED
    # EIGEN without a basis / IDENTITY with one
    assert L.stc_state_init(128, 0, None, lam_p, bits_p, None, ctypes.byref(info), fake, None) == _abi.STC_EINVAL
    # width > 8
    bad = bits.copy(); bad[3] = 9
    assert L.stc_state_init(128, 1, None, lam_p, bad.ctypes.data_as(P(ctypes.c_uint8)), None, ctypes.byref(info),
                            fake, None) == _abi.STC_EBUDGET
    # misaligned / NULL state
    assert L.stc_state_init(128, 1, None, lam_p, bits_p, None, ctypes.byref(info), ctypes.c_void_p(4100),
                            None) == _abi.STC_EINVAL
    assert L.stc_state_init(128, 1, None, lam_p, bits_p, None, ctypes.byref(info), None, None) == _abi.STC_EINVAL
    # calibrate: widths not summing to the budget; budget above 8 d
    assert L.stc_calibrate_head(128, 16, fake, _abi.BF16, 128, 1.0, bits_p, 0, ctypes.byref(info), fake,
                                None) == _abi.STC_EBUDGET
    assert L.stc_calibrate_head(128, 16, fake, _abi.BF16, 128, 9.0, None, 0, ctypes.byref(info), fake,
                                None) == _abi.STC_EBUDGET
    assert L.stc_calibrate_head(128, 16, fake, 7, 128, 2.0, None, 0, ctypes.byref(info), fake,
                                None) == _abi.STC_EUNSUPPORTED
    assert L.stc_calibrate_head(128, 0, fake, _abi.BF16, 128, 2.0, None, 0, ctypes.byref(info), fake,
                                None) == _abi.STC_EINVAL
    # rht: sign not +-1, codebook not increasing
    sg = np.ones(128, np.int8); sg[5] = 0
    cb = np.linspace(-1, 1, 8).astype(np.float32)
    assert L.stc_rht_state_init(128, sg.ctypes.data_as(P(ctypes.c_int8)), cb.ctypes.data_as(P(ctypes.c_float)),
                                ctypes.byref(info), fake, None) == _abi.STC_EINVAL
    sg[5] = 1
    cb2 = cb[::-1].copy()
    assert L.stc_rht_state_init(128, sg.ctypes.data_as(P(ctypes.c_int8)), cb2.ctypes.data_as(P(ctypes.c_float)),
                                ctypes.byref(info), fake, None) == _abi.STC_EINVAL
    # encode/decode: bad infos, dtype, strides, alignment
    good = _abi.HeadInfo(); good.d = 128; good.xform = 0; good.total_bits = 256
    assert L.stc_encode_kv(ctypes.byref(good), fake, 10, fake, 5, 128, fake, None, None) == _abi.STC_EUNSUPPORTED
    assert L.stc_encode_kv(ctypes.byref(good), fake, 10, fake, _abi.BF16, 100, fake, None, None) == _abi.STC_EINVAL
    assert L.stc_encode_kv(ctypes.byref(good), fake, 10, ctypes.c_void_p(4098), _abi.BF16, 128, fake, None,
                           None) == _abi.STC_EINVAL
    assert L.stc_encode_kv(ctypes.byref(good), fake, -1, fake, _abi.BF16, 128, fake, None, None) == _abi.STC_EINVAL
    bad_info = _abi.HeadInfo(); bad_info.d = 64
    assert L.stc_decode_kv(ctypes.byref(bad_info), fake, 10, fake, None, fake, _abi.BF16, 128,
                           None) == _abi.STC_EUNSUPPORTED
    rht_info = _abi.HeadInfo(); rht_info.d = 128; rht_info.xform = 2; rht_info.total_bits = 384
    assert L.stc_encode_kv(ctypes.byref(rht_info), fake, 10, fake, _abi.BF16, 128, fake, None,
                           None) == _abi.STC_EINVAL          # RHT needs norms
    # batched: packed stride too small, mixed families
    infos = (_abi.HeadInfo * 2)(good, rht_info)
    assert L.stc_encode_kv_batched(fake, 2, None, infos, 2, 16, fake, _abi.BF16, 128, 2048, fake, 512, fake,
                                   None) == _abi.STC_EINVAL
    infos2 = (_abi.HeadInfo * 1)(good)
    assert L.stc_encode_kv_batched(fake, 1, None, infos2, 2, 100, fake, _abi.BF16, 128, 128 * 100, fake, 16,
                                   None, None) == _abi.STC_EINVAL
    # attention: group out of range, workspace too small, RHT states
    assert L.stc_attend_compressed(ctypes.byref(good), fake, ctypes.byref(good), fake, 100, fake, fake, 17, fake,
                                   fake, 0.1, fake, 1 << 20, None) == _abi.STC_EUNSUPPORTED
    assert L.stc_attend_compressed(ctypes.byref(good), fake, ctypes.byref(good), fake, 100, fake, fake, 4, fake,
                                   fake, 0.1, fake, 16, None) == _abi.STC_EWORKSPACE
    assert L.stc_attend_compressed(ctypes.byref(rht_info), fake, ctypes.byref(good), fake, 100, fake, fake, 4,
                                   fake, fake, 0.1, fake, 1 << 20, None) == _abi.STC_EUNSUPPORTED
    assert L.stc_last_error()
    assert L.stc_status_str(_abi.STC_EBUDGET) == b"bit budget"


def test_allocation_variants_match_oracle():
    """The library's allocation variants equal the oracle's on random and
    structured spectra (written independently on each side)."""
    rng = np.random.default_rng(70)
    spectra = [np.arange(1, 129, dtype=np.float64) ** -a for a in (0.8, 1.2, 2.0)]
    spectra.append(np.sort(rng.exponential(1.0, 128))[::-1])
    spectra.append(np.concatenate([np.linspace(3.0, 1.0, 20), np.full(108, 2e-4)]))
    z = np.sort(rng.exponential(1.0, 128))[::-1]
    z[100:] = 0.0
    spectra.append(z)
    cases = [("greedy", 0), ("operational", 0), ("grouped", 4), ("grouped", 8), ("floor", 1), ("gap", 50.0)]
    for lam in spectra:
        for B in (170, 256, 512):
            for variant, param in cases:
                want = codec.allocate_bits(lam, B, variant, param)
                got = stc.allocate_bits(lam, B, variant, param)
                assert np.array_equal(got, want), (variant, param, B)



def test_check_state_map_validates_arguments_without_device_work():
    L = _abi.lib()
    assert L.stc_check_state_map(None, 0, 4, None) == _abi.STC_OK
    assert L.stc_check_state_map(None, 3, 4, None) == _abi.STC_EINVAL
    assert b"NULL map" in L.stc_last_error()
    assert L.stc_check_state_map(None, -1, 4, None) == _abi.STC_EINVAL


def test_rht_encode_kernel_choice():
    """The Walsh-Hadamard encode kernel choice takes the two declared kinds and
    refuses others, leaving the previous choice in place."""
    L = _abi.lib()
    before = L.stc_get_rht_encode_kernel()
    try:
        assert L.stc_set_rht_encode_kernel(1) == _abi.STC_OK
        assert L.stc_get_rht_encode_kernel() == 1
        assert L.stc_set_rht_encode_kernel(2) == _abi.STC_EINVAL
        assert L.stc_set_rht_encode_kernel(-1) == _abi.STC_EINVAL
        assert L.stc_get_rht_encode_kernel() == 1
        assert L.stc_set_rht_encode_kernel(0) == _abi.STC_OK
        assert L.stc_get_rht_encode_kernel() == 0
    finally:
        L.stc_set_rht_encode_kernel(before)


def test_batched_calibration_validates_arguments_without_device_work():
    L = _abi.lib()
    infos = (_abi.HeadInfo * 4)()
    fake = ctypes.c_void_p(4096)           # aligned, never dereferenced on these paths
    call = L.stc_calibrate_heads_batched
    # head dim, dtype, negative counts, budget
    assert call(64, 4, 2048, fake, _abi.BF16, 128, 2048 * 128, 2.0, 1, infos, fake, None) == _abi.STC_EUNSUPPORTED
    assert call(128, 4, 2048, fake, 7, 128, 2048 * 128, 2.0, 1, infos, fake, None) == _abi.STC_EUNSUPPORTED
    assert call(128, -1, 2048, fake, _abi.BF16, 128, 2048 * 128, 2.0, 1, infos, fake, None) == _abi.STC_EINVAL
    assert call(128, 4, 0, fake, _abi.BF16, 128, 2048 * 128, 2.0, 1, infos, fake, None) == _abi.STC_EINVAL
    assert call(128, 4, 2048, fake, _abi.BF16, 128, 2048 * 128, 9.0, 1, infos, fake, None) == _abi.STC_EBUDGET
    # stream stride that does not cover n_calib rows; misaligned rows; NULL summaries
    assert call(128, 4, 2048, fake, _abi.BF16, 128, 2047 * 128, 2.0, 1, infos, fake, None) == _abi.STC_EINVAL
    assert call(128, 4, 2048, ctypes.c_void_p(4098), _abi.BF16, 128, 2048 * 128, 2.0, 1, infos, fake,
                None) == _abi.STC_EINVAL
    assert call(128, 4, 2048, fake, _abi.BF16, 128, 2048 * 128, 2.0, 1, None, fake, None) == _abi.STC_EINVAL
    # no streams: nothing to do
    assert call(128, 0, 2048, fake, _abi.BF16, 128, 0, 2.0, 1, infos, fake, None) == _abi.STC_OK


def test_stream_copy_validates_arguments_without_device_work():
    L = _abi.lib()
    fake = ctypes.c_void_p(4096)
    assert L.stc_stream_copy(fake, fake, 0, None) == _abi.STC_OK
    assert L.stc_stream_copy(fake, fake, 24, None) == _abi.STC_EINVAL
    assert L.stc_stream_copy(fake, fake, -16, None) == _abi.STC_EINVAL
    assert L.stc_stream_copy(ctypes.c_void_p(4100), fake, 32, None) == _abi.STC_EINVAL
    assert L.stc_stream_copy(None, fake, 32, None) == _abi.STC_EINVAL
