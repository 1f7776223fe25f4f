"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (floating point tolerances are the ones the target states):
  - quantize+pack fed the oracle's fp32 coefficients and the oracle's state:
    byte-identical streams;
  - end-to-end codes (GPU calibration and projection): at most 1e-4 of codes
    differ, each by one level, and each at a decision threshold: the oracle's
    coefficient lies within the derived projection error of the threshold
    between the two codes (tests/parity_bounds.py); calibrated widths
    identical;
  - reconstruction relMSE within 1e-3 (relative) of the oracle's;
  - attention: max |o - o*| <= 2e-3 max |o*|.
"""
import math

import numpy as np
import pytest
import torch

import att_variants
import synth
from oracle import codec, rht
from parity_bounds import (assert_rht_code_diffs_at_boundaries, check_eigen_codes, decode_arith, decode_w16,
                           rht_rotation_eps)

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"


def dev_tensor(x32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).to(DEV)


def gpu_state(st) -> "stc.State":
    if st["xform"] == codec.XFORM_IDENTITY:
        return stc.state_init(None, st["lam"], st["bits"], st["steps"], xform=stc.XFORM_IDENTITY)
    return stc.state_init(st["U"], st["lam"], st["bits"], st["steps"], xform=stc.XFORM_EIGEN)


def codes(packed, bits, n):
    p = packed.cpu().numpy() if isinstance(packed, torch.Tensor) else packed
    return codec.unpack(p, bits, n)


def rel_err(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max() / np.abs(b).max())


def stream_case(cfg, n, head=0, kind=0, layer=0):
    w = synth.WORKLOADS[cfg]
    return w, synth.stream(w, layer, 0, head, kind, n=n)


# ------------------------------------------------------------ G1: bit-exact
G1_CASES = [
    ("cfg1_2.0", 1, 1000, 2.0, codec.XFORM_EIGEN, None),
    ("cfg2_4.0", 2, 4133, 4.0, codec.XFORM_EIGEN, None),
    ("cfg2_2.0", 2, 2600, 2.0, codec.XFORM_EIGEN, None),
    ("cfg2_1.33", 2, 2600, 1.33, codec.XFORM_EIGEN, None),
    ("identity_3.0", 2, 700, 3.0, codec.XFORM_IDENTITY, None),
    ("all8", 2, 300, 8.0, codec.XFORM_EIGEN, None),
    ("tiny_budget_odd", 2, 513, 0.1, codec.XFORM_EIGEN, None),
    ("uniform2", 2, 600, 2.0, codec.XFORM_EIGEN, np.full(128, 2, np.uint8)),
]


@pytest.mark.parametrize("name,cfg,n,avg,xform,bits", G1_CASES, ids=[c[0] for c in G1_CASES])
def test_quantize_pack_bitexact(name, cfg, n, avg, xform, bits):
    w, x = stream_case(cfg, n)
    n_c = min(w.n_calib, n)
    st = codec.calibrate_head(x, n_c, avg, bits=bits, xform=xform)
    c32 = codec.project(st, x).astype(np.float32)
    # edge values: exact thresholds, neighbours, NaN, +-Inf, huge
    kept = np.flatnonzero(st["bits"])
    for i, j in enumerate(kept[:40]):
        t = st["thresholds"][j]
        c32[0, j] = t[len(t) // 2]
        c32[1, j] = np.nextafter(t[0], np.float32(-np.inf))
        c32[2, j] = t[-1]
    c32[3, :] = np.nan
    c32[4, :] = np.inf
    c32[5, :] = -np.inf
    c32[6, :] = 3e38
    c32[7, :] = -0.0
    gst = gpu_state(st)
    got = stc.quantize_pack_f32(gst, torch.from_numpy(c32).to(DEV)).cpu().numpy()
    want = codec.quantize_pack(st, c32.astype(np.float64))
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


def test_quantize_pack_zero_step_channel():
    """A kept channel with a zero step (variance <= 0): every threshold is 0."""
    lam = np.linspace(2.0, 0.5, 128)
    lam[5] = 0.0
    bits = np.full(128, 8, np.uint8)
    st = codec.make_state(np.eye(128), lam, bits, codec.XFORM_IDENTITY)
    c = np.random.default_rng(50).standard_normal((300, 128)).astype(np.float32)
    c[:4, 5] = [0.0, -0.0, -1e-30, 1e-30]
    gst = stc.state_init(None, lam, bits, st["steps"], xform=stc.XFORM_IDENTITY)
    got = stc.quantize_pack_f32(gst, torch.from_numpy(c).to(DEV)).cpu().numpy()
    assert np.array_equal(got, codec.quantize_pack(st, c.astype(np.float64)))


def test_zero_tokens_is_a_noop():
    w, x = stream_case(2, 64)
    st = codec.calibrate_head(x, 64, 2.0)
    gst = gpu_state(st)
    packed, _ = stc.encode_kv(gst, dev_tensor(x[:0], "bf16"))
    assert packed.numel() == 0


# ------------------------------------------------------ G2: end-to-end codes
E2E_CASES = [(1, 4096, 2.0, "f32"), (2, 8192, 4.0, "bf16"), (2, 8192, 2.0, "bf16"), (2, 8192, 1.33, "bf16"),
             (5, 4500, 1.33, "bf16")]


@pytest.mark.parametrize("cfg,n,avg,dtype", E2E_CASES)
def test_encode_end_to_end(cfg, n, avg, dtype):
    w, x = stream_case(cfg, n, head=1, kind=1)
    n_c = w.n_calib
    xd = dev_tensor(x, dtype)
    gst = stc.calibrate_head(xd, n_c, avg)
    ost = codec.calibrate_head(x, n_c, avg)
    assert np.array_equal(gst.bits, ost["bits"])
    assert np.abs(gst.lam - ost["lam"]).max() <= 1e-11 * ost["lam"][0]
    assert np.abs(gst.basis() - ost["U"]).max() <= 1e-6
    packed, _ = stc.encode_kv(gst, xd)
    assert packed.numel() == codec.packed_bytes(ost["total_bits"], n)
    qg = codes(packed, ost["bits"], n)
    check_eigen_codes(qg, ost, x, gpu_state=gst)


def test_encode_with_oracle_state_isolates_projection():
    w, x = stream_case(2, 5000, head=2)
    ost = codec.calibrate_head(x, 2048, 2.0)
    packed, _ = stc.encode_kv(gpu_state(ost), dev_tensor(x, "bf16"))
    qg = codes(packed, ost["bits"], 5000)
    check_eigen_codes(qg, ost, x)


# ---------------------------------------------------------- G3: reconstruction
@pytest.mark.parametrize("cfg,n,avg,dtype", E2E_CASES + [(2, 777, 8.0, "bf16")])
def test_decode_matches_oracle(cfg, n, avg, dtype):
    w, x = stream_case(cfg, n, head=3)
    ost = codec.calibrate_head(x, min(w.n_calib, n), avg)
    po = codec.encode_kv(ost, x)
    out = stc.decode_kv(gpu_state(ost), torch.from_numpy(po).to(DEV), n,
                        dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    xg = out.float().cpu().numpy().astype(np.float64)
    xo = codec.decode_kv(ost, po, n, dtype)
    r_o, r_g = codec.rel_mse(x, xo), codec.rel_mse(x, xg)
    assert abs(r_g - r_o) <= 1e-3 * r_o, (r_g, r_o)
    # element-wise: one rounding step of the output dtype apart, plus the
    # error of the GPU's arithmetic before rounding (parity_bounds.decode_arith:
    # the bf16 pair of W, or for low budgets with bf16 output one fp16 pass)
    exact = codec.reconstruct_exact(ost, po, n)
    ulp = np.abs(exact) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
    arith = decode_arith(ost, dtype)
    assert np.all(np.abs(xg - xo) <= ulp + arith[None, :])


@pytest.mark.parametrize("scale,avg", [(2.0 ** -12, 2.0), (2.0 ** -12, 1.33), (1.0, 3.0)])
def test_decode_low_budget_bf16_pair(scale, avg):
    """bf16 output of records of at most 256 bits whose steps fall below
    2^-7 (tiny activations), or budgets above 2 bits: the bf16 hi / lo pair
    instead of the fp16 pass, for short records and long ones, against the
    oracle as above (the ragged last block included)."""
    w, x = stream_case(2, 3001, head=5)
    x = x * scale
    ost = codec.calibrate_head(x, 2048, avg)
    assert not decode_w16(ost, "bf16")
    po = codec.encode_kv(ost, x)
    xg = stc.decode_kv(gpu_state(ost), torch.from_numpy(po).to(DEV), 3001).float().cpu().numpy().astype(np.float64)
    xo = codec.decode_kv(ost, po, 3001, "bf16")
    exact = codec.reconstruct_exact(ost, po, 3001)
    assert np.all(np.abs(xg - xo) <= np.abs(exact) * 2.0 ** -7 + decode_arith(ost, "bf16")[None, :])


@pytest.mark.parametrize("cfg,n,avg,dtype", [(1, 4096, 2.0, "f32"), (2, 8192, 2.0, "bf16")])
def test_relmse_end_to_end(cfg, n, avg, dtype):
    w, x = stream_case(cfg, n, head=4, kind=1)
    xd = dev_tensor(x, dtype)
    gst = stc.calibrate_head(xd, w.n_calib, avg)
    packed, _ = stc.encode_kv(gst, xd)
    xg = stc.decode_kv(gst, packed, n, dtype=xd.dtype).float().cpu().numpy()
    ost = codec.calibrate_head(x, w.n_calib, avg)
    xo = codec.decode_kv(ost, codec.encode_kv(ost, x), n, dtype)
    r_o, r_g = codec.rel_mse(x, xo), codec.rel_mse(x, xg)
    assert abs(r_g - r_o) <= 1e-3 * r_o, (r_g, r_o)


# --------------------------------------------------------------- G4: attention
@pytest.mark.parametrize("cfg,n,avg", [(1, 4096, 2.0), (2, 32768, 2.0), (2, 9000, 4.0), (2, 3000, 1.33),
                                       (5, 2500, 1.33), (2, 1, 2.0), (2, 300, 2.0)])
def test_attention_matches_oracle(cfg, n, avg):
    w = synth.WORKLOADS[cfg]
    k = synth.stream(w, 0, 0, 1, 0, n=n)
    v = synth.stream(w, 0, 0, 1, 1, n=n)
    n_c = min(w.n_calib, n)
    ks, vs = codec.calibrate_head(k, n_c, avg), codec.calibrate_head(v, n_c, avg)
    kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
    q = synth.queries(w, 0, 0, 1)
    want = codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64))
    got = stc.attend_compressed(gpu_state(ks), gpu_state(vs), torch.from_numpy(kp).to(DEV),
                                torch.from_numpy(vp).to(DEV), n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    assert rel_err(got, want) <= 2e-3, rel_err(got, want)


def test_attention_near_uniform_long_context():
    """A query of small norm spreads the softmax over all 32768 tokens: every
    value code enters the weighted mean with about the same weight, so any
    rounding that grows with the offset the kernel adds to the codes shows up."""
    w = synth.WORKLOADS[2]
    n = 32768
    k = synth.stream(w, 0, 0, 6, 0, n=n)
    v = synth.stream(w, 0, 0, 6, 1, n=n)
    ks, vs = codec.calibrate_head(k, 2048, 2.0), codec.calibrate_head(v, 2048, 2.0)
    kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
    q = (1e-3 * synth.queries(w, 0, 0, 6)).astype(np.float32)
    want = codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64))
    got = stc.attend_compressed(gpu_state(ks), gpu_state(vs), torch.from_numpy(kp).to(DEV),
                                torch.from_numpy(vp).to(DEV), n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    assert rel_err(got, want) <= 2e-3, rel_err(got, want)


@pytest.mark.parametrize("avg", [7.8, 8.0])
def test_attention_wide_records_last_dims(avg):
    """Records of 998 / 1024 bits leave room for 12 waves per workgroup only
    (the a table is then built by 6 parts of 22 rows): a query that lives on
    the last latent dimensions checks that every row of U_K is summed."""
    w = synth.WORKLOADS[2]
    n = 3000
    k = synth.stream(w, 0, 0, 1, 0, n=n)
    v = synth.stream(w, 0, 0, 1, 1, n=n)
    ks, vs = codec.calibrate_head(k, 2048, avg), codec.calibrate_head(v, 2048, avg)
    kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
    rng = np.random.default_rng(5)
    q = np.zeros((4, 128), np.float32)
    q[:, 120:] = rng.standard_normal((4, 8)).astype(np.float32) * 3.0
    q = (q + 0.01 * rng.standard_normal((4, 128))).astype(np.float32)
    qr = (q.astype(np.float64) @ ks["U"].T).astype(np.float32)  # query along the last latent directions
    want = codec.attend_compressed(ks, vs, kp, vp, n, qr.astype(np.float64))
    got = stc.attend_compressed(gpu_state(ks), gpu_state(vs), torch.from_numpy(kp).to(DEV),
                                torch.from_numpy(vp).to(DEV), n, torch.from_numpy(qr).to(DEV)).cpu().numpy()
    assert rel_err(got, want) <= 2e-3, rel_err(got, want)


def test_attention_end_to_end_gpu_codes():
    w = synth.WORKLOADS[2]
    n = 8192
    k = synth.stream(w, 0, 0, 5, 0, n=n)
    v = synth.stream(w, 0, 0, 5, 1, n=n)
    kd, vd = dev_tensor(k, "bf16"), dev_tensor(v, "bf16")
    gk, gv = stc.calibrate_head(kd, 2048, 2.0), stc.calibrate_head(vd, 2048, 2.0)
    kp, _ = stc.encode_kv(gk, kd)
    vp, _ = stc.encode_kv(gv, vd)
    q = synth.queries(w, 0, 0, 5)
    got = stc.attend_compressed(gk, gv, kp, vp, n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    ks, vs = codec.calibrate_head(k, 2048, 2.0), codec.calibrate_head(v, 2048, 2.0)
    want = codec.attend_compressed(ks, vs, codec.encode_kv(ks, k), codec.encode_kv(vs, v), n, q.astype(np.float64))
    assert rel_err(got, want) <= 2e-3


def test_attention_batched_gqa7():
    w = synth.WORKLOADS[5]
    n, pairs = 2100, 3
    states, kps, vps, qs, wants = [], [], [], [], []
    for hd in range(pairs):
        k = synth.stream(w, 0, 0, hd, 0, n=n)
        v = synth.stream(w, 0, 0, hd, 1, n=n)
        ks, vs = codec.calibrate_head(k, 2048, 1.33), codec.calibrate_head(v, 2048, 1.33)
        kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
        q = synth.queries(w, 0, 0, hd)
        wants.append(codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64)))
        states += [gpu_state(ks), gpu_state(vs)]
        kps.append(kp); vps.append(vp); qs.append(q)
    arr = stc.StateArray(states)
    stride = stc.packed_bytes(arr.max_bits, n)
    kb = np.zeros((pairs, stride), np.uint8); vb = np.zeros((pairs, stride), np.uint8)
    for i in range(pairs):
        kb[i, :kps[i].shape[0]] = kps[i]; vb[i, :vps[i].shape[0]] = vps[i]
    kmap = torch.tensor([0, 2, 4], dtype=torch.int32, device=DEV)
    vmap = torch.tensor([1, 3, 5], dtype=torch.int32, device=DEV)
    out = stc.attend_compressed_batched(arr, kmap, vmap, torch.from_numpy(kb).to(DEV), torch.from_numpy(vb).to(DEV),
                                        n, torch.from_numpy(np.stack(qs)).to(DEV)).cpu().numpy()
    for i in range(pairs):
        assert rel_err(out[i], wants[i]) <= 2e-3


def test_attention_one_split_per_pair():
    """With a full round of pairs each pair gets one workgroup, which forms
    the output itself instead of leaving a partial for the merge kernel. 3072
    copies of one GQA-7 pair (one split each: whole rounds at 1, 3 or 4
    workgroups per CU) against the same pair alone
    (four splits and the merge): the copies agree bit for bit, and both paths
    agree with the oracle within 2e-3 (they differ from each other by the
    fp16 rounding of the softmax weights, which each split scales by its own
    running maximum)."""
    w = synth.WORKLOADS[5]
    n, pairs = 1000, 3072
    k = synth.stream(w, 0, 0, 2, 0, n=n)
    v = synth.stream(w, 0, 0, 2, 1, n=n)
    ks, vs = codec.calibrate_head(k, n, 1.33), codec.calibrate_head(v, n, 1.33)
    kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
    q = synth.queries(w, 0, 0, 2)
    want = codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64))
    arr = stc.StateArray([gpu_state(ks), gpu_state(vs)])
    stride = stc.packed_bytes(arr.max_bits, n)
    kb = torch.zeros((pairs, stride), dtype=torch.uint8, device=DEV)
    vb = torch.zeros((pairs, stride), dtype=torch.uint8, device=DEV)
    kb[:, :kp.shape[0]] = torch.from_numpy(kp).to(DEV)
    vb[:, :vp.shape[0]] = torch.from_numpy(vp).to(DEV)
    qd = torch.from_numpy(q).to(DEV)
    zeros = torch.zeros(pairs, dtype=torch.int32, device=DEV)
    many = stc.attend_compressed_batched(arr, zeros, zeros + 1, kb, vb, n,
                                         qd.unsqueeze(0).expand(pairs, -1, -1).contiguous()).cpu().numpy()
    one = stc.attend_compressed_batched(arr, zeros[:1], zeros[:1] + 1, kb[:1], vb[:1], n,
                                        qd.unsqueeze(0)).cpu().numpy()[0]
    assert np.all(many == many[0])
    assert rel_err(many[0], want) <= 2e-3, rel_err(many[0], want)
    assert rel_err(one, want) <= 2e-3, rel_err(one, want)


@pytest.mark.parametrize("case", att_variants.CASES, ids=lambda c: f"cfg{c[0]}-{c[1]:.3f}-g{c[2]}")
def test_attention_kernel_variants(case):
    """One case per instance of the packed-bit attention kernel (record
    widths, value-column counts and groups that select each one)."""
    cfg, avg, g, n, spec = case
    w = synth.WORKLOADS[cfg]
    k = synth.stream(w, 0, 0, 1, 0, n=n)
    v = synth.stream(w, 0, 0, 1, 1, n=n)
    n_c = min(w.n_calib, n)
    bits = None if spec is None else att_variants.widths(spec)
    ks, vs = codec.calibrate_head(k, n_c, avg, bits=bits), codec.calibrate_head(v, n_c, avg, bits=bits)
    kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
    q = np.random.default_rng(cfg * 100 + g).standard_normal((g, 128)).astype(np.float32)
    want = codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64))
    got = stc.attend_compressed(gpu_state(ks), gpu_state(vs), torch.from_numpy(kp).to(DEV),
                                torch.from_numpy(vp).to(DEV), n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    assert rel_err(got, want) <= 2e-3, rel_err(got, want)


def test_attention_zero_bit_streams():
    """KV heads whose K or V keeps no channel (a 0.0-bit budget: empty
    records): no K bits give equal scores, so the output is the mean of the
    reconstructed V; no V bits give a zero output. Mixed in one batched call
    with a regular pair; garbage-filled record bytes beyond each stream."""
    w = synth.WORKLOADS[2]
    n = 1700
    budgets = [(0.0, 2.0), (2.0, 0.0), (2.0, 2.0), (0.0, 0.0)]
    states, kps, vps, qs, wants = [], [], [], [], []
    for hd, (bk, bv) in enumerate(budgets):
        k = synth.stream(w, 0, 0, hd, 0, n=n)
        v = synth.stream(w, 0, 0, hd, 1, n=n)
        ks, vs = codec.calibrate_head(k, 1024, bk), codec.calibrate_head(v, 1024, bv)
        kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
        q = synth.queries(w, 0, 0, hd)
        wants.append(codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64)))
        states += [gpu_state(ks), gpu_state(vs)]
        kps.append(kp); vps.append(vp); qs.append(q)
    assert np.abs(wants[1]).max() == 0.0 and np.abs(wants[0] - wants[0][0]).max() == 0.0
    arr = stc.StateArray(states)
    stride = stc.packed_bytes(arr.max_bits, n)
    rng = np.random.default_rng(3)
    kb = rng.integers(0, 256, (len(budgets), stride), dtype=np.uint8)
    vb = rng.integers(0, 256, (len(budgets), stride), dtype=np.uint8)
    for i in range(len(budgets)):
        kb[i, :kps[i].shape[0]] = kps[i]; vb[i, :vps[i].shape[0]] = vps[i]
    kmap = torch.arange(0, 2 * len(budgets), 2, dtype=torch.int32, device=DEV)
    out = stc.attend_compressed_batched(arr, kmap, kmap + 1, torch.from_numpy(kb).to(DEV),
                                        torch.from_numpy(vb).to(DEV), n,
                                        torch.from_numpy(np.stack(qs)).to(DEV)).cpu().numpy()
    for i in range(len(budgets)):
        if np.abs(wants[i]).max() == 0.0:
            assert np.abs(out[i]).max() == 0.0, i
        else:
            assert rel_err(out[i], wants[i]) <= 2e-3, (i, rel_err(out[i], wants[i]))


@pytest.mark.parametrize("budget", [1.0, 2.0, 4.0, 8.0])
def test_attention_record_layouts_agree(budget):
    """Records of 32 * 2^s bits (here 128, 256, 512, 1024) are staged one per
    word-aligned slot; a state array that also holds a 1.33-bit state (170-bit
    records) makes the same pairs go through the packed stream layout. The
    two layouts feed the same codes to the same arithmetic: outputs agree
    bit for bit, and both match the oracle."""
    w = synth.WORKLOADS[2]
    n = 1700
    states, kps, vps, qs, wants = [], [], [], [], []
    for hd in range(3):
        k = synth.stream(w, 0, 0, hd, 0, n=n)
        v = synth.stream(w, 0, 0, hd, 1, n=n)
        ks, vs = codec.calibrate_head(k, 1024, budget), codec.calibrate_head(v, 1024, budget)
        assert int(ks["bits"].sum()) == int(vs["bits"].sum()) == round(128 * budget)
        kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
        q = synth.queries(w, 0, 0, hd)
        wants.append(codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64)))
        states += [gpu_state(ks), gpu_state(vs)]
        kps.append(kp); vps.append(vp); qs.append(q)
    odd = gpu_state(codec.calibrate_head(synth.stream(w, 0, 0, 7, 0, n=n), 1024, 1.33))
    outs = []
    for arr in (stc.StateArray(states), stc.StateArray(states + [odd])):
        stride = stc.packed_bytes(arr.max_bits, n)
        kb = np.zeros((3, stride), dtype=np.uint8)
        vb = np.zeros((3, stride), dtype=np.uint8)
        for i in range(3):
            kb[i, :kps[i].shape[0]] = kps[i]; vb[i, :vps[i].shape[0]] = vps[i]
        kmap = torch.arange(0, 6, 2, dtype=torch.int32, device=DEV)
        outs.append(stc.attend_compressed_batched(arr, kmap, kmap + 1, torch.from_numpy(kb).to(DEV),
                                                  torch.from_numpy(vb).to(DEV), n,
                                                  torch.from_numpy(np.stack(qs)).to(DEV)).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    for i in range(3):
        assert rel_err(outs[0][i], wants[i]) <= 2e-3, (i, rel_err(outs[0][i], wants[i]))


# ---------------------------------------------------------- batched codec
def test_batched_encode_decode_shared_states():
    w = synth.WORKLOADS[5]
    n = 3000
    xs = [synth.stream(w, 0, b, 0, 0, n=n) for b in range(4)]
    st0 = codec.calibrate_head(xs[0], 2048, 1.33)
    st1 = codec.calibrate_head(synth.stream(w, 0, 0, 1, 0, n=n), 2048, 1.33)
    arr = stc.StateArray([gpu_state(st0), gpu_state(st1)])
    smap = [0, 1, 1, 0]
    x = torch.stack([dev_tensor(xi, "bf16") for xi in xs])
    packed, _ = stc.encode_kv_batched(arr, x, torch.tensor(smap, dtype=torch.int32, device=DEV))
    dec = stc.decode_kv_batched(arr, packed, n, state_of_stream=torch.tensor(smap, dtype=torch.int32, device=DEV))
    for i, si in enumerate(smap):
        st = st0 if si == 0 else st1
        qg = codes(packed[i, :codec.packed_bytes(st["total_bits"], n)], st["bits"], n)
        check_eigen_codes(qg, st, xs[i])
        single, _ = stc.encode_kv(gpu_state(st), dev_tensor(xs[i], "bf16"))
        assert torch.equal(single, packed[i, :single.numel()])
        xo = codec.decode_kv(st, codec.pack(qg, st["bits"]), n, "bf16")
        xg = dec[i].float().cpu().numpy()
        assert abs(codec.rel_mse(xs[i], xg) - codec.rel_mse(xs[i], xo)) <= 1e-3 * codec.rel_mse(xs[i], xo)


# ----------------------------------------------------------------- RHT path
@pytest.fixture(scope="module")
def rht_codebook():
    c, _ = rht.lloyd_max(synth.sphere_coordinate_samples(100000))
    return rht.codebook_fp32(c)


@pytest.fixture(params=[stc.RHT_ENCODE_MFMA, stc.RHT_ENCODE_BUTTERFLY], ids=["mfma", "butterfly"])
def rht_kernel(request):
    """Runs the test once per Walsh-Hadamard encode kernel."""
    before = stc.get_rht_encode_kernel()
    stc.set_rht_encode_kernel(request.param)
    yield request.param
    stc.set_rht_encode_kernel(before)


@pytest.mark.parametrize("n", [1, 1000, 32768])
def test_rht_encode_matches_oracle(rht_codebook, rht_kernel, n):
    w = synth.WORKLOADS[3]
    x = synth.stream(w, 0, 0, 2, 0, n=n)
    signs = synth.random_signs(3, 0, 0, 2, 0)
    ost = rht.make_state(signs, rht_codebook)
    gst = stc.rht_state_init(signs, rht_codebook)
    packed, norms = stc.encode_kv(gst, dev_tensor(x, "bf16"))
    po, no = rht.encode_kv(ost, x)
    assert packed.numel() == po.shape[0]
    qg, qo = codes(packed, ost["bits"], n), codec.unpack(po, ost["bits"], n)
    y = rht.rotate(x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=1))[:, None], signs)
    assert_rht_code_diffs_at_boundaries(qg, qo, y, ost["thresholds"], rht_rotation_eps(x))
    # fp32 sum of 128 squares then sqrt: relative error <= (127/2 + 1) 2^-24
    ng = norms.cpu().numpy()
    assert np.all(np.abs(ng - no) <= 4e-6 * no)


def test_rht_decode_matches_oracle(rht_codebook):
    w = synth.WORKLOADS[3]
    n = 5000
    x = synth.stream(w, 0, 0, 3, 1, n=n)
    signs = synth.random_signs(3, 0, 0, 3, 1)
    ost = rht.make_state(signs, rht_codebook)
    po, no = rht.encode_kv(ost, x)
    gst = stc.rht_state_init(signs, rht_codebook)
    xg = stc.decode_kv(gst, torch.from_numpy(po).to(DEV), n, torch.from_numpy(no).to(DEV)).float().cpu().numpy()
    xo = rht.decode_kv(ost, po, no, n, "bf16")
    r_o, r_g = codec.rel_mse(x, xo), codec.rel_mse(x, xg)
    assert abs(r_g - r_o) <= 1e-3 * r_o
    exact = rht.reconstruct_exact(ost, po, no, n)
    assert np.all(np.abs(xg - xo) <= 1.01 * np.abs(exact) * 2.0 ** -7 + 1e-6 * np.abs(exact).max())


def test_rht_batched(rht_codebook, rht_kernel):
    w = synth.WORKLOADS[3]
    n = 2000
    xs = [synth.stream(w, 0, 0, h, 0, n=n) for h in range(3)]
    sg = [synth.random_signs(3, 0, 0, h, 0) for h in range(3)]
    arr = stc.StateArray([stc.rht_state_init(s, rht_codebook) for s in sg])
    packed, norms = stc.encode_kv_batched(arr, torch.stack([dev_tensor(xi, "bf16") for xi in xs]))
    dec = stc.decode_kv_batched(arr, packed, n, norms=norms)
    for i in range(3):
        ost = rht.make_state(sg[i], rht_codebook)
        po, no = rht.encode_kv(ost, xs[i])
        qg, qo = codes(packed[i], ost["bits"], n), codec.unpack(po, ost["bits"], n)
        y = rht.rotate(xs[i] / np.sqrt(np.sum(xs[i].astype(np.float64) ** 2, axis=1))[:, None], sg[i])
        assert_rht_code_diffs_at_boundaries(qg, qo, y, ost["thresholds"], rht_rotation_eps(xs[i]))
        r_o = codec.rel_mse(xs[i], rht.decode_kv(ost, po, no, n, "bf16"))
        assert abs(codec.rel_mse(xs[i], dec[i].float().cpu().numpy()) - r_o) <= 1e-3 * r_o


def test_attention_workspace_reused_across_shapes():
    """One workspace (garbage-filled, no initialisation needed) serves calls
    of different shapes in turn."""
    w = synth.WORKLOADS[2]
    cases = [(3, 7, 2100, 2.0), (1, 4, 5000, 4.0), (3, 7, 2100, 2.0), (2, 16, 700, 1.33)]
    need = max(stc.attend_workspace_bytes(pairs, g, n) for pairs, g, n, _ in cases)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(77)
    for pairs, g, n, avg in cases:
        states, kps, vps, qs, wants = [], [], [], [], []
        for hd in range(pairs):
            k = synth.stream(w, 0, 0, hd, 0, n=n)
            v = synth.stream(w, 0, 0, hd, 1, n=n)
            ks, vs = codec.calibrate_head(k, min(2048, n), avg), codec.calibrate_head(v, min(2048, n), avg)
            kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
            q = rng.standard_normal((g, 128)).astype(np.float32)
            wants.append(codec.attend_compressed(ks, vs, kp, vp, n, q.astype(np.float64)))
            states += [gpu_state(ks), gpu_state(vs)]
            kps.append(kp); vps.append(vp); qs.append(q)
        arr = stc.StateArray(states)
        stride = stc.packed_bytes(arr.max_bits, n)
        kb = np.zeros((pairs, stride), np.uint8); vb = np.zeros((pairs, stride), np.uint8)
        for i in range(pairs):
            kb[i, :kps[i].shape[0]] = kps[i]; vb[i, :vps[i].shape[0]] = vps[i]
        kmap = torch.arange(0, 2 * pairs, 2, dtype=torch.int32, device=DEV)
        vmap = kmap + 1
        out = stc.attend_compressed_batched(arr, kmap, vmap, torch.from_numpy(kb).to(DEV),
                                            torch.from_numpy(vb).to(DEV), n, torch.from_numpy(np.stack(qs)).to(DEV),
                                            ws=ws).cpu().numpy()
        for i in range(pairs):
            assert rel_err(out[i], wants[i]) <= 2e-3, (pairs, g, n, i, rel_err(out[i], wants[i]))


@pytest.mark.parametrize("n", [700, 200])
def test_out_of_range_state_map_entries(n):
    """A map entry outside [0, n_states) never codes a stream with another
    state: encode leaves its bytes untouched, decode writes NaN rows, attention
    NaN outputs; the other streams are unaffected and check_state_map names it.
    700 tokens: three splits per pair and the merge kernel; 200: one split,
    whose workgroup writes the output itself."""
    w = synth.WORKLOADS[2]
    xs = [synth.stream(w, 0, 0, h, kind, n=n) for h in range(2) for kind in (0, 1)]
    sts = [codec.calibrate_head(x, min(512, n), 2.0) for x in xs]
    arr = stc.StateArray([gpu_state(st) for st in sts])
    x = torch.stack([dev_tensor(xi, "bf16") for xi in xs])
    good = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=DEV)
    bad = torch.tensor([0, 1, 7, -1], dtype=torch.int32, device=DEV)
    stc.check_state_map(good, 4)
    with pytest.raises(stc.StcError):
        stc.check_state_map(bad, 4)
    ref, _ = stc.encode_kv_batched(arr, x, good)
    packed = torch.full_like(ref, 0x5A)
    stc.encode_kv_batched(arr, x, bad, packed=packed)
    assert torch.equal(packed[:2], ref[:2]) and torch.all(packed[2:] == 0x5A)
    dec = stc.decode_kv_batched(arr, ref, n, state_of_stream=bad)
    want = stc.decode_kv_batched(arr, ref, n, state_of_stream=good)
    assert torch.equal(dec[:2], want[:2]) and torch.all(torch.isnan(dec[2:].float()))
    q = torch.from_numpy(np.stack([synth.queries(w, 0, 0, h) for h in range(2)])).to(DEV)
    out = stc.attend_compressed_batched(arr, bad[0::2].contiguous(), bad[1::2].contiguous(), ref[0::2], ref[1::2],
                                        n, q).cpu().numpy()
    ok = stc.attend_compressed_batched(arr, good[0::2].contiguous(), good[1::2].contiguous(), ref[0::2], ref[1::2],
                                       n, q).cpu().numpy()
    assert np.array_equal(out[0], ok[0]) and np.all(np.isnan(out[1]))


def test_stream_copy():
    """The measurement helper's copy moves every byte (ragged tail of the
    grid-stride loop included)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    for nb in (16, 4096 + 48, (1 << 22) + 16 * 7):
        src = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=DEV, generator=g)
        dst = torch.zeros_like(src)
        stc.stream_copy(dst, src)
        assert torch.equal(dst, src)
