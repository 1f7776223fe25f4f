"""Append-only cache on the GPU (SPECTRA summary, "La Pipeline" steps 2-3:
tokens are quantized one at a time as they arrive and their records
appended): appends in chunks of any size give exactly the stream of one
encode of all tokens (the prefix invariant), and one generation step
(append the new K and V token, then attend) equals attention over the
fully encoded cache. Capacity past the stream is filled with garbage first:
the calls must not depend on it."""
import numpy as np
import pytest
import torch

import synth
from oracle import codec, rht
from parity_bounds import check_eigen_codes

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"
CHUNKS = [0, 1, 2, 33, 64, 65, 100, 517, 1000]


def dev_tensor(x32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).to(DEV)


def gpu_state(st):
    return stc.state_init(st["U"], st["lam"], st["bits"], st["steps"], xform=stc.XFORM_EIGEN)


def garbage(shape, dtype=torch.uint8):
    return torch.full(shape, 0xA5, dtype=dtype, device=DEV)


@pytest.mark.parametrize("cfg,avg,dtype", [(2, 4.0, "bf16"), (2, 2.0, "bf16"), (2, 1.33, "bf16"),
                                            (1, 2.0, "f32")])
def test_append_prefix_invariant(cfg, avg, dtype):
    w = synth.WORKLOADS[cfg]
    n = CHUNKS[-1]
    xs = [synth.stream(w, 0, 0, h, 0, n=n) for h in range(3)]
    sts = [codec.calibrate_head(xs[h], min(w.n_calib, n), avg) for h in range(2)]
    arr = stc.StateArray([gpu_state(s) for s in sts])
    smap = torch.tensor([0, 1, 0], dtype=torch.int32, device=DEV)
    x = torch.stack([dev_tensor(xi, dtype) for xi in xs])
    full, _ = stc.encode_kv_batched(arr, x, smap)
    buf = garbage(tuple(full.shape))
    for a, b in zip(CHUNKS[:-1], CHUNKS[1:]):
        stc.append_kv_batched(arr, x[:, a:b], a, buf, state_of_stream=smap)
    for i in range(3):
        st = sts[int(smap[i])]
        nb = codec.packed_bytes(st["total_bits"], n)
        assert torch.equal(buf[i, :nb], full[i, :nb]), i
        qg = codec.unpack(buf[i, :nb].cpu().numpy(), st["bits"], n)
        check_eigen_codes(qg, st, xs[i])


def test_append_one_token_at_a_time_matches_oracle_append():
    """Single-token appends, checked against the oracle's own append of the
    GPU's codes (F1 bit layout) as well as against one encode."""
    w = synth.WORKLOADS[2]
    n = 70
    x = synth.stream(w, 0, 0, 3, 1, n=n)
    st = codec.calibrate_head(synth.stream(w, 0, 0, 3, 1, n=4096), 2048, 1.33)   # B = 170
    arr = stc.StateArray([gpu_state(st)])
    xd = dev_tensor(x, "bf16")[None]
    full, _ = stc.encode_kv_batched(arr, xd)
    buf = garbage(tuple(full.shape))
    ref = codec.pack(np.zeros((0, 128), np.int64), st["bits"])
    for t in range(n):
        stc.append_kv_batched(arr, xd[:, t:t + 1], t, buf)
        q_t = codec.unpack(buf[0].cpu().numpy(), st["bits"], t + 1)[t:t + 1]
        ref = codec.append_pack(ref, t, q_t, st["bits"])
        nb = codec.packed_bytes(st["total_bits"], t + 1)
        assert np.array_equal(buf[0, :nb].cpu().numpy(), ref), t
    assert torch.equal(buf, full)


@pytest.fixture(scope="module")
def rht_codebook():
    c, _ = rht.lloyd_max(synth.sphere_coordinate_samples(100000))
    return rht.codebook_fp32(c)


@pytest.mark.parametrize("kernel", [stc.RHT_ENCODE_MFMA, stc.RHT_ENCODE_BUTTERFLY], ids=["mfma", "butterfly"])
def test_append_walsh_hadamard(rht_codebook, kernel):
    before = stc.get_rht_encode_kernel()
    stc.set_rht_encode_kernel(kernel)
    try:
        _append_walsh_hadamard(rht_codebook)
    finally:
        stc.set_rht_encode_kernel(before)


def _append_walsh_hadamard(rht_codebook):
    w = synth.WORKLOADS[3]
    n = CHUNKS[-1]
    xs = [synth.stream(w, 0, 0, h, 0, n=n) for h in range(2)]
    arr = stc.StateArray([stc.rht_state_init(synth.random_signs(3, 0, 0, h, 0), rht_codebook) for h in range(2)])
    x = torch.stack([dev_tensor(xi, "bf16") for xi in xs])
    full, fnorm = stc.encode_kv_batched(arr, x)
    buf = garbage(tuple(full.shape))
    norms = torch.full((2, n + 5), float("nan"), dtype=torch.float32, device=DEV)
    for a, b in zip(CHUNKS[:-1], CHUNKS[1:]):
        stc.append_kv_batched(arr, x[:, a:b], a, buf, norms=norms)
    assert torch.equal(buf, full)
    assert torch.equal(norms[:, :n], fnorm)


# The new tokens' records are formed inside the attention's first launch for
# bf16 rows; fp32 rows, groups above 8 and records above 512 bits take the
# appends' own launch. Both must equal an encode of the whole stream.
@pytest.mark.parametrize("n_old,g,dtype,budget", [(777, 4, "bf16", 2.0), (31, 7, "bf16", 2.0), (0, 4, "bf16", 2.0),
                                                  (500, 4, "f32", 2.0), (95, 8, "f32", 4.0),
                                                  (300, 16, "bf16", 2.0), (200, 4, "bf16", 6.0)])
def test_decode_step_equals_attention_over_full_cache(n_old, g, dtype, budget):
    w = synth.WORKLOADS[2]
    pairs = 3
    n = n_old + 1
    ks = [synth.stream(w, 0, 0, h, 0, n=n) for h in range(pairs)]
    vs = [synth.stream(w, 0, 0, h, 1, n=n) for h in range(pairs)]
    sk = [codec.calibrate_head(synth.stream(w, 0, 0, h, 0, n=2048), 2048, budget) for h in range(pairs)]
    sv = [codec.calibrate_head(synth.stream(w, 0, 0, h, 1, n=2048), 2048, budget) for h in range(pairs)]
    arr = stc.StateArray([gpu_state(s) for pair in zip(sk, sv) for s in pair])
    kmap = torch.arange(0, 2 * pairs, 2, dtype=torch.int32, device=DEV)
    vmap = kmap + 1
    kx = torch.stack([dev_tensor(k, dtype) for k in ks])
    vx = torch.stack([dev_tensor(v, dtype) for v in vs])
    rng = np.random.default_rng(5 + n_old)
    q = torch.from_numpy(rng.standard_normal((pairs, g, 128)).astype(np.float32)).to(DEV)
    stride = stc.packed_bytes(arr.max_bits, n)
    kbuf, vbuf = garbage((pairs, stride)), garbage((pairs, stride))
    if n_old:
        stc.append_kv_batched(arr, kx[:, :n_old], 0, kbuf, state_of_stream=kmap)
        stc.append_kv_batched(arr, vx[:, :n_old], 0, vbuf, state_of_stream=vmap)
    out = stc.decode_step_batched(arr, kmap, vmap, n_old, kx[:, n_old].contiguous(), vx[:, n_old].contiguous(),
                                  kbuf, vbuf, q)
    kfull, _ = stc.encode_kv_batched(arr, kx, kmap, packed=torch.zeros_like(kbuf))
    vfull, _ = stc.encode_kv_batched(arr, vx, vmap, packed=torch.zeros_like(vbuf))
    for i in range(pairs):
        nk = codec.packed_bytes(sk[i]["total_bits"], n)
        nv = codec.packed_bytes(sv[i]["total_bits"], n)
        assert torch.equal(kbuf[i, :nk], kfull[i, :nk]) and torch.equal(vbuf[i, :nv], vfull[i, :nv])
    want_gpu = stc.attend_compressed_batched(arr, kmap, vmap, kfull, vfull, n, q)
    assert torch.equal(out, want_gpu)
    qn = q.cpu().numpy().astype(np.float64)
    for i in range(pairs):
        kp = kfull[i, :codec.packed_bytes(sk[i]["total_bits"], n)].cpu().numpy()
        vp = vfull[i, :codec.packed_bytes(sv[i]["total_bits"], n)].cpu().numpy()
        want = codec.attend_compressed(sk[i], sv[i], kp, vp, n, qn[i])
        got = out[i].cpu().numpy()
        assert np.abs(got - want).max() <= 2e-3 * np.abs(want).max()
