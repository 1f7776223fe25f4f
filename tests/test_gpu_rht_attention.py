"""Decode-step attention over Walsh-Hadamard caches on the GPU against the
oracle (exact fp64 reconstructions, the same softmax core as the eigen
cache): max |o - o*| <= 2e-3 max |o*|."""
import numpy as np
import pytest
import torch

import synth
from oracle import rht

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"


@pytest.fixture(scope="module")
def cb():
    c, _ = rht.lloyd_max(synth.sphere_coordinate_samples(100000))
    return rht.codebook_fp32(c)


def rel_err(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max() / np.abs(b).max())


def run_case(cb, n, g, pairs, amp=1.0, gpu_codes=False):
    w = synth.WORKLOADS[3]
    ks_sig = [synth.random_signs(3, 0, 0, h, 0) for h in range(pairs)]
    vs_sig = [synth.random_signs(3, 0, 0, h, 1) for h in range(pairs)]
    kx = [amp * synth.stream(w, 0, 0, h, 0, n=n) for h in range(pairs)]
    vx = [amp * synth.stream(w, 0, 0, h, 1, n=n) for h in range(pairs)]
    arr = stc.StateArray([stc.rht_state_init(s, cb) for pair in zip(ks_sig, vs_sig) for s in pair])
    kmap = torch.arange(0, 2 * pairs, 2, dtype=torch.int32, device=DEV)
    vmap = kmap + 1
    stride = stc.packed_bytes(384, n)
    if gpu_codes:
        x = torch.stack([torch.from_numpy(t.astype(np.float32)) for pair in zip(kx, vx) for t in pair]).to(
            DEV, torch.bfloat16)
        packed, norms = stc.encode_kv_batched(arr, x)
        kp, vp = packed[0::2], packed[1::2]
        kn, vn = norms[0::2], norms[1::2]
        kp_np, vp_np = kp.cpu().numpy(), vp.cpu().numpy()
        kn_np, vn_np = kn.cpu().numpy(), vn.cpu().numpy()
    else:
        kp_np = np.zeros((pairs, stride), np.uint8); vp_np = np.zeros((pairs, stride), np.uint8)
        kn_np = np.zeros((pairs, n), np.float32); vn_np = np.zeros((pairs, n), np.float32)
        for h in range(pairs):
            st_k, st_v = rht.make_state(ks_sig[h], cb), rht.make_state(vs_sig[h], cb)
            p, nn = rht.encode_kv(st_k, kx[h]); kp_np[h, :p.shape[0]] = p; kn_np[h] = nn
            p, nn = rht.encode_kv(st_v, vx[h]); vp_np[h, :p.shape[0]] = p; vn_np[h] = nn
        kp, vp = torch.from_numpy(kp_np).to(DEV), torch.from_numpy(vp_np).to(DEV)
        kn, vn = torch.from_numpy(kn_np).to(DEV), torch.from_numpy(vn_np).to(DEV)
    rng = np.random.default_rng(40 + n + g)
    q = rng.standard_normal((pairs, g, 128)).astype(np.float32)
    out = stc.attend_rht_batched(arr, kmap, vmap, kp, kn, vp, vn, n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    for h in range(pairs):
        st_k, st_v = rht.make_state(ks_sig[h], cb), rht.make_state(vs_sig[h], cb)
        want = rht.attend_compressed(st_k, st_v, kp_np[h], kn_np[h], vp_np[h], vn_np[h], n, q[h].astype(np.float64))
        assert rel_err(out[h], want) <= 2e-3, (h, rel_err(out[h], want))


@pytest.mark.parametrize("n,g", [(1, 4), (300, 4), (3000, 7), (2049, 16)])
def test_rht_attention_oracle_codes(cb, n, g):
    run_case(cb, n, g, pairs=3)


def test_rht_attention_gpu_codes_full_length(cb):
    run_case(cb, 32768, 4, pairs=2, gpu_codes=True)


def test_rht_attention_large_norms(cb):
    """Value norms far above the fp16 range: P is scaled per block."""
    run_case(cb, 1000, 4, pairs=2, amp=3e4)
