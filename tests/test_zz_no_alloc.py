"""The attention entry point that allocates nothing (for callers that cannot
call hipMalloc): through the C ABI, its outputs equal those of
stc_attend_compressed_batched with a caller workspace, bit for bit, on two
calls in a row (the second smaller, so the shared scratch holds the first
call's partials when it starts); a shape needing more partials than the
scratch holds is refused before any device work."""
import numpy as np
import pytest
import torch

import synth
from oracle import codec

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"


def _case(pairs, n, avg, g, seed):
    w = synth.WORKLOADS[2]
    states, kps, vps = [], [], []
    for hd in range(pairs):
        k = synth.stream(w, 0, 0, hd, 0, n=n)
        v = synth.stream(w, 0, 0, hd, 1, n=n)
        ks, vs = codec.calibrate_head(k, min(2048, n), avg), codec.calibrate_head(v, min(2048, n), avg)
        kps.append(codec.encode_kv(ks, k))
        vps.append(codec.encode_kv(vs, v))
        for st in (ks, vs):
            states.append(stc.state_init(st["U"], st["lam"], st["bits"], st["steps"], xform=stc.XFORM_EIGEN))
    arr = stc.StateArray(states)
    stride = stc.packed_bytes(arr.max_bits, n)
    kb = np.zeros((pairs, stride), np.uint8)
    vb = np.zeros((pairs, stride), np.uint8)
    for i in range(pairs):
        kb[i, :kps[i].shape[0]] = kps[i]
        vb[i, :vps[i].shape[0]] = vps[i]
    q = np.random.default_rng(seed).standard_normal((pairs, g, 128)).astype(np.float32)
    kmap = torch.arange(0, 2 * pairs, 2, dtype=torch.int32, device=DEV)
    return (arr, kmap, kmap + 1, torch.from_numpy(kb).to(DEV), torch.from_numpy(vb).to(DEV), n,
            torch.from_numpy(q).to(DEV))


def test_noalloc_equals_workspace_entry_point_twice():
    first = _case(4, 9000, 2.0, 7, 11)
    second = _case(2, 1300, 1.33, 4, 12)     # smaller: starts on the first call's partials
    for arr, km, vm, kp, vp, n, q in (first, second):
        want = stc.attend_compressed_batched(arr, km, vm, kp, vp, n, q)
        out = torch.full_like(want, float("nan"))
        stc.attend_compressed_batched_noalloc(arr, km, vm, kp, vp, n, q, out)
        torch.cuda.synchronize()
        assert torch.equal(out, want)


def test_noalloc_refuses_a_shape_beyond_the_scratch():
    """4096 KV heads of one token with 16 query heads need more partials than
    the scratch holds: STC_EWORKSPACE, and nothing is written. (The buffers
    are real and the maps valid, so even a launch would stay in bounds.)"""
    arr, _, _, _, _, _, _ = _case(1, 64, 2.0, 4, 13)
    pairs, g = 4096, 16
    assert stc.attend_workspace_bytes(pairs, g, 1) > stc.attend_noalloc_max_bytes()
    km = torch.zeros(pairs, dtype=torch.int32, device=DEV)
    vm = torch.ones(pairs, dtype=torch.int32, device=DEV)
    kp = torch.zeros((pairs, stc.packed_bytes(arr.max_bits, 1)), dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    q = torch.zeros((pairs, g, 128), dtype=torch.float32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(stc.StcError):
        stc.attend_compressed_batched_noalloc(arr, km, vm, kp, vp, 1, q, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
