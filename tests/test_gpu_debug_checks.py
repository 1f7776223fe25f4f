"""The debug build on the GPU (libstc_debug.so: every kernel family checks
the LDS stream words, record byte ranges, staging offsets and value rows it
computes, and records a failed check instead of making the access):
representative calls of each family set no check bit and give exactly the
bytes the release library gives (the checks change no arithmetic). Covers
encode, append and decode of records in the slot layout (2.0 bits) and the
packed stream (1.33 bits), attention and the fused generation step, both
Walsh-Hadamard encode kernels, its decode and attention over its cache."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")
from spectral_transform_codec_amd import _abi  # noqa: E402

DEV = "cuda"


def _flags():
    f = ctypes.c_uint32(0)
    torch.cuda.synchronize()
    assert _abi.lib().stc_debug_flags(ctypes.byref(f), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    return f.value


@pytest.fixture(scope="module")
def inputs():
    w = synth.WORKLOADS[2]
    n = 3001
    xs = np.stack([synth.stream(w, 0, 0, h // 2, h % 2, n=n) for h in range(4)]).astype(np.float32)
    x = torch.from_numpy(xs).to(DEV).to(torch.bfloat16)
    arrays = {b: stc.calibrate_heads_batched(x, 2048, b) for b in (2.0, 1.33)}
    cb = stc.lloyd_max(synth.sphere_coordinate_samples(100000))[0].astype(np.float32)
    rht = stc.StateArray([stc.rht_state_init(synth.random_signs(3, 0, 0, h, 0), cb) for h in range(4)])
    rng = np.random.default_rng(3)
    q = torch.from_numpy(rng.standard_normal((2, 4, 128)).astype(np.float32)).to(DEV)
    return x, arrays, rht, q


def _run(inputs):
    x, arrays, rht, q = inputs
    n = x.shape[1]
    kmap = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    vmap = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    out = {}
    for b, arr in arrays.items():
        packed, _ = stc.encode_kv_batched(arr, x)
        out[f"enc{b}"] = packed
        out[f"dec{b}"] = stc.decode_kv_batched(arr, packed, n)
        app = torch.full_like(packed, 0xA5)
        for a0, a1 in ((0, 1000), (1000, 2999)):
            stc.append_kv_batched(arr, x[:, a0:a1], a0, app)
        kp, vp = app[0::2].contiguous(), app[1::2].contiguous()
        out[f"step{b}"] = stc.decode_step_batched(arr, kmap, vmap, 2999, x[0::2, 2999].contiguous(),
                                                  x[1::2, 2999].contiguous(), kp, vp, q)
        out[f"app{b}"] = torch.cat([kp, vp])
        out[f"att{b}"] = stc.attend_compressed_batched(arr, kmap, vmap, packed[0::2], packed[1::2], n, q)
    before = stc.get_rht_encode_kernel()
    try:
        for kind in (stc.RHT_ENCODE_MFMA, stc.RHT_ENCODE_BUTTERFLY):
            stc.set_rht_encode_kernel(kind)
            rp, rn = stc.encode_kv_batched(rht, x)
            out[f"rht_enc{kind}"] = torch.cat([rp.flatten(), rn.flatten().view(torch.uint8)])
    finally:
        stc.set_rht_encode_kernel(before)
    out["rht_dec"] = stc.decode_kv_batched(rht, rp, n, norms=rn)
    out["rht_att"] = stc.attend_rht_batched(rht, kmap, vmap, rp[0::2].contiguous(), rn[0::2].contiguous(),
                                            rp[1::2].contiguous(), rn[1::2].contiguous(), n, q)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def test_debug_build_checks_pass_and_match_release(inputs):
    rel = _run(inputs)
    with _abi.use_library(_abi.DEBUG_LIB_PATH) as L:
        assert L.stc_debug_build() == 1
        _flags()  # (start from a clear word)
        dbg = _run(inputs)
        assert _flags() == 0
    for k in rel:
        assert torch.equal(rel[k], dbg[k]), k
