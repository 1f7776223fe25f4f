"""Strided token rows on the GPU: K and V of a head side by side in one
buffer (row stride 256 values, as a fused K/V projection writes them), both
dtypes. Tokens are read where the model wrote them (SPECTRA summary, "La
Pipeline di SPECTRA" step 3: tokens are projected as they arrive), so
calibration, encode and decode take the row stride as given; results equal
those of contiguous rows and meet the oracle bars (widths identical, codes
at thresholds, relMSE within 1e-3 relative, decode written back into the
strided buffer without touching the other half)."""
import numpy as np
import pytest
import torch

import synth
from oracle import codec
from parity_bounds import check_eigen_codes

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"


def interleaved(k, v, dtype):
    kv = np.concatenate([k, v], axis=1).astype(np.float32)       # [n][256]
    t = torch.from_numpy(np.ascontiguousarray(kv))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).to(DEV)


@pytest.mark.parametrize("cfg,n,avg,dtype", [(2, 5000, 2.0, "bf16"), (2, 4133, 1.33, "bf16"),
                                             (1, 4096, 2.0, "f32")])
def test_kv_interleaved_rows(cfg, n, avg, dtype):
    w = synth.WORKLOADS[cfg]
    k = synth.stream(w, 0, 0, 2, 0, n=n)
    v = synth.stream(w, 0, 0, 2, 1, n=n)
    kv = interleaved(k, v, dtype)
    assert kv.stride(0) == 256
    xk, xv = kv[:, :128], kv[:, 128:]
    n_c = w.n_calib
    gk, gv = stc.calibrate_head(xk, n_c, avg), stc.calibrate_head(xv, n_c, avg)
    ok, ov = codec.calibrate_head(k, n_c, avg), codec.calibrate_head(v, n_c, avg)
    assert np.array_equal(gk.bits, ok["bits"]) and np.array_equal(gv.bits, ov["bits"])
    # the same calibration as contiguous rows
    ck = stc.calibrate_head(xk.contiguous(), n_c, avg)
    assert np.array_equal(ck.basis(), gk.basis()) and np.array_equal(ck.lam, gk.lam)
    kp, _ = stc.encode_kv(gk, xk)
    vp, _ = stc.encode_kv(gv, xv)
    assert torch.equal(kp, stc.encode_kv(gk, xk.contiguous())[0])
    check_eigen_codes(codec.unpack(kp.cpu().numpy(), ok["bits"], n), ok, k, gpu_state=gk)
    check_eigen_codes(codec.unpack(vp.cpu().numpy(), ov["bits"], n), ov, v, gpu_state=gv)
    # decode into the strided buffer: K half first, V half untouched, then V
    out = torch.full_like(kv, 7.0)
    stc.decode_kv(gk, kp, n, out=out[:, :128])
    assert torch.all(out[:, 128:] == 7.0)
    stc.decode_kv(gv, vp, n, out=out[:, 128:])
    dec = out.float().cpu().numpy().astype(np.float64)
    for half, x, st, packed in ((0, k, ok, kp), (1, v, ov, vp)):
        xg = dec[:, 128 * half:128 * half + 128]
        contig = stc.decode_kv(gk if half == 0 else gv, packed, n, dtype=kv.dtype).float().cpu().numpy()
        assert np.array_equal(xg, contig.astype(np.float64))
        xo = codec.decode_kv(st, codec.encode_kv(st, x), n, dtype)
        r_o, r_g = codec.rel_mse(x, xo), codec.rel_mse(x, xg)
        assert abs(r_g - r_o) <= 1e-3 * r_o, (half, r_g, r_o)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_interleaved_rows_batched(dtype):
    """Several heads' K halves of [S][n][256] buffers in one batched encode and
    decode (row stride 256, stream stride n * 256)."""
    w = synth.WORKLOADS[2]
    n, S, avg = 3000, 3, 2.0
    ks = [synth.stream(w, 0, 0, h, 0, n=n) for h in range(S)]
    vs = [synth.stream(w, 0, 0, h, 1, n=n) for h in range(S)]
    buf = torch.stack([interleaved(ks[h], vs[h], dtype) for h in range(S)])
    x = buf[:, :, :128]
    assert x.stride(1) == 256 and x.stride(0) == n * 256
    osts = [codec.calibrate_head(ks[h], 2048, avg) for h in range(S)]
    arr = stc.StateArray([stc.state_init(st["U"], st["lam"], st["bits"], st["steps"]) for st in osts])
    packed, _ = stc.encode_kv_batched(arr, x)
    ref, _ = stc.encode_kv_batched(arr, x.contiguous())
    assert torch.equal(packed, ref)
    out = torch.full_like(buf, -3.0)
    stc.decode_kv_batched(arr, packed, n, out=out[:, :, :128])
    assert torch.all(out[:, :, 128:] == -3.0)
    dec = out[:, :, :128].float().cpu().numpy().astype(np.float64)
    for h in range(S):
        st = osts[h]
        qg = codec.unpack(packed[h].cpu().numpy(), st["bits"], n)
        check_eigen_codes(qg, st, ks[h])
        xo = codec.decode_kv(st, codec.pack(qg, st["bits"]), n, dtype)
        assert abs(codec.rel_mse(ks[h], dec[h]) - codec.rel_mse(ks[h], xo)) <= 1e-3 * codec.rel_mse(ks[h], xo)
