"""Batched calibration on the GPU: one call forms the second moment of every
stream (SPECTRA summary, "Metodologia" observation 3) and builds each
stream's state; every state must equal, byte for byte, the one the
single-stream call builds from the same rows (which the parity tests pin to
the oracle: widths identical, eigenvalues and basis within their bounds).
Covers both dtypes, K/V-interleaved rows (row stride 256) and a stream whose
rows hold a NaN (the call fails and names that stream)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"


def _same_state(arr, i, single):
    assert torch.equal(arr.blob[i], single.blob)
    a, b = arr.states[i], single
    assert a.total_bits == b.total_bits
    assert np.array_equal(a.bits, b.bits)
    assert np.array_equal(a.lam, b.lam) and np.array_equal(a.steps, b.steps)


@pytest.mark.parametrize("dtype,avg,n_streams", [("bf16", 2.0, 6), ("f32", 1.33, 3), ("bf16", 4.0, 1)])
def test_batched_equals_single(dtype, avg, n_streams):
    w = synth.WORKLOADS[2]
    n = 2500
    xs = np.stack([synth.stream(w, 0, 0, h // 2, h % 2, n=n) for h in range(n_streams)]).astype(np.float32)
    x = torch.from_numpy(xs).to(DEV)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    arr = stc.calibrate_heads_batched(x, w.n_calib, avg)
    assert arr.n == n_streams
    for i in range(n_streams):
        _same_state(arr, i, stc.calibrate_head(x[i], w.n_calib, avg))


def test_batched_interleaved_rows():
    """K and V of each head side by side (row stride 256): the K halves of
    three heads as one batch with stream stride n * 256."""
    w = synth.WORKLOADS[2]
    n = 2300
    kv = np.stack([np.concatenate([synth.stream(w, 0, 0, h, 0, n=n), synth.stream(w, 0, 0, h, 1, n=n)], axis=1)
                   for h in range(3)]).astype(np.float32)
    t = torch.from_numpy(kv).to(torch.bfloat16).to(DEV)       # [3][n][256]
    xk = t[:, :, :128]
    assert xk.stride() == (n * 256, 256, 1)
    arr = stc.calibrate_heads_batched(xk, w.n_calib, 2.0)
    for i in range(3):
        _same_state(arr, i, stc.calibrate_head(xk[i], w.n_calib, 2.0))


def test_batched_non_finite_stream_named():
    w = synth.WORKLOADS[2]
    xs = np.stack([synth.stream(w, 0, 0, h, 0, n=2048) for h in range(4)]).astype(np.float32)
    xs[2, 100, 7] = np.nan
    x = torch.from_numpy(xs).to(torch.bfloat16).to(DEV)
    with pytest.raises(stc.StcError, match="stream 2"):
        stc.calibrate_heads_batched(x, 2048, 2.0)


def test_batched_chunk_boundaries():
    """More streams than one host chunk (256): states on both sides of the
    chunk boundaries equal the single-stream call's."""
    w = synth.WORKLOADS[2]
    base = np.stack([synth.stream(w, 0, 0, h // 2, h % 2, n=2048) for h in range(6)]).astype(np.float32)
    xs = np.concatenate([base] * 50)           # 300 streams
    x = torch.from_numpy(xs).to(torch.bfloat16).to(DEV)
    arr = stc.calibrate_heads_batched(x, 2048, 2.0)
    assert arr.n == 300
    for i in (0, 255, 256, 299):
        _same_state(arr, i, stc.calibrate_head(x[i], 2048, 2.0))
