"""Allocation variants on the GPU: widths from each variant (grouped,
floor, spectral-gap pruning, operational) drive the same kernels; encode and
decode meet the end-to-end bars against the oracle with the same widths
(codes: <= 1e-4 differ, each by one level; relMSE within 1e-3 relative)."""
import numpy as np
import pytest
import torch

import synth
from oracle import codec
from parity_bounds import check_eigen_codes

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"
VARIANTS = [("operational", 0), ("grouped", 4), ("grouped", 16), ("floor", 1), ("gap", 20.0)]


@pytest.mark.parametrize("variant,param", VARIANTS)
@pytest.mark.parametrize("avg", [2.0, 1.33])
def test_variant_widths_end_to_end(variant, param, avg):
    w = synth.WORKLOADS[2]
    n = 6000
    x = synth.stream(w, 0, 0, 4, 0, n=n)
    base = codec.calibrate_head(x, 2048, avg)
    B = int(base["total_bits"])
    if variant == "floor" and B < 128 * int(param):
        pytest.skip("budget below the floor")
    bits = codec.allocate_bits(base["lam"], B, variant, param)
    assert np.array_equal(stc.allocate_bits(base["lam"], B, variant, param), bits)
    st = codec.make_state(base["U"], base["lam"], bits, codec.XFORM_EIGEN)
    gst = stc.state_init(st["U"], st["lam"], st["bits"], st["steps"], xform=stc.XFORM_EIGEN)
    xd = torch.from_numpy(x.astype(np.float32)).to(DEV, torch.bfloat16)
    packed, _ = stc.encode_kv(gst, xd)
    qg = codec.unpack(packed.cpu().numpy(), st["bits"], n)
    check_eigen_codes(qg, st, x)
    xg = stc.decode_kv(gst, packed, n).float().cpu().numpy()
    xo = codec.decode_kv(st, codec.encode_kv(st, x), n, "bf16")
    r_g, r_o = codec.rel_mse(x, xg), codec.rel_mse(x, xo)
    assert abs(r_g - r_o) <= 1e-3 * r_o, (r_g, r_o)
