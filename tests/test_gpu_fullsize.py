"""GPU parity at the workloads' full sizes, in the batched launch configuration
the benchmark times, against the CPU oracle.

* Llama layer (16 streams x 32768 bf16 tokens, budgets 4.0 / 2.0 / 1.33):
  GPU calibration, batched encode, batched decode and batched GQA-4 attention
  exactly as bench.py calls them. Widths and all codes are compared with the
  oracle's; decode on a seeded sample of tokens per stream; attention on every
  KV head.
* Llama cache (131072 tokens, per-layer spectrum exponent, 2.0 bits): a seeded
  sample of streams (first and last layer, first and last KV head) at full
  length, codes on a token sample, decode, GQA-4 attention.
* Qwen batch (32768 tokens, 1.33 bits, states calibrated on batch sequence 0
  and shared across the batch): a sample of layers / batch entries / heads at
  full length, batched encode / decode with the state map, GQA-7 attention.

Bars as in test_gpu_parity.py: calibrated widths identical; <= 1e-4 of codes
differ, each by one level at a decision threshold; decode within one output rounding plus the hi/lo
arithmetic bound and relMSE within 1e-3 relative; attention relative max-abs
error <= 2e-3.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import codec
from parity_bounds import check_eigen_codes, decode_arith

pytestmark = pytest.mark.gpu

stc = pytest.importorskip("spectral_transform_codec_amd")

DEV = "cuda"
SAMPLE = 1024          # tokens per stream for the sampled checks


def f1_codes_of_tokens(packed: np.ndarray, bits: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Codes of the given tokens read straight from F1 bytes: token t, channel
    j, code bit k sits at stream bit t*B + o_j + k, bit (i & 7) of byte i >> 3."""
    bits = bits.astype(np.int64)
    B = int(bits.sum())
    off = np.concatenate([[0], np.cumsum(bits)[:-1]])
    k = np.arange(8)
    pos = tokens[:, None, None].astype(np.int64) * B + off[None, :, None] + k[None, None, :]
    valid = k[None, None, :] < bits[None, :, None]
    pos = np.where(valid, pos, 0)
    b = (packed[pos >> 3] >> (pos & 7).astype(np.uint8)) & 1
    b = np.where(valid, b, 0).astype(np.int64)
    return (b << k[None, None, :]).sum(axis=2)


def check_codes(q_gpu, st, x_tokens, gpu_state):
    """<= 1e-4 of codes differ, each by one level and at a decision threshold
    (within the derived projection error, GPU-calibrated basis included)."""
    check_eigen_codes(q_gpu, st, x_tokens, gpu_state=gpu_state)


def check_decode(st, q_gpu, x_tokens, x_gpu_tokens):
    """x_gpu_tokens: GPU decode (bf16 -> f64) of the sampled tokens whose GPU
    codes are q_gpu. Elementwise against the oracle's reconstruction of the
    same codes, and relMSE on the sample against the oracle's own codes."""
    exact = codec.reconstruct_exact(st, codec.pack(q_gpu, st["bits"]), q_gpu.shape[0])
    xo = codec.round_to_bf16(exact)
    ulp = np.abs(exact) * 2.0 ** -7
    arith = decode_arith(st, "bf16")
    assert np.all(np.abs(x_gpu_tokens - xo) <= ulp + arith[None, :])
    q_or = codec.quantize(st, codec.project(st, x_tokens))
    x_or = codec.decode_kv(st, codec.pack(q_or, st["bits"]), q_or.shape[0], "bf16")
    r_o, r_g = codec.rel_mse(x_tokens, x_or), codec.rel_mse(x_tokens, x_gpu_tokens)
    assert abs(r_g - r_o) <= 1e-3 * r_o, (r_g, r_o)


def attention_want(ks, vs, qk, qv, n, q):
    return codec.attend_compressed(ks, vs, codec.pack(qk, ks["bits"]), codec.pack(qv, vs["bits"]), n,
                                   q.astype(np.float64))


def rel_err(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max())


# ------------------------------------------------------------- Llama layer
@pytest.fixture(scope="module")
def llama_layer():
    w = synth.WORKLOADS[2]
    xs = [synth.stream(w, 0, 0, s // 2, s % 2) for s in range(2 * w.kv_heads)]
    x = torch.empty((len(xs), w.n_tokens, 128), dtype=torch.bfloat16, device=DEV)
    for s, xi in enumerate(xs):
        x[s] = torch.from_numpy(xi).to(DEV, torch.bfloat16)
    q = np.stack([synth.queries(w, 0, 0, h) for h in range(w.kv_heads)])
    return w, xs, x, q


@pytest.mark.parametrize("avg", [4.0, 2.0, 1.33])
def test_llama_layer_bench_configuration(llama_layer, avg):
    w, xs, x, q = llama_layer
    n, S, heads = w.n_tokens, len(xs), w.kv_heads
    print(f"llama layer: {S} streams x {n} tokens at {avg} bits", flush=True)
    arr = stc.StateArray([stc.calibrate_head(x[s], w.n_calib, avg) for s in range(S)])
    packed = torch.empty((S, stc.packed_bytes(arr.max_bits, n)), dtype=torch.uint8, device=DEV)
    stc.encode_kv_batched(arr, x, packed=packed)
    xhat = torch.empty_like(x)
    stc.decode_kv_batched(arr, packed, n, out=xhat)
    kmap = torch.arange(0, S, 2, dtype=torch.int32, device=DEV)
    vmap = torch.arange(1, S, 2, dtype=torch.int32, device=DEV)
    out = stc.attend_compressed_batched(arr, kmap, vmap, packed[0::2], packed[1::2], n,
                                        torch.from_numpy(q).to(DEV)).cpu().numpy()
    pk = packed.cpu().numpy()
    rng = np.random.default_rng(1234)
    states, q_all = [], []
    for s in range(S):
        st = codec.calibrate_head(xs[s], w.n_calib, avg)
        assert np.array_equal(arr.states[s].bits, st["bits"]), s
        qg = codec.unpack(pk[s, :codec.packed_bytes(st["total_bits"], n)], st["bits"], n)
        check_codes(qg, st, xs[s], arr.states[s])
        idx = np.sort(rng.choice(n, SAMPLE, replace=False))
        idx[-1] = n - 1
        xg = xhat[s, torch.from_numpy(idx).to(DEV)].float().cpu().numpy().astype(np.float64)
        check_decode(st, qg[idx], xs[s][idx], xg)
        states.append(st)
        q_all.append(qg)
    for h in range(heads):
        want = attention_want(states[2 * h], states[2 * h + 1], q_all[2 * h], q_all[2 * h + 1], n, q[h])
        assert rel_err(out[h], want) <= 2e-3, (h, rel_err(out[h], want))


# -------------------------------------------------------------- Llama cache
def test_llama_cache_sampled_streams_full_length():
    w = synth.WORKLOADS[4]
    n, avg = w.n_tokens, 2.0
    picks = [(0, 0), (0, 7), (31, 0), (31, 7)]          # (layer, KV head)
    xs = []
    for layer, h in picks:
        for kind in (0, 1):
            xs.append(synth.stream(w, layer, 0, h, kind))
    S = len(xs)
    print(f"llama cache: {S} streams x {n} tokens at {avg} bits", flush=True)
    x = torch.empty((S, n, 128), dtype=torch.bfloat16, device=DEV)
    for s, xi in enumerate(xs):
        x[s] = torch.from_numpy(xi).to(DEV, torch.bfloat16)
    arr = stc.StateArray([stc.calibrate_head(x[s], w.n_calib, avg) for s in range(S)])
    packed, _ = stc.encode_kv_batched(arr, x)
    xhat = stc.decode_kv_batched(arr, packed, n)
    q = np.stack([synth.queries(w, layer, 0, h) for layer, h in picks])
    kmap = torch.arange(0, S, 2, dtype=torch.int32, device=DEV)
    vmap = torch.arange(1, S, 2, dtype=torch.int32, device=DEV)
    out = stc.attend_compressed_batched(arr, kmap, vmap, packed[0::2], packed[1::2], n,
                                        torch.from_numpy(q).to(DEV)).cpu().numpy()
    pk = packed.cpu().numpy()
    rng = np.random.default_rng(4321)
    states, q_all = [], []
    for s in range(S):
        st = codec.calibrate_head(xs[s], w.n_calib, avg)
        assert np.array_equal(arr.states[s].bits, st["bits"]), s
        qg = codec.unpack(pk[s, :codec.packed_bytes(st["total_bits"], n)], st["bits"], n)
        idx = np.sort(rng.choice(n, SAMPLE, replace=False))
        idx[-1] = n - 1
        check_codes(qg[idx], st, xs[s][idx], arr.states[s])
        assert np.array_equal(f1_codes_of_tokens(pk[s], st["bits"], idx), qg[idx])
        xg = xhat[s, torch.from_numpy(idx).to(DEV)].float().cpu().numpy().astype(np.float64)
        check_decode(st, qg[idx], xs[s][idx], xg)
        states.append(st)
        q_all.append(qg)
    for p in range(len(picks)):
        want = attention_want(states[2 * p], states[2 * p + 1], q_all[2 * p], q_all[2 * p + 1], n, q[p])
        assert rel_err(out[p], want) <= 2e-3, (picks[p], rel_err(out[p], want))


# --------------------------------------------------------------- Qwen batch
def test_qwen_batch_shared_states_full_length():
    w = synth.WORKLOADS[5]
    n, avg = w.n_tokens, 1.33
    layers, batches, heads = (0, 27), (0, 9, 15), range(w.kv_heads)
    # states: one per (layer, head, kind), calibrated on batch sequence 0
    st_key = [(layer, h, kind) for layer in layers for h in heads for kind in (0, 1)]
    st_index = {k: i for i, k in enumerate(st_key)}
    calib_x = {k: synth.stream(w, k[0], 0, k[1], k[2]) for k in st_key}
    streams = [(layer, b, h, kind) for layer in layers for b in batches for h in heads for kind in (0, 1)]
    S = len(streams)
    print(f"qwen batch: {S} streams x {n} tokens at {avg} bits, {len(st_key)} shared states", flush=True)
    arr = stc.StateArray([stc.calibrate_head(torch.from_numpy(calib_x[k]).to(DEV, torch.bfloat16), w.n_calib, avg)
                          for k in st_key])
    smap_l = [st_index[(layer, h, kind)] for layer, b, h, kind in streams]
    smap = torch.tensor(smap_l, dtype=torch.int32, device=DEV)
    xs = [calib_x[(layer, h, kind)] if b == 0 else synth.stream(w, layer, b, h, kind)
          for layer, b, h, kind in streams]
    x = torch.empty((S, n, 128), dtype=torch.bfloat16, device=DEV)
    for s, xi in enumerate(xs):
        x[s] = torch.from_numpy(xi).to(DEV, torch.bfloat16)
    packed, _ = stc.encode_kv_batched(arr, x, smap)
    xhat = stc.decode_kv_batched(arr, packed, n, state_of_stream=smap)
    q = np.stack([synth.queries(w, layer, b, h) for layer, b, h, kind in streams[0::2]])
    out = stc.attend_compressed_batched(arr, smap[0::2].contiguous(), smap[1::2].contiguous(), packed[0::2],
                                        packed[1::2], n, torch.from_numpy(q).to(DEV)).cpu().numpy()
    ost = {k: codec.calibrate_head(calib_x[k], w.n_calib, avg) for k in st_key}
    for k in st_key:
        assert np.array_equal(arr.states[st_index[k]].bits, ost[k]["bits"]), k
    pk = packed.cpu().numpy()
    rng = np.random.default_rng(5678)
    q_all = []
    for s, (layer, b, h, kind) in enumerate(streams):
        st = ost[(layer, h, kind)]
        qg = codec.unpack(pk[s, :codec.packed_bytes(st["total_bits"], n)], st["bits"], n)
        idx = np.sort(rng.choice(n, SAMPLE // 2, replace=False))
        idx[-1] = n - 1
        check_codes(qg[idx], st, xs[s][idx], arr.states[st_index[(layer, h, kind)]])
        if s % 6 == 0:
            xg = xhat[s, torch.from_numpy(idx).to(DEV)].float().cpu().numpy().astype(np.float64)
            check_decode(st, qg[idx], xs[s][idx], xg)
        q_all.append(qg)
    for p in range(S // 2):
        layer, b, h, _ = streams[2 * p]
        want = attention_want(ost[(layer, h, 0)], ost[(layer, h, 1)], q_all[2 * p], q_all[2 * p + 1], n, q[p])
        assert rel_err(out[p], want) <= 2e-3, (streams[2 * p], rel_err(out[p], want))
