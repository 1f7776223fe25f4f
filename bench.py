#!/usr/bin/env python3
"""Benchmark of the spectral transform KV-cache codec on one MI355X.

Default workload (one "step" = one pass of the whole hot path over one batch):
the two full-size caches, resident in HBM:
  * Qwen2.5-7B-shaped batched decode: 28 layers x batch 16 x 4 KV heads x
    {K, V} = 3584 streams of 32768 bf16 tokens (head dim 128), spiked-Gaussian
    synthetic data (lambda_i = i^-1.0, 3 outlier channels at 30x), 224 states
    calibrated on the first 2048 tokens of batch entry 0 and shared over the
    batch, 1.33 bits (170-bit records);
  * Llama-3.1-8B-shaped cache: 32 layers x 8 KV heads x {K, V} = 512 streams
    of 131072 bf16 tokens (lambda_i = i^-alpha, alpha per layer in
    [0.8, 1.5], 2 outlier channels at 20x), 2.0 bits (256-bit records).
  For each: one batched encode of every stream (prefill), one batched decode
  of every stream, and one decode-step attention over every KV head (GQA 7 /
  GQA 4) reading only the packed cache. Calibration runs once, before timing.
  Streams are generated on the device from the seeded recipe.

Prints ONE JSON line. `value` is the algorithmic bytes of the K timed steps
divided by their wall time on the launch stream (GB/s); per-op figures are in
`breakdown`; `roofline` is for the kernel launch with the largest time share;
`cpu_baseline` times the CPU oracle on a labelled sample of the same two
workloads. `layer` holds the figures of the smaller Llama-layer step (16
streams x 32768 tokens, budgets 4.0 / 2.0 / 1.33, Walsh-Hadamard path, warm
and with cold caches), which are not part of `value`.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
WORKLOAD = 2
RHT_WORKLOAD = 3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=None, help="override tokens per stream (testing only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the workload, copy a buffer of this many MiB three times (untimed): "
                         "the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-mib N` into a traffic summary for --kernel")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR", default=None,
                    help="no GPU work: print the kernel statistics of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR", default=None,
                    help="no GPU work: per-kernel averages of the counters of rocprofv3 --pmc runs of the step")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (no generation step, Walsh-Hadamard attention, sketch or cold "
                         "passes); for counter runs whose per-launch averages must cover the step's launches only")
    ap.add_argument("--workload", default="full", choices=["full", "llama_layer", "llama_cache", "qwen_batch"],
                    help="full: the step above (the bench line); llama_layer: the Llama-layer step alone (its own "
                         "line); llama_cache / qwen_batch: one of the two caches alone, timed the same way (for "
                         "counter runs whose per-launch figures must cover one workload)")
    ap.add_argument("--kernel", default=None, help="kernel name prefix for --summarize")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    return ap.parse_args()


# Kernel launched by each timed op that is a single kernel; the roofline is
# reported for the kernel with the largest share of the step.
KERNEL_OF_OP = {"encode": "k_encode_eigen<bf16>", "decode": "k_decode_eigen<bf16>",
                "attend": "k_att2", "rht_encode": "k_rht_encode", "rht_decode": "k_rht_decode"}
# rocprofv3 kernel names of the same kernels (the variants the step runs:
# records of 32 * 2^s bits at 4.0 and 2.0 bits take the slot-layout variant,
# the 170-bit records at 1.33 bits the packed-stream one)
PROFILE_NAME = {"k_encode_eigen<bf16>": ("void stc::k_encode_eigen<0, true>(stc::EncK)",
                                         "void stc::k_encode_eigen<0, false>(stc::EncK)"),
                "k_decode_eigen<bf16>": ("void stc::k_decode_eigen<0, *",),
                "k_att2": ("void stc::k_att2<*",),  # (every instance; a trailing * matches a prefix)
                "k_att_main": ("void stc::k_att_main<8, false, false, true>(stc::AttK)",
                               "void stc::k_att_main<8, false, false, false>(stc::AttK)"),
                "k_rht_encode": ("void stc::k_rht_encode<false>(stc::RhtK)",),
                "k_rht_decode": ("stc::k_rht_decode(stc::RhtK)",)}
KERNEL_SOURCE = os.path.join(ROOT, "spectral_transform_codec_amd", "csrc", "stc_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def _present(pnames, names):
    """The profiled kernel names among `names` that the patterns pnames cover."""
    out = []
    for pn in pnames:
        if pn.endswith("*"):
            out += sorted(n for n in names if n.startswith(pn[:-1]))
        elif pn in names:
            out.append(pn)
    return out


def kernel_of(op_name):
    base = op_name.split("@")[0]
    return KERNEL_OF_OP.get(base)


def source_digest():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter
    summary, or None if there is none or the kernel source changed since it
    was taken."""
    path = os.path.join(PROFILES, "traffic_" + kernel.replace("<", "_").replace(">", "") + f"_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(total_bits, n, streams, elem=2):
    """Encode or decode: read/write the tokens plus the packed records."""
    return streams * n * (128 * elem + total_bits / 8.0)


def main():
    args = parse()
    if args.summarize or args.summarize_trace or args.summarize_counters:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mib:
        # the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "llama_layer":
        line = layer_step(args, dev)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(args.cpu_seconds, layer=True)
        print(json.dumps(line), flush=True)
        return
    full_step(args, dev)


def layer_step(args, dev):
    """The Llama-layer step (16 streams x 32768 tokens, budgets 4.0 / 2.0 /
    1.33 bits, plus the Walsh-Hadamard path on 16 Student-t streams): its own
    timing, per-op breakdown, cold-cache pass and extras. Returns a dict."""
    import numpy as np
    import torch

    import synth
    import spectral_transform_codec_amd as stc

    w = synth.WORKLOADS[WORKLOAD]
    w3 = synth.WORKLOADS[RHT_WORKLOAD]
    n = args.tokens or w.n_tokens
    heads = w.kv_heads
    S = 2 * heads                       # K and V of every KV head
    g = w.group

    # ------------------------------------------------------------ inputs
    t_setup = time.time()
    x2 = torch.empty((S, n, 128), dtype=torch.bfloat16, device=dev)
    x3 = torch.empty((S, n, 128), dtype=torch.bfloat16, device=dev)
    for h in range(heads):
        for kind in (0, 1):
            x2[2 * h + kind] = torch.from_numpy(synth.stream(w, 0, 0, h, kind, n=n)).to(dev, torch.bfloat16)
            x3[2 * h + kind] = torch.from_numpy(synth.stream(w3, 0, 0, h, kind, n=n)).to(dev, torch.bfloat16)
    q = torch.from_numpy(np.stack([synth.queries(w, 0, 0, h) for h in range(heads)])).to(dev)

    # ------------------------------------------------ calibration (untimed)
    t_cal = time.time()
    budgets = list(w.budgets)
    arrays = {}
    for b in budgets:
        arrays[b] = stc.calibrate_heads_batched(x2, w.n_calib, b)
    torch.cuda.synchronize()
    cal_s = time.time() - t_cal
    cb, _ = stc.lloyd_max(synth.sphere_coordinate_samples())
    cb32 = cb.astype(np.float32)
    rht_arr = stc.StateArray([stc.rht_state_init(synth.random_signs(3, 0, 0, s // 2, s % 2), cb32)
                              for s in range(S)])
    kmap = torch.arange(0, S, 2, dtype=torch.int32, device=dev)
    vmap = torch.arange(1, S, 2, dtype=torch.int32, device=dev)

    # ---------------------------------------------------- buffers (untimed)
    packed = {b: torch.empty((S, stc.packed_bytes(arrays[b].max_bits, n)), dtype=torch.uint8, device=dev)
              for b in budgets}
    xhat = torch.empty((S, n, 128), dtype=torch.bfloat16, device=dev)
    attn_out = {b: torch.empty((heads, g, 128), dtype=torch.float32, device=dev) for b in budgets}
    ws = torch.zeros(stc.attend_workspace_bytes(heads, g, n), dtype=torch.uint8, device=dev)
    rpacked = torch.empty((S, stc.packed_bytes(384, n)), dtype=torch.uint8, device=dev)
    rnorms = torch.empty((S, n), dtype=torch.float32, device=dev)
    setup_s = time.time() - t_setup

    ops = []  # (name, fn, algorithmic bytes)
    for b in budgets:
        B = arrays[b].max_bits
        ops.append((f"encode@{b}", (lambda b=b: stc.encode_kv_batched(arrays[b], x2, packed=packed[b])),
                    algorithmic_bytes(B, n, S)))
        ops.append((f"decode@{b}", (lambda b=b: stc.decode_kv_batched(arrays[b], packed[b], n, out=xhat)),
                    algorithmic_bytes(B, n, S)))
        kp, vp = packed[b][0::2], packed[b][1::2]
        ops.append((f"attend@{b}",
                    (lambda b=b, kp=kp, vp=vp: stc.attend_compressed_batched(arrays[b], kmap, vmap, kp, vp, n, q,
                                                                            ws=ws, out=attn_out[b])),
                    heads * n * 2 * B / 8.0 + 2 * q.numel() * 4))
    ops.append(("rht_encode", lambda: stc.encode_kv_batched(rht_arr, x3, packed=rpacked, norms=rnorms),
                S * n * (256 + 48 + 4)))
    ops.append(("rht_decode", lambda: stc.decode_kv_batched(rht_arr, rpacked, n, norms=rnorms, out=xhat),
                S * n * (256 + 48 + 4)))

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, fn, _ in ops:
            fn()
    torch.cuda.synchronize()

    # ------------------------------------------------------- timed region
    # (1) the step as a whole: events only around the K steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for k in range(args.steps):
        for _, fn, _ in ops:
            fn()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    # (2) per-op durations: events on the launch stream around every op
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        for i, (_, fn, _) in enumerate(ops):
            ev[k][i][0].record(stream)
            fn()
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()

    step_us, cold, achievable = {}, {}, {}
    if not args.no_extras:
        # (3) one generation step per budget (append the last token's K and V to
        # every KV head, then attend over all n): it rewrites record n - 1 with
        # the same codes, so the caches stay as they are
        kn = x2[0::2, n - 1].contiguous()
        vn = x2[1::2, n - 1].contiguous()
        for b in budgets:
            kp, vp = packed[b][0::2], packed[b][1::2]
            fn = (lambda b=b, kp=kp, vp=vp: stc.decode_step_batched(arrays[b], kmap, vmap, n - 1, kn, vn, kp, vp, q,
                                                                    ws=ws, out=attn_out[b]))
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            step_us[f"decode_step@{b}"] = round(1e3 * e0.elapsed_time(e1) / args.steps, 2)

        # (4) one attention step over the Walsh-Hadamard caches of the same layer
        rk, rv = rpacked[0::2], rpacked[1::2]
        rkn, rvn = rnorms[0::2], rnorms[1::2]
        rht_out = torch.empty((heads, g, 128), dtype=torch.float32, device=dev)
        rfn = lambda: stc.attend_rht_batched(rht_arr, kmap, vmap, rk, rkn, rv, rvn, n, q, ws=ws, out=rht_out)
        for _ in range(3):
            rfn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            rfn()
        e1.record(stream)
        torch.cuda.synchronize()
        step_us["attend_rht"] = round(1e3 * e0.elapsed_time(e1) / args.steps, 2)

        # (5) the key residual sketch on the same layer: sketch encode of the 8 K
        # streams, then attention with the score correction
        sk_states = []
        for s_ in range(S):
            sg = synth.random_signs(3, 0, 0, s_ // 2, s_ % 2)
            sk_states.append(stc.rht_sketch_state_init(sg, cb32, synth.sketch_matrix(3, 0, 0, s_ // 2, 0))
                             if s_ % 2 == 0 else stc.rht_state_init(sg, cb32))
        sk_arr = stc.StateArray(sk_states)
        kx3 = x3[0::2]
        sk_packed = torch.empty((S, stc.packed_bytes(384, n)), dtype=torch.uint8, device=dev)[0::2]  # V's strides
        sk_norms = torch.empty((S, n), dtype=torch.float32, device=dev)[0::2]
        sk_bits = torch.empty((heads, stc.packed_bytes(128, n)), dtype=torch.uint8, device=dev)
        sk_rn = torch.empty((heads, n), dtype=torch.float32, device=dev)
        kmap_sk = torch.arange(0, S, 2, dtype=torch.int32, device=dev)
        sfn = lambda: stc.append_rht_sketch_batched(sk_arr, kx3, 0, sk_packed, sk_norms, sk_bits, sk_rn,
                                                    state_of_stream=kmap_sk)
        afn = lambda: stc.attend_rht_batched(sk_arr, kmap, vmap, sk_packed, sk_norms, rv, rvn, n, q, ws=ws,
                                             out=rht_out, k_sketch=sk_bits, k_rnorm=sk_rn)
        for name, fn in (("rht_sketch_encode_K", sfn), ("attend_rht_sketch", afn)):
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            step_us[name] = round(1e3 * e0.elapsed_time(e1) / args.steps, 2)

        # (5b) the selective residual sketch on the eigen caches at 2.0 bits:
        # sketch of the 8 K streams, then attention with the second score table
        b2 = 2.0 if 2.0 in budgets else budgets[0]
        es_states = []
        for s_, st in enumerate(arrays[b2].states):
            es_states.append(stc.state_init(st.basis(), st.lam, st.bits, st.steps,
                                            sketch=synth.sketch_matrix(2, 0, 0, s_ // 2, 0))
                             if s_ % 2 == 0 else st)
        es_arr = stc.StateArray(es_states)
        es_bits = torch.empty((heads, stc.packed_bytes(128, n)), dtype=torch.uint8, device=dev)
        es_rn = torch.empty((heads, n), dtype=torch.float32, device=dev)
        kp2, vp2 = packed[b2][0::2], packed[b2][1::2]
        stc.encode_kv_batched(arrays[b2], x2, packed=packed[b2])
        kx2 = x2[0::2]
        efn = lambda: stc.sketch_kv_batched(es_arr, kx2, 0, es_bits, es_rn, state_of_stream=kmap)
        eafn = lambda: stc.attend_compressed_sketch_batched(es_arr, kmap, vmap, kp2, vp2, es_bits, es_rn, n, q,
                                                            ws=ws, out=attn_out[b2])
        for name, fn in ((f"eigen_sketch_K@{b2}", efn), (f"attend_sketch@{b2}", eafn)):
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            step_us[name] = round(1e3 * e0.elapsed_time(e1) / args.steps, 2)

        # (6) cold caches: each op of the step once more, after 1 GiB of writes
        # has pushed the L2s and the 256 MiB memory-side cache out
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for name, fn, nbytes in ops:
            ms = []
            for _ in range(3):
                scratch.fill_(1.0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            cold[name] = {"us": round(1e3 * min(ms), 2),
                          "pct_hbm_peak": round(100.0 * nbytes / (min(ms) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
        del scratch

        # (7) what a plain device copy achieves (bytes read + written per
        # second): at 1 GiB, and at the size of one encode launch's traffic
        def copy_gbps(nbytes):
            src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(10):
                dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            return round(2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        enc_bytes = int(ops[0][2])
        achievable = {"copy_GBps_1GiB": copy_gbps(1 << 30),
                      "copy_GBps_encode_size": copy_gbps(enc_bytes // 2),
                      "encode_size_bytes": enc_bytes}

    per_op = {}
    for i, (name, _, nbytes) in enumerate(ops):
        ms = [ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)]
        avg = sum(ms) / len(ms)
        per_op[name] = {"ms": round(avg, 5), "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                        "pct_hbm_peak": round(100.0 * nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
                        "bytes": int(nbytes)}
    step_bytes = sum(o[2] for o in ops)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # roofline of the single-kernel op family with the largest time share:
    # algorithmic bytes per launch / average launch duration (HIP events on
    # the launch stream), averaged over the family's launches in a step
    fam = {}
    for name, _, nbytes in ops:
        kname = kernel_of(name)
        if kname:
            t = fam.setdefault(kname, [0.0, 0.0, 0])
            t[0] += per_op[name]["ms"]
            t[1] += nbytes
            t[2] += 1
    dname = max(fam, key=lambda k: fam[k][0])
    d_ms, d_bytes, d_n = fam[dname]
    achieved = d_bytes / (d_ms * 1e-3) / 1e9
    traffic = stored_traffic(dname, "llama_layer")
    # the same figures for every single-kernel family of the step
    families = {}
    for kname, (f_ms, f_bytes, f_n) in sorted(fam.items(), key=lambda kv: -kv[1][0]):
        f_tr = stored_traffic(kname, "llama_layer")
        families[kname] = {"launches_per_step": f_n, "avg_launch_us": round(1e3 * f_ms / f_n, 2),
                           "algorithmic_bytes_per_launch": int(f_bytes / f_n),
                           "achieved": round(f_bytes / (f_ms * 1e-3) / 1e9, 1),
                           "frac": round(f_bytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                           "traffic": None if f_tr is None else int(f_tr)}
    codec_names = [o[0] for o in ops if o[0].startswith(("encode", "decode"))]
    codec_bytes = sum(o[2] for o in ops if o[0] in codec_names)
    codec_ms = sum(per_op[nm]["ms"] for nm in codec_names)
    attn_names = [o[0] for o in ops if o[0].startswith("attend")]

    line = {
        "metric": "KV codec encode/decode GB/s (% of HBM peak); compressed decode-attn tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped layer: 8 KV heads x K/V = 16 streams x "
                               f"{n} bf16 tokens, head_dim 128, budgets {budgets} bits, "
                               "GQA-4 decode attention; plus 16 Student-t(3) streams through the "
                               "Walsh-Hadamard 3-bit path",
                   "streams": S, "tokens": n, "budgets": budgets, "group": g},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 1),
        "codec_GBps": round(codec_bytes / (codec_ms * 1e-3) / 1e9, 1),
        "attn_tokens_per_s": {nm: round(1e3 / per_op[nm]["ms"], 1) for nm in attn_names},
        # not in value: a generation step per budget (append one K/V token per KV head, then attend over
        # n), one attention step over the Walsh-Hadamard caches, and the key residual sketches of both
        # caches (their encode of the 8 K streams, attention with the score correction)
        "extra_us": step_us,
        "breakdown": per_op,
        "breakdown_cold": cold,  # each op alone after 1 GiB of writes (not in value)
        "achievable": achievable,  # plain device copies, read + write bytes per second (not in value)
        "roofline": {"bound": "hbm", "kernel": dname, "launches_per_step": d_n,
                     "algorithmic_bytes_per_launch": int(d_bytes / d_n),
                     "avg_launch_us": round(1e3 * d_ms / d_n, 2),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic)},
        "roofline_by_kernel": families,
        "setup_s": round(setup_s, 2),
        "calibrate_s": round(cal_s, 2),
    }
    return line


def build_cache(w, n, dev):
    """One full-size cache on the device: every stream generated from the
    workload's recipe (per-stream Haar rotation and outlier channels from the
    seeded numpy generators, lambda_i = i^-alpha per layer, Gaussian samples
    from a seeded device generator: the same distribution as the host
    generator, not the same numbers), calibrated on its first 2048 tokens (the
    Qwen batch: one state per layer, KV head and K/V, from batch entry 0,
    shared over the batch). Returns a dict of device tensors and sizes."""
    import numpy as np
    import torch

    import synth
    import spectral_transform_codec_amd as stc

    L, Bt, H, g = w.layers, w.batch, w.kv_heads, w.group
    budget = w.budgets[0]
    S = L * Bt * H * 2                      # streams ordered (layer, batch, head, K/V)
    P = S // 2                              # KV heads attended per step
    t_setup = time.time()
    x = torch.empty((S, n, 128), dtype=torch.bfloat16, device=dev)
    gen = torch.Generator(device=dev)
    rot = {}
    for l in range(L):
        lam = torch.arange(1, 129, dtype=torch.float64, device=dev) ** (-synth.layer_alpha(w, l))
        for b in range(Bt):
            bs = 0 if w.share_over_batch else b
            for h in range(H):
                for kind in (0, 1):
                    key = (l, bs, h, kind)
                    if key not in rot:
                        q = synth.haar_orthogonal(synth.rng_for(w.cfg, l, bs, h, kind, synth.P_ROT))
                        idx = synth.rng_for(w.cfg, l, bs, h, kind, synth.P_OUTLIER).permutation(128)[:w.n_outliers]
                        sc = np.ones(128)
                        sc[idx] = w.outlier_scale
                        # x = (z sqrt(lambda)) Q^T, then the outlier channels scaled
                        rot[key] = (torch.from_numpy(q.T * sc[None, :]).to(dev) * lam.sqrt()[:, None]).float()
                    gen.manual_seed(((((w.cfg * 64 + l) * 64 + b) * 64 + h) * 2 + kind) * 8 + synth.P_SAMPLES)
                    z = torch.randn((n, 128), generator=gen, device=dev, dtype=torch.float32)
                    x[((l * Bt + b) * H + h) * 2 + kind] = (z @ rot[key]).to(torch.bfloat16)
                    del z
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    t_cal = time.time()
    n_c = min(w.n_calib, n)
    if w.share_over_batch:
        # batch entry 0 of every (layer, KV head, K/V), gathered into one
        # [L * H * 2][n_calib][128] tensor; state index (l, h, kind)
        xc = x.view(L, Bt, H * 2, n, 128)[:, 0, :, :n_c].reshape(L * H * 2, n_c, 128)
        smap = [(l * H + h) * 2 + kind for l in range(L) for b in range(Bt) for h in range(H) for kind in (0, 1)]
    else:
        xc = x[:, :n_c]
        smap = list(range(S))
    arr = stc.calibrate_heads_batched(xc, n_c, budget)
    del xc
    torch.cuda.synchronize()
    cal_s = time.time() - t_cal
    smap_t = torch.tensor(smap, dtype=torch.int32, device=dev)
    B = arr.max_bits
    return {"w": w, "n": n, "S": S, "P": P, "g": g, "Bt": Bt, "B": B, "budget": budget, "x": x, "arr": arr,
            "smap": smap_t, "kmap": smap_t[0::2].contiguous(), "vmap": smap_t[1::2].contiguous(),
            "packed": torch.empty((S, stc.packed_bytes(B, n)), dtype=torch.uint8, device=dev),
            "xhat": torch.empty_like(x),
            "q": torch.randn((P, g, 128), generator=gen.manual_seed(w.cfg * 8 + synth.P_QUERY), device=dev),
            "ws": torch.empty(stc.attend_workspace_bytes(P, g, n), dtype=torch.uint8, device=dev),
            "out": torch.empty((P, g, 128), dtype=torch.float32, device=dev),
            "setup_s": setup_s, "calibrate_s": cal_s}


def cache_ops(c, tag):
    """(name, fn, algorithmic bytes, workload tag) of one cache's step:
    encode every stream, decode every stream, one attention step."""
    import spectral_transform_codec_amd as stc
    n, S, P, B = c["n"], c["S"], c["P"], c["B"]
    codec_bytes = S * n * (256 + B / 8.0)
    kp, vp = c["packed"][0::2], c["packed"][1::2]
    return [
        (f"encode@{tag}", lambda: stc.encode_kv_batched(c["arr"], c["x"], state_of_stream=c["smap"],
                                                        packed=c["packed"]), codec_bytes, tag),
        (f"decode@{tag}", lambda: stc.decode_kv_batched(c["arr"], c["packed"], n, state_of_stream=c["smap"],
                                                        out=c["xhat"]), codec_bytes, tag),
        (f"attend@{tag}", lambda: stc.attend_compressed_batched(c["arr"], c["kmap"], c["vmap"], kp, vp, n, c["q"],
                                                                ws=c["ws"], out=c["out"]),
         P * n * 2 * B / 8.0 + 2 * c["q"].numel() * 4, tag),
    ]


def rht_encode_kernels(c, args, dev):
    """Walsh-Hadamard encode of the whole cache input (every stream, 3-bit
    codebook) with each encode kernel in turn: the +-1 matrix on the matrix
    cores and the register butterfly. Average of K launches (HIP events on the
    launch stream), bytes = bf16 tokens in + 48-byte records + fp32 norms out.
    Not part of value."""
    import torch

    import synth
    import spectral_transform_codec_amd as stc
    n, S = c["n"], c["S"]
    import numpy as np
    cb = stc.lloyd_max(synth.sphere_coordinate_samples())[0].astype(np.float32)
    n_st = 16
    arr = stc.StateArray([stc.rht_state_init(synth.random_signs(4, 0, 0, h, 0), cb) for h in range(n_st)])
    smap = torch.arange(S, dtype=torch.int32, device=dev) % n_st
    packed = torch.empty((S, stc.packed_bytes(384, n)), dtype=torch.uint8, device=dev)
    norms = torch.empty((S, n), dtype=torch.float32, device=dev)
    nbytes = S * n * (256 + 48 + 4)
    stream = torch.cuda.current_stream()
    out = {}
    before = stc.get_rht_encode_kernel()
    try:
        for name, kind in (("mfma", stc.RHT_ENCODE_MFMA), ("butterfly", stc.RHT_ENCODE_BUTTERFLY)):
            stc.set_rht_encode_kernel(kind)
            fn = lambda: stc.encode_kv_batched(arr, c["x"], state_of_stream=smap, packed=packed, norms=norms)
            for _ in range(2):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            out[name] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
    finally:
        stc.set_rht_encode_kernel(before)
    out["bytes"] = int(nbytes)
    out["streams"], out["tokens"] = S, n
    del packed, norms
    return out


def copy_ceiling(args, dev):
    """The practical ceiling of a read + write pattern: device copies of
    4 GiB (far past the 256 MiB memory-side cache), read + written bytes per
    second, with the library's streaming copy kernel and with torch's copy.
    Not part of value."""
    import torch

    import spectral_transform_codec_amd as stc
    nbytes = 4 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    out = {"bytes_copied": nbytes}
    for name, fn in (("stream_copy", lambda: stc.stream_copy(dst, src)), ("torch_copy", lambda: dst.copy_(src))):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = 2 * nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        out[name] = {"GBps": round(gbps, 1), "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 1)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def full_step(args, dev):
    import torch

    import synth

    tags = ["qwen_batch", "llama_cache"] if args.workload == "full" else [args.workload]
    caches = {}
    for tag in tags:
        w = synth.WORKLOADS[5 if tag == "qwen_batch" else 4]
        caches[tag] = build_cache(w, args.tokens or w.n_tokens, dev)
        print(f"bench: {tag} built ({caches[tag]['S']} streams x {caches[tag]['n']} tokens, "
              f"setup {caches[tag]['setup_s']:.1f} s, calibration {caches[tag]['calibrate_s']:.1f} s)",
              file=sys.stderr, flush=True)
    ops = [op for tag in tags for op in cache_ops(caches[tag], tag)]
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for op in ops:
            op[1]()
    torch.cuda.synchronize()
    # (1) the step as a whole: events only around the K steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        for op in ops:
            op[1]()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # (2) per-op durations: events on the launch stream around every op
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        for i, op in enumerate(ops):
            ev[k][i][0].record(stream)
            op[1]()
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()
    per_op = {}
    for i, (name, _, nbytes, tag) in enumerate(ops):
        ms = [ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)]
        avg = sum(ms) / len(ms)
        per_op[name] = {"ms": round(avg, 5), "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                        "pct_hbm_peak": round(100.0 * nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
                        "bytes": int(nbytes)}
    step_bytes = sum(op[2] for op in ops)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # roofline of the kernel launch with the largest time share (one launch
    # per op and step): algorithmic bytes / average duration (HIP events on
    # the launch stream); traffic from the committed counter summary of that
    # kernel on that workload, if it matches the kernel source
    by_kernel = {}
    for name, _, nbytes, tag in ops:
        kname = kernel_of(name)
        a_ms = per_op[name]["ms"]
        tr = stored_traffic(kname, tag)
        by_kernel[f"{kname}@{tag}"] = {"avg_launch_us": round(1e3 * a_ms, 2),
                                      "algorithmic_bytes_per_launch": int(nbytes),
                                      "achieved": round(nbytes / (a_ms * 1e-3) / 1e9, 1),
                                      "frac": round(nbytes / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                      "traffic": None if tr is None else int(tr)}
    dom = max(ops, key=lambda op: per_op[op[0]]["ms"])
    dkey = f"{kernel_of(dom[0])}@{dom[3]}"
    d = by_kernel[dkey]
    att = {}
    for tag in tags:
        a_ms = per_op[f"attend@{tag}"]["ms"]
        att[tag] = {"us_per_step": round(1e3 * a_ms, 1), "steps_per_s": round(1e3 / a_ms, 1),
                    "tokens_per_s": round(caches[tag]["Bt"] * 1e3 / a_ms, 1),
                    "pct_hbm_peak": per_op[f"attend@{tag}"]["pct_hbm_peak"]}
    codec_names = [op[0] for op in ops if op[0].startswith(("encode", "decode"))]
    codec_bytes = sum(op[2] for op in ops if op[0] in codec_names)
    codec_ms = sum(per_op[nm]["ms"] for nm in codec_names)
    cfg = {"workload": " + ".join(caches[t]["w"].name + f" ({caches[t]['S']} streams x {caches[t]['n']} bf16 "
                                                        f"tokens, {caches[t]['budget']} bits)" for t in tags),
           "step": "per cache: batched encode of every stream, batched decode of every stream, one decode-attention "
                   "step over every KV head reading only the packed cache",
           "streams": {t: caches[t]["S"] for t in tags}, "tokens": {t: caches[t]["n"] for t in tags},
           "budget_bits": {t: caches[t]["budget"] for t in tags}, "group": {t: caches[t]["g"] for t in tags}}
    line = {
        "metric": "KV codec encode/decode GB/s (% of HBM peak); compressed decode-attn tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (device-generated, seeded)", "config": cfg,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 1),
        "codec_GBps": round(codec_bytes / (codec_ms * 1e-3) / 1e9, 1),
        "codec_pct_hbm_peak": round(100.0 * codec_bytes / (codec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
        "attention": att,
        "breakdown": per_op,
        "roofline": {"bound": "hbm", "kernel": dkey, "launches_per_step": 1,
                     "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_launch"],
                     "avg_launch_us": d["avg_launch_us"], "achieved": d["achieved"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": d["frac"], "traffic": d["traffic"]},
        "roofline_by_kernel": by_kernel,
        "setup_s": {t: round(caches[t]["setup_s"], 1) for t in tags},
        "calibrate_s": {t: round(caches[t]["calibrate_s"], 1) for t in tags},
    }
    if "llama_cache" in caches and not args.no_extras:
        line["rht_encode_llama_cache"] = rht_encode_kernels(caches["llama_cache"], args, dev)
    # the caches are not needed any more: free them before the extras
    del ops, caches
    torch.cuda.empty_cache()
    if not args.no_extras:
        line["achievable"] = copy_ceiling(args, dev)
    if not args.no_extras and args.workload == "full":
        line["layer"] = layer_step(args, dev)
    if not args.no_cpu_baseline and args.workload == "full":
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


def _profile_rows(d, want_counters):
    """(kernel name, dispatch id, value) rows of a rocprofv3 output folder:
    counter values of a --pmc run, or durations (ns) of a kernel trace. Reads
    the rocpd database, or the CSV files when that is what the run wrote."""
    import csv
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    rows = []
    if dbs:
        for db in dbs:
            con = sqlite3.connect(db)
            if want_counters:
                q = "select name, dispatch_id, counter_name, counter_value from pmc_events"
                rows += [(r[0], r[1], r[2], float(r[3])) for r in con.execute(q)]
            else:
                rows += [(r[0], None, None, float(r[1] - r[2]))
                         for r in con.execute("select name, end, start from kernels")]
        return rows
    pat = "*counter_collection.csv" if want_counters else "*kernel_trace.csv"
    for fn in sorted(glob.glob(os.path.join(d, "**", pat), recursive=True)):
        for r in csv.DictReader(open(fn)):
            if want_counters:
                rows.append((r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"], float(r["Counter_Value"])))
            else:
                rows.append((r["Kernel_Name"], None, None,
                             float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    return rows


def summarize(args):
    """Text summaries for profiles/: kernel statistics of a trace run, or the
    HBM traffic per launch of one kernel from FETCH_SIZE and WRITE_SIZE runs,
    each counter scaled by what it reads for a plain device copy of known size
    (`bench.py --copy-mib N` runs one before the workload)."""
    import collections
    out = []
    if args.command:
        out.append("command: " + args.command)
    if args.summarize_counters:
        # per kernel: the average over its dispatches of each counter (summed
        # over the counter's instances within a dispatch)
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for d in args.summarize_counters:
            acc = collections.defaultdict(lambda: collections.defaultdict(float))
            for name, disp, cname, v in _profile_rows(d, True):
                acc[(name, disp)][cname] += v
            for (name, _), cs in acc.items():
                for cname, v in cs.items():
                    per[name][cname].append(v)
        out.append(f"kernel_source_sha256_16: {source_digest()}")
        # 32-token blocks per launch of the codec kernels and of attention:
        # Llama layer 16 streams / 8 KV heads x 32768 tokens; Llama cache 512
        # streams / 256 KV heads x 131072; Qwen batch 3584 streams / 1792 KV
        # heads x 32768
        codec_tok, att_tok = {"llama_cache": (512 * 131072, 256 * 131072),
                              "qwen_batch": (3584 * 32768, 1792 * 32768)}.get(args.workload,
                                                                            (16 * 32768, 8 * 32768))
        blocks = {"k_att_main": att_tok // 32, "k_att2": att_tok // 32}
        for kname, pats in PROFILE_NAME.items():
            pnames = _present(pats, per)
            if not pnames:
                continue
            cs = collections.defaultdict(list)  # dispatches of every variant
            for pn in pnames:
                for c, v in per.get(pn, {}).items():
                    cs[c] += v
            pname = " + ".join(pn for pn in pnames if pn in per)
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            nb = blocks.get(kname, codec_tok // 32)
            out.append(f"== {kname}  ({pname}; {len(next(iter(cs.values())))} dispatches per counter)")
            for c in sorted(avg):
                out.append(f"   {c:40s} {avg[c]:18.1f}")
            if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
                out.append(f"   per 32-token block: VALU {avg['SQ_INSTS_VALU'] / nb:.1f} (MFMA included), "
                           f"MFMA {avg['SQ_INSTS_MFMA'] / nb:.1f}, LDS {avg.get('SQ_INSTS_LDS', 0) / nb:.1f}, "
                           f"VMEM read {avg.get('SQ_INSTS_VMEM_RD', 0) / nb:.2f}, "
                           f"VMEM write {avg.get('SQ_INSTS_VMEM_WR', 0) / nb:.2f}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                out.append(f"   MFMA busy cycles per SIMD (1024 SIMDs): {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:.0f}")
            if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_ACTIVE_INST_LDS" in avg:
                out.append(f"   LDS bank-conflict cycles / LDS active cycles: "
                           f"{avg['SQ_LDS_BANK_CONFLICT'] / max(1.0, avg['SQ_ACTIVE_INST_LDS']):.3f}")
            if "SQ_WAVE_CYCLES" in avg:
                for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
                          "SQ_WAIT_ANY"):
                    if c in avg:
                        out.append(f"   {c} / SQ_WAVE_CYCLES: {avg[c] / avg['SQ_WAVE_CYCLES']:.3f}")
        print("\n".join(out))
        return
    if args.summarize_trace:
        agg = collections.defaultdict(list)
        for name, _, _, ns in _profile_rows(args.summarize_trace, False):
            if args.kernel is None or args.kernel in name:  # (--kernel: a name filter, e.g. the namespace)
                agg[name].append(ns)
        tot = sum(sum(v) for v in agg.values())
        out.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share%':>7}  kernel")
        for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{len(v):6d} {sum(v) / len(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} {max(v) / 1e3:10.2f} "
                       f"{100 * sum(v) / tot:7.2f}  {name}")
        print("\n".join(out))
        return
    fetch_dir, write_dir = args.summarize
    kernel = args.kernel
    pats = PROFILE_NAME.get(kernel, (kernel,))

    def per_kernel(d, counter):
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        for name, disp, cname, v in _profile_rows(d, True):
            if cname == counter:
                vals[name][disp] += v       # sums the per-instance values of a dispatch
        return {k: list(v.values()) for k, v in vals.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_name = max((k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()),
                    key=lambda k: max(fetch[k]))
    copy_bytes = args.copy_mib << 20
    f_copy = max(fetch[copy_name]) * 1024.0
    w_copy = max(write[copy_name]) * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    pnames = _present(pats, fetch)
    fk = [v for pn in pnames for v in fetch.get(pn, [])]  # every variant's launches
    wk = [v for pn in pnames for v in write.get(pn, [])]
    pname = " + ".join(pn for pn in pnames if pn in fetch)
    f_avg = sum(fk) / len(fk) * 1024.0
    w_avg = sum(wk) / len(wk) * 1024.0
    traffic = f_avg * f_scale + w_avg * w_scale
    out += [
        f"kernel: {kernel}",
        f"profiled_name: {pname}",
        f"kernel_source_sha256_16: {source_digest()}",
        f"copy_kernel: {copy_name}",
        f"copy_bytes: {copy_bytes}",
        f"copy_FETCH_SIZE_bytes: {f_copy:.0f}",
        f"copy_WRITE_SIZE_bytes: {w_copy:.0f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"launches: {len(fk)} (FETCH run), {len(wk)} (WRITE run)",
        f"FETCH_SIZE_bytes_per_launch: {f_avg:.0f}",
        f"WRITE_SIZE_bytes_per_launch: {w_avg:.0f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        "  (= FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale, averaged over the launches)",
        "per launch (FETCH KiB, scaled read bytes):",
    ]
    out += [f"  {v:.1f} KiB -> {v * 1024 * f_scale:.0f}" for v in fk]
    out.append("per launch (WRITE KiB, scaled write bytes):")
    out += [f"  {v:.1f} KiB -> {v * 1024 * w_scale:.0f}" for v in wk]
    print("\n".join(out))


def _cpu_worker(args):
    """One process of the CPU baseline: the oracle, as it stands, on KV head
    pairs of the full-size workloads at their full length, BLAS on one
    thread: calibrate K and V (2048 tokens), encode and decode both streams,
    one attention step. The pairs alternate between the Qwen batch (32768
    tokens, 1.33 bits) and the Llama cache (131072 tokens, 2.0 bits), starting
    at a different pair in each process, until `seconds` have passed (a pair
    in progress is finished). Input generation is not timed. With `layer`,
    the sample is the Llama layer instead (4096-token KV head pairs at 2.0
    bits plus a Walsh-Hadamard stream). Returns (algorithmic bytes,
    description of the pairs done, seconds)."""
    proc, seconds, layer = args
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import codec, rht

    done, total_bytes, busy = [], 0.0, 0.0
    with threadpool_limits(limits=1):
        k_ = 0
        while busy < seconds:
            if layer:
                w = synth.WORKLOADS[WORKLOAD]
                cfg, lyr, b, h, n, avg = WORKLOAD, 0, 0, (proc + k_) % w.kv_heads, 4096, 2.0
            else:
                cfg = 5 if (proc + k_) % 2 == 0 else 4
                w = synth.WORKLOADS[cfg]
                j = proc * 7 + k_
                lyr, b, h = j % w.layers, (j // w.layers) % w.batch, j % w.kv_heads
                n, avg = w.n_tokens, w.budgets[0]
            k = synth.stream(w, lyr, b, h, 0, n=n)
            v = synth.stream(w, lyr, b, h, 1, n=n)
            q = synth.queries(w, lyr, b, h).astype(np.float64)
            t0 = time.perf_counter()
            ks, vs = codec.calibrate_head(k, 2048, avg), codec.calibrate_head(v, 2048, avg)
            kp, vp = codec.encode_kv(ks, k), codec.encode_kv(vs, v)
            codec.decode_kv(ks, kp, n, "bf16")
            codec.decode_kv(vs, vp, n, "bf16")
            codec.attend_compressed(ks, vs, kp, vp, n, q)
            B = int(ks["total_bits"])
            nbytes = 2 * 2 * algorithmic_bytes(B, n, 1) + n * 2 * B / 8.0
            if layer:
                w3 = synth.WORKLOADS[RHT_WORKLOAD]
                x3 = synth.stream(w3, 0, 0, h, 0, n=n)
                cb = rht.codebook_fp32(rht.lloyd_max(synth.sphere_coordinate_samples(200000))[0])
                rst = rht.make_state(synth.random_signs(3, 0, 0, h, 0), cb)
                t1 = time.perf_counter()
                p3, n3 = rht.encode_kv(rst, x3)
                rht.decode_kv(rst, p3, n3, n, "bf16")
                busy += time.perf_counter() - t1
                nbytes += 2 * n * (256 + 48 + 4)
            busy += time.perf_counter() - t0
            total_bytes += nbytes
            done.append(f"cfg{cfg}:L{lyr}/b{b}/h{h}")
            k_ += 1
    return total_bytes, done, busy


def cpu_baseline(seconds, layer=False):
    """The CPU oracle, as it stands, on a bounded sample of the workload (see
    _cpu_worker), in one process per host core (at most 16, the host share of
    one GPU), BLAS on one thread each; falls back to one process if a
    process pool cannot be started. GB/s = the sample's algorithmic bytes
    over the longest process's busy time."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        with mp.get_context("spawn").Pool(cores) as pool:
            res = pool.map(_cpu_worker, [(p, seconds, layer) for p in range(cores)])
    except (OSError, RuntimeError):
        cores = 1
        res = [_cpu_worker((0, seconds, layer))]
    total = sum(r[0] for r in res)
    el = max(r[2] for r in res)
    pairs = [p for r in res for p in r[1]]
    n5 = sum(1 for p in pairs if p.startswith("cfg5"))
    n4 = sum(1 for p in pairs if p.startswith("cfg4"))
    what = (f"{len(pairs)} Llama-layer KV head pairs x 4096 tokens at 2.0 bits (+ a Walsh-Hadamard stream each)"
            if layer else
            f"{n5} Qwen-batch KV head pairs x 32768 tokens at 1.33 bits and {n4} Llama-cache KV head pairs x "
            f"131072 tokens at 2.0 bits, full length ({', '.join(pairs[:6])}, ...)")
    return {"value": round(total / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{cores} processes, BLAS 1 thread each, {el:.1f} s busy in the longest: {what}; per pair "
                      f"calibrate K and V, encode, decode, one attention step; host CPU: {model}"}


if __name__ == "__main__":
    main()
