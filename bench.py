"""Benchmark of the CCA / CCGQA layer on one MI355X.

Headline: CCGQA prefill (B=1, S=16384, E=2048, 4 query heads x 128, 2 KV heads
x 128, conv kernels 2, QK-mean, value shift on d/2 channels, RoPE base 1e4),
bf16 storage with fp32 accumulation, synthetic seeded inputs resident in HBM.
A step is one cca_forward_prefill: down-projection, mix, attention,
up-projection.  Prints one JSON line (rank 0) with tokens/s over K timed steps,
the roofline of the dominant kernel (attention) timed with HIP events on the
launch stream over a second loop of K steps (the events add to the step time,
so the first loop runs without them), and the float64 CPU oracle's forward over
the same workload, timed once.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--rows prefill,decode,backward]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def attention_flops(S: int, Hq: int, d: int) -> float:
    # QK^T and PV over the S(S+1)/2 visible (query, key) pairs, 2 flops per MAC
    return 4.0 * Hq * d * S * (S + 1) / 2


def prefill_flops(w) -> dict:
    S, E, d = w.B * w.S, w.E, w.d
    nq, nk = w.Hq * d, w.Hkv * d
    return {
        "proj_down": 2.0 * S * E * (nq + 2 * nk),
        "mix": 2.0 * S * (w.Hq * w.kq + w.Hkv * w.kk) * d * d,
        "attn": w.B * attention_flops(w.S, w.Hq, d),
        "proj_up": 2.0 * S * nq * E,
    }


def attention_traffic_bytes():
    """HBM bytes per attention launch from the committed rocprofv3 PMC record
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the counter
    reads for a plain copy of known size), or None when the attention kernel's
    source has changed since the counters were taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "attn_prefill_16k_traffic.txt")
    src_path = os.path.join(ROOT, "compressed_latent_attention_amd", "csrc", "attn_mfma.hip")
    try:
        rec = {}
        for line in open(rec_path):
            if line.strip() and not line.startswith("#"):
                k, v = line.split()[:2]
                rec[k] = v
        if hashlib.sha256(open(src_path, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        return (float(rec["fetch_kib"]) * 1024 * float(rec["fetch_scale"]) +
                float(rec["write_kib"]) * 1024 * float(rec["write_scale"]))
    except (OSError, KeyError, ValueError):
        return None


def time_oracle_forward(w, inp):
    """The float64 oracle's forward over the whole workload (every token, every
    step: projections, convolution, QK-mean, shift, RoPE, attention, W_o),
    timed once, wall clock, on the host cores numpy's BLAS uses."""
    from oracle import cca as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    spec = O.Spec(E=w.E, C=w.C, Hq=w.Hq, Hkv=w.Hkv, kq=w.kq, kk=w.kk, rope_base=w.rope_base,
                  s_v=w.s_v)
    p = {k: inp[k] for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    t0 = time.perf_counter()
    O.forward(inp["x"], p, spec)
    sec = time.perf_counter() - t0
    return {"value": w.B * w.S / sec, "unit": "tokens/s", "cores": int(threads),
            "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": (f"the whole workload, not a sample: float64 numpy oracle forward over "
                       f"all {w.B * w.S} tokens in {sec:.1f} s, one run, BLAS threads "
                       f"{threads} of {os.cpu_count()} host CPUs")}


def bench_prefill(args, torch, cca, w, inp, fused=False):
    dt = torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, w.capacity, w.kq, w.kk, w.s_v, w.flags,
                         w.rope_base, w.dtype)
    if fused:
        layer.set_prefill_fusion(True)
    wts = {k: dev(inp[k]) for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    x = dev(inp["x"])
    B, S = w.B, w.S
    y = torch.empty_like(x)
    ws = layer.workspace(cca.CCA_OP_PREFILL, B, S)
    stream = torch.cuda.current_stream()

    def step():
        cca.cca_forward_prefill(layer.handle, wts, x, B, S, y, None, None, None, None, ws, stream)

    # W warm-up steps, then more until at least args.warm_s seconds of steps
    # have run: the shader clock takes ~0.1 s of load to settle
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_steps = args.warmup
    while time.perf_counter() - t0 < args.warm_s:
        for _ in range(20):
            step()
        warm_steps += 20
        torch.cuda.synchronize()
    # the step time: K steps with nothing recorded between the kernels
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the kernel durations: K more steps with HIP events recorded around every
    # launch on the launch stream (the events themselves add ~7 us per kernel
    # to the step, so this loop's step time is reported apart)
    cca.cca_profile_enable(layer.handle, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - t0
    prof = cca.cca_profile_read(layer.handle)
    cca.cca_profile_enable(layer.handle, False)
    return elapsed, elapsed_prof, prof, layer, warm_steps


def mix_bytes(w) -> dict:
    """Algorithmic HBM bytes of the mix over one prefill: the bf16 latent
    q~|k~|v~ read once, the conv taps, and Q'', K'', V' written once; plus the
    fp32 cos/sin rows of the RoPE table this implementation reads (listed
    apart)."""
    d, nq, nk = w.d, w.Hq * w.d, w.Hkv * w.d
    tokens = w.B * w.S
    return {"latent_in": tokens * (nq + 2 * nk) * 2.0,
            "taps": (w.Hq * w.kq + w.Hkv * w.kk) * d * d * 2.0,
            "out": tokens * (nq + 2 * nk) * 2.0,
            "rope_table": w.S * (d // 2) * 8.0}


def bench_mix_cold(args, torch, cca, w, inp):
    """The mix kernel of the 16k prefill timed alone with cold caches: before
    each timed launch the library writes a 1 GiB buffer (evicting L2 and the
    256 MB MALL), so its inputs come from HBM."""
    dt = torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, w.capacity, w.kq, w.kk, w.s_v, w.flags,
                         w.rope_base, w.dtype)
    wts = {k: dev(inp[k]) for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    x = dev(inp["x"])
    y = torch.empty_like(x)
    ws = layer.workspace(cca.CCA_OP_PREFILL, w.B, w.S)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        cca.cca_forward_prefill(layer.handle, wts, x, w.B, w.S, y, None, None, None, None, ws,
                                stream)

    _time_warm(torch, step, 10)
    cca.cca_profile_enable(layer.handle, True)
    cca.cca_profile_flush(layer.handle, flush)
    n = max(args.steps // 5, 5)
    _time_loop(torch, step, n, 0)
    prof = cca.cca_profile_read(layer.handle)
    cca.cca_profile_flush(layer.handle, None)
    cca.cca_profile_enable(layer.handle, False)
    layer.close()
    del flush
    torch.cuda.empty_cache()
    launches, total = prof["mix"]
    ms = total / max(launches, 1)
    by = mix_bytes(w)
    alg = by["latent_in"] + by["taps"] + by["out"]
    return {"workload": f"ccgqa_prefill_16k mix (conv, QK-mean, value shift, RoPE): S={w.S}, "
                        f"Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, bf16",
            "avg_ms_cold": ms, "launches": launches,
            "bytes_algorithmic": alg,
            "bytes_note": "bf16 latent q~|k~|v~ read once + taps + Q'', K'', V' written once; "
                          f"the fp32 RoPE table rows ({by['rope_table'] / 1e6:.1f} MB) not counted",
            "GBps": alg / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "timing": "HIP events around each mix launch, a 1 GiB write before each (L2 and MALL "
                      "evicted)",
            "other_kernels_cold_ms": {k: v[1] / max(v[0], 1) for k, v in prof.items()}}


DECODE_BYTES_NOTE = ("K and V caches over positions 0..pos of every sequence + all weights "
                     "+ x_new, y_new, the rolling state and the new cache rows")


def decode_bytes(w, positions=None) -> float:
    """Algorithmic HBM bytes of one decode step: the cache rows attention reads
    (positions 0..pos, K and V), every weight once, and the per-token
    activations (x_new, y_new, the state read and written, the cache rows
    written)."""
    es = 2
    d, nq, nk = w.d, w.Hq * w.d, w.Hkv * w.d
    keys = w.B * (w.S + 1) if positions is None else sum(int(p) + 1 for p in positions)
    cache = 2.0 * w.Hkv * keys * d * es
    weights = (w.E * (nq + 2 * nk) + w.E * nq + (w.Hq * w.kq + w.Hkv * w.kk) * d * d) * es
    state_w = (w.kq - 1) * nq + (w.kk - 1) * nk + nk
    acts = w.B * (2 * w.E + 2 * state_w + 2 * nk) * es
    return cache + weights + acts


def backward_flops(w) -> dict:
    """Algorithmic FLOPs of one backward pass: the attention backward as five
    causal matmuls (S recompute, dP, dV, dQ, dK), the four projection GEMM
    gradients (dx and dW for W_o and for W_qkv) and the conv gradients."""
    S, E, d = w.B * w.S, w.E, w.d
    nq, nk = w.Hq * d, w.Hkv * d
    attn = 5.0 / 2.0 * w.B * attention_flops(w.S, w.Hq, d)
    gemm = 2.0 * (2.0 * S * nq * E) + 2.0 * (2.0 * S * E * (nq + 2 * nk))
    conv = 2.0 * (2.0 * S * (w.Hq * w.kq + w.Hkv * w.kk) * d * d)
    return {"attn": attn, "gemm": gemm, "conv": conv}


def _time_loop(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def _time_warm(torch, fn, steps, warm_s=0.15):
    """Mean seconds per call over `steps` calls after at least `warm_s` seconds
    of untimed calls (sized from one probe call): the shader clock takes tens
    of milliseconds of load to settle after the host-side set-up between
    configurations."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-5)
    return _time_loop(torch, fn, steps, max(steps, int(warm_s / one)))


def ragged_positions(B=32, cap=32768, seed=13):
    """A ragged decode batch: a quarter of the sequences long (16k..32k cached
    tokens), the rest short (512..4096), seeded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_long = B // 4
    pos = [int(rng.integers(16384, cap)) for _ in range(n_long)]
    pos += [int(rng.integers(512, 4097)) for _ in range(B - n_long)]
    rng.shuffle(pos)
    return pos


def bench_decode(args, torch, cca, hkv=None, w=None, positions=None):
    """32-sequence CCGQA decode step over a 32768-token cache.  The cache, the
    state and x_new are drawn on the GPU from a seeded torch generator (N(0,1),
    the same law as the parity workload; the timing does not depend on the
    values), the weights from the seeded parity recipe."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs
    w = w or WORKLOADS["ccgqa_decode_32k"]
    if hkv is not None:
        w = w.replace(Hkv=hkv)
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, w.capacity, w.kq, w.kk, w.s_v, w.flags,
                         w.rope_base, w.dtype)
    wi = make_inputs(w.replace(S=1, B=1))     # weights only (same draw order and seed)
    dt = torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    wts = {k: dev(wi[k]) for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    shape = (w.B, w.Hkv, w.capacity, w.d)
    kc = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dt)
    vc = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dt)
    st = torch.randn((w.B, layer.state_width()), generator=gen, device="cuda").to(dt)
    xn = torch.randn((w.B, w.E), generator=gen, device="cuda").to(dt)
    pos = [w.S] * w.B if positions is None else list(positions)
    ws = layer.workspace(cca.CCA_OP_DECODE, w.B, 0)
    yn = torch.empty_like(xn)
    stream = torch.cuda.current_stream()
    arr_pos = pos

    def step():
        cca.cca_decode_step(layer.handle, wts, xn, arr_pos, w.B, kc, vc, st, yn, ws, stream)

    steps = max(args.steps, 10)
    sec = _time_warm(torch, step, steps)
    cca.cca_profile_enable(layer.handle, True)
    _time_loop(torch, step, 5, 0)
    prof = cca.cca_profile_read(layer.handle)
    cca.cca_profile_enable(layer.handle, False)
    byts = decode_bytes(w, positions)
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0]} for k, v in prof.items()}
    attn_ms = kernels.get("decode_attn", {}).get("avg_ms", float("nan"))
    cache_bytes = 2.0 * w.Hkv * sum(p + 1 for p in pos) * w.d * 2
    layer.close()
    cached = (f"cache {w.S} tokens" if positions is None else
              f"ragged caches of {min(pos)}..{max(pos)} tokens ({sum(pos)} in all)")
    return {
        "workload": f"{w.name}: B={w.B}, {cached}, E={w.E}, Hq={w.Hq}, "
                    f"Hkv={w.Hkv}, d={w.d}, bf16",
        "tokens_per_s": w.B / sec,
        "ms_per_step": sec * 1e3,
        "hbm_bytes_per_step": byts,
        "bytes_note": DECODE_BYTES_NOTE,
        "GBps": byts / sec / 1e9,
        "frac_of_hbm_peak": byts / sec / 1e9 / PEAK_HBM_GBS,
        "attn_kernel": {"avg_ms": attn_ms, "cache_bytes": cache_bytes,
                        "GBps": cache_bytes / (attn_ms * 1e-3) / 1e9,
                        "frac_of_hbm_peak": cache_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "kernels": kernels,
    }


def bench_backward(args, torch, cca, w=None):
    """CCGQA backward at S=16384 from a saved prefill of the same seeded x."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs
    w = w or WORKLOADS["ccgqa_backward_16k"]
    inp = make_inputs(w)
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, w.capacity, w.kq, w.kk, w.s_v, w.flags,
                         w.rope_base, w.dtype)
    dt = torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    wts = {k: dev(inp[k]) for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    x, dy = dev(inp["x"]), dev(inp["dy"])
    saved = torch.empty(layer.saved_bytes(w.B, w.S), dtype=torch.uint8, device="cuda")
    layer.forward_prefill(wts, x, saved=saved)
    grads = {"dx": torch.empty_like(x)}
    for n in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k"):
        grads["d" + n] = torch.empty(wts[n].shape, dtype=torch.float32, device="cuda")
    ws = layer.workspace(cca.CCA_OP_BACKWARD, w.B, w.S)
    stream = torch.cuda.current_stream()

    def step():
        cca.cca_backward(layer.handle, wts, x, dy, saved, w.B, w.S, grads, ws, stream)

    steps = max(1, args.bwd_steps)
    sec = _time_warm(torch, step, steps)
    cca.cca_profile_enable(layer.handle, True)
    _time_loop(torch, step, 1, 0)
    prof = cca.cca_profile_read(layer.handle)
    cca.cca_profile_enable(layer.handle, False)
    fl = backward_flops(w)
    total = sum(fl.values())
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0]} for k, v in prof.items()}
    layer.close()
    return {
        "workload": f"{w.name}: B={w.B}, S={w.S}, E={w.E}, Hq={w.Hq}, Hkv={w.Hkv}, "
                    f"d={w.d}, bf16 storage, fp32 accumulation",
        "tokens_per_s": w.B * w.S / sec,
        "ms_per_step": sec * 1e3,
        "flops_per_step": total,
        "flops_note": "attention backward as 5 causal matmuls (S recompute, dP, dV, dQ, dK) + "
                      "4 projection GEMM gradients + conv tap and input gradients",
        "TFLOPs": total / sec / 1e12,
        "frac_of_bf16_peak": total / sec / 1e12 / PEAK_BF16_TFLOPS,
        "kernels": kernels,
    }


def bench_fused(args, torch, cca, w, inp):
    """The 16k prefill with the query side of the mix fused into the attention
    (cca_set_prefill_fusion) against the separate passes, alternately on the
    same layer, same warm-up: step times and kernel times of both."""
    out = {"note": "fused: the attention forms Q'' from the bf16 latent and the mix writes no Q''; "
                   "separate: the default path (the headline row)"}
    a2 = argparse.Namespace(**vars(args))
    a2.steps = 30
    res = {}
    for rep_i in range(2):
        for mode in ("separate", "fused"):
            elapsed, _, prof, layer, _ = bench_prefill(a2, torch, cca, w, inp,
                                                       fused=(mode == "fused"))
            layer.close()
            ms = elapsed * 1e3 / a2.steps
            kern = {k: round(v[1] / max(v[0], 1) * 1e3, 2) for k, v in prof.items()}
            if mode not in res or ms < res[mode]["ms_per_step"]:
                res[mode] = {"ms_per_step": ms, "kernels_us": kern}
    out.update(res)
    out["fused_over_separate"] = res["fused"]["ms_per_step"] / res["separate"]["ms_per_step"]
    return out


def bench_varlen(args, torch, cca):
    """Chunked variable-length prefill of the CCGQA layer (16 chunks, 16384 new
    tokens in all, over caches of up to 32768 tokens): tokens/s and the
    attention kernel's MFMA fraction (algorithmic FLOPs: every new query
    against its cached and earlier new keys)."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs, varlen_layout
    w = WORKLOADS["ccgqa_prefill_16k"]
    cap = 32768
    offsets, starts = varlen_layout(cap=cap)
    T = int(offsets[-1])
    wi = make_inputs(w.replace(S=1, B=1))
    dt = torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    wts = {k: dev(wi[k]) for k in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, cap, w.kq, w.kk, w.s_v, w.flags, w.rope_base,
                         w.dtype)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    B = len(starts)
    shape = (B, w.Hkv, cap, w.d)
    kc = torch.randn(shape, generator=gen, device="cuda").to(dt)
    vc = torch.randn(shape, generator=gen, device="cuda").to(dt)
    st = torch.randn((B, layer.state_width()), generator=gen, device="cuda").to(dt)
    x = torch.randn((T, w.E), generator=gen, device="cuda").to(dt)
    y = torch.empty_like(x)
    n = cca.cca_varlen_workspace_bytes(layer.handle, offsets.tolist(), starts.tolist())
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    offs, sts = offsets.tolist(), starts.tolist()

    def step():
        # the caches and states advance every call; the positions stay the
        # same, so every call does the same work
        cca.cca_forward_prefill_varlen(layer.handle, wts, x, offs, sts, y, kc, vc, st, ws, stream)

    sec = _time_warm(torch, step, 20)
    cca.cca_profile_enable(layer.handle, True)
    _time_loop(torch, step, 10, 0)
    prof = cca.cca_profile_read(layer.handle)
    cca.cca_profile_enable(layer.handle, False)
    layer.close()
    lens = np.diff(offsets)
    pairs = float(sum(int(n) * int(s) + int(n) * (int(n) + 1) // 2 for n, s in zip(lens, starts)))
    attn_fl = 4.0 * w.Hq * w.d * pairs
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0]} for k, v in prof.items()}
    attn_ms = kernels.get("varlen_attn", {}).get("avg_ms", float("nan"))
    return {"workload": f"ccgqa chunked prefill: {B} chunks, {T} new tokens (lengths "
                        f"{int(lens.min())}..{int(lens.max())}) at cached lengths "
                        f"{int(starts.min())}..{int(starts.max())}, capacity {cap}, E={w.E}, "
                        f"Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, bf16",
            "tokens_per_s": T / sec, "ms_per_call": sec * 1e3,
            "attn_flops": attn_fl, "attn_tflops": attn_fl / (attn_ms * 1e-3) / 1e12,
            "attn_frac_of_bf16_peak": attn_fl / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "kernels": kernels}


def bench_d64(args, torch, cca):
    """The CCGQA layer with head dimension 64 (8 query and 4 KV heads of 64:
    the same latent widths and KV-cache size as the d = 128 layer): the 16k
    prefill with its kernel times and the attention's MFMA fraction, the
    decode step over a 32k cache and the 16k backward."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs
    w = WORKLOADS["ccgqa_d64_prefill_16k"]
    inp = make_inputs(w)
    a2 = argparse.Namespace(**vars(args))
    a2.steps = 20
    elapsed, _, prof, layer, _ = bench_prefill(a2, torch, cca, w, inp)
    layer.close()
    ms = elapsed * 1e3 / a2.steps
    fl = prefill_flops(w)
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0],
                   "tflops": (fl[k] / (v[1] / max(v[0], 1) * 1e-3) / 1e12) if k in fl else None}
               for k, v in prof.items()}
    attn = kernels.get("attn", {})
    pre = {"workload": f"{w.name}: B={w.B}, S={w.S}, E={w.E}, C={w.C}, Hq={w.Hq}, Hkv={w.Hkv}, "
                       f"d={w.d}, bf16",
           "tokens_per_s": w.B * w.S / elapsed * a2.steps, "ms_per_step": ms,
           "layer_frac_of_bf16_peak": sum(fl.values()) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "attn_frac_of_bf16_peak": (attn.get("tflops") or float("nan")) / PEAK_BF16_TFLOPS,
           "kernels": kernels}
    dec = bench_decode(args, torch, cca,
                       w=WORKLOADS["ccgqa_decode_32k"].replace(name="ccgqa_d64_decode_32k", Hq=8,
                                                               Hkv=4))
    bwd = bench_backward(args, torch, cca,
                         w=w.replace(name="ccgqa_d64_backward_16k", kind="backward"))
    return {"prefill": pre, "decode": dec, "backward": bwd}


def bench_cca4k(args, torch, cca):
    """The CCA prefill at S = 4096 (B = 1, E = 2048, C = 4, 4 query and 4 KV
    heads of 128, no head sharing): tokens/s, the layer's and the attention's
    fraction of the dense bf16 peak and the kernel times.  A shorter sequence
    puts more of the layer in the projections (attention is ~32% of its FLOPs)."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs
    w = WORKLOADS["cca_prefill_4k"]
    inp = make_inputs(w)
    a2 = argparse.Namespace(**vars(args))
    a2.steps = max(args.steps, 50)
    elapsed, _, prof, layer, warm = bench_prefill(a2, torch, cca, w, inp)
    layer.close()
    ms = elapsed * 1e3 / a2.steps
    fl = prefill_flops(w)
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0],
                   "tflops": (fl[k] / (v[1] / max(v[0], 1) * 1e-3) / 1e12) if k in fl else None}
               for k, v in prof.items()}
    attn = kernels.get("attn", {})
    return {"workload": f"{w.name}: B={w.B}, S={w.S}, E={w.E}, C={w.C}, Hq={w.Hq}, Hkv={w.Hkv}, "
                        f"d={w.d}, bf16",
            "tokens_per_s": w.B * w.S / elapsed * a2.steps, "ms_per_step": ms,
            "warmup_steps": warm,
            "layer_tflops": sum(fl.values()) / (ms * 1e-3) / 1e12,
            "layer_frac_of_bf16_peak": sum(fl.values()) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "attn_frac_of_bf16_peak": (attn.get("tflops") or float("nan")) / PEAK_BF16_TFLOPS,
            "kernels": kernels}


def _gpu_layer(torch, cca, w, gen):
    """A layer of workload w with weights drawn on the GPU (seeded N(0, 1)
    scaled like the parity recipe; the timing does not depend on the values)."""
    layer = cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, w.capacity, w.kq, w.kk, w.s_v, w.flags,
                         w.rope_base, w.dtype)
    d, E = w.d, w.E
    rnd = lambda shape, std: (torch.randn(shape, generator=gen, device="cuda") * std).to(
        torch.bfloat16)
    wts = {"w_q": rnd((w.Hq * d, E), E ** -0.5), "w_k": rnd((w.Hkv * d, E), E ** -0.5),
           "w_v": rnd((w.Hkv * d, E), E ** -0.5), "w_o": rnd((E, w.Hq * d), E ** -0.5),
           "conv_q": rnd((w.Hq, w.kq, d, d), (w.kq * d) ** -0.5),
           "conv_k": rnd((w.Hkv, w.kk, d, d), (w.kk * d) ** -0.5)}
    return layer, wts, rnd


N1_SWEEP = (4096, 8192, 16384, 32768, 65536)





def bench_n1(args, torch, cca):
    """The same-GPU comparators: prefill of the CCGQA layer and of MHA and GQA
    of the same hidden size through the same kernels (C = 1, 16 query heads of
    128, a one-tap convolution, no QK-mean or value shift) over S = 4k .. 64k,
    and the backward of all three at 16k.  MHA's layer time includes the mix
    pass its one-tap convolution still runs; `mha_core_ms` sums only its
    projections and attention (kernel events, a second loop)."""
    from compressed_latent_attention_amd.synthetic import WORKLOADS
    base = {n: WORKLOADS[k] for n, k in (("ccgqa", "ccgqa_prefill_16k"),
                                         ("mha", "mha_prefill_16k"),
                                         ("gqa", "gqa_prefill_16k"),
                                         ("ccgqa16", "ccgqa16_prefill_16k"))}
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    sweep = []
    for S in N1_SWEEP:
        row = {"S": S}
        for name, w0 in base.items():
            w = w0.replace(S=S)
            gen.manual_seed(w.seed)
            layer, wts, rnd = _gpu_layer(torch, cca, w, gen)
            x = rnd((1, S, w.E), 1.0)
            y = torch.empty_like(x)
            ws = layer.workspace(cca.CCA_OP_PREFILL, 1, S)

            def step():
                cca.cca_forward_prefill(layer.handle, wts, x, 1, S, y, None, None, None, None,
                                        ws, stream)

            steps = 20 if S <= 8192 else 5
            row[name + "_ms"] = _time_warm(torch, step, steps) * 1e3
            if name == "mha":
                cca.cca_profile_enable(layer.handle, True)
                _time_loop(torch, step, steps, 0)
                prof = cca.cca_profile_read(layer.handle)
                cca.cca_profile_enable(layer.handle, False)
                row["mha_core_ms"] = sum(v[1] / max(v[0], 1) for k, v in prof.items()
                                         if k in ("proj_down", "attn", "proj_up"))
            layer.close()
            del x, y, ws, wts
        row["mha_over_ccgqa"] = row["mha_ms"] / row["ccgqa_ms"]
        row["mha_core_over_ccgqa"] = row["mha_core_ms"] / row["ccgqa_ms"]
        row["gqa_over_ccgqa"] = row["gqa_ms"] / row["ccgqa_ms"]
        row["ccgqa16_over_ccgqa"] = row["ccgqa16_ms"] / row["ccgqa_ms"]
        sweep.append(row)
        torch.cuda.empty_cache()
    bwd = {}
    for name, w0 in base.items():
        w = w0.replace(kind="backward")
        gen.manual_seed(w.seed)
        layer, wts, rnd = _gpu_layer(torch, cca, w, gen)
        x, dy = rnd((1, w.S, w.E), 1.0), rnd((1, w.S, w.E), 1.0)
        saved = torch.empty(layer.saved_bytes(1, w.S), dtype=torch.uint8, device="cuda")
        layer.forward_prefill(wts, x, saved=saved)
        grads = {"dx": torch.empty_like(x)}
        for n in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k"):
            grads["d" + n] = torch.empty(wts[n].shape, dtype=torch.float32, device="cuda")
        ws = layer.workspace(cca.CCA_OP_BACKWARD, 1, w.S)

        def bstep():
            cca.cca_backward(layer.handle, wts, x, dy, saved, 1, w.S, grads, ws, stream)

        bwd[name + "_ms"] = _time_warm(torch, bstep, max(1, args.bwd_steps)) * 1e3
        layer.close()
        del x, dy, saved, grads, ws, wts
        torch.cuda.empty_cache()
    bwd["mha_over_ccgqa"] = bwd["mha_ms"] / bwd["ccgqa_ms"]
    bwd["gqa_over_ccgqa"] = bwd["gqa_ms"] / bwd["ccgqa_ms"]
    bwd["ccgqa16_over_ccgqa"] = bwd["ccgqa16_ms"] / bwd["ccgqa_ms"]
    # decode over a 32k-token cache: one KV head halves the cache the step reads
    d2 = bench_decode(args, torch, cca)
    d1 = bench_decode(args, torch, cca, hkv=1)
    dec = {"ccgqa_ms": d2["ms_per_step"], "ccgqa16_ms": d1["ms_per_step"],
           "ccgqa16_over_ccgqa": d1["ms_per_step"] / d2["ms_per_step"],
           "ccgqa16_frac_of_hbm_peak": d1["frac_of_hbm_peak"]}
    return {"note": "same-GPU comparators through the same kernels: MHA = C 1, 16 heads of 128, "
                    "one-tap convolution, RoPE, no QK-mean or value shift; GQA = the same with "
                    "2 KV heads (the CCGQA layer's KV-cache size); ccgqa16 = the CCGQA layer "
                    "with one KV head (16x); E = 2048, B = 1, bf16",
            "prefill": sweep, "backward_16k": bwd, "decode_32k": dec}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~0.1 s of prefill steps: fewer left the shader clock still ramping in the
    # timed loop (0.475 vs 0.451 ms per step after 5 and after ~100 steps)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-s", type=float, default=0.3,
                    help="untimed prefill steps continue past --warmup until this many seconds")
    ap.add_argument("--rows", default="prefill,cca4k,mix,fused,varlen,decode,backward,d64",
                    help="comma list: prefill (headline, always run), cca4k (the CCA prefill at "
                         "S = 4096, four query and four KV heads), mix (the mix kernel with "
                         "cold caches), fused (the prefill with the query side of the mix in "
                         "the attention, against the separate passes), varlen (the chunked "
                         "variable-length prefill), decode, backward, d64 "
                         "(the head-dimension-64 layer: prefill, decode, backward); n1 adds the "
                         "MHA / GQA comparators over S = 4k .. 64k (not run by default)")
    ap.add_argument("--bwd-steps", type=int, default=3, help="timed backward steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (steps times), the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": args.steps}), flush=True)
        return
    import compressed_latent_attention_amd as cca
    from compressed_latent_attention_amd.synthetic import WORKLOADS, make_inputs

    w = WORKLOADS["ccgqa_prefill_16k"]
    inp = make_inputs(w)
    elapsed, elapsed_prof, prof, _, warm_steps = bench_prefill(args, torch, cca, w, inp)
    ms = elapsed * 1000.0 / args.steps
    tokens = w.B * w.S * args.steps
    fl = prefill_flops(w)
    launches, total_ms = prof.get("attn", (0, 0.0))
    attn_ms = total_ms / max(launches, 1)
    attn_tflops = fl["attn"] / (attn_ms * 1e-3) / 1e12
    kernels = {k: {"avg_ms": v[1] / max(v[0], 1), "launches": v[0],
                   "tflops": (fl[k] / (v[1] / max(v[0], 1) * 1e-3) / 1e12) if k in fl else None}
               for k, v in prof.items()}
    total_flops = sum(fl.values())
    out = {
        "metric": "CCGQA prefill tokens/sec at S=16k, E=2048 (1 GPU) + % bf16 MFMA peak",
        "value": tokens / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_note": f"{warm_steps} untimed steps ran before the timed ones: the {args.warmup} "
                       f"asked for, then more until {args.warm_s} s of steps had run (the "
                       f"shader clock settles after ~0.1 s of load)",
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ccgqa_prefill_16k", "global_batch": w.B, "seq_len": w.S,
                   "E": w.E, "C": w.C, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "conv_kernels": [w.kq, w.kk], "parallelism": "none (1 GPU)"},
        "layer_tflops": total_flops / (ms * 1e-3) / 1e12,
        "layer_frac_of_bf16_peak": total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "attn", "achieved": attn_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": attention_traffic_bytes(),
                     "flops_per_launch": fl["attn"], "avg_launch_ms": attn_ms,
                     "timing": f"HIP events around each launch on the launch stream over a second "
                               f"timed loop of {args.steps} steps"},
        "kernels": kernels,
        "ms_per_step_with_kernel_events": elapsed_prof * 1000.0 / args.steps,
    }
    rows = [r.strip() for r in args.rows.split(",") if r.strip()]
    if "cca4k" in rows:
        out["cca_prefill_4k"] = bench_cca4k(args, torch, cca)
    if "mix" in rows:
        out["mix_cold"] = bench_mix_cold(args, torch, cca, w, inp)
    if "fused" in rows:
        out["fused_q"] = bench_fused(args, torch, cca, w, inp)
    if "varlen" in rows:
        out["varlen"] = bench_varlen(args, torch, cca)
    if "decode" in rows:
        out["decode"] = bench_decode(args, torch, cca)
        out["decode_ragged"] = bench_decode(args, torch, cca, positions=ragged_positions())
    if "backward" in rows:
        out["backward"] = bench_backward(args, torch, cca)
    if "d64" in rows:
        out["d64"] = bench_d64(args, torch, cca)
    if "n1" in rows:
        out["n1"] = bench_n1(args, torch, cca)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = time_oracle_forward(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
