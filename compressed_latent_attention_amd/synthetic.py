"""Seeded synthetic workloads for the CCA / CCGQA layer.

This module only draws random numbers and describes shapes. It holds none of
the layer's arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it without sharing any computation.

Recipe (the pages publish no workload beyond "16k tokens", so these shapes and
distributions stand in for it):

* generator: ``numpy.random.Generator(PCG64(seed))``, ``standard_normal`` in
  float64, drawn in chunks of at most 2**24 values, scaled, cast to float32;
  for bf16 workloads then rounded to bf16 with round-to-nearest-even before
  either side sees the value;
* draw order: x, W_q, W_k, W_v, W_o, A_q, A_k, then dY (backward workload) or
  K cache, V cache, rolling state, x_new (decode workload; that workload has no
  x and starts at W_q);
* x, dY, caches, state ~ N(0, 1); projections ~ N(0, 1/E); conv taps
  ~ N(0, 1/(kernel * head_dim)).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int                 # prefill length (decode: cached tokens per sequence)
    E: int
    C: int
    Hq: int
    Hkv: int
    kq: int = 2
    kk: int = 2
    sv: Optional[int] = None   # shifted V channels per KV head; None = d/2
    rope_base: float = 10000.0
    dtype: str = "bf16"        # "f32" or "bf16"
    seed: int = 0
    kind: str = "prefill"      # "prefill" | "decode" | "backward"
    max_seq_len: Optional[int] = None
    flags: int = 15

    @property
    def d(self) -> int:
        return self.E // (self.C * self.Hq)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def s_v(self) -> int:
        return self.d // 2 if self.sv is None else self.sv

    @property
    def capacity(self) -> int:
        if self.max_seq_len is not None:
            return self.max_seq_len
        return self.S + 64 if self.kind == "decode" else self.S

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny fp32 CCA, CCA prefill at 4k, CCGQA prefill at 16k,
# CCGQA decode over a 32768-token cache, CCGQA backward at 16k; then the two
# same-GPU comparators of the same hidden size run through the same kernels:
# MHA (no compression, 16 heads of 128, one-tap convolution, no QK-mean, no
# value shift, RoPE kept) and GQA (the same with 2 KV heads, the KV-cache
# size of the CCGQA layer); and the CCGQA layer with one KV head (16x).
WORKLOADS: Dict[str, Workload] = {
    "cca_tiny_f32": Workload("cca_tiny_f32", B=1, S=128, E=256, C=4, Hq=4, Hkv=4,
                             dtype="f32", seed=1),
    "cca_prefill_4k": Workload("cca_prefill_4k", B=1, S=4096, E=2048, C=4, Hq=4, Hkv=4,
                               seed=2),
    "ccgqa_prefill_16k": Workload("ccgqa_prefill_16k", B=1, S=16384, E=2048, C=4, Hq=4,
                                  Hkv=2, seed=3),
    "ccgqa_decode_32k": Workload("ccgqa_decode_32k", B=32, S=32768, E=2048, C=4, Hq=4,
                                 Hkv=2, seed=4, kind="decode", max_seq_len=32832),
    "ccgqa_backward_16k": Workload("ccgqa_backward_16k", B=1, S=16384, E=2048, C=4, Hq=4,
                                   Hkv=2, seed=5, kind="backward"),
    "mha_prefill_16k": Workload("mha_prefill_16k", B=1, S=16384, E=2048, C=1, Hq=16, Hkv=16,
                                kq=1, kk=1, flags=4, seed=6),
    "gqa_prefill_16k": Workload("gqa_prefill_16k", B=1, S=16384, E=2048, C=1, Hq=16, Hkv=2,
                                kq=1, kk=1, flags=4, seed=7),
    # the 16x-compressed variant: one KV head (half the CCGQA layer's KV cache)
    "ccgqa16_prefill_16k": Workload("ccgqa16_prefill_16k", B=1, S=16384, E=2048, C=4, Hq=4,
                                    Hkv=1, seed=8),
    # head dimension 64: the same latent (512 query, 256 KV channels) as 8 query
    # heads and 4 KV heads of 64, so the same 8x smaller KV cache than MHA
    "ccgqa_d64_prefill_16k": Workload("ccgqa_d64_prefill_16k", B=1, S=16384, E=2048, C=4, Hq=8,
                                      Hkv=4, seed=9),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "value is not bf16-exact"
    return (u >> 16).astype(np.uint16)


class _Drawer:
    def __init__(self, seed: int, dtype: str):
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.dtype = dtype

    def normal(self, shape, std: float) -> np.ndarray:
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for s in range(0, n, _CHUNK):
            e = min(n, s + _CHUNK)
            out[s:e] = (self.rng.standard_normal(e - s) * std).astype(np.float32)
        if self.dtype == "bf16":
            for s in range(0, n, _CHUNK):
                out[s:s + _CHUNK] = round_bf16(out[s:s + _CHUNK])
        return out.reshape(shape)


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of workload ``w`` as float32 arrays (bf16-exact when
    ``w.dtype == 'bf16'``).  Shapes:

    x [B,S,E]; w_q [Hq*d,E]; w_k, w_v [Hkv*d,E]; w_o [E,Hq*d];
    conv_q [Hq,kq,d,d]; conv_k [Hkv,kk,d,d] (tap j multiplies lag j);
    backward: dy [B,S,E];
    decode: k_cache, v_cache [B,Hkv,cap,d] (slots >= S are zero), state
    [B, (kq-1)*Hq*d + (kk-1)*Hkv*d + Hkv*d], x_new [B,E], pos [B] int32 (= S).
    """
    dr = _Drawer(w.seed if seed is None else seed, w.dtype)
    d, E = w.d, w.E
    wstd = 1.0 / np.sqrt(E)
    out: Dict[str, np.ndarray] = {}
    if w.kind != "decode":
        out["x"] = dr.normal((w.B, w.S, E), 1.0)
    out["w_q"] = dr.normal((w.Hq * d, E), wstd)
    out["w_k"] = dr.normal((w.Hkv * d, E), wstd)
    out["w_v"] = dr.normal((w.Hkv * d, E), wstd)
    out["w_o"] = dr.normal((E, w.Hq * d), wstd)
    out["conv_q"] = dr.normal((w.Hq, w.kq, d, d), 1.0 / np.sqrt(w.kq * d))
    out["conv_k"] = dr.normal((w.Hkv, w.kk, d, d), 1.0 / np.sqrt(w.kk * d))
    if w.kind == "backward":
        out["dy"] = dr.normal((w.B, w.S, E), 1.0)
    if w.kind == "decode":
        cap = w.capacity
        for name in ("k_cache", "v_cache"):
            c = np.zeros((w.B, w.Hkv, cap, d), dtype=np.float32)
            for b in range(w.B):
                c[b, :, :w.S, :] = dr.normal((w.Hkv, w.S, d), 1.0)
            out[name] = c
        out["state"] = dr.normal((w.B, state_width(w)), 1.0)
        out["x_new"] = dr.normal((w.B, E), 1.0)
        out["pos"] = np.full((w.B,), w.S, dtype=np.int32)
    return out


def varlen_layout(total: int = 16384, nseq: int = 16, cap: int = 32768, seed: int = 11):
    """A serving-like chunked prefill batch: nseq chunks of ragged lengths
    (uniform in [total / (2 nseq), 3 total / (2 nseq)], scaled to sum to
    total) continuing sequences at ragged cached lengths (uniform below
    cap - chunk).  Returns (offsets [nseq + 1], starts [nseq]) as int64."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.uniform(0.5, 1.5, nseq)
    lens = np.floor(lens / lens.sum() * total).astype(np.int64)
    lens[-1] += total - lens.sum()
    starts = np.array([int(rng.integers(0, cap - n + 1)) for n in lens], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(lens)])
    return offsets, starts


def state_width(w: Workload) -> int:
    """Elements of rolling decode state per sequence: [q lags 1..kq-1 |
    k lags 1..kk-1 | v at lag 1], most recent lag first."""
    return (w.kq - 1) * w.Hq * w.d + (w.kk - 1) * w.Hkv * w.d + w.Hkv * w.d


def identity_taps(H: int, k: int, d: int) -> np.ndarray:
    """Taps that make the convolution a pass-through (tap 0 = I, others 0)."""
    a = np.zeros((H, k, d, d), dtype=np.float32)
    for h in range(H):
        a[h, 0] = np.eye(d, dtype=np.float32)
    return a
