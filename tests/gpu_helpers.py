"""Shared plumbing of the GPU parity tests: moving seeded inputs to the
device, running the library through its C ABI, and the oracle spec matching a
workload.  No layer arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import compressed_latent_attention_amd as cca
from compressed_latent_attention_amd.synthetic import Workload, make_inputs
from oracle import cca as O

WEIGHT_NAMES = ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")
# relative L2 error bounds: fp32 workloads 1e-5, bf16 workloads 1e-2
TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def tdtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(a: np.ndarray, w: Workload) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        device="cuda", dtype=tdtype(w))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def block_rel(a, b, axis: int, block: int = 128) -> float:
    """The largest relative L2 error over blocks of `block` rows along `axis`
    (the token axis), so that one wrong tile cannot hide in a whole-tensor
    norm."""
    a = np.moveaxis(np.asarray(a, np.float64), axis, 0)
    b = np.moveaxis(np.asarray(b, np.float64), axis, 0)
    worst = 0.0
    for t0 in range(0, a.shape[0], block):
        worst = max(worst, rel(a[t0:t0 + block], b[t0:t0 + block]))
    return worst


def spec_of(w: Workload) -> O.Spec:
    return O.Spec(E=w.E, C=w.C, Hq=w.Hq, Hkv=w.Hkv, kq=w.kq, kk=w.kk, rope_base=w.rope_base,
                  qk_pre=bool(w.flags & 1), qk_post=bool(w.flags & 2),
                  use_rope=bool(w.flags & 4), use_vshift=bool(w.flags & 8), s_v=w.s_v)


def layer_of(w: Workload, max_seq_len=None) -> cca.CCALayer:
    return cca.CCALayer(w.E, w.C, w.Hq, w.Hkv, max_seq_len or w.capacity, w.kq, w.kk, w.s_v,
                        w.flags, w.rope_base, w.dtype)


def params_of(inp):
    return {n: inp[n] for n in WEIGHT_NAMES}


def dev_weights(inp, w: Workload):
    return {n: dev(inp[n], w) for n in WEIGHT_NAMES}


def saved_views(layer: cca.CCALayer, saved: torch.Tensor, w: Workload, B: int, S: int):
    """Typed views of the regions of a prefill's saved buffer."""
    offs = layer.saved_offsets(B, S)
    es = 2 if w.dtype == "bf16" else 4
    d = w.d
    shapes = [(B * S, (w.Hq + 2 * w.Hkv) * d), (B, w.Hq, S, d), (B, w.Hkv, S, d),
              (B, w.Hkv, S, d), (B, S, w.Hq * d), (B, w.Hq, S), (B, S, w.Hq * d)]
    names = ["qkv", "q_rope", "k_rope", "v_shift", "o", "lse", "o32"]
    out = {}
    for name, off, shp in zip(names, offs, shapes):
        n = int(np.prod(shp))
        if name in ("lse", "qkv", "o32"):
            out[name] = saved[off:off + 4 * n].view(torch.float32).view(shp)
        else:
            out[name] = saved[off:off + es * n].view(tdtype(w)).view(shp)
    return out


def run_prefill(w: Workload, inp, with_saved=True, with_cache=False, layer=None):
    layer = layer or layer_of(w)
    x = dev(inp["x"], w)
    wts = dev_weights(inp, w)
    B, S = x.shape[0], x.shape[1]
    saved = torch.empty(layer.saved_bytes(B, S), dtype=torch.uint8, device="cuda") \
        if with_saved else None
    kc = vc = st = None
    if with_cache:
        kc = torch.zeros((B, w.Hkv, layer.max_seq_len, w.d), dtype=tdtype(w), device="cuda")
        vc = torch.zeros_like(kc)
        st = torch.zeros((B, layer.state_width()), dtype=tdtype(w), device="cuda")
    y = layer.forward_prefill(wts, x, saved=saved, k_cache=kc, v_cache=vc, state=st)
    torch.cuda.synchronize()
    return dict(layer=layer, y=y, saved=saved, k_cache=kc, v_cache=vc, state=st, x=x, w=wts)
