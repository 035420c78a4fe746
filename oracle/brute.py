"""Scalar pure-Python loops for tiny shapes (test infrastructure only).

Written separately from ``cca.py`` (no numpy, no shared helper) so that the
vectorised oracle can be pinned against a second, loop-by-loop statement of the
same definitions on inputs of a few tokens:

* ``mha_bruteforce``: textbook causal multi-head attention with input and
  output projections, optionally with rotate-half RoPE.  With compression C = 1,
  identity convolutions, no QK-mean and no value shift, a CCA layer is exactly
  this (CCA-es §2.A: CCA is attention run in a latent of size E/C).
* ``cca_loops``: the whole CCA / CCGQA layer written as loops over tokens,
  heads and channels, following CCA-es §2.A-2.C and §3 item 2 with the
  readings stated in ``cca.py``.
"""
from __future__ import annotations

import math
from typing import List, Optional

Vec = List[float]


def _matvec(w, x) -> Vec:
    return [sum(w[i][j] * x[j] for j in range(len(x))) for i in range(len(w))]


def _rope_vec(u: Vec, p: int, base: float) -> Vec:
    d = len(u)
    h = d // 2
    out = list(u)
    for i in range(h):
        ang = p * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = u[i] * c - u[i + h] * s
        out[i + h] = u[i + h] * c + u[i] * s
    return out


def _causal_attend(qs, ks, vs, scale):
    """qs, ks, vs: per-token vectors of one head; returns per-token outputs."""
    S = len(qs)
    outs = []
    for t in range(S):
        sc = [scale * sum(qs[t][c] * ks[s][c] for c in range(len(qs[t]))) for s in range(t + 1)]
        m = max(sc)
        e = [math.exp(z - m) for z in sc]
        tot = sum(e)
        outs.append([sum(e[s] / tot * vs[s][c] for s in range(t + 1)) for c in range(len(vs[0]))])
    return outs


def mha_bruteforce(x, wq, wk, wv, wo, H: int, rope_base: Optional[float] = None):
    """Causal multi-head attention on one sequence x [S][E]; weights [out][in]."""
    x = [list(map(float, r)) for r in x]
    S = len(x)
    q = [_matvec(wq, x[t]) for t in range(S)]
    k = [_matvec(wk, x[t]) for t in range(S)]
    v = [_matvec(wv, x[t]) for t in range(S)]
    dh = len(q[0]) // H
    out = [[0.0] * (H * dh) for _ in range(S)]
    for h in range(H):
        qs = [q[t][h * dh:(h + 1) * dh] for t in range(S)]
        ks = [k[t][h * dh:(h + 1) * dh] for t in range(S)]
        vs = [v[t][h * dh:(h + 1) * dh] for t in range(S)]
        if rope_base is not None:
            qs = [_rope_vec(qs[t], t, rope_base) for t in range(S)]
            ks = [_rope_vec(ks[t], t, rope_base) for t in range(S)]
        o = _causal_attend(qs, ks, vs, 1.0 / math.sqrt(dh))
        for t in range(S):
            out[t][h * dh:(h + 1) * dh] = o[t]
    return [_matvec(wo, out[t]) for t in range(S)]


def cca_loops(x, w_q, w_k, w_v, w_o, conv_q, conv_k, Hq: int, Hkv: int,
              rope_base: float, qk_pre: bool, qk_post: bool, use_rope: bool,
              vmask):
    """The CCA / CCGQA layer on one sequence x [S][E], all in scalar loops.

    conv_q [Hq][k][d][d], conv_k [Hkv][k][d][d]; vmask [Hkv][d] (truthy =
    channel taken from the previous token).
    """
    x = [list(map(float, r)) for r in x]
    S = len(x)
    G = Hq // Hkv
    ql = [_matvec(w_q, x[t]) for t in range(S)]          # flat [Hq*d]
    kl = [_matvec(w_k, x[t]) for t in range(S)]
    vl = [_matvec(w_v, x[t]) for t in range(S)]
    d = len(ql[0]) // Hq

    def head(vecs, t, h):
        return vecs[t][h * d:(h + 1) * d]

    def conv(vecs, taps, t, h):
        acc = [0.0] * d
        for j in range(len(taps[h])):
            if t - j < 0:
                continue
            src = head(vecs, t - j, h)
            for c in range(d):
                acc[c] += sum(taps[h][j][c][e] * src[e] for e in range(d))
        return acc

    qc = [[conv(ql, conv_q, t, h) for h in range(Hq)] for t in range(S)]
    kc = [[conv(kl, conv_k, t, g) for g in range(Hkv)] for t in range(S)]
    a = 1.0 if qk_pre else 0.0
    b = 1.0 if qk_post else 0.0
    qm = [[None] * Hq for _ in range(S)]
    km = [[None] * Hkv for _ in range(S)]
    for t in range(S):
        for h in range(Hq):
            g = h // G
            qm[t][h] = [qc[t][h][c]
                        + a * 0.5 * (head(ql, t, h)[c] + head(kl, t, g)[c])
                        + b * 0.5 * (qc[t][h][c] + kc[t][g][c]) for c in range(d)]
        for g in range(Hkv):
            members = range(g * G, (g + 1) * G)
            mean_pre = [sum(head(ql, t, h)[c] for h in members) / G for c in range(d)]
            mean_post = [sum(qc[t][h][c] for h in members) / G for c in range(d)]
            km[t][g] = [kc[t][g][c]
                        + a * 0.5 * (mean_pre[c] + head(kl, t, g)[c])
                        + b * 0.5 * (mean_post[c] + kc[t][g][c]) for c in range(d)]
    vs = [[[(head(vl, t - 1, g)[c] if t > 0 else 0.0) if vmask[g][c] else head(vl, t, g)[c]
            for c in range(d)] for g in range(Hkv)] for t in range(S)]
    if use_rope:
        qm = [[_rope_vec(qm[t][h], t, rope_base) for h in range(Hq)] for t in range(S)]
        km = [[_rope_vec(km[t][g], t, rope_base) for g in range(Hkv)] for t in range(S)]
    o = [[0.0] * (Hq * d) for _ in range(S)]
    for h in range(Hq):
        g = h // G
        oh = _causal_attend([qm[t][h] for t in range(S)], [km[t][g] for t in range(S)],
                            [vs[t][g] for t in range(S)], 1.0 / math.sqrt(d))
        for t in range(S):
            o[t][h * d:(h + 1) * d] = oh[t]
    return [_matvec(w_o, o[t]) for t in range(S)]
