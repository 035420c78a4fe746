"""Float64 numpy oracle of one CCA / CCGQA attention layer (test infrastructure).

Each function states the passage it follows (page keys are defined in
``oracle/__init__.py``).  Nothing here is blocked, fused or reordered beyond
what the definition needs to fit in memory: attention is processed in blocks
of query rows so that the S x S score matrix is never held whole, which does
not change the definition.

Readings taken where the pages leave a step open (each is repeated in the
build's design notes):

* R-conv: the "convolutional mixing" along the sequence and across the
  channels of one head (CCA-es §2.B.1; CCA-fr §2 "Mélange Convolutif") is one
  causal grouped convolution per head: k taps, each a d x d matrix; tap j
  multiplies the token at lag j; zero history before the first token; no bias,
  no activation.  Q and K have their own taps; V is not convolved.
* R-qkmean: "the mean of Q and K before and after the convolution" (CCA-es
  §2.B.2; CCA-fr §2 "Moyenne Q-K") is added to the post-convolution Q and K:
  q' = q^ + a(q~ + k~)/2 + b(q^ + k^)/2 and the same for k'.  Under head
  sharing the Q side takes its own KV head's k and the K side takes the mean of
  its group's query heads.  a, b switch the pre- and post-convolution terms.
* R-shift: "each head receives value vectors from the current and from the
  previous input" (CCA-es §2.B.3; CCA-fr §2 "Décalage de Valeur"): within every
  KV head a channel mask (default: the last d/2 channels) takes the projected
  value of token t-1 (zero at t = 0); the other channels take token t.
* R-rope: RoPE "directly in the latent" (CCA-es §3 item 2; CCA-fr §2
  "Intégration Native de RoPE") is rotate-half RoPE over the full head dim,
  pairs (i, i + d/2), angle p * base^(-2i/d), applied last to q' and k' only.
* R-attn: scale 1/sqrt(d) with d the latent head dim; causal (key <= query);
  KV head of query head h is h // G (CCA-es §2.C; CCA-fr §2 "Extension
  CCGQA").
* R-out: the output projection W_o maps the query latent back to E; the "no
  up-projection" of CCA-es §2.A is MLA's per-head K/V up-projection.
* R-cache: the compressed cache holds post-RoPE K and post-shift V; the rolling
  decode state holds pre-convolution q~ and k~ for lags 1..k-1 and the
  projected v~ of the previous token, most recent lag first.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

f64 = np.float64


@dataclasses.dataclass
class Spec:
    """Shape and switches of one layer.

    d = E / (C * Hq) is the latent head dim (CCA-es §2.A: latent size E/C),
    G = Hq / Hkv query heads share one KV head (CCA-es §2.C).
    """
    E: int
    C: int
    Hq: int
    Hkv: int
    kq: int = 2
    kk: int = 2
    rope_base: float = 10000.0
    qk_pre: bool = True
    qk_post: bool = True
    use_rope: bool = True
    use_vshift: bool = True
    s_v: Optional[int] = None
    vmask: Optional[np.ndarray] = None   # [Hkv, d] bool overrides s_v

    @property
    def d(self) -> int:
        assert self.E % (self.C * self.Hq) == 0
        return self.E // (self.C * self.Hq)

    @property
    def G(self) -> int:
        assert self.Hq % self.Hkv == 0
        return self.Hq // self.Hkv

    def mask(self) -> np.ndarray:
        if not self.use_vshift:
            return np.zeros((self.Hkv, self.d), dtype=bool)
        if self.vmask is not None:
            return np.asarray(self.vmask, dtype=bool)
        return default_vmask(self.Hkv, self.d, self.d // 2 if self.s_v is None else self.s_v)


def default_vmask(Hkv: int, d: int, s_v: int) -> np.ndarray:
    """The last s_v channels of every KV head are shifted (R-shift)."""
    m = np.zeros((Hkv, d), dtype=bool)
    if s_v > 0:
        m[:, d - s_v:] = True
    return m


# ---------------------------------------------------------------- stages

def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Linear map to (or from) the latent: x @ w.T with w stored [out, in].

    Down-projection of Q, K, V to the latent of size E/C: CCA-es §2.A; CCA-fr §2
    "Projection vers l'Espace Latent"; CCA-blog "Introducing CCA".
    """
    return np.asarray(x, f64) @ np.asarray(w, f64).T


def conv_causal(u: np.ndarray, taps: np.ndarray,
                history: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal grouped convolution along the sequence, mixing channels within a
    head (CCA-es §2.B.1 "Mezcla Convolucional"; CCA-fr §2 "Mélange Convolutif";
    reading R-conv).

    u [S, H, d]; taps [H, k, d, d]; history [k-1, H, d] holds the tokens before
    u[0], most recent first (None = zero history).
    out[t, h] = sum_j taps[h, j] @ u[t - j, h].
    """
    u = np.asarray(u, f64)
    taps = np.asarray(taps, f64)
    S, H, d = u.shape
    k = taps.shape[1]
    hist = np.zeros((k - 1, H, d), f64) if history is None else np.asarray(history, f64)
    # extended sequence, oldest first: position k-1 of `ext` is token 0
    ext = np.concatenate([hist[::-1], u], axis=0)
    out = np.zeros((S, H, d), f64)
    for j in range(k):
        lagged = ext[k - 1 - j:k - 1 - j + S]              # token t - j
        out += np.einsum("hcx,thx->thc", taps[:, j], lagged)
    return out


def qk_mean(q_pre: np.ndarray, k_pre: np.ndarray, q_post: np.ndarray,
            k_post: np.ndarray, G: int, pre: bool, post: bool
            ) -> Tuple[np.ndarray, np.ndarray]:
    """QK-mean: adds the mean of Q and K, taken before and after the
    convolution, to the convolved Q and K (CCA-es §2.B.2 "Operación QK-Mean";
    CCA-fr §2 "Moyenne Q-K"; reading R-qkmean).

    q_* [S, Hq, d], k_* [S, Hkv, d].
    """
    a = 1.0 if pre else 0.0
    b = 1.0 if post else 0.0
    S, Hq, d = q_pre.shape
    Hkv = Hq // G

    def per_query_head(kv):          # kv head of query head h is h // G
        return np.repeat(kv, G, axis=1)

    def group_mean(q):               # mean of the G query heads of each group
        return q.reshape(S, Hkv, G, d).mean(axis=2)

    q_out = q_post + a * 0.5 * (q_pre + per_query_head(k_pre)) \
                   + b * 0.5 * (q_post + per_query_head(k_post))
    k_out = k_post + a * 0.5 * (group_mean(q_pre) + k_pre) \
                   + b * 0.5 * (group_mean(q_post) + k_post)
    return q_out, k_out


def value_shift(v: np.ndarray, mask: np.ndarray,
                prev: Optional[np.ndarray] = None) -> np.ndarray:
    """Value shift: masked channels of each KV head come from the previous
    token (CCA-es §2.B.3 "Desplazamiento de Valores"; CCA-fr §2 "Décalage de
    Valeur"; reading R-shift).

    v [S, Hkv, d]; mask [Hkv, d]; prev [Hkv, d] is the value before v[0]
    (None = zeros).
    """
    v = np.asarray(v, f64)
    before = np.zeros_like(v[:1]) if prev is None else np.asarray(prev, f64)[None]
    shifted = np.concatenate([before, v[:-1]], axis=0)
    return np.where(mask[None], shifted, v)


def rope_angles(positions: np.ndarray, d: int, base: float) -> np.ndarray:
    """phi[p, i] = p * base^(-2i/d), i < d/2, in float64 (reading R-rope)."""
    i = np.arange(d // 2, dtype=f64)
    inv = np.power(f64(base), -2.0 * i / d)
    return np.asarray(positions, f64)[:, None] * inv[None, :]


def rope(u: np.ndarray, positions: np.ndarray, base: float,
         inverse: bool = False) -> np.ndarray:
    """Rotary position embedding applied in the latent heads (CCA-es §3 item 2
    "Integración Nativa de RoPE"; CCA-fr §2 "Intégration Native de RoPE";
    reading R-rope).  u [S, H, d]; positions [S].  ``inverse`` rotates by -phi
    (used by the backward pass).
    """
    u = np.asarray(u, f64)
    d = u.shape[-1]
    h = d // 2
    phi = rope_angles(positions, d, base)
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    if inverse:
        s = -s
    lo, hi = u[..., :h], u[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, G: int,
              q_pos: Optional[np.ndarray] = None, block: int = 256,
              return_probs: bool = False):
    """Causal softmax attention carried out entirely on the latent heads, with
    KV heads shared by groups of G query heads (CCA-es §2.A "Principio
    Fundamental" and §2.C "CCGQA"; CCA-fr §2 "Opération d'Attention
    Compressée" and "Extension CCGQA"; reading R-attn).

    q [Sq, Hq, d]; k, v [Sk, Hkv, d]; the query at row i sits at position
    q_pos[i] (default i) and sees keys 0..q_pos[i].
    Returns o [Sq, Hq, d], lse [Hq, Sq] (natural log of the softmax
    denominator of the scaled scores) and, if asked, P [Hq, Sq, Sk].
    """
    q = np.asarray(q, f64)
    k = np.asarray(k, f64)
    v = np.asarray(v, f64)
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((Sq, Hq, d), f64)
    lse = np.zeros((Hq, Sq), f64)
    probs = np.zeros((Hq, Sq, Sk), f64) if return_probs else None
    for h in range(Hq):
        g = h // G
        for t0 in range(0, Sq, block):
            t1 = min(Sq, t0 + block)
            p_blk = pos[t0:t1]
            n = int(p_blk.max()) + 1                   # keys any row may see
            s = (q[t0:t1, h] @ k[:n, g].T) * scale
            s = np.where(np.arange(n)[None, :] <= p_blk[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            p = e / l
            o[t0:t1, h] = p @ v[:n, g]
            lse[h, t0:t1] = (m + np.log(l))[:, 0]
            if return_probs:
                probs[h, t0:t1, :n] = p
    if return_probs:
        return o, lse, probs
    return o, lse


# ---------------------------------------------------------------- the layer

def _split_heads(a: np.ndarray, H: int) -> np.ndarray:
    return a.reshape(a.shape[0], H, -1)


def forward(x: np.ndarray, params: Dict[str, np.ndarray], spec: Spec,
            return_saved: bool = False):
    """Forward prefill of one layer over x [B, S, E] -> y [B, S, E].

    Order of the steps (CCA-es §2.A then §2.B.1-3, RoPE per §3 item 2,
    attention per §2.A/§2.C, output projection per reading R-out):
    project -> conv -> QK-mean -> value shift -> RoPE -> attention -> W_o.

    With ``return_saved`` also returns a dict of per-sequence stage outputs
    (lists over the batch) plus the decode cache and rolling state a prefill
    leaves behind (reading R-cache).
    """
    x = np.asarray(x, f64)
    B, S, E = x.shape
    Hq, Hkv, G, d = spec.Hq, spec.Hkv, spec.G, spec.d
    mask = spec.mask()
    pos = np.arange(S)
    ys = []
    saved = {key: [] for key in ("q_lat", "k_lat", "v_lat", "q_conv", "k_conv", "q_mix",
                                 "k_mix", "q_rope", "k_rope", "v_shift", "o", "lse", "state")}
    for b in range(B):
        q_lat = _split_heads(project(x[b], params["w_q"]), Hq)
        k_lat = _split_heads(project(x[b], params["w_k"]), Hkv)
        v_lat = _split_heads(project(x[b], params["w_v"]), Hkv)
        q_conv = conv_causal(q_lat, params["conv_q"])
        k_conv = conv_causal(k_lat, params["conv_k"])
        q_mix, k_mix = qk_mean(q_lat, k_lat, q_conv, k_conv, G, spec.qk_pre, spec.qk_post)
        v_sh = value_shift(v_lat, mask)
        if spec.use_rope:
            q_r = rope(q_mix, pos, spec.rope_base)
            k_r = rope(k_mix, pos, spec.rope_base)
        else:
            q_r, k_r = q_mix, k_mix
        o, lse = attention(q_r, k_r, v_sh, G)
        y = project(o.reshape(S, Hq * d), params["w_o"])
        ys.append(y)
        if return_saved:
            for key, val in (("q_lat", q_lat), ("k_lat", k_lat), ("v_lat", v_lat),
                             ("q_conv", q_conv), ("k_conv", k_conv), ("q_mix", q_mix),
                             ("k_mix", k_mix), ("q_rope", q_r), ("k_rope", k_r),
                             ("v_shift", v_sh), ("o", o), ("lse", lse)):
                saved[key].append(val)
            saved["state"].append(_state_after(q_lat, k_lat, v_lat, spec))
    y = np.stack(ys)
    if return_saved:
        return y, saved
    return y


def _lags(u: np.ndarray, n: int) -> np.ndarray:
    """Tokens S-1, S-2, ..., S-n of u [S, H, d] (zero where the index < 0)."""
    S = u.shape[0]
    out = np.zeros((n,) + u.shape[1:], f64)
    for j in range(1, n + 1):
        if S - j >= 0:
            out[j - 1] = u[S - j]
    return out


def _state_after(q_lat, k_lat, v_lat, spec: Spec) -> np.ndarray:
    parts = [_lags(q_lat, spec.kq - 1).reshape(-1), _lags(k_lat, spec.kk - 1).reshape(-1),
             _lags(v_lat, 1).reshape(-1)]
    return np.concatenate(parts)


def _unpack_state(state: np.ndarray, spec: Spec):
    Hq, Hkv, d = spec.Hq, spec.Hkv, spec.d
    nq = (spec.kq - 1) * Hq * d
    nk = (spec.kk - 1) * Hkv * d
    st = np.asarray(state, f64)
    q_hist = st[:nq].reshape(spec.kq - 1, Hq, d)
    k_hist = st[nq:nq + nk].reshape(spec.kk - 1, Hkv, d)
    v_prev = st[nq + nk:nq + nk + Hkv * d].reshape(Hkv, d)
    return q_hist, k_hist, v_prev


def decode_step(x_new: np.ndarray, params: Dict[str, np.ndarray], spec: Spec,
                k_cache: np.ndarray, v_cache: np.ndarray, state: np.ndarray,
                pos: np.ndarray):
    """One autoregressive step per sequence over the compressed latent cache
    (CCA-es §1 item 2 and §2.C on the cache; CCA-fr §4 "Décodage"; readings
    R-cache and R-conv for the rolling state).

    x_new [B, E]; k_cache, v_cache [B, Hkv, cap, d] hold post-RoPE K and
    post-shift V; state [B, W]; pos [B] = tokens already cached.
    Returns y_new [B, E] and updated copies of (k_cache, v_cache, state).
    """
    x_new = np.asarray(x_new, f64)
    B, E = x_new.shape
    Hq, Hkv, G, d = spec.Hq, spec.Hkv, spec.G, spec.d
    mask = spec.mask()
    kc = np.array(k_cache, f64)
    vc = np.array(v_cache, f64)
    st_out = np.zeros((B, np.asarray(state).shape[1]), f64)
    y = np.zeros((B, E), f64)
    for b in range(B):
        p = int(pos[b])
        q_hist, k_hist, v_prev = _unpack_state(state[b], spec)
        q_lat = project(x_new[b][None], params["w_q"]).reshape(1, Hq, d)
        k_lat = project(x_new[b][None], params["w_k"]).reshape(1, Hkv, d)
        v_lat = project(x_new[b][None], params["w_v"]).reshape(1, Hkv, d)
        q_conv = conv_causal(q_lat, params["conv_q"], history=q_hist)
        k_conv = conv_causal(k_lat, params["conv_k"], history=k_hist)
        q_mix, k_mix = qk_mean(q_lat, k_lat, q_conv, k_conv, G, spec.qk_pre, spec.qk_post)
        v_sh = value_shift(v_lat, mask, prev=v_prev)
        if spec.use_rope:
            q_r = rope(q_mix, np.array([p]), spec.rope_base)
            k_r = rope(k_mix, np.array([p]), spec.rope_base)
        else:
            q_r, k_r = q_mix, k_mix
        kc[b, :, p] = k_r[0]
        vc[b, :, p] = v_sh[0]
        k_seq = np.transpose(kc[b, :, :p + 1], (1, 0, 2))      # [p+1, Hkv, d]
        v_seq = np.transpose(vc[b, :, :p + 1], (1, 0, 2))
        o, _ = attention(q_r, k_seq, v_seq, G, q_pos=np.array([p]))
        y[b] = project(o.reshape(1, Hq * d), params["w_o"])[0]
        # roll the state: the new token becomes lag 1
        q_h = np.concatenate([q_lat, q_hist[:spec.kq - 2]], axis=0) if spec.kq > 1 else q_hist
        k_h = np.concatenate([k_lat, k_hist[:spec.kk - 2]], axis=0) if spec.kk > 1 else k_hist
        st_out[b] = np.concatenate([q_h.reshape(-1), k_h.reshape(-1), v_lat.reshape(-1)])
    return y, kc, vc, st_out


def prefill_chunks(x: np.ndarray, offsets, starts, params: Dict[str, np.ndarray], spec: Spec,
                   k_cache: np.ndarray, v_cache: np.ndarray, state: np.ndarray):
    """Chunked, variable-length batched prefill over the compressed latent
    cache (CCA-es §1 item 2 and §2.C on the cache; CCA-fr §4 "Décodage").

    Sequence b brings the packed rows offsets[b] .. offsets[b+1]-1 of x [T, E]
    as new tokens at positions starts[b] ..; each is taken through
    ``decode_step`` in order (a chunk is its tokens decoded one after another:
    conv and shift history from the state, attention over the cache up to the
    token's own row).  Returns y [T, E] and updated copies of (k_cache,
    v_cache, state).
    """
    x = np.asarray(x, f64)
    B = len(offsets) - 1
    kc = np.array(k_cache, f64)
    vc = np.array(v_cache, f64)
    st = np.array(state, f64)
    y = np.zeros((x.shape[0], x.shape[1]), f64)
    for b in range(B):
        p0 = 0 if starts is None else int(starts[b])
        for i, row in enumerate(range(int(offsets[b]), int(offsets[b + 1]))):
            yb, kcb, vcb, stb = decode_step(x[row][None], params, spec, kc[b:b + 1],
                                            vc[b:b + 1], st[b:b + 1], np.array([p0 + i]))
            y[row] = yb[0]
            kc[b], vc[b], st[b] = kcb[0], vcb[0], stb[0]
    return y, kc, vc, st


# ---------------------------------------------------------------- backward

def _attention_backward(q, k, v, o, lse, do, G, block=256):
    """Gradients of causal softmax attention (reading R-attn) given the
    forward's o and lse; P is recomputed from q, k and lse."""
    Sq, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros((k.shape[0], Hkv, d), f64)
    dv = np.zeros((v.shape[0], Hkv, d), f64)
    for h in range(Hq):
        g = h // G
        D = np.sum(do[:, h] * o[:, h], axis=1)                # rowsum(dO * O)
        for t0 in range(0, Sq, block):
            t1 = min(Sq, t0 + block)
            n = t1
            s = (q[t0:t1, h] @ k[:n, g].T) * scale
            causal = np.arange(n)[None, :] <= np.arange(t0, t1)[:, None]
            p = np.exp(np.where(causal, s, -np.inf) - lse[h, t0:t1, None])
            dv[:n, g] += p.T @ do[t0:t1, h]
            dp = do[t0:t1, h] @ v[:n, g].T
            ds = p * (dp - D[t0:t1, None]) * scale
            dq[t0:t1, h] = ds @ k[:n, g]
            dk[:n, g] += ds.T @ q[t0:t1, h]
    return dq, dk, dv


def _conv_backward(u: np.ndarray, taps: np.ndarray, dout: np.ndarray):
    """Adjoint of ``conv_causal`` (zero history): returns (du, dtaps)."""
    S, H, d = u.shape
    k = taps.shape[1]
    du = np.zeros_like(u)
    dtaps = np.zeros(taps.shape, f64)
    for j in range(k):
        if j >= S:
            continue
        # out[t] += A_j u[t-j]  for t >= j
        du[:S - j] += np.einsum("hcx,thc->thx", taps[:, j], dout[j:])
        dtaps[:, j] = np.einsum("thc,thx->hcx", dout[j:], u[:S - j])
    return du, dtaps


def backward(x: np.ndarray, dy: np.ndarray, params: Dict[str, np.ndarray], spec: Spec):
    """Gradients of L = <dy, forward(x)> with respect to x, the four
    projections and the conv taps (training backward pass, CCA-es §4 latency
    results "Entrenamiento (Backward)"; CCA-fr §4 "Rétropropagation").

    Each step is the adjoint of the matching forward step, taken in reverse
    order: W_o, attention (P recomputed from lse), RoPE (rotation by -phi),
    QK-mean, convolution, value shift, down-projections.
    Returns a dict with dx [B,S,E], dw_q, dw_k, dw_v, dw_o, dconv_q, dconv_k.
    """
    x = np.asarray(x, f64)
    dy = np.asarray(dy, f64)
    B, S, E = x.shape
    Hq, Hkv, G, d = spec.Hq, spec.Hkv, spec.G, spec.d
    a = 1.0 if spec.qk_pre else 0.0
    bb = 1.0 if spec.qk_post else 0.0
    mask = spec.mask()
    pos = np.arange(S)
    _, sv = forward(x, params, spec, return_saved=True)
    g = {name: np.zeros(np.shape(params[name]), f64)
         for name in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")}
    dx = np.zeros_like(x)
    for b in range(B):
        o = sv["o"][b]
        o_flat = o.reshape(S, Hq * d)
        g["w_o"] += dy[b].T @ o_flat
        do = (dy[b] @ np.asarray(params["w_o"], f64)).reshape(S, Hq, d)
        dq_r, dk_r, dv_sh = _attention_backward(sv["q_rope"][b], sv["k_rope"][b],
                                                sv["v_shift"][b], o, sv["lse"][b], do, G)
        if spec.use_rope:
            dq_mix = rope(dq_r, pos, spec.rope_base, inverse=True)
            dk_mix = rope(dk_r, pos, spec.rope_base, inverse=True)
        else:
            dq_mix, dk_mix = dq_r, dk_r
        # QK-mean adjoint
        sum_dq_group = dq_mix.reshape(S, Hkv, G, d).sum(axis=2)          # [S,Hkv,d]
        dk_per_q = np.repeat(dk_mix, G, axis=1)                            # [S,Hq,d]
        dq_conv = (1 + bb / 2) * dq_mix + (bb / (2 * G)) * dk_per_q
        dk_conv = (1 + bb / 2) * dk_mix + (bb / 2) * sum_dq_group
        dq_lat = (a / 2) * dq_mix + (a / (2 * G)) * dk_per_q
        dk_lat = (a / 2) * sum_dq_group + (a / 2) * dk_mix
        # convolution adjoint
        du, dA = _conv_backward(sv["q_lat"][b], params["conv_q"], dq_conv)
        dq_lat += du
        g["conv_q"] += dA
        du, dA = _conv_backward(sv["k_lat"][b], params["conv_k"], dk_conv)
        dk_lat += du
        g["conv_k"] += dA
        # value shift adjoint
        dv_next = np.concatenate([dv_sh[1:], np.zeros_like(dv_sh[:1])], axis=0)
        dv_lat = np.where(mask[None], dv_next, dv_sh)
        # down-projections
        dqf, dkf, dvf = (dq_lat.reshape(S, -1), dk_lat.reshape(S, -1), dv_lat.reshape(S, -1))
        dx[b] = dqf @ np.asarray(params["w_q"], f64) + dkf @ np.asarray(params["w_k"], f64) \
            + dvf @ np.asarray(params["w_v"], f64)
        g["w_q"] += dqf.T @ x[b]
        g["w_k"] += dkf.T @ x[b]
        g["w_v"] += dvf.T @ x[b]
    return {"dx": dx, "dw_q": g["w_q"], "dw_k": g["w_k"], "dw_v": g["w_v"], "dw_o": g["w_o"],
            "dconv_q": g["conv_q"], "dconv_k": g["conv_k"]}


# ---------------------------------------------------------------- accounting

def attention_flops(S: int, Hq: int, d: int) -> int:
    """FLOPs of causal attention counting only visible (query, key) pairs:
    QK^T and PV each cost 2*d per pair per query head.  The pages state that
    working in the latent divides attention FLOPs by C (CCA-es §2.A; CCA-fr §4
    "Réduction des FLOPs")."""
    return 4 * Hq * d * (S * (S + 1) // 2)


def kv_cache_values_per_token(Hkv: int, d: int) -> int:
    """Cached values per token: one K and one V vector per KV head (CCA-es
    §2.C; CCA-fr §2 "Extension CCGQA")."""
    return 2 * Hkv * d


def param_count(spec: Spec) -> int:
    """Parameters of the layer: W_q, W_k, W_v, W_o and the conv taps (CCA-es
    §3 item 1 on the parameter reduction)."""
    d = spec.d
    E = spec.E
    return (E * spec.Hq * d + 2 * E * spec.Hkv * d + E * spec.Hq * d
            + spec.Hq * spec.kq * d * d + spec.Hkv * spec.kk * d * d)
