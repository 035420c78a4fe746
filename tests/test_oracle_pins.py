"""Pins of the float64 oracle against things other than itself (CPU only).

Each test ties an oracle function to brute force on tiny inputs, to textbook
multi-head attention, to a closed form or to an invariant the pages fix.
"""
import math

import numpy as np
import pytest

from oracle import cca as O
from oracle import brute


def rand_params(spec: O.Spec, rng, scale_taps=None):
    E, d = spec.E, spec.d
    p = {
        "w_q": rng.standard_normal((spec.Hq * d, E)) / math.sqrt(E),
        "w_k": rng.standard_normal((spec.Hkv * d, E)) / math.sqrt(E),
        "w_v": rng.standard_normal((spec.Hkv * d, E)) / math.sqrt(E),
        "w_o": rng.standard_normal((E, spec.Hq * d)) / math.sqrt(E),
        "conv_q": rng.standard_normal((spec.Hq, spec.kq, d, d)) / math.sqrt(spec.kq * d),
        "conv_k": rng.standard_normal((spec.Hkv, spec.kk, d, d)) / math.sqrt(spec.kk * d),
    }
    return p


def identity_taps(H, k, d):
    a = np.zeros((H, k, d, d))
    for h in range(H):
        a[h, 0] = np.eye(d)
    return a


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------- reduction to MHA

@pytest.mark.parametrize("use_rope", [False, True])
@pytest.mark.parametrize("k", [1, 2])
def test_reduces_to_bruteforce_mha(use_rope, k):
    """C = 1, Hq = Hkv, identity convolutions, no QK-mean, no value shift:
    the layer is plain causal multi-head attention (CCA-es §2.A)."""
    rng = np.random.default_rng(11)
    spec = O.Spec(E=8, C=1, Hq=2, Hkv=2, kq=k, kk=k, qk_pre=False, qk_post=False,
                  use_rope=use_rope, use_vshift=False)
    p = rand_params(spec, rng)
    p["conv_q"] = identity_taps(2, k, spec.d)
    p["conv_k"] = identity_taps(2, k, spec.d)
    x = rng.standard_normal((1, 7, 8))
    y = O.forward(x, p, spec)[0]
    ref = np.array(brute.mha_bruteforce(x[0], p["w_q"], p["w_k"], p["w_v"], p["w_o"], 2,
                                        rope_base=10000.0 if use_rope else None))
    assert rel(y, ref) < 1e-12


# ------------------------------------------------------- loop-by-loop layer

@pytest.mark.parametrize("Hq,Hkv,kq,kk,flags", [
    (2, 2, 2, 2, (True, True, True)),
    (4, 2, 2, 3, (True, True, True)),
    (4, 1, 3, 1, (True, False, True)),
    (2, 1, 1, 2, (False, True, False)),
    (4, 2, 2, 2, (False, False, True)),
])
def test_matches_scalar_loops(Hq, Hkv, kq, kk, flags):
    """The vectorised oracle equals the scalar-loop statement of the whole
    layer on tiny shapes, for several head sharings, kernel sizes and switch
    settings, with a random (not half-split) value-shift mask."""
    pre, post, use_rope = flags
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + kq + kk)
    E, C = 16, 2
    vmask = rng.random((Hkv, E // (C * Hq))) < 0.5
    spec = O.Spec(E=E, C=C, Hq=Hq, Hkv=Hkv, kq=kq, kk=kk, qk_pre=pre, qk_post=post,
                  use_rope=use_rope, vmask=vmask)
    p = rand_params(spec, rng)
    x = rng.standard_normal((1, 6, E))
    y = O.forward(x, p, spec)[0]
    ref = np.array(brute.cca_loops(x[0], p["w_q"], p["w_k"], p["w_v"], p["w_o"],
                                   p["conv_q"], p["conv_k"], Hq, Hkv, 10000.0, pre, post,
                                   use_rope, vmask))
    assert rel(y, ref) < 1e-12


def test_default_shift_mask_is_last_half():
    m = O.default_vmask(2, 8, 4)
    assert m.tolist() == [[False] * 4 + [True] * 4] * 2
    spec = O.Spec(E=64, C=4, Hq=2, Hkv=1)
    assert spec.mask().sum() == spec.d // 2 and spec.mask()[0, -1] and not spec.mask()[0, 0]


# ------------------------------------------------------- attention invariants

def test_attention_rows_sum_to_one_and_causal():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((37, 4, 8))
    k = rng.standard_normal((37, 2, 8))
    v = rng.standard_normal((37, 2, 8))
    o, lse, P = O.attention(q, k, v, G=2, block=16, return_probs=True)
    assert np.max(np.abs(P.sum(axis=2) - 1.0)) < 1e-13
    upper = np.triu(np.ones((37, 37), bool), 1)
    assert np.all(P[:, upper] == 0.0)
    assert np.all(P[:, ~upper] > 0.0)
    # lse is the log of the softmax denominator of the scaled scores
    s = np.einsum("thc,shc->hts", q, np.repeat(k, 2, axis=1)) / math.sqrt(8)
    s = np.where(upper[None], -np.inf, s)
    assert np.max(np.abs(lse - np.log(np.exp(s).sum(axis=2)))) < 1e-12
    # visible pairs = S(S+1)/2 per head: the count behind attention_flops
    assert int((P[0] > 0).sum()) == 37 * 38 // 2


def test_attention_single_token_returns_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 4))
    k = rng.standard_normal((1, 1, 4))
    v = rng.standard_normal((1, 1, 4))
    o, lse = O.attention(q, k, v, G=2)
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[0, 1], v[0, 0])


def test_gqa_head_mapping_uses_contiguous_groups():
    """Query head h reads KV head h // G: make KV heads' values constant and
    distinct; every output row of head h equals KV head h // G's constant."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((5, 6, 4))
    k = rng.standard_normal((5, 3, 4))
    v = np.zeros((5, 3, 4))
    for g in range(3):
        v[:, g, :] = 10.0 * (g + 1)
    o, _ = O.attention(q, k, v, G=2)
    for h in range(6):
        assert np.allclose(o[:, h, :], 10.0 * (h // 2 + 1), rtol=0, atol=1e-12)


def test_causality_bit_identical():
    """Changing tokens t >= t0 leaves every output row t < t0 bit-identical."""
    rng = np.random.default_rng(6)
    spec = O.Spec(E=64, C=4, Hq=4, Hkv=2)
    p = rand_params(spec, rng)
    x = rng.standard_normal((1, 300, 64))
    y0 = O.forward(x, p, spec)
    x2 = x.copy()
    t0 = 171
    x2[:, t0:] = rng.standard_normal(x2[:, t0:].shape)
    y1 = O.forward(x2, p, spec)
    assert np.array_equal(y0[:, :t0], y1[:, :t0])
    assert not np.allclose(y0[:, t0], y1[:, t0])


# ------------------------------------------------------- stage identities

def test_conv_impulse_response_is_lag_ordered():
    """A single nonzero token at t0 produces tap j's response at t0 + j, and
    nothing before t0 (causal, tap j multiplies lag j)."""
    rng = np.random.default_rng(7)
    taps = rng.standard_normal((2, 3, 4, 4))
    u = np.zeros((9, 2, 4))
    u[4] = rng.standard_normal((2, 4))
    out = O.conv_causal(u, taps)
    assert np.all(out[:4] == 0) and np.all(out[7:] == 0)
    for j in range(3):
        for h in range(2):
            assert np.allclose(out[4 + j, h], taps[h, j] @ u[4, h], rtol=0, atol=1e-14)


def test_conv_identity_taps_pass_through_and_linear_in_taps():
    rng = np.random.default_rng(8)
    u = rng.standard_normal((10, 3, 4))
    assert np.array_equal(O.conv_causal(u, identity_taps(3, 2, 4)), u)
    a1 = rng.standard_normal((3, 2, 4, 4))
    a2 = rng.standard_normal((3, 2, 4, 4))
    lhs = O.conv_causal(u, 2.0 * a1 - a2)
    rhs = 2.0 * O.conv_causal(u, a1) - O.conv_causal(u, a2)
    assert rel(lhs, rhs) < 1e-14


def test_conv_history_equals_prepended_tokens():
    rng = np.random.default_rng(9)
    taps = rng.standard_normal((2, 3, 4, 4))
    u = rng.standard_normal((8, 2, 4))
    full = O.conv_causal(u, taps)
    hist = u[3:5][::-1]                       # tokens 4, 3: most recent first
    part = O.conv_causal(u[5:], taps, history=hist)
    assert rel(part, full[5:]) < 1e-14


def test_qk_mean_switches_and_plain_case():
    rng = np.random.default_rng(10)
    qp, qc = rng.standard_normal((2, 5, 4, 6))
    kp, kc = rng.standard_normal((2, 5, 2, 6))
    q, k = O.qk_mean(qp, kp, qc, kc, G=2, pre=False, post=False)
    assert np.array_equal(q, qc) and np.array_equal(k, kc)
    # G = 1: the same vector is added to q and k
    qp1, qc1, kp1, kc1 = rng.standard_normal((4, 5, 3, 6))
    q, k = O.qk_mean(qp1, kp1, qc1, kc1, G=1, pre=True, post=True)
    assert rel(q - qc1, k - kc1) < 1e-15
    # and that vector is the average of the four tensors times two halves
    assert rel(q - qc1, (qp1 + kp1 + qc1 + kc1) / 2) < 1e-15


def test_value_shift_indexing():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((6, 2, 4))
    assert np.array_equal(O.value_shift(v, np.zeros((2, 4), bool)), v)
    m = O.default_vmask(2, 4, 2)
    s = O.value_shift(v, m)
    assert np.all(s[0, :, 2:] == 0)
    assert np.array_equal(s[1:, :, 2:], v[:-1, :, 2:])
    assert np.array_equal(s[:, :, :2], v[:, :, :2])
    prev = rng.standard_normal((2, 4))
    s2 = O.value_shift(v, m, prev=prev)
    assert np.array_equal(s2[0, :, 2:], prev[:, 2:])


def test_rope_identities():
    rng = np.random.default_rng(12)
    u = rng.standard_normal((1, 3, 16))
    assert np.array_equal(O.rope(u, np.array([0]), 10000.0), u)
    pos = np.arange(50)
    w = rng.standard_normal((50, 3, 16))
    r = O.rope(w, pos, 10000.0)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(w, axis=-1), rtol=1e-14)
    assert rel(O.rope(r, pos, 10000.0, inverse=True), w) < 1e-14
    # pair 0 turns by exactly p radians
    assert np.array_equal(O.rope_angles(np.arange(5), 16, 10000.0)[:, 0], np.arange(5.0))
    # relative position: <R_t q, R_s k> depends only on t - s
    qv, kv = rng.standard_normal((2, 1, 1, 16))
    def dot(t, s):
        return float(np.sum(O.rope(qv, np.array([t]), 1e4) * O.rope(kv, np.array([s]), 1e4)))
    assert abs(dot(9, 4) - dot(105, 100)) < 1e-12 and abs(dot(5, 0) - dot(9, 4)) < 1e-12
    # the last pair turns by p * base^(-(d-2)/d)
    ang = O.rope_angles(np.array([3]), 16, 10000.0)[0, -1]
    assert abs(ang - 3 * 10000.0 ** (-14 / 16)) < 1e-15


def test_head_sharing_equals_duplicated_kv_heads():
    """With QK-mean off, CCGQA (Hkv = 1, G = 2) equals CCA whose KV heads are
    copies (same W_k, W_v rows, taps and mask per head)."""
    rng = np.random.default_rng(13)
    sh = O.Spec(E=32, C=2, Hq=2, Hkv=1, qk_pre=False, qk_post=False)
    p = rand_params(sh, rng)
    x = rng.standard_normal((1, 9, 32))
    y_sh = O.forward(x, p, sh)
    dup = O.Spec(E=32, C=2, Hq=2, Hkv=2, qk_pre=False, qk_post=False)
    p2 = dict(p)
    p2["w_k"] = np.concatenate([p["w_k"], p["w_k"]])
    p2["w_v"] = np.concatenate([p["w_v"], p["w_v"]])
    p2["conv_k"] = np.concatenate([p["conv_k"], p["conv_k"]])
    assert rel(O.forward(x, p2, dup), y_sh) < 1e-13


# ------------------------------------------------------- decode == prefill

@pytest.mark.parametrize("Hq,Hkv,kq,kk", [(4, 2, 2, 2), (2, 2, 3, 1), (4, 1, 1, 3)])
def test_decode_equals_prefill(Hq, Hkv, kq, kk):
    """Prefill over S tokens, then decode of token S, reproduces row S of a
    prefill over S + 1 tokens, and leaves the cache and state a prefill over
    S + 1 tokens leaves."""
    rng = np.random.default_rng(14 + kq)
    spec = O.Spec(E=64, C=4, Hq=Hq, Hkv=Hkv, kq=kq, kk=kk)
    p = rand_params(spec, rng)
    B, S = 2, 11
    x = rng.standard_normal((B, S + 1, 64))
    y_full, sv_full = O.forward(x, p, spec, return_saved=True)
    _, sv = O.forward(x[:, :S], p, spec, return_saved=True)
    cap = S + 5
    kc = np.zeros((B, Hkv, cap, spec.d))
    vc = np.zeros((B, Hkv, cap, spec.d))
    for b in range(B):
        kc[b, :, :S] = np.transpose(sv["k_rope"][b], (1, 0, 2))
        vc[b, :, :S] = np.transpose(sv["v_shift"][b], (1, 0, 2))
    state = np.stack(sv["state"])
    y, kc2, vc2, st2 = O.decode_step(x[:, S], p, spec, kc, vc, state, np.full(B, S))
    assert rel(y, y_full[:, S]) < 1e-12
    for b in range(B):
        assert rel(kc2[b, :, S], sv_full["k_rope"][b][S]) < 1e-12
        assert rel(vc2[b, :, S], sv_full["v_shift"][b][S]) < 1e-12
        assert rel(st2[b], sv_full["state"][b]) < 1e-14
        assert np.array_equal(kc2[b, :, :S], kc[b, :, :S])


def test_decode_first_token_from_zero_state_equals_prefill_of_one():
    rng = np.random.default_rng(15)
    spec = O.Spec(E=64, C=4, Hq=4, Hkv=2)
    p = rand_params(spec, rng)
    x = rng.standard_normal((3, 1, 64))
    y_ref = O.forward(x, p, spec)[:, 0]
    W = (spec.kq - 1) * 4 * spec.d + (spec.kk - 1) * 2 * spec.d + 2 * spec.d
    y, *_ = O.decode_step(x[:, 0], p, spec, np.zeros((3, 2, 4, spec.d)),
                          np.zeros((3, 2, 4, spec.d)), np.zeros((3, W)), np.zeros(3, int))
    assert rel(y, y_ref) < 1e-13


# ------------------------------------------------------- chunked prefill

def _fresh_caches(spec, B, cap):
    W = (spec.kq - 1) * spec.Hq * spec.d + (spec.kk - 1) * spec.Hkv * spec.d + spec.Hkv * spec.d
    return (np.zeros((B, spec.Hkv, cap, spec.d)), np.zeros((B, spec.Hkv, cap, spec.d)),
            np.zeros((B, W)))


def test_chunked_prefill_of_new_sequences_equals_prefill():
    """Ragged new sequences (start 0, zero state) in one packed batch give each
    sequence's prefill output, cache rows and final state."""
    rng = np.random.default_rng(16)
    spec = O.Spec(E=64, C=4, Hq=4, Hkv=2, kq=3, kk=2)
    p = rand_params(spec, rng)
    lens = [1, 6, 0, 4]
    offs = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((offs[-1], 64))
    kc, vc, st = _fresh_caches(spec, len(lens), 8)
    y, kc2, vc2, st2 = O.prefill_chunks(x, offs, None, p, spec, kc, vc, st)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(kc2[b] == 0) and np.all(st2[b] == 0)
            continue
        yb, sv = O.forward(x[None, offs[b]:offs[b + 1]], p, spec, return_saved=True)
        assert rel(y[offs[b]:offs[b + 1]], yb[0]) < 1e-12
        assert rel(kc2[b, :, :n], np.transpose(sv["k_rope"][0], (1, 0, 2))) < 1e-12
        assert rel(vc2[b, :, :n], np.transpose(sv["v_shift"][0], (1, 0, 2))) < 1e-12
        assert rel(st2[b], sv["state"][0]) < 1e-14
        assert np.all(kc2[b, :, n:] == 0)


def test_chunked_prefill_is_independent_of_the_chunking():
    """A sequence fed as one chunk of 7 tokens, or as chunks of 3 and 4 (the
    second starting where the first left the cache and state), gives the same
    outputs, cache and state."""
    rng = np.random.default_rng(17)
    spec = O.Spec(E=64, C=4, Hq=4, Hkv=1, kq=2, kk=3)
    p = rand_params(spec, rng)
    x = rng.standard_normal((7, 64))
    kc, vc, st = _fresh_caches(spec, 1, 10)
    y1, kc1, vc1, st1 = O.prefill_chunks(x, [0, 7], [0], p, spec, kc, vc, st)
    ya, kca, vca, sta = O.prefill_chunks(x[:3], [0, 3], [0], p, spec, kc, vc, st)
    yb, kcb, vcb, stb = O.prefill_chunks(x[3:], [0, 4], [3], p, spec, kca, vca, sta)
    assert rel(np.concatenate([ya, yb]), y1) < 1e-13
    assert rel(kcb, kc1) < 1e-13 and rel(vcb, vc1) < 1e-13 and rel(stb, st1) < 1e-13


# ------------------------------------------------------- backward

def _loss(x, dy, p, spec):
    return float(np.sum(dy * O.forward(x, p, spec)))


@pytest.mark.parametrize("Hq,Hkv,flags", [(4, 2, (True, True, True, True)),
                                           (2, 2, (True, False, True, True)),
                                           (4, 1, (False, True, False, True)),
                                           (2, 1, (True, True, True, False))])
def test_backward_matches_central_differences(Hq, Hkv, flags):
    """Directional central differences of <dy, forward> agree with the
    oracle's gradient for x and for every parameter separately."""
    pre, post, use_rope, vsh = flags
    rng = np.random.default_rng(16 + Hq + Hkv)
    spec = O.Spec(E=32, C=2, Hq=Hq, Hkv=Hkv, kq=2, kk=3, qk_pre=pre, qk_post=post,
                  use_rope=use_rope, use_vshift=vsh)
    p = rand_params(spec, rng)
    x = rng.standard_normal((2, 13, 32))
    dy = rng.standard_normal((2, 13, 32))
    g = O.backward(x, dy, p, spec)
    eps = 1e-5
    names = {"dx": None, "dw_q": "w_q", "dw_k": "w_k", "dw_v": "w_v", "dw_o": "w_o",
             "dconv_q": "conv_q", "dconv_k": "conv_k"}
    for gname, pname in names.items():
        base = x if pname is None else p[pname]
        delta = rng.standard_normal(base.shape)
        def at(s):
            if pname is None:
                return _loss(x + s * delta, dy, p, spec)
            q = dict(p)
            q[pname] = p[pname] + s * delta
            return _loss(x, dy, q, spec)
        fd = (at(eps) - at(-eps)) / (2 * eps)
        an = float(np.sum(g[gname] * delta))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (gname, fd, an)


def test_backward_elementwise_tiny():
    """Per-entry central differences for a handful of entries of every
    gradient on a tiny CCGQA layer."""
    rng = np.random.default_rng(17)
    spec = O.Spec(E=16, C=2, Hq=2, Hkv=1, kq=2, kk=2)
    p = rand_params(spec, rng)
    x = rng.standard_normal((1, 5, 16))
    dy = rng.standard_normal((1, 5, 16))
    g = O.backward(x, dy, p, spec)
    eps = 1e-6
    for gname, pname in {"dx": None, "dw_q": "w_q", "dw_v": "w_v", "dconv_q": "conv_q",
                         "dconv_k": "conv_k", "dw_o": "w_o", "dw_k": "w_k"}.items():
        arr = x if pname is None else p[pname]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            def at(s):
                a2 = arr.copy()
                a2[idx] += s
                if pname is None:
                    return _loss(a2, dy, p, spec)
                q = dict(p)
                q[pname] = a2
                return _loss(x, dy, q, spec)
            fd = (at(eps) - at(-eps)) / (2 * eps)
            assert abs(fd - g[gname][idx]) < 1e-7 * max(1.0, abs(fd)), (gname, idx)
