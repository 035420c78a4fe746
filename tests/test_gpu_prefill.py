"""GPU parity of the forward prefill against the float64 oracle.

Element-by-element on every stage the library saves (q~|k~|v~, Q'', K'', V',
O, lse) and on y, for small workloads that span several tiles with ragged
tails; on the 16k CCGQA workload, y on sampled rows (the oracle computes K''
and V' for every token and attention only for the sampled query rows).
Bounds: relative L2 <= 1e-5 (fp32 storage), <= 1e-2 (bf16 storage).
"""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import WORKLOADS, Workload, make_inputs
from oracle import cca as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import (TOL, host, params_of, rel, run_prefill, saved_views, say,  # noqa: E402
                         spec_of)


def check_prefill(w: Workload, inp, stages=True):
    say(f"[prefill] {w}")
    r = run_prefill(w, inp)
    spec = spec_of(w)
    y_ref, sv = O.forward(inp["x"], params_of(inp), spec, return_saved=True)
    tol = TOL[w.dtype]
    errs = {"y": rel(host(r["y"]), y_ref)}
    if stages:
        B, S = w.B, w.S
        v = saved_views(r["layer"], r["saved"], w, B, S)
        qkv_ref = np.concatenate([np.stack(sv["q_lat"]).reshape(B, S, -1),
                                  np.stack(sv["k_lat"]).reshape(B, S, -1),
                                  np.stack(sv["v_lat"]).reshape(B, S, -1)], axis=2)
        errs["qkv"] = rel(host(v["qkv"]).reshape(B, S, -1), qkv_ref)
        errs["q_rope"] = rel(host(v["q_rope"]), np.stack(sv["q_rope"]).transpose(0, 2, 1, 3))
        errs["k_rope"] = rel(host(v["k_rope"]), np.stack(sv["k_rope"]).transpose(0, 2, 1, 3))
        errs["v_shift"] = rel(host(v["v_shift"]), np.stack(sv["v_shift"]).transpose(0, 2, 1, 3))
        errs["o"] = rel(host(v["o"]), np.stack(sv["o"]).reshape(B, S, -1))
        errs["lse"] = rel(host(v["lse"]), np.stack(sv["lse"]))
        errs["o32"] = rel(host(v["o32"]), np.stack(sv["o"]).reshape(B, S, -1))
    say(f"  rel errors {errs}")
    for k, e in errs.items():
        assert e <= tol, (k, e, tol)
    return r


SMALL_F32 = [
    WORKLOADS["cca_tiny_f32"],
    Workload("f32_gqa_ragged", B=2, S=37, E=128, C=2, Hq=4, Hkv=2, dtype="f32", seed=21),
    Workload("f32_k3_k1", B=1, S=70, E=96, C=1, Hq=2, Hkv=1, kq=3, kk=1, dtype="f32", seed=22),
    Workload("f32_single_token", B=3, S=1, E=64, C=2, Hq=2, Hkv=2, dtype="f32", seed=23),
    Workload("f32_no_extras", B=1, S=50, E=64, C=1, Hq=4, Hkv=4, flags=0, dtype="f32", seed=24),
    Workload("f32_pre_only", B=1, S=50, E=64, C=1, Hq=4, Hkv=1, flags=1 | 8, dtype="f32", seed=25),
    Workload("f32_post_rope", B=1, S=50, E=64, C=1, Hq=4, Hkv=2, flags=2 | 4, sv=3, dtype="f32",
             seed=26),
    Workload("f32_d128_g8", B=1, S=40, E=1024, C=1, Hq=8, Hkv=1, dtype="f32", seed=27),
]


@pytest.mark.parametrize("w", SMALL_F32, ids=[w.name for w in SMALL_F32])
def test_prefill_f32(w):
    check_prefill(w, make_inputs(w))


SMALL_BF16 = [
    Workload("bf16_gqa_ragged", B=1, S=300, E=512, C=1, Hq=4, Hkv=2, seed=31),
    Workload("bf16_cca_b2", B=2, S=257, E=1024, C=2, Hq=4, Hkv=4, seed=32),
    Workload("bf16_g4_k3", B=1, S=200, E=512, C=1, Hq=4, Hkv=1, kq=3, kk=2, seed=33),
    Workload("bf16_single_token", B=2, S=1, E=512, C=1, Hq=4, Hkv=2, seed=34),
    Workload("bf16_no_extras", B=1, S=130, E=512, C=1, Hq=4, Hkv=4, flags=0, seed=35),
    # the same-GPU comparators of the 16k layer at small S: MHA (no compression,
    # 16 heads of 128, one-tap convolution, RoPE only) and GQA (2 KV heads)
    Workload("bf16_mha_c1", B=1, S=200, E=2048, C=1, Hq=16, Hkv=16, kq=1, kk=1, flags=4,
             seed=36),
    Workload("bf16_gqa_c1", B=1, S=200, E=2048, C=1, Hq=16, Hkv=2, kq=1, kk=1, flags=4,
             seed=37),
    # the 16x variant (one KV head) and d = 64 (the generic kernels)
    Workload("bf16_ccgqa16", B=1, S=200, E=2048, C=4, Hq=4, Hkv=1, seed=38),
    Workload("bf16_d64", B=1, S=150, E=512, C=2, Hq=4, Hkv=2, seed=39),
    Workload("bf16_tiny_tail", B=1, S=65, E=512, C=2, Hq=2, Hkv=1, flags=1 | 4 | 8, sv=40,
             seed=36),
]


@pytest.mark.parametrize("w", SMALL_BF16, ids=[w.name for w in SMALL_BF16])
def test_prefill_bf16(w):
    check_prefill(w, make_inputs(w))


def test_prefill_cca_4k_bf16():
    w = WORKLOADS["cca_prefill_4k"]
    check_prefill(w, make_inputs(w))


def check_sampled_rows(w: Workload, n_random=43):
    """y of a large prefill on sampled rows (the first and last included): the
    oracle computes K'' and V' for every token and attention only for the
    sampled query rows."""
    inp = make_inputs(w)
    say(f"[prefill sampled] {w}")
    r = run_prefill(w, inp, with_saved=False)
    y = host(r["y"])[0]
    spec = spec_of(w)
    p = params_of(inp)
    x = inp["x"][0].astype(np.float64)
    S, G, d = w.S, w.G, w.d
    q_lat = O.project(x, p["w_q"]).reshape(S, w.Hq, d)
    k_lat = O.project(x, p["w_k"]).reshape(S, w.Hkv, d)
    v_lat = O.project(x, p["w_v"]).reshape(S, w.Hkv, d)
    q_c = O.conv_causal(q_lat, p["conv_q"])
    k_c = O.conv_causal(k_lat, p["conv_k"])
    q_m, k_m = O.qk_mean(q_lat, k_lat, q_c, k_c, G, True, True)
    v_s = O.value_shift(v_lat, spec.mask())
    pos = np.arange(S)
    k_r = O.rope(k_m, pos, w.rope_base)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, S - 1], rng.integers(0, S, n_random)]))
    q_r = O.rope(q_m[rows], rows, w.rope_base)
    o, _ = O.attention(q_r, k_r, v_s, G, q_pos=rows)
    y_ref = O.project(o.reshape(len(rows), -1), p["w_o"])
    e = rel(y[rows], y_ref)
    say(f"  sampled rows rel error {e:.3e}")
    assert e <= TOL["bf16"]
    assert np.all(np.isfinite(y))


def test_prefill_ccgqa_16k_sampled_rows():
    """Full-size CCGQA prefill (S = 16384) in the launch configuration the
    benchmark times."""
    check_sampled_rows(WORKLOADS["ccgqa_prefill_16k"])


def test_prefill_ragged_large_sampled_rows():
    """S = 5000 at E = 2048: the 256 x 256 projection GEMMs with a ragged last
    row tile (5000 = 19 * 256 + 136) and the attention's ragged last block."""
    check_sampled_rows(Workload("ccgqa_ragged_5000", B=1, S=5000, E=2048, C=4, Hq=4, Hkv=2,
                                seed=43), n_random=60)


def test_causality_bit_identical_on_gpu():
    """Perturbing tokens t >= t0 leaves y[:t0] bitwise unchanged."""
    w = Workload("bf16_causal", B=1, S=700, E=512, C=1, Hq=4, Hkv=2, seed=41)
    inp = make_inputs(w)
    y0 = run_prefill(w, inp, with_saved=False)["y"].clone()
    inp2 = dict(inp)
    x2 = inp["x"].copy()
    t0 = 333
    x2[:, t0:] = np.asarray(np.random.default_rng(1).standard_normal(x2[:, t0:].shape),
                            np.float32)
    from compressed_latent_attention_amd.synthetic import round_bf16
    inp2["x"] = round_bf16(x2)
    y1 = run_prefill(w, inp2, with_saved=False)["y"]
    assert torch.equal(y0[:, :t0], y1[:, :t0])
    assert not torch.equal(y0[:, t0], y1[:, t0])


def test_prefill_is_deterministic():
    w = Workload("bf16_det", B=1, S=513, E=512, C=1, Hq=4, Hkv=2, seed=42)
    inp = make_inputs(w)
    a = run_prefill(w, inp)
    b = run_prefill(w, inp)
    assert torch.equal(a["y"], b["y"])
    va = saved_views(a["layer"], a["saved"], w, w.B, w.S)
    vb = saved_views(b["layer"], b["saved"], w, w.B, w.S)
    for k in va:
        assert torch.equal(va[k], vb[k]), k


def test_empty_batch_or_sequence_is_rejected():
    """B = 0 or S = 0: prefill and backward return CCA_ERR_INVALID_ARG before
    any launch and leave their outputs as they were."""
    import ctypes

    import compressed_latent_attention_amd as cca
    w = Workload("bf16_empty", B=1, S=8, E=512, C=1, Hq=4, Hkv=2, seed=43)
    r = run_prefill(w, make_inputs(w), with_saved=True)
    lib, h = cca.load(), r["layer"].handle
    wts = cca._weights(r["w"])
    y = torch.full_like(r["y"], 7.0)
    ws = r["layer"].workspace(cca.CCA_OP_PREFILL, 1, 8)
    for B, S in ((0, 8), (1, 0)):
        st = lib.cca_forward_prefill(h, ctypes.byref(wts), cca._ptr(r["x"]), B, S, cca._ptr(y),
                                     None, None, None, None, cca._ptr(ws), None)
        assert st == cca.CCA_ERR_INVALID_ARG, (B, S, st)
    g = cca.cca_grads()
    dx = torch.full_like(r["x"], 7.0)
    g.dx = cca._ptr(dx)
    grads = {n: torch.zeros(r["w"][n[1:]].shape, dtype=torch.float32, device="cuda")
             for n in ("dw_q", "dw_k", "dw_v", "dw_o", "dconv_q", "dconv_k")}
    for n, t in grads.items():
        setattr(g, n, cca._ptr(t))
    wsb = r["layer"].workspace(cca.CCA_OP_BACKWARD, 1, 8)
    for B, S in ((0, 8), (1, 0)):
        st = lib.cca_backward(h, ctypes.byref(wts), cca._ptr(r["x"]), cca._ptr(r["x"]),
                              cca._ptr(r["saved"]), B, S, ctypes.byref(g), cca._ptr(wsb), None)
        assert st == cca.CCA_ERR_INVALID_ARG, (B, S, st)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((dx == 7.0).all())
    assert all(int(torch.count_nonzero(t)) == 0 for t in grads.values())
