"""GPU parity of the backward pass against the float64 oracle: dx and every
weight and tap gradient, element by element (relative L2 per tensor; dx also
per block of 128 tokens), up to the full 16k CCGQA backward the benchmark
times, and with upstream gradients scaled down to the size a token-mean loss
gives (2^-20, 2^-24)."""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import WORKLOADS, Workload, make_inputs
from oracle import cca as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import (TOL, block_rel, dev, host, params_of, rel, run_prefill,  # noqa: E402
                         say, spec_of)

CASES = [
    Workload("f32_bwd_tiny", B=1, S=128, E=256, C=4, Hq=4, Hkv=4, dtype="f32", seed=61,
             kind="backward"),
    Workload("f32_bwd_gqa", B=2, S=45, E=128, C=2, Hq=4, Hkv=2, kq=3, kk=1, dtype="f32",
             seed=62, kind="backward"),
    Workload("f32_bwd_flags", B=1, S=33, E=64, C=1, Hq=2, Hkv=1, flags=2 | 8, sv=5,
             dtype="f32", seed=63, kind="backward"),
    # d = 128 in fp32: the tiled conv-input and tap-gradient kernels, ragged tiles
    Workload("f32_bwd_d128", B=2, S=300, E=256, C=1, Hq=2, Hkv=1, kq=3, kk=2, dtype="f32",
             seed=68, kind="backward"),
    Workload("bf16_bwd_gqa", B=1, S=300, E=512, C=1, Hq=4, Hkv=2, seed=64, kind="backward"),
    Workload("bf16_bwd_b2", B=2, S=129, E=1024, C=2, Hq=4, Hkv=4, kq=2, kk=3, seed=65,
             kind="backward"),
    # d = 128 with four and eight query heads per KV head (the group-size
    # instances of the pointwise adjoint); the second without the post-conv
    # QK-mean and with a 40-channel value shift
    Workload("bf16_bwd_g4", B=1, S=200, E=512, C=1, Hq=4, Hkv=1, kq=3, kk=2, seed=69,
             kind="backward"),
    Workload("bf16_bwd_g8_flags", B=1, S=150, E=1024, C=1, Hq=8, Hkv=1, flags=1 | 4 | 8, sv=40,
             seed=70, kind="backward"),
    # a single token: one step in each attention backward kernel, the weight
    # gradients on the transposed-copy path
    Workload("bf16_bwd_single", B=2, S=1, E=512, C=1, Hq=4, Hkv=2, seed=73, kind="backward"),
    # three query heads per KV head: the attention backward splits each head's
    # query range between the two work-groups of a key block (odd group size)
    # and a separate kernel adds the second partial; ragged S
    Workload("bf16_bwd_g3", B=1, S=97, E=768, C=1, Hq=6, Hkv=2, seed=71, kind="backward"),
    # two heads per KV head over a longer ragged sequence: the work-groups of a
    # key block take one head each, query blocks in descending order
    Workload("bf16_bwd_s1000", B=1, S=1000, E=512, C=1, Hq=4, Hkv=2, kq=3, kk=2, seed=72,
             kind="backward"),
    # the MHA and GQA comparators of the 16k layer (C = 1, 16 heads of 128,
    # one-tap convolution, RoPE only; GQA with 2 KV heads)
    Workload("bf16_bwd_mha_c1", B=1, S=150, E=2048, C=1, Hq=16, Hkv=16, kq=1, kk=1, flags=4,
             seed=74, kind="backward"),
    Workload("bf16_bwd_gqa_c1", B=1, S=150, E=2048, C=1, Hq=16, Hkv=2, kq=1, kk=1, flags=4,
             seed=75, kind="backward"),
    # the 16x variant (one KV head) and d = 64: group sizes 2, 1 (two
    # sequences) and 4 (four parts per key block), three taps, the flag
    # subsets, several key blocks with ragged tails
    Workload("bf16_bwd_ccgqa16", B=1, S=150, E=2048, C=4, Hq=4, Hkv=1, seed=76, kind="backward"),
    Workload("bf16_bwd_d64", B=1, S=120, E=512, C=2, Hq=4, Hkv=2, seed=77, kind="backward"),
    Workload("bf16_bwd_d64_g1_b2", B=2, S=200, E=512, C=2, Hq=4, Hkv=4, seed=81, kind="backward"),
    Workload("bf16_bwd_d64_g4_k3", B=1, S=300, E=1024, C=2, Hq=8, Hkv=2, kq=3, kk=2, seed=82,
             kind="backward"),
    Workload("bf16_bwd_d64_flags", B=1, S=129, E=512, C=2, Hq=4, Hkv=2, flags=1 | 4 | 8, sv=20,
             seed=83, kind="backward"),
    # large enough that the weight gradients run split over K (16 partial sums)
    # on the 256 x 256 kernel, and the attention backward spans 16 key blocks
    Workload("bf16_bwd_splitk", B=1, S=2048, E=1024, C=2, Hq=4, Hkv=2, seed=67,
             kind="backward"),
    # two sequences of 4500 tokens: 18 blocks of tap-gradient partials (the
    # batched reduce loop) with a ragged last block, split-K weight gradients
    # over 9000 tokens
    Workload("bf16_bwd_taps18", B=2, S=4500, E=512, C=1, Hq=4, Hkv=2, seed=78,
             kind="backward"),
]


def check_backward(w, inp, block_check=True):
    say(f"[backward] {w}")
    r = run_prefill(w, inp, with_saved=True)
    dy = dev(inp["dy"], w)
    g = r["layer"].backward(r["w"], r["x"], dy, r["saved"])
    torch.cuda.synchronize()
    ref = O.backward(inp["x"], inp["dy"], params_of(inp), spec_of(w))
    # With one token every query sees only its own key: P = 1, O = V, dP = D,
    # so dS and every gradient that flows through Q or K are exactly zero and
    # the oracle's are rounding noise.  Those are checked against the scale of
    # the gradients that do not vanish instead of relative to themselves.
    vanish = {"dw_q", "dw_k", "dconv_q", "dconv_k"} if w.S == 1 else set()
    got = {k: host(g[k]) for k in ref}
    errs = {k: rel(got[k], ref[k]) for k in ref if k not in vanish}
    say(f"  rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[w.dtype], (k, e)
    assert all(np.all(np.isfinite(a)) for a in got.values())
    if block_check:
        e_blk = block_rel(got["dx"], ref["dx"], 1)
        say(f"  dx worst 128-token block {e_blk:.2e}")
        assert e_blk <= TOL[w.dtype], ("dx block", e_blk)
    if vanish:
        scale = max(float(np.linalg.norm(ref[k])) for k in ("dw_v", "dw_o"))
        small = {k: float(np.linalg.norm(host(g[k]).astype(np.float64))) / scale for k in vanish}
        say(f"  vanishing gradients / scale {small}")
        for k, e in small.items():
            assert e <= 1e-4, (k, e)
    return g


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_backward(w):
    check_backward(w, make_inputs(w))


def test_backward_ccgqa_16k_full():
    """The full-size CCGQA backward (S = 16384, E = 2048) the benchmark times:
    the eight-wave dx GEMM, split-K weight gradients over 16384 tokens and 32
    blocks of tap-gradient partials, every gradient against the oracle."""
    w = WORKLOADS["ccgqa_backward_16k"]
    check_backward(w, make_inputs(w))


def test_backward_ccgqa_d64_16k_full():
    """The d = 64 CCGQA layer's backward at full size (S = 16384, E = 2048, 8
    query and 4 KV heads of 64), every gradient against the oracle."""
    w = WORKLOADS["ccgqa_d64_prefill_16k"].replace(name="ccgqa_d64_backward_16k", kind="backward")
    check_backward(w, make_inputs(w))


@pytest.mark.parametrize("dy_log2", [-20, -24])
def test_backward_small_upstream_gradient(dy_log2):
    """dY scaled by 2^-20 and 2^-24, the size of the upstream gradient of a
    loss averaged over many tokens.  Every gradient is linear in dY, so the
    relative error bound is the same as at dY ~ N(0, 1)."""
    w = Workload(f"bf16_bwd_dy_2^{dy_log2}", B=1, S=300, E=512, C=1, Hq=4, Hkv=2, seed=79,
                 kind="backward")
    inp = make_inputs(w)
    inp["dy"] = inp["dy"] * np.float32(2.0 ** dy_log2)
    check_backward(w, inp)


def test_backward_small_input():
    """x scaled by 2^-12 (Q'', K'' and V' of order 2^-12)."""
    w = Workload("bf16_bwd_x_small", B=1, S=300, E=512, C=1, Hq=4, Hkv=2, seed=80,
                 kind="backward")
    inp = make_inputs(w)
    inp["x"] = inp["x"] * np.float32(2.0 ** -12)
    check_backward(w, inp)


def test_backward_is_deterministic():
    w = Workload("bf16_bwd_det", B=1, S=260, E=512, C=1, Hq=4, Hkv=2, seed=66, kind="backward")
    inp = make_inputs(w)
    r = run_prefill(w, inp, with_saved=True)
    dy = dev(inp["dy"], w)
    g1 = r["layer"].backward(r["w"], r["x"], dy, r["saved"])
    g2 = r["layer"].backward(r["w"], r["x"], dy, r["saved"])
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
