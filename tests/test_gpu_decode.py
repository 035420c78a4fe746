"""GPU parity of the decode step against the float64 oracle.

* decode == prefill: a GPU prefill of S tokens (writing the cache and the
  rolling state) followed by GPU decode steps reproduces the oracle's prefill
  rows S, S+1, and the cache rows and state the oracle leaves;
* the 32-sequence CCGQA decode over a seeded 32768-token cache, every output
  element against the oracle's decode step.
"""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import (WORKLOADS, Workload, make_inputs,
                                                       round_bf16)
from oracle import cca as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import (TOL, dev, dev_weights, host, layer_of, params_of, rel,  # noqa: E402
                         run_prefill, say, spec_of)

CASES = [
    Workload("f32_decode", B=2, S=29, E=128, C=2, Hq=4, Hkv=2, dtype="f32", seed=51),
    Workload("f32_decode_k3", B=1, S=5, E=64, C=1, Hq=2, Hkv=2, kq=3, kk=1, dtype="f32", seed=52),
    Workload("bf16_decode", B=3, S=150, E=512, C=1, Hq=4, Hkv=2, seed=53),
    Workload("bf16_decode_g4", B=2, S=64, E=512, C=1, Hq=4, Hkv=1, kq=3, kk=2, seed=54),
    Workload("bf16_decode_first", B=2, S=1, E=512, C=1, Hq=4, Hkv=2, seed=55),
    # one query head per KV head, and eight: the other group-size instances
    Workload("bf16_decode_mha", B=2, S=90, E=512, C=1, Hq=4, Hkv=4, seed=57),
    Workload("bf16_decode_g8", B=2, S=70, E=1024, C=1, Hq=8, Hkv=1, seed=58),
    # one sequence over a longer cache: several work-groups per head, waves
    # with no block, a partly valid last block
    Workload("bf16_decode_long", B=1, S=1000, E=512, C=1, Hq=4, Hkv=2, seed=59),
    # head dimension 64: group sizes 2, 1 and 4, three taps, a longer cache
    Workload("bf16_decode_d64", B=3, S=150, E=512, C=2, Hq=4, Hkv=2, seed=60),
    Workload("bf16_decode_d64_mha", B=2, S=90, E=256, C=1, Hq=4, Hkv=4, seed=61),
    Workload("bf16_decode_d64_g4_k3", B=2, S=700, E=1024, C=2, Hq=8, Hkv=2, kq=3, kk=2, seed=62),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_decode_continues_prefill(w):
    say(f"[decode] {w}")
    steps = 2
    full = w.replace(S=w.S + steps)
    inp = make_inputs(full)
    spec = spec_of(w)
    y_ref, sv = O.forward(inp["x"], params_of(inp), spec, return_saved=True)
    pre = dict(inp)
    pre["x"] = inp["x"][:, :w.S]
    r = run_prefill(w.replace(max_seq_len=w.S + 8), pre, with_saved=False, with_cache=True)
    layer, kc, vc, st, wts = r["layer"], r["k_cache"], r["v_cache"], r["state"], r["w"]
    tol = TOL[w.dtype]
    for i in range(steps):
        p = w.S + i
        xn = dev(inp["x"][:, p], w)
        y = layer.decode_step(wts, xn, [p] * w.B, kc, vc, st)
        torch.cuda.synchronize()
        e_y = rel(host(y), y_ref[:, p])
        e_k = rel(host(kc[:, :, p]), np.stack([s[p] for s in sv["k_rope"]]))
        e_v = rel(host(vc[:, :, p]), np.stack([s[p] for s in sv["v_shift"]]))
        say(f"  step {i}: y {e_y:.2e} k {e_k:.2e} v {e_v:.2e}")
        assert e_y <= tol and e_k <= tol and e_v <= tol
    # the state after the last step is the state a prefill of S + steps leaves
    e_s = rel(host(st), np.stack(sv["state"]))
    assert e_s <= tol, e_s


def test_prefill_writes_cache_and_state():
    w = Workload("bf16_cache", B=2, S=77, E=512, C=1, Hq=4, Hkv=2, seed=56, max_seq_len=100)
    inp = make_inputs(w)
    r = run_prefill(w, inp, with_saved=False, with_cache=True)
    _, sv = O.forward(inp["x"], params_of(inp), spec_of(w), return_saved=True)
    kc = host(r["k_cache"])
    assert rel(kc[:, :, :w.S], np.stack(sv["k_rope"]).transpose(0, 2, 1, 3)) <= TOL["bf16"]
    assert rel(host(r["v_cache"])[:, :, :w.S],
               np.stack(sv["v_shift"]).transpose(0, 2, 1, 3)) <= TOL["bf16"]
    assert np.all(kc[:, :, w.S:] == 0)           # rows past S are untouched
    assert rel(host(r["state"]), np.stack(sv["state"])) <= TOL["bf16"]


def test_decode_ccgqa_32k_full_size():
    """32 sequences, each with a 32768-token seeded cache, one new token each:
    y, the written cache row and the advanced state, every element."""
    w = WORKLOADS["ccgqa_decode_32k"]
    say(f"[decode32k] {w}")
    inp = make_inputs(w)
    layer = layer_of(w)
    wts = dev_weights(inp, w)
    kc = dev(inp["k_cache"], w)
    vc = dev(inp["v_cache"], w)
    st = dev(inp["state"], w)
    xn = dev(inp["x_new"], w)
    y = layer.decode_step(wts, xn, inp["pos"].tolist(), kc, vc, st)
    torch.cuda.synchronize()
    y_ref, kc_ref, vc_ref, st_ref = O.decode_step(inp["x_new"], params_of(inp), spec_of(w),
                                                  inp["k_cache"], inp["v_cache"], inp["state"],
                                                  inp["pos"])
    p = w.S
    errs = {"y": rel(host(y), y_ref), "k": rel(host(kc[:, :, p]), kc_ref[:, :, p]),
            "v": rel(host(vc[:, :, p]), vc_ref[:, :, p]), "state": rel(host(st), st_ref)}
    say(f"  rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
    # rows before p are untouched
    assert torch.equal(kc[:, :, :p], dev(inp["k_cache"][:, :, :p], w))


@pytest.mark.parametrize("heads", [(4, 2), (8, 4)], ids=["d128", "d64"])
def test_decode_ragged_positions_32k_cache(heads):
    """One batch whose sequences sit at different positions over a seeded
    32768-token cache: a new sequence (pos 0), the first blocks' edges (1, 31,
    32, 33), a mid-length one (1000) and the last slot of the capacity (32767).
    Cache slots past each sequence's position hold random values, so a read past
    a sequence's keys would change its output.  y, the written cache rows and
    the advanced state against the oracle, and every other cache row untouched.
    Heads of 128 (4 query, 2 KV) and of 64 (8 query, 4 KV)."""
    positions = [0, 1, 31, 32, 33, 1000, 32767]
    w = Workload("ccgqa_decode_ragged", B=len(positions), S=32767, E=2048, C=4, Hq=heads[0],
                 Hkv=heads[1], seed=44, kind="decode", max_seq_len=32768)
    say(f"[decode ragged] {w} positions {positions}")
    inp = make_inputs(w)
    pos = np.asarray(positions, np.int32)
    layer = layer_of(w)
    wts = dev_weights(inp, w)
    kc = dev(inp["k_cache"], w)
    vc = dev(inp["v_cache"], w)
    kc0, vc0 = kc.clone(), vc.clone()
    st = dev(inp["state"], w)
    xn = dev(inp["x_new"], w)
    y = layer.decode_step(wts, xn, positions, kc, vc, st)
    torch.cuda.synchronize()
    y_ref, kc_ref, vc_ref, st_ref = O.decode_step(inp["x_new"], params_of(inp), spec_of(w),
                                                  inp["k_cache"], inp["v_cache"], inp["state"],
                                                  pos)
    bi = np.arange(w.B)
    tbi, tpos = torch.as_tensor(bi, device="cuda"), torch.as_tensor(pos.astype(np.int64),
                                                                     device="cuda")
    errs = {"y": rel(host(y), y_ref),
            "k": rel(host(kc[tbi, :, tpos]), kc_ref[bi, :, pos]),
            "v": rel(host(vc[tbi, :, tpos]), vc_ref[bi, :, pos]),
            "state": rel(host(st), st_ref)}
    per_seq = [rel(host(y[b]), y_ref[b]) for b in range(w.B)]
    say(f"  rel errors {errs}; y per sequence {['%.1e' % e for e in per_seq]}")
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
    for b, e in enumerate(per_seq):
        assert e <= TOL["bf16"], (positions[b], e)
    # every cache row other than (b, pos[b]) is untouched
    for b, p in enumerate(positions):
        for c, c0 in ((kc, kc0), (vc, vc0)):
            assert torch.equal(c[b, :, :p], c0[b, :, :p]), (b, p)
            assert torch.equal(c[b, :, p + 1:], c0[b, :, p + 1:]), (b, p)


def test_decode_rejects_positions_beyond_capacity():
    import compressed_latent_attention_amd as cca
    w = Workload("bf16_cap", B=1, S=4, E=512, C=1, Hq=4, Hkv=2, seed=57, max_seq_len=8)
    layer = layer_of(w)
    inp = make_inputs(w.replace(kind="prefill"))
    wts = dev_weights(inp, w)
    kc = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    st = torch.zeros((1, layer.state_width()), dtype=torch.bfloat16, device="cuda")
    xn = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cca.CCAError) as ei:
        layer.decode_step(wts, xn, [8], kc, vc, st)
    assert ei.value.status == cca.CCA_ERR_CAPACITY
    with pytest.raises(cca.CCAError):
        layer.decode_step(wts, xn, [-1], kc, vc, st)
    assert torch.count_nonzero(kc) == 0
