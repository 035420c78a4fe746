"""GPU parity of the fused-Q prefill (cca_set_prefill_fusion): the attention
forms Q'' from the latent itself and the mix writes only K'', V' and the
cache.  y, the cache and the state against the oracle (relative L2 <= 1e-2,
whole and per 128-token block), and against the separate passes of the same
library: identical where the separate attention runs one work-group per query
block (the attention forms Q'' with the mix's operations), within 2e-3 where it
splits each block's keys over two work-groups (fewer than 512 work-groups and
more than 8 blocks), which changes only the order of the softmax sums.  A prefill
that saves for the backward ignores the switch (bit-identical)."""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import WORKLOADS, Workload, make_inputs
from oracle import cca as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import (TOL, block_rel, host, layer_of, params_of, rel, run_prefill,  # noqa: E402
                         saved_views, say, spec_of)


def separate_attention_splits(w: Workload) -> bool:
    """Whether the separate inference prefill splits its attention's keys
    (fewer than 512 work-groups of 128 queries, and more than 8 blocks)."""
    nqb = (w.S + 127) // 128
    return nqb * w.Hq * w.B < 512 and nqb > 8


def check_fused(w: Workload):
    say(f"[fused] {w}")
    inp = make_inputs(w)
    layer = layer_of(w)
    plain = run_prefill(w, inp, with_saved=False, with_cache=True, layer=layer)
    layer.set_prefill_fusion(True)
    fused = run_prefill(w, inp, with_saved=False, with_cache=True, layer=layer)
    y_ref, sv = O.forward(inp["x"], params_of(inp), spec_of(w), return_saved=True)
    S = w.S
    pairs = {"y": (host(fused["y"]), y_ref, 1),
             "cache K''": (host(fused["k_cache"])[:, :, :S],
                           np.stack(sv["k_rope"]).transpose(0, 2, 1, 3), 2),
             "cache V'": (host(fused["v_cache"])[:, :, :S],
                          np.stack(sv["v_shift"]).transpose(0, 2, 1, 3), 2),
             "state": (host(fused["state"]), np.stack(sv["state"]), 0)}
    errs = {k: rel(a, b) for k, (a, b, _) in pairs.items()}
    blk = {k: block_rel(a, b, ax) for k, (a, b, ax) in pairs.items() if k != "state"}
    vs_plain = rel(host(fused["y"]), host(plain["y"]))
    say(f"  rel errors {errs}; worst block {blk}; fused vs separate y {vs_plain:.2e} "
        f"(identical: {torch.equal(fused['y'], plain['y'])})")
    for k, e in list(errs.items()) + list(blk.items()):
        assert e <= TOL[w.dtype], (k, e)
    # K'', V' and the state come from the same mix arithmetic: identical
    for k in ("k_cache", "v_cache", "state"):
        assert torch.equal(fused[k], plain[k]), k
    # the prologue forms Q'' with the mix's operations, so y is identical too
    # (up to the order of the softmax sums where the separate attention splits)
    if separate_attention_splits(w):
        assert vs_plain <= 2e-3, vs_plain
    else:
        assert torch.equal(fused["y"], plain["y"]), vs_plain
    # a saving prefill is unaffected by the switch
    s_on = run_prefill(w, inp, with_saved=True, layer=layer)
    layer.set_prefill_fusion(False)
    s_off = run_prefill(w, inp, with_saved=True, layer=layer)
    assert torch.equal(s_on["y"], s_off["y"])
    v_on = saved_views(layer, s_on["saved"], w, w.B, w.S)
    v_off = saved_views(layer, s_off["saved"], w, w.B, w.S)
    for k in v_on:
        assert torch.equal(v_on[k], v_off[k]), k
    layer.close()


CASES = [
    Workload("fq_gqa_ragged", B=1, S=300, E=512, C=1, Hq=4, Hkv=2, seed=91),
    Workload("fq_g1_b2", B=2, S=257, E=1024, C=2, Hq=4, Hkv=4, seed=92),
    Workload("fq_g4_k3", B=1, S=200, E=512, C=1, Hq=4, Hkv=1, kq=3, kk=2, seed=93),
    Workload("fq_k1_flags", B=1, S=130, E=512, C=1, Hq=4, Hkv=2, kq=1, kk=3, flags=1 | 8,
             seed=94),
    Workload("fq_single_token", B=2, S=1, E=512, C=1, Hq=4, Hkv=2, seed=95),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_fused_q_prefill(w):
    check_fused(w)


def test_fused_q_prefill_ccgqa_16k():
    check_fused(WORKLOADS["ccgqa_prefill_16k"])
