"""The allocation-free decode entry point (cca_decode_step_noalloc) against
cca_decode_step, through the C ABI: two calls in a row on the same GPU, the
second with fewer sequences, each compared with the workspace-taking call on
identical copies of the inputs.  Both run the same kernels, so y, the written
cache rows and the advanced state must agree bit for bit (inside the 1e-2
relative bound of the bf16 parity tests)."""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import Workload, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import compressed_latent_attention_amd as cca  # noqa: E402
from gpu_helpers import dev, dev_weights, layer_of, say  # noqa: E402


def _run_both(layer, w, inp, positions):
    B = len(positions)
    wts = dev_weights(inp, w)
    xn = dev(inp["x_new"][:B], w)
    outs = []
    for noalloc in (False, True):
        kc = dev(inp["k_cache"][:B], w)
        vc = dev(inp["v_cache"][:B], w)
        st = dev(inp["state"][:B], w)
        y = torch.empty_like(xn)
        if noalloc:
            cca.cca_decode_step_noalloc(layer.handle, wts, xn, positions, B, kc, vc, st, y)
        else:
            ws = layer.workspace(cca.CCA_OP_DECODE, B, 0)
            cca.cca_decode_step(layer.handle, wts, xn, positions, B, kc, vc, st, y, ws)
        torch.cuda.synchronize()
        outs.append((y, kc, vc, st))
    return outs


def test_noalloc_decode_matches_workspace_decode():
    w = Workload("noalloc_decode", B=5, S=3000, E=2048, C=4, Hq=4, Hkv=2, seed=91,
                 kind="decode", max_seq_len=3072)
    inp = make_inputs(w)
    layer = layer_of(w)
    for positions in ([0, 17, 999, 2048, 3071], [5, 3000, 64]):
        say(f"[noalloc] {w.name} positions {positions}")
        (y0, k0, v0, s0), (y1, k1, v1, s1) = _run_both(layer, w, inp, positions)
        assert torch.equal(y0, y1)
        assert torch.equal(k0, k1) and torch.equal(v0, v1)
        assert torch.equal(s0, s1)
        assert bool(torch.isfinite(y1.float()).all())
    layer.close()


def test_noalloc_decode_rejects_what_the_workspace_call_rejects():
    w = Workload("noalloc_reject", B=1, S=4, E=512, C=1, Hq=4, Hkv=2, seed=92, kind="decode",
                 max_seq_len=8)
    inp = make_inputs(w)
    layer = layer_of(w)
    wts = dev_weights(inp, w)
    kc = dev(inp["k_cache"], w)
    vc, st, xn = dev(inp["v_cache"], w), dev(inp["state"], w), dev(inp["x_new"], w)
    y = torch.empty_like(xn)
    for pos, status in (([8], cca.CCA_ERR_CAPACITY), ([-1], cca.CCA_ERR_CAPACITY)):
        with pytest.raises(cca.CCAError) as ei:
            cca.cca_decode_step_noalloc(layer.handle, wts, xn, pos, 1, kc, vc, st, y)
        assert ei.value.status == status
    layer.close()
