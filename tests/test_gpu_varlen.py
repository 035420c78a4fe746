"""GPU parity of the chunked, variable-length batched prefill
(cca_forward_prefill_varlen) against the oracle's chunked prefill (each new
token decoded in turn over the cache and the rolling state).

* new sequences of ragged lengths (start 0, zero state) in one call;
* continuation chunks over seeded caches and states at ragged start positions,
  including an empty chunk and a chunk that ends at the cache capacity;
* the same sequence as one chunk and as two chunks;
* rejection of out-of-range lengths and positions before any launch.
Relative L2 <= 1e-2 (bf16 storage) on y, the written cache rows and the state;
cache rows outside the chunks must be untouched.
"""
import numpy as np
import pytest

from compressed_latent_attention_amd.synthetic import WORKLOADS, Workload, make_inputs, varlen_layout
from oracle import cca as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import compressed_latent_attention_amd as cca  # noqa: E402
from gpu_helpers import TOL, dev, dev_weights, host, layer_of, params_of, rel, say, spec_of  # noqa: E402


def _inputs(w, lens, cap, seed, fresh):
    """Packed x for the chunks; caches and state seeded N(0, 1) (fresh: zero)."""
    T = int(sum(lens))
    x = make_inputs(Workload("x", B=1, S=max(T, 1), E=w.E, C=w.C, Hq=w.Hq, Hkv=w.Hkv,
                             seed=seed))["x"][0, :T]
    dinp = make_inputs(w.replace(B=len(lens), S=cap, kind="decode", max_seq_len=cap,
                                 seed=seed + 1))
    kc, vc, st = dinp["k_cache"], dinp["v_cache"], dinp["state"]
    if fresh:
        kc, vc, st = np.zeros_like(kc), np.zeros_like(vc), np.zeros_like(st)
    return x, dinp, kc, vc, st


def check_varlen(w, lens, starts, cap, seed, fresh=False):
    say(f"[varlen] {w.name} lens {lens} starts {starts} cap {cap}")
    x, pin, kc0, vc0, st0 = _inputs(w, lens, cap, seed, fresh)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    layer = layer_of(w, max_seq_len=cap)
    wts = dev_weights(pin, w)
    kc, vc, st = dev(kc0, w), dev(vc0, w), dev(st0, w)
    kc_in, vc_in = kc.clone(), vc.clone()
    y = layer.forward_prefill_varlen(wts, dev(x, w), offs.tolist(), starts, kc, vc, st)
    torch.cuda.synchronize()
    y_ref, kc_ref, vc_ref, st_ref = O.prefill_chunks(x, offs, starts, params_of(pin), spec_of(w),
                                                     kc0, vc0, st0)
    errs = {"y": rel(host(y), y_ref), "state": rel(host(st), st_ref)}
    kh, vh = host(kc), host(vc)
    rows_k, rows_v, ref_k, ref_v = [], [], [], []
    for b, n in enumerate(lens):
        s0 = 0 if starts is None else starts[b]
        rows_k.append(kh[b, :, s0:s0 + n]); ref_k.append(kc_ref[b, :, s0:s0 + n])
        rows_v.append(vh[b, :, s0:s0 + n]); ref_v.append(vc_ref[b, :, s0:s0 + n])
        # rows outside the chunk are untouched
        assert torch.equal(kc[b, :, :s0], kc_in[b, :, :s0]), b
        assert torch.equal(kc[b, :, s0 + n:], kc_in[b, :, s0 + n:]), b
        assert torch.equal(vc[b, :, :s0], vc_in[b, :, :s0]), b
        assert torch.equal(vc[b, :, s0 + n:], vc_in[b, :, s0 + n:]), b
        if n:
            e = rel(host(y)[offs[b]:offs[b + 1]], y_ref[offs[b]:offs[b + 1]])
            assert e <= TOL[w.dtype], ("y of sequence", b, e)
    errs["k"] = rel(np.concatenate([r.reshape(-1) for r in rows_k]),
                    np.concatenate([r.reshape(-1) for r in ref_k]))
    errs["v"] = rel(np.concatenate([r.reshape(-1) for r in rows_v]),
                    np.concatenate([r.reshape(-1) for r in ref_v]))
    say(f"  rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[w.dtype], (k, e)
    assert np.all(np.isfinite(host(y)))
    layer.close()
    return host(y)


W_CCGQA = Workload("varlen_ccgqa", B=1, S=1, E=2048, C=4, Hq=4, Hkv=2, seed=0)


def test_varlen_new_sequences_ragged():
    """Four new sequences (1, 64, 200 and 130 tokens) in one packed call."""
    check_varlen(W_CCGQA, [1, 64, 200, 130], None, cap=256, seed=101, fresh=True)


def test_varlen_continuation_chunks():
    """Chunks over seeded caches: starts 0, 5, 300 and 190 (an empty chunk),
    the last ending at the capacity."""
    check_varlen(W_CCGQA, [37, 130, 212, 0], [0, 5, 300, 190], cap=512, seed=103)


def test_varlen_group_sizes_and_taps():
    """One KV head per 4 query heads (the general mix) with 3 and 1 taps, and
    one query head per KV head."""
    w4 = Workload("varlen_g4", B=1, S=1, E=512, C=1, Hq=4, Hkv=1, kq=3, kk=1, seed=0)
    check_varlen(w4, [70, 3], [10, 0], cap=128, seed=105)
    w1 = Workload("varlen_g1", B=1, S=1, E=512, C=1, Hq=4, Hkv=4, seed=0)
    check_varlen(w1, [65, 129], [63, 1], cap=256, seed=107)


def test_varlen_one_chunk_equals_two():
    """A 300-token sequence as one chunk, and as chunks of 111 and 189 tokens
    (the second from the cache and state the first left), give the same y."""
    w = W_CCGQA
    x, pin, kc0, vc0, st0 = _inputs(w, [300], 320, 109, fresh=True)
    layer = layer_of(w, max_seq_len=320)
    wts = dev_weights(pin, w)
    kc, vc, st = dev(kc0, w), dev(vc0, w), dev(st0, w)
    y1 = layer.forward_prefill_varlen(wts, dev(x, w), [0, 300], [0], kc, vc, st)
    kc2, vc2, st2 = dev(kc0, w), dev(vc0, w), dev(st0, w)
    ya = layer.forward_prefill_varlen(wts, dev(x[:111], w), [0, 111], [0], kc2, vc2, st2)
    yb = layer.forward_prefill_varlen(wts, dev(x[111:], w), [0, 189], [111], kc2, vc2, st2)
    torch.cuda.synchronize()
    e = rel(host(torch.cat([ya, yb])), host(y1))
    say(f"[varlen] one chunk vs two: y {e:.2e}")
    assert e <= TOL["bf16"]
    assert rel(host(kc2), host(kc)) <= TOL["bf16"] and rel(host(st2), host(st)) <= TOL["bf16"]
    layer.close()


def test_varlen_bench_layout_sampled():
    """The benchmark's launch configuration: 16 chunks (583..1598 tokens,
    16384 in all) continuing sequences at cached lengths 4298..30930 over
    32768-token caches, all in one call.  The oracle decodes the first 128
    tokens of two of the chunks one by one (a chunk's first tokens depend on
    nothing after them); their y rows and cache rows are compared."""
    w = WORKLOADS["ccgqa_prefill_16k"]
    cap = 32768
    offsets, starts = varlen_layout(cap=cap)
    B, T = len(starts), int(offsets[-1])
    say(f"[varlen] bench layout: {B} chunks, {T} tokens, cap {cap}")
    x = make_inputs(Workload("varlen_bench_x", B=1, S=T, E=w.E, C=w.C, Hq=w.Hq, Hkv=w.Hkv,
                             seed=21))["x"][0]
    pin = make_inputs(w.replace(name="varlen_bench_cache", B=B, S=cap, kind="decode",
                                max_seq_len=cap, seed=23))
    layer = layer_of(w, max_seq_len=cap)
    kc, vc, st = dev(pin["k_cache"], w), dev(pin["v_cache"], w), dev(pin["state"], w)
    y = layer.forward_prefill_varlen(dev_weights(pin, w), dev(x, w), offsets.tolist(),
                                     starts.tolist(), kc, vc, st)
    torch.cuda.synchronize()
    yh = host(y)
    m = 128
    for b in (10, 3):
        s0, r0 = int(starts[b]), int(offsets[b])
        rows = slice(0, s0 + m)
        y_ref, kc_ref, vc_ref, _ = O.prefill_chunks(
            x[r0:r0 + m], np.array([0, m]), np.array([s0]), params_of(pin), spec_of(w),
            pin["k_cache"][b:b + 1, :, rows], pin["v_cache"][b:b + 1, :, rows],
            pin["state"][b:b + 1])
        errs = {"y": rel(yh[r0:r0 + m], y_ref),
                "k": rel(host(kc[b, :, s0:s0 + m]), kc_ref[0, :, s0:s0 + m]),
                "v": rel(host(vc[b, :, s0:s0 + m]), vc_ref[0, :, s0:s0 + m])}
        say(f"  sequence {b} (start {s0}): rel errors {errs}")
        for k, e in errs.items():
            assert e <= TOL["bf16"], (b, k, e)
    assert np.all(np.isfinite(yh))
    layer.close()


def test_varlen_rejects_bad_layouts():
    w = W_CCGQA
    layer = layer_of(w, max_seq_len=64)
    lib, h = cca.load(), layer.handle
    i32 = cca._i32
    assert lib.cca_varlen_workspace_bytes(h, i32([0, 10, 5]), None, 2) == 0       # negative length
    assert lib.cca_varlen_workspace_bytes(h, i32([1, 10]), None, 1) == 0          # offsets[0] != 0
    assert lib.cca_varlen_workspace_bytes(h, i32([0, 10]), i32([60]), 1) == 0     # past capacity
    assert lib.cca_varlen_workspace_bytes(h, i32([0, 10]), i32([54]), 1) > 0
    x = torch.zeros((10, w.E), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, w.Hkv, 64, 128), dtype=torch.bfloat16, device="cuda")
    vc, st = torch.zeros_like(kc), torch.zeros((1, layer.state_width()), dtype=torch.bfloat16,
                                                 device="cuda")
    inp = make_inputs(Workload("wts", B=1, S=1, E=w.E, C=w.C, Hq=w.Hq, Hkv=w.Hkv, seed=3))
    wts = dev_weights(inp, w)
    with pytest.raises(cca.CCAError) as ei:
        layer.forward_prefill_varlen(wts, x, [0, 10], [60], kc, vc, st)
    assert ei.value.status == cca.CCA_ERR_CAPACITY
    with pytest.raises(cca.CCAError) as ei:
        layer.forward_prefill_varlen(wts, x, [0, 10], [-1], kc, vc, st)
    assert ei.value.status == cca.CCA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(kc)) == 0 and int(torch.count_nonzero(st)) == 0
    layer.close()
    # head dimension 64: not built for chunks, refused before any launch
    w64 = Workload("varlen_d64", B=1, S=1, E=512, C=2, Hq=4, Hkv=2, seed=0)
    l64 = layer_of(w64, max_seq_len=64)
    inp64 = make_inputs(Workload("wts64", B=1, S=1, E=512, C=2, Hq=4, Hkv=2, seed=3))
    x64 = torch.zeros((10, 512), dtype=torch.bfloat16, device="cuda")
    kc64 = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    st64 = torch.zeros((1, l64.state_width()), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cca.CCAError) as ei:
        l64.forward_prefill_varlen(dev_weights(inp64, w64), x64, [0, 10], [0], kc64,
                                   torch.zeros_like(kc64), st64)
    assert ei.value.status == cca.CCA_ERR_UNSUPPORTED
    l64.close()
