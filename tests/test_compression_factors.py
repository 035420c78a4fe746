"""Pins the oracle's cost accounting to the compression factors the pages
state (tests/golden/compression_factors.txt): attention FLOPs fall by C and
the CCGQA KV cache is 8x (or 16x) smaller than same-E multi-head attention.

The oracle's counts are also checked against direct counting: visible
(query, key) pairs by brute force on small S, cached values by the shapes the
oracle's decode actually reads, parameters by the arrays the layer holds."""
import os

import numpy as np
import pytest

from oracle import cca as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "compression_factors.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, value = line.split()[:2]
        out[name] = int(value)
    return out


def mha_spec(E, heads):
    # standard multi-head attention of the same hidden size: C = 1, d = E / heads
    return O.Spec(E=E, C=1, Hq=heads, Hkv=heads)


def test_visible_pair_count_matches_brute_force():
    for S in (1, 2, 7, 64):
        pairs = sum(1 for t in range(S) for s in range(S) if s <= t)
        assert O.attention_flops(S, 1, 1) == 4 * pairs


@pytest.mark.parametrize("C", [1, 2, 4, 8])
def test_attention_flops_fall_by_C(C):
    g = golden()
    E, heads, S = 2048, 16, 4096
    d_mha = E // heads
    cca = O.Spec(E=E, C=C, Hq=4, Hkv=4)
    ratio = O.attention_flops(S, heads, d_mha) / O.attention_flops(S, cca.Hq, cca.d)
    assert ratio == C * g["attention_flops_reduction_is_C"]
    if C == 4:
        assert ratio == g["attention_flops_reduction_C4"]


def test_ccgqa_kv_cache_is_8x_smaller_than_mha():
    g = golden()
    mha = mha_spec(2048, 16)
    ccgqa = O.Spec(E=2048, C=4, Hq=4, Hkv=2)          # the 16k prefill / decode layer
    ratio = O.kv_cache_values_per_token(mha.Hkv, mha.d) / \
        O.kv_cache_values_per_token(ccgqa.Hkv, ccgqa.d)
    assert ratio == g["ccgqa_kv_cache_compression"] == g["ccgqa_extreme_compression_a"]
    # one KV head instead of two: the 16x variant
    ratio16 = O.kv_cache_values_per_token(mha.Hkv, mha.d) / \
        O.kv_cache_values_per_token(1, ccgqa.d)
    assert ratio16 == g["ccgqa_extreme_compression_b"]
    # GQA with 4 KV heads of 128 (4x) holds twice the CCGQA cache
    gqa = O.kv_cache_values_per_token(4, 128)
    assert gqa / O.kv_cache_values_per_token(ccgqa.Hkv, ccgqa.d) == g["ccgqa_half_of_gqa_mla_cache"]


def test_kv_count_matches_what_decode_reads():
    # the decode step reads exactly k_cache and v_cache of shape [Hkv, L, d]
    spec = O.Spec(E=64, C=2, Hq=4, Hkv=2)
    rng = np.random.default_rng(0)
    L = 5
    k = rng.standard_normal((L, spec.Hkv, spec.d))
    per_token = 2 * k[0].size
    assert per_token == O.kv_cache_values_per_token(spec.Hkv, spec.d)


def test_param_count_matches_arrays():
    spec = O.Spec(E=256, C=4, Hq=4, Hkv=2, kq=2, kk=3)
    d = spec.d
    shapes = [(spec.Hq * d, 256), (spec.Hkv * d, 256), (spec.Hkv * d, 256), (256, spec.Hq * d),
              (spec.Hq, spec.kq, d, d), (spec.Hkv, spec.kk, d, d)]
    assert O.param_count(spec) == sum(int(np.prod(s)) for s in shapes)
    # fewer parameters than same-E MHA (4 E^2) once C > 1
    assert O.param_count(spec) < 4 * 256 * 256
