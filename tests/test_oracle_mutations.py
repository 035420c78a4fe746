"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle's source (a dropped term, a wrong
sign, index or direction, a transposed operand), loads the mutant in place of
the real function, and checks that at least one pin of
``test_oracle_pins.py`` fails.  Mistakes are planted in the oracle on the CPU
only; nothing here touches the HIP library.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import cca as O
import test_oracle_pins as P


def _battery():
    return [
        lambda: P.test_reduces_to_bruteforce_mha(True, 2),
        lambda: P.test_reduces_to_bruteforce_mha(False, 1),
        lambda: P.test_matches_scalar_loops(4, 2, 2, 3, (True, True, True)),
        lambda: P.test_matches_scalar_loops(4, 1, 3, 1, (True, False, True)),
        lambda: P.test_matches_scalar_loops(2, 1, 1, 2, (False, True, False)),
        P.test_attention_rows_sum_to_one_and_causal,
        P.test_gqa_head_mapping_uses_contiguous_groups,
        P.test_causality_bit_identical,
        P.test_conv_impulse_response_is_lag_ordered,
        P.test_value_shift_indexing,
        P.test_rope_identities,
        P.test_qk_mean_switches_and_plain_case,
        lambda: P.test_decode_equals_prefill(4, 2, 2, 2),
        lambda: P.test_decode_equals_prefill(2, 2, 3, 1),
        lambda: P.test_backward_matches_central_differences(4, 2, (True, True, True, True)),
        lambda: P.test_backward_matches_central_differences(4, 1, (False, True, False, True)),
    ]


# (function, exact source fragment, replacement, what the mistake is)
MUTANTS = [
    ("conv_causal", "lagged = ext[k - 1 - j:k - 1 - j + S]", "lagged = ext[k - 1:k - 1 + S]",
     "every tap reads the current token"),
    ("conv_causal", 'np.einsum("hcx,thx->thc", taps[:, j], lagged)',
     'np.einsum("hxc,thx->thc", taps[:, j], lagged)', "taps transposed"),
    ("conv_causal", "hist[::-1], u", "hist, u", "history in the wrong order"),
    ("qk_mean", "+ b * 0.5 * (q_post + per_query_head(k_post))",
     "+ b * 0.5 * (q_post)", "post-conv k dropped from q"),
    ("qk_mean", "a * 0.5 * (group_mean(q_pre) + k_pre)", "a * 0.5 * (q_pre[:, ::G] + k_pre)",
     "K side takes the first head instead of the group mean"),
    ("qk_mean", "return np.repeat(kv, G, axis=1)", "return np.tile(kv, (1, G, 1))",
     "query head h reads KV head h % Hkv"),
    ("value_shift", "shifted = np.concatenate([before, v[:-1]], axis=0)",
     "shifted = np.concatenate([v[1:], before], axis=0)", "shift from the next token"),
    ("value_shift", "np.where(mask[None], shifted, v)", "np.where(mask[None], v, shifted)",
     "mask inverted"),
    ("rope", "lo * c - hi * s, hi * c + lo * s", "lo * c + hi * s, hi * c - lo * s",
     "rotation sign flipped"),
    ("rope_angles", "-2.0 * i / d", "-1.0 * i / d", "wrong frequency exponent"),
    ("attention", "scale = 1.0 / math.sqrt(d)", "scale = 1.0", "missing 1/sqrt(d)"),
    ("attention", "<= p_blk[:, None]", "< p_blk[:, None] + 2", "mask lets one future key in"),
    ("attention", "g = h // G", "g = h % (k.shape[1])", "KV head h % Hkv"),
    ("attention", "lse[h, t0:t1] = (m + np.log(l))[:, 0]", "lse[h, t0:t1] = np.log(l)[:, 0]",
     "lse without the row max"),
    ("_state_after", "_lags(v_lat, 1)", "_lags(k_lat, 1)", "state keeps k instead of v"),
    ("decode_step", "kc[b, :, p] = k_r[0]", "kc[b, :, p] = k_mix[0]", "cache holds pre-RoPE K"),
    ("decode_step", "q_pos=np.array([p])", "q_pos=np.array([p - 1])", "decode misses its own key"),
    ("_attention_backward", "ds = p * (dp - D[t0:t1, None]) * scale",
     "ds = p * dp * scale", "softmax adjoint without the rowsum term"),
    ("_attention_backward", "dk[:n, g] += ds.T @ q[t0:t1, h]", "dk[:n, g] += ds.T @ k[t0:t1, g]",
     "dK uses K instead of Q"),
    ("_conv_backward", 'np.einsum("hcx,thc->thx", taps[:, j], dout[j:])',
     'np.einsum("hxc,thc->thx", taps[:, j], dout[j:])', "conv adjoint not transposed"),
    ("backward", "dq_conv = (1 + bb / 2) * dq_mix + (bb / (2 * G)) * dk_per_q",
     "dq_conv = (1 + bb / 2) * dq_mix", "QK-mean adjoint drops the K path"),
    ("backward", "dv_lat = np.where(mask[None], dv_next, dv_sh)",
     "dv_lat = dv_sh", "shift adjoint ignored"),
    ("backward", "dq_mix = rope(dq_r, pos, spec.rope_base, inverse=True)",
     "dq_mix = rope(dq_r, pos, spec.rope_base)", "RoPE adjoint rotates forward"),
    ("backward", "dk_lat = (a / 2) * sum_dq_group + (a / 2) * dk_mix",
     "dk_lat = (a / 2) * dk_mix", "pre-conv QK-mean adjoint drops the Q path"),
]


@pytest.mark.parametrize("fname,old,new,why", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_pins_kill_mutant(monkeypatch, fname, old, new, why):
    src = textwrap.dedent(inspect.getsource(getattr(O, fname)))
    assert src.count(old) == 1, f"fragment not found once in {fname}: {old}"
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), ns)
    monkeypatch.setattr(O, fname, ns[fname])
    killed = []
    with np.errstate(all="ignore"):
        for pin in _battery():
            try:
                pin()
            except Exception:          # a failed assertion or a shape error
                killed.append(pin)
                break
    assert killed, f"no pin caught the mutant: {why}"


def test_battery_passes_on_the_real_oracle():
    for pin in _battery():
        pin()
