"""CPU oracle for the CCA / CCGQA layer: TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy statement of what one Compressed Convolutional
Attention layer computes (forward prefill, single-token decode, backward).
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The HIP library never calls it, and it shares no
code, table or constant with the HIP library.

Sources cited in this package (page titles; the section named after each
citation is the one on that page):

* CCA-es: "Compressed Convolutional Attention: Efficient Attention in a
  Compressed Latent Space", technical summary on gist.science, Spanish.
* CCA-fr: the same title, summary on gist.science, French (its technical part,
  sections 1-5 after the lay explanation).
* CCA-blog: "Compressed Convolutional Attention: Revolutionizing Efficiency in
  Transformers", aimodelkit.com.

Pin status: every function in ``cca.py`` is pinned by a test in
``tests/test_oracle_*.py`` against brute force on tiny inputs (``brute.py``,
pure-Python loops written separately), against textbook multi-head attention
(the reduction the pages imply when the compression and the three extras are
removed), against closed forms and invariants, and the backward against
central finite differences of the forward.  The exact composed function rests
on the readings listed in ``Spec``'s docstring: the pages print no numeric
output of the layer, so no printed value pins the composition itself.
"""
from .cca import (Spec, project, conv_causal, qk_mean, value_shift, rope_angles, rope,
                  attention, forward, decode_step, prefill_chunks, backward, default_vmask,
                  attention_flops, kv_cache_values_per_token, param_count)

__all__ = ["Spec", "project", "conv_causal", "qk_mean", "value_shift", "rope_angles",
           "rope", "attention", "forward", "decode_step", "prefill_chunks", "backward",
           "default_vmask",
           "attention_flops", "kv_cache_values_per_token", "param_count"]
