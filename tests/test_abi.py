"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and validates configs in host code (no GPU call is made here)."""
import ctypes
import os
import re

import pytest

import compressed_latent_attention_amd as cca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cca.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cca_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("cca_create", "cca_forward_prefill", "cca_decode_step", "cca_backward",
              "cca_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = cca.load()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding wraps each of them
    assert set(declared_functions()) == set(cca._SIGNATURES)


def test_library_exports_no_cxx_mangled_api():
    out = os.popen(f"nm -D --defined-only {cca.LIB_PATH}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported


def cfg(**kw):
    base = dict(E=2048, C=4, n_q_heads=4, n_kv_heads=2, max_seq_len=16384, dtype="bf16")
    base.update(kw)
    return cca.make_config(**base)


def status(c):
    return cca.cca_validate_config(c)[0]


def test_valid_configs_pass():
    assert status(cfg()) == cca.CCA_OK
    assert status(cfg(E=256, C=4, n_q_heads=4, n_kv_heads=4, max_seq_len=128,
                      dtype="f32")) == cca.CCA_OK
    assert status(cfg(n_kv_heads=1)) == cca.CCA_OK


@pytest.mark.parametrize("kw", [
    dict(E=2050),                     # E % (C * Hq) != 0
    dict(n_kv_heads=3),               # Hq % Hkv != 0
    dict(E=12, C=4, n_q_heads=1),     # odd head dim
    dict(conv_kernel_q=0),
    dict(conv_kernel_k=0),
    dict(v_shift_channels=129),
    dict(v_shift_channels=-1),
    dict(max_seq_len=0),
    dict(C=0),
    dict(flags=16),
    dict(rope_base=1.0),
])
def test_invalid_configs_are_rejected(kw):
    assert status(cfg(**kw)) == cca.CCA_ERR_INVALID_CONFIG


@pytest.mark.parametrize("kw", [
    dict(E=4096, C=4, n_q_heads=4, n_kv_heads=2),   # d = 256 > 128
    dict(conv_kernel_q=5),
    dict(n_q_heads=16, n_kv_heads=1, C=1),          # G = 16
    dict(E=80, C=2, n_q_heads=2, n_kv_heads=1),     # bf16 with d = 20 (not a multiple of 8)
])
def test_unsupported_configs_are_reported(kw):
    assert status(cfg(**kw)) == cca.CCA_ERR_UNSUPPORTED


def test_struct_size_mismatch_is_rejected():
    c = cfg()
    c.struct_size = ctypes.sizeof(cca.cca_config) - 8
    assert status(c) == cca.CCA_ERR_INVALID_CONFIG
    assert ctypes.sizeof(cca.cca_config) == 56


def test_null_arguments_are_rejected_before_any_gpu_call():
    lib = cca.load()
    assert lib.cca_validate_config(None, None, 0) == cca.CCA_ERR_INVALID_CONFIG
    assert lib.cca_create(ctypes.byref(cfg()), None) == cca.CCA_ERR_INVALID_ARG
    assert lib.cca_forward_prefill(None, None, None, 1, 1, None, None, None, None, None, None,
                                   None) == cca.CCA_ERR_INVALID_ARG
    assert lib.cca_decode_step(None, None, None, None, 1, None, None, None, None, None,
                               None) == cca.CCA_ERR_INVALID_ARG
    assert lib.cca_backward(None, None, None, None, None, 1, 1, None, None,
                            None) == cca.CCA_ERR_INVALID_ARG
    assert lib.cca_decode_step_noalloc(None, None, None, None, 1, None, None, None, None,
                                       None) == cca.CCA_ERR_INVALID_ARG
    assert lib.cca_workspace_bytes(None, 0, 1, 1) == 0
    assert lib.cca_saved_bytes(None, 1, 1) == 0
    assert lib.cca_state_bytes(None, 1) == 0
    assert lib.cca_profile_read(None, None, 0) == -1
    assert lib.cca_profile_flush(None, None, 0) == cca.CCA_ERR_INVALID_ARG
    lib.cca_destroy(None)


def test_status_strings():
    lib = cca.load()
    for s in range(8):
        assert lib.cca_status_string(s)
    assert lib.cca_status_string(99) == b"unknown status"


def test_stale_library_is_refused(monkeypatch):
    """load() compares the source hash compiled into the library with the
    hash of the sources beside it and raises on a mismatch."""
    import compressed_latent_attention_amd.build as build
    lib = cca.load()
    assert lib.cca_source_hash().decode() == build.source_hash()
    monkeypatch.setattr(cca, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 64)
    with pytest.raises(ImportError, match="stale"):
        cca.load()


def test_invalid_config_message():
    st, msg = cca.cca_validate_config(cfg(n_kv_heads=3))
    assert st == cca.CCA_ERR_INVALID_CONFIG and "n_kv_heads" in msg
