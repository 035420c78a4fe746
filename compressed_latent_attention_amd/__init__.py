"""Python binding of libcca.so, the MI355X (gfx950) CCA / CCGQA layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
the shared library.  PyTorch supplies device memory and the stream; tensors are
passed as raw device pointers.  The functions keep the C names
(``cca_create``, ``cca_forward_prefill``, ``cca_decode_step``,
``cca_backward``, ``cca_destroy`` ...); ``CCALayer`` wraps them for torch
tensors.  There is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, byref, c_char, c_char_p, c_double, c_int, c_int32,
                    c_size_t, c_uint32, c_void_p)
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcca.so")

CCA_OK, CCA_ERR_INVALID_CONFIG, CCA_ERR_INVALID_ARG, CCA_ERR_UNSUPPORTED = 0, 1, 2, 3
CCA_ERR_CAPACITY, CCA_ERR_HIP, CCA_ERR_OOM, CCA_ERR_SCRATCH = 4, 5, 6, 7
CCA_F32, CCA_BF16 = 0, 1
CCA_QKMEAN_PRE, CCA_QKMEAN_POST, CCA_ROPE, CCA_VSHIFT, CCA_DEFAULT_FLAGS = 1, 2, 4, 8, 15
CCA_OP_PREFILL, CCA_OP_DECODE, CCA_OP_BACKWARD = 0, 1, 2


class cca_config(Structure):
    _fields_ = [("struct_size", c_uint32), ("E", c_int32), ("C", c_int32),
                ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("max_seq_len", c_int32),
                ("conv_kernel_q", c_int32), ("conv_kernel_k", c_int32),
                ("v_shift_channels", c_int32), ("flags", c_uint32), ("rope_base", c_double),
                ("dtype", c_int32)]


class cca_weights(Structure):
    _fields_ = [(n, c_void_p) for n in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k")]


class cca_grads(Structure):
    _fields_ = [(n, c_void_p) for n in ("dx", "dw_q", "dw_k", "dw_v", "dw_o", "dconv_q",
                                        "dconv_k")]


class cca_kernel_time(Structure):
    _fields_ = [("name", c_char * 48), ("launches", c_int32), ("total_ms", c_double)]


# every symbol include/cca.h declares, with its ctypes signature
_SIGNATURES = {
    "cca_validate_config": (c_int, [POINTER(cca_config), c_char_p, c_size_t]),
    "cca_create": (c_int, [POINTER(cca_config), POINTER(c_void_p)]),
    "cca_destroy": (None, [c_void_p]),
    "cca_workspace_bytes": (c_size_t, [c_void_p, c_int, c_int32, c_int32]),
    "cca_saved_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
    "cca_saved_offsets": (c_int, [c_void_p, c_int32, c_int32, POINTER(c_size_t)]),
    "cca_state_bytes": (c_size_t, [c_void_p, c_int32]),
    "cca_forward_prefill": (c_int, [c_void_p, POINTER(cca_weights), c_void_p, c_int32, c_int32,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p]),
    "cca_decode_step": (c_int, [c_void_p, POINTER(cca_weights), c_void_p, POINTER(c_int32),
                                c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]),
    "cca_decode_step_noalloc": (c_int, [c_void_p, POINTER(cca_weights), c_void_p,
                                        POINTER(c_int32), c_int32, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p]),
    "cca_forward_prefill_varlen": (c_int, [c_void_p, POINTER(cca_weights), c_void_p,
                                           POINTER(c_int32), POINTER(c_int32), c_int32, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "cca_varlen_workspace_bytes": (c_size_t, [c_void_p, POINTER(c_int32), POINTER(c_int32),
                                              c_int32]),
    "cca_backward": (c_int, [c_void_p, POINTER(cca_weights), c_void_p, c_void_p, c_void_p,
                             c_int32, c_int32, POINTER(cca_grads), c_void_p, c_void_p]),
    "cca_profile_enable": (c_int, [c_void_p, c_int]),
    "cca_profile_read": (c_int, [c_void_p, POINTER(cca_kernel_time), c_int]),
    "cca_profile_flush": (c_int, [c_void_p, c_void_p, c_size_t]),
    "cca_set_prefill_fusion": (c_int, [c_void_p, c_int32]),
    "cca_status_string": (c_char_p, [c_int]),
    "cca_source_hash": (c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libcca.so (built by ``build.py``); raises if it is missing or was
    built from sources other than the ones beside it (its compiled-in source
    hash differs from the hash of csrc/ and include/cca.h)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m compressed_latent_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    from .build import source_hash
    built, now = lib.cca_source_hash().decode(), source_hash()
    if built != now:
        raise ImportError(f"{path} is stale: built from sources with hash {built[:16]}, the "
                          f"sources now hash to {now[:16]}; rebuild with "
                          "`python -m compressed_latent_attention_amd.build`")
    _lib = lib
    return lib


class CCAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().cca_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str) -> None:
    if status != CCA_OK:
        raise CCAError(status, where)


def make_config(E: int, C: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int,
                conv_kernel_q: int = 2, conv_kernel_k: int = 2,
                v_shift_channels: Optional[int] = None, flags: int = CCA_DEFAULT_FLAGS,
                rope_base: float = 10000.0, dtype: str = "bf16") -> cca_config:
    d = E // (C * n_q_heads) if C * n_q_heads else 0
    cfg = cca_config()
    cfg.struct_size = ctypes.sizeof(cca_config)
    cfg.E, cfg.C, cfg.n_q_heads, cfg.n_kv_heads = E, C, n_q_heads, n_kv_heads
    cfg.max_seq_len = max_seq_len
    cfg.conv_kernel_q, cfg.conv_kernel_k = conv_kernel_q, conv_kernel_k
    cfg.v_shift_channels = d // 2 if v_shift_channels is None else v_shift_channels
    cfg.flags = flags
    cfg.rope_base = rope_base
    cfg.dtype = CCA_BF16 if dtype == "bf16" else CCA_F32
    return cfg


# --------------------------------------------------------------- C-named calls

def cca_validate_config(cfg: cca_config):
    buf = ctypes.create_string_buffer(256)
    st = load().cca_validate_config(byref(cfg), buf, 256)
    return st, buf.value.decode()


def cca_create(cfg: cca_config) -> c_void_p:
    h = c_void_p()
    _check(load().cca_create(byref(cfg), byref(h)), "cca_create")
    return h


def cca_destroy(h) -> None:
    load().cca_destroy(h)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _weights(w: Dict[str, "object"]) -> cca_weights:
    cw = cca_weights()
    for n in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k"):
        setattr(cw, n, _ptr(w[n]))
    return cw


def cca_forward_prefill(h, w, x, B, S, y, saved, k_cache, v_cache, state, workspace,
                        stream=None) -> None:
    _check(load().cca_forward_prefill(h, byref(_weights(w)), _ptr(x), B, S, _ptr(y),
                                      _ptr(saved), _ptr(k_cache), _ptr(v_cache), _ptr(state),
                                      _ptr(workspace), _stream(stream)),
           "cca_forward_prefill")


def cca_decode_step(h, w, x_new, pos, B, k_cache, v_cache, state, y_new, workspace,
                    stream=None) -> None:
    arr = (c_int32 * B)(*[int(p) for p in pos])
    _check(load().cca_decode_step(h, byref(_weights(w)), _ptr(x_new), arr, B, _ptr(k_cache),
                                  _ptr(v_cache), _ptr(state), _ptr(y_new), _ptr(workspace),
                                  _stream(stream)),
           "cca_decode_step")


def cca_decode_step_noalloc(h, w, x_new, pos, B, k_cache, v_cache, state, y_new,
                            stream=None) -> None:
    arr = (c_int32 * B)(*[int(p) for p in pos])
    _check(load().cca_decode_step_noalloc(h, byref(_weights(w)), _ptr(x_new), arr, B,
                                          _ptr(k_cache), _ptr(v_cache), _ptr(state),
                                          _ptr(y_new), _stream(stream)),
           "cca_decode_step_noalloc")


def _i32(vals):
    return None if vals is None else (c_int32 * len(vals))(*[int(v) for v in vals])


def cca_varlen_workspace_bytes(h, offsets, starts=None) -> int:
    return load().cca_varlen_workspace_bytes(h, _i32(offsets), _i32(starts), len(offsets) - 1)


def cca_forward_prefill_varlen(h, w, x, offsets, starts, y, k_cache, v_cache, state, workspace,
                               stream=None) -> None:
    """offsets: B + 1 token offsets into the packed rows of x and y; starts: B
    cached-token counts or None (all 0)."""
    _check(load().cca_forward_prefill_varlen(h, byref(_weights(w)), _ptr(x), _i32(offsets),
                                             _i32(starts), len(offsets) - 1, _ptr(y),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(state),
                                             _ptr(workspace), _stream(stream)),
           "cca_forward_prefill_varlen")


def cca_backward(h, w, x, dy, saved, B, S, grads, workspace, stream=None) -> None:
    g = cca_grads()
    for n in ("dx", "dw_q", "dw_k", "dw_v", "dw_o", "dconv_q", "dconv_k"):
        setattr(g, n, _ptr(grads[n]))
    _check(load().cca_backward(h, byref(_weights(w)), _ptr(x), _ptr(dy), _ptr(saved), B, S,
                               byref(g), _ptr(workspace), _stream(stream)),
           "cca_backward")


def cca_profile_enable(h, enable: bool) -> None:
    _check(load().cca_profile_enable(h, 1 if enable else 0), "cca_profile_enable")


def cca_profile_flush(h, buf) -> None:
    """Cold-cache timing: write over the torch uint8 tensor `buf` before every
    timed launch (None turns it off)."""
    _check(load().cca_profile_flush(h, _ptr(buf), 0 if buf is None else buf.numel()),
           "cca_profile_flush")


def cca_set_prefill_fusion(h, on: bool) -> None:
    """Inference prefill with the query side of the mix inside the attention."""
    _check(load().cca_set_prefill_fusion(h, 1 if on else 0), "cca_set_prefill_fusion")


def cca_profile_read(h) -> Dict[str, tuple]:
    lib = load()
    n = lib.cca_profile_read(h, None, 0)
    if n < 0:
        raise CCAError(CCA_ERR_HIP, "cca_profile_read")
    arr = (cca_kernel_time * max(n, 1))()
    lib.cca_profile_read(h, arr, n)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


# --------------------------------------------------------------- torch wrapper

class CCALayer:
    """One CCA / CCGQA layer bound to a libcca handle.  Tensors are torch CUDA
    tensors of the config's dtype (torch.bfloat16 or torch.float32)."""

    def __init__(self, E, C, n_q_heads, n_kv_heads, max_seq_len, conv_kernel_q=2,
                 conv_kernel_k=2, v_shift_channels=None, flags=CCA_DEFAULT_FLAGS,
                 rope_base=10000.0, dtype="bf16"):
        import torch
        self.cfg = make_config(E, C, n_q_heads, n_kv_heads, max_seq_len, conv_kernel_q,
                               conv_kernel_k, v_shift_channels, flags, rope_base, dtype)
        self.handle = cca_create(self.cfg)
        self.E, self.Hq, self.Hkv = E, n_q_heads, n_kv_heads
        self.d = E // (C * n_q_heads)
        self.max_seq_len = max_seq_len
        self.dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self._ws = {}

    def close(self):
        if self.handle is not None:
            cca_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, op: int, B: int, S: int, device="cuda"):
        import torch
        n = load().cca_workspace_bytes(self.handle, op, B, S)
        key = (op, str(device))
        buf = self._ws.get(key)
        if buf is None or buf.numel() < n:
            buf = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self._ws[key] = buf
        return buf

    def set_prefill_fusion(self, on: bool) -> None:
        cca_set_prefill_fusion(self.handle, on)

    def saved_bytes(self, B, S) -> int:
        return load().cca_saved_bytes(self.handle, B, S)

    def saved_offsets(self, B, S):
        offs = (c_size_t * 8)()
        _check(load().cca_saved_offsets(self.handle, B, S, offs), "cca_saved_offsets")
        return list(offs)

    def state_width(self) -> int:
        es = 2 if self.cfg.dtype == CCA_BF16 else 4
        return load().cca_state_bytes(self.handle, 1) // es

    def forward_prefill(self, w, x, saved=None, k_cache=None, v_cache=None, state=None,
                        stream=None):
        import torch
        B, S, E = x.shape
        y = torch.empty_like(x)
        ws = None if saved is not None else self.workspace(CCA_OP_PREFILL, B, S, x.device)
        cca_forward_prefill(self.handle, w, x, B, S, y, saved, k_cache, v_cache, state, ws,
                            stream)
        return y

    def decode_step(self, w, x_new, pos, k_cache, v_cache, state, stream=None):
        import torch
        B = x_new.shape[0]
        y = torch.empty_like(x_new)
        ws = self.workspace(CCA_OP_DECODE, B, 0, x_new.device)
        cca_decode_step(self.handle, w, x_new, pos, B, k_cache, v_cache, state, y, ws, stream)
        return y

    def forward_prefill_varlen(self, w, x, offsets, starts, k_cache, v_cache, state,
                               stream=None):
        """Chunked variable-length prefill of packed rows x [T, E]; returns y."""
        import torch
        y = torch.empty_like(x)
        n = load().cca_varlen_workspace_bytes(self.handle, _i32(offsets), _i32(starts),
                                              len(offsets) - 1)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
        cca_forward_prefill_varlen(self.handle, w, x, offsets, starts, y, k_cache, v_cache,
                                   state, ws, stream)
        return y

    def backward(self, w, x, dy, saved, stream=None):
        import torch
        B, S, E = x.shape
        grads = {"dx": torch.empty_like(x)}
        for n in ("w_q", "w_k", "w_v", "w_o", "conv_q", "conv_k"):
            grads["d" + n] = torch.empty(w[n].shape, dtype=torch.float32, device=x.device)
        ws = self.workspace(CCA_OP_BACKWARD, B, S, x.device)
        cca_backward(self.handle, w, x, dy, saved, B, S, grads, ws, stream)
        return grads
