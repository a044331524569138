"""ctypes binding of libdsa.so: same names and argument order as include/dsa.h.

Pointer arguments take a device address (int), any object with
``data_ptr()`` (a torch tensor), or None for NULL.  Streams take a
``hipStream_t`` address (``torch.cuda.current_stream().cuda_stream``), an
object with ``cuda_stream``, or None for the null stream.  A negative status
raises DsaError with the library's message.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _build

DSA_F32, DSA_BF16, DSA_MXFP8 = 0, 1, 2
(DSA_POLICY_DIAGONAL, DSA_POLICY_DIAGONAL_SINK4, DSA_POLICY_SLIDING_WINDOW, DSA_POLICY_STREAMING_LLM, DSA_POLICY_TOVA,
 DSA_POLICY_H2O) = range(6)

_c_int, _c_size, _P = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGNATURES = {
    "dsa_state_workspace_bytes": (_c_size, [_c_int] * 8),
    "dsa_state_init": (_c_int, [ctypes.POINTER(_P)] + [_c_int] * 8 + [_P, _c_size, _P]),
    "dsa_policy_workspace_bytes": (_c_size, [_c_int] * 8),
    "dsa_policy_state_init": (_c_int, [ctypes.POINTER(_P)] + [_c_int] * 8 + [_P, _c_size, _P]),
    "dsa_set_stream": (_c_int, [_P, _P]),
    "dsa_append_prompt": (_c_int, [_P, _P, _P]),
    "dsa_append_kv": (_c_int, [_P, _P, _P]),
    "dsa_decode_step": (_c_int, [_P, _P, _P, _P]),
    "dsa_append_decode_step": (_c_int, [_P, _P, _P, _P, _P, _P]),
    "dsa_read_state": (_c_int, [_P, _P, _P, _P]),
    "dense_state_workspace_bytes": (_c_size, [_c_int] * 6),
    "dense_state_init": (_c_int, [ctypes.POINTER(_P)] + [_c_int] * 6 + [_P, _c_size, _P]),
    "dense_append_prompt": (_c_int, [_P, _P, _P]),
    "dense_append_kv": (_c_int, [_P, _P, _P]),
    "dense_decode_step": (_c_int, [_P, _P, _P]),
    "dense_append_decode_step": (_c_int, [_P, _P, _P, _P, _P]),
    "dsa_profile_workspace_bytes": (_c_size, [_c_int] * 5),
    "dsa_attention_profile": (_c_int, [_P, _P, _P] + [_c_int] * 7 + [_P, _c_size, _P, _P, _P, _P]),
    "dsa_attention_profile_static": (_c_int, [_P, _P, _P] + [_c_int] * 7 + [_P, _P, _P, _P]),
    "dsa_hbm_read_probe": (_c_int, [_P, _c_size, _c_int, _c_int, _c_int, _P, _P]),
    "dsa_set_waves": (_c_int, [_P, _c_int]),
    "dsa_set_splits": (_c_int, [_P, _c_int]),
    "dsa_state_step": (_c_int, [_P]),
    "dsa_state_destroy": (_c_int, [_P]),
    "dsa_strerror": (ctypes.c_char_p, [_c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
}

_lib = None


def library_path() -> str:
    return _build.LIB


def library():
    """Load libdsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError("libdsa.so is not built: run python -m autoregressive_image_generation_amd._build")
        lib = ctypes.CDLL(_build.LIB)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    """Names of the C ABI entry points the binding expects the library to export."""
    return list(_SIGNATURES)


class DsaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("%s (%s)" % (message, dsa_strerror(code)))
        self.code = code
        self.message = message


def _check(rc: int) -> int:
    if rc < 0:
        raise DsaError(rc, dsa_last_error())
    return rc


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


class State:
    """Host handle of a sparse or dense state plus the sizes the binding needs."""

    def __init__(self, handle, kind, lanes, list_len, workspace):
        self.handle = handle
        self.kind = kind
        self.lanes = lanes
        self.list_len = list_len
        self.workspace = workspace  # kept alive with the handle

    @property
    def _as_parameter_(self):
        if self.handle is None:
            raise DsaError(-1, "state already destroyed")
        return self.handle

    def __del__(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.dsa_state_destroy(self.handle)
            self.handle = None


def dsa_strerror(code: int) -> str:
    return library().dsa_strerror(code).decode()


def dsa_last_error() -> str:
    return library().dsa_last_error().decode()


def dsa_state_workspace_bytes(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype) -> int:
    return int(library().dsa_state_workspace_bytes(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype))


def dsa_state_init(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype, workspace, workspace_bytes, stream=None):
    h = _P()
    _check(library().dsa_state_init(ctypes.byref(h), batch, L_p, N_r, N_att, heads, head_dim, sink, dtype,
                                    _ptr(workspace), workspace_bytes, _stream(stream)))
    return State(h, "sparse", batch * heads, N_att - sink, workspace)


def dsa_policy_workspace_bytes(policy, batch, L_p, N_r, N_att, heads, head_dim, dtype) -> int:
    return int(library().dsa_policy_workspace_bytes(policy, batch, L_p, N_r, N_att, heads, head_dim, dtype))


def dsa_policy_state_init(policy, batch, L_p, N_r, N_att, heads, head_dim, dtype, workspace, workspace_bytes,
                          stream=None):
    h = _P()
    _check(library().dsa_policy_state_init(ctypes.byref(h), policy, batch, L_p, N_r, N_att, heads, head_dim, dtype,
                                           _ptr(workspace), workspace_bytes, _stream(stream)))
    sink = 4 if policy in (DSA_POLICY_DIAGONAL_SINK4, DSA_POLICY_STREAMING_LLM) else 0
    return State(h, "sparse", batch * heads, N_att - sink, workspace)


def dsa_set_stream(st, stream):
    return _check(library().dsa_set_stream(st, _stream(stream)))


def dsa_append_prompt(st, k_p, v_p):
    return _check(library().dsa_append_prompt(st, _ptr(k_p), _ptr(v_p)))


def dsa_append_kv(st, k_t, v_t):
    return _check(library().dsa_append_kv(st, _ptr(k_t), _ptr(v_t)))


def dsa_decode_step(st, q_t, out, trace=None):
    return _check(library().dsa_decode_step(st, _ptr(q_t), _ptr(out), _ptr(trace)))


def dsa_append_decode_step(st, k_t, v_t, q_t, out, trace=None):
    return _check(library().dsa_append_decode_step(st, _ptr(k_t), _ptr(v_t), _ptr(q_t), _ptr(out), _ptr(trace)))


def dsa_read_state(st):
    """Returns (t, offsets [lanes][N_att - sink] int16 padded with -1, counts [lanes] int32).

    TOVA / H2O states list N_att offsets (sink 0)."""
    t = ctypes.c_int32()
    offs = np.empty((st.lanes, st.list_len), np.int16)
    cnt = np.empty(st.lanes, np.int32)
    _check(library().dsa_read_state(st, ctypes.byref(t), offs.ctypes.data_as(_P), cnt.ctypes.data_as(_P)))
    return int(t.value), offs, cnt


def dense_state_workspace_bytes(batch, L_p, L_max, heads, head_dim, dtype) -> int:
    return int(library().dense_state_workspace_bytes(batch, L_p, L_max, heads, head_dim, dtype))


def dense_state_init(batch, L_p, L_max, heads, head_dim, dtype, workspace, workspace_bytes, stream=None):
    h = _P()
    _check(library().dense_state_init(ctypes.byref(h), batch, L_p, L_max, heads, head_dim, dtype, _ptr(workspace),
                                      workspace_bytes, _stream(stream)))
    return State(h, "dense", batch * heads, 0, workspace)


def dense_append_prompt(st, k_p, v_p):
    return _check(library().dense_append_prompt(st, _ptr(k_p), _ptr(v_p)))


def dense_append_kv(st, k_t, v_t):
    return _check(library().dense_append_kv(st, _ptr(k_t), _ptr(v_t)))


def dense_decode_step(st, q_t, out):
    return _check(library().dense_decode_step(st, _ptr(q_t), _ptr(out)))


def dense_append_decode_step(st, k_t, v_t, q_t, out):
    return _check(library().dense_append_decode_step(st, _ptr(k_t), _ptr(v_t), _ptr(q_t), _ptr(out)))


def dsa_profile_workspace_bytes(batch, heads, L_p, T, max_dist) -> int:
    return int(library().dsa_profile_workspace_bytes(batch, heads, L_p, T, max_dist))


def dsa_attention_profile(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist, workspace, workspace_bytes,
                          mass, vert, diag, stream=None):
    return _check(library().dsa_attention_profile(_ptr(q), _ptr(k), _ptr(k_p), batch, heads, head_dim, L_p, T, dtype,
                                                  max_dist, _ptr(workspace), workspace_bytes, _ptr(mass), _ptr(vert),
                                                  _ptr(diag), _stream(stream)))


DSA_PROFILE_STATIC_SCRATCH_BYTES = 64 << 20


def dsa_attention_profile_static(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist, mass, vert, diag,
                                 stream=None):
    return _check(library().dsa_attention_profile_static(_ptr(q), _ptr(k), _ptr(k_p), batch, heads, head_dim, L_p, T,
                                                         dtype, max_dist, _ptr(mass), _ptr(vert), _ptr(diag),
                                                         _stream(stream)))


def dsa_hbm_read_probe(src, nbytes, blocks, threads, unroll, sink, stream=None):
    return _check(library().dsa_hbm_read_probe(_ptr(src), nbytes, blocks, threads, unroll, _ptr(sink),
                                               _stream(stream)))


def dsa_set_waves(st, waves_per_lane):
    return _check(library().dsa_set_waves(st, waves_per_lane))


def dsa_set_splits(st, splits_per_lane):
    return _check(library().dsa_set_splits(st, splits_per_lane))


def dsa_state_step(st) -> int:
    return _check(library().dsa_state_step(st))


def dsa_state_destroy(st):
    if isinstance(st, State):
        if st.handle is not None:
            library().dsa_state_destroy(st.handle)
            st.handle = None
        return 0
    return library().dsa_state_destroy(st)
