"""CPU oracle for diagonal-aware sparse decode attention and its baselines (fp64).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library.  The algorithms live in C: ``dsa_oracle.c`` (Algorithm 1 of
"Understanding and Exploiting Diagonal Attention Sparsity in Autoregressive
Image Generation", Section 4, and the dense step) and ``baselines_oracle.c``
(SlidingWindow, StreamingLLM, TOVA and H2O as Sections 2.3 and 5.1 describe
them); this module compiles them with gcc and marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_baselines.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, n) for n in ("dsa_oracle.c", "baselines_oracle.c", "mxfp8_oracle.c")]
_LIB = os.path.join(_HERE, "_liboracle.so")

_P = ctypes.c_void_p


def build() -> str:
    """Compile the oracle's C files into _liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp] + _SRCS + ["-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(f) for f in _SRCS):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_dsa_lane.restype = ctypes.c_int
        lib.oracle_dsa_lane.argtypes = [ctypes.c_int] * 6 + [_P] * 13
        lib.oracle_dense_lane.restype = ctypes.c_int
        lib.oracle_dense_lane.argtypes = [ctypes.c_int] * 3 + [_P] * 6
        lib.oracle_window_lane.restype = ctypes.c_int
        lib.oracle_window_lane.argtypes = [ctypes.c_int] * 5 + [_P] * 8
        lib.oracle_score_lane.restype = ctypes.c_int
        lib.oracle_score_lane.argtypes = [ctypes.c_int] * 6 + [_P] * 12
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_mxfp8_quantize.restype = ctypes.c_int
        lib.oracle_mxfp8_quantize.argtypes = [_P, ctypes.c_int, _P, _P]
        lib.oracle_mxfp8_dequantize.restype = ctypes.c_int
        lib.oracle_mxfp8_dequantize.argtypes = [_P, _P, ctypes.c_int, _P]
        _lib = lib
    return _lib


def widen(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp64 copy of generator output: uint16 bf16 bit patterns (dtype 1) or float32 (dtype 0)."""
    if dtype == 1:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _f64(a, shape):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.shape != shape:
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a


def run_lane(L_p, N_r, N_att, sink, q, kp, vp, k, v, follow=None, masks=False, gaps=False):
    """Algorithm 1 on one lane for T = len(q) decode steps.

    q, k, v: [T][d] (k, v indexed by decode position); kp, vp: [L_p][d]; all fp64.
    follow: optional int array [T]: at selection steps append follow[t] to the
    skip set instead of the oracle's own argmin (it must be a candidate).
    Returns a dict with out [T][d], choice [T], evicted [T], n_dec [T] and,
    on request, gap [T], att_mask [T][T] and skip_mask [T][T].
    """
    T, d = np.shape(q)
    q = _f64(q, (T, d))
    k = _f64(k, (T, d))
    v = _f64(v, (T, d))
    kp = _f64(kp, (L_p, d))
    vp = _f64(vp, (L_p, d))
    out = np.empty((T, d), np.float64)
    choice = np.empty(T, np.int32)
    evicted = np.empty(T, np.int32)
    n_dec = np.empty(T, np.int32)
    fol = None if follow is None else np.ascontiguousarray(follow, dtype=np.int32)
    gap = np.zeros(T, np.float64) if (gaps or follow is not None) else None
    att = np.zeros((T, T), np.uint8) if masks else None
    skp = np.zeros((T, T), np.uint8) if masks else None
    rc = _load().oracle_dsa_lane(L_p, N_r, N_att, sink, d, T, _ptr(q), _ptr(kp), _ptr(vp), _ptr(k), _ptr(v),
                                 _ptr(fol), _ptr(out), _ptr(choice), _ptr(evicted), _ptr(n_dec), _ptr(gap),
                                 _ptr(att), _ptr(skp))
    if rc == -2:
        raise ValueError("follow names a position that is not a candidate")
    if rc != 0:
        raise ValueError("oracle_dsa_lane failed (%d)" % rc)
    res = {"out": out, "choice": choice, "evicted": evicted, "n_dec": n_dec}
    if gap is not None:
        res["gap"] = gap
    if masks:
        res["att_mask"] = att.astype(bool)
        res["skip_mask"] = skp.astype(bool)
    return res


def run_dense_lane(L_p, q, kp, vp, k, v):
    """Dense decode attention: step t attends all prompt rows and decode positions 0..t."""
    T, d = np.shape(q)
    q = _f64(q, (T, d))
    k = _f64(k, (T, d))
    v = _f64(v, (T, d))
    kp = _f64(kp, (L_p, d))
    vp = _f64(vp, (L_p, d))
    out = np.empty((T, d), np.float64)
    rc = _load().oracle_dense_lane(L_p, d, T, _ptr(q), _ptr(kp), _ptr(vp), _ptr(k), _ptr(v), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dense_lane failed (%d)" % rc)
    return out


def run_window_lane(L_p, N_att, sink, q, kp, vp, k, v, masks=False):
    """SlidingWindow (sink 0) or StreamingLLM (sink 4) on one lane for T = len(q) steps.

    Returns out [T][d], n_dec [T] and, on request, att_mask [T][T].
    """
    T, d = np.shape(q)
    q, k, v = _f64(q, (T, d)), _f64(k, (T, d)), _f64(v, (T, d))
    kp, vp = _f64(kp, (L_p, d)), _f64(vp, (L_p, d))
    out = np.empty((T, d), np.float64)
    n_dec = np.empty(T, np.int32)
    att = np.zeros((T, T), np.uint8) if masks else None
    rc = _load().oracle_window_lane(L_p, N_att, sink, d, T, _ptr(q), _ptr(kp), _ptr(vp), _ptr(k), _ptr(v),
                                    _ptr(out), _ptr(n_dec), _ptr(att))
    if rc != 0:
        raise ValueError("oracle_window_lane failed (%d)" % rc)
    res = {"out": out, "n_dec": n_dec}
    if masks:
        res["att_mask"] = att.astype(bool)
    return res


TOVA, H2O = 0, 1


def run_score_lane(policy, L_p, N_att, q, kp, vp, k, v, N_recent=0, follow=None, masks=False, scores=False):
    """TOVA (policy 0) or H2O (policy 1, N_recent protected recent positions) on one lane.

    follow: optional int array [T]: at eviction steps the entry that leaves is
    follow[t] instead of the oracle's own choice (it must be a candidate).
    Returns out [T][d], choice [T] (position the step's own rule evicts, -1 if
    none), n_dec [T], gap [T] (with follow) and, on request, att_mask [T][T]
    and score [T][T] (H2O accumulated scores after each step).
    """
    T, d = np.shape(q)
    q, k, v = _f64(q, (T, d)), _f64(k, (T, d)), _f64(v, (T, d))
    kp, vp = _f64(kp, (L_p, d)), _f64(vp, (L_p, d))
    out = np.empty((T, d), np.float64)
    choice = np.empty(T, np.int32)
    n_dec = np.empty(T, np.int32)
    fol = None if follow is None else np.ascontiguousarray(follow, dtype=np.int32)
    gap = np.zeros(T, np.float64) if follow is not None else None
    att = np.zeros((T, T), np.uint8) if masks else None
    sc = np.zeros((T, T), np.float64) if scores else None
    rc = _load().oracle_score_lane(policy, L_p, N_att, N_recent, d, T, _ptr(q), _ptr(kp), _ptr(vp), _ptr(k),
                                   _ptr(v), _ptr(fol), _ptr(out), _ptr(choice), _ptr(n_dec), _ptr(gap), _ptr(att),
                                   _ptr(sc))
    if rc == -2:
        raise ValueError("follow names a position that is not a candidate")
    if rc != 0:
        raise ValueError("oracle_score_lane failed (%d)" % rc)
    res = {"out": out, "choice": choice, "n_dec": n_dec}
    if gap is not None:
        res["gap"] = gap
    if masks:
        res["att_mask"] = att.astype(bool)
    if scores:
        res["score"] = sc
    return res


def e4m3_value(code):
    """Value of an OCP E4M3 code (NaN for the two NaN codes)."""
    return float(_load().oracle_e4m3_value(int(code)))


def quantize_mxfp8(x):
    """MXFP8 E4M3 quantisation of the last axis (a multiple of 32) of x.

    Returns (codes uint8, same shape as x; scales uint8, shape [..., n / 32])."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if x.shape[-1] % 32:
        raise ValueError("last axis must be a multiple of 32")
    nb = x.size // 32
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), np.uint8)
    _load().oracle_mxfp8_quantize(_ptr(x), nb, _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_mxfp8(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if scales.size * 32 != codes.size:
        raise ValueError("one scale per 32 codes")
    out = np.empty(codes.shape, np.float64)
    _load().oracle_mxfp8_dequantize(_ptr(codes), _ptr(scales), scales.size, _ptr(out))
    return out


def mxfp8_roundtrip(x):
    """The values an MXFP8 cache holds for x (rows along the last axis)."""
    return dequantize_mxfp8(*quantize_mxfp8(x))


def lane_inputs(workload, layer, b, h, T=None):
    """fp64 inputs of one lane from the shared seeded generator: (q, kp, vp, k, v).

    For a workload with an MXFP8 cache the K / V rows come back as the cache
    holds them (quantised and dequantised); q stays bf16."""
    import synth

    T = workload.L_dec if T is None else T
    dt = workload.input_dtype
    q = widen(workload.lane(layer, b, h, synth.Q, 0, T), dt)
    k = widen(workload.lane(layer, b, h, synth.K, 0, T), dt)
    v = widen(workload.lane(layer, b, h, synth.V, 0, T), dt)
    kp = widen(workload.lane(layer, b, h, synth.KP), dt)
    vp = widen(workload.lane(layer, b, h, synth.VP), dt)
    if workload.dtype == synth.MXFP8:
        # an MXFP8 cache holds every K / V row (prompt and decode) quantised
        k, v, kp, vp = (mxfp8_roundtrip(x) if x.size else x for x in (k, v, kp, vp))
    return q, kp, vp, k, v
