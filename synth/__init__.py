"""Seeded synthetic decode-attention inputs (grid 2D-rotary + N(0, 0.1) noise).

The generator itself is ``synth.c`` (its header states the recipe).  This module
builds it with gcc, wraps it with ctypes and names the workloads.  It is shared
by the oracle's tests, the GPU tests and the benchmark, and holds none of the
attention method's arithmetic.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "_libsynth.so")

Q, K, V, KP, VP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
# A workload whose KV cache is MXFP8: its inputs are generated in bf16 (the
# quantisation belongs to the cache, not to the inputs).
MXFP8 = 2


def build() -> str:
    """Compile synth.c into _libsynth.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_uint64] + [ctypes.c_int] * 10 + [ctypes.c_longlong] * 3 + [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n:
        return max(1, int(n))
    return max(1, min(16, os.cpu_count() or 1))


def fill(seed, stream, layer, d, grid_w, b0, nb, h0, nh, tok0, ntok, shape, strides, dtype, threads=None,
         out=None):
    """Generate into ``out`` (or a new array) of ``shape`` with element ``strides`` (tok, b, h).

    ``out`` must be C-contiguous with that shape and the dtype's element type
    (float32 for F32, uint16 bit patterns for BF16); reusing one buffer avoids
    paying first-touch page faults on every call.
    """
    want = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(shape, dtype=want)
    elif out.dtype != want or tuple(out.shape) != tuple(shape) or not out.flags.c_contiguous:
        raise ValueError("out must be a C-contiguous %s array of shape %s" % (np.dtype(want).name, shape))
    rc = _load().synth_fill(ctypes.c_uint64(seed), stream, layer, d, grid_w, b0, nb, h0, nh, tok0, ntok,
                            strides[0], strides[1], strides[2], dtype,
                            out.ctypes.data_as(ctypes.c_void_p), threads or default_threads())
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


@dataclass(frozen=True)
class Workload:
    """One decode-attention workload: model shape plus (N_r, N_att, sink)."""
    name: str
    batch: int
    layers: int
    heads: int
    head_dim: int
    L_p: int
    L_dec: int
    N_r: int
    N_att: int
    sink: int = 0
    dtype: int = BF16
    seed: int = 0

    @property
    def grid_w(self) -> int:
        return max(1, int(round(math.sqrt(self.L_dec))))

    @property
    def lanes(self) -> int:
        return self.batch * self.heads

    @property
    def input_dtype(self) -> int:
        """dtype of the generated q, k, v (MXFP8 caches take bf16 inputs)."""
        return BF16 if self.dtype == MXFP8 else self.dtype

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # ---- generation in the layouts the library takes ----
    def decode(self, layer, stream, tok0=0, ntok=None, threads=None, out=None):
        """Q, K or V of decode tokens, step-major ``[ntok][B][H][d]``."""
        ntok = self.L_dec - tok0 if ntok is None else ntok
        B, H, d = self.batch, self.heads, self.head_dim
        return fill(self.seed, stream, layer, d, self.grid_w, 0, B, 0, H, tok0, ntok,
                    (ntok, B, H, d), (B * H * d, H * d, d), self.input_dtype, threads, out)

    def prompt(self, layer, stream, threads=None, out=None):
        """Prompt K or V in the model layout ``[B][L_p][H][d]``."""
        B, H, d, L = self.batch, self.heads, self.head_dim, self.L_p
        return fill(self.seed, stream, layer, d, self.grid_w, 0, B, 0, H, 0, L,
                    (B, L, H, d), (H * d, L * H * d, d), self.input_dtype, threads, out)

    def lane(self, layer, b, h, stream, tok0=0, ntok=None, threads=None):
        """One (layer, batch, head) lane, ``[ntok][d]``; prompt streams give all L_p tokens."""
        if stream in (KP, VP):
            tok0, ntok = 0, self.L_p
        ntok = self.L_dec - tok0 if ntok is None else ntok
        d = self.head_dim
        return fill(self.seed, stream, layer, d, self.grid_w, b, 1, h, 1, tok0, ntok,
                    (ntok, d), (d, 0, 0), self.input_dtype, threads)


def n_att_for(L_dec: int, sparsity: float) -> int:
    """N_att from a sparsity ratio 1 - N_att / L_dec, rounded to nearest."""
    return int(math.floor(L_dec * (1.0 - sparsity) + 0.5))


# The five workloads: shapes from the pages' models (Table 1 token counts) with
# N_r = L_dec / 2 and N_att from the sparsity ratio.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", batch=1, layers=1, heads=4, head_dim=64, L_p=16, L_dec=64,
                          N_r=32, N_att=8, sink=0, dtype=F32),
    "janus_pro_1b": Workload("janus_pro_1b", batch=32, layers=24, heads=16, head_dim=128, L_p=64, L_dec=576,
                             N_r=288, N_att=58),
    "janus_pro_7b": Workload("janus_pro_7b", batch=96, layers=30, heads=32, head_dim=128, L_p=64, L_dec=576,
                             N_r=288, N_att=29),
    "lumina_mgpt_7b_1024": Workload("lumina_mgpt_7b_1024", batch=16, layers=32, heads=32, head_dim=128, L_p=96,
                                    L_dec=4096, N_r=2048, N_att=205),
    "hires_8100_sink4": Workload("hires_8100_sink4", batch=8, layers=32, heads=32, head_dim=128, L_p=96,
                                 L_dec=8100, N_r=4050, N_att=810, sink=4),
}
