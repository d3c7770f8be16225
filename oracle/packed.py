"""ctypes binding of the packed C oracle (mdr_packed.c).

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and the ``cpu_baseline`` leg of
``bench.py``.  The C file computes what ``mdr_oracle`` computes for one (batch,
head) -- summaries, addresses, posting lists, probes, rerank, top-R, and exact
softmax over the selected tokens -- with plain loops and gathers instead of a
dense mask, so that its running time is a meaningful CPU baseline (the pages
time a packed CPU routing implementation: aitechinspire.com write-up,
"Scaling behavior and implementation notes").  Drop policy, no forced target.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mdr_packed.c")
LIB = os.path.join(HERE, "libmdr_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-shared", "-fPIC"]

_lib = None


def build() -> str:
    """Compile mdr_packed.c with gcc into oracle/libmdr_oracle.so."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        fp, ip, dp, i = (ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32),
                         ctypes.POINTER(ctypes.c_double), ctypes.c_int)
        lib.mdr_packed_forward.argtypes = [fp, fp, fp, i, i, fp, fp, i, i, i, i, i, i, i, i, i, i, ip, dp]
        lib.mdr_packed_forward.restype = i
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def packed_forward(q, k, v, codebook, bias, w, t0: int = 0, t1: int | None = None):
    """One (batch, head): q, k, v [S, D]; codebook [G, C, D]; bias [G, C] or None; ``w`` carries the
    sizes (block, capacity, probes, max_cand, remote, local).  Returns (sel [n, R] int64 in rank order,
    -1 beyond the last; out [n, D] float64) for the tokens t0 .. t1 - 1."""
    lib = _load()
    S, D = q.shape
    G, C, _ = codebook.shape
    t1 = S if t1 is None else t1
    n = t1 - t0
    q, k, v, cb = _f32(q), _f32(k), _f32(v), _f32(codebook)
    bs = None if bias is None else _f32(bias)
    sel = np.empty((n, w.remote), dtype=np.int32)
    out = np.empty((n, D), dtype=np.float64)
    P = ctypes.POINTER
    fptr = lambda a: a.ctypes.data_as(P(ctypes.c_float))  # noqa: E731
    rc = lib.mdr_packed_forward(fptr(q), fptr(k), fptr(v), S, D, fptr(cb), None if bs is None else fptr(bs), G, C,
                                w.block, w.capacity, w.probes, w.max_cand, w.remote, w.local, t0, t1,
                                sel.ctypes.data_as(P(ctypes.c_int32)), out.ctypes.data_as(P(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"mdr_packed_forward failed ({rc})")
    return sel.astype(np.int64), out
