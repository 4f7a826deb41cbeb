"""Loader for the oracle's C part (oracle/csrc/*.c -> oracle/liboracle.so). TEST INFRASTRUCTURE ONLY.

Built by __graft_entry__.build(); compiled here on first use if missing or older than its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "csrc", "pool.c")]
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]

_lib = None


def build() -> str:
    # a private temporary name per process: parallel test workers may all build at once
    tmp = f"{LIB}.tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, *SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        stale = not os.path.exists(LIB) or any(os.path.getmtime(s) > os.path.getmtime(LIB) for s in SRC)
        if stale:
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.oracle_pool.restype = None
        L.oracle_pool.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int32, P, P]
        _lib = L
    return _lib


def pool(cK: np.ndarray, cV: np.ndarray, W: np.ndarray, f: int, bf16: bool):
    cK = np.ascontiguousarray(cK, dtype=np.float32)
    cV = np.ascontiguousarray(cV, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    g, _, d = cK.shape
    assert d <= 256 and W.shape == (d, d)
    NK = np.empty((g, d), np.float32)
    NV = np.empty((g, d), np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    lib().oracle_pool(g, f, d, p(cK), p(cV), p(W), 1 if bf16 else 0, p(NK), p(NV))
    return NK, NV
