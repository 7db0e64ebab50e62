"""Loader for the oracle's C integer GEMM (``oracle/gemm_i64.c``).

TEST INFRASTRUCTURE ONLY.  Builds ``oracle/_gemm_i64.so`` with gcc (-O2, OpenMP)
when it is missing or older than its source, then binds it with ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_i64.c")
LIB = os.path.join(HERE, "_gemm_i64.so")

_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        L.oracle_gemm_i64.restype = ctypes.c_int
        L.oracle_gemm_i64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        _lib = L
    return _lib
