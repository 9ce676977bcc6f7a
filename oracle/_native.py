"""TEST INFRASTRUCTURE ONLY: builds and loads the fp64 C reference (attention_ref.c).

The shared object is compiled with the host C compiler (gcc, -O2, OpenMP, no fast-math,
so every sum runs in plain loop order).  It is rebuilt when the source is newer.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_ref.c")
# ORACLE_ATTENTION_LIB loads another build of the same source instead (the sanitizer
# test builds one with AddressSanitizer / UndefinedBehaviorSanitizer)
_LIB_OVERRIDE = os.environ.get("ORACLE_ATTENTION_LIB")
_LIB = os.path.join(_HERE, "liboracle_attention.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile attention_ref.c into liboracle_attention.so next to it; return the path."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                h = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                build()
                h = ctypes.CDLL(_LIB)
            h.oracle_attention_rows.restype = ctypes.c_int
            h.oracle_attention_rows.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            h.oracle_max_threads.restype = ctypes.c_int
            h.oracle_max_threads.argtypes = []
            _lib = h
    return _lib


def default_threads() -> int:
    """Host threads available to this process (affinity mask), capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)
