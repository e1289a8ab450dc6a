"""Build and call the oracle's plain C contraction -- test infrastructure.

``contract.c`` holds the triple loop of the DeepGEMM page's golden
reference (section 3.2) in float64.  It is compiled with gcc into
``oracle/liboracle_contract.so`` (no vectorising or contracting flags beyond
-O2 and -ffp-contract=off) the first time it is needed, or by ``build()``;
it shares no code, header or build step with the GPU library.

Thread count: ``TGEMM_ORACLE_THREADS`` when set, else the CPUs this process
may run on, at most 16.  Rows are split between threads and each row is
computed by one thread, so results do not depend on the count.
"""

import ctypes
import os
import shutil
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "contract.c")
LIB = os.path.join(HERE, "liboracle_contract.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-std=c99"]

_lock = threading.Lock()
_lib = None


def build():
    """Compile contract.c (always) and return the library path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found to build the oracle's contraction")
    tmp = LIB + f".tmp{os.getpid()}"
    res = subprocess.run([cc] + CFLAGS + [SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        stale = (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC)
        if stale:
            build()
        lib = ctypes.CDLL(LIB)
        f = lib.oracle_contract_f64
        f.restype = ctypes.c_int
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        f.argtypes = [P, i64, P, i64, P, P, i64, i64, i64, i64, ctypes.c_int]
        _lib = lib
        return lib


def default_threads():
    env = os.environ.get("TGEMM_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _row_major(x):
    """x itself when its rows are unit-stride with a row stride >= its width
    (in whole elements), else a contiguous copy."""
    rows, cols = x.shape
    ok = (cols <= 1 or x.strides[1] == 8) and (rows <= 1 or (x.strides[0] % 8 == 0 and x.strides[0] >= 8 * cols))
    return x if ok else np.ascontiguousarray(x)


def contract(a, b, threads=None):
    """(y, d) = (a @ b, |a| @ |b|) by the plain k-ascending loop in float64.

    a: float64 [M, K]; b: float64 [K, N] (any row strides, unit inner
    stride; other layouts are copied first).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shape mismatch: a{a.shape} b{b.shape}")
    a = _row_major(a)
    b = _row_major(b)
    M, K = a.shape
    N = b.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    d = np.empty((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return y, d
    if K == 0:
        y.fill(0.0)
        d.fill(0.0)
        return y, d
    lda = a.strides[0] // 8 if M > 1 else K
    ldb = b.strides[0] // 8 if K > 1 else N
    lib = _load()
    rc = lib.oracle_contract_f64(a.ctypes.data, lda, b.ctypes.data, ldb, y.ctypes.data, d.ctypes.data,
                                 N, M, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_contract_f64 rejected its arguments")
    return y, d
