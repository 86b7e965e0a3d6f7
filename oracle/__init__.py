"""CPU oracle for OUT_PROD (double precision) and the parity checker.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library and
its Python binding never import it; the two implementations share no code.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over output columns,
double accumulation in ascending k, its own decoders of every a type).
This module compiles it with gcc on first use, loads it with ctypes and adds
the element-wise gate that a GPU result must pass:

* no NaN or Inf anywhere;
* ``|gpu - ref| <= tol * den`` per element, with ``den = sum_k |a||b|``
  (``den == 0`` therefore demands ``gpu == 0``), ``tol = 1e-5``.

Pages: "metal: OUT_PROD runs batched, broadcast and narrow shapes on the GPU"
(review "VERIFIED BY READING": dst shape, divisibility contract, the CPU
backend's slice rule i02 = i2/dps2) and "metal: OUT_PROD multiplies in float
staging" (body: half staging turned gradients past 65504 into Inf and NaN and
left ~1e-3 relative error; the tolerance here is far below that).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

# GGUF type ids of the a (src0) types the oracle decodes
F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0 = 0, 1, 2, 3, 6, 7, 8
Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16 = 10, 11, 12, 13, 14, 30
BLOCK_VALUES = {F32: 1, F16: 1, BF16: 1, Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32,
                Q2_K: 256, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {F32: 4, F16: 2, BF16: 2, Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34,
               Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_I64P = ctypes.POINTER(ctypes.c_int64)
_DBLP = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-std=c99", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_out_prod.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                            _I64P, _I64P, _I64P, ctypes.c_int64, _DBLP, _DBLP]
            lib.oracle_out_prod.restype = ctypes.c_int
            lib.oracle_dequant_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
            lib.oracle_dequant_rows.restype = ctypes.c_int
            lib.oracle_mul_mat_id_back.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                   ctypes.c_void_p, _I64P, _I64P, _I64P,
                                                   ctypes.c_int64, _DBLP, _DBLP]
            lib.oracle_mul_mat_id_back.restype = ctypes.c_int
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def _i64(arr) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(arr, dtype=np.int64))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def dequant_rows(a: np.ndarray, a_type: int, ne00: int, nrows: int, row_stride: int) -> np.ndarray:
    """Decode ``nrows`` rows of ``ne00`` values (row r at byte r*row_stride) to float32."""
    buf = np.ascontiguousarray(a)
    out = np.empty((nrows, ne00), dtype=np.float32)
    rc = _load().oracle_dequant_rows(buf.ctypes.data, a_type, ne00, nrows, row_stride,
                                     out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_dequant_rows failed: %d" % rc)
    return out


def out_prod(a: np.ndarray, a_type: int, b: np.ndarray, ne, nb, cols=None):
    """Reference OUT_PROD.  ``a``/``b`` are host buffers addressed by ``nb`` (bytes)
    from their first byte.  Returns ``(ref, den)`` as float64.

    With ``cols=None`` the arrays have shape ``(ne13, ne12, ne10, ne00)`` (dst
    order).  Otherwise ``cols`` is an (n, 3) array of (i1, i2, i3) and the
    arrays have shape ``(n, ne00)``.
    """
    ne = _i64(ne)
    nb = _i64(nb)
    ne00, ne10, ne12, ne13 = (int(x) for x in (ne[0], ne[4], ne[6], ne[7]))
    if cols is None:
        n = ne10 * ne12 * ne13
        shape = (ne13, ne12, ne10, ne00)
        cols_arr = None
    else:
        cols_arr = _i64(cols).reshape(-1, 3)
        n = cols_arr.shape[0]
        shape = (n, ne00)
    ref = np.zeros(n * ne00, dtype=np.float64)
    den = np.zeros(n * ne00, dtype=np.float64)
    a_c = np.ascontiguousarray(a) if a is not None else None
    b_c = np.ascontiguousarray(b) if b is not None else None
    rc = _load().oracle_out_prod(
        a_c.ctypes.data if a_c is not None and a_c.size else None, a_type,
        b_c.ctypes.data if b_c is not None and b_c.size else None,
        ne.ctypes.data_as(_I64P), nb.ctypes.data_as(_I64P),
        cols_arr.ctypes.data_as(_I64P) if cols_arr is not None else None, n,
        ref.ctypes.data_as(_DBLP), den.ctypes.data_as(_DBLP))
    if rc != 0:
        raise ValueError("oracle_out_prod failed: %d" % rc)
    return ref.reshape(shape), den.reshape(shape)


def mul_mat_id_back(as_: np.ndarray, as_type: int, g: np.ndarray, ids: np.ndarray, ne, nb,
                    slots=None):
    """Reference MUL_MAT_ID_BACK (the input gradient of MUL_MAT_ID through frozen
    experts): for slot s = i + n_used*t, row c of the result is
    sum_r expert[ids[i,t]](c, r) * g(r, i, t).  ``ne``/``nb`` (16 each) describe
    as, g, ids and dst (see oracle.c).  Returns ``(ref, den)`` as float64 of
    shape ``(n_tokens, n_used, ne00)``, or ``(len(slots), ne00)``."""
    ne = _i64(ne)
    nb = _i64(nb)
    ne00, n_used, n_tokens = int(ne[0]), int(ne[5]), int(ne[6])
    if slots is None:
        n = n_used * n_tokens
        shape = (n_tokens, n_used, ne00)
        sl = None
    else:
        sl = _i64(slots).reshape(-1)
        n = sl.size
        shape = (n, ne00)
    ref = np.zeros(max(1, n * ne00), dtype=np.float64)
    den = np.zeros(max(1, n * ne00), dtype=np.float64)
    a_c = np.ascontiguousarray(as_) if as_ is not None else None
    g_c = np.ascontiguousarray(g) if g is not None else None
    i_c = np.ascontiguousarray(ids) if ids is not None else None
    rc = _load().oracle_mul_mat_id_back(
        a_c.ctypes.data if a_c is not None and a_c.size else None, as_type,
        g_c.ctypes.data if g_c is not None and g_c.size else None,
        i_c.ctypes.data if i_c is not None and i_c.size else None,
        ne.ctypes.data_as(_I64P), nb.ctypes.data_as(_I64P),
        sl.ctypes.data_as(_I64P) if sl is not None else None, n,
        ref.ctypes.data_as(_DBLP), den.ctypes.data_as(_DBLP))
    if rc != 0:
        raise ValueError("oracle_mul_mat_id_back failed: %d" % rc)
    return ref[: n * ne00].reshape(shape), den[: n * ne00].reshape(shape)


def check(gpu, ref, den, tol: float = 1e-5) -> dict:
    """The parity gate.  Returns a summary; ``ok`` is True only if every element passes."""
    g = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    if g.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, ref.shape))
    finite = np.isfinite(g)
    n_nonfinite = int(g.size - np.count_nonzero(finite))
    err = np.abs(np.where(finite, g, 0.0) - ref)
    bad = (err > tol * den) | ~finite
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    return {
        "ok": bool(not bad.any()),
        "n_bad": int(np.count_nonzero(bad)),
        "n_nonfinite": n_nonfinite,
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "size": int(g.size),
    }
