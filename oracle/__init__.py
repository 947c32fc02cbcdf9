"""TEST INFRASTRUCTURE ONLY -- the CPU oracle of the chunked GDP forward.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import, call or load anything in this package.  The product path (the HIP
library and its Python binding) never does.

Contents
* ``gdp_oracle.c`` (built to ``libgdp_oracle.so`` with gcc): the fp64 serial
  recurrence over the Householder-expanded stream and the per-chunk WY factors
  by forward substitution.  See the header of that file for the definitions and
  their sources.
* ``prepare.py``: the prefill prepare step in numpy with float32-per-op gates.

The C library is built by :func:`build` (called by the package build entry
point); :func:`lib` loads what is built and builds only if nothing is.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import prepare  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gdp_oracle.c")
LIB_PATH = os.path.join(_HERE, "libgdp_oracle.so")

_lib = None


def build():
    """Compile the C oracle with the host gcc (IEEE semantics, no contraction)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-o", tmp, SRC, "-lm",
    ])
    os.replace(tmp, LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        L.gdp_oracle_recurrence.restype = i32
        L.gdp_oracle_recurrence.argtypes = [
            i64, i32, i32, i32,
            fp, i64, fp, i64, fp, i64, fp, i64, fp, i64,
            dbl, dbl, i32, dp, dp, dp, dp, dp]
        L.gdp_oracle_wy.restype = i32
        L.gdp_oracle_wy.argtypes = [
            i64, i32, i32, i32,
            fp, i64, fp, i64, fp, i64, fp, i64,
            dbl, i32, dp, dp]
        _lib = L
    return _lib


def _f32_rows(a, name, ndim):
    """Return (pointer, row stride in elements) for a float32 view whose last
    dimension is contiguous (ndim 2) or a strided 1-D float32 view (ndim 1)."""
    if a.dtype != np.float32:
        raise TypeError("%s must be float32" % name)
    if a.ndim != ndim:
        raise ValueError("%s must be %d-D" % (name, ndim))
    if ndim == 2 and a.shape[1] > 1 and a.strides[1] != 4:
        raise ValueError("%s: last dimension must be contiguous" % name)
    stride = a.strides[0] // 4 if a.shape[0] > 0 else 0
    if a.strides[0] % 4:
        raise ValueError("%s: misaligned stride" % name)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), stride


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, beta, g, M, scale=None, chunk=64, h0=None, eps=1e-6,
               want_vnew=True, want_h=True):
    """Serial fp64 recurrence for one sequence and one value head.

    q [L, K], k [L*M, K], v [L*M, V]: float32, last dim contiguous (views OK).
    beta [L*M], g [L] (or None for no decay): float32 1-D views.
    Returns dict with o [L, V], v_new [L*M, V], h [ceil(L*M/chunk), V, K],
    h_final [V, K] (float64).
    """
    L, K = q.shape
    V = v.shape[1]
    if k.shape != (L * M, K) or v.shape[0] != L * M or beta.shape != (L * M,):
        raise ValueError("inconsistent shapes")
    if g is not None and g.shape != (L,):
        raise ValueError("g must be [L]")
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    qp, qs = _f32_rows(q, "q", 2)
    kp, ks = _f32_rows(k, "k", 2)
    vp, vs = _f32_rows(v, "v", 2)
    bp, bs = _f32_rows(beta, "beta", 1)
    if g is not None:
        gp, gs = _f32_rows(g, "g", 1)
    else:
        gp, gs = None, 0
    nc = -(-(L * M) // chunk)
    o = np.zeros((L, V), np.float64)
    vn = np.zeros((L * M, V), np.float64) if want_vnew else None
    h = np.zeros((nc, V, K), np.float64) if want_h else None
    hf = np.zeros((V, K), np.float64)
    h0a = None
    if h0 is not None:
        h0a = np.ascontiguousarray(h0, dtype=np.float64)
        if h0a.shape != (V, K):
            raise ValueError("h0 must be [V, K]")
    rc = lib().gdp_oracle_recurrence(
        L, M, K, V, qp, qs, kp, ks, vp, vs, bp, bs, gp, gs,
        float(scale), float(eps), int(chunk), _dptr(h0a),
        _dptr(o), _dptr(vn), _dptr(h), _dptr(hf))
    if rc != 0:
        raise RuntimeError("gdp_oracle_recurrence failed: %d" % rc)
    return {"o": o, "v_new": vn, "h": h, "h_final": hf}


def wy(k, v, beta, g, M, chunk=64, eps=1e-6):
    """Per-chunk WY factors (w [L*M, K], u [L*M, V]) for one sequence/head."""
    LM, K = k.shape
    V = v.shape[1]
    if LM % M:
        raise ValueError("rows must be a multiple of M")
    L = LM // M
    kp, ks = _f32_rows(k, "k", 2)
    vp, vs = _f32_rows(v, "v", 2)
    bp, bs = _f32_rows(beta, "beta", 1)
    if g is not None:
        gp, gs = _f32_rows(g, "g", 1)
    else:
        gp, gs = None, 0
    w = np.zeros((LM, K), np.float64)
    u = np.zeros((LM, V), np.float64)
    rc = lib().gdp_oracle_wy(L, M, K, V, kp, ks, vp, vs, bp, bs, gp, gs,
                             float(eps), int(chunk), _dptr(w), _dptr(u))
    if rc != 0:
        raise RuntimeError("gdp_oracle_wy failed: %d" % rc)
    return w, u
