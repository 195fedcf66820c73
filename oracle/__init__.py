"""fp64 CPU oracle for the Orthros per-layer attention step.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library and its Python binding never import it, and it imports nothing from
them: the two share no code.

``oracle.c`` holds the loop form of the definition (one query at a time,
fp64); ``brute.py`` holds the dense-matrix form for tiny sizes.  This module
is the ctypes wrapper around ``oracle.c`` plus its build step (plain gcc).

Tensors passed in are contiguous CPU torch tensors in float32 or bfloat16
(the call's storage type).  Outputs are float64 tensors; caches are returned
in the storage type, as byte copies of the inputs.
"""
import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("nthreads", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
    ]


def build(force=True):
    """Compile oracle.c with gcc into oracle/liboracle.so."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        sp = ctypes.POINTER(Shape)
        L.oracle_prefill.argtypes = [sp, i64] + [vp] * 2 + [vp] + [vp] * 8 + [i64, vp, vp]
        L.oracle_prefill.restype = ctypes.c_int
        L.oracle_swa_rows.argtypes = [sp, i64] + [vp] * 5 + [i64, vp, vp]
        L.oracle_swa_rows.restype = ctypes.c_int
        L.oracle_swa_rows_given_q.argtypes = [sp, i64] + [vp] * 5 + [i64, vp, vp]
        L.oracle_swa_rows_given_q.restype = ctypes.c_int
        L.oracle_decode_step.argtypes = [sp] + [vp] * 10 + [i64, vp, vp, vp]
        L.oracle_copies.argtypes = [sp, i64, i64] + [vp] * 6 + [i64, vp]
        L.oracle_copies.restype = ctypes.c_int
        L.oracle_decode_step.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise TypeError(f"oracle takes float32 or bfloat16 storage, got {t.dtype}")


def _p(t):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, window, dtype, softmax_scale=None, nthreads=None):
    return Shape(
        batch, n_q_heads, n_kv_heads, head_dim, window,
        0 if dtype == torch.float32 else 1,
        nthreads or default_threads(),
        softmax_scale if softmax_scale else head_dim ** -0.5,
    )


def prefill(q, q_out, out_pos, k, v, alpha, beta, alpha_out, beta_out, window,
            softmax_scale=None, k_cache=None, v_cache=None, cap=None,
            swa=True, glob=True, nthreads=None):
    """One prefill call.  q [B,T,Hq,d] (may be None when swa is False),
    q_out [B,Hq,d], k/v [B,T,Hkv,d], out_pos: ints [B].

    k_cache / v_cache ([B,Hkv,cap,d], storage dtype) are updated in place
    when given, else created zero-filled.  Returns dict(o, o_out, k_cache,
    v_cache); o / o_out are None when swa / glob is False.
    """
    B, T, Hkv, d = k.shape
    Hq = q_out.shape[1]
    dt = k.dtype
    assert q is not None or not swa, "q is needed for the base stream"
    for t in (q, q_out, k, v, alpha, beta, alpha_out, beta_out):
        assert t is None or t.dtype == dt, "one storage type per call"
    cap = cap or (k_cache.shape[2] if k_cache is not None else T)
    if k_cache is None:
        k_cache = torch.zeros(B, Hkv, cap, d, dtype=dt)
        v_cache = torch.zeros(B, Hkv, cap, d, dtype=dt)
    pos = torch.as_tensor(list(out_pos), dtype=torch.int64)
    o = torch.zeros(B, T, Hq, d, dtype=torch.float64) if swa else None
    o_out = torch.zeros(B, Hq, d, dtype=torch.float64) if glob else None
    s = make_shape(B, Hq, Hkv, d, window, dt, softmax_scale, nthreads)
    rc = lib().oracle_prefill(
        ctypes.byref(s), T, _p(q), _p(q_out), _p(pos), _p(k), _p(v),
        _p(alpha), _p(beta), _p(alpha_out), _p(beta_out),
        _p(k_cache), _p(v_cache), cap, _p(o), _p(o_out))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return dict(o=o, o_out=o_out, k_cache=k_cache, v_cache=v_cache)


def swa_rows(q, k, v, alpha, beta, window, rows, softmax_scale=None, nthreads=None):
    """Eq. (4) at selected rows.  rows: int64 tensor [n, 3] of (b, t, h)."""
    B, T, Hq, d = q.shape
    rows = torch.as_tensor(rows, dtype=torch.int64).contiguous()
    out = torch.zeros(rows.shape[0], d, dtype=torch.float64)
    s = make_shape(B, Hq, k.shape[2], d, window, q.dtype, softmax_scale, nthreads)
    rc = lib().oracle_swa_rows(ctypes.byref(s), T, _p(q), _p(k), _p(v), _p(alpha), _p(beta),
                               rows.shape[0], _p(rows), _p(out))
    if rc != 0:
        raise ValueError("oracle_swa_rows rejected its arguments")
    return out


def swa_rows_given_q(qrows, k, v, alpha, beta, window, rows, n_q_heads, softmax_scale=None, nthreads=None):
    """Eq. (4) at selected rows whose raw queries are given row by row.

    qrows [n, d] (row u is the base-stream query of rows[u] = (b, t, h));
    k, v [B,T,Hkv,d].  Same result as swa_rows on a full q holding those
    rows."""
    B, T, Hkv, d = k.shape
    rows = torch.as_tensor(rows, dtype=torch.int64).contiguous()
    assert qrows.shape == (rows.shape[0], d) and qrows.is_contiguous()
    out = torch.zeros(rows.shape[0], d, dtype=torch.float64)
    s = make_shape(B, n_q_heads, Hkv, d, window, k.dtype, softmax_scale, nthreads)
    rc = lib().oracle_swa_rows_given_q(ctypes.byref(s), T, _p(qrows), _p(k), _p(v), _p(alpha), _p(beta),
                                       rows.shape[0], _p(rows), _p(out))
    if rc != 0:
        raise ValueError("oracle_swa_rows_given_q rejected its arguments")
    return out


def decode_step(q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, window,
                k_cache, v_cache, cache_len, softmax_scale=None, compute=True, nthreads=None):
    """One decode step; updates k_cache, v_cache and cache_len (int32 [B]) in place.

    q, q_out [B,Hq,d]; k_new, v_new [B,Hkv,d].  Returns (o, o_out) as
    float64 [B,Hq,d], or (None, None) when compute is False (append only).
    """
    B, Hq, d = q.shape
    Hkv = k_new.shape[1]
    assert cache_len.dtype == torch.int32 and cache_len.is_contiguous()
    o = torch.zeros(B, Hq, d, dtype=torch.float64) if compute else None
    o_out = torch.zeros(B, Hq, d, dtype=torch.float64) if compute else None
    s = make_shape(B, Hq, Hkv, d, window, q.dtype, softmax_scale, nthreads)
    rc = lib().oracle_decode_step(
        ctypes.byref(s), _p(q), _p(q_out), _p(k_new), _p(v_new),
        _p(alpha), _p(beta), _p(alpha_out), _p(beta_out),
        _p(k_cache), _p(v_cache), k_cache.shape[2], _p(cache_len), _p(o), _p(o_out))
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    return o, o_out


def copies(q_out, pos, alpha_out, beta_out, k_cache, v_cache, T, softmax_scale=None, nthreads=None):
    """Eq. (5) for T_out output copies per sequence (the PT / SFT modes).

    q_out [B,T_out,Hq,d]; pos [B,T_out] original positions (any order,
    0 <= pos < T); k_cache, v_cache [B,Hkv,cap,d] with slots [0, T) filled.
    Returns o_out as float64 [B,T_out,Hq,d].
    """
    B, T_out, Hq, d = q_out.shape
    Hkv = k_cache.shape[1]
    pos = torch.as_tensor(pos, dtype=torch.int32).reshape(B, T_out).contiguous()
    o_out = torch.zeros(B, T_out, Hq, d, dtype=torch.float64)
    s = make_shape(B, Hq, Hkv, d, 1, q_out.dtype, softmax_scale, nthreads)
    rc = lib().oracle_copies(ctypes.byref(s), T, T_out, _p(q_out), _p(pos), _p(alpha_out), _p(beta_out),
                             _p(k_cache), _p(v_cache), k_cache.shape[2], _p(o_out))
    if rc != 0:
        raise ValueError("oracle_copies rejected its arguments")
    return o_out
