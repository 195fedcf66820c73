"""ctypes binding of liborthros.so (the C ABI in include/orthros.h).

Argument marshalling only: tensors become raw pointers, the stream is
torch's current HIP stream, and a negative status raises OrthrosError with
the library's message.  Every step of the computation runs in the library's
HIP kernels; nothing here computes, and nothing falls back to the CPU.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborthros.so")

F32, BF16 = 0, 1
STATUS = {0: "ORTHROS_OK", -1: "ORTHROS_E_NULL", -2: "ORTHROS_E_SHAPE", -3: "ORTHROS_E_DTYPE",
          -4: "ORTHROS_E_POS", -5: "ORTHROS_E_CAPACITY", -6: "ORTHROS_E_WORKSPACE", -7: "ORTHROS_E_HIP",
          -8: "ORTHROS_E_ALIGN"}


class OrthrosError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Loads liborthros.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run phase_aware_swa_amd/build.py "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(Desc)
        L.orthros_prefill_workspace_size.argtypes = [dp, i64]
        L.orthros_prefill_workspace_size.restype = sz
        L.orthros_decode_workspace_size.argtypes = [dp, i64]
        L.orthros_decode_workspace_size.restype = sz
        L.orthros_prefill.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
        L.orthros_prefill.restype = ctypes.c_int
        L.orthros_swa_prefill.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp]
        L.orthros_swa_prefill.restype = ctypes.c_int
        L.orthros_global_xattn.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
        L.orthros_global_xattn.restype = ctypes.c_int
        L.orthros_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp, vp,
                                          sz, vp]
        L.orthros_decode_step.restype = ctypes.c_int
        L.orthros_decode_step_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, vp,
                                                  vp, vp]
        L.orthros_decode_step_noalloc.restype = ctypes.c_int
        L.orthros_copies.argtypes = [dp, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp]
        L.orthros_copies.restype = ctypes.c_int
        L.orthros_project.argtypes = [dp, i64, i64, i64] + [vp] * 13 + [i64, vp]
        L.orthros_project.restype = ctypes.c_int
        L.orthros_status_str.argtypes = [ctypes.c_int]
        L.orthros_status_str.restype = ctypes.c_char_p
        L.orthros_last_error.argtypes = []
        L.orthros_last_error.restype = ctypes.c_char_p
        L.orthros_abi_version.argtypes = []
        L.orthros_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def make_desc(batch, n_q_heads, n_kv_heads, head_dim, window, dtype, softmax_scale=0.0):
    """dtype: torch.float32 / torch.bfloat16, or the ORTHROS_F32 / ORTHROS_BF16 code."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: F32, torch.bfloat16: BF16}.get(dtype, -1)
    return Desc(batch, n_q_heads, n_kv_heads, head_dim, window, softmax_scale, dtype)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status):
    if status != 0:
        raise OrthrosError(status, lib().orthros_last_error().decode())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def prefill_workspace_size(desc, T):
    return lib().orthros_prefill_workspace_size(ctypes.byref(desc), T)


def decode_workspace_size(desc, max_len):
    return lib().orthros_decode_workspace_size(ctypes.byref(desc), max_len)


def prefill(desc, T, q, q_out, out_pos, k, v, alpha, beta, alpha_out, beta_out, k_cache, v_cache, o, o_out,
            workspace, stream=None):
    """orthros_prefill; out_pos is a sequence of B ints (host)."""
    pos = (ctypes.c_int64 * len(out_pos))(*[int(p) for p in out_pos])
    _check(lib().orthros_prefill(
        ctypes.byref(desc), T, _ptr(q), _ptr(q_out), pos, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(alpha_out), _ptr(beta_out), _ptr(k_cache), _ptr(v_cache), k_cache.shape[2] if k_cache is not None
        else 0, _ptr(o), _ptr(o_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def swa_prefill(desc, T, q, k, v, alpha, beta, k_cache, v_cache, o, stream=None):
    _check(lib().orthros_swa_prefill(
        ctypes.byref(desc), T, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(k_cache),
        _ptr(v_cache), k_cache.shape[2] if k_cache is not None else 0, _ptr(o), _stream(stream)))


def global_xattn(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, o_out, workspace, stream=None):
    pos = (ctypes.c_int64 * len(out_pos))(*[int(p) for p in out_pos])
    _check(lib().orthros_global_xattn(
        ctypes.byref(desc), T, _ptr(q_out), pos, _ptr(alpha_out), _ptr(beta_out), _ptr(k_cache),
        _ptr(v_cache), k_cache.shape[2] if k_cache is not None else 0, _ptr(o_out), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def decode_step(desc, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache, v_cache, cache_len,
                max_len_hint, o, o_out, workspace, stream=None):
    _check(lib().orthros_decode_step(
        ctypes.byref(desc), _ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new), _ptr(alpha), _ptr(beta),
        _ptr(alpha_out), _ptr(beta_out), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[2] if k_cache is not None else 0, _ptr(cache_len), max_len_hint, _ptr(o), _ptr(o_out),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def decode_step_noalloc(desc, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache, v_cache,
                        cache_len, max_len_hint, o, o_out, stream=None):
    """orthros_decode_step_noalloc: the decode step on the library's own scratch (no workspace)."""
    _check(lib().orthros_decode_step_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new), _ptr(alpha), _ptr(beta),
        _ptr(alpha_out), _ptr(beta_out), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[2] if k_cache is not None else 0, _ptr(cache_len), max_len_hint, _ptr(o), _ptr(o_out),
        _stream(stream)))


def copies(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, o_out, stream=None):
    """orthros_copies; q_out / o_out [B, T_out, Hq, d]; out_pos a device int32 tensor [B, T_out]."""
    _check(lib().orthros_copies(
        ctypes.byref(desc), T, q_out.shape[1] if q_out is not None else 0, _ptr(q_out), _ptr(out_pos),
        _ptr(alpha_out), _ptr(beta_out), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[2] if k_cache is not None else 0, _ptr(o_out), _stream(stream)))


def project(desc, T, d_model, x, x_out, w_q, w_k, w_v, alpha, beta, alpha_out, beta_out, q, q_out, k_cache,
            v_cache, stream=None):
    """orthros_project; x [B,T,d_model], x_out [B,T_out,d_model] or None; alpha..beta_out may be None."""
    T_out = x_out.shape[1] if x_out is not None else 0
    _check(lib().orthros_project(
        ctypes.byref(desc), T, T_out, d_model, _ptr(x), _ptr(x_out), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(alpha),
        _ptr(beta), _ptr(alpha_out), _ptr(beta_out), _ptr(q), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[2] if k_cache is not None else 0, _stream(stream)))


def abi_version():
    return lib().orthros_abi_version()


def status_str(status):
    return lib().orthros_status_str(status).decode()
