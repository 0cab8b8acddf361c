"""ctypes binding of libla.so (include/la.h): argument marshalling only.

Every step of the decoding path runs in the library's HIP kernels; this
module only converts Python / torch arguments to the C-ABI and back.  PyTorch
provides device memory (weights, workspace) and the stream.  If the library
is missing, loading fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libla.so")

LA_OK, LA_DONE = 0, 1
LA_EINVAL, LA_ENOMEM, LA_ECTX, LA_EHIP, LA_ESTATE = -1, -2, -3, -4, -5
LA_F32, LA_BF16 = 0, 1
LA_MAX_N = 16
LA_PROBE_BLOCKS = 256
LA_NOALLOC_SCRATCH_BYTES = 32 << 20
LA_PROMPT_REF, LA_AR, LA_NO_GRAPH, LA_POOL_LRU, LA_POOL_CONTEXT = 1, 2, 8, 16, 32
LA_ADAPTIVE_G, LA_DEBUG_LOGITS = 64, 4

EXPORTS = [
    "la_model_load", "la_model_free", "la_session_bytes", "la_prefill", "la_step",
    "la_pool_stats", "la_debug_logits", "la_session_rows", "la_session_free", "la_last_error",
    "la_kernel_attention", "la_kernel_gemm", "la_kernel_gemm_ws_bytes", "la_step_profile",
    "la_kernel_attention_ws_bytes", "la_packed_bytes", "la_pack_weight", "la_probe_read",
    "la_step_trace", "la_step_trace_bytes", "la_philox_uniform", "la_kernel_gemm_noalloc",
]

PROF_KINDS = ["gemm", "lm_head", "attention", "norm", "epilogue", "argmax", "bookkeeping"]


class LaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"la error {code}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("W", ctypes.c_int32), ("G", ctypes.c_int32),
                ("pool_cap", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("max_new", ctypes.c_int32), ("eos_id", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("temperature", ctypes.c_float),
                ("top_k", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("top_p", ctypes.c_float), ("reserved", ctypes.c_uint32)]


class PoolStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("tokens", ctypes.c_int64),
                ("accept_hist", ctypes.c_int64 * (LA_MAX_N + 1)),
                ("pool_ngrams", ctypes.c_int64), ("pool_keys_nonempty", ctypes.c_int64),
                ("inserts", ctypes.c_int64), ("dup_skips", ctypes.c_int64),
                ("evictions", ctypes.c_int64), ("gathers_nonempty", ctypes.c_int64),
                ("cand_total", ctypes.c_int64), ("rows_total", ctypes.c_int64)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "accept_hist"}
        d["accept_hist"] = list(self.accept_hist)
        return d


class Profile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32 * 7), ("ms", ctypes.c_double * 7),
                ("bytes", ctypes.c_double * 7), ("flops", ctypes.c_double * 7)]

    def as_dict(self) -> dict:
        return {k: {"launches": self.launches[i], "ms": self.ms[i], "bytes": self.bytes[i],
                    "flops": self.flops[i]} for i, k in enumerate(PROF_KINDS)}


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libla.so not built ({path}); run exact_decoding_amd/build.py")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.la_model_load.argtypes = [ctypes.POINTER(ModelDesc), ctypes.POINTER(P), ctypes.c_int, P,
                                  ctypes.POINTER(P)]
    lib.la_model_free.argtypes = [P]
    lib.la_model_free.restype = None
    lib.la_session_bytes.argtypes = [P, ctypes.POINTER(DecodeParams), ctypes.POINTER(SZ)]
    lib.la_prefill.argtypes = [P, ctypes.POINTER(DecodeParams), ctypes.POINTER(I32), I32,
                               ctypes.POINTER(I32), P, SZ, P, ctypes.POINTER(P)]
    lib.la_step.argtypes = [P, ctypes.POINTER(I32), I32, ctypes.POINTER(I32)]
    lib.la_pool_stats.argtypes = [P, ctypes.POINTER(PoolStats)]
    lib.la_step_profile.argtypes = [P, ctypes.POINTER(I32), I32, ctypes.POINTER(I32),
                                    ctypes.POINTER(Profile)]
    lib.la_debug_logits.argtypes = [P, ctypes.POINTER(ctypes.c_float), I32]
    lib.la_step_trace.argtypes = [P, ctypes.POINTER(I32), I32, ctypes.POINTER(I32), P,
                                  ctypes.c_size_t]
    lib.la_step_trace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.la_session_rows.argtypes = [P, ctypes.POINTER(I32)]
    lib.la_session_free.argtypes = [P]
    lib.la_session_free.restype = None
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_kernel_attention.argtypes = [P, P, P, I32, I32, P, P, P, I32, I32, I32, I32, I32, I32,
                                        I32, P, SZ, P]
    lib.la_kernel_attention_ws_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.la_kernel_attention_ws_bytes.restype = SZ
    lib.la_kernel_gemm.argtypes = [P, I32, I32, P, I32, P, I32, P, SZ, P]
    lib.la_kernel_gemm_noalloc.argtypes = [P, I32, I32, P, I32, P, I32, P]
    lib.la_probe_read.argtypes = [P, SZ, P, P]
    lib.la_philox_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, I32, P, P]
    lib.la_packed_bytes.argtypes = [I32, I32]
    lib.la_packed_bytes.restype = SZ
    lib.la_pack_weight.argtypes = [P, I32, I32, P, P]
    lib.la_kernel_gemm_ws_bytes.argtypes = [I32, I32, I32]
    lib.la_kernel_gemm_ws_bytes.restype = SZ
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc < 0:
        raise LaError(rc, _lib.la_last_error().decode())
    return rc


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int:
    return 0 if stream is None else int(stream.cuda_stream)


# ---------------------------------------------------------------------------
# same-named wrappers of the C-ABI calls
# ---------------------------------------------------------------------------

def la_model_load(desc: ModelDesc, weights, stream) -> ctypes.c_void_p:
    lib = load_library()
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    out = ctypes.c_void_p()
    _check(lib.la_model_load(ctypes.byref(desc), arr, len(weights),
                             ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(out)))
    return out


def la_session_bytes(model, params: DecodeParams) -> int:
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.la_session_bytes(model, ctypes.byref(params), ctypes.byref(n)))
    return n.value


def la_prefill(model, params: DecodeParams, prompt, init_window, workspace, stream):
    lib = load_library()
    pr = np.ascontiguousarray(prompt, dtype=np.int32)
    win = None if init_window is None else np.ascontiguousarray(init_window, dtype=np.int32)
    out = ctypes.c_void_p()
    _check(lib.la_prefill(
        model, ctypes.byref(params), pr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(pr),
        None if win is None else win.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        ctypes.c_void_p(_ptr(workspace)), workspace.numel() * workspace.element_size(),
        ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(out)))
    return out


def la_step(session, out_cap: int) -> tuple[int, list[int]]:
    lib = load_library()
    buf = (ctypes.c_int32 * out_cap)()
    n = ctypes.c_int32()
    rc = _check(lib.la_step(session, buf, out_cap, ctypes.byref(n)))
    return rc, list(buf[:n.value])


def la_step_profile(session, out_cap: int) -> tuple[int, list[int], dict]:
    lib = load_library()
    buf = (ctypes.c_int32 * out_cap)()
    n = ctypes.c_int32()
    prof = Profile()
    rc = _check(lib.la_step_profile(session, buf, out_cap, ctypes.byref(n), ctypes.byref(prof)))
    return rc, list(buf[:n.value]), prof.as_dict()


def la_step_trace_bytes(session) -> int:
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.la_step_trace_bytes(session, ctypes.byref(n)))
    return n.value


def la_step_trace(session, out_cap: int, trace, nbytes: int) -> tuple[int, list[int]]:
    """One step with the per-layer trace written to device memory `trace`
    (a device pointer or a tensor exposing data_ptr())."""
    lib = load_library()
    buf = (ctypes.c_int32 * out_cap)()
    n = ctypes.c_int32()
    rc = _check(lib.la_step_trace(session, buf, out_cap, ctypes.byref(n), _ptr(trace), nbytes))
    return rc, list(buf[:n.value])


def la_pool_stats(session) -> dict:
    lib = load_library()
    st = PoolStats()
    _check(lib.la_pool_stats(session, ctypes.byref(st)))
    return st.as_dict()


def la_debug_logits(session, rows: int, vocab: int) -> np.ndarray:
    lib = load_library()
    out = np.empty((rows, vocab), dtype=np.float32)
    _check(lib.la_debug_logits(session, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), rows))
    return out


def la_session_rows(session) -> int:
    lib = load_library()
    n = ctypes.c_int32()
    _check(lib.la_session_rows(session, ctypes.byref(n)))
    return n.value


def la_session_free(session) -> None:
    load_library().la_session_free(session)


def la_model_free(model) -> None:
    load_library().la_model_free(model)


def la_kernel_attention_ws_bytes(ld_ctx, H, hd, N, W, G, dtype) -> int:
    return int(load_library().la_kernel_attention_ws_bytes(ld_ctx, H, hd, N, W, G, dtype))


def la_kernel_attention(q, k_cache, v_cache, P, ld_ctx, k_blk, v_blk, out, H, Hkv, hd, N, W, G,
                        dtype, ws, stream) -> None:
    lib = load_library()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.la_kernel_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), P, ld_ctx, _ptr(k_blk),
                                   _ptr(v_blk), _ptr(out), H, Hkv, hd, N, W, G, dtype, _ptr(ws),
                                   nbytes, ctypes.c_void_p(_stream_handle(stream))))


def la_philox_uniform(seed: int, step: int, n: int, out, stream) -> None:
    """out[i] = draw i of `step` under `seed` (device float32 tensor of >= n)."""
    _check(load_library().la_philox_uniform(seed, step, n, _ptr(out),
                                            ctypes.c_void_p(_stream_handle(stream))))


def la_probe_read(buf, nbytes: int, out, stream) -> None:
    _check(load_library().la_probe_read(_ptr(buf), nbytes, _ptr(out),
                                        ctypes.c_void_p(_stream_handle(stream))))


def la_packed_bytes(N: int, K: int) -> int:
    return int(load_library().la_packed_bytes(N, K))


def la_pack_weight(src, N: int, K: int, dst, stream) -> None:
    _check(load_library().la_pack_weight(_ptr(src), N, K, _ptr(dst),
                                         ctypes.c_void_p(_stream_handle(stream))))


def la_kernel_gemm_ws_bytes(M: int, K: int, N: int) -> int:
    return int(load_library().la_kernel_gemm_ws_bytes(M, K, N))


def la_kernel_gemm(x, M, K, w, N, y, dtype, ws, stream) -> None:
    lib = load_library()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.la_kernel_gemm(_ptr(x), M, K, _ptr(w), N, _ptr(y), dtype, _ptr(ws), nbytes,
                              ctypes.c_void_p(_stream_handle(stream))))


def la_kernel_gemm_noalloc(x, M, K, w, N, y, dtype, stream) -> None:
    _check(load_library().la_kernel_gemm_noalloc(_ptr(x), M, K, _ptr(w), N, _ptr(y), dtype,
                                                 ctypes.c_void_p(_stream_handle(stream))))
