"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every call include/la.h declares, and rejects bad arguments before any
device work."""
import ctypes
import os
import re

import pytest

from exact_decoding_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "la.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = B.load_library()
    names = _declared()
    assert "la_step" in names and "la_prefill" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTS) == set(names)


def test_flag_values_match_header():
    src = open(os.path.join(ROOT, "include", "la.h")).read()
    defs = dict(re.findall(r"#define (LA_[A-Z_]+) (\d+)u", src))
    assert defs == {"LA_PROMPT_REF": str(B.LA_PROMPT_REF), "LA_AR": str(B.LA_AR),
                    "LA_NO_GRAPH": str(B.LA_NO_GRAPH), "LA_POOL_LRU": str(B.LA_POOL_LRU),
                    "LA_POOL_CONTEXT": str(B.LA_POOL_CONTEXT),
                    "LA_ADAPTIVE_G": str(B.LA_ADAPTIVE_G),
                    "LA_DEBUG_LOGITS": str(B.LA_DEBUG_LOGITS)}


def _model(dtype=B.LA_BF16, L=2, d=512, H=4, Hkv=4, hd=128, F=1408, V=4000):
    desc = B.ModelDesc(L, d, H, Hkv, hd, F, V, 10000.0, 1e-5, dtype)
    # la_model_load only records the pointers: fake non-null values are fine
    fake = [ctypes.c_void_p(0x1000 + 256 * i) for i in range(3 + 9 * L)]
    arr = (ctypes.c_void_p * len(fake))(*fake)
    lib = B.load_library()
    out = ctypes.c_void_p()
    rc = lib.la_model_load(ctypes.byref(desc), arr, len(fake), None, ctypes.byref(out))
    return rc, out


def test_model_load_validation():
    rc, m = _model()
    assert rc == B.LA_OK and m.value
    B.la_model_free(m)
    assert _model(hd=96)[0] == B.LA_EINVAL
    assert _model(H=4, Hkv=3)[0] == B.LA_EINVAL
    assert _model(d=500)[0] == B.LA_EINVAL          # bf16 needs d % 64 == 0
    # every model: d a multiple of 64 (the norm epilogue's whole waves per row)
    assert _model(dtype=B.LA_F32, d=500, H=4, hd=16, F=100)[0] == B.LA_EINVAL
    rc, m = _model(dtype=B.LA_F32, d=64, H=4, hd=16, F=100)
    assert rc == B.LA_OK
    B.la_model_free(m)
    assert _model(dtype=7)[0] == B.LA_EINVAL


def test_session_bytes_and_param_validation():
    rc, m = _model()
    p = B.DecodeParams(5, 15, 15, 0, 400, 256, -1, B.LA_PROMPT_REF)
    n = B.la_session_bytes(m, p)
    assert n > 0
    p_ar = B.DecodeParams(5, 15, 15, 0, 400, 256, -1, B.LA_AR)
    assert 0 < B.la_session_bytes(m, p_ar) < n
    # a temperature adds the sampling weights of row 0 and the 60
    # verification rows (vocab floats each, plus their sums; 256-byte aligned)
    p_s = B.DecodeParams(5, 15, 15, 0, 400, 256, -1, B.LA_PROMPT_REF, 0.8, 0, 12345)
    ns = B.la_session_bytes(m, p_s)
    align = lambda b: (b + 255) // 256 * 256
    assert ns == n + align(61 * 4000 * 4) + align(61 * 4)
    # the seed changes nothing
    assert B.la_session_bytes(m, B.DecodeParams(5, 15, 15, 0, 400, 256, -1, B.LA_PROMPT_REF, 0.8, 0, 7)) == ns
    # nor does the pool's eviction policy
    p_l = B.DecodeParams(5, 15, 15, 0, 400, 256, -1,
                         B.LA_PROMPT_REF | B.LA_POOL_LRU | B.LA_POOL_CONTEXT)
    assert B.la_session_bytes(m, p_l) == n
    # nor do top-K / top-P (K past the vocabulary and p = 1 are no cut)
    for k, pp in [(40, 0.9), (1, 0.0), (10 ** 6, 1.0)]:
        p_k = B.DecodeParams(5, 15, 15, 0, 400, 256, -1, B.LA_PROMPT_REF, 0.8, k, 12345, pp)
        assert B.la_session_bytes(m, p_k) == ns
    for bad in [B.DecodeParams(1, 4, 4, 0, 100, 10, -1, 0), B.DecodeParams(17, 4, 4, 0, 100, 10, -1, 0),
                B.DecodeParams(3, -1, 4, 0, 100, 10, -1, 0), B.DecodeParams(3, 4, 4, 0, 100, 0, -1, 0),
                B.DecodeParams(3, 4, 4, 0, 100, 10, 4000, 0), B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 128),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 128 * 2),
                B.DecodeParams(2, 0, 1025, 0, 4000, 10, -1, 0),
                B.DecodeParams(16, 100, 100, 0, 100, 10, -1, 0),
                # sampling: negative or non-finite temperature, reserved field set
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, -0.5, 0, 1),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, float("nan"), 0, 1),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, float("inf"), 0, 1),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, 1.0, 0, 1, 0.0, 7),
                # top-K / top-P out of range
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, 1.0, -1, 1),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, 1.0, 0, 1, 1.5),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, 1.0, 0, 1, -0.1),
                B.DecodeParams(3, 4, 4, 0, 100, 10, -1, 0, 1.0, 0, 1, float("nan"))]:
        with pytest.raises(B.LaError) as e:
            B.la_session_bytes(m, bad)
        assert e.value.code == B.LA_EINVAL
    B.la_model_free(m)


def test_prefill_rejects_before_device_work():
    lib = B.load_library()
    rc, m = _model()
    p = B.DecodeParams(3, 4, 4, 0, 64, 8, -1, B.LA_NO_GRAPH)
    prompt = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    out = ctypes.c_void_p()
    ws = ctypes.c_void_p(0x10000)
    # workspace too small
    assert lib.la_prefill(m, ctypes.byref(p), prompt, 4, None, ws, 16, None, ctypes.byref(out)) == B.LA_ENOMEM
    need = B.la_session_bytes(m, p)
    # token out of range
    bad = (ctypes.c_int32 * 4)(1, 2, 3, 4000)
    assert lib.la_prefill(m, ctypes.byref(p), bad, 4, None, ws, need, None, ctypes.byref(out)) == B.LA_EINVAL
    # empty prompt
    assert lib.la_prefill(m, ctypes.byref(p), prompt, 0, None, ws, need, None, ctypes.byref(out)) == B.LA_EINVAL
    # prompt too long for max_ctx
    long_prompt = (ctypes.c_int32 * 70)(*([1] * 70))
    assert lib.la_prefill(m, ctypes.byref(p), long_prompt, 70, None, ws, need, None, ctypes.byref(out)) == B.LA_ECTX
    # graph mode needs a stream
    p2 = B.DecodeParams(3, 4, 4, 0, 64, 8, -1, 0)
    assert lib.la_prefill(m, ctypes.byref(p2), prompt, 4, None, ws, need, None, ctypes.byref(out)) == B.LA_EINVAL
    assert b"stream" in lib.la_last_error()
    B.la_model_free(m)


def test_step_null_args():
    lib = B.load_library()
    n = ctypes.c_int32()
    assert lib.la_step(None, None, 4, ctypes.byref(n)) == B.LA_EINVAL
    buf = (ctypes.c_int32 * 4)()
    assert lib.la_step_trace(None, buf, 4, ctypes.byref(n), None, 0) == B.LA_EINVAL
    assert lib.la_step_trace(None, buf, 4, ctypes.byref(n), 256, 1 << 20) == B.LA_EINVAL
    nb = ctypes.c_size_t()
    assert lib.la_step_trace_bytes(None, ctypes.byref(nb)) == B.LA_EINVAL


def test_kernel_hooks_validate():
    lib = B.load_library()
    P = ctypes.c_void_p(0x1000)
    # bad head_dim / N
    assert lib.la_kernel_attention(P, P, P, 4, 8, P, P, P, 4, 4, 100, 3, 2, 2, 1, None, 0, None) == B.LA_EINVAL
    assert lib.la_kernel_attention(P, P, P, 4, 8, P, P, P, 4, 4, 128, 1, 2, 2, 1, None, 0, None) == B.LA_EINVAL
    assert lib.la_kernel_attention(P, P, P, 9, 8, P, P, P, 4, 4, 128, 3, 2, 2, 1, None, 0, None) == B.LA_EINVAL
    # bf16 head_dim 128 needs the partial-state scratch
    assert B.la_kernel_attention_ws_bytes(512, 32, 128, 5, 15, 15, B.LA_BF16) > 0
    assert lib.la_kernel_attention(P, P, P, 4, 8, P, P, P, 4, 4, 128, 3, 2, 2, 1, None, 0, None) == B.LA_ENOMEM
    # W + G past INT_MAX: widened before the row count is formed, then refused
    imax = 2**31 - 1
    assert lib.la_kernel_attention(P, P, P, 4, 8, P, P, P, 4, 4, 128, 3, imax, 2, 1, None, 0, None) == B.LA_EINVAL
    assert lib.la_kernel_attention(P, P, P, 4, 8, P, P, P, 4, 4, 128, 3, imax, imax, 1, None, 0, None) == B.LA_EINVAL
    assert B.la_kernel_attention_ws_bytes(512, 32, 128, 3, imax, 2, B.LA_BF16) == 0
    assert B.la_kernel_attention_ws_bytes(512, 32, 128, 3, imax, imax, B.LA_BF16) == 0
    # bf16 GEMM needs K % 64 == 0
    assert lib.la_kernel_gemm(P, 4, 100, P, 64, P, B.LA_BF16, None, 0, None) == B.LA_EINVAL
    assert B.la_kernel_gemm_ws_bytes(121, 4096, 4096) > 0
    # the allocation-free variant: same argument checks, and partial sums
    # beyond its static scratch are refused before any device work
    assert lib.la_kernel_gemm_noalloc(None, 4, 64, P, 64, P, B.LA_BF16, None) == B.LA_EINVAL
    assert lib.la_kernel_gemm_noalloc(P, 4, 100, P, 64, P, B.LA_BF16, None) == B.LA_EINVAL
    assert lib.la_kernel_gemm_noalloc(P, 0, 64, P, 64, P, B.LA_BF16, None) == B.LA_EINVAL
    assert B.la_kernel_gemm_ws_bytes(2048, 4096, 4096) > B.LA_NOALLOC_SCRATCH_BYTES
    assert lib.la_kernel_gemm_noalloc(P, 2048, 4096, P, 4096, P, B.LA_BF16, None) == B.LA_ENOMEM
    assert b"static scratch" in lib.la_last_error()


def test_binding_constants_match_header():
    """Every numeric constant la.h defines has the same value in the binding."""
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "la.h")).read()
    consts = {m.group(1): int(m.group(2)) for m in
              re.finditer(r"^#define (LA_[A-Z_0-9]+) (-?\d+)u?\b", text, re.M)}
    consts.update({m.group(1): int(m.group(2)) for m in
                   re.finditer(r"^\s+(LA_[A-Z_0-9]+) = (-?\d+),?", text, re.M)
                   if not m.group(1).startswith("LA_PROF_")})
    assert len(consts) >= 12
    for k, v in consts.items():
        assert getattr(B, k) == v, k
