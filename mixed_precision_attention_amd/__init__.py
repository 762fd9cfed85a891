"""Python binding of libtilemix, the MI355X (gfx950) TileMix prefill library.

Argument marshalling only: every step of the path (routing words, work plan,
quantisation, fused attention) runs inside libtilemix.so -- the host steps in
its C++ half, the device steps in its HIP kernels.  PyTorch supplies device
memory and the current HIP stream.  The functions carry the names of the C
entry points declared in include/tilemix.h; ``TileMixPrefill`` bundles them
for one packed batch shape, ``TileMixDecode`` for one decode step over an
INT8 key/value cache and ``TileMixStack`` for a synthetic stack of
attention + residual layers.

The library must be built first (``python -m mixed_precision_attention_amd.build``);
importing works without it, but every call raises ``TileMixError`` when the
shared library is missing -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; TILEMIX_LIB may name one of build.py's checking builds
# (``_build/debug`` or ``_build/host_sanitize``) instead.
LIB_PATH = os.environ.get("TILEMIX_LIB") or os.path.join(_HERE, "libtilemix.so")

BLOCK_M = 128
BLOCK_N = 64

TEMPLATE_IDS = {"band": 0, "global": 1, "rowrandom": 2, "alignedsparse": 3, "bigbird": 4,
                "sptrans": 5}

_STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EHIP"}


class TileMixError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"tilemix {_STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64

_SIGNATURES = {
    "tilemix_last_error": ([], ctypes.c_char_p),
    "tilemix_query_sizes": ([_P, _I32, _P, _P, _P], ctypes.c_int),
    "tilemix_build_routing": ([_P, _I32, _I32, _I32, _I32, _U64, _P, _P, _P, _P], ctypes.c_int),
    "tilemix_plan_size": ([_P, _I32, _I32, _I32, _I32, _P], ctypes.c_int),
    "tilemix_build_plan": ([_P, _I32, _I32, _I32, _I32, _P, _I64], ctypes.c_int),
    "tilemix_quantize_qk": ([_P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "tilemix_prefill_varlen": ([_P] * 12, ctypes.c_int),
    "tilemix_quantize_k": ([_P] * 6, ctypes.c_int),
    "tilemix_prefill_varlen_qinline": ([_P] * 10, ctypes.c_int),
    "tilemix_quantize_k_fp8": ([_P] * 6, ctypes.c_int),
    "tilemix_quantize_k_i8_fp8": ([_P] * 8, ctypes.c_int),
    "tilemix_prefill_varlen3_qinline": ([_P] * 13, ctypes.c_int),
    "tilemix_debug_qk_i32_tile": ([_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "tilemix_debug_qk_f8_tile": ([_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "tilemix_quantize_kv": ([_P] * 9, ctypes.c_int),
    "tilemix_build_routing3": ([_P, _I32, _I32, _I32, _I32, _I32, _U64, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "tilemix_quantize_qk_fp8": ([_P] * 9, ctypes.c_int),
    "tilemix_prefill_varlen3": ([_P] * 17, ctypes.c_int),
    "tilemix_build_routing_adaptive": ([_P, _I32, _I32, _P, _I32, _P, _P, _P, _P], ctypes.c_int),
    "tilemix_importance_workspace_size": ([_P, _P], ctypes.c_int),
    "tilemix_routing_importance": ([_P] * 7 + [_I64, _P, _P], ctypes.c_int),
    "tilemix_select_routing_adaptive": ([_P, _P, _P, _I32, _P, _P, _P, _P], ctypes.c_int),
    "tilemix_decode_workspace_size": ([_P, _P], ctypes.c_int),
    "tilemix_decode_varlen": ([_P] * 9 + [_I64, _P, _P], ctypes.c_int),
    "tilemix_decode_varlen_noalloc": ([_P] * 10, ctypes.c_int),
    "tilemix_stack_rms_norm": ([_P, _P, _I64, _I32, _I32, _I32, ctypes.c_float, _P], ctypes.c_int),
    "tilemix_stack_qkv": ([_P] * 5 + [_I64, _I32, _I32, _I32, _P], ctypes.c_int),
    "tilemix_stack_out_residual": ([_P] * 3 + [_I64, _I32, _I32, _I32, _P], ctypes.c_int),
    "tilemix_stack_workspace_size": ([_P, _P], ctypes.c_int),
    "tilemix_stack_layer": ([_P] * 6 + [ctypes.c_float, _P, _I64, _P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """Load libtilemix.so (raises TileMixError when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TileMixError(-3, f"{LIB_PATH} is not built; run "
                                   "`python -m mixed_precision_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        msg = lib().tilemix_last_error()
        raise TileMixError(rc, msg.decode() if msg else "")


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _hptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def _dptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous torch tensor on a GPU."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TileMixError(-1, f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TileMixError(-1, f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TileMixError(-1, f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dims(plan_h):
    """(T, B, Hq, Hkv, d, total_q_tiles, total_k_tiles) from a plan's header."""
    p = np.asarray(plan_h)
    if p.dtype != np.int32 or p.ndim != 1 or p.size < 16:
        raise TileMixError(-1, "plan_h must be the int32 array tilemix_build_plan returned")
    return int(p[6]), int(p[2]), int(p[3]), int(p[4]), int(p[5]), int(p[7]), int(p[8])


def _sizes(plan_h, plan_d=None, **need):
    """Refuse, before any launch, a tensor smaller than the plan makes the
    kernels touch (name=(tensor, elements)), and a device plan that is not
    plan_h's size."""
    if plan_d is not None and plan_d.numel() != np.asarray(plan_h).size:
        raise TileMixError(-1, f"plan_d holds {plan_d.numel()} int32, plan_h {np.asarray(plan_h).size}: "
                               "plan_d must be the device copy of plan_h")
    for name, (t, n) in need.items():
        if t is None:
            if n > 0:
                raise TileMixError(-1, f"{name} is missing")
            continue
        if t.numel() < n:
            raise TileMixError(-1, f"{name} holds {t.numel()} elements; the plan needs {n}")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------- host calls

def tilemix_last_error() -> str:
    msg = lib().tilemix_last_error()
    return msg.decode() if msg else ""


def tilemix_query_sizes(cu_seqlens):
    cu = _host_i32(cu_seqlens)
    out = (ctypes.c_int64 * 3)()
    _check(lib().tilemix_query_sizes(_hptr(cu), len(cu) - 1, ctypes.byref(out, 0),
                                     ctypes.byref(out, 8), ctypes.byref(out, 16)))
    return int(out[0]), int(out[1]), int(out[2])


def tilemix_build_routing(cu_seqlens, num_kv_heads: int, template, coverage_bp: int, seed: int = 0):
    """Returns (words uint64 [Hkv, sum Tm], g int32 [B], n_int8 int64 [B], n_legal int64 [B])."""
    cu = _host_i32(cu_seqlens)
    batch = len(cu) - 1
    tmpl = TEMPLATE_IDS[template] if isinstance(template, str) else int(template)
    _, tq, _ = tilemix_query_sizes(cu)
    words = np.zeros((max(num_kv_heads, 0), tq), dtype=np.uint64)
    g = np.zeros(batch, dtype=np.int32)
    n8 = np.zeros(batch, dtype=np.int64)
    nl = np.zeros(batch, dtype=np.int64)
    _check(lib().tilemix_build_routing(_hptr(cu), batch, int(num_kv_heads), tmpl, int(coverage_bp),
                                       ctypes.c_uint64(seed & (2 ** 64 - 1)), _hptr(words),
                                       _hptr(g), _hptr(n8), _hptr(nl)))
    return words, g, n8, nl


def tilemix_build_routing3(cu_seqlens, num_kv_heads: int, template, int8_bp: int, fp8_bp: int, seed: int = 0):
    """Returns (INT8 words, FP8 words, g, N8, Nf8, N_legal)."""
    cu = _host_i32(cu_seqlens)
    batch = len(cu) - 1
    tmpl = TEMPLATE_IDS[template] if isinstance(template, str) else int(template)
    _, tq, _ = tilemix_query_sizes(cu)
    w8 = np.zeros((max(num_kv_heads, 0), tq), dtype=np.uint64)
    wf = np.zeros_like(w8)
    g = np.zeros(batch, dtype=np.int32)
    n8 = np.zeros(batch, dtype=np.int64)
    nf = np.zeros(batch, dtype=np.int64)
    nl = np.zeros(batch, dtype=np.int64)
    _check(lib().tilemix_build_routing3(_hptr(cu), batch, int(num_kv_heads), tmpl, int(int8_bp), int(fp8_bp),
                                        ctypes.c_uint64(seed & (2 ** 64 - 1)), _hptr(w8), _hptr(wf), _hptr(g),
                                        _hptr(n8), _hptr(nf), _hptr(nl)))
    return w8, wf, g, n8, nf, nl


def tilemix_build_routing_adaptive(cu_seqlens, importance, coverage_bp: int):
    """Words from group importances float32 [Hkv, sum Tm, 64]; returns as
    tilemix_build_routing."""
    cu = _host_i32(cu_seqlens)
    batch = len(cu) - 1
    imp = np.ascontiguousarray(np.asarray(importance, dtype=np.float32))
    hkv = imp.shape[0]
    _, tq, _ = tilemix_query_sizes(cu)
    words = np.zeros((hkv, tq), dtype=np.uint64)
    g = np.zeros(batch, dtype=np.int32)
    n8 = np.zeros(batch, dtype=np.int64)
    nl = np.zeros(batch, dtype=np.int64)
    _check(lib().tilemix_build_routing_adaptive(_hptr(cu), batch, hkv, _hptr(imp), int(coverage_bp),
                                                _hptr(words), _hptr(g), _hptr(n8), _hptr(nl)))
    return words, g, n8, nl


def tilemix_build_plan(cu_seqlens, hq: int, hkv: int, head_dim: int) -> np.ndarray:
    cu = _host_i32(cu_seqlens)
    n = ctypes.c_int64(0)
    _check(lib().tilemix_plan_size(_hptr(cu), len(cu) - 1, hq, hkv, head_dim, ctypes.byref(n)))
    plan = np.zeros(n.value, dtype=np.int32)
    _check(lib().tilemix_build_plan(_hptr(cu), len(cu) - 1, hq, hkv, head_dim, _hptr(plan), n.value))
    return plan


# --------------------------------------------------------------- device calls

def tilemix_quantize_qk(plan_h, plan_d, q, k, q_i8, k_i8, q_scale, k_scale, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), q_i8=(q_i8, T * hq * d), k_i8=(k_i8, T * hkv * d),
           q_scale=(q_scale, hq * tq), k_scale=(k_scale, hkv * tk))
    _check(lib().tilemix_quantize_qk(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(q_i8, torch.int8, "q_i8"), _dptr(k_i8, torch.int8, "k_i8"),
        _dptr(q_scale, torch.float32, "q_scale"), _dptr(k_scale, torch.float32, "k_scale"),
        _stream(stream)))


def tilemix_prefill_varlen(plan_h, plan_d, q, k, v, q_i8, k_i8, q_scale, k_scale, words_d, out,
                           stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), v=(v, T * hkv * d), q_i8=(q_i8, T * hq * d),
           k_i8=(k_i8, T * hkv * d), q_scale=(q_scale, hq * tq), k_scale=(k_scale, hkv * tk),
           words_d=(words_d, hkv * tq), out=(out, T * hq * d))
    _check(lib().tilemix_prefill_varlen(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(v, torch.float16, "v"), _dptr(q_i8, torch.int8, "q_i8"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(q_scale, torch.float32, "q_scale"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(words_d, torch.int64, "words_d"),
        _dptr(out, torch.float16, "out"), _stream(stream)))


def tilemix_quantize_k(plan_h, plan_d, k, k_i8, k_scale, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, k=(k, T * hkv * d), k_i8=(k_i8, T * hkv * d), k_scale=(k_scale, hkv * tk))
    _check(lib().tilemix_quantize_k(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(k, torch.float16, "k"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(k_scale, torch.float32, "k_scale"), _stream(stream)))


def tilemix_prefill_varlen_qinline(plan_h, plan_d, q, k, v, k_i8, k_scale, words_d, out, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), v=(v, T * hkv * d), k_i8=(k_i8, T * hkv * d),
           k_scale=(k_scale, hkv * tk), words_d=(words_d, hkv * tq), out=(out, T * hq * d))
    _check(lib().tilemix_prefill_varlen_qinline(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(v, torch.float16, "v"), _dptr(k_i8, torch.int8, "k_i8"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(words_d, torch.int64, "words_d"),
        _dptr(out, torch.float16, "out"), _stream(stream)))


def tilemix_quantize_k_fp8(plan_h, plan_d, k, k_f8, k_scale_f8, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, k=(k, T * hkv * d), k_f8=(k_f8, T * hkv * d), k_scale_f8=(k_scale_f8, hkv * tk))
    _check(lib().tilemix_quantize_k_fp8(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(k, torch.float16, "k"),
        _dptr(k_f8, torch.uint8, "k_f8"), _dptr(k_scale_f8, torch.float32, "k_scale_f8"), _stream(stream)))


def tilemix_quantize_k_i8_fp8(plan_h, plan_d, k, k_i8, k_scale, k_f8, k_scale_f8, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, k=(k, T * hkv * d), k_i8=(k_i8, T * hkv * d), k_scale=(k_scale, hkv * tk),
           k_f8=(k_f8, T * hkv * d), k_scale_f8=(k_scale_f8, hkv * tk))
    _check(lib().tilemix_quantize_k_i8_fp8(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(k, torch.float16, "k"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(k_scale, torch.float32, "k_scale"), _dptr(k_f8, torch.uint8, "k_f8"),
        _dptr(k_scale_f8, torch.float32, "k_scale_f8"), _stream(stream)))


def tilemix_prefill_varlen3_qinline(plan_h, plan_d, q, k, v, k_i8, k_scale, k_f8, k_scale_f8, words_i8_d,
                                    words_f8_d, out, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), v=(v, T * hkv * d), k_i8=(k_i8, T * hkv * d),
           k_scale=(k_scale, hkv * tk), k_f8=(k_f8, T * hkv * d), k_scale_f8=(k_scale_f8, hkv * tk),
           words_i8_d=(words_i8_d, hkv * tq), words_f8_d=(words_f8_d, hkv * tq), out=(out, T * hq * d))
    _check(lib().tilemix_prefill_varlen3_qinline(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(v, torch.float16, "v"), _dptr(k_i8, torch.int8, "k_i8"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(k_f8, torch.uint8, "k_f8"),
        _dptr(k_scale_f8, torch.float32, "k_scale_f8"), _dptr(words_i8_d, torch.int64, "words_i8_d"),
        _dptr(words_f8_d, torch.int64, "words_f8_d"), _dptr(out, torch.float16, "out"), _stream(stream)))


def tilemix_quantize_qk_fp8(plan_h, plan_d, q, k, q_f8, k_f8, q_scale_f8, k_scale_f8, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), q_f8=(q_f8, T * hq * d), k_f8=(k_f8, T * hkv * d),
           q_scale_f8=(q_scale_f8, hq * tq), k_scale_f8=(k_scale_f8, hkv * tk))
    _check(lib().tilemix_quantize_qk_fp8(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(q_f8, torch.uint8, "q_f8"), _dptr(k_f8, torch.uint8, "k_f8"),
        _dptr(q_scale_f8, torch.float32, "q_scale_f8"), _dptr(k_scale_f8, torch.float32, "k_scale_f8"),
        _stream(stream)))


def tilemix_prefill_varlen3(plan_h, plan_d, q, k, v, q_i8, k_i8, q_scale, k_scale, q_f8, k_f8, q_scale_f8,
                            k_scale_f8, words_i8_d, words_f8_d, out, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, T * hq * d), k=(k, T * hkv * d), v=(v, T * hkv * d), q_i8=(q_i8, T * hq * d),
           k_i8=(k_i8, T * hkv * d), q_scale=(q_scale, hq * tq), k_scale=(k_scale, hkv * tk),
           q_f8=(q_f8, T * hq * d), k_f8=(k_f8, T * hkv * d), q_scale_f8=(q_scale_f8, hq * tq),
           k_scale_f8=(k_scale_f8, hkv * tk), words_i8_d=(words_i8_d, hkv * tq), words_f8_d=(words_f8_d, hkv * tq),
           out=(out, T * hq * d))
    _check(lib().tilemix_prefill_varlen3(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(v, torch.float16, "v"), _dptr(q_i8, torch.int8, "q_i8"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(q_scale, torch.float32, "q_scale"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(q_f8, torch.uint8, "q_f8"),
        _dptr(k_f8, torch.uint8, "k_f8"), _dptr(q_scale_f8, torch.float32, "q_scale_f8"),
        _dptr(k_scale_f8, torch.float32, "k_scale_f8"), _dptr(words_i8_d, torch.int64, "words_i8_d"),
        _dptr(words_f8_d, torch.int64, "words_f8_d"), _dptr(out, torch.float16, "out"), _stream(stream)))


def tilemix_debug_qk_i32_tile(plan_h, plan_d, q_i8, k_i8, seq: int, head: int, r: int, t: int,
                              acc, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q_i8=(q_i8, T * hq * d), k_i8=(k_i8, T * hkv * d), acc=(acc, 128 * 64))
    _check(lib().tilemix_debug_qk_i32_tile(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q_i8, torch.int8, "q_i8"),
        _dptr(k_i8, torch.int8, "k_i8"), seq, head, r, t, _dptr(acc, torch.int32, "acc"),
        _stream(stream)))


def tilemix_debug_qk_f8_tile(plan_h, plan_d, q_f8, k_f8, seq: int, head: int, r: int, t: int, acc,
                             stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q_f8=(q_f8, T * hq * d), k_f8=(k_f8, T * hkv * d), acc=(acc, 128 * 64))
    _check(lib().tilemix_debug_qk_f8_tile(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q_f8, torch.uint8, "q_f8"),
        _dptr(k_f8, torch.uint8, "k_f8"), seq, head, r, t, _dptr(acc, torch.float32, "acc"),
        _stream(stream)))


def tilemix_importance_workspace_size(plan_h) -> int:
    n = ctypes.c_int64(0)
    _check(lib().tilemix_importance_workspace_size(_hptr(plan_h), ctypes.byref(n)))
    return int(n.value)


def tilemix_routing_importance(plan_h, plan_d, q_i8, k_i8, q_scale, k_scale, workspace, importance,
                               stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q_i8=(q_i8, T * hq * d), k_i8=(k_i8, T * hkv * d), q_scale=(q_scale, hq * tq),
           k_scale=(k_scale, hkv * tk), importance=(importance, hkv * tq * 64))
    _check(lib().tilemix_routing_importance(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q_i8, torch.int8, "q_i8"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(q_scale, torch.float32, "q_scale"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _dptr(importance, torch.float32, "importance"),
        _stream(stream)))


def tilemix_select_routing_adaptive(plan_h, plan_d, importance, coverage_bp: int, words_d, stream=None):
    """Adaptive words selected on the device into ``words_d`` (int64 tensor
    holding the uint64 words, [Hkv, total_q_tiles]); returns the per-sequence
    (int8_groups, legal_groups) counts."""
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, importance=(importance, hkv * tq * 64), words_d=(words_d, hkv * tq))
    n8 = np.zeros(max(B, 1), dtype=np.int64)
    nl = np.zeros(max(B, 1), dtype=np.int64)
    _check(lib().tilemix_select_routing_adaptive(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(importance, torch.float32, "importance"),
        int(coverage_bp), _dptr(words_d, torch.int64, "words_d"), _hptr(n8), _hptr(nl), _stream(stream)))
    return n8[:B], nl[:B]


def tilemix_quantize_kv(plan_h, plan_d, k, v, k_i8, v_i8, k_scale, v_scale, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, k=(k, T * hkv * d), v=(v, T * hkv * d), k_i8=(k_i8, T * hkv * d),
           v_i8=(v_i8, T * hkv * d), k_scale=(k_scale, hkv * tk), v_scale=(v_scale, hkv * tk))
    _check(lib().tilemix_quantize_kv(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(k, torch.float16, "k"),
        _dptr(v, torch.float16, "v"), _dptr(k_i8, torch.int8, "k_i8"), _dptr(v_i8, torch.int8, "v_i8"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(v_scale, torch.float32, "v_scale"),
        _stream(stream)))


def tilemix_decode_workspace_size(plan_h) -> int:
    n = ctypes.c_int64(0)
    _check(lib().tilemix_decode_workspace_size(_hptr(plan_h), ctypes.byref(n)))
    return int(n.value)


def tilemix_decode_varlen(plan_h, plan_d, q, k_i8, v_i8, k_scale, v_scale, words_d, workspace, out,
                          stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, B * hq * d), k_i8=(k_i8, T * hkv * d), v_i8=(v_i8, T * hkv * d),
           k_scale=(k_scale, hkv * tk), v_scale=(v_scale, hkv * tk), words_d=(words_d, hkv * tq),
           out=(out, B * hq * d))
    _check(lib().tilemix_decode_varlen(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(v_i8, torch.int8, "v_i8"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(v_scale, torch.float32, "v_scale"),
        _dptr(words_d, torch.int64, "words_d"), _dptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _dptr(out, torch.float16, "out"),
        _stream(stream)))


def tilemix_decode_varlen_noalloc(plan_h, plan_d, q, k_i8, v_i8, k_scale, v_scale, words_d, out,
                                  stream=None):
    """tilemix_decode_varlen with its scratch in the library's static device
    array (nothing allocated; calls that overlap on one GPU race)."""
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    _sizes(plan_h, plan_d, q=(q, B * hq * d), k_i8=(k_i8, T * hkv * d), v_i8=(v_i8, T * hkv * d),
           k_scale=(k_scale, hkv * tk), v_scale=(v_scale, hkv * tk), words_d=(words_d, hkv * tq),
           out=(out, B * hq * d))
    _check(lib().tilemix_decode_varlen_noalloc(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(q, torch.float16, "q"),
        _dptr(k_i8, torch.int8, "k_i8"), _dptr(v_i8, torch.int8, "v_i8"),
        _dptr(k_scale, torch.float32, "k_scale"), _dptr(v_scale, torch.float32, "v_scale"),
        _dptr(words_d, torch.int64, "words_d"), _dptr(out, torch.float16, "out"), _stream(stream)))


def tilemix_stack_rms_norm(x, u, hq: int, hkv: int, head_dim: int, eps: float, stream=None):
    import torch
    _check(lib().tilemix_stack_rms_norm(
        _dptr(x, torch.float32, "x"), _dptr(u, torch.float16, "u"), x.shape[0], hq, hkv, head_dim, eps,
        _stream(stream)))


def tilemix_stack_qkv(u, wqkv, q, k, v, hq: int, hkv: int, head_dim: int, stream=None):
    import torch
    _check(lib().tilemix_stack_qkv(
        _dptr(u, torch.float16, "u"), _dptr(wqkv, torch.float16, "wqkv"), _dptr(q, torch.float16, "q"),
        _dptr(k, torch.float16, "k"), _dptr(v, torch.float16, "v"), u.shape[0], hq, hkv, head_dim,
        _stream(stream)))


def tilemix_stack_out_residual(o, wo, x, hq: int, hkv: int, head_dim: int, stream=None):
    import torch
    _check(lib().tilemix_stack_out_residual(
        _dptr(o, torch.float16, "o"), _dptr(wo, torch.float16, "wo"), _dptr(x, torch.float32, "x"),
        x.shape[0], hq, hkv, head_dim, _stream(stream)))


def tilemix_stack_workspace_size(plan_h) -> int:
    n = ctypes.c_int64(0)
    _check(lib().tilemix_stack_workspace_size(_hptr(plan_h), ctypes.byref(n)))
    return int(n.value)


def tilemix_stack_layer(plan_h, plan_d, words_d, x, wqkv, wo, eps: float, workspace, stream=None):
    import torch
    T, B, hq, hkv, d, tq, tk = _dims(plan_h)
    W = (hq // hkv) * d
    _sizes(plan_h, plan_d, words_d=(words_d, hkv * tq), x=(x, T * hq * d),
           wqkv=(wqkv, hkv * (W + 2 * d) * W), wo=(wo, hkv * W * W))
    _check(lib().tilemix_stack_layer(
        _hptr(plan_h), _dptr(plan_d, torch.int32, "plan_d"), _dptr(words_d, torch.int64, "words_d"),
        _dptr(x, torch.float32, "x"), _dptr(wqkv, torch.float16, "wqkv"), _dptr(wo, torch.float16, "wo"),
        eps, _dptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream)))


# ------------------------------------------------------------------ bundle

class TileMixPrefill:
    """One packed batch shape: host/device plan, routing words and the
    quantised-operand buffers, reused across calls (the pages reuse a static
    template across layers, batch entries and KV heads)."""

    def __init__(self, cu_seqlens, hq: int, hkv: int, head_dim: int, template, coverage_bp: int,
                 seed: int = 0, device="cuda"):
        import torch
        self.cu = _host_i32(cu_seqlens)
        self.hq, self.hkv, self.d = hq, hkv, head_dim
        self.tokens, self.tq, self.tk = tilemix_query_sizes(self.cu)
        self.plan_h = tilemix_build_plan(self.cu, hq, hkv, head_dim)
        self.plan_d = torch.from_numpy(self.plan_h).to(device)
        self.device = device
        self.set_routing(template, coverage_bp, seed)
        t = max(self.tokens, 1)
        self.q_i8 = torch.empty((t, hq, head_dim), dtype=torch.int8, device=device)
        self.k_i8 = torch.empty((t, hkv, head_dim), dtype=torch.int8, device=device)
        self.q_scale = torch.empty((hq, max(self.tq, 1)), dtype=torch.float32, device=device)
        self.k_scale = torch.empty((hkv, max(self.tk, 1)), dtype=torch.float32, device=device)

    def set_routing(self, template, coverage_bp: int, seed: int = 0):
        import torch
        self.words, self.g, self.n_int8, self.n_legal = tilemix_build_routing(
            self.cu, self.hkv, template, coverage_bp, seed)
        w = self.words if self.words.size else np.zeros((1, 1), dtype=np.uint64)
        self.words_d = torch.from_numpy(w.view(np.int64)).to(self.device)

    def set_routing_adaptive(self, coverage_bp: int, stream=None, on_device: bool = True):
        """Content-dependent words from the quantised Q and K of the last
        ``quantize`` call: the device statistic, then the selection on the
        device (``words_d`` written in place, nothing crosses to the host;
        ``words`` is set to None, ``words_host()`` downloads them) and the
        device importances returned, or with ``on_device=False`` the ranking
        on the host and an upload (the importances returned as numpy).  Both
        give the same words, bit for bit."""
        import torch
        if not hasattr(self, "imp_ws"):
            self.imp_ws = torch.empty(max(tilemix_importance_workspace_size(self.plan_h), 16),
                                      dtype=torch.uint8, device=self.device)
            self.importance = torch.empty((self.hkv, max(self.tq, 1), 64), dtype=torch.float32,
                                          device=self.device)
        tilemix_routing_importance(self.plan_h, self.plan_d, self.q_i8, self.k_i8, self.q_scale,
                                   self.k_scale, self.imp_ws, self.importance, stream)
        if on_device:
            shape = (self.hkv, max(self.tq, 1))
            if self.words_d is None or tuple(self.words_d.shape) != shape:
                self.words_d = torch.zeros(shape, dtype=torch.int64, device=self.device)
            self.n_int8, self.n_legal = tilemix_select_routing_adaptive(
                self.plan_h, self.plan_d, self.importance, coverage_bp, self.words_d, stream)
            self.words = None
            return self.importance
        imp = self.importance.cpu().numpy()[:, :self.tq]
        self.words, self.g, self.n_int8, self.n_legal = tilemix_build_routing_adaptive(
            self.cu, imp, coverage_bp)
        w = self.words if self.words.size else np.zeros((1, 1), dtype=np.uint64)
        self.words_d = torch.from_numpy(w.view(np.int64)).to(self.device)
        return imp

    def words_host(self):
        """The routing words in use, [Hkv, total_q_tiles] uint64 on the host
        (downloads them when they were selected on the device)."""
        if self.words is None:
            self.words = self.words_d.cpu().numpy().view(np.uint64)[:, :self.tq].copy()
        return self.words

    def quantize(self, q, k, stream=None):
        tilemix_quantize_qk(self.plan_h, self.plan_d, q, k, self.q_i8, self.k_i8, self.q_scale,
                            self.k_scale, stream)

    def attend(self, q, k, v, out, stream=None):
        tilemix_prefill_varlen(self.plan_h, self.plan_d, q, k, v, self.q_i8, self.k_i8,
                               self.q_scale, self.k_scale, self.words_d, out, stream)

    def quantize_k(self, k, stream=None):
        """The key half of ``quantize`` (for ``attend_qinline``)."""
        tilemix_quantize_k(self.plan_h, self.plan_d, k, self.k_i8, self.k_scale, stream)

    def attend_qinline(self, q, k, v, out, stream=None):
        """``attend`` with Q quantised inside the prefill kernel; needs the
        key codes of ``quantize_k`` (or ``quantize``)."""
        tilemix_prefill_varlen_qinline(self.plan_h, self.plan_d, q, k, v, self.k_i8, self.k_scale,
                                       self.words_d, out, stream)

    def __call__(self, q, k, v, out=None, stream=None, inline_q: bool = False):
        """One prefill step.  By default the quantiser writes Q's and K's
        codes (kept in ``q_i8``/``k_i8`` and the scales) and the prefill reads
        them; ``inline_q=True`` quantises K alone and lets the prefill quantise
        each Q block in registers (the same output, bit for bit, and faster;
        ``q_i8``/``q_scale`` are then left untouched)."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        if inline_q:
            self.quantize_k(k, stream)
            self.attend_qinline(q, k, v, out, stream)
        else:
            self.quantize(q, k, stream)
            self.attend(q, k, v, out, stream)
        return out


class TileMixPrefill3(TileMixPrefill):
    """Three score paths per group -- FP16, FP8 (E4M3) and INT8 -- from a
    template at INT8 coverage ``int8_bp`` and FP8 coverage ``fp8_bp``."""

    def __init__(self, cu_seqlens, hq: int, hkv: int, head_dim: int, template, int8_bp: int, fp8_bp: int,
                 seed: int = 0, device="cuda"):
        import torch
        super().__init__(cu_seqlens, hq, hkv, head_dim, template, int8_bp, seed, device)
        self.set_routing3(template, int8_bp, fp8_bp, seed)
        t = max(self.tokens, 1)
        self.q_f8 = torch.empty((t, hq, head_dim), dtype=torch.uint8, device=device)
        self.k_f8 = torch.empty((t, hkv, head_dim), dtype=torch.uint8, device=device)
        self.q_scale_f8 = torch.empty((hq, max(self.tq, 1)), dtype=torch.float32, device=device)
        self.k_scale_f8 = torch.empty((hkv, max(self.tk, 1)), dtype=torch.float32, device=device)

    def set_routing3(self, template, int8_bp: int, fp8_bp: int, seed: int = 0):
        import torch
        self.words, self.words_f8, self.g, self.n_int8, self.n_fp8, self.n_legal = tilemix_build_routing3(
            self.cu, self.hkv, template, int8_bp, fp8_bp, seed)
        for name, w in (("words_d", self.words), ("words_f8_d", self.words_f8)):
            w = w if w.size else np.zeros((1, 1), dtype=np.uint64)
            setattr(self, name, torch.from_numpy(w.view(np.int64)).to(self.device))

    def quantize_k(self, k, stream=None):
        """The key halves of both quantisers, in one pass over K (for
        ``attend_qinline``)."""
        tilemix_quantize_k_i8_fp8(self.plan_h, self.plan_d, k, self.k_i8, self.k_scale, self.k_f8,
                                  self.k_scale_f8, stream)

    def attend_qinline(self, q, k, v, out, stream=None):
        """``attend`` with Q's INT8 and FP8 codes made inside the kernel."""
        tilemix_prefill_varlen3_qinline(self.plan_h, self.plan_d, q, k, v, self.k_i8, self.k_scale, self.k_f8,
                                        self.k_scale_f8, self.words_d, self.words_f8_d, out, stream)

    def quantize(self, q, k, stream=None):
        super().quantize(q, k, stream)
        tilemix_quantize_qk_fp8(self.plan_h, self.plan_d, q, k, self.q_f8, self.k_f8, self.q_scale_f8,
                                self.k_scale_f8, stream)

    def attend(self, q, k, v, out, stream=None):
        tilemix_prefill_varlen3(self.plan_h, self.plan_d, q, k, v, self.q_i8, self.k_i8, self.q_scale,
                                self.k_scale, self.q_f8, self.k_f8, self.q_scale_f8, self.k_scale_f8,
                                self.words_d, self.words_f8_d, out, stream)


class TileMixDecode:
    """One decode step's shape over an INT8 key/value cache: the plan and
    routing words of the cache lengths, the int8 cache with its scales, and
    the workspace of the split-key merge."""

    def __init__(self, cu_seqlens, hq: int, hkv: int, head_dim: int, template, coverage_bp: int,
                 seed: int = 0, device="cuda"):
        import torch
        self.cu = _host_i32(cu_seqlens)
        self.batch = len(self.cu) - 1
        self.hq, self.hkv, self.d = hq, hkv, head_dim
        self.tokens, self.tq, self.tk = tilemix_query_sizes(self.cu)
        self.plan_h = tilemix_build_plan(self.cu, hq, hkv, head_dim)
        self.plan_d = torch.from_numpy(self.plan_h).to(device)
        self.device = device
        self.words, self.g, self.n_int8, self.n_legal = tilemix_build_routing(
            self.cu, hkv, template, coverage_bp, seed)
        w = self.words if self.words.size else np.zeros((1, 1), dtype=np.uint64)
        self.words_d = torch.from_numpy(w.view(np.int64)).to(device)
        t = max(self.tokens, 1)
        self.k_i8 = torch.empty((t, hkv, head_dim), dtype=torch.int8, device=device)
        self.v_i8 = torch.empty((t, hkv, head_dim), dtype=torch.int8, device=device)
        self.k_scale = torch.empty((hkv, max(self.tk, 1)), dtype=torch.float32, device=device)
        self.v_scale = torch.empty((hkv, max(self.tk, 1)), dtype=torch.float32, device=device)
        self.workspace = torch.empty(max(tilemix_decode_workspace_size(self.plan_h), 16),
                                     dtype=torch.uint8, device=device)

    def fill_cache(self, k, v, stream=None):
        """Quantise fp16 K, V [T, Hkv, d] into the INT8 cache."""
        tilemix_quantize_kv(self.plan_h, self.plan_d, k, v, self.k_i8, self.v_i8, self.k_scale,
                            self.v_scale, stream)

    def step(self, q, out=None, stream=None, noalloc: bool = False):
        """q: fp16 [B, Hq, d], the newest query of each sequence.  With
        ``noalloc`` the step keeps its partial records in the library's static
        scratch instead of ``self.workspace`` (the same output)."""
        import torch
        if out is None:
            out = torch.empty((self.batch, self.hq, self.d), dtype=torch.float16, device=q.device)
        if noalloc:
            tilemix_decode_varlen_noalloc(self.plan_h, self.plan_d, q, self.k_i8, self.v_i8, self.k_scale,
                                          self.v_scale, self.words_d, out, stream)
        else:
            tilemix_decode_varlen(self.plan_h, self.plan_d, q, self.k_i8, self.v_i8, self.k_scale,
                                  self.v_scale, self.words_d, self.workspace, out, stream)
        return out


class TileMixStack:
    """A synthetic stack of attention + residual layers over one packed batch
    shape: the plan and routing words (one template for every layer), the
    layers' weights on the device and one layer's workspace."""

    def __init__(self, cu_seqlens, hq: int, hkv: int, head_dim: int, template, coverage_bp: int,
                 seed: int = 0, eps: float = 1e-6, device="cuda"):
        import torch
        self.cu = _host_i32(cu_seqlens)
        self.hq, self.hkv, self.d = hq, hkv, head_dim
        self.eps = eps
        self.device = device
        self.tokens, self.tq, self.tk = tilemix_query_sizes(self.cu)
        self.plan_h = tilemix_build_plan(self.cu, hq, hkv, head_dim)
        self.plan_d = torch.from_numpy(self.plan_h).to(device)
        self.set_routing(template, coverage_bp, seed)
        self.workspace = torch.empty(max(tilemix_stack_workspace_size(self.plan_h), 16),
                                     dtype=torch.uint8, device=device)
        self.wqkv = self.wo = None

    def set_routing(self, template, coverage_bp: int, seed: int = 0):
        import torch
        self.words, self.g, self.n_int8, self.n_legal = tilemix_build_routing(
            self.cu, self.hkv, template, coverage_bp, seed)
        w = self.words if self.words.size else np.zeros((1, 1), dtype=np.uint64)
        self.words_d = torch.from_numpy(w.view(np.int64)).to(self.device)

    def set_weights(self, wqkv, wo):
        """wqkv: fp16 [layers, Hkv, W + 2d, W]; wo: fp16 [layers, Hkv, W, W]
        (device tensors, kept by reference)."""
        self.wqkv, self.wo = wqkv, wo

    @property
    def layers(self) -> int:
        return 0 if self.wqkv is None else self.wqkv.shape[0]

    def layer(self, x, l: int, stream=None):
        """Layer l in place on x (fp32 [T, Hq*d])."""
        tilemix_stack_layer(self.plan_h, self.plan_d, self.words_d, x, self.wqkv[l], self.wo[l], self.eps,
                            self.workspace, stream)

    def forward(self, x, record=None, stream=None):
        """Run every layer in place on x; returns {depth: copy of x} for the
        depths (1-based) listed in ``record``."""
        snaps = {}
        for l in range(self.layers):
            self.layer(x, l, stream)
            if record is not None and l + 1 in record:
                snaps[l + 1] = x.clone()
        return snaps
