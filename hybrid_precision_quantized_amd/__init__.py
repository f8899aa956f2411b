"""Python binding of libhq.so, the HyQuant hybrid-precision attention library
for AMD Instinct MI355X (gfx950).

Argument marshalling only: every function forwards torch tensors' device
pointers and plain sizes to the C ABI declared in include/hq.h (same names,
same argument order apart from dtypes, which are taken from the tensors).
PyTorch provides device memory and the current HIP stream; all computation
runs in the library's HIP kernels. There is no fallback: if libhq.so is
missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhq.so")

HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_WORKSPACE, HQ_ERR_HIP = range(5)
HQ_F32, HQ_BF16, HQ_F16 = 0, 1, 2
HQ_LAYOUT_ROWS, HQ_LAYOUT_TILE16 = 0, 1
HQ_DETECT_MATMUL, HQ_DETECT_QSUM = 0, 1
HQ_KV_DROP_INT4 = 1

_DT = {torch.float32: HQ_F32, torch.bfloat16: HQ_BF16, torch.float16: HQ_F16}


class HQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hq status {status}: {message}")
        self.status = status


class HybridKV(ctypes.Structure):
    """Mirror of hq_hybrid_kv (include/hq.h)."""
    _fields_ = [
        ("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("D", ctypes.c_int), ("group", ctypes.c_int),
        ("T", ctypes.c_int64), ("W", ctypes.c_int), ("k", ctypes.c_int), ("t_cap", ctypes.c_int64),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_sz", ctypes.c_void_p), ("v_sz", ctypes.c_void_p),
        ("vl_bits", ctypes.c_void_p),
        ("vl_k", ctypes.c_void_p), ("vl_v", ctypes.c_void_p),
        ("win_k", ctypes.c_void_p), ("win_v", ctypes.c_void_p),
        ("win_offset", ctypes.c_int), ("hp_dtype", ctypes.c_int), ("flags", ctypes.c_int),
        ("win_cap", ctypes.c_int),
    ]


_lib_handle = None

_SIGS = {
    "hq_quantize_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p]),
    "hq_quantize_kv_pair": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_void_p]),
    "hq_gather_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "hq_vl_bitmap": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "hq_detect_vlines": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int), ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "hq_detect_vlines_cache": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                              ctypes.POINTER(HybridKV), ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int),
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "hq_detect_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int]),
    "hq_detect_vlines_mass": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int), ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]),
    "hq_detect_mass_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_int64, ctypes.c_int64]),
    "hq_decode_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(HybridKV), ctypes.c_float, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]),
    "hq_decode_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(HybridKV), ctypes.c_float, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p]),
    "hq_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HybridKV), ctypes.c_int, ctypes.c_int]),
    "hq_decode_attn_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                              ctypes.POINTER(HybridKV), ctypes.c_float, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "hq_vl_update": (ctypes.c_int, [ctypes.POINTER(HybridKV), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_void_p]),
    "hq_vl_redetect": (ctypes.c_int, [ctypes.POINTER(HybridKV), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]),
    "hq_vl_redetect_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HybridKV)]),
    "hq_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "hq_stream_read_sink_bytes": (ctypes.c_size_t, []),
    "hq_decode_auto_splits": (ctypes.c_int, [ctypes.POINTER(HybridKV), ctypes.c_int]),
    "hq_prefill_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "hq_prefill_attn_i8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "hq_prefill_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int64, ctypes.c_int, ctypes.c_int]),
    "hq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hq_last_error": (ctypes.c_char_p, []),
    "hq_abi_version": (ctypes.c_int, []),
}

EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m hybrid_precision_quantized_amd.build`")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib_handle = h
    return _lib_handle


def library_path() -> str:
    return _LIB_PATH


def _check(status: int) -> None:
    if status != HQ_OK:
        msg = lib().hq_last_error().decode(errors="replace")
        raise HQError(status, msg)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


# ---------------------------------------------------------------- calls
def hq_quantize_kv(x, n_heads, n_rows, D, x_head_stride, x_row_stride, codes, sz, layout,
                   dst_head_rows, dst_row0, group=32, stream=None):
    """Pack rows of x into INT4 codes and fp16 scale/zero (see include/hq.h)."""
    if x.device.type != "cuda":
        raise ValueError("x must live on the GPU")
    _check(lib().hq_quantize_kv(x.data_ptr(), _dt(x), n_heads, n_rows, D, group, x_head_stride,
                                x_row_stride, _ptr(codes), _ptr(sz), layout, dst_head_rows,
                                dst_row0, _stream(stream)))


def hq_quantize_kv_pair(xk, xv, n_heads, n_rows, D, x_head_stride, x_row_stride, k_codes, k_sz,
                        v_codes, v_sz, dst_head_rows, dst_row0, group=32, stream=None):
    """K rows (row layout) and V rows (16-token tiles) in one launch (see include/hq.h)."""
    if xk.device.type != "cuda" or xv.device.type != "cuda":
        raise ValueError("xk and xv must live on the GPU")
    if xk.dtype != xv.dtype:
        raise TypeError("xk and xv must share a dtype")
    _check(lib().hq_quantize_kv_pair(xk.data_ptr(), xv.data_ptr(), _dt(xk), n_heads, n_rows, D, group,
                                     x_head_stride, x_row_stride, _ptr(k_codes), _ptr(k_sz),
                                     _ptr(v_codes), _ptr(v_sz), dst_head_rows, dst_row0,
                                     _stream(stream)))


def hq_gather_rows(src, n_heads, src_rows, D, idx, k, dst, stream=None):
    _check(lib().hq_gather_rows(_ptr(src), _dt(src), n_heads, src_rows, D, _ptr(idx), k,
                                _ptr(dst), _stream(stream)))


def hq_vl_bitmap(vl_idx, n_heads, k, t_cap, bits, stream=None):
    _check(lib().hq_vl_bitmap(_ptr(vl_idx), n_heads, k, t_cap, _ptr(bits), _stream(stream)))


def hq_detect_workspace_size(B, Hkv, cand_end, k_top) -> int:
    return int(lib().hq_detect_workspace_size(B, Hkv, cand_end, k_top))


def hq_detect_vlines(q_new, q_acc, B, Hq, Hkv, D, R, step, force, k, k_rows, cand_end, k_top,
                     method, idx_out, score_out=None, ws=None, stream=None) -> bool:
    """Accumulate q_new into the ring q_acc and, on the last slot or when
    forced, score and select the vertical lines. Returns True if detection
    was enqueued."""
    ran = ctypes.c_int(0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_detect_vlines(_ptr(q_new), _ptr(q_acc), _dt(q_acc), B, Hq, Hkv, D, R, step,
                                  int(force), _ptr(k), k_rows, cand_end, k_top, method,
                                  _ptr(idx_out), _ptr(score_out), ctypes.byref(ran), _ptr(ws),
                                  ws_bytes, _stream(stream)))
    return bool(ran.value)


def hq_detect_vlines_cache(q_new, q_acc, Hq, R, step, force, kv: HybridKV, cand_end, k_top, idx_out,
                           score_out=None, ws=None, stream=None) -> bool:
    """The detector scored from the INT4 key cache described by kv (see
    include/hq.h). Returns True if detection was enqueued."""
    ran = ctypes.c_int(0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_detect_vlines_cache(_ptr(q_new), _ptr(q_acc), _dt(q_acc), Hq, R, step, int(force),
                                        ctypes.byref(kv), cand_end, k_top, _ptr(idx_out), _ptr(score_out),
                                        ctypes.byref(ran), _ptr(ws), ws_bytes, _stream(stream)))
    return bool(ran.value)


def hq_detect_mass_workspace_size(B, Hq, Hkv, R, k_rows, cand_end) -> int:
    return int(lib().hq_detect_mass_workspace_size(B, Hq, Hkv, R, k_rows, cand_end))


def hq_detect_vlines_mass(q_new, q_acc, B, Hq, Hkv, D, R, step, force, k, k_rows, cand_end, k_top,
                          idx_out, score_out=None, ws=None, sm_scale=0.0, stream=None) -> bool:
    """The detector scored by attention mass (see include/hq.h). Returns True
    if detection was enqueued."""
    ran = ctypes.c_int(0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_detect_vlines_mass(_ptr(q_new), _ptr(q_acc), _dt(q_acc), B, Hq, Hkv, D, R, step,
                                       int(force), _ptr(k), k_rows, cand_end, k_top, float(sm_scale),
                                       _ptr(idx_out), _ptr(score_out), ctypes.byref(ran), _ptr(ws),
                                       ws_bytes, _stream(stream)))
    return bool(ran.value)


def hq_decode_workspace_size(kv: HybridKV, Hq: int, n_splits: int = 0) -> int:
    return int(lib().hq_decode_workspace_size(ctypes.byref(kv), Hq, n_splits))


def hq_decode_auto_splits(kv: HybridKV, Hq: int) -> int:
    return int(lib().hq_decode_auto_splits(ctypes.byref(kv), Hq))


def hq_decode_attn(q, Hq, kv: HybridKV, sm_scale, n_splits, out, lse, ws, stream=None):
    """One decode step over the hybrid cache described by kv (see include/hq.h)."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_decode_attn(_ptr(q), _dt(q), Hq, ctypes.byref(kv), float(sm_scale),
                                n_splits, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                _stream(stream)))


def hq_decode_attn_noalloc(q, Hq, kv: HybridKV, sm_scale, n_splits, out, lse, stream=None):
    """hq_decode_attn with the split partials in the library's fixed device
    array instead of a workspace (for callers that cannot allocate)."""
    _check(lib().hq_decode_attn_noalloc(_ptr(q), _dt(q), Hq, ctypes.byref(kv), float(sm_scale),
                                        n_splits, _ptr(out), _ptr(lse), _stream(stream)))


HQ_DECODE_SCRATCH_BYTES = 16 << 20


def hq_vl_update(kv: HybridKV, vl_idx, p0, scores, score_stride, stream=None):
    """Apply a re-detection to a rolling cache in place: the k best of the
    current VL set and the positions [p0, T - W) still in the ring (see
    include/hq.h)."""
    _check(lib().hq_vl_update(ctypes.byref(kv), _ptr(vl_idx), int(p0), _ptr(scores), int(score_stride),
                              _stream(stream)))


def hq_vl_redetect_workspace_size(kv: HybridKV) -> int:
    return int(lib().hq_vl_redetect_workspace_size(ctypes.byref(kv)))


def hq_vl_redetect(kv: HybridKV, vl_idx, p0, q_acc, Hq, R, ws, stream=None):
    """A whole re-detection: the summed query ring, the column scores of the
    candidates only (current VL set and [p0, T - W)) from the INT4 keys, and
    the update of hq_vl_update (see include/hq.h)."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_vl_redetect(ctypes.byref(kv), _ptr(vl_idx), int(p0), _ptr(q_acc), _dt(q_acc), int(Hq), int(R),
                                _ptr(ws), ws_bytes, _stream(stream)))


def hq_stream_read(buf, sink, stream=None):
    """One sequential read of the whole tensor `buf` (measurement utility)."""
    _check(lib().hq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def hq_stream_read_sink_bytes() -> int:
    return int(lib().hq_stream_read_sink_bytes())


def hq_decode_step(q, Hq, kv: HybridKV, sm_scale, n_splits, out, lse, ws, q_acc=None, R=64, step=0,
                   evict=False, stream=None):
    """hq_decode_attn plus the step's upkeep: q into the detector ring and the
    window's oldest row into INT4 row T - W (see include/hq.h)."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hq_decode_step(_ptr(q), _dt(q), Hq, ctypes.byref(kv), float(sm_scale),
                                n_splits, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                _ptr(q_acc), int(R), int(step), 1 if evict else 0,
                                _stream(stream)))


def hq_prefill_workspace_size(B, Hq, Hkv, T, D, k_vl) -> int:
    return int(lib().hq_prefill_workspace_size(B, Hq, Hkv, T, D, k_vl))


def hq_prefill_attn(q, k, v, B, Hq, Hkv, T, D, W, vl_idx, k_vl, sm_scale, out, lse, ws, group=32,
                    stream=None, form="split"):
    """Causal hybrid-precision prefill attention (see include/hq.h). form:
    "split" (hq_prefill_attn, split fp16 planes) or "i8" (hq_prefill_attn_i8,
    int8 MFMA over the codes)."""
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share a dtype")
    if form not in ("split", "i8"):
        raise ValueError(f"unknown prefill form {form!r}")
    fn = lib().hq_prefill_attn if form == "split" else lib().hq_prefill_attn_i8
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _dt(q), B, Hq, Hkv, T, D, group, W, _ptr(vl_idx), k_vl,
              float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def hq_status_string(s: int) -> str:
    return lib().hq_status_string(s).decode()


def hq_last_error() -> str:
    return lib().hq_last_error().decode(errors="replace")


def hq_abi_version() -> int:
    return int(lib().hq_abi_version())


from .cache import HybridCache, RollingCache  # noqa: E402,F401
