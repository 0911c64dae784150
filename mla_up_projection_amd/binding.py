"""Thin ctypes binding of libmlaqup.so (include/mla_qup.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C entry point of the same name, and raises on any status other than
MLA_OK. Nothing here computes any part of the operation, and there is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p

import torch  # imported before the library so both share torch's HIP runtime

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmlaqup.so")

MLA_FWD_FP8_MFMA = 1
MLA_OK, MLA_EINVAL, MLA_EROPE_TABLE, MLA_EALIAS, MLA_EUNSUPPORTED, MLA_EDEVICE, MLA_EWORKSPACE = range(7)
DTYPE_BF16, DTYPE_FP32, DTYPE_MXFP8 = 0, 1, 2
FMT_BSHD, FMT_SBHD, FMT_THD = 0, 1, 2

FUNCTIONS = ("rope_cache_build", "mxfp8_quantize", "mxfp8_quantize_t", "mla_qup_fwd", "mla_qup_bwd",
             "mla_qup_bwd_workspace_size", "mla_qup_bwd_mxfp8", "mla_qup_bwd_mxfp8_workspace_size",
             "mla_kv_rope", "mla_status_str")


class mla_tokens(Structure):
    _fields_ = [("fmt", c_int32), ("B", c_int32), ("S", c_int32), ("T", c_int64),
                ("cu_seqlens", c_void_p), ("nseq", c_int32), ("max_seqlen", c_int32)]


class mla_yarn(Structure):
    _fields_ = [("factor", c_double), ("orig_max_pos", c_int32), ("beta_fast", c_double),
                ("beta_slow", c_double), ("mscale", c_double)]


class mla_rope(Structure):
    _fields_ = [("cos", c_void_p), ("sin", c_void_p), ("rows", c_int32), ("pairs", c_int32)]


class mla_qup_fwd_args(Structure):
    _fields_ = [("x", c_void_p), ("x_scales", c_void_p), ("x_dtype", c_int32),
                ("w", c_void_p), ("w_scales", c_void_p), ("w_dtype", c_int32),
                ("bias", c_void_p), ("K", c_int32), ("H", c_int32), ("d_nope", c_int32),
                ("d_rope", c_int32), ("tokens", mla_tokens), ("rope", mla_rope),
                ("out_dtype", c_int32), ("out", c_void_p), ("out_scales", c_void_p),
                ("flags", c_int32)]


class mla_kv_args(Structure):
    _fields_ = [("kv", c_void_p), ("k_pe", c_void_p), ("H", c_int32), ("d_nope", c_int32),
                ("d_rope", c_int32), ("d_v", c_int32), ("tokens", mla_tokens), ("rope", mla_rope),
                ("out_dtype", c_int32), ("key", c_void_p), ("key_scales", c_void_p),
                ("value", c_void_p), ("value_scales", c_void_p)]


class mla_qup_bwd_args(Structure):
    _fields_ = [("dq", c_void_p), ("x", c_void_p), ("w", c_void_p), ("K", c_int32),
                ("H", c_int32), ("d_nope", c_int32), ("d_rope", c_int32),
                ("tokens", mla_tokens), ("rope", mla_rope), ("dq_pre", c_void_p),
                ("dx", c_void_p), ("dw", c_void_p), ("dw_dtype", c_int32),
                ("use_bias", c_int32), ("db", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmlaqup.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mla_up_projection_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.rope_cache_build.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_double,
                                       POINTER(mla_yarn), c_void_p]
        L.mxfp8_quantize.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int64, c_void_p,
                                     c_void_p, c_void_p]
        L.mxfp8_quantize_t.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_int64, c_void_p,
                                       c_void_p, c_void_p]
        L.mla_qup_fwd.argtypes = [POINTER(mla_qup_fwd_args), c_void_p]
        L.mla_qup_bwd.argtypes = [POINTER(mla_qup_bwd_args), c_void_p]
        L.mla_qup_bwd_workspace_size.argtypes = [POINTER(mla_qup_bwd_args)]
        L.mla_qup_bwd_workspace_size.restype = c_size_t
        L.mla_qup_bwd_mxfp8.argtypes = [POINTER(mla_qup_bwd_args), c_int32, c_void_p]
        L.mla_qup_bwd_mxfp8_workspace_size.argtypes = [POINTER(mla_qup_bwd_args)]
        L.mla_qup_bwd_mxfp8_workspace_size.restype = c_size_t
        L.mla_kv_rope.argtypes = [POINTER(mla_kv_args), c_void_p]
        L.mla_status_str.argtypes = [c_int32]
        L.mla_status_str.restype = c_char_p
        for f in ("rope_cache_build", "mxfp8_quantize", "mxfp8_quantize_t", "mla_qup_fwd", "mla_qup_bwd",
                  "mla_qup_bwd_mxfp8", "mla_kv_rope"):
            getattr(L, f).restype = c_int32
        _lib = L
    return _lib


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mla_status_str(status)}")
        self.status = status


def mla_status_str(status: int) -> str:
    return lib().mla_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmlaqup must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tokens(T, fmt, B, S, cu_seqlens, max_seqlen) -> mla_tokens:
    tk = mla_tokens()
    tk.fmt = fmt
    tk.T = T
    if fmt == FMT_THD:
        tk.B, tk.S = 1, T
        tk.cu_seqlens = _ptr(cu_seqlens)
        tk.nseq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 0
        tk.max_seqlen = int(max_seqlen) if max_seqlen is not None else 0
    else:
        tk.B = B
        tk.S = S if S is not None else (T // B if B else 0)
    return tk


def _rope(cos, sin, d_rope) -> mla_rope:
    r = mla_rope()
    if cos is not None:
        r.cos, r.sin = _ptr(cos), _ptr(sin)
        r.rows = cos.shape[0]
        r.pairs = cos.shape[1] if cos.dim() == 2 else d_rope // 2
    return r


def _yarn(yarn) -> mla_yarn | None:
    if yarn is None:
        return None
    y = mla_yarn()
    y.factor, y.orig_max_pos, y.beta_fast, y.beta_slow, y.mscale = yarn
    return y


# ------------------------------------------------------------- entry points --
def rope_cache_build(cos, sin, d_rope: int, base: float = 10000.0, yarn=None, stream=None):
    """Fill fp32 device tables cos/sin [rows, d_rope/2]; yarn = (factor, L,
    beta_fast, beta_slow, mscale) or None."""
    y = _yarn(yarn)
    st = lib().rope_cache_build(_ptr(cos), _ptr(sin), cos.shape[0], d_rope, float(base),
                                ctypes.byref(y) if y is not None else None, _stream(stream))
    _check(st, "rope_cache_build")


def mxfp8_quantize(x, codes, scales, stream=None):
    """x [rows, cols] bf16/fp32 (row stride may exceed cols) -> codes uint8
    [rows, cols], scales uint8 [rows, cols/32]."""
    if x.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    dt = DTYPE_FP32 if x.dtype == torch.float32 else DTYPE_BF16 if x.dtype == torch.bfloat16 else -1
    st = lib().mxfp8_quantize(x.data_ptr(), dt, x.shape[0], x.shape[1], x.stride(0),
                              _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "mxfp8_quantize")


def mxfp8_quantize_t(x, codes_t, scales_t, rows_pad=None, stream=None):
    """x bf16 [rows, cols] (row stride may exceed cols) -> codes_t uint8
    [cols, rows_pad], scales_t uint8 [cols, rows_pad/32]: quantized along the
    columns, stored transposed; rows_pad defaults to codes_t.shape[1]."""
    if x.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    rp = codes_t.shape[1] if rows_pad is None else rows_pad
    st = lib().mxfp8_quantize_t(x.data_ptr(), x.shape[0], x.shape[1], x.stride(0), rp,
                                _ptr(codes_t), _ptr(scales_t), _stream(stream))
    _check(st, "mxfp8_quantize_t")


def make_fwd_args(x, w, out, *, H, d_nope, d_rope, cos=None, sin=None, x_scales=None,
                  w_scales=None, bias=None, out_scales=None, fmt=FMT_BSHD, B=1, S=None,
                  cu_seqlens=None, max_seqlen=None, fp8_mfma=False) -> mla_qup_fwd_args:
    a = mla_qup_fwd_args()
    a.flags = MLA_FWD_FP8_MFMA if fp8_mfma else 0
    mx_in = x.dtype == torch.uint8
    a.x, a.x_scales, a.x_dtype = _ptr(x), _ptr(x_scales), DTYPE_MXFP8 if mx_in else DTYPE_BF16
    a.w, a.w_scales = _ptr(w), _ptr(w_scales)
    a.w_dtype = DTYPE_MXFP8 if w.dtype == torch.uint8 else DTYPE_BF16
    a.bias = _ptr(bias)
    a.K, a.H, a.d_nope, a.d_rope = x.shape[1], H, d_nope, d_rope
    a.tokens = _tokens(x.shape[0], fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(cos, sin, d_rope)
    a.out_dtype = DTYPE_MXFP8 if out.dtype == torch.uint8 else DTYPE_BF16
    a.out, a.out_scales = _ptr(out), _ptr(out_scales)
    return a


def mla_qup_fwd(x, w, out, *, stream=None, **kw):
    """Fused forward. x: bf16 [T,K] or uint8 codes with x_scales; w likewise
    [N,K]; out: bf16 or uint8 BHSD [B,H,S,D] (THD: [1,H,T,D]); out_scales
    uint8 [.., D/32] for MXFP8 output. fp8_mfma=True puts MXFP8 operands on
    the scaled FP8 MFMA (faster, lower accumulation precision)."""
    a = make_fwd_args(x, w, out, **kw)
    _check(lib().mla_qup_fwd(ctypes.byref(a), _stream(stream)), "mla_qup_fwd")


def make_bwd_args(dq, x, w, dq_pre, *, H, d_nope, d_rope, cos=None, sin=None, dx=None, dw=None,
                  db=None, use_bias=False, workspace=None, fmt=FMT_BSHD, B=1, S=None,
                  cu_seqlens=None, max_seqlen=None) -> mla_qup_bwd_args:
    a = mla_qup_bwd_args()
    a.dq, a.x, a.w = _ptr(dq), _ptr(x), _ptr(w)
    a.K, a.H, a.d_nope, a.d_rope = x.shape[1], H, d_nope, d_rope
    a.tokens = _tokens(x.shape[0], fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(cos, sin, d_rope)
    a.dq_pre, a.dx, a.dw = _ptr(dq_pre), _ptr(dx), _ptr(dw)
    a.dw_dtype = DTYPE_FP32 if (dw is not None and dw.dtype == torch.float32) else DTYPE_BF16
    a.use_bias = 1 if use_bias else 0
    a.db = _ptr(db)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return a


def mla_qup_bwd_workspace_size(dq, x, w, dq_pre, **kw) -> int:
    kw.pop("stream", None)
    a = make_bwd_args(dq, x, w, dq_pre, **kw)
    return int(lib().mla_qup_bwd_workspace_size(ctypes.byref(a)))


def mla_qup_bwd(dq, x, w, dq_pre, *, stream=None, **kw):
    """Backward. dq bf16 [T,H,D], x bf16 [T,K], w bf16 [N,K] -> dq_pre bf16
    [T,N], dx bf16 [T,K] (optional), dw bf16/fp32 [N,K] (optional), db bf16
    [N] (use_bias). workspace: uint8 device tensor of at least
    mla_qup_bwd_workspace_size() bytes (None if that is 0)."""
    a = make_bwd_args(dq, x, w, dq_pre, **kw)
    _check(lib().mla_qup_bwd(ctypes.byref(a), _stream(stream)), "mla_qup_bwd")


def mla_qup_bwd_mxfp8_workspace_size(dq, x, w, dq_pre, **kw) -> int:
    kw.pop("stream", None)
    kw.pop("fp8_mfma", None)
    a = make_bwd_args(dq, x, w, dq_pre, **kw)
    return int(lib().mla_qup_bwd_mxfp8_workspace_size(ctypes.byref(a)))


def mla_qup_bwd_mxfp8(dq, x, w, dq_pre, *, fp8_mfma=False, stream=None, **kw):
    """MXFP8 backward: arguments and outputs as mla_qup_bwd; the dx and dw
    products take MXFP8 operands quantized along their reduction axes.
    workspace: at least mla_qup_bwd_mxfp8_workspace_size() bytes."""
    a = make_bwd_args(dq, x, w, dq_pre, **kw)
    _check(lib().mla_qup_bwd_mxfp8(ctypes.byref(a), 1 if fp8_mfma else 0, _stream(stream)),
           "mla_qup_bwd_mxfp8")


def mla_kv_rope(kv, k_pe, key, value, *, H, d_nope, d_rope, d_v, cos=None, sin=None,
                key_scales=None, value_scales=None, fmt=FMT_BSHD, B=1, S=None, cu_seqlens=None,
                max_seqlen=None, stream=None):
    """KV side: kv bf16 [T,H,d_nope+d_v], k_pe bf16 [T,d_rope] -> key [B,H,S,d_nope+d_rope]
    and value [B,H,S,d_v] (BHSD; THD: B=1, S=T), bf16 or uint8 E4M3 codes with
    key_scales / value_scales uint8 [.., D/32]."""
    a = mla_kv_args()
    a.kv, a.k_pe = _ptr(kv), _ptr(k_pe)
    a.H, a.d_nope, a.d_rope, a.d_v = H, d_nope, d_rope, d_v
    a.tokens = _tokens(kv.shape[0], fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(cos, sin, d_rope)
    a.out_dtype = DTYPE_MXFP8 if key.dtype == torch.uint8 else DTYPE_BF16
    a.key, a.key_scales, a.value, a.value_scales = _ptr(key), _ptr(key_scales), _ptr(value), _ptr(value_scales)
    _check(lib().mla_kv_rope(ctypes.byref(a), _stream(stream)), "mla_kv_rope")
