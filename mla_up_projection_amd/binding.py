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
(MLA_OK, MLA_EINVAL, MLA_EROPE_TABLE, MLA_EALIAS, MLA_EUNSUPPORTED, MLA_EDEVICE, MLA_EWORKSPACE,
 MLA_ESCRATCH) = range(8)
MLA_BWD_SCRATCH_BYTES = 64 << 20
DTYPE_BF16, DTYPE_FP32, DTYPE_MXFP8 = 0, 1, 2
FMT_BSHD, FMT_SBHD, FMT_THD = 0, 1, 2

FUNCTIONS = ("rope_cache_build", "mxfp8_quantize", "mxfp8_quantize_t", "mla_qup_fwd", "mla_qup_bwd",
             "mla_qup_bwd_workspace_size", "mla_qup_bwd_noalloc", "mla_qup_bwd_mxfp8",
             "mla_qup_bwd_mxfp8_workspace_size", "mla_kv_rope", "mla_status_str")


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
        L.mla_qup_bwd_noalloc.argtypes = [POINTER(mla_qup_bwd_args), c_void_p]
        L.mla_qup_bwd_mxfp8.argtypes = [POINTER(mla_qup_bwd_args), c_int32, c_void_p]
        L.mla_qup_bwd_mxfp8_workspace_size.argtypes = [POINTER(mla_qup_bwd_args)]
        L.mla_qup_bwd_mxfp8_workspace_size.restype = c_size_t
        L.mla_kv_rope.argtypes = [POINTER(mla_kv_args), c_void_p]
        L.mla_status_str.argtypes = [c_int32]
        L.mla_status_str.restype = c_char_p
        for f in ("rope_cache_build", "mxfp8_quantize", "mxfp8_quantize_t", "mla_qup_fwd", "mla_qup_bwd",
                  "mla_qup_bwd_noalloc", "mla_qup_bwd_mxfp8", "mla_kv_rope"):
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


# Device type every tensor argument must live on (the library receives raw
# device pointers and cannot tell a host address from a device one).
DEVICE_TYPE = "cuda"

_BF16, _FP32, _U8, _I32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32


class _Dev:
    """Checks of one call's tensor arguments before any pointer crosses the C
    ABI: every tensor on one device of DEVICE_TYPE, contiguous, of an
    accepted dtype and with the element count the C call will assume."""

    def __init__(self, where: str):
        self.where = where
        self.device = None

    def __call__(self, t, name: str, dtypes, numel=None, min_numel=None) -> int | None:
        if t is None:
            return None
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{self.where}: {name} must be a torch tensor")
        if t.device.type != DEVICE_TYPE:
            raise ValueError(f"{self.where}: {name} is on {t.device}, not on the GPU")
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            raise ValueError(f"{self.where}: {name} is on {t.device}, other arguments on {self.device}")
        if t.dtype not in dtypes:
            raise ValueError(f"{self.where}: {name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.where}: {name} must be contiguous")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{self.where}: {name} has {t.numel()} elements, expected {numel}")
        if min_numel is not None and t.numel() < min_numel:
            raise ValueError(f"{self.where}: {name} has {t.numel()} elements, at least {min_numel} needed")
        return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tokens(chk: _Dev, T, fmt, B, S, cu_seqlens, max_seqlen) -> mla_tokens:
    tk = mla_tokens()
    tk.fmt = fmt
    tk.T = T
    if fmt == FMT_THD:
        tk.B, tk.S = 1, T
        tk.cu_seqlens = chk(cu_seqlens, "cu_seqlens", (_I32,), min_numel=2)
        tk.nseq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 0
        tk.max_seqlen = int(max_seqlen) if max_seqlen is not None else 0
    else:
        tk.B = B
        tk.S = S if S is not None else (T // B if B else 0)
    return tk


def _rope(chk: _Dev, cos, sin, d_rope) -> mla_rope:
    r = mla_rope()
    if cos is not None or sin is not None:
        if cos is None or sin is None or cos.dim() != 2 or cos.shape != sin.shape:
            raise ValueError(f"{chk.where}: cos and sin must be two tables of one shape [rows, pairs]")
        r.cos, r.sin = chk(cos, "cos", (_FP32,)), chk(sin, "sin", (_FP32,))
        r.rows = cos.shape[0]
        r.pairs = cos.shape[1]
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
    chk = _Dev("rope_cache_build")
    if cos.dim() != 2 or cos.shape != sin.shape or cos.shape[1] != d_rope // 2:
        raise ValueError("rope_cache_build: cos and sin must both be [rows, d_rope/2]")
    pc, ps = chk(cos, "cos", (_FP32,)), chk(sin, "sin", (_FP32,))
    st = lib().rope_cache_build(pc, ps, cos.shape[0], d_rope, float(base),
                                ctypes.byref(y) if y is not None else None, _stream(stream))
    _check(st, "rope_cache_build")


def mxfp8_quantize(x, codes, scales, stream=None):
    """x [rows, cols] bf16/fp32 (row stride may exceed cols) -> codes uint8
    [rows, cols], scales uint8 [rows, cols/32]."""
    chk = _Dev("mxfp8_quantize")
    if x.dim() != 2 or x.stride(-1) != 1:
        raise ValueError("mxfp8_quantize: x must be 2-D with contiguous rows")
    rows, cols = x.shape
    # x may be a row-strided view: check it as the rows it spans
    span = x.as_strided(((rows - 1) * x.stride(0) + cols,) if rows else (0,), (1,))
    px = chk(span, "x", (_BF16, _FP32))
    dt = DTYPE_FP32 if x.dtype == torch.float32 else DTYPE_BF16
    pc = chk(codes, "codes", (_U8,), numel=rows * cols)
    psc = chk(scales, "scales", (_U8,), numel=rows * cols // 32)
    st = lib().mxfp8_quantize(px if rows else x.data_ptr(), dt, rows, cols, x.stride(0), pc, psc,
                              _stream(stream))
    _check(st, "mxfp8_quantize")


def mxfp8_quantize_t(x, codes_t, scales_t, rows_pad=None, stream=None):
    """x bf16 [rows, cols] (row stride may exceed cols) -> codes_t uint8
    [cols, rows_pad], scales_t uint8 [cols, rows_pad/32]: quantized along the
    columns, stored transposed; rows_pad defaults to codes_t.shape[1]."""
    chk = _Dev("mxfp8_quantize_t")
    if x.dim() != 2 or x.stride(-1) != 1:
        raise ValueError("mxfp8_quantize_t: x must be 2-D with contiguous rows")
    rows, cols = x.shape
    span = x.as_strided(((rows - 1) * x.stride(0) + cols,) if rows else (0,), (1,))
    px = chk(span, "x", (_BF16,))
    rp = codes_t.shape[1] if rows_pad is None else rows_pad
    pc = chk(codes_t, "codes_t", (_U8,), numel=cols * rp)
    psc = chk(scales_t, "scales_t", (_U8,), numel=cols * rp // 32)
    st = lib().mxfp8_quantize_t(px if rows else x.data_ptr(), rows, cols, x.stride(0), rp, pc, psc,
                                _stream(stream))
    _check(st, "mxfp8_quantize_t")


def make_fwd_args(x, w, out, *, H, d_nope, d_rope, cos=None, sin=None, x_scales=None,
                  w_scales=None, bias=None, out_scales=None, fmt=FMT_BSHD, B=1, S=None,
                  cu_seqlens=None, max_seqlen=None, fp8_mfma=False) -> mla_qup_fwd_args:
    chk = _Dev("mla_qup_fwd")
    a = mla_qup_fwd_args()
    a.flags = MLA_FWD_FP8_MFMA if fp8_mfma else 0
    if x.dim() != 2:
        raise ValueError("mla_qup_fwd: x must be [T, K]")
    T, K = x.shape
    N = H * (d_nope + d_rope)
    mx_in = x.dtype == torch.uint8
    a.x = chk(x, "x", (_BF16, _U8))
    a.x_scales = chk(x_scales, "x_scales", (_U8,), numel=T * K // 32)
    a.x_dtype = DTYPE_MXFP8 if mx_in else DTYPE_BF16
    a.w = chk(w, "w", (_BF16, _U8), numel=N * K)
    a.w_scales = chk(w_scales, "w_scales", (_U8,), numel=N * K // 32)
    a.w_dtype = DTYPE_MXFP8 if w.dtype == torch.uint8 else DTYPE_BF16
    a.bias = chk(bias, "bias", (_BF16,), numel=N)
    a.K, a.H, a.d_nope, a.d_rope = K, H, d_nope, d_rope
    a.tokens = _tokens(chk, T, fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(chk, cos, sin, d_rope)
    a.out_dtype = DTYPE_MXFP8 if out.dtype == torch.uint8 else DTYPE_BF16
    a.out = chk(out, "out", (_BF16, _U8), numel=T * N)
    a.out_scales = chk(out_scales, "out_scales", (_U8,), numel=T * N // 32)
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
    chk = _Dev("mla_qup_bwd")
    a = mla_qup_bwd_args()
    if x.dim() != 2:
        raise ValueError("mla_qup_bwd: x must be [T, K]")
    T, K = x.shape
    N = H * (d_nope + d_rope)
    a.dq = chk(dq, "dq", (_BF16,), numel=T * N)
    a.x = chk(x, "x", (_BF16,))
    a.w = chk(w, "w", (_BF16,), numel=N * K)
    a.K, a.H, a.d_nope, a.d_rope = K, H, d_nope, d_rope
    a.tokens = _tokens(chk, T, fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(chk, cos, sin, d_rope)
    a.dq_pre = chk(dq_pre, "dq_pre", (_BF16,), numel=T * N)
    a.dx = chk(dx, "dx", (_BF16,), numel=T * K)
    a.dw = chk(dw, "dw", (_BF16, _FP32), numel=N * K)
    a.dw_dtype = DTYPE_FP32 if (dw is not None and dw.dtype == torch.float32) else DTYPE_BF16
    a.use_bias = 1 if use_bias else 0
    a.db = chk(db, "db", (_BF16,), numel=N)
    if workspace is not None:
        a.workspace = chk(workspace, "workspace", (_U8,))
        a.workspace_bytes = workspace.numel()
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


def mla_qup_bwd_noalloc(dq, x, w, dq_pre, *, stream=None, **kw):
    """Backward as mla_qup_bwd, with the partial sums in the library's static
    scratch instead of a workspace (nothing is allocated; calls that overlap on
    one GPU race on that scratch). No workspace argument."""
    if kw.get("workspace") is not None:
        raise ValueError("mla_qup_bwd_noalloc takes no workspace")
    a = make_bwd_args(dq, x, w, dq_pre, **kw)
    _check(lib().mla_qup_bwd_noalloc(ctypes.byref(a), _stream(stream)), "mla_qup_bwd_noalloc")


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
    chk = _Dev("mla_kv_rope")
    a = mla_kv_args()
    T = kv.shape[0]
    Dk, Dv = d_nope + d_rope, d_v
    a.kv = chk(kv, "kv", (_BF16,), numel=T * H * (d_nope + d_v))
    a.k_pe = chk(k_pe, "k_pe", (_BF16,), numel=T * d_rope)
    a.H, a.d_nope, a.d_rope, a.d_v = H, d_nope, d_rope, d_v
    a.tokens = _tokens(chk, T, fmt, B, S, cu_seqlens, max_seqlen)
    a.rope = _rope(chk, cos, sin, d_rope)
    out_dt = key.dtype if key is not None else value.dtype
    a.out_dtype = DTYPE_MXFP8 if out_dt == torch.uint8 else DTYPE_BF16
    a.key = chk(key, "key", (out_dt,), numel=T * H * Dk)
    a.value = chk(value, "value", (out_dt,), numel=T * H * Dv)
    a.key_scales = chk(key_scales, "key_scales", (_U8,), numel=T * H * Dk // 32)
    a.value_scales = chk(value_scales, "value_scales", (_U8,), numel=T * H * Dv // 32)
    _check(lib().mla_kv_rope(ctypes.byref(a), _stream(stream)), "mla_kv_rope")
