"""Python binding of the MI355X GDPA library (libgdpa.so, C ABI in include/gdpa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C entry points.  PyTorch provides device memory and the
current stream.  The functions keep the C names (gdpa_fwd, gdpa_varlen_fwd,
gdpa_bwd, gdpa_varlen_bwd); outputs are caller-allocated tensors, as in C.
Small helpers (`varlen_forward`, `varlen_backward`, ...) allocate the outputs
with torch and call the same entry points; `GDPAFunction` makes them
differentiable, and `flash_attn_func`, `flash_attn_varlen_func` and
`generalized_dot_product_attention` take the call forms of the GDPA README's
usage examples ("CUTE-DSL" and "Triton").

The library must have been built (`python generalized_attention_amd/build.py`);
importing this module fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdpa.so")

ACT = {
    "identity": 0, "gelu": 1, "gelu_tanh": 2, "gelu_approx": 2, "fast_gelu": 3, "fast_gelu_bf16": 4,
    "relu": 5, "relu2": 6, "relu_squared": 6, "leaky_relu": 7, "silu": 8, "fast_silu": 9,
    "hardswish": 10,
}
MASK = {"none": 0, "causal": 1, "window": 2, "sliding_window": 2}
DTYPE_BF16, DTYPE_FP16, DTYPE_FP8_E4M3, DTYPE_FP32 = 0, 1, 2, 3
STATUS = {0: "GDPA_OK", 1: "GDPA_ERR_INVALID_ARG", 2: "GDPA_ERR_UNSUPPORTED",
          3: "GDPA_ERR_WORKSPACE_TOO_SMALL", 4: "GDPA_ERR_HIP", 5: "GDPA_ERR_DEVICE_WAIT"}

EXPORTED = (
    "gdpa_fwd", "gdpa_varlen_fwd", "gdpa_bwd", "gdpa_varlen_bwd", "gdpa_varlen_bwd_noalloc", "gdpa_varlen_fwd_mxfp8",
    "gdpa_varlen_fwd_mxfp4", "gdpa_varlen_bwd_lowp", "gdpa_varlen_bwd_lowp_workspace_size",
    "gdpa_fwd_workspace_size", "gdpa_varlen_fwd_workspace_size",
    "gdpa_bwd_workspace_size", "gdpa_varlen_bwd_workspace_size",
    "gdpa_status_string", "gdpa_abi_version",
)


class GDPAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python generalized_attention_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    # head dims: head_dim (Q, K) then head_dim_v (V, O)
    lib.gdpa_fwd.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32, I32, I32, I32, I32, F32,
                             I32, I32, I32, F32, F32, P, SZ, P]
    lib.gdpa_varlen_fwd.argtypes = [P, P, P, P, P, P, I32, I32, I32, I64, I64, I32, I32, I32, I32, F32, I32, I32,
                                    I32, I32, F32, I32, I32, I32, F32, F32, P, SZ, P]
    lib.gdpa_varlen_fwd_mxfp8.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I64, I64, I32, I32, I32, F32, I32,
                                          I32, I32, I32, F32, I32, P, SZ, P]
    lib.gdpa_varlen_fwd_mxfp4.argtypes = lib.gdpa_varlen_fwd_mxfp8.argtypes
    lib.gdpa_varlen_bwd_lowp.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I64, I64, I32, I32, I32, F32,
                                         I32, I32, I32, I32, F32, I32, F32, F32, I32, P, SZ, P]
    lib.gdpa_varlen_bwd_lowp.restype = ctypes.c_int
    lib.gdpa_varlen_bwd_lowp_workspace_size.argtypes = [I32, I32, I32, I64, I64, I32, I32, I32, I32, I32]
    lib.gdpa_varlen_bwd_lowp_workspace_size.restype = SZ
    lib.gdpa_bwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32, I32, I32, I32, I32, F32,
                             I32, I32, P, SZ, P]
    lib.gdpa_varlen_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I64, I64, I32, I32, I32, I32, F32,
                                    I32, I32, I32, I32, F32, I32, I32, P, SZ, P]
    lib.gdpa_varlen_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I64, I64, I32, I32, I32, I32,
                                            F32, I32, I32, I32, I32, F32, I32, I32, P]
    for n in ("gdpa_fwd", "gdpa_varlen_fwd", "gdpa_bwd", "gdpa_varlen_bwd"):
        getattr(lib, n).restype = ctypes.c_int
    for n in ("gdpa_fwd_workspace_size", "gdpa_varlen_fwd_workspace_size"):
        getattr(lib, n).argtypes = [I32] * 6
        getattr(lib, n).restype = SZ
    lib.gdpa_bwd_workspace_size.argtypes = [I32] * 7
    lib.gdpa_bwd_workspace_size.restype = SZ
    lib.gdpa_varlen_bwd_workspace_size.argtypes = [I32, I32, I32, I64, I32, I32, I32, I32]
    lib.gdpa_varlen_bwd_workspace_size.restype = SZ
    lib.gdpa_status_string.argtypes = [ctypes.c_int]
    lib.gdpa_status_string.restype = ctypes.c_char_p
    lib.gdpa_abi_version.restype = I32
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(st, where):
    if st != 0:
        raise GDPAError(st, where)


def _act(a):
    return ACT[a] if isinstance(a, str) else int(a)


def _mask(m):
    return MASK[m] if isinstance(m, str) else int(m)


def _qk_dtype(t):
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DTYPE_FP8_E4M3
    if t.dtype == torch.float16:
        return DTYPE_FP16
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _out_dtype(t):
    if t.dtype == torch.float32:
        return DTYPE_FP32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_FP16
    raise TypeError(f"unsupported output dtype {t.dtype}")


def _grad_dtype(dq, dk, dv):
    given = [t for t in (dq, dk, dv) if t is not None]
    if not given:
        return DTYPE_FP32
    kinds = {_out_dtype(t) for t in given}
    if len(kinds) != 1:
        raise TypeError(f"dq, dk and dv must share one dtype, got {[t.dtype for t in given]}")
    return kinds.pop()


def _expect(name, t, shape, device, dtypes=None):
    """Checks that tensor `t` has the layout the C entry points assume
    (contiguous, on `device`, of `shape`, of one of `dtypes`) before any call
    into the library, which takes raw pointers on trust."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {tuple(dtypes)}")


_IN16 = (torch.bfloat16, torch.float16)
_QK = (torch.bfloat16, torch.float16, torch.float8_e4m3fn, torch.uint8)
_OUT = (torch.float32, torch.bfloat16, torch.float16)


def _check_fwd_args(q, k, v, o, jagged):
    dev = q.device
    if jagged:
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("jagged q/k/v are [total, heads, head_dim]")
        _expect("k", k, (k.shape[0], k.shape[1], q.shape[2]), dev, _QK)
        _expect("v", v, (k.shape[0], k.shape[1], v.shape[2]), dev, _IN16)
        _expect("o", o, (q.shape[0], q.shape[1], v.shape[2]), dev, _OUT)
    else:
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("fixed-length q/k/v are [batch, seqlen, heads, head_dim]")
        _expect("k", k, (q.shape[0], k.shape[1], k.shape[2], q.shape[3]), dev, _QK)
        _expect("v", v, (q.shape[0], k.shape[1], k.shape[2], v.shape[3]), dev, _IN16)
        _expect("o", o, (*q.shape[:3], v.shape[-1]), dev, _OUT)
    _expect("q", q, q.shape, dev, _QK)
    if _qk_dtype(q) != _qk_dtype(k):
        raise TypeError(f"q and k must share one dtype, got {q.dtype} and {k.dtype}")


def _check_bwd_args(q, k, v, dout, dq, dk, dv, jagged):
    dev = q.device
    _check_fwd_args(q, k, v, None, jagged)
    if not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise TypeError(f"q, k, v and dout must share one dtype, got {q.dtype}, {k.dtype}, {v.dtype}, {dout.dtype}")
    _expect("dout", dout, (*q.shape[:-1], v.shape[-1]), dev, _IN16)
    _expect("dq", dq, q.shape, dev, _OUT)
    _expect("dk", dk, k.shape, dev, _OUT)
    _expect("dv", dv, v.shape, dev, _OUT)
    if (dk is None) != (dv is None):
        raise ValueError("dk and dv are requested together (both tensors or both None)")


def _check_cu(cu_q, cu_k, device):
    for name, t in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous int32 vector on {device}")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ---------------------------------------------------------------- C-name calls
def gdpa_fwd(q, k, v, o, scale, act="fast_gelu", act_param=0.01, mask="none", window_left=-1,
             window_right=-1, q_descale=1.0, k_descale=1.0):
    """Fixed-length forward: q/o [B, Lq, Hq, D], k/v [B, Lk, Hkv, D]; writes o."""
    _check_fwd_args(q, k, v, o, jagged=False)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    ws, nws = _workspace(_lib.gdpa_fwd_workspace_size(B, Lq, Lk, Hq, Hkv, D), q.device)
    st = _lib.gdpa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Lq, Lk, Hq, Hkv, D, v.shape[-1], float(scale),
                       _mask(mask),
                       window_left, window_right, _act(act), float(act_param), _qk_dtype(q), _qk_dtype(v),
                       _out_dtype(o), float(q_descale), float(k_descale), _ptr(ws), nws, _stream(q.device))
    _check(st, "gdpa_fwd")
    return o


def gdpa_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale,
                    act="fast_gelu", act_param=0.01, mask="none", window_left=-1, window_right=-1,
                    q_descale=1.0, k_descale=1.0):
    """Jagged forward: q/o [total_q, Hq, D], k/v [total_k, Hkv, D], cu_seqlens int32 [B+1]."""
    _check_fwd_args(q, k, v, o, jagged=True)
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    B = cu_seqlens_q.numel() - 1
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    ws, nws = _workspace(_lib.gdpa_varlen_fwd_workspace_size(B, max_seqlen_q, max_seqlen_k, Hq, Hkv, D), q.device)
    st = _lib.gdpa_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
                              int(max_seqlen_q), int(max_seqlen_k), q.shape[0], k.shape[0], Hq, Hkv, D,
                              v.shape[-1], float(scale), _mask(mask), window_left, window_right, _act(act), float(act_param),
                              _qk_dtype(q), _qk_dtype(v), _out_dtype(o), float(q_descale), float(k_descale),
                              _ptr(ws), nws, _stream(q.device))
    _check(st, "gdpa_varlen_fwd")
    return o


def gdpa_varlen_fwd_mxfp8(q, q_scale, k, k_scale, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          scale, act="fast_gelu", act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """Jagged forward with MXFP8 q/k: E4M3 codes [total, heads, D] (uint8 or
    float8_e4m3fn) and E8M0 scales [total, heads, D / 32] (uint8 or
    float8_e8m0fnu), v bf16."""
    _check_fwd_args(q, k, v, o, jagged=True)
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    if _qk_dtype(q) != DTYPE_FP8_E4M3:
        raise TypeError(f"MXFP8 q/k hold E4M3 codes, got {q.dtype}")
    D = q.shape[2]
    if D % 32:
        raise ValueError("MXFP8 head dim must be a multiple of 32")
    _SC = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    _expect("q_scale", q_scale, (q.shape[0], q.shape[1], D // 32), q.device, _SC)
    _expect("k_scale", k_scale, (k.shape[0], k.shape[1], D // 32), q.device, _SC)
    B = cu_seqlens_q.numel() - 1
    Hq, Hkv = q.shape[1], k.shape[1]
    ws, nws = _workspace(_lib.gdpa_varlen_fwd_workspace_size(B, max_seqlen_q, max_seqlen_k, Hq, Hkv, D), q.device)
    st = _lib.gdpa_varlen_fwd_mxfp8(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(o),
                                    _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k),
                                    q.shape[0], k.shape[0], Hq, Hkv, D, float(scale), _mask(mask), window_left,
                                    window_right, _act(act), float(act_param), _out_dtype(o), _ptr(ws), nws,
                                    _stream(q.device))
    _check(st, "gdpa_varlen_fwd_mxfp8")
    return o


def gdpa_varlen_fwd_mxfp4(q, q_scale, k, k_scale, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          scale, act="fast_gelu", act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """Jagged forward with MXFP4 q/k: uint8 [total, heads, D / 2], two E2M1
    elements per byte (element 2 i in the low nibble of byte i), E8M0 scales
    [total, heads, D / 32] (uint8 or float8_e8m0fnu), v bf16 [total, heads_kv, D]."""
    _check_fwd_args(q, k, v, o, jagged=True)
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    if q.dtype != torch.uint8 or k.dtype != torch.uint8:
        raise TypeError(f"MXFP4 q/k are uint8 bytes of E2M1 pairs, got {q.dtype} and {k.dtype}")
    D = 2 * q.shape[2]
    if D != v.shape[2] or D % 32:
        raise ValueError("MXFP4: 2 * q.shape[2] is the head dim, equal to v's and a multiple of 32")
    _SC = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    _expect("q_scale", q_scale, (q.shape[0], q.shape[1], D // 32), q.device, _SC)
    _expect("k_scale", k_scale, (k.shape[0], k.shape[1], D // 32), q.device, _SC)
    B = cu_seqlens_q.numel() - 1
    Hq, Hkv = q.shape[1], k.shape[1]
    ws, nws = _workspace(_lib.gdpa_varlen_fwd_workspace_size(B, max_seqlen_q, max_seqlen_k, Hq, Hkv, D), q.device)
    st = _lib.gdpa_varlen_fwd_mxfp4(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(o),
                                    _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k),
                                    q.shape[0], k.shape[0], Hq, Hkv, D, float(scale), _mask(mask), window_left,
                                    window_right, _act(act), float(act_param), _out_dtype(o), _ptr(ws), nws,
                                    _stream(q.device))
    _check(st, "gdpa_varlen_fwd_mxfp4")
    return o


LOWP = {"fp8": 2, "mxfp8": 4, "mxfp4": 5}


def gdpa_varlen_bwd_lowp(q, q_scale, k, k_scale, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                         max_seqlen_k, scale, qk_format, q_descale=1.0, k_descale=1.0, act="fast_gelu", act_param=0.01,
                         mask="none", window_left=-1, window_right=-1):
    """Jagged backward from 8- or 4-bit q/k (qk_format "fp8": E4M3 codes with
    per-tensor descales, q_scale = k_scale = None; "mxfp8": E4M3 codes with
    E8M0 block scales; "mxfp4": bytes of E2M1 pairs [total, heads, D / 2] with
    E8M0 block scales); v, dout bf16; dq/dk/dv as in gdpa_varlen_bwd."""
    fmt = LOWP[qk_format]
    D = v.shape[2]
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn) or k.dtype != q.dtype:
        raise TypeError(f"8- and 4-bit q/k are uint8 (or float8_e4m3fn) codes, got {q.dtype} and {k.dtype}")
    qcols = D // 2 if qk_format == "mxfp4" else D
    dev = q.device
    _expect("q", q, (q.shape[0], q.shape[1], qcols), dev)
    _expect("k", k, (k.shape[0], k.shape[1], qcols), dev)
    _expect("v", v, (k.shape[0], k.shape[1], D), dev, (torch.bfloat16,))
    _expect("dout", dout, (q.shape[0], q.shape[1], D), dev, (torch.bfloat16,))
    _expect("dq", dq, (q.shape[0], q.shape[1], D), dev, _OUT)
    _expect("dk", dk, (k.shape[0], k.shape[1], D), dev, _OUT)
    _expect("dv", dv, v.shape, dev, _OUT)
    if (dk is None) != (dv is None):
        raise ValueError("dk and dv are requested together (both tensors or both None)")
    _check_cu(cu_seqlens_q, cu_seqlens_k, dev)
    if qk_format == "fp8":
        if q_scale is not None or k_scale is not None:
            raise ValueError("FP8 q/k take per-tensor descales, not block scales")
    else:
        _SC = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
        _expect("q_scale", q_scale, (q.shape[0], q.shape[1], D // 32), dev, _SC)
        _expect("k_scale", k_scale, (k.shape[0], k.shape[1], D // 32), dev, _SC)
    B = cu_seqlens_q.numel() - 1
    Hq, Hkv = q.shape[1], k.shape[1]
    gd = _grad_dtype(dq, dk, dv)
    ws, nws = _workspace(_lib.gdpa_varlen_bwd_lowp_workspace_size(B, max_seqlen_q, max_seqlen_k, q.shape[0],
                                                                  k.shape[0], Hq, Hkv, D, fmt, gd), dev)
    st = _lib.gdpa_varlen_bwd_lowp(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(dout), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q),
                                   int(max_seqlen_k), q.shape[0], k.shape[0], Hq, Hkv, D, float(scale), _mask(mask),
                                   window_left, window_right, _act(act), float(act_param), fmt, float(q_descale),
                                   float(k_descale), gd, _ptr(ws), nws, _stream(dev))
    _check(st, "gdpa_varlen_bwd_lowp")
    return dq, dk, dv


def gdpa_bwd(q, k, v, dout, dq, dk, dv, scale, act="fast_gelu", act_param=0.01, mask="none",
             window_left=-1, window_right=-1):
    """Fixed-length backward; writes dq (may be None) and dk/dv (both may be None)."""
    _check_bwd_args(q, k, v, dout, dq, dk, dv, jagged=False)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    gd = _grad_dtype(dq, dk, dv)
    ws, nws = _workspace(_lib.gdpa_bwd_workspace_size(B, Lq, Lk, Hq, Hkv, D, gd), q.device)
    st = _lib.gdpa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, Lq, Lk, Hq, Hkv,
                       D, v.shape[-1], float(scale), _mask(mask), window_left, window_right, _act(act), float(act_param),
                       _qk_dtype(q), gd, _ptr(ws), nws, _stream(q.device))
    _check(st, "gdpa_bwd")
    return dq, dk, dv


def gdpa_varlen_bwd(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale,
                    act="fast_gelu", act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """Jagged backward; writes dq (may be None) and dk/dv (both may be None)."""
    _check_bwd_args(q, k, v, dout, dq, dk, dv, jagged=True)
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    B = cu_seqlens_q.numel() - 1
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    gd = _grad_dtype(dq, dk, dv)
    ws, nws = _workspace(_lib.gdpa_varlen_bwd_workspace_size(B, max_seqlen_q, max_seqlen_k, q.shape[0], Hq, Hkv, D, gd),
                         q.device)
    st = _lib.gdpa_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k),
                              q.shape[0], k.shape[0], Hq, Hkv, D, v.shape[-1], float(scale), _mask(mask),
                              window_left,
                              window_right, _act(act), float(act_param), _qk_dtype(q), gd, _ptr(ws),
                              nws, _stream(q.device))
    _check(st, "gdpa_varlen_bwd")
    return dq, dk, dv


def gdpa_varlen_bwd_noalloc(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                            scale, act="fast_gelu", act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """Jagged backward that allocates nothing (the library's per-GPU scratch
    array replaces the workspace); same results as gdpa_varlen_bwd."""
    _check_bwd_args(q, k, v, dout, dq, dk, dv, jagged=True)
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    B = cu_seqlens_q.numel() - 1
    Hq, D = q.shape[1], q.shape[2]
    st = _lib.gdpa_varlen_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q),
                                      int(max_seqlen_k), q.shape[0], k.shape[0], Hq, k.shape[1], D, v.shape[-1],
                                      float(scale), _mask(mask), window_left, window_right, _act(act),
                                      float(act_param), _qk_dtype(q), _grad_dtype(dq, dk, dv), _stream(q.device))
    _check(st, "gdpa_varlen_bwd_noalloc")
    return dq, dk, dv


# ------------------------------------------------------ allocating conveniences
def varlen_forward(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                   activation="fast_gelu", out_dtype=torch.float32, **kw):
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    o = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=out_dtype, device=q.device)
    return gdpa_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale,
                           act=activation, **kw)


def varlen_backward(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                    activation="fast_gelu", grad_dtype=torch.float32, **kw):
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    return gdpa_varlen_bwd(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                           scale, act=activation, **kw)


def forward(q, k, v, scale=None, activation="fast_gelu", out_dtype=torch.float32, **kw):
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    o = torch.empty(q.shape[0], q.shape[1], q.shape[2], v.shape[3], dtype=out_dtype, device=q.device)
    return gdpa_fwd(q, k, v, o, scale, act=activation, **kw)


def backward(q, k, v, dout, scale=None, activation="fast_gelu", grad_dtype=torch.float32, **kw):
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    return gdpa_bwd(q, k, v, dout, dq, dk, dv, scale, act=activation, **kw)


# ------------------------------------------------------------------- autograd
def _mask_args(causal, window_size):
    """(causal, window_size=(left, right)) of the flash-attention call form ->
    (mask, window_left, window_right); -1 is an unbounded side."""
    left, right = window_size
    if left >= 0 or right >= 0:
        return "window", int(left), 0 if causal else int(right)
    return ("causal" if causal else "none"), -1, -1


class GDPAFunction(torch.autograd.Function):
    """Differentiable GDPA over the C entry points: forward calls gdpa_fwd /
    gdpa_varlen_fwd, backward calls gdpa_bwd / gdpa_varlen_bwd (gradients in
    the inputs' dtype, dO rounded to it).  cu_seqlens_q is None for the
    fixed-length layout [B, L, H, D]."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, act, act_param,
                mask, window_left, window_right, out_dtype):
        kw = dict(act=act, act_param=act_param, mask=mask, window_left=window_left, window_right=window_right)
        if cu_seqlens_q is None:
            o = torch.empty(*q.shape[:3], v.shape[3], dtype=out_dtype, device=q.device)
            gdpa_fwd(q, k, v, o, scale, **kw)
        else:
            o = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=out_dtype, device=q.device)
            gdpa_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, **kw)
        ctx.save_for_backward(q, k, v, cu_seqlens_q, cu_seqlens_k)
        ctx.args = (max_seqlen_q, max_seqlen_k, scale, kw)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, scale, kw = ctx.args
        do = do.to(q.dtype).contiguous()
        want_q, want_k, want_v = ctx.needs_input_grad[:3]
        dq = torch.empty_like(q) if want_q else None
        dk = torch.empty_like(k) if (want_k or want_v) else None
        dv = torch.empty_like(v) if (want_k or want_v) else None
        if dq is not None or dk is not None:
            if cu_q is None:
                gdpa_bwd(q, k, v, do, dq, dk, dv, scale, **kw)
            else:
                gdpa_varlen_bwd(q, k, v, do, dq, dk, dv, cu_q, cu_k, max_q, max_k, scale, **kw)
        return (dq, dk if want_k else None, dv if want_v else None) + (None,) * 11


def flash_attn_func(q, k, v, softmax_scale=None, causal=False, activation="fast_gelu", window_size=(-1, -1),
                    act_param=0.01, out_dtype=None):
    """The README's fixed-length call form: q [B, Lq, Hq, D], k/v [B, Lk, Hkv, D].
    Returns (out, None): there is no log-sum-exp without a softmax."""
    scale = q.shape[-1] ** -0.5 if softmax_scale is None else softmax_scale
    mask, wl, wr = _mask_args(causal, window_size)
    o = GDPAFunction.apply(q.contiguous(), k.contiguous(), v.contiguous(), None, None, q.shape[1], k.shape[1],
                           float(scale), activation, float(act_param), mask, wl, wr, out_dtype or q.dtype)
    return o, None


def flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                           causal=False, activation="fast_gelu", window_size=(-1, -1), act_param=0.01,
                           out_dtype=None):
    """The README's jagged call form: q [total_q, Hq, D], k/v [total_k, Hkv, D],
    cu_seqlens int32 [B+1].  Returns (out, None)."""
    scale = q.shape[-1] ** -0.5 if softmax_scale is None else softmax_scale
    mask, wl, wr = _mask_args(causal, window_size)
    o = GDPAFunction.apply(q.contiguous(), k.contiguous(), v.contiguous(), cu_seqlens_q.to(torch.int32),
                           cu_seqlens_k.to(torch.int32), int(max_seqlen_q), int(max_seqlen_k), float(scale),
                           activation, float(act_param), mask, wl, wr, out_dtype or q.dtype)
    return o, None


def generalized_dot_product_attention(query, key, value, query_offset, key_offset, max_seq_len_q, max_seq_len_kv,
                                      activation="fast_gelu", scale=None, causal=False, window_size=(-1, -1),
                                      act_param=0.01, out_dtype=None):
    """The README's Triton call form: jagged tensors with query_offset /
    key_offset (the cu_seqlens prefix sums) and max_seq_len_q / max_seq_len_kv."""
    o, _ = flash_attn_varlen_func(query, key, value, query_offset, key_offset, max_seq_len_q, max_seq_len_kv,
                                  softmax_scale=scale, causal=causal, activation=activation,
                                  window_size=window_size, act_param=act_param, out_dtype=out_dtype)
    return o
