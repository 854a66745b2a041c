"""Weight-only MXFP4 / INT4 single-token decode projections for MI355X.

A thin ctypes binding over ``libtt.so`` (declared in ``include/tt.h``).
Every step of every projection runs in the library's HIP kernels; this module
only checks tensors, allocates outputs with torch and passes raw pointers and
the current torch stream.  There is no fallback: if ``libtt.so`` is missing
the import fails.

Device calls take torch tensors on a ROCm device:
  * packed weights: ``torch.uint8`` tensors holding a pack made by the
    ``pack_*`` functions (host numpy arrays, copied to the device by the
    caller);
  * activations: ``torch.bfloat16`` (or their ``int16`` bit patterns).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtt.so")

TT_F32, TT_BF16 = 0, 1
TT_FMT_MXFP4, TT_FMT_INT4_AFFINE = 0, 1
INT4_GROUP = 128
MAX_BATCH = 32

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_weight_only_mxfp4_amd.build`")

_P, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
_SIGS = {
    "tt_abi_version": (_I32, []),
    "tt_last_error": (ctypes.c_char_p, []),
    "tt_status_str": (ctypes.c_char_p, [_I32]),
    "tt_format_info": (_I32, [_I32, _P, _P, _P, _P]),
    "tt_mxfp4_matrix_pack_bytes": (_I64, [_I64, _I64]),
    "tt_pack_mxfp4_matrix": (_I32, [_P, _P, _P, _I64, _I64, _P, _I64]),
    "tt_mxfp4_gateup_pack_bytes": (_I64, [_I64, _I64]),
    "tt_pack_mxfp4_gateup": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _P, _I64]),
    "tt_quantize_mxfp4": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "tt_quantize_int4_affine": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "tt_int4_pack_bytes": (_I64, [_I64, _I64, _I64]),
    "tt_fp8_pack_bytes": (_I64, [_I64, _I64]),
    "tt_pack_fp8_matrix": (_I32, [_P, _P, _I64, _I64, _P, _I64]),
    "tt_pack_int4": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _I64]),
    "tt_mxfp4_gateup_swiglu": (_I32, [_P, _I64, _I64, _P, _I64, _P, _I32, _P]),
    "tt_moe_route_topk": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "tt_moe_mxfp4_gateup_swiglu": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P,
                                          _I32, _P]),
    "tt_moe_mxfp4_route_gateup_swiglu": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P,
                                                _P, _P, _I32, _P]),
    "tt_moe_mxfp4_down_combine": (_I32, [_P, _I64, _I64, _I64, _P, _I32, _P, _P, _I64,
                                         _I64, _P, _I32, _P]),
    "tt_int4_gemv": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I32, _P]),
    "tt_fp8_gemv": (_I32, [_P, _I64, _I64, _P, _I32, _I64, _P, _I32, _P]),
    "tt_gqa_attention_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64]),
    "tt_gqa_attention_decode": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                        ctypes.c_float, _P, _I32, _P, _I64, _P]),
    "tt_gqa_attention_decode_noalloc": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                                ctypes.c_float, _P, _I32, _P]),
    "tt_mxfp4_dequantize": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "tt_mxfp4_gateup_dequantize": (_I32, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "tt_int4_dequantize": (_I32, [_P, _I64, _I64, _I64, _P, _P]),
    "tt_fp8_dequantize": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "tt_stream_read": (_I32, [_P, _I64, _I32, _P, _P]),
}

# libtt.so needs libamdhip64.so.7.  torch bundles its own HIP runtime under that
# soname; importing torch first makes the loader bind libtt.so to the runtime
# that owns torch's streams and device memory instead of loading a second one.
import torch as _torch_runtime  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args
EXPORTS = tuple(_SIGS)


class TTError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{lib.tt_status_str(status).decode()}: {message}")
        self.status = status


def _check(status):
    if status != 0:
        raise TTError(status, lib.tt_last_error().decode())


def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _host(a, dtype, need=None, name="array"):
    """Contiguous host copy (or view) of ``a``; with ``need``, ``a`` must hold
    at least that many elements (the library reads them through a raw
    pointer and cannot check)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    if need is not None and a.size < need:
        raise ValueError(f"{name} holds {a.size} elements, the call reads {need}")
    return a


def abi_version() -> int:
    return lib.tt_abi_version()


def format_info(fmt: int):
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(lib.tt_format_info(fmt, *[ctypes.byref(v) for v in vals]))
    return dict(zip(("bits", "group", "scale_kind", "has_zero"), (v.value for v in vals)))


# ---- host packers ---------------------------------------------------------

def _size(n):
    if n < 0:
        raise TTError(int(n), lib.tt_last_error().decode())
    return int(n)


def mxfp4_matrix_pack_bytes(n: int, k: int) -> int:
    return _size(lib.tt_mxfp4_matrix_pack_bytes(n, k))


def mxfp4_gateup_pack_bytes(inter: int, hidden: int) -> int:
    return _size(lib.tt_mxfp4_gateup_pack_bytes(inter, hidden))


def int4_pack_bytes(n: int, k: int, group: int = INT4_GROUP) -> int:
    return _size(lib.tt_int4_pack_bytes(n, k, group))


def pack_mxfp4_matrix(codes, scales, ps, n, k, out=None):
    """Canonical MXFP4 (codes u8[n][k/2], scales u8[n][k/32], ps f32[n] or
    None) -> packed uint8 numpy array (or into ``out``)."""
    nbytes = mxfp4_matrix_pack_bytes(n, k)
    c = _host(codes, np.uint8, n * (k // 2), "codes")
    s = _host(scales, np.uint8, n * (k // 32), "scales")
    p = _host(ps, np.float32, n, "ps")
    dst = np.empty(nbytes, np.uint8) if out is None else out
    _check(lib.tt_pack_mxfp4_matrix(_np_ptr(c), _np_ptr(s), _np_ptr(p), n, k, _np_ptr(dst),
                                    dst.nbytes))
    return dst


def pack_mxfp4_gateup(g, u, inter, hidden, out=None):
    """g and u are canonical (codes, scales, ps) triples of [inter][hidden]."""
    nbytes = mxfp4_gateup_pack_bytes(inter, hidden)
    nc, ns = inter * (hidden // 2), inter * (hidden // 32)
    gc, gs = _host(g[0], np.uint8, nc, "gate codes"), _host(g[1], np.uint8, ns, "gate scales")
    uc, us = _host(u[0], np.uint8, nc, "up codes"), _host(u[1], np.uint8, ns, "up scales")
    gp, up = _host(g[2], np.float32, inter, "gate ps"), _host(u[2], np.float32, inter, "up ps")
    dst = np.empty(nbytes, np.uint8) if out is None else out
    _check(lib.tt_pack_mxfp4_gateup(_np_ptr(gc), _np_ptr(gs), _np_ptr(gp), _np_ptr(uc),
                                    _np_ptr(us), _np_ptr(up), inter, hidden, _np_ptr(dst),
                                    dst.nbytes))
    return dst


def fp8_pack_bytes(n: int, k: int) -> int:
    return _size(lib.tt_fp8_pack_bytes(n, k))


def pack_fp8_matrix(codes, scale, n, k, out=None):
    """Canonical FP8 E4M3 codes u8[n][k] and row scales f32[n] (or None) ->
    packed uint8 numpy array (or into ``out``)."""
    nbytes = fp8_pack_bytes(n, k)
    c, sc = _host(codes, np.uint8, n * k, "codes"), _host(scale, np.float32, n, "scale")
    dst = np.empty(nbytes, np.uint8) if out is None else out
    _check(lib.tt_pack_fp8_matrix(_np_ptr(c), _np_ptr(sc), n, k, _np_ptr(dst), dst.nbytes))
    return dst


def quantize_mxfp4(w, fit_postscale: bool = True):
    """fp32 [n][k] -> (codes u8[n][k/2], scales u8[n][k/32], ps f32[n] or
    None): MXFP4 blocks by the OCP shared-exponent rule, then the
    least-squares row postscale when fit_postscale."""
    w = _host(w, np.float32)
    n, k = w.shape
    codes = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, max(k // 32, 1)), np.uint8)
    ps = np.empty(n, np.float32) if fit_postscale else None
    _check(lib.tt_quantize_mxfp4(_np_ptr(w), n, k, _np_ptr(codes), _np_ptr(scales),
                                 _np_ptr(ps) if ps is not None else None))
    return codes, scales, ps


def quantize_int4_affine(w, group: int = INT4_GROUP):
    """fp32 [n][k] -> (q u8[n][k/2], s u16[n][G], z u16[n][G])."""
    w = _host(w, np.float32)
    n, k = w.shape
    G = -(-k // group)
    q = np.empty((n, k // 2), np.uint8)
    s = np.empty((n, G), np.uint16)
    z = np.empty((n, G), np.uint16)
    _check(lib.tt_quantize_int4_affine(_np_ptr(w), n, k, group, _np_ptr(q), _np_ptr(s),
                                       _np_ptr(z)))
    return q, s, z


def pack_int4(q, s, z, n, k, group: int = INT4_GROUP, out=None):
    nbytes = int4_pack_bytes(n, k, group)
    G = -(-k // group)
    q = _host(q, np.uint8, n * (k // 2), "q")
    s, z = _host(s, np.uint16, n * G, "s"), _host(z, np.uint16, n * G, "z")
    dst = np.empty(nbytes, np.uint8) if out is None else out
    _check(lib.tt_pack_int4(_np_ptr(q), _np_ptr(s), _np_ptr(z), n, k, group, _np_ptr(dst),
                            dst.nbytes))
    return dst


# ---- device calls -----------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _same_device(ref, **tensors):
    """Every tensor of a call on ref's device (the call runs on ref's current
    stream; a buffer on another device would be read or written from there)."""
    for name, t in tensors.items():
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {ref.device}")


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return TT_F32
    if dt == torch.bfloat16:
        return TT_BF16
    raise TypeError(f"output dtype {dt} is not float32 or bfloat16")


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _acts(x, name="x"):
    torch = _torch()
    _dev_ptr(x, name, (torch.bfloat16, torch.int16, torch.uint16))
    return x


# The library cannot see buffer sizes (it takes raw pointers), so every size
# is checked here before a call: a short buffer would otherwise become an
# out-of-bounds device access.

def _rows_of(x, k, name="x"):
    """Tokens in x [batch][k]; x must hold a whole number of rows."""
    if k <= 0 or x.numel() % k:
        raise ValueError(f"{name} holds {x.numel()} elements, not a multiple of {k}")
    return x.numel() // k


def _holds(t, n, name):
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _packed(t, nbytes, name, count=1):
    if t.numel() < nbytes * count:
        what = f"{count} packs of {nbytes} bytes" if count > 1 else f"{nbytes} bytes"
        raise ValueError(f"{name} holds {t.numel()} bytes, the call reads {what}")


def mxfp4_gateup_swiglu(w_gu, inter, hidden, x, out=None, out_dtype=None):
    """SwiGLU(gate, up) of a packed gate/up pair for x [batch][hidden] bf16."""
    torch = _torch()
    _acts(x)
    batch = _rows_of(x, hidden)
    _packed(w_gu, mxfp4_gateup_pack_bytes(inter, hidden), "w_gu")
    if out is None:
        out = torch.empty((batch, inter), dtype=out_dtype or torch.float32, device=x.device)
    _holds(out, batch * inter, "out")
    _same_device(x, w_gu=w_gu, out=out)
    _check(lib.tt_mxfp4_gateup_swiglu(_dev_ptr(w_gu, "w_gu", (torch.uint8,)), inter, hidden,
                                      _dev_ptr(x, "x"), batch, _dev_ptr(out, "out"),
                                      _dtype_code(out.dtype), _stream(x)))
    return out


def moe_route_topk(logits, topk, ids=None, w=None):
    torch = _torch()
    _acts(logits, "logits")
    batch, n_exp = logits.shape
    if ids is None:
        ids = torch.empty((batch, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((batch, topk), dtype=torch.float32, device=logits.device)
    _holds(ids, batch * topk, "ids")
    _holds(w, batch * topk, "w")
    _same_device(logits, ids=ids, w=w)
    _check(lib.tt_moe_route_topk(_dev_ptr(logits, "logits"), batch, n_exp, topk,
                                 _dev_ptr(ids, "ids", (torch.int32,)),
                                 _dev_ptr(w, "w", (torch.float32,)), _stream(logits)))
    return ids, w


def moe_mxfp4_gateup_swiglu(bank, n_experts, inter, hidden, x, ids, out=None, out_dtype=None):
    torch = _torch()
    _acts(x)
    batch = _rows_of(x, hidden)
    topk = ids.shape[-1]
    _holds(ids, batch * topk, "ids")
    _packed(bank, mxfp4_gateup_pack_bytes(inter, hidden), "bank", n_experts)
    if out is None:
        out = torch.empty((batch, topk, inter), dtype=out_dtype or torch.float32,
                          device=x.device)
    _holds(out, batch * topk * inter, "h")
    _same_device(x, bank=bank, ids=ids, h=out)
    _check(lib.tt_moe_mxfp4_gateup_swiglu(_dev_ptr(bank, "bank", (torch.uint8,)), n_experts,
                                          inter, hidden, _dev_ptr(x, "x"), batch,
                                          _dev_ptr(ids, "ids", (torch.int32,)), topk,
                                          _dev_ptr(out, "h"), _dtype_code(out.dtype),
                                          _stream(x)))
    return out


def moe_mxfp4_route_gateup_swiglu(bank, n_experts, inter, hidden, x, logits, topk, ids=None,
                                  w=None, out=None, out_dtype=None):
    """Routing fused into the expert gate/up; returns (h, ids, w)."""
    torch = _torch()
    _acts(x)
    _acts(logits, "logits")
    batch = _rows_of(x, hidden)
    _holds(logits, batch * n_experts, "logits")
    _packed(bank, mxfp4_gateup_pack_bytes(inter, hidden), "bank", n_experts)
    if ids is None:
        ids = torch.empty((batch, topk), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((batch, topk), dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((batch, topk, inter), dtype=out_dtype or torch.float32,
                          device=x.device)
    _holds(ids, batch * topk, "ids")
    _holds(w, batch * topk, "w")
    _holds(out, batch * topk * inter, "h")
    _same_device(x, bank=bank, logits=logits, ids=ids, w=w, h=out)
    _check(lib.tt_moe_mxfp4_route_gateup_swiglu(
        _dev_ptr(bank, "bank", (torch.uint8,)), n_experts, inter, hidden, _dev_ptr(x, "x"), batch,
        _dev_ptr(logits, "logits"), topk, _dev_ptr(ids, "ids", (torch.int32,)),
        _dev_ptr(w, "w", (torch.float32,)), _dev_ptr(out, "h"), _dtype_code(out.dtype),
        _stream(x)))
    return out, ids, w


def moe_mxfp4_down_combine(down_bank, n_experts, hidden, inter, h, ids, w, out=None,
                           out_dtype=None):
    torch = _torch()
    batch, topk = ids.shape
    if tuple(h.shape) != (batch, topk, inter):
        raise ValueError(f"h has shape {tuple(h.shape)}, expected {(batch, topk, inter)}")
    _holds(w, batch * topk, "w")
    _packed(down_bank, mxfp4_matrix_pack_bytes(hidden, inter), "down_bank", n_experts)
    if out is None:
        out = torch.empty((batch, hidden), dtype=out_dtype or torch.float32, device=h.device)
    _holds(out, batch * hidden, "y")
    _same_device(h, down_bank=down_bank, ids=ids, w=w, y=out)
    _check(lib.tt_moe_mxfp4_down_combine(
        _dev_ptr(down_bank, "down_bank", (torch.uint8,)), n_experts, hidden, inter,
        _dev_ptr(h, "h", (torch.float32, torch.bfloat16)), _dtype_code(h.dtype),
        _dev_ptr(ids, "ids", (torch.int32,)), _dev_ptr(w, "w", (torch.float32,)), batch, topk,
        _dev_ptr(out, "y"), _dtype_code(out.dtype), _stream(h)))
    return out


def int4_gemv(w_packed, n, k, x, group=INT4_GROUP, out=None, out_dtype=None):
    torch = _torch()
    _acts(x)
    batch = _rows_of(x, k)
    _packed(w_packed, int4_pack_bytes(n, k, group), "w_packed")
    if out is None:
        out = torch.empty((batch, n), dtype=out_dtype or torch.float32, device=x.device)
    _holds(out, batch * n, "y")
    _same_device(x, w_packed=w_packed, y=out)
    _check(lib.tt_int4_gemv(_dev_ptr(w_packed, "w_packed", (torch.uint8,)), n, k, group,
                            _dev_ptr(x, "x"), batch, _dev_ptr(out, "y"),
                            _dtype_code(out.dtype), _stream(x)))
    return out


def fp8_gemv(w_packed, n, k, x, out=None, out_dtype=None):
    """y[b][r] = scale[r] * sum_k w[r][k] x[b][k] for x [batch][k] fp32 or
    bf16 (e.g. the gate/up SwiGLU output h)."""
    torch = _torch()
    _dev_ptr(x, "x", (torch.float32, torch.bfloat16))
    batch = _rows_of(x, k)
    _packed(w_packed, fp8_pack_bytes(n, k), "w_packed")
    if out is None:
        out = torch.empty((batch, n), dtype=out_dtype or torch.float32, device=x.device)
    _holds(out, batch * n, "y")
    _same_device(x, w_packed=w_packed, y=out)
    _check(lib.tt_fp8_gemv(_dev_ptr(w_packed, "w_packed", (torch.uint8,)), n, k,
                           _dev_ptr(x, "x"), _dtype_code(x.dtype), batch, _dev_ptr(out, "y"),
                           _dtype_code(out.dtype), _stream(x)))
    return out


def gqa_attention_workspace_bytes(hq, hkv, d, T) -> int:
    return _size(lib.tt_gqa_attention_workspace_bytes(hq, hkv, d, T))


def gqa_attention_decode(q, k_cache, v_cache, hq, hkv, d, T, scale, out=None, out_dtype=None,
                         workspace=None):
    """Single-token GQA attention: q bf16 [hq][d], k_cache / v_cache bf16
    [hkv][tcap][d] (positions 0..T-1 attended).  ``workspace`` (uint8 device
    tensor) is allocated here when not given."""
    torch = _torch()
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _acts(t, name)
    tcap = k_cache.numel() // (hkv * d)
    _holds(q, hq * d, "q")
    if v_cache.numel() != k_cache.numel() or k_cache.numel() != hkv * tcap * d:
        raise ValueError("k_cache and v_cache must both hold [hkv][tcap][d] elements")
    if out is None:
        out = torch.empty((hq, d), dtype=out_dtype or torch.float32, device=q.device)
    _holds(out, hq * d, "out")
    need = gqa_attention_workspace_bytes(hq, hkv, d, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _same_device(q, k_cache=k_cache, v_cache=v_cache, out=out, workspace=workspace)
    _check(lib.tt_gqa_attention_decode(
        _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), hq, hkv,
        d, tcap, T, float(scale), _dev_ptr(out, "out"), _dtype_code(out.dtype),
        _dev_ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(q)))
    return out


def gqa_attention_decode_noalloc(q, k_cache, v_cache, hq, hkv, d, T, scale, out=None,
                                 out_dtype=None):
    """gqa_attention_decode with the partials in the library's own
    per-device array instead of a workspace (the call allocates nothing on
    the device; ``out`` is allocated here only when not given).  Calls that
    overlap on one device share that array and must be ordered."""
    torch = _torch()
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _acts(t, name)
    tcap = k_cache.numel() // (hkv * d)
    _holds(q, hq * d, "q")
    if v_cache.numel() != k_cache.numel() or k_cache.numel() != hkv * tcap * d:
        raise ValueError("k_cache and v_cache must both hold [hkv][tcap][d] elements")
    if out is None:
        out = torch.empty((hq, d), dtype=out_dtype or torch.float32, device=q.device)
    _holds(out, hq * d, "out")
    _same_device(q, k_cache=k_cache, v_cache=v_cache, out=out)
    _check(lib.tt_gqa_attention_decode_noalloc(
        _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), hq, hkv,
        d, tcap, T, float(scale), _dev_ptr(out, "out"), _dtype_code(out.dtype), _stream(q)))
    return out


def mxfp4_dequantize(packed, n, k):
    torch = _torch()
    _packed(packed, mxfp4_matrix_pack_bytes(n, k), "packed")
    w = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    ps = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _check(lib.tt_mxfp4_dequantize(_dev_ptr(packed, "packed", (torch.uint8,)), n, k,
                                   _dev_ptr(w, "w"), _dev_ptr(ps, "ps"), _stream(packed)))
    return w, ps


def mxfp4_gateup_dequantize(packed, inter, hidden):
    torch = _torch()
    _packed(packed, mxfp4_gateup_pack_bytes(inter, hidden), "packed")
    mk = lambda *s: torch.empty(s, dtype=torch.float32, device=packed.device)  # noqa: E731
    g, u, gp, up = mk(inter, hidden), mk(inter, hidden), mk(inter), mk(inter)
    _check(lib.tt_mxfp4_gateup_dequantize(_dev_ptr(packed, "packed", (torch.uint8,)), inter,
                                          hidden, _dev_ptr(g, "g"), _dev_ptr(u, "u"),
                                          _dev_ptr(gp, "g_ps"), _dev_ptr(up, "u_ps"),
                                          _stream(packed)))
    return g, u, gp, up


def int4_dequantize(packed, n, k, group=INT4_GROUP):
    torch = _torch()
    _packed(packed, int4_pack_bytes(n, k, group), "packed")
    w = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    _check(lib.tt_int4_dequantize(_dev_ptr(packed, "packed", (torch.uint8,)), n, k, group,
                                  _dev_ptr(w, "w"), _stream(packed)))
    return w


def fp8_dequantize(packed, n, k):
    torch = _torch()
    _packed(packed, fp8_pack_bytes(n, k), "packed")
    w = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    sc = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _check(lib.tt_fp8_dequantize(_dev_ptr(packed, "packed", (torch.uint8,)), n, k,
                                 _dev_ptr(w, "w"), _dev_ptr(sc, "scale"), _stream(packed)))
    return w, sc


def stream_read(buf, loads_per_lane=4, sink=None, nbytes=None):
    """Measurement helper: read ``nbytes`` (default: all) of a uint8 device
    tensor with 16-byte loads (the read ceiling of a streaming kernel)."""
    torch = _torch()
    n = buf.numel() if nbytes is None else int(nbytes)
    _holds(buf, n, "buf")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    _same_device(buf, sink=sink)
    _check(lib.tt_stream_read(_dev_ptr(buf, "buf", (torch.uint8,)), n, loads_per_lane,
                              _dev_ptr(sink, "sink"), _stream(buf)))
    return sink


def normalize_device(dev):
    """Accept "cuda", "cuda:N", an int or a torch.device (the ThinTensor
    fix list's device-normalisation item); returns a torch.device."""
    torch = _torch()
    if isinstance(dev, int):
        return torch.device("cuda", dev)
    d = torch.device(dev)
    if d.type != "cuda":
        raise ValueError(f"not a ROCm device: {dev}")
    return torch.device("cuda", d.index if d.index is not None else torch.cuda.current_device())
