"""CPU oracle for the weight-only MXFP4 / INT4 decode projections.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
(``bit_weight_only_mxfp4_amd``) never imports it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64 sums, one fp32 rounding
per decoded weight); this module only builds it with gcc and marshals numpy
arrays into it.  Every function documents the passage of the ThinTensor
developer logs (or of the OCP MX v1.0 format definition) it follows in
``oracle.c``.

Parity is pinned for every function here by the CPU tests (decode table
against the OCP values, exact rational brute force, closed forms,
invariants, library routines); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same source with its row loops split over OpenMP threads, for the
# benchmark's CPU timing only (the parity tests use the plain build)
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")

# Plain build: no fast-math, no vector intrinsics, default rounding mode.
GCC_CMD = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]


def _build_one(path: str, extra, force: bool) -> str:
    if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        tmp = path + ".tmp"
        cmd = GCC_CMD[:-3] + list(extra) + ["-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return path


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (and the OpenMP timing build
    liboracle_omp.so) with gcc; returns the plain library's path."""
    _build_one(_LIB_OMP, ["-fopenmp"], force)
    return _build_one(_LIB, [], force)


_libs = {}


def lib(parallel: bool = False) -> ctypes.CDLL:
    """The oracle library (the plain build, or the OpenMP timing build).
    TT_ORACLE_LIB names another build of the same source to load instead of
    the plain one (the sanitizer test runs the pins against an
    AddressSanitizer / UBSan build this way)."""
    if parallel not in _libs:
        override = None if parallel else os.environ.get("TT_ORACLE_LIB")
        if override:
            path = override
        elif parallel:
            path = _build_one(_LIB_OMP, ["-fopenmp"], False)
        else:
            path = build(force=False)
        L = ctypes.CDLL(path)
        P, I64, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        sig = {
            "or_e2m1_value": (D, [ctypes.c_int]),
            "or_e8m0_value": (D, [ctypes.c_int]),
            "or_mxfp4_weight": (ctypes.c_float, [ctypes.c_int, ctypes.c_int]),
            "or_bf16_value": (D, [ctypes.c_uint16]),
            "or_f16_value": (D, [ctypes.c_uint16]),
            "or_f16_from_double": (ctypes.c_uint16, [D]),
            "or_silu": (D, [D]),
            "or_mxfp4_dequantize": (None, [P, P, I64, I64, P]),
            "or_mxfp4_gemv": (None, [P, P, P, I64, I64, P, I64, P, I64, P, P]),
            "or_mxfp4_gateup_swiglu": (None, [P, P, P, P, P, P, I64, I64, P, I64,
                                              P, I64, P, P, P, P, P]),
            "or_moe_route_topk": (None, [P, I64, I64, I64, P, P]),
            "or_moe_gateup_swiglu": (None, [P, P, P, P, P, P, I64, I64, I64, P,
                                            I64, P, I64, P, I64, P, P, P]),
            "or_moe_down_combine": (None, [P, P, P, I64, I64, I64, P, P, P, I64,
                                           I64, P, I64, P, P]),
            "or_mxfp4_quantize": (ctypes.c_int, [P, I64, I64, P, P, P]),
            "or_fp8e4m3_value": (D, [ctypes.c_int]),
            "or_gqa_attention": (None, [P, P, P, I64, I64, I64, I64, I64, D, P, P, P]),
            "or_fp8_gemv": (None, [P, P, I64, I64, P, ctypes.c_int, I64, P, I64, P, P]),
            "or_int4_quantize": (ctypes.c_int, [P, I64, I64, I64, P, P, P]),
            "or_int4_dequantize": (None, [P, P, P, I64, I64, I64, P]),
            "or_int4_gemv": (None, [P, P, P, I64, I64, I64, P, I64, P, I64, P, P]),
            "or_threads": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _libs[parallel] = L
    return _libs[parallel]


def threads(parallel: bool = False) -> int:
    """Threads the oracle's row loops use (1 for the plain build)."""
    return int(lib(parallel).or_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _rows(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


# ---- scalar formats ------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(int(code))


def e8m0_value(e: int) -> float:
    return lib().or_e8m0_value(int(e))


def mxfp4_weight(code: int, e: int) -> np.float32:
    return np.float32(lib().or_mxfp4_weight(int(code), int(e)))


def bf16_value(bits: int) -> float:
    return lib().or_bf16_value(int(bits))


def f16_value(bits: int) -> float:
    return lib().or_f16_value(int(bits))


def f16_from_double(v: float) -> int:
    return int(lib().or_f16_from_double(float(v)))


def silu(z: float) -> float:
    return lib().or_silu(float(z))


# ---- MXFP4 ---------------------------------------------------------------

def mxfp4_dequantize(codes, scales, n, k):
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    out = np.empty((n, k), np.float32)
    lib().or_mxfp4_dequantize(_p(codes), _p(scales), n, k, _p(out))
    return out


def mxfp4_gemv(codes, scales, ps, n, k, x_bf16, rows=None):
    """Returns (y, S), each [batch][nrows] fp64."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    ps = _c(ps, np.float32)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    r, nr = _rows(rows, n)
    y = np.empty((x.shape[0], nr))
    S = np.empty_like(y)
    lib().or_mxfp4_gemv(_p(codes), _p(scales), _p(ps), n, k, _p(x), x.shape[0],
                        _p(r), nr, _p(y), _p(S))
    return y, S


def mxfp4_gateup_swiglu(g, u, inter, hidden, x_bf16, rows=None, parallel=False):
    """g and u are (codes, scales, ps) triples.  Returns a dict with h, g,
    u, Sg, Su, each [batch][nrows] fp64.  parallel=True runs the OpenMP
    timing build of the same loops (same bits)."""
    gc, gs, gp = _c(g[0], np.uint8), _c(g[1], np.uint8), _c(g[2], np.float32)
    uc, us, up = _c(u[0], np.uint8), _c(u[1], np.uint8), _c(u[2], np.float32)
    x = _c(x_bf16, np.uint16).reshape(-1, hidden)
    r, nr = _rows(rows, inter)
    out = {k: np.empty((x.shape[0], nr)) for k in ("h", "g", "u", "Sg", "Su")}
    lib(parallel).or_mxfp4_gateup_swiglu(_p(gc), _p(gs), _p(gp), _p(uc), _p(us), _p(up),
                                 inter, hidden, _p(x), x.shape[0], _p(r), nr,
                                 _p(out["h"]), _p(out["g"]), _p(out["u"]),
                                 _p(out["Sg"]), _p(out["Su"]))
    return out


# ---- routed experts -------------------------------------------------------

def moe_route_topk(logits_bf16, topk):
    lg = _c(logits_bf16, np.uint16)
    batch, n_exp = lg.shape
    if topk > 64:
        raise ValueError("oracle routing supports topk <= 64")
    ids = np.empty((batch, topk), np.int32)
    w = np.empty((batch, topk))
    lib().or_moe_route_topk(_p(lg), batch, n_exp, topk, _p(ids), _p(w))
    return ids, w


def moe_gateup_swiglu(g_bank, u_bank, n_exp, inter, hidden, x_bf16, ids,
                      rows=None):
    """Banks are (codes[E][I][H/2], scales[E][I][H/32], ps[E][I]).  Returns
    (h, Sg, Su), each [batch][topk][nrows]."""
    gc, gs, gp = (_c(g_bank[0], np.uint8), _c(g_bank[1], np.uint8),
                  _c(g_bank[2], np.float32))
    uc, us, up = (_c(u_bank[0], np.uint8), _c(u_bank[1], np.uint8),
                  _c(u_bank[2], np.float32))
    x = _c(x_bf16, np.uint16).reshape(-1, hidden)
    ids = _c(ids, np.int32)
    batch, topk = ids.shape
    r, nr = _rows(rows, inter)
    h = np.empty((batch, topk, nr))
    Sg, Su = np.empty_like(h), np.empty_like(h)
    lib().or_moe_gateup_swiglu(_p(gc), _p(gs), _p(gp), _p(uc), _p(us), _p(up),
                               n_exp, inter, hidden, _p(x), batch, _p(ids), topk,
                               _p(r), nr, _p(h), _p(Sg), _p(Su))
    return h, Sg, Su


def moe_down_combine(d_bank, n_exp, hidden, inter, h, ids, w, rows=None):
    """h is [batch][topk][inter] (any float dtype, converted exactly to
    fp64), w is [batch][topk].  Returns (y, S), each [batch][nrows]."""
    dc, ds, dp = (_c(d_bank[0], np.uint8), _c(d_bank[1], np.uint8),
                  _c(d_bank[2], np.float32))
    ids = _c(ids, np.int32)
    batch, topk = ids.shape
    hh = _c(np.asarray(h).astype(np.float64), np.float64).reshape(batch, topk, inter)
    ww = _c(np.asarray(w).astype(np.float64), np.float64).reshape(batch, topk)
    r, nr = _rows(rows, hidden)
    y = np.empty((batch, nr))
    S = np.empty_like(y)
    lib().or_moe_down_combine(_p(dc), _p(ds), _p(dp), n_exp, hidden, inter,
                              _p(hh), _p(ids), _p(ww), batch, topk, _p(r), nr,
                              _p(y), _p(S))
    return y, S


# ---- INT4 ---------------------------------------------------------------

def gqa_attention(q, K, V, hq, hkv, d, tcap, T, scale):
    """Single-token GQA attention (bf16 bit patterns q [hq][d], K and V
    [hkv][tcap][d]).  Returns (out, A, Smax) in fp64: out [hq][d], A =
    sum_t p_t |V| [hq][d], Smax = max_t scale * sum |K q| [hq]."""
    q, K, V = _c(q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    out = np.empty((hq, d), np.float64)
    A = np.empty((hq, d), np.float64)
    Sm = np.empty(hq, np.float64)
    lib().or_gqa_attention(_p(q), _p(K), _p(V), hq, hkv, d, tcap, T, float(scale), _p(out),
                           _p(A), _p(Sm))
    return out, A, Sm


def fp8e4m3_value(code):
    return lib().or_fp8e4m3_value(int(code))


def fp8_gemv(w, scale, n, k, x, rows=None):
    """y[b][r] = scale[r] * sum_k w[r][k] x[b][k] (E4M3 bytes w [n][k];
    x bf16 bit patterns (uint16) or fp32).  Returns (y, S), fp64
    [batch][len(rows) or n]."""
    w = _c(w, np.uint8)
    scale = _c(scale, np.float32)
    x = np.asarray(x)
    if x.dtype.kind == "f":
        x_f32 = 1
    elif x.dtype in (np.uint16, np.int16):
        x_f32 = 0
    else:
        raise TypeError("x must be floating point (fp32 values) or bf16 bit patterns")
    x = _c(x, np.float32 if x_f32 else np.uint16).reshape(-1, k)
    batch = x.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    m = n if r is None else r.size
    y = np.empty((batch, m), np.float64)
    S = np.empty((batch, m), np.float64)
    lib().or_fp8_gemv(_p(w), _p(scale), n, k, _p(x), x_f32, batch, _p(r), m, _p(y), _p(S))
    return y, S


def mxfp4_quantize(w, fit_postscale=True):
    """fp32 [N][K] -> (codes u8[N][K/2], scales u8[N][K/32], ps f32[N] or
    None): the OCP MX shared-exponent rule, then the least-squares row
    postscale when fit_postscale."""
    w = _c(w, np.float32)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, k // 32), np.uint8)
    ps = np.empty(n, np.float32) if fit_postscale else None
    rc = lib().or_mxfp4_quantize(_p(w), n, k, _p(codes), _p(scales), _p(ps))
    if rc != 0:
        raise ValueError("non-finite input")
    return codes, scales, ps


def int4_quantize(w, group=128):
    """Returns (q packed u8[N][K/2], s u16[N][G], z u16[N][G])."""
    w = _c(w, np.float32)
    n, k = w.shape
    if k % 2:
        raise ValueError("K must be even")
    G = (k + group - 1) // group
    q = np.empty((n, k // 2), np.uint8)
    s = np.empty((n, G), np.uint16)
    z = np.empty((n, G), np.uint16)
    rc = lib().or_int4_quantize(_p(w), n, k, group, _p(q), _p(s), _p(z))
    if rc != 0:
        raise OverflowError("INT4 scale overflows binary16")
    return q, s, z


def int4_dequantize(q, s, z, n, k, group=128):
    q, s, z = _c(q, np.uint8), _c(s, np.uint16), _c(z, np.uint16)
    out = np.empty((n, k), np.float32)
    lib().or_int4_dequantize(_p(q), _p(s), _p(z), n, k, group, _p(out))
    return out


def int4_gemv(q, s, z, n, k, group, x_bf16, rows=None):
    q, s, z = _c(q, np.uint8), _c(s, np.uint16), _c(z, np.uint16)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    r, nr = _rows(rows, n)
    y = np.empty((x.shape[0], nr))
    S = np.empty_like(y)
    lib().or_int4_gemv(_p(q), _p(s), _p(z), n, k, group, _p(x), x.shape[0],
                       _p(r), nr, _p(y), _p(S))
    return y, S
