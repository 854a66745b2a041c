"""Tolerances and comparisons shared by the parity tests.

The bar: every output within 2e-3 of the sum of |w x| magnitudes behind it
(propagated through SwiGLU for the fused call), cosine >= 0.99999 per call,
bf16 outputs with one extra bf16 rounding allowed; decoded weights bit-exact.
"""
import numpy as np
import torch

import oracle

REL = 2e-3
COS_MIN = 0.99999
SILU_LIP = 1.1   # max |silu'(z)| is about 1.0998


def silu_vec(z):
    return np.array([oracle.silu(float(v)) for v in np.ravel(z)]).reshape(np.shape(z))


def h_tol(ref, bf16=False):
    """Bound on |h - h_ref| for h = silu(g) * u, g and u each within
    REL * S of the exact projections."""
    g, u, Sg, Su, h = ref["g"], ref["u"], ref["Sg"], ref["Su"], ref["h"]
    tol = REL * (SILU_LIP * Sg * np.abs(u) + np.abs(silu_vec(g)) * Su) \
        + SILU_LIP * REL * REL * Sg * Su
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(h)
    return tol


def gemv_tol(S, ref, bf16=False):
    tol = REL * S
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    return tol


def cosine(a, b):
    a = np.ravel(a).astype(np.float64)
    b = np.ravel(b).astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(got, ref, tol, what, cos_min=COS_MIN):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(got[ok] - ref[ok])
    t = np.asarray(np.broadcast_to(tol, ref.shape))[ok]
    worst = float((err / np.maximum(t, 1e-300)).max()) if err.size else 0.0
    cos = cosine(got[ok], ref[ok]) if err.size else 1.0
    print(f"{what}: n={err.size} max|err|={err.max() if err.size else 0:.3e} "
          f"max err/tol={worst:.3e} cosine={cos:.9f}")
    assert np.all(err <= t), f"{what}: {int((err > t).sum())} outputs exceed the tolerance"
    assert cos >= cos_min, f"{what}: cosine {cos} < {cos_min}"


def dev_u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def dev_bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


# ---- guard bands around device outputs ---------------------------------------

GUARD = 64   # canary elements before and after an output
_CANARY = {4: 0x7FA5A5A5, 2: 0x7FA5}


def guarded(shape, dtype, dev):
    """An output tensor that is a view into a larger buffer with canary bands
    of GUARD elements on both sides (a NaN bit pattern no kernel writes).
    Returns (view, check); check() asserts both bands are untouched."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device=dev)
    isz = buf.element_size()
    bits = buf.view(torch.int32 if isz == 4 else torch.int16)
    bits.fill_(_CANARY[isz])
    view = buf[GUARD:GUARD + n].view(shape)

    def check():
        torch.cuda.synchronize()
        b = bits.cpu().numpy()
        pat = np.array(_CANARY[isz], dtype=b.dtype)
        assert np.all(b[:GUARD] == pat), "canary before the output was overwritten"
        assert np.all(b[GUARD + n:] == pat), "canary after the output was overwritten"
    return view, check
