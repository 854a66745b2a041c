"""Seeded synthetic inputs for the decode-projection workloads.

This module is shared by the tests, the benchmark and the smoke check, and by
both sides of every parity comparison.  It holds none of the method's
arithmetic: it only draws random numbers and lays them out in the canonical
formats (packed nibbles, E8M0 bytes, fp32 postscales, bf16 activation bits).
The only rounding here is of the drawn fp32 activations to the bf16 inputs
the method consumes.

The workloads are shaped like the projections of the models the ThinTensor
developer logs run (SmolLM3-3B, Phi-4, gpt-oss-20b); the real checkpoints are
not used -- random codes and scales of the same shapes stand in for them.

Distributions (one numpy Generator per tensor, seeded by
``[seed, workload, layer, tensor, expert]``):
  * activations x: standard normal fp32, rounded to bf16 (nearest-even);
  * FP4 codes: uniform over 0..15 (drawn as uniform bytes, i.e. two
    independent uniform nibbles);
  * E8M0 scale bytes: uniform over 119..125, i.e. 2^-8 .. 2^-2;
  * row postscales: uniform(0.5, 1.5) fp32;
  * router logits: standard normal, rounded to bf16;
  * INT4 source weights: 0.02 * standard normal fp32 (quantized by the caller).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids in the seed sequence
T_X, T_GC, T_GE, T_GP, T_UC, T_UE, T_UP, T_DC, T_DE, T_DP, T_LOGITS, T_INT4W, T_OX = range(13)
T_F8C, T_F8S, T_H = 13, 14, 15

E8M0_LO, E8M0_HI = 119, 125          # 2^-8 .. 2^-2 inclusive


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    hidden: int
    inter: int
    layers: int = 1
    batches: tuple = (1,)
    n_experts: int = 0
    topk: int = 0
    # INT4 attention projections (q heads, kv heads, head dim)
    heads: tuple = ()


TINY = Workload(0, "tiny-gateup-h256-i512", 256, 512)
SMOLLM3 = Workload(1, "smollm3-3b-gateup-h2048-i11008", 2048, 11008, layers=24)
PHI4 = Workload(2, "phi4-14b-h5120-i17920", 5120, 17920, layers=8,
                heads=(40, 10, 128))
GPTOSS = Workload(3, "gpt-oss-20b-moe-h2880-e32-top4", 2880, 2880, layers=24,
                  n_experts=32, topk=4)
BATCHED = Workload(4, "smollm3-3b-gateup-batched", 2048, 11008, layers=24,
                   batches=(1, 4, 8, 16, 32))
ALL = (TINY, SMOLLM3, PHI4, GPTOSS, BATCHED)


def rng(wid: int, layer: int, tensor: int, expert: int = 0, seed: int = 0):
    return np.random.default_rng([seed, wid, layer, tensor, expert])


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bit
    patterns as uint16.  Inputs here are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def activations(wid: int, layer: int, batch: int, hidden: int,
                tensor: int = T_X, seed: int = 0) -> np.ndarray:
    x = rng(wid, layer, tensor, seed=seed).standard_normal((batch, hidden),
                                                           dtype=np.float32)
    return bf16_bits(x)


def mxfp4_matrix(wid: int, layer: int, n: int, k: int, which: str = "gate",
                 expert: int = 0, seed: int = 0):
    """Random canonical MXFP4 matrix: (codes u8[n][k/2], scales u8[n][k/32],
    ps f32[n]).  ``which`` selects the tensor ids (gate / up / down)."""
    assert k % 32 == 0
    tc, te, tp = {"gate": (T_GC, T_GE, T_GP), "up": (T_UC, T_UE, T_UP),
                  "down": (T_DC, T_DE, T_DP)}[which]
    codes = rng(wid, layer, tc, expert, seed).integers(0, 256, (n, k // 2),
                                                       dtype=np.uint8)
    scales = rng(wid, layer, te, expert, seed).integers(
        E8M0_LO, E8M0_HI + 1, (n, k // 32), dtype=np.uint8)
    ps = rng(wid, layer, tp, expert, seed).uniform(0.5, 1.5, n).astype(np.float32)
    return codes, scales, ps


def gateup(w: Workload, layer: int = 0, expert: int = 0, seed: int = 0):
    g = mxfp4_matrix(w.wid, layer, w.inter, w.hidden, "gate", expert, seed)
    u = mxfp4_matrix(w.wid, layer, w.inter, w.hidden, "up", expert, seed)
    return g, u


def expert_bank(w: Workload, layer: int = 0, which: str = "gate",
                n_experts: int | None = None, seed: int = 0):
    """Canonical bank: (codes[E][N][K/2], scales[E][N][K/32], ps[E][N]).
    gate/up banks are [E][inter][hidden]; the down bank is [E][hidden][inter]."""
    E = w.n_experts if n_experts is None else n_experts
    n, k = (w.hidden, w.inter) if which == "down" else (w.inter, w.hidden)
    mats = [mxfp4_matrix(w.wid, layer, n, k, which, e, seed) for e in range(E)]
    return tuple(np.stack([m[i] for m in mats]) for i in range(3))


def router_logits(wid: int, step: int, batch: int, n_experts: int,
                  seed: int = 0) -> np.ndarray:
    lg = rng(wid, step, T_LOGITS, seed=seed).standard_normal(
        (batch, n_experts), dtype=np.float32)
    return bf16_bits(lg)


def int4_source(wid: int, layer: int, n: int, k: int, tensor: int = T_INT4W,
                seed: int = 0) -> np.ndarray:
    return (0.02 * rng(wid, layer, tensor, seed=seed).standard_normal(
        (n, k), dtype=np.float32)).astype(np.float32)


def fp8_matrix(wid: int, layer: int, n: int, k: int, seed: int = 0):
    """FP8 E4M3 codes u8[n][k] drawn uniformly over the finite codes (the
    two NaN patterns are excluded) and row scales U(0.5, 1.5) / 448."""
    c = rng(wid, layer, T_F8C, seed=seed).integers(0, 254, (n, k), dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c).astype(np.uint8)   # skip 0x7F; 0xFF is above
    s = (rng(wid, layer, T_F8S, seed=seed).uniform(0.5, 1.5, n) / 448.0).astype(np.float32)
    return c, s


def swiglu_like(wid: int, layer: int, batch: int, k: int, seed: int = 0) -> np.ndarray:
    """fp32 activations shaped like a gate/up SwiGLU output: silu(a) * b for
    a, b ~ N(0, 1)."""
    g = rng(wid, layer, T_H, seed=seed)
    a = g.standard_normal((batch, k))
    b = g.standard_normal((batch, k))
    return (a / (1.0 + np.exp(-a)) * b).astype(np.float32)


def attention_shapes(w: Workload):
    """(N, K) of the fused QKV projection (q heads, then k, then v, heads
    contiguous) and of the O projection."""
    hq, hkv, d = w.heads
    return (hq * d + 2 * hkv * d, w.hidden), (w.hidden, hq * d)


def random_bits_bf16(gen: np.random.Generator, shape, lo_exp=-20, hi_exp=20):
    """Finite random bf16 patterns with unbiased exponents in [lo_exp, hi_exp]
    (for brute-force tests)."""
    sign = gen.integers(0, 2, shape, dtype=np.uint16)
    expo = gen.integers(lo_exp + 127, hi_exp + 128, shape).astype(np.uint16)
    mant = gen.integers(0, 128, shape, dtype=np.uint16)
    return (sign << np.uint16(15)) | (expo << np.uint16(7)) | mant
