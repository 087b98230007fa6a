"""Crafted bf16 inputs that drive the group quantizer into its edge cases.

Each group (the channels of a per-token group, or the tokens of one channel of a per-channel
key group) is filled by one of these kinds, in rotation so that every kind reaches every
position of the layout:

  ties      quotients x / s that are exact half-integers k + 1/2 (positive and negative), with
            the scale an exact fp16 value and every element exact in bf16; the element
            carrying the group's extreme sits at a random position
  zero      all +0.0
  negzero   all -0.0 (a zero-point of -0.0 for asymmetric groups)
  underflow the fp32 scale lands at or just around 2^-25, where fp16 rounding sends it to 0
            or to the smallest subnormal 2^-24
  tiny      magnitudes near 1e-30: finite in bf16, far below fp16's subnormal range
  huge      magnitudes near the fp16 scale limit (scale up to 0.9 * 65504)
  constant  every element equal (max == min: an asymmetric scale of 0)
  random    N(0, 1) scaled by a random power of two

Only the quantizer's integer ranges (Q = 2^(b-1) - 1, M = 2^b - 1) are used, to place the
ties; no code, scale or zero-point is computed here -- the expected bytes come from the
oracle.  Every value is checked to be exactly representable in bf16.
"""
from __future__ import annotations

import numpy as np

D = 128
KINDS = ("ties", "zero", "negzero", "underflow", "tiny", "huge", "constant", "random")


def bf16_exact(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return (bf16_exact(x).view(np.uint32) >> 16).astype(np.uint16)


def _ties(n, bits, scheme, rng):
    if scheme == 0:
        Q = (1 << (bits - 1)) - 1
        mult = 1 if bits == 8 else int(rng.choice([1, 3, 5]))
        sf = np.float32(mult) * np.float32(2.0) ** int(rng.integers(-10, 6))
        k = rng.integers(-Q, Q, size=n)              # x / s = k + 1/2 in [-Q + 1/2, Q - 1/2]
        x = ((2 * k + 1).astype(np.float32) / 2) * sf
        i = int(rng.integers(n))
        x[i] = np.float32(Q * (1 if rng.integers(2) else -1)) * sf  # the extreme: |x| = Q s
        return x
    M = (1 << bits) - 1
    mult = 1 if bits == 8 else int(rng.choice([1, 3, 5]))
    sf = np.float32(mult) * np.float32(2.0) ** int(rng.integers(-10, 4))
    j0 = (M + 1) // 2 if bits == 8 else int(rng.integers(0, M + 1))  # lo = -j0 s
    k = rng.integers(0, M, size=n)                    # (x - lo) / s = k + 1/2
    x = ((2 * (k - j0) + 1).astype(np.float32) / 2) * sf
    i0, i1 = rng.choice(n, size=2, replace=False)
    x[i0] = np.float32(-j0) * sf                      # the minimum
    x[i1] = np.float32(M - j0) * sf                   # the maximum: hi - lo = M s
    return x


def _bf16_round(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16).astype(np.uint32).view(np.float32)


def group(kind: str, n: int, bits: int, scheme: int, rng) -> np.ndarray:
    """n float32 values, exact in bf16, of one crafted group."""
    Q = (1 << (bits - 1)) - 1
    M = (1 << bits) - 1
    if kind == "ties":
        x = _ties(n, bits, scheme, rng)
    elif kind == "zero":
        x = np.zeros(n, np.float32)
    elif kind == "negzero":
        x = np.full(n, -0.0, np.float32)
    elif kind == "underflow":
        # a scale of 2^-25 exactly (fp16 tie between 0 and 2^-24), or just above / below it
        f = float(rng.choice([1.0, 1.0 + 2.0 ** -6, 1.0 - 2.0 ** -7, 3.0]))
        span = (Q if scheme == 0 else M) * 2.0 ** -25 * f
        if scheme == 0:
            x = _bf16_round(rng.uniform(-span, span, n))
            x[int(rng.integers(n))] = _bf16_round(np.float32(span * (1 if rng.integers(2) else -1)))
        else:
            lo = float(_bf16_round(np.float32(rng.choice([0.0, -span, 0.25]))))
            x = _bf16_round(lo + rng.uniform(0, span, n))
            x[0] = lo
    elif kind == "tiny":
        x = _bf16_round(rng.standard_normal(n) * 1e-30)
    elif kind == "huge":
        if scheme == 0:
            m = 65504.0 * Q * rng.uniform(0.2, 0.9)
            x = _bf16_round(rng.uniform(-m, m, n))
        else:
            lo = -65504.0 * rng.uniform(0.0, 0.9)
            rngw = 65504.0 * M * rng.uniform(0.2, 0.9)
            x = _bf16_round(lo + rng.uniform(0, rngw, n))
            x[0] = _bf16_round(np.float32(lo))
    elif kind == "constant":
        x = np.full(n, _bf16_round(np.float32(rng.standard_normal() * 3)), np.float32)
    elif kind == "random":
        x = _bf16_round(rng.standard_normal(n) * 2.0 ** int(rng.integers(-6, 6)))
    else:
        raise ValueError(kind)
    return bf16_exact(x.astype(np.float32))


def crafted_rows(side, T: int, H: int, rng, kinds=KINDS, start: int = 0) -> np.ndarray:
    """float32 [T][H][128] for one side (bits, scheme, axis, group): every group of the layout
    gets a kind, rotating through `kinds` (per-token: groups of channels of one row;
    per-channel: one channel over `group` consecutive tokens, aligned to token 0)."""
    bits, scheme, axis, G = side
    x = np.zeros((T, H, D), np.float32)
    r = start
    if axis == 0:
        for t in range(T):
            for h in range(H):
                for g in range(D // G):
                    x[t, h, g * G:(g + 1) * G] = group(kinds[r % len(kinds)], G, bits, scheme, rng)
                    r += 1
    else:
        assert T % G == 0
        for t0 in range(0, T, G):
            for h in range(H):
                for c in range(D):
                    x[t0:t0 + G, h, c] = group(kinds[r % len(kinds)], G, bits, scheme, rng)
                    r += 1
    return x
