"""CPU pins of the oracle's group quantizers on crafted edge-case groups (ties, signed zeros,
fp16 scale underflow, magnitudes far below fp16 and near its scale limit, constant groups).

Each expected result is written out from the quantizer's definition [P2 = llmdaily.org
"KV-cache quantization -- making long-context inference fit in memory", "From BF16 to INT8,
INT4, or even fewer bits"] with numpy's IEEE float32 arithmetic for the steps the definition fixes in fp32
(the scale m / Q, the difference x - z, the quotient by the stored scale), numpy's float16 cast
for the scale's fp16 storage, and round-half-away-from-zero in exact rational arithmetic
(Python fractions):

  symmetric   s = fp16(fl32(max|x| / Q)),   q = clip(round_half_away(x / s), -Q, Q), u = q + 2^(b-1)
  asymmetric  s = fp16(fl32(fl32(hi - lo) / M)), z = fp16(lo),
              u = clip(round_half_away((x - z) / s), 0, M)
  a scale of 0 gives u = 2^(b-1) (symmetric) or u = 0 (asymmetric).

The tie groups make half-even or round-toward-zero implementations fail; the signed-zero groups
pin the sign of a zero-point of -0.0.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import codec_edges as ce


def _half_away(fr: Fraction) -> int:
    a = abs(fr)
    n = int(a + Fraction(1, 2))  # floor(|y| + 1/2)
    return n if fr >= 0 else -n


def _f16_bits(x: np.float32) -> int:
    return int(np.array([x], np.float32).astype(np.float16).view(np.uint16)[0])


def _f16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def expected_sym(x: np.ndarray, bits: int):
    Q = (1 << (bits - 1)) - 1
    m = np.float32(np.max(np.abs(x)))
    s16 = _f16_bits(np.float32(m / np.float32(Q)))
    sf = _f16_value(s16)
    if sf == 0:
        return s16, [1 << (bits - 1)] * x.size
    sf32 = np.float32(sf)
    u = [max(-Q, min(Q, _half_away(Fraction(float(np.float32(v) / sf32))))) + (1 << (bits - 1))
         for v in x]
    return s16, u


def expected_asym(x: np.ndarray, bits: int):
    M = (1 << bits) - 1
    lo, hi = np.float32(np.min(x)), np.float32(np.max(x))
    if lo == 0 and np.any(np.signbit(x[x == 0])):
        lo = x[np.argmin(x)]  # the group's own zero (all zeros share one sign here)
    s16 = _f16_bits(np.float32(np.float32(hi - lo) / np.float32(M)))
    z16 = _f16_bits(lo)
    sf, zf = _f16_value(s16), _f16_value(z16)
    if sf == 0:
        return s16, z16, [0] * x.size
    sf32, zf32 = np.float32(sf), np.float32(zf)
    u = [max(0, min(M, _half_away(Fraction(float((np.float32(v) - zf32) / sf32))))) for v in x]
    return s16, z16, u


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("scheme", [0, 1])
@pytest.mark.parametrize("kind", ce.KINDS)
def test_oracle_quantizer_on_crafted_groups(orc, bits, scheme, kind):
    rng = np.random.default_rng(100 * bits + 10 * scheme + ce.KINDS.index(kind))
    for _ in range(60):
        n = int(rng.choice([16, 32, 64, 128]))
        x = ce.group(kind, n, bits, scheme, rng)
        if scheme == 0:
            s16, u = orc.quant_sym(x, bits)
            es, eu = expected_sym(x, bits)
            assert s16 == es, (kind, x[:4], hex(s16), hex(es))
            assert list(u) == eu, (kind, x[:8], list(u)[:8], eu[:8])
        else:
            s16, z16, u = orc.quant_asym(x, bits)
            es, ez, eu = expected_asym(x, bits)
            assert (s16, z16) == (es, ez), (kind, hex(s16), hex(es), hex(z16), hex(ez))
            assert list(u) == eu, (kind, x[:8], list(u)[:8], eu[:8])


def test_ties_round_half_away_from_zero(orc):
    """Every non-extreme element of a tie group is an exact half-integer multiple of the scale;
    its code is the integer away from zero (symmetric), or the next integer up (asymmetric:
    quotients are non-negative)."""
    rng = np.random.default_rng(7)
    seen_neg = seen_pos = 0
    for bits in (2, 4, 8):
        Q, M = (1 << (bits - 1)) - 1, (1 << bits) - 1
        for _ in range(50):
            x = ce.group("ties", 64, bits, 0, rng)
            s16, u = orc.quant_sym(x, bits)
            sf = _f16_value(s16)
            for v, c in zip(x, (int(c) for c in u)):
                y = Fraction(float(v)) / sf
                if abs(y) == Q:
                    assert c - (1 << (bits - 1)) == int(y)
                    continue
                assert y.denominator == 2, "not a tie"
                want = int(y + Fraction(1, 2)) if y > 0 else int(y - Fraction(1, 2))
                assert c - (1 << (bits - 1)) == want
                seen_neg += y < 0
                seen_pos += y > 0
            x = ce.group("ties", 32, bits, 1, rng)
            s16, z16, u = orc.quant_asym(x, bits)
            sf, zf = _f16_value(s16), _f16_value(z16)
            for v, c in zip(x, (int(c) for c in u)):
                y = (Fraction(float(v)) - zf) / sf
                if y in (0, M):
                    assert c == int(y)
                    continue
                assert y.denominator == 2
                assert c == int(y + Fraction(1, 2))
    assert seen_neg > 100 and seen_pos > 100


def test_signed_zero_and_underflow_groups(orc):
    """All -0.0: the asymmetric zero-point is fp16 -0.0 (0x8000) with scale 0 and codes 0; the
    symmetric scale is +0 with every code at the offset.  A symmetric scale of exactly 2^-25
    is an fp16 tie between 0 and 2^-24 and rounds to 0 (even)."""
    x = np.full(32, -0.0, np.float32)
    s16, z16, u = orc.quant_asym(x, 2)
    assert (s16, z16, list(u)) == (0, 0x8000, [0] * 32)
    s16, u = orc.quant_sym(x, 4)
    assert (s16, list(u)) == (0, [8] * 32)
    for bits in (2, 4, 8):
        Q = (1 << (bits - 1)) - 1
        x = np.zeros(16, np.float32)
        x[3] = np.float32(Q) * np.float32(2.0 ** -25)
        s16, u = orc.quant_sym(x, bits)
        assert s16 == 0 and list(u) == [1 << (bits - 1)] * 16
        x[3] = np.float32(Q) * np.float32(2.0 ** -25) * np.float32(1 + 2.0 ** -6)
        s16, u = orc.quant_sym(x, bits)
        assert s16 == 1 and int(u[3]) == (1 << (bits - 1)) + min(Q, round(float(x[3]) * 2 ** 24))
