"""Pins of the CPU oracle to things other than itself (no GPU).

Each test checks the oracle against what the pages or the mathematics fix: values printed on
the pages (fixtures under tests/golden/, each with its source), closed forms, exhaustive or
brute-force searches, invariants and special cases.

Pages: [P1] chipfoundryservices.com "KV Cache Quantization"; [P2] llmdaily.org "KV-cache
quantization -- making long-context inference fit in memory"; [P3] oh-bug.com "KV Cache
Quantization in Practice: Managing Memory and Throughput for Long-Context Inference".
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng(20261202)


def bf16_values(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return them as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def f16_np(bits) -> np.ndarray:
    """numpy's own binary16 decoder (independent of the oracle's)."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def read_rows(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([float(v) for v in line.split()])
    return rows


# ------------------------------------------------------------------------------------------
# binary16 conversions
# ------------------------------------------------------------------------------------------

def test_f32_to_f16_exhaustive_against_numpy(orc):
    """Every binary32 pattern in [2^-26, 2^16) (and a sample of negatives) rounds exactly as
    numpy's nearest-even float16 cast."""
    lo, hi, step = 0x32800000, 0x47800000, 1 << 24
    bad = 0
    for a in range(lo, hi, step):
        bits = np.arange(a, min(a + step, hi), dtype=np.uint32)
        x = bits.view(np.float32)
        with np.errstate(over="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        bad += int((orc.f32_to_f16_bits(x) != ref).sum())
    assert bad == 0
    neg = (RNG.integers(0, 0x7F800000, 1 << 20, dtype=np.uint64).astype(np.uint32) | 0x80000000)
    x = neg.view(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16_bits(x), ref)


def test_f16_to_f32_all_patterns(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def f16_rne_of_rational(fr: Fraction) -> int:
    """Exact rational -> binary16 bits, nearest-even, positive finite inputs (from the
    definition: count quanta of the binade, round, re-encode)."""
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    qexp = -24 if e < -14 else e - 10
    n = fr / Fraction(2) ** qexp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if qexp == -24:
        return fl
    val = ((e + 15) << 10) + (fl - 1024)
    return min(val, 0x7C00)


def test_scale_is_single_rounding_of_exact_ratio(orc):
    """For bf16 maxima, fp16(fl32(m / Q)) equals the exact m / Q rounded once to fp16."""
    checked = 0
    for ex in range(-20, 9):
        for mant in range(128):
            m = float((1 + mant / 128) * 2.0**ex)
            for bits in (8, 4, 2):
                Q = (1 << (bits - 1)) - 1
                x = np.array([m, -m / 3, m / 7], np.float32)
                s16, _ = orc.quant_sym(bf16_values(x), bits)
                assert s16 == f16_rne_of_rational(Fraction(m) / Q), (m, bits)
                checked += 1
    assert checked == 29 * 128 * 3


# ------------------------------------------------------------------------------------------
# Quantizers: brute-force codebooks, error bounds, extremal codes, exact reconstruction
# [P2, "From BF16 to INT8, INT4, or even fewer bits"]
# ------------------------------------------------------------------------------------------

def random_groups(n_groups, G):
    mags = RNG.choice([1e-3, 1.0, 20.0, 300.0], size=(n_groups, 1))
    x = RNG.standard_normal((n_groups, G)) * mags
    return bf16_values(x.astype(np.float32))


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_sym_codes_equal_brute_force_codebook(orc, bits):
    """q_i = argmin over q in [-Q, Q] of |x_i - s q| (exact fp64), ties away from zero."""
    Q = (1 << (bits - 1)) - 1
    cand = np.arange(-Q, Q + 1, dtype=np.float64)
    for x in random_groups(300, 64):
        s16, u = orc.quant_sym(x, bits)
        sf = float(f16_np(s16))
        q = u.astype(np.int64) - (1 << (bits - 1))
        if sf == 0.0:
            assert not q.any()
            continue
        dist = np.abs(x.astype(np.float64)[:, None] - sf * cand[None, :])
        best = dist.min(axis=1, keepdims=True)
        ties = np.where(dist == best, np.abs(cand)[None, :], -1)
        pick = cand[np.argmax(ties, axis=1)]
        assert np.array_equal(q, pick.astype(np.int64))


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_asym_codes_equal_brute_force_codebook(orc, bits):
    """u_i = argmin over u in [0, M] of |x_i - (z + s u)|, ties upward; elements whose exact
    quotient (x - z) / s lies within 2^-20 of a half-integer are exempt (the fp32 subtraction
    and division may legitimately round across such a tie)."""
    M = (1 << bits) - 1
    cand = np.arange(0, M + 1, dtype=np.float64)
    exempt = 0
    for x in random_groups(300, 32):
        s16, z16, u = orc.quant_asym(x, bits)
        sf, zf = float(f16_np(s16)), float(f16_np(z16))
        assert z16 == int(np.float32(x.min()).astype(np.float16).view(np.uint16))
        if sf == 0.0:
            assert not u.any()
            continue
        xd = x.astype(np.float64)
        dist = np.abs(xd[:, None] - (zf + sf * cand[None, :]))
        best = dist.min(axis=1, keepdims=True)
        ties = np.where(dist == best, cand[None, :], -1)
        pick = cand[np.argmax(ties, axis=1)].astype(np.int64)
        y = (xd - zf) / sf
        near_tie = np.abs(y - np.floor(y) - 0.5) < 2.0**-20
        exempt += int(near_tie.sum())
        assert np.array_equal(u.astype(np.int64)[~near_tie], pick[~near_tie])
    assert exempt < 0.01 * 300 * 32


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_sym_error_bound_and_extremal_code(orc, bits):
    """|x^ - x| <= s/2 for every element (s the stored scale), and the element of largest
    magnitude gets +-Q whenever the stored scale is a normal fp16 number (relative error at
    most 2^-11, so x_max / s stays within Q * 2^-11 < 1/2 of Q)."""
    Q = (1 << (bits - 1)) - 1
    for x in random_groups(2000, 64):
        s16, u = orc.quant_sym(x, bits)
        sf = float(f16_np(s16))
        xh = orc.dequant(bits, 0, u, s16)
        assert np.all(np.abs(xh - x.astype(np.float64)) <= sf / 2)
        if sf >= 2.0**-14:
            i = int(np.argmax(np.abs(x)))
            assert int(u[i]) - (1 << (bits - 1)) == (Q if x[i] > 0 else -Q)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_asym_error_bound_and_extremal_codes(orc, bits):
    """|x^ - x| <= max(s/2, |z - lo| + M |s - (hi - lo)/M|): the s/2 bound widened by the fp16
    rounding of the stored scale and zero-point; hi -> M and lo -> 0 when the scale is a
    normal fp16 number and the zero-point rounding is small against the step."""
    M = (1 << bits) - 1
    for x in random_groups(2000, 32):
        s16, z16, u = orc.quant_asym(x, bits)
        sf, zf = float(f16_np(s16)), float(f16_np(z16))
        lo, hi = float(x.min()), float(x.max())
        xh = orc.dequant(bits, 1, u, s16, z16)
        bound = max(sf / 2, abs(zf - lo) + M * abs(sf - (hi - lo) / M)) + 1e-300
        assert np.all(np.abs(xh - x.astype(np.float64)) <= bound * (1 + 1e-12))
        if sf >= 2.0**-14 and abs(zf - lo) < 0.25 * sf:
            assert u[int(np.argmax(x))] == M and u[int(np.argmin(x))] == 0


def test_zero_group_and_reconstruction_exact_in_fp32(orc):
    """An all-zero group stores scale 0 and signed code 0; s * q has at most 19 significant
    bits, so the fp32 product equals the exact one."""
    s16, u = orc.quant_sym(np.zeros(64, np.float32), 4)
    assert s16 == 0 and np.all(u == 8)
    for x in random_groups(200, 64):
        for bits in (8, 4, 2):
            s16, u = orc.quant_sym(x, bits)
            q = u.astype(np.int64) - (1 << (bits - 1))
            sf32 = np.float32(f16_np(s16))
            assert np.array_equal((sf32 * q.astype(np.float32)).astype(np.float64), float(sf32) * q)


# ------------------------------------------------------------------------------------------
# Sizing [P2, "Why the KV cache grows so quickly" and "Worked example"; P1, "The KV Cache
# Problem" and "Practical Impact"]
# ------------------------------------------------------------------------------------------

def test_worked_example_sizes(orc):
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    L, H, d, T = g["L"], g["H_kv"], g["d_h"], g["T"]
    MiB, GiB = 2**20, 2**30
    bf16 = orc.mkv_bytes(L, T, H, d, 2)
    assert bf16 == g["bf16_bytes"] == GiB
    assert orc.mkv_bytes(L, T, H, d, 0.5) == 256 * MiB
    bpe = orc.bytes_per_element(4, g["scale_every_elements"], g["scale_bytes"])
    assert bpe == g["bytes_per_element"]
    q = orc.mkv_bytes(L, T, H, d, bpe)
    assert q == g["quantized_label_mib"] * MiB
    assert f"{bf16 / q:.2f}x" == g["reduction_label"]
    assert round(g["contexts"] * q / GiB, 1) == g["contexts_quantized_label_gib"]
    assert g["contexts"] * bf16 / GiB == g["contexts_bf16_label_gib"]
    # The same figure from the oracle's own storage images: one layer's codes and fp16
    # scales, times L layers.
    side = (4, orc.SYM, orc.PER_TOKEN, 64)
    im = orc.empty_images(side, side, 1, H, 0, capacity=T)
    per_layer = sum(im[n].nbytes for n in ("k_codes", "v_codes", "k_scale", "v_scale"))
    assert per_layer == 8_912_896
    assert L * per_layer == 272 * MiB


def test_memory_formula_every_width(orc):
    for b in (2, 1, 0.5, 0.25):
        assert orc.mkv_bytes(3, 5, 7, 11, b) == 2 * 3 * 5 * 7 * 11 * b
    r = json.load(open(os.path.join(GOLD, "storage_ratios.json")))
    for bits, ratio in r["ratios"].items():
        assert orc.mkv_bytes(1, 1, 1, 128, 2) / orc.mkv_bytes(1, 1, 1, 128, int(bits) / 8) == ratio


def test_p1_kv_problem_numbers(orc):
    g = json.load(open(os.path.join(GOLD, "kv_problem_p1.json")))
    per_tok = orc.p1_bytes_per_token(g["num_layers"], g["hidden_dim"], g["fp16_bytes"])
    assert per_tok == 524_288 and g["per_token_label"].startswith(str(per_tok // 1000))
    assert per_tok * g["tokens"] == 2**30
    assert per_tok * g["tokens"] * g["batch"] == g["users_32"]["fp16_GB"] * 2**30
    for key, bits in (("int8_GB", 8), ("int4_GB", 4)):
        assert per_tok * g["tokens"] * g["batch"] * bits // 16 == g["users_32"][key] * 2**30


# ------------------------------------------------------------------------------------------
# Worked illustrations [P2, "Why scales and groups matter"; "Why key errors and value errors
# are different"]
# ------------------------------------------------------------------------------------------

def test_outlier_vector_single_scale_vs_groups(orc):
    x = bf16_values(np.array(read_rows("outlier_vector.txt")[0], np.float32))
    s16, u = orc.quant_sym(x, 4)
    q = u.astype(int) - 8
    assert list(q[:4]) == [0, 0, 0, 0] and q[4] == 7  # small values all round to zero
    _, u2 = orc.quant_sym(x, 2)
    assert list(u2.astype(int) - 2) == [0, 0, 0, 0, 1]
    _, u8 = orc.quant_sym(x, 8)
    assert list(u8.astype(int) - 128) == [1, -1, 2, 2, 127]
    sA, uA = orc.quant_sym(x[:4], 4)  # first group: small magnitudes, hence a small scale
    qA = uA.astype(int) - 8
    assert list(qA) == [2, -4, 7, 5]
    err_single = np.abs(orc.dequant(4, 0, u[:4], s16) - x[:4])
    err_group = np.abs(orc.dequant(4, 0, uA, sA) - x[:4])
    assert err_group.max() < err_single.min()
    sB, uB = orc.quant_sym(x[4:], 4)
    assert f16_np(sB) > f16_np(sA) and int(uB[0]) - 8 == 7  # group B: larger scale


def test_logit_flip_softmax_closed_form(orc):
    (a, b), (a2, b2) = read_rows("logit_flip.txt")
    q = np.array([1.0, 0.0])
    kh = np.array([[a, 0.0], [b, 0.0]])
    vh = np.eye(2)
    w = orc.attend_rows(q, kh, vh, 1.0)
    pa = 1.0 / (1.0 + math.exp(-(a - b)))
    assert abs(w[0] - pa) < 1e-15 and abs(w[1] - (1 - pa)) < 1e-15
    assert f"{w[0]:.6f}" == "0.549834"
    w2 = orc.attend_rows(q, np.array([[a2, 0.0], [b2, 0.0]]), vh, 1.0)
    assert abs(w2[0] - w[1]) < 1e-15 and abs(w2[1] - w[0]) < 1e-15  # the preference flips


# ------------------------------------------------------------------------------------------
# Attention special cases and brute force [P2, attention equation]
# ------------------------------------------------------------------------------------------

def test_attention_special_cases(orc):
    d = 16
    q = RNG.standard_normal(d)
    kh = RNG.standard_normal((9, d))
    vh = RNG.standard_normal((9, d))
    assert np.allclose(orc.attend_rows(q, kh[:1], vh[:1], 0.25), vh[0], rtol=0, atol=0)
    same = np.repeat(kh[:1], 9, axis=0)
    assert np.allclose(orc.attend_rows(q, same, vh, 0.25), vh.mean(axis=0), atol=1e-15)
    assert np.allclose(orc.attend_rows(np.zeros(d), kh, vh, 0.25), vh.mean(axis=0), atol=1e-15)
    base = orc.attend_rows(q, kh, vh, 0.25)
    shifted = orc.attend_rows(np.concatenate([q, [1.0]]),
                              np.concatenate([kh, np.full((9, 1), 3.7)], axis=1),
                              np.concatenate([vh, np.zeros((9, 1))], axis=1), 0.25)[:d]
    assert np.allclose(base, shifted, atol=1e-14)
    perm = RNG.permutation(9)
    assert np.allclose(base, orc.attend_rows(q, kh[perm], vh[perm], 0.25), atol=1e-14)


def python_reference_attention(seq, q_bits, sm_scale):
    """Pure-Python fp64 attention over a Sequence's logical state: its own dequantization
    (numpy's float16 decoder), math.fsum sums, math.exp."""
    k_bits, k_scheme, k_axis, k_group = seq.k_side
    v_bits, v_scheme, v_axis, v_group = seq.v_side
    H, d = seq.H, seq.d
    Hq = q_bits.shape[0]
    qf = (q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def bf16(x):
        return float((np.asarray(x, np.uint32) << 16).view(np.float32))

    def deq(u, s16, z16, bits, scheme):
        s = float(f16_np(s16))
        if scheme == 0:
            return s * (int(u) - (1 << (bits - 1)))
        return s * int(u) + float(f16_np(z16))

    def meta(side, S, Z, h, p, c):
        bits, scheme, axis, group = side
        if axis == 0:
            i = (h, p, c // group)
        else:
            i = (h, p // group, c)
        return S[i], (Z[i] if scheme == 1 else 0)

    out = np.zeros((Hq, d))
    for hq in range(Hq):
        h = hq * H // Hq
        keys, vals = [], []
        for p in range(seq.n_quant):
            if k_bits == 16:
                keys.append([bf16(seq.kb[h, p, c]) for c in range(d)])
            else:
                keys.append([deq(seq.ku[h, p, c], *meta(seq.k_side, seq.ks, seq.kz, h, p, c),
                                 k_bits, k_scheme) for c in range(d)])
            if v_bits == 16:
                vals.append([bf16(seq.vb[h, p, c]) for c in range(d)])
            else:
                vals.append([deq(seq.vu[h, p, c], *meta(seq.v_side, seq.vs, seq.vz, h, p, c),
                                 v_bits, v_scheme) for c in range(d)])
        for r in range(seq.n_res):
            keys.append(list((seq.kres[h, r].astype(np.uint32) << 16).view(np.float32).astype(float)))
            vals.append(list((seq.vres[h, r].astype(np.uint32) << 16).view(np.float32).astype(float)))
        scores = [math.fsum(qf[hq, c] * k[c] for c in range(d)) * sm_scale for k in keys]
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        l = math.fsum(w)
        for c in range(d):
            out[hq, c] = math.fsum(w[t] * vals[t][c] for t in range(len(w))) / l
    return out


@pytest.mark.parametrize("case", [
    ((8, 0, 0, 128), (8, 0, 0, 128), 0, 40),
    ((4, 0, 0, 64), (4, 0, 0, 64), 16, 45),
    ((2, 1, 1, 16), (2, 1, 0, 32), 32, 61),
    ((4, 1, 0, 32), (8, 1, 0, 64), 16, 33),
    ((16, 0, 0, 128), (16, 0, 0, 128), 16, 37),
])
def test_attention_brute_force_tiny(orc, case):
    """The oracle's attention over its own state equals a pure-Python fsum computation to
    fp32 output rounding."""
    k_side, v_side, R, T = case
    H, Hq = 2, 4
    seq = orc.Sequence(k_side, v_side, H, R, capacity=128)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kbits = kv.view(np.uint32) >> 16
    seq.append(kbits[0].astype(np.uint16), kbits[1].astype(np.uint16))
    q = (bf16_values(RNG.standard_normal((Hq, 128)).astype(np.float32)).view(np.uint32) >> 16)
    q = q.astype(np.uint16)
    sm = float(np.float32(1 / math.sqrt(128)))
    got = seq.attend(q, sm)
    ref = python_reference_attention(seq, q, sm)
    assert np.allclose(got, ref, rtol=2.0**-23, atol=1e-30)


# ------------------------------------------------------------------------------------------
# BF16 storage (bits 16): the unquantized baseline [P2, "From BF16 to INT8, INT4, or even fewer
# bits"; P3, "Go-Live Checklist": a BF16 baseline and fallback]
# ------------------------------------------------------------------------------------------

BF16_SIDE = (16, 0, 0, 128)


def test_bf16_storage_keeps_every_bit(orc):
    H, T, R = 2, 77, 16
    seq = orc.Sequence(BF16_SIDE, BF16_SIDE, H, R, capacity=128)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32) * 100)
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kb[0], kb[1])
    nq = seq.n_quant
    assert nq == T - seq.n_res and seq.n_res == (T - 1) % R + 1
    assert np.array_equal(seq.kb[:, :nq], kb[0, :nq].transpose(1, 0, 2))
    assert np.array_equal(seq.vb[:, :nq], kb[1, :nq].transpose(1, 0, 2))


def test_bf16_equals_int8_where_int8_is_exact(orc):
    """Rows of integers in [-127, 127] that reach +-127 in every row: the INT8 per-token
    quantizer (group 128) gets scale exactly 1 and reproduces them, so attention over the INT8
    cache and over the BF16 cache sees identical values and must agree to the last bit."""
    H, T, Hq = 2, 70, 4
    x = RNG.integers(-127, 128, size=(2, T, H, 128)).astype(np.float32)
    x[..., 5] = np.where(RNG.random((2, T, H)) < 0.5, 127.0, -127.0)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # integers below 256 are exact in bf16
    a = orc.Sequence(BF16_SIDE, BF16_SIDE, H, 0, capacity=128)
    b = orc.Sequence((8, 0, 0, 128), (8, 0, 0, 128), H, 0, capacity=128)
    a.append(xb[0], xb[1])
    b.append(xb[0], xb[1])
    assert np.all(b.ks[:, :T] == 0x3C00) and np.all(b.vs[:, :T] == 0x3C00)  # fp16 1.0
    q = (bf16_values(RNG.standard_normal((Hq, 128)).astype(np.float32) * 0.01).view(np.uint32)
         >> 16).astype(np.uint16)
    assert np.array_equal(a.attend(q, 0.088), b.attend(q, 0.088))


def test_bf16_layout_and_paged_roundtrip(orc):
    # V: element (t, c) is halfword 4 (c % 8) + t % 4 of chunk (t / 4) 16 + c / 8, whose 16-byte
    # piece i lives in slab i (1 KiB) at 16 chunk; K: channels 8 p .. 8 p + 7 of row t form
    # piece p % 4 of slice 4 t + p / 4
    for t in range(16):
        for c in range(128):
            chunk = (t // 4) * 16 + c // 8
            hb = 2 * (4 * (c % 8) + t % 4)
            assert orc.v_bit(16, t, c) == 8 * (1024 * (hb // 16) + 16 * chunk + hb % 16)
            p_ = c // 8
            assert orc.k_bit(16, t, c) == 8 * (1024 * (p_ % 4) + 16 * (4 * t + p_ // 4) + 2 * (c % 8))
    H, T = 2, 90
    seq = orc.Sequence(BF16_SIDE, BF16_SIDE, H, 0, capacity=128)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kb[0], kb[1])
    table = RNG.permutation(8).astype(np.int32)
    im = orc.empty_images(BF16_SIDE, BF16_SIDE, 1, H, 0, num_blocks=8)
    seq.pack(0, im, table)
    # every K element is its bf16 bit pattern, little-endian, at the slab offset
    for p_ in (0, 17, 89):
        for h in range(H):
            tile = table[p_ // 16] * H + h
            img = im["k_codes"][tile * 4096:(tile + 1) * 4096]
            got = [int(img[orc.k_bit(16, p_ % 16, c) // 8]) | int(img[orc.k_bit(16, p_ % 16, c) // 8 + 1]) << 8
                   for c in range(128)]
            assert got == [int(x) for x in kb[0, p_, h]]
    back = orc.Sequence(BF16_SIDE, BF16_SIDE, H, 0, capacity=128)
    back.set_counters(T, 0)
    back.unpack_codes(0, im, table)
    assert np.array_equal(back.kb[:, :T], seq.kb[:, :T])
    assert np.array_equal(back.vb[:, :T], seq.vb[:, :T])


# ------------------------------------------------------------------------------------------
# FP8 E4M3 with per-tensor / per-head scales [P3, "Step 3: Deploy a Fallback-Capable FP8 First"]
# ------------------------------------------------------------------------------------------

def torch_e4m3(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_values_match_torch(orc):
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x01) == 2.0**-9


def test_e4m3_encode_matches_torch_cast_exhaustively(orc):
    """Every finite bf16 value below 464 in magnitude (torch's cast turns larger ones into NaN;
    here they saturate to +-448), plus random fp32 values around every binade."""
    b = np.arange(65536, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464)]
    assert np.array_equal(orc.e4m3_encode_array(x), torch_e4m3(x))
    y = (RNG.standard_normal(200000) * np.exp2(RNG.integers(-12, 9, 200000))).astype(np.float32)
    y = y[np.abs(y) < 464]
    assert np.array_equal(orc.e4m3_encode_array(y), torch_e4m3(y))
    big = np.array([448.0, 463.9, 464.0, 1e4, 3e38, -500.0], np.float32)
    assert list(orc.e4m3_encode_array(big)) == [0x7E] * 5 + [0xFE]


def test_fp8_cache_follows_definition_and_attention(orc):
    """Per-head scales: head h stores E4M3(x / s_h) (numpy fp32 division, torch's cast); the
    oracle's attention equals a pure-Python fsum over s_h * E4M3 value."""
    import torch
    H, Hq, T, R = 2, 4, 45, 16
    ks, vs = np.array([0.02, 0.5], np.float32), np.array([0.01, 0.75], np.float32)
    side_k, side_v = (8, 2, 3, 0), (8, 2, 3, 0)
    seq = orc.Sequence(side_k, side_v, H, R, capacity=128, k_fp8_scale=ks, v_fp8_scale=vs)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kbits = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kbits[0], kbits[1])
    nq = seq.n_quant
    for h in range(H):
        assert np.array_equal(seq.ku[h, :nq], torch_e4m3(kv[0, :nq, h] / ks[h]))
        assert np.array_equal(seq.vu[h, :nq], torch_e4m3(kv[1, :nq, h] / vs[h]))
    q = (bf16_values(RNG.standard_normal((Hq, 128)).astype(np.float32)).view(np.uint32) >> 16)
    q = q.astype(np.uint16)
    sm = float(np.float32(1 / math.sqrt(128)))
    got = seq.attend(q, sm)
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for hq in range(Hq):
        h = hq * H // Hq
        keys = [list(float(ks[h]) * dec[seq.ku[h, p]]) for p in range(nq)]
        vals = [list(float(vs[h]) * dec[seq.vu[h, p]]) for p in range(nq)]
        for r in range(seq.n_res):
            keys.append(list((seq.kres[h, r].astype(np.uint32) << 16).view(np.float32).astype(float)))
            vals.append(list((seq.vres[h, r].astype(np.uint32) << 16).view(np.float32).astype(float)))
        scores = [math.fsum(qf[hq, c] * kk[c] for c in range(128)) * sm for kk in keys]
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        l = math.fsum(w)
        ref = [math.fsum(w[t] * vals[t][c] for t in range(len(w))) / l for c in range(128)]
        assert np.allclose(got[hq], ref, rtol=2.0**-23, atol=1e-30)


# ------------------------------------------------------------------------------------------
# Window state machine [P2, "Why some systems keep a full-precision window"]
# ------------------------------------------------------------------------------------------

def _seq_arrays(seq):
    return [seq.ku, seq.vu, seq.ks, seq.kz, seq.vs, seq.vz]


@pytest.mark.parametrize("k_side,R", [((4, 0, 0, 64), 32), ((2, 1, 1, 32), 64), ((8, 0, 0, 128), 0)])
def test_window_invariants_and_flush_is_optional(orc, k_side, R):
    H, T = 2, 200
    v_side = (4, 0, 0, 64)
    a = orc.Sequence(k_side, v_side, H, R, capacity=512)
    b = orc.Sequence(k_side, v_side, H, R, capacity=512)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    pos = 0
    while pos < T:
        n = int(RNG.integers(1, 23))
        n = min(n, T - pos)
        a.append(kb[0, pos:pos + n], kb[1, pos:pos + n])
        for j in range(n):  # b: one token at a time, flushing eagerly before each
            b.flush()
            b.append(kb[0, pos + j:pos + j + 1], kb[1, pos + j:pos + j + 1])
        pos += n
        if R:
            assert a.n_res == (pos - 1) % R + 1 and a.n_quant == pos - a.n_res
        else:
            assert a.n_quant == pos and a.n_res == 0
    for x, y in zip(_seq_arrays(a), _seq_arrays(b)):
        assert np.array_equal(x, y)
    q = (bf16_values(RNG.standard_normal((4, 128)).astype(np.float32)).view(np.uint32) >> 16)
    q = q.astype(np.uint16)
    assert np.array_equal(a.attend(q, 0.088), b.attend(q, 0.088))


def test_per_channel_key_groups_follow_definition(orc):
    """Per-channel keys: for each channel, one scale and zero-point per group of Gt
    consecutive compressed tokens (numpy float32 arithmetic and numpy's float16 cast)."""
    Gt, R, H = 16, 32, 1
    seq = orc.Sequence((2, 1, 1, Gt), (2, 1, 0, 32), H, R, capacity=256)
    T = 100
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kb[0], kb[1])
    assert seq.n_quant == 96 and seq.n_res == 4
    for tau in range(seq.n_quant // Gt):
        blk = kv[0, tau * Gt:(tau + 1) * Gt, 0, :]  # [Gt][d]
        lo, hi = blk.min(axis=0), blk.max(axis=0)
        s = ((hi - lo) / np.float32(3)).astype(np.float16).view(np.uint16)
        z = lo.astype(np.float16).view(np.uint16)
        assert np.array_equal(seq.ks[0, tau], s) and np.array_equal(seq.kz[0, tau], z)


# ------------------------------------------------------------------------------------------
# Storage layout (a format of this project): bijection, pack/unpack, block permutations
# [P2, "How this connects to paging and prefix caching": block tables]
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [16, 8, 4, 2])
def test_layout_is_a_bijection(orc, bits):
    S = min(16, 4 * bits)  # bytes of a slice piece; slab i holds piece i of all 64 slices
    vb = sorted(orc.v_bit(bits, t, c) for t in range(16) for c in range(128))
    assert vb == list(range(0, 16 * 128 * bits, bits))
    kb = sorted(orc.k_bit(bits, t, c) for t in range(16) for c in range(128))
    assert kb == list(range(0, 16 * 128 * bits, bits))
    for t in range(16):
        for c in range(128):
            # V: slice (t/4)*16 + c/8 holds channels c&~7.., tokens 4(t/4)..; K: slice 4t + c/32
            vbyte, kbyte = orc.v_bit(bits, t, c) // 8, orc.k_bit(bits, t, c) // 8
            assert (vbyte % (64 * S)) // S == (t // 4) * 16 + c // 8
            assert (kbyte % (64 * S)) // S == 4 * t + c // 32
            if bits <= 4:  # one piece per slice: K rows are plain row-major rows
                assert orc.k_bit(bits, t, c) == (t * 128 + c) * bits


@pytest.mark.parametrize("k_side,v_side", [((4, 0, 0, 64), (4, 0, 0, 64)),
                                           ((2, 1, 0, 32), (8, 1, 0, 128)),
                                           ((8, 2, 3, 0), (8, 2, 2, 0))])
def test_paged_pack_roundtrip_any_block_permutation(orc, k_side, v_side):
    H, R, T = 2, 16, 150
    seq = orc.Sequence(k_side, v_side, H, R, capacity=256)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kb[0], kb[1])
    nblk = 16
    imgs = []
    for trial in range(2):
        table = RNG.permutation(nblk).astype(np.int32)
        im = orc.empty_images(k_side, v_side, 1, H, R, num_blocks=nblk)
        seq.pack(0, im, table)
        back = orc.Sequence(k_side, v_side, H, R, capacity=256)
        back.set_counters(seq.n_quant, 0)
        back.unpack_codes(0, im, table)
        assert np.array_equal(back.ku[:, :seq.n_quant], seq.ku[:, :seq.n_quant])
        assert np.array_equal(back.vu[:, :seq.n_quant], seq.vu[:, :seq.n_quant])
        tile_bytes = 16 * 128 * k_side[0] // 8
        logical = [im["k_codes"][(table[j] * H) * tile_bytes:(table[j] * H + H) * tile_bytes]
                   for j in range(nblk)]
        imgs.append(np.concatenate(logical))
    assert np.array_equal(imgs[0], imgs[1])  # same logical content under either permutation


@pytest.mark.parametrize("gt", [16, 32, 64])
def test_paged_per_channel_metadata_travels_with_the_group_block(orc, gt):
    """Paged per-channel keys: key group tau's scale/zero row is stored with the physical block
    of the group's first token, whatever the block permutation [P2, "How this connects to paging
    and prefix caching"; P3, "Why Can't You Quantize the KV Cache Like Ordinary Activations?"]."""
    H, R, T = 2, 64, 300
    k_side, v_side = (2, 1, 1, gt), (2, 1, 0, 32)
    seq = orc.Sequence(k_side, v_side, H, R, capacity=512)
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    seq.append(kb[0], kb[1])
    nblk = 32
    table = RNG.permutation(nblk).astype(np.int32)
    im = orc.empty_images(k_side, v_side, 1, H, R, num_blocks=nblk)
    assert im["k_scale"].size == nblk * H * 128
    seq.pack(0, im, table)
    for tau in range(seq.n_quant // gt):
        blk = table[tau * gt // 16]
        for h in range(H):
            row = slice((blk * H + h) * 128, (blk * H + h + 1) * 128)
            assert np.array_equal(im["k_scale"][row], seq.ks[h, tau])
            assert np.array_equal(im["k_zero"][row], seq.kz[h, tau])
    back = orc.Sequence(k_side, v_side, H, R, capacity=512)
    back.set_counters(seq.n_quant, 0)
    back.unpack_codes(0, im, table)
    assert np.array_equal(back.ku[:, :seq.n_quant], seq.ku[:, :seq.n_quant])


@pytest.mark.parametrize("k_side,v_side", [((4, 0, 0, 64), (4, 0, 0, 64)),
                                           ((16, 0, 0, 128), (16, 0, 0, 128))])
def test_multi_query_is_causal_single_query_over_prefixes(orc, k_side, v_side):
    """Multi-query decode: query i of the last n_q tokens equals single-query decode over a
    sequence that holds only the first T - n_q + i + 1 tokens (without a window the codes of a
    token do not depend on what follows, so the prefixes are the same cache state)."""
    H, Hq, T, nq = 2, 8, 75, 6
    kv = bf16_values(RNG.standard_normal((2, T, H, 128)).astype(np.float32))
    kb = (kv.view(np.uint32) >> 16).astype(np.uint16)
    full = orc.Sequence(k_side, v_side, H, 0, capacity=128)
    full.append(kb[0], kb[1])
    q = (bf16_values(RNG.standard_normal((nq, Hq, 128)).astype(np.float32)).view(np.uint32) >> 16)
    q = q.astype(np.uint16)
    got = full.attend_mq(q, 0.088)
    for i in range(nq):
        pre = orc.Sequence(k_side, v_side, H, 0, capacity=128)
        pre.append(kb[0, :T - nq + i + 1], kb[1, :T - nq + i + 1])
        assert np.array_equal(got[i], pre.attend(q[i], 0.088))
    assert np.array_equal(full.attend_mq(q[-1:], 0.088)[0], full.attend(q[-1], 0.088))
    # a query before the first token attends nothing
    tiny = orc.Sequence(k_side, v_side, H, 0, capacity=128)
    tiny.append(kb[0, :2], kb[1, :2])
    out = tiny.attend_mq(q[:4], 0.088)
    assert np.all(out[0] == 0) and np.all(out[1] == 0) and np.any(out[3] != 0)
