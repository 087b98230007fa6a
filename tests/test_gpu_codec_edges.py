"""GPU parity of the quantize-append path on crafted edge-case groups: every byte of the codes,
scales and zero-points written by the HIP kernels equals the oracle's image.

The groups (tests/codec_edges.py) hold exact half-integer quotients (positive and negative),
all +0.0 or all -0.0, fp32 scales at the fp16 underflow boundary 2^-25, magnitudes near 1e-30
and near the fp16 scale limit, and constant groups (for per-channel keys: a channel constant over
its token group).  Every bit width (2, 4, 8) and scheme (symmetric, asymmetric) is covered with
per-token keys and with per-channel keys, contiguous and paged, through bulk appends and through
single-token appends that flush full windows.
"""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest
import torch

import codec_edges as ce
import kvq_cases as kc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


CODEC_CASES = [
    # name, k side, v side, R, paged, tokens per sequence, single-token tail
    ("sym8-g128", (8, 0, 0, 128), (8, 0, 0, 128), 0, False, [80, 37], 6),
    ("sym8-g32-paged-window", (8, 0, 0, 32), (8, 0, 0, 64), 32, True, [100, 64], 40),
    ("sym4-g64-window", (4, 0, 0, 64), (4, 0, 0, 64), 32, False, [100, 70], 40),
    ("sym4-g32-paged", (4, 0, 0, 32), (4, 0, 0, 128), 0, True, [90, 31], 5),
    ("sym2-g32-window", (2, 0, 0, 32), (2, 0, 0, 32), 16, False, [90, 50], 20),
    ("sym2-g128-paged", (2, 0, 0, 128), (2, 0, 0, 64), 0, True, [70, 17], 5),
    ("asym8-g64-paged", (8, 1, 0, 64), (8, 1, 0, 64), 0, True, [80, 33], 6),
    ("asym8-g128-window", (8, 1, 0, 128), (8, 1, 0, 32), 16, False, [70, 40], 20),
    ("asym4-g32-window", (4, 1, 0, 32), (4, 1, 0, 32), 32, False, [100, 65], 40),
    ("asym4-g64-paged-window", (4, 1, 0, 64), (4, 1, 0, 128), 16, True, [90, 48], 20),
    ("asym2-g32-paged-window", (2, 1, 0, 32), (2, 1, 0, 32), 16, True, [90, 47], 20),
    ("asym2-g64", (2, 1, 0, 64), (2, 1, 0, 64), 0, False, [77, 20], 5),
    # keys and values in different integer formats
    ("mix-k8s-v4a-window", (8, 0, 0, 64), (4, 1, 0, 32), 16, False, [90, 40], 20),
    ("mix-k2a-v8s-paged", (2, 1, 0, 32), (8, 0, 0, 128), 0, True, [70, 33], 5),
    ("mix-kpc4a-v2s-paged", (4, 1, 1, 32), (2, 0, 0, 64), 64, True, [192, 96], 70),
    # per-channel keys: groups over tokens, formed when a window flushes
    ("kpc2-asym-g32", (2, 1, 1, 32), (2, 1, 0, 32), 64, False, [192, 128], 70),
    ("kpc2-sym-g64-paged", (2, 0, 1, 64), (2, 0, 0, 32), 128, True, [320, 192], 140),
    ("kpc4-sym-g16-paged", (4, 0, 1, 16), (4, 0, 0, 64), 32, True, [160, 96], 40),
    ("kpc4-asym-g32", (4, 1, 1, 32), (4, 1, 0, 32), 64, False, [192, 96], 70),
    ("kpc8-asym-g64", (8, 1, 1, 64), (8, 1, 0, 128), 64, False, [192, 128], 70),
    ("kpc8-sym-g16-paged", (8, 0, 1, 16), (8, 0, 0, 32), 16, True, [96, 48], 20),
]


def crafted_pair(name, k, v, R, paged, lens, tail, H=2, Hq=4):
    """The crafted cache of one case and the largest |value| among its inputs."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k_rows, v_rows, vmax = [], [], 1.0
    for b, T in enumerate(lens):
        kx = ce.crafted_rows(k, T, H, rng, start=b)
        vx = ce.crafted_rows(v, T, H, rng, start=3 + b)
        vmax = max(vmax, float(np.abs(vx).max()))
        k_rows.append(ce.to_bf16_bits(kx))
        v_rows.append(ce.to_bf16_bits(vx))
    pr = kc.build_pair_rows(k, v, Hq, H, R, k_rows, v_rows, paged=paged,
                            seed=zlib.crc32(name.encode()) % 1000, single_tail=tail)
    return pr, vmax


@pytest.mark.parametrize("name,k,v,R,paged,lens,tail", CODEC_CASES, ids=[c[0] for c in CODEC_CASES])
def test_crafted_groups_bit_exact(name, k, v, R, paged, lens, tail):
    print("case:", name, flush=True)
    sys.stdout.flush()
    pr, _ = crafted_pair(name, k, v, R, paged, lens, tail)
    kc.compare_state(pr)


@pytest.mark.parametrize("name,k,v,R,paged,lens,tail", CODEC_CASES, ids=[c[0] for c in CODEC_CASES])
def test_attention_over_crafted_groups(name, k, v, R, paged, lens, tail):
    """Decode attention over the crafted caches (zero, underflowing, tiny and huge groups among
    ordinary ones): within the bar scaled by the largest |value| (the outputs scale with it)."""
    print("case:", name, "attention", flush=True)
    pr, vmax = crafted_pair(name, k, v, R, paged, lens, tail)
    kc.compare_attention(pr, tol_scale=vmax)


SYM4 = (4, 0, 0, 64)
KPC2 = (2, 1, 1, 32)
ASYM2_32 = (2, 1, 0, 32)
DOMAIN_FORMATS = [
    # name, k, v, Hq, H, R, lens, paged
    ("int4-gqa4-window", SYM4, SYM4, 8, 2, 32, [300, 77], False),
    ("kivi-int2-paged", KPC2, ASYM2_32, 8, 2, 64, [300, 140], True),
    ("int8-mha", (8, 0, 0, 128), (8, 0, 0, 128), 2, 2, 0, [200, 33], False),
    ("asym4-g32-gqa2", (4, 1, 0, 32), (4, 1, 0, 32), 4, 2, 16, [250, 99], False),
    ("int2-g64-gqa8", (2, 0, 0, 64), (2, 0, 0, 64), 16, 2, 16, [260, 50], True),
    ("kpc8-sym-g16", (8, 0, 1, 16), (8, 0, 0, 64), 4, 2, 32, [200, 64], False),
    ("fp8-head-gqa4", (8, 2, 3, 0), (8, 2, 3, 0), 8, 2, 16, [300, 77], False),
]


@pytest.mark.parametrize("q_scale", [1e5, 3e3, 1e-6, 1e-30, 0.0])
@pytest.mark.parametrize("name,k,v,Hq,H,R,lens,paged", DOMAIN_FORMATS, ids=[c[0] for c in DOMAIN_FORMATS])
def test_query_magnitudes(name, k, v, Hq, H, R, lens, paged, q_scale):
    """Queries of any bf16 magnitude: each query row enters the matrix cores after an exact
    power-of-two prescale, so |q| near 1e5 (beyond f16) and near 1e-30 (below f16) attend
    like ordinary queries; q = 0 gives the mean of the values."""
    print("case:", name, "q_scale", q_scale, flush=True)
    pr = kc.build_pair(k, v, len(lens), Hq, H, R, lens, paged=paged,
                       seed=zlib.crc32(name.encode()) % 1000)
    kc.compare_attention(pr, q_scale=q_scale)


VALUE_SCALE_CASES = [
    # name, k, v, value multiplier c, offset: values c x (symmetric) or c |x| + offset
    # (asymmetric: the minimum, stored as the fp16 zero-point, stays within fp16), x ~ N(0, 1);
    # the largest fp16 value scale reaches 50-65k
    ("int2-sym-g32", (2, 0, 0, 32), (2, 0, 0, 32), 15000.0, 0.0, 16, False),
    ("int4-sym-g64", SYM4, SYM4, 1.0e5, 0.0, 32, True),
    ("int8-sym-g128", (8, 0, 0, 128), (8, 0, 0, 128), 1.8e6, 0.0, 0, False),
    ("kivi-asym2-g32", KPC2, ASYM2_32, 4.2e4, -6.0e4, 64, False),
    ("asym4-g32", (4, 1, 0, 32), (4, 1, 0, 32), 2.1e5, -6.0e4, 16, True),
]


@pytest.mark.parametrize("name,k,v,c,off,R,paged", VALUE_SCALE_CASES, ids=[c[0] for c in VALUE_SCALE_CASES])
def test_value_scales_near_fp16_limit(name, k, v, c, off, R, paged):
    """Values whose fp16 group scales approach 65504: the PV weights times those scales stay
    within the hi + lo f16 operand parts (weights <= 2), so the outputs match the oracle within
    the bar scaled by the value magnitude."""
    print("case:", name, "value scale", c, flush=True)
    H, Hq, lens = 2, 8, [260, 90]
    w = kc.ki.Workload("vs", zlib.crc32(name.encode()) % 1000, 2, Hq, H, 260,
                       kc.ki.Side(*k), kc.ki.Side(*v), residual=R)
    k_rows, v_rows, vmax = [], [], 1.0
    for b, T in enumerate(lens):
        kk, vv = kc.ki.prefill_kv(w, b, T)
        x = vv.float()
        vv = (x * c if v[1] == 0 else x.abs() * c + off).to(torch.bfloat16)
        vmax = max(vmax, float(vv.float().abs().max()))
        k_rows.append(kc.ki.bf16_bits(kk))
        v_rows.append(kc.ki.bf16_bits(vv))
    pr = kc.build_pair_rows(k, v, Hq, H, R, k_rows, v_rows, paged=paged, seed=w.seed,
                            single_tail=20)
    kc.compare_state(pr)
    # the value scales really reach the top binade of fp16
    shared = k[2] == 0 and v[2] == 0
    vs = (pr.cache.k_scale if shared else pr.cache.v_scale).view(torch.float16).float()
    assert float(vs.abs().max()) > 32768, float(vs.abs().max())
    kc.compare_attention(pr, tol_scale=vmax)


DENSE_FORMATS = [
    # name, k, v, Hq, H, R, lens, paged: formats the dense multi-query kernel serves
    ("int4-g64-gqa4-window", SYM4, SYM4, 8, 2, 32, [300, 77], False),
    ("asym4-g32-gqa2-paged", (4, 1, 0, 32), (4, 1, 0, 32), 4, 2, 16, [250, 99], True),
    ("int8-g128-mha", (8, 0, 0, 128), (8, 0, 0, 128), 2, 2, 0, [200, 33], False),
    ("int2-g64-gqa8", (2, 0, 0, 64), (2, 0, 0, 64), 16, 2, 16, [260, 50], True),
    ("fp8-head-gqa4-paged", (8, 2, 3, 0), (8, 2, 3, 0), 8, 2, 16, [300, 77], True),
    ("bf16-mha-window", (16, 0, 0, 128), (16, 0, 0, 128), 2, 2, 32, [260, 99], False),
]


@pytest.mark.parametrize("q_scale", [1e5, 1e-30, 0.0])
@pytest.mark.parametrize("name,k,v,Hq,H,R,lens,paged", DENSE_FORMATS, ids=[c[0] for c in DENSE_FORMATS])
def test_dense_multi_query_magnitudes(name, k, v, Hq, H, R, lens, paged, q_scale, monkeypatch):
    """The dense multi-query kernel (forced from 16 rows) takes the same exact power-of-two query
    prescale: queries beyond f16 and below it attend like ordinary ones, q = 0 gives the mean of
    the values visible to each query."""
    print("case:", name, "dense multi-query q_scale", q_scale, flush=True)
    monkeypatch.setenv("KVQ_MQ_DENSE", "1")
    pr = kc.build_pair(k, v, len(lens), Hq, H, R, lens, paged=paged,
                       seed=zlib.crc32(name.encode()) % 1000)
    kc.compare_attention_mq(pr, 8, q_scale=q_scale)


@pytest.mark.parametrize("name,k,v,c,off,R,paged",
                         [cse for cse in VALUE_SCALE_CASES if cse[1][2] == 0],
                         ids=[cse[0] for cse in VALUE_SCALE_CASES if cse[1][2] == 0])
def test_dense_multi_query_value_scales_near_fp16_limit(name, k, v, c, off, R, paged, monkeypatch):
    """Value scales near 65504 through the dense multi-query kernel: the values enter its
    products as s (u - off) 2^-8 (or (s u + z) 2^-8) in f16, which stays finite for every fp16
    scale, and the outputs match the oracle within the bar scaled by the value magnitude."""
    print("case:", name, "dense multi-query value scale", c, flush=True)
    monkeypatch.setenv("KVQ_MQ_DENSE", "1")
    H, Hq, lens = 2, 8, [260, 90]
    w = kc.ki.Workload("vs", zlib.crc32(name.encode()) % 1000, 2, Hq, H, 260,
                       kc.ki.Side(*k), kc.ki.Side(*v), residual=R)
    k_rows, v_rows, vmax = [], [], 1.0
    for b, T in enumerate(lens):
        kk, vv = kc.ki.prefill_kv(w, b, T)
        x = vv.float()
        vv = (x * c if v[1] == 0 else x.abs() * c + off).to(torch.bfloat16)
        vmax = max(vmax, float(vv.float().abs().max()))
        k_rows.append(kc.ki.bf16_bits(kk))
        v_rows.append(kc.ki.bf16_bits(vv))
    pr = kc.build_pair_rows(k, v, Hq, H, R, k_rows, v_rows, paged=paged, seed=w.seed,
                            single_tail=20)
    kc.compare_attention_mq(pr, 6, tol_scale=vmax)
