"""Randomised GPU parity over formats and shapes: 48 seeded cases drawn over key and value
formats (2/4/8 bits, symmetric or asymmetric, chosen independently; per-token groups of
32/64/128 channels, per-channel key groups of 16/32/64 tokens; FP8 and BF16 storage), GQA
ratios 1/2/4/8, 1-4 kv heads, windows of 0-128 tokens, lengths 0-300 per sequence, contiguous
or paged caches.  Each case: codes, scales and windows bit-exact after the prefill, attention
within the bar, one decode step (window flushes where due), both again.  The draw is fixed by
the case index, so a failure names a reproducible case.

A second set of 24 draws goes through the dense multi-query kernel (forced from 16 query rows
per kv head): one format on both sides (2/4/8 bits, symmetric or asymmetric, per-token key
groups of 32/64/128; some draws FP8 E4M3 or BF16), GQA 1/2/4/8, 16-96 query rows per kv head,
windows, lengths 0-400, contiguous or paged.

A third set of 24 draws takes the first set's formats and shapes (keys and values in independent
formats, per-channel keys included) through multi-query decode with 2-12 query tokens per
sequence (the blocked kernel's query blocks; the dense kernel where one format with enough rows
takes it)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import kvq_cases as kc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def draw(i: int):
    rng = np.random.default_rng(9000 + i)
    special = rng.random()
    G = int(rng.choice([1, 2, 4, 8]))
    H = int(rng.choice([1, 2, 4]))
    if special < 0.1:
        k = v = (16, 0, 0, 128)
        R = int(rng.choice([0, 16, 32]))
    elif special < 0.2:
        k = (8, 2, int(rng.choice([2, 3])), 0)
        v = (8, 2, int(rng.choice([2, 3])), 0)
        R = int(rng.choice([0, 16, 64]))
    else:
        while True:
            kb, vb = int(rng.choice([2, 4, 8])), int(rng.choice([2, 4, 8]))
            ks, vs = int(rng.integers(2)), int(rng.integers(2))
            vg = int(rng.choice([32, 64, 128]))
            if rng.random() < 0.35:  # per-channel keys
                gt = int(rng.choice([16, 32, 64]))
                R = gt * int(rng.choice([1, 2])) if gt < 128 else 128
                k = (kb, ks, 1, gt)
                ok = True
            else:
                kg = int(rng.choice([32, 64, 128]))
                R = int(rng.choice([0, 16, 32, 128]))
                k = (kb, ks, 0, kg)
                ok = (128 // kg) * G <= 16
            v = (vb, vs, 0, vg)
            if ok and 2 * G * (128 // vg) <= 32:
                break
    B = int(rng.integers(1, 4))
    lens = [int(rng.integers(0, 301)) for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 1
    paged = bool(rng.integers(2))
    return k, v, B, G * H, H, R, lens, paged


@pytest.mark.parametrize("i", range(48))
def test_random_case(i):
    k, v, B, Hq, H, R, lens, paged = draw(i)
    print("case:", i, dict(k=k, v=v, B=B, Hq=Hq, H=H, R=R, lens=lens, paged=paged), flush=True)
    sys.stdout.flush()
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, paged=paged, seed=500 + i)
    kc.compare_state(pr)
    kc.compare_attention(pr)
    kc.step(pr, flush_first=bool(i % 2))
    kc.compare_state(pr)
    kc.compare_attention(pr, q_seed_step=1)


def draw_dense(i: int):
    rng = np.random.default_rng(7100 + i)
    bits, sch = int(rng.choice([2, 4, 8])), int(rng.integers(2))
    side = (bits, sch, 0, int(rng.choice([32, 64, 128])))
    if i % 6 == 5:  # FP8 E4M3, one scale per kv head or per tensor
        side = (8, 2, int(rng.choice([2, 3])), 0)
    elif i % 8 == 6:  # BF16 storage
        side = (16, 0, 0, 128)
    G = int(rng.choice([1, 2, 4, 8]))
    H = int(rng.choice([1, 2]))
    R = int(rng.choice([0, 16, 32, 64, 128]))
    n_q = int(rng.integers(max(2, -(-16 // G)), 96 // G + 1))
    B = int(rng.integers(1, 4))
    lens = [int(rng.integers(0, 401)) for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 1
    paged = bool(rng.integers(2))
    return side, B, G * H, H, R, lens, paged, n_q


@pytest.mark.parametrize("i", range(24))
def test_random_dense_multi_query(i, monkeypatch):
    side, B, Hq, H, R, lens, paged, n_q = draw_dense(i)
    print("case:", i, dict(side=side, B=B, Hq=Hq, H=H, R=R, lens=lens, paged=paged, n_q=n_q),
          flush=True)
    monkeypatch.setenv("KVQ_MQ_DENSE", "1")
    pr = kc.build_pair(side, side, B, Hq, H, R, lens, paged=paged, seed=700 + i,
                       extra_tokens=64 + n_q)
    for _ in range(min(n_q, 8)):  # the last query tokens are appended (windows flush where due)
        kc.step(pr)
    kc.compare_state(pr)
    kc.compare_attention_mq(pr, n_q)


@pytest.mark.parametrize("i", range(24))
def test_random_multi_query(i):
    k, v, B, Hq, H, R, lens, paged = draw(3000 + i)
    n_q = int(np.random.default_rng(8800 + i).integers(2, 13))
    lens[0] = max(lens[0], n_q)
    print("case:", i, dict(k=k, v=v, B=B, Hq=Hq, H=H, R=R, lens=lens, paged=paged, n_q=n_q),
          flush=True)
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, paged=paged, seed=900 + i, extra_tokens=64 + n_q)
    for _ in range(min(n_q, 4)):  # the last query tokens are appended (windows flush where due)
        kc.step(pr)
    kc.compare_state(pr)
    kc.compare_attention_mq(pr, n_q)
