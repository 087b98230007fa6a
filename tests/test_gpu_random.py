"""Randomised GPU parity over formats and shapes: 48 seeded cases drawn over key and value
formats (2/4/8 bits, symmetric or asymmetric, chosen independently; per-token groups of
32/64/128 channels, per-channel key groups of 16/32/64 tokens; FP8 and BF16 storage), GQA
ratios 1/2/4/8, 1-4 kv heads, windows of 0-128 tokens, lengths 0-300 per sequence, contiguous
or paged caches.  Each case: codes, scales and windows bit-exact after the prefill, attention
within the bar, one decode step (window flushes where due), both again.  The draw is fixed by
the case index, so a failure names a reproducible case."""
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
