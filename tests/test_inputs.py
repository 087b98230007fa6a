"""The seeded input recipe: determinism, distributions and structure (no GPU)."""
import numpy as np
import torch

import kvq_inputs as ki


def test_counter_generator_is_deterministic_and_offset_consistent():
    a = ki.counter_bf16(7, ki.S_K, 3, (64, 2, 128), "cpu")
    b = ki.counter_bf16(7, ki.S_K, 3, (64, 2, 128), "cpu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    tail = ki.counter_bf16(7, ki.S_K, 3, (32, 2, 128), "cpu", offset=32 * 2 * 128)
    assert torch.equal(a[32:].view(torch.int16), tail.view(torch.int16))
    c = ki.counter_bf16(7, ki.S_K, 4, (64, 2, 128), "cpu")
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_normal_and_laplace_tables():
    x = ki.counter_bf16(1, ki.S_V, 0, (1 << 20,), "cpu").float().numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01 and np.abs(x).max() < 4.5
    lap = ki.counter_bf16(1, ki.S_V, 0, (1 << 20,), "cpu", kind="laplace3").float().numpy()
    assert abs(np.median(np.abs(lap)) - 3 * np.log(2)) < 0.05   # median |X| = b ln 2


def test_workload_structure():
    w = ki.CONFIGS["c3"]
    k, v = ki.prefill_kv(w, 0, 256)
    frac = (k.float().abs() > 4.4).float().mean().item()
    assert 0.002 < frac < 0.01  # Laplace(0,3) entries beyond the normal table's reach
    w2 = ki.CONFIGS["c2"]
    ch = ki.outlier_channels(w2)
    assert len(ch) == 4 and len(set(ch)) == 4
    k2, _ = ki.prefill_kv(w2, 0, 512)
    std = k2.float().std(dim=(0, 1))
    assert all(std[c] > 10 for c in ch) and float(np.median(std.numpy())) < 1.2
    w5 = ki.CONFIGS["c5"]
    lens = ki.lengths(w5)
    assert len(lens) == 64 and min(lens) >= 1024 and max(lens) <= 131072
    assert all(lens[b] % 128 == 0 for b in range(0, 64, 16))
    tab, pool = ki.block_tables(w5, lens)
    used = tab[tab >= 0]
    assert len(used) == pool and np.array_equal(np.sort(used), np.arange(pool))
