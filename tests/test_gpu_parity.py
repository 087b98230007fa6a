"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Codes, scales, zero-points, window rows and counters must be bit-exact; attention outputs must
lie within 2e-3 + 1e-2 |ref| of the oracle's fp64 attention on the same dequantized values.
Sizes span several 16-slot tiles, several decode chunks and ragged tails.
"""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest
import torch

import kvq_cases as kc

pytestmark = pytest.mark.gpu

SYM8 = (8, 0, 0, 128)
SYM4 = (4, 0, 0, 64)
SYM2_32 = (2, 0, 0, 32)
ASYM4_32 = (4, 1, 0, 32)
ASYM2_32 = (2, 1, 0, 32)
KPC2 = (2, 1, 1, 32)
KPC4S = (4, 0, 1, 16)
BF16 = (16, 0, 0, 128)  # unquantized BF16 storage
FP8H = (8, 2, 3, 0)     # FP8 E4M3, one scale per kv head
FP8T = (8, 2, 2, 0)     # FP8 E4M3, one scale per tensor


def announce(**kw):
    print("case:", kw, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


CASES = [
    # k, v, B, Hq, H, R, lens, paged
    ("int8-mha-tiny", SYM8, SYM8, 1, 1, 1, 0, [256], False),
    ("int8-mha-ragged", SYM8, SYM8, 3, 4, 4, 0, [5, 300, 1031], False),
    # MHA 8-bit with several key groups per head (the vector-ALU QK build scales per group)
    ("int8-g32-mha-window-paged", (8, 0, 0, 32), (8, 0, 0, 32), 2, 4, 4, 64, [700, 33], True),
    ("int8-g64-mha", (8, 0, 0, 64), (8, 0, 0, 64), 2, 2, 2, 0, [1031, 300], False),
    ("int4-gqa4", SYM4, SYM4, 2, 8, 2, 0, [777, 1500], False),
    ("int4-gqa4-window", SYM4, SYM4, 2, 8, 2, 32, [777, 190], False),
    ("int4-paged-window", SYM4, SYM4, 3, 8, 2, 128, [1000, 129, 40], True),
    ("int2-sym-g32", SYM2_32, SYM2_32, 2, 4, 2, 0, [333, 64], False),
    ("asym4-g32", ASYM4_32, ASYM4_32, 2, 4, 2, 16, [250, 999], False),
    ("kivi-int2", KPC2, ASYM2_32, 2, 8, 2, 128, [700, 1300], False),
    ("kpc4-sym-g16", KPC4S, SYM4, 2, 4, 1, 32, [100, 50], False),
    ("gqa8-int8", SYM8, SYM8, 1, 16, 2, 0, [600], False),
    ("gqa2-int4-paged", SYM4, SYM4, 2, 4, 2, 0, [300, 17], True),
    ("bf16-gqa4-window", BF16, BF16, 2, 8, 2, 32, [777, 190], False),
    ("bf16-mha-paged", BF16, BF16, 3, 4, 4, 0, [300, 17, 1031], True),
    ("bf16-gqa8-paged-window", BF16, BF16, 1, 16, 2, 16, [600], True),
    ("asym8-g64-paged", (8, 1, 0, 64), (8, 1, 0, 64), 2, 8, 2, 16, [500, 77], True),
    ("fp8-head-gqa4-window", FP8H, FP8H, 2, 16, 4, 32, [777, 190], False),
    ("fp8-tensor-paged-mha", FP8T, FP8T, 3, 4, 4, 0, [300, 17, 1031], True),
    ("fp8-mixed-axes-gqa8-paged", FP8H, FP8T, 1, 16, 2, 16, [600], True),
    ("kivi-int2-paged", KPC2, ASYM2_32, 2, 8, 2, 128, [700, 1300], True),
    ("kpc4-sym-g16-paged", KPC4S, SYM4, 2, 4, 1, 32, [100, 50], True),
    ("kpc4-asym-g64-paged", (4, 1, 1, 64), (4, 1, 0, 32), 1, 8, 2, 64, [500], True),
    # asymmetric per-channel keys in 16-token groups: tiles A and B of a unit belong to two
    # groups with their own zero-point terms
    ("kpc4-asym-g16-gqa8-paged", (4, 1, 1, 16), (4, 0, 0, 128), 1, 16, 2, 16, [260], True),
    ("kpc2-asym-g16", (2, 1, 1, 16), (2, 1, 0, 32), 2, 8, 2, 32, [300, 77], False),
    # two PV row blocks (hi and lo parts of one set of value-group rows), symmetric and GQA-8
    ("int4-g32-gqa4-two-row-blocks", (4, 0, 0, 32), (4, 0, 0, 32), 2, 8, 2, 0, [345, 1200], False),
    ("kpc8-asym-gqa8-two-row-blocks", (8, 1, 1, 32), (8, 1, 0, 64), 1, 16, 2, 64, [900], False),
    # symmetric 2-bit per-channel keys: raw codes with every field scale 1..256 and a bias
    ("kpc2-sym-g64", (2, 0, 1, 64), (2, 0, 0, 32), 2, 4, 2, 128, [500, 260], False),
    # value codes as f16 subnormals: every bit width and scheme, one and two row blocks, GQA 1..8
    ("asym2-g64-per-token-keys", (2, 1, 0, 64), (2, 1, 0, 64), 2, 8, 2, 32, [613, 97], True),
    ("int2-mha-g128", (2, 0, 0, 128), (2, 0, 0, 128), 2, 4, 4, 0, [1000, 33], False),
    ("int2-g64-gqa8-two-row-blocks", (2, 0, 0, 64), (2, 0, 0, 64), 1, 16, 2, 16, [1200], False),
    ("int8-g32-gqa4-two-row-blocks", (8, 0, 0, 32), (8, 0, 0, 32), 2, 8, 2, 0, [321, 1029], True),
    ("asym8-g128-gqa2", (8, 1, 0, 128), (8, 1, 0, 128), 2, 4, 2, 64, [700, 65], False),
    # keys and values in different integer formats (bit widths and/or schemes)
    ("mix-k8-v4-gqa4-window", SYM8, SYM4, 2, 8, 2, 32, [777, 190], False),
    ("mix-k4-v2asym-paged", SYM4, ASYM2_32, 3, 8, 2, 16, [500, 77, 1000], True),
    ("mix-kivi2-v4sym", KPC2, SYM4, 2, 8, 2, 128, [700, 1300], False),
    ("mix-k4asym-v8-gqa8-paged", (4, 1, 0, 64), (8, 0, 0, 128), 1, 16, 2, 16, [600], True),
    ("mix-k2-v8asym-mha", (2, 0, 0, 32), (8, 1, 0, 64), 2, 4, 4, 0, [300, 1031], False),
    ("mix-kpc8sym-v2-paged", (8, 0, 1, 16), (2, 0, 0, 32), 2, 4, 2, 32, [200, 90], True),
    ("mix-k8asym-v8sym", (8, 1, 0, 64), SYM8, 2, 8, 2, 0, [321, 64], False),
    ("mix-k2asym-v4asym-g32", ASYM2_32, ASYM4_32, 2, 4, 2, 16, [400, 33], True),
    # more sequences than one wave scans (the prologue's workgroup-wide prefix sum)
    ("int4-batch70-ragged", SYM4, SYM4, 70, 4, 2, 16, [20 + (37 * i) % 113 for i in range(70)], True),
]


@pytest.mark.parametrize("name,k,v,B,Hq,H,R,lens,paged", CASES, ids=[c[0] for c in CASES])
def test_prefill_step_and_attention(name, k, v, B, Hq, H, R, lens, paged):
    announce(test="prefill_step_and_attention", name=name)
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, paged=paged, seed=zlib.crc32(name.encode()) % 1000)
    kc.compare_state(pr)
    kc.compare_attention(pr)
    kc.step(pr, flush_first=False)
    kc.step(pr, flush_first=True)
    kc.compare_state(pr)
    kc.compare_attention(pr, q_seed_step=1)


def test_bulk_append_equals_single_appends():
    """One n_new = 37 call equals 37 one-token calls (both compared to the oracle, which
    appends one token at a time by definition)."""
    announce(test="bulk_append")
    pr = kc.build_pair(SYM4, SYM4, 2, 8, 2, 32, [100, 100], bulk=True, seed=5)
    kc.compare_state(pr)
    kc.step(pr, n_new=37)
    kc.compare_state(pr)
    kc.compare_attention(pr)
    pr2 = kc.build_pair(KPC2, ASYM2_32, 1, 4, 1, 64, [70], seed=6)
    kc.step(pr2, n_new=150)
    kc.compare_state(pr2)
    kc.compare_attention(pr2)


def test_window_edge_states():
    """Windows exactly full, empty compressed part, single token."""
    announce(test="window_edges")
    pr = kc.build_pair(SYM4, SYM4, 4, 8, 2, 32, [32, 1, 33, 64])
    kc.compare_state(pr)
    kc.compare_attention(pr)
    for _ in range(3):
        kc.step(pr)
    kc.compare_state(pr)
    kc.compare_attention(pr)


# Uniform batches use segment-aligned unit ranges; a forced grid size drives each choice:
# segments split m ways, k whole segments per range (k dividing S), and the fall-back to plain
# ranges when no aligned count keeps half of the workgroups.
ALIGN_CASES = [
    # name, k, v, B, Hq, H, R, lens, workgroups
    ("segments-split-2-ways", SYM4, SYM4, 2, 8, 4, 0, [700, 700], 20),
    ("two-segments-per-range", SYM4, SYM4, 2, 8, 4, 0, [700, 700], 7),
    ("four-segments-per-range-window", SYM8, SYM8, 2, 4, 4, 32, [650, 650], 3),
    ("prime-segment-count-falls-back", SYM4, SYM4, 7, 2, 1, 0, [300] * 7, 5),
    ("uniform-with-empty-sequence", SYM4, SYM4, 3, 8, 2, 0, [0, 500, 500], 5),
    ("ragged-keeps-plain-ranges", SYM4, SYM4, 3, 8, 2, 0, [100, 500, 500], 5),
    # one workgroup: no combine launch; it writes the empty sequence's zeros itself
    ("single-workgroup-with-empty-sequence", SYM4, SYM4, 3, 8, 2, 32, [300, 0, 77], 1),
    ("single-workgroup-kivi", KPC2, ASYM2_32, 2, 8, 2, 64, [200, 90], 1),
]


@pytest.mark.parametrize("name,k,v,B,Hq,H,R,lens,nb", ALIGN_CASES, ids=[c[0] for c in ALIGN_CASES])
def test_unit_range_choices(name, k, v, B, Hq, H, R, lens, nb, monkeypatch):
    announce(test="unit_range_choices", name=name, workgroups=nb)
    monkeypatch.setenv("KVQ_DECODE_BLOCKS", str(nb))
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, seed=zlib.crc32(name.encode()) % 1000)
    kc.compare_attention(pr)
    kc.step(pr, flush_first=False)
    kc.compare_attention(pr, q_seed_step=1)


def test_more_workgroups_than_units(monkeypatch):
    """A max_tokens far above the lengths sizes the grid for units that do not exist: most unit
    ranges are empty, and the empty ones that start inside a segment count in a neutral partial."""
    announce(test="more_workgroups_than_units")
    monkeypatch.setenv("KVQ_DECODE_BLOCKS", "64")
    pr = kc.build_pair(SYM4, SYM4, 2, 8, 2, 0, [100, 40], seed=31)
    kc.compare_attention(pr, max_tokens=4096)
    pr = kc.build_pair(SYM4, SYM4, 2, 8, 2, 32, [130, 7], seed=32)
    kc.compare_attention_mq(pr, 9, max_tokens=4096)


def test_workspace_needs_no_initialisation():
    """One workspace filled with garbage serves calls of different shapes in a row: nothing in
    it is read before the call writes it."""
    announce(test="workspace_reuse")
    K = kc.kvq()
    a = kc.build_pair(SYM4, SYM4, 3, 8, 2, 0, [900, 40, 333], seed=5)
    b = kc.build_pair(KPC2, ASYM2_32, 2, 8, 2, 128, [700, 1300], seed=6)
    c = kc.build_pair(SYM4, SYM4, 2, 8, 2, 32, [777, 190], seed=7)
    mt = lambda pr: max(s.n_quant + s.n_res for s in pr.seqs)
    need = max(K.workspace_bytes(a.cache, 8, mt(a)), K.workspace_bytes(b.cache, 8, mt(b)),
               K.workspace_bytes_mq(c.cache, 8, 9, mt(c)))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        kc.compare_attention(a, q_seed_step=rep, workspace=ws)
        kc.compare_attention(b, q_seed_step=rep, workspace=ws)
        kc.compare_attention_mq(c, 9, workspace=ws)


# Mixed-length batches with windows: a window unit counts its bytes' weight in units (and every
# segment opens with slots of no work), so range boundaries fall inside window units and inside
# those slots; forced grid sizes move them around.
WINDOW_SPLIT_CASES = [
    # name, k, v, B, Hq, H, R, lens, workgroups
    ("int4-window-split-7", SYM4, SYM4, 3, 8, 2, 64, [150, 47, 300], 7),
    ("int4-window-split-13", SYM4, SYM4, 3, 8, 2, 64, [150, 47, 300], 13),
    ("int2-window-split-11", SYM2_32, SYM2_32, 3, 4, 2, 96, [130, 75, 200], 11),
    ("int8-window-split-5", SYM8, SYM8, 2, 4, 4, 128, [600, 100], 5),
    ("kivi-window-split-9", KPC2, ASYM2_32, 2, 8, 2, 128, [700, 300], 9),
]


@pytest.mark.parametrize("name,k,v,B,Hq,H,R,lens,nb", WINDOW_SPLIT_CASES, ids=[c[0] for c in WINDOW_SPLIT_CASES])
def test_window_units_split_across_ranges(name, k, v, B, Hq, H, R, lens, nb, monkeypatch):
    announce(test="window_split", name=name, workgroups=nb)
    monkeypatch.setenv("KVQ_DECODE_BLOCKS", str(nb))
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, seed=zlib.crc32(name.encode()) % 1000)
    kc.compare_attention(pr)
    kc.step(pr, flush_first=False)
    kc.compare_attention(pr, q_seed_step=1)


def test_empty_sequence_gives_zeros():
    announce(test="empty_sequence")
    pr = kc.build_pair(SYM8, SYM8, 3, 2, 2, 0, [0, 40, 0])
    err, got = kc.compare_attention(pr, max_tokens=64)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    # small enough for one workgroup (two units per wave at most): the decode launch alone
    pr = kc.build_pair(SYM8, SYM8, 2, 1, 1, 0, [0, 40])
    err, got = kc.compare_attention(pr, max_tokens=40)
    assert np.all(got[0] == 0)


def test_deterministic_and_paged_equals_contiguous():
    announce(test="determinism_paging")
    a = kc.build_pair(SYM4, SYM4, 2, 8, 2, 128, [900, 333], paged=False, seed=9)
    b = kc.build_pair(SYM4, SYM4, 2, 8, 2, 128, [900, 333], paged=True, seed=9)
    _, o1 = kc.compare_attention(a)
    _, o2 = kc.compare_attention(a)
    assert np.array_equal(o1, o2)
    _, o3 = kc.compare_attention(b)
    assert np.array_equal(o1, o3)


def test_device_faults_leave_other_sequences_intact():
    """A block-table entry outside the pool and a full contiguous cache set error bits; the
    faulty sequence's counters do not move and the other sequences proceed."""
    announce(test="device_faults")
    K = kc.kvq()
    pr = kc.build_pair(SYM4, SYM4, 2, 4, 2, 0, [30, 30], paged=True, seed=12, extra_tokens=16)
    bad = pr.cache.block_table.clone()
    bad[1, 1] = pr.num_blocks + 5  # slot 30's block for sequence 1 is now outside the pool
    pr.cache.block_table.copy_(bad)
    pr.cache.desc = pr.cache._describe()
    nq0 = pr.cache.n_quant.cpu().tolist()
    k, v = kc.ki.step_kv(pr.w, 0)
    K.quantize_append(pr.cache, k.cuda().contiguous(), v.cuda().contiguous())
    torch.cuda.synchronize()
    assert K.read_error(pr.cache) & K.ERR_BLOCK
    nq1 = pr.cache.n_quant.cpu().tolist()
    assert nq1[1] == nq0[1] and nq1[0] == nq0[0] + 1
    # contiguous cache that is full
    pr2 = kc.build_pair(SYM8, SYM8, 2, 2, 2, 0, [16, 5], capacity=16, seed=13)
    k, v = kc.ki.step_kv(pr2.w, 0)
    K.quantize_append(pr2.cache, k.cuda().contiguous(), v.cuda().contiguous())
    torch.cuda.synchronize()
    assert K.read_error(pr2.cache) & K.ERR_CAPACITY
    assert pr2.cache.n_quant.cpu().tolist() == [16, 6]


def test_per_channel_flush_inside_a_group_is_refused():
    """Per-channel keys: a sequence whose n_quant is not a multiple of the key group (a corrupt
    or misaligned prefix) would flush into the middle of a group.  The append sets
    KVQ_ERR_GROUP, writes nothing of that sequence and leaves its counters; the other sequence
    flushes and appends as usual."""
    announce(test="per_channel_group_fault")
    K = kc.kvq()
    pr = kc.build_pair(KPC2, ASYM2_32, 2, 8, 2, 64, [64, 64], seed=44)
    kc.compare_state(pr)
    pr.cache.n_quant[1] = 16  # not a multiple of the 32-token key group; window full (64)
    codes0 = pr.cache.k_codes.clone()
    k, v = kc.ki.step_kv(pr.w, 0)
    K.quantize_append(pr.cache, k.cuda().contiguous(), v.cuda().contiguous())
    torch.cuda.synchronize()
    assert K.read_error(pr.cache) & K.ERR_GROUP
    assert pr.cache.n_quant.tolist() == [64, 16] and pr.cache.n_res.tolist() == [1, 64]
    # sequence 1's slots (the second half of the contiguous buffer) are untouched
    half = codes0.numel() // 2
    assert torch.equal(pr.cache.k_codes[half:], codes0[half:])


def test_prefix_shared_blocks_are_read_not_written():
    """Prefix sharing through the block table [P2, "How this connects to paging and prefix
    caching"]: sequence 1 maps sequence 0's first P/16 physical blocks (its compressed prefix,
    per-channel key metadata included) and sets its counters to (P, 0); then both sequences
    take their own single-token steps, with window flushes.  Codes, metadata and windows equal
    two oracle sequences (the second = the same P tokens, flushed, then its own tokens), the
    shared blocks never change, and both attention outputs match."""
    announce(test="prefix_sharing")
    K = kc.kvq()
    k_side, v_side, R, H, Hq, P = KPC2, ASYM2_32, 64, 2, 8, 256
    w = kc.ki.Workload("share", 21, 2, Hq, H, P + 10, kc.ki.Side(*k_side), kc.ki.Side(*v_side),
                       residual=R, paged=True)
    nbs = (P + 10 + R + 160) // 16 + 1  # logical blocks per sequence
    pool = 2 * nbs
    perm = np.random.default_rng(3).permutation(pool).astype(np.int32)
    table = np.full((2, nbs), -1, np.int32)
    table[0] = perm[:nbs]
    table[1, :P // 16] = table[0, :P // 16]  # shared prefix blocks
    table[1, P // 16:] = perm[nbs:2 * nbs - P // 16]
    cache = K.Cache(k_side, v_side, 2, H, residual=R, block_table=torch.from_numpy(table),
                    num_blocks=pool)
    k, v = kc.ki.prefill_kv(w, 0, P + 10)
    K.quantize_append(cache, k[None].cuda().contiguous(), v[None].cuda().contiguous(),
                      desc=cache.sequence(0))
    torch.cuda.synchronize()
    assert cache.n_quant.tolist() == [P, 0] and cache.n_res.tolist() == [10, 0]
    cache.n_quant[1] = P  # sequence 1 adopts the compressed prefix
    s0 = kc.oracle.Sequence(k_side, v_side, H, R, nbs * 16)
    s1 = kc.oracle.Sequence(k_side, v_side, H, R, nbs * 16)
    s0.append(kc.ki.bf16_bits(k), kc.ki.bf16_bits(v))
    s1.append(kc.ki.bf16_bits(k[:P]), kc.ki.bf16_bits(v[:P]))
    s1.flush()
    assert (s1.n_quant, s1.n_res) == (P, 0)
    shared = [int(bk) for bk in table[0, :P // 16]]
    tile_bytes = 16 * 128 * k_side[0] // 8

    def shared_bytes():
        kcodes = cache.k_codes.cpu().numpy().reshape(pool * H, tile_bytes)
        ks = kc._u16(cache.k_scale).reshape(pool, H, 128)
        return [kcodes[[bk * H + h for bk in shared for h in range(H)]].copy(), ks[shared].copy()]

    before = shared_bytes()
    pr = kc.Pair(w, cache, [s0, s1], [P + 10, P], table, pool, 0)
    for _ in range(90):  # each sequence flushes its window once, into its own blocks
        kc.step(pr)
    kc.compare_state(pr)
    after = shared_bytes()
    assert all(np.array_equal(x, y) for x, y in zip(before, after))
    assert cache.n_quant.tolist() == [s0.n_quant, s1.n_quant] == [P + R, P + R]
    kc.compare_attention(pr)


MQ_CASES = [
    # name, k, v, B, Hq, H, R, lens, paged, n_q (queries per sequence)
    ("mq-int4-gqa4-window", SYM4, SYM4, 2, 8, 2, 32, [777, 190], False, 16),
    ("mq-int8-mha-paged", SYM8, SYM8, 3, 4, 4, 0, [300, 17, 1031], True, 5),
    ("mq-kivi-int2", KPC2, ASYM2_32, 2, 8, 2, 128, [700, 1300], False, 8),
    ("mq-fp8-gqa8-paged", FP8H, FP8H, 1, 16, 2, 16, [600], True, 3),
    ("mq-bf16-gqa2", BF16, BF16, 2, 4, 2, 0, [333, 64], False, 16),
    # one query block per wave, with idle waves in the last group and a sequence shorter than n_q
    ("mq-int4-gqa4-ragged-idle-waves", SYM4, SYM4, 3, 8, 2, 16, [50, 3, 200], False, 13),
    ("mq-int4-paged-idle-waves", SYM4, SYM4, 2, 8, 2, 32, [900, 70], True, 9),
    ("mq-int8-g32-two-row-blocks", (8, 0, 0, 32), (8, 0, 0, 32), 2, 8, 2, 0, [400, 1100], False, 12),
    # two query blocks of two waves each (2 or 3 blocks per sequence and kv head)
    ("mq-int4-gqa4-two-blocks", SYM4, SYM4, 2, 8, 2, 32, [777, 190], False, 4),
    ("mq-kivi-int2-three-blocks", KPC2, ASYM2_32, 2, 8, 2, 128, [700, 1300], False, 3),
    ("mq-asym4-paged-two-blocks", ASYM4_32, ASYM4_32, 2, 4, 2, 16, [250, 999], True, 3),
    # keys and values in different formats (query blocks of the blocked kernel: four blocks of one
    # wave, two of two waves, one of four)
    ("mq-mix-k8-v4-gqa4-window", SYM8, SYM4, 2, 8, 2, 32, [777, 190], False, 16),
    ("mq-mix-k4-v2asym-paged", SYM4, ASYM2_32, 3, 8, 2, 16, [500, 77, 1000], True, 3),
    ("mq-mix-kivi2-v4sym", KPC2, SYM4, 2, 8, 2, 128, [700, 1300], False, 2),
    ("mq-mix-k2-v8asym-mha", (2, 0, 0, 32), (8, 1, 0, 64), 2, 4, 4, 0, [300, 1031], False, 5),
    ("mq-mix-k4asym-v8-gqa8-paged", (4, 1, 0, 64), SYM8, 1, 16, 2, 16, [600], True, 4),
    # the dense kernel: 16 query rows per wave, four blocks per workgroup (key groups of 64 or
    # 128); it takes 64 or more rows per kv head by itself, and these cases force it from 16 rows
    # on (KVQ_MQ_DENSE=1) for idle waves, partial blocks and segments split over workgroups
    ("mq-dense-asym4-g64-gqa4", (4, 1, 0, 64), (4, 1, 0, 64), 2, 8, 2, 32, [600, 130], False, 8),
    ("mq-dense-int8-mha-paged", SYM8, SYM8, 2, 2, 2, 16, [500, 77], True, 16),
    ("mq-dense-int2-g64-gqa8", (2, 0, 0, 64), (2, 0, 0, 64), 1, 16, 2, 0, [900], False, 4),
    ("mq-dense-asym8-gqa2-long", (8, 1, 0, 128), (8, 1, 0, 128), 1, 4, 2, 128, [3000], False, 32),
    ("mq-dense-int4-gqa4-two-segments", SYM4, SYM4, 2, 8, 2, 0, [700, 1500], False, 24),
    ("mq-dense-asym2-g64-paged-window", (2, 1, 0, 64), (2, 1, 0, 64), 2, 8, 2, 64, [333, 1100], True, 5),
    ("mq-dense-int2-g32-gqa4", (2, 0, 0, 32), (2, 0, 0, 32), 2, 8, 2, 0, [900, 260], False, 16),
    ("mq-dense-asym4-g32-paged-window", (4, 1, 0, 32), (4, 1, 0, 32), 2, 16, 2, 32, [700, 90], True, 4),
    ("mq-dense-asym8-g32-mha", (8, 1, 0, 32), (8, 1, 0, 32), 1, 2, 2, 0, [1200], False, 17),
    ("mq-dense-int4-k64-v32-window", (4, 0, 0, 64), (4, 0, 0, 32), 2, 8, 2, 32, [500, 140], False, 8),
    ("mq-dense-asym2-k128-v64-paged", (2, 1, 0, 128), (2, 1, 0, 64), 2, 4, 2, 16, [420, 77], True, 12),
    ("mq-dense-fp8-head-gqa4-window", (8, 2, 3, 0), (8, 2, 3, 0), 2, 8, 2, 32, [600, 45], False, 8),
    ("mq-dense-fp8-tensor-mha-paged", (8, 2, 2, 0), (8, 2, 2, 0), 2, 4, 4, 16, [333, 700], True, 16),
    ("mq-dense-fp8-k-head-v-tensor-gqa8", (8, 2, 3, 0), (8, 2, 2, 0), 1, 16, 2, 0, [1000], False, 3),
    ("mq-dense-bf16-gqa4-window", BF16, BF16, 2, 8, 2, 32, [500, 61], False, 8),
    ("mq-dense-bf16-mha-paged", BF16, BF16, 2, 2, 2, 16, [300, 777], True, 19),
    ("mq-dense-int2-g64-paged-window", (2, 0, 0, 64), (2, 0, 0, 64), 2, 8, 2, 64, [777, 1300], True, 9),
    ("mq-dense-int2-g128-gqa4", (2, 0, 0, 128), (2, 0, 0, 128), 1, 8, 2, 0, [640], False, 16),
]


@pytest.mark.parametrize("name,k,v,B,Hq,H,R,lens,paged,nq", MQ_CASES, ids=[c[0] for c in MQ_CASES])
def test_multi_query_decode(name, k, v, B, Hq, H, R, lens, paged, nq, monkeypatch):
    """Multi-query decode: append the n_q query tokens (single-token steps, so windows flush
    where due), then attend with each query seeing the tokens up to its own."""
    announce(test="multi_query", name=name)
    if name.startswith("mq-dense"):
        monkeypatch.setenv("KVQ_MQ_DENSE", "1")
    pr = kc.build_pair(k, v, B, Hq, H, R, lens, paged=paged, seed=zlib.crc32(name.encode()) % 1000,
                       extra_tokens=64 + nq)
    for _ in range(nq):
        kc.step(pr)
    kc.compare_state(pr)
    kc.compare_attention_mq(pr, nq)


def test_multi_query_edges():
    """n_q = 1 is single-query decode bit for bit; queries that precede every cached token of
    their sequence (a sequence shorter than n_q) get zeros."""
    announce(test="multi_query_edges")
    K = kc.kvq()
    pr = kc.build_pair(SYM4, SYM4, 3, 8, 2, 16, [50, 3, 200], seed=31, extra_tokens=80)
    q1 = kc.mq_queries(pr, 1)
    mt = max(s.n_quant + s.n_res for s in pr.seqs)
    a = K.decode_attention_mq(pr.cache, q1, max_tokens=mt, sm_scale=kc.SM_SCALE)
    b_ = K.decode_attention(pr.cache, q1[:, 0].contiguous(), max_tokens=mt, sm_scale=kc.SM_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b_)
    _, got = kc.compare_attention_mq(pr, 6)
    assert np.all(got[1, :3] == 0) and np.any(got[1, 3] != 0)  # sequence 1 holds 3 tokens
