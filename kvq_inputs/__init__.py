"""Seeded synthetic inputs and the workload table for the quantized KV cache.

This module holds only the input recipe: shapes, formats, value distributions and a
counter-based generator.  It contains none of the method's arithmetic (no quantizer, no
attention) and is the only code that both the GPU path's tests/benchmark and the CPU oracle's
callers share.

Generator: every bf16 element is a pure function of (config seed, stream, sequence, token,
head, channel).  A 32-bit integer hash of that counter picks one of 65536 equiprobable
quantiles of the target distribution (a table of bf16 values computed once in fp64), so the
same torch code yields bit-identical tensors on the CPU and on the GPU.  The N(0, 1) table is
truncated at about +-4.3 sigma (the 0.5/65536 quantile).
"""
from __future__ import annotations

import dataclasses
import math
from statistics import NormalDist

import numpy as np
import torch

D_HEAD = 128
SYM, ASYM = 0, 1
PER_TOKEN, PER_CHANNEL = 0, 1

# streams
S_K, S_V, S_Q, S_KNEW, S_VNEW, S_MASK, S_LAPLACE, S_CHANNELS, S_LEN, S_PERM = range(10)

_M32 = 0xFFFFFFFF


def hash32_int(x: int) -> int:
    """32-bit integer mixing hash (two multiply-xorshift rounds), on Python ints."""
    x &= _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def hash32(x: torch.Tensor) -> torch.Tensor:
    """Same hash on an int64 tensor holding values in [0, 2^32); products stay below 2^59."""
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def _salt(seed: int, stream: int, seq: int) -> tuple[int, int]:
    a = hash32_int(seed * 1000003 + stream * 7919 + seq * 104729 + 0x9E3779B9)
    b = hash32_int(a ^ 0x85EBCA6B ^ (seq * 31 + stream))
    return a, b


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16  # round to nearest even
    return r.astype(np.uint16)


def _table(kind: str) -> np.ndarray:
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    if kind == "normal":
        nd = NormalDist()
        z = np.array([nd.inv_cdf(v) for v in p])
    elif kind == "laplace3":  # Laplace(0, b=3)
        z = -3.0 * np.sign(p - 0.5) * np.log(1.0 - 2.0 * np.abs(p - 0.5))
    else:
        raise ValueError(kind)
    return _f32_to_bf16_bits(z.astype(np.float32))


_TABLES: dict = {}


def table(kind: str, device) -> torch.Tensor:
    key = (kind, str(device))
    if key not in _TABLES:
        host = _TABLES.get((kind, "cpu-np"))
        if host is None:
            host = _table(kind)
            _TABLES[(kind, "cpu-np")] = host
        _TABLES[key] = torch.from_numpy(host.view(np.int16).copy()).to(device)
    return _TABLES[key]


def counter_bf16(seed: int, stream: int, seq: int, shape, device, kind: str = "normal",
                 offset: int = 0) -> torch.Tensor:
    """bf16 tensor of `shape`; element with flat index i uses counter offset + i."""
    n = int(np.prod(shape))
    a, b = _salt(seed, stream, seq)
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    u = hash32(hash32((idx & _M32) ^ a) ^ b)
    vals = table(kind, device)[u >> 16]
    return vals.view(torch.bfloat16).reshape(shape)


def counter_u32(seed: int, stream: int, seq: int, n: int, device="cpu", offset: int = 0):
    a, b = _salt(seed, stream, seq)
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    return hash32(hash32((idx & _M32) ^ a) ^ b)


@dataclasses.dataclass(frozen=True)
class Side:
    bits: int
    scheme: int = SYM
    axis: int = PER_TOKEN
    group: int = 128

    def astuple(self):
        return (self.bits, self.scheme, self.axis, self.group)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    tokens: int                    # cached tokens before the step (c5: upper bound)
    k: Side
    v: Side
    residual: int = 0
    paged: bool = False
    k_outlier_channels: int = 0    # number of persistent key outlier channels
    k_outlier_scale: float = 1.0
    laplace_outliers: float = 0.0  # fraction of entries replaced by Laplace(0, 3)
    step_append: bool = False      # the step appends one token (and flushes where due)
    mixed_lengths: bool = False    # log-uniform lengths in [1024, tokens]
    description: str = ""

    @property
    def group_q(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    "c1": Workload("c1", 1, 1, 1, 1, 256, Side(8, SYM, PER_TOKEN, 128), Side(8, SYM, PER_TOKEN, 128),
                   description="tiny: batch 1, H_q=H_kv=1, T=256, INT8 symmetric per-token group 128"),
    "c2": Workload("c2", 2, 1, 32, 8, 8192, Side(4, SYM, PER_TOKEN, 64), Side(4, SYM, PER_TOKEN, 64),
                   k_outlier_channels=4, k_outlier_scale=20.0,
                   description="worked-example layer: batch 1, H_q=32, H_kv=8, T=8192, INT4 "
                               "symmetric group 64, fp16 scale, 4 key outlier channels x20"),
    "c3": Workload("c3", 3, 32, 32, 32, 2048, Side(8, SYM, PER_TOKEN, 128), Side(8, SYM, PER_TOKEN, 128),
                   laplace_outliers=0.01, step_append=True,
                   description="MHA 7B-like layer: batch 32, H=32/32, T=2048, INT8 symmetric "
                               "per-token group 128, 1% Laplace(0,3) outliers, append 1"),
    "c4": Workload("c4", 4, 16, 32, 8, 32768, Side(2, ASYM, PER_CHANNEL, 32), Side(2, ASYM, PER_TOKEN, 32),
                   residual=128, k_outlier_channels=4, k_outlier_scale=15.0, step_append=True,
                   description="KIVI-style 2-bit asymmetric: batch 16, H_q=32, H_kv=8, T=32768, "
                               "keys per-channel over 32 tokens, values per-token groups of 32, "
                               "BF16 window 128, key outlier channels x15"),
    "c4p": Workload("c4p", 4, 16, 32, 8, 32768, Side(2, ASYM, PER_CHANNEL, 32), Side(2, ASYM, PER_TOKEN, 32),
                    residual=128, k_outlier_channels=4, k_outlier_scale=15.0, step_append=True,
                    paged=True,
                    description="KIVI-style 2-bit asymmetric, paged: the c4 batch (same inputs) "
                                "in 16-token blocks of a shuffled pool, per-channel key metadata "
                                "kept with each group's first block"),
    "c5": Workload("c5", 5, 64, 32, 8, 131072, Side(4, SYM, PER_TOKEN, 64), Side(4, SYM, PER_TOKEN, 64),
                   residual=128, paged=True, step_append=True, mixed_lengths=True,
                   description="paged mixed batch: 64 sequences, lengths log-uniform in "
                               "[1024, 131072], block 16, H_q=32, H_kv=8, INT4 group 64, "
                               "BF16 window 128"),
}


def outlier_channels(w: Workload) -> list[int]:
    if not w.k_outlier_channels:
        return []
    u = counter_u32(w.seed, S_CHANNELS, 0, D_HEAD).numpy()
    return sorted(int(c) for c in np.argsort(u, kind="stable")[: w.k_outlier_channels])


def lengths(w: Workload) -> list[int]:
    """Cached tokens per sequence before the step."""
    if not w.mixed_lengths:
        return [w.tokens] * w.batch
    lo, hi = math.log(1024), math.log(w.tokens)
    out = []
    for b in range(w.batch):
        u = counter_u32(w.seed, S_LEN, b, 2).numpy()
        x = (int(u[0]) * 2.0**32 + int(u[1]) + 0.5) / 2.0**64
        out.append(int(math.floor(math.exp(lo + x * (hi - lo)))))
    if w.residual:
        # a quarter of the sequences end on a window boundary, so the step flushes them
        for b in range(0, w.batch, 16):
            out[b] = min(w.tokens, w.residual * -(-out[b] // w.residual))
    return out


def _kv_values(w: Workload, stream: int, seq: int, shape, device, offset: int, is_key: bool):
    x = counter_bf16(w.seed, stream, seq, shape, device, offset=offset)
    if w.laplace_outliers:
        n = int(np.prod(shape))
        m = counter_u32(w.seed, S_MASK + 16 * stream, seq, n, device, offset=offset)
        lap = counter_bf16(w.seed, S_LAPLACE + 16 * stream, seq, shape, device, "laplace3", offset)
        thresh = int(round(w.laplace_outliers * 65536))
        x = torch.where((m & 0xFFFF).reshape(shape) < thresh, lap, x)
    if is_key and w.k_outlier_channels:
        ch = torch.tensor(outlier_channels(w), device=device)
        xs = x.float()
        xs[..., ch] = xs[..., ch] * w.k_outlier_scale
        x = xs.to(torch.bfloat16)
    return x


def prefill_kv(w: Workload, seq: int, n_tokens: int, device="cpu", t0: int = 0):
    """K and V rows of tokens [t0, t0 + n_tokens) of sequence `seq`: bf16 [n][H_kv][d]."""
    shape = (n_tokens, w.n_kv_heads, D_HEAD)
    off = t0 * w.n_kv_heads * D_HEAD
    k = _kv_values(w, S_K, seq, shape, device, off, True)
    v = _kv_values(w, S_V, seq, shape, device, off, False)
    return k, v


def step_kv(w: Workload, step: int, device="cpu"):
    """The token appended by decode step `step`: bf16 [B][1][H_kv][d] for K and V."""
    shape = (1, w.n_kv_heads, D_HEAD)
    ks, vs = [], []
    for b in range(w.batch):
        off = step * w.n_kv_heads * D_HEAD
        ks.append(_kv_values(w, S_KNEW, b, shape, device, off, True))
        vs.append(_kv_values(w, S_VNEW, b, shape, device, off, False))
    return torch.stack(ks), torch.stack(vs)


def queries(w: Workload, step: int = 0, device="cpu"):
    """bf16 [B][H_q][d]."""
    shape = (w.batch, w.n_q_heads, D_HEAD)
    return counter_bf16(w.seed, S_Q, step, shape, device)


def block_tables(w: Workload, lens: list[int], extra_tokens: int = 256, block: int = 16):
    """Per-sequence block tables over a shared pool, in shuffled physical order.

    Sequence b gets ceil((len_b + residual + extra_tokens) / block) logical blocks; physical
    ids are a seeded permutation of the pool.  Returns (table int32 [B][max_blocks] with -1 in
    unused entries, num_blocks)."""
    nb = [-(-(n + w.residual + extra_tokens) // block) for n in lens]
    pool = int(sum(nb))
    u = counter_u32(w.seed, S_PERM, 0, pool).numpy()
    perm = np.argsort(u, kind="stable").astype(np.int32)
    maxb = max(nb)
    tab = np.full((len(lens), maxb), -1, np.int32)
    pos = 0
    for b, n in enumerate(nb):
        tab[b, :n] = perm[pos:pos + n]
        pos += n
    return tab, pool


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor (for the oracle)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
