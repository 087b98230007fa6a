"""The C-ABI library without a GPU: it loads, exports every function its headers declare, sizes
buffers like the storage layout the oracle writes, and rejects host-detectable misuse with a
status before launching anything."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    from quantized_kv_cache_07_amd import kvq
    return kvq


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(kvq_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(K):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(K.lib, n), n
    assert sorted(K.EXPORTS) == names


@pytest.mark.parametrize("k,v,R", [((4, 0, 0, 64), (4, 0, 0, 64), 0),
                                   ((8, 0, 0, 128), (8, 0, 0, 128), 16),
                                   ((2, 1, 1, 32), (2, 1, 0, 32), 128),
                                   ((4, 1, 0, 32), (4, 1, 0, 32), 32),
                                   ((16, 0, 0, 128), (16, 0, 0, 128), 16),
                                   ((8, 2, 3, 0), (8, 2, 2, 0), 16),
                                   ((8, 0, 0, 64), (4, 1, 0, 32), 16),
                                   ((4, 1, 0, 64), (2, 0, 0, 32), 0),
                                   ((2, 1, 1, 32), (4, 0, 0, 64), 64)])
def test_buffer_sizes_match_the_storage_layout(K, orc, k, v, R):
    fmt = K.make_format(k, v, R)
    B, H = 3, 2
    for cap, nblk in ((256, 0), (0, 40)):
        im = orc.empty_images(k, v, B, H, R, capacity=cap, num_blocks=nblk)
        for which, name in enumerate(["k_codes", "v_codes", "k_scale", "v_scale", "k_zero",
                                      "v_zero", "k_res", "v_res"]):
            got = K.lib.kvq_buffer_bytes(ctypes.byref(fmt), B, H, cap, nblk, which)
            side = k if name[0] == "k" else v
            if side[1] == 2 and name.endswith("scale"):  # FP8: fp32 scale per head or tensor
                assert got == 4 * (H if side[2] == 3 else 1)
            elif side[1] == 2 and name.endswith("zero"):
                assert got == 0
            elif name == "k_zero" and k[2] == 0 and v[1] == 1:
                assert got == im[name].nbytes > 0  # shared record: the values' zero rows
            elif name.endswith("zero") and side[1] == 0:
                assert got == 0
            elif name.endswith("res") and R == 0:
                assert got == 0
            else:
                assert got == im[name].nbytes, (name, got, im[name].nbytes)


def test_worked_example_footprint(K):
    """One layer of the worked example (H_kv=8, T=8192, INT4, one fp16 scale per 64 elements),
    times 32 layers, is the 272 MiB of the page's worked example."""
    fmt = K.make_format((4, 0, 0, 64), (4, 0, 0, 64), 0)
    per_layer = sum(K.lib.kvq_buffer_bytes(ctypes.byref(fmt), 1, 8, 8192, 0, w) for w in range(4))
    assert per_layer * 32 == 272 * 2**20


@pytest.mark.parametrize("k,v,R,status", [
    ((4, 0, 0, 64), (4, 0, 0, 64), 0, 0),
    ((3, 0, 0, 64), (3, 0, 0, 64), 0, 2),
    ((4, 0, 0, 48), (4, 0, 0, 64), 0, 2),
    ((4, 0, 1, 32), (4, 0, 0, 64), 0, 1),     # per-channel keys need a window
    ((4, 0, 1, 32), (4, 0, 0, 64), 48, 1),    # ... whose length the group divides
    ((4, 0, 0, 64), (4, 0, 1, 32), 64, 2),    # per-channel values are not implemented
    ((8, 0, 0, 64), (4, 0, 0, 64), 0, 0),     # K and V widths chosen independently
    ((2, 1, 1, 32), (4, 0, 0, 32), 64, 0),    # ... and schemes
    ((4, 0, 0, 64), (8, 1, 0, 128), 0, 0),
    ((4, 2, 0, 64), (4, 0, 0, 64), 0, 1),
    ((4, 0, 0, 64), (4, 0, 0, 64), 24, 1),    # window not a multiple of 16
    ((16, 0, 0, 128), (16, 0, 0, 128), 0, 0),  # unquantized BF16 cache
    ((16, 0, 0, 128), (16, 0, 0, 128), 32, 0),
    ((16, 1, 0, 128), (16, 1, 0, 128), 0, 1),  # BF16 storage has no scheme ...
    ((16, 0, 0, 64), (16, 0, 0, 64), 0, 1),    # ... and no groups
    ((16, 0, 0, 128), (8, 0, 0, 128), 0, 2),   # BF16 storage on one side only
    ((8, 2, 3, 0), (8, 2, 2, 0), 16, 0),       # FP8 E4M3: per-head keys, per-tensor values
    ((8, 2, 0, 0), (8, 2, 0, 0), 0, 1),        # FP8 scales are per tensor or per head
    ((8, 2, 3, 64), (8, 2, 3, 0), 0, 1),       # ... with no group
    ((4, 2, 3, 0), (4, 2, 3, 0), 0, 1),        # ... on 8-bit codes
    ((8, 2, 3, 0), (8, 0, 0, 128), 0, 2),      # FP8 on one side only
])
def test_check_format(K, k, v, R, status):
    fmt = K.make_format(k, v, R)
    assert K.lib.kvq_check_format(ctypes.byref(fmt)) == status


def fake_cache(K, **over):
    d = K.CacheDesc()
    d.fmt = K.make_format((4, 0, 0, 64), (4, 0, 0, 64), 32)
    d.batch, d.n_kv_heads, d.capacity = 2, 2, 256
    for i, name in enumerate(("k_codes", "v_codes", "k_scale", "v_scale", "k_res", "v_res",
                              "n_quant", "n_res", "err")):
        setattr(d, name, 0x100000 + 0x1000 * i)  # never dereferenced on these paths
    for key, val in over.items():
        setattr(d, key, val)
    return d


def test_host_errors_return_before_launch(K):
    L = K.lib
    d = fake_cache(K)
    assert L.kvq_quantize_append(None, 0x1000, 0x1000, 1, None) == 1
    assert L.kvq_quantize_append(ctypes.byref(d), 0x1000, 0x1000, 0, None) == 1
    assert L.kvq_quantize_append(ctypes.byref(d), 0x1008, 0x1000, 1, None) == 3
    assert L.kvq_quantize_append(ctypes.byref(fake_cache(K, k_codes=0x100004)), 0x1000, 0x1000, 1,
                                 None) == 3
    assert L.kvq_quantize_append(ctypes.byref(fake_cache(K, k_res=None)), 0x1000, 0x1000, 1,
                                 None) == 1
    assert L.kvq_quantize_append(ctypes.byref(fake_cache(K, capacity=100)), 0x1000, 0x1000, 1,
                                 None) == 1
    assert L.kvq_flush_residual(ctypes.byref(fake_cache(K, err=None)), None) == 1
    ws = L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 1000)
    assert ws > 0
    assert L.kvq_decode_attention(ctypes.byref(d), 0x1000, 8, 0.1, 1000, 0x2000, 0x3000, ws - 1,
                                  None) == 4
    assert L.kvq_decode_attention(ctypes.byref(d), 0x1000, 5, 0.1, 1000, 0x2000, 0x3000, ws,
                                  None) == 1      # H_q not a multiple of H_kv
    assert L.kvq_decode_attention(ctypes.byref(d), 0x1000, 32, 0.1, 1000, 0x2000, 0x3000, ws,
                                  None) == 2      # 16 query heads per kv head
    d2 = fake_cache(K)
    d2.fmt = K.make_format((4, 0, 0, 32), (4, 0, 0, 64), 32)
    assert L.kvq_decode_attention(ctypes.byref(d2), 0x1000, 16, 0.1, 1000, 0x2000, 0x3000, 1 << 40,
                                  None) == 2      # 4 key groups x 8 heads > 16 MFMA columns
    d3 = fake_cache(K)
    d3.fmt = K.make_format((4, 0, 0, 32), (8, 0, 0, 64), 32)
    ws3 = L.kvq_decode_workspace_bytes_mq(ctypes.byref(d3), 16, 4, 1000)
    assert L.kvq_decode_attention_mq(ctypes.byref(d3), 0x1000, 4, 16, 0.1, 1000, 0x2000, 0x3000, ws3,
                                     None) == 2   # mixed K/V formats: 4 key groups x 8 heads > 16 columns
    assert L.kvq_status_str(6).startswith(b"KVQ_EDEVICE")


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing library is an ImportError."""
    import importlib
    import quantized_kv_cache_07_amd.kvq as mod
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mod._load()
    importlib.reload(mod)


def test_multi_query_workspace_grows_with_the_blocks_a_segment_holds(K, monkeypatch):
    """Multi-query decode sizes its partial slots by the query blocks one segment holds: one
    block (the waves interleave its units), two blocks of two waves, or four of one wave each.
    Per workgroup a slot pair holds qpw x G rows of 132 floats.  With 32 or more query rows per
    kv head (4-bit codes) the dense kernel takes the call: four blocks of 16 rows (from 16 rows
    on when KVQ_MQ_DENSE=1 forces it)."""
    L = K.lib
    d = fake_cache(K)  # INT4 group 64, H_kv = 2, GQA-4 with 8 query heads: G = 8 rows per block
    one = L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 1000)
    assert L.kvq_decode_workspace_bytes_mq(ctypes.byref(d), 8, 1, 1000) == one

    def sizes():
        s = {nq: L.kvq_decode_workspace_bytes_mq(ctypes.byref(d), 8, nq, 1000) for nq in (2, 4, 6, 8, 16)}
        assert all(v > 0 for v in s.values())
        return s
    # blocked kernel: 2 is one block of two tokens, 4 and 6 two or three blocks (two per
    # segment), 8 four blocks (four per segment): the per-workgroup slots grow 1 : 2 : 4
    monkeypatch.setenv("KVQ_MQ_DENSE", "0")
    off = sizes()
    assert off[4] > off[2] and off[8] > off[4]
    # by default n_q = 8 and 16 (32 and 64 rows) are dense: four 16-row blocks per workgroup,
    # twice the rows of the blocked kernel's four 8-row blocks
    monkeypatch.delenv("KVQ_MQ_DENSE")
    auto = sizes()
    assert all(auto[nq] == off[nq] for nq in (2, 4, 6))
    assert auto[8] == auto[16] and off[8] < auto[8] < 2 * off[8]
    # forced from 16 rows (n_q = 4) on
    monkeypatch.setenv("KVQ_MQ_DENSE", "1")
    forced = sizes()
    assert forced[2] == off[2] and forced[4] == forced[6] == forced[8] == forced[16] == auto[16]
