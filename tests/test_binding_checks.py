"""The Python binding validates every tensor it hands to the C ABI (shape, dtype, layout,
device) and raises ValueError before any library call: a mismatch would otherwise make a
kernel read or write outside the buffers.  Runs without a GPU: the caches live on the CPU, so
every call that passes the shape checks stops at the device check."""
from __future__ import annotations

import pytest
import torch


@pytest.fixture(scope="module")
def K():
    from quantized_kv_cache_07_amd import kvq
    return kvq


@pytest.fixture(scope="module")
def cache(K):
    return K.Cache((4, 0, 0, 64), (4, 0, 0, 64), 2, 2, residual=16, capacity=64, device="cpu")


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("k_shape,v_shape,why", [
    ((3, 1, 2, 128), (3, 1, 2, 128), "batch"),
    ((2, 1, 3, 128), (2, 1, 3, 128), "H_kv"),
    ((2, 1, 2, 64), (2, 1, 2, 64), "head_dim"),
    ((2, 0, 2, 128), (2, 0, 2, 128), "n_new"),
    ((2, 2, 128), (2, 2, 128), "rank"),
    ((2, 1, 2, 128), (2, 2, 2, 128), "k/v mismatch"),
])
def test_append_shapes(K, cache, k_shape, v_shape, why):
    with pytest.raises(ValueError):
        K.quantize_append(cache, bf(*k_shape), bf(*v_shape))


def test_append_dtype_layout_device(K, cache):
    with pytest.raises(ValueError):
        K.quantize_append(cache, torch.zeros(2, 1, 2, 128), bf(2, 1, 2, 128))
    with pytest.raises(ValueError):
        K.quantize_append(cache, bf(2, 1, 2, 128), torch.zeros(2, 1, 2, 128, dtype=torch.float16))
    nc = bf(2, 2, 1, 128).transpose(1, 2)
    with pytest.raises(ValueError):
        K.quantize_append(cache, nc, nc)
    with pytest.raises(ValueError, match="not on a GPU"):
        K.quantize_append(cache, bf(2, 1, 2, 128), bf(2, 1, 2, 128))
    with pytest.raises(ValueError, match="not on a GPU"):
        K.flush_residual(cache)
    # a one-sequence view takes batch 1
    with pytest.raises(ValueError, match="batch=1"):
        K.quantize_append(cache, bf(2, 1, 2, 128), bf(2, 1, 2, 128), desc=cache.sequence(0))


@pytest.mark.parametrize("q_shape", [(3, 4, 128), (2, 3, 128), (2, 4, 64), (2, 0, 128), (2, 4)])
def test_decode_query_shapes(K, cache, q_shape):
    with pytest.raises(ValueError):
        K.decode_attention(cache, bf(*q_shape), max_tokens=16)
    with pytest.raises(ValueError):
        K.decode_attention_noalloc(cache, bf(*q_shape), max_tokens=16)


def test_decode_out_and_workspace(K, cache):
    q = bf(2, 4, 128)
    with pytest.raises(ValueError, match="out"):
        K.decode_attention(cache, q, 16, out=torch.zeros(2, 4, 64))
    with pytest.raises(ValueError, match="out"):
        K.decode_attention(cache, q, 16, out=torch.zeros(2, 4, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="out"):
        K.decode_attention_noalloc(cache, q, 16, out=torch.zeros(2, 8, 128))
    with pytest.raises(ValueError, match="workspace"):
        K.decode_attention(cache, q, 16, workspace=torch.zeros(1 << 20, dtype=torch.float32))
    with pytest.raises(ValueError, match="not on a GPU"):
        K.decode_attention(cache, q, 16)
    with pytest.raises(ValueError, match="not on a GPU"):
        K.decode_attention_noalloc(cache, q, 16)
    with pytest.raises(ValueError):
        K.decode_attention(cache, q.float(), 16)


def test_multi_query_shapes(K, cache):
    with pytest.raises(ValueError):
        K.decode_attention_mq(cache, bf(2, 4, 128), max_tokens=16)        # rank 3
    with pytest.raises(ValueError):
        K.decode_attention_mq(cache, bf(2, 3, 4, 64), max_tokens=16)      # head_dim
    with pytest.raises(ValueError):
        K.decode_attention_mq(cache, bf(1, 3, 4, 128), max_tokens=16)     # batch
    with pytest.raises(ValueError, match="out"):
        K.decode_attention_mq(cache, bf(2, 3, 4, 128), 16, out=torch.zeros(2, 4, 128))
    with pytest.raises(ValueError, match="not on a GPU"):
        K.decode_attention_mq(cache, bf(2, 3, 4, 128), max_tokens=16)
