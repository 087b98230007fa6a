"""kvq_decode_attention_noalloc: decode attention with the library's own device workspace.

Two calls in a row through the C ABI, the second on a smaller batch, each against
kvq_decode_attention (caller workspace) on the same cache and queries: the same kernels run
in the same launch configuration, so the outputs must be identical, and both within
2e-3 + 1e-2 |ref| of the oracle.  A shape whose workspace exceeds the library's array is
refused on the host with KVQ_ENOSPACE before anything is launched.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import kvq_cases as kc

pytestmark = pytest.mark.gpu

SYM4 = (4, 0, 0, 64)
KPC2 = (2, 1, 1, 32)
ASYM2_32 = (2, 1, 0, 32)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _noalloc_vs_workspace(pr, q_seed_step):
    K = kc.kvq()
    q = kc.ki.queries(pr.w, q_seed_step, "cuda")
    mt = max(s.n_quant + s.n_res for s in pr.seqs)
    ref = K.decode_attention(pr.cache, q, max_tokens=mt, sm_scale=kc.SM_SCALE)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device="cuda")
    st = K.lib.kvq_decode_attention_noalloc(ctypes.byref(pr.cache.desc), q.data_ptr(),
                                            q.shape[1], ctypes.c_float(kc.SM_SCALE), mt,
                                            out.data_ptr(), K._stream(None))
    assert st == 0, K.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert K.read_error(pr.cache) == 0
    assert torch.equal(out, ref)
    got = out.cpu().numpy()
    qb = kc.ki.bf16_bits(q)
    oref = np.stack([s.attend(qb[b], kc.SM_SCALE) for b, s in enumerate(pr.seqs)])
    err = np.abs(got - oref)
    assert np.all(err <= kc.ATOL + kc.RTOL * np.abs(oref)), float(err.max())


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    print("case: noalloc large then small", flush=True)
    sys.stdout.flush()
    big = kc.build_pair(SYM4, SYM4, 3, 8, 2, 32, [900, 40, 333], seed=41)
    _noalloc_vs_workspace(big, 0)
    small = kc.build_pair(KPC2, ASYM2_32, 1, 8, 2, 64, [200], seed=42)
    _noalloc_vs_workspace(small, 1)
    # the big case once more after the small one: nothing left over is read
    _noalloc_vs_workspace(big, 2)


def test_noalloc_refuses_a_workspace_beyond_its_array(monkeypatch):
    print("case: noalloc ENOSPACE", flush=True)
    K = kc.kvq()
    monkeypatch.setenv("KVQ_DECODE_BLOCKS", "65536")
    pr = kc.build_pair(SYM4, SYM4, 3, 16, 2, 32, [64, 40, 33], seed=43)
    mt = 1 << 17
    limit = 16 << 20
    assert K.workspace_bytes(pr.cache, 16, mt) > limit
    q = kc.ki.queries(pr.w, 0, "cuda")
    out = torch.zeros((3, 16, 128), dtype=torch.float32, device="cuda")
    st = K.lib.kvq_decode_attention_noalloc(ctypes.byref(pr.cache.desc), q.data_ptr(), 16,
                                            ctypes.c_float(kc.SM_SCALE), mt, out.data_ptr(),
                                            K._stream(None))
    assert st == 4  # KVQ_ENOSPACE, nothing launched
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
