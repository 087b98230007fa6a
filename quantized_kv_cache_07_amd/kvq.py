"""Thin ctypes binding of libkvq (include/kvq.h).

Argument marshalling only: every step of the path runs in the HIP kernels of libkvq.so.  PyTorch
supplies device memory (tensors) and the stream (torch.cuda.current_stream()).  Importing this
module loads the library and raises if it is missing; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may name another build of the same sources (build.py --qk-valu)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

SYM, ASYM = 0, 1
PER_TOKEN, PER_CHANNEL = 0, 1
HEAD_DIM = 128
BLOCK = 16
(BUF_K_CODES, BUF_V_CODES, BUF_K_SCALE, BUF_V_SCALE, BUF_K_ZERO, BUF_V_ZERO, BUF_K_RES,
 BUF_V_RES) = range(8)
ERR_CAPACITY, ERR_BLOCK, ERR_TOKENS, ERR_GROUP = 1, 2, 4, 8

STATUS = {0: "KVQ_OK", 1: "KVQ_EINVAL", 2: "KVQ_ENOTSUP", 3: "KVQ_EALIGN", 4: "KVQ_ENOSPACE",
          5: "KVQ_ELAUNCH", 6: "KVQ_EDEVICE"}

# Every function declared in include/kvq.h and include/kvq_measure.h.
EXPORTS = ["kvq_buffer_bytes", "kvq_check_format", "kvq_quantize_append", "kvq_flush_residual",
           "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_workspace_bytes_mq",
           "kvq_decode_attention_mq", "kvq_decode_attention_noalloc", "kvq_read_error",
           "kvq_status_str", "kvq_measure_read", "kvq_measure_read_sink_floats",
           "kvq_measure_copy"]


SCHEME_FP8 = 2  # KVQ_FP8


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class Side(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("scheme", ctypes.c_int32), ("axis", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class Format(ctypes.Structure):
    _fields_ = [("k", Side), ("v", Side), ("residual", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("fmt", Format), ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_zero", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
                ("n_quant", ctypes.c_void_p), ("n_res", ctypes.c_void_p),
                ("err", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python -m quantized_kv_cache_07_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.kvq_buffer_bytes.argtypes = [P, i32, i32, i32, i32, i32]
    L.kvq_buffer_bytes.restype = sz
    L.kvq_check_format.argtypes = [P]
    L.kvq_quantize_append.argtypes = [P, P, P, i32, P]
    L.kvq_flush_residual.argtypes = [P, P]
    L.kvq_decode_workspace_bytes.argtypes = [P, i32, i32]
    L.kvq_decode_workspace_bytes.restype = sz
    L.kvq_decode_attention.argtypes = [P, P, i32, f32, i32, P, P, sz, P]
    L.kvq_decode_workspace_bytes_mq.argtypes = [P, i32, i32, i32]
    L.kvq_decode_workspace_bytes_mq.restype = sz
    L.kvq_decode_attention_mq.argtypes = [P, P, i32, i32, f32, i32, P, P, sz, P]
    L.kvq_decode_attention_noalloc.argtypes = [P, P, i32, f32, i32, P, P]
    L.kvq_read_error.argtypes = [P, P, P]
    L.kvq_status_str.argtypes = [ctypes.c_int]
    L.kvq_status_str.restype = ctypes.c_char_p
    L.kvq_measure_read.argtypes = [P, sz, P, P]
    L.kvq_measure_read_sink_floats.restype = i32
    L.kvq_measure_copy.argtypes = [P, P, sz, P]
    for f in ("kvq_check_format", "kvq_quantize_append", "kvq_flush_residual",
              "kvq_decode_attention", "kvq_decode_attention_mq", "kvq_decode_attention_noalloc",
              "kvq_read_error",
              "kvq_measure_read", "kvq_measure_copy"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()


def make_format(k, v, residual: int = 0, head_dim: int = HEAD_DIM) -> Format:
    """k, v: (bits, scheme, axis, group) tuples."""
    return Format(Side(*k), Side(*v), residual, head_dim)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvqError(status, what)


class Cache:
    """A batch cache whose buffers are torch tensors (zero-initialised) sized by
    kvq_buffer_bytes.  Contiguous when `block_table` is None, else paged over `num_blocks`."""

    def __init__(self, k, v, batch: int, n_kv_heads: int, residual: int = 0, capacity: int = 0,
                 block_table: torch.Tensor | None = None, num_blocks: int = 0,
                 device="cuda", fp8_scales=None):
        """fp8_scales: for FP8 sides, (k_scales, v_scales), each one value (per tensor) or
        n_kv_heads values (per head); copied into the float32 scale buffers."""
        self.fmt = make_format(k, v, residual)
        st = lib.kvq_check_format(ctypes.byref(self.fmt))
        _check(st, "format")
        self.k_side, self.v_side = tuple(k), tuple(v)
        self.batch, self.n_kv_heads, self.residual = batch, n_kv_heads, residual
        self.paged = block_table is not None
        self.capacity = 0 if self.paged else capacity
        self.num_blocks = num_blocks if self.paged else 0
        self.device = device

        def buf(which, dtype):
            n = lib.kvq_buffer_bytes(ctypes.byref(self.fmt), batch, n_kv_heads, self.capacity,
                                     self.num_blocks, which)
            if n == 0:
                return None
            itemsize = torch.tensor([], dtype=dtype).element_size()
            return torch.zeros(n // itemsize, dtype=dtype, device=device)

        self.k_codes = buf(BUF_K_CODES, torch.uint8)
        self.v_codes = buf(BUF_V_CODES, torch.uint8)
        self.k_scale = buf(BUF_K_SCALE, torch.int16)
        self.v_scale = buf(BUF_V_SCALE, torch.int16)
        self.k_zero = buf(BUF_K_ZERO, torch.int16)
        self.v_zero = buf(BUF_V_ZERO, torch.int16)
        self.k_res = buf(BUF_K_RES, torch.int16)
        self.v_res = buf(BUF_V_RES, torch.int16)
        if k[1] == SCHEME_FP8:
            if fp8_scales is None:
                raise ValueError("an FP8 cache needs its scales (fp8_scales=(k, v))")
            for buf_, vals in ((self.k_scale, fp8_scales[0]), (self.v_scale, fp8_scales[1])):
                f = buf_.view(torch.float32)
                f.copy_(torch.as_tensor(vals, dtype=torch.float32).reshape(-1).expand(f.numel()))
        self.n_quant = torch.zeros(batch, dtype=torch.int32, device=device)
        self.n_res = torch.zeros(batch, dtype=torch.int32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self.block_table = None
        if self.paged:
            self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        self.desc = self._describe()

    def _describe(self, seq: int | None = None) -> CacheDesc:
        d = CacheDesc()
        d.fmt = self.fmt
        d.n_kv_heads = self.n_kv_heads
        d.capacity = self.capacity
        d.num_blocks = self.num_blocks
        d.max_blocks = 0 if not self.paged else self.block_table.shape[1]
        d.err = _ptr(self.err)
        names = ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero", "k_res", "v_res")
        if seq is None:
            d.batch = self.batch
            d.block_table = _ptr(self.block_table)
            for name in names:
                setattr(d, name, _ptr(getattr(self, name)))
            d.n_quant, d.n_res = _ptr(self.n_quant), _ptr(self.n_res)
            return d
        # A one-sequence view: the same pool (paged) or the sequence's slice (contiguous).
        d.batch = 1
        d.n_quant = self.n_quant[seq:seq + 1].data_ptr()
        d.n_res = self.n_res[seq:seq + 1].data_ptr()
        if self.paged:
            d.block_table = self.block_table[seq].data_ptr()
            for name in names:
                t = getattr(self, name)
                if name in ("k_res", "v_res"):
                    t = None if t is None else t.view(self.batch, -1)[seq]
                setattr(d, name, _ptr(t))
        else:
            d.block_table = None
            for name in names:
                t = getattr(self, name)
                shared = name in ("k_scale", "v_scale") and \
                    (self.k_side if name[0] == "k" else self.v_side)[1] == SCHEME_FP8
                if t is None or shared:  # FP8 scales belong to the whole cache
                    setattr(d, name, _ptr(t))
                else:
                    setattr(d, name, t.view(self.batch, -1)[seq].data_ptr())
        return d

    def sequence(self, seq: int) -> CacheDesc:
        return self._describe(seq)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_device(cache: Cache, *tensors) -> None:
    """Every tensor on the cache's GPU (checked last, after shapes and dtypes)."""
    dev = cache.n_quant.device
    _need(dev.type == "cuda", f"the cache's buffers are on {dev}, not on a GPU")
    for t in tensors:
        if t is not None:
            _need(t.device == dev, f"a tensor on {t.device} for a cache on {dev}")


def quantize_append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None,
                    desc: CacheDesc | None = None) -> None:
    """k_new, v_new: bf16 [batch][n_new][H_kv][128] on the cache's device (batch of `desc`,
    1 for a one-sequence view)."""
    batch = (desc or cache.desc).batch
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16,
              f"{name} must be a bfloat16 tensor")
        _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(t.dim() == 4 and t.shape[0] == batch and t.shape[1] >= 1 and
              t.shape[2] == cache.n_kv_heads and t.shape[3] == HEAD_DIM,
              f"{name} must be [batch={batch}][n_new>=1][H_kv={cache.n_kv_heads}][{HEAD_DIM}], "
              f"got {tuple(t.shape)}")
    _need(k_new.shape == v_new.shape, "k_new and v_new must have the same shape")
    _on_device(cache, k_new, v_new)
    st = lib.kvq_quantize_append(ctypes.byref(desc or cache.desc), k_new.data_ptr(),
                                 v_new.data_ptr(), k_new.shape[1], _stream(stream))
    _check(st, "kvq_quantize_append")


def flush_residual(cache: Cache, stream=None, desc: CacheDesc | None = None) -> None:
    _on_device(cache)
    _check(lib.kvq_flush_residual(ctypes.byref(desc or cache.desc), _stream(stream)),
           "kvq_flush_residual")


def _check_query(cache: Cache, q: torch.Tensor, dims: int) -> None:
    """q: bf16, contiguous, [batch][H_q][128] (dims 3) or [batch][n_q][H_q][128] (dims 4)."""
    _need(isinstance(q, torch.Tensor) and q.dtype == torch.bfloat16, "q must be a bfloat16 tensor")
    _need(q.is_contiguous(), "q must be contiguous")
    _need(q.dim() == dims and q.shape[0] == cache.batch and q.shape[-1] == HEAD_DIM and
          q.shape[-2] >= 1 and q.shape[-2] % cache.n_kv_heads == 0 and
          (dims == 3 or q.shape[1] >= 1),
          f"q must be [batch={cache.batch}]{'[n_q]' if dims == 4 else ''}[H_q, a multiple of "
          f"H_kv={cache.n_kv_heads}][{HEAD_DIM}], got {tuple(q.shape)}")


def _check_out(out: torch.Tensor, q: torch.Tensor) -> None:
    _need(isinstance(out, torch.Tensor) and out.dtype == torch.float32, "out must be float32")
    _need(out.is_contiguous() and tuple(out.shape) == tuple(q.shape),
          f"out must be a contiguous {tuple(q.shape)} tensor, got {tuple(out.shape)}")


def _check_workspace(ws: torch.Tensor) -> None:
    _need(isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and ws.is_contiguous() and
          ws.dim() == 1, "workspace must be a contiguous 1-D uint8 tensor")


def workspace_bytes(cache: Cache, n_q_heads: int, max_tokens: int) -> int:
    return lib.kvq_decode_workspace_bytes(ctypes.byref(cache.desc), n_q_heads, max_tokens)


def decode_attention(cache: Cache, q: torch.Tensor, max_tokens: int, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, sm_scale: float | None = None,
                     stream=None) -> torch.Tensor:
    """q: bf16 [batch][H_q][128] -> fp32 [batch][H_q][128]."""
    _check_query(cache, q, 3)
    hq = q.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check_out(out, q)
    need = workspace_bytes(cache, hq, max_tokens)
    if need == 0:
        raise KvqError(1, "kvq_decode_workspace_bytes")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    _on_device(cache, q, out, workspace)
    st = lib.kvq_decode_attention(ctypes.byref(cache.desc), q.data_ptr(), hq, float(sm_scale),
                                  max_tokens, out.data_ptr(), workspace.data_ptr(),
                                  workspace.numel(), _stream(stream))
    _check(st, "kvq_decode_attention")
    return out


def workspace_bytes_mq(cache: Cache, n_q_heads: int, n_q: int, max_tokens: int) -> int:
    return lib.kvq_decode_workspace_bytes_mq(ctypes.byref(cache.desc), n_q_heads, n_q, max_tokens)


def decode_attention_mq(cache: Cache, q: torch.Tensor, max_tokens: int,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        sm_scale: float | None = None, stream=None) -> torch.Tensor:
    """q: bf16 [batch][n_q][H_q][128], the queries of each sequence's last n_q cached tokens
    -> fp32 [batch][n_q][H_q][128] (causal)."""
    _check_query(cache, q, 4)
    nq, hq = q.shape[1], q.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check_out(out, q)
    need = workspace_bytes_mq(cache, hq, nq, max_tokens)
    if need == 0:
        raise KvqError(1, "kvq_decode_workspace_bytes_mq")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    _on_device(cache, q, out, workspace)
    st = lib.kvq_decode_attention_mq(ctypes.byref(cache.desc), q.data_ptr(), nq, hq,
                                     float(sm_scale), max_tokens, out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "kvq_decode_attention_mq")
    return out


def decode_attention_noalloc(cache: Cache, q: torch.Tensor, max_tokens: int,
                             out: torch.Tensor | None = None, sm_scale: float | None = None,
                             stream=None) -> torch.Tensor:
    """kvq_decode_attention_noalloc: as decode_attention, with the library's own workspace (no
    device allocation by the library; `out` may be preallocated by the caller)."""
    _check_query(cache, q, 3)
    hq = q.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check_out(out, q)
    _on_device(cache, q, out)
    st = lib.kvq_decode_attention_noalloc(ctypes.byref(cache.desc), q.data_ptr(), hq,
                                          float(sm_scale), max_tokens, out.data_ptr(),
                                          _stream(stream))
    _check(st, "kvq_decode_attention_noalloc")
    return out


def read_error(cache: Cache, stream=None) -> int:
    v = ctypes.c_int32(0)
    st = lib.kvq_read_error(ctypes.byref(cache.desc), ctypes.byref(v), _stream(stream))
    if st not in (0, 6):
        raise KvqError(st, "kvq_read_error")
    return v.value


def measure_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    _need(buf.is_cuda and sink.is_cuda and buf.is_contiguous() and sink.dtype == torch.float32 and
          sink.numel() >= lib.kvq_measure_read_sink_floats(),
          "measure_read: contiguous GPU buffer and a float32 GPU sink of "
          "kvq_measure_read_sink_floats() values")
    _check(lib.kvq_measure_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                _stream(stream)), "kvq_measure_read")


def measure_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    _need(dst.is_cuda and src.is_cuda and dst.is_contiguous() and src.is_contiguous() and
          dst.numel() * dst.element_size() >= src.numel() * src.element_size(),
          "measure_copy: contiguous GPU tensors, dst at least as large as src")
    _check(lib.kvq_measure_copy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(),
                                _stream(stream)), "kvq_measure_copy")
