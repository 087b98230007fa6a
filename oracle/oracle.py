"""CPU oracle for the quantized KV cache and decode attention -- Python side.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``; never by the GPU library or its binding.  It wraps the plain C
oracle in ``kvq_oracle.c`` (built with ``gcc -O2 -fno-fast-math -ffp-contract=off``) and adds
the sizing arithmetic of the pages.

Pages (cited by title and section):
  [P1] chipfoundryservices.com, "KV Cache Quantization"
  [P2] llmdaily.org, "KV-cache quantization -- making long-context inference fit in memory"
  [P3] oh-bug.com, "KV Cache Quantization in Practice: Managing Memory and Throughput for
       Long-Context Inference"
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
SO = os.path.join(HERE, "libkvq_oracle.so")

SYM, ASYM, FP8 = 0, 1, 2
PER_TOKEN, PER_CHANNEL, PER_TENSOR, PER_HEAD = 0, 1, 2, 3
D_HEAD = 128
TILE = 16

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
             "-fPIC", "-shared", "-std=c99", "-Wall"]


def build() -> str:
    """Compile the C oracle in place (host gcc; no GPU code involved)."""
    tmp = SO + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, SRC, "-lm"])
    os.replace(tmp, SO)
    return SO


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(SO) or os.path.getmtime(SO) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(SO)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.orc_f32_to_f16.argtypes, L.orc_f32_to_f16.restype = [f32], ctypes.c_uint16
        L.orc_f16_to_f32.argtypes, L.orc_f16_to_f32.restype = [ctypes.c_uint16], f32
        L.orc_f32_to_f16_array.argtypes = [P, P, i64]
        L.orc_f16_to_f32_array.argtypes = [P, P, i64]
        L.orc_quant_sym.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.orc_quant_asym.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
        L.orc_dequant.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint8, ctypes.c_uint16,
                                  ctypes.c_uint16]
        L.orc_dequant.restype = f64
        L.orc_append.argtypes = [P, P, P, i32]
        L.orc_append.restype = ctypes.c_int
        L.orc_flush.argtypes = [P]
        L.orc_flush.restype = ctypes.c_int
        L.orc_attend.argtypes = [P, P, i32, f32, P]
        L.orc_attend_mq.argtypes = [P, P, i32, i32, f32, P]
        L.orc_attend_rows.argtypes = [P, P, P, i32, i32, f64, P]
        L.orc_pack.argtypes = [P, i32, P, P, P, P, P, P, P, P, P]
        L.orc_unpack_codes.argtypes = [P, i32, P, P, P]
        L.orc_k_bit.argtypes, L.orc_k_bit.restype = [i32, i32, i32], i64
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [f32], ctypes.c_uint8
        L.orc_e4m3_value.argtypes, L.orc_e4m3_value.restype = [ctypes.c_uint8], f64
        L.orc_e4m3_encode_array.argtypes = [P, P, i64]
        L.orc_v_bit.argtypes, L.orc_v_bit.restype = [i32, i32, i32, i32], i64
        _LIB = L
    return _LIB


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------------------------------
# Scalar / vector conversions and the group quantizers
# ------------------------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    y = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_p(x), _p(y), x.size)
    return y


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    y = np.empty(h.shape, dtype=np.float32)
    lib().orc_f16_to_f32_array(_p(h), _p(y), h.size)
    return y


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quant_sym(x, bits: int):
    """Symmetric group quantizer of [P2, "From BF16 to INT8, INT4, or even fewer bits"].
    Returns (fp16 scale bits, offset-binary codes u = q + 2^(bits-1))."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    s = np.zeros(1, np.uint16)
    u = np.zeros(x.size, np.uint8)
    lib().orc_quant_sym(_p(x), x.size, bits, _p(s), _p(u))
    return int(s[0]), u


def quant_asym(x, bits: int):
    """Asymmetric (min-max, zero-point) group quantizer; returns (scale bits, zero bits, codes)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    u = np.zeros(x.size, np.uint8)
    lib().orc_quant_asym(_p(x), x.size, bits, _p(s), _p(z), _p(u))
    return int(s[0]), int(z[0]), u


def dequant(bits: int, scheme: int, codes, s16: int, z16: int = 0) -> np.ndarray:
    L = lib()
    return np.array([L.orc_dequant(bits, scheme, int(c), s16, z16) for c in np.asarray(codes)],
                    dtype=np.float64)


def attend_rows(q, khat, vhat, sm_scale: float) -> np.ndarray:
    """fp64 softmax(q K^T * sm_scale) V on already reconstructed rows."""
    q = np.ascontiguousarray(np.asarray(q, np.float64))
    kh = np.ascontiguousarray(np.asarray(khat, np.float64))
    vh = np.ascontiguousarray(np.asarray(vhat, np.float64))
    T, d = kh.shape
    out = np.zeros(d, np.float64)
    lib().orc_attend_rows(_p(q), _p(kh), _p(vh), T, d, float(sm_scale), _p(out))
    return out


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(float(y))


def e4m3_encode_array(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    out = np.zeros(y.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(y), _p(out), y.size)
    return out


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def k_bit(bits: int, t: int, c: int) -> int:
    """Bit offset of (tile row t, channel c) inside a K tile."""
    return lib().orc_k_bit(bits, t, c)


def v_bit(bits: int, t: int, c: int, d: int = D_HEAD) -> int:
    return lib().orc_v_bit(bits, d, t, c)


# ------------------------------------------------------------------------------------------
# One sequence's cache state
# ------------------------------------------------------------------------------------------

class _Side(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("scheme", ctypes.c_int32),
                ("axis", ctypes.c_int32), ("group", ctypes.c_int32)]


class _Seq(ctypes.Structure):
    _fields_ = [("k", _Side), ("v", _Side), ("d", ctypes.c_int32), ("H", ctypes.c_int32),
                ("R", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("ku", ctypes.c_void_p), ("vu", ctypes.c_void_p),
                ("ks", ctypes.c_void_p), ("kz", ctypes.c_void_p),
                ("vs", ctypes.c_void_p), ("vz", ctypes.c_void_p),
                ("kres", ctypes.c_void_p), ("vres", ctypes.c_void_p),
                ("n_quant", ctypes.c_int32), ("n_res", ctypes.c_int32),
                ("kb", ctypes.c_void_p), ("vb", ctypes.c_void_p),
                ("kf8", ctypes.c_void_p), ("vf8", ctypes.c_void_p)]


class OracleError(RuntimeError):
    pass


class Sequence:
    """Logical cache of one sequence (all kv heads): one code byte per element plus fp16
    metadata, and the BF16 window.  ``k_side``/``v_side`` are (bits, scheme, axis, group);
    bits 16 is the unquantized BF16 cache (elements kept in ``kb``/``vb``, no metadata)."""

    def __init__(self, k_side, v_side, n_kv_heads: int, residual: int, capacity: int,
                 d: int = D_HEAD, k_fp8_scale=None, v_fp8_scale=None):
        self.k_side, self.v_side = tuple(k_side), tuple(v_side)
        self.H, self.R, self.cap, self.d = n_kv_heads, residual, capacity, d
        H, cap = n_kv_heads, capacity
        self.ku = np.zeros((H, cap, d), np.uint8)
        self.vu = np.zeros((H, cap, d), np.uint8)
        self.kb = np.zeros((H, cap, d) if self.k_side[0] == 16 else 1, np.uint16)
        self.vb = np.zeros((H, cap, d) if self.v_side[0] == 16 else 1, np.uint16)

        def fp8_scales(side, given):
            # FP8: the caller's scale per tensor (one value) or per kv head, as float32 [H]
            if side[1] != FP8:
                return np.ones(1, np.float32)
            g = np.atleast_1d(np.asarray(1.0 if given is None else given, np.float32))
            return np.ascontiguousarray(np.broadcast_to(g, (H,)) if g.size == 1 else g, np.float32)

        self.kf8 = fp8_scales(self.k_side, k_fp8_scale)
        self.vf8 = fp8_scales(self.v_side, v_fp8_scale)

        def meta(side):
            bits, scheme, axis, group = side
            if scheme == FP8:  # no per-slot metadata
                return np.zeros(1, np.uint16), np.zeros(1, np.uint16)
            shape = (H, cap, d // group) if axis == PER_TOKEN else (H, cap // group, d)
            s = np.zeros(shape, np.uint16)
            z = np.zeros(shape, np.uint16) if scheme == ASYM else np.zeros(1, np.uint16)
            return s, z

        self.ks, self.kz = meta(self.k_side)
        self.vs, self.vz = meta(self.v_side)
        self.kres = np.zeros((H, max(residual, 1), d), np.uint16)
        self.vres = np.zeros((H, max(residual, 1), d), np.uint16)
        self._s = _Seq(_Side(*self.k_side), _Side(*self.v_side), d, H, residual, cap,
                       _p(self.ku), _p(self.vu), _p(self.ks), _p(self.kz), _p(self.vs),
                       _p(self.vz), _p(self.kres), _p(self.vres), 0, 0, _p(self.kb), _p(self.vb),
                       _p(self.kf8), _p(self.vf8))

    @property
    def n_quant(self) -> int:
        return self._s.n_quant

    @property
    def n_res(self) -> int:
        return self._s.n_res

    def set_counters(self, n_quant: int, n_res: int) -> None:
        self._s.n_quant, self._s.n_res = n_quant, n_res

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """k_new, v_new: bf16 bits [n_new][H][d]."""
        k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
        v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
        assert k_new.shape[1:] == (self.H, self.d) and v_new.shape == k_new.shape
        rc = lib().orc_append(ctypes.byref(self._s), _p(k_new), _p(v_new), k_new.shape[0])
        if rc:
            raise OracleError(f"append failed (code {rc})")

    def flush(self) -> None:
        rc = lib().orc_flush(ctypes.byref(self._s))
        if rc:
            raise OracleError(f"flush failed (code {rc})")

    def attend(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """q: bf16 bits [Hq][d] -> fp32 [Hq][d]."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        out = np.zeros(q.shape, np.float32)
        lib().orc_attend(ctypes.byref(self._s), _p(q), q.shape[0], float(sm_scale), _p(out))
        return out

    def attend_mq(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """q: bf16 bits [n_q][Hq][d] for the last n_q cached tokens -> fp32 [n_q][Hq][d];
        query i attends the first T - n_q + i + 1 tokens (causal)."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        out = np.zeros(q.shape, np.float32)
        lib().orc_attend_mq(ctypes.byref(self._s), _p(q), q.shape[0], q.shape[1],
                            float(sm_scale), _p(out))
        return out

    def pack(self, b: int, images: dict, table_row: np.ndarray | None = None) -> None:
        """Write the valid state into batch byte images (see ``empty_images``)."""
        tr = None if table_row is None else np.ascontiguousarray(table_row, dtype=np.int32)
        g = images.get
        lib().orc_pack(ctypes.byref(self._s), b, _p(tr), _p(g("k_codes")), _p(g("v_codes")),
                       _p(g("k_scale")), _p(g("k_zero")), _p(g("v_scale")), _p(g("v_zero")),
                       _p(g("k_res")), _p(g("v_res")))

    def unpack_codes(self, b: int, images: dict, table_row: np.ndarray | None = None) -> None:
        tr = None if table_row is None else np.ascontiguousarray(table_row, dtype=np.int32)
        lib().orc_unpack_codes(ctypes.byref(self._s), b, _p(tr), _p(images["k_codes"]),
                               _p(images["v_codes"]))


def empty_images(k_side, v_side, batch: int, n_kv_heads: int, residual: int, capacity: int = 0,
                 num_blocks: int = 0, d: int = D_HEAD) -> dict:
    """Zero-filled byte images of every buffer of a batch cache in the storage layout:
    contiguous when ``num_blocks == 0`` (``capacity`` tokens per sequence), else a paged pool."""
    H = n_kv_heads
    tiles = num_blocks * H if num_blocks else batch * H * (capacity // TILE)
    out = {}
    for name, side in (("k", k_side), ("v", v_side)):
        bits, scheme, axis, group = side
        out[f"{name}_codes"] = np.zeros(tiles * TILE * d * bits // 8, np.uint8)
        if scheme == FP8:  # the caller's fp32 scales: one per tensor or per kv head
            out[f"{name}_codes"] = np.zeros(tiles * TILE * d, np.uint8)
            out[f"{name}_scale"] = np.zeros(0, np.uint16)
            out[f"{name}_zero"] = np.zeros(0, np.uint16)
            out[f"{name}_res"] = np.zeros(batch * H * max(residual, 1) * d, np.uint16)
            continue
        if bits == 16:  # BF16 storage has no metadata
            out[f"{name}_scale"] = np.zeros(0, np.uint16)
            out[f"{name}_zero"] = np.zeros(0, np.uint16)
            out[f"{name}_res"] = np.zeros(batch * H * max(residual, 1) * d, np.uint16)
            continue
        if axis == PER_TOKEN:
            n = tiles * (d // group) * TILE
            if k_side[2] == PER_TOKEN:  # both per-token: one record per tile in the key buffers
                n = tiles * (d // k_side[3] + d // v_side[3]) * TILE if name == "k" else 0
        elif num_blocks:  # paged per-channel keys: one metadata row per (block, head)
            n = num_blocks * H * d
        else:
            n = batch * H * (capacity // group) * d
        out[f"{name}_scale"] = np.zeros(n, np.uint16)
        # zero-points: the side's own, or, in a shared per-tile record, those of either side
        has_zero = scheme == ASYM or (name == "k" and axis == PER_TOKEN and v_side[1] == ASYM)
        out[f"{name}_zero"] = np.zeros(n if has_zero else (1 if n else 0), np.uint16)
        out[f"{name}_res"] = np.zeros(batch * H * max(residual, 1) * d, np.uint16)
    return out


# ------------------------------------------------------------------------------------------
# Sizing [P2, "Why the KV cache grows so quickly", memory formula; "Worked example"]
# ------------------------------------------------------------------------------------------

def mkv_bytes(L: int, T: int, H_kv: int, d_h: int, b: float) -> float:
    """M_KV = 2 L T H_kv d_h b (keys and values; b = bytes per stored element)."""
    return 2 * L * T * H_kv * d_h * b


def bytes_per_element(bits: int, group: int, scale_bytes: int = 2, zero_point: bool = False) -> float:
    """Packed code bytes plus one scale (and zero-point) per ``group`` elements."""
    return bits / 8 + (scale_bytes * (2 if zero_point else 1)) / group


def p1_bytes_per_token(num_layers: int, hidden: int, elem_bytes: int) -> int:
    """[P1, "The KV Cache Problem"]: 2 x num_layers x hidden_dim x bytes per element."""
    return 2 * num_layers * hidden * elem_bytes
