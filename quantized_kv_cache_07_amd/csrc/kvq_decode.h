// kvq_decode.h -- decode attention over the quantized cache (gfx950 kernels).
//
//   out[b][hq] = softmax(sm_scale * q K^T) V          [P2 = llmdaily.org "KV-cache quantization --
//   making long-context inference fit in memory", "Why the KV cache grows so quickly", attention
//   equation], over the compressed tokens, dequantized in registers as they stream in (P3 =
//   oh-bug.com "KV Cache Quantization in Practice", "Misconception 1": a kernel gains from
//   quantization only when the dequantization is fused into it), followed by the BF16 window.
//
// Work decomposition.  A work unit is 32 compressed slots (a pair of 16-slot tiles) or 32 window
// rows of one (sequence, kv head).  Units are numbered sequence by sequence, kv head by kv head,
// from a prefix sum every workgroup rebuilds from the device counters (no host sync).  Workgroup
// k of NB owns the contiguous unit range [k U / NB, (k+1) U / NB): the load is balanced to one
// unit whatever the length mix.  A window unit counts window_weight units (about its bytes
// against a compressed unit's), so ranges that hold many sequence ends carry no more bytes.  Inside a workgroup the four waves interleave the units of each
// (sequence, kv head) segment; at a segment end the waves merge in LDS and the workgroup writes
// either the normalised output (the segment was the whole sequence) or a partial (max, sum,
// o[128]) that combine_kernel merges with a log-sum-exp rescale.  Multi-query decode with two or
// more query blocks per (sequence, kv head) puts two (mode 3: two waves each) or four (mode 2:
// one wave each) blocks in a segment, their waves walking the same units.
//
// One unit on one wave (lane = 16 g + n):
//   QK^T  4 MFMA 16x16x32 f16 per tile: D[token][col] = sum_k A[token][k] B[k][col], A = key
//         codes of token n as f16 operands (a masked field under the exponent of 1024, or, for
//         per-channel keys, under a zero exponent: an exact subnormal), B = the query rows of
//         the GQA group divided by each field's power-of-two position factor, one column per
//         (key group, query head) with the other groups' channels zeroed, so per-token group
//         scales apply to the products; per-channel key scales are folded into the query (hi +
//         lo f16 parts) once per key group.
//   softmax  online, in log2 units; the running max is only raised when a score exceeds it by
//         more than 1 (weights stay <= 2), so the accumulator is rescaled a few times per segment.
//   PV    8 MFMA 16x16x32 f16 per row block: D[row][ch] = sum_t P[row][t] V[t][ch] with rows
//         (hi/lo part, value group, query head) of w * s_v, 32 tokens (both tiles) deep; value
//         codes enter as f16 subnormals (one AND per two codes), the symmetric offset as one
//         more product per unit.
//   Codes of the next unit are loaded as soon as the current ones are consumed.
#pragma once

#include <cfloat>
#include <climits>
#include <mutex>
#include <type_traits>

#include "kvq_dev.h"

// QK of single-query MHA (G = 1) 8-bit symmetric per-token caches on the vector ALU instead of
// the matrix cores: v_dot2_f32_f16 over the raw code pairs, then DPP row sums.  Off by default
// (the two run at the same HBM-bound speed); a build with -DKVQ_QK_VALU=1 selects it, for the
// comparison of the two.
#ifndef KVQ_QK_VALU
#define KVQ_QK_VALU 0
#endif

namespace kvq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVES = 4;
constexpr int RED_STRIDE = D + 4;  // floats per LDS row of the merge buffer
// Raise the running max only past this margin (log2 units): weights stay <= 2, so a weight times
// any finite fp16 value scale (<= 65504) stays within the hi + lo f16 parts of the PV operand
// (v_cvt_pkrtz_f16_f32 saturates at 65504: hi = 65504, lo = w s - 65504 <= 65504).
constexpr float LAZY_LOG2 = 1.0f;
// Query rows enter the matrix cores as f16 after a power-of-two prescale 2^-e per row, so any
// bf16 query fits: the row maximum lands in [2^QE_RAW, 2^(QE_RAW+1)) for raw-code keys (the
// largest f16 operand q 2^-e / alpha stays below 65504) and in [2^QE_FOLD, 2^(QE_FOLD+1)) when
// the query is multiplied by per-channel key scales first (q s 2^-e stays below 65504 for any
// fp16 scale).  The scores come out multiplied by 2^-e and the softmax scale by 2^e.
constexpr int QE_RAW = 13, QE_FOLD = -1;

// ---- small helpers ------------------------------------------------------------------------

// 2^x for an integer |x| <= 126, exactly.
__device__ __forceinline__ float exp2i(int x) { return __uint_as_float(static_cast<uint32_t>(127 + x) << 23); }

// Exponent e of a query row's prescale 2^-e: the row maximum mx times 2^-e lies in
// [2^target, 2^(target+1)); 0 for an all-zero row; clamped to [-100, 100].
__device__ __forceinline__ int q_exponent(float mx, int target) {
  if (!(mx > 0.0f)) return 0;
  const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu) - 127;  // floor(log2 mx)
  return min(max(E - target, -100), 100);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t h2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
// Two f32 to two f16, rounding toward zero (v_cvt_pkrtz_f16_f32).
__device__ __forceinline__ f16x2 pkrtz(float a, float b) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ f16x2 h2s(float x) { return f16x2{(_Float16)x, (_Float16)x}; }
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, static_cast<unsigned short>(u & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, static_cast<unsigned short>(u >> 16));
}

// DPP row rotate (within 16-lane rows) by S lanes.
template <int S>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(S >= 1 && S <= 15, "row_ror");
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + S, 0xF, 0xF, true));
}

// Values every lane of a wave agrees on, made scalar (the compiler cannot see it for LDS loads).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long uni(long v) {
  const unsigned long long u = static_cast<unsigned long long>(v);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u >> 32));
  return static_cast<long>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// A load through the scalar data cache: `ptr` must be the same on every lane and the memory
// must not change while the kernel runs (block tables and counters).
__device__ __forceinline__ int ld_uniform(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)(ptr);
}

// max(a, b, c) in one instruction; the operands are never NaN here.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- code unpacking -----------------------------------------------------------------------
// Constants of the unpacking, held in registers: gfx950 VOP3 instructions (v_and_or_b32) take
// no literal operands, so with literals every and-or would split into two instructions.
struct UnpackRegs {
  uint32_t magic;       // VGPR: 0x64006400, f16 1024.0 in both halves
  uint32_t m_lo, m_hi;  // SGPRs: masks of the fields a pair needs (per bit width)
  uint32_t m2[4];       // 2-bit codes: 0x00030003 << 2k, k = 0..3
};

template <int KB>
__device__ __forceinline__ UnpackRegs unpack_regs() {
  UnpackRegs r;
  r.magic = 0x64006400u;
  if constexpr (KB == 16) {  // BF16 storage: nothing to unpack
    r.m_lo = r.m_hi = 0;
    return r;
  }
  asm volatile("" : "+v"(r.magic));
  if constexpr (KB == 8) {
    asm volatile("s_mov_b32 %0, 0x00ff00ff" : "=s"(r.m_lo));
    r.m_hi = r.m_lo;
  } else if constexpr (KB == 4) {
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(r.m_lo));
    asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(r.m_hi));
  } else {
    asm volatile("s_mov_b32 %0, 0x00030003" : "=s"(r.m2[0]));
    asm volatile("s_mov_b32 %0, 0x000c000c" : "=s"(r.m2[1]));
    asm volatile("s_mov_b32 %0, 0x00300030" : "=s"(r.m2[2]));
    asm volatile("s_mov_b32 %0, 0x00c000c0" : "=s"(r.m2[3]));
    r.m_lo = r.m_hi = 0;
  }
  return r;
}

// A word holds E = 32 / KB fields; pair k (0 <= k < E/2) is (field k, field k + E/2): the
// same field of the word's two 16-bit halves, so one mask under an f16 exponent turns a pair into
// two f16 values.  2-bit pairs 4..7 are taken from the word shifted right by 8.

// Scale of pair k's fields in the bias-free form: the masked field reads as 1024 + alpha u.
template <int KB>
__device__ __forceinline__ constexpr int pair_alpha(int k) {
  if constexpr (KB == 8) return 1;
  else if constexpr (KB == 4) return (k & 1) ? 16 : 1;
  else return 1 << (2 * (k & 3));
}

// Pair r as two f16 subnormals alpha u 2^-24 (the masked fields under a zero exponent; one
// and).  The matrix cores take f16 subnormal operands exactly, so these products need no bias
// removal: the other operand carries 1 / alpha and the result is scaled by 2^24 afterwards.
template <int KB>
__device__ __forceinline__ uint32_t subpair(const uint32_t* w, int r, const UnpackRegs& u) {
  constexpr int HH = 16 / KB;
  const uint32_t x = w[r / HH];
  const int k = r % HH;
  if constexpr (KB == 8) {
    return (k ? (x >> 8) : x) & u.m_lo;
  } else if constexpr (KB == 4) {
    const uint32_t s = (k >= 2) ? (x >> 8) : x;
    return s & ((k & 1) ? u.m_hi : u.m_lo);
  } else {
    const uint32_t s = (k >= 4) ? (x >> 8) : x;
    return s & u.m2[k & 3];
  }
}

// Pair r as the raw f16 values 1024 + alpha u (one and-or, no bias removal).  The bias is
// removed inside the matrix products: the other operand is divided by alpha and a constant
// operand holding -(1024 + alpha off) cancels the rest.
template <int KB>
__device__ __forceinline__ uint32_t rawpair(const uint32_t* w, int r, const UnpackRegs& u) {
  return subpair<KB>(w, r, u) | u.magic;
}

// alpha of element i of QK MFMA j (pair 4 j + i / 2) and of element i of a PV B operand
// (pairs 2 j, 2 j + 1 of tile A, then of tile B)
template <int KB>
__device__ __forceinline__ constexpr int kelem_alpha(int j, int i) {
  return pair_alpha<KB>((4 * j + i / 2) % (16 / KB));
}
template <int KB>
__device__ __forceinline__ constexpr int velem_alpha(int j, int i) {
  return pair_alpha<KB>((2 * j + (i / 2) % 2) % (16 / KB));
}

// 1 / alpha of natural channel k (0..7) of a per-channel folding lane's block in QK column block
// jp: natural channels k and k + 4 are the two halves of pair (4 jp + k % 4) mod 16 / KB
template <int KB>
__device__ __forceinline__ float fold_inv_alpha(int jp, int k) {
  return 1.0f / static_cast<float>(pair_alpha<KB>((4 * jp + (k & 3)) % (16 / KB)));
}

template <int KB>
__device__ __forceinline__ f16x8 kop_raw(const uint32_t* w, int j, const UnpackRegs& u) {
  return __builtin_bit_cast(f16x8, uint4{rawpair<KB>(w, 4 * j, u), rawpair<KB>(w, 4 * j + 1, u),
                                         rawpair<KB>(w, 4 * j + 2, u), rawpair<KB>(w, 4 * j + 3, u)});
}
template <int KB>
__device__ __forceinline__ f16x8 kop_sub(const uint32_t* w, int j, const UnpackRegs& u) {
  return __builtin_bit_cast(f16x8, uint4{subpair<KB>(w, 4 * j, u), subpair<KB>(w, 4 * j + 1, u),
                                         subpair<KB>(w, 4 * j + 2, u), subpair<KB>(w, 4 * j + 3, u)});
}
template <int KB>
__device__ __forceinline__ f16x8 vop_sub(const uint32_t* wa, const uint32_t* wb, int j, const UnpackRegs& u) {
  return __builtin_bit_cast(f16x8, uint4{subpair<KB>(wa, 2 * j, u), subpair<KB>(wa, 2 * j + 1, u),
                                         subpair<KB>(wb, 2 * j, u), subpair<KB>(wb, 2 * j + 1, u)});
}
// alpha of value MFMA j's channel factor (element i's alpha is vchan_alpha(j) * vtok_alpha(i))
template <int KB>
__device__ __forceinline__ constexpr int vchan_alpha(int j) {
  return velem_alpha<KB>(j, 0);
}

// FP8 E4M3 bytes to exact f16 (every E4M3 value is an f16 value): bytes (0, 1) and (2, 3) of
// each word, in that order.
__device__ __forceinline__ f16x8 f8_to_f16x8(uint32_t w0, uint32_t w1) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Channel (0..31 inside a lane's 32-channel key slice) of element i of QK MFMA j: element i is
// half i % 2 of pair 4 j + i / 2.
template <int KB>
__device__ __forceinline__ constexpr int kchan(int j, int i) {
  constexpr int HH = 16 / KB;
  const int r = 4 * j + i / 2;
  return (r / HH) * 2 * HH + (r % HH) + HH * (i % 2);
}

// Eight f16/bf16 values at channels base + kchan(j, 0..7) from a natural-order LDS row.
template <int KB>
__device__ __forceinline__ u16x8 gather_kchan(const uint16_t* row, int j) {
  if constexpr (KB == 2) {
    const int c0 = 16 * (j / 2) + 4 * (j % 2);
    const u16x4 a = *reinterpret_cast<const u16x4*>(row + c0);
    const u16x4 b = *reinterpret_cast<const u16x4*>(row + c0 + 8);
    return __builtin_shufflevector(a, b, 0, 4, 1, 5, 2, 6, 3, 7);
  } else {
    const u16x8 a = *reinterpret_cast<const u16x8*>(row + 8 * j);
    if constexpr (KB == 16) return a;
    if constexpr (KB == 4) return __builtin_shufflevector(a, a, 0, 4, 1, 5, 2, 6, 3, 7);
    else return __builtin_shufflevector(a, a, 0, 2, 1, 3, 4, 6, 5, 7);
  }
}

// Streaming loads of data read once per call: the nontemporal hint lets them pass through the
// caches without displacing anything (measured on MI355X: ~7.1 TB/s against ~6.4 TB/s for
// plain 128-bit loads).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream4(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 ld_stream2(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return uint2{v[0], v[1]};
}

// Buffer loads from a wave-uniform base: the base sits in the scalar resource and each lane
// adds a 32-bit byte offset, so a load costs no 64-bit address arithmetic per lane.  The
// resource's last word is the raw-buffer setting of this GPU family; the record count is the
// 2 GiB maximum (every offset here is within a tile or a scale row).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
constexpr int BUF_NT = 2;  // nontemporal cache policy (as the streaming loads above)
__device__ __forceinline__ uint4 bld4(rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, BUF_NT));
}
template <int AUX = BUF_NT>
__device__ __forceinline__ uint2 bld2(rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
}

// A lane's slice of a tile (4 KB bytes) at byte `off` of the tile's resource; 8- and 16-bit
// slices are stored as 16-byte pieces one 1 KiB slab apart, so each load instruction of a wave
// reads 1 KiB contiguously.
template <int KB>
__device__ __forceinline__ void load_words(rsrc_t r, unsigned off, uint32_t (&w)[KB]) {
  if constexpr (KB == 16) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 a = bld4(r, off + 1024 * i);
      w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
    }
  } else if constexpr (KB == 8) {
    const uint4 a = bld4(r, off);
    const uint4 b = bld4(r, off + 1024);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (KB == 4) {
    const uint4 a = bld4(r, off);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else {
    const uint2 a = bld2(r, off);
    w[0] = a.x; w[1] = a.y;
  }
}

template <int KB>
__device__ __forceinline__ void load_words(const uint8_t* ptr, uint32_t (&w)[KB]) {
  if constexpr (KB == 16) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 a = ld_stream4(ptr + 1024 * i);
      w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
    }
  } else if constexpr (KB == 8) {
    const uint4 a = ld_stream4(ptr);
    const uint4 b = ld_stream4(ptr + 1024);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (KB == 4) {
    const uint4 a = ld_stream4(ptr);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else {
    const uint2 a = ld_stream2(ptr);
    w[0] = a.x; w[1] = a.y;
  }
}

// ---- per-unit register data ----------------------------------------------------------------

// PV row blocks and the value-scale rows a lane needs.  Rows are (hi/lo part, value group, query
// head); with two row blocks there are exactly 16 (group, head) rows, so block pp is part pp and
// both blocks read the same value group: one set of scale rows serves both.
template <int NP>
constexpr int scale_rows() { return NP == 2 ? 1 : NP; }

template <int KB, int VB, int NP, bool KPC>
struct UnitData {
  uint32_t kw[2][KB];  // key slices of tiles A and B (token n, channels 32 g .. 32 g + 31)
  uint32_t vw[2][VB];  // value chunks of tiles A and B (tokens 4 g .. 4 g + 3, channels 8 n ..)
  uint2 ks[2];         // per-token keys: scale of tokens 4 g .. 4 g + 3 (column's group)
  uint2 kz[2];         // per-token asymmetric keys: zero-points
  uint2 vs[scale_rows<NP>()][2];  // value scales of tokens 4 g .. 4 g + 3 (row's group), tiles A, B
  uint2 vz[scale_rows<NP>()][2];  // asymmetric values: zero-points
  uint4 fs, fz;        // per-channel keys: scale / zero of the folding lane's 8 channels
};

// ---- the kernel ----------------------------------------------------------------------------

template <int MQ>
struct DecodeLds {
  // byte offsets inside the dynamic LDS block
  static constexpr int red = 0;                                   // [WAVES][16][RED_STRIDE] f32
  static constexpr int mw = red + WAVES * 16 * RED_STRIDE * 4;    // [WAVES][8] f32
  static constexpr int lw = mw + WAVES * 8 * 4;                   // [WAVES][8] f32
  static constexpr int zw = lw + WAVES * 8 * 4;                   // [WAVES][32] f32
  static constexpr int ztw = zw + WAVES * 32 * 4;                 // [WAVES][8] f32
  static constexpr int QB = MQ == 2 ? 4 : MQ == 3 ? 2 : 1;        // query-row blocks
  static constexpr int qs = ztw + WAVES * 8 * 4;                  // [QB][8][D] bf16
  static constexpr int ustat = qs + QB * 8 * D * 2;               // [WAVES][3] int: min, max,
                                                                  // count of units (> 0)
  static constexpr int qe = ustat + WAVES * 3 * 4;                // [QB][8] int: query row
                                                                  // prescale exponents
  static constexpr int pre = qe + QB * 8 * 4;                     // [B + 1] int
  // per-channel key folding buffer [WAVES][2][8][D] f16 overlays `red` (never live together)
  static constexpr int kf = red;
  static_assert(WAVES * 2 * 8 * D * 2 <= WAVES * 16 * RED_STRIDE * 4, "kf overlay");
  // then [B][2] int: each sequence's counters (n_quant, n_res) as the prologue read them
  __host__ __device__ static size_t cnt(int B) { return static_cast<size_t>(pre) + 4 * static_cast<size_t>(B + 1); }
  static size_t bytes(int B) { return cnt(B) + 8 * static_cast<size_t>(B); }
};

// Weighted work units of one sequence (per kv head): its compressed units plus ww per window
// unit, or -1 when its counters are out of range.
__device__ __forceinline__ int seq_units(const CacheDev& c, int max_tokens, int b, int ww) {
  const int nq = c.n_quant[b], nr = c.R > 0 ? c.n_res[b] : 0;
  if (nq < 0 || nr < 0 || nr > c.R || (!c.table && nq > c.cap) ||
      (c.table && (nq + TILE - 1) / TILE > c.max_blocks) || nq > max_tokens - nr)
    return -1;
  return (nq + 31) / 32 + ww * ((nr + 31) / 32);
}

// Ranges actually used of nb workgroups over S segments.  When every segment has the same number
// of units, ranges that end on segment boundaries save a segment restart and a partial per
// workgroup: nb rounded down to a multiple of S (each segment split m ways), or S / k with k | S
// (k whole segments per range), whichever aligned count is largest, if it keeps at least half of
// the workgroups.  Otherwise all nb ranges (Stream-K over the unit sequence).
// floor(a / b) for 0 <= a < 2^53 and b > 0 through one f64 division (a few instructions, where
// a 64-bit integer division is a long sequence).  The quotient is rounded to nearest; one that
// falls short of an integer n falls short by at least 1 / b, more than the rounding error
// q 2^-53 while a < 2^53, so it cannot round up to n.
__device__ __forceinline__ long long floor_div(long long a, long long b) {
  return static_cast<long long>(static_cast<double>(a) / static_cast<double>(b));
}

__device__ __forceinline__ int aligned_ranges(int nb, int S, bool uniform) {
  if (!uniform || S <= 0) return nb;
  if (S <= nb) return (nb / S) * S;
  int k = (S + nb - 1) / nb;
  while (S % k) k++;
  return (S / k >= (nb + 1) / 2) ? S / k : nb;
}

// KB, SCH: key bits and scheme; VB, VSCH: value bits and scheme (equal to the key's for FP8 and
// BF16 storage).
template <int KB, int G, bool KPC, int NP, int SCH, int MQ, int VB, int VSCH>
__global__ __launch_bounds__(256, (KB != 16 && MQ != 2 && MQ != 3 && (NP == 1 || G <= 4)) ? 3 : 2) void decode_kernel(DecodeParams p) {
  // multi-query geometry; single-query instantiations fold it to constants
  const int nqt = MQ ? p.nqt : 1, qbs = MQ ? p.qbs : 1, nqb = MQ ? p.nqb : 1, gkv = MQ ? p.gkv : G;
  // query blocks per segment, one per wave (1: the waves interleave the units of one block),
  // and segments per (sequence, kv head)
  constexpr int qpw = MQ == 2 ? 4 : MQ == 3 ? 2 : 1;
  constexpr int WPQ = WAVES / qpw;  // waves per query block
  const int nqs = MQ ? p.nqs : 1;
  constexpr bool KASYM = SCH == KVQ_ASYM, VASYM = VSCH == KVQ_ASYM;
  static_assert((SCH == KVQ_FP8) == (VSCH == KVQ_FP8) && (KB == 16) == (VB == 16), "formats");
  constexpr bool F8 = SCH == KVQ_FP8;  // E4M3 bytes, one scale per kv head (or tensor) per side
  // A segment's units are its compressed units, then WW slots per window unit; a window unit
  // belongs to the workgroup whose range holds its first slot.
  constexpr int WW = window_weight2(KB, VB);
  // In a batch of mixed lengths every segment also starts with SEG_W slots of no work, the cost
  // of a segment start (query staging, first loads) in units, so that a range holding many short
  // segments holds fewer units.  Batches of equal lengths (segment-aligned ranges) have none.
  constexpr int SEG_W = SEGMENT_START_WEIGHT;
  extern __shared__ __align__(16) unsigned char smem[];
  const CacheDev& c = p.c;
  const int B = c.B, H = c.H;
  const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;

  float* red = reinterpret_cast<float*>(smem + DecodeLds<MQ>::red);
  float* mw = reinterpret_cast<float*>(smem + DecodeLds<MQ>::mw);
  float* lw = reinterpret_cast<float*>(smem + DecodeLds<MQ>::lw);
  float* zw = reinterpret_cast<float*>(smem + DecodeLds<MQ>::zw);
  float* ztw = reinterpret_cast<float*>(smem + DecodeLds<MQ>::ztw);
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + DecodeLds<MQ>::qs);
  int* pre = reinterpret_cast<int*>(smem + DecodeLds<MQ>::pre);
  int* cnt = reinterpret_cast<int*>(smem + DecodeLds<MQ>::cnt(c.B));
  int* ustat = reinterpret_cast<int*>(smem + DecodeLds<MQ>::ustat);
  int* qe = reinterpret_cast<int*>(smem + DecodeLds<MQ>::qe);
  uint16_t* kf = reinterpret_cast<uint16_t*>(smem + DecodeLds<MQ>::kf) + wave * 2 * 8 * D;

  // ---- units per sequence, prefix sum (every workgroup; workgroup 0 publishes it) ----
  if (B <= 64) {
    // one wave: lane i takes sequence i, an in-register scan, one barrier
    if (wave == 0) {
      int un = 0;
      if (lane < B) {
        un = seq_units(c, p.max_tokens, lane, WW);
        cnt[2 * lane] = c.n_quant[lane];
        cnt[2 * lane + 1] = c.R > 0 ? c.n_res[lane] : 0;
        if (un < 0 && blockIdx.x == 0) atomicOr(c.err, KVQ_ERR_TOKENS);
      }
      int umin = (un > 0) ? un : INT_MAX, umax = max(un, 0), useq = (un > 0) ? 1 : 0;
      for (int off = 32; off > 0; off >>= 1) {
        umin = min(umin, __shfl_xor(umin, off));
        umax = max(umax, __shfl_xor(umax, off));
        useq += __shfl_xor(useq, off);
      }
      const int segw = umin != umax ? SEG_W : 0;
      const int own = (un > 0 ? un + segw : 0) * H * nqs;
      int incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      if (lane < B) pre[lane] = incl - own;
      if (lane == 63) pre[B] = incl;
      if (lane < WAVES) {  // this wave's totals in slot 0, neutral ones for the others
        ustat[3 * lane] = lane == 0 ? umin : INT_MAX;
        ustat[3 * lane + 1] = lane == 0 ? umax : 0;
        ustat[3 * lane + 2] = lane == 0 ? useq : 0;
      }
    }
    __syncthreads();
  } else {
    const int per = (B + 255) / 256;
    int* scan = reinterpret_cast<int*>(red);
    int umin = INT_MAX, umax = 0, useq = 0;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) {
      const int un = seq_units(c, p.max_tokens, i, WW);
      cnt[2 * i] = c.n_quant[i];  // kept for the segment starts (the loads above hit the cache)
      cnt[2 * i + 1] = c.R > 0 ? c.n_res[i] : 0;
      if (un < 0) {
        if (blockIdx.x == 0) atomicOr(c.err, KVQ_ERR_TOKENS);
      } else if (un > 0) {
        umin = min(umin, un);
        umax = max(umax, un);
        useq++;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      umin = min(umin, __shfl_xor(umin, off));
      umax = max(umax, __shfl_xor(umax, off));
      useq += __shfl_xor(useq, off);
    }
    if (lane == 0) {
      ustat[3 * wave] = umin;
      ustat[3 * wave + 1] = umax;
      ustat[3 * wave + 2] = useq;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WAVES; w++) {
      umin = min(umin, ustat[3 * w]);
      umax = max(umax, ustat[3 * w + 1]);
    }
    const int segw = umin != umax ? SEG_W : 0;
    auto weighted = [&](int i) {
      const int un = seq_units(c, p.max_tokens, i, WW);
      return (un > 0 ? un + segw : 0) * H * nqs;
    };
    int s = 0;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) s += weighted(i);
    scan[tid] = s;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int run = scan[tid] - s;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) {
      pre[i] = run;
      run += weighted(i);
    }
    if (tid == 255) pre[B] = scan[255];
    __syncthreads();
  }

  const int U = uni(pre[B]);
  // ranges in use (the combine reads the count back): segment-aligned for uniform batches
  int umin = ustat[0], umax = ustat[1], useq = ustat[2];
#pragma unroll
  for (int w = 1; w < WAVES; w++) {
    umin = min(umin, ustat[3 * w]);
    umax = max(umax, ustat[3 * w + 1]);
    useq += ustat[3 * w + 2];
  }
  const int nbe = uni(aligned_ranges(gridDim.x, useq * H * nqs, umin == umax));
  if (blockIdx.x == 0) {
    for (int i = tid; i <= B; i += 256) p.ws_pre[i] = pre[i];
    if (tid == 0) p.ws_pre[B + 1] = nbe;
  }
  if (static_cast<int>(blockIdx.x) >= nbe) return;
  if (gridDim.x == 1) {
    // a single workgroup: no combine runs after this launch, so empty sequences get their
    // zeros here
    for (int bb = 0; bb < B; bb++) {
      if (pre[bb + 1] != pre[bb]) continue;
      float* o = p.out + static_cast<size_t>(bb) * nqt * p.Hq * D;
      for (int i = tid; i < nqt * p.Hq * D; i += 256) o[i] = 0.0f;
    }
  }
  const long long NBl = nbe;
  const int u0 = static_cast<int>(floor_div(static_cast<long long>(blockIdx.x) * U, NBl));
  const int u1 = static_cast<int>(floor_div(static_cast<long long>(blockIdx.x + 1) * U, NBl));
  // Even progress of the workgroups that share a compute unit.  The issue arbiter favours the
  // oldest waves, so the first workgroup dispatched to a CU would finish its range well before
  // the last one, which then runs alone at a fraction of the CU's throughput (on the KIVI layer
  // the three workgroups of a CU ended at 68, 82 and 96 us on average).  Each wave starts at the
  // top priority and drops a level when its workgroup has done 50%, 75% and 90% of its range:
  // a workgroup ahead of the others on its CU yields issue slots until they catch up, and the
  // last band, where the order is again by age, is short.
  const int span = u1 - u0;
  int band = 0;
  __builtin_amdgcn_s_setprio(3);
  auto pace = [&](int done) {
    const int nb = (20 * done >= 18 * span) ? 3 : (20 * done >= 15 * span) ? 2 : (20 * done >= 10 * span) ? 1 : 0;
    if (nb == band) return;
    band = nb;
    switch (nb) {
      case 1: __builtin_amdgcn_s_setprio(2); break;
      case 2: __builtin_amdgcn_s_setprio(1); break;
      default: __builtin_amdgcn_s_setprio(0); break;
    }
  };
  if (u0 == u1) {
    // An empty range still owns slot 0, which the combine may read: make it neutral.
    float* part = p.ws_part + static_cast<size_t>(blockIdx.x) * 2 * qpw * G * PART_STRIDE;
    for (int i = tid; i < qpw * G * PART_STRIDE; i += 256) part[i] = (i % PART_STRIDE == 0) ? -FLT_MAX : 0.0f;
    return;
  }

  const int kgroup = (F8 || KB == 16) ? D : c.k.group, vgroup = (F8 || KB == 16) ? D : c.v.group;
  const int ngk = KPC ? 2 : D / kgroup;  // QK columns per head: key groups, or hi/lo parts
  const int ngv = D / vgroup;
  constexpr float koff = KASYM ? 0.0f : static_cast<float>(1 << (KB - 1));
  constexpr float voff = VASYM ? 0.0f : static_cast<float>(1 << (VB - 1));
  // Integer value codes enter PV as f16 subnormals alpha u 2^-24 (one and per pair).  alpha is
  // a token-position factor VT (at i % 4 >= 2; the weights come out of the exponential divided
  // by it) times a channel factor of MFMA j, removed with the 2^24 when the compressed units are
  // done.  The offset of symmetric codes (-off times the sum of w s_v) is accumulated apart (zo).
  constexpr bool VBF = !F8 && VB != 16;
  constexpr float VLG = VB == 4 ? 4.0f : VB == 2 ? 2.0f : 0.0f;  // log2 VT
  constexpr float VT = VB == 4 ? 16.0f : VB == 2 ? 4.0f : 1.0f;
  constexpr bool BF = KB == 16;  // unquantized BF16 storage: bf16 matrix products, no scales
  // QK on the vector ALU (KVQ_QK_VALU builds): lane (g, n) dots token 4 g + n % 4 with the
  // query over channel block n / 4, scales by its (token, key group) scale and sums the four
  // blocks along its row; every column of the row then holds the token's whole score
  constexpr bool VQK = KVQ_QK_VALU && G == 1 && KB == 8 && VB == 8 && SCH == KVQ_SYM &&
                       VSCH == KVQ_SYM && !KPC && MQ == 0;
  const int hh = n % G;          // query head of QK column n and of PV row 16 pp + n
  const int cg = (n / G) % ngk;  // key group (or hi/lo part) of QK column n
  constexpr long K_TILE_BYTES = static_cast<long>(TILE) * D * KB / 8;
  constexpr long V_TILE_BYTES = static_cast<long>(TILE) * D * VB / 8;

  int u = u0;
  bool first_seg = true;
  while (u < u1) {
    // ---- locate the segment: sequence b, kv head h, query block qblk, first slot kk ----
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int b = uni(lo);
    const int pb0 = uni(pre[b]);
    const int ub = uni((pre[b + 1] - pb0) / (H * nqs));
    const int sidx = (u - pb0) / ub, kk = (u - pb0) % ub;
    const int h = sidx / nqs, qgrp = sidx % nqs;
    const int qi = wave / WPQ;  // this wave's query block within the segment
    const int qblk = qgrp * qpw + qi;
    const int seg_abs_end = pb0 + (sidx + 1) * ub;
    const int uend = min(u1, seg_abs_end);
    const bool complete = (kk == 0) && (uend == seg_abs_end);
    const int slot = first_seg ? 0 : 1;
    const int nq = uni(cnt[2 * b]);
    const int nr = uni(cnt[2 * b + 1]);
    const int uq = (nq + 31) / 32;
    const int segw = umin != umax ? SEG_W : 0;
    const int ku = max(kk - segw, 0), xend = max(kk + (uend - u) - segw, 0);  // in units

    // ---- issue the segment's first loads before staging its query: the query rows, the
    // block-table entries and the first unit's codes and scales are in flight together ----
    // query row v of block bi = query token (qgrp qpw + bi) qbs + v / gkv, query head
    // h gkv + v % gkv (zero past the last); up to two 16-byte pieces per thread
    constexpr int QPC = MQ == 2 ? 2 : 1;
    uint4 qval[QPC];
#pragma unroll
    for (int k = 0; k < QPC; k++) {
      qval[k] = uint4{0u, 0u, 0u, 0u};
      const int piece = tid + 256 * k;
      if (piece < qpw * G * (D / 8)) {
        const int row = piece / (D / 8), bi = row / G, v = row % G;
        const int qg = (qgrp * qpw + bi) * qbs + v / gkv;
        if (qg < nqt)
          qval[k] = reinterpret_cast<const uint4*>(
              p.q + ((static_cast<size_t>(b) * nqt + qg) * p.Hq +
                     static_cast<size_t>(h) * gkv + v % gkv) * D)[piece % (D / 8)];
      }
    }
    // the WPQ waves of a block interleave its units; waves past the last block idle
    const int xstep = WPQ;
    int x = (qblk < nqb) ? ku + wave % WPQ : xend;
    const int xq_end = min(xend, uq);

    // PV row roles: row 16 pp + n is (part, value group, head hh)
    int rpart[NP], rgv[NP];
#pragma unroll
    for (int pp = 0; pp < NP; pp++) {
      const int row = 16 * pp + n;
      rpart[pp] = row / (G * ngv);
      rgv[pp] = (row / G) % ngv;
    }

    const int seq_tile0 = (b * H + h) * (c.cap / TILE);  // < 2^31 tiles (host check)
    const int* trow = c.table ? c.table + static_cast<size_t>(b) * c.max_blocks : nullptr;
    // physical tile of sequence tile t, or -1 for an unusable block-table entry
    auto phys_of = [&](int t) -> int {
      if (!trow) return seq_tile0 + t;
      const int blk = ld_uniform(trow + t);
      if (blk < 0 || blk >= c.num_blocks) return -1;
      return blk * H + h;
    };
    // Per-channel keys: lane l folds the eight channels of QK MFMA block (g', j') = (blk / 4,
    // blk % 4), blk = l % 16, for head l / 16 (and + 4): channels 32 g' + kchan(j', 0..7), which
    // are the run 8 blk .. 8 blk + 7 (8- and 4-bit) or two runs of four (2-bit).
    const int fold_blk = lane & 15;
    const int fold_c0 = (KB == 2) ? 32 * (fold_blk / 4) + 16 * ((fold_blk % 4) / 2) + 4 * (fold_blk % 2)
                                  : 8 * fold_blk;
    // per-channel key group tau's metadata row: contiguous [b][h][cap / Gt], paged with the
    // block of the group's first token (an unusable entry reads row 0; the block error is
    // reported where the codes are read)
    // (the row's first element; a lane reads its 8 channels from fold_c0 on)
    auto kpc_meta = [&](int tau) -> size_t {
      if (!trow) return ((static_cast<size_t>(b) * H + h) * (c.cap / kgroup) + tau) * D;
      const int blk = ld_uniform(trow + (tau * kgroup) / TILE);
      const int pb_ = (blk < 0 || blk >= c.num_blocks) ? 0 : blk;
      return (static_cast<size_t>(pb_) * H + h) * D;
    };
    auto load_meta8 = [&](const uint16_t* row) -> uint4 {
      const rsrc_t r = buf(row);
      if constexpr (KB == 2) {
        const uint2 a = bld2<0>(r, 2 * fold_c0);
        const uint2 bb = bld2<0>(r, 2 * fold_c0 + 16);
        return uint4{a.x, a.y, bb.x, bb.y};
      } else {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * fold_c0, 0, 0));
      }
    };
    UnitData<KB, VB, NP, KPC> d{};
    const UnpackRegs ur = unpack_regs<KB>();   // key code masks
    const UnpackRegs urv = unpack_regs<VB>();  // value code masks
    bool bad_block = false;
    // Every unit issues the same loads (an unusable or absent tile reads tile 0 of the buffer
    // and is ignored), so the compiler can count outstanding loads exactly.
    // Loads address a wave-uniform tile base (scalar registers) plus a 32-bit lane offset
    // that is fixed for the segment, so no per-lane 64-bit address arithmetic is needed.
    constexpr unsigned SPK = (4 * KB < 16) ? 4 * KB : 16;  // bytes of a key slice piece
    constexpr unsigned SPV = (4 * VB < 16) ? 4 * VB : 16;  // bytes of a value slice piece
    const unsigned k_lane = VQK ? SPK * (4 * (4 * g + (n & 3)) + (n >> 2))  // token 4 g + n % 4
                                : SPK * (4 * n + g);                    // slice 4 n + g (token n)
    const unsigned v_lane = SPV * (16 * g + n);              // chunk 16 g + n
    // scales of tokens 4 g .. 4 g + 3 in the lane's key group (VQK: the group of block n / 4)
    const unsigned ks_lane = (VQK ? (32 * (n >> 2)) / kgroup : cg) * TILE + 4 * g;
    auto load_k = [&](int xx, int pA, int pB) {
      pA = max(pA, 0);
      pB = max(pB, 0);
      if constexpr (BF || F8) {  // (measured: buffer loads made the BF16 kernel need more
                                 // registers, and the FP8 multi-query kernels 15% slower)
        load_words<KB>(c.kc + static_cast<size_t>(pA) * K_TILE_BYTES + k_lane, d.kw[0]);
        load_words<KB>(c.kc + static_cast<size_t>(pB) * K_TILE_BYTES + k_lane, d.kw[1]);
      } else {
        load_words<KB>(buf(c.kc + static_cast<size_t>(pA) * K_TILE_BYTES), k_lane, d.kw[0]);
        load_words<KB>(buf(c.kc + static_cast<size_t>(pB) * K_TILE_BYTES), k_lane, d.kw[1]);
      }
      if constexpr (BF || F8) {
      } else if constexpr (KPC) {
        // a paged key group of 16 or 32 tokens starts at this unit's tile A, whose block then
        // holds the group's metadata row: no second block-table read
        const size_t mrow = (trow && kgroup <= 2 * TILE) ? static_cast<size_t>(pA) * D
                                                         : kpc_meta((32 * xx) / kgroup);
        d.fs = load_meta8(c.ks + mrow);
        if constexpr (KASYM) d.fz = load_meta8(c.kz + mrow);
      } else {
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const size_t tb = static_cast<size_t>(t ? pB : pA) * c.ks_tile;
          d.ks[t] = bld2<0>(buf(c.ks + tb), 2 * ks_lane);
          if constexpr (KASYM) d.kz[t] = bld2<0>(buf(c.kz + tb), 2 * ks_lane);
        }
      }
    };
    auto load_v = [&](int pA, int pB) {
      pA = max(pA, 0);
      pB = max(pB, 0);
      if constexpr (BF || F8) {
        load_words<VB>(c.vc + static_cast<size_t>(pA) * V_TILE_BYTES + v_lane, d.vw[0]);
        load_words<VB>(c.vc + static_cast<size_t>(pB) * V_TILE_BYTES + v_lane, d.vw[1]);
      } else {
        load_words<VB>(buf(c.vc + static_cast<size_t>(pA) * V_TILE_BYTES), v_lane, d.vw[0]);
        load_words<VB>(buf(c.vc + static_cast<size_t>(pB) * V_TILE_BYTES), v_lane, d.vw[1]);
      }
      if constexpr (!BF && !F8)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const size_t tb = static_cast<size_t>(t ? pB : pA) * c.vs_tile;
#pragma unroll
        for (int pp = 0; pp < scale_rows<NP>(); pp++) {
          const unsigned lo = rgv[pp] * TILE + 4 * g;
          d.vs[pp][t] = bld2<0>(buf(c.vs + tb), 2 * lo);
          if constexpr (VASYM) d.vz[pp][t] = bld2<0>(buf(c.vz + tb), 2 * lo);
        }
      }
    };
    int pA = -1, pB = -1;
    if (x < xq_end) {
      pA = phys_of(2 * x);
      pB = (32 * x + 16 < nq) ? phys_of(2 * x + 1) : -1;
      load_k(x, pA, pB);
      load_v(pA, pB);
    }

    // ---- stage the segment's G query rows (bf16) and each row's prescale exponent ----
    // A row's 16 pieces sit on the 16 lanes of one DPP row: its |q| maximum is a row reduction.
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPC; k++) {
      const int piece = tid + 256 * k;
      float mx = 0.0f;
      if constexpr (!BF) {
        const uint32_t w4[4] = {qval[k].x, qval[k].y, qval[k].z, qval[k].w};
#pragma unroll
        for (int i = 0; i < 4; i++)
          mx = max3f(mx, __uint_as_float((w4[i] << 16) & 0x7FFF0000u), __uint_as_float(w4[i] & 0x7FFF0000u));
        mx = fmaxf(mx, row_ror<8>(mx));
        mx = fmaxf(mx, row_ror<4>(mx));
        mx = fmaxf(mx, row_ror<2>(mx));
        mx = fmaxf(mx, row_ror<1>(mx));
      }
      if (piece < qpw * G * (D / 8)) {
        const int row = piece / (D / 8);
        reinterpret_cast<uint4*>(qs + ((row / G) * 8 + row % G) * D)[piece % (D / 8)] = qval[k];
        if (piece % (D / 8) == 0) qe[(row / G) * 8 + row % G] = q_exponent(mx, KPC ? QE_FOLD : QE_RAW);
      }
    }
    __syncthreads();
    // this lane's QK column head: its query prescale 2^-e and the softmax scale of its scores
    // over compressed units, sm_scale log2(e) 2^e (BF16 storage: no prescale)
    const int qe_h = BF ? 0 : qe[qi * 8 + hh];
    const float qsc = exp2i(-qe_h);
    const float sl2 = p.sm_log2 * exp2i(qe_h);
    const uint16_t* qsw = qs + qi * 8 * D;  // this wave's query rows
    // causal limit (multi-query): the block's first query token sees the first lim_min cached
    // tokens (the query tokens are the last nqt), column n's token lim_min + hh / gkv of them;
    // single-query decode has no limit
    const int lim_min = MQ ? uni(nq + nr - nqt + qblk * qbs + 1) : INT_MAX;

    // ---- QK operand: f16 query, masked to the column's key group ----
    f16x8 qb[4];
    f16x2 qv[16];       // VQK: query pairs of the lane's channel block, in code-pair order
    float qbias = 0.0f;  // VQK: -(1024 + off) times the sum of those query values
    bf16x8 qbf[4];                            // BF16 storage: the bf16 query as it is
    f32x4 dq0 = f32x4{0.f, 0.f, 0.f, 0.f};  // QK accumulator start of every tile
    float qsum = 0.0f;  // asymmetric per-token keys: sum of q over the column's group
    float zt = 0.0f;    // asymmetric per-channel keys: sum of q * zero over the key group
    float f8k = 1.0f, f8v = 1.0f;  // FP8: the key and value scales of kv head h
    if constexpr (BF) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        qbf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qsw + hh * D + 32 * g + 8 * j));
    } else if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const u16x8 raw = *reinterpret_cast<const u16x8*>(qsw + hh * D + 32 * g + 8 * j);
#pragma unroll
        for (int i = 0; i < 8; i++) qb[j][i] = static_cast<_Float16>(bf16_to_f32(raw[i]) * qsc);
      }
      const int32_t* fks = reinterpret_cast<const int32_t*>(c.ks);
      const int32_t* fvs = reinterpret_cast<const int32_t*>(c.vs);
      f8k = __int_as_float(ld_uniform(fks + (c.k.axis == KVQ_PER_HEAD ? h : 0)));
      f8v = __int_as_float(ld_uniform(fvs + (c.v.axis == KVQ_PER_HEAD ? h : 0)));
    } else if constexpr (VQK) {
      // pair r of a code word holds channels 4 (r / 2) + r % 2 and that + 2 (bytes 0, 2 or 1, 3)
      const uint16_t* qrow = qsw + 32 * (n >> 2);
      float qs_ = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int c0 = 4 * (r / 2) + r % 2;
        qv[r] = f16x2{static_cast<_Float16>(bf16_to_f32(qrow[c0]) * qsc),
                      static_cast<_Float16>(bf16_to_f32(qrow[c0 + 2]) * qsc)};
        qs_ += static_cast<float>(qv[r][0]) + static_cast<float>(qv[r][1]);
      }
      qbias = -(1024.0f + koff) * qs_;
    } else if constexpr (!KPC) {
      const bool in_grp = ((32 * g) / kgroup) == cg;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const u16x8 raw = gather_kchan<KB>(qsw + hh * D + 32 * g, j);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float x = in_grp ? bf16_to_f32(raw[i]) * qsc : 0.0f;  // exact: a power of two
          qb[j][i] = static_cast<_Float16>(x * (1.0f / static_cast<float>(kelem_alpha<KB>(j, i))));
          if constexpr (KASYM) qsum += x;
        }
      }
      if constexpr (KASYM) {
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
      }
      // every token row starts at -sum_i qb_i (1024 + alpha_i off): the bias of the raw codes
#pragma unroll
      for (int j = 0; j < 4; j++) {
        f16x8 bias;
#pragma unroll
        for (int i = 0; i < 8; i++)
          bias[i] = static_cast<_Float16>(-(1024.0f + static_cast<float>(kelem_alpha<KB>(j, i)) * koff));
        dq0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(bias, qb[j], dq0, 0, 0, 0);
      }
    }

    float m_run = -FLT_MAX, l_run = 0.0f;
    // PV accumulator: 16 rows.  With one P operand the rows are (hi/lo part, value group,
    // query head); with two (NP == 2: 16 (value group, head) rows) the hi and lo operands are
    // two products into the same rows, so the parts are summed by the matrix cores.
    constexpr bool PARTS_IN_ROWS = NP == 1;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // symmetric subnormal value codes: -off times the sum of each row's products, one product
    // per unit against a constant operand, the same for every channel
    f32x4 zo = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 voffop;
#pragma unroll
    for (int i = 0; i < 8; i++)
      voffop[i] = static_cast<_Float16>(-voff * ((i & 2) ? VT : 1.0f) * 0x1p-24f);
    float zacc = 0.0f;  // asymmetric values: sum of w z of the lane's row

    // ---- online softmax over the 8 raw scores of a pair; returns the weights in s2 ----
    // m_run is in log2 units; weights are exp2(score * sm_log2 - m_run).  The running max starts
    // at a finite sentinel, so empty waves never form inf - inf.
    // With vfold, element i's weight comes out divided by alpha_i of the value codes it meets
    // (the raw-code PV operand), which only shifts its exponent.
    auto softmax = [&](float (&s2)[8], int nvA, int nvB, auto vfold, int tok0, float sl2_) {
      const bool full = nvA == 16 && nvB == 16;
      if (!full) {
#pragma unroll
        for (int i = 0; i < 8; i++)
          if (4 * g + (i & 3) >= (i < 4 ? nvA : nvB)) s2[i] = -INFINITY;
      }
      if (tok0 + 32 > lim_min) {  // tokens at or past a column's limit are hidden
        const int lim = lim_min + hh / gkv;
#pragma unroll
        for (int i = 0; i < 8; i++)
          if (tok0 + 16 * (i >> 2) + 4 * g + (i & 3) >= lim) s2[i] = -INFINITY;
      }
      const float m01 = max3f(s2[0], s2[1], s2[2]);
      const float m02 = max3f(s2[3], s2[4], s2[5]);
      float tmax = max3f(max3f(s2[6], s2[7], m01), m02, m02);
      tmax *= sl2_;
      if (__ballot(tmax > m_run + LAZY_LOG2) != 0) {
        float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
        hm = fmaxf(hm, __shfl_xor(hm, 32));
        const float mn = fmaxf(m_run, hm);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= alpha;
        zacc *= alpha;
        float al[G];
#pragma unroll
        for (int q = 0; q < G; q++)
          al[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), q));
#pragma unroll
        for (int r = 0; r < 4; r++) {
          float a;
          if constexpr (G <= 4) a = al[r % G];
          else a = (g & 1) ? al[4 + r] : al[r];
#pragma unroll
          for (int j = 0; j < 8; j++) acc[j][r] *= a;
          zo[r] *= a;
        }
        m_run = mn;
      }
      constexpr bool AT = decltype(vfold)::value && VT > 1.0f;  // factor VT at i % 4 >= 2
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float a = (AT && (i & 2)) ? VLG : 0.0f;  // log2 of element i's token factor
        s2[i] = __builtin_amdgcn_exp2f(fmaf(s2[i], sl2_, -m_run - a));  // -inf -> 0
      }
      const float l1 = (s2[0] + s2[1]) + (s2[4] + s2[5]);
      const float l16 = (s2[2] + s2[3]) + (s2[6] + s2[7]);
      l_run += AT ? fmaf(l16, VT, l1) : l1 + l16;
    };

    // sum the per-group (or hi/lo) columns of one head, for 8 scores at once
    auto fold_cols8 = [&](float (&v)[8]) {
      if (ngk >= 2) {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = row_ror<G>(v[i]) + v[i];
        if constexpr (2 * G < 16) {
          if (ngk >= 4) {
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = row_ror<2 * G>(v[i]) + v[i];
          }
        }
      }
    };

    // ---------------------------- compressed units ----------------------------
    if (x < xq_end) {
      // the query of the folding lane's channels, in MFMA element order, as f32 (per segment)
      // the query of the folding lane's 8 channels (natural order, as their scales arrive),
      // prescaled and as f16 pairs, once per segment: exact for every element within 2^31 of the
      // row's maximum (a bf16 significand fits an f16 one)
      f16x2 qn[(G + 3) / 4][4];
      if constexpr (KPC) {
#pragma unroll
        for (int r0 = 0; r0 < G; r0 += 4) {
          const int hw = min(r0 + (lane >> 4), G - 1);
          const uint16_t* qrow = qsw + hw * D + fold_c0;
          u16x8 q8;
          if constexpr (KB == 2) {  // channels c0 .. c0 + 3 and c0 + 8 .. c0 + 11
            const u16x4 a = *reinterpret_cast<const u16x4*>(qrow);
            const u16x4 b4 = *reinterpret_cast<const u16x4*>(qrow + 8);
            q8 = __builtin_shufflevector(a, b4, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            q8 = *reinterpret_cast<const u16x8*>(qrow);
          }
          const float fsc = exp2i(-qe[qi * 8 + hw]);  // the folded head's prescale
#pragma unroll
          for (int w = 0; w < 4; w++)
            qn[r0 / 4][w] = f16x2{static_cast<_Float16>(bf16_to_f32(q8[2 * w]) * fsc),
                                  static_cast<_Float16>(bf16_to_f32(q8[2 * w + 1]) * fsc)};
        }
      }

      // Raw key codes read as 1024 + alpha u: the folded query carries 1 / alpha of each
      // channel (a power of two), applied to the folding lane's 8 scales as they arrive.
      f16x2 ia2[4];
      if constexpr (KPC) {
#pragma unroll
        for (int w = 0; w < 4; w++)
          ia2[w] = f16x2{static_cast<_Float16>(fold_inv_alpha<KB>(fold_blk % 4, 2 * w)),
                         static_cast<_Float16>(fold_inv_alpha<KB>(fold_blk % 4, 2 * w + 1))};
      }

      // per-channel keys: fold one key group's scales (and zero-points) into the query, then
      // start the group's QK accumulator at minus the bias of the raw codes (plus, for
      // asymmetric keys, the zero-point term sum_i q_i z_i in the hi column)
      auto kpc_fold = [&](uint4 fs, uint4 fz) {
        // metadata words hold the lane's 8 channels in natural order; element i of the MFMA
        // block is natural index (0,4,1,5,2,6,3,7)[i] (2- and 4-bit) or (0,2,1,3,4,6,5,7)[i]
        uint32_t sw[4] = {fs.x, fs.y, fs.z, fs.w};
        const uint32_t zwd[4] = {fz.x, fz.y, fz.z, fz.w};
        if constexpr (KB != 8) {
#pragma unroll
          for (int w = 0; w < 4; w++) sw[w] = h2_bits(as_h2(sw[w]) * ia2[w]);
        }
#pragma unroll
        for (int r0 = 0; r0 < G; r0 += 4) {
          const int hw = r0 + (lane >> 4);
          float zp = 0.0f;
          if (hw < G) {
            // q s as f16 hi + lo on packed f16 math: hi = q s rounded, lo = q s - hi by one
            // fused op, exact (q s has at most 8 + 11 significant bits; q < 1, s <= 65504)
            f16x8 hn, ln;
#pragma unroll
            for (int w = 0; w < 4; w++) {
              const f16x2 sc = as_h2(sw[w]);
              const f16x2 h2 = qn[r0 / 4][w] * sc;
              const f16x2 l2 = __builtin_elementwise_fma(qn[r0 / 4][w], sc, -h2);
              hn[2 * w] = h2[0];
              hn[2 * w + 1] = h2[1];
              ln[2 * w] = l2[0];
              ln[2 * w + 1] = l2[1];
              if constexpr (KASYM) zp = __builtin_amdgcn_fdot2(qn[r0 / 4][w], as_h2(zwd[w]), zp, false);
            }
            f16x8 he, le;
            if constexpr (KB == 8) {
              he = __builtin_shufflevector(hn, hn, 0, 2, 1, 3, 4, 6, 5, 7);
              le = __builtin_shufflevector(ln, ln, 0, 2, 1, 3, 4, 6, 5, 7);
            } else {
              he = __builtin_shufflevector(hn, hn, 0, 4, 1, 5, 2, 6, 3, 7);
              le = __builtin_shufflevector(ln, ln, 0, 4, 1, 5, 2, 6, 3, 7);
            }
            *reinterpret_cast<f16x8*>(kf + hw * D + 8 * fold_blk) = he;
            *reinterpret_cast<f16x8*>(kf + (8 + hw) * D + 8 * fold_blk) = le;
          }
          if constexpr (KASYM) {
            zp += row_ror<8>(zp);
            zp += row_ror<4>(zp);
            zp += row_ror<2>(zp);
            zp += row_ror<1>(zp);
            if ((lane & 15) == 0 && hw < G) ztw[wave * 8 + hw] = zp;
          }
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; j++)
          qb[j] = *reinterpret_cast<const f16x8*>(kf + (cg * 8 + hh) * D + 8 * (4 * g + j));
        if constexpr (KASYM) zt = ztw[wave * 8 + hh];
        wave_lds_sync();
        // subnormal key codes alpha u 2^-24: symmetric codes start at minus the offset,
        // -off alpha 2^-24 against the same operand; asymmetric ones start at the zero-point
        // term sum_i q_i z_i, in the same 2^-24 units, in the hi column of each head
        dq0 = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!KASYM) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            f16x8 bias;
#pragma unroll
            for (int i = 0; i < 8; i++)
              bias[i] = static_cast<_Float16>(-static_cast<float>(kelem_alpha<KB>(j, i)) * koff * 0x1p-24f);
            dq0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(bias, qb[j], dq0, 0, 0, 0);
          }
        }
        if constexpr (KASYM) {
          const float z0 = (cg == 0) ? zt * 0x1p-24f : 0.0f;
          dq0 = f32x4{z0, z0, z0, z0};
        }
      };

      for (; x < xq_end; x += xstep) {
        pace((u - u0) + (x - ku));
        const int xn = x + xstep;
        const bool more = xn < xq_end;
        // after the last unit, reload the current tiles (cache hits) so the load count per
        // iteration stays fixed
        const int nA = more ? phys_of(2 * xn) : pA;
        const int nB = more ? ((32 * xn + 16 < nq) ? phys_of(2 * xn + 1) : -1) : pB;
        // valid tokens of tiles A and B (a tile whose block is unusable counts as empty)
        const int nvA = pA >= 0 ? min(16, nq - 32 * x) : 0;
        const int nvB = pB >= 0 ? min(16, nq - 32 * x - 16) : 0;
        bad_block |= pA < 0 || (32 * x + 16 < nq && pB < 0);

        // ---- QK^T of both tiles (two independent MFMA chains, interleaved) ----
        // Tiles past the sequence end hold finite codes of a stand-in tile; their scores are
        // masked below, so the MFMAs run unconditionally.
        if constexpr (KPC) kpc_fold(d.fs, d.fz);
        f32x4 dq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (KPC) {
          if (kgroup == 16 && nvB > 0) {
            // tile B opens its own key group: finish tile A with the current fold first
            dq[0] = dq0;
#pragma unroll
            for (int j = 0; j < 4; j++)
              dq[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_sub<KB>(d.kw[0], j, ur), qb[j], dq[0], 0, 0, 0);
            const size_t mrow = trow ? static_cast<size_t>(max(pB, 0)) * D : kpc_meta(2 * x + 1);
            const uint4 fs2 = load_meta8(c.ks + mrow);
            uint4 fz2 = uint4{0, 0, 0, 0};
            if constexpr (KASYM) fz2 = load_meta8(c.kz + mrow);
            kpc_fold(fs2, fz2);
            dq[1] = dq0;
#pragma unroll
            for (int j = 0; j < 4; j++)
              dq[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_sub<KB>(d.kw[1], j, ur), qb[j], dq[1], 0, 0, 0);
          } else {
            dq[0] = dq0;
            dq[1] = dq0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
              dq[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_sub<KB>(d.kw[0], j, ur), qb[j], dq[0], 0, 0, 0);
              dq[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_sub<KB>(d.kw[1], j, ur), qb[j], dq[1], 0, 0, 0);
            }
          }
        } else if constexpr (F8) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            dq[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f8_to_f16x8(d.kw[0][2 * j], d.kw[0][2 * j + 1]), qb[j], dq[0], 0, 0, 0);
            dq[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f8_to_f16x8(d.kw[1][2 * j], d.kw[1][2 * j + 1]), qb[j], dq[1], 0, 0, 0);
          }
        } else if constexpr (BF) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const bf16x8 ka = __builtin_bit_cast(bf16x8, uint4{d.kw[0][4 * j], d.kw[0][4 * j + 1], d.kw[0][4 * j + 2], d.kw[0][4 * j + 3]});
            const bf16x8 kb = __builtin_bit_cast(bf16x8, uint4{d.kw[1][4 * j], d.kw[1][4 * j + 1], d.kw[1][4 * j + 2], d.kw[1][4 * j + 3]});
            dq[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qbf[j], dq[0], 0, 0, 0);
            dq[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qbf[j], dq[1], 0, 0, 0);
          }
        } else if constexpr (VQK) {
#pragma unroll
          for (int t = 0; t < 2; t++) {
            float part = qbias;  // this lane's block: sum of (1024 + u) q, less (1024 + off) sum q
#pragma unroll
            for (int r = 0; r < 16; r++)
              part = __builtin_amdgcn_fdot2(as_h2(rawpair<KB>(d.kw[t], r, ur)), qv[r], part, false);
            const uint2 k2 = d.ks[t];
            const uint32_t kw2 = (n & 2) ? k2.y : k2.x;
            part *= (n & 1) ? f16_hi(kw2) : f16_lo(kw2);
            part = row_ror<4>(part) + part;
            part = row_ror<8>(part) + part;
            // token 4 g + r's score is in lanes 4 i + r of the row: broadcast it (quad_perm r)
            const int pi = __float_as_int(part);
            dq[t][0] = __int_as_float(__builtin_amdgcn_mov_dpp(pi, 0x00, 0xF, 0xF, true));
            dq[t][1] = __int_as_float(__builtin_amdgcn_mov_dpp(pi, 0x55, 0xF, 0xF, true));
            dq[t][2] = __int_as_float(__builtin_amdgcn_mov_dpp(pi, 0xAA, 0xF, 0xF, true));
            dq[t][3] = __int_as_float(__builtin_amdgcn_mov_dpp(pi, 0xFF, 0xF, 0xF, true));
          }
        } else {
          dq[0] = dq0;
          dq[1] = dq0;
#pragma unroll
          for (int j = 0; j < 4; j++) {
            dq[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_raw<KB>(d.kw[0], j, ur), qb[j], dq[0], 0, 0, 0);
            dq[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop_raw<KB>(d.kw[1], j, ur), qb[j], dq[1], 0, 0, 0);
          }
        }
        float s2[8];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          if constexpr (BF) {
#pragma unroll
            for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[t][r];
          } else if constexpr (F8) {
#pragma unroll
            for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[t][r] * f8k;
          } else if constexpr (KPC || VQK) {  // KPC: hi + lo columns are summed below, in 2^-24 units
#pragma unroll
            for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[t][r];
          } else {
            const uint2 k2 = d.ks[t];
            s2[4 * t + 0] = fmaf(dq[t][0], f16_lo(k2.x), 0.0f);
            s2[4 * t + 1] = fmaf(dq[t][1], f16_hi(k2.x), 0.0f);
            s2[4 * t + 2] = fmaf(dq[t][2], f16_lo(k2.y), 0.0f);
            s2[4 * t + 3] = fmaf(dq[t][3], f16_hi(k2.y), 0.0f);
            if constexpr (KASYM) {
              const uint2 z2 = d.kz[t];
              s2[4 * t + 0] += f16_lo(z2.x) * qsum;
              s2[4 * t + 1] += f16_hi(z2.x) * qsum;
              s2[4 * t + 2] += f16_lo(z2.y) * qsum;
              s2[4 * t + 3] += f16_hi(z2.y) * qsum;
            }
          }
        }
        load_k(more ? xn : x, nA, nB);  // key registers are free again
        if constexpr (!VQK) fold_cols8(s2);

        softmax(s2, nvA, nvB, std::integral_constant<bool, VBF>{}, 32 * x,
                KPC ? sl2 * 0x1p24f : sl2);  // s2: weights / alpha

        // ---- P rows (hi / lo f16 parts of w * s_v) and PV ----
        // Rows 16 pp + n with part >= 2 are never read back, so they are left as computed.
        // A stand-in tile's scales may be anything: its tokens' products are selected away.
        const bool full = nvA == 16 && nvB == 16;
        if constexpr (BF) {
          // bf16 hi / lo parts of w (truncations; hi + lo carries 16 significant bits); a
          // stand-in tile's tokens have w = 0 and its finite rows contribute nothing
          bf16x8 pb;
          uint32_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            uint32_t e2[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++) {
              const float wv = s2[2 * i + k2];
              const float lo_v = wv - __uint_as_float(__float_as_uint(wv) & 0xFFFF0000u);
              e2[k2] = __float_as_uint(rpart[0] == 1 ? lo_v : wv) >> 16;
            }
            pk[i] = e2[0] | (e2[1] << 16);
          }
          pb = __builtin_bit_cast(bf16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
          if (!full) {
            // stored bytes past the sequence end (or of a stand-in tile) may be anything, and
            // 0 * NaN is NaN: clear the lane's value halves of tokens it must not read
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
              const int nv = tt ? nvB : nvA;
#pragma unroll
              for (int w = 0; w < 16; w++) {
                // word w of the chunk holds tokens 2 (w % 2) and 2 (w % 2) + 1 of channel w / 2
                const int r0 = 4 * g + 2 * (w % 2);
                const uint32_t keep = (r0 < nv ? 0x0000FFFFu : 0u) | (r0 + 1 < nv ? 0xFFFF0000u : 0u);
                d.vw[tt][w] &= keep;
              }
            }
          }
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const bf16x8 vb = __builtin_bit_cast(bf16x8, uint4{d.vw[0][2 * j], d.vw[0][2 * j + 1], d.vw[1][2 * j], d.vw[1][2 * j + 1]});
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vb, acc[j], 0, 0, 0);
          }
          load_v(nA, nB);  // value registers are free again
          pA = nA;
          pB = nB;
          continue;
        }
        // With two P operands, operand 0 takes the hi parts and operand 1 the lo parts of the
        // same products w * s_v, formed once; with one, each lane's row picks its own part.
        f16x8 pa[NP];
        float neg1 = -1.0f;
        asm volatile("" : "+s"(neg1));
#pragma unroll
        for (int pp = 0; pp < scale_rows<NP>(); pp++) {
          const float sel = (rpart[pp] == 1) ? 1.0f : 0.0f;
          float ws[8];
#pragma unroll
          for (int t = 0; t < 2; t++) {
            if constexpr (F8) {
              // the head's value scale; P element order follows the converted bytes of a V
              // word, tokens (0, 2, 1, 3) of each tile
#pragma unroll
              for (int r = 0; r < 4; r++) ws[4 * t + r] = s2[4 * t + ((r == 1) ? 2 : (r == 2) ? 1 : r)] * f8v;
              continue;
            }
            const uint2 s2v = d.vs[pp][t];
            ws[4 * t + 0] = fmaf(s2[4 * t + 0], f16_lo(s2v.x), 0.0f);
            ws[4 * t + 1] = fmaf(s2[4 * t + 1], f16_hi(s2v.x), 0.0f);
            ws[4 * t + 2] = fmaf(s2[4 * t + 2], f16_lo(s2v.y), 0.0f);
            ws[4 * t + 3] = fmaf(s2[4 * t + 3], f16_hi(s2v.y), 0.0f);
            if constexpr (VASYM) {
              uint2 z2v = d.vz[pp][t];
              if (!full) {  // a token past the end may sit on a stand-in tile with any zero-point:
                            // clear the fp16 bits of tokens with no weight
                z2v.x &= (s2[4 * t] != 0.0f ? 0x0000FFFFu : 0u) | (s2[4 * t + 1] != 0.0f ? 0xFFFF0000u : 0u);
                z2v.y &= (s2[4 * t + 2] != 0.0f ? 0x0000FFFFu : 0u) | (s2[4 * t + 3] != 0.0f ? 0xFFFF0000u : 0u);
              }
              const float zv[4] = {f16_lo(z2v.x), f16_hi(z2v.x), f16_lo(z2v.y), f16_hi(z2v.y)};
              float zp = 0.0f;
#pragma unroll
              for (int r = 0; r < 4; r++) {
                const float wa = VBF ? s2[4 * t + r] * static_cast<float>(velem_alpha<VB>(0, r)) : s2[4 * t + r];
                zp = fmaf(zv[r], wa, zp);  // one mixed-precision fma on the fp16 zero-point
              }
              zacc += zp;
            }
          }
          if (!full) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
              const int si = F8 ? (i & 4) + (((i & 3) == 1) ? 2 : ((i & 3) == 2) ? 1 : (i & 3)) : i;
              ws[i] = (s2[si] != 0.0f) ? ws[i] : 0.0f;
            }
          }
          uint32_t pk[4], pl[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const f16x2 hi2 = pkrtz(ws[2 * i], ws[2 * i + 1]);
            if constexpr (NP == 2) {
              pk[i] = h2_bits(hi2);
              // ws - hi, exact, as one mixed-precision fma on the fp16 hi part (the -1 is kept in
              // a register: as a literal the fma folds to a subtraction of a converted hi)
              pl[i] = h2_bits(pkrtz(fmaf(static_cast<float>(hi2[0]), neg1, ws[2 * i]),
                                    fmaf(static_cast<float>(hi2[1]), neg1, ws[2 * i + 1])));
            } else {
              const float r0 = fmaf(-sel, static_cast<float>(hi2[0]), ws[2 * i]);
              const float r1 = fmaf(-sel, static_cast<float>(hi2[1]), ws[2 * i + 1]);
              pk[i] = h2_bits(pkrtz(r0, r1));
            }
          }
          pa[pp] = __builtin_bit_cast(f16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
          if constexpr (NP == 2) pa[1] = __builtin_bit_cast(f16x8, uint4{pl[0], pl[1], pl[2], pl[3]});
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
          if constexpr (VBF) {
            // subnormal codes alpha u 2^-24 against weights / token factor
            const f16x8 vb = vop_sub<VB>(d.vw[0], d.vw[1], j, urv);
#pragma unroll
            for (int pp = 0; pp < NP; pp++)
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[pp], vb, acc[j], 0, 0, 0);
            if constexpr (!VASYM) {
              if (j == 0) {
#pragma unroll
                for (int pp = 0; pp < NP; pp++)
                  zo = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[pp], voffop, zo, 0, 0, 0);
              }
            }
          } else if constexpr (F8) {
            // word j of each tile's chunk: channel 8 n + j of tokens (0, 2, 1, 3)
            const f16x8 vb = f8_to_f16x8(d.vw[0][j], d.vw[1][j]);
#pragma unroll
            for (int pp = 0; pp < NP; pp++)
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[pp], vb, acc[j], 0, 0, 0);
          }
        }
        load_v(nA, nB);  // value registers are free again
        pA = nA;
        pB = nB;
      }
      if (bad_block && lane == 0) atomicOr(c.err, KVQ_ERR_BLOCK);
    }
    // the compressed units' products are in units of 2^-24 / (channel factor of MFMA j); the
    // window rows below add true values
    if constexpr (VBF) {
#pragma unroll
      for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 4; r++)
          acc[j][r] = fmaf(acc[j][r], 16777216.0f / static_cast<float>(vchan_alpha<VB>(j)),
                           VASYM ? 0.0f : zo[r] * 16777216.0f);
    }

    // ---------------------------- BF16 window units ----------------------------
    // window units whose first slot lies in this range, interleaved over the block's waves
    const int wend = xend > uq ? (xend - uq + WW - 1) / WW : 0;
    int jw = (qblk < nqb) ? (max(ku, uq) - uq + WW - 1) / WW + wave % WPQ : wend;
    if (jw < wend) {
      // bf16 query operand in natural channel order, masked like the f16 one
      bf16x8 qw[4];
      const bool keep = KPC ? (cg == 0) : (((32 * g) / kgroup) == cg);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        u16x8 raw = *reinterpret_cast<const u16x8*>(qsw + hh * D + 32 * g + 8 * j);
        if (!keep) raw = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        qw[j] = __builtin_bit_cast(bf16x8, raw);
      }
      const uint16_t* kr = c.kres + (static_cast<size_t>(b) * H + h) * c.R * D;
      const uint16_t* vr = c.vres + (static_cast<size_t>(b) * H + h) * c.R * D;
      for (; jw < wend; jw += xstep) {
        const int r0 = 32 * jw;
        const int nvA = min(16, nr - r0), nvB = max(0, min(16, nr - r0 - 16));
        float s2[8];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          f32x4 dq = f32x4{0.f, 0.f, 0.f, 0.f};
          if ((t ? nvB : nvA) > 0) {
            const uint4* rowp = reinterpret_cast<const uint4*>(kr + (r0 + 16 * t + n) * D + 32 * g);
#pragma unroll
            for (int j = 0; j < 4; j++)
              dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rowp[j]), qw[j],
                                                           dq, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[r];
        }
        fold_cols8(s2);
        softmax(s2, nvA, nvB, std::false_type{}, nq + r0, p.sm_log2);
        // P rows: bf16 hi / lo parts of w (truncation; hi + lo carries 16 significant bits)
        bf16x8 pb[NP];
#pragma unroll
        for (int pp = 0; pp < NP; pp++) {
          uint32_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            uint32_t e2[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++) {
              const float wv = s2[2 * i + k2];
              const float lo_v = wv - __uint_as_float(__float_as_uint(wv) & 0xFFFF0000u);
              e2[k2] = __float_as_uint(rpart[pp] == 1 ? lo_v : wv) >> 16;
            }
            pk[i] = e2[0] | (e2[1] << 16);
          }
          pb[pp] = __builtin_bit_cast(bf16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
        }
        // V rows of tokens (tile A 4g..4g+3, tile B 4g..4g+3), channels 8n .. 8n+7, in two halves
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          uint2 vrow[8];
#pragma unroll
          for (int i = 0; i < 8; i++) {
            const int t = i / 4, row = r0 + 16 * t + 4 * g + (i % 4);
            const bool ok = 4 * g + (i % 4) < (t ? nvB : nvA);
            vrow[i] = ok ? *reinterpret_cast<const uint2*>(vr + row * D + 8 * n + 4 * hf) : uint2{0, 0};
          }
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            u16x8 col;
#pragma unroll
            for (int i = 0; i < 8; i++) {
              const uint32_t wv = (jj < 2) ? vrow[i].x : vrow[i].y;
              col[i] = static_cast<unsigned short>((jj & 1) ? (wv >> 16) : (wv & 0xFFFFu));
            }
            const int j = 4 * hf + jj;
#pragma unroll
            for (int pp = 0; pp < NP; pp++)
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[pp], __builtin_bit_cast(bf16x8, col),
                                                               acc[j], 0, 0, 0);
          }
        }
      }
    }

    // ---------------------------- merge the four waves ----------------------------
    float lsum = l_run + __shfl_xor(l_run, 16);
    lsum += __shfl_xor(lsum, 32);
    float zs = zacc + __shfl_xor(zacc, 16);
    zs += __shfl_xor(zs, 32);
    __syncthreads();  // every wave is done with kf (overlays red)
    if (lane < G) {
      mw[wave * 8 + lane] = m_run;
      lw[wave * 8 + lane] = lsum;
    }
    if (lane < 16) {
#pragma unroll
      for (int pp = 0; pp < 2; pp++) zw[wave * 32 + 16 * pp + lane] = pp ? 0.0f : zs;
    }
    if constexpr (MQ == 2) {
      // one query block per wave: each wave normalises (or writes the partial of) its own
      // block from its own rows of the merge buffer, no merge across waves
      constexpr int NOW = (G * D) / 64;  // outputs per lane
      float Ow[NOW];
      {
        wave_lds_sync();  // the m / l / z stores are done
#pragma unroll
        for (int j = 0; j < 8; j++)
#pragma unroll
          for (int r = 0; r < 4; r++) red[(wave * 16 + 4 * g + r) * RED_STRIDE + 8 * n + j] = acc[j][r];
        wave_lds_sync();
#pragma unroll
        for (int oi = 0; oi < NOW; oi++) {
          const int o = lane + 64 * oi;
          const int oh = o / D, ch = o % D;
          const int gv = ch / vgroup;
          Ow[oi] = VASYM ? zw[wave * 32 + gv * G + oh] : 0.0f;
#pragma unroll
          for (int part = 0; part < (PARTS_IN_ROWS ? 2 : 1); part++) {
            const int row = (part * ngv + gv) * G + oh;
            Ow[oi] += red[(wave * 16 + row) * RED_STRIDE + ch];
          }
        }
      }
#pragma unroll
      for (int oi = 0; oi < NOW; oi++) {
        const int o = lane + 64 * oi;
        const int oh = o / D, ch = o % D;
        const float L = lw[wave * 8 + oh];
        if (complete) {
          const int qg = qblk * qbs + oh / gkv;
          if (qg < nqt)
            p.out[((static_cast<size_t>(b) * nqt + qg) * p.Hq + static_cast<size_t>(h) * gkv +
                   oh % gkv) * D + ch] = (L > 0.0f) ? Ow[oi] / L : 0.0f;
        } else {
          float* part = p.ws_part +
                        (((static_cast<size_t>(blockIdx.x) * 2 + slot) * qpw + qi) * G + oh) * PART_STRIDE;
          if (ch == 0) {
            part[0] = mw[wave * 8 + oh];
            part[1] = L;
          }
          part[4 + ch] = Ow[oi];
        }
      }
      u = uend;
      first_seg = false;
      continue;
    }
    // merge the WPQ waves of each of the qpw blocks (one block of all four waves unless mode 3)
    constexpr int NO = (qpw * G * D + 255) / 256;
    float O[NO], Mx[NO], e[NO][WPQ];
    {
#pragma unroll
      for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) red[(wave * 16 + 4 * g + r) * RED_STRIDE + 8 * n + j] = acc[j][r];
      __syncthreads();
#pragma unroll
      for (int oi = 0; oi < NO; oi++) {
        const int o = tid + 256 * oi;
        if (o >= qpw * G * D) continue;
        const int qo = o / (G * D), oh = (o % (G * D)) / D, ch = o % D;  // block, row, channel
        const int w0 = qo * WPQ;                                           // its first wave
        const int gv = ch / vgroup;
        {
          float M = -FLT_MAX;
#pragma unroll
          for (int k = 0; k < WPQ; k++) M = fmaxf(M, mw[(w0 + k) * 8 + oh]);
          Mx[oi] = M;
          O[oi] = 0.0f;
#pragma unroll
          for (int k = 0; k < WPQ; k++) {
            const float mv = mw[(w0 + k) * 8 + oh];
            e[oi][k] = __builtin_amdgcn_exp2f(mv - M);  // waves without tokens hold -FLT_MAX
          }
          if constexpr (VASYM) {
            const int row0 = gv * G + oh;
#pragma unroll
            for (int k = 0; k < WPQ; k++) O[oi] += e[oi][k] * zw[(w0 + k) * 32 + row0];
          }
        }
#pragma unroll
        for (int part = 0; part < (PARTS_IN_ROWS ? 2 : 1); part++) {
          const int row = (part * ngv + gv) * G + oh;
#pragma unroll
          for (int k = 0; k < WPQ; k++)
            O[oi] += e[oi][k] * red[((w0 + k) * 16 + row) * RED_STRIDE + ch];
        }
      }
    }
#pragma unroll
    for (int oi = 0; oi < NO; oi++) {
      const int o = tid + 256 * oi;
      if (o >= qpw * G * D) continue;
      const int qo = o / (G * D), oh = (o % (G * D)) / D, ch = o % D;
      const int w0 = qo * WPQ;
      float L = 0.0f;
#pragma unroll
      for (int k = 0; k < WPQ; k++) L += e[oi][k] * lw[(w0 + k) * 8 + oh];
      if (complete) {
        const int qg = (qgrp * qpw + qo) * qbs + oh / gkv;
        if (qg < nqt)
          p.out[((static_cast<size_t>(b) * nqt + qg) * p.Hq + static_cast<size_t>(h) * gkv +
                 oh % gkv) * D + ch] = (L > 0.0f) ? O[oi] / L : 0.0f;
      } else {
        float* part = p.ws_part +
                      (((static_cast<size_t>(blockIdx.x) * 2 + slot) * qpw + qo) * G + oh) * PART_STRIDE;
        if (ch == 0) {
          part[0] = Mx[oi];
          part[1] = L;
        }
        part[4 + ch] = O[oi];
      }
    }
    u = uend;
    first_seg = false;
  }
}

// First workgroup whose unit range [k U / NB, (k+1) U / NB) contains unit u.
__device__ __forceinline__ int block_of(long long u, long long U, long long NB) {
  return static_cast<int>(floor_div((u + 1) * NB - 1, U));
}

// Merge the partials of each (sequence, kv head) that more than one workgroup worked on; write
// zeros for empty sequences.  Each output is merged by CG threads over interleaved partials,
// then across them in LDS.
//
// Grid (B * H * query blocks, S) with S slices of a block's G x D outputs; T threads per
// workgroup.  A workgroup takes OPP = min(G D / S, 256) outputs per pass with CG = T / OPP
// threads each; thread (cgi, oi) folds partials kf + cgi, kf + cgi + CG, ... with the
// log-sum-exp rule, and the OPP threads of a group read contiguous floats of one partial.
// S and T are chosen on the host from the partials a segment has on average: many slices and
// 1024 threads when few segments are split many ways (one long sequence), one slice of 256
// threads when many short segments have a partial or two each (a smaller launch).
template <int G, int S, int T>
__global__ __launch_bounds__(T) void combine_kernel(DecodeParams p) {
  static_assert((G * D) % S == 0 && (G * D) / S >= 32, "combine slices");
  __shared__ float sm[T], sl[T], so[T];
  const int H = p.c.H, B = p.c.B;
  // one workgroup per (sequence, kv head, query block); the decode segment holding the block is
  // (kv head, group of qpw blocks), the block's partials sit at position qi of each slot
  const int QB = H * p.nqb;
  const int b = blockIdx.x / QB, hq = blockIdx.x % QB;
  const int h = hq / p.nqb, qblk = hq % p.nqb;
  const int qpw = p.qpw, qi = qblk % qpw, sidx = h * p.nqs + qblk / qpw;
  constexpr int opb = (G * D) / S;
  constexpr int opp = opb < 256 ? opb : 256;
  constexpr int cg = T / opp;
  const int oi = threadIdx.x % opp, cgi = threadIdx.x / opp;
  const int* pre = p.ws_pre;
  const long long U = pre[B], NB = pre[B + 1];  // ranges the decode launch used
  const int ub = (pre[b + 1] - pre[b]) / (H * p.nqs);
  // output element o of the segment's G x D block (row o / D: query token, query head)
  auto dst = [&](int o) -> float* {
    const int row = o / D, qg = qblk * p.qbs + row / p.gkv;
    if (qg >= p.nqt) return nullptr;
    return p.out + ((static_cast<size_t>(b) * p.nqt + qg) * p.Hq + static_cast<size_t>(h) * p.gkv +
                    row % p.gkv) * D + o % D;
  };
  if (ub == 0) {
    for (int o = threadIdx.x; o < opb; o += T)
      if (float* d = dst(static_cast<int>(blockIdx.y) * opb + o)) *d = 0.0f;
    return;
  }
  const long long us = pre[b] + static_cast<long long>(sidx) * ub, ue = us + ub;
  const int kf = block_of(us, U, NB), kl = block_of(ue - 1, U, NB);
  if (kf == kl) return;  // one workgroup saw the whole sequence and wrote the output
  const int s0 = (floor_div(static_cast<long long>(kf) * U, NB) == us) ? 0 : 1;
  for (int o0 = 0; o0 < opb; o0 += opp) {
    const int o = static_cast<int>(blockIdx.y) * opb + o0 + oi;
    const int oh = o / D, ch = o % D;
    float M = -FLT_MAX, L = 0.0f, O = 0.0f;
#pragma unroll 4
    for (int k = kf + cgi; k <= kl; k += cg) {
      const float* pt =
          p.ws_part + (((static_cast<size_t>(k) * 2 + (k == kf ? s0 : 0)) * qpw + qi) * G + oh) * PART_STRIDE;
      const float m = pt[0], l = pt[1], v = pt[4 + ch];
      const float mn = fmaxf(M, m);
      const float a = __builtin_amdgcn_exp2f(M - mn), e = __builtin_amdgcn_exp2f(m - mn);
      L = L * a + l * e;
      O = O * a + v * e;
      M = mn;
    }
    sm[threadIdx.x] = M;
    sl[threadIdx.x] = L;
    so[threadIdx.x] = O;
    __syncthreads();
    if (cgi == 0) {
      float Mt = -FLT_MAX;
#pragma unroll
      for (int q = 0; q < cg; q++) Mt = fmaxf(Mt, sm[q * opp + oi]);
      float Lt = 0.0f, Ot = 0.0f;
#pragma unroll
      for (int q = 0; q < cg; q++) {
        const float e = __builtin_amdgcn_exp2f(sm[q * opp + oi] - Mt);
        Lt += e * sl[q * opp + oi];
        Ot += e * so[q * opp + oi];
      }
      if (float* d = dst(o)) *d = (Lt > 0.0f) ? Ot / Lt : 0.0f;
    }
    __syncthreads();
  }
}

// Workgroups of decode_kernel that are resident at once on the current device.  Each workgroup
// owns 1/NB of the units, so the grid must never exceed what runs concurrently.  The answer
// depends on the device and the LDS size alone and is cached per instantiation.
template <int KB, int G, bool KPC, int NP, int SCH, int MQ, int VB, int VSCH>
int decode_resident_blocks(size_t lds) {
  static std::mutex mu;
  static int cached_dev = -1, cached_blocks = 0;
  static size_t cached_lds = 0;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> g(mu);
    if (dev == cached_dev && lds == cached_lds) return cached_blocks;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<KB, G, KPC, NP, SCH, MQ, VB, VSCH>,
                                                   256, lds) != hipSuccess)
    return 0;
  std::lock_guard<std::mutex> g(mu);
  cached_dev = dev;
  cached_lds = lds;
  cached_blocks = cus * per_cu;
  return cached_blocks;
}

template <int KB, int G, bool KPC, int NP, int SCH, int MQ, int VB, int VSCH>
hipError_t launch_decode_t(const DecodeParams& p0, hipStream_t s) {
  DecodeParams p = p0;
  const size_t lds = DecodeLds<MQ>::bytes(p.c.B);
  const int resident = decode_resident_blocks<KB, G, KPC, NP, SCH, MQ, VB, VSCH>(lds);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  if (p.nblocks > resident) p.nblocks = resident;
  decode_kernel<KB, G, KPC, NP, SCH, MQ, VB, VSCH><<<p.nblocks, 256, lds, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup saw every segment whole and wrote every output (empty sequences included):
  // nothing to combine
  if (p.nblocks == 1) return hipSuccess;
  // slices: about one per 4 partials a segment has on average, 32 outputs per slice at most
  const int avg = p.nblocks / (p.c.B * p.c.H * p.nqs);
  int slices = 1;
  while (slices < 16 && slices * 2 <= avg / 4 && (G * D) / (slices * 2) >= 32) slices *= 2;
  const dim3 grid(p.c.B * p.c.H * p.nqb, slices);
  switch (avg < 8 ? 0 : slices) {  // 0: one slice, 256 threads for short partial chains
    case 0: combine_kernel<G, 1, 256><<<grid, 256, 0, s>>>(p); break;
    case 1: combine_kernel<G, 1, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 2: combine_kernel<G, 2, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 4: combine_kernel<G, 4, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 8: if constexpr (G >= 2) combine_kernel<G, 8, 1024><<<grid, 1024, 0, s>>>(p); break;
    default: if constexpr (G >= 4) combine_kernel<G, 16, 1024><<<grid, 1024, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

template <int KB, int SCH, int MQ, int VB, int VSCH>
hipError_t launch_decode_mq(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  if constexpr (KB == 16 || SCH == KVQ_FP8) {  // whole-row formats: at most 16 PV rows
    if (kpc || NP != 1) return hipErrorInvalidValue;
    switch (G) {
      case 1: return launch_decode_t<KB, 1, false, 1, SCH, MQ, VB, VSCH>(p, s);
      case 2: return launch_decode_t<KB, 2, false, 1, SCH, MQ, VB, VSCH>(p, s);
      case 4: return launch_decode_t<KB, 4, false, 1, SCH, MQ, VB, VSCH>(p, s);
      case 8: return launch_decode_t<KB, 8, false, 1, SCH, MQ, VB, VSCH>(p, s);
      default: return hipErrorInvalidValue;
    }
  } else {
#define KVQ_CASE(GG, NN)                                                        \
  if (G == GG && NP == NN)                                                      \
    return kpc ? launch_decode_t<KB, GG, true, NN, SCH, MQ, VB, VSCH>(p, s)    \
               : launch_decode_t<KB, GG, false, NN, SCH, MQ, VB, VSCH>(p, s);
  KVQ_CASE(1, 1)
  KVQ_CASE(2, 1)
  KVQ_CASE(4, 1)
  KVQ_CASE(4, 2)
  KVQ_CASE(8, 1)
  KVQ_CASE(8, 2)
#undef KVQ_CASE
    return hipErrorInvalidValue;
  }
}

// Single-query decode and the three multi-query modes are separate instantiations, so the
// single-query kernel carries none of the query-block bookkeeping: mode 1 has the four waves of
// a workgroup interleave the units of one query block, mode 3 gives two blocks two waves each,
// mode 2 gives each wave its own block.
template <int KB, int SCH>
hipError_t launch_decode_bits(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  if (p.nqt <= 1) return launch_decode_mq<KB, SCH, 0, KB, SCH>(p, G, NP, kpc, s);
  switch (p.qpw) {
    case 4: return launch_decode_mq<KB, SCH, 2, KB, SCH>(p, G, NP, kpc, s);
    case 2: return launch_decode_mq<KB, SCH, 3, KB, SCH>(p, G, NP, kpc, s);
    default: return launch_decode_mq<KB, SCH, 1, KB, SCH>(p, G, NP, kpc, s);
  }
}

// Keys and values in different integer formats (bits and/or scheme): single-query decode and the
// three multi-query modes, as for one format.
template <int KB, int SCH>
hipError_t launch_decode_mixed(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc,
                               hipStream_t s) {
#define KVQ_VFMT(VBB, VS)                                                        \
  if constexpr (VBB != KB || VS != SCH)                                          \
    if (vb == VBB && vsch == VS) {                                               \
      if (p.nqt <= 1) return launch_decode_mq<KB, SCH, 0, VBB, VS>(p, G, NP, kpc, s); \
      switch (p.qpw) {                                                           \
        case 4: return launch_decode_mq<KB, SCH, 2, VBB, VS>(p, G, NP, kpc, s);  \
        case 2: return launch_decode_mq<KB, SCH, 3, VBB, VS>(p, G, NP, kpc, s);  \
        default: return launch_decode_mq<KB, SCH, 1, VBB, VS>(p, G, NP, kpc, s); \
      }                                                                          \
    }
  KVQ_VFMT(2, KVQ_SYM)
  KVQ_VFMT(2, KVQ_ASYM)
  KVQ_VFMT(4, KVQ_SYM)
  KVQ_VFMT(4, KVQ_ASYM)
  KVQ_VFMT(8, KVQ_SYM)
  KVQ_VFMT(8, KVQ_ASYM)
#undef KVQ_VFMT
  return hipErrorInvalidValue;
}

}  // namespace kvq
