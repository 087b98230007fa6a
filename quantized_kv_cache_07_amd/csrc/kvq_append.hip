// kvq_append.hip -- quantize-and-append and window flush kernels (gfx950).
//
// Quantizers [P2 = llmdaily.org "KV-cache quantization -- making long-context inference fit in
// memory", section "From BF16 to INT8, INT4, or even fewer bits"]:
//   symmetric   s = max|x| / (2^(b-1) - 1),  q = clip(round(x / s), -Q, Q)
//   asymmetric  s = (max - min) / (2^b - 1), z = min, u = clip(round((x - z) / s), 0, 2^b - 1)
// with the fp32 scale rounded once to fp16 (nearest even) and x / s an IEEE fp32 division by the
// stored scale; round() is half away from zero.  Groups [P2, "Why scales and groups matter"]:
// per token over `group` channels, or, for keys, per channel over `group` tokens [P3 =
// oh-bug.com "KV Cache Quantization in Practice", "Why Can't You Quantize the KV Cache Like
// Ordinary Activations?"].  The window [P2, "Why some systems keep a full-precision window"]:
// new tokens enter a BF16 window of R rows; when a token finds it full, the R rows are
// quantized into the compressed cache first.
//
// One call = two kernels on one stream:
//   quantize_kernel  grid (segments, B * H_kv): every slot the call moves into the compressed
//                    cache -- window rows and/or new rows -- is quantized into LDS, then packed
//                    into the storage layout (K rows, token-interleaved V tiles, fp16 metadata).
//                    A segment is 16 slots (one tile), or one per-channel key group.
//   tail_kernel      grid (B): checks the whole slot range, copies the new window rows and only
//                    then advances the counters, so a faulty sequence is left unchanged.
#include "kvq_dev.h"

#pragma clang fp contract(off)

namespace kvq {

// --- group quantizers; `get(i)` returns element i as fp32 (exact bf16 widening) --------------

template <class Get>
__device__ __forceinline__ void quant_sym(Get get, int n, int bits, uint16_t& s16out,
                                          uint8_t* codes, int stride) {
  const int Q = (1 << (bits - 1)) - 1;
  float m = 0.0f;
  for (int i = 0; i < n; i++) m = fmaxf(m, fabsf(get(i)));
  const float s32 = m / static_cast<float>(Q);
  const __half sh = __float2half_rn(s32);
  const float sf = __half2float(sh);
  for (int i = 0; i < n; i++) {
    int q = 0;
    if (sf != 0.0f) {
      float r = roundf(get(i) / sf);
      r = fminf(fmaxf(r, static_cast<float>(-Q)), static_cast<float>(Q));
      q = static_cast<int>(r);
    }
    codes[i * stride] = static_cast<uint8_t>(q + (1 << (bits - 1)));
  }
  s16out = __half_as_ushort(sh);
}

template <class Get>
__device__ __forceinline__ void quant_asym(Get get, int n, int bits, uint16_t& s16out,
                                           uint16_t& z16out, uint8_t* codes, int stride) {
  const int M = (1 << bits) - 1;
  float lo = get(0), hi = lo;
  for (int i = 1; i < n; i++) {
    const float x = get(i);
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  const float range = hi - lo;
  const float s32 = range / static_cast<float>(M);
  const __half sh = __float2half_rn(s32);
  const __half zh = __float2half_rn(lo);
  const float sf = __half2float(sh), zf = __half2float(zh);
  for (int i = 0; i < n; i++) {
    int u = 0;
    if (sf != 0.0f) {
      const float diff = get(i) - zf;
      float r = roundf(diff / sf);
      r = fminf(fmaxf(r, 0.0f), static_cast<float>(M));
      u = static_cast<int>(r);
    }
    codes[i * stride] = static_cast<uint8_t>(u);
  }
  s16out = __half_as_ushort(sh);
  z16out = __half_as_ushort(zh);
}

// OCP FP8 E4M3 code of y: the nearest E4M3 value (ties to the even code, i.e. round-half-even
// on the integer significand), saturating at +-448; the sign is kept (-0 -> 0x80).
__device__ __forceinline__ uint8_t e4m3_rne_sat(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return static_cast<uint8_t>(sign | 0x7Eu);
  if (a < 0.015625f)  // below 2^-6: subnormal codes m 2^-9, m = 0..8 (8 is the smallest normal)
    return static_cast<uint8_t>(sign | static_cast<uint32_t>(rintf(a * 512.0f)));
  const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
  const float m8 = rintf(a * __uint_as_float(static_cast<uint32_t>(127 + 3 - e) << 23));  // 8..16
  const int code = ((e + 7) << 3) + (static_cast<int>(m8) - 8);  // 16 carries into the exponent
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(code > 0x7E ? 0x7E : code));
}

// Row j of the slots this call moves into the compressed cache: the window rows first, then
// the new rows.
__device__ __forceinline__ const uint16_t* pending_row(const CacheDev& c, const uint16_t* fresh,
                                                       int n_new, int b, int h, int j, int nr,
                                                       bool key) {
  if (j < nr) return (key ? c.kres : c.vres) + ((static_cast<size_t>(b) * c.H + h) * c.R + j) * D;
  return fresh + ((static_cast<size_t>(b) * n_new + (j - nr)) * c.H + h) * D;
}

// Position (slot-in-tile t, channel ch) of field f of word q of a V tile (inverse of the layout).
__device__ __forceinline__ void v_field_owner(int bits, int q, int f, int& t, int& ch) {
  const int E = 32 / bits, Hh = E / 2;
  const int chunk = q / bits, word = q % bits;
  const int g = chunk / (D / 8), n = chunk % (D / 8);
  const int k = f % Hh, half = f / Hh;
  const int r = word * Hh + k;
  const int jj = r / 2, p = r % 2;
  t = 4 * g + 2 * p + half;
  ch = 8 * n + jj;
}

template <int S>
__global__ __launch_bounds__(256) void quantize_kernel(CacheDev c, const uint16_t* knew,
                                                       const uint16_t* vnew, int n_new, int mode) {
  __shared__ uint8_t lk[S][D];
  __shared__ uint8_t lv[S][D];
  __shared__ __align__(16) uint16_t xs[S][2][D];  // pending bf16 rows (keys, values)
  __shared__ uint16_t mk_s[S * 4], mk_z[S * 4], mv_s[S * 4], mv_z[S * 4];
  __shared__ uint16_t pc_s[D], pc_z[D];
  __shared__ int s_ok;

  const int tid = threadIdx.x;
  const int b = blockIdx.y / c.H, h = blockIdx.y % c.H;
  constexpr int PIECES = D * 2 / 16;  // 16-byte pieces of a bf16 row
  // One new token and no window (a decode step): the token is this workgroup's only slot
  // wherever the counters put it, so its two rows load in parallel with the counters.
  const bool one_row = mode == MODE_APPEND && c.R == 0 && n_new == 1;
  uint4 row_piece = uint4{0u, 0u, 0u, 0u};
  if (one_row && tid < 2 * PIECES)
    row_piece = reinterpret_cast<const uint4*>((tid < PIECES ? knew : vnew) +
                                               (static_cast<size_t>(b) * c.H + h) * D)[tid % PIECES];
  const int nq = c.n_quant[b];
  int nr = c.R > 0 ? c.n_res[b] : 0;
  if (nq < 0 || nr < 0 || nr > c.R) return;  // corrupt counters: reported by tail_kernel
  int F, total, nra;
  step_counts(mode, c.R, nr, n_new, F, total, nra);
  if (F <= 0) return;
  const int seg0 = (nq / S) * S + static_cast<int>(blockIdx.x) * S;
  const int lo = max(seg0, nq), hi = min(seg0 + S, nq + F);
  if (lo >= hi) return;
  if (!c.table && nq + F > c.cap) return;  // reported by tail_kernel; nothing written
  // per-channel key groups start at multiples of S: a sequence whose n_quant is not one would
  // split a group (reported by tail_kernel; nothing of the sequence is written)
  if (c.k.axis == KVQ_PER_CHANNEL && (nq % S != 0 || lo != seg0 || hi != seg0 + S)) return;
  if (tid == 0) {
    int ok = 1;
    if (c.table)
      for (int t = seg0 / TILE; t < (seg0 + S) / TILE; t++) {
        bool tok = true;
        (void)tile_index(c, b, h, t, tok);
        if (!tok) ok = 0;
      }
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) return;

  const SideDev K = c.k, V = c.v;
  const bool fp8 = K.scheme == KVQ_FP8;  // both sides share the scheme
  const int ngk = (!fp8 && K.axis == KVQ_PER_TOKEN) ? D / K.group : 0;
  const int ngv = fp8 ? 0 : D / V.group;

  // Phase 0: the pending bf16 rows of this segment into LDS (16-byte pieces).
  if (one_row) {
    if (tid < 2 * PIECES) reinterpret_cast<uint4*>(&xs[lo - seg0][tid / PIECES][0])[tid % PIECES] = row_piece;
  } else {
    const int pieces = PIECES;
    const int n_items = (hi - lo) * 2 * pieces;
    for (int it = tid; it < n_items; it += blockDim.x) {
      const int piece = it % pieces;
      const int side = (it / pieces) % 2;
      const int slot = lo + it / (2 * pieces);
      const uint16_t* row =
          pending_row(c, side ? vnew : knew, n_new, b, h, slot - nq, nr, side == 0);
      reinterpret_cast<uint4*>(&xs[slot - seg0][side][0])[piece] =
          reinterpret_cast<const uint4*>(row)[piece];
    }
  }
  __syncthreads();

  // BF16 storage (bits 16): the elements go in unchanged, into the same slice layout as codes
  // (K: channels 8 p .. 8 p + 7 of row t are piece p % 4 of slice 4 t + p / 4; V: channel ch of
  // row t is halfword 4 (ch % 8) + t % 4 of chunk (t / 4) (D / 8) + ch / 8), and there is no
  // metadata.
  if (K.bits == 16) {
    for (int it = tid; it < (hi - lo) * PIECES; it += blockDim.x) {
      const int slot = lo + it / PIECES, pc = it % PIECES;
      bool ok = true;
      const long tile = tile_index(c, b, h, slot / TILE, ok);
      const long off = slab_byte(16, 4 * (slot % TILE) + pc / 4, 128 * (pc % 4));
      *reinterpret_cast<uint4*>(c.kc + tile * TILE * (D * 2) + off) =
          reinterpret_cast<const uint4*>(&xs[slot - seg0][0][0])[pc];
    }
    for (int it = tid; it < (hi - lo) * D; it += blockDim.x) {
      const int slot = lo + it / D, ch = it % D, tr = slot % TILE;
      bool ok = true;
      const long tile = tile_index(c, b, h, slot / TILE, ok);
      const int chunk = (tr / 4) * (D / 8) + ch / 8;
      const long off = slab_byte(16, chunk, 16 * (4 * (ch % 8) + tr % 4));
      *reinterpret_cast<uint16_t*>(c.vc + tile * TILE * (D * 2) + off) = xs[slot - seg0][1][ch];
    }
    return;
  }

  // FP8: every element is E4M3(x / s) with the side's scale for this kv head (or tensor).
  if (fp8) {
    const float* fks = reinterpret_cast<const float*>(c.ks);
    const float* fvs = reinterpret_cast<const float*>(c.vs);
    const float sk = fks[K.axis == KVQ_PER_HEAD ? h : 0], sv = fvs[V.axis == KVQ_PER_HEAD ? h : 0];
    for (int it = tid; it < (hi - lo) * 2 * D; it += blockDim.x) {
      const int j = lo - seg0 + it / (2 * D), side = (it / D) % 2, ch = it % D;
      const float x = bf16_to_f32(xs[j][side][ch]);
      (side ? lv : lk)[j][ch] = e4m3_rne_sat(x / (side ? sv : sk));
    }
  }

  // Phase 1a: per-token groups.  One wave per (slot, side) row; lane l holds channels 2l and
  // 2l + 1, and the group's maximum (or minimum and maximum) is reduced across its lanes.
  if (!fp8) {
    const int wave = tid >> 6, lane = tid & 63;
    const bool k_pt = K.axis == KVQ_PER_TOKEN;
    const int nside = k_pt ? 2 : 1;  // per-channel keys are quantized in phase 1b
    const int rows = (hi - lo) * nside;
    for (int it = wave; it < rows; it += blockDim.x >> 6) {
      const int side = k_pt ? (it % 2) : 1;
      const int j = lo - seg0 + it / nside;
      const SideDev& sd = side ? V : K;
      const int gl = sd.group / 2;  // lanes per group
      const float x0 = bf16_to_f32(xs[j][side][2 * lane]);
      const float x1 = bf16_to_f32(xs[j][side][2 * lane + 1]);
      uint8_t* codes = side ? &lv[j][0] : &lk[j][0];
      uint16_t s16, z16 = 0;
      int u0, u1;
      if (sd.scheme == KVQ_SYM) {
        const int Q = (1 << (sd.bits - 1)) - 1;
        float m = fmaxf(fabsf(x0), fabsf(x1));
        for (int o = 1; o < gl; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float s32 = m / static_cast<float>(Q);
        const __half sh = __float2half_rn(s32);
        const float sf = __half2float(sh);
        int q0 = 0, q1 = 0;
        if (sf != 0.0f) {
          q0 = static_cast<int>(fminf(fmaxf(roundf(x0 / sf), static_cast<float>(-Q)), static_cast<float>(Q)));
          q1 = static_cast<int>(fminf(fmaxf(roundf(x1 / sf), static_cast<float>(-Q)), static_cast<float>(Q)));
        }
        u0 = q0 + (1 << (sd.bits - 1));
        u1 = q1 + (1 << (sd.bits - 1));
        s16 = __half_as_ushort(sh);
      } else {
        const int M = (1 << sd.bits) - 1;
        float lo_v = fminf(x0, x1), hi_v = fmaxf(x0, x1);
        for (int o = 1; o < gl; o <<= 1) {
          lo_v = fminf(lo_v, __shfl_xor(lo_v, o));
          hi_v = fmaxf(hi_v, __shfl_xor(hi_v, o));
        }
        const float range = hi_v - lo_v;
        const float s32 = range / static_cast<float>(M);
        const __half sh = __float2half_rn(s32);
        const __half zh = __float2half_rn(lo_v);
        const float sf = __half2float(sh), zf = __half2float(zh);
        int a0 = 0, a1 = 0;
        if (sf != 0.0f) {
          const float d0 = x0 - zf, d1 = x1 - zf;
          a0 = static_cast<int>(fminf(fmaxf(roundf(d0 / sf), 0.0f), static_cast<float>(M)));
          a1 = static_cast<int>(fminf(fmaxf(roundf(d1 / sf), 0.0f), static_cast<float>(M)));
        }
        u0 = a0;
        u1 = a1;
        s16 = __half_as_ushort(sh);
        z16 = __half_as_ushort(zh);
      }
      codes[2 * lane] = static_cast<uint8_t>(u0);
      codes[2 * lane + 1] = static_cast<uint8_t>(u1);
      if ((lane % gl) == 0) {
        const int g = lane / gl;
        if (side) {
          mv_s[j * 4 + g] = s16;
          mv_z[j * 4 + g] = z16;
        } else {
          mk_s[j * 4 + g] = s16;
          mk_z[j * 4 + g] = z16;
        }
      }
    }
  }

  // Phase 1b: per-channel keys: the segment is exactly one group of S tokens (lo == seg0, hi ==
  // seg0 + S: flushes move whole windows, R is a multiple of the group); a thread per channel.
  if (!fp8 && K.axis == KVQ_PER_CHANNEL) {
    for (int ch = tid; ch < D; ch += blockDim.x) {
      auto get = [&](int j) { return bf16_to_f32(xs[j][0][ch]); };
      uint16_t s16 = 0, z16 = 0;
      if (K.scheme == KVQ_SYM)
        quant_sym(get, S, K.bits, s16, &lk[0][ch], D);
      else
        quant_asym(get, S, K.bits, s16, z16, &lk[0][ch], D);
      pc_s[ch] = s16;
      pc_z[ch] = z16;
    }
  }
  __syncthreads();

  // Phase 2a: K rows, one 32-bit word per item.
  {
    const int E = 32 / K.bits, DW = D / E, RB = D * K.bits / 8;
    const int n_items = (hi - lo) * DW;
    for (int it = tid; it < n_items; it += blockDim.x) {
      const int slot = lo + it / DW, w = it % DW;
      bool ok = true;
      const long tile = tile_index(c, b, h, slot / TILE, ok);
      uint32_t word = 0;
      for (int f = 0; f < E; f++)
        word |= static_cast<uint32_t>(lk[slot - seg0][w * E + f]) << (f * K.bits);
      // word w of row t: channels w E .. w E + E - 1, slice 4 t + w E / 32
      const long off = slab_byte(K.bits, 4 * (slot % TILE) + (w * E) / 32, ((w * E) % 32) * K.bits);
      *reinterpret_cast<uint32_t*>(c.kc + tile * TILE * RB + off) = word;
    }
  }
  // Phase 2b: V tiles, one 32-bit word per item; words shared with slots outside [lo, hi)
  // keep those slots' bits (read-modify-write by the single owner of the tile).  8-bit codes
  // are whole bytes: a tile the range covers only in part gets byte stores instead, with no
  // read of the words it shares with other slots.
  const bool v_bytes = V.bits == 8 && (lo % TILE != 0 || hi % TILE != 0);
  if (v_bytes) {
    const long tile_bytes = static_cast<long>(TILE) * D;
    for (int it = tid; it < (hi - lo) * D; it += blockDim.x) {
      const int slot = lo + it / D, ch = it % D, t = slot % TILE;
      bool ok = true;
      const long tile = tile_index(c, b, h, slot / TILE, ok);
      // inverse of v_field_owner for 8-bit fields: chunk, word in the chunk, field in the word
      const int chunk = (t / 4) * (D / 8) + ch / 8;
      const int r = 2 * (ch % 8) + (t % 4) / 2;
      const int fld = r % 2 + 2 * (t % 2);
      c.vc[tile * tile_bytes + slab_byte(8, chunk, 32 * (r / 2) + 8 * fld)] = lv[slot - seg0][ch];
    }
  }
  if (!v_bytes) {
    const int E = 32 / V.bits;
    const int words = (D / 8) * 4 * V.bits;  // per tile
    const int t_first = seg0 / TILE, n_tiles = S / TILE;
    const long tile_bytes = static_cast<long>(TILE) * D * V.bits / 8;
    for (int it = tid; it < n_tiles * words; it += blockDim.x) {
      const int tl = t_first + it / words, q = it % words;
      const int base_slot = tl * TILE;
      if (base_slot + TILE <= lo || base_slot >= hi) continue;
      bool ok = true;
      const long tile = tile_index(c, b, h, tl, ok);
      uint32_t val = 0, mask = 0;
      for (int f = 0; f < E; f++) {
        int t, ch;
        v_field_owner(V.bits, q, f, t, ch);
        const int slot = base_slot + t;
        if (slot >= lo && slot < hi) {
          val |= static_cast<uint32_t>(lv[slot - seg0][ch]) << (f * V.bits);
          mask |= ((1u << V.bits) - 1u) << (f * V.bits);
        }
      }
      // word q of the chunk sequence: word q % bits of chunk q / bits
      uint32_t* dst = reinterpret_cast<uint32_t*>(c.vc + tile * tile_bytes +
                                                  slab_byte(V.bits, q / V.bits, 32 * (q % V.bits)));
      if (mask == 0xFFFFFFFFu) {
        *dst = val;
      } else if (mask != 0u) {
        // fields of slots outside [lo, hi) keep their bits: clear this range's fields, then set
        // them (two atomics from one thread to one word apply in order; nothing waits on them,
        // where a read-modify-write would put a memory round trip on the append's path)
        atomicAnd(dst, ~mask);
        atomicOr(dst, val);
      }
    }
  }
  // Phase 2c: metadata (none for FP8: its scales are the caller's).
  if (fp8) return;
  if (K.axis == KVQ_PER_TOKEN) {
    for (int it = tid; it < (hi - lo) * ngk; it += blockDim.x) {
      const int slot = lo + it / ngk, g = it % ngk;
      bool ok = true;
      const long tile = tile_index(c, b, h, slot / TILE, ok);
      const size_t idx = static_cast<size_t>(tile) * c.ks_tile + g * TILE + slot % TILE;
      c.ks[idx] = mk_s[(slot - seg0) * 4 + g];
      if (K.scheme == KVQ_ASYM) c.kz[idx] = mk_z[(slot - seg0) * 4 + g];
    }
  } else {
    // the group's row: per (sequence, head) in order, or with the block of its first token
    const int tau = seg0 / S;
    bool ok = true;
    const size_t row = c.table ? static_cast<size_t>(tile_index(c, b, h, seg0 / TILE, ok))
                               : (static_cast<size_t>(b) * c.H + h) * (c.cap / S) + tau;
    for (int ch = tid; ch < D; ch += blockDim.x) {
      const size_t idx = row * D + ch;
      c.ks[idx] = pc_s[ch];
      if (K.scheme == KVQ_ASYM) c.kz[idx] = pc_z[ch];
    }
  }
  for (int it = tid; it < (hi - lo) * ngv; it += blockDim.x) {
    const int slot = lo + it / ngv, g = it % ngv;
    bool ok = true;
    const long tile = tile_index(c, b, h, slot / TILE, ok);
    const size_t idx = static_cast<size_t>(tile) * c.vs_tile + g * TILE + slot % TILE;
    c.vs[idx] = mv_s[(slot - seg0) * 4 + g];
    if (V.scheme == KVQ_ASYM) c.vz[idx] = mv_z[(slot - seg0) * 4 + g];
  }
}

__global__ __launch_bounds__(256) void tail_kernel(CacheDev c, const uint16_t* knew,
                                                   const uint16_t* vnew, int n_new, int mode) {
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int nq = c.n_quant[b];
  const int nr = c.R > 0 ? c.n_res[b] : 0;
  int F, total, nra;
  step_counts(mode, c.R, nr, n_new, F, total, nra);
  if (tid == 0) {
    s_bad = (nq < 0 || nr < 0 || nr > c.R) ? KVQ_ERR_CAPACITY : 0;
    if (!s_bad && F > 0 && c.k.axis == KVQ_PER_CHANNEL && nq % c.k.group != 0) s_bad = KVQ_ERR_GROUP;
  }
  __syncthreads();
  if (F > 0 && !s_bad) {
    if (!c.table) {
      if (nq + F > c.cap && tid == 0) s_bad = KVQ_ERR_CAPACITY;
    } else {
      for (int t = nq / TILE + tid; t <= (nq + F - 1) / TILE; t += blockDim.x) {
        bool ok = true;
        (void)tile_index(c, b, 0, t, ok);
        if (!ok) atomicOr(&s_bad, KVQ_ERR_BLOCK);
      }
    }
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) atomicOr(c.err, s_bad);
    return;
  }
  if (mode == MODE_APPEND && c.R > 0) {
    // window rows j' in [max(0, nr - F), nra) receive new row F + j' - nr
    const int j0 = max(0, nr - F);
    const int rows = nra - j0;
    const int per_row = D * 2 / 16;  // 16-byte pieces per bf16 row
    const int n_items = 2 * c.H * rows * per_row;
    for (int it = tid; it < n_items; it += blockDim.x) {
      const int piece = it % per_row;
      int rest = it / per_row;
      const int jr = j0 + rest % rows;
      rest /= rows;
      const int h = rest % c.H;
      const bool key = rest / c.H == 0;
      const uint16_t* src = (key ? knew : vnew) +
                            ((static_cast<size_t>(b) * n_new + (F + jr - nr)) * c.H + h) * D;
      uint16_t* dst = (key ? c.kres : c.vres) + ((static_cast<size_t>(b) * c.H + h) * c.R + jr) * D;
      reinterpret_cast<uint4*>(dst)[piece] = reinterpret_cast<const uint4*>(src)[piece];
    }
  }
  __syncthreads();
  if (tid == 0) {
    c.n_quant[b] = nq + F;
    c.n_res[b] = nra;
  }
}

// Host-side launch of one append/flush call.
hipError_t launch_append(const CacheDev& c, const uint16_t* knew, const uint16_t* vnew, int n_new,
                         int mode, hipStream_t stream) {
  const int S = (c.k.axis == KVQ_PER_CHANNEL) ? c.k.group : TILE;
  // slots one call can move: n_new without a window, else whole windows: R floor((n_res + n_new
  // - 1) / R) <= R floor((R + n_new - 1) / R)
  const int f_max = (mode == MODE_FLUSH) ? c.R
                    : (c.R == 0 ? n_new : c.R * ((c.R + n_new - 1) / c.R));
  // S-slot segments a range of f_max slots can touch, wherever it starts
  const int segs = (f_max + S - 2) / S + 1;
  dim3 grid(segs, c.B * c.H);
  switch (S) {
    case 16: quantize_kernel<16><<<grid, 256, 0, stream>>>(c, knew, vnew, n_new, mode); break;
    case 32: quantize_kernel<32><<<grid, 256, 0, stream>>>(c, knew, vnew, n_new, mode); break;
    case 64: quantize_kernel<64><<<grid, 256, 0, stream>>>(c, knew, vnew, n_new, mode); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tail_kernel<<<c.B, 256, 0, stream>>>(c, knew, vnew, n_new, mode);
  return hipGetLastError();
}

}  // namespace kvq
