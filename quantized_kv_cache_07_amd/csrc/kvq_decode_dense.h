// kvq_decode_dense.h -- causal multi-query decode with sixteen query rows per wave (gfx950).
//
//   out[b][i][hq] = softmax(sm_scale q_i K^T + causal mask) V    [P2 = llmdaily.org "KV-cache
//   quantization -- making long-context inference fit in memory", "Why the KV cache grows so
//   quickly", attention equation; the query tokens are the last n_q cached tokens], over the
//   compressed tokens dequantized in registers as they stream in (P3 = oh-bug.com "KV Cache
//   Quantization in Practice", "Misconception 1"), then the BF16 window.
//
// For caches with one format on both sides -- integer with per-token key groups of 32, 64 or 128
// channels, FP8 E4M3 or BF16 -- and n_q x (query heads per kv head) >= 16 (the host takes it from
// 32 rows, from 16 for 8- and 16-bit codes).  A query block is 16 rows (query tokens x GQA
// heads); a workgroup's four waves take four blocks of one (sequence, kv head) and walk the same
// units, so the codes stream once for up to 64 rows.  Per unit (32 tokens) each wave unpacks a
// quarter of the unit's operands into LDS, one barrier, then every wave reads all of them:
//   QK^T  raw key codes as f16 (1024 + alpha u, one and-or per pair), re-ordered so that product
//         j takes key slice j (channels 32 j .. 32 j + 31, inside one key group), against the 16
//         query rows divided by alpha; the bias is removed by the accumulator start and each
//         group's sum is multiplied by the token's group scale: exact products, as in the
//         single-query kernel.
//   PV    P = the 16 rows' weights as f16; the values dequantized to f16, s (u - off) 2^-8 (or
//         (s u + z) 2^-8), one subtraction and one multiply (or fma) per two codes after the
//         raw-form unpack.  Rounding w and v to f16 (11 bits) keeps the output within the
//         pages' tolerance; the 2^-8 keeps every finite fp16 scale times a code below the f16
//         limit and is removed before the window rows add true values.
//   FP8   E4M3 bytes convert exactly to f16 on both sides; the head's key scale goes into the
//         softmax scale and its value scale multiplies the output.
//   BF16  the stored bf16 words are the operands as they are (bf16 products; weights as bf16
//         hi and lo parts).
// Split segments leave partials for combine_kernel, as in the single-query kernel.
#pragma once

#include "kvq_decode.h"

namespace kvq {

constexpr int DROWS = 16;  // query rows of a dense block

struct DenseLds {
  static constexpr int red = 0;                                  // [WAVES][16][RED_STRIDE] f32
  static constexpr int mw = red + WAVES * 16 * RED_STRIDE * 4;   // [WAVES][16] f32
  static constexpr int lw = mw + WAVES * DROWS * 4;              // [WAVES][16] f32
  static constexpr int qs = lw + WAVES * DROWS * 4;              // [4][16][D] bf16
  static constexpr int ustat = qs + 4 * DROWS * D * 2;           // [WAVES][3] int
  static constexpr int qe = ustat + WAVES * 3 * 4;               // [4][16] int
  static constexpr int pre = qe + 4 * DROWS * 4;                 // [B + 1] int
  // a unit's operands, unpacked once per workgroup, in the merge rows (which hold nothing while
  // units stream): values dequantized [2 units][8 products][64 lanes] x 16 bytes, then raw key
  // codes [2 units][2 tiles][4 key slices][64 lanes] x 16 bytes
  static constexpr int vbuf = red;
  static constexpr int kbuf = red + 2 * 8 * 64 * 16;
  __host__ __device__ static size_t cnt(int B) { return static_cast<size_t>(pre) + 4 * static_cast<size_t>(B + 1); }
  static size_t bytes(int B) { return cnt(B) + 8 * static_cast<size_t>(B); }
};
static_assert(WAVES * 16 * RED_STRIDE * 4 >= 2 * (8 + 8) * 64 * 16, "unit operands fit the merge rows");

// Code words of a value chunk (or key slice) that wave w unpacks: pairs 4 w .. 4 w + 3, i.e.
// words 2 w, 2 w + 1 of 8-bit codes, word w of 4-bit codes and half of word w / 2 of 2-bit codes
// (the wave shifts odd halves down by 8 bits); value products 2 w and 2 w + 1 use these pairs,
// and so does the part of a key slice that lane group w of a QK product takes.  BF16 storage
// (16-byte pieces one 1 KiB slab apart): piece w of a key slice (8 channels) or of a value chunk
// (channels 2 w and 2 w + 1 of its four tokens).
template <int KB>
constexpr int vwords() { return KB == 16 ? 4 : KB == 8 ? 2 : 1; }
template <int KB>
__device__ __forceinline__ unsigned vword_off(int w) {
  if constexpr (KB == 16) return 1024u * w;
  else if constexpr (KB == 8) return 1024u * (w / 2) + 8u * (w % 2);
  else if constexpr (KB == 4) return 4u * w;
  else return 4u * (w / 2);
}
// The key words at byte voff + soff of resource r (soff: the tile's byte offset, wave-uniform).
template <int KB>
__device__ __forceinline__ void load_vwords(rsrc_t r, unsigned voff, int soff, uint32_t (&x)[vwords<KB>()]) {
  if constexpr (KB == 16) {
    const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, BUF_NT));
    x[0] = a.x;
    x[1] = a.y;
    x[2] = a.z;
    x[3] = a.w;
  } else if constexpr (KB == 8) {
    const uint2 a = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, BUF_NT));
    x[0] = a.x;
    x[1] = a.y;
  } else {
    x[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, BUF_NT);
  }
}

// The loaded words of wave w as the array rawpair() indexes: 2-bit codes of an odd wave are the
// upper halves' fields, shifted down here (at use, not at the load, which would wait for it).
template <int KB>
__device__ __forceinline__ void vwords_at_use(const uint32_t (&x)[vwords<KB>()], int w, uint32_t (&y)[vwords<KB>()]) {
#pragma unroll
  for (int i = 0; i < vwords<KB>(); i++) y[i] = (KB == 2) ? x[i] >> (8 * (w & 1)) : x[i];
}
// 8 bytes of scale (or zero-point) rows at byte voff + soff of resource r
__device__ __forceinline__ uint2 ld_rows(rsrc_t r, unsigned voff, int soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// KB: code bits of keys and values (the same format on both sides; 16: BF16 storage); SCH:
// KVQ_SYM, KVQ_ASYM or KVQ_FP8 (E4M3 bytes with one fp32 scale per kv head or tensor; KB 8,
// NGK 1);
// NGK: key groups per row (1: groups of 128 channels, 2: of 64, 4: of 32).  Three workgroups per
// CU for key groups of 64 or 128 (168 VGPRs; the few spills the compiler makes fall outside the
// unit loop: 16 queries ran 7-19% faster than at two, symmetric 2-bit codes in groups of 64 17%),
// two for asymmetric 2-bit codes (the same time at three) and for groups of 32 (slower at three:
// four key groups' accumulators, 3-4% for 4- and 2-bit codes, 40% for asymmetric 2-bit ones).
template <int KB, int SCH, int NGK>
__global__ __launch_bounds__(256, (NGK == 4 || (KB == 2 && SCH == KVQ_ASYM)) ? 2 : 3) void dense_kernel(DecodeParams p) {
  constexpr int G = DROWS;
  constexpr int qpw = 4;  // query blocks per segment, one per wave
  constexpr bool ASYM = SCH == KVQ_ASYM;
  constexpr bool F8 = SCH == KVQ_FP8;
  constexpr bool BF = KB == 16;
  static_assert(!F8 || (KB == 8 && NGK == 1), "FP8 caches: bytes, no groups");
  static_assert(!BF || (SCH == KVQ_SYM && NGK == 1), "BF16 caches: no scales, no groups");
  constexpr int WW = window_weight2(KB, KB);
  constexpr int SEG_W = SEGMENT_START_WEIGHT;
  const int nqt = p.nqt, qbs = p.qbs, nqb = p.nqb, gkv = p.gkv, nqs = p.nqs;
  extern __shared__ __align__(16) unsigned char smem[];
  const CacheDev& c = p.c;
  const int B = c.B, H = c.H;
  const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;

  float* red = reinterpret_cast<float*>(smem + DenseLds::red);
  float* mw = reinterpret_cast<float*>(smem + DenseLds::mw);
  float* lw = reinterpret_cast<float*>(smem + DenseLds::lw);
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + DenseLds::qs);
  int* pre = reinterpret_cast<int*>(smem + DenseLds::pre);
  int* cnt = reinterpret_cast<int*>(smem + DenseLds::cnt(c.B));
  int* ustat = reinterpret_cast<int*>(smem + DenseLds::ustat);
  int* qe = reinterpret_cast<int*>(smem + DenseLds::qe);

  // ---- units per sequence and their prefix sum (every workgroup; workgroup 0 publishes it) ----
  {
    const int per = (B + 255) / 256;
    int* scan = reinterpret_cast<int*>(red);
    int umin = INT_MAX, umax = 0, useq = 0;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) {
      const int un = seq_units(c, p.max_tokens, i, WW);
      cnt[2 * i] = c.n_quant[i];
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
  if (gridDim.x == 1) {  // no combine runs after a one-workgroup launch: empty sequences here
    for (int bb = 0; bb < B; bb++) {
      if (pre[bb + 1] != pre[bb]) continue;
      float* o = p.out + static_cast<size_t>(bb) * nqt * p.Hq * D;
      for (int i = tid; i < nqt * p.Hq * D; i += 256) o[i] = 0.0f;
    }
  }
  const long long NBl = nbe;
  const int u0 = static_cast<int>(floor_div(static_cast<long long>(blockIdx.x) * U, NBl));
  const int u1 = static_cast<int>(floor_div(static_cast<long long>(blockIdx.x + 1) * U, NBl));
  if (u0 == u1) {
    float* part = p.ws_part + static_cast<size_t>(blockIdx.x) * 2 * qpw * G * PART_STRIDE;
    for (int i = tid; i < qpw * G * PART_STRIDE; i += 256) part[i] = (i % PART_STRIDE == 0) ? -FLT_MAX : 0.0f;
    return;
  }

  const int vgroup = c.v.group;
  constexpr float off = ASYM ? 0.0f : static_cast<float>(1 << (KB - 1));
  constexpr long TILE_BYTES = static_cast<long>(TILE) * D * KB / 8;
  constexpr unsigned SP = (4 * KB < 16) ? 4 * KB : 16;  // bytes of a slice piece
  // key slice 4 n + g (token n, channels 32 g ..): the words this wave unpacks for lane group
  // `wave` of QK product g
  const unsigned kw_lane = SP * (4 * n + g) + vword_off<KB>(wave);
  // value chunk 16 g + n (tokens 4 g .., channels 8 n ..): the words this wave dequantizes
  const unsigned vw_lane = SP * (16 * g + n) + vword_off<KB>(wave);
  const unsigned vs_lane = ((8 * n) / vgroup) * TILE + 4 * g;  // value scale row of this lane
  const int qi = wave;
  const UnpackRegs ur = unpack_regs<KB>();

  int u = u0;
  bool first_seg = true;
  while (u < u1) {
    // ---- the segment: sequence b, kv head h, query-block group qgrp, first unit kk ----
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
    const int qblk = qgrp * qpw + qi;
    const int seg_abs_end = pb0 + (sidx + 1) * ub;
    const int uend = min(u1, seg_abs_end);
    const bool complete = (kk == 0) && (uend == seg_abs_end);
    const int slot = first_seg ? 0 : 1;
    const int nq = uni(cnt[2 * b]);
    const int nr = uni(cnt[2 * b + 1]);
    const int uq = (nq + 31) / 32;
    const int segw = umin != umax ? SEG_W : 0;
    const int ku = max(kk - segw, 0), xend = max(kk + (uend - u) - segw, 0);
    // causal limit: block qblk's first query token sees the first lim_min cached tokens, row v's
    // token lim_min + v / gkv of them
    const int lim_min = uni(nq + nr - nqt + qblk * qbs + 1);

    // query rows of the four blocks: row v of block bi = query token (qgrp 4 + bi) qbs + v / gkv,
    // head h gkv + v % gkv (zero past the last); four 16-byte pieces per thread
    uint4 qval[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      qval[k] = uint4{0u, 0u, 0u, 0u};
      const int piece = tid + 256 * k;
      const int row = piece / (D / 8), bi = row / G, v = row % G;
      const int qg = (qgrp * qpw + bi) * qbs + v / gkv;
      if (qg < nqt)
        qval[k] = reinterpret_cast<const uint4*>(
            p.q + ((static_cast<size_t>(b) * nqt + qg) * p.Hq + static_cast<size_t>(h) * gkv + v % gkv) *
                      D)[piece % (D / 8)];
    }
    // every wave walks all units: an active wave for its block, and every wave dequantizes its
    // quarter of each unit's values for the others
    const bool active = qblk < nqb;
    int x = ku;
    const int xq_end = min(xend, uq);

    // Tiles are addressed from a base per segment: the sequence's first tile (contiguous) or the
    // pool's (paged), one buffer resource per array, and a tile's byte offset from that base as the
    // load's scalar offset (the host admits only caches whose offsets stay below 2^31).
    const int* trow = c.table ? c.table + static_cast<size_t>(b) * c.max_blocks : nullptr;
    const size_t tile_base = trow ? 0 : static_cast<size_t>(b * H + h) * (c.cap / TILE);
    const rsrc_t rK = buf(c.kc + tile_base * TILE_BYTES);
    const rsrc_t rV = buf(c.vc + tile_base * TILE_BYTES);
    const rsrc_t rS = buf(c.ks + tile_base * c.ks_tile);  // key rows, then value rows, per tile
    const rsrc_t rZ = buf(ASYM ? c.kz + tile_base * c.ks_tile : c.ks);
    const int rec_bytes = 2 * c.ks_tile;
    const unsigned vrow_off = static_cast<unsigned>(c.vs - c.ks) * 2;  // value rows in the record
    // tile index from the base (-1: an unusable table entry)
    auto phys_of = [&](int t) -> int {
      if (!trow) return t;
      const int blk = ld_uniform(trow + t);
      if (blk < 0 || blk >= c.num_blocks) return -1;
      return blk * H + h;
    };
    constexpr int VW = vwords<KB>();
    uint32_t kw[2][VW], vw[2][VW];
    uint2 ks[NGK][2], kz[NGK][2], vsc[2], vz[2];
    auto load_k = [&](int pA, int pB) {
      load_vwords<KB>(rK, kw_lane, max(pA, 0) * static_cast<int>(TILE_BYTES), kw[0]);
      load_vwords<KB>(rK, kw_lane, max(pB, 0) * static_cast<int>(TILE_BYTES), kw[1]);
    };
    auto load_ks = [&](int pA, int pB) {  // key scales (and zero-points): the scores only
      if constexpr (F8 || BF) return;
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int so = max(t ? pB : pA, 0) * rec_bytes;
#pragma unroll
        for (int gi = 0; gi < NGK; gi++) {
          ks[gi][t] = ld_rows(rS, 2 * (gi * TILE + 4 * g), so);
          if constexpr (ASYM) kz[gi][t] = ld_rows(rZ, 2 * (gi * TILE + 4 * g), so);
        }
      }
    };
    auto load_v = [&](int pA, int pB) {
      load_vwords<KB>(rV, vw_lane, max(pA, 0) * static_cast<int>(TILE_BYTES), vw[0]);
      load_vwords<KB>(rV, vw_lane, max(pB, 0) * static_cast<int>(TILE_BYTES), vw[1]);
      if constexpr (F8 || BF) return;  // one scale per head or tensor, or none
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int so = max(t ? pB : pA, 0) * rec_bytes;
        vsc[t] = ld_rows(rS, vrow_off + 2 * vs_lane, so);
        if constexpr (ASYM) vz[t] = ld_rows(rZ, vrow_off + 2 * vs_lane, so);
      }
    };
    // tiles of unit y, and how many of their tokens are valid (0 for a bad block entry)
    auto tiles_of = [&](int y, int& a, int& b) {
      a = phys_of(2 * y);
      b = (32 * y + 16 < nq) ? phys_of(2 * y + 1) : -1;
    };
    auto valid_of = [&](int y, int a, int b, int& va, int& vb) {
      va = a >= 0 ? min(16, nq - 32 * y) : 0;
      vb = b >= 0 ? min(16, nq - 32 * y - 16) : 0;
    };
    int pA = -1, pB = -1, nA = -1, nB = -1;  // tiles of units x and x + 1
    if (x < xq_end) {
      tiles_of(x, pA, pB);
      load_k(pA, pB);
      if (active) load_ks(pA, pB);
      load_v(pA, pB);
      if (x + 1 < xq_end) tiles_of(x + 1, nA, nB);
    }

    // ---- stage the 64 query rows and each row's prescale exponent ----
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int piece = tid + 256 * k;
      float mx = 0.0f;
      const uint32_t w4[4] = {qval[k].x, qval[k].y, qval[k].z, qval[k].w};
#pragma unroll
      for (int i = 0; i < 4; i++)
        mx = max3f(mx, __uint_as_float((w4[i] << 16) & 0x7FFF0000u), __uint_as_float(w4[i] & 0x7FFF0000u));
      mx = fmaxf(mx, row_ror<8>(mx));
      mx = fmaxf(mx, row_ror<4>(mx));
      mx = fmaxf(mx, row_ror<2>(mx));
      mx = fmaxf(mx, row_ror<1>(mx));
      const int row = piece / (D / 8);
      reinterpret_cast<uint4*>(qs + row * D)[piece % (D / 8)] = qval[k];
      if (piece % (D / 8) == 0) qe[row] = q_exponent(mx, QE_RAW);
    }
    __syncthreads();
    // this lane's QK column = row n of the wave's block: its prescale 2^-e and the softmax
    // scale of its scores, sm_scale log2(e) 2^e
    const int qe_n = qe[qi * G + n];
    const float qsc = exp2i(-qe_n);
    // FP8: the key scale of kv head h multiplies every score, the value scale the output
    float f8k = 1.0f, f8v = 1.0f;
    if constexpr (F8) {
      f8k = __int_as_float(ld_uniform(reinterpret_cast<const int32_t*>(c.ks) + (c.k.axis == KVQ_PER_HEAD ? h : 0)));
      f8v = __int_as_float(ld_uniform(reinterpret_cast<const int32_t*>(c.vs) + (c.v.axis == KVQ_PER_HEAD ? h : 0)));
    }
    // (BF16 storage: the bf16 query as it is, no prescale)
    const float sl2 = BF ? p.sm_log2 : p.sm_log2 * exp2i(qe_n) * f8k;
    const uint16_t* qrow = qs + (qi * G + n) * D;

    // ---- QK operands: product j takes key slice j (channels 32 j .. 32 j + 31, one key group),
    // lane group g its pairs 4 g .. 4 g + 3; the row's query over the same channels, prescaled and
    // divided by each field's alpha.  Every tile's accumulator for group gi starts at minus the
    // group's raw-code bias. ----
    f16x8 qn[4];
    f32x4 dq0[NGK];
    float qsum[NGK];  // asymmetric keys: sum of the prescaled query over the group's channels
#pragma unroll
    for (int gi = 0; gi < NGK; gi++) {
      qsum[gi] = 0.0f;
      dq0[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f16x8 bias;
#pragma unroll
    for (int i = 0; i < 8; i++)
      bias[i] = static_cast<_Float16>(-(1024.0f + static_cast<float>(pair_alpha<KB>(i / 2)) * off));
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int gi = j / (4 / NGK);
      // FP8 bytes convert in natural channel order (no fields, no bias); BF16 keys take the bf16
      // query bits as they are
      const u16x8 raw = (F8 || BF) ? *reinterpret_cast<const u16x8*>(qrow + 32 * j + 8 * g) : gather_kchan<KB>(qrow + 32 * j, g);
      if constexpr (BF) {
        qn[j] = __builtin_bit_cast(f16x8, raw);
        continue;
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float xq = bf16_to_f32(raw[i]) * qsc;
        qn[j][i] = static_cast<_Float16>(F8 ? xq : xq * (1.0f / static_cast<float>(pair_alpha<KB>(i / 2))));
        if constexpr (ASYM) qsum[gi] += xq;
      }
      if constexpr (!F8) dq0[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bias, qn[j], dq0[gi], 0, 0, 0);
    }
    if constexpr (ASYM) {
#pragma unroll
      for (int gi = 0; gi < NGK; gi++) {
        qsum[gi] += __shfl_xor(qsum[gi], 16);
        qsum[gi] += __shfl_xor(qsum[gi], 32);
      }
    }

    float m_run = -FLT_MAX, l_run = 0.0f;
    f32x4 acc[8];  // rows 4 g + r (query rows), columns = channels 8 n + j of product j
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- online softmax of the 8 scores of a unit (column n, tokens 4 g + r of tiles A, B) ----
    auto softmax = [&](float (&s2)[8], int nvA, int nvB, int tok0, float sl2_) {
      if (!(nvA == 16 && nvB == 16)) {
#pragma unroll
        for (int i = 0; i < 8; i++)
          if (4 * g + (i & 3) >= (i < 4 ? nvA : nvB)) s2[i] = -INFINITY;
      }
      if (tok0 + 32 > lim_min) {
        const int lim = lim_min + n / gkv;
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
        // accumulator row 4 g + r belongs to column (row) 4 g + r, whose alpha lane 4 g + r holds
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r));
          const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + r));
          const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 8 + r));
          const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 12 + r));
          const float a = (g == 0) ? a0 : (g == 1) ? a1 : (g == 2) ? a2 : a3;
#pragma unroll
          for (int j = 0; j < 8; j++) acc[j][r] *= a;
        }
        m_run = mn;
      }
#pragma unroll
      for (int i = 0; i < 8; i++) s2[i] = __builtin_amdgcn_exp2f(fmaf(s2[i], sl2_, -m_run));
      l_run += (s2[0] + s2[1]) + (s2[2] + s2[3]) + ((s2[4] + s2[5]) + (s2[6] + s2[7]));
    };

    // ---------------------------- compressed units ----------------------------
    // Unit y's value operands go to LDS buffer y & 1, one quarter per wave: products 2 wave and
    // 2 wave + 1.  Element i of product j is raw pair (2 j + (i / 2) % 2) of tile i / 4, field
    // i % 2; its scale is token 4 g + i % 4's of the lane's value group, times 2^-8 / alpha.
    uint4* vbuf = reinterpret_cast<uint4*>(smem + DenseLds::vbuf);
    auto put_values = [&](int y, int nvA, int nvB) {
      if constexpr (BF) {
        // BF16 values as they are: word 2 jj + h of the wave's piece holds tokens 4 g + 2 h and
        // + 1 of channel 8 n + 2 wave + jj, so product 2 wave + jj is words 2 jj, 2 jj + 1 of
        // each tile.  Halves of tokens past the end are cleared (they may hold NaN).
        uint32_t w[2][4];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const int nv = t ? nvB : nvA;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int r0 = 4 * g + 2 * (q % 2);
            const uint32_t keep = (r0 < nv ? 0x0000FFFFu : 0u) | (r0 + 1 < nv ? 0xFFFF0000u : 0u);
            w[t][q] = (nvA == 16 && nvB == 16) ? vw[t][q] : vw[t][q] & keep;
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++)
          vbuf[((y & 1) * 8 + 2 * wave + jj) * 64 + lane] = uint4{w[0][2 * jj], w[0][2 * jj + 1], w[1][2 * jj], w[1][2 * jj + 1]};
        return;
      }
      if constexpr (F8) {
        // E4M3 bytes convert exactly to f16 (the head's scale multiplies the output); byte b of
        // a value word is token 4 g + (0, 2, 1, 3)[b].  Bytes of tokens past the end are
        // cleared (they may hold NaN codes).
        uint32_t keep[2] = {~0u, ~0u};
        if (!(nvA == 16 && nvB == 16)) {
#pragma unroll
          for (int t = 0; t < 2; t++) {
            const int nv = t ? nvB : nvA;
            keep[t] = (4 * g < nv ? 0x000000FFu : 0u) | (4 * g + 2 < nv ? 0x0000FF00u : 0u) |
                      (4 * g + 1 < nv ? 0x00FF0000u : 0u) | (4 * g + 3 < nv ? 0xFF000000u : 0u);
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++)
          vbuf[((y & 1) * 8 + 2 * wave + jj) * 64 + lane] =
              __builtin_bit_cast(uint4, f8_to_f16x8(vw[0][jj] & keep[0], vw[1][jj] & keep[1]));
        return;
      }
      uint32_t svb[4] = {vsc[0].x, vsc[0].y, vsc[1].x, vsc[1].y};
      uint32_t zvb[4] = {vz[0].x, vz[0].y, vz[1].x, vz[1].y};
      // a tile past the sequence end may hold any bytes (0 * NaN is NaN): clear the fp16 bits
      // of the scales and zero-points of tokens past the end.  (By validity, not by weight: a
      // value operand serves every query row, and a token one row's causal limit hides is seen
      // by the next.)
      if (!(nvA == 16 && nvB == 16)) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int nv = (q < 2) ? nvA : nvB, t0 = 4 * g + 2 * (q % 2);
          const uint32_t keep = (t0 < nv ? 0x0000FFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
          svb[q] &= keep;
          if constexpr (ASYM) zvb[q] &= keep;
        }
      }
      uint32_t vu[2][VW];
      vwords_at_use<KB>(vw[0], wave, vu[0]);
      vwords_at_use<KB>(vw[1], wave, vu[1]);
      f16x2 sv[4], zv2[4];
      const f16x2 k8 = h2s(0x1p-8f);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        sv[q] = as_h2(svb[q]) * k8;
        if constexpr (ASYM) zv2[q] = as_h2(zvb[q]) * k8;
      }
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        uint32_t vbw[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          // q = 2 t + (pair parity): tile t, the wave's pair 2 jj + q % 2
          const int t = q / 2, pr = 2 * jj + (q % 2);
          const f16x2 raw = as_h2(rawpair<KB>(vu[t], pr, ur));
          const float a0 = static_cast<float>(pair_alpha<KB>(pr));
          const f16x2 inva = h2s(1.0f / a0);
          f16x2 v2;
          if constexpr (ASYM) {
            const f16x2 tt = raw - h2s(1024.0f);                    // alpha u, exact
            v2 = __builtin_elementwise_fma(tt, sv[q] * inva, zv2[q]);  // (s u + z) 2^-8
          } else {
            const f16x2 tt = raw - h2s(1024.0f + a0 * off);         // alpha (u - off), exact
            v2 = tt * (sv[q] * inva);                                // s (u - off) 2^-8
          }
          vbw[q] = __builtin_bit_cast(uint32_t, v2);
        }
        vbuf[((y & 1) * 8 + 2 * wave + jj) * 64 + lane] = uint4{vbw[0], vbw[1], vbw[2], vbw[3]};
      }
    };
    // unit y's raw key codes to LDS buffer y & 1: this wave's part (lane group `wave`) of key slice
    // 4 n + g of each tile, as QK product g's operand for token n
    uint4* kbuf = reinterpret_cast<uint4*>(smem + DenseLds::kbuf);
    auto put_keys = [&](int y) {
#pragma unroll
      for (int t = 0; t < 2; t++) {
        uint32_t ku[VW];
        vwords_at_use<KB>(kw[t], wave, ku);
        uint4 op;
        if constexpr (BF) op = uint4{ku[0], ku[VW > 1 ? 1 : 0], ku[VW > 2 ? 2 : 0], ku[VW > 3 ? 3 : 0]};
        else if constexpr (F8) op = __builtin_bit_cast(uint4, f8_to_f16x8(ku[0], ku[VW - 1]));
        else op = __builtin_bit_cast(uint4, kop_raw<KB>(ku, 0, ur));
        kbuf[(((y & 1) * 2 + t) * 4 + g) * 64 + 16 * wave + n] = op;
      }
    };
    if (x < xq_end) {
      bool bad_block = false;
      for (; x < xq_end; x++) {
        int nvA, nvB;
        valid_of(x, pA, pB, nvA, nvB);
        bad_block |= pA < 0 || (32 * x + 16 < nq && pB < 0);
        // wave priorities per phase: a wave past the barrier (QK, softmax) issues before one in
        // its PV products, and both before one unpacking (16 queries: INT4 355-360 -> 338-339 us,
        // INT8 345-348 -> 332-333 us against no priorities; the opposite order was slower)
        __builtin_amdgcn_s_setprio(0);
        put_keys(x);
        put_values(x, nvA, nvB);
        int nnA = -1, nnB = -1;  // tiles of unit x + 2
        if (x + 2 < xq_end) tiles_of(x + 2, nnA, nnB);
        // code registers are free again: the next unit's codes (past the last unit a stand-in
        // tile, so every path issues the same loads and no register copies join them: 16 INT4
        // queries 356-360 -> 340-346 us, INT8 343-346 -> 328-336 us)
        load_k(nA, nB);
        load_v(nA, nB);
        // every wave's quarter of unit x is in LDS (and every wave is done reading unit x - 1's)
        __syncthreads();
        __builtin_amdgcn_s_setprio(2);

        f16x8 pa;
        bf16x8 ph, pl;  // BF16 storage: the weights' bf16 hi and lo parts (16 significant bits)
        if (active) {
          // QK^T: one accumulator per (tile, key group); stand-in tiles are masked by the softmax
          uint4 kop[2][4];
#pragma unroll
          for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) kop[t][j] = kbuf[(((x & 1) * 2 + t) * 4 + j) * 64 + lane];
          f32x4 dq[2][NGK];
#pragma unroll
          for (int t = 0; t < 2; t++)
#pragma unroll
            for (int gi = 0; gi < NGK; gi++) dq[t][gi] = dq0[gi];
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int t = 0; t < 2; t++) {
              const int gi = j / (4 / NGK);
              if constexpr (BF)
                dq[t][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[t][j]),
                                                                    __builtin_bit_cast(bf16x8, qn[j]), dq[t][gi], 0, 0, 0);
              else
                dq[t][gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kop[t][j]), qn[j], dq[t][gi], 0, 0, 0);
            }
          float s2[8];
#pragma unroll
          for (int t = 0; t < 2; t++) {
#pragma unroll
            for (int r = 0; r < 4; r++) s2[4 * t + r] = 0.0f;
            if constexpr (F8 || BF) {  // FP8: the head's key scale is in sl2
#pragma unroll
              for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[t][0][r];
              continue;
            }
#pragma unroll
            for (int gi = 0; gi < NGK; gi++) {
              const uint2 k2 = ks[gi][t];
              const float sc[4] = {f16_lo(k2.x), f16_hi(k2.x), f16_lo(k2.y), f16_hi(k2.y)};
#pragma unroll
              for (int r = 0; r < 4; r++) s2[4 * t + r] = fmaf(dq[t][gi][r], sc[r], s2[4 * t + r]);
              if constexpr (ASYM) {
                const uint2 z2 = kz[gi][t];
                const float zk[4] = {f16_lo(z2.x), f16_hi(z2.x), f16_lo(z2.y), f16_hi(z2.y)};
#pragma unroll
                for (int r = 0; r < 4; r++) s2[4 * t + r] = fmaf(zk[r], qsum[gi], s2[4 * t + r]);
              }
            }
          }
          load_ks(nA, nB);  // scale registers are free again
          softmax(s2, nvA, nvB, 32 * x, sl2);

          // P: the weights as f16, element i: token 4 g + i % 4 of tile i / 4 (FP8: token
          // 4 g + (0, 2, 1, 3)[i % 4], the order of the converted value bytes)
          if constexpr (BF) {
            uint32_t hk[4], lk[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
              uint32_t eh[2], el[2];
#pragma unroll
              for (int k2 = 0; k2 < 2; k2++) {
                const float wv = s2[2 * i + k2];
                const float hv = __uint_as_float(__float_as_uint(wv) & 0xFFFF0000u);
                eh[k2] = __float_as_uint(hv) >> 16;
                el[k2] = __float_as_uint(wv - hv) >> 16;
              }
              hk[i] = eh[0] | (eh[1] << 16);
              lk[i] = el[0] | (el[1] << 16);
            }
            ph = __builtin_bit_cast(bf16x8, uint4{hk[0], hk[1], hk[2], hk[3]});
            pl = __builtin_bit_cast(bf16x8, uint4{lk[0], lk[1], lk[2], lk[3]});
          } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int a = F8 ? 4 * (i / 2) + (i % 2) : 2 * i, b = F8 ? a + 2 : a + 1;
              const f16x2 w2 = pkrtz(s2[a], s2[b]);
              pa[2 * i] = w2[0];
              pa[2 * i + 1] = w2[1];
            }
          }
        }
        __builtin_amdgcn_s_setprio(1);
        if (active) {
          uint4 vop[8];
#pragma unroll
          for (int j = 0; j < 8; j++) vop[j] = vbuf[((x & 1) * 8 + j) * 64 + lane];
#pragma unroll
          for (int j = 0; j < 8; j++) {
            if constexpr (BF) {
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, __builtin_bit_cast(bf16x8, vop[j]), acc[j], 0, 0, 0);
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, __builtin_bit_cast(bf16x8, vop[j]), acc[j], 0, 0, 0);
            } else {
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(f16x8, vop[j]), acc[j], 0, 0, 0);
            }
          }
        }
        pA = nA;
        pB = nB;
        nA = nnA;
        nB = nnB;
      }
      if (bad_block && lane == 0) atomicOr(c.err, KVQ_ERR_BLOCK);
    }
    // the compressed units' values were taken times 2^-8 (FP8: without the head's value scale)
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) acc[j][r] *= F8 ? f8v : BF ? 1.0f : 256.0f;

    // ---------------------------- BF16 window units ----------------------------
    const int wend = xend > uq ? (xend - uq + WW - 1) / WW : 0;
    int jw = (qblk < nqb) ? (max(ku, uq) - uq + WW - 1) / WW : wend;
    if (jw < wend) {
      bf16x8 qw[4];
#pragma unroll
      for (int j = 0; j < 4; j++)
        qw[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qrow + 32 * g + 8 * j));
      const uint16_t* kr = c.kres + (static_cast<size_t>(b) * H + h) * c.R * D;
      const uint16_t* vr = c.vres + (static_cast<size_t>(b) * H + h) * c.R * D;
      for (; jw < wend; jw++) {
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
              dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rowp[j]), qw[j], dq, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; r++) s2[4 * t + r] = dq[r];
        }
        softmax(s2, nvA, nvB, nq + r0, p.sm_log2);
        // P: bf16 hi and lo parts of the weights (hi + lo carries 16 significant bits)
        bf16x8 ph, pl;
        {
          uint32_t hk[4], lk[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            uint32_t eh[2], el[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++) {
              const float wv = s2[2 * i + k2];
              const float hv = __uint_as_float(__float_as_uint(wv) & 0xFFFF0000u);
              eh[k2] = __float_as_uint(hv) >> 16;
              el[k2] = __float_as_uint(wv - hv) >> 16;
            }
            hk[i] = eh[0] | (eh[1] << 16);
            lk[i] = el[0] | (el[1] << 16);
          }
          ph = __builtin_bit_cast(bf16x8, uint4{hk[0], hk[1], hk[2], hk[3]});
          pl = __builtin_bit_cast(bf16x8, uint4{lk[0], lk[1], lk[2], lk[3]});
        }
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
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, __builtin_bit_cast(bf16x8, col), acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, __builtin_bit_cast(bf16x8, col), acc[j], 0, 0, 0);
          }
        }
      }
    }

    // ---------------------------- the wave's block: output or partial ----------------------------
    float lsum = l_run + __shfl_xor(l_run, 16);
    lsum += __shfl_xor(lsum, 32);
    __syncthreads();  // every wave is done with the previous segment's rows of red
    if (lane < G) {
      mw[wave * G + lane] = m_run;
      lw[wave * G + lane] = lsum;
    }
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) red[(wave * 16 + 4 * g + r) * RED_STRIDE + 8 * n + j] = acc[j][r];
    wave_lds_sync();
    if (qblk < nqb) {
#pragma unroll 4
      for (int oi = 0; oi < (G * D) / 64; oi++) {
        const int o = lane + 64 * oi;
        const int oh = o / D, ch = o % D;
        const float O = red[(wave * 16 + oh) * RED_STRIDE + ch];
        const float L = lw[wave * G + oh];
        if (complete) {
          const int qg = qblk * qbs + oh / gkv;
          if (qg < nqt)
            p.out[((static_cast<size_t>(b) * nqt + qg) * p.Hq + static_cast<size_t>(h) * gkv + oh % gkv) * D + ch] =
                (L > 0.0f) ? O / L : 0.0f;
        } else {
          float* part = p.ws_part + (((static_cast<size_t>(blockIdx.x) * 2 + slot) * qpw + qi) * G + oh) * PART_STRIDE;
          if (ch == 0) {
            part[0] = mw[wave * G + oh];
            part[1] = L;
          }
          part[4 + ch] = O;
        }
      }
    } else if (!complete) {
      // a block past the last one still owns its partial rows: neutral
#pragma unroll 4
      for (int oi = 0; oi < (G * D) / 64; oi++) {
        const int o = lane + 64 * oi;
        const int oh = o / D, ch = o % D;
        float* part = p.ws_part + (((static_cast<size_t>(blockIdx.x) * 2 + slot) * qpw + qi) * G + oh) * PART_STRIDE;
        if (ch == 0) {
          part[0] = -FLT_MAX;
          part[1] = 0.0f;
        }
        part[4 + ch] = 0.0f;
      }
    }
    u = uend;
    first_seg = false;
  }
}

// Launch of the dense multi-query kernel and of the combine that merges its partials.
template <int KB, int SCH, int NGK>
hipError_t launch_dense_t(const DecodeParams& p0, hipStream_t s) {
  DecodeParams p = p0;
  const size_t lds = DenseLds::bytes(p.c.B);
  static std::mutex mu;
  static int cached_dev = -1, cached_blocks = 0;
  static size_t cached_lds = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  int resident = 0;
  {
    std::lock_guard<std::mutex> gd(mu);
    if (dev == cached_dev && lds == cached_lds) resident = cached_blocks;
  }
  if (resident == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dense_kernel<KB, SCH, NGK>, 256, lds) != hipSuccess)
      return hipErrorInvalidConfiguration;
    resident = cus * per_cu;
    std::lock_guard<std::mutex> gd(mu);
    cached_dev = dev;
    cached_lds = lds;
    cached_blocks = resident;
  }
  if (resident <= 0) return hipErrorInvalidConfiguration;
  if (p.nblocks > resident) p.nblocks = resident;
  dense_kernel<KB, SCH, NGK><<<p.nblocks, 256, lds, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nblocks == 1) return hipSuccess;
  const int avg = p.nblocks / (p.c.B * p.c.H * p.nqs);
  int slices = 1;
  while (slices < 16 && slices * 2 <= avg / 4 && (DROWS * D) / (slices * 2) >= 32) slices *= 2;
  const dim3 grid(p.c.B * p.c.H * p.nqb, slices);
  switch (avg < 8 ? 0 : slices) {
    case 0: combine_kernel<DROWS, 1, 256><<<grid, 256, 0, s>>>(p); break;
    case 1: combine_kernel<DROWS, 1, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 2: combine_kernel<DROWS, 2, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 4: combine_kernel<DROWS, 4, 1024><<<grid, 1024, 0, s>>>(p); break;
    case 8: combine_kernel<DROWS, 8, 1024><<<grid, 1024, 0, s>>>(p); break;
    default: combine_kernel<DROWS, 16, 1024><<<grid, 1024, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
