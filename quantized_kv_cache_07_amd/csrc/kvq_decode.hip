// kvq_decode.hip -- single-query decode attention over the quantized cache (gfx950).
//
//   out[b][hq] = softmax(sm_scale * q K^T) V          [P2 = llmdaily.org "KV-cache quantization --
//   making long-context inference fit in memory", "Why the KV cache grows so quickly", attention
//   equation], over the compressed tokens (dequantized in registers as they stream in, as P3 =
//   oh-bug.com "KV Cache Quantization in Practice", "Misconception 1", asks of a kernel that is
//   to gain from quantization) followed by the BF16 window rows.
//
// Work split (split-K over the sequence): a work unit is (sequence b, chunk of `chunk` compressed
// slots, kv head h) and is processed by ONE wavefront; the last chunk of a sequence also takes
// the window rows.  Units are numbered sequence by sequence from a prefix sum of per-sequence
// chunk counts that every workgroup rebuilds in LDS from the device counters, so mixed lengths
// need no host sync; waves stride over the units (persistent grid).  Each unit writes a partial
// (running max m, sum l, unnormalised o[GQ][128]); combine_kernel merges a sequence's partials
// with a log-sum-exp rescale.
//
// Per 16-slot tile, per wave (64 lanes; lane = 16 * g + n):
//   QK^T on MFMA 16x16x16 f16:  D[token][col] = sum_k A[token][k] B[k][col], A = key codes
//     (lane (g, n): 32 channels of token n), B = the query rows of the GQA group, one column per
//     (key group, query head) with the other groups' channels zeroed, so per-token group scales
//     apply after the product; per-channel key scales are folded into the query (hi + lo f16
//     parts) once per key group.  8 MFMAs cover 128 channels.
//   PV on MFMA 16x16x16 f16:  D[row][ch] = sum_t P[row][t] V[t][ch], rows = (hi/lo part, value
//     group, query head) of w * s_v, columns 16 channels; the token-interleaved V tile gives each
//     lane exactly the 4 tokens x 8 channels it needs in one 128-bit load.
//   Codes are turned into exact f16 integers with the 0x6400 exponent trick (two codes per
//   and-or, then one packed f16 add/fma removes the bias), so A/B operands are exact and the
//   only roundings are the fp32 accumulations; softmax weights enter PV as hi + lo f16 parts.
#include "kvq_dev.h"

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ h2 splat(float x) { return h2{(_Float16)x, (_Float16)x}; }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3); }

// ---- code unpacking: 16 pairs (field k, field k + E/2) of each word, as exact f16 (u - off) --

template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t* w, h2 (&o)[16], float off) {
  constexpr uint32_t MAGIC = 0x64006400u;  // f16 1024.0 in both halves; low mantissa = code
  if constexpr (BITS == 8) {
    const h2 s1 = splat(1024.0f + off);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      o[2 * i] = as_h2((w[i] & 0x00FF00FFu) | MAGIC) - s1;
      o[2 * i + 1] = as_h2(((w[i] >> 8) & 0x00FF00FFu) | MAGIC) - s1;
    }
  } else if constexpr (BITS == 4) {
    const h2 s1 = splat(1024.0f + off), s16 = splat(64.0f + off), r16 = splat(0.0625f);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t w8 = w[i] >> 8;
      o[4 * i + 0] = as_h2((w[i] & 0x000F000Fu) | MAGIC) - s1;
      o[4 * i + 1] = as_h2((w[i] & 0x00F000F0u) | MAGIC) * r16 - s16;
      o[4 * i + 2] = as_h2((w8 & 0x000F000Fu) | MAGIC) - s1;
      o[4 * i + 3] = as_h2((w8 & 0x00F000F0u) | MAGIC) * r16 - s16;
    }
  } else {
    static_assert(BITS == 2, "bits");
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t w10 = w[i] >> 10;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int sh = (k < 5) ? 2 * k : 2 * (k - 5);
        const uint32_t src = (k < 5) ? w[i] : w10;
        const float scl = 1.0f / static_cast<float>(1 << sh);  // (1024 + 2^sh u) * 2^-sh
        o[8 * i + k] = as_h2((src & (0x00030003u << sh)) | MAGIC) * splat(scl) -
                       splat(1024.0f * scl + off);
      }
    }
  }
}

// Channel (0..31, relative to the lane's 32-channel slice) of slot s (0..3) of MFMA step j for a
// row-major key row: pair P = 2j + s/2 of the slice, word P / (E/2), field (P mod E/2) + (E/2)(s mod 2).
template <int BITS>
__device__ __forceinline__ constexpr int kslot_channel(int j, int s) {
  constexpr int E = 32 / BITS, Hh = E / 2;
  const int P = 2 * j + s / 2;
  return (P / Hh) * E + (P % Hh) + Hh * (s % 2);
}

template <int BITS>
struct Codes {
  uint32_t w[BITS];
};

template <int BITS>
__device__ __forceinline__ Codes<BITS> load_codes(const uint8_t* p) {
  Codes<BITS> c;
  if constexpr (BITS == 8) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = a.z; c.w[3] = a.w;
    c.w[4] = b.x; c.w[5] = b.y; c.w[6] = b.z; c.w[7] = b.w;
  } else if constexpr (BITS == 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = a.z; c.w[3] = a.w;
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    c.w[0] = a.x; c.w[1] = a.y;
  }
  return c;
}

__device__ __forceinline__ void f16x4_to_f32(uint2 u, float (&o)[4]) {
  o[0] = __half2float(__ushort_as_half(static_cast<unsigned short>(u.x & 0xFFFF)));
  o[1] = __half2float(__ushort_as_half(static_cast<unsigned short>(u.x >> 16)));
  o[2] = __half2float(__ushort_as_half(static_cast<unsigned short>(u.y & 0xFFFF)));
  o[3] = __half2float(__ushort_as_half(static_cast<unsigned short>(u.y >> 16)));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Chunks of sequence b (0 when it is empty or exceeds the host bound).
__device__ __forceinline__ int seq_chunks(const DecodeParams& p, int b) {
  const int nq = p.c.n_quant[b];
  const int nr = p.c.R > 0 ? p.c.n_res[b] : 0;
  if (nq < 0 || nr < 0 || nr > p.c.R || (!p.c.table && nq > p.c.cap)) return 0;
  if (nq + nr <= 0 || nq + nr > p.max_tokens) return 0;
  return max(1, (nq + p.chunk - 1) / p.chunk);
}

constexpr int RED_STRIDE = D + 4;  // padded LDS row (floats)

template <int KB, int GQ, int NP, bool KPC>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  extern __shared__ int smem[];
  const CacheDev& c = p.c;
  const int B = c.B, H = c.H;
  int* prefix = smem;                                          // [B + 1]
  float* red_all = reinterpret_cast<float*>(smem + ((B + 1 + 3) & ~3));

  // ---- prefix sum of chunk counts (every workgroup; block 0 also publishes it) ----
  {
    const int tid = threadIdx.x;
    const int per = (B + 255) / 256;
    int s = 0;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) s += seq_chunks(p, i);
    prefix[B] = 0;
    __syncthreads();
    // inclusive scan of the 256 partial sums through the window of prefix[] (B + 1 >= 1 ints
    // are enough only when B >= 256; use red_all as scratch instead)
    float* scr = red_all;
    reinterpret_cast<int*>(scr)[tid] = s;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = (tid >= off) ? reinterpret_cast<int*>(scr)[tid - off] : 0;
      __syncthreads();
      reinterpret_cast<int*>(scr)[tid] += v;
      __syncthreads();
    }
    int run = reinterpret_cast<int*>(scr)[tid] - s;
    for (int i = tid * per; i < min(B, (tid + 1) * per); i++) {
      prefix[i] = run;
      run += seq_chunks(p, i);
      if (blockIdx.x == 0 && seq_chunks(p, i) == 0 &&
          (p.c.n_quant[i] != 0 || (p.c.R > 0 && p.c.n_res[i] != 0)))
        atomicOr(c.err, KVQ_ERR_TOKENS);  // counters out of range or above max_tokens
    }
    if (tid == 255) prefix[B] = reinterpret_cast<int*>(scr)[255];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += 256) p.ws_prefix[i] = prefix[i];
    __syncthreads();
  }
  const int total_items = min(prefix[B], p.items_cap);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  float* red = red_all + wave * 16 * RED_STRIDE;

  const SideDev K = c.k, V = c.v;
  const int ngk = KPC ? 1 : D / K.group;
  const int ngv = D / V.group;
  const int np_rt = (2 * GQ * ngv + 15) / 16;
  const bool k_asym = K.scheme == KVQ_ASYM, v_asym = V.scheme == KVQ_ASYM;
  const float k_off = k_asym ? 0.0f : static_cast<float>(1 << (KB - 1));
  const float v_off = v_asym ? 0.0f : static_cast<float>(1 << (KB - 1));
  // lane roles
  const int hq_n = n % GQ;                        // query head of QK column n / PV row n
  const int gk_n = KPC ? 0 : (n / GQ) % ngk;      // key group of QK column n
  const int kpart_n = KPC ? ((n / GQ) & 1) : 0;   // hi/lo part of QK column n (per-channel keys)
  const int RBK = D * KB / 8;                     // key row bytes
  const long TILE_BYTES = static_cast<long>(TILE) * RBK;

  const long n_units = static_cast<long>(total_items) * H;
  for (long u = static_cast<long>(blockIdx.x) * 4 + wave; u < n_units;
       u += static_cast<long>(gridDim.x) * 4) {
    const int item = static_cast<int>(u / H), h = static_cast<int>(u % H);
    // sequence of this item: largest b with prefix[b] <= item
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int cidx = item - prefix[b];
    const int nchunks = prefix[b + 1] - prefix[b];
    const int nq = c.n_quant[b];
    const int nr = c.R > 0 ? c.n_res[b] : 0;
    const bool last = cidx == nchunks - 1;
    const int t0 = cidx * p.chunk;
    const int t1 = min(nq, t0 + p.chunk);
    const int ntiles = t1 > t0 ? (t1 - t0 + TILE - 1) / TILE : 0;
    const uint16_t* qrow = p.q + (static_cast<size_t>(b) * p.Hq + static_cast<size_t>(h) * GQ) * D;

    // ---- query operand ----
    h4 bq[8];
    float qf[32];       // per-channel keys: q of the lane's head in slot order
    float qsum = 0.0f;  // asymmetric per-token keys: sum of q over the column's key group
#pragma unroll
    for (int j = 0; j < 8; j++) {
      h2 lo2, hi2;
      float v[4];
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const int ch = 32 * g + kslot_channel<KB>(j, s);
        const float x = bf16_to_f32(qrow[hq_n * D + ch]);
        const bool in_group = KPC || (ch / K.group) == gk_n;
        v[s] = in_group ? x : 0.0f;
        if (KPC) qf[4 * j + s] = x;
        qsum += v[s];
      }
      lo2 = h2{(_Float16)v[0], (_Float16)v[1]};
      hi2 = h2{(_Float16)v[2], (_Float16)v[3]};
      bq[j] = cat(lo2, hi2);
    }
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);

    float m_run = -INFINITY, l_run = 0.0f;
    f4 acc[NP][8];
#pragma unroll
    for (int pp = 0; pp < NP; pp++)
#pragma unroll
      for (int j = 0; j < 8; j++) acc[pp][j] = f4{0.f, 0.f, 0.f, 0.f};
    float zacc[NP];
#pragma unroll
    for (int pp = 0; pp < NP; pp++) zacc[pp] = 0.0f;
    float zt = 0.0f;  // per-channel keys: sum_i q_i z_i of the current key group

    // block-table slice of this chunk (one entry per lane; chunk <= 1024 slots = 64 tiles)
    int tbl = 0;
    if (c.table && lane < ntiles) {
      const int tt = t0 / TILE + lane;
      tbl = (tt < c.max_blocks) ? c.table[static_cast<size_t>(b) * c.max_blocks + tt] : -1;
    }
    const long contig_base = (static_cast<long>(b) * H + h) * (c.cap / TILE) + t0 / TILE;

    for (int it = 0; it < ntiles; it++) {
      const int tslot = t0 + it * TILE;
      long phys;
      if (c.table) {
        const int blk = __builtin_amdgcn_readlane(tbl, it);
        if (blk < 0 || blk >= c.num_blocks) {
          if (lane == 0) atomicOr(c.err, KVQ_ERR_BLOCK);
          continue;
        }
        phys = static_cast<long>(blk) * H + h;
      } else {
        phys = contig_base + it;
      }
      // per-channel keys: refresh the folded query at each key group boundary
      if constexpr (KPC) {
        if ((tslot % K.group) == 0 || it == 0) {
          const int tau = tslot / K.group;
          const uint16_t* sp =
              c.ks + ((static_cast<size_t>(b) * H + h) * (c.cap / K.group) + tau) * D + 32 * g;
          const uint16_t* zp =
              k_asym ? c.kz + ((static_cast<size_t>(b) * H + h) * (c.cap / K.group) + tau) * D + 32 * g
                     : nullptr;
          uint16_t sv[32], zv[32];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint4 a = reinterpret_cast<const uint4*>(sp)[i];
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
              sv[8 * i + 2 * e] = aw[e] & 0xFFFF;
              sv[8 * i + 2 * e + 1] = aw[e] >> 16;
            }
            if (k_asym) {
              const uint4 z = reinterpret_cast<const uint4*>(zp)[i];
              const uint32_t zw[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
              for (int e = 0; e < 4; e++) {
                zv[8 * i + 2 * e] = zw[e] & 0xFFFF;
                zv[8 * i + 2 * e + 1] = zw[e] >> 16;
              }
            }
          }
          float zpart = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; j++) {
            float hv[4];
#pragma unroll
            for (int s = 0; s < 4; s++) {
              const int ch = kslot_channel<KB>(j, s);
              const float qs = qf[4 * j + s] * __half2float(__ushort_as_half(sv[ch]));
              const float hi_part = static_cast<float>(static_cast<_Float16>(qs));
              hv[s] = kpart_n ? (qs - hi_part) : qs;
              if (k_asym) zpart += qf[4 * j + s] * __half2float(__ushort_as_half(zv[ch]));
            }
            bq[j] = cat(h2{(_Float16)hv[0], (_Float16)hv[1]}, h2{(_Float16)hv[2], (_Float16)hv[3]});
          }
          zpart += __shfl_xor(zpart, 16);
          zpart += __shfl_xor(zpart, 32);
          zt = zpart;
        }
      }

      // ---- loads ----
      const Codes<KB> kc = load_codes<KB>(c.kc + phys * TILE_BYTES + n * RBK + g * (RBK / 4));
      const Codes<KB> vc =
          load_codes<KB>(c.vc + phys * TILE_BYTES + (g * (D / 8) + n) * (4 * KB));
      uint2 ksc = {0, 0}, kzc = {0, 0};
      if constexpr (!KPC) {
        const size_t mi = (static_cast<size_t>(phys) * ngk + gk_n) * TILE + 4 * g;
        ksc = *reinterpret_cast<const uint2*>(c.ks + mi);
        if (k_asym) kzc = *reinterpret_cast<const uint2*>(c.kz + mi);
      }

      // ---- QK^T ----
      h2 kp[16];
      unpack16<KB>(kc.w, kp, k_off);
      f4 dk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; j++)
        dk = __builtin_amdgcn_mfma_f32_16x16x16f16(cat(kp[2 * j], kp[2 * j + 1]), bq[j], dk, 0, 0, 0);

      float sc[4];
      if constexpr (KPC) {
#pragma unroll
        for (int r = 0; r < 4; r++) sc[r] = dk[r] + __shfl_xor(dk[r], GQ) + zt;
      } else {
        float ks4[4], kz4[4];
        f16x4_to_f32(ksc, ks4);
        if (k_asym) f16x4_to_f32(kzc, kz4);
#pragma unroll
        for (int r = 0; r < 4; r++) sc[r] = dk[r] * ks4[r] + (k_asym ? kz4[r] * qsum : 0.0f);
        for (int st = GQ; st < ngk * GQ; st <<= 1)
#pragma unroll
          for (int r = 0; r < 4; r++) sc[r] += __shfl_xor(sc[r], st);
      }
      bool tv[4];
      float s2[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        tv[r] = tslot + 4 * g + r < t1;
        s2[r] = tv[r] ? sc[r] * p.sm_log2 : -INFINITY;
      }

      // ---- online softmax (per lane: head hq_n) ----
      float tmax = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      if (__ballot(m_new > m_run) != 0) {
        const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        float al[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; hh++)
          al[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hh));
#pragma unroll
        for (int pp = 0; pp < NP; pp++) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            float a;
            if constexpr (GQ <= 4) a = al[r % GQ];
            else a = (g & 1) ? al[(4 + r) % GQ] : al[r % GQ];
#pragma unroll
            for (int j = 0; j < 8; j++) acc[pp][j][r] *= a;
          }
          zacc[pp] *= alpha;
        }
        l_run *= alpha;
        m_run = m_new;
      }
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; r++) w[r] = tv[r] ? __builtin_amdgcn_exp2f(s2[r] - m_run) : 0.0f;
      l_run += (w[0] + w[1]) + (w[2] + w[3]);

      // ---- PV ----
      h2 vp[16];
      unpack16<KB>(vc.w, vp, v_off);
#pragma unroll
      for (int pp = 0; pp < NP; pp++) {
        if (pp >= np_rt) break;
        const int mrow = 16 * pp + n;
        const int gv = (mrow / GQ) % ngv;
        const int part = (mrow / (GQ * ngv)) & 1;
        const bool row_ok = mrow < 2 * GQ * ngv;
        const size_t mi = (static_cast<size_t>(phys) * ngv + gv) * TILE + 4 * g;
        float vs4[4], vz4[4];
        f16x4_to_f32(*reinterpret_cast<const uint2*>(c.vs + mi), vs4);
        if (v_asym) f16x4_to_f32(*reinterpret_cast<const uint2*>(c.vz + mi), vz4);
        float a[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float ws = tv[r] ? w[r] * vs4[r] : 0.0f;
          const float hi_part = static_cast<float>(static_cast<_Float16>(ws));
          a[r] = row_ok ? (part ? ws - hi_part : ws) : 0.0f;
          if (v_asym && part == 0 && row_ok && tv[r]) zacc[pp] += w[r] * vz4[r];
        }
        const h4 ap = cat(h2{(_Float16)a[0], (_Float16)a[1]}, h2{(_Float16)a[2], (_Float16)a[3]});
#pragma unroll
        for (int j = 0; j < 8; j++)
          acc[pp][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap, cat(vp[2 * j], vp[2 * j + 1]),
                                                             acc[pp][j], 0, 0, 0);
      }
    }

    // ---- fold the MFMA accumulators into o[head][ch], ch = lane and lane + 64 ----
    float lsum = l_run + __shfl_xor(l_run, 16);
    lsum += __shfl_xor(lsum, 32);
    float o[GQ][2];
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) o[hh][0] = o[hh][1] = 0.0f;
#pragma unroll
    for (int pp = 0; pp < NP; pp++) {
      if (pp >= np_rt) break;
      float zs = zacc[pp] + __shfl_xor(zacc[pp], 16);
      zs += __shfl_xor(zs, 32);  // lane n now holds sum over tokens of w * z for row 16 pp + n
#pragma unroll
      for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) red[(4 * g + r) * RED_STRIDE + 8 * n + j] = acc[pp][j][r];
      wave_lds_sync();
#pragma unroll
      for (int ci = 0; ci < 2; ci++) {
        const int ch = lane + 64 * ci;
        const int gv = ch / V.group;
#pragma unroll
        for (int hh = 0; hh < GQ; hh++)
#pragma unroll
          for (int part = 0; part < 2; part++) {
            const int mrow = (part * ngv + gv) * GQ + hh;
            const float zz = v_asym ? __shfl(zs, mrow % 16) : 0.0f;  // all lanes take part
            if (mrow / 16 == pp) {
              o[hh][ci] += red[(mrow % 16) * RED_STRIDE + ch];
              if (part == 0) o[hh][ci] += zz;
            }
          }
      }
      wave_lds_sync();
    }
    float mh[GQ], lh[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) {
      mh[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), hh));
      lh[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), hh));
    }

    // ---- BF16 window rows (last chunk of the sequence) ----
    if (last && nr > 0) {
      float qv[GQ][2];
#pragma unroll
      for (int hh = 0; hh < GQ; hh++) {
        qv[hh][0] = bf16_to_f32(qrow[hh * D + lane]);
        qv[hh][1] = bf16_to_f32(qrow[hh * D + lane + 64]);
      }
      const uint16_t* kr = c.kres + (static_cast<size_t>(b) * H + h) * c.R * D;
      const uint16_t* vr = c.vres + (static_cast<size_t>(b) * H + h) * c.R * D;
      for (int t = 0; t < nr; t++) {
        const float k0 = bf16_to_f32(kr[t * D + lane]), k1 = bf16_to_f32(kr[t * D + lane + 64]);
        const float v0 = bf16_to_f32(vr[t * D + lane]), v1 = bf16_to_f32(vr[t * D + lane + 64]);
#pragma unroll
        for (int hh = 0; hh < GQ; hh++) {
          const float s = wave_sum(qv[hh][0] * k0 + qv[hh][1] * k1) * p.sm_log2;
          const float mn = fmaxf(mh[hh], s);
          const float alpha = __builtin_amdgcn_exp2f(mh[hh] - mn);
          const float wt = __builtin_amdgcn_exp2f(s - mn);
          lh[hh] = lh[hh] * alpha + wt;
          o[hh][0] = o[hh][0] * alpha + wt * v0;
          o[hh][1] = o[hh][1] * alpha + wt * v1;
          mh[hh] = mn;
        }
      }
    }

    // ---- partial ----
    if (item < p.items_cap) {
      const size_t base = (static_cast<size_t>(item) * H + h) * GQ;
#pragma unroll
      for (int hh = 0; hh < GQ; hh++) {
        if (lane == 0) {
          p.ws_ml[(base + hh) * 2] = mh[hh];
          p.ws_ml[(base + hh) * 2 + 1] = lh[hh];
        }
        p.ws_acc[(base + hh) * D + lane] = o[hh][0];
        p.ws_acc[(base + hh) * D + lane + 64] = o[hh][1];
      }
    }
  }
}

// Merge the partials of each (sequence, query head) with a log-sum-exp rescale.
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p, int GQ) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int p0 = p.ws_prefix[b], p1 = p.ws_prefix[b + 1];
  const int H = p.c.H;
  for (int idx = threadIdx.x; idx < GQ * D; idx += blockDim.x) {
    const int hh = idx / D, ch = idx % D;
    float* dst = p.out + (static_cast<size_t>(b) * p.Hq + static_cast<size_t>(h) * GQ + hh) * D + ch;
    if (p1 <= p0 || p1 > p.items_cap) {
      *dst = 0.0f;
      continue;
    }
    float M = -INFINITY;
    for (int it = p0; it < p1; it++)
      M = fmaxf(M, p.ws_ml[((static_cast<size_t>(it) * H + h) * GQ + hh) * 2]);
    float L = 0.0f, O = 0.0f;
    for (int it = p0; it < p1; it++) {
      const size_t base = (static_cast<size_t>(it) * H + h) * GQ + hh;
      const float m = p.ws_ml[base * 2];
      const float e = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      L += e * p.ws_ml[base * 2 + 1];
      O += e * p.ws_acc[base * D + ch];
    }
    *dst = (L > 0.0f) ? O / L : 0.0f;
  }
}

size_t decode_lds_bytes(int B) {
  return static_cast<size_t>((B + 1 + 3) & ~3) * 4 + 4 * 16 * RED_STRIDE * sizeof(float);
}

template <int KB, int GQ, int NP, bool KPC>
static hipError_t launch_t(const DecodeParams& p, int grid, hipStream_t s) {
  const size_t lds = decode_lds_bytes(p.c.B);
  decode_kernel<KB, GQ, NP, KPC><<<grid, 256, lds, s>>>(p);
  return hipGetLastError();
}

template <int KB>
static hipError_t launch_bits(const DecodeParams& p, int GQ, int NP, bool kpc, int grid,
                              hipStream_t s) {
#define KVQ_CASE(G, N)                                                     \
  if (GQ == G && NP == N)                                                  \
    return kpc ? launch_t<KB, G, N, true>(p, grid, s) : launch_t<KB, G, N, false>(p, grid, s);
  KVQ_CASE(1, 1)
  KVQ_CASE(2, 1)
  KVQ_CASE(4, 1)
  KVQ_CASE(4, 2)
  KVQ_CASE(8, 1)
  KVQ_CASE(8, 2)
  KVQ_CASE(8, 4)
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int bits, int GQ, int NP, bool kpc, int grid,
                         hipStream_t s) {
  hipError_t e;
  switch (bits) {
    case 8: e = launch_bits<8>(p, GQ, NP, kpc, grid, s); break;
    case 4: e = launch_bits<4>(p, GQ, NP, kpc, grid, s); break;
    case 2: e = launch_bits<2>(p, GQ, NP, kpc, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  combine_kernel<<<dim3(p.c.B, p.c.H), 256, 0, s>>>(p, GQ);
  return hipGetLastError();
}

}  // namespace kvq
