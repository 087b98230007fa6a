// kvq_dev.h -- device-side definitions shared by the HIP sources of libkvq (gfx950).
//
// The storage layout and the quantizer rules are the ones documented in include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int D = 128;    // head dimension
constexpr int TILE = 16;  // compressed slots per tile (and tokens per paged block)

struct SideDev {
  int bits, scheme, axis, group;
};

// A cache descriptor as the kernels see it (passed by value).
struct CacheDev {
  SideDev k, v;
  int R, B, H, cap, num_blocks, max_blocks;
  const int32_t* table;  // nullptr: contiguous
  uint8_t* kc;
  uint8_t* vc;
  uint16_t* ks;
  uint16_t* vs;
  uint16_t* kz;
  uint16_t* vz;
  uint16_t* kres;
  uint16_t* vres;
  int32_t* n_quant;
  int32_t* n_res;
  int32_t* err;
  // Per-token scale (and zero) rows: fp16 elements from one tile's rows to the next.  When both
  // sides use per-token groups they share one record per tile in the key buffers (key rows,
  // then value rows) and vs / vz point at the value rows of tile 0.
  int ks_tile, vs_tile;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Tile index of compressed slot `slot` of (b, h); ok=false when a paged entry is unusable.
__device__ __forceinline__ long tile_index(const CacheDev& c, int b, int h, int tile, bool& ok) {
  if (c.table) {
    if (tile >= c.max_blocks) {
      ok = false;
      return 0;
    }
    int blk = c.table[static_cast<size_t>(b) * c.max_blocks + tile];
    if (blk < 0 || blk >= c.num_blocks) {
      ok = false;
      return 0;
    }
    return static_cast<long>(blk) * c.H + h;
  }
  return (static_cast<long>(b) * c.H + h) * (c.cap / TILE) + tile;
}

// Decode-attention launch parameters.
struct DecodeParams {
  CacheDev c;
  const uint16_t* q;  // [B][nqt][Hq][D] bf16
  float* out;         // [B][nqt][Hq][D] fp32
  int32_t* ws_pre;    // [B + 1] prefix over sequences of work units (all kv heads), then
                      // the number of unit ranges in use
  float* ws_part;     // [nblocks][2][qpw][G][PART_STRIDE] partial (max, sum, pad, pad, o[D])
  int Hq, max_tokens, nblocks;
  float sm_log2;      // sm_scale * log2(e)
  // Queries per sequence: nqt query tokens, the last nqt cached tokens (1: single-query decode).
  // A query block has G rows, qbs query tokens x gkv query heads (G = qbs * gkv); there are
  // nqb = ceil(nqt / qbs) blocks per (sequence, kv head).  A segment is one (sequence, kv head,
  // group of qpw blocks): with qpw = 4 each wave of a workgroup takes one block and all waves
  // walk the same units (the codes are fetched once for four blocks), with qpw = 2 two waves
  // share each of two blocks, with qpw = 1 the four waves interleave the units of one block.
  // nqs = ceil(nqb / qpw) segments per (sequence, kv head).
  int nqt, qbs, nqb, gkv, qpw, nqs;
};

constexpr int PART_STRIDE = D + 4;

// Work weight of a BF16 window unit (32 rows of bf16 keys and values, 16 KB) against a
// compressed unit of `bits`-bit codes (32 slots of codes plus their scale rows): about the ratio
// of their HBM bytes, so that unit ranges of equal weight carry about equal bytes.
__host__ __device__ constexpr int window_weight(int bits) {
  return bits == 2 ? 5 : bits == 4 ? 4 : bits == 8 ? 2 : 1;
}
// The same for keys of kb bits and values of vb bits (the mean of the two, rounded up).
__host__ __device__ constexpr int window_weight2(int kb, int vb) {
  return (window_weight(kb) + window_weight(vb) + 1) / 2;
}

// Work weight of starting a segment (query staging, first loads), in units, given to every
// segment of a batch of mixed lengths.
constexpr int SEGMENT_START_WEIGHT = 6;

// Slots one append/flush call moves into the compressed cache (F), window tokens before the
// call plus new tokens (total), and window length afterwards.  Equal, by construction, to
// n_new single-token appends each flushing a full window before copying the token in.
enum { MODE_APPEND = 0, MODE_FLUSH = 1 };

// Storage slices: a tile is 64 lane-sized slices of 4 * bits bytes (K: 32 channels of one row,
// slice 4 t + c / 32; V: a chunk of 4 tokens x 8 channels), stored in pieces of
// S = min(16, 4 bits) bytes, piece i of slice s at byte 64 S i + S s (slab i).  A wave reading
// piece i of all slices reads one contiguous 64 S-byte run.  Byte of bit `bit` of slice `s`:
__device__ __forceinline__ long slab_byte(int bits, int s, int bit) {
  const int S = (4 * bits < 16) ? 4 * bits : 16;
  return 64L * S * (bit / (8 * S)) + static_cast<long>(S) * s + (bit % (8 * S)) / 8;
}

__device__ __forceinline__ void step_counts(int mode, int R, int nr, int n_new, int& F,
                                            int& total, int& nr_after) {
  if (R == 0) nr = 0;
  if (mode == MODE_FLUSH) {
    F = (R > 0 && nr == R) ? R : 0;
    total = nr;
    nr_after = nr - F;
    return;
  }
  total = nr + n_new;
  if (R == 0)
    F = n_new;
  else
    F = total > R ? R * ((total - 1) / R) : 0;
  nr_after = total - F;
}

}  // namespace kvq
