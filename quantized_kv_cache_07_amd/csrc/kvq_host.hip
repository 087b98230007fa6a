// kvq_host.hip -- the C ABI of libkvq: validation, sizing, launch configuration.
//
// Everything a host can check is checked here before any launch; see include/kvq.h for the
// contract of each call.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kvq_dev.h"
#include "kvq_measure.h"

// Decode workspace of kvq_decode_attention_noalloc(): a device-resident array of the library,
// one copy per GPU, held until the process ends.  Host code never passes its name to a kernel
// (on the host that name is a stand-in, not a device address); it passes the address
// hipGetSymbolAddress() returned for the current device.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_WORKSPACE_BYTES];

namespace kvq {

hipError_t launch_append(const CacheDev& c, const uint16_t* knew, const uint16_t* vnew, int n_new,
                         int mode, hipStream_t stream);
hipError_t launch_decode_b2s(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b4s(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b8s(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b2a(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b4a(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b8a(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b16(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_b8f(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s);
// keys and values in different integer formats, one function per key format (v: value format)
hipError_t launch_decode_mixed_k2s(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_mixed_k2a(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_mixed_k4s(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_mixed_k4a(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_mixed_k8s(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
hipError_t launch_decode_mixed_k8a(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc, hipStream_t s);
// multi-query decode with 16 query rows per wave (kvq_decode_dense.h)
hipError_t launch_decode_dense(const DecodeParams& p, int bits, int scheme, hipStream_t s);

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Both sides use per-token groups: their scale (and zero) rows share one record per tile in
// the key buffers, so the rows of a tile are one contiguous run (one 128-byte line for 4-bit
// groups of 64) instead of two half-used lines.
bool shared_scale_records(const kvq_format& f) {
  return f.k.bits != 16 && f.k.scheme != KVQ_FP8 && f.k.axis == KVQ_PER_TOKEN;
}

kvq_status check_side(const kvq_side& s, bool is_key, int residual) {
  if (s.scheme == KVQ_FP8) {  // E4M3 bytes, one fp32 scale per tensor or kv head
    if (s.bits != 8 || (s.axis != KVQ_PER_TENSOR && s.axis != KVQ_PER_HEAD) || s.group != 0)
      return KVQ_EINVAL;
    return KVQ_OK;
  }
  if (s.bits == 16) {  // unquantized BF16 storage: one "group" per row, no scale
    if (s.scheme != KVQ_SYM || s.axis != KVQ_PER_TOKEN || s.group != D) return KVQ_EINVAL;
    return KVQ_OK;
  }
  if (s.bits != 2 && s.bits != 4 && s.bits != 8) return KVQ_ENOTSUP;
  if (s.scheme != KVQ_SYM && s.scheme != KVQ_ASYM) return KVQ_EINVAL;
  if (s.axis == KVQ_PER_TOKEN) {
    if (s.group != 32 && s.group != 64 && s.group != 128) return KVQ_ENOTSUP;
  } else if (s.axis == KVQ_PER_CHANNEL) {
    if (!is_key) return KVQ_ENOTSUP;
    if (s.group != 16 && s.group != 32 && s.group != 64) return KVQ_ENOTSUP;
    if (residual <= 0 || residual % s.group != 0) return KVQ_EINVAL;
  } else {
    return KVQ_EINVAL;
  }
  return KVQ_OK;
}

kvq_status check_format(const kvq_format* f) {
  if (!f) return KVQ_EINVAL;
  if (f->head_dim != D) return KVQ_ENOTSUP;
  if (f->residual < 0 || f->residual > 256 || f->residual % TILE != 0) return KVQ_EINVAL;
  kvq_status s = check_side(f->k, true, f->residual);
  if (s != KVQ_OK) return s;
  s = check_side(f->v, false, f->residual);
  if (s != KVQ_OK) return s;
  // FP8 and BF16 storage on one side only is not implemented; integer sides combine freely
  if ((f->k.scheme == KVQ_FP8) != (f->v.scheme == KVQ_FP8)) return KVQ_ENOTSUP;
  if ((f->k.bits == 16) != (f->v.bits == 16)) return KVQ_ENOTSUP;
  return KVQ_OK;
}

// Keys and values in different formats (integer widths or schemes).
bool mixed_format(const kvq_format& f) {
  return f.k.bits != f.v.bits || f.k.scheme != f.v.scheme;
}

kvq_status check_cache(const kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  kvq_status s = check_format(&c->fmt);
  if (s != KVQ_OK) return s;
  if (c->batch < 1 || c->batch > 4096 || c->n_kv_heads < 1) return KVQ_EINVAL;
  if (static_cast<long>(c->batch) * c->n_kv_heads > 65535) return KVQ_ENOTSUP;
  if (c->block_table) {
    if (c->num_blocks < 1 || c->max_blocks < 1) return KVQ_EINVAL;
  } else {
    if (c->capacity < TILE || c->capacity % TILE != 0) return KVQ_EINVAL;
    if (c->fmt.k.axis == KVQ_PER_CHANNEL && c->capacity % c->fmt.k.group != 0) return KVQ_EINVAL;
  }
  const bool scaled = c->fmt.k.bits != 16;
  const bool shared = shared_scale_records(c->fmt);  // value rows live in the key buffers
  if (!c->k_codes || !c->v_codes || (scaled && !c->k_scale) ||
      (scaled && !shared && !c->v_scale) || !c->n_quant || !c->n_res || !c->err)
    return KVQ_EINVAL;
  if (c->fmt.k.scheme == KVQ_ASYM && !c->k_zero) return KVQ_EINVAL;
  if (c->fmt.v.scheme == KVQ_ASYM && !(shared ? c->k_zero : c->v_zero)) return KVQ_EINVAL;
  if (c->fmt.residual > 0 && (!c->k_res || !c->v_res)) return KVQ_EINVAL;
  // kernels index 16-slot tiles with 32-bit integers
  const long tiles = c->block_table ? static_cast<long>(c->num_blocks) * c->n_kv_heads
                                    : static_cast<long>(c->batch) * c->n_kv_heads * (c->capacity / TILE);
  if (tiles >= (1L << 31)) return KVQ_ENOTSUP;
  const void* al[] = {c->k_codes, c->v_codes};
  for (const void* p : al)
    if (!aligned16(p)) return KVQ_EALIGN;
  if ((c->k_scale && !aligned16(c->k_scale)) || (c->v_scale && !aligned16(c->v_scale)))
    return KVQ_EALIGN;
  if ((c->k_zero && !aligned16(c->k_zero)) || (c->v_zero && !aligned16(c->v_zero)) ||
      (c->k_res && !aligned16(c->k_res)) || (c->v_res && !aligned16(c->v_res)))
    return KVQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(c->n_quant) & 3u) || (reinterpret_cast<uintptr_t>(c->n_res) & 3u) ||
      (reinterpret_cast<uintptr_t>(c->err) & 3u))
    return KVQ_EALIGN;
  return KVQ_OK;
}

CacheDev to_dev(const kvq_cache* c) {
  CacheDev d;
  d.k = {c->fmt.k.bits, c->fmt.k.scheme, c->fmt.k.axis, c->fmt.k.group};
  d.v = {c->fmt.v.bits, c->fmt.v.scheme, c->fmt.v.axis, c->fmt.v.group};
  d.R = c->fmt.residual;
  d.B = c->batch;
  d.H = c->n_kv_heads;
  d.cap = c->block_table ? 0 : c->capacity;
  d.num_blocks = c->block_table ? c->num_blocks : 0;
  d.max_blocks = c->block_table ? c->max_blocks : 0;
  d.table = c->block_table;
  d.kc = c->k_codes;
  d.vc = c->v_codes;
  d.ks = c->k_scale;
  d.vs = c->v_scale;
  d.kz = c->k_zero;
  d.vz = c->v_zero;
  d.ks_tile = d.vs_tile = 0;
  const bool rows = c->fmt.k.bits != 16 && c->fmt.k.scheme != KVQ_FP8;  // per-slot scale rows
  if (rows) {
    const int ngv = D / c->fmt.v.group;
    if (shared_scale_records(c->fmt)) {
      const int ngk = D / c->fmt.k.group;
      d.ks_tile = d.vs_tile = (ngk + ngv) * TILE;
      d.vs = c->k_scale + ngk * TILE;
      d.vz = c->k_zero ? c->k_zero + ngk * TILE : nullptr;
    } else {
      d.vs_tile = ngv * TILE;
    }
  }
  d.kres = c->k_res;
  d.vres = c->v_res;
  d.n_quant = c->n_quant;
  d.n_res = c->n_res;
  d.err = c->err;
  return d;
}

// Decode work units are 32 compressed slots or 32 window rows of one (sequence, kv head); the
// grid is persistent (about four workgroups per compute unit), each workgroup owning a
// contiguous range of units.  The workspace holds the unit prefix sum and two partial slots
// per workgroup.
struct WsLayout {
  int G, nblocks;  // G: rows of a segment (query tokens per block x query heads per kv head)
  int qbs, nqb;    // query tokens per block, query blocks per (sequence, kv head)
  int qpw, nqs;    // query blocks per segment (one per wave, or 1), segments per (seq, kv head)
  size_t pre_off, part_off, total;
};

long units_bound(const kvq_cache* c, int max_tokens) {
  // weighted units of a sequence: at most one unit more than ceil(max_tokens / 32) when a window
  // exists (the two parts round up separately), window_weight - 1 more per window unit, and the
  // segment start weight of a batch of mixed lengths
  const long R = c->fmt.residual;
  const long wu = R > 0 ? (std::min<long>(R, max_tokens) + 31) / 32 : 0;
  const long per_seq = (static_cast<long>(max_tokens) + 31) / 32 + (R > 0 ? 1 : 0) +
                       (window_weight2(c->fmt.k.bits, c->fmt.v.bits) - 1) * wu + SEGMENT_START_WEIGHT;
  return static_cast<long>(c->batch) * c->n_kv_heads * per_seq;
}

int device_cus();

// Query tokens per segment for multi-query decode: the largest power of two (at most the
// next power of two >= n_q) that keeps the segment within 8 rows, 16 QK columns (one per key
// group and row) and 32 PV rows (hi / lo part, value group, row).
// Multi-query decode takes the dense kernel (16 query rows per wave, the four waves of a
// workgroup on four blocks of one (sequence, kv head), keys and values unpacked once per
// workgroup) for caches with the same format on both sides (integer with per-token key groups of
// 32, 64 or 128 channels, FP8 E4M3 or BF16) whose tiles lie within 2 GiB of their base, once a kv
// head has query rows for two of its blocks (n_q x GQA heads >= 32; the waves of empty blocks
// only unpack their share), for 8- and 16-bit codes from one block on.  KVQ_MQ_DENSE=0 turns it off, KVQ_MQ_DENSE=1 takes
// it from 16 rows on.
bool dense_mq(const kvq_cache* c, int gkv, int n_q) {
  const kvq_side& k = c->fmt.k;
  const kvq_side& v = c->fmt.v;
  if (n_q < 2 || n_q * gkv < 16 || 16 % gkv != 0) return false;
  if (k.bits != v.bits || k.scheme != v.scheme) return false;
  const bool f8 = k.scheme == KVQ_FP8;  // E4M3 on both sides (per-head or per-tensor scales)
  const bool bf = k.bits == 16;         // BF16 storage on both sides
  if (!f8 && !bf) {
    if (k.scheme != KVQ_SYM && k.scheme != KVQ_ASYM) return false;
    if (k.bits != 2 && k.bits != 4 && k.bits != 8) return false;
    if (k.axis != KVQ_PER_TOKEN || v.axis != KVQ_PER_TOKEN) return false;
    if (k.group != 32 && k.group != 64 && k.group != 128) return false;
  }
  // tiles are addressed by 31-bit byte offsets from the sequence's first tile (contiguous) or
  // the pool's (paged)
  const long tiles = c->block_table ? static_cast<long>(c->num_blocks) * c->n_kv_heads
                                    : c->capacity / TILE;
  const long rec = (f8 || bf) ? 0 : 2L * (D / k.group + D / v.group) * TILE;  // a tile's scale record
  if (tiles * (static_cast<long>(TILE) * D * k.bits / 8) >= (1L << 31) || tiles * rec >= (1L << 31))
    return false;
  // measured on the GQA-4 sweep: from 32 rows the dense kernel beats the blocked one (4-bit
  // 287 against 326 us, 2-bit group 32 341 against 489 us), 8-bit codes already at 16 (268
  // against 312 us); formats the blocked kernel cannot serve for this GQA group (more than 16 QK
  // columns or 32 PV rows per query token) take it from 16 rows on
  const bool blocked_fits = f8 || bf || ((D / k.group) * gkv <= 16 && 2 * gkv * (D / v.group) <= 32);
  int rows_min = (!blocked_fits || k.bits >= 8) ? 16 : 32;
  if (const char* e = std::getenv("KVQ_MQ_DENSE")) {
    if (e[0] == '0') return false;
    if (e[0] == '1') rows_min = 16;
  }
  return n_q * gkv >= rows_min;
}

int query_block(const kvq_cache* c, int gkv, int n_q) {
  if (n_q <= 1) return 1;
  if (dense_mq(c, gkv, n_q)) return 16 / gkv;
  const bool whole_row = c->fmt.k.scheme == KVQ_FP8 || c->fmt.k.bits == 16;
  const bool kpc = c->fmt.k.axis == KVQ_PER_CHANNEL;
  const int ngk = kpc ? 2 : whole_row ? 1 : D / c->fmt.k.group;
  const int ngv = whole_row ? 1 : D / c->fmt.v.group;
  int qbs = 1;
  while (qbs < n_q && gkv * qbs * 2 <= 8 && ngk * gkv * qbs * 2 <= 16 && 2 * ngv * gkv * qbs * 2 <= 32)
    qbs *= 2;
  return qbs;
}

WsLayout ws_layout(const kvq_cache* c, int n_q_heads, int max_tokens, int n_q = 1) {
  WsLayout w;
  const int gkv = n_q_heads / c->n_kv_heads;
  w.qbs = query_block(c, gkv, n_q);
  w.nqb = (n_q + w.qbs - 1) / w.qbs;
  w.G = gkv * w.qbs;
  // several blocks share a segment, so the waves of a workgroup read the same codes: four blocks
  // one per wave, or two blocks of two waves each (with more blocks than waves would idle); the
  // dense kernel always has one block per wave
  w.qpw = dense_mq(c, gkv, n_q) ? 4 : w.nqb >= 4 ? 4 : w.nqb >= 2 ? 2 : 1;
  w.nqs = (w.nqb + w.qpw - 1) / w.qpw;
  long nb = static_cast<long>(device_cus()) * 4;
  if (const char* e = std::getenv("KVQ_DECODE_BLOCKS")) {
    const long v = std::atol(e);
    if (v >= 1 && v <= 65536) nb = v;
  }
  // small batches get fewer, fuller workgroups: about two units per wave (on the 8 K-token
  // worked example 12.7 us per call against 16.0 us at one unit per wave and 14.1 us at four)
  // (the 4 / qpw waves of a block share its units)
  // (the segment-start weight is not work: a batch that one workgroup covers in three units
  // per wave runs on one workgroup, with no partials and no combine launch, which costs more
  // than the third unit: the one-sequence 256-token layer took 8.6 us per call on two
  // workgroups with the combine)
  const long wpq = 4 / w.qpw;
  const long work = units_bound(c, max_tokens) -
                    static_cast<long>(c->batch) * c->n_kv_heads * SEGMENT_START_WEIGHT;
  const long ub = (work * w.nqs <= 3 * wpq) ? 1 : (work * w.nqs + 2 * wpq - 1) / (2 * wpq);
  if (nb > ub) nb = ub;
  if (nb < 1) nb = 1;
  w.nblocks = static_cast<int>(nb);
  w.pre_off = 0;
  w.part_off = ((static_cast<size_t>(c->batch) + 2) * 4 + 255) & ~static_cast<size_t>(255);
  w.total = w.part_off + static_cast<size_t>(w.nblocks) * 2 * w.qpw * w.G * PART_STRIDE * 4;
  return w;
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept; nullptr when the lookup fails.
void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace

// ---- measurement kernels ------------------------------------------------------------------

constexpr int MEASURE_BLOCKS = 2048;  // eight 256-thread workgroups per compute unit

__global__ __launch_bounds__(256) void measure_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                           float* __restrict__ sink) {
  uint32_t x = 0;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 256; i++) r ^= red[i];
    sink[blockIdx.x] = static_cast<float>(r & 0xFFFF);
  }
}

__global__ __launch_bounds__(256) void measure_copy_kernel(uint4* __restrict__ dst,
                                                           const uint4* __restrict__ src, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

}  // namespace kvq

using namespace kvq;

extern "C" {

size_t kvq_buffer_bytes(const kvq_format* fmt, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                        int32_t num_blocks, int32_t which) {
  if (check_format(fmt) != KVQ_OK || batch < 1 || n_kv_heads < 1) return 0;
  const bool paged = num_blocks > 0;
  if (!paged && (capacity < TILE || capacity % TILE)) return 0;
  const size_t tiles = paged ? static_cast<size_t>(num_blocks) * n_kv_heads
                             : static_cast<size_t>(batch) * n_kv_heads * (capacity / TILE);
  const kvq_side& s = (which == KVQ_BUF_K_CODES || which == KVQ_BUF_K_SCALE ||
                       which == KVQ_BUF_K_ZERO || which == KVQ_BUF_K_RES)
                          ? fmt->k
                          : fmt->v;
  switch (which) {
    case KVQ_BUF_K_CODES:
    case KVQ_BUF_V_CODES:
      return tiles * TILE * D * s.bits / 8;
    case KVQ_BUF_K_SCALE:
    case KVQ_BUF_V_SCALE:
    case KVQ_BUF_K_ZERO:
    case KVQ_BUF_V_ZERO: {
      if (s.bits == 16) return 0;
      if (s.scheme == KVQ_FP8) {
        if (which == KVQ_BUF_K_ZERO || which == KVQ_BUF_V_ZERO) return 0;
        return (s.axis == KVQ_PER_HEAD ? static_cast<size_t>(n_kv_heads) : 1) * sizeof(float);
      }
      if (shared_scale_records(*fmt)) {  // one record per tile in the key buffers
        if (which == KVQ_BUF_V_SCALE || which == KVQ_BUF_V_ZERO) return 0;
        // zero rows exist when either side is asymmetric (a symmetric side's rows are unused)
        if (which == KVQ_BUF_K_ZERO && fmt->k.scheme != KVQ_ASYM && fmt->v.scheme != KVQ_ASYM)
          return 0;
        return tiles * (D / fmt->k.group + D / fmt->v.group) * TILE * 2;
      }
      if ((which == KVQ_BUF_K_ZERO || which == KVQ_BUF_V_ZERO) && s.scheme != KVQ_ASYM) return 0;
      if (s.axis == KVQ_PER_TOKEN) return tiles * (D / s.group) * TILE * 2;
      if (paged) return static_cast<size_t>(num_blocks) * n_kv_heads * D * 2;  // per block
      if (capacity % s.group) return 0;
      return static_cast<size_t>(batch) * n_kv_heads * (capacity / s.group) * D * 2;
    }
    case KVQ_BUF_K_RES:
    case KVQ_BUF_V_RES:
      return static_cast<size_t>(batch) * n_kv_heads * fmt->residual * D * 2;
    default:
      return 0;
  }
}

kvq_status kvq_check_format(const kvq_format* fmt) { return check_format(fmt); }

kvq_status kvq_quantize_append(const kvq_cache* cache, const void* k_new, const void* v_new,
                               int32_t n_new, void* stream) {
  kvq_status s = check_cache(cache);
  if (s != KVQ_OK) return s;
  if (n_new < 1 || !k_new || !v_new) return KVQ_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_EALIGN;
  const CacheDev d = to_dev(cache);
  hipError_t e = launch_append(d, static_cast<const uint16_t*>(k_new),
                               static_cast<const uint16_t*>(v_new), n_new, MODE_APPEND,
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

kvq_status kvq_flush_residual(const kvq_cache* cache, void* stream) {
  kvq_status s = check_cache(cache);
  if (s != KVQ_OK) return s;
  if (cache->fmt.residual == 0) return KVQ_OK;
  const CacheDev d = to_dev(cache);
  hipError_t e = launch_append(d, nullptr, nullptr, 0, MODE_FLUSH, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t n_q_heads, int32_t max_tokens) {
  return kvq_decode_workspace_bytes_mq(cache, n_q_heads, 1, max_tokens);
}

size_t kvq_decode_workspace_bytes_mq(const kvq_cache* cache, int32_t n_q_heads, int32_t n_q,
                                     int32_t max_tokens) {
  if (check_cache(cache) != KVQ_OK || n_q_heads < 1 || max_tokens < 1 || n_q < 1 ||
      n_q > max_tokens || n_q_heads % cache->n_kv_heads)
    return 0;
  return ws_layout(cache, n_q_heads, max_tokens, n_q).total;
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t n_q_heads,
                                float sm_scale, int32_t max_tokens, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return kvq_decode_attention_mq(cache, q, 1, n_q_heads, sm_scale, max_tokens, out, workspace,
                                 workspace_bytes, stream);
}

kvq_status kvq_decode_attention_mq(const kvq_cache* cache, const void* q, int32_t n_q,
                                   int32_t n_q_heads, float sm_scale, int32_t max_tokens,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  kvq_status s = check_cache(cache);
  if (s != KVQ_OK) return s;
  if (!q || !out || !workspace || n_q_heads < 1 || max_tokens < 1) return KVQ_EINVAL;
  if (n_q < 1 || n_q > max_tokens) return KVQ_EINVAL;
  if (n_q_heads % cache->n_kv_heads) return KVQ_EINVAL;
  const int gkv = n_q_heads / cache->n_kv_heads;
  if (gkv != 1 && gkv != 2 && gkv != 4 && gkv != 8) return KVQ_ENOTSUP;
  const bool kpc = cache->fmt.k.axis == KVQ_PER_CHANNEL;
  // groups per row: FP8 and BF16 rows have one scale (or none) for all 128 channels
  const bool whole_row = cache->fmt.k.scheme == KVQ_FP8 || cache->fmt.k.bits == 16;
  const int kgroup = whole_row ? D : cache->fmt.k.group;
  const int vgroup = whole_row ? D : cache->fmt.v.group;
  const bool dense = dense_mq(cache, gkv, n_q);
  if (!kpc && (D / kgroup) * gkv > 16 && !dense) return KVQ_ENOTSUP;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_EALIGN;
  const WsLayout w = ws_layout(cache, n_q_heads, max_tokens, n_q);
  if (workspace_bytes < w.total) return KVQ_ENOSPACE;
  const int G = w.G;
  const int ngv = D / vgroup;
  const int rows = 2 * G * ngv;  // PV rows: (hi/lo part, value group, row)
  if (rows > 32 && !dense) return KVQ_ENOTSUP;
  const int NP = rows > 16 ? 2 : 1;
  if (units_bound(cache, max_tokens) * w.nqb * 64 >= (1L << 31)) return KVQ_ENOTSUP;

  DecodeParams p;
  p.c = to_dev(cache);
  p.q = static_cast<const uint16_t*>(q);
  p.out = out;
  char* ws = static_cast<char*>(workspace);
  p.ws_pre = reinterpret_cast<int32_t*>(ws + w.pre_off);
  p.ws_part = reinterpret_cast<float*>(ws + w.part_off);
  p.Hq = n_q_heads;
  p.max_tokens = max_tokens;
  p.nblocks = w.nblocks;
  p.sm_log2 = sm_scale * 1.4426950408889634f;
  p.nqt = n_q;
  p.qbs = w.qbs;
  p.nqb = w.nqb;
  p.gkv = gkv;
  p.qpw = w.qpw;
  p.nqs = w.nqs;

  if (std::getenv("KVQ_DEBUG"))
    fprintf(stderr, "[kvq] decode B=%d H=%d G=%d (n_q %d, %d per block) bits=%d NP=%d kpc=%d blocks=%d ws=%zu\n",
            cache->batch, cache->n_kv_heads, G, n_q, w.qbs, cache->fmt.k.bits, NP, kpc ? 1 : 0,
            w.nblocks, w.total);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool asym = cache->fmt.k.scheme == KVQ_ASYM;
  if (dense) {
    e = launch_decode_dense(p, cache->fmt.k.bits, cache->fmt.k.scheme, st);
    return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
  }
  if (mixed_format(cache->fmt)) {
    const int vb = cache->fmt.v.bits, vs = cache->fmt.v.scheme;
    switch (cache->fmt.k.bits) {
      case 2: e = asym ? launch_decode_mixed_k2a(p, vb, vs, G, NP, kpc, st) : launch_decode_mixed_k2s(p, vb, vs, G, NP, kpc, st); break;
      case 4: e = asym ? launch_decode_mixed_k4a(p, vb, vs, G, NP, kpc, st) : launch_decode_mixed_k4s(p, vb, vs, G, NP, kpc, st); break;
      case 8: e = asym ? launch_decode_mixed_k8a(p, vb, vs, G, NP, kpc, st) : launch_decode_mixed_k8s(p, vb, vs, G, NP, kpc, st); break;
      default: return KVQ_ENOTSUP;
    }
    return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
  }
  switch (cache->fmt.k.bits) {
    case 2: e = asym ? launch_decode_b2a(p, G, NP, kpc, st) : launch_decode_b2s(p, G, NP, kpc, st); break;
    case 4: e = asym ? launch_decode_b4a(p, G, NP, kpc, st) : launch_decode_b4s(p, G, NP, kpc, st); break;
    case 16: e = launch_decode_b16(p, G, NP, kpc, st); break;
    case 8:
      e = cache->fmt.k.scheme == KVQ_FP8 ? launch_decode_b8f(p, G, NP, kpc, st)
          : asym ? launch_decode_b8a(p, G, NP, kpc, st) : launch_decode_b8s(p, G, NP, kpc, st);
      break;
    default: return KVQ_ENOTSUP;  // unreachable: check_cache accepted the width
  }
  return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t n_q_heads,
                                        float sm_scale, int32_t max_tokens, float* out,
                                        void* stream) {
  kvq_status s = check_cache(cache);
  if (s != KVQ_OK) return s;
  if (n_q_heads < 1 || max_tokens < 1 || n_q_heads % cache->n_kv_heads) return KVQ_EINVAL;
  const size_t need = ws_layout(cache, n_q_heads, max_tokens).total;
  if (need > KVQ_NOALLOC_WORKSPACE_BYTES) return KVQ_ENOSPACE;
  void* ws = scratch_address();
  if (!ws) return KVQ_ELAUNCH;
  return kvq_decode_attention_mq(cache, q, 1, n_q_heads, sm_scale, max_tokens, out, ws,
                                 KVQ_NOALLOC_WORKSPACE_BYTES, stream);
}

kvq_status kvq_read_error(const kvq_cache* cache, int32_t* host_err, void* stream) {
  if (!cache || !cache->err || !host_err) return KVQ_EINVAL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KVQ_ELAUNCH;
  if (hipMemcpy(host_err, cache->err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return KVQ_ELAUNCH;
  return *host_err ? KVQ_EDEVICE : KVQ_OK;
}

const char* kvq_status_str(kvq_status status) {
  // a C caller may pass any int: read the value as one (an out-of-range enum load is undefined
  // in C++)
  int v;
  std::memcpy(&v, &status, sizeof v);
  switch (v) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_EINVAL: return "KVQ_EINVAL: invalid argument or descriptor";
    case KVQ_ENOTSUP: return "KVQ_ENOTSUP: combination not implemented";
    case KVQ_EALIGN: return "KVQ_EALIGN: buffer not 16-byte aligned";
    case KVQ_ENOSPACE: return "KVQ_ENOSPACE: workspace too small";
    case KVQ_ELAUNCH: return "KVQ_ELAUNCH: HIP launch failed";
    case KVQ_EDEVICE: return "KVQ_EDEVICE: device error bits set";
    default: return "unknown kvq_status";
  }
}

int32_t kvq_measure_read_sink_floats(void) { return MEASURE_BLOCKS; }

kvq_status kvq_measure_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16) return KVQ_EINVAL;
  if (!aligned16(buf)) return KVQ_EALIGN;
  measure_read_kernel<<<MEASURE_BLOCKS, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

kvq_status kvq_measure_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes == 0 || bytes % 16) return KVQ_EINVAL;
  if (!aligned16(dst) || !aligned16(src)) return KVQ_EALIGN;
  measure_copy_kernel<<<MEASURE_BLOCKS, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

}  // extern "C"
