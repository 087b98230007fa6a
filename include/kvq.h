/*
 * kvq.h -- C ABI of libkvq: a quantized KV cache with fused single-query decode attention,
 * implemented as hand-written HIP kernels for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The operations follow three pages:
 *   [P1] chipfoundryservices.com, "KV Cache Quantization"
 *   [P2] llmdaily.org, "KV-cache quantization -- making long-context inference fit in memory"
 *   [P3] oh-bug.com, "KV Cache Quantization in Practice: Managing Memory and Throughput for
 *        Long-Context Inference"
 * P1 "How KV Cache Quantization Works" gives the shape of the API: quantize keys and values
 * after they are computed, store the quantized tensors, dequantize when attention needs them.
 * P2 "How this connects to paging and prefix caching" requires that a cached block be read with
 * its own quantization format and scales, so the format travels with every cache descriptor.
 *
 * Conventions for every call:
 *   - All buffer pointers are DEVICE pointers owned by the caller (for example torch tensors);
 *     the library allocates no device memory and keeps no per-cache state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous and
 *     stream-ordered; only kvq_read_error() synchronises.
 *   - Misuse that the host can see (null pointers, unsupported formats, misaligned buffers,
 *     inconsistent sizes) returns a status before anything is launched.  Faults only the device
 *     can see (a full cache, a block-table entry outside the pool) set bits in the caller's
 *     device error word `err` (atomic OR), skip the offending sequence without advancing its
 *     counters, and leave the other sequences' results intact.
 *   - Reentrant for distinct caches; two calls that write the same cache must be ordered on one
 *     stream.  No C++ exception crosses this boundary.
 *
 * Storage layout (a format of this library; all multi-byte values little-endian):
 *   tile        16 consecutive compressed token slots of one (sequence, kv head).
 *   tile index  contiguous: (b * H_kv + h) * (capacity / 16) + slot / 16
 *               paged:      block_table[b][slot / 16] * H_kv + h     (a block holds 16 tokens)
 *   slices      a tile is 64 slices of 4 * bits bytes (one per lane of the wave that reads it),
 *               stored in pieces of S = min(16, 4 * bits) bytes: piece i of slice s (its bits
 *               8 S i .. 8 S (i + 1) - 1) sits at byte 64 S i + S s of the tile.  2- and 4-bit
 *               slices are one piece; 8-bit slices two and 16-bit slices four, 1 KiB apart.
 *   K codes     slice 4 * t + c / 32 holds channels 32 * (c / 32) .. + 31 of tile row t, channel
 *               c at bit (c % 32) * bits of the slice (little-endian inside each byte); for 2-
 *               and 4-bit codes this is plain row-major order.
 *   V codes     token-interleaved: slice (chunk) (t / 4) * (head_dim / 8) + c / 8 holds channels
 *               8 * (c / 8) .. + 7 of tile rows 4 * (t / 4) .. + 3.  Inside a chunk, with
 *               E = 32 / bits fields per 32-bit word and r = 2 * (c % 8) + (t % 4) / 2, element
 *               (t, c) is field (r % (E/2)) + (E/2) * (t % 2) of word r / (E/2).
 *   codes       offset binary: symmetric q in [-Q, Q] is stored as q + 2^(bits-1); asymmetric
 *               codes are stored as they are (0 .. 2^bits - 1); FP8 codes are E4M3 bytes; bits
 *               16 stores the bf16 elements.
 *   scales/zeros fp16.  Per-token groups: [tile][head_dim / group][16]; when both sides use
 *               per-token groups they share one record per tile in k_scale (and k_zero):
 *               [tile][head_dim / k_group + head_dim / v_group][16], the key rows then the value
 *               rows, so a tile's rows are one contiguous run (one 128-byte line for 4-bit groups
 *               of 64); v_scale / v_zero are then unused (NULL, 0 bytes), and k_zero exists when
 *               either side is asymmetric (the rows of a symmetric side are unused).  Per-channel key groups:
 *               contiguous [b][h][capacity / group][head_dim]; paged [block][h][head_dim], the
 *               row of key group tau kept with the block of its first token,
 *               block_table[b][tau * group / 16] (other blocks' rows are unused).  FP8: fp32
 *               [1] or [n_kv_heads], the caller's.
 *   window      bf16 [b][h][residual][head_dim].
 *   counters    n_quant[b] compressed tokens, n_res[b] window tokens (int32, device).
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,   /* null pointer, non-positive size, inconsistent descriptor */
  KVQ_ENOTSUP = 2,  /* a combination this library does not implement (see each call) */
  KVQ_EALIGN = 3,   /* a buffer pointer that is not 16-byte aligned */
  KVQ_ENOSPACE = 4, /* workspace smaller than kvq_decode_workspace_bytes() */
  KVQ_ELAUNCH = 5,  /* the HIP runtime refused a launch */
  KVQ_EDEVICE = 6   /* kvq_read_error() found device error bits */
} kvq_status;

/* Quantization scheme of one side [P2, "From BF16 to INT8, INT4, or even fewer bits"]:
 *   KVQ_SYM   s = max|x| / (2^(b-1) - 1), q = clip(round(x / s), -Q, Q), x^ = s q
 *   KVQ_ASYM  min-max with a zero-point: s = (max - min) / (2^b - 1), z = min,
 *             u = clip(round((x - z) / s), 0, 2^b - 1), x^ = s u + z
 * round() is half away from zero; x / s is an IEEE fp32 division by the stored fp16 scale;
 * the fp32 scale is rounded once to fp16 (nearest even).  A group whose scale is 0 stores
 * code 0 (symmetric) or u = 0 (asymmetric). */
enum { KVQ_SYM = 0, KVQ_ASYM = 1, KVQ_FP8 = 2 };

/* Grouping direction [P2, "Why scales and groups matter"; P3, "Why Can't You Quantize the KV
 * Cache Like Ordinary Activations?"]: one scale (and zero-point) per group of `group` channels
 * of one token, or, for keys only, per channel over `group` consecutive tokens. */
enum { KVQ_PER_TOKEN = 0, KVQ_PER_CHANNEL = 1, KVQ_PER_TENSOR = 2, KVQ_PER_HEAD = 3 };

/* KVQ_FP8: elements stored as OCP FP8 E4M3 bytes with one fp32 scale per tensor (axis
 * KVQ_PER_TENSOR) or per kv head (KVQ_PER_HEAD) [P3, "Step 3: Deploy a Fallback-Capable FP8
 * First": FP8 caches scaled per tensor or per attention head; "FP8 / INT8: Engineering Baseline"]:
 * code = E4M3(x / s) with x / s an IEEE fp32 division, rounded to the nearest E4M3 value (ties to
 * the even code) and saturated at +-448; x^ = s * E4M3 value.  bits 8, group 0 (else
 * KVQ_EINVAL); both sides FP8, each with its own axis.  k_scale / v_scale then point to float32
 * scales (1 or n_kv_heads of them, kvq_buffer_bytes gives the size) that the caller sets before
 * the first append and keeps for the cache's lifetime; the library only reads them.  The codes
 * use the 8-bit layout.  There are no zero buffers. */

/* Device error bits. */
enum {
  KVQ_ERR_CAPACITY = 1, /* append: a contiguous sequence has no free compressed slot */
  KVQ_ERR_BLOCK = 2,    /* a block-table entry outside [0, num_blocks) or beyond max_blocks */
  KVQ_ERR_TOKENS = 4,   /* decode: n_quant + n_res exceeded max_tokens (sequence skipped) */
  KVQ_ERR_GROUP = 8     /* append/flush with per-channel keys: n_quant is not a multiple of the
                           key group, so a flush would start inside a group (sequence skipped) */
};

/* Buffers of a cache, for kvq_buffer_bytes(). */
enum {
  KVQ_BUF_K_CODES = 0, KVQ_BUF_V_CODES = 1, KVQ_BUF_K_SCALE = 2, KVQ_BUF_V_SCALE = 3,
  KVQ_BUF_K_ZERO = 4, KVQ_BUF_V_ZERO = 5, KVQ_BUF_K_RES = 6, KVQ_BUF_V_RES = 7
};

/* bits = 16 selects the unquantized BF16 cache, the baseline and fallback the compressed
 * formats are measured against [P2, "From BF16 to INT8, INT4, or even fewer bits"; P3, "Step 3:
 * Deploy a Fallback-Capable FP8 First", "Go-Live Checklist"]: both sides 16, scheme KVQ_SYM,
 * axis KVQ_PER_TOKEN, group 128 (else KVQ_EINVAL).  Elements are stored as given -- K rows as
 * bf16 rows, V in the same token-interleaved tile layout as the codes, two bytes per field --
 * and there are no scale or zero buffers (kvq_buffer_bytes returns 0, the pointers may be
 * NULL).  Stored bytes past a sequence's end are never read into a result. */
typedef struct {
  int32_t bits;   /* 2, 4 or 8; 16 = unquantized BF16 */
  int32_t scheme; /* KVQ_SYM or KVQ_ASYM */
  int32_t axis;   /* KVQ_PER_TOKEN or KVQ_PER_CHANNEL (keys only) */
  int32_t group;  /* PER_TOKEN: channels per group, 32, 64 or 128.
                     PER_CHANNEL: tokens per group, 16, 32 or 64, dividing `residual`. */
} kvq_side;

typedef struct {
  kvq_side k, v;
  int32_t residual; /* BF16 window length R in tokens: 0 (none) or a multiple of 16, <= 256
                       [P2, "Why some systems keep a full-precision window"] */
  int32_t head_dim; /* 128 */
} kvq_format;

/* A batch cache.  Contiguous when block_table == NULL (capacity slots per sequence); paged
 * otherwise [P2, "How this connects to paging and prefix caching"]: each sequence's
 * compressed slots live in 16-token blocks of a shared pool, found through its row of the
 * block table.  Blocks that a call writes must belong to that sequence alone.
 * Prefix sharing: a sequence may start its table with blocks another sequence already wrote
 * (a shared, already-quantized prefix).  The caller then sets its counters to n_quant = the
 * prefix length (a multiple of 16 and of a per-channel key group) and n_res = 0; calls only
 * write slots >= n_quant, so shared blocks are read, never written.
 * Calls return KVQ_ENOTSUP when batch * n_kv_heads > 65535 or when a buffer would hold 2^31 or
 * more 16-slot tiles (batch * n_kv_heads * capacity / 16, or num_blocks * n_kv_heads). */
typedef struct {
  kvq_format fmt;
  int32_t batch;      /* sequences B, 1 .. 4096 */
  int32_t n_kv_heads; /* H_kv */
  int32_t capacity;   /* contiguous: compressed slots per sequence, a multiple of 16 and of a
                         per-channel key group; paged: 0 */
  int32_t num_blocks; /* paged: blocks in the pool; contiguous: 0 */
  int32_t max_blocks; /* paged: row length of block_table; contiguous: 0 */
  const int32_t *block_table; /* paged: [batch][max_blocks] int32; contiguous: NULL */
  uint8_t *k_codes, *v_codes;   /* sized by kvq_buffer_bytes(), 16-byte aligned */
  uint16_t *k_scale, *v_scale;  /* fp16 bit patterns; NULL allowed for bits 16 */
  uint16_t *k_zero, *v_zero;    /* fp16 bit patterns; NULL for a KVQ_SYM side */
  uint16_t *k_res, *v_res;      /* bf16 window; NULL when residual == 0 */
  int32_t *n_quant, *n_res;     /* [batch] counters; zero for an empty cache */
  int32_t *err;                 /* one int32 error word; the caller zero-initialises it */
} kvq_cache;

/* Bytes of buffer `which` (KVQ_BUF_*) for a contiguous cache (num_blocks == 0, `capacity`
 * slots per sequence) or a paged pool of `num_blocks` blocks.  Returns 0 for a buffer the
 * format does not use, or for an invalid format.  Pure host arithmetic.
 * The code buffers follow the memory formula of [P2, "Why the KV cache grows so quickly"]:
 * keys and values together hold 2 * T * H_kv * d_h * b bytes for T slots of b = bits / 8 bytes
 * per element; the scale (and zero-point) buffers add the per-group fp16 metadata that
 * [P2, "Worked example: an 8,192-token context"] counts on top (one two-byte scale per 64
 * elements gives 0.53125 bytes per element at 4 bits: 8,912,896 bytes per layer at H_kv = 8,
 * T = 8192). */
size_t kvq_buffer_bytes(const kvq_format *fmt, int32_t batch, int32_t n_kv_heads,
                        int32_t capacity, int32_t num_blocks, int32_t which);

/* Check a format without a cache: KVQ_OK, KVQ_EINVAL or KVQ_ENOTSUP.  Supported: head_dim 128;
 * each side 2, 4 or 8 bits, symmetric or asymmetric, chosen independently for keys and values
 * (keys and values may warrant different treatment [P2, "Why scales and groups matter"; P3,
 * "Why Can't You Quantize the KV Cache Like Ordinary Activations?"]); per-token groups
 * 32/64/128; per-channel grouping for keys only (contiguous or paged), with residual > 0
 * divisible by the group; FP8 and bits 16 as described above, on both sides (one side FP8 or
 * BF16 and the other not: KVQ_ENOTSUP).  Keys and values of different integer formats are
 * served by single-query and multi-query decode alike.  Pure host code. */
kvq_status kvq_check_format(const kvq_format *fmt);

/* Append n_new >= 1 new tokens to every sequence of the batch.
 *   k_new, v_new: bf16 [batch][n_new][n_kv_heads][head_dim], device, 16-byte aligned.
 * The result equals n_new single-token appends, each of which (P1 "How KV Cache Quantization
 * Works": quantize after computation; P2 "Why some systems keep a full-precision window"):
 *   - without a window, quantizes the token into compressed slot n_quant (n_quant += 1);
 *   - with a window of R tokens, first flushes it if it already holds R tokens (quantizes the
 *     R window rows into slots n_quant .. n_quant+R-1, n_quant += R, n_res = 0), then copies
 *     the token into window row n_res (n_res += 1).
 * After T appends to an empty sequence with R > 0: n_res = (T-1) mod R + 1.
 * Paged caches: the block table must already map every slot the call may write.
 * Device faults: KVQ_ERR_CAPACITY (contiguous slots exhausted), KVQ_ERR_BLOCK (a needed table
 * entry is outside [0, num_blocks) or beyond max_blocks), KVQ_ERR_GROUP (per-channel keys and
 * an n_quant that is not a multiple of the key group); the sequence is left unchanged.
 * Launches two kernels on `stream`. */
kvq_status kvq_quantize_append(const kvq_cache *cache, const void *k_new, const void *v_new,
                               int32_t n_new, void *stream);

/* Flush every sequence whose window holds exactly R tokens; other sequences are untouched
 * [P2, "Why some systems keep a full-precision window": once the BF16 buffer of recent tokens
 * fills, its contents are quantized and moved into the compressed cache].  The R window rows
 * are quantized into compressed slots n_quant .. n_quant + R - 1 with the side formats (per-
 * channel key groups are formed here, over whole groups of the window), then n_quant += R and
 * n_res = 0.  Optional: kvq_quantize_append() flushes by itself when a token finds the window
 * full, and calling this first never changes any result.  No-op launch-free return when R == 0.
 * Paged caches: the block table must map the R slots.  Device faults as kvq_quantize_append()
 * (the sequence is left unchanged).  Launches two kernels on `stream`. */
kvq_status kvq_flush_residual(const kvq_cache *cache, void *stream);

/* Workspace bytes kvq_decode_attention() needs for n_q_heads and a host bound max_tokens on
 * n_quant[b] + n_res[b] over the batch.  Pure host arithmetic. */
size_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t n_q_heads, int32_t max_tokens);

/* Single-query decode attention [P2, "Why the KV cache grows so quickly", attention equation]:
 * for each sequence b and query head hq, with kv head h = floor(hq * H_kv / H_q),
 *   out[b][hq] = softmax(sm_scale * q[b][hq] . K^T) V
 * over the dequantized compressed tokens 0 .. n_quant[b]-1 followed by the BF16 window rows
 * 0 .. n_res[b]-1.  K and V are dequantized in registers as they stream from HBM (P3,
 * "Misconception 1": the dequantization must be fused into the attention kernel).
 *   q:   bf16 [batch][n_q_heads][head_dim], device; n_q_heads = G * n_kv_heads, G in 1,2,4,8
 *   out: fp32 [batch][n_q_heads][head_dim], device; an empty sequence gets zeros
 *   sm_scale: typically 1 / sqrt(head_dim)
 *   max_tokens: host upper bound on n_quant[b] + n_res[b] (sizes the split over the sequence)
 *   workspace: >= kvq_decode_workspace_bytes(cache, n_q_heads, max_tokens) bytes, device
 * KVQ_ENOTSUP for a per-token key format with (head_dim / key group) * G > 16, or for
 * 2 * G * (head_dim / value group) > 32.
 * The workspace needs no initialisation and holds nothing between calls; two calls that run at
 * the same time need two workspaces.
 * Device faults: KVQ_ERR_BLOCK (a table entry outside the pool: that tile is skipped).
 * Launches two kernels on `stream`. */
kvq_status kvq_decode_attention(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                                float sm_scale, int32_t max_tokens, float *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Workspace bytes kvq_decode_attention_mq() needs for n_q query tokens per sequence;
 * kvq_decode_workspace_bytes(c, hq, mt) equals kvq_decode_workspace_bytes_mq(c, hq, 1, mt).
 * 0 for invalid arguments (n_q < 1 or n_q > max_tokens included).  Pure host arithmetic. */
size_t kvq_decode_workspace_bytes_mq(const kvq_cache *cache, int32_t n_q_heads, int32_t n_q,
                                     int32_t max_tokens);

/* Multi-query decode attention (speculative rows, a prefill chunk) over the same cache: the
 * last n_q cached tokens of every sequence are the queries' own tokens (append them first), and
 * query i attends the tokens up to and including its own, the first n_quant + n_res - n_q + i + 1
 * of the sequence (causal; a query with no such token gets zeros) [P2, "Why the KV cache grows
 * so quickly", attention equation, one row per query; P3, "Step 3: Deploy a Fallback-Capable FP8
 * First": prefill-heavy workloads gain least].  The K/V tiles streamed from HBM are dequantized
 * once per block of query rows and multiplied against all of them on the matrix cores.  With 32
 * or more query rows per kv head (n_q * n_q_heads / n_kv_heads; 16 for 8- and 16-bit codes) on a
 * cache whose two sides share one format (2/4/8-bit with per-token key groups of 32, 64 or 128,
 * FP8 E4M3 or BF16), one pass over the codes serves up to 64 rows: the values are dequantized once
 * per workgroup to f16 (FP8 exactly; BF16 values are used as stored) and the weights rounded to
 * f16 (each within 2^-11 relative; BF16: bf16 hi + lo parts; the result stays within
 * 2e-3 + 1e-2 |ref| of the exact attention over the dequantized cache).
 * Formats beyond kvq_decode_attention's column limits (for example key groups of 32 with G = 8)
 * take that path from 16 rows on (n_q * G >= 16) instead of returning KVQ_ENOTSUP.  Keys and
 * values of different formats, and per-channel keys, run on the blocks of query rows (at most 8
 * rows, 16 QK columns and 32 PV rows per block; beyond that KVQ_ENOTSUP).  Environment
 * KVQ_MQ_DENSE=0 turns that path off.
 *   q:   bf16 [batch][n_q][n_q_heads][head_dim], device, 16-byte aligned
 *   out: fp32 [batch][n_q][n_q_heads][head_dim], device
 *   n_q: 1 .. max_tokens; n_q = 1 is kvq_decode_attention.
 *   workspace: >= kvq_decode_workspace_bytes_mq(cache, n_q_heads, n_q, max_tokens) bytes
 * Other arguments, errors and device faults as kvq_decode_attention.  Launches two kernels. */
kvq_status kvq_decode_attention_mq(const kvq_cache *cache, const void *q, int32_t n_q,
                                   int32_t n_q_heads, float sm_scale, int32_t max_tokens,
                                   float *out, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Bytes of the library's own decode workspace (see kvq_decode_attention_noalloc). */
#define KVQ_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)

/* kvq_decode_attention() without a caller-supplied workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a device array of KVQ_NOALLOC_WORKSPACE_BYTES bytes inside the
 * library, one copy per GPU, held until the process ends; this call allocates nothing (no
 * hipMalloc, no allocating library routine).  Its first call on a device looks the array's
 * address up on that device.
 *   Arguments, output, results and device faults: as kvq_decode_attention().
 *   KVQ_ENOSPACE when kvq_decode_workspace_bytes(cache, n_q_heads, max_tokens) exceeds
 *   KVQ_NOALLOC_WORKSPACE_BYTES (nothing is launched); KVQ_ELAUNCH when the array's device
 *   address cannot be found.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one device (two
 * streams, or two host threads) race and give undefined results; order them on one stream.
 * Nothing in the array needs to start at zero, and a call reads nothing an earlier call left. */
kvq_status kvq_decode_attention_noalloc(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                                        float sm_scale, int32_t max_tokens, float *out,
                                        void *stream);

/* Synchronise `stream`, copy the device error word into *host_err and return KVQ_EDEVICE if
 * any bit is set, KVQ_OK otherwise.  The word is not cleared. */
kvq_status kvq_read_error(const kvq_cache *cache, int32_t *host_err, void *stream);

/* A static string naming a status. */
const char *kvq_status_str(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
