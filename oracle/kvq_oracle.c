/*
 * kvq_oracle.c -- CPU oracle for the quantized KV cache and single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg of the
 * benchmark load this library; the GPU library never does, and the two share no source,
 * header, table or helper.  Everything here is plain scalar C, written to be read against
 * the pages it follows, not to be fast.  Build: gcc -O2 -fno-fast-math -ffp-contract=off.
 *
 * Pages (cited by title and section only):
 *   [P1] chipfoundryservices.com, "KV Cache Quantization"
 *   [P2] llmdaily.org, "KV-cache quantization -- making long-context inference fit in memory"
 *   [P3] oh-bug.com, "KV Cache Quantization in Practice: Managing Memory and Throughput for
 *        Long-Context Inference"
 *
 * What it computes:
 *   - symmetric group quantizer  s = max|x| / (2^(b-1) - 1),  q = clip(round(x / s), -Q, Q),
 *     reconstruction x^ = s q                    [P2, "From BF16 to INT8, INT4, or even fewer bits"]
 *   - asymmetric (zero-point) group quantizer; the pages name it without a formula
 *     [P2 same section; P3 "4-bit / 3-bit / 2-bit", KIVI]; reading: min-max affine,
 *     s = (hi - lo) / (2^b - 1), z = lo, u = clip(round((x - z) / s), 0, 2^b - 1), x^ = s u + z
 *   - one scale per group of elements              [P2, "Why scales and groups matter"]
 *   - keys grouped per channel (over tokens), values per token
 *                                                  [P2 same section, last paragraph; P3 "Why Can't
 *                                                   You Quantize the KV Cache Like Ordinary Activations?"]
 *   - fp16 scale                                   [P2, "Worked example", one two-byte FP16 scale]
 *   - a BF16 window of recent tokens; once it holds R tokens they are quantized into the main cache
 *                                                  [P2, "Why some systems keep a full-precision window"]
 *   - block-table addressing of fixed-size blocks  [P2, "How this connects to paging and prefix caching"]
 *   - FP8 (scheme 2): elements stored as OCP FP8 E4M3 with one fp32 scale per tensor or per
 *     attention head, supplied by the caller  [P3, "Step 3: Deploy a Fallback-Capable FP8
 *     First": FP8 caches scaled per tensor or per attention head; "FP8 / INT8:
 *     Engineering Baseline"].  Reading: code = E4M3(x / s), x / s an IEEE fp32 division, the
 *     nearest E4M3 value with ties to the even code, saturating at +-448; x^ = s * E4M3 value.
 *   - bits = 16: the unquantized BF16 cache, the baseline the compressed formats are measured
 *     against and the fallback kept beside them  [P2, "From BF16 to INT8, INT4, or even fewer
 *     bits": two bytes per value; P3, "Step 3: Deploy a Fallback-Capable FP8 First" and
 *     "Go-Live Checklist": a BF16 baseline and fallback].  Elements are stored as given, with no
 *     scale; in the byte images they are 16-bit fields of the same K-row and V-tile layouts.
 *   - Attention(q_t, K, V) = softmax(q_t K^T / sqrt(d_h)) V, in fp64 on the dequantized values
 *                                                  [P2, "Why the KV cache grows so quickly", attention eq.]
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   round() is half away from zero; x / s is an IEEE fp32 division by the *stored* fp16 scale;
 *   the fp32 scale is rounded once to fp16 (nearest-even); an all-zero group (or a scale that
 *   underflows fp16) stores scale 0 and all-zero signed codes; codes are stored offset-binary
 *   (u = q + 2^(b-1) for symmetric), little-endian within a byte.
 *
 * Storage layout of the byte images this file writes (a format of this project, not of the pages):
 *   tile        = 16 consecutive compressed token slots of one (sequence, kv head)
 *   tile index  contiguous: (b * H + h) * (cap / 16) + slot / 16
 *               paged:      block_table[b][slot / 16] * H + h      (block = 16 tokens)
 *   K codes     slice (t, c / 32) of tile row t holds channels 32 (c / 32) .. + 31 at bit
 *               (c % 32) * bits of the slice (little-endian within each byte), see orc_k_bit()
 *   V codes     token-interleaved chunks of 4 tokens x 8 channels, see orc_v_bit()
 *   slices      a tile is 64 slices of 4 * bits bytes, stored in pieces of S = min(16, 4 bits)
 *               bytes: piece i of slice s at byte 64 S i + S s of the tile (slab i), so the
 *               slices' piece i form one contiguous run (for bits <= 4 a slice is one piece)
 *   scales/zeros per-token groups: fp16 [tile][d / G][16]; when both sides use per-token groups
 *               they share one record per tile in the key buffers, [tile][d/Gk + d/Gv][16]:
 *               the key rows, then the value rows (one 128-byte line for 4-bit groups of 64)
 *               per-channel key groups: contiguous fp16 [b][h][cap / Gt][d]; paged fp16
 *               [block][h][d], the row of key group tau kept with the block that holds the
 *               group's first token (block_table[b][tau * Gt / 16]), so blocks shared between
 *               sequences carry their groups' metadata with them
 *   residual    bf16 [b][h][R][d]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_SYM 0
#define ORC_ASYM 1
#define ORC_FP8 2
#define ORC_PER_TOKEN 0
#define ORC_PER_CHANNEL 1
#define ORC_PER_TENSOR 2
#define ORC_PER_HEAD 3

/* ------------------------------------------------------------------------------------------ */
/* Scalar conversions, written from the IEEE-754 / bfloat16 definitions.                       */
/* ------------------------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* binary16 -> value, exactly: subnormal m * 2^-24, normal (1024 + m) * 2^(e - 25). */
float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m | 0x400), e - 25);
  return (float)(sign ? -v : v);
}

/* binary32 -> binary16, round to nearest, ties to even; subnormals kept, overflow to inf.
 * The value is mant * 2^(e-150).  Its binary16 neighbours are multiples of the quantum
 * 2^qexp (qexp = E - 10 for a normal result, -24 in the subnormal range); the result is the
 * integer number of quanta, rounded to nearest-even, re-encoded. */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return sign | (a > 0x7f800000u ? 0x7e00 : 0x7c00);
  int e = (int)(a >> 23);
  if (e == 0) return sign; /* below 2^-126: far under half the smallest subnormal (2^-25) */
  uint64_t mant = (a & 0x7fffffu) | 0x800000u;
  int E = e - 127;
  if (E > 15) return sign | 0x7c00;
  int qexp = (E < -14) ? -24 : E - 10;
  int shift = qexp - (e - 150); /* >= 13 */
  uint64_t n;
  if (shift >= 40) {
    n = 0;
  } else {
    n = mant >> shift;
    uint64_t rem = mant & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (n & 1))) n++;
  }
  if (qexp == -24) return sign | (uint16_t)n; /* n <= 1024; 1024 encodes 2^-14 */
  return sign | (uint16_t)(((uint64_t)(E + 15) << 10) + (n - 1024)); /* carry may reach inf */
}

/* Round half away from zero of a binary32 value (exact in double). */
static double orc_round_half_away(float y) { return round((double)y); }

/* ------------------------------------------------------------------------------------------ */
/* Group quantizers [P2, "From BF16 to INT8, INT4, or even fewer bits"].                       */
/* ------------------------------------------------------------------------------------------ */

/* Symmetric: Q = 2^(b-1) - 1, s = max|x| / Q (fp32 division), stored as fp16; codes
 * q = clip(round(x / s), -Q, Q) with s the stored scale; written offset-binary q + 2^(b-1). */
void orc_quant_sym(const float *x, int n, int bits, uint16_t *scale16, uint8_t *codes) {
  int Q = (1 << (bits - 1)) - 1;
  float m = 0.0f;
  for (int i = 0; i < n; i++) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  float s32 = m / (float)Q;
  uint16_t s16 = orc_f32_to_f16(s32);
  float sf = orc_f16_to_f32(s16);
  for (int i = 0; i < n; i++) {
    int q = 0;
    if (sf != 0.0f) {
      float y = x[i] / sf;
      double r = orc_round_half_away(y);
      if (r > Q) r = Q;
      if (r < -Q) r = -Q;
      q = (int)r;
    }
    codes[i] = (uint8_t)(q + (1 << (bits - 1)));
  }
  *scale16 = s16;
}

/* Asymmetric (reading of "asymmetric zero-points"): M = 2^b - 1, s = (hi - lo) / M with an
 * fp32 subtraction then an fp32 division, z = lo; both stored fp16; u = clip(round((x - z) / s),
 * 0, M) with the stored s and z (fp32 subtraction then division). */
void orc_quant_asym(const float *x, int n, int bits, uint16_t *scale16, uint16_t *zero16,
                    uint8_t *codes) {
  int M = (1 << bits) - 1;
  float lo = x[0], hi = x[0];
  for (int i = 1; i < n; i++) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  float range = hi - lo;
  float s32 = range / (float)M;
  uint16_t s16 = orc_f32_to_f16(s32);
  uint16_t z16 = orc_f32_to_f16(lo);
  float sf = orc_f16_to_f32(s16), zf = orc_f16_to_f32(z16);
  for (int i = 0; i < n; i++) {
    int u = 0;
    if (sf != 0.0f) {
      float diff = x[i] - zf;
      float y = diff / sf;
      double r = orc_round_half_away(y);
      if (r > M) r = M;
      if (r < 0) r = 0;
      u = (int)r;
    }
    codes[i] = (uint8_t)u;
  }
  *scale16 = s16;
  *zero16 = z16;
}

/* Reconstruction, evaluated exactly in fp64: symmetric s * q, asymmetric s * u + z. */
/* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
 * (m / 8 * 2^-6); no infinities; S.1111.111 is NaN.  Value of a code, exactly. */
double orc_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* The E4M3 code nearest to y (ties: the code with an even mantissa), by search over every
 * finite non-negative code; |y| >= 448 saturates to +-448.  The sign of y is kept (-0 -> 0x80). */
uint8_t orc_e4m3_encode(float y) {
  double a = fabs((double)y);
  uint8_t sign = signbit(y) ? 0x80 : 0;
  if (a >= 448.0) return sign | 0x7E;
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    double d = fabs(orc_e4m3_value((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(sign | best);
}

double orc_dequant(int bits, int scheme, uint8_t code, uint16_t s16, uint16_t z16) {
  double s = (double)orc_f16_to_f32(s16);
  if (scheme == ORC_SYM) return s * (double)((int)code - (1 << (bits - 1)));
  return s * (double)code + (double)orc_f16_to_f32(z16);
}

/* ------------------------------------------------------------------------------------------ */
/* One sequence's cache: logical state (one code byte per element), plus the window.          */
/* Memory is owned by the caller (numpy arrays); this struct only points at it.               */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int32_t bits, scheme, axis, group;
} orc_side;

typedef struct {
  orc_side k, v;
  int32_t d, H, R, cap;
  uint8_t *ku, *vu;                /* codes [H][cap][d] */
  uint16_t *ks, *kz, *vs, *vz;     /* per-token [H][cap][d/G]; per-channel keys [H][cap/Gt][d] */
  uint16_t *kres, *vres;           /* [H][R][d] bf16 */
  int32_t n_quant, n_res;
  uint16_t *kb, *vb;               /* bits 16: the stored bf16 elements [H][cap][d] */
  float *kf8, *vf8;                /* FP8: the scale of each kv head [H] (per tensor: all equal) */
} orc_seq;

enum { ORC_OK = 0, ORC_ERR_CAPACITY = 1, ORC_ERR_FORMAT = 2 };

static size_t meta_index(const orc_seq *s, const orc_side *sd, int h, int slot, int c) {
  if (sd->axis == ORC_PER_TOKEN)
    return ((size_t)h * s->cap + slot) * (s->d / sd->group) + c / sd->group;
  return ((size_t)h * (s->cap / sd->group) + slot / sd->group) * s->d + c;
}

/* Quantize `n` bf16 rows rows[j][h][d] (row j at stride row_stride elements between tokens)
 * into compressed slots [slot0, slot0 + n). Per-token sides quantize each row's groups of G
 * channels; per-channel keys quantize each channel over groups of Gt consecutive slots. */
static void quantize_rows(orc_seq *s, int is_k, const uint16_t *rows, size_t tok_stride,
                          size_t head_stride, int n, int slot0) {
  const orc_side *sd = is_k ? &s->k : &s->v;
  if (sd->bits == 16) { /* BF16 storage: the element itself, no scale */
    uint16_t *E = is_k ? s->kb : s->vb;
    for (int h = 0; h < s->H; h++)
      for (int j = 0; j < n; j++)
        memcpy(E + ((size_t)h * s->cap + slot0 + j) * s->d,
               rows + (size_t)j * tok_stride + (size_t)h * head_stride, 2 * (size_t)s->d);
    return;
  }
  uint8_t *U = is_k ? s->ku : s->vu;
  if (sd->scheme == ORC_FP8) { /* one scale per head (or tensor), elementwise codes */
    const float *F = is_k ? s->kf8 : s->vf8;
    for (int h = 0; h < s->H; h++)
      for (int j = 0; j < n; j++)
        for (int c = 0; c < s->d; c++) {
          float x = orc_bf16_to_f32(rows[(size_t)j * tok_stride + (size_t)h * head_stride + c]);
          U[((size_t)h * s->cap + slot0 + j) * s->d + c] = orc_e4m3_encode(x / F[h]);
        }
    return;
  }
  uint16_t *S = is_k ? s->ks : s->vs;
  uint16_t *Z = is_k ? s->kz : s->vz;
  int d = s->d;
  float *x = (float *)malloc(sizeof(float) * (size_t)(d > sd->group ? d : sd->group));
  uint8_t *cq = (uint8_t *)malloc((size_t)(d > sd->group ? d : sd->group));
  for (int h = 0; h < s->H; h++) {
    if (sd->axis == ORC_PER_TOKEN) {
      int G = sd->group;
      for (int j = 0; j < n; j++) {
        const uint16_t *row = rows + (size_t)j * tok_stride + (size_t)h * head_stride;
        int slot = slot0 + j;
        for (int g = 0; g < d / G; g++) {
          for (int i = 0; i < G; i++) x[i] = orc_bf16_to_f32(row[g * G + i]);
          uint16_t s16 = 0, z16 = 0;
          if (sd->scheme == ORC_SYM)
            orc_quant_sym(x, G, sd->bits, &s16, cq);
          else
            orc_quant_asym(x, G, sd->bits, &s16, &z16, cq);
          for (int i = 0; i < G; i++) U[((size_t)h * s->cap + slot) * d + g * G + i] = cq[i];
          S[meta_index(s, sd, h, slot, g * G)] = s16;
          if (sd->scheme == ORC_ASYM) Z[meta_index(s, sd, h, slot, g * G)] = z16;
        }
      }
    } else {
      int Gt = sd->group; /* n is a multiple of Gt and slot0 is Gt-aligned (checked by caller) */
      for (int j0 = 0; j0 < n; j0 += Gt) {
        for (int c = 0; c < d; c++) {
          for (int j = 0; j < Gt; j++)
            x[j] = orc_bf16_to_f32(rows[(size_t)(j0 + j) * tok_stride + (size_t)h * head_stride + c]);
          uint16_t s16 = 0, z16 = 0;
          if (sd->scheme == ORC_SYM)
            orc_quant_sym(x, Gt, sd->bits, &s16, cq);
          else
            orc_quant_asym(x, Gt, sd->bits, &s16, &z16, cq);
          for (int j = 0; j < Gt; j++) U[((size_t)h * s->cap + slot0 + j0 + j) * d + c] = cq[j];
          S[meta_index(s, sd, h, slot0 + j0, c)] = s16;
          if (sd->scheme == ORC_ASYM) Z[meta_index(s, sd, h, slot0 + j0, c)] = z16;
        }
      }
    }
  }
  free(x);
  free(cq);
}

/* Move a full window into the compressed cache [P2, "Why some systems keep a
 * full-precision window"]: only when it holds exactly R tokens. */
int orc_flush(orc_seq *s) {
  if (s->R == 0 || s->n_res != s->R) return ORC_OK;
  if (s->n_quant + s->R > s->cap) return ORC_ERR_CAPACITY;
  size_t hs = (size_t)s->R * s->d; /* residual is [H][R][d] */
  quantize_rows(s, 1, s->kres, s->d, hs, s->R, s->n_quant);
  quantize_rows(s, 0, s->vres, s->d, hs, s->R, s->n_quant);
  s->n_quant += s->R;
  s->n_res = 0;
  return ORC_OK;
}

/* Append one token (rows k[h][d], v[h][d], bf16).  Without a window the token is quantized
 * straight into the next slot; with one, a full window is flushed first (the new token finds
 * no room), then the token is copied into the window. */
static int append_one(orc_seq *s, const uint16_t *k, const uint16_t *v) {
  if (s->R == 0) {
    if (s->k.axis == ORC_PER_CHANNEL) return ORC_ERR_FORMAT;
    if (s->n_quant + 1 > s->cap) return ORC_ERR_CAPACITY;
    quantize_rows(s, 1, k, 0, s->d, 1, s->n_quant);
    quantize_rows(s, 0, v, 0, s->d, 1, s->n_quant);
    s->n_quant += 1;
    return ORC_OK;
  }
  if (s->n_res == s->R) {
    int rc = orc_flush(s);
    if (rc) return rc;
  }
  for (int h = 0; h < s->H; h++) {
    memcpy(s->kres + ((size_t)h * s->R + s->n_res) * s->d, k + (size_t)h * s->d, 2 * (size_t)s->d);
    memcpy(s->vres + ((size_t)h * s->R + s->n_res) * s->d, v + (size_t)h * s->d, 2 * (size_t)s->d);
  }
  s->n_res += 1;
  return ORC_OK;
}

/* Append n_new tokens, k_new/v_new laid out [n_new][H][d] bf16: by definition, one at a time. */
int orc_append(orc_seq *s, const uint16_t *k_new, const uint16_t *v_new, int32_t n_new) {
  size_t row = (size_t)s->H * s->d;
  for (int j = 0; j < n_new; j++) {
    int rc = append_one(s, k_new + j * row, v_new + j * row);
    if (rc) return rc;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Decode attention in fp64 [P2, "Why the KV cache grows so quickly", attention equation].     */
/* ------------------------------------------------------------------------------------------ */

static double khat(const orc_seq *s, int h, int slot, int c) {
  if (s->k.bits == 16) return (double)orc_bf16_to_f32(s->kb[((size_t)h * s->cap + slot) * s->d + c]);
  uint8_t u = s->ku[((size_t)h * s->cap + slot) * s->d + c];
  if (s->k.scheme == ORC_FP8) return (double)s->kf8[h] * orc_e4m3_value(u);
  size_t mi = meta_index(s, &s->k, h, slot, c);
  return orc_dequant(s->k.bits, s->k.scheme, u, s->ks[mi], s->k.scheme == ORC_ASYM ? s->kz[mi] : 0);
}

static double vhat(const orc_seq *s, int h, int slot, int c) {
  if (s->v.bits == 16) return (double)orc_bf16_to_f32(s->vb[((size_t)h * s->cap + slot) * s->d + c]);
  uint8_t u = s->vu[((size_t)h * s->cap + slot) * s->d + c];
  if (s->v.scheme == ORC_FP8) return (double)s->vf8[h] * orc_e4m3_value(u);
  size_t mi = meta_index(s, &s->v, h, slot, c);
  return orc_dequant(s->v.bits, s->v.scheme, u, s->vs[mi], s->v.scheme == ORC_ASYM ? s->vz[mi] : 0);
}

/* q: [Hq][d] bf16, out: [Hq][d] fp32.  Query head hq reads kv head floor(hq * H / Hq).  The
 * attended sequence is the first T of: the compressed tokens 0..n_quant-1, then the window rows
 * 0..n_res-1.  score_t = (sum_i q_i k^_ti) * sm_scale; o = sum_t e^(score_t - max) v^_t / sum. */
static void attend_first(const orc_seq *s, const uint16_t *q, int32_t Hq, float sm_scale,
                         float *out, int T) {
  int d = s->d;
  if (T < 0) T = 0;
  double *sc = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double *qd = (double *)malloc(sizeof(double) * (size_t)d);
  double *o = (double *)malloc(sizeof(double) * (size_t)d);
  for (int hq = 0; hq < Hq; hq++) {
    int h = (int)(((long long)hq * s->H) / Hq);
    for (int i = 0; i < d; i++) qd[i] = (double)orc_bf16_to_f32(q[(size_t)hq * d + i]);
    double mx = -INFINITY;
    for (int t = 0; t < T; t++) {
      double acc = 0.0;
      if (t < s->n_quant) {
        for (int i = 0; i < d; i++) acc += qd[i] * khat(s, h, t, i);
      } else {
        const uint16_t *kr = s->kres + ((size_t)h * s->R + (t - s->n_quant)) * d;
        for (int i = 0; i < d; i++) acc += qd[i] * (double)orc_bf16_to_f32(kr[i]);
      }
      sc[t] = acc * (double)sm_scale;
      if (sc[t] > mx) mx = sc[t];
    }
    double l = 0.0;
    for (int i = 0; i < d; i++) o[i] = 0.0;
    for (int t = 0; t < T; t++) {
      double w = exp(sc[t] - mx);
      l += w;
      if (t < s->n_quant) {
        for (int i = 0; i < d; i++) o[i] += w * vhat(s, h, t, i);
      } else {
        const uint16_t *vr = s->vres + ((size_t)h * s->R + (t - s->n_quant)) * d;
        for (int i = 0; i < d; i++) o[i] += w * (double)orc_bf16_to_f32(vr[i]);
      }
    }
    for (int i = 0; i < d; i++) out[(size_t)hq * d + i] = (T > 0) ? (float)(o[i] / l) : 0.0f;
  }
  free(sc);
  free(qd);
  free(o);
}

/* Single-query decode: the query attends every cached token. */
void orc_attend(const orc_seq *s, const uint16_t *q, int32_t Hq, float sm_scale, float *out) {
  attend_first(s, q, Hq, sm_scale, out, s->n_quant + s->n_res);
}

/* Multi-query decode (speculative rows or a prefill chunk): the last n_q cached tokens are the
 * queries' own, and query i (0-based, q [n_q][Hq][d], out [n_q][Hq][d]) attends the tokens up
 * to and including its own, the first T - n_q + i + 1 of them (causal).  A query with no token
 * before it outputs zeros.  [P2, "Why the KV cache grows so quickly", attention equation, per
 * query row; P3, "Step 3: Deploy a Fallback-Capable FP8 First": prefill-heavy workloads] */
void orc_attend_mq(const orc_seq *s, const uint16_t *q, int32_t n_q, int32_t Hq, float sm_scale,
                   float *out) {
  int T = s->n_quant + s->n_res;
  for (int i = 0; i < n_q; i++)
    attend_first(s, q + (size_t)i * Hq * s->d, Hq, sm_scale, out + (size_t)i * Hq * s->d,
                 T - n_q + i + 1);
}

/* Same, but on already dequantized fp64 rows khat/vhat [T][d] (used by the pins). */
void orc_attend_rows(const double *q, const double *kh, const double *vh, int32_t T, int32_t d,
                     double sm_scale, double *out) {
  double *sc = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double mx = -INFINITY;
  for (int t = 0; t < T; t++) {
    double acc = 0.0;
    for (int i = 0; i < d; i++) acc += q[i] * kh[(size_t)t * d + i];
    sc[t] = acc * sm_scale;
    if (sc[t] > mx) mx = sc[t];
  }
  double l = 0.0;
  for (int i = 0; i < d; i++) out[i] = 0.0;
  for (int t = 0; t < T; t++) {
    double w = exp(sc[t] - mx);
    l += w;
    for (int i = 0; i < d; i++) out[i] += w * vh[(size_t)t * d + i];
  }
  for (int i = 0; i < d; i++) out[i] = (T > 0) ? out[i] / l : 0.0;
  free(sc);
}

/* ------------------------------------------------------------------------------------------ */
/* Byte images in the storage layout (see the header comment).                                 */
/* ------------------------------------------------------------------------------------------ */

/* Bit offset, inside its tile, of bit `bit` of slice `slice` (see the header comment). */
static int64_t slab_bit(int bits, int64_t slice, int64_t bit) {
  int64_t S = 4 * bits < 16 ? 4 * bits : 16;
  return 8 * (64 * S * (bit / (8 * S)) + S * slice) + bit % (8 * S);
}

/* Bit offset of (tile row t, channel c) inside a K tile: slice 4 t + c / 32, bit (c % 32) bits.
 * For 2- and 4-bit codes this is the row-major order t * d * bits + c * bits. */
int64_t orc_k_bit(int32_t bits, int32_t t, int32_t c) {
  return slab_bit(bits, 4 * (int64_t)t + c / 32, (int64_t)(c % 32) * bits);
}

/* Bit offset of (tile row t in 0..15, channel c) inside a 16-token V tile of d channels.
 * The tile is 4 * (d / 8) chunks (slices) of 4 * bits bytes; chunk (t / 4) * (d / 8) + c / 8 holds the
 * 8 channels c & ~7 .. (c & ~7) + 7 of the 4 tokens 4 (t / 4) .. 4 (t / 4) + 3.  Inside a
 * chunk, E = 32 / bits fields per 32-bit word; pair index r = 2 (c % 8) + (t % 4) / 2 picks
 * word r / (E / 2) and field r % (E / 2) in the low 16 bits for even t % 4, the same field of
 * the high 16 bits (+ E / 2) for odd t % 4. */
int64_t orc_v_bit(int32_t bits, int32_t d, int32_t t, int32_t c) {
  int64_t chunk = (int64_t)(t / 4) * (d / 8) + c / 8;
  int E = 32 / bits, Hh = E / 2;
  int tt = t % 4, jj = c % 8;
  int r = 2 * jj + tt / 2;
  int word = r / Hh, k = r % Hh;
  int field = k + Hh * (tt % 2);
  return slab_bit(bits, chunk, (int64_t)word * 32 + (int64_t)field * bits);
}

static void put_field(uint8_t *base, int64_t bit, int bits, uint8_t code) {
  uint8_t *byte = base + bit / 8;
  int sh = (int)(bit % 8);
  uint8_t mask = (uint8_t)(((1u << bits) - 1u) << sh);
  *byte = (uint8_t)((*byte & ~mask) | ((code << sh) & mask));
}

static uint8_t get_field(const uint8_t *base, int64_t bit, int bits) {
  return (uint8_t)((base[bit / 8] >> (bit % 8)) & ((1u << bits) - 1u));
}

/* 16-bit fields (BF16 storage) start on a byte boundary; little-endian. */
static void put16(uint8_t *base, int64_t bit, uint16_t x) {
  base[bit / 8] = (uint8_t)(x & 0xff);
  base[bit / 8 + 1] = (uint8_t)(x >> 8);
}

static uint16_t get16(const uint8_t *base, int64_t bit) {
  return (uint16_t)(base[bit / 8] | (base[bit / 8 + 1] << 8));
}

static int64_t tile_index(const orc_seq *s, int b, int h, int slot, const int32_t *table_row) {
  if (table_row) return (int64_t)table_row[slot / 16] * s->H + h;
  return ((int64_t)b * s->H + h) * (s->cap / 16) + slot / 16;
}

/* Write this sequence's valid state (slots < n_quant, window rows < n_res) into the batch
 * images.  table_row: this sequence's block-table row (NULL for a contiguous cache, where
 * the images hold [B][H][cap] and the sequence is index b). Unused slots are not touched. */
void orc_pack(const orc_seq *s, int32_t b, const int32_t *table_row, uint8_t *kc, uint8_t *vc,
              uint16_t *ksc, uint16_t *kzc, uint16_t *vsc, uint16_t *vzc, uint16_t *kres_img,
              uint16_t *vres_img) {
  int d = s->d;
  int64_t RBk = d * s->k.bits / 8, RBv = d * s->v.bits / 8;
  /* per-slot metadata groups; FP8 and BF16 rows have none */
  int meta = s->k.scheme != ORC_FP8 && s->k.bits != 16;
  int ngk = (meta && s->k.axis == ORC_PER_TOKEN) ? d / s->k.group : 0;
  int ngv = meta ? d / s->v.group : 0;
  for (int h = 0; h < s->H; h++) {
    for (int p = 0; p < s->n_quant; p++) {
      int64_t tile = tile_index(s, b, h, p, table_row);
      uint8_t *ktile = kc + tile * 16 * RBk;
      uint8_t *vtile = vc + tile * 16 * RBv;
      for (int c = 0; c < d; c++) {
        size_t e = ((size_t)h * s->cap + p) * d + c;
        if (s->k.bits == 16)
          put16(ktile, orc_k_bit(16, p % 16, c), s->kb[e]);
        else
          put_field(ktile, orc_k_bit(s->k.bits, p % 16, c), s->k.bits, s->ku[e]);
        if (s->v.bits == 16)
          put16(vtile, orc_v_bit(16, d, p % 16, c), s->vb[e]);
        else
          put_field(vtile, orc_v_bit(s->v.bits, d, p % 16, c), s->v.bits, s->vu[e]);
      }
      if (s->k.bits == 16 || s->k.scheme == ORC_FP8) continue; /* no per-slot metadata */
      /* shared record: key rows then value rows of each tile in the key buffers */
      int shared = s->k.axis == ORC_PER_TOKEN;
      int rows = shared ? ngk + ngv : ngv;
      uint16_t *vs_img = shared ? ksc : vsc, *vz_img = shared ? kzc : vzc;
      int v0 = shared ? ngk : 0;
      if (shared) {
        for (int g = 0; g < ngk; g++) {
          size_t mi = meta_index(s, &s->k, h, p, g * s->k.group);
          ksc[(tile * rows + g) * 16 + p % 16] = s->ks[mi];
          if (s->k.scheme == ORC_ASYM) kzc[(tile * rows + g) * 16 + p % 16] = s->kz[mi];
        }
      }
      for (int g = 0; g < ngv; g++) {
        size_t mi = meta_index(s, &s->v, h, p, g * s->v.group);
        vs_img[(tile * rows + v0 + g) * 16 + p % 16] = s->vs[mi];
        if (s->v.scheme == ORC_ASYM) vz_img[(tile * rows + v0 + g) * 16 + p % 16] = s->vz[mi];
      }
    }
    if (s->k.bits != 16 && s->k.scheme != ORC_FP8 && s->k.axis == ORC_PER_CHANNEL) {
      int Gt = s->k.group, ntau = s->n_quant / Gt;
      for (int tau = 0; tau < ntau; tau++)
        for (int c = 0; c < d; c++) {
          size_t mi = meta_index(s, &s->k, h, tau * Gt, c);
          size_t img = table_row ? ((size_t)table_row[tau * Gt / 16] * s->H + h) * d + c
                                 : (((size_t)b * s->H + h) * (s->cap / Gt) + tau) * d + c;
          ksc[img] = s->ks[mi];
          if (s->k.scheme == ORC_ASYM) kzc[img] = s->kz[mi];
        }
    }
    for (int r = 0; r < s->n_res; r++) {
      size_t src = ((size_t)h * s->R + r) * d;
      size_t dst = (((size_t)b * s->H + h) * s->R + r) * d;
      memcpy(kres_img + dst, s->kres + src, 2 * (size_t)d);
      memcpy(vres_img + dst, s->vres + src, 2 * (size_t)d);
    }
  }
}

/* Inverse of orc_pack for the code bytes only: read the codes of slots < n_quant back from
 * the images into ku/vu of `s` (used to check that the layout is a bijection). */
void orc_unpack_codes(orc_seq *s, int32_t b, const int32_t *table_row, const uint8_t *kc,
                      const uint8_t *vc) {
  int d = s->d;
  int64_t RBk = d * s->k.bits / 8, RBv = d * s->v.bits / 8;
  for (int h = 0; h < s->H; h++)
    for (int p = 0; p < s->n_quant; p++) {
      int64_t tile = tile_index(s, b, h, p, table_row);
      const uint8_t *ktile = kc + tile * 16 * RBk;
      const uint8_t *vtile = vc + tile * 16 * RBv;
      for (int c = 0; c < d; c++) {
        size_t e = ((size_t)h * s->cap + p) * d + c;
        if (s->k.bits == 16)
          s->kb[e] = get16(ktile, orc_k_bit(16, p % 16, c));
        else
          s->ku[e] = get_field(ktile, orc_k_bit(s->k.bits, p % 16, c), s->k.bits);
        if (s->v.bits == 16)
          s->vb[e] = get16(vtile, orc_v_bit(16, d, p % 16, c));
        else
          s->vu[e] = get_field(vtile, orc_v_bit(s->v.bits, d, p % 16, c), s->v.bits);
      }
    }
}

/* Vectorised helpers for the tests. */
void orc_f32_to_f16_array(const float *x, uint16_t *y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_f32_to_f16(x[i]);
}

void orc_e4m3_encode_array(const float *x, uint8_t *y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_e4m3_encode(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *x, float *y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_f16_to_f32(x[i]);
}

int32_t orc_abi_version(void) { return 4; }
