/*
 * oracle_check.c -- drives every entry point of the C oracle (quantizers, the append / flush
 * state machine, fp64 attention single- and multi-query, packing into byte images and back)
 * over every supported format, with every buffer allocated to its exact size, so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build reports any out-of-bounds access,
 * overflow or undefined conversion.  Test infrastructure: built and run by
 * tests/test_sanitizers.py with gcc -fsanitize=address,undefined; prints "ok" and exits 0.
 */
#include "kvq_oracle.c"

#include <stdio.h>

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state;
}
/* a bf16 value of about N(0, 1) (sum of uniforms), with a rare large outlier */
static uint16_t rand_bf16(void) {
  float x = 0.0f;
  for (int i = 0; i < 4; i++) x += (float)(next_u32() >> 8) / 16777216.0f - 0.5f;
  x *= 1.7f;
  if ((next_u32() & 255u) == 0) x *= 40.0f;
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

typedef struct {
  orc_side k, v;
  int R;
} fmt_t;

static size_t meta_elems(const orc_side *sd, int H, int cap, int d) {
  if (sd->bits == 16 || sd->scheme == ORC_FP8) return 1;
  if (sd->axis == ORC_PER_TOKEN) return (size_t)H * cap * (d / sd->group);
  return (size_t)H * (cap / sd->group) * d;
}

/* bytes of the batch images for B sequences (contiguous: cap slots each; paged: nblk blocks) */
static size_t img_codes(const orc_side *sd, int B, int H, int cap, int nblk, int d) {
  size_t tiles = nblk ? (size_t)nblk * H : (size_t)B * H * (cap / 16);
  return tiles * 16 * d * sd->bits / 8;
}

static int run_format(const fmt_t *f, int paged) {
  const int d = 128, H = 2, B = 2, cap = 256, Hq = 4;
  orc_seq s[2];
  void *owned[64];
  int no = 0;
#define ALLOC(p, n, T) do { p = (T *)calloc((n), sizeof(T)); owned[no++] = p; } while (0)
  for (int b = 0; b < B; b++) {
    orc_seq *q = &s[b];
    memset(q, 0, sizeof(*q));
    q->k = f->k;
    q->v = f->v;
    q->d = d;
    q->H = H;
    q->R = f->R;
    q->cap = cap;
    ALLOC(q->ku, (size_t)H * cap * d, uint8_t);
    ALLOC(q->vu, (size_t)H * cap * d, uint8_t);
    ALLOC(q->ks, meta_elems(&f->k, H, cap, d), uint16_t);
    ALLOC(q->kz, meta_elems(&f->k, H, cap, d), uint16_t);
    ALLOC(q->vs, meta_elems(&f->v, H, cap, d), uint16_t);
    ALLOC(q->vz, meta_elems(&f->v, H, cap, d), uint16_t);
    ALLOC(q->kres, (size_t)H * (f->R > 0 ? f->R : 1) * d, uint16_t);
    ALLOC(q->vres, (size_t)H * (f->R > 0 ? f->R : 1) * d, uint16_t);
    ALLOC(q->kb, f->k.bits == 16 ? (size_t)H * cap * d : 1, uint16_t);
    ALLOC(q->vb, f->v.bits == 16 ? (size_t)H * cap * d : 1, uint16_t);
    ALLOC(q->kf8, H, float);
    ALLOC(q->vf8, H, float);
    for (int h = 0; h < H; h++) {
      q->kf8[h] = 0.02f * (float)(h + 1);
      q->vf8[h] = 0.05f;
    }
  }
  /* appends: a bulk piece, then single tokens (windows flush where due), then a flush */
  const int T = 150;
  uint16_t *kx, *vx;
  ALLOC(kx, (size_t)T * H * d, uint16_t);
  ALLOC(vx, (size_t)T * H * d, uint16_t);
  for (size_t i = 0; i < (size_t)T * H * d; i++) {
    kx[i] = rand_bf16();
    vx[i] = rand_bf16();
  }
  for (int b = 0; b < B; b++) {
    int n0 = 100 - 37 * b;
    if (orc_append(&s[b], kx, vx, n0)) return 1;
    for (int t = n0; t < T; t++)
      if (orc_append(&s[b], kx + (size_t)t * H * d, vx + (size_t)t * H * d, 1)) return 2;
    if (b == 0 && orc_flush(&s[b])) return 3;
  }
  /* attention, single- and multi-query */
  uint16_t *q;
  float *out;
  ALLOC(q, (size_t)3 * Hq * d, uint16_t);
  ALLOC(out, (size_t)3 * Hq * d, float);
  for (size_t i = 0; i < (size_t)3 * Hq * d; i++) q[i] = rand_bf16();
  for (int b = 0; b < B; b++) {
    orc_attend(&s[b], q, Hq, 0.08838834764831845f, out);
    orc_attend_mq(&s[b], q, 3, Hq, 0.08838834764831845f, out);
    for (size_t i = 0; i < (size_t)3 * Hq * d; i++)
      if (out[i] != out[i]) return 4; /* NaN */
  }
  /* byte images, contiguous or paged over a permuted pool, and the codes read back */
  int nblk = paged ? B * (cap / 16) : 0;
  int32_t *table;
  ALLOC(table, (size_t)B * (cap / 16), int32_t);
  for (int i = 0; i < B * (cap / 16); i++) table[i] = (int32_t)((i * 7 + 3) % (B * (cap / 16)));
  size_t kcb = img_codes(&f->k, B, H, cap, nblk, d), vcb = img_codes(&f->v, B, H, cap, nblk, d);
  int meta = f->k.bits != 16 && f->k.scheme != ORC_FP8;
  int shared = meta && f->k.axis == ORC_PER_TOKEN;
  size_t tiles = nblk ? (size_t)nblk * H : (size_t)B * H * (cap / 16);
  size_t ks_n = 1, vs_n = 1;
  if (meta) {
    if (shared) {
      ks_n = tiles * (d / f->k.group + d / f->v.group) * 16;
      vs_n = 1;
    } else {
      ks_n = nblk ? (size_t)nblk * H * d : (size_t)B * H * (cap / f->k.group) * d;
      vs_n = tiles * (d / f->v.group) * 16;
    }
  }
  uint8_t *kc, *vc;
  uint16_t *ksi, *kzi, *vsi, *vzi, *kri, *vri;
  ALLOC(kc, kcb, uint8_t);
  ALLOC(vc, vcb, uint8_t);
  ALLOC(ksi, ks_n, uint16_t);
  ALLOC(kzi, ks_n, uint16_t);
  ALLOC(vsi, vs_n, uint16_t);
  ALLOC(vzi, vs_n, uint16_t);
  ALLOC(kri, (size_t)B * H * (f->R > 0 ? f->R : 1) * d, uint16_t);
  ALLOC(vri, (size_t)B * H * (f->R > 0 ? f->R : 1) * d, uint16_t);
  for (int b = 0; b < B; b++) {
    const int32_t *row = paged ? table + (size_t)b * (cap / 16) : NULL;
    orc_pack(&s[b], b, row, kc, vc, ksi, kzi, vsi, vzi, kri, vri);
  }
  for (int b = 0; b < B; b++) {
    const int32_t *row = paged ? table + (size_t)b * (cap / 16) : NULL;
    uint8_t *ku0 = s[b].ku, *vu0 = s[b].vu;
    uint16_t *kb0 = s[b].kb, *vb0 = s[b].vb;
    uint8_t *ku1, *vu1;
    uint16_t *kb1, *vb1;
    ALLOC(ku1, (size_t)H * cap * d, uint8_t);
    ALLOC(vu1, (size_t)H * cap * d, uint8_t);
    ALLOC(kb1, f->k.bits == 16 ? (size_t)H * cap * d : 1, uint16_t);
    ALLOC(vb1, f->v.bits == 16 ? (size_t)H * cap * d : 1, uint16_t);
    s[b].ku = ku1; s[b].vu = vu1; s[b].kb = kb1; s[b].vb = vb1;
    orc_unpack_codes(&s[b], b, row, kc, vc);
    for (int h = 0; h < H; h++)
      for (int p = 0; p < s[b].n_quant; p++)
        for (int c = 0; c < d; c++) {
          size_t e = ((size_t)h * cap + p) * d + c;
          if (f->k.bits == 16 ? kb1[e] != kb0[e] : ku1[e] != ku0[e]) return 5;
          if (f->v.bits == 16 ? vb1[e] != vb0[e] : vu1[e] != vu0[e]) return 6;
        }
  }
  for (int i = 0; i < no; i++) free(owned[i]);
  return 0;
}

int main(void) {
  const fmt_t fmts[] = {
      {{8, ORC_SYM, ORC_PER_TOKEN, 128}, {8, ORC_SYM, ORC_PER_TOKEN, 128}, 0},
      {{4, ORC_SYM, ORC_PER_TOKEN, 64}, {4, ORC_SYM, ORC_PER_TOKEN, 64}, 32},
      {{2, ORC_ASYM, ORC_PER_CHANNEL, 32}, {2, ORC_ASYM, ORC_PER_TOKEN, 32}, 64},
      {{4, ORC_ASYM, ORC_PER_CHANNEL, 16}, {8, ORC_SYM, ORC_PER_TOKEN, 128}, 16},
      {{8, ORC_ASYM, ORC_PER_TOKEN, 32}, {2, ORC_SYM, ORC_PER_TOKEN, 64}, 16},
      {{2, ORC_SYM, ORC_PER_TOKEN, 32}, {4, ORC_ASYM, ORC_PER_TOKEN, 32}, 0},
      {{16, ORC_SYM, ORC_PER_TOKEN, 128}, {16, ORC_SYM, ORC_PER_TOKEN, 128}, 16},
      {{8, ORC_FP8, ORC_PER_HEAD, 0}, {8, ORC_FP8, ORC_PER_TENSOR, 0}, 32},
  };
  for (size_t i = 0; i < sizeof(fmts) / sizeof(fmts[0]); i++)
    for (int paged = 0; paged < 2; paged++) {
      int rc = run_format(&fmts[i], paged);
      if (rc) {
        printf("format %zu paged %d failed: %d\n", i, paged, rc);
        return 1;
      }
    }
  /* conversions over wide ranges of bit patterns */
  for (uint32_t u = 0; u < 0xFFFFFFFFu - 0x00010000u; u += 0x00010001u) {
    float x;
    memcpy(&x, &u, 4);
    if (x == x) (void)orc_f16_to_f32(orc_f32_to_f16(x));
    (void)orc_e4m3_encode(x);
  }
  printf("ok\n");
  return 0;
}
