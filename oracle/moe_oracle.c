/*
 * moe_oracle — fp64 CPU reference of the routed-expert MoE FFN layer.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing); the
 * product path never loads it. Build: gcc -O2, no fast-math, no FP contraction,
 * so that the fp32 steps of the activation recipe are plain IEEE fp32 ops.
 *
 * Every function follows the definition of what the layer computes, in the
 * order the description gives it; nothing is blocked, fused or reordered.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ decoders */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_fp16(uint16_t bits) {
  int s = bits >> 15, E = (bits >> 10) & 31, m = bits & 1023;
  double v;
  if (E == 0) v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
  else if (E == 31) v = m ? NAN : INFINITY;
  else v = ldexp(1.0 + (double)m / 1024.0, E - 15);
  return s ? -v : v;
}

/* OCP MX v1.0 E8M0 scale: 2^(e - 127); e = 255 is NaN (never produced here). */
double or_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* OCP FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, subnormal at E = 0. */
double or_e2m1(uint8_t code) {
  int s = (code >> 3) & 1, E = (code >> 1) & 3, m = code & 1;
  double v = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
  return s ? -v : v;
}

/* OCP FP8 E4M3 (MX v1.0, §5.3.3): sign bit 7, exponent bits 6..3 (bias 7),
 * mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); 0x7F/0xFF are
 * NaN; no infinities. */
double or_e4m3(uint8_t code) {
  int s = code >> 7, ex = (code >> 3) & 15, m = code & 7;
  if (ex == 15 && m == 7) return NAN;
  double v = ex == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, ex - 7);
  return s ? -v : v;
}

/* Nearest finite E4M3 magnitude by exhaustive comparison over the 127 codes
 * 0x00..0x7E (ties: the even code); beyond 448 every value saturates. */
uint8_t or_e4m3_round(double v) {
  double a = fabs(v);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(or_e4m3((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  if (best == 0) return 0;
  return (uint8_t)(v < 0 ? (best | 0x80) : best);
}

void or_quantize_mx8(const float* x, int n, uint8_t* q, uint8_t* e) {
  for (int b = 0; b < n / 32; ++b) {
    const float* xb = x + (size_t)b * 32;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      e[b] = 0;
      for (int i = 0; i < 32; ++i) q[(size_t)b * 32 + i] = 0;
      continue;
    }
    int k;
    frexp((double)amax, &k);          /* amax = f 2^k, f in [0.5, 1): floor(log2) = k - 1 */
    int sb = (k - 1) - 8 + 127;
    if (sb < 0) sb = 0;
    if (sb > 254) sb = 254;
    e[b] = (uint8_t)sb;
    for (int i = 0; i < 32; ++i)
      q[(size_t)b * 32 + i] = or_e4m3_round(ldexp((double)xb[i], 127 - sb));  /* exact */
  }
}

double or_row_dot_mx8(const uint8_t* row, int K, const uint8_t* q, const uint8_t* e) {
  double acc = 0.0;
  for (int b = 0; b < K / 32; ++b) {
    const uint8_t* blk = row + (size_t)b * 17;
    double s = 0.0;  /* exact: products and their sum are well inside fp64 */
    for (int i = 0; i < 32; ++i) {
      uint8_t code = i < 16 ? (blk[1 + i] & 15) : (blk[1 + i - 16] >> 4);
      s += or_e2m1(code) * or_e4m3(q[(size_t)b * 32 + i]);
    }
    acc += or_e8m0(blk[0]) * or_e8m0(e[b]) * s;
  }
  return acc;
}

int or_block_elems(int fmt) {
  return (fmt == OR_MXFP4 || fmt == OR_Q4_0 || fmt == OR_Q5_1) ? 32 : 256;
}
int or_block_bytes(int fmt) {
  switch (fmt) {
    case OR_Q4_K: return 144;
    case OR_Q6_K: return 210;
    case OR_Q5_K: return 176;
    case OR_Q2_K: return 84;
    case OR_Q3_K: return 110;
    case OR_Q4_0: return 18;
    case OR_Q5_1: return 24;
    default: return 17;
  }
}
/* Activation quant block for rows of this format: q8 blocks of 32 for the
 * 32-weight formats, of 256 (with 16-element sums) for the 256-weight ones. */
int or_act_block(int fmt) { return or_block_elems(fmt) == 32 ? 32 : 256; }

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_K (and Q5_K) 6-bit sub-block scales and mins. The 12 scale bytes hold, for
 * sub-blocks 0..3, sc and m in the low 6 bits of bytes 0..3 and 4..7; for
 * sub-blocks 4..7 the low 4 bits sit in bytes 8..11 (sc low nibble, m high
 * nibble) and the top 2 bits in bits 6..7 of bytes 0..3 (sc) and 4..7 (m). */
static void q4k_scales(const uint8_t* blk, int* sc, int* m) {
  const uint8_t* s = blk + 4;
  for (int j = 0; j < 4; ++j) {
    sc[j] = s[j] & 63;
    m[j] = s[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* Q3_K's sixteen 6-bit sub-block scales (used as sc - 32): sub-block s takes
 * its low 4 bits from byte s mod 8 of the 12 scale bytes (at byte 96; the low
 * nibble for s < 8, the high nibble for s >= 8) and its top 2 bits from bits
 * 2 (s / 4).. of scale byte 8 + s mod 4. */
static void q3k_scales(const uint8_t* blk, int* sc) {
  const uint8_t* s = blk + 96;
  for (int i = 0; i < 16; ++i) {
    int lo = i < 8 ? (s[i % 8] & 15) : (s[i % 8] >> 4);
    int hi = (s[8 + i % 4] >> (2 * (i / 4))) & 3;
    sc[i] = lo | (hi << 4);
  }
}

void or_block_quants(int fmt, const uint8_t* blk, int32_t* q) {
  if (fmt == OR_Q3_K) {
    /* halves of 128: weight 32j + l (l < 32) of half h has its low 2 bits in
     * bits 2j..2j+1 of qs[32h + l] (qs at byte 32) and its high bit in bit
     * 4h + j of hmask[l] (byte l); q = low + 4 * high - 4, in -4..3 */
    const uint8_t* hm = blk;
    const uint8_t* qs = blk + 32;
    for (int n = 0; n < 256; ++n) {
      int h = n / 128, r = n % 128, j = r / 32, l = r % 32;
      int lo = (qs[32 * h + l] >> (2 * j)) & 3;
      int hi = (hm[l] >> (4 * h + j)) & 1;
      q[n] = lo + 4 * hi - 4;
    }
  } else if (fmt == OR_Q4_0 || fmt == OR_Q5_1) {
    /* byte j of the nibbles holds element j (low) and element j + 16 (high);
     * Q5_1 adds bit j of its 32-bit qh (byte 4) as the fifth bit of element j */
    const uint8_t* qs = blk + (fmt == OR_Q4_0 ? 2 : 8);
    uint32_t qh = 0;
    if (fmt == OR_Q5_1) qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) |
                             ((uint32_t)blk[6] << 16) | ((uint32_t)blk[7] << 24);
    for (int n = 0; n < 32; ++n) {
      int lo = n < 16 ? (qs[n] & 15) : (qs[n - 16] >> 4);
      q[n] = lo | (int)(((qh >> n) & 1) << 4);
    }
  } else if (fmt == OR_Q4_K) {
    /* 4 chunks of 64 weights over 32 quant bytes each: byte i of chunk c holds
     * weight 64c+i in its low nibble and weight 64c+32+i in its high nibble. */
    const uint8_t* qs = blk + 16;
    for (int n = 0; n < 256; ++n) {
      int c = n / 64, i = n % 64;
      q[n] = i < 32 ? (qs[32 * c + i] & 15) : (qs[32 * c + i - 32] >> 4);
    }
  } else if (fmt == OR_Q5_K) {
    /* Q4_K's nibble layout (at byte 48) plus a fifth bit: qh[l] (l < 32, at
     * byte 16) holds, in bit 2c, the high bit of weight 64c+l and, in bit
     * 2c+1, that of weight 64c+32+l. */
    const uint8_t* qh = blk + 16;
    const uint8_t* qs = blk + 48;
    for (int n = 0; n < 256; ++n) {
      int c = n / 64, i = n % 64, l = i % 32;
      int lo = i < 32 ? (qs[32 * c + l] & 15) : (qs[32 * c + l] >> 4);
      int hi = (qh[l] >> (2 * c + (i < 32 ? 0 : 1))) & 1;
      q[n] = lo | (hi << 4);
    }
  } else if (fmt == OR_Q2_K) {
    /* Two halves of 128 over qs[32h .. 32h+31] (byte 16): in half h, weight
     * 32j + l (l < 32) is bits 2j..2j+1 of qs[32h + l]. */
    const uint8_t* qs = blk + 16;
    for (int n = 0; n < 256; ++n) {
      int h = n / 128, r = n % 128, j = r / 32, l = r % 32;
      q[n] = (qs[32 * h + l] >> (2 * j)) & 3;
    }
  } else if (fmt == OR_Q6_K) {
    /* Two halves of 128; in half h, element r = 32*quarter + i takes its low
     * 4 bits from ql and its high 2 bits from qh[32h+i] bits 2*quarter.. */
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    for (int n = 0; n < 256; ++n) {
      int h = n / 128, r = n % 128, quarter = r / 32, i = r % 32;
      int lo = (quarter & 1) ? ql[64 * h + 32 + i] : ql[64 * h + i];
      lo = (quarter >= 2) ? (lo >> 4) : (lo & 15);
      int hi = (qh[32 * h + i] >> (2 * quarter)) & 3;
      q[n] = lo | (hi << 4);
    }
  } else {
    /* MXFP4: byte i holds element i (low nibble) and element i+16 (high). */
    const uint8_t* qs = blk + 1;
    for (int n = 0; n < 32; ++n) {
      uint8_t code = n < 16 ? (qs[n] & 15) : (qs[n - 16] >> 4);
      q[n] = (int32_t)lrint(2.0 * or_e2m1(code)); /* exact: 2*e2m1 is an integer */
    }
  }
}

void or_dequant_block(int fmt, const uint8_t* blk, double* out) {
  int32_t q[256];
  or_block_quants(fmt, blk, q);
  if (fmt == OR_Q4_K || fmt == OR_Q5_K) {  /* same scales and formula; q < 16 or < 32 */
    double d = or_fp16(rd16(blk)), dmin = or_fp16(rd16(blk + 2));
    int sc[8], m[8];
    q4k_scales(blk, sc, m);
    for (int n = 0; n < 256; ++n) out[n] = d * sc[n / 32] * q[n] - dmin * m[n / 32];
  } else if (fmt == OR_Q2_K) {
    /* scales[s] (s = n / 16): low nibble scale, high nibble min */
    double d = or_fp16(rd16(blk + 80)), dmin = or_fp16(rd16(blk + 82));
    for (int n = 0; n < 256; ++n)
      out[n] = d * (blk[n / 16] & 15) * q[n] - dmin * (blk[n / 16] >> 4);
  } else if (fmt == OR_Q6_K) {
    double d = or_fp16(rd16(blk + 208));
    const int8_t* sc = (const int8_t*)(blk + 192);
    for (int n = 0; n < 256; ++n) out[n] = d * sc[n / 16] * (q[n] - 32);
  } else if (fmt == OR_Q3_K) {
    double d = or_fp16(rd16(blk + 108));
    int sc[16];
    q3k_scales(blk, sc);
    for (int n = 0; n < 256; ++n) out[n] = d * (sc[n / 16] - 32) * q[n];
  } else if (fmt == OR_Q4_0) {
    double d = or_fp16(rd16(blk));
    for (int n = 0; n < 32; ++n) out[n] = d * (q[n] - 8);
  } else if (fmt == OR_Q5_1) {
    double d = or_fp16(rd16(blk)), m = or_fp16(rd16(blk + 2));
    for (int n = 0; n < 32; ++n) out[n] = d * q[n] + m;
  } else {
    double s = or_e8m0(blk[0]);
    for (int n = 0; n < 32; ++n) out[n] = s * 0.5 * q[n];
  }
}

void or_dequant_row(int fmt, const uint8_t* row, int K, double* out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  for (int b = 0; b < K / be; ++b) or_dequant_block(fmt, row + (size_t)b * bb, out + b * be);
}

/* ------------------------------------------------------- activation quantization */
void or_quantize_q8(const float* x, int n, int B, int8_t* qs, float* d, int16_t* bsums) {
  for (int b = 0; b < n / B; ++b) {
    const float* xb = x + (size_t)b * B;
    float amax = 0.0f;
    for (int i = 0; i < B; ++i) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      d[b] = 0.0f;
      for (int i = 0; i < B; ++i) qs[(size_t)b * B + i] = 0;
    } else {
      float iscale = 127.0f / amax;            /* IEEE fp32 division */
      for (int i = 0; i < B; ++i) {
        float v = xb[i] * iscale;              /* fp32 product */
        long r = lrintf(v);                    /* round to nearest, ties to even */
        if (r > 127) r = 127;
        if (r < -127) r = -127;
        qs[(size_t)b * B + i] = (int8_t)r;
      }
      d[b] = amax / 127.0f;
    }
    if (bsums && B == 256)
      for (int g = 0; g < 16; ++g) {
        int s = 0;
        for (int i = 0; i < 16; ++i) s += qs[(size_t)b * B + 16 * g + i];
        bsums[b * 16 + g] = (int16_t)s;
      }
  }
}

/* ------------------------------------------------------------ block dots */
void or_block_partials(int fmt, const uint8_t* row, int K, const int8_t* qs,
                       const int16_t* bsums, int32_t* out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  int32_t q[256];
  for (int b = 0; b < K / be; ++b) {
    const uint8_t* blk = row + (size_t)b * bb;
    const int8_t* a = qs + (size_t)b * be;
    or_block_quants(fmt, blk, q);
    if (fmt == OR_Q4_K || fmt == OR_Q5_K) {
      int sc[8], m[8];
      q4k_scales(blk, sc, m);
      const int16_t* bs = bsums + (size_t)b * 16;
      int64_t S1 = 0, S2 = 0;
      for (int j = 0; j < 8; ++j) {
        int64_t dot = 0;
        for (int i = 0; i < 32; ++i) dot += (int64_t)q[32 * j + i] * a[32 * j + i];
        S1 += sc[j] * dot;
        S2 += (int64_t)m[j] * (bs[2 * j] + bs[2 * j + 1]);
      }
      out[2 * b] = (int32_t)S1;
      out[2 * b + 1] = (int32_t)S2;
    } else if (fmt == OR_Q2_K) {
      /* per sub-block of 16: S1 += sc_s * dot_s, S2 += m_s * (sum of its activations) */
      const int16_t* bs = bsums + (size_t)b * 16;
      int64_t S1 = 0, S2 = 0;
      for (int s = 0; s < 16; ++s) {
        int64_t dot = 0;
        for (int i = 0; i < 16; ++i) dot += (int64_t)q[16 * s + i] * a[16 * s + i];
        S1 += (int64_t)(blk[s] & 15) * dot;
        S2 += (int64_t)(blk[s] >> 4) * bs[s];
      }
      out[2 * b] = (int32_t)S1;
      out[2 * b + 1] = (int32_t)S2;
    } else if (fmt == OR_Q6_K) {
      const int8_t* sc = (const int8_t*)(blk + 192);
      const int16_t* bs = bsums + (size_t)b * 16;
      int64_t S = 0;
      for (int s = 0; s < 16; ++s) {
        int64_t dot = 0;
        for (int i = 0; i < 16; ++i) dot += (int64_t)q[16 * s + i] * a[16 * s + i];
        S += (int64_t)sc[s] * (dot - 32 * (int64_t)bs[s]);
      }
      out[2 * b] = (int32_t)S;
      out[2 * b + 1] = 0;
    } else if (fmt == OR_Q3_K) {
      /* S = sum over sub-blocks of 16 of (sc_s - 32) * (dot of signed q with a) */
      int sc[16];
      q3k_scales(blk, sc);
      int64_t S = 0;
      for (int s = 0; s < 16; ++s) {
        int64_t dot = 0;
        for (int i = 0; i < 16; ++i) dot += (int64_t)q[16 * s + i] * a[16 * s + i];
        S += (int64_t)(sc[s] - 32) * dot;
      }
      out[2 * b] = (int32_t)S;
      out[2 * b + 1] = 0;
    } else if (fmt == OR_Q4_0) {
      /* S = sum of (q - 8) * a */
      int64_t S = 0;
      for (int i = 0; i < 32; ++i) S += (int64_t)(q[i] - 8) * a[i];
      out[2 * b] = (int32_t)S;
      out[2 * b + 1] = 0;
    } else if (fmt == OR_Q5_1) {
      /* S1 = sum of q * a, S2 = sum of a (the min term) */
      int64_t S1 = 0, S2 = 0;
      for (int i = 0; i < 32; ++i) {
        S1 += (int64_t)q[i] * a[i];
        S2 += a[i];
      }
      out[2 * b] = (int32_t)S1;
      out[2 * b + 1] = (int32_t)S2;
    } else {
      int64_t S = 0;
      for (int i = 0; i < 32; ++i) S += (int64_t)q[i] * a[i];
      out[2 * b] = (int32_t)S;
      out[2 * b + 1] = 0;
    }
  }
}

double or_block_value(int fmt, const uint8_t* blk, const int32_t* p, float d8) {
  if (fmt == OR_Q4_K || fmt == OR_Q5_K) {
    double d = or_fp16(rd16(blk)), dmin = or_fp16(rd16(blk + 2));
    return (double)d8 * (d * p[0] - dmin * p[1]);
  } else if (fmt == OR_Q2_K) {
    double d = or_fp16(rd16(blk + 80)), dmin = or_fp16(rd16(blk + 82));
    return (double)d8 * (d * p[0] - dmin * p[1]);
  } else if (fmt == OR_Q6_K) {
    return (double)d8 * or_fp16(rd16(blk + 208)) * p[0];
  } else if (fmt == OR_Q3_K) {
    return (double)d8 * or_fp16(rd16(blk + 108)) * p[0];
  } else if (fmt == OR_Q4_0) {
    return (double)d8 * or_fp16(rd16(blk)) * p[0];
  } else if (fmt == OR_Q5_1) {
    return (double)d8 * (or_fp16(rd16(blk)) * p[0] + or_fp16(rd16(blk + 2)) * p[1]);
  }
  /* e2m1 = k/2, so value = d8 * 2^(e-127) * S/2 */
  return (double)d8 * or_e8m0(blk[0]) * 0.5 * p[0];
}

double or_row_dot(int fmt, const uint8_t* row, int K, const int8_t* qs, const float* d8,
                  const int16_t* bsums) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt), nb = K / be;
  int32_t* p = (int32_t*)malloc(sizeof(int32_t) * 2 * (size_t)nb);
  or_block_partials(fmt, row, K, qs, bsums, p);
  double acc = 0.0;
  for (int b = 0; b < nb; ++b) acc += or_block_value(fmt, row + (size_t)b * bb, p + 2 * b, d8[b]);
  free(p);
  return acc;
}

/* ------------------------------------------------------------------- router */
void or_router_logits(const float* W, const float* x, int E, int H, float* logits) {
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int h = 0; h < H; ++h) acc += (double)W[(size_t)e * H + h] * (double)x[h];
    logits[e] = (float)acc;
  }
}

typedef struct { float key; int idx; } kv_t;
static int kv_cmp(const void* a, const void* b) {
  const kv_t* p = (const kv_t*)a;
  const kv_t* q = (const kv_t*)b;
  if (p->key > q->key) return -1;   /* larger key first */
  if (p->key < q->key) return 1;
  return p->idx < q->idx ? -1 : (p->idx > q->idx); /* tie: lower index first */
}

void or_topk(const float* logits, const float* sel_bias, int E, int k, int32_t* ids) {
  kv_t* v = (kv_t*)malloc(sizeof(kv_t) * (size_t)E);
  for (int e = 0; e < E; ++e) {
    float key = sel_bias ? logits[e] + sel_bias[e] : logits[e]; /* one fp32 add */
    if (key == 0.0f) key = 0.0f;                                 /* -0 -> +0 */
    v[e].key = key;
    v[e].idx = e;
  }
  qsort(v, (size_t)E, sizeof(kv_t), kv_cmp);
  for (int j = 0; j < k; ++j) ids[j] = v[j].idx;
  free(v);
}

void or_route_weights(const float* logits, const int32_t* ids, int E, int k, int router,
                      int norm_topk, double route_scale, double* w) {
  if (router == OR_SOFTMAX) {
    if (norm_topk) {
      double mx = -INFINITY, z = 0.0;
      for (int j = 0; j < k; ++j) if (logits[ids[j]] > mx) mx = logits[ids[j]];
      for (int j = 0; j < k; ++j) z += exp((double)logits[ids[j]] - mx);
      for (int j = 0; j < k; ++j) w[j] = exp((double)logits[ids[j]] - mx) / z;
    } else {
      double mx = -INFINITY, z = 0.0;
      for (int e = 0; e < E; ++e) if (logits[e] > mx) mx = logits[e];
      for (int e = 0; e < E; ++e) z += exp((double)logits[e] - mx);
      for (int j = 0; j < k; ++j) w[j] = exp((double)logits[ids[j]] - mx) / z;
    }
  } else {
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
      w[j] = 1.0 / (1.0 + exp(-(double)logits[ids[j]]));
      z += w[j];
    }
    if (norm_topk)
      for (int j = 0; j < k; ++j) w[j] /= z;
  }
  for (int j = 0; j < k; ++j) w[j] *= route_scale;
}

/* ------------------------------------------------------------------ experts */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

double or_act(int act, double alpha, double limit, double g, double u) {
  if (act == OR_SWIGLU) return g * sigmoid(g) * u;
  /* clamped SwiGLU (gpt-oss): gate clamped from above, up clamped to +-limit,
   * gate * sigmoid(alpha * gate) * (up + 1) */
  double gc = g < limit ? g : limit;
  double uc = u < -limit ? -limit : (u > limit ? limit : u);
  return gc * sigmoid(alpha * gc) * (uc + 1.0);
}

/* MXFP8 mode of one expert: x already quantized (codes xq8, scales xe). */
static void expert_ffn_mx8(const or_layer* L, const uint8_t* gate, const uint8_t* up,
                           const uint8_t* down, const float* bg, const float* bu,
                           const float* bd, const uint8_t* xq8, const uint8_t* xe, double* out,
                           float* h32) {
  const int H = L->H, F = L->F;
  float* h = (float*)malloc(sizeof(float) * (size_t)F);
  uint8_t* hq = (uint8_t*)malloc((size_t)F);
  uint8_t* he = (uint8_t*)malloc((size_t)(F / 32));
  for (int r = 0; r < F; ++r) {
    double g = or_row_dot_mx8(gate + (size_t)r * L->stride_gate, H, xq8, xe);
    double u = or_row_dot_mx8(up + (size_t)r * L->stride_up, H, xq8, xe);
    if (bg) g += bg[r];
    if (bu) u += bu[r];
    h[r] = (float)or_act(L->act, L->act_alpha, L->act_limit, g, u);
  }
  if (h32) memcpy(h32, h, sizeof(float) * (size_t)F);
  or_quantize_mx8(h, F, hq, he);
  for (int i = 0; i < H; ++i) {
    double o = or_row_dot_mx8(down + (size_t)i * L->stride_down, F, hq, he);
    if (bd) o += bd[i];
    out[i] = o;
  }
  free(h); free(hq); free(he);
}

void or_expert_ffn(const or_layer* L, const uint8_t* gate, const uint8_t* up,
                   const uint8_t* down, const float* bg, const float* bu, const float* bd,
                   const int8_t* xq, const float* xd, const int16_t* xbs, double* out,
                   float* h32) {
  const int H = L->H, F = L->F;
  const int Bh = or_act_block(L->fmt_down);
  float* h = (float*)malloc(sizeof(float) * (size_t)F);
  int8_t* hq = (int8_t*)malloc((size_t)F);
  float* hd = (float*)malloc(sizeof(float) * (size_t)(F / 32));
  int16_t* hbs = (int16_t*)malloc(sizeof(int16_t) * (size_t)(F / 16));
  for (int r = 0; r < F; ++r) {
    double g = or_row_dot(L->fmt_gate, gate + (size_t)r * L->stride_gate, H, xq, xd, xbs);
    double u = or_row_dot(L->fmt_up, up + (size_t)r * L->stride_up, H, xq, xd, xbs);
    if (bg) g += bg[r];
    if (bu) u += bu[r];
    h[r] = (float)or_act(L->act, L->act_alpha, L->act_limit, g, u);
  }
  if (h32) memcpy(h32, h, sizeof(float) * (size_t)F);
  or_quantize_q8(h, F, Bh, hq, hd, hbs);
  for (int i = 0; i < H; ++i) {
    double o = or_row_dot(L->fmt_down, down + (size_t)i * L->stride_down, F, hq, hd, hbs);
    if (bd) o += bd[i];
    out[i] = o;
  }
  free(h); free(hq); free(hd); free(hbs);
}

/* x quantized as the layer's gate/up rows consume it: q8 (q, d, bs), or
 * MXFP8 (codes in q, scale bytes in e). */
typedef struct { int8_t* q; float* d; int16_t* bs; uint8_t* e; } q8buf;
static q8buf q8_of(const or_layer* L, const float* x) {
  const int Bx = or_act_block(L->fmt_gate);
  q8buf b;
  b.q = (int8_t*)malloc((size_t)L->H);
  b.d = (float*)malloc(sizeof(float) * (size_t)(L->H / 32));
  b.bs = (int16_t*)malloc(sizeof(int16_t) * (size_t)(L->H / 16));
  b.e = (uint8_t*)malloc((size_t)(L->H / 32));
  if (L->act_quant == OR_ACTQ_MXFP8)
    or_quantize_mx8(x, L->H, (uint8_t*)b.q, b.e);
  else
    or_quantize_q8(x, L->H, Bx, b.q, b.d, b.bs);
  return b;
}
static void q8_free(q8buf b) { free(b.q); free(b.d); free(b.bs); free(b.e); }

static void run_expert(const or_layer* L, const uint8_t* gate, const uint8_t* up,
                       const uint8_t* down, const float* bg, const float* bu, const float* bd,
                       const q8buf* xq, double* out, float* h32) {
  if (L->act_quant == OR_ACTQ_MXFP8)
    expert_ffn_mx8(L, gate, up, down, bg, bu, bd, (const uint8_t*)xq->q, xq->e, out, h32);
  else
    or_expert_ffn(L, gate, up, down, bg, bu, bd, xq->q, xq->d, xq->bs, out, h32);
}

static double shared_weight(const or_layer* L, const float* x) {
  if (!L->sh_gate_vec) return 1.0;
  double acc = 0.0;
  for (int h = 0; h < L->H; ++h) acc += (double)L->sh_gate_vec[h] * (double)x[h];
  return sigmoid(acc);
}

static void add_experts(const or_layer* L, const float* x, const int32_t* ids,
                        const double* w, double* y, float* h32) {
  const int H = L->H, F = L->F;
  q8buf xq = q8_of(L, x);
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
  for (int i = 0; i < H; ++i) y[i] = 0.0;
  for (int j = 0; j < L->k; ++j) {
    int e = ids[j];
    /* an id outside [0, E) or a NULL expert is a slot that is "not mine": it
       contributes nothing (given routing may carry such ids) */
    if (e < 0 || e >= L->E || !L->gate[e]) continue;
    run_expert(L, L->gate[e], L->up[e], L->down[e], L->b_gate ? L->b_gate[e] : NULL,
               L->b_up ? L->b_up[e] : NULL, L->b_down ? L->b_down[e] : NULL, &xq, o,
               h32 ? h32 + (size_t)j * F : NULL);
    for (int i = 0; i < H; ++i) y[i] += w[j] * o[i];
  }
  if (L->sh_gate) {
    double ws = shared_weight(L, x);
    run_expert(L, L->sh_gate, L->sh_up, L->sh_down, NULL, NULL, NULL, &xq, o,
               h32 ? h32 + (size_t)L->k * F : NULL);
    for (int i = 0; i < H; ++i) y[i] += ws * o[i];
  }
  free(o);
  q8_free(xq);
}

void or_layer_token(const or_layer* L, const float* x, double* y, int32_t* ids, double* w,
                    float* logits, float* h32) {
  or_router_logits(L->w_router, x, L->E, L->H, logits);
  or_topk(logits, L->sel_bias, L->E, L->k, ids);
  or_route_weights(logits, ids, L->E, L->k, L->router, L->norm_topk, L->route_scale, w);
  add_experts(L, x, ids, w, y, h32);
}

void or_expert_part_token(const or_layer* L, const float* x, const int32_t* ids,
                          const float* w, double* y) {
  double wd[64];
  for (int j = 0; j < L->k && j < 64; ++j) wd[j] = w[j];
  add_experts(L, x, ids, wd, y, NULL);
}
