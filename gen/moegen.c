/*
 * moegen — seeded synthetic inputs (see moegen.h). Test and benchmark data only.
 *
 * The weight encoders are plain "covering" quantizers computed in fp64: every
 * sub-block gets a scale (and for Q4_K / Q5_K an offset) large enough that the
 * whole sub-block lies inside the representable range, so every element has the
 * closed-form round-trip bound |x - xhat| <= step/2 (Q4_K, Q5_K, Q6_K) or <= 2^E
 * inside the MXFP4 grid. The pages do not say how float weights become blocks;
 * these encoders exist to make test data with known error bounds.
 */
#include "moegen.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t mg_stream(uint64_t seed, uint32_t tensor, uint32_t expert, uint32_t row) {
  uint64_t s = mix64(seed + GAMMA);
  s = mix64(s + ((uint64_t)tensor + 1) * GAMMA);
  s = mix64(s + ((uint64_t)expert + 1) * GAMMA);
  s = mix64(s + ((uint64_t)row + 1) * GAMMA);
  return s;
}

uint64_t mg_u64(uint64_t stream, uint64_t n) { return mix64(stream + (n + 1) * GAMMA); }

void mg_normal_row(uint64_t seed, uint32_t tensor, uint32_t expert, uint32_t row, int n,
                   double std_, float* out) {
  /* Marsaglia's polar method: draw (u, v) uniform in (-1, 1)^2 from consecutive
   * counter values until 0 < s = u^2 + v^2 < 1, then u*f and v*f with
   * f = sqrt(-2 ln s / s) are two independent N(0, 1) values. */
  const uint64_t st = mg_stream(seed, tensor, expert, row);
  uint64_t ctr = 0;
  for (int i = 0; i < n; i += 2) {
    double u, v, s;
    do {
      u = (double)(mg_u64(st, ctr++) >> 11) * 0x1.0p-52 - 1.0;
      v = (double)(mg_u64(st, ctr++) >> 11) * 0x1.0p-52 - 1.0;
      s = u * u + v * v;
    } while (s >= 1.0 || s == 0.0);
    double f = sqrt(-2.0 * log(s) / s);
    out[i] = (float)(std_ * u * f);
    if (i + 1 < n) out[i + 1] = (float)(std_ * v * f);
  }
}

/* ---- simple row-parallel loop ------------------------------------------------ */
typedef void (*row_fn)(void* ctx, int r0, int r1);
struct par_job { row_fn fn; void* ctx; int r0, r1; };
static void* par_thread(void* p) {
  struct par_job* j = (struct par_job*)p;
  j->fn(j->ctx, j->r0, j->r1);
  return NULL;
}
static void par_rows(int rows, int threads, row_fn fn, void* ctx) {
  if (threads < 1) threads = 1;
  if (threads > rows) threads = rows > 0 ? rows : 1;
  if (threads == 1) { fn(ctx, 0, rows); return; }
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * threads);
  struct par_job* jobs = (struct par_job*)malloc(sizeof(struct par_job) * threads);
  for (int t = 0; t < threads; ++t) {
    jobs[t].fn = fn; jobs[t].ctx = ctx;
    jobs[t].r0 = (int)((long long)rows * t / threads);
    jobs[t].r1 = (int)((long long)rows * (t + 1) / threads);
    pthread_create(&tid[t], NULL, par_thread, &jobs[t]);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
  free(tid); free(jobs);
}

struct nm_ctx { uint64_t seed; uint32_t tensor, expert; int cols; double std_; float* out; };
static void nm_rows(void* p, int r0, int r1) {
  struct nm_ctx* c = (struct nm_ctx*)p;
  for (int r = r0; r < r1; ++r)
    mg_normal_row(c->seed, c->tensor, c->expert, (uint32_t)r, c->cols, c->std_,
                  c->out + (size_t)r * c->cols);
}
void mg_normal_matrix(uint64_t seed, uint32_t tensor, uint32_t expert, int rows, int cols,
                      double std_, float* out, int threads) {
  struct nm_ctx c = {seed, tensor, expert, cols, std_, out};
  par_rows(rows, threads, nm_rows, &c);
}

void mg_round_bf16(const float* in, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &in[i], 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    out[i] = (uint16_t)(b >> 16);
  }
}

/* ---- fp16 ------------------------------------------------------------------- */
uint16_t mg_fp16_ceil_bits(double v) {
  if (!(v > 0.0)) return 0;
  if (v > 65504.0) return 0x7C00; /* +inf: never reached by the data here */
  int ex;
  double f = frexp(v, &ex); /* v = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;           /* v = (2f) * 2^e, 2f in [1, 2) */
  if (e < -14) {            /* subnormal range, quantum 2^-24 */
    double n = ceil(ldexp(v, 24));
    return (uint16_t)n;     /* n == 1024 is the smallest normal, same bits */
  }
  double m = ceil((2.0 * f - 1.0) * 1024.0);
  if (m >= 1024.0) { m = 0.0; e += 1; }
  if (e > 15) return 0x7C00;
  return (uint16_t)(((e + 15) << 10) | (int)m);
}

static double fp16_value(uint16_t h) { /* positive finite values only */
  int E = (h >> 10) & 31, m = h & 1023;
  if (E == 0) return ldexp((double)m, -24);
  return ldexp((double)(1024 + m), E - 25);
}

/* Round to nearest, ties to even, for |v| < 2^51: adding and subtracting
 * 1.5 * 2^52 leaves no fraction bits, and the default IEEE rounding mode
 * breaks ties to even (needs strict double evaluation, no contraction). */
static inline double rne(double v) {
  volatile double t = v + 0x1.8p52;
  return t - 0x1.8p52;
}

size_t mg_block_bytes(int fmt) {
  switch (fmt) {
    case MG_Q4_K: return 144;
    case MG_Q6_K: return 210;
    case MG_Q5_K: return 176;
    case MG_Q2_K: return 84;
    case MG_Q3_K: return 110;
    case MG_Q4_0: return 18;
    case MG_Q5_1: return 24;
    default: return 17;
  }
}
int mg_block_elems(int fmt) {
  return (fmt == MG_MXFP4 || fmt == MG_Q4_0 || fmt == MG_Q5_1) ? 32 : 256;
}

/* ---- packers ------------------------------------------------------------------ */
void mg_pack_q4k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk) {
  blk[0] = (uint8_t)d_bits; blk[1] = (uint8_t)(d_bits >> 8);
  blk[2] = (uint8_t)dmin_bits; blk[3] = (uint8_t)(dmin_bits >> 8);
  uint8_t* s = blk + 4;
  for (int j = 0; j < 4; ++j) {
    s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
    s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
    s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
  }
  uint8_t* qs = blk + 16;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 32; ++i)
      qs[32 * c + i] = (uint8_t)((q[64 * c + i] & 15) | ((q[64 * c + 32 + i] & 15) << 4));
}

/* Q5_K (176 B): Q4_K's d, dmin and scales, then qh[32] (bit 2c of qh[l]: fifth bit
 * of weight 64c+l; bit 2c+1: of weight 64c+32+l), then Q4_K's nibbles. */
void mg_pack_q5k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk) {
  uint8_t tmp[144];
  mg_pack_q4k(d_bits, dmin_bits, sc, m, q, tmp);  /* low nibbles (masked), header */
  memcpy(blk, tmp, 16);
  memcpy(blk + 48, tmp + 16, 128);
  uint8_t* qh = blk + 16;
  for (int l = 0; l < 32; ++l) {
    uint8_t h = 0;
    for (int c = 0; c < 4; ++c)
      h |= (uint8_t)((((q[64 * c + l] >> 4) & 1) << (2 * c)) |
                     (((q[64 * c + 32 + l] >> 4) & 1) << (2 * c + 1)));
    qh[l] = h;
  }
}

/* Q2_K (84 B): scales[16] (scale low nibble, min high nibble, one per 16
 * weights), qs[64] (half h: bits 2j..2j+1 of qs[32h + l] is weight 128h + 32j + l),
 * fp16 d at 80, dmin at 82. */
void mg_pack_q2k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk) {
  for (int s = 0; s < 16; ++s) blk[s] = (uint8_t)((sc[s] & 15) | ((m[s] & 15) << 4));
  uint8_t* qs = blk + 16;
  for (int h = 0; h < 2; ++h)
    for (int l = 0; l < 32; ++l) {
      uint8_t v = 0;
      for (int j = 0; j < 4; ++j) v |= (uint8_t)((q[128 * h + 32 * j + l] & 3) << (2 * j));
      qs[32 * h + l] = v;
    }
  blk[80] = (uint8_t)d_bits; blk[81] = (uint8_t)(d_bits >> 8);
  blk[82] = (uint8_t)dmin_bits; blk[83] = (uint8_t)(dmin_bits >> 8);
}

void mg_pack_q6k(uint16_t d_bits, const int8_t* sc, const uint8_t* q, uint8_t* blk) {
  uint8_t* ql = blk;
  uint8_t* qh = blk + 128;
  for (int h = 0; h < 2; ++h) {
    const uint8_t* qq = q + 128 * h;
    for (int i = 0; i < 32; ++i) {
      ql[64 * h + i] = (uint8_t)((qq[i] & 15) | ((qq[64 + i] & 15) << 4));
      ql[64 * h + 32 + i] = (uint8_t)((qq[32 + i] & 15) | ((qq[96 + i] & 15) << 4));
      qh[32 * h + i] = (uint8_t)(((qq[i] >> 4) & 3) | (((qq[32 + i] >> 4) & 3) << 2) |
                                 (((qq[64 + i] >> 4) & 3) << 4) | (((qq[96 + i] >> 4) & 3) << 6));
    }
  }
  memcpy(blk + 192, sc, 16);
  blk[208] = (uint8_t)d_bits; blk[209] = (uint8_t)(d_bits >> 8);
}

/* Q3_K (110 B): hmask[32] @0, qs[64] @32, scales[12] @96, fp16 d @108. Weight
 * n = 128 h + 32 j + l (l < 32) keeps bits 0..1 of q + 4 in bits 2j..2j+1 of
 * qs[32 h + l] and bit 2 of q + 4 in bit 4h + j of hmask[l]. The 6-bit value
 * of sub-block s (n / 16) keeps its low 4 bits in byte s mod 8 of scales (low
 * nibble for s < 8, high nibble for s >= 8) and its top 2 bits in bits
 * 2 (s / 4).. of scales[8 + s mod 4]. q in -4..3, sc in 0..63. */
void mg_pack_q3k(uint16_t d_bits, const uint8_t* sc, const int8_t* q, uint8_t* blk) {
  memset(blk, 0, 110);
  for (int n = 0; n < 256; ++n) {
    int h = n / 128, r = n % 128, j = r / 32, l = r % 32;
    int u = q[n] + 4;
    blk[32 + 32 * h + l] |= (uint8_t)((u & 3) << (2 * j));
    blk[l] |= (uint8_t)((u >> 2) << (4 * h + j));
  }
  for (int s2 = 0; s2 < 16; ++s2) {
    int lo = sc[s2] & 15, hi = sc[s2] >> 4;
    blk[96 + s2 % 8] |= (uint8_t)(s2 < 8 ? lo : lo << 4);
    blk[104 + s2 % 4] |= (uint8_t)(hi << (2 * (s2 / 4)));
  }
  blk[108] = (uint8_t)(d_bits & 0xFF);
  blk[109] = (uint8_t)(d_bits >> 8);
}

/* Q4_0 (18 B): fp16 d @0, qs[16] @2; byte j holds element j (low nibble) and
 * element j + 16 (high nibble); q in 0..15. */
void mg_pack_q40(uint16_t d_bits, const uint8_t* q, uint8_t* blk) {
  blk[0] = (uint8_t)(d_bits & 0xFF);
  blk[1] = (uint8_t)(d_bits >> 8);
  for (int j = 0; j < 16; ++j) blk[2 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
}

/* Q5_1 (24 B): fp16 d @0, fp16 m @2, qh (32 bits, little-endian) @4, qs[16] @8;
 * bit j of qh is the fifth bit of element j; byte j of qs holds the low 4 bits
 * of element j (low nibble) and of element j + 16 (high nibble); q in 0..31. */
void mg_pack_q51(uint16_t d_bits, uint16_t m_bits, const uint8_t* q, uint8_t* blk) {
  uint32_t qh = 0;
  for (int j = 0; j < 32; ++j) qh |= (uint32_t)((q[j] >> 4) & 1) << j;
  blk[0] = (uint8_t)(d_bits & 0xFF);
  blk[1] = (uint8_t)(d_bits >> 8);
  blk[2] = (uint8_t)(m_bits & 0xFF);
  blk[3] = (uint8_t)(m_bits >> 8);
  for (int i = 0; i < 4; ++i) blk[4 + i] = (uint8_t)(qh >> (8 * i));
  for (int j = 0; j < 16; ++j) blk[8 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
}

void mg_pack_mxfp4(uint8_t e, const uint8_t* codes, uint8_t* blk) {
  blk[0] = e;
  for (int i = 0; i < 16; ++i)
    blk[1 + i] = (uint8_t)((codes[i] & 15) | ((codes[i + 16] & 15) << 4));
}

/* ---- covering encoders ----------------------------------------------------------- */
/* Scales, mins and quants (0..qmax) of a Q4_K (qmax 15) or Q5_K (qmax 31) block. */
static void encode_scale_min(const float* x, int qmax, uint16_t* d_out, uint16_t* dmin_out,
                             uint8_t* sc, uint8_t* m, uint8_t* q) {
  double mn[8], mx[8], off[8], need[8], maxoff = 0.0, maxneed = 0.0;
  for (int j = 0; j < 8; ++j) {
    double lo = 0.0, hi = -INFINITY;
    for (int i = 0; i < 32; ++i) {
      double v = x[32 * j + i];
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    mn[j] = lo; mx[j] = hi; off[j] = -lo;
    if (off[j] > maxoff) maxoff = off[j];
  }
  uint16_t dmin_bits = mg_fp16_ceil_bits(maxoff / 63.0);
  double dmin = fp16_value(dmin_bits);
  double mhat[8];
  for (int j = 0; j < 8; ++j) {
    double mj = dmin > 0.0 ? ceil(off[j] / dmin) : 0.0;
    if (mj > 63.0) mj = 63.0;
    m[j] = (uint8_t)mj;
    mhat[j] = dmin * mj;
    need[j] = (mx[j] + mhat[j]) / qmax;
    if (need[j] < 0.0) need[j] = 0.0;
    if (need[j] > maxneed) maxneed = need[j];
  }
  (void)mn;
  uint16_t d_bits = mg_fp16_ceil_bits(maxneed / 63.0);
  double d = fp16_value(d_bits);
  for (int j = 0; j < 8; ++j) {
    double s = d > 0.0 ? ceil(need[j] / d) : 0.0;
    if (s > 63.0) s = 63.0;
    sc[j] = (uint8_t)s;
    double shat = d * s;
    for (int i = 0; i < 32; ++i) {
      double v = shat > 0.0 ? rne(((double)x[32 * j + i] + mhat[j]) / shat) : 0.0;
      if (v < 0.0) v = 0.0;
      if (v > qmax) v = qmax;
      q[32 * j + i] = (uint8_t)v;
    }
  }
  *d_out = d_bits;
  *dmin_out = dmin_bits;
}

void mg_encode_q4k(const float* x, uint8_t* blk) {
  uint16_t d_bits, dmin_bits;
  uint8_t sc[8], m[8], q[256];
  encode_scale_min(x, 15, &d_bits, &dmin_bits, sc, m, q);
  mg_pack_q4k(d_bits, dmin_bits, sc, m, q, blk);
}

/* Q2_K: 16 sub-blocks of 16 with 4-bit scale and min, 2-bit quants. Covering:
 * m_s * dmin >= -min of the sub-block, sc_s * d * 3 >= max + m_s * dmin. */
void mg_encode_q2k(const float* x, uint8_t* blk) {
  double mx[16], off[16], need[16], maxoff = 0.0, maxneed = 0.0;
  for (int s = 0; s < 16; ++s) {
    double lo = 0.0, hi = -INFINITY;
    for (int i = 0; i < 16; ++i) {
      double v = x[16 * s + i];
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    mx[s] = hi; off[s] = -lo;
    if (off[s] > maxoff) maxoff = off[s];
  }
  uint16_t dmin_bits = mg_fp16_ceil_bits(maxoff / 15.0);
  double dmin = fp16_value(dmin_bits);
  uint8_t sc[16], m[16], q[256];
  double mhat[16];
  for (int s = 0; s < 16; ++s) {
    double ms = dmin > 0.0 ? ceil(off[s] / dmin) : 0.0;
    if (ms > 15.0) ms = 15.0;
    m[s] = (uint8_t)ms;
    mhat[s] = dmin * ms;
    need[s] = (mx[s] + mhat[s]) / 3.0;
    if (need[s] < 0.0) need[s] = 0.0;
    if (need[s] > maxneed) maxneed = need[s];
  }
  uint16_t d_bits = mg_fp16_ceil_bits(maxneed / 15.0);
  double d = fp16_value(d_bits);
  for (int s = 0; s < 16; ++s) {
    double c = d > 0.0 ? ceil(need[s] / d) : 0.0;
    if (c > 15.0) c = 15.0;
    sc[s] = (uint8_t)c;
    double shat = d * c;
    for (int i = 0; i < 16; ++i) {
      double v = shat > 0.0 ? rne(((double)x[16 * s + i] + mhat[s]) / shat) : 0.0;
      if (v < 0.0) v = 0.0;
      if (v > 3.0) v = 3.0;
      q[16 * s + i] = (uint8_t)v;
    }
  }
  mg_pack_q2k(d_bits, dmin_bits, sc, m, q, blk);
}

void mg_encode_q5k(const float* x, uint8_t* blk) {
  uint16_t d_bits, dmin_bits;
  uint8_t sc[8], m[8], q[256];
  encode_scale_min(x, 31, &d_bits, &dmin_bits, sc, m, q);
  mg_pack_q5k(d_bits, dmin_bits, sc, m, q, blk);
}

void mg_encode_q6k(const float* x, uint8_t* blk) {
  double need[16], maxneed = 0.0;
  for (int s = 0; s < 16; ++s) {
    double lo = 0.0, hi = 0.0;
    for (int i = 0; i < 16; ++i) {
      double v = x[16 * s + i];
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    double n = hi / 31.0;
    if (-lo / 32.0 > n) n = -lo / 32.0;
    need[s] = n;
    if (n > maxneed) maxneed = n;
  }
  uint16_t d_bits = mg_fp16_ceil_bits(maxneed / 127.0);
  double d = fp16_value(d_bits);
  int8_t sc[16];
  uint8_t q[256];
  for (int s = 0; s < 16; ++s) {
    double c = d > 0.0 ? ceil(need[s] / d) : 0.0;
    if (c > 127.0) c = 127.0;
    sc[s] = (int8_t)c;
    double shat = d * c;
    for (int i = 0; i < 16; ++i) {
      double v = shat > 0.0 ? rne((double)x[16 * s + i] / shat) : 0.0;
      if (v < -32.0) v = -32.0;
      if (v > 31.0) v = 31.0;
      q[16 * s + i] = (uint8_t)(v + 32.0);
    }
  }
  mg_pack_q6k(d_bits, sc, q, blk);
}

/* Q3_K: 16 sub-blocks of 16 with a signed scale (stored + 32) and q in -4..3.
 * Covering: need_s = max(max x / 3, -min x / 4, 0); d = fp16_ceil(max need / 31);
 * c_s = ceil(need_s / d) <= 31; every x of the sub-block lies in [-4 d c_s,
 * 3 d c_s], so |x - x^| <= d c_s / 2. */
void mg_encode_q3k(const float* x, uint8_t* blk) {
  double need[16], maxneed = 0.0;
  for (int s2 = 0; s2 < 16; ++s2) {
    double lo = 0.0, hi = 0.0;
    for (int i = 0; i < 16; ++i) {
      double v = x[16 * s2 + i];
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    need[s2] = hi / 3.0 > -lo / 4.0 ? hi / 3.0 : -lo / 4.0;
    if (need[s2] > maxneed) maxneed = need[s2];
  }
  uint16_t d_bits = mg_fp16_ceil_bits(maxneed / 31.0);
  double d = fp16_value(d_bits);
  uint8_t sc[16];
  int8_t q[256];
  for (int s2 = 0; s2 < 16; ++s2) {
    double c = d > 0.0 ? ceil(need[s2] / d) : 0.0;
    if (c > 31.0) c = 31.0;
    sc[s2] = (uint8_t)(c + 32.0);
    double shat = d * c;
    for (int i = 0; i < 16; ++i) {
      double v = shat > 0.0 ? rne((double)x[16 * s2 + i] / shat) : 0.0;
      if (v < -4.0) v = -4.0;
      if (v > 3.0) v = 3.0;
      q[16 * s2 + i] = (int8_t)v;
    }
  }
  mg_pack_q3k(d_bits, sc, q, blk);
}

/* Q4_0: d = fp16_ceil(max(max x / 7, -min x / 8, 0)), q = clamp(rne(x / d), -8, 7)
 * + 8; every x lies in [-8 d, 7 d], so |x - x^| <= d / 2. */
void mg_encode_q40(const float* x, uint8_t* blk) {
  double lo = 0.0, hi = 0.0;
  for (int i = 0; i < 32; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  double need = hi / 7.0 > -lo / 8.0 ? hi / 7.0 : -lo / 8.0;
  uint16_t d_bits = mg_fp16_ceil_bits(need);
  double d = fp16_value(d_bits);
  uint8_t q[32];
  for (int i = 0; i < 32; ++i) {
    double v = d > 0.0 ? rne((double)x[i] / d) : 0.0;
    if (v < -8.0) v = -8.0;
    if (v > 7.0) v = 7.0;
    q[i] = (uint8_t)(v + 8.0);
  }
  mg_pack_q40(d_bits, q, blk);
}

/* Q5_1: m = -fp16_ceil(-min x) (0 when min x >= 0), d = fp16_ceil((max x - m) / 31),
 * q = clamp(rne((x - m) / d), 0, 31); every x lies in [m, m + 31 d], so
 * |x - x^| <= d / 2. */
void mg_encode_q51(const float* x, uint8_t* blk) {
  double lo = 0.0, hi = 0.0;
  for (int i = 0; i < 32; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  uint16_t mneg = mg_fp16_ceil_bits(-lo);  /* lo <= 0 */
  double m = -fp16_value(mneg);
  uint16_t m_bits = (uint16_t)(mneg ? (mneg | 0x8000) : 0);
  uint16_t d_bits = mg_fp16_ceil_bits((hi - m) / 31.0);
  double d = fp16_value(d_bits);
  uint8_t q[32];
  for (int i = 0; i < 32; ++i) {
    double v = d > 0.0 ? rne(((double)x[i] - m) / d) : 0.0;
    if (v < 0.0) v = 0.0;
    if (v > 31.0) v = 31.0;
    q[i] = (uint8_t)v;
  }
  mg_pack_q51(d_bits, m_bits, q, blk);
}

/* OCP MX v1.0: shared exponent floor(log2 amax) - emax(e2m1 = 2); elements rounded
 * to nearest on the e2m1 grid, ties to the even mantissa, saturating at 6. */
void mg_encode_mxfp4(const float* x, uint8_t* blk) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  uint8_t codes[32];
  if (amax == 0.0) {
    memset(codes, 0, sizeof codes);
    mg_pack_mxfp4(0, codes, blk);
    return;
  }
  int ex;
  frexp(amax, &ex);
  int E = (ex - 1) - 2;
  if (E < -127) E = -127;
  if (E > 127) E = 127;
  for (int i = 0; i < 32; ++i) {
    double v = ldexp(fabs((double)x[i]), -E);
    int best = 7;
    if (v < 6.0) {
      best = 0;
      for (int c = 1; c < 8; ++c) {
        double dc = fabs(v - grid[c]), db = fabs(v - grid[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
      }
    }
    codes[i] = (uint8_t)(best | ((x[i] < 0.0f && best != 0) ? 8 : 0));
  }
  mg_pack_mxfp4((uint8_t)(E + 127), codes, blk);
}

struct enc_ctx { int fmt; const float* x; int K; size_t stride; uint8_t* out; };
static void enc_rows(void* p, int r0, int r1) {
  struct enc_ctx* c = (struct enc_ctx*)p;
  const int be = mg_block_elems(c->fmt);
  const size_t bb = mg_block_bytes(c->fmt);
  const int nb = c->K / be;
  for (int r = r0; r < r1; ++r) {
    uint8_t* row = c->out + (size_t)r * c->stride;
    const float* xr = c->x + (size_t)r * c->K;
    for (int b = 0; b < nb; ++b) {
      if (c->fmt == MG_Q4_K) mg_encode_q4k(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q5_K) mg_encode_q5k(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q2_K) mg_encode_q2k(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q6_K) mg_encode_q6k(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q3_K) mg_encode_q3k(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q4_0) mg_encode_q40(xr + b * be, row + b * bb);
      else if (c->fmt == MG_Q5_1) mg_encode_q51(xr + b * be, row + b * bb);
      else mg_encode_mxfp4(xr + b * be, row + b * bb);
    }
    memset(row + nb * bb, 0, c->stride - nb * bb);
  }
}
void mg_encode_matrix(int fmt, const float* x, int rows, int K, size_t stride, uint8_t* out,
                      int threads) {
  struct enc_ctx c = {fmt, x, K, stride, out};
  par_rows(rows, threads, enc_rows, &c);
}

struct wm_ctx {
  uint64_t seed; uint32_t tensor, expert; int fmt, K; size_t stride; double std_; uint8_t* out;
};
static void wm_rows(void* p, int r0, int r1) {
  struct wm_ctx* c = (struct wm_ctx*)p;
  float* buf = (float*)malloc(sizeof(float) * (size_t)c->K);
  struct enc_ctx e = {c->fmt, buf, c->K, c->stride, NULL};
  for (int r = r0; r < r1; ++r) {
    mg_normal_row(c->seed, c->tensor, c->expert, (uint32_t)r, c->K, c->std_, buf);
    e.out = c->out + (size_t)r * c->stride;
    enc_rows(&e, 0, 1);
  }
  free(buf);
}
void mg_weight_matrix(uint64_t seed, uint32_t tensor, uint32_t expert, int fmt, int rows, int K,
                      size_t stride, double std_, uint8_t* out, int threads) {
  struct wm_ctx c = {seed, tensor, expert, fmt, K, stride, std_, out};
  par_rows(rows, threads, wm_rows, &c);
}

void mg_zipf_bias(uint64_t seed, int E, double s, float* out) {
  int* perm = (int*)malloc(sizeof(int) * (size_t)E);
  for (int i = 0; i < E; ++i) perm[i] = i;
  const uint64_t st = mg_stream(seed, MG_T_ZIPF, 0, 0);
  for (int i = E - 1; i >= 1; --i) {
    int j = (int)(mg_u64(st, (uint64_t)(E - 1 - i)) % (uint64_t)(i + 1));
    int t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
  double z = 0.0;
  for (int r = 0; r < E; ++r) z += pow((double)(r + 1), -s);
  for (int r = 0; r < E; ++r) out[perm[r]] = (float)log(pow((double)(r + 1), -s) / z);
  free(perm);
}
