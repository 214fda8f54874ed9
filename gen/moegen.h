/*
 * moegen — seeded synthetic inputs for the routed-expert FFN layer.
 *
 * This module produces test and benchmark data only: fp32 tensors drawn from
 * N(0, std), and weight matrices turned into the stored block formats by plain
 * "covering" encoders. It holds none of the layer's arithmetic (no activation
 * quantization, no block decoding, no routing). The oracle and the HIP library
 * both consume the bytes it writes; neither includes this header.
 *
 * Randomness: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based generator: the n-th
 * value of a stream with state S is mix64(S + (n+1)*GAMMA), so any element can
 * be produced independently and the output does not depend on thread count.
 * Normals use Marsaglia's polar method in fp64 (one stream per row).
 *
 * Block formats written (little-endian, the ggml/GGUF on-disk conventions):
 *   Q4_K  144 B / 256 weights: fp16 d @0, fp16 dmin @2, 12 B packed 6-bit
 *         sub-block scales and mins @4, 128 B of 4-bit quants @16.
 *   Q6_K  210 B / 256 weights: ql[128] @0, qh[64] @128, int8 scales[16] @192,
 *         fp16 d @208.
 *   MXFP4 17 B / 32 weights: E8M0 scale byte @0, 16 B of e2m1 nibbles @1
 *         (OCP Microscaling Formats v1.0).
 *   Q5_K 176 B, Q2_K 84 B, Q3_K 110 B (256 weights), Q4_0 18 B and Q5_1 24 B
 *         (32 weights): see the packers in moegen.c.
 */
#ifndef MOEGEN_H
#define MOEGEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MG_Q4_K = 0, MG_Q6_K = 1, MG_MXFP4 = 2, MG_Q5_K = 3, MG_Q2_K = 4, MG_Q3_K = 5,
       MG_Q4_0 = 6, MG_Q5_1 = 7 };

/* Tensor identifiers that key the random streams. */
enum {
  MG_T_ROUTER = 1, MG_T_X = 2, MG_T_GATE = 3, MG_T_UP = 4, MG_T_DOWN = 5,
  MG_T_BGATE = 6, MG_T_BUP = 7, MG_T_BDOWN = 8, MG_T_ZIPF = 9, MG_T_SHVEC = 10
};

uint64_t mg_stream(uint64_t seed, uint32_t tensor, uint32_t expert, uint32_t row);
uint64_t mg_u64(uint64_t stream, uint64_t n);

/* n normals * std, rounded to fp32, from stream (seed, tensor, expert, row). */
void mg_normal_row(uint64_t seed, uint32_t tensor, uint32_t expert, uint32_t row,
                   int n, double std_, float* out);
/* rows x cols fp32 tensor; row r uses stream (seed, tensor, expert, r). */
void mg_normal_matrix(uint64_t seed, uint32_t tensor, uint32_t expert, int rows, int cols,
                      double std_, float* out, int threads);

/* Round fp32 to bf16 (round to nearest, ties to even). */
void mg_round_bf16(const float* in, uint16_t* out, size_t n);

/* Smallest fp16 value >= v (v >= 0), as bits. */
uint16_t mg_fp16_ceil_bits(double v);

/* Covering encoders: one block from 256 (Q4_K, Q5_K, Q6_K) or 32 (MXFP4) fp32 values. */
void mg_encode_q4k(const float* x, uint8_t* blk);
void mg_encode_q5k(const float* x, uint8_t* blk);
void mg_encode_q2k(const float* x, uint8_t* blk);
void mg_encode_q6k(const float* x, uint8_t* blk);
void mg_encode_mxfp4(const float* x, uint8_t* blk);
void mg_encode_q3k(const float* x, uint8_t* blk);
void mg_encode_q40(const float* x, uint8_t* blk);
void mg_encode_q51(const float* x, uint8_t* blk);
/* Encode a [rows x K] fp32 matrix into block rows at byte stride `stride`
 * (padding bytes are zeroed). K must be a multiple of the block size. */
void mg_encode_matrix(int fmt, const float* x, int rows, int K, size_t stride, uint8_t* out,
                      int threads);

/* Pack explicit fields into one block (for hand-built test blocks).
 * q4k: sc[8], m[8] in 0..63, q[256] in 0..15.
 * q6k: sc[16] int8, q[256] in 0..63.
 * mxfp4: e = E8M0 byte, codes[32] in 0..15. */
void mg_pack_q4k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk);
void mg_pack_q6k(uint16_t d_bits, const int8_t* sc, const uint8_t* q, uint8_t* blk);
/* q2k: sc[16], m[16] in 0..15, q[256] in 0..3. */
void mg_pack_q2k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk);
/* q5k: as q4k with q[256] in 0..31. */
void mg_pack_q5k(uint16_t d_bits, uint16_t dmin_bits, const uint8_t* sc, const uint8_t* m,
                 const uint8_t* q, uint8_t* blk);
void mg_pack_mxfp4(uint8_t e, const uint8_t* codes, uint8_t* blk);
void mg_pack_q3k(uint16_t d_bits, const uint8_t* sc, const int8_t* q, uint8_t* blk);
void mg_pack_q40(uint16_t d_bits, const uint8_t* q, uint8_t* blk);
void mg_pack_q51(uint16_t d_bits, uint16_t m_bits, const uint8_t* q, uint8_t* blk);

size_t mg_block_bytes(int fmt);
int mg_block_elems(int fmt);

/* Generate one quantized weight matrix directly (normals -> blocks), row-parallel.
 * Rows use streams (seed, tensor, expert, r). */
void mg_weight_matrix(uint64_t seed, uint32_t tensor, uint32_t expert, int fmt, int rows, int K,
                      size_t stride, double std_, uint8_t* out, int threads);

/* Zipf(s) selection bias over a seeded permutation of E experts:
 * b[perm[r]] = log(p_r), p_r proportional to (r+1)^-s. */
void mg_zipf_bias(uint64_t seed, int E, double s, float* out);

#ifdef __cplusplus
}
#endif
#endif
