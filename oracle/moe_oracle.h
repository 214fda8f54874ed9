/*
 * moe_oracle — plain, slow, single-threaded CPU reference of the routed-expert
 * MoE FFN layer, in fp64. TEST INFRASTRUCTURE ONLY: it is used by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg, and by
 * nothing on the product path. It shares no code with the HIP library.
 *
 * What is computed (sources: the Pulsar README — model list, "expert resolve"
 * and numerics notes; the DGX Spark article on running Kimi K3 with Pulsar):
 *   1. Activations are quantized per block to int8 with one fp32 scale
 *      (q8_K: blocks of 256 with 16-element sums; q8_32: blocks of 32).
 *   2. A router scores every expert (fp32 weights, fp64 accumulation, one fp32
 *      rounding), top-k picks k experts (ties to the lowest index), and the k
 *      weights come from a softmax or a sigmoid over the selected logits.
 *   3. For each selected expert, gate/up rows are integer dot products of the
 *      stored weight quants with the activation quants, rescaled per quant
 *      block; SwiGLU (or the clamped gpt-oss variant) gives h, which is
 *      re-quantized to int8 and multiplied by the down rows the same way.
 *   4. The expert outputs are summed with the routing weights, plus an
 *      always-on shared expert (weight 1, or a sigmoid gate).
 * A NULL expert pointer means "not present here": that slot adds nothing and
 * the remaining weights are not renormalized.
 *
 * Block layouts are the ggml/GGUF conventions (the pages name the formats
 * only): Q4_K 144 B / 256, Q6_K 210 B / 256, MXFP4 17 B / 32 (OCP MX v1.0);
 * further formats the pages list: Q5_K 176 B, Q2_K 84 B, Q3_K 110 B (256
 * weights), Q4_0 18 B, Q5_1 24 B (32 weights). Rows of 32-weight formats
 * consume q8 activations in blocks of 32, the others in blocks of 256.
 * GGUF byte-level interoperability is parity unpinned: no GGUF file or
 * reference decoder is available to check against.
 *
 * MXFP8 activation mode (act_quant = OR_ACTQ_MXFP8, MXFP4 layers only): the
 * numerics of a block-scaled MX matrix path (memra ARCHITECTURE.md, §0 item 3
 * and the §2 ledger row on MXFP4 / block-scale mma). x and h are quantized per
 * block of 32 to OCP MX v1.0 MXFP8 (E4M3 elements, one E8M0 scale; the
 * shared-scale rule of the MX spec, §6.3) instead of q8, and every block dot
 * is the exact fp64 value 2^(ew-127) 2^(ea-127) sum_i e2m1(w_i) e4m3(a_i).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_Q4_K = 0, OR_Q6_K = 1, OR_MXFP4 = 2, OR_Q5_K = 3, OR_Q2_K = 4, OR_Q3_K = 5,
       OR_Q4_0 = 6, OR_Q5_1 = 7 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };
enum { OR_SWIGLU = 0, OR_SWIGLU_OAI = 1 };
enum { OR_ACTQ_Q8 = 0, OR_ACTQ_MXFP8 = 1 };

/* ---- scalar decoders ---- */
double or_fp16(uint16_t bits);      /* IEEE binary16 -> double */
double or_e8m0(uint8_t e);          /* 2^(e - 127) */
double or_e2m1(uint8_t code);       /* OCP FP4 E2M1 value of a 4-bit code */
double or_e4m3(uint8_t code);       /* OCP FP8 E4M3 value of a byte (NaN for 0x7F, 0xFF) */
/* The finite E4M3 code nearest to v (ties to the even code), saturating at
 * +-448; a result of magnitude zero is +0 (code 0x00). */
uint8_t or_e4m3_round(double v);

/* ---- block formats ---- */
int or_block_elems(int fmt);
int or_block_bytes(int fmt);
/* q8 block size of the activations that rows of this format consume (32 or 256). */
int or_act_block(int fmt);
/* Raw integer quants of one block: Q4_K 0..15, Q5_K 0..31, Q6_K 0..63, Q2_K 0..3,
 * Q3_K -4..3, Q4_0 0..15, Q5_1 0..31, MXFP4 2*e2m1 (signed). */
void or_block_quants(int fmt, const uint8_t* blk, int32_t* q);
/* Dequantize one block / one row of K values to fp64. */
void or_dequant_block(int fmt, const uint8_t* blk, double* out);
void or_dequant_row(int fmt, const uint8_t* row, int K, double* out);

/* ---- activation quantization (fp32 recipe) ----
 * Per block of B (256 or 32): amax = max |x|; amax == 0 -> d = 0, q = 0;
 * else iscale = 127/amax, q = clamp(rne(x*iscale), -127, 127), d = amax/127,
 * all in IEEE fp32. bsums (B = 256 only, may be NULL) = sum of q over each 16. */
void or_quantize_q8(const float* x, int n, int B, int8_t* qs, float* d, int16_t* bsums);

/* ---- MXFP8 activation quantization (OCP MX v1.0, §6.3) ----
 * Per block of 32: amax = max |x| (fp32); amax == 0 -> scale byte 0 and all
 * codes 0; else the shared exponent is floor(log2(amax)) - 8 (8 = E4M3's
 * largest normal exponent), scale byte e = shared + 127 clamped to [0, 254],
 * and code_i = or_e4m3_round(x_i / 2^(e - 127)). q[n] codes, e[n / 32]. */
void or_quantize_mx8(const float* x, int n, uint8_t* q, uint8_t* e);
/* Exact fp64 dot of one MXFP4 row (K values) with MXFP8 activations. */
double or_row_dot_mx8(const uint8_t* row, int K, const uint8_t* q, const uint8_t* e);

/* ---- integer block partials of one weight row against q8 activations ----
 * out[2b], out[2b+1] for block b:
 *   Q4_K : S1 = sum_j sc_j * dot_j,  S2 = sum_j m_j * (bsums[2j] + bsums[2j+1])
 *   Q6_K : S  = sum_s sc_s * (dot_s - 32 * bsums[s]),       second value 0
 *   MXFP4: S  = sum_i k_i * a_i with k = 2 * e2m1,          second value 0
 *   Q5_K and Q2_K as Q4_K (sub-blocks of 32 and 16)
 *   Q3_K : S  = sum_s (sc_s - 32) * dot_s (q in -4..3),     second value 0
 *   Q4_0 : S  = sum_i (q_i - 8) * a_i,                      second value 0
 *   Q5_1 : S1 = sum_i q_i * a_i,  S2 = sum_i a_i */
void or_block_partials(int fmt, const uint8_t* row, int K, const int8_t* qs,
                       const int16_t* bsums, int32_t* out);
/* fp64 value of one block from its partials and scales. */
double or_block_value(int fmt, const uint8_t* blk, const int32_t* partial, float d8);
/* Sum over the row's blocks of the block values (fp64). */
double or_row_dot(int fmt, const uint8_t* row, int K, const int8_t* qs, const float* d8,
                  const int16_t* bsums);

/* ---- router ---- */
void or_router_logits(const float* w_router, const float* x, int E, int H, float* logits);
void or_topk(const float* logits, const float* sel_bias, int E, int k, int32_t* ids);
void or_route_weights(const float* logits, const int32_t* ids, int E, int k, int router,
                      int norm_topk, double route_scale, double* w);

/* ---- layer ---- */
typedef struct {
  int H, F, E, k;
  int router, norm_topk;
  double route_scale;
  const float* w_router;                 /* [E, H] */
  const float* sel_bias;                 /* [E] or NULL */
  int fmt_gate, fmt_up, fmt_down;
  size_t stride_gate, stride_up, stride_down;
  const uint8_t* const* gate;            /* [E] pointers, NULL = expert not present */
  const uint8_t* const* up;
  const uint8_t* const* down;
  const float* const* b_gate;            /* [E] pointers to [F], or NULL */
  const float* const* b_up;              /* [E] pointers to [F], or NULL */
  const float* const* b_down;            /* [E] pointers to [H], or NULL */
  int act;
  double act_alpha, act_limit;
  const uint8_t* sh_gate;                /* shared expert, or NULL */
  const uint8_t* sh_up;
  const uint8_t* sh_down;
  const float* sh_gate_vec;              /* [H] or NULL (weight 1) */
  int act_quant;                         /* OR_ACTQ_Q8, or OR_ACTQ_MXFP8 (MXFP4 only) */
} or_layer;

/* Activation function on one (g, u) pair, fp64. */
double or_act(int act, double alpha, double limit, double g, double u);

/* One expert FFN on one token's q8 activations. Returns 0 if run.
 * out[H] fp64 (includes b_down); h32[F] fp32 h, optional. */
void or_expert_ffn(const or_layer* L, const uint8_t* gate, const uint8_t* up,
                   const uint8_t* down, const float* bg, const float* bu, const float* bd,
                   const int8_t* xq, const float* xd, const int16_t* xbs, double* out,
                   float* h32);

/* Whole layer for one token. x: [H] fp32 (bf16 inputs already upcast).
 * y[H] fp64; ids[k]; w[k] fp64; logits[E] fp32; h32 optional [(k+1) * F]
 * (slot k holds the shared expert's h). */
void or_layer_token(const or_layer* L, const float* x, double* y, int32_t* ids, double* w,
                    float* logits, float* h32);

/* Expert part only, with given ids and weights (fp32 w as the caller passes). */
void or_expert_part_token(const or_layer* L, const float* x, const int32_t* ids,
                          const float* w, double* y);

#ifdef __cplusplus
}
#endif
#endif
