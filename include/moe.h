/*
 * moe.h — C ABI of the routed-expert MoE FFN layer for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer, per token t of a chunk of T tokens:
 *   1. x[t] is quantized per block to int8 with one fp32 scale (q8 activations).
 *   2. A router scores all E experts, top-k picks k of them (ties go to the
 *      lower expert index) and gives them routing weights (softmax or sigmoid).
 *   3. Each selected expert's block-quantized gate/up rows are integer dot
 *      products with q8(x), rescaled per quant block; SwiGLU gives h, which is
 *      re-quantized to q8 and multiplied by the expert's down rows the same way.
 *   4. y[t] = sum over the k slots of weight * expert output, plus an optional
 *      always-on shared expert.
 * Sources: the Pulsar README (model list: routers and experts of the supported
 * families; numerics notes: activations quantized to q8_0/q8_K with integer
 * dots; MoE expert resolve: launches get explicit per-expert gate/up/down
 * device pointers and a NULL one means "not mine"; prefill notes: grouped
 * int8 tensor-core MoE that rescales per quant block). Block layouts follow the
 * ggml/GGUF conventions for Q4_K (144 B / 256 weights), Q6_K (210 B / 256) and
 * OCP MX v1.0 for MXFP4 (17 B / 32).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; descriptors
 *    and moe_qact structs are HOST structs read during the call only.
 *  - Work is enqueued on the caller's stream and nothing else: no allocation,
 *    no host synchronization, no device-to-host copy. Calls can be captured
 *    into a HIP graph. Results are valid once the stream has synchronized.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and the status says why. A failed kernel launch
 *    returns MOE_EHIP. No C++ exception crosses this boundary.
 *  - The library keeps no global mutable state; calls are reentrant. Two calls
 *    that share a workspace must be ordered on one stream.
 *  - Same inputs on the same path give the same bytes (no float atomics).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_ABI_VERSION 5
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,         /* bad argument: NULL, shape, stride, alignment, enum */
  MOE_EUNSUPPORTED = 2,   /* valid but not implemented combination */
  MOE_ENOWORKSPACE = 3,   /* workspace smaller than moe_workspace_size() */
  MOE_EHIP = 4            /* a HIP launch failed */
} moe_status;

/* Stored weight block formats (GGUF block layouts; MXFP4 as OCP MX v1.0):
 * Q4_K 144 B / 256 weights, Q6_K 210 B / 256, MXFP4 17 B / 32, Q5_K 176 B / 256
 * (Q4_K's fp16 d, dmin and 6-bit scales, 32 B of fifth bits, 128 B of nibbles),
 * Q2_K 84 B / 256 (16 scale/min nibble pairs, 64 B of 2-bit quants, fp16 d,
 * dmin), Q3_K 110 B / 256 (32 B of high bits, 64 B of 2-bit quants, 12 B of
 * 6-bit scales, fp16 d), Q4_0 18 B / 32 (fp16 d, 16 B of nibbles) and Q5_1
 * 24 B / 32 (fp16 d and m, 32 fifth bits, 16 B of nibbles). Layers with a
 * matrix in any format other than Q4_K and Q6_K take the per-(token, slot)
 * GEMV path for every T. */
typedef enum {
  MOE_WFMT_Q4_K = 0,
  MOE_WFMT_Q6_K = 1,
  MOE_WFMT_MXFP4 = 2,
  MOE_WFMT_Q5_K = 3,
  MOE_WFMT_Q2_K = 4,
  MOE_WFMT_Q3_K = 5,
  MOE_WFMT_Q4_0 = 6,
  MOE_WFMT_Q5_1 = 7
} moe_wfmt;
/* Activation quant formats: Q8_K = blocks of 256 with 16-element sums
 * (consumed by Q4_K, Q5_K, Q2_K, Q3_K and Q6_K rows); Q8_32 = blocks of 32
 * (MXFP4, Q4_0 and Q5_1 rows); MXFP8 = OCP MX v1.0 blocks of 32 E4M3 values
 * with one E8M0 scale (MXFP4 rows of layers with act_quant = MXFP8). */
typedef enum { MOE_AFMT_Q8_K = 0, MOE_AFMT_Q8_32 = 1, MOE_AFMT_MXFP8 = 2 } moe_afmt;
/* Activation numerics of a layer (which quantization x and h get before the
 * expert rows). Q8: q8_K / q8_32 by weight format, integer block dots (Pulsar
 * README, numerics notes). MXFP8: MXFP4 experts only, x and h quantized per
 * block of 32 to MXFP8 (shared exponent floor(log2 amax) - 8, E4M3 elements
 * rounded to nearest-even and saturated at 448) and multiplied on the
 * block-scaled MFMA path at every T (memra ARCHITECTURE.md, §0 item 3 and the
 * §2 ledger row on MXFP4 / block-scale mma). */
typedef enum { MOE_ACTQ_Q8 = 0, MOE_ACTQ_MXFP8 = 1 } moe_actq;
typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;
typedef enum { MOE_ROUTER_SOFTMAX = 0, MOE_ROUTER_SIGMOID = 1 } moe_router;
/* SWIGLU: h = silu(g) * u. SWIGLU_OAI (gpt-oss): g' = min(g, limit),
 * u' = clamp(u, -limit, limit), h = g' * sigmoid(alpha * g') * (u' + 1). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SWIGLU_OAI = 1 } moe_act;
/* Expert-FFN path of a chunk. AUTO: layers with a matrix in a format without
 * tile kernels (all but Q4_K and Q6_K) take the per-(token, slot) GEMV path; the
 * others take the expert-grouped int8-MFMA path when one expert's block bytes
 * reach 8 MB, or when T * (k + shared) * (block bytes of one expert) reaches
 * 160 MB, or when the GEMV kernels do not take the shape (LDS budget), else
 * the GEMV path (the measured crossover: the grouped path reads
 * each selected expert once per 16 tokens at the cost of more launches, and
 * streams large experts faster even for one token). GEMV and GROUPED force a
 * path (GROUPED only where the formats allow it). */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GROUPED = 2 } moe_path;
/* Order of the blocks of every expert matrix of a layer (gate, up, down and the
 * shared expert's). The blocks themselves are the stored format's; only their
 * order differs.
 *  ROWS: row r of a matrix at r * stride, its blocks in order along the row
 *    (the GGUF tensor order).
 *  TILE64: rows form tiles of 64, and tile i holds super-block 0 of its 64
 *    rows (row 64 i first), then their super-block 1, and so on: block b of
 *    row r of a matrix with nb blocks per row sits at byte
 *    ((r / 64) * nb + b) * 64 * BB + (r % 64) * BB (BB: block bytes), and the
 *    stride fields are not used. One stage of the grouped tile kernels (one
 *    super-block of 64 or 128 rows) is then a single contiguous read instead of
 *    a block from each of 64 rows. Needs Q4_K gate and up, Q4_K or Q6_K down,
 *    no biases, Q8 activations and a path other than GEMV (MOE_EUNSUPPORTED
 *    otherwise); such layers take the grouped path at every T.
 *    moe_repack_tile64 converts a matrix from ROWS order.
 *  MX16: MXFP4 rows with the fields of their 17-byte blocks regrouped: row r
 *    at r * stride holds the 16 nibble bytes of block b at byte 16 b (the
 *    block's bytes 1..16, unchanged) and, after all of them, the scale byte of
 *    block b at byte 16 nb + b (nb = blocks per row); the scale run is read as
 *    whole dwords, so strides must reach 16 nb + nb rounded up to 4. Every
 *    field is aligned, so the per-pair GEMV kernels load each block straight
 *    into registers instead of realigning 17-byte blocks. Needs MXFP4 gate, up
 *    and down, Q8 activations, a path other than GROUPED, and widths the
 *    per-pair MXFP4 kernels take (up to 256 blocks per row within their LDS
 *    budget) (MOE_EUNSUPPORTED otherwise); such layers take the GEMV path at
 *    every T. moe_repack_mx16 converts a matrix from ROWS order. */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILE64 = 1, MOE_LAYOUT_MX16 = 2 } moe_layout;

/* Quantized activations of T rows of width H, structure-of-arrays:
 *   qs    int8  [T, H]      q8 quants, |q| <= 127 (Q8_K, Q8_32); MXFP8: E4M3
 *                           codes, each block of 32 pair-interleaved (byte 2j =
 *                           element j, byte 2j + 1 = element j + 16, the pairing
 *                           of an MXFP4 block's nibble bytes)
 *   d     fp32  [T, H / B]  q8 per-block scale (B = 256 for Q8_K, 32 for Q8_32),
 *                           a = d * q; NULL for MXFP8
 *   bsums int16 [T, H / 16] sum of the quants of each 16 elements (Q8_K only)
 *   scales uint8 [T, S]     MXFP8 only: E8M0 block scales, rows padded to
 *                           S = 16 * ceil(H / 512) bytes; a = 2^(s - 127) e4m3(q)
 * Device pointers, 16-byte aligned. */
typedef struct {
  int8_t* qs;
  float* d;
  int16_t* bsums;
  int32_t fmt; /* moe_afmt */
  int32_t T;
  int32_t H;
  uint8_t* scales;
} moe_qact;

/* One MoE layer. Host struct; every pointer in it is a device pointer.
 *  hidden (H), ffn (F): H and F must be multiples of the block size of the
 *    formats that consume them (256 for Q4_K/Q6_K, 32 for MXFP4).
 *  n_expert (E) in [1, MOE_MAX_EXPERTS], top_k (k) in [1, min(E, MOE_MAX_TOPK)].
 *  router, norm_topk: SOFTMAX with norm_topk = 1 is the softmax over the k
 *    selected logits; norm_topk = 0 is the softmax over all E evaluated at the
 *    selected experts. SIGMOID: sigmoid of the selected logits, divided by
 *    their sum when norm_topk = 1. Weights are then multiplied by route_scale.
 *  w_router fp32 [E, H] row-major. Logits are accumulated in fp64 and rounded
 *    once to fp32.
 *  sel_bias fp32 [E] or NULL: added (one fp32 add) to the logits for selection
 *    only; routing weights use the unbiased logits.
 *  fmt_* / stride_*: weight format and row stride in bytes of the gate and up
 *    matrices ([F rows of H]) and of down ([H rows of F]). Rows are contiguous
 *    block streams; stride >= row bytes, stride % 16 == 0, and each matrix
 *    spans rows * stride bytes (rows are read in whole 16-byte pieces, up to
 *    the next multiple of 16 past a row's last block). gate and up must have
 *    the same format.
 *  gate, up, down: device arrays of E device pointers to each expert's
 *    matrices (16-byte aligned). gate[e] == NULL means expert e is not present
 *    here: its slots contribute nothing and the other weights are not
 *    renormalized. When gate[e] != NULL, up[e] and down[e] must be valid.
 *  b_gate, b_up ([F]) and b_down ([H]): NULL, or device arrays of E device
 *    pointers to fp32 biases. Gate/up biases are added before the activation,
 *    the down bias to the expert output before the routing weight.
 *  act, act_alpha, act_limit: moe_act and its constants.
 *  sh_gate, sh_up, sh_down: the shared expert (same formats, strides and
 *    shape as the routed experts) or all NULL. sh_gate_vec fp32 [H] or NULL:
 *    shared-expert weight sigmoid(sh_gate_vec . x), or 1 when NULL.
 *  path: moe_path (0 = AUTO).
 *  act_quant: moe_actq (0 = Q8). MXFP8 needs MXFP4 gate, up and down and a
 *    path other than GEMV (MOE_EUNSUPPORTED otherwise).
 *  layout: moe_layout (0 = ROWS) of every expert matrix.
 */
typedef struct {
  int32_t hidden;
  int32_t ffn;
  int32_t n_expert;
  int32_t top_k;
  int32_t router;
  int32_t norm_topk;
  float route_scale;
  const float* w_router;
  const float* sel_bias;
  int32_t fmt_gate, fmt_up, fmt_down;
  size_t stride_gate, stride_up, stride_down;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const float* const* b_gate;
  const float* const* b_up;
  const float* const* b_down;
  int32_t act;
  float act_alpha;
  float act_limit;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
  const float* sh_gate_vec;
  int32_t path;
  int32_t act_quant;
  int32_t layout;
} moe_layer_desc;

/* ABI version (MOE_ABI_VERSION) and a static message for a status. */
MOE_API int moe_abi_version(void);
MOE_API const char* moe_status_str(moe_status s);

/* Bytes of device workspace (256-byte aligned base) that moe_route_topk,
 * moe_expert_ffn and moe_layer_forward need for T tokens of this layer.
 * Returns 0 if the descriptor or T is invalid. A valid layer whose expert FFN
 * no kernel takes (a per-pair shape past the GEMV kernels' LDS budget, in
 * formats without tile kernels) still gets its size: routing works, and
 * moe_expert_ffn / moe_layer_forward return MOE_EUNSUPPORTED. The workspace is
 * scratch: its contents on entry do not matter. */
MOE_API size_t moe_workspace_size(const moe_layer_desc* desc, int T);

/* Activation quantization. x: device [T, H] fp32 or bf16 (bf16 is upcast
 * exactly). Per block of B values: amax = max |x|; amax == 0 gives d = 0 and
 * q = 0; otherwise iscale = 127/amax, q = clamp(rne(x * iscale), -127, 127) and
 * d = amax/127, every step in IEEE fp32. MXFP8 (H % 32 == 0): per block of 32,
 * scale byte s = floor(log2 amax) - 8 + 127 within [0, 254] (0 for amax 0) and
 * codes rne_e4m3(x / 2^(s - 127)) saturated at +-448, zero as +0, stored
 * pair-interleaved (see moe_qact). out: host struct whose qs, d (and bsums for
 * Q8_K; scales for MXFP8) point to caller device buffers; fmt, T and H are
 * filled in. Sources: Pulsar README, numerics notes (activations quantized to
 * q8_0/q8_K); OCP MX v1.0 §6.3 for MXFP8. */
MOE_API moe_status moe_quantize_act_q8k(const void* x, moe_dtype dtype, int T, int H, moe_afmt fmt,
                                moe_qact* out, hipStream_t stream);

/* Router + top-k. x: device [T, H] (fp32 or bf16). Writes ids int32 [T, k]
 * (experts in rank order: key descending, index ascending on ties, where key is
 * the fp32 logit, plus sel_bias if set, with -0 treated as +0), w fp32 [T, k]
 * routing weights, and logits fp32 [T, E] if non-NULL. ws: workspace of at
 * least moe_workspace_size(desc, T) bytes.
 * Source: Pulsar README, model list (softmax routers of qwen3moe/gpt-oss,
 * sigmoid-gated routers with shared experts of the deepseek/qwen35 families). */
MOE_API moe_status moe_route_topk(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                          int32_t* ids, float* w, float* logits, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Expert FFN for given routing. xq: q8 of x in the format the gate/up rows
 * consume (Q8_K for Q4_K/Q6_K, Q8_32 for MXFP4). x: the unquantized input, only
 * read when sh_gate_vec is set (else may be NULL). ids int32 [T, k], w fp32
 * [T, k] device arrays (ids must lie in [0, E)). y fp32 [T, H] is overwritten.
 * Source: Pulsar README, MoE expert resolve and numerics notes. */
MOE_API moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_qact* xq, const void* x,
                          moe_dtype dtype, int T, const int32_t* ids, const float* w, float* y,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer: quantize, route, expert FFN. y fp32 [T, H] overwritten;
 * ids_out [T, k] and w_out [T, k] are optional copies of the routing (device,
 * int32 / fp32, or NULL). ws: workspace of at least moe_workspace_size(desc, T)
 * bytes, 256-byte aligned, caller-owned; its contents on entry do not matter.
 * The routing never leaves the device: the selected experts' pointers are
 * resolved in the kernels, so the call is one enqueue with no readback.
 * Errors: as above (MOE_EINVAL, MOE_EUNSUPPORTED when a launch shape does not
 * fit the kernels, MOE_ENOWORKSPACE, MOE_EHIP), nothing enqueued on failure.
 * Source: Pulsar README, MoE expert resolve (per-token router ids pick the
 * experts whose gate/up/down pointers the launch gets; NULL = "not mine") and
 * numerics notes (q8_K activations, integer dots); the DGX Spark article on
 * running Kimi K3 with Pulsar (router readbacks and per-layer launches as the
 * fixed cost of a token). */
MOE_API moe_status moe_layer_forward(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                             float* y, int32_t* ids_out, float* w_out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, with the workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends. The caller passes inputs and outputs only.
 * Returns MOE_ENOWORKSPACE, with nothing enqueued, when
 * moe_workspace_size(desc, T) exceeds that size (32 MiB covers up to 64 tokens
 * of the Kimi-K2-shaped layer; larger chunks need moe_layer_forward and a
 * caller workspace). It calls no allocation routine; the first call on a
 * device looks the array's address up once. All calls on one GPU share its
 * array: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be serialized by the caller. Other arguments and
 * errors as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
MOE_API moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* x,
                                     moe_dtype dtype, int T, float* y, int32_t* ids_out,
                                     float* w_out, hipStream_t stream);

/* moe_layer_forward with timing hooks: events holds n_events HIP events (may
 * be NULL); kernel i of the call records events[2i] when it starts and
 * events[2i + 1] when it ends (hipExtLaunchKernel start/stop events), for the
 * pairs that fit in n_events. moe_layer_stage_count() gives how many kernels
 * the call launches and moe_layer_stage_name() names them. */
MOE_API moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const void* x, moe_dtype dtype,
                                   int T, float* y, int32_t* ids_out, float* w_out, void* ws,
                                   size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                                   int n_events);
MOE_API int moe_layer_stage_count(const moe_layer_desc* desc, int T);
MOE_API const char* moe_layer_stage_name(const moe_layer_desc* desc, int T, int stage);

/* Reorders one expert matrix from ROWS to TILE64 order (moe_layout): n_rows
 * rows of K weights in format fmt (Q4_K or Q6_K), row r at src + r * src_stride,
 * into n_rows * (K / 256) * BB bytes at dst. Whole blocks move; no byte of a
 * block changes. Needs n_rows % 64 == 0, K % 256 == 0, src_stride >= the row's
 * bytes and even, src and dst 16-byte aligned and not overlapping (MOE_EINVAL
 * otherwise); a failed launch gives MOE_EHIP. Enqueued on stream; the caller
 * owns both buffers. Source: Pulsar README, formats paragraph (routed experts
 * as stored GGUF quant blocks); the order of the blocks in device memory is
 * this library's choice. */
MOE_API moe_status moe_repack_tile64(moe_wfmt fmt, const void* src, size_t src_stride, int n_rows,
                                     int K, void* dst, hipStream_t stream);

/* Reorders one MXFP4 matrix from ROWS to MX16 order (moe_layout): n_rows rows
 * of K weights (K % 32 == 0), row r at src + r * src_stride (>= 17 K / 32),
 * into rows at dst + r * dst_stride (dst_stride a multiple of 16 and at least
 * 16 nb + nb rounded up to 4, nb = K / 32). Only the order of each block's
 * bytes changes (nibble fields first, then the scale bytes); the bytes past
 * the scale run up to the next multiple of 4 are written as zero, the rest of
 * each dst row is not touched. src and dst 16-byte aligned and not
 * overlapping (MOE_EINVAL otherwise); a failed launch gives MOE_EHIP. Enqueued
 * on stream; the caller owns both buffers. Source: Pulsar README, formats
 * paragraph (MXFP4 routed experts as stored quant blocks); the order of the
 * fields in device memory is this library's choice. */
MOE_API moe_status moe_repack_mx16(const void* src, size_t src_stride, int n_rows, int K, void* dst,
                                   size_t dst_stride, hipStream_t stream);

/* Test export: integer block partials of n_rows weight rows (device, K
 * columns, byte stride `stride`) against token `token` of xq, computed by the
 * same device routines the FFN kernels use (MXFP4 rows of up to 256 blocks:
 * the realigning routine of the MXFP4 GEMV kernels; longer rows: the per-block
 * routine). out int32 [n_rows, K / Bw, 2] (device):
 *   Q4_K, Q5_K, Q2_K: (S1, S2) with S1 = sum_j sc_j * dot_j, S2 = sum_j m_j * (activation sums of sub-block j)
 *   Q6_K : (S, 0)   with S  = sum_s sc_s * sum_i (q_i - 32) * a_i
 *   MXFP4: (S, 0)   with S  = sum_i (2 * e2m1_i) * a_i
 *   Q3_K : (S, 0)   with S  = sum_s (sc_s - 32) * sum_i q_i * a_i, q in -4..3
 *   Q4_0 : (S, 0)   with S  = sum_i (q_i - 8) * a_i
 *   Q5_1 : (S1, S2) with S1 = sum_i q_i * a_i, S2 = sum_i a_i
 * Errors: MOE_EINVAL for a bad format, pointer, width, stride or token.
 * Source: Pulsar README, numerics notes (activations quantized to q8_0/q8_K,
 * integer dp4a dots, rescaled per quant block). */
MOE_API moe_status moe_test_block_dots(moe_wfmt fmt, const void* rows, int n_rows, int K, size_t stride,
                               const moe_qact* xq, int token, int32_t* out, hipStream_t stream);

/* Test export: the same partials (S = 2 dot, 0) for MXFP4 rows in the MX16
 * order (row stride >= 16 nb + nb rounded up to 4, a multiple of 16; K / 32 <=
 * 256), through the loads and dots of the MX16 GEMV kernels. xq: Q8_32.
 * Errors: MOE_EINVAL for a bad pointer, width, stride or token;
 * MOE_EUNSUPPORTED past 256 blocks per row. Source: Pulsar README, numerics
 * notes (integer dots rescaled per quant block). */
MOE_API moe_status moe_test_block_dots_mx16(const void* rows, int n_rows, int K, size_t stride,
                                            const moe_qact* xq, int token, int32_t* out,
                                            hipStream_t stream);

/* Test export: the integer super-block sums of the multi-token path's int8
 * MFMA tile kernels, computed by their production bodies (LDS ring, MFMA
 * tiles) on one tile of n_tok (1..16) activation rows (tokens 0..n_tok-1 of
 * xq, Q8_K, width K % 256 == 0) against n_rows weight rows (device, byte
 * stride `stride`):
 *   mode 0: Q4_K gate/up body, the rows serving as both the gate and the up
 *           matrix, n_rows % 64 == 0: out int32 [2][n_tok][n_rows][K/256] = S1
 *   mode 1: Q4_K down body, n_rows % 128 == 0: out [n_tok][n_rows][K/256] = S1
 *   mode 2: Q6_K down body, n_rows % 64 == 0:  out [n_tok][n_rows][K/256] = S
 * with S1 and S as in moe_test_block_dots. ws: device scratch of at least
 * moe_test_tile_dots_ws(mode, n_rows, K, n_tok) bytes, 256-byte aligned.
 * Errors: MOE_EINVAL, MOE_ENOWORKSPACE. Source: Pulsar README, prefill notes
 * (grouped int8 tensor-core MoE that rescales per quant block). */
MOE_API moe_status moe_test_tile_dots(int mode, const void* rows, int n_rows, int K, size_t stride,
                              const moe_qact* xq, int n_tok, int32_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream);
MOE_API size_t moe_test_tile_dots_ws(int mode, int n_rows, int K, int n_tok);

/* Test export: the gate (which = 0) or up (which = 1) pre-activations, bias
 * included, that moe_expert_ffn's gate/up stage computes for the given routing
 * (ids int32 [T, k]), by the same kernels and path (per-pair GEMV or
 * expert-grouped MFMA tiles) with the activation replaced by the identity.
 * out fp32 [T * k + T * (shared expert ? 1 : 0), F] (device): row t k + s for
 * token t, slot s, then the shared expert's rows; rows of absent experts are
 * left untouched. Other arguments and errors as moe_expert_ffn.
 * Source: Pulsar README, numerics notes (integer dots rescaled per quant block). */
MOE_API moe_status moe_test_preact(const moe_layer_desc* desc, const moe_qact* xq, int T,
                           const int32_t* ids, int which, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* Measurement probes (not part of the layer): ceilings measured on the chip
 * that runs the layer, reported beside the datasheet peaks. Source: the memra
 * architecture plan, header (a measured memory-read wall stated beside the
 * peak bandwidth).
 * moe_probe_read_wall: reads `bytes` (a multiple of 16) of the device buffer
 * buf (16-byte aligned) once, as non-temporal 16-byte loads from nwg
 * workgroups of 256 threads, eight loads in flight per thread. sink: one
 * device uint32 that is written only in a practically impossible case (it
 * keeps the loads live). Time it with events on `stream`.
 * moe_probe_mfma_i8: nwg workgroups of four waves; every wave issues `iters`
 * rounds of eight independent int8 MFMAs (k64 = 0: 16x16x32, the shape the
 * tile kernels use; 1: 16x16x64). int8 operations per launch:
 * nwg * 4 * iters * 8 * 16 * 16 * (k64 ? 64 : 32) * 2. sink as above.
 * Errors: MOE_EINVAL for a bad pointer, size or count; MOE_EHIP. */
MOE_API moe_status moe_probe_read_wall(const void* buf, size_t bytes, int nwg, uint32_t* sink,
                               hipStream_t stream);
/* moe_probe_empty_chain: n (1..4096) launches of an empty kernel back to back
 * on `stream`: the launch-chain floor of a layer call with that many kernels
 * (time it with events, or capture it in a graph as the layer calls are). */
MOE_API moe_status moe_probe_empty_chain(int n, hipStream_t stream);
MOE_API moe_status moe_probe_mfma_i8(int k64, int iters, int nwg, int32_t* sink,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
