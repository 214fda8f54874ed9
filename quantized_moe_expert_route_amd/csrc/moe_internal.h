// Internal interface between the C ABI (moe_api.cpp) and the HIP kernels
// (moe_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/moe.h"

namespace moe {

enum { FMT_Q4_K = 0, FMT_Q6_K = 1, FMT_MXFP4 = 2, FMT_Q5_K = 3, FMT_Q2_K = 4, FMT_Q3_K = 5,
       FMT_Q4_0 = 6, FMT_Q5_1 = 7 };

// Rows of 32-weight formats consume q8 activations in blocks of 32 (MXFP4 as
// fp16 pairs inside its kernels, Q4_0 and Q5_1 as int8); the others blocks of
// 256 with 16-element sums.
__host__ __device__ inline bool act32(int fmt) {
  return fmt == FMT_MXFP4 || fmt == FMT_Q4_0 || fmt == FMT_Q5_1;
}

// Activation codes beyond moe_act, used only by the test export of the gate/up
// pre-activations: the gate/up kernels then store g (or u) where h would go.
enum { ACT_PRE_GATE = 100, ACT_PRE_UP = 101 };

// Unsigned division by a runtime constant d >= 1 without a divide sequence
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): q = (umulhi(n, m) + n) >> s with
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1; exact for n < 2^31.
struct Div {
  uint32_t d, m, s;
  static Div make(uint32_t d_) {
    uint32_t sh = 0;
    while ((1ull << sh) < d_) ++sh;
    const uint64_t m64 = ((1ull << 32) * ((1ull << sh) - d_)) / d_ + 1;
    return Div{d_, static_cast<uint32_t>(m64), sh};
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> 32);
    return (hi + n) >> s;
  }
  __host__ __device__ __forceinline__ uint32_t mod(uint32_t n, uint32_t q) const {
    return n - q * d;
  }
};

// One token tile of the expert-grouped path: up to 16 (token, slot) pairs routed
// to one expert, with that expert's resolved pointers. Written by k_bucket.
struct GTile {
  int32_t e;      // expert id (E: the shared expert)
  int32_t start;  // first entry in the sorted pair list
  int32_t cnt;    // pairs in the tile, 1..16
  int32_t pad;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const float* b_gate;  // nullptr: no biases
  const float* b_up;
  const float* b_down;
};

// Down-projection pointers of one (token, slot) pair, resolved by k_gateup.
struct SlotRef {
  const uint8_t* down;  // nullptr: expert not present (slot contributes nothing)
  const float* bias;
};

// Everything a kernel may need, resolved on the host. Passed by value.
struct KArgs {
  int H, F, E, k, T;
  int router, norm_topk;
  float route_scale;
  const float* w_router;
  const float* sel_bias;
  int fmt_gu, fmt_d;
  size_t stride_gate, stride_up, stride_down;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const float* const* b_gate;
  const float* const* b_up;
  const float* const* b_down;
  int act;
  float act_alpha, act_limit;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
  const float* sh_gate_vec;
  int has_shared;
  // inputs / outputs / scratch (device)
  const void* x;
  int x_dtype;
  int8_t* xqs;      // [T, H]
  float* xd;        // [T, H / Bx]
  int16_t* xbs;     // [T, H / 16] (Q8_K) or nullptr
  float* logits;    // [T, E]
  int32_t* ids;     // [T, k]
  float* w;         // [T, k]
  float* shw;       // [T] shared-expert weight
  SlotRef* slots;   // [T, k]
  float* h;         // [P, F], P = T * k + T * has_shared
  float* y;         // [T, H]
  uint32_t* counters;  // one word per (token, slot) pair, reset by the router kernel
  // grouped path
  double* rpart;       // [KS, T, E1] router partial sums (E1 = E + shared gate row)
  int2* plist;         // [P] (pair, token), sorted by (expert, pair); shared expert last
  int32_t* present;    // [P] 1 if the pair's expert is present
  GTile* tiles;        // [max tiles]
  int8_t* hqs;         // [P, F] int8 (grouped); [P, F / 2] fp16 pairs (GEMV path, MXFP4 down)
  float* hd;           // [P, F / 256] (grouped); [P, F / 32] (GEMV path, MXFP4 down)
  int16_t* hbs;        // [P, F / 16]
  float* part;         // [P, H] routing-weighted expert outputs per pair
  // test export of the tile kernels' integer super-block sums (nullptr otherwise)
  int32_t* dump;
  // MXFP8 activation numerics (MXFP4 layers on the block-scaled MFMA path):
  // x codes in xqs and h codes in hqs (E4M3, pair-interleaved per block), their
  // E8M0 scale rows here (pitch mx8_pitch(K) bytes)
  int mx8;
  uint8_t* xe;         // [T, mx8_pitch(H)]
  uint8_t* he;         // [P, mx8_pitch(F)]
  // expert matrices in 64-row tiles, super-block-major inside a tile (block b
  // of row r at ((r / 64) nb + b) 64 BB + (r % 64) BB); strides unused
  int tiled;
  // MXFP4 rows in the MX16 order (nibble fields of all blocks, then the scale
  // bytes): read by the MX16 variants of k_gateup_mx and k_down_mx
  int mx16;
};

// Workspace layout (byte offsets from the base, each 256-aligned).
struct WsLayout {
  size_t counters, xqs, xd, xbs, logits, ids, w, shw, slots, h, hqs, hd, hbs, rpart, plist,
      present, tiles, part, xe, he, total;
};
WsLayout ws_layout(int H, int F, int E, int k, int T, int has_shared, bool grouped, bool mx8);

// Dynamic LDS a workgroup may use (bytes).
constexpr size_t kMaxLds = 64 * 1024;

// Largest chunk (tokens) of one call, and so at most kMaxTokens * MOE_MAX_TOPK
// routed (token, slot) pairs.
constexpr int kMaxTokens = 2048;

// Whether the GEMV kernels' LDS needs fit for this layer and chunk.
bool gemv_fits(const KArgs& a);
// GEMV path: whether the down projection takes h quantized once per pair by a
// kernel of its own (an MXFP4 down too large for the fused kernel, or MX16
// rows). Otherwise every down workgroup quantizes h itself, overlapped with
// its row stream.
bool gemv_hquant(int fmt_down, int F, int k, int has_shared, bool mx16);

// Whether the per-pair MXFP4 kernels (k_gateup_mx, k_down_mx) take this
// layer's gate/up and down rows: the widths their row plans cover, within the
// LDS budget. MX16 layers need both.
bool mx16_fits(const KArgs& a);
// Bytes an MXFP4 row of nb blocks spans in the MX16 order: the nibble fields,
// then the scale bytes, read as whole dwords.
__host__ __device__ inline size_t mx16_row_bytes(int nb) {
  return 16 * static_cast<size_t>(nb) + ((static_cast<size_t>(nb) + 3) & ~static_cast<size_t>(3));
}

// Which expert-FFN path a chunk of T tokens takes (fixed rule, see moe_api.cpp).
bool use_grouped(const moe_layer_desc* d, int T);

// Router split of the grouped path: K slices of `len` elements (multiple of 16).
struct RouterSplit { int ks, len; };
RouterSplit router_split(int T, int E1, int H);

// Upper bound on the tiles k_bucket can emit.
int max_tiles(int T, int k, int E, int has_shared);

// Optional per-kernel timing events, recorded by the dispatch itself
// (hipExtLaunchKernel start/stop), i.e. the kernel's execution window.
struct Ev {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launchers. Each returns hipSuccess or the launch error.
hipError_t launch_quant(const void* x, int dtype, int T, int H, int B, int8_t* qs, float* d,
                        int16_t* bs, hipStream_t s);
hipError_t launch_zero(uint32_t* p, int n, hipStream_t s, Ev ev);
hipError_t launch_shared_gate(const KArgs& a, hipStream_t s);
// Router logits; quant: also q8 of x; n_clear: counters to reset for k_gateup.
hipError_t launch_router(const KArgs& a, bool quant, int n_clear, hipStream_t s, Ev ev);
hipError_t launch_topk(const KArgs& a, hipStream_t s);
hipError_t launch_gateup(const KArgs& a, bool routing_given, hipStream_t s, Ev ev);
hipError_t launch_down(const KArgs& a, hipStream_t s, Ev ev);
hipError_t launch_hquant_pairs(const KArgs& a, hipStream_t s, Ev ev);
// grouped path
hipError_t launch_router_grouped(const KArgs& a, bool quant, RouterSplit rs, hipStream_t s, Ev ev);
hipError_t launch_topk_sum(const KArgs& a, RouterSplit rs, hipStream_t s, Ev ev);
hipError_t launch_bucket(const KArgs& a, hipStream_t s, Ev ev);
// One matrix (n_rows of nb blocks of BB bytes, row stride `stride`) from row
// order into 64-row tiles.
hipError_t launch_repack_tile64(const uint8_t* src, size_t stride, int n_rows, int nb, int BB,
                                uint8_t* dst, hipStream_t s);
// One MXFP4 matrix (n_rows of nb 17-byte blocks, row stride `stride`) into the
// MX16 order at dst (row stride dst_stride).
hipError_t launch_repack_mx16(const uint8_t* src, size_t stride, int n_rows, int nb, uint8_t* dst,
                              size_t dst_stride, hipStream_t s);
hipError_t launch_gateup_grouped(const KArgs& a, hipStream_t s, Ev ev);
hipError_t launch_hquant(const KArgs& a, hipStream_t s, Ev ev);
hipError_t launch_down_grouped(const KArgs& a, hipStream_t s, Ev ev);
hipError_t launch_combine(const KArgs& a, hipStream_t s, Ev ev);
// MX path (moe_mx.hip): bytes per row of MXFP8 scales of a row of width K (K /
// 32 rounded up to a multiple of 16); standalone MXFP8 quantization, tile
// kernels and h quantization.
__host__ __device__ inline int mx8_pitch(int K) { return ((K / 32 + 15) / 16) * 16; }
hipError_t launch_quant_mx8(const void* x, int dtype, int T, int H, uint8_t* q, uint8_t* e,
                            hipStream_t s, Ev ev);
hipError_t launch_gateup_mx(const KArgs& a, int max_tiles, hipStream_t s, Ev ev);
hipError_t launch_hquant_mx8(const KArgs& a, hipStream_t s, Ev ev);
hipError_t launch_down_mx(const KArgs& a, int max_tiles, hipStream_t s, Ev ev);
hipError_t launch_block_dots(int fmt, const void* rows, int n_rows, int K, size_t stride,
                             const int8_t* qs, const float* d, const int16_t* bs,
                             int32_t* out, hipStream_t s);
// The same for MXFP4 rows in the MX16 order, through the MX16 kernels' routine.
hipError_t launch_block_dots_mx16(const void* rows, int n_rows, int K, size_t stride,
                                  const int8_t* qs, const float* d, int32_t* out, hipStream_t s);
// Test export: one token tile (n_tok <= 16 activation rows) through the grouped
// path's LDS-ring tile kernel of `mode` (0: Q4_K gate/up body, 1: Q4_K down
// body, 2: Q6_K down body), dumping the int32 super-block sums. ws >= tile_dots_ws().
size_t tile_dots_ws(int mode, int n_rows, int K, int n_tok);
// Measurement probes (moe_probe.hip).
hipError_t launch_read_wall(const void* buf, size_t bytes, uint32_t* sink, int nwg, hipStream_t s);
hipError_t launch_mfma_i8(int k64, int iters, int nwg, int32_t* sink, hipStream_t s);
hipError_t launch_empty_chain(int n, hipStream_t s);
hipError_t launch_tile_dots(int mode, const void* rows, int n_rows, int K, size_t stride,
                            const int8_t* qs, const float* d, const int16_t* bs, int n_tok,
                            int32_t* out, void* ws, hipStream_t s);

}  // namespace moe
