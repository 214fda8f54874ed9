// Expert-grouped HIP kernels of the routed-expert MoE FFN layer for gfx950,
// for chunks of several tokens (verify and prefill chunks) with K-quant experts.
//
// Each selected expert's weights are streamed once per 16-token tile instead of
// once per (token, slot) pair:
//   k_router_mfma   router GEMM [T, H] x [H, E] on fp64 MFMA (16x16x4), split
//                   over K slices into fp64 partials; extra waves quantize x
//   k_topk_sum      per token: the K-slice partials summed in slice order, one
//                   fp32 rounding, then top-k and routing weights
//   k_bucket        one workgroup: stable counting sort of the (token, slot)
//                   pairs by expert; tiles of <= 16 pairs with the expert's
//                   resolved pointers; presence flags
//   k_gu_grouped    per (tile, row block): gate and up rows against the
//                   tile's q8(x) rows, one int8 MFMA (16x16x32) per weight
//                   sub-block, integer sub-block scaling, fp32 block rescale;
//                   SwiGLU -> h
//   k_hquant        q8 of h per present pair (blocks of 256)
//   k_down_grouped  per (tile, row block of H): down rows against q8(h);
//                   bias and routing weight applied -> per-pair rows
//   k_combine       y[t] = per-pair rows summed in slot order, shared expert last
// The integer block partials are the same ones the decode path computes; only
// the fp32 order of the block rescale differs. No float atomics.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

using namespace dev;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename K, typename... Args>
hipError_t launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Ev ev,
                  Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, ev.start, ev.stop,
                          0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ long pk64(uint32_t lo, uint32_t hi) {
  return static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ uint2 ld8(const void* p) {
  const u32x2 v = *gp<u32x2>(p);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(gp<u32x2>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = *gp<u32x4>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 8 bytes at a 2-byte aligned address, cached (dword reads that each hold at
// least one byte of [p, p + 8), as load8_unaligned).
__device__ __forceinline__ uint2 ld8_a2(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(a & ~static_cast<uintptr_t>(3));
  const uint8_t* w_last = reinterpret_cast<const uint8_t*>((a + 7) & ~static_cast<uintptr_t>(3));
  const uint32_t sh = static_cast<uint32_t>(a & 3);
  const uint32_t w0 = *gp<uint32_t>(w), w1 = *gp<uint32_t>(w + 4), w2 = *gp<uint32_t>(w_last);
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}
__device__ __forceinline__ float4 ldg_f4(const void* p) {
  const v4f v = *gp<v4f>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}
// c + a * b with 24-bit signed operands (full-rate v_mad_i32_i24); every
// product here is a 6- or 8-bit scale times a sub-block dot of |.| < 2^17.
__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }
__device__ __forceinline__ v4i mma_i8(long a, long b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
}

// Lane roles in a 16x16 MFMA tile (wave64): g = lane / 16, c = lane % 16.
// int8 16x16x32 and fp32 16x16x4: A[row c][k in lane group g], B[k in g][col c],
// C[row 4g + i][col c] for i = 0..3. Rows are tokens, columns weight rows.
// fp64 16x16x4: A[row c][k g], B[k g][col c], C[row g + 4i][col c].

// q8 activations of one 256-element super-block as one lane feeds the MFMAs:
// q[m] holds elements 32m + 8g .. 32m + 8g + 7 of the lane's A-row token
// (group m is Q4_K sub-block m and Q6_K sub-blocks 2m, 2m + 1).
struct ActSB {
  uint2 q[8];
  uint32_t bs[2];  // two int16 16-element sums = sub-block 4h + g's sum (Q4_K)
  float dA;        // block scale of the A-row token
  float dC[4];     // block scales of the C-row tokens 4g + i
};

struct ActRows {
  const int8_t* qa;
  const int16_t* bsa;
  const float* da;
  const float* dc[4];
};

template <bool BS>
__device__ __forceinline__ void load_act(ActSB& r, const ActRows& x, int b, int g) {
  const int8_t* p = x.qa + 256 * b + 8 * g;
#pragma unroll
  for (int m = 0; m < 8; ++m) r.q[m] = ld8(p + 32 * m);
  if constexpr (BS) {
#pragma unroll
    for (int h = 0; h < 2; ++h) r.bs[h] = *gp<uint32_t>(x.bsa + 16 * b + 2 * (4 * h + g));
  }
  r.dA = *gp<float>(x.da + b);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.dC[i] = *gp<float>(x.dc[i] + b);
}

// ---- Q4_K: sub-block j of 32, w = d sc_j q - dmin m_j.
struct WQ4K {
  uint4 hdr;
  uint2 q[4];  // qs bytes 32c + 8g .. + 7: low nibbles sub-block 2c, high 2c + 1
  static constexpr bool kBS = true;
  __device__ __forceinline__ void load(const uint8_t* blk, int g) {
    hdr = ld16(blk);
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = ld8(blk + 16 + 32 * c + 8 * g);
  }
  // S[i] = S1 of C-row token 4g + i against this lane's weight row: the int32
  // sub-block dots (two int8 MFMAs per 32-weight group: low and high nibbles)
  // times the 6-bit scales sc_j, summed over the super-block.
  __device__ __forceinline__ v4i sums(const ActSB& x) const {
    const uint32_t s0 = hdr.y, s2 = hdr.w;
    const uint32_t sc03 = s0 & 0x3F3F3F3Fu;
    const uint32_t sc47 = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
    v4i S = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t lx = q[c].x, ly = q[c].y;
      const v4i clo = mma_i8(pk64(x.q[2 * c].x, x.q[2 * c].y),
                             pk64(lx & 0x0F0F0F0Fu, ly & 0x0F0F0F0Fu));
      const v4i chi = mma_i8(pk64(x.q[2 * c + 1].x, x.q[2 * c + 1].y),
                             pk64((lx >> 4) & 0x0F0F0F0Fu, (ly >> 4) & 0x0F0F0F0Fu));
      const uint32_t scw = c < 2 ? sc03 : sc47;
      const int sl = (scw >> (16 * (c & 1))) & 0xFF, sh = (scw >> (16 * (c & 1) + 8)) & 0xFF;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = mad24(sh, chi[i], mad24(sl, clo[i], S[i]));
    }
    return S;
  }
  // acc += dC * d * S1; mn += dA * bsum_j * dmin * m_j (min term, fp32 MFMA
  // over the sub-blocks).
  __device__ __forceinline__ void scale(const ActSB& x, int g, const v4i& S, v4f& acc,
                                        v4f& mn) const {
    const uint32_t s1 = hdr.z, s2 = hdr.w;
    const uint32_t m03 = s1 & 0x3F3F3F3Fu;
    const uint32_t m47 = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
    const float d = half_bits_to_f32(hdr.x & 0xFFFF), dmin = half_bits_to_f32(hdr.x >> 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t mw = h ? m47 : m03;
      const float mj = static_cast<float>((mw >> (8 * g)) & 0xFF);
      const int bsum = static_cast<int>(static_cast<int16_t>(x.bs[h] & 0xFFFF)) +
                       static_cast<int>(static_cast<int16_t>(x.bs[h] >> 16));
      mn = __builtin_amdgcn_mfma_f32_16x16x4f32(x.dA * static_cast<float>(bsum), dmin * mj, mn,
                                                0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += (x.dC[i] * d) * static_cast<float>(S[i]);
  }
  __device__ __forceinline__ void mma(const ActSB& x, int g, v4f& acc, v4f& mn) const {
    scale(x, g, sums(x), acc, mn);
  }
};

// ---- Q6_K: sub-block s of 16, w = d sc_s (q - 32), q - 32 fits int8.
struct WQ6K {
  uint2 l0[2], l1[2], qh[2], sc[2];
  uint32_t dbits;
  static constexpr bool kBS = false;
  __device__ __forceinline__ void load(const uint8_t* blk, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      l0[h] = ld8_a2(blk + 64 * h + 8 * g);
      l1[h] = ld8_a2(blk + 64 * h + 32 + 8 * g);
      qh[h] = ld8_a2(blk + 128 + 32 * h + 8 * g);
    }
    sc[0] = ld8_a2(blk + 192);
    sc[1] = ld8_a2(blk + 200);
    dbits = *gp<uint16_t>(blk + 208);
  }
  // S[i] = sum over the 16-weight sub-blocks s of sc_s * (int8 dot of q - 32
  // with C-row token 4g + i). Group m = 4h + qq covers sub-blocks 2m (lane
  // groups 0, 1) and 2m + 1 (groups 2, 3): two MFMAs, each with the other half
  // of B zeroed.
  __device__ __forceinline__ v4i sums(const ActSB& x, int g) const {
    v4i S = {0, 0, 0, 0};
    const bool first = g < 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int m = 4 * h + qq;
        const uint2 lo = (qq & 1) ? l1[h] : l0[h];
        const int lsh = (qq >> 1) * 4, hsh = 2 * qq;
        uint32_t w0 = ((lo.x >> lsh) & 0x0F0F0F0Fu) | (((qh[h].x >> hsh) & 0x03030303u) << 4);
        uint32_t w1 = ((lo.y >> lsh) & 0x0F0F0F0Fu) | (((qh[h].y >> hsh) & 0x03030303u) << 4);
        // bytes 0..63 -> q - 32 as int8, per byte without carries between bytes
        w0 = ((w0 | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
        w1 = ((w1 | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
        const long av = pk64(x.q[m].x, x.q[m].y);
        const long wv = pk64(w0, w1);
        const v4i ca = mma_i8(av, first ? wv : 0L);
        const v4i cb = mma_i8(av, first ? 0L : wv);
        const uint2 sv = m < 4 ? sc[0] : sc[1];
        const uint32_t sw = (m & 3) < 2 ? sv.x : sv.y;
        const int sh = 16 * (m & 1);
        const int sa = static_cast<int8_t>((sw >> sh) & 0xFF);
        const int sb = static_cast<int8_t>((sw >> (sh + 8)) & 0xFF);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[i] = mad24(sb, cb[i], mad24(sa, ca[i], S[i]));
      }
    }
    return S;
  }
  __device__ __forceinline__ void scale(const ActSB& x, const v4i& S, v4f& acc) const {
    const float d = half_bits_to_f32(dbits);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += (x.dC[i] * d) * static_cast<float>(S[i]);
  }
  __device__ __forceinline__ void mma(const ActSB& x, int g, v4f& acc, v4f&) const {
    scale(x, sums(x, g), acc);
  }
};

template <int FMT> struct WOf;
template <> struct WOf<FMT_Q4_K> { using T = WQ4K; };
template <> struct WOf<FMT_Q6_K> { using T = WQ6K; };

// Work item of a grouped launch: items (tile, row block) are numbered tile-major;
// each XCD (workgroup id % 8) takes a contiguous range, so the row blocks of a
// tile (same activations) and the tiles of an expert (same weights) share an L2.
// Returns -1 for workgroups beyond the chunk's items.
__device__ __forceinline__ int grouped_item(int n_items) {
  const int bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
  const int chunk = (n_items + 7) >> 3;
  const int item = xcd * chunk + j;
  return (j < chunk && item < n_items) ? item : -1;
}

// Streams nb super-blocks of NM weight rows (one per matrix) against the tile's
// activations. Two register stages: the loads of super-block b + 1 are in
// flight while b is computed. Scheduling barriers keep the compiler from
// sinking the loads below the compute (which would serialize every super-block
// behind a full memory round trip).
template <class W, int NM>
__device__ __forceinline__ void stream_rows(const uint8_t* const (&wrow)[NM], const ActRows& x,
                                            int nb, int g, v4f (&acc)[NM], v4f (&mn)[NM]) {
  constexpr int BB = W::kBS ? 144 : 210;
  ActSB xs[2];
  W ws[2][NM];
  auto ld = [&](ActSB& xa, W (&wa)[NM], int b) {
    load_act<W::kBS>(xa, x, b, g);
#pragma unroll
    for (int j = 0; j < NM; ++j) wa[j].load(wrow[j] + static_cast<size_t>(b) * BB, g);
  };
  auto mm = [&](const ActSB& xa, const W (&wa)[NM]) {
#pragma unroll
    for (int j = 0; j < NM; ++j) wa[j].mma(xa, g, acc[j], mn[j]);
  };
  ld(xs[0], ws[0], 0);
  for (int b = 0; b < nb; b += 2) {
    ld(xs[1], ws[1], min(b + 1, nb - 1));
    __builtin_amdgcn_sched_barrier(0);
    mm(xs[0], ws[0]);
    __builtin_amdgcn_sched_barrier(0);
    ld(xs[0], ws[0], min(b + 2, nb - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < nb) mm(xs[1], ws[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Test export of a tile kernel's integer super-block sums: dump[((m T + ts) n_rows
// + row) nb + b] = S of token slot ts (= 4 g + i) against weight row `row` of
// matrix m, super-block b.
__device__ __forceinline__ void dump_sums(int32_t* dump, int m, int T, int n_rows, int nb,
                                          int row, int b, int g, int cnt, const v4i& S) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ts = 4 * g + i;
    if (ts < cnt) dump[((static_cast<size_t>(m) * T + ts) * n_rows + row) * nb + b] = S[i];
  }
}

// ------------------------------------------------ LDS-staged Q4_K tile stream
// One work item streams the Q4_K rows of a few consecutive row blocks of one
// tile through a 2-slot LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4), one super-block ahead of the compute, so no
// weight bytes sit in registers while in flight. A slot holds one super-block
// of 128 weight rows (gate/up: 64 rows of each; down: 128 rows) and of the
// tile's 16 activation rows:
constexpr int kStA = 128 * 144;          // 16 rows x 256 B of q8, 16-byte pieces XOR-swizzled
constexpr int kStB = kStA + 16 * 256;    // 16 rows x 32 B of 16-element sums (+ 512 B pad)
constexpr int kStD = kStB + 1024;        // 16 block scales (+ pad)
constexpr int kStBytes = kStD + 256;     // 23808 B per slot

// MODE 0: gate/up (streams: gate and up rows of one 16-row tile per wave, 64
// rows per row block). MODE 1: down (two 16-row tiles per wave, 128 rows per
// row block). grid 8 * ceil(max items / 8), block 256 (4 waves). Two slots
// (47.6 KB) let three workgroups share a compute unit, so each ring's stage
// waits and barriers are covered by two others (three slots, one more stage
// in flight per ring but only two workgroups per unit, measured slower).
// Item = (tile, ii): row blocks [ii RBG, min(RB, (ii + 1) RBG)). Layers without
// expert biases only (those take the register-staged kernels).
// DUMP: also write the integer super-block sums to a.dump (test export).
template <int MODE, bool DUMP>
__global__ __launch_bounds__(256, DUMP ? 2 : 3) void k_glds_q4k(KArgs a, Div dIPT, int RBG, int RB) {
  // separate arrays: with the slot known at each access the compiler can tell
  // a slot being filled from the slot being read (no forced vmcnt(0))
  __shared__ __align__(16) uint8_t lds0[kStBytes];
  __shared__ __align__(16) uint8_t lds1[kStBytes];
  const int n_tiles = static_cast<int>(*gp<uint32_t>(a.counters));
  const int item = grouped_item(n_tiles * static_cast<int>(dIPT.d));
  if (item < 0) return;
  const uint32_t tile = dIPT.div(item);
  const int ii = dIPT.mod(item, tile);
  const int rb0 = ii * RBG, rb1 = min(RB, rb0 + RBG);
  const GTile tl = a.tiles[tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int cnt = tl.cnt;
  const int K = MODE == 0 ? a.H : a.F;  // reduction length
  const int nb = K >> 8;
  // activation rows of token slot ts (slots >= cnt repeat the last pair)
  auto pair_of = [&](int ts) { return a.plist[tl.start + min(ts, cnt - 1)]; };
  auto act_q = [&](int2 pr) -> const uint8_t* {
    return MODE == 0 ? reinterpret_cast<const uint8_t*>(a.xqs) + static_cast<size_t>(pr.y) * K
                     : reinterpret_cast<const uint8_t*>(a.hqs) + static_cast<size_t>(pr.x) * K;
  };
  auto act_bs = [&](int2 pr) -> const uint8_t* {
    return MODE == 0 ? reinterpret_cast<const uint8_t*>(a.xbs + static_cast<size_t>(pr.y) * (K >> 4))
                     : reinterpret_cast<const uint8_t*>(a.hbs + static_cast<size_t>(pr.x) * (K >> 4));
  };
  auto act_d = [&](int2 pr) -> const uint8_t* {
    return MODE == 0 ? reinterpret_cast<const uint8_t*>(a.xd + static_cast<size_t>(pr.y) * nb)
                     : reinterpret_cast<const uint8_t*>(a.hd + static_cast<size_t>(pr.x) * nb);
  };
  // ---- per-lane DMA sources. Wave w issues slot pieces j = w + 4u, u = 0..5:
  // j < 18 weights (piece i = 64 j + lane: row R = i / 9, 16-byte part i % 9),
  // 18..21 activation q8 (LDS piece (ts, ql) holds global piece ql ^ ts),
  // 22 the 16-element sums, 23 (4-byte) the block scales.
  // Row order: piece (R, q) of super-block b at row R's start + 144 b + 16 q.
  // 64-row tiles: the 64 blocks of a tile's super-block are one 9216-byte run
  // in row order, so a stage is one run per 64 rows.
  const uint8_t* wsrc[5];
  size_t wrbs[5];  // bytes between consecutive row blocks
  const size_t bstep = a.tiled ? 9216 : 144;  // bytes between consecutive super-blocks
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int j = min(wave + 4 * u, 17);
    const int i = 64 * j + lane, R = i / 9, q = i - 9 * R;
    const uint8_t* W;
    size_t st;
    int r;
    if (MODE == 0) {
      W = R < 64 ? tl.gate : tl.up;
      st = R < 64 ? a.stride_gate : a.stride_up;
      r = R & 63;
    } else {
      W = tl.down;
      st = a.stride_down;
      r = R;
    }
    if (a.tiled) {
      // row block rb = tile rb (gate/up) or tiles 2 rb, 2 rb + 1 (down)
      const size_t tile_bytes = static_cast<size_t>(nb) * 9216;
      wsrc[u] = W + (MODE == 0 ? 0 : static_cast<size_t>(R >> 6) * tile_bytes) +
                16 * (i - 576 * (R >> 6));
      wrbs[u] = (MODE == 0 ? 1 : 2) * tile_bytes;
    } else {
      wsrc[u] = W + static_cast<size_t>(r) * st + 16 * q;
      wrbs[u] = (MODE == 0 ? 64 : 128) * st;
    }
  }
  const uint8_t* asrc;  // activation q8 piece (waves 0..3: slot piece 20, 21, 18, 19)
  {
    const int j = wave < 2 ? 20 + wave : 16 + wave;
    const int i = 64 * (j - 18) + lane, ts = i >> 4, ql = i & 15;
    asrc = act_q(pair_of(ts)) + 16 * (ql ^ ts);
  }
  const uint8_t* xsrc;  // wave 2: sums (lanes 32..63 repeat 0..31); wave 3: scales
  if (wave == 2) {
    const int l = lane & 31;
    xsrc = act_bs(pair_of(l >> 1)) + 16 * (l & 1);
  } else {
    xsrc = act_d(pair_of(lane & 15));
  }
  auto issue = [&](uint8_t* L, int rb, int b) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dma16(wsrc[u] + rb * wrbs[u] + bstep * b, L + 1024 * (wave + 4 * u));
    if (wave < 2) {
      dma16(wsrc[4] + rb * wrbs[4] + bstep * b, L + 1024 * (wave + 16));
      dma16(asrc + 256 * b, L + 1024 * (wave + 20));
    } else {
      dma16(asrc + 256 * b, L + 1024 * (wave + 16));
      if (wave == 2) dma16(xsrc + 32 * b, L + kStB);
      else dma4(xsrc + 4 * b, L + kStD);
    }
  };
  // ---- compute-side lane roles
  int2 pC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pC[i] = pair_of(4 * g + i);
  int Rj[2];
  if (MODE == 0) { Rj[0] = wave * 16 + c; Rj[1] = 64 + wave * 16 + c; }
  else { Rj[0] = wave * 32 + c; Rj[1] = wave * 32 + 16 + c; }
  auto row_of = [&](int j, int rb) {
    return MODE == 0 ? rb * 64 + wave * 16 + c : rb * 128 + wave * 32 + 16 * j + c;
  };
  const int Tk = a.T * a.k;
  float wp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = pC[i].x;
      wp[i] = p < Tk ? *gp<float>(a.w + p) : (a.sh_gate_vec ? *gp<float>(a.shw + p - Tk) : 1.0f);
    }
  }
  // make every register load complete here, before the ring is filled: a wait
  // for them later (across the loop) would drain the in-flight slot loads
#pragma unroll
  for (int i = 0; i < 4; ++i) __asm__ volatile("" ::"v"(wp[i]), "v"(pC[i].x));
  const int nst = (rb1 - rb0) * nb;
  issue(lds0, rb0, 0);
  v4f acc[2], mn[2];
  int rb = rb0, b = 0;          // stage s: row block rb, super-block b
  int rbn = rb0, bn = 0;        // stage s + 1
  if (++bn == nb) { bn = 0; ++rbn; }
  // stage s: read slot s % 2, refill the other slot with stage s + 1
  auto step = [&](int s, const uint8_t* L, uint8_t* Lw) {
    // this wave's loads of stage s are the only ones outstanding: once they
    // are done, the barrier publishes every wave's share of the slot
    wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (b == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mn[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // the slot of stage s - 1 is free: every wave has passed its compute
    if (s + 1 < nst) issue(Lw, rbn, bn);
    if (++bn == nb) { bn = 0; ++rbn; }
    __builtin_amdgcn_sched_barrier(0);
    ActSB x;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int qg = 2 * m + (g >> 1);
      x.q[m] = *reinterpret_cast<const uint2*>(L + kStA + c * 256 + 16 * (qg ^ c) + 8 * (g & 1));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      x.bs[h] = *reinterpret_cast<const uint32_t*>(L + kStB + 32 * c + 4 * (4 * h + g));
    x.dA = *reinterpret_cast<const float*>(L + kStD + 4 * c);
    {
      const float4 dc = *reinterpret_cast<const float4*>(L + kStD + 16 * g);
      x.dC[0] = dc.x; x.dC[1] = dc.y; x.dC[2] = dc.z; x.dC[3] = dc.w;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      WQ4K w;
      const uint8_t* blk = L + Rj[j] * 144;
      w.hdr = *reinterpret_cast<const uint4*>(blk);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) w.q[cc] = *reinterpret_cast<const uint2*>(blk + 16 + 32 * cc + 8 * g);
      if constexpr (DUMP) {
        const v4i S = w.sums(x);
        dump_sums(a.dump, MODE == 0 ? j : 0, a.T, MODE == 0 ? a.F : a.H, nb,
                  MODE == 0 ? row_of(0, rb) : row_of(j, rb), b, g, cnt, S);
        w.scale(x, g, S, acc[j], mn[j]);
      } else {
        w.mma(x, g, acc[j], mn[j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (b == nb - 1) {  // row block done
      if (MODE == 0) {
        const int row = row_of(0, rb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (4 * g + i < cnt) {
            const float gv = acc[0][i] - mn[0][i];
            const float uv = acc[1][i] - mn[1][i];
            a.h[static_cast<size_t>(pC[i].x) * a.F + row] =
                act_fn(a.act, a.act_alpha, a.act_limit, gv, uv);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = row_of(j, rb);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (4 * g + i < cnt)
              a.part[static_cast<size_t>(pC[i].x) * a.H + row] = wp[i] * (acc[j][i] - mn[j][i]);
          }
        }
      }
    }
    if (++b == nb) { b = 0; ++rb; }
  };
  for (int s = 0; s < nst; s += 2) {
    step(s, lds0, lds1);
    if (s + 1 < nst) step(s + 1, lds1, lds0);
  }
}

// ------------------------------------------------ LDS-staged Q6_K down stream
// Q6_K blocks are 210 bytes, so a row's super-block b is not 16-byte aligned:
// a slot holds, per row, the 16-byte pieces that cover it (at most 14; the
// block starts at byte (210 b) mod 16 of them; row pitch 240) for 64 rows,
// plus the tile's 16 activation rows and block scales. Every piece loaded
// holds at least one byte of the block, so no load leaves its page.
constexpr int kQ6Row = 240;
constexpr int kS6A = 64 * kQ6Row;        // 15360: 16 rows x 256 B of q8 (XOR-swizzled pieces)
constexpr int kS6D = kS6A + 16 * 256;    // 19456: 16 block scales (+ pad)
constexpr int kS6Bytes = kS6D + 256;     // 19712 B per slot

// 8 bytes at byte offset off (even) of a 16-byte aligned LDS slot: dword
// reads + byte align (offset arithmetic keeps the LDS address space visible).
__device__ __forceinline__ uint2 lds8_a2(const uint8_t* L, int off) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(L + (off & ~3));
  const uint32_t* wl = reinterpret_cast<const uint32_t*>(L + ((off + 7) & ~3));
  const uint32_t sh = static_cast<uint32_t>(off & 3);
  const uint32_t w0 = w[0], w1 = w[1], w2 = *wl;
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}

// Down rows of Q6_K experts: item = (tile, ii), row blocks of 64 rows of H,
// wave w takes rows 16 w .. 16 w + 15 of a block. Same 2-slot ring protocol
// as k_glds_q4k, 5 slot loads per wave and stage. Layers without down biases.
// TILED (64-row tiles): a stage is one 13440-byte run, held in the slot's
// weight pieces as is (row pitch 210 instead of kQ6Row). Two slots of 19712
// bytes let four 4-wave workgroups share a compute unit's 160 KB of LDS, so
// each ring's stage waits and barriers are covered by three others.
template <bool DUMP, bool TILED>
__global__ __launch_bounds__(256, DUMP ? 2 : 4) void k_glds_q6k_down(KArgs a, Div dIPT, int RBG,
                                                                     int RB) {
  static_assert(4 * 2 * kS6Bytes <= 160 * 1024, "four workgroups per compute unit");
  __shared__ __align__(16) uint8_t lds0[kS6Bytes];
  __shared__ __align__(16) uint8_t lds1[kS6Bytes];
  const int n_tiles = static_cast<int>(*gp<uint32_t>(a.counters));
  const int item = grouped_item(n_tiles * static_cast<int>(dIPT.d));
  if (item < 0) return;
  const uint32_t tile = dIPT.div(item);
  const int ii = dIPT.mod(item, tile);
  const int rb0 = ii * RBG, rb1 = min(RB, rb0 + RBG);
  const GTile tl = a.tiles[tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int cnt = tl.cnt;
  const int K = a.F, nb = K >> 8;
  auto pair_of = [&](int ts) { return a.plist[tl.start + min(ts, cnt - 1)]; };
  // slot loads j = wave + 4 u, u = 0..4: j < 15 weight pieces (i = 64 j + lane:
  // row R = i / 15, piece i % 15), 15..18 q8(h) pieces, 19 (4-byte) scales
  const uint8_t* wsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = min(wave + 4 * u, 14);
    const int i = 64 * j + lane;
    if (TILED) {
      // 840 pieces per stage; lanes past them reload the last one (their LDS
      // bytes lie past the 64 blocks and are not read)
      wsrc[u] = tl.down + 16 * min(i, 839);
    } else {
      // a block needs at most 14 pieces (sh + 210 <= 224 bytes); the 15th of a
      // row reloads the 14th, so no load starts past the block (the last block
      // of the last row of an expert may end its allocation)
      const int R = i / 15, q = min(i - 15 * R, 13);
      wsrc[u] = tl.down + static_cast<size_t>(R) * a.stride_down + 16 * q;
    }
  }
  const size_t rbs = TILED ? static_cast<size_t>(nb) * 13440 : 64 * a.stride_down;
  const uint8_t* asrc;
  {
    const int j = wave == 3 ? 15 : 16 + wave;
    const int i = 64 * (j - 15) + lane, ts = i >> 4, ql = i & 15;
    asrc = reinterpret_cast<const uint8_t*>(a.hqs) + static_cast<size_t>(pair_of(ts).x) * K +
           16 * (ql ^ ts);
  }
  const uint8_t* dsrc =
      reinterpret_cast<const uint8_t*>(a.hd + static_cast<size_t>(pair_of(lane & 15).x) * nb);
  auto issue = [&](uint8_t* L, int rb, int b) {
    const size_t wo = rb * rbs + (TILED ? static_cast<size_t>(13440) * b : (210 * b) & ~15);
#pragma unroll
    for (int u = 0; u < 3; ++u) dma16(wsrc[u] + wo, L + 1024 * (wave + 4 * u));
    if (wave < 3) {
      dma16(wsrc[3] + wo, L + 1024 * (wave + 12));
      dma16(asrc + 256 * b, L + 1024 * (wave + 16));
    } else {
      dma16(asrc + 256 * b, L + 1024 * 15);
      dma4(dsrc + 4 * b, L + kS6D);
    }
  };
  int2 pC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pC[i] = pair_of(4 * g + i);
  const int Tk = a.T * a.k;
  float wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = pC[i].x;
    wp[i] = p < Tk ? *gp<float>(a.w + p) : (a.sh_gate_vec ? *gp<float>(a.shw + p - Tk) : 1.0f);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) __asm__ volatile("" ::"v"(wp[i]), "v"(pC[i].x));
  const int nst = (rb1 - rb0) * nb;
  issue(lds0, rb0, 0);
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f}, mn = acc;
  int rb = rb0, b = 0, rbn = rb0, bn = 0;
  if (++bn == nb) { bn = 0; ++rbn; }  // stage s + 1
  auto step = [&](int s, const uint8_t* L, uint8_t* Lw) {
    wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (b == 0) acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if (s + 1 < nst) issue(Lw, rbn, bn);
    if (++bn == nb) { bn = 0; ++rbn; }
    __builtin_amdgcn_sched_barrier(0);
    ActSB x;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int qg = 2 * m + (g >> 1);
      x.q[m] = *reinterpret_cast<const uint2*>(L + kS6A + c * 256 + 16 * (qg ^ c) + 8 * (g & 1));
    }
    {
      const float4 dc = *reinterpret_cast<const float4*>(L + kS6D + 16 * g);
      x.dC[0] = dc.x; x.dC[1] = dc.y; x.dC[2] = dc.z; x.dC[3] = dc.w;
    }
    WQ6K w;
    const int blk = TILED ? (wave * 16 + c) * 210 : (wave * 16 + c) * kQ6Row + ((210 * b) & 15);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w.l0[h] = lds8_a2(L, blk + 64 * h + 8 * g);
      w.l1[h] = lds8_a2(L, blk + 64 * h + 32 + 8 * g);
      w.qh[h] = lds8_a2(L, blk + 128 + 32 * h + 8 * g);
    }
    w.sc[0] = lds8_a2(L, blk + 192);
    w.sc[1] = lds8_a2(L, blk + 200);
    w.dbits = *reinterpret_cast<const uint16_t*>(L + blk + 208);
    if constexpr (DUMP) {
      const v4i S = w.sums(x, g);
      dump_sums(a.dump, 0, a.T, a.H, nb, rb * 64 + wave * 16 + c, b, g, cnt, S);
      w.scale(x, S, acc);
    } else {
      w.mma(x, g, acc, mn);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (b == nb - 1) {
      const int row = rb * 64 + wave * 16 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < cnt) a.part[static_cast<size_t>(pC[i].x) * a.H + row] = wp[i] * acc[i];
    }
    if (++b == nb) { b = 0; ++rb; }
  };
  for (int s = 0; s < nst; s += 2) {
    step(s, lds0, lds1);
    if (s + 1 < nst) step(s + 1, lds1, lds0);
  }
}

// Row order -> 64-row tiles, one 2-byte unit per thread (blocks are 2-byte
// aligned in both orders): destination block (tile, b, r) is source block
// (64 tile + r, b).
__global__ __launch_bounds__(256) void k_repack_tile64(const uint8_t* src, size_t stride, int nb,
                                                       int BB, uint8_t* dst, size_t units) {
  const size_t n_thr = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t u = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += n_thr) {
    const size_t byte = 2 * u, blk = byte / BB;
    const int off = static_cast<int>(byte - blk * BB);
    const int r = static_cast<int>(blk & 63);
    const size_t tb = blk >> 6, tile = tb / nb;
    const int b = static_cast<int>(tb - tile * nb);
    const uint8_t* p = src + (64 * tile + r) * stride + static_cast<size_t>(b) * BB + off;
    reinterpret_cast<uint16_t*>(dst)[u] = *reinterpret_cast<const uint16_t*>(p);
  }
}

// ================================================================== kernels

// q8 of one 256-element piece of x (job = token * pieces + piece), one wave;
// MXFP8 layers: MXFP8 of the piece (H a multiple of 32: the last piece may be
// partial, with whole blocks).
__device__ __forceinline__ void router_quant_wave(const KArgs& a, int job, int lane) {
  if (a.mx8) {
    const int pieces = (a.H + 255) >> 8;
    const int t = job / pieces, pc = job - t * pieces;
    if (t >= a.T) return;
    const int e0 = pc * 256 + 4 * lane;
    const bool valid = e0 < a.H;
    float v[4];
    load_x4(a.x, a.x_dtype, static_cast<size_t>(t) * a.H + (valid ? e0 : 0), v);
    quant_wave_mx8(v, valid, lane,
                   reinterpret_cast<uint8_t*>(a.xqs) + static_cast<size_t>(t) * a.H + pc * 256,
                   a.xe + static_cast<size_t>(t) * mx8_pitch(a.H) + pc * 8);
    return;
  }
  const int pieces = a.H >> 8;
  const int t = job / pieces, pc = job - t * pieces;
  if (t >= a.T) return;
  float v[4];
  load_x4(a.x, a.x_dtype, static_cast<size_t>(t) * a.H + pc * 256 + 4 * lane, v);
  const size_t base = static_cast<size_t>(t) * a.H + pc * 256;
  quant_wave<256>(v, true, lane, a.xqs + base, a.xd + base / 256, a.xbs + base / 16);
}

// Router logits for many tokens: fp32 inputs, fp64 MFMA products and sums (the
// products of fp32 values are exact in fp64). grid nwg_r + quant workgroups,
// block 256. Router workgroup w: K slice w % KS of (token tile, expert tile)
// w / KS, its four waves taking every fourth 16-k step of the slice (four
// short MFMA chains on four SIMDs instead of one long one), their fp64 sums
// added in wave order in LDS; column E of the expert tiles is the
// shared-expert gate vector when present. Quant waves: q8 of one 256-element
// piece of x. BF: x in bf16 (else fp32), a template argument so that no dtype
// branch sits between the batched loads.
template <bool BF>
__global__ __launch_bounds__(256) void k_router_mfma(KArgs a, int quant, int KS, int L, int n_et,
                                                     int n_work, int nwg_r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) >= nwg_r) {
    if (quant) router_quant_wave(a, (blockIdx.x - nwg_r) * 4 + wave, lane);
    return;
  }
  const int wv = blockIdx.x;  // workgroup-uniform: the early exit skips no barrier
  if (wv >= n_work) return;
  __shared__ v4d red[3][64];
  const int E1 = a.E + (a.sh_gate_vec ? 1 : 0);
  const int ks = wv % KS, r = wv / KS, et = r % n_et, tt = r / n_et;
  const int g = lane >> 4, c = lane & 15;
  const int t = min(tt * 16 + c, a.T - 1);
  const int e = min(et * 16 + c, E1 - 1);
  const float* wr = e < a.E ? a.w_router + static_cast<size_t>(e) * a.H : a.sh_gate_vec;
  const int k0 = ks * L;
  const int nst = (min(a.H, k0 + L) - k0) >> 4;  // steps of 16 (4 per lane group)
  v4d acc = {0.0, 0.0, 0.0, 0.0};
  auto step = [&](const float4& xv, const float4& wv4) {
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(xv.x),
                                               static_cast<double>(wv4.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(xv.y),
                                               static_cast<double>(wv4.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(xv.z),
                                               static_cast<double>(wv4.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(xv.w),
                                               static_cast<double>(wv4.w), acc, 0, 0, 0);
  };
  auto load_xv = [&](int kk) -> float4 {
    const size_t o = static_cast<size_t>(t) * a.H + kk;
    if constexpr (!BF) return ldg_f4(static_cast<const float*>(a.x) + o);
    const uint2 bb = ld8(static_cast<const uint16_t*>(a.x) + o);
    return make_float4(bf16_bits_to_f32(bb.x & 0xFFFF), bf16_bits_to_f32(bb.x >> 16),
                       bf16_bits_to_f32(bb.y & 0xFFFF), bf16_bits_to_f32(bb.y >> 16));
  };
  // MFMA step n (wave n % 4), lane group g: k = k0 + 16 n + 4 g + s for
  // s = 0..3 (the same k for A and B, so the k order is only a reordering of
  // the sum). The loads of U steps are issued before their MFMAs: one memory
  // round trip per U steps of the wave (a slice of up to 256 k is one round
  // trip; short batches keep the registers, and so the waves per SIMD, in
  // bounds); steps past the slice reload its last step and are not multiplied.
  constexpr int U = 4;
  for (int n = wave; n < nst; n += 4 * U) {
    float4 xv[U], wv4[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + 16 * min(n + 4 * u, nst - 1) + 4 * g;
      xv[u] = load_xv(kk);
      wv4[u] = ldg_f4(wr + kk);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (n + 4 * u < nst) step(xv[u], wv4[u]);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const v4d o = red[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += o[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = tt * 16 + g + 4 * i, ex = et * 16 + c;
    if (tok < a.T && ex < E1)
      a.rpart[(static_cast<size_t>(ks) * a.T + tok) * E1 + ex] = acc[i];
  }
}

// Router logits, 2 x 2 register blocking (chunks of more than 16 tokens and
// 16 experts): a router workgroup computes token tiles 2 tt .. 2 tt + 1
// against expert tiles 2 et .. 2 et + 1 over one of 8 K slices, its four waves
// taking every fourth 16-k step and adding their fp64 sums in wave order in
// LDS. Each loaded x and W fragment feeds two MFMAs, and the four accumulators
// are independent chains. K slice s is computed by workgroups s, s + 8, s + 16,
// ..., the ones that run on XCD s (dispatch order), so each slice's x and W are
// read into one L2. Same sums and partial layout as k_router_mfma (the k order
// inside a slice is only a reordering of the sum). grid nwg_r (8 per tile
// pair) + quant workgroups, block 256. BF as in k_router_mfma.
template <bool BF>
__global__ __launch_bounds__(256) void k_router_mfma22(KArgs a, int quant, int KS, int L,
                                                       int n_et2, int n_work, int nwg_r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) >= nwg_r) {
    if (quant) router_quant_wave(a, (blockIdx.x - nwg_r) * 4 + wave, lane);
    return;
  }
  const int ks = blockIdx.x & 7;  // KS == 8
  const int r = blockIdx.x >> 3;  // tile pair (workgroup-uniform: the exit skips no barrier)
  if (r >= n_work || ks >= KS) return;
  __shared__ v4d red[3][2][2][64];
  const int E1 = a.E + (a.sh_gate_vec ? 1 : 0);
  const int et2 = r % n_et2, tt2 = r / n_et2;
  const int g = lane >> 4, c = lane & 15;
  int t[2];
  const float* wr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    t[i] = min((2 * tt2 + i) * 16 + c, a.T - 1);
    const int e = min((2 * et2 + i) * 16 + c, E1 - 1);
    wr[i] = e < a.E ? a.w_router + static_cast<size_t>(e) * a.H : a.sh_gate_vec;
  }
  const int k0 = ks * L;
  const int nst = (min(a.H, k0 + L) - k0) >> 4;  // steps of 16 (4 per lane group)
  v4d acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
  auto load_xv = [&](int tok, int kk) -> float4 {
    const size_t o = static_cast<size_t>(tok) * a.H + kk;
    if constexpr (!BF) return ldg_f4(static_cast<const float*>(a.x) + o);
    const uint2 bb = ld8(static_cast<const uint16_t*>(a.x) + o);
    return make_float4(bf16_bits_to_f32(bb.x & 0xFFFF), bf16_bits_to_f32(bb.x >> 16),
                       bf16_bits_to_f32(bb.y & 0xFFFF), bf16_bits_to_f32(bb.y >> 16));
  };
  auto step = [&](const float4 (&xv)[2], const float4 (&wv4)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            static_cast<double>(xv[i].x), static_cast<double>(wv4[j].x), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            static_cast<double>(xv[i].y), static_cast<double>(wv4[j].y), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            static_cast<double>(xv[i].z), static_cast<double>(wv4[j].z), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            static_cast<double>(xv[i].w), static_cast<double>(wv4[j].w), acc[i][j], 0, 0, 0);
      }
  };
  // MFMA step n (wave n % 4), lane group g: k = k0 + 16 n + 4 g + s for s = 0..3
  // (steps past the slice reload its last step and are not multiplied)
  constexpr int U = 2;  // steps of the wave whose loads are issued together
  for (int n = wave; n < nst; n += 4 * U) {
    float4 xv[U][2], wv4[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + 16 * min(n + 4 * u, nst - 1) + 4 * g;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xv[u][i] = load_xv(t[i], kk);
        wv4[u][i] = ldg_f4(wr[i] + kk);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (n + 4 * u < nst) step(xv[u], wv4[u]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (wave > 0) red[wave - 1][i][j][lane] = acc[i][j];
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const v4d o = red[w][i][j][lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] += o[q];
      }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tok = (2 * tt2 + i) * 16 + g + 4 * q, ex = (2 * et2 + j) * 16 + c;
        if (tok < a.T && ex < E1)
          a.rpart[(static_cast<size_t>(ks) * a.T + tok) * E1 + ex] = acc[i][j][q];
      }
}

// Per token (one wave): logit = fp32(sum of the K-slice partials in slice order),
// then top-k and weights; the shared gate sigmoid from column E.
template <int NC>
__global__ __launch_bounds__(256) void k_topk_sum(KArgs a, int KS) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const int E1 = a.E + (a.sh_gate_vec ? 1 : 0);
  const double* rp = a.rpart + static_cast<size_t>(t) * E1;
  const size_t kstride = static_cast<size_t>(a.T) * E1;
  double s[NC], sg = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) s[i] = 0.0;
  // column E (the shared-expert gate, when present) rides in the same batches
  const int col_sh = a.sh_gate_vec ? a.E : a.E - 1;
  // slices in batches whose loads are all issued before the first add (one
  // memory round trip per batch); the sums still run in slice order
  constexpr int KB = NC <= 4 ? 16 : NC <= 8 ? 8 : 4;
  for (int k0 = 0; k0 < KS; k0 += KB) {
    double v[KB][NC], vs[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int ks = min(k0 + kb, KS - 1);
#pragma unroll
      for (int i = 0; i < NC; ++i) v[kb][i] = rp[ks * kstride + min(lane + 64 * i, a.E - 1)];
      vs[kb] = rp[ks * kstride + col_sh];
    }
    // keep the compiler from interleaving the adds with the loads (it would
    // otherwise keep only a few loads in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (k0 + kb < KS) {
#pragma unroll
        for (int i = 0; i < NC; ++i) s[i] += v[kb][i];
        sg += vs[kb];
      }
    }
  }
  float lg[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    lg[i] = static_cast<float>(s[i]);
    if (lane + 64 * i < a.E) a.logits[static_cast<size_t>(t) * a.E + lane + 64 * i] = lg[i];
  }
  if (a.sh_gate_vec && lane == 0) a.shw[t] = static_cast<float>(1.0 / (1.0 + exp(-sg)));
  wave_topk_regs<NC>(lg, a.sel_bias, a.E, a.k, a.router, a.norm_topk, a.route_scale,
                     a.ids + t * a.k, a.w + t * a.k);
}

// Stable counting sort of the pairs by expert (one workgroup of 1024 threads).
// Pair p = t * k + slot is present when its id is in range and the expert's
// gate pointer is not NULL; the shared expert is pseudo-expert E with pairs
// T * k + t. Output: plist sorted by (expert, pair), tiles of <= 16 consecutive
// entries of one expert, the tile count in counters[0], the presence flags.
// Every global load (ids, the experts' pointers) is issued at the start; the
// sort itself runs in LDS (pair and expert ids fit 16 bits).
constexpr int kMaxPairs = kMaxTokens * MOE_MAX_TOPK;
static_assert(kMaxPairs <= 65536 && MOE_MAX_EXPERTS < 65535, "16-bit pair and expert ids");
__global__ __launch_bounds__(1024) void k_bucket(KArgs a) {
  __shared__ int cnt[MOE_MAX_EXPERTS + 1];
  __shared__ int off[MOE_MAX_EXPERTS + 2];
  __shared__ int toff[MOE_MAX_EXPERTS + 2];
  __shared__ int cur[MOE_MAX_EXPERTS + 1];
  __shared__ uint8_t have[MOE_MAX_EXPERTS];  // gate[e] != NULL
  __shared__ uint16_t s_e[kMaxPairs];        // expert of pair p, 0xFFFF when absent
  __shared__ uint16_t s_grp[kMaxPairs];      // pairs grouped by expert, unordered inside
  const int tid = threadIdx.x, E = a.E, NE = E + 1, Tk = a.T * a.k;
  constexpr uint16_t kNone = 0xFFFF;
  // this thread's expert (tid < E <= 1024): its pointers, loaded up front
  const void *pg = nullptr, *pu = nullptr, *pd = nullptr;
  const float *bg = nullptr, *bu = nullptr, *bd = nullptr;
  if (tid < E) {
    pg = a.gate[tid];
    pu = a.up[tid];
    pd = a.down[tid];
    if (a.b_gate) { bg = a.b_gate[tid]; bu = a.b_up[tid]; }
    if (a.b_down) bd = a.b_down[tid];
  }
  for (int p = tid; p < Tk; p += 1024) {
    const int e = a.ids[p];
    s_e[p] = static_cast<unsigned>(e) < static_cast<unsigned>(E) ? static_cast<uint16_t>(e) : kNone;
  }
  for (int i = tid; i < NE; i += 1024) {
    cnt[i] = 0;
    cur[i] = 0;
  }
  if (tid < E) have[tid] = pg != nullptr;
  __syncthreads();
  for (int p = tid; p < Tk; p += 1024) {
    const int e = s_e[p];
    const bool ok = e != kNone && have[e];
    if (!ok) s_e[p] = kNone;
    a.present[p] = ok;
    if (ok) atomicAdd(&cnt[e], 1);
  }
  if (a.has_shared)
    for (int t = tid; t < a.T; t += 1024) a.present[Tk + t] = 1;
  if (tid == 0) cnt[E] = a.has_shared ? a.T : 0;
  __syncthreads();
  if (tid < 64) {  // exclusive scans of pair counts and tile counts (wave 0)
    int cc = 0, ct = 0;
    for (int base = 0; base < NE; base += 64) {
      const int i = base + tid;
      const int c = i < NE ? cnt[i] : 0, nt = (c + 15) >> 4;
      int ic = c, it = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int oc = __shfl_up(ic, d), ot = __shfl_up(it, d);
        if (tid >= d) {
          ic += oc;
          it += ot;
        }
      }
      if (i < NE) {
        off[i] = cc + ic - c;
        toff[i] = ct + it - nt;
      }
      cc += __shfl(ic, 63);
      ct += __shfl(it, 63);
    }
    if (tid == 0) {
      off[NE] = cc;
      toff[NE] = ct;
      a.counters[0] = static_cast<uint32_t>(ct);
    }
  }
  __syncthreads();
  for (int e = tid; e < NE; e += 1024) {
    const int c = cnt[e];
    if (c == 0) continue;
    GTile tl;
    tl.e = e;
    tl.pad = 0;
    if (e < E) {  // e == tid: this thread's pointers
      tl.gate = static_cast<const uint8_t*>(pg);
      tl.up = static_cast<const uint8_t*>(pu);
      tl.down = static_cast<const uint8_t*>(pd);
      tl.b_gate = bg;
      tl.b_up = bu;
      tl.b_down = bd;
    } else {
      tl.gate = static_cast<const uint8_t*>(a.sh_gate);
      tl.up = static_cast<const uint8_t*>(a.sh_up);
      tl.down = static_cast<const uint8_t*>(a.sh_down);
      tl.b_gate = tl.b_up = tl.b_down = nullptr;
    }
    for (int j = 0; 16 * j < c; ++j) {
      tl.start = off[e] + 16 * j;
      tl.cnt = min(16, c - 16 * j);
      a.tiles[toff[e] + j] = tl;
    }
  }
  for (int p = tid; p < Tk; p += 1024) {
    const int e = s_e[p];
    if (e != kNone) s_grp[off[e] + atomicAdd(&cur[e], 1)] = static_cast<uint16_t>(p);
  }
  if (a.has_shared)
    for (int t = tid; t < a.T; t += 1024) a.plist[off[E] + t] = make_int2(Tk + t, t);
  __syncthreads();
  // sorted position = bucket start + number of smaller pair ids in the bucket
  const int nr = off[E];
  for (int i = tid; i < nr; i += 1024) {
    const int p = s_grp[i];
    const int e = s_e[p];
    const int b0 = off[e], n = cnt[e];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += s_grp[b0 + j] < p;
    a.plist[b0 + rank] = make_int2(p, p / a.k);
  }
}

// Row tiles of 16 per wave: gate/up (two weight streams per tile) and down.
// Q6_K blocks hold more registers in flight than Q4_K, so they take fewer.
template <int FMT> constexpr int gu_tiles() { return FMT == FMT_Q4_K ? 2 : 1; }
template <int FMT> constexpr int down_tiles() { return FMT == FMT_Q4_K ? 4 : 2; }

// Gate/up rows of one tile: grid 8 * ceil(max items / 8), block 256. Item =
// (tile, block of 64 NT rows of F); wave w takes row tiles 16 (NT w + r),
// r < NT; its 2 NT weight streams (gate and up of each row tile) share one
// activation stage.
template <int FMT, int NT>
__global__ __launch_bounds__(256) void k_gu_grouped(KArgs a, Div dRB) {
  using W = typename WOf<FMT>::T;
  const int n_tiles = static_cast<int>(*gp<uint32_t>(a.counters));
  const int item = grouped_item(n_tiles * static_cast<int>(dRB.d));
  if (item < 0) return;
  const uint32_t tile = dRB.div(item);
  const int rb = dRB.mod(item, tile);
  const GTile tl = a.tiles[tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int cnt = tl.cnt;
  const int2 pA = a.plist[tl.start + min(c, cnt - 1)];
  int2 pC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pC[i] = a.plist[tl.start + min(4 * g + i, cnt - 1)];
  const int H = a.H, nb = H >> 8;
  ActRows x;
  x.qa = a.xqs + static_cast<size_t>(pA.y) * H;
  x.bsa = a.xbs + static_cast<size_t>(pA.y) * (H >> 4);
  x.da = a.xd + static_cast<size_t>(pA.y) * nb;
#pragma unroll
  for (int i = 0; i < 4; ++i) x.dc[i] = a.xd + static_cast<size_t>(pC[i].y) * nb;
  const int row0 = (rb * 4 + wave) * 16 * NT + c;  // row tile r: row0 + 16 r
  const uint8_t* wrow[2 * NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    wrow[2 * r] = tl.gate + static_cast<size_t>(row0 + 16 * r) * a.stride_gate;
    wrow[2 * r + 1] = tl.up + static_cast<size_t>(row0 + 16 * r) * a.stride_up;
  }
  v4f acc[2 * NT], mn[2 * NT];
#pragma unroll
  for (int j = 0; j < 2 * NT; ++j) acc[j] = mn[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  stream_rows<W, 2 * NT>(wrow, x, nb, g, acc, mn);
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int row = row0 + 16 * r;
    const float bg = tl.b_gate ? tl.b_gate[row] : 0.0f;
    const float bu = tl.b_up ? tl.b_up[row] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g + i < cnt) {
        const float gv = acc[2 * r][i] - mn[2 * r][i] + bg;
        const float uv = acc[2 * r + 1][i] - mn[2 * r + 1][i] + bu;
        a.h[static_cast<size_t>(pC[i].x) * a.F + row] =
            act_fn(a.act, a.act_alpha, a.act_limit, gv, uv);
      }
    }
  }
}

// q8 of h (blocks of 256, fp32 recipe) per present pair: one wave per
// (pair, 256-element piece). grid ceil(P * F / 256 / 4), block 256.
__global__ __launch_bounds__(256) void k_hquant(KArgs a, int P) {
  const int lane = threadIdx.x & 63;
  const int job = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int pieces = a.F >> 8;
  const int p = job / pieces, pc = job - p * pieces;
  if (p >= P || !a.present[p]) return;
  const float4 hv = ldg_f4(a.h + static_cast<size_t>(p) * a.F + pc * 256 + 4 * lane);
  const float v[4] = {hv.x, hv.y, hv.z, hv.w};
  quant_wave<256>(v, true, lane, a.hqs + static_cast<size_t>(p) * a.F + pc * 256,
                  a.hd + static_cast<size_t>(p) * (a.F >> 8) + pc,
                  a.hbs + static_cast<size_t>(p) * (a.F >> 4) + pc * 16);
}

// Down rows of one tile: item = (tile, block of 64 NT rows of H); wave w takes
// row tiles 16 (NT w + r), r < NT. Writes part[p] = w_p * (W_d q8(h_p) + b_d)
// for the tile's pairs.
template <int FMT, int NT>
__global__ __launch_bounds__(256) void k_down_grouped(KArgs a, Div dRB) {
  using W = typename WOf<FMT>::T;
  const int n_tiles = static_cast<int>(*gp<uint32_t>(a.counters));
  const int item = grouped_item(n_tiles * static_cast<int>(dRB.d));
  if (item < 0) return;
  const uint32_t tile = dRB.div(item);
  const int rb = dRB.mod(item, tile);
  const GTile tl = a.tiles[tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int cnt = tl.cnt;
  const int2 pA = a.plist[tl.start + min(c, cnt - 1)];
  int2 pC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pC[i] = a.plist[tl.start + min(4 * g + i, cnt - 1)];
  const int F = a.F, nb = F >> 8;
  ActRows x;
  x.qa = a.hqs + static_cast<size_t>(pA.x) * F;
  x.bsa = a.hbs + static_cast<size_t>(pA.x) * (F >> 4);
  x.da = a.hd + static_cast<size_t>(pA.x) * nb;
#pragma unroll
  for (int i = 0; i < 4; ++i) x.dc[i] = a.hd + static_cast<size_t>(pC[i].x) * nb;
  const int row0 = (rb * 4 + wave) * 16 * NT + c;  // row tile r: row0 + 16 r
  const uint8_t* wrow[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) wrow[r] = tl.down + static_cast<size_t>(row0 + 16 * r) * a.stride_down;
  v4f acc[NT], mn[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = mn[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  stream_rows<W, NT>(wrow, x, nb, g, acc, mn);
  const int Tk = a.T * a.k;
  float wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = pC[i].x;
    wp[i] = p < Tk ? a.w[p] : (a.sh_gate_vec ? a.shw[p - Tk] : 1.0f);
  }
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int row = row0 + 16 * r;
    const float bd = tl.b_down ? tl.b_down[row] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g + i < cnt)
        a.part[static_cast<size_t>(pC[i].x) * a.H + row] = wp[i] * (acc[r][i] - mn[r][i] + bd);
    }
  }
}

// y[t] = sum of the token's present pair rows in slot order, then the shared
// expert's. grid (ceil(H / 1024), T), block 256, 4 outputs per thread.
__global__ __launch_bounds__(256) void k_combine(KArgs a) {
  const int t = blockIdx.y, h0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h0 >= a.H) return;
  float r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;
  for (int s = 0; s < a.k; ++s) {
    const int p = t * a.k + s;
    if (a.present[p]) {
      const float4 v = ldg_f4(a.part + static_cast<size_t>(p) * a.H + h0);
      r0 += v.x; r1 += v.y; r2 += v.z; r3 += v.w;
    }
  }
  if (a.has_shared) {
    const float4 v = ldg_f4(a.part + static_cast<size_t>(a.T * a.k + t) * a.H + h0);
    r0 += v.x; r1 += v.y; r2 += v.z; r3 += v.w;
  }
  *reinterpret_cast<float4*>(a.y + static_cast<size_t>(t) * a.H + h0) = make_float4(r0, r1, r2, r3);
}

int grouped_grid(int n_items_max) { return 8 * ((n_items_max + 7) / 8); }

// One token tile for the tile-dots export: one tile of n_tok pairs (pair i =
// token i) over the given rows as gate, up and down of expert 0, weight 1.
__global__ void k_tile_setup(KArgs a, const uint8_t* rows, int n_tok) {
  const int i = threadIdx.x;
  if (i == 0) {
    a.counters[0] = 1;
    GTile tl;
    tl.e = 0;
    tl.start = 0;
    tl.cnt = n_tok;
    tl.pad = 0;
    tl.gate = tl.up = tl.down = rows;
    tl.b_gate = tl.b_up = tl.b_down = nullptr;
    a.tiles[0] = tl;
  }
  if (i < n_tok) {
    a.plist[i] = make_int2(i, i);
    a.w[i] = 1.0f;
  }
}

// Row blocks per LDS-staged work item: long enough streams to amortize the
// ring fill, while keeping about 9216 items at the bound on tiles (12 rounds
// of the Q4_K kernel's three workgroups per compute unit, 9 of the Q6_K
// kernel's four: a short tail).
int glds_group(int RB, int max_tiles) {
  int g = (RB * max_tiles + 9215) / 9216;
  if (g < 1) g = 1;
  if (g > RB) g = RB;
  return g;
}

}  // namespace

// The 2 x 2 blocked router kernel for chunks of more than 16 tokens and experts.
bool router_blocked(int T, int E) { return T > 16 && E + 1 > 16; }

RouterSplit router_split(int T, int E, int H) {
  const int E1 = E + 1;
  int ks;
  if (router_blocked(T, E)) {  // 8 slices, one per XCD (H / 16 >= 16)
    ks = 8;
  } else {
    const int tiles = ((T + 15) / 16) * ((E1 + 15) / 16);
    ks = (2048 + tiles - 1) / tiles;
  }
  if (ks > 16) ks = 16;
  if (ks < 1) ks = 1;
  const int steps = (H + 15) / 16;
  if (ks > steps) ks = steps;
  const int len = 16 * ((steps + ks - 1) / ks);
  return RouterSplit{(H + len - 1) / len, len};
}

int max_tiles(int T, int k, int E, int has_shared) {
  const int Tk = T * k;
  return (E < Tk ? E : Tk) + Tk / 16 + (has_shared ? (T + 15) / 16 : 0);
}

hipError_t launch_router_grouped(const KArgs& a, bool quant, RouterSplit rs, hipStream_t s,
                                 Ev ev) {
  const int E1 = a.E + (a.sh_gate_vec ? 1 : 0);
  const int pieces = a.mx8 ? (a.H + 255) / 256 : a.H / 256;
  const int nq = quant ? (a.T * pieces + 3) / 4 : 0;
  if (router_blocked(a.T, a.E)) {
    const int n_et2 = (E1 + 31) / 32, n_tt2 = (a.T + 31) / 32;
    const int n_work = n_tt2 * n_et2;  // tile pairs, each in all 8 K slices
    const int nwg_r = 8 * n_work;
    return launch(a.x_dtype ? k_router_mfma22<true> : k_router_mfma22<false>, dim3(nwg_r + nq),
                  256, 0, s, ev, a, quant ? 1 : 0, rs.ks, rs.len, n_et2, n_work, nwg_r);
  }
  const int n_et = (E1 + 15) / 16, n_tt = (a.T + 15) / 16;
  const int n_work = n_tt * n_et * rs.ks;  // one workgroup per (tile pair, slice)
  const int nwg_r = n_work;
  return launch(a.x_dtype ? k_router_mfma<true> : k_router_mfma<false>, dim3(nwg_r + nq), 256,
                0, s, ev, a, quant ? 1 : 0, rs.ks, rs.len, n_et, n_work, nwg_r);
}

hipError_t launch_topk_sum(const KArgs& a, RouterSplit rs, hipStream_t s, Ev ev) {
  const dim3 grid((a.T + 3) / 4);
  if (a.E <= 256) return launch(k_topk_sum<4>, grid, 256, 0, s, ev, a, rs.ks);
  if (a.E <= 512) return launch(k_topk_sum<8>, grid, 256, 0, s, ev, a, rs.ks);
  return launch(k_topk_sum<16>, grid, 256, 0, s, ev, a, rs.ks);
}

hipError_t launch_repack_tile64(const uint8_t* src, size_t stride, int n_rows, int nb, int BB,
                                uint8_t* dst, hipStream_t s) {
  const size_t units = static_cast<size_t>(n_rows) * nb * BB / 2;
  const size_t want = (units + 255) / 256;
  const int grid = static_cast<int>(want < 8192 ? want : 8192);
  return launch(k_repack_tile64, dim3(grid), 256, 0, s, Ev{}, src, stride, nb, BB, dst, units);
}

hipError_t launch_bucket(const KArgs& a, hipStream_t s, Ev ev) {
  return launch(k_bucket, dim3(1), 1024, 0, s, ev, a);
}

hipError_t launch_gateup_grouped(const KArgs& a, hipStream_t s, Ev ev) {
  const int mt = max_tiles(a.T, a.k, a.E, a.has_shared);
  if (a.fmt_gu == FMT_Q4_K && a.b_gate == nullptr) {
    const int RB = a.F / 64, RBG = glds_group(RB, mt), IPT = (RB + RBG - 1) / RBG;
    return launch(k_glds_q4k<0, false>, dim3(grouped_grid(mt * IPT)), 256, 0, s, ev, a, Div::make(IPT),
                  RBG, RB);
  }
  if (a.fmt_gu == FMT_Q4_K) {
    constexpr int NT = gu_tiles<FMT_Q4_K>();
    const int RB = a.F / (64 * NT);
    return launch(k_gu_grouped<FMT_Q4_K, NT>, dim3(grouped_grid(mt * RB)), 256, 0, s, ev, a,
                  Div::make(RB));
  }
  constexpr int NT = gu_tiles<FMT_Q6_K>();
  const int RB = a.F / (64 * NT);
  return launch(k_gu_grouped<FMT_Q6_K, NT>, dim3(grouped_grid(mt * RB)), 256, 0, s, ev, a,
                Div::make(RB));
}

hipError_t launch_hquant(const KArgs& a, hipStream_t s, Ev ev) {
  const int P = a.T * a.k + a.T * a.has_shared;
  const int jobs = P * (a.F / 256);
  return launch(k_hquant, dim3((jobs + 3) / 4), 256, 0, s, ev, a, P);
}

hipError_t launch_down_grouped(const KArgs& a, hipStream_t s, Ev ev) {
  const int mt = max_tiles(a.T, a.k, a.E, a.has_shared);
  if (a.fmt_d == FMT_Q4_K && a.b_down == nullptr) {
    const int RB = a.H / 128, RBG = glds_group(RB, mt), IPT = (RB + RBG - 1) / RBG;
    return launch(k_glds_q4k<1, false>, dim3(grouped_grid(mt * IPT)), 256, 0, s, ev, a, Div::make(IPT),
                  RBG, RB);
  }
  if (a.fmt_d == FMT_Q4_K) {
    constexpr int NT = down_tiles<FMT_Q4_K>();
    const int RB = a.H / (64 * NT);
    return launch(k_down_grouped<FMT_Q4_K, NT>, dim3(grouped_grid(mt * RB)), 256, 0, s, ev, a,
                  Div::make(RB));
  }
  if (a.b_down == nullptr) {
    const int RB = a.H / 64, RBG = glds_group(RB, mt), IPT = (RB + RBG - 1) / RBG;
    return launch(a.tiled ? k_glds_q6k_down<false, true> : k_glds_q6k_down<false, false>,
                  dim3(grouped_grid(mt * IPT)), 256, 0, s, ev, a, Div::make(IPT), RBG, RB);
  }
  constexpr int NT = down_tiles<FMT_Q6_K>();
  const int RB = a.H / (64 * NT);
  return launch(k_down_grouped<FMT_Q6_K, NT>, dim3(grouped_grid(mt * RB)), 256, 0, s, ev, a,
                Div::make(RB));
}

hipError_t launch_combine(const KArgs& a, hipStream_t s, Ev ev) {
  return launch(k_combine, dim3((a.H + 1023) / 1024, a.T), 256, 0, s, ev, a);
}

// Scratch of the tile-dots export: tile count, tile, pair list, weights (one
// 256-byte region each), then the kernel's h (mode 0) or per-pair rows.
size_t tile_dots_ws(int, int n_rows, int, int n_tok) {
  return 1024 + 4 * static_cast<size_t>(n_tok) * n_rows;
}

hipError_t launch_tile_dots(int mode, const void* rows, int n_rows, int K, size_t stride,
                            const int8_t* qs, const float* d, const int16_t* bs, int n_tok,
                            int32_t* out, void* ws, hipStream_t s) {
  KArgs a;
  memset(&a, 0, sizeof a);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  a.T = n_tok;
  a.k = 1;
  a.E = 1;
  a.counters = reinterpret_cast<uint32_t*>(w8);
  a.tiles = reinterpret_cast<GTile*>(w8 + 256);
  a.plist = reinterpret_cast<int2*>(w8 + 512);
  a.w = reinterpret_cast<float*>(w8 + 768);
  a.h = a.part = reinterpret_cast<float*>(w8 + 1024);
  a.xqs = a.hqs = const_cast<int8_t*>(qs);
  a.xd = a.hd = const_cast<float*>(d);
  a.xbs = a.hbs = const_cast<int16_t*>(bs);
  a.dump = out;
  if (mode == 0) {
    a.H = K;
    a.F = n_rows;
    a.stride_gate = a.stride_up = stride;
  } else {
    a.F = K;
    a.H = n_rows;
    a.stride_down = stride;
  }
  hipError_t e = launch(k_tile_setup, dim3(1), 64, 0, s, Ev{}, a,
                        static_cast<const uint8_t*>(rows), n_tok);
  if (e != hipSuccess) return e;
  // two row blocks per work item where there are two, as the production
  // grouping uses on long expert matrices (the ring then runs across them)
  const int RB = mode == 0 ? n_rows / 64 : mode == 1 ? n_rows / 128 : n_rows / 64;
  const int RBG = RB >= 2 ? 2 : 1, IPT = (RB + RBG - 1) / RBG;
  const dim3 grid(grouped_grid(IPT));
  if (mode == 0) return launch(k_glds_q4k<0, true>, grid, 256, 0, s, Ev{}, a, Div::make(IPT), RBG, RB);
  if (mode == 1) return launch(k_glds_q4k<1, true>, grid, 256, 0, s, Ev{}, a, Div::make(IPT), RBG, RB);
  return launch(k_glds_q6k_down<true, false>, grid, 256, 0, s, Ev{}, a, Div::make(IPT), RBG, RB);
}

}  // namespace moe
