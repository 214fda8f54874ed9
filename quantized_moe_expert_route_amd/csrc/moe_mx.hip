// MX-native expert-grouped kernels for gfx950: MXFP4 experts against MXFP8
// activations on the block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4),
// for layers whose activation numerics are MXFP8 (memra ARCHITECTURE.md, §0
// item 3 and the §2 ledger row on MXFP4 / block-scale mma: block-scaled FP4 /
// FP8 products as the compute lever of batched and prefill chunks).
//
// The chunk runs the grouped path's router, top-k and bucketing (tiles of up
// to 16 (token, slot) pairs of one expert), then:
//   k_gmx<0>       per (tile, 32 rows of F): gate and up rows against MXFP8(x)
//                  of the tile's tokens, block scales applied by the MFMA;
//                  bias, SwiGLU -> h
//   k_hquant_mx8   MXFP8 of h per present pair
//   k_gmx<1>       per (tile, 64 rows of H): down rows against MXFP8(h); bias
//                  and routing weight -> per-pair rows
//   k_combine      (grouped path) slot-order sum per token
//
// Operand layout of the 16x16x128 block-scaled MFMA (A: 16 token rows of
// E4M3, B: 16 weight columns of E2M1, K = 128 = four 32-value scale blocks;
// lane = 16 g + c):
//   B: lane (c, g) holds scale block g of column c, 16 bytes, low nibble of
//      byte j first: K positions 2j, 2j + 1; its scale byte is scale_b.
//   A: lane (r, g) holds bytes 16 (g % 2) .. + 15 of scale blocks g / 2 and
//      2 + g / 2 of row r (32 bytes); scale_a of lane (r, g) is block g's.
//   C: lane (c, g) holds rows 4 g + i, column c.
// An MXFP4 block's byte j holds elements j (low) and j + 16 (high), so K
// position 2j is element j and 2j + 1 is element j + 16; MXFP8 activation
// blocks are stored in that order (pair-interleaved) so both operands agree.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

using namespace dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

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

// Work item of a grouped launch: items (tile, row-block group) tile-major, each
// XCD (workgroup id % 8) a contiguous range; -1 past the chunk's items.
__device__ __forceinline__ int mx_item(int n_items) {
  const int bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
  const int chunk = (n_items + 7) >> 3;
  const int item = xcd * chunk + j;
  return (j < chunk && item < n_items) ? item : -1;
}

// Ring slot: one stage = 16 scale blocks (K = 512) of 64 weight rows (272
// bytes = 17 aligned 16-byte pieces per row) and of the tile's 16 activation
// rows (512 bytes each, pieces XOR-swizzled by row), 16 scale bytes per
// activation row, and the row block's 64 bias values.
constexpr int kMxBlocks = 16;
constexpr int kMxRow = 17 * kMxBlocks;        // 272
constexpr int kMxA = 64 * kMxRow;             // 17408
constexpr int kMxE = kMxA + 16 * 512;         // 25600
constexpr int kMxBias = kMxE + 256;           // 25856
constexpr int kMxSlot = kMxBias + 256;        // 26112 B per slot

// MODE 0: gate/up. Row block = 32 rows of F; LDS rows 0..31 are the gate rows,
// 32..63 the up rows; wave w computes F rows 8 w .. 8 w + 7 as MFMA columns
// 0..7 (gate) and 8..15 (up). MODE 1: down. Row block = 64 rows of H; wave w
// computes rows 16 w .. 16 w + 15. Item = (tile, ii): row blocks [ii RBG,
// min(RB, (ii + 1) RBG)). grid 8 * ceil(max items / 8), block 256.
template <int MODE>
__global__ __launch_bounds__(256, 3) void k_gmx(KArgs a, Div dIPT, int RBG, int RB) {
  // two slots (52.2 KB): three workgroups share a compute unit
  __shared__ __align__(16) uint8_t lds0[kMxSlot];
  __shared__ __align__(16) uint8_t lds1[kMxSlot];
  const int n_tiles = static_cast<int>(*gp<uint32_t>(a.counters));
  const int item = mx_item(n_tiles * static_cast<int>(dIPT.d));
  if (item < 0) return;
  const uint32_t tile = dIPT.div(item);
  const int ii = dIPT.mod(item, tile);
  const int rb0 = ii * RBG, rb1 = min(RB, rb0 + RBG);
  const GTile tl = a.tiles[tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int cnt = tl.cnt;
  const int K = MODE == 0 ? a.H : a.F;      // reduction length
  const int N = MODE == 0 ? a.F : a.H;      // output rows
  const int nb = K >> 5;                    // scale blocks per row
  const int nbs = (nb + kMxBlocks - 1) / kMxBlocks;  // stages per row block
  const int spitch = mx8_pitch(K);
  const int qmax_w = (17 * nb - 1) >> 4;    // last 16-byte piece holding weight bytes
  const int qmax_a = (K >> 4) - 1;          // last piece of an activation row
  const bool has_bias = MODE == 0 ? tl.b_gate != nullptr : tl.b_down != nullptr;
  auto pair_of = [&](int ts) { return a.plist[tl.start + min(ts, cnt - 1)]; };
  auto act_row = [&](int2 pr) -> const uint8_t* {
    return MODE == 0 ? reinterpret_cast<const uint8_t*>(a.xqs) + static_cast<size_t>(pr.y) * K
                     : reinterpret_cast<const uint8_t*>(a.hqs) + static_cast<size_t>(pr.x) * K;
  };
  auto scale_row = [&](int2 pr) -> const uint8_t* {
    return MODE == 0 ? a.xe + static_cast<size_t>(pr.y) * spitch
                     : a.he + static_cast<size_t>(pr.x) * spitch;
  };
  // ---- DMA roles. Wave w issues slot pieces j = w + 4 u, u = 0..6: j < 17
  // weights (piece i = 64 j + lane: row R = i / 17, part q = i % 17), 17..24
  // activations (LDS piece (ts, ql) holds global piece ql ^ ts; only the
  // slots holding one of the tile's cnt token rows), 25 scale bytes (4 per
  // lane), 26 biases (4 bytes per lane; layers with biases). The issue code
  // indexes no register array dynamically (a spill to scratch would add
  // memory operations of its own).
  int wR[5], wq[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int j = wave + 4 * u;  // <= 19: u < 5 covers every weight slot (j < 17)
    const int i = 64 * min(j, 16) + lane;
    wR[u] = i / 17;
    wq[u] = i - 17 * wR[u];
  }
  // activation slots of wave w: 17 + (w + 3) % 4 and 4 more
  const uint8_t* arow[2];
  int aq[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int j = 17 + ((wave + 3) & 3) + 4 * v;
    const int i = 64 * (j - 17) + lane, ts = i >> 5, ql = i & 31;
    arow[v] = act_row(pair_of(ts));
    aq[v] = ql ^ ts;
  }
  const uint8_t* srow = scale_row(pair_of(lane >> 2));
  auto weight_src = [&](int R, int q, int rb, int s) -> const uint8_t* {
    const int qq = min(17 * s + q, qmax_w);
    if (MODE == 0) {
      const int row = rb * 32 + (R & 31);
      return (R < 32 ? static_cast<const uint8_t*>(tl.gate) + static_cast<size_t>(row) * a.stride_gate
                     : static_cast<const uint8_t*>(tl.up) + static_cast<size_t>(row) * a.stride_up) +
             16 * qq;
    }
    const int row = min(rb * 64 + R, N - 1);
    return static_cast<const uint8_t*>(tl.down) + static_cast<size_t>(row) * a.stride_down +
           16 * qq;
  };
  // the wave's activation slots: 17 + (w + 3) % 4 and 4 more (token rows
  // 2 (j - 17) and 2 (j - 17) + 1 each)
  const int ja = 17 + ((wave + 3) & 3);
  // issue order inside a stage is free: the ring waits for whole stages
  auto issue = [&](uint8_t* L, int rb, int s) {
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int j = wave + 4 * u;  // wave-uniform; j < 17 for u < 4, and for wave 0 at u = 4
      // non-temporal: a stage's 272 bytes per row end mid 64-byte segment, so
      // the segment it shares with the next stage is fetched twice (HBM
      // traffic 1.2x); cached loads avoid that but evict the router weights
      // the next forward reads, which costs more than the tiles gain
      if (j < 17) dma16_nt(weight_src(wR[u], wq[u], rb, s), L + 1024 * j);
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int j = ja + 4 * v;
      if (2 * (j - 17) >= cnt) continue;  // rows past the tile's count: not loaded
      dma16(arow[v] + 16 * min(32 * s + aq[v], qmax_a), L + kMxA + 1024 * (j - 17));
    }
    if (wave == 1) dma4(srow + 16 * s + 4 * (lane & 3), L + kMxE);
    if (wave == 2 && has_bias) {
      const float* bsrc;
      if (MODE == 0) bsrc = lane < 32 ? tl.b_gate + rb * 32 + lane : tl.b_up + rb * 32 + lane - 32;
      else bsrc = tl.b_down + min(rb * 64 + lane, N - 1);
      dma4(reinterpret_cast<const uint8_t*>(bsrc), L + kMxBias);
    }
  };
  // ---- compute-side lane roles
  int2 pC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pC[i] = pair_of(4 * g + i);
  // B column c of this wave: LDS weight row
  const int Rb = MODE == 0 ? (c < 8 ? 8 * wave + c : 32 + 8 * wave + c - 8) : 16 * wave + c;
  const int Tk = a.T * a.k;
  float wp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = pC[i].x;
      wp[i] = p < Tk ? *gp<float>(a.w + p) : (a.sh_gate_vec ? *gp<float>(a.shw + p - Tk) : 1.0f);
    }
  }
  // every register load completes here, before the ring is filled
#pragma unroll
  for (int i = 0; i < 4; ++i) __asm__ volatile("" ::"v"(wp[i]), "v"(pC[i].x));
  const int nst = (rb1 - rb0) * nbs;
  // stage st -> (row block, stage within the row block)
  issue(lds0, rb0, 0);
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int rb = rb0, sb = 0, rbn = rb0, sbn = 0;
  if (++sbn == nbs) { sbn = 0; ++rbn; }  // stage st + 1
  // stage st: read slot st % 2, refill the other slot with stage st + 1
  auto step = [&](int st, const uint8_t* L, uint8_t* Lw) {
    // this wave's loads of stage st are the only ones outstanding: once they
    // are done, the barrier publishes every wave's share of the slot
    wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (sb == 0) acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // the slot of stage st - 1 is free: every wave has passed its compute
    if (st + 1 < nst) issue(Lw, rbn, sbn);
    if (++sbn == nbs) { sbn = 0; ++rbn; }
    __builtin_amdgcn_sched_barrier(0);
    const int nbv = min(kMxBlocks, nb - sb * kMxBlocks);  // valid blocks in this stage
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (4 * m < nbv) {  // wave-uniform
        const int bl = 4 * m + g;
        const bool ok = bl < nbv;
        // B: the lane's 17-byte block of row Rb (scale byte, then 16 nibble bytes)
        const int o = Rb * kMxRow + 17 * bl;
        const uint32_t* wp32 = reinterpret_cast<const uint32_t*>(L + (o & ~3));
        const uint32_t sh = static_cast<uint32_t>(o & 3);
        uint32_t w[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) w[k] = wp32[k];
        v8i B = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          B[k] = static_cast<int>(sh == 3 ? w[k + 1] : __builtin_amdgcn_alignbyte(w[k + 1], w[k], sh + 1));
        int sbw = static_cast<int>((w[0] >> (8 * sh)) & 0xFF);
        // A: bytes 16 (g % 2) .. of blocks 4m + g/2 and 4m + 2 + g/2 of token row c
        // token rows past the tile's count are not loaded: their MFMA rows
        // (garbage, rows are independent) are never stored
        const uint8_t* arow_l = L + kMxA + 512 * c;
        const int p0 = 8 * m + g, p1 = 8 * m + 4 + g;  // global pieces of the stage row
        const uint4 a0 = *reinterpret_cast<const uint4*>(arow_l + 16 * (p0 ^ c));
        const uint4 a1 = *reinterpret_cast<const uint4*>(arow_l + 16 * (p1 ^ c));
        const v8i A = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                       static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                       static_cast<int>(a1.z), static_cast<int>(a1.w)};
        int sab = L[kMxE + 16 * c + bl];
        if (!ok) {  // block past the row: no contribution (finite scales, zero B)
#pragma unroll
          for (int k = 0; k < 4; ++k) B[k] = 0;
          sbw = 127;
          sab = 127;
        }
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 4, 0, sab, 0, sbw);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (sb == nbs - 1) {  // row block done
      const float* bias = reinterpret_cast<const float*>(L + kMxBias);
      if (MODE == 0) {
        // up values of columns 8..15 to lanes c - 8 (rotate the 16-lane row by 8)
        v4f up;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          up[i] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[i]), 0x128, 0xF, 0xF, false));
        if (c < 8) {
          const int row = rb * 32 + 8 * wave + c;
          const float bg = has_bias ? bias[8 * wave + c] : 0.0f;
          const float bu = has_bias ? bias[32 + 8 * wave + c] : 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (4 * g + i < cnt)
              a.h[static_cast<size_t>(pC[i].x) * a.F + row] =
                  act_fn(a.act, a.act_alpha, a.act_limit, acc[i] + bg, up[i] + bu);
          }
        }
      } else {
        const int row = rb * 64 + 16 * wave + c;
        if (row < N) {
          const float bd = has_bias ? bias[16 * wave + c] : 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * g + i < cnt) a.part[static_cast<size_t>(pC[i].x) * a.H + row] = wp[i] * (acc[i] + bd);
        }
      }
    }
    if (++sb == nbs) { sb = 0; ++rb; }
  };
  for (int st = 0; st < nst; st += 2) {
    step(st, lds0, lds1);
    if (st + 1 < nst) step(st + 1, lds1, lds0);
  }
}

// MXFP8 of h per present pair: one wave per (pair, 256-value piece). grid
// ceil(P * pieces / 4), block 256.
__global__ __launch_bounds__(256) void k_hquant_mx8(KArgs a, int P, Div dpc) {
  const int lane = threadIdx.x & 63;
  const int job = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = dpc.div(job), pc = dpc.mod(job, p);
  if (p >= P || !a.present[p]) return;
  const int e0 = pc * 256 + 4 * lane;
  const bool valid = e0 < a.F;
  const float4 hv = *reinterpret_cast<const float4*>(a.h + static_cast<size_t>(p) * a.F +
                                                      (valid ? e0 : 0));
  const float v[4] = {hv.x, hv.y, hv.z, hv.w};
  quant_wave_mx8(v, valid, lane, reinterpret_cast<uint8_t*>(a.hqs) + static_cast<size_t>(p) * a.F + pc * 256,
                 a.he + static_cast<size_t>(p) * mx8_pitch(a.F) + pc * 8);
}

// MXFP8 of x (standalone quantization): grid (ceil(H / 256), T), block 64.
__global__ __launch_bounds__(64) void k_quant_mx8(const void* x, int dtype, int H, uint8_t* q,
                                                  uint8_t* e) {
  const int lane = threadIdx.x, t = blockIdx.y;
  const int e0 = blockIdx.x * 256 + 4 * lane;
  const bool valid = e0 < H;
  float v[4];
  load_x4(x, dtype, static_cast<size_t>(t) * H + (valid ? e0 : 0), v);
  quant_wave_mx8(v, valid, lane, q + static_cast<size_t>(t) * H + blockIdx.x * 256,
                 e + static_cast<size_t>(t) * mx8_pitch(H) + blockIdx.x * 8);
}

int mx_grid(int n_items_max) { return 8 * ((n_items_max + 7) / 8); }

// Row blocks per work item, about 9216 items at the bound on tiles (measured
// on the gpt-oss shape at 16 and 64 tokens: one row block per item beat groups
// sized for one or two rounds of workgroups by 20-25%; the finer items balance
// the chip better than a long ring per item saves on fills).
int mx_group(int RB, int max_tiles) {
  int g = (RB * max_tiles + 9215) / 9216;
  return g < 1 ? 1 : (g > RB ? RB : g);
}

}  // namespace

hipError_t launch_quant_mx8(const void* x, int dtype, int T, int H, uint8_t* q, uint8_t* e,
                            hipStream_t s, Ev ev) {
  return launch(k_quant_mx8, dim3((H + 255) / 256, T), 64, 0, s, ev, x, dtype, H, q, e);
}

hipError_t launch_gateup_mx(const KArgs& a, int max_tiles, hipStream_t s, Ev ev) {
  const int RB = a.F / 32, RBG = mx_group(RB, max_tiles), IPT = (RB + RBG - 1) / RBG;
  return launch(k_gmx<0>, dim3(mx_grid(max_tiles * IPT)), 256, 0, s, ev, a, Div::make(IPT), RBG,
                RB);
}

hipError_t launch_hquant_mx8(const KArgs& a, hipStream_t s, Ev ev) {
  const int P = a.T * a.k + a.T * a.has_shared;
  const int pieces = (a.F + 255) / 256;
  return launch(k_hquant_mx8, dim3((P * pieces + 3) / 4), 256, 0, s, ev, a, P, Div::make(pieces));
}

hipError_t launch_down_mx(const KArgs& a, int max_tiles, hipStream_t s, Ev ev) {
  const int RB = (a.H + 63) / 64, RBG = mx_group(RB, max_tiles), IPT = (RB + RBG - 1) / RBG;
  return launch(k_gmx<1>, dim3(mx_grid(max_tiles * IPT)), 256, 0, s, ev, a, Div::make(IPT), RBG,
                RB);
}

}  // namespace moe
