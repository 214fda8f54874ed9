// Decode-path HIP kernels of the routed-expert MoE FFN layer for gfx950 (MI355X).
//
// moe_layer_forward on a small chunk (T tokens, every (token, slot) pair
// handled on its own) is three kernels:
//   k_router     router GEMV with fp64 accumulation (one wave per expert row)
//                + q8 of x (extra waves)
//   k_gateup     per (token, slot) pair and row tile: top-k of the token (one
//                wave, DPP reductions) -> expert pointers -> gate/up dequant-GEMV
//                against q8(x) staged in LDS -> SwiGLU -> h (fp32); workgroup
//                0 of each pair publishes the slot's id, weight and down pointers
//   k_down       per token and row tile: q8 of each present slot's h (in LDS),
//                down rows against it, routing-weighted sum in slot order
//                (+ shared expert) -> y
// Cross-workgroup communication is only through kernel boundaries: on this
// chip fences and same-address atomics cost more than a launch.
// plus k_quant (moe_quantize_act_q8k), k_topk (moe_route_topk) and the
// block-dot export. No float atomics; every reduction has a fixed order.
#include <algorithm>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

using namespace dev;

namespace {

// Rows of more blocks than this are summed in this many fixed chunks first.
constexpr int kSumChunks = 8;

// LDS layout of the down kernels: q8 of h per slot (qs, d, bsums), block
// values [ns][R][nb], slot outputs [R][ns]; the LDS-staged variant then holds
// the rows, 16-byte aligned.
__host__ __device__ inline int down_lds_weights_offset(int ns, int K, int R, int nb) {
  const int o = ns * K + ns * 4 * (K / 32) + ns * 2 * (K / 16) + 4 * ns * R * nb + 4 * ns * R;
  return (o + 15) & ~15;
}

// ---------------------------------------------------------------- launching
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

// ================================================================== kernels

// x [T, H] -> q8. grid (ceil(H / 256), T), block 64.
template <int B>
__global__ __launch_bounds__(64) void k_quant(const void* x, int dtype, int H, int8_t* qs,
                                              float* d, int16_t* bs) {
  const int lane = threadIdx.x, t = blockIdx.y;
  const int e0 = blockIdx.x * 256 + 4 * lane;
  const bool valid = e0 < H;
  float v[4];
  load_x4(x, dtype, static_cast<size_t>(t) * H + (valid ? e0 : 0), v);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = valid ? v[i] : 0.0f;
  const size_t base = static_cast<size_t>(t) * H + blockIdx.x * 256;
  quant_wave<B>(v, valid, lane, qs + base, d + base / B, bs ? bs + base / 16 : nullptr);
}

__global__ void k_zero(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Shared-expert gate sigmoid(v . x) per token, fp64 dot. grid T, block 256.
__global__ __launch_bounds__(256) void k_shared_gate(KArgs a) {
  __shared__ double red[4];
  const int t = blockIdx.x;
  double acc = 0.0;
#pragma unroll 8
  for (int h = threadIdx.x; h < a.H; h += 256)
    acc += static_cast<double>(a.sh_gate_vec[h]) *
           static_cast<double>(load_x(a.x, a.x_dtype, static_cast<size_t>(t) * a.H + h));
  acc = wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double s = red[0] + red[1] + red[2] + red[3];
    a.shw[t] = static_cast<float>(1.0 / (1.0 + exp(-s)));
  }
}

// Router logits (fp32 inputs, fp64 accumulation, one fp32 rounding).
// grid E + (shared gate row) + quant jobs, block 64. Waves [0, E) compute the
// logit of one expert for every token (TT at a time); wave E (if present) the
// shared-expert gate; the remaining waves quantize x in 256-value pieces when
// `quant` is set. Wave 0 also clears n_clear counters for the next kernel.
// Each pass over the row issues all of its W_r and x loads (U float4 pieces
// per lane and token) before the first multiply, so a row of up to 256 U
// values costs one memory round trip. Pieces past H read a valid address and
// are zeroed. XBF: x is bf16 (else fp32).
template <int TT, int U, bool XBF>
__global__ __launch_bounds__(64) void k_router(KArgs a, int quant, int n_clear) {
  const int lane = threadIdx.x, e = blockIdx.x;
  if (e == 0)
    for (int i = lane; i < n_clear; i += 64) a.counters[i] = 0;
  const int nrow = a.E + (a.sh_gate_vec ? 1 : 0);
  if (e >= nrow) {
    if (!quant) return;
    const int pieces = (a.H + 255) / 256;
    const int job = e - nrow, t = job / pieces, pc = job % pieces;
    const int e0 = pc * 256 + 4 * lane;
    const bool valid = e0 < a.H;
    float v[4];
    load_x4(a.x, XBF ? 1 : 0, static_cast<size_t>(t) * a.H + (valid ? e0 : 0), v);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = valid ? v[i] : 0.0f;
    const size_t base = static_cast<size_t>(t) * a.H + pc * 256;
    if (act32(a.fmt_gu))
      quant_wave<32>(v, valid, lane, a.xqs + base, a.xd + base / 32, nullptr);
    else
      quant_wave<256>(v, valid, lane, a.xqs + base, a.xd + base / 256, a.xbs + base / 16);
    return;
  }
  const float* wrow = e < a.E ? a.w_router + static_cast<size_t>(e) * a.H : a.sh_gate_vec;
  for (int t0 = 0; t0 < a.T; t0 += TT) {
    double acc[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) acc[i] = 0.0;
    for (int hb = 0; hb < a.H; hb += 256 * U) {
      float4 wv[U];
      float xv[TT][U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = hb + 256 * u + 4 * lane;
        wv[u] = *reinterpret_cast<const float4*>(wrow + (h < a.H ? h : 0));
      }
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        const int t = min(t0 + i, a.T - 1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int h = hb + 256 * u + 4 * lane;
          const size_t xo = static_cast<size_t>(t) * a.H + (h < a.H ? h : 0);
          if constexpr (XBF) {
            const uint2 bb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + xo);
            xv[i][u][0] = bf16_bits_to_f32(bb.x & 0xFFFF); xv[i][u][1] = bf16_bits_to_f32(bb.x >> 16);
            xv[i][u][2] = bf16_bits_to_f32(bb.y & 0xFFFF); xv[i][u][3] = bf16_bits_to_f32(bb.y >> 16);
          } else {
            const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + xo);
            xv[i][u][0] = f.x; xv[i][u][1] = f.y; xv[i][u][2] = f.z; xv[i][u][3] = f.w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = hb + 256 * u + 4 * lane < a.H;
        const double w0 = ok ? static_cast<double>(wv[u].x) : 0.0;
        const double w1 = ok ? static_cast<double>(wv[u].y) : 0.0;
        const double w2 = ok ? static_cast<double>(wv[u].z) : 0.0;
        const double w3 = ok ? static_cast<double>(wv[u].w) : 0.0;
#pragma unroll
        for (int i = 0; i < TT; ++i) {
          acc[i] = fma(w0, static_cast<double>(xv[i][u][0]), acc[i]);
          acc[i] = fma(w1, static_cast<double>(xv[i][u][1]), acc[i]);
          acc[i] = fma(w2, static_cast<double>(xv[i][u][2]), acc[i]);
          acc[i] = fma(w3, static_cast<double>(xv[i][u][3]), acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const double s = wave_sum_d(acc[i]);
      if (lane == 0 && t0 + i < a.T) {
        if (e < a.E) a.logits[static_cast<size_t>(t0 + i) * a.E + e] = static_cast<float>(s);
        else a.shw[t0 + i] = static_cast<float>(1.0 / (1.0 + exp(-s)));
      }
    }
  }
}

// Top-k for many tokens: one wave per token. grid ceil(T / 4), block 256.
template <int NC>
__global__ __launch_bounds__(256) void k_topk(KArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  wave_topk<NC>(a.logits + static_cast<size_t>(t) * a.E, a.sel_bias, a.E, a.k, a.router, a.norm_topk,
            a.route_scale, a.ids + t * a.k, a.w + t * a.k);
}

// -------------------------------------------------------------- gate/up GEMV
// grid (ceil(F / R), P), block 256. Pair p < T*k: token p / k, slot p % k;
// p >= T*k: shared expert of token p - T*k. routing_given: ids/w are inputs;
// otherwise wave 0 runs top-k for the token and workgroup x == 0 of each pair
// writes its slot's id and weight. Tasks (m in {gate, up}, row, block) are
// spread over lane groups; block values go to LDS and one thread per row sums
// them in block order.
template <int FMT, int TPG, int NC>
__global__ __launch_bounds__(256) void k_gateup(KArgs a, int R, int routing_given, Div dnb,
                                                Div dR) {
  using F = typename FmtOf<FMT>::T;
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr bool I32 = ActMode<FMT>::v == ACT_I8_32;  // int8 q8_32 (no 16-element sums)
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_e;
  __shared__ int s_ids[16];
  __shared__ float s_w[16];
  const int p = blockIdx.y, row0 = blockIdx.x * R;
  const int Tk = a.T * a.k;
  const bool routed = p < Tk;
  const int t = routed ? p / a.k : p - Tk;
  const int K = a.H, nb = K / F::BE;
  int8_t* lqs = reinterpret_cast<int8_t*>(smem);
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  const int act_bytes = MX ? K * 5 / 2 : K;  // MXFP4: 80 bytes per 32-value block
  float* ld = reinterpret_cast<float*>(smem + act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + act_bytes + 4 * (K / 32));
  float* vals = reinterpret_cast<float*>(smem + act_bytes + 4 * (K / 32) + 2 * (K / 16));
  // gate/up pointer tables of all experts, read while wave 0 runs the top-k
  const void** ltab = reinterpret_cast<const void**>(
      smem + act_bytes + 4 * (K / 32) + 2 * (K / 16) + 4 * ((2 * R * nb + 2 * R * kSumChunks + 1) & ~1));
  const int G = 256 / F::LPB;
  const int grp = threadIdx.x / F::LPB, sub = threadIdx.x % F::LPB;
  const int total = 2 * R * nb;
  typename F::Raw raw[TPG];
  const uint8_t* gbase = nullptr;
  const uint8_t* ubase = nullptr;
  // Every lane issues all TPG loads unconditionally (idle tasks read a dummy
  // 256-byte workspace region), so the compiler can count outstanding loads.
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.counters);
  auto issue_loads = [&]() {
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int task = grp + G * i;
      const uint32_t q1 = dnb.div(task), q2 = dR.div(q1);
      const int b = dnb.mod(task, q1), r = dR.mod(q1, q2), m = q2;
      const int row = row0 + r;
      const uint8_t* base = m ? ubase : gbase;
      const size_t stride = m ? a.stride_up : a.stride_gate;
      const uint8_t* blk = (task < total && row < a.F)
                               ? base + static_cast<size_t>(row) * stride + static_cast<size_t>(b) * F::BB
                               : dummy;
      F::load(raw[i], blk, sub);
    }
  };
  // q8 activations (not MXFP4): this thread's first slice is loaded before the
  // role work below, so that the selection wave does not issue it after its
  // dependent chain; it goes to LDS after the roles.
  int4 pre_q = make_int4(0, 0, 0, 0);
  int16_t pre_bs = 0;
  float pre_d = 0.0f;
  if constexpr (!MX) {
    const int tid = threadIdx.x;
    if (tid < K / 16) {
      pre_q = reinterpret_cast<const int4*>(a.xqs + static_cast<size_t>(t) * K)[tid];
      if constexpr (!I32) pre_bs = a.xbs[static_cast<size_t>(t) * (K / 16) + tid];
    }
    if (tid < K / F::BE) pre_d = a.xd[static_cast<size_t>(t) * (K / F::BE) + tid];
  }
  // The selection runs on one wave, chosen by the workgroup's place among
  // those resident on a compute unit (dispatch order: 256 per round), so that
  // the selection waves of co-resident workgroups run on different SIMDs.
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tkw = ((blockIdx.x + blockIdx.y * gridDim.x) >> 8) & 3;
  if (routed && wave != tkw) {
    // E <= 1024: at most 6 entries per thread; issue the loads, then store
    const int li = (wave - (wave > tkw ? 1 : 0)) * 64 + lane;  // 0..191
    const void* g[6];
    const void* u[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      if (192 * j < a.E) {  // wave-uniform: no loads past the table
        const int i = min(li + 192 * j, a.E - 1);
        g[j] = a.gate[i];
        u[j] = a.up[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int i = li + 192 * j;
      if (i < a.E) {
        ltab[2 * i] = g[j];
        ltab[2 * i + 1] = u[j];
      }
    }
  } else if (routed) {
    const int slot = p - t * a.k;
    // the selection is one long dependent chain: issue priority over the
    // co-resident workgroups' block arithmetic on this SIMD
    __builtin_amdgcn_s_setprio(3);
    if (routing_given) {
      if (lane == 0) s_e = a.ids[p];
    } else if (!MX && blockIdx.x != 0) {
      // only the slot's expert is needed here: ranks 0..slot, no weights (not
      // for MXFP4, whose kernels lose occupancy to the extra registers)
      float lg[NC];
#pragma unroll
      for (int i = 0; i < NC; ++i)
        lg[i] = a.logits[static_cast<size_t>(t) * a.E + min(lane + 64 * i, a.E - 1)];
      uint32_t key[NC];
      topk_keys<NC>(lg, a.sel_bias, a.E, key);
      const int e = topk_nth<NC>(key, a.E, slot);
      if (lane == 0) s_e = e;
    } else {
      wave_topk<NC>(a.logits + static_cast<size_t>(t) * a.E, a.sel_bias, a.E, a.k, a.router,
                    a.norm_topk, a.route_scale, s_ids, s_w);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane == 0) {
        s_e = s_ids[slot];
        if (blockIdx.x == 0) {
          a.ids[p] = s_ids[slot];
          a.w[p] = s_w[slot];
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (MX) {
    stage_act<ACT_PAIRS>(a.xqs + static_cast<size_t>(t) * K,
                         a.xd + static_cast<size_t>(t) * (K / 32), nullptr, K, lqs, ld, lbs, lap);
  } else {
    const int tid = threadIdx.x;
    const int8_t* qs = a.xqs + static_cast<size_t>(t) * K;
    const float* dd = a.xd + static_cast<size_t>(t) * (K / F::BE);
    if (tid < K / 16) {
      reinterpret_cast<int4*>(lqs)[tid] = pre_q;
      if constexpr (!I32) lbs[tid] = pre_bs;
    }
    if (tid < K / F::BE) ld[tid] = pre_d;
    for (int i = tid + 256; i < K / 16; i += 256) {
      reinterpret_cast<int4*>(lqs)[i] = reinterpret_cast<const int4*>(qs)[i];
      if constexpr (!I32) lbs[i] = a.xbs[static_cast<size_t>(t) * (K / 16) + i];
    }
    for (int i = tid + 256; i < K / F::BE; i += 256) ld[i] = dd[i];
  }
  __syncthreads();
  const float* bg = nullptr;
  const float* bu = nullptr;
  if (routed) {
    const int e = s_e;
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(a.E)) {  // invalid id: no-op
      if (blockIdx.x == 0 && threadIdx.x == 0) a.slots[p] = SlotRef{nullptr, nullptr};
      return;
    }
    gbase = static_cast<const uint8_t*>(ltab[2 * e]);
    if (gbase == nullptr) {  // expert not present: the slot contributes nothing
      if (blockIdx.x == 0 && threadIdx.x == 0) a.slots[p] = SlotRef{nullptr, nullptr};
      return;
    }
    ubase = static_cast<const uint8_t*>(ltab[2 * e + 1]);
    if (a.b_gate) { bg = a.b_gate[e]; bu = a.b_up[e]; }
  } else {
    gbase = static_cast<const uint8_t*>(a.sh_gate);
    ubase = static_cast<const uint8_t*>(a.sh_up);
  }
  // One issue site for both kinds of pair, after the bias pointer loads: a
  // pointer loaded after the blocks could only be used once all of them had
  // arrived (loads complete in issue order), and block registers merged from
  // two issue sites are copied, which waits for every load in flight.
  issue_loads();
  ActView av{lqs, ld, lbs, lap};
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int task = grp + G * i;
    const uint32_t q1 = dnb.div(task), q2 = dR.div(q1);
    const int b = dnb.mod(task, q1), r = dR.mod(q1, q2), m = q2;
    if (task < total && row0 + r < a.F) {
      const float v = block_value<F>(raw[i], av, b, sub);
      if (sub == 0) vals[(m * R + r) * nb + b] = v;
    }
  }
  __syncthreads();
  float* hrow = a.h + static_cast<size_t>(p) * a.F;
  // long rows (MXFP4: 32-value blocks): fixed chunks of blocks summed in
  // parallel first, then the chunks in order
  float* chunk = vals + 2 * R * nb;  // [2 R][kSumChunks]
  const bool chunked = nb > kSumChunks;
  if (chunked) {
    const int L = (nb + kSumChunks - 1) / kSumChunks;
    for (int i = threadIdx.x; i < 2 * R * kSumChunks; i += 256) {
      const int mr = i / kSumChunks, c = i - mr * kSumChunks;
      float o = 0.0f;
      for (int b = c * L; b < min(nb, (c + 1) * L); ++b) o += vals[mr * nb + b];
      chunk[i] = o;
    }
    __syncthreads();
  }
  for (int r = threadIdx.x; r < R; r += 256) {
    const int row = row0 + r;
    if (row >= a.F) break;
    float g = 0.0f, u = 0.0f;
    if (chunked) {
      for (int c = 0; c < kSumChunks; ++c) g += chunk[r * kSumChunks + c];
      for (int c = 0; c < kSumChunks; ++c) u += chunk[(R + r) * kSumChunks + c];
    } else {
      for (int b = 0; b < nb; ++b) g += vals[r * nb + b];
      for (int b = 0; b < nb; ++b) u += vals[(R + r) * nb + b];
    }
    if (bg) { g += bg[row]; u += bu[row]; }
    hrow[row] = act_fn(a.act, a.act_alpha, a.act_limit, g, u);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && routed) {
    // resolved down-projection pointers for k_down (one dependent load instead of three)
    SlotRef ref;
    ref.down = static_cast<const uint8_t*>(a.down[s_e]);
    ref.bias = a.b_down ? a.b_down[s_e] : nullptr;
    a.slots[p] = ref;
  }
}

// q8 (32-value blocks) of every pair's h for an MXFP4 down, once per pair,
// stored as the down kernel's LDS image: fp16 pairs (a[32b + i], a[32b + 16 + i])
// block-major and padded ([block][kApPitch], as ActView reads them) and one
// scale per block. grid ceil(P pieces / 4), block 256: one wave per
// 256-value piece (fp32 recipe; values past F belong to no block).
__global__ __launch_bounds__(256) void k_hquant_pairs(KArgs a, int P, Div dpc) {
  const int lane = threadIdx.x & 63;
  const int job = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = dpc.div(job), pc = dpc.mod(job, p);
  if (p >= P) return;
  const int e0 = pc * 256 + 4 * lane;
  const bool valid = e0 < a.F;
  const float4 hv = *reinterpret_cast<const float4*>(a.h + static_cast<size_t>(p) * a.F +
                                                      (valid ? e0 : 0));
  const float v[4] = {valid ? hv.x : 0.0f, valid ? hv.y : 0.0f, valid ? hv.z : 0.0f,
                      valid ? hv.w : 0.0f};
  quant_wave_pairs(v, valid, lane,
                   reinterpret_cast<half2_t*>(a.hqs) +
                       (static_cast<size_t>(p) * (a.F / 32) + pc * 8) * kApPitch,
                   a.hd + static_cast<size_t>(p) * (a.F / 32) + pc * 8);
}

// MXFP4 gate/up (the rows realigned per wave, see mx_pair). grid
// (ceil(F / (4 RPW)), P), block 256: wave w takes the row pairs (gate row r,
// up row r), r = row0 + w + 4 i for i < RPW. Routing and pointer tables as in
// k_gateup; each wave issues all its 16-byte row pieces as soon as the expert
// is known, then reduces each pair and applies the activation on lane 0.
// LDS: activation pairs [nb][kApPitch], scales [nb], 4 wave scratches, [E][2]
// gate/up pointers.
__host__ __device__ inline int mx_gu_scratch_offset(int nb) { return (84 * nb + 15) & ~15; }

// NS = 0: rows of 17-byte blocks (realigned through LDS); NS > 0: rows in the
// MX16 order, NS blocks per lane and row pair straight into registers.
template <int RPW, int NL, int NBL, int NC, int NS>
__global__ __launch_bounds__(256) void k_gateup_mx(KArgs a, int routing_given) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_e;
  __shared__ int s_ids[16];
  __shared__ float s_w[16];
  const int p = blockIdx.y, row0 = blockIdx.x * (4 * RPW);
  const int Tk = a.T * a.k;
  const bool routed = p < Tk;
  const int t = routed ? p / a.k : p - Tk;
  const int K = a.H, nb = K / 32, npc = mx_row_pieces(nb);
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  float* ld = reinterpret_cast<float*>(smem + 80 * nb);
  const int scr_bytes = mx_scratch_bytes(nb);
  uint8_t* scr0 = smem + mx_gu_scratch_offset(nb);
  const void** ltab = reinterpret_cast<const void**>(scr0 + 4 * scr_bytes);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* gbase = nullptr;
  const uint8_t* ubase = nullptr;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.counters);
  uint4 pcs[RPW][NS ? 1 : NL];
  Mx16Unit<NS ? NS : 1> u16[NS ? RPW : 1];
  auto issue = [&]() {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = row0 + wave + 4 * i;
      if constexpr (NS > 0) {
        const bool ok = r < a.F;
        mx16_issue<NS>(u16[i], gbase + static_cast<size_t>(r) * a.stride_gate,
                       ubase + static_cast<size_t>(r) * a.stride_up, ok, ok, nb, lane, dummy);
        continue;
      }
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const int j = lane + 64 * m;
        const bool up = j >= npc;
        const int q = up ? j - npc : j;
        const uint8_t* src = (j < 2 * npc && r < a.F)
                                 ? (up ? ubase + static_cast<size_t>(r) * a.stride_up
                                       : gbase + static_cast<size_t>(r) * a.stride_gate) + 16 * q
                                 : dummy;
        pcs[i][m] = ld_nt16(src);
      }
    }
  };
  // selection on one wave, rotated by the workgroup's residency index (see k_gateup)
  const int tkw = ((blockIdx.x + blockIdx.y * gridDim.x) >> 8) & 3;
  // the other three waves stage x's q8 as fp16 pairs, one 32-value block per
  // thread; the first block's loads are issued before the role work
  const int li = (wave - (wave > tkw ? 1 : 0)) * 64 + lane;  // 0..191 off the selection wave
  const int8_t* xq = a.xqs + static_cast<size_t>(t) * K;
  const float* xd = a.xd + static_cast<size_t>(t) * nb;
  int4 xq0 = make_int4(0, 0, 0, 0), xq1 = xq0;
  float xdv = 0.0f;
  if (wave != tkw && li < nb) {
    xq0 = reinterpret_cast<const int4*>(xq)[2 * li];
    xq1 = reinterpret_cast<const int4*>(xq)[2 * li + 1];
    xdv = xd[li];
  }
  if (routed && wave != tkw) {
    const void* g[6];
    const void* u[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      if (192 * j < a.E) {  // wave-uniform: no loads past the table
        const int i = min(li + 192 * j, a.E - 1);
        g[j] = a.gate[i];
        u[j] = a.up[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int i = li + 192 * j;
      if (i < a.E) {
        ltab[2 * i] = g[j];
        ltab[2 * i + 1] = u[j];
      }
    }
  } else if (routed) {
    const int slot = p - t * a.k;
    __builtin_amdgcn_s_setprio(3);
    if (routing_given) {
      if (lane == 0) s_e = a.ids[p];
    } else if (blockIdx.x != 0) {
      // only the slot's expert is needed here: ranks 0..slot, no weights
      float lg[NC];
#pragma unroll
      for (int i = 0; i < NC; ++i)
        lg[i] = a.logits[static_cast<size_t>(t) * a.E + min(lane + 64 * i, a.E - 1)];
      uint32_t key[NC];
      topk_keys<NC>(lg, a.sel_bias, a.E, key);
      const int e = topk_nth<NC>(key, a.E, slot);
      if (lane == 0) s_e = e;
    } else {
      wave_topk<NC>(a.logits + static_cast<size_t>(t) * a.E, a.sel_bias, a.E, a.k, a.router,
                    a.norm_topk, a.route_scale, s_ids, s_w);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane == 0) {
        s_e = s_ids[slot];
        if (blockIdx.x == 0) {
          a.ids[p] = s_ids[slot];
          a.w[p] = s_w[slot];
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if (wave != tkw) {
    for (int b = li; b < nb; b += 192) {
      if (b != li) {
        xq0 = reinterpret_cast<const int4*>(xq)[2 * b];
        xq1 = reinterpret_cast<const int4*>(xq)[2 * b + 1];
        xdv = xd[b];
      }
      const uint32_t lo[4] = {static_cast<uint32_t>(xq0.x), static_cast<uint32_t>(xq0.y),
                              static_cast<uint32_t>(xq0.z), static_cast<uint32_t>(xq0.w)};
      const uint32_t hi[4] = {static_cast<uint32_t>(xq1.x), static_cast<uint32_t>(xq1.y),
                              static_cast<uint32_t>(xq1.z), static_cast<uint32_t>(xq1.w)};
      uint4* dst = reinterpret_cast<uint4*>(lap + b * kApPitch);
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // pairs 4c..4c+3: (a[4c + j], a[16 + 4c + j])
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = __builtin_bit_cast(
              uint32_t, half2_t{static_cast<_Float16>(static_cast<int8_t>(lo[c] >> (8 * j))),
                                static_cast<_Float16>(static_cast<int8_t>(hi[c] >> (8 * j)))});
        dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      ld[b] = xdv;
    }
  }
  __syncthreads();
  const float* bg = nullptr;
  const float* bu = nullptr;
  if (routed) {
    const int e = s_e;
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(a.E)) {  // invalid id: no-op
      if (blockIdx.x == 0 && threadIdx.x == 0) a.slots[p] = SlotRef{nullptr, nullptr};
      return;
    }
    gbase = static_cast<const uint8_t*>(ltab[2 * e]);
    if (gbase == nullptr) {  // expert not present: the slot contributes nothing
      if (blockIdx.x == 0 && threadIdx.x == 0) a.slots[p] = SlotRef{nullptr, nullptr};
      return;
    }
    ubase = static_cast<const uint8_t*>(ltab[2 * e + 1]);
    if (a.b_gate) { bg = a.b_gate[e]; bu = a.b_up[e]; }
  } else {
    gbase = static_cast<const uint8_t*>(a.sh_gate);
    ubase = static_cast<const uint8_t*>(a.sh_up);
  }
  // One issue site for both kinds of pair, after the bias pointer loads: loads
  // complete in issue order, so a pointer loaded after the rows could only be
  // used once all of them had arrived, and row registers merged from two
  // issue sites are copied, which waits for every load in flight. Either way
  // the first pair's dots would wait for the wave's whole stream.
  issue();
  MxAct<NBL> A;
  mx_act_load(A, lap, ld, nb, lane);
  float* hrow = a.h + static_cast<size_t>(p) * a.F;
  uint8_t* scr = scr0 + wave * scr_bytes;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = row0 + wave + 4 * i;
    if (r < a.F) {
      float2 gu;
      if constexpr (NS > 0) gu = mx16_pair<NS, NBL>(u16[i], A, nb, lane);
      else gu = mx_pair<NL, NBL>(pcs[i], scr, nb, A, lane);
      if (lane == 0) {
        float g = gu.x, u = gu.y;
        if (bg) { g += bg[r]; u += bu[r]; }
        hrow[r] = act_fn(a.act, a.act_alpha, a.act_limit, g, u);
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && routed) {
    SlotRef ref;
    ref.down = static_cast<const uint8_t*>(a.down[s_e]);
    ref.bias = a.b_down ? a.b_down[s_e] : nullptr;
    a.slots[p] = ref;
  }
}

// Row tile and token of a down workgroup (grid: row tiles x tokens). When
// tokens of a chunk share an expert, the workgroups of one row tile read the
// same rows. Workgroups go to the 8 XCDs round robin by linear id, so the
// tokens of a row tile are given adjacent ids with one residue mod 8: they run
// at the same time on one XCD, and a shared expert's rows come from HBM once
// and from that XCD's L2 for the other tokens. One token: the identity.
__device__ __forceinline__ void down_tile_token(int& x, int& t) {
  const int gx = gridDim.x, T = gridDim.y;
  const int lin = blockIdx.x + gx * blockIdx.y;
  const int full = gx & ~7;  // row tiles in whole groups of 8
  if (lin < full * T) {
    const int rest = lin >> 3;
    t = rest % T;
    x = (rest / T) * 8 + (lin & 7);
  } else {
    const int r = lin - full * T, tail = gx - full;
    t = r / tail;
    x = full + (r - t * tail);
  }
}

// ---------------------------------------------------------------- down GEMV
// grid (ceil(H / R), T), block 512. For each present slot of token t (and the
// shared expert): down rows [row0, row0 + R) against q8(h), then
// y = sum_slot w * (o + b_down) + shw * o_shared in slot order.
// Waves 0-3 stream the down rows (TPG block tasks per lane) and multiply them;
// waves 4-7 meanwhile quantize h into LDS (fp32 recipe), so the VALU work of
// the quantization overlaps the weight stream instead of queueing behind the
// load issue.
template <int FMT, int TPG, int JB, bool PRE>
__global__ __launch_bounds__(512) void k_down(KArgs a, int R, Div dnb, Div dR, Div dpc) {
  using F = typename FmtOf<FMT>::T;
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int B = F::BE == 32 ? 32 : 256;  // q8 block of h
  extern __shared__ __align__(16) unsigned char smem[];
  int tile, t;
  down_tile_token(tile, t);
  const int row0 = tile * R;
  const int K = a.F, nb = K / F::BE;
  const int ns = a.k + a.has_shared;
  const int act_bytes = MX ? K * 5 / 2 : K;  // MXFP4: 80 bytes per 32-value block
  unsigned char* p_act = smem;
  float* ld = reinterpret_cast<float*>(smem + ns * act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + ns * act_bytes + ns * 4 * (K / 32));
  float* vals = reinterpret_cast<float*>(smem + ns * act_bytes + ns * 4 * (K / 32) +
                                         ns * 2 * (K / 16));
  __shared__ const uint8_t* dptr[17];
  __shared__ const float* dbias[17];
  __shared__ float wslot[17];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool streamer = wave < 4;  // wave-uniform role
  const int G = 256 / F::LPB;
  const int grp = threadIdx.x / F::LPB, sub = threadIdx.x % F::LPB;  // streamers only
  const int total = ns * R * nb;
  // loads are unconditional (idle ones read a dummy workspace region) so the
  // compiler can count outstanding loads
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.counters);
  // Quantizer jobs: 256-value pieces of h. h rows sit at fixed places (pair
  // t k + s, shared T k + t), so a quantizer wave loads its first JB jobs
  // before the slot table is read (an absent slot's row is loaded and ignored).
  const int qw = wave - 4;
  const int pieces = (K + 255) / 256;
  const int njobs = ns * pieces;
  auto load_h = [&](int job) {
    const int jc = min(job, njobs - 1);
    const int s = dpc.div(jc), e0 = dpc.mod(jc, s) * 256 + 4 * lane;
    const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
    const bool ok = job < njobs && e0 < K;
    const float* src = ok ? a.h + static_cast<size_t>(ps) * K + e0
                          : reinterpret_cast<const float*>(dummy);
    return *reinterpret_cast<const float4*>(src);
  };
  float4 hv[JB];
  if (!streamer && !PRE) {
#pragma unroll
    for (int u = 0; u < JB; ++u) hv[u] = load_h(qw + 4 * u);
  }
  if (threadIdx.x < ns) {
    const int s = threadIdx.x;
    if (s < a.k) {
      const SlotRef ref = a.slots[t * a.k + s];
      dptr[s] = ref.down;
      dbias[s] = ref.bias;
      wslot[s] = a.w[t * a.k + s];
    } else {
      dptr[s] = static_cast<const uint8_t*>(a.sh_down);
      dbias[s] = nullptr;
      wslot[s] = a.sh_gate_vec ? a.shw[t] : 1.0f;
    }
  }
  __syncthreads();
  // present slots as a wave-uniform bit mask (ns <= 17)
  const uint32_t present = static_cast<uint32_t>(
      __builtin_amdgcn_ballot_w64(lane < ns && dptr[min(lane, ns - 1)] != nullptr));
  typename F::Raw raw[TPG];
  if (streamer) {
    // all slot-pointer reads first, then all weight loads
    const uint8_t* wp[TPG];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int tc = min(grp + G * i, total - 1);
      wp[i] = dptr[dR.div(dnb.div(tc))];
    }
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int task = grp + G * i;
      const int tc = min(task, total - 1);
      const uint32_t q1 = dnb.div(tc), q2 = dR.div(q1);
      const int b = dnb.mod(tc, q1), r = dR.mod(q1, q2);
      const bool ok = task < total && row0 + r < a.H && wp[i] != nullptr;
      F::load(raw[i], ok ? wp[i] + static_cast<size_t>(row0 + r) * a.stride_down +
                               static_cast<size_t>(b) * F::BB
                         : dummy, sub);
    }
  } else if constexpr (PRE) {
    // h already quantized per pair (MXFP4 down): copy the LDS image of every
    // present slot, 16 bytes per thread and step
    const int qt = threadIdx.x - 256;
    const int n16 = act_bytes / 16;  // 16-byte pieces of one slot's fp16 pairs
    for (int i = qt; i < ns * n16; i += 256) {
      const int s = i / n16, j = i - s * n16;
      if ((present >> s) & 1u) {
        const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
        reinterpret_cast<int4*>(p_act + s * act_bytes)[j] =
            reinterpret_cast<const int4*>(a.hqs + static_cast<size_t>(ps) * act_bytes)[j];
      }
    }
    for (int i = qt; i < ns * (K / 32); i += 256) {
      const int s = i / (K / 32), j = i - s * (K / 32);
      if ((present >> s) & 1u) {
        const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
        ld[s * (K / 32) + j] = a.hd[static_cast<size_t>(ps) * (K / 32) + j];
      }
    }
  } else {
    auto quant_h = [&](int job, const float4& hv1) {
      const int s = dpc.div(job), pc = dpc.mod(job, s);
      const bool valid = pc * 256 + 4 * lane < K;
      const float v[4] = {hv1.x, hv1.y, hv1.z, hv1.w};
      if constexpr (!MX) {
        quant_wave<B>(v, valid, lane, reinterpret_cast<int8_t*>(p_act + s * act_bytes) + pc * 256,
                      ld + s * (K / 32) + pc * (256 / B), lbs + s * (K / 16) + pc * 16);
      } else {
        quant_wave_pairs(v, valid, lane,
                         reinterpret_cast<half2_t*>(p_act + s * act_bytes) + pc * 8 * kApPitch,
                         ld + s * (K / 32) + pc * 8);
      }
    };
    if constexpr (!MX) {
      int q[JB][4];
      float dv[JB];
      quant_wave_batch<B, JB>(hv, q, dv);
#pragma unroll
      for (int u = 0; u < JB; ++u) {
        const int job = qw + 4 * u;  // wave-uniform
        const int js = dpc.div(job);
        if (job < njobs && ((present >> js) & 1u)) {
          const int s = js, pc = dpc.mod(job, js);
          if (pc * 256 + 4 * lane < K) {
            reinterpret_cast<uint32_t*>(p_act + s * act_bytes + pc * 256)[lane] = pack_q8x4(q[u]);
            if (B == 32 && (lane & 7) == 0) ld[s * (K / 32) + pc * 8 + (lane >> 3)] = dv[u];
            if (B == 256 && lane == 0) ld[s * (K / 32) + pc] = dv[u];
          }
          if constexpr (B == 256) {
            const int sm = sum4(q[u][0] + q[u][1] + q[u][2] + q[u][3]);
            if ((lane & 3) == 0 && pc * 256 + 4 * lane < K)
              lbs[s * (K / 16) + pc * 16 + (lane >> 2)] = static_cast<int16_t>(sm);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < JB; ++u) {
        const int job = qw + 4 * u;
        if (job < njobs && ((present >> dpc.div(job)) & 1u)) quant_h(job, hv[u]);
      }
    }
    for (int job = qw + 4 * JB; job < njobs; job += 4) {  // jobs beyond the first batch
      const float4 v = load_h(job);
      if ((present >> dpc.div(job)) & 1u) quant_h(job, v);
    }
  }
  __syncthreads();
  if (streamer) {
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int task = grp + G * i;
      const uint32_t q1 = dnb.div(task), q2 = dR.div(q1);
      const int b = dnb.mod(task, q1), r = dR.mod(q1, q2), s = q2;
      if (task < total && row0 + r < a.H && ((present >> s) & 1u)) {
        ActView av{reinterpret_cast<const int8_t*>(p_act + s * act_bytes), ld + s * (K / 32),
                   lbs + s * (K / 16), reinterpret_cast<const half2_t*>(p_act + s * act_bytes)};
        const float v = block_value<F>(raw[i], av, b, sub);
        if (sub == 0) vals[(s * R + r) * nb + b] = v;
      }
    }
  }
  __syncthreads();
  // weighted slot outputs, one thread per (row, slot), then the sum over the
  // slots in slot order (shared expert last). Long rows (MXFP4: 32-value
  // blocks) first sum fixed chunks of blocks in parallel, then the chunks in
  // order.
  float* part = vals + ns * R * nb;  // [R][ns]
  float* chunk = part + ns * R;      // [ns R][kSumChunks]
  const bool chunked = nb > kSumChunks;
  if (chunked) {
    const int L = (nb + kSumChunks - 1) / kSumChunks;
    for (int i = threadIdx.x; i < ns * R * kSumChunks; i += 512) {
      const int sr = i / kSumChunks, c = i - sr * kSumChunks;
      float o = 0.0f;
      for (int b = c * L; b < min(nb, (c + 1) * L); ++b) o += vals[sr * nb + b];
      chunk[i] = o;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < R * ns; i += 512) {
    const int r = i / ns, s = i - r * ns, row = row0 + r;
    float v = 0.0f;
    if (row < a.H && ((present >> s) & 1u)) {
      float o = 0.0f;
      if (chunked) {
        for (int c = 0; c < kSumChunks; ++c) o += chunk[(s * R + r) * kSumChunks + c];
      } else {
        for (int b = 0; b < nb; ++b) o += vals[(s * R + r) * nb + b];
      }
      if (dbias[s]) o += dbias[s][row];
      v = wslot[s] * o;
    }
    part[i] = v;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 512) {
    const int row = row0 + r;
    if (row >= a.H) break;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) acc += part[r * ns + s];
    a.y[static_cast<size_t>(t) * a.H + row] = acc;
  }
}

// Q4_K / Q5_K / Q2_K down with the rows staged in LDS. grid (ceil(H / R), T),
// block 512. Same result as k_down. Waves 0-2 copy the down rows [row0, row0 +
// R) of every present slot straight into LDS (global->LDS loads of the 16-byte
// pieces covering each row; every block field the lanes read is dword-aligned
// in LDS) while waves 3-7 quantize h (the
// longer of the two paths: 3:5 measured best of 2:6, 3:5 and 4:4); then all
// eight waves multiply out of LDS, TPG block tasks per 8-lane group.
constexpr int kStreamers = 3, kQuantizers = 8 - kStreamers;
template <int FMT, int TPG, int JB>
__global__ __launch_bounds__(512) void k_down_lds(KArgs a, int R, Div dnb, Div dR, Div dpc,
                                                  Div dq) {
  using F = typename FmtOf<FMT>::T;
  extern __shared__ __align__(16) unsigned char smem[];
  int tile, t;
  down_tile_token(tile, t);
  const int row0 = tile * R;
  const int K = a.F, nb = K / 256;
  const int ns = a.k + a.has_shared;
  // rows staged as whole 16-byte pieces (the last may run into the row's stride padding)
  const int npc = (nb * F::BB + 15) / 16, pitch = 16 * npc;
  unsigned char* p_act = smem;
  float* ld = reinterpret_cast<float*>(smem + ns * K);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + ns * K + ns * 4 * (K / 32));
  float* vals = reinterpret_cast<float*>(smem + ns * K + ns * 4 * (K / 32) + ns * 2 * (K / 16));
  float* part = vals + ns * R * nb;  // [R][ns]
  uint8_t* wl = smem + down_lds_weights_offset(ns, K, R, nb);
  __shared__ const uint8_t* dptr[17];
  __shared__ const float* dbias[17];
  __shared__ float wslot[17];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool streamer = wave < kStreamers;  // wave-uniform role
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.counters);
  const int qw = wave - kStreamers;
  const int pieces = K / 256;
  const int njobs = ns * pieces;
  auto load_h = [&](int job) {
    const int jc = min(job, njobs - 1);
    const int s = dpc.div(jc), e0 = dpc.mod(jc, s) * 256 + 4 * lane;
    const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
    const float* src = job < njobs ? a.h + static_cast<size_t>(ps) * K + e0
                                   : reinterpret_cast<const float*>(dummy);
    return *reinterpret_cast<const float4*>(src);
  };
  float4 hv[JB];
  if (!streamer) {
#pragma unroll
    for (int u = 0; u < JB; ++u) hv[u] = load_h(qw + kQuantizers * u);
  }
  if (threadIdx.x < ns) {
    const int s = threadIdx.x;
    if (s < a.k) {
      const SlotRef ref = a.slots[t * a.k + s];
      dptr[s] = ref.down;
      dbias[s] = ref.bias;
      wslot[s] = a.w[t * a.k + s];
    } else {
      dptr[s] = static_cast<const uint8_t*>(a.sh_down);
      dbias[s] = nullptr;
      wslot[s] = a.sh_gate_vec ? a.shw[t] : 1.0f;
    }
  }
  __syncthreads();
  const uint32_t present = static_cast<uint32_t>(
      __builtin_amdgcn_ballot_w64(lane < ns && dptr[min(lane, ns - 1)] != nullptr));
  if (streamer) {
    // piece j = ((s R + r) npc + q) -> LDS bytes [16 j, 16 j + 16); one
    // instruction moves 64 consecutive pieces. Pieces of absent slots, rows
    // past H and the tail of the last instruction read the dummy region.
    const int npieces = ns * R * npc;
    for (int j0 = wave * 64; j0 < npieces; j0 += 64 * kStreamers) {
      const int j = j0 + lane;
      const int jc = min(j, npieces - 1);
      const uint32_t sr = dq.div(jc), sl = dR.div(sr);
      const int q = dq.mod(jc, sr), r = dR.mod(sr, sl);
      const uint8_t* src = dptr[sl];
      const bool ok = j < npieces && src != nullptr && row0 + r < a.H;
      dma16_nt(ok ? src + static_cast<size_t>(row0 + r) * a.stride_down + 16 * q : dummy,
               wl + 16 * j0);
    }
  } else {
    int q[JB][4];
    float dv[JB];
    quant_wave_batch<256, JB>(hv, q, dv);
#pragma unroll
    for (int u = 0; u < JB; ++u) {
      const int job = qw + kQuantizers * u;  // wave-uniform
      const int js = dpc.div(job);
      if (job < njobs && ((present >> js) & 1u)) {
        const int pc = dpc.mod(job, js);
        reinterpret_cast<uint32_t*>(p_act + js * K + pc * 256)[lane] = pack_q8x4(q[u]);
        if (lane == 0) ld[js * (K / 32) + pc] = dv[u];
        const int sm = sum4(q[u][0] + q[u][1] + q[u][2] + q[u][3]);
        if ((lane & 3) == 0) lbs[js * (K / 16) + pc * 16 + (lane >> 2)] = static_cast<int16_t>(sm);
      }
    }
    for (int job = qw + kQuantizers * JB; job < njobs; job += kQuantizers) {  // jobs beyond the first batch
      const float4 v4 = load_h(job);
      const int js = dpc.div(job), pc = dpc.mod(job, js);
      if ((present >> js) & 1u) {
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
        quant_wave<256>(v, true, lane, reinterpret_cast<int8_t*>(p_act + js * K) + pc * 256,
                        ld + js * (K / 32) + pc, lbs + js * (K / 16) + pc * 16);
      }
    }
  }
  wait_vm<0>();  // this wave's LDS copies have landed
  __syncthreads();
  {
    const int grp = threadIdx.x >> 3, sub = threadIdx.x & 7;  // 64 groups of 8 lanes
    const int total = ns * R * nb;
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int task = grp + 64 * i;
      if (task < total) {
        const uint32_t q1 = dnb.div(task), sl = dR.div(q1);
        const int b = dnb.mod(task, q1), r = dR.mod(q1, sl);
        if (row0 + r < a.H && ((present >> sl) & 1u)) {
          const uint8_t* blk = wl + static_cast<size_t>(q1) * pitch + b * F::BB;
          typename F::Raw raw;
          F::lds_load(raw, blk, sub);
          const ActView av{reinterpret_cast<const int8_t*>(p_act + sl * K), ld + sl * (K / 32),
                           lbs + sl * (K / 16), nullptr};
          const float v = block_value<F>(raw, av, b, sub);
          if (sub == 0) vals[task] = v;
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * ns; i += 512) {
    const int r = i / ns, s = i - r * ns, row = row0 + r;
    float v = 0.0f;
    if (row < a.H && ((present >> s) & 1u)) {
      float o = 0.0f;
      for (int b = 0; b < nb; ++b) o += vals[(s * R + r) * nb + b];
      if (dbias[s]) o += dbias[s][row];
      v = wslot[s] * o;
    }
    part[i] = v;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 512) {
    const int row = row0 + r;
    if (row >= a.H) break;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) acc += part[r * ns + s];
    a.y[static_cast<size_t>(t) * a.H + row] = acc;
  }
}

// MXFP4 down with the rows realigned per wave (see mx_pair). grid
// (ceil(H / R), T), block 512, R even. Units are (slot s, row pair r, r + 1)
// for s < ns, taken slot-major; wave w owns units [w upw, (w + 1) upw), upw <=
// RPW (the host plan), and issues them at once. Each wave first loads the h pieces of
// its quantization jobs (256 values of one slot's h, job = wave + 8 u), then
// its first weight batch, then quantizes (32-value blocks, fp32 recipe) into
// the LDS image: loads complete in issue order, so the quantization waits for
// h only. The weighted slot outputs are then summed in slot order, as in
// k_down.
// LDS: activation pairs [ns][nb][kApPitch], scales [ns][nb], 8 wave
// scratches, slot outputs [R][ns].
// h quantization jobs per wave (256-value pieces of every slot over 8 waves);
// the host keeps ns * ceil(F / 256) <= 8 * kMxDownJobs.
constexpr int kMxDownJobs = 8;
__host__ __device__ inline int mx_down_scratch_offset(int ns, int nb) {
  return (84 * ns * nb + 15) & ~15;
}

// NS as in k_gateup_mx.
template <int RPW, int NL, int NBL, int NS>
__global__ __launch_bounds__(512) void k_down_mx(KArgs a, int R) {
  extern __shared__ __align__(16) unsigned char smem[];
  int tile, t;
  down_tile_token(tile, t);
  const int row0 = tile * R;
  const int K = a.F, nb = K / 32, npc = mx_row_pieces(nb);
  const int ns = a.k + a.has_shared;
  const int act_bytes = 80 * nb;
  unsigned char* p_act = smem;
  float* ld = reinterpret_cast<float*>(smem + ns * act_bytes);
  const int scr_bytes = mx_scratch_bytes(nb);
  uint8_t* scr = smem + mx_down_scratch_offset(ns, nb) + (threadIdx.x >> 6) * scr_bytes;
  // [R][ns] slot outputs (MX16 rows: the only LDS the kernel uses)
  float* part = reinterpret_cast<float*>(NS ? smem : smem + mx_down_scratch_offset(ns, nb) + 8 * scr_bytes);
  __shared__ const uint8_t* dptr[17];
  __shared__ const float* dbias[17];
  __shared__ float wslot[17];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.counters);
  if (threadIdx.x < ns) {
    const int s = threadIdx.x;
    if (s < a.k) {
      const SlotRef ref = a.slots[t * a.k + s];
      dptr[s] = ref.down;
      dbias[s] = ref.bias;
      wslot[s] = a.w[t * a.k + s];
    } else {
      dptr[s] = static_cast<const uint8_t*>(a.sh_down);
      dbias[s] = nullptr;
      wslot[s] = a.sh_gate_vec ? a.shw[t] : 1.0f;
    }
  }
  __syncthreads();
  const uint32_t present = static_cast<uint32_t>(
      __builtin_amdgcn_ballot_w64(lane < ns && dptr[min(lane, ns - 1)] != nullptr));
  const int nrp = (R + 1) / 2, units = ns * nrp, upw = (units + 7) / 8;
  const int u0 = wave * upw, u1 = min(u0 + upw, units);
  uint4 pcs[RPW][NS ? 1 : NL];
  Mx16Unit<NS ? NS : 1> u16[NS ? RPW : 1];
  auto issue = [&](int ub) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int u = ub + i;
      const int s = u < u1 ? u / nrp : 0;
      const int r = row0 + 2 * (u - s * nrp);
      const uint8_t* base = (u < u1 && ((present >> s) & 1u)) ? dptr[s] : nullptr;
      if constexpr (NS > 0) {
        const uint8_t* rb = base ? base : dummy;
        mx16_issue<NS>(u16[i], rb + static_cast<size_t>(r) * a.stride_down,
                       rb + static_cast<size_t>(r + 1) * a.stride_down, base && r < a.H,
                       base && r + 1 < a.H, nb, lane, dummy);
        continue;
      }
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const int j = lane + 64 * m;
        const int hi = j >= npc ? 1 : 0;
        const int rr = r + hi;
        const bool ok = base != nullptr && j < 2 * npc && rr < a.H;
        pcs[i][m] = ld_nt16(ok ? base + static_cast<size_t>(rr) * a.stride_down +
                                     16 * (j - hi * npc)
                               : dummy);
      }
    }
  };
  const int pieces = (K + 255) / 256, njobs = ns * pieces;
  MxAct<NBL> A;
  int cur = -1;  // slot whose activations A holds (wave-uniform)
  // MX16 rows (NS > 0): h was quantized once per pair by k_hquant_pairs into
  // this kernel's LDS image in the workspace, and each lane reads its
  // activation blocks from there (L2). Those of the wave's first slot are
  // loaded before the rows, so they arrive first.
  auto act_of = [&](int s) {
    const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
    mx_act_load(A, reinterpret_cast<const half2_t*>(a.hqs) + static_cast<size_t>(ps) * nb * kApPitch,
                a.hd + static_cast<size_t>(ps) * nb, nb, lane);
    cur = s;
  };
  if constexpr (NS > 0) {
    if (u0 < u1) act_of(u0 / nrp);
    issue(u0);
  }
  float4 hv[NS ? 1 : kMxDownJobs];
#pragma unroll
  for (int u = 0; u < (NS ? 0 : kMxDownJobs); ++u) {
    const int job = wave + 8 * u;  // wave-uniform
    hv[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (job < njobs) {
      const int s = job / pieces, e0 = (job - s * pieces) * 256 + 4 * lane;
      const int ps = s < a.k ? t * a.k + s : a.T * a.k + t;
      if (e0 < K) hv[u] = *reinterpret_cast<const float4*>(a.h + static_cast<size_t>(ps) * K + e0);
    }
  }
  if constexpr (NS == 0) issue(u0);
#pragma unroll
  for (int u = 0; u < (NS ? 0 : kMxDownJobs); ++u) {
    const int job = wave + 8 * u;
    if (job < njobs) {
      const int s = job / pieces, pc = job - s * pieces;
      if ((present >> s) & 1u) {
        const float v[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
        quant_wave_pairs(v, pc * 256 + 4 * lane < K, lane,
                         reinterpret_cast<half2_t*>(p_act + s * act_bytes) + pc * 8 * kApPitch,
                         ld + s * nb + pc * 8);
      }
    }
  }
  if constexpr (NS == 0) __syncthreads();
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int u = u0 + i;
    if (u < u1) {
      const int s = u / nrp, rp = u - s * nrp, r = row0 + 2 * rp;
      if (((present >> s) & 1u) && r < a.H) {
        if (s != cur) {
          if constexpr (NS > 0) {
            act_of(s);
          } else {
            mx_act_load(A, reinterpret_cast<const half2_t*>(p_act + s * act_bytes), ld + s * nb,
                        nb, lane);
            cur = s;
          }
        }
        float2 o;
        if constexpr (NS > 0) o = mx16_pair<NS, NBL>(u16[i], A, nb, lane);
        else o = mx_pair<NL, NBL>(pcs[i], scr, nb, A, lane);
        if (lane == 0) {
          const float* bias = dbias[s];
          part[(2 * rp) * ns + s] = wslot[s] * (o.x + (bias ? bias[r] : 0.0f));
          if (2 * rp + 1 < R && r + 1 < a.H)
            part[(2 * rp + 1) * ns + s] = wslot[s] * (o.y + (bias ? bias[r + 1] : 0.0f));
        }
      }
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 512) {
    const int row = row0 + r;
    if (row >= a.H) break;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s)
      if ((present >> s) & 1u) acc += part[r * ns + s];
    a.y[static_cast<size_t>(t) * a.H + row] = acc;
  }
}

// Integer block partials export through the same format routines.
// grid n_rows, block 256.
template <int FMT>
__global__ __launch_bounds__(256) void k_block_dots(const uint8_t* rows, int K, size_t stride,
                                                    const int8_t* qs, const float* d,
                                                    const int16_t* bs, int32_t* out) {
  using F = typename FmtOf<FMT>::T;
  constexpr bool MX = FMT == FMT_MXFP4;
  extern __shared__ __align__(16) unsigned char smem[];
  const int act_bytes = MX ? K * 5 / 2 : K;
  int8_t* lqs = reinterpret_cast<int8_t*>(smem);
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  float* ld = reinterpret_cast<float*>(smem + act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + act_bytes + 4 * (K / 32));
  stage_act<ActMode<FMT>::v>(qs, d, bs, K, lqs, ld, lbs, lap);
  __syncthreads();
  ActView av{lqs, ld, lbs, lap};
  const int r = blockIdx.x, nb = K / F::BE;
  const int G = 256 / F::LPB, grp = threadIdx.x / F::LPB, sub = threadIdx.x % F::LPB;
  for (int b = grp; b < nb; b += G) {
    typename F::Raw raw;
    F::load(raw, rows + static_cast<size_t>(r) * stride + static_cast<size_t>(b) * F::BB, sub);
    const int2 pr = F::partials(raw, av, b, sub);
    if (sub == 0) {
      out[(static_cast<size_t>(r) * nb + b) * 2] = pr.x;
      out[(static_cast<size_t>(r) * nb + b) * 2 + 1] = pr.y;
    }
  }
}

// MXFP4 block partials through the routine the MXFP4 GEMV kernels run
// (k_gateup_mx, k_down_mx): row pairs read as coalesced 16-byte pieces,
// realigned through the wave's scratch by mx_pair_blocks and dotted against
// fp16 activation pairs in registers; S = 2 * dot (exact). grid ceil(n_rows /
// 2), block 64 (one wave per row pair). LDS as k_gateup_mx: activation pairs
// [nb][kApPitch], scales [nb], then the scratch.
template <int NL, int NBL>
__global__ __launch_bounds__(64) void k_block_dots_mx(const uint8_t* rows, int n_rows, int K,
                                                      size_t stride, const int8_t* qs,
                                                      const float* d, int32_t* out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nb = K / 32, npc = mx_row_pieces(nb), lane = threadIdx.x;
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  float* ld = reinterpret_cast<float*>(smem + 80 * nb);
  uint8_t* scr = smem + mx_gu_scratch_offset(nb);
  stage_act<ACT_PAIRS>(qs, d, nullptr, K, nullptr, ld, nullptr, lap);
  __syncthreads();
  const int r0 = 2 * blockIdx.x;
  uint4 pcs[NL];
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    const int j = lane + 64 * m;
    const int hi = j >= npc ? 1 : 0;
    const int r = r0 + hi;
    const bool ok = j < 2 * npc && r < n_rows;
    pcs[m] = ld_nt16(ok ? rows + static_cast<size_t>(r) * stride + 16 * (j - hi * npc) : rows);
  }
  MxAct<NBL> A;
  mx_act_load(A, lap, ld, nb, lane);
  mx_pair_blocks<NL, NBL>(pcs, scr, nb, A, lane, [&](int row, int b, int, float dot, int) {
    const int r = r0 + row;
    if (r < n_rows) {
      out[(static_cast<size_t>(r) * nb + b) * 2] = static_cast<int>(2.0f * dot);
      out[(static_cast<size_t>(r) * nb + b) * 2 + 1] = 0;
    }
  });
}

// The same export for MXFP4 rows in the MX16 order, through the MX16 kernels'
// loads and dots (mx16_issue, mx16_pair_blocks). grid ceil(n_rows / 2), block
// 64; LDS: activation pairs [nb][kApPitch], scales [nb].
template <int NS, int NBL>
__global__ __launch_bounds__(64) void k_block_dots_mx16(const uint8_t* rows, int n_rows, int K,
                                                        size_t stride, const int8_t* qs,
                                                        const float* d, int32_t* out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nb = K / 32, lane = threadIdx.x;
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  float* ld = reinterpret_cast<float*>(smem + 80 * nb);
  stage_act<ACT_PAIRS>(qs, d, nullptr, K, nullptr, ld, nullptr, lap);
  __syncthreads();
  const int r0 = 2 * blockIdx.x;
  Mx16Unit<NS> u;
  mx16_issue<NS>(u, rows + static_cast<size_t>(r0) * stride,
                 rows + static_cast<size_t>(min(r0 + 1, n_rows - 1)) * stride, true,
                 r0 + 1 < n_rows, nb, lane, rows);
  MxAct<NBL> A;
  mx_act_load(A, lap, ld, nb, lane);
  mx16_pair_blocks<NS, NBL>(u, A, nb, lane, [&](int row, int b, int, float dot, int) {
    const int r = r0 + row;
    if (r < n_rows) {
      out[(static_cast<size_t>(r) * nb + b) * 2] = static_cast<int>(2.0f * dot);
      out[(static_cast<size_t>(r) * nb + b) * 2 + 1] = 0;
    }
  });
}

// One MXFP4 matrix from rows of 17-byte blocks into the MX16 order, one output
// byte per thread (row r, byte o < mx16_row_bytes(nb)): the nibble fields,
// then the scale bytes, then zeros up to the next dword.
__global__ __launch_bounds__(256) void k_repack_mx16(const uint8_t* src, size_t stride, int nb,
                                                     uint8_t* dst, size_t dst_stride, int rb,
                                                     size_t total) {
  const size_t n_thr = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += n_thr) {
    const size_t r = i / rb;
    const int o = static_cast<int>(i - r * rb);
    const uint8_t* row = src + r * stride;
    uint8_t v = 0;
    if (o < 16 * nb) v = row[17 * (o >> 4) + 1 + (o & 15)];
    else if (o < 17 * nb) v = row[17 * (o - 16 * nb)];
    dst[r * dst_stride + o] = v;
  }
}

// Calls f(std::integral_constant<int, FMT>) for a format enum (nothing for
// an unknown one).
template <class Fn>
void with_fmt(int fmt, Fn&& f) {
  switch (fmt) {
    case FMT_Q4_K: f(std::integral_constant<int, FMT_Q4_K>{}); break;
    case FMT_Q6_K: f(std::integral_constant<int, FMT_Q6_K>{}); break;
    case FMT_MXFP4: f(std::integral_constant<int, FMT_MXFP4>{}); break;
    case FMT_Q5_K: f(std::integral_constant<int, FMT_Q5_K>{}); break;
    case FMT_Q2_K: f(std::integral_constant<int, FMT_Q2_K>{}); break;
    case FMT_Q3_K: f(std::integral_constant<int, FMT_Q3_K>{}); break;
    case FMT_Q4_0: f(std::integral_constant<int, FMT_Q4_0>{}); break;
    case FMT_Q5_1: f(std::integral_constant<int, FMT_Q5_1>{}); break;
    default: break;
  }
}

// Rows per workgroup and tasks per lane group for a GEMV launch: at least
// min_wgs workgroups while keeping every lane group busy.
struct GemvShape { int R, tpg; };
GemvShape gemv_shape(int rows_total, int nmat, int nb, int lpb, int grid_y, int tpg_max,
                     int min_wgs) {
  const int G = 256 / lpb;
  int R = (G * tpg_max) / (nmat * nb);
  if (R < 1) R = 1;
  if (R > rows_total) R = rows_total;
  while (R > 1 && static_cast<long>((rows_total + R - 1) / R) * grid_y < min_wgs) R = (R + 1) / 2;
  const int tpg = (nmat * R * nb + G - 1) / G;
  return {R, tpg};
}

int tpg_bucket(int tpg) { return tpg <= 1 ? 1 : tpg <= 2 ? 2 : tpg <= 4 ? 4 : 8; }

template <int FMT>
size_t gateup_lds(const KArgs& a, GemvShape* out) {
  using F = typename FmtOf<FMT>::T;
  const int P = a.T * a.k + a.T * a.has_shared;
  const int nb = a.H / F::BE;
  const int tpg_max = FMT == FMT_Q6_K || FMT == FMT_Q5_K || FMT == FMT_Q3_K ? 4 : 8;  // Raw registers per task
  GemvShape sh = gemv_shape(a.F, 2, nb, F::LPB, P, tpg_max, 512);
  if (out) *out = sh;
  const bool MX = FMT == FMT_MXFP4;
  return (MX ? 5 * a.H / 2 : a.H) + 4 * (a.H / 32) + 2 * (a.H / 16) +
         4 * static_cast<size_t>((2 * sh.R * nb + 2 * sh.R * kSumChunks + 1) & ~1) +
         16 * static_cast<size_t>(a.E);
}

template <int FMT>
size_t down_lds(const KArgs& a, GemvShape* out) {
  using F = typename FmtOf<FMT>::T;
  const int ns = a.k + a.has_shared;
  const int nb = a.F / F::BE;
  const int tpg_max = FMT == FMT_Q6_K || FMT == FMT_Q5_K || FMT == FMT_Q3_K ? 4 : 8;  // Raw registers per task
  // Every workgroup re-quantizes its token's h (VALU work), so the target is
  // one workgroup per compute unit (R = ceil(H T / 256)), as far as the cap
  // on loads per lane allows.
  const int G = 256 / F::LPB;
  const int per_token = max(1, 256 / max(a.T, 1));
  int R = min((G * tpg_max) / (ns * nb), (a.H + per_token - 1) / per_token);
  R = max(1, min(R, a.H));
  GemvShape sh{R, (ns * R * nb + G - 1) / G};
  if (out) *out = sh;
  const bool MX = FMT == FMT_MXFP4;
  return ns * ((MX ? 5 * a.F / 2 : a.F) + 4 * (a.F / 32) + 2 * (a.F / 16)) +
         4 * static_cast<size_t>(ns * sh.R * nb) + 4 * static_cast<size_t>(ns * sh.R) +
         4 * static_cast<size_t>(ns * sh.R * kSumChunks);
}

template <int FMT, int NC>
hipError_t gateup_dispatch_nc(const KArgs& a, int routing_given, hipStream_t s, Ev ev) {
  const int P = a.T * a.k + a.T * a.has_shared;
  GemvShape sh;
  const size_t lds = gateup_lds<FMT>(a, &sh);
  dim3 grid((a.F + sh.R - 1) / sh.R, P);
  using F = typename FmtOf<FMT>::T;
  const Div dnb = Div::make(a.H / F::BE), dR = Div::make(sh.R);
  switch (tpg_bucket(sh.tpg)) {
    case 1: return launch(k_gateup<FMT, 1, NC>, grid, 256, lds, s, ev, a, sh.R, routing_given, dnb, dR);
    case 2: return launch(k_gateup<FMT, 2, NC>, grid, 256, lds, s, ev, a, sh.R, routing_given, dnb, dR);
    case 4: return launch(k_gateup<FMT, 4, NC>, grid, 256, lds, s, ev, a, sh.R, routing_given, dnb, dR);
    default: return launch(k_gateup<FMT, 8, NC>, grid, 256, lds, s, ev, a, sh.R, routing_given, dnb, dR);
  }
}

// MXFP4 plans of k_gateup_mx / k_down_mx: NL 16-byte pieces per lane and row
// pair, NBL blocks per lane, RPW row pairs per wave in flight (at most nine
// pieces per lane).
struct MxPlan { int nl, nbl, rpw; };
bool mx_plan(int K, MxPlan* out) {
  const int nb = K / 32, npc = mx_row_pieces(nb);
  const int nl = (2 * npc + 63) / 64, nbl = (nb + 63) / 64;
  if (nbl == 1) *out = {nl, 1, 3};  // nl <= 3
  else if (nbl == 2) *out = nl <= 3 ? MxPlan{3, 2, 3} : MxPlan{5, 2, 1};
  else if (nbl <= 4) *out = {9, 4, 1};
  else return false;
  return true;
}

size_t mx_gateup_lds(const KArgs& a) {
  const int nb = a.H / 32;
  return static_cast<size_t>(mx_gu_scratch_offset(nb)) + 4 * mx_scratch_bytes(nb) +
         16 * static_cast<size_t>(a.E);
}

// Rows per k_down_mx workgroup: all (slot, row pair) units in one batch per
// wave where ns <= 8 RPW.
int mx_down_rows(const KArgs& a, const MxPlan& pl) {
  const int ns = a.k + a.has_shared;
  return 2 * max(1, 8 * pl.rpw / ns);
}

size_t mx_down_lds(const KArgs& a, const MxPlan& pl) {
  const int ns = a.k + a.has_shared, nb = a.F / 32;
  return static_cast<size_t>(mx_down_scratch_offset(ns, nb)) + 8 * mx_scratch_bytes(nb) +
         4 * static_cast<size_t>(mx_down_rows(a, pl)) * ns;
}

bool mx_gateup_fits(const KArgs& a) {
  MxPlan pl;
  return a.fmt_gu == FMT_MXFP4 && mx_plan(a.H, &pl) && mx_gateup_lds(a) <= kMaxLds;
}
bool mx_down_fits(const KArgs& a) {
  MxPlan pl;
  if (a.fmt_d != FMT_MXFP4 || !mx_plan(a.F, &pl)) return false;
  const int ns = a.k + a.has_shared;
  const int units = ns * (mx_down_rows(a, pl) / 2);  // every wave's units in one batch
  return mx_down_lds(a, pl) <= kMaxLds && (units + 7) / 8 <= pl.rpw &&
         ns * ((a.F + 255) / 256) <= 8 * kMxDownJobs;
}

template <int RPW, int NL, int NBL, int NS>
hipError_t gateup_mx_launch(const KArgs& a, int routing_given, hipStream_t s, Ev ev) {
  const int P = a.T * a.k + a.T * a.has_shared;
  const dim3 grid((a.F + 4 * RPW - 1) / (4 * RPW), P);
  const size_t lds = mx_gateup_lds(a);
  if (a.E <= 256)
    return launch(k_gateup_mx<RPW, NL, NBL, 4, NS>, grid, 256, lds, s, ev, a, routing_given);
  return launch(k_gateup_mx<RPW, NL, NBL, 16, NS>, grid, 256, lds, s, ev, a, routing_given);
}

// Blocks per lane and row pair of the MX16 kernels for rows of nb blocks.
int mx16_ns(int nb) { return nb <= 64 ? 2 : nb <= 96 ? 3 : nb <= 128 ? 4 : 8; }

// Calls f(RPW, NL, NBL, NS) as integral constants for the plan of rows of K
// weights (NS = 0: 17-byte rows; else the MX16 slots).
template <class Fn>
hipError_t with_mx_plan(int K, bool mx16, Fn&& f) {
  using std::integral_constant;
  MxPlan pl;
  mx_plan(K, &pl);
  const int ns = mx16 ? mx16_ns(K / 32) : 0;
  auto go = [&](auto rpw, auto nl, auto nbl) -> hipError_t {
    constexpr int NBL = decltype(nbl)::value;
    switch (ns) {
      case 0: return f(rpw, nl, nbl, integral_constant<int, 0>{});
      case 2: if constexpr (NBL == 1) return f(rpw, nl, nbl, integral_constant<int, 2>{}); break;
      case 3: if constexpr (NBL == 2) return f(rpw, nl, nbl, integral_constant<int, 3>{}); break;
      case 4: if constexpr (NBL == 2) return f(rpw, nl, nbl, integral_constant<int, 4>{}); break;
      case 8: if constexpr (NBL == 4) return f(rpw, nl, nbl, integral_constant<int, 8>{}); break;
    }
    return hipErrorInvalidValue;
  };
  switch (pl.nl) {
    case 1: return go(integral_constant<int, 3>{}, integral_constant<int, 1>{}, integral_constant<int, 1>{});
    case 2: return go(integral_constant<int, 3>{}, integral_constant<int, 2>{}, integral_constant<int, 1>{});
    case 3:
      if (pl.nbl == 1)
        return go(integral_constant<int, 3>{}, integral_constant<int, 3>{}, integral_constant<int, 1>{});
      return go(integral_constant<int, 3>{}, integral_constant<int, 3>{}, integral_constant<int, 2>{});
    case 5: return go(integral_constant<int, 1>{}, integral_constant<int, 5>{}, integral_constant<int, 2>{});
    default: return go(integral_constant<int, 1>{}, integral_constant<int, 9>{}, integral_constant<int, 4>{});
  }
}

hipError_t gateup_mx(const KArgs& a, int routing_given, hipStream_t s, Ev ev) {
  return with_mx_plan(a.H, a.mx16, [&](auto rpw, auto nl, auto nbl, auto ns) {
    return gateup_mx_launch<decltype(rpw)::value, decltype(nl)::value, decltype(nbl)::value,
                            decltype(ns)::value>(a, routing_given, s, ev);
  });
}

template <int RPW, int NL, int NBL, int NS>
hipError_t down_mx_launch(const KArgs& a, const MxPlan& pl, hipStream_t s, Ev ev) {
  const int R = mx_down_rows(a, pl);
  const dim3 grid((a.H + R - 1) / R, a.T);
  const size_t lds = NS ? 4 * static_cast<size_t>(R) * (a.k + a.has_shared) : mx_down_lds(a, pl);
  return launch(k_down_mx<RPW, NL, NBL, NS>, grid, 512, lds, s, ev, a, R);
}

hipError_t down_mx(const KArgs& a, hipStream_t s, Ev ev) {
  MxPlan pl;
  mx_plan(a.F, &pl);
  return with_mx_plan(a.F, a.mx16, [&](auto rpw, auto nl, auto nbl, auto ns) {
    return down_mx_launch<decltype(rpw)::value, decltype(nl)::value, decltype(nbl)::value,
                          decltype(ns)::value>(a, pl, s, ev);
  });
}

// Candidates per lane of the in-kernel top-k: 4 covers E <= 256.
template <int FMT>
hipError_t gateup_dispatch(const KArgs& a, int routing_given, hipStream_t s, Ev ev) {
  if (FMT == FMT_MXFP4 && mx_gateup_fits(a)) return gateup_mx(a, routing_given, s, ev);
  if (a.E <= 256) return gateup_dispatch_nc<FMT, 4>(a, routing_given, s, ev);
  return gateup_dispatch_nc<FMT, 16>(a, routing_given, s, ev);
}

// h pieces quantized in lock-step per wave: 2, 5 or 8 (more run one at a time).
template <int FMT, int TPG>
hipError_t down_jb(int jobs_per_wave, dim3 grid, size_t lds, hipStream_t s, Ev ev, const KArgs& a,
                   int R, Div dnb, Div dR, Div dpc) {
  if constexpr (FMT == FMT_MXFP4)  // h quantized beforehand (k_hquant_pairs)
    return launch(k_down<FMT, TPG, 2, true>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc);
  if (jobs_per_wave <= 2) return launch(k_down<FMT, TPG, 2, false>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc);
  if (jobs_per_wave <= 5) return launch(k_down<FMT, TPG, 5, false>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc);
  return launch(k_down<FMT, TPG, 8, false>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc);
}

// Plan of the LDS-staged down kernel (Q4_K, Q5_K, Q2_K): one workgroup per
// compute unit where the LDS (q8 of h + R rows per slot) and 8 tasks per lane
// group allow.
int down_lds_bb(int fmt) { return fmt == FMT_Q4_K ? 144 : fmt == FMT_Q5_K ? 176 : fmt == FMT_Q2_K ? 84 : 0; }
struct DownLdsPlan { int R, tpg; size_t lds; };
bool down_lds_plan(const KArgs& a, DownLdsPlan* out) {
  if (down_lds_bb(a.fmt_d) == 0) return false;
  const int ns = a.k + a.has_shared, K = a.F, nb = K / 256;
  const int npc = (nb * down_lds_bb(a.fmt_d) + 15) / 16;  // 16-byte pieces per row
  const int per_token = max(1, 256 / max(a.T, 1));
  int R = max(1, min((a.H + per_token - 1) / per_token, a.H));
  auto lds_of = [&](int r) {
    const size_t pcs = static_cast<size_t>(ns) * r * npc;
    return static_cast<size_t>(down_lds_weights_offset(ns, K, r, nb)) + 16 * ((pcs + 63) / 64 * 64);
  };
  while (R > 1 && (lds_of(R) > kMaxLds || ns * R * nb > 64 * 8)) --R;
  if (lds_of(R) > kMaxLds || ns * R * nb > 64 * 8) return false;
  *out = {R, (ns * R * nb + 63) / 64, lds_of(R)};
  return true;
}

template <int FMT, int TPG>
hipError_t down_lds_jb(int jobs_per_wave, dim3 grid, size_t lds, hipStream_t s, Ev ev,
                       const KArgs& a, int R, Div dnb, Div dR, Div dpc, Div dq) {
  if (jobs_per_wave <= 2) return launch(k_down_lds<FMT, TPG, 2>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc, dq);
  if (jobs_per_wave <= 5) return launch(k_down_lds<FMT, TPG, 5>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc, dq);
  return launch(k_down_lds<FMT, TPG, 8>, grid, 512, lds, s, ev, a, R, dnb, dR, dpc, dq);
}

template <int FMT>
hipError_t down_dispatch(const KArgs& a, hipStream_t s, Ev ev) {
  if (FMT == FMT_MXFP4 && mx_down_fits(a)) return down_mx(a, s, ev);
  if constexpr (FMT == FMT_Q4_K || FMT == FMT_Q5_K || FMT == FMT_Q2_K) {
    DownLdsPlan pl;
    if (down_lds_plan(a, &pl)) {
      const int nb = a.F / 256, pieces = a.F / 256;
      const dim3 grid((a.H + pl.R - 1) / pl.R, a.T);
      const Div dnb = Div::make(nb), dR = Div::make(pl.R), dpc = Div::make(pieces),
                dq = Div::make((nb * FmtOf<FMT>::T::BB + 15) / 16);
      const int jpw = ((a.k + a.has_shared) * pieces + kQuantizers - 1) / kQuantizers;
      switch (tpg_bucket(pl.tpg)) {
        case 1: return down_lds_jb<FMT, 1>(jpw, grid, pl.lds, s, ev, a, pl.R, dnb, dR, dpc, dq);
        case 2: return down_lds_jb<FMT, 2>(jpw, grid, pl.lds, s, ev, a, pl.R, dnb, dR, dpc, dq);
        case 4: return down_lds_jb<FMT, 4>(jpw, grid, pl.lds, s, ev, a, pl.R, dnb, dR, dpc, dq);
        default: return down_lds_jb<FMT, 8>(jpw, grid, pl.lds, s, ev, a, pl.R, dnb, dR, dpc, dq);
      }
    }
  }
  GemvShape sh;
  const size_t lds = down_lds<FMT>(a, &sh);
  dim3 grid((a.H + sh.R - 1) / sh.R, a.T);
  using F = typename FmtOf<FMT>::T;
  const int pieces = (a.F + 255) / 256;
  const Div dnb = Div::make(a.F / F::BE), dR = Div::make(sh.R), dpc = Div::make(pieces);
  const int jobs_per_wave = ((a.k + a.has_shared) * pieces + 3) / 4;
  switch (tpg_bucket(sh.tpg)) {
    case 1: return down_jb<FMT, 1>(jobs_per_wave, grid, lds, s, ev, a, sh.R, dnb, dR, dpc);
    case 2: return down_jb<FMT, 2>(jobs_per_wave, grid, lds, s, ev, a, sh.R, dnb, dR, dpc);
    case 4: return down_jb<FMT, 4>(jobs_per_wave, grid, lds, s, ev, a, sh.R, dnb, dR, dpc);
    default: return down_jb<FMT, 8>(jobs_per_wave, grid, lds, s, ev, a, sh.R, dnb, dR, dpc);
  }
}

}  // namespace

bool gemv_hquant(int fmt_down, int F, int k, int has_shared, bool mx16) {
  if (fmt_down != FMT_MXFP4) return false;
  if (mx16) return true;
  KArgs a{};
  a.fmt_d = fmt_down;
  a.F = F;
  a.k = k;
  a.has_shared = has_shared;
  return !mx_down_fits(a);
}

bool mx16_fits(const KArgs& a) { return mx_gateup_fits(a) && mx_down_fits(a); }

bool gemv_fits(const KArgs& a) {
  GemvShape gs{1, 1}, ds{1, 1};
  size_t g = 0, d = 0;
  with_fmt(a.fmt_gu, [&](auto f) { g = gateup_lds<decltype(f)::value>(a, &gs); });
  with_fmt(a.fmt_d, [&](auto f) { d = down_lds<decltype(f)::value>(a, &ds); });
  DownLdsPlan pl;
  if (down_lds_plan(a, &pl)) {
    d = pl.lds;
    ds.tpg = pl.tpg;
  }
  if (mx_gateup_fits(a)) {
    g = 0;
    gs.tpg = 1;
  }
  if (mx_down_fits(a)) {
    d = 0;
    ds.tpg = 1;
  }
  // the GEMV kernels are instantiated for at most 8 block tasks per lane
  // group (tpg_bucket): wider rows would leave blocks uncomputed
  return g <= kMaxLds && d <= kMaxLds && gs.tpg <= 8 && ds.tpg <= 8;
}

hipError_t launch_quant(const void* x, int dtype, int T, int H, int B, int8_t* qs, float* d,
                        int16_t* bs, hipStream_t s) {
  dim3 grid((H + 255) / 256, T);
  if (B == 256) return launch(k_quant<256>, grid, 64, 0, s, Ev{}, x, dtype, H, qs, d, bs);
  return launch(k_quant<32>, grid, 64, 0, s, Ev{}, x, dtype, H, qs, d,
                static_cast<int16_t*>(nullptr));
}

hipError_t launch_zero(uint32_t* p, int n, hipStream_t s, Ev ev) {
  return launch(k_zero, dim3(1), 256, 0, s, ev, p, n);
}

hipError_t launch_shared_gate(const KArgs& a, hipStream_t s) {
  return launch(k_shared_gate, dim3(a.T), 256, 0, s, Ev{}, a);
}

hipError_t launch_router(const KArgs& a, bool quant, int n_clear, hipStream_t s, Ev ev) {
  const int nq = quant ? a.T * ((a.H + 255) / 256) : 0;
  dim3 grid(a.E + (a.sh_gate_vec ? 1 : 0) + nq);
  const int q = quant ? 1 : 0;
  if (a.T == 1) {
    if (a.x_dtype) return launch(k_router<1, 8, true>, grid, 64, 0, s, ev, a, q, n_clear);
    return launch(k_router<1, 8, false>, grid, 64, 0, s, ev, a, q, n_clear);
  }
  if (a.x_dtype) return launch(k_router<4, 4, true>, grid, 64, 0, s, ev, a, q, n_clear);
  return launch(k_router<4, 4, false>, grid, 64, 0, s, ev, a, q, n_clear);
}

hipError_t launch_topk(const KArgs& a, hipStream_t s) {
  if (a.E <= 256) return launch(k_topk<4>, dim3((a.T + 3) / 4), 256, 0, s, Ev{}, a);
  return launch(k_topk<16>, dim3((a.T + 3) / 4), 256, 0, s, Ev{}, a);
}

hipError_t launch_gateup(const KArgs& a, bool routing_given, hipStream_t s, Ev ev) {
  hipError_t e = hipErrorInvalidValue;
  with_fmt(a.fmt_gu, [&](auto f) { e = gateup_dispatch<decltype(f)::value>(a, routing_given, s, ev); });
  return e;
}

hipError_t launch_hquant_pairs(const KArgs& a, hipStream_t s, Ev ev) {
  const int P = a.T * a.k + a.T * a.has_shared;
  const int pieces = (a.F + 255) / 256;
  return launch(k_hquant_pairs, dim3((P * pieces + 3) / 4), 256, 0, s, ev, a, P, Div::make(pieces));
}

hipError_t launch_down(const KArgs& a, hipStream_t s, Ev ev) {
  hipError_t e = hipErrorInvalidValue;
  with_fmt(a.fmt_d, [&](auto f) { e = down_dispatch<decltype(f)::value>(a, s, ev); });
  return e;
}

template <int NL, int NBL>
hipError_t block_dots_mx_launch(const uint8_t* r, int n_rows, int K, size_t stride,
                                const int8_t* qs, const float* d, int32_t* out, hipStream_t s) {
  const int nb = K / 32;
  const size_t lds = static_cast<size_t>(mx_gu_scratch_offset(nb)) + mx_scratch_bytes(nb);
  return launch(k_block_dots_mx<NL, NBL>, dim3((n_rows + 1) / 2), 64, lds, s, Ev{}, r, n_rows, K,
                stride, qs, d, out);
}

hipError_t launch_block_dots(int fmt, const void* rows, int n_rows, int K, size_t stride,
                             const int8_t* qs, const float* d, const int16_t* bs, int32_t* out,
                             hipStream_t s) {
  const uint8_t* r = static_cast<const uint8_t*>(rows);
  const size_t lds = (fmt == FMT_MXFP4 ? 5 * K / 2 : K) + 4 * (K / 32) + 2 * (K / 16);
  if (fmt < FMT_Q4_K || fmt > FMT_Q5_1) return hipErrorInvalidValue;
  MxPlan pl;
  if (fmt == FMT_MXFP4 && mx_plan(K, &pl)) {
    // rows the realigning MXFP4 kernels take (the same plans as k_gateup_mx)
    switch (pl.nl) {
      case 1: return block_dots_mx_launch<1, 1>(r, n_rows, K, stride, qs, d, out, s);
      case 2: return block_dots_mx_launch<2, 1>(r, n_rows, K, stride, qs, d, out, s);
      case 3:
        if (pl.nbl == 1) return block_dots_mx_launch<3, 1>(r, n_rows, K, stride, qs, d, out, s);
        return block_dots_mx_launch<3, 2>(r, n_rows, K, stride, qs, d, out, s);
      case 5: return block_dots_mx_launch<5, 2>(r, n_rows, K, stride, qs, d, out, s);
      default: return block_dots_mx_launch<9, 4>(r, n_rows, K, stride, qs, d, out, s);
    }
  }
  hipError_t e = hipErrorInvalidValue;
  // MXFP4 rows past the realigning kernels' plans take the per-block routine
  with_fmt(fmt, [&](auto f) {
    e = launch(k_block_dots<decltype(f)::value>, dim3(n_rows), 256, lds, s, Ev{}, r, K, stride, qs,
               d, bs, out);
  });
  return e;
}

hipError_t launch_block_dots_mx16(const void* rows, int n_rows, int K, size_t stride,
                                  const int8_t* qs, const float* d, int32_t* out, hipStream_t s) {
  const uint8_t* r = static_cast<const uint8_t*>(rows);
  const size_t lds = static_cast<size_t>(84) * (K / 32);
  return with_mx_plan(K, true, [&](auto, auto, auto nbl, auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value, NBL = decltype(nbl)::value;
    if constexpr (NS == 0) return hipErrorInvalidValue;
    else
      return launch(k_block_dots_mx16<NS, NBL>, dim3((n_rows + 1) / 2), 64, lds, s, Ev{}, r,
                    n_rows, K, stride, qs, d, out);
  });
}

hipError_t launch_repack_mx16(const uint8_t* src, size_t stride, int n_rows, int nb, uint8_t* dst,
                              size_t dst_stride, hipStream_t s) {
  const int rb = static_cast<int>(mx16_row_bytes(nb));
  const size_t total = static_cast<size_t>(n_rows) * rb;
  const size_t grid = std::min<size_t>((total + 255) / 256, 65536);
  return launch(k_repack_mx16, dim3(static_cast<unsigned>(grid)), 256, 0, s, Ev{}, src, stride, nb,
                dst, dst_stride, rb, total);
}

}  // namespace moe
