#pragma once
// Device-side building blocks of the routed-expert MoE FFN kernels (gfx950):
// block formats, q8 activation quantization, lane reductions and top-k.
//
// Block formats (ggml/GGUF conventions; OCP MX v1.0 for MXFP4):
//   Q4_K  144 B / 256: fp16 d, fp16 dmin, 12 B of 6-bit sub-block scales and
//         mins, 128 B of nibbles (byte i of 32-byte chunk c: weight 64c+i low,
//         64c+32+i high). w = d*sc_j*q - dmin*m_j, j = sub-block of 32.
//   Q6_K  210 B / 256: ql[128], qh[64], int8 scales[16], fp16 d.
//         w = d*sc_s*(q - 32), s = sub-block of 16.
//   MXFP4 17 B / 32: E8M0 scale byte, 16 B of e2m1 nibbles (byte i: element i
//         low, element i+16 high). w = e2m1 * 2^(e-127).
// Every dot product is an integer (or exact fp32) sum of weight quants times
// activation quants per block, rescaled per block in fp32: the integer-dot
// numerics the Pulsar README describes for its q8_K/q8_0 activations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace dev {


typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global-address-space views. Weight pointers often come from LDS tables, where
// the compiler cannot prove they are global and would emit FLAT loads; FLAT
// loads also count against lgkmcnt, so any later LDS wait would drain them.
#define MOE_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const MOE_GLOBAL T* gp(const void* p) {
  return (const MOE_GLOBAL T*)(p);
}

// Streaming (non-temporal) 16-byte load: expert weights are read once per call.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(gp<u32x4>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt4(const void* p) {
  return __builtin_nontemporal_load(gp<uint32_t>(p));
}
__device__ __forceinline__ uint16_t ld_nt2(const void* p) {
  return __builtin_nontemporal_load(gp<uint16_t>(p));
}

#define MOE_LDS __attribute__((address_space(3)))

// Direct global->LDS loads. Written as inline asm so that the compiler does not
// track their LDS writes: its tracking loses count across the ring's loop and
// would wait for every slot load in flight before any LDS read. Completion is
// ordered by the explicit vmcnt waits and workgroup barriers of the ring. (The
// compiler's own vmcnt waits for other loads stay sufficient: loads complete
// in issue order, so extra ops it does not see only make them stronger.)
// Lane l of one instruction writes its 16 (or 4) bytes at M0 + 16 l (4 l).
// LDS byte address of a (wave-uniform) pointer into a __shared__ array, as an
// SGPR value for M0.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* l) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const MOE_LDS uint8_t*)(l))));
}
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* l) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr(l))
               : "memory", "m0");
}
// Non-temporal variant for weights read once (keeps them from displacing
// reused lines in the caches).
__device__ __forceinline__ void dma16_nt(const uint8_t* g, uint8_t* l) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_addr(l))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint8_t* l) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_addr(l))
               : "memory", "m0");
}
// Wait until at most N vector memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}


__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float load_x(const void* x, int dtype, size_t i) {
  return dtype == 0 ? static_cast<const float*>(x)[i]
                    : bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// Four consecutive x values (i a multiple of 4) with one load.
__device__ __forceinline__ void load_x4(const void* x, int dtype, size_t i, float (&v)[4]) {
  if (dtype == 0) {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + i);
    v[0] = bf16_bits_to_f32(b.x & 0xFFFF); v[1] = bf16_bits_to_f32(b.x >> 16);
    v[2] = bf16_bits_to_f32(b.y & 0xFFFF); v[3] = bf16_bits_to_f32(b.y >> 16);
  }
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Sum over aligned groups of 8 lanes with DPP; every lane of the group gets the sum.
__device__ __forceinline__ int sum8(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return v;
}

// ---- DPP reductions. Prefix over 16-lane rows with row_shr 1/2/4/8, then
// row_bcast 15/31 carry row results upward; lane 63 ends with the full value,
// which readlane makes wave-uniform. For sums, lanes without a source add 0;
// for max, they keep their own value.
// Where 0 is the identity (sums, maxima of non-negative values) lanes without a
// source read 0 (bound_ctrl), which lets the move fold into the DPP form of the
// arithmetic instruction.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_f(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true);
  return v + __int_as_float(o);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_amax_f(float v) {  // v >= 0
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true);
  return fmaxf(v, __int_as_float(o));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_f(float v) {
  const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK,
                                            0xF, false);
  return fmaxf(v, __int_as_float(o));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, ROW_MASK, 0xF,
                                             false);
  return v + __longlong_as_double((static_cast<long long>(hi) << 32) |
                                  static_cast<uint32_t>(lo));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add_f<0x111, 0xF>(v);
  v = dpp_add_f<0x112, 0xF>(v);
  v = dpp_add_f<0x114, 0xF>(v);
  v = dpp_add_f<0x118, 0xF>(v);
  v = dpp_add_f<0x142, 0xA>(v);
  v = dpp_add_f<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max_f<0x111, 0xF>(v);
  v = dpp_max_f<0x112, 0xF>(v);
  v = dpp_max_f<0x114, 0xF>(v);
  v = dpp_max_f<0x118, 0xF>(v);
  v = dpp_max_f<0x142, 0xA>(v);
  v = dpp_max_f<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Max of non-negative values over the wave.
__device__ __forceinline__ float wave_amax(float v) {
  v = dpp_amax_f<0x111, 0xF>(v);
  v = dpp_amax_f<0x112, 0xF>(v);
  v = dpp_amax_f<0x114, 0xF>(v);
  v = dpp_amax_f<0x118, 0xF>(v);
  v = dpp_amax_f<0x142, 0xA>(v);
  v = dpp_amax_f<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ double wave_sum_d(double v) {
  v = dpp_add_d<0x111, 0xF>(v);
  v = dpp_add_d<0x112, 0xF>(v);
  v = dpp_add_d<0x114, 0xF>(v);
  v = dpp_add_d<0x118, 0xF>(v);
  v = dpp_add_d<0x142, 0xA>(v);
  v = dpp_add_d<0x143, 0xC>(v);
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Max of non-negative values over aligned groups of 8 lanes (every lane of the
// group gets it; quad_perm and row_half_mirror give every lane a source).
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true)));
  return v;
}

// Sum over aligned groups of 4 lanes (every lane of the quad gets it).
__device__ __forceinline__ int sum4(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  return v;
}

// ------------------------------------------------------------ q8 quantization
// One wave quantizes 256 consecutive values, 4 per lane (lane l: 4l..4l+3), as
// blocks of B = 256 (one block) or B = 32 (eight blocks of 8 lanes).
// fp32 recipe: amax; iscale = 127/amax (IEEE division); q = rne(v * iscale)
// clamped to +-127; d = amax/127; amax == 0 gives d = 0 and q = 0.
// Lanes past the end pass zeros (whole blocks only) and store nothing.
template <int B>
__device__ __forceinline__ float quant_wave_q(const float v[4], int q[4]) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  static_assert(B == 256 || B == 32, "block of 256 (one per wave) or 32 (8 lanes)");
  amax = B == 256 ? wave_amax(amax) : max8(amax);
  if (amax == 0.0f) {
    q[0] = q[1] = q[2] = q[3] = 0;
    return 0.0f;
  }
  const float iscale = 127.0f / amax;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = __builtin_rintf(v[i] * iscale);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    q[i] = static_cast<int>(r);
  }
  return amax / 127.0f;
}

// NJ independent 256-value pieces quantized in lock-step by one wave, so the
// dependent chains (DPP max, divisions) of different pieces interleave.
// Same fp32 recipe as quant_wave_q.
template <int B, int NJ>
__device__ __forceinline__ void quant_wave_batch(const float4 (&hv)[NJ], int (&q)[NJ][4],
                                                 float (&dv)[NJ]) {
  float am[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    am[j] = fmaxf(fmaxf(fabsf(hv[j].x), fabsf(hv[j].y)), fmaxf(fabsf(hv[j].z), fabsf(hv[j].w)));
  if constexpr (B == 256) {
#define MOE_BSTEP(CTRL, RM) _Pragma("unroll") for (int j = 0; j < NJ; ++j) am[j] = dpp_amax_f<CTRL, RM>(am[j]);
    MOE_BSTEP(0x111, 0xF) MOE_BSTEP(0x112, 0xF) MOE_BSTEP(0x114, 0xF) MOE_BSTEP(0x118, 0xF)
    MOE_BSTEP(0x142, 0xA) MOE_BSTEP(0x143, 0xC)
#undef MOE_BSTEP
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      am[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am[j]), 63));
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) am[j] = max8(am[j]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float v[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w};
    if (am[j] == 0.0f) {
      q[j][0] = q[j][1] = q[j][2] = q[j][3] = 0;
      dv[j] = 0.0f;
    } else {
      const float iscale = 127.0f / am[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float r = __builtin_rintf(v[i] * iscale);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q[j][i] = static_cast<int>(r);
      }
      dv[j] = am[j] / 127.0f;
    }
  }
}

__device__ __forceinline__ uint32_t pack_q8x4(const int q[4]) {
  return (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) |
         (static_cast<uint32_t>(q[3] & 0xFF) << 24);
}

// Stores as int8 quants + scales (+ 16-element sums for B = 256).
template <int B>
__device__ __forceinline__ void quant_wave(const float v[4], bool valid, int lane, int8_t* qs,
                                           float* d, int16_t* bs) {
  int q[4];
  const float dv = quant_wave_q<B>(v, q);
  constexpr int G = B / 4;
  if (valid) {
    const uint32_t packed = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) |
                            (static_cast<uint32_t>(q[3] & 0xFF) << 24);
    reinterpret_cast<uint32_t*>(qs)[lane] = packed;
    if ((lane % G) == 0) d[lane / G] = dv;
  }
  if (B == 256) {
    const int sm = sum4(q[0] + q[1] + q[2] + q[3]);
    if (valid && (lane & 3) == 0) bs[lane >> 2] = static_cast<int16_t>(sm);
  }
}

// ---------------------------------------------------------------- MXFP8
// OCP MX v1.0 MXFP8 (E4M3 elements, one E8M0 scale per 32). Code of the E4M3
// value nearest to y (ties to even), saturating at +-448; zero -> +0.
// Normal range (|y| >= 2^-6): the fp32 bits rounded to 3 mantissa bits (the
// carry moves into the exponent), rebiased from 127 to 7; below: multiples of
// the smallest subnormal 2^-9 (8 of them is the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t bits = __float_as_uint(y), mag = bits & 0x7FFFFFFFu;
  uint32_t c;
  if (mag >= 0x3C800000u) {  // 2^-6
    const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
    c = min((r >> 20) - (120u << 3), 0x7Eu);
  } else {
    c = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(mag) * 512.0f));
  }
  return c == 0 ? 0u : (c | ((bits >> 24) & 0x80u));
}

// Scale byte of a block with maximum magnitude amax: floor(log2 amax) - 8
// (8 = E4M3's largest normal exponent) + 127, within [0, 254]; 0 for amax 0.
__device__ __forceinline__ int mx8_scale_byte(float amax) {
  if (amax == 0.0f) return 0;
  const int k = __builtin_amdgcn_frexp_expf(amax);  // amax = f 2^k, f in [0.5, 1)
  return min(max(k - 1 - 8 + 127, 0), 254);
}

// One wave quantizes a 256-value piece (lane l holds elements 4l .. 4l + 3;
// 8 lanes per block of 32) to MXFP8 and stores each block pair-interleaved:
// byte 2j = element j, byte 2j + 1 = element j + 16 (the pairing of an MXFP4
// block's nibble bytes, and the K order of the block-scaled MFMA). q points at
// the piece's first block, e at its first scale byte. valid: lane's 4 values
// exist (whole blocks are valid or not).
__device__ __forceinline__ void quant_wave_mx8(const float (&v)[4], bool valid, int lane,
                                               uint8_t* q, uint8_t* e) {
  float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  am = max8(am);
  const int sb = mx8_scale_byte(am);
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = e4m3_code(__builtin_ldexpf(v[i], 127 - sb));
  const uint32_t mine = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  // the lane 4 ahead holds elements 16.. of the same positions (row_shl:4)
  const uint32_t other = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(mine), 0x104, 0xF, 0xF, false));
  const int bl = lane >> 3, j = lane & 7;  // block, lane in block
  if (valid && j < 4) {
    const uint32_t lo = __builtin_amdgcn_perm(other, mine, 0x05010400u);
    const uint32_t hi = __builtin_amdgcn_perm(other, mine, 0x07030602u);
    *reinterpret_cast<uint2*>(q + 32 * bl + 8 * j) = make_uint2(lo, hi);
  }
  if (valid && j == 0) e[bl] = static_cast<uint8_t>(sb);
}

// fp16 pairs per block in the MXFP4 activation layout: 16 used + 4 of padding
// (80 bytes), so that lanes reading consecutive blocks with 16-byte loads hit
// different LDS banks.
constexpr int kApPitch = 20;

// B = 32 quantization stored as fp16 pairs (a[i], a[i+16]) per block, the layout
// the MXFP4 dot reads: ap gets the 8 blocks of the 256-value piece.
// Stores the pairs block-major: ap[block * kApPitch + q] (see ActView), with ap
// pointing at the piece's first block; each lane writes 4 consecutive pairs.
__device__ __forceinline__ void store_pairs(const int (&q)[4], float dv, bool valid, int lane,
                                            half2_t* ap, float* d) {
  int o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // partner 16 elements ahead: lane + 4 (DPP row_shl:4)
    o[i] = __builtin_amdgcn_update_dpp(0, q[i], 0x104, 0xF, 0xF, false);
  const int bl = lane >> 3, off = 4 * (lane & 7);
  if (valid && off < 16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(uint32_t, half2_t{static_cast<_Float16>(q[i]), static_cast<_Float16>(o[i])});
    *reinterpret_cast<uint4*>(ap + bl * kApPitch + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (valid && (lane & 7) == 0) d[bl] = dv;
}
__device__ __forceinline__ void quant_wave_pairs(const float v[4], bool valid, int lane,
                                                 half2_t* ap, float* d) {
  int q[4];
  const float dv = quant_wave_q<32>(v, q);
  store_pairs(q, dv, valid, lane, ap, d);
}

// Activations of one row vector as the dot routines read them (LDS).
struct ActView {
  const int8_t* qs;     // [K] (Q8_K)
  const float* d;       // [K / B]
  const int16_t* bs;    // [K / 16] (Q8_K)
  // [K / 32][kApPitch] fp16 pairs (Q8_32), block-major: ap[b * kApPitch + i] =
  // (a[32b+i], a[32b+16+i]) for i < 16 (then padding): one block is four
  // 16-byte reads, and lanes that take consecutive blocks start 80 bytes
  // apart (different banks)
  const half2_t* ap;
};

// ------------------------------------------------------------------ formats
// Each format: BE elements and BB bytes per block, LPB lanes cooperate on one
// block. load() reads the lane's share of a block from global memory;
// partials() returns the block's integer partials (summed over the LPB lanes);
// value() turns them into the fp32 block value d8 * (...).

struct FmtQ4K {
  static constexpr int BE = 256, BB = 144, LPB = 8;
  struct Raw { uint4 hdr, q; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int sub) {
    r.hdr = ld_nt16(blk);
    r.q = ld_nt16(blk + 16 + 16 * sub);
  }
  // the same share from a block staged in LDS
  __device__ static __forceinline__ void lds_load(Raw& r, const uint8_t* blk, int sub) {
    r.hdr = *reinterpret_cast<const uint4*>(blk);
    r.q = *reinterpret_cast<const uint4*>(blk + 16 + 16 * sub);
  }
  // Lane `sub` holds qs bytes 16*sub..16*sub+15: chunk c = sub/2, half hh = sub%2, i.e.
  // weights 64c+16hh+i (low nibbles, sub-block 2c) and 64c+32+16hh+i (high, 2c+1).
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int sub) {
    const int c = sub >> 1, hh = sub & 1;
    const int4* ax = reinterpret_cast<const int4*>(a.qs + b * 256);
    const int4 alo = ax[4 * c + hh];
    const int4 ahi = ax[4 * c + 2 + hh];
    int dl = 0, dh = 0;
    dl = sdot4(r.q.x & 0x0F0F0F0F, alo.x, dl);
    dl = sdot4(r.q.y & 0x0F0F0F0F, alo.y, dl);
    dl = sdot4(r.q.z & 0x0F0F0F0F, alo.z, dl);
    dl = sdot4(r.q.w & 0x0F0F0F0F, alo.w, dl);
    dh = sdot4((r.q.x >> 4) & 0x0F0F0F0F, ahi.x, dh);
    dh = sdot4((r.q.y >> 4) & 0x0F0F0F0F, ahi.y, dh);
    dh = sdot4((r.q.z >> 4) & 0x0F0F0F0F, ahi.z, dh);
    dh = sdot4((r.q.w >> 4) & 0x0F0F0F0F, ahi.w, dh);
    return scaled(r.hdr, dl, dh, a, b, sub);
  }
  // The lane's share of the block partials from its two sub-block dots (dl:
  // sub-block 2c, dh: 2c + 1; c = sub / 2): sum over the 8 lanes of sc * dot and
  // of m * (16-element activation sums).
  __device__ static __forceinline__ int2 scaled(const uint4& hdr, int dl, int dh,
                                                const ActView& a, int b, int sub) {
    const int c = sub >> 1, hh = sub & 1;
    // 6-bit scales/mins of the 8 sub-blocks as bytes: sub-blocks 0..3 sit in the
    // low 6 bits of scale bytes 0..3 (sc) and 4..7 (m); 4..7 take their low 4
    // bits from bytes 8..11 and their top 2 bits from bits 6..7 of bytes 0..7.
    const uint32_t s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;
    const uint32_t sc03 = s0 & 0x3F3F3F3Fu, m03 = s1 & 0x3F3F3F3Fu;
    const uint32_t sc47 = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
    const uint32_t m47 = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
    const uint32_t scw = c < 2 ? sc03 : sc47, mw = c < 2 ? m03 : m47;
    const int sh = 16 * (c & 1);
    const int sc0 = (scw >> sh) & 0xFF, sc1 = (scw >> (sh + 8)) & 0xFF;
    const int m0 = (mw >> sh) & 0xFF, m1 = (mw >> (sh + 8)) & 0xFF;
    const int16_t* bs = a.bs + b * 16;
    const int S1 = sc0 * dl + sc1 * dh;
    const int S2 = m0 * bs[4 * c + hh] + m1 * bs[4 * c + 2 + hh];
    return make_int2(sum8(S1), sum8(S2));
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    const float d = half_bits_to_f32(r.hdr.x & 0xFFFF), dmin = half_bits_to_f32(r.hdr.x >> 16);
    return d8 * (d * static_cast<float>(p.x) - dmin * static_cast<float>(p.y));
  }
};

// 8 bytes at a 2-byte aligned address: dwords at p & ~3, the next one, and the
// one holding byte p + 7, so no dword read lies wholly outside [p, p + 8).
__device__ __forceinline__ uint2 load8_unaligned(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(a & ~static_cast<uintptr_t>(3));
  const uint8_t* w_last = reinterpret_cast<const uint8_t*>((a + 7) & ~static_cast<uintptr_t>(3));
  const uint32_t sh = static_cast<uint32_t>(a & 3);
  const uint32_t w0 = ld_nt4(w), w1 = ld_nt4(w + 4), w2 = ld_nt4(w_last);
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}

// Q5_K: Q4_K's header and nibble layout (nibbles at byte 48) plus 32 bytes of
// fifth bits at byte 16: bit 2c of qh[l] belongs to weight 64c + l, bit 2c + 1
// to weight 64c + 32 + l. Lane `sub` (chunk c = sub / 2, half hh = sub % 2)
// needs qh[16 hh .. 16 hh + 15], the same l as its nibble bytes.
struct FmtQ5K {
  static constexpr int BE = 256, BB = 176, LPB = 8;
  struct Raw { uint4 hdr, qh, q; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int sub) {
    r.hdr = ld_nt16(blk);
    r.qh = ld_nt16(blk + 16 + 16 * (sub & 1));
    r.q = ld_nt16(blk + 48 + 16 * sub);
  }
  __device__ static __forceinline__ void lds_load(Raw& r, const uint8_t* blk, int sub) {
    r.hdr = *reinterpret_cast<const uint4*>(blk);
    r.qh = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (sub & 1));
    r.q = *reinterpret_cast<const uint4*>(blk + 48 + 16 * sub);
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int sub) {
    const int c = sub >> 1, hh = sub & 1;
    const int4* ax = reinterpret_cast<const int4*>(a.qs + b * 256);
    const int4 alo = ax[4 * c + hh];
    const int4 ahi = ax[4 * c + 2 + hh];
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    const uint32_t h[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
    const int al[4] = {alo.x, alo.y, alo.z, alo.w}, ah[4] = {ahi.x, ahi.y, ahi.z, ahi.w};
    int dl = 0, dh = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (q[i] & 0x0F0F0F0Fu) | (((h[i] >> (2 * c)) & 0x01010101u) << 4);
      const uint32_t hi = ((q[i] >> 4) & 0x0F0F0F0Fu) | (((h[i] >> (2 * c + 1)) & 0x01010101u) << 4);
      dl = sdot4(static_cast<int>(lo), al[i], dl);
      dh = sdot4(static_cast<int>(hi), ah[i], dh);
    }
    return FmtQ4K::scaled(r.hdr, dl, dh, a, b, sub);
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    const float d = half_bits_to_f32(r.hdr.x & 0xFFFF), dmin = half_bits_to_f32(r.hdr.x >> 16);
    return d8 * (d * static_cast<float>(p.x) - dmin * static_cast<float>(p.y));
  }
};

// Q2_K (84 B): scales[16] (scale | min << 4, one per 16 weights), qs[64] at
// byte 16 (half h: bits 2j..2j+1 of qs[32h + l] is weight 128h + 32j + l), fp16 d
// and dmin at byte 80. Lane `sub` (half h = sub / 4, k = sub % 4) takes qs bytes
// 32h + 8k .. + 8, i.e. weights 128h + 32j + 8k + i (j < 4, i < 8) of sub-blocks
// 8h + 2j + k / 2; all its fields are dword-aligned in the block.
struct FmtQ2K {
  static constexpr int BE = 256, BB = 84, LPB = 8;
  struct Raw { uint2 q, sc; uint32_t dd; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int sub) {
    const int h = sub >> 2, k = sub & 3;
    const uint8_t* qs = blk + 16 + 32 * h + 8 * k;
    r.q = make_uint2(ld_nt4(qs), ld_nt4(qs + 4));
    r.sc = make_uint2(ld_nt4(blk + 8 * h), ld_nt4(blk + 8 * h + 4));
    r.dd = ld_nt4(blk + 80);
  }
  // from a block staged in LDS at a dword-aligned address: dword reads only
  __device__ static __forceinline__ void lds_load(Raw& r, const uint8_t* blk, int sub) {
    const int h = sub >> 2, k = sub & 3;
    const uint32_t* qs = reinterpret_cast<const uint32_t*>(blk + 16 + 32 * h + 8 * k);
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(blk + 8 * h);
    r.q = make_uint2(qs[0], qs[1]);
    r.sc = make_uint2(sc[0], sc[1]);
    r.dd = *reinterpret_cast<const uint32_t*>(blk + 80);
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int sub) {
    const int h = sub >> 2, k = sub & 3;
    const int8_t* ab = a.qs + b * 256 + 128 * h + 8 * k;
    const int16_t* bs = a.bs + b * 16 + 8 * h + (k >> 1);
    int S1 = 0, S2 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int2 av = *reinterpret_cast<const int2*>(ab + 32 * j);
      int dot = sdot4(static_cast<int>((r.q.x >> (2 * j)) & 0x03030303u), av.x, 0);
      dot = sdot4(static_cast<int>((r.q.y >> (2 * j)) & 0x03030303u), av.y, dot);
      // scale byte 2j + k / 2 of the eight at 8h
      const uint32_t sw = j < 2 ? r.sc.x : r.sc.y;
      const int byte = (sw >> (8 * (2 * (j & 1) + (k >> 1)))) & 0xFF;
      S1 += (byte & 15) * dot;
      if ((k & 1) == 0) S2 += (byte >> 4) * bs[2 * j];  // one lane of each pair adds the min term
    }
    return make_int2(sum8(S1), sum8(S2));
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    const float d = half_bits_to_f32(r.dd & 0xFFFF), dmin = half_bits_to_f32(r.dd >> 16);
    return d8 * (d * static_cast<float>(p.x) - dmin * static_cast<float>(p.y));
  }
};

struct FmtQ6K {
  static constexpr int BE = 256, BB = 210, LPB = 8;
  // Lane `sub`: half h = sub/4, j = sub%4 holds element i in [8j, 8j+8) of the four
  // quarters of half h: ql[64h+8j..], ql[64h+32+8j..], qh[32h+8j..].
  struct Raw { uint2 l0, l1, qh, sc; uint32_t dbits; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int sub) {
    const int h = sub >> 2, j = sub & 3;
    r.l0 = load8_unaligned(blk + 64 * h + 8 * j);
    r.l1 = load8_unaligned(blk + 64 * h + 32 + 8 * j);
    r.qh = load8_unaligned(blk + 128 + 32 * h + 8 * j);
    r.sc = load8_unaligned(blk + 192 + 8 * h);
    r.dbits = ld_nt2(blk + 208);
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int sub) {
    const int h = sub >> 2, j = sub & 3;
    const int8_t* ab = a.qs + b * 256 + 128 * h + 8 * j;
    const int16_t* bs = a.bs + b * 16;
    int S = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint2 lo = (qq & 1) ? r.l1 : r.l0;
      const int lsh = (qq >> 1) * 4;
      const int hsh = 2 * qq;
      const uint32_t w0 = ((lo.x >> lsh) & 0x0F0F0F0Fu) | (((r.qh.x >> hsh) & 0x03030303u) << 4);
      const uint32_t w1 = ((lo.y >> lsh) & 0x0F0F0F0Fu) | (((r.qh.y >> hsh) & 0x03030303u) << 4);
      const int2 av = *reinterpret_cast<const int2*>(ab + 32 * qq);
      int dot = sdot4(static_cast<int>(w0), av.x, 0);
      dot = sdot4(static_cast<int>(w1), av.y, dot);
      const int sidx = 2 * qq + (j >> 1);  // sub-block 8h + sidx
      const uint32_t scw = sidx < 4 ? r.sc.x : r.sc.y;
      const int sc = static_cast<int>(static_cast<int8_t>((scw >> (8 * (sidx & 3))) & 0xFF));
      // q is stored with +32: subtract 32 * (sum of a over the sub-block) once per sub-block
      const int corr = (j & 1) ? 0 : 32 * bs[8 * h + sidx];
      S += sc * (dot - corr);
    }
    return make_int2(sum8(S), 0);
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    return d8 * half_bits_to_f32(r.dbits) * static_cast<float>(p.x);
  }
};

struct FmtMXFP4 {
  static constexpr int BE = 32, BB = 17, LPB = 1;
  struct Raw { uint32_t w[5]; uint32_t sh; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(blk);
    const uint8_t* p = reinterpret_cast<const uint8_t*>(a & ~static_cast<uintptr_t>(3));
    r.sh = static_cast<uint32_t>(a & 3);
#pragma unroll
    for (int i = 0; i < 5; ++i) r.w[i] = ld_nt4(p + 4 * i);
  }
  __device__ static __forceinline__ uint32_t scale_byte(const Raw& r) {
    return (r.w[0] >> (8 * r.sh)) & 0xFF;
  }
  // Exact: e2m1 values and int8 activations are exact in fp16, products exact in
  // fp32 and every partial sum is a multiple of 0.5 below 2^23.
  __device__ static __forceinline__ float dot(const Raw& r, const ActView& a, int b) {
    const uint4* ap = reinterpret_cast<const uint4*>(a.ap + kApPitch * b);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qw = r.sh == 3 ? r.w[i + 1]
                                    : __builtin_amdgcn_alignbyte(r.w[i + 1], r.w[i], r.sh + 1);
      const uint4 pr = ap[i];  // pairs 4 i .. 4 i + 3 (byte j of qw holds pair 4 i + j)
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 0),
                                   __builtin_bit_cast(half2_t, pr.x), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 1),
                                   __builtin_bit_cast(half2_t, pr.y), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 2),
                                   __builtin_bit_cast(half2_t, pr.z), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 3),
                                   __builtin_bit_cast(half2_t, pr.w), acc, false);
    }
    return acc;
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int) {
    return make_int2(static_cast<int>(2.0f * dot(r, a, b)), 0);
  }
  __device__ static __forceinline__ float value_from_dot(const Raw& r, float s, float d8) {
    return d8 * __builtin_ldexpf(s, static_cast<int>(scale_byte(r)) - 127);
  }
};

// Q3_K (110 B): hmask[32] @0, qs[64] @32, 12 scale bytes @96, fp16 d @108.
// Weight 128h + 32j + l has low bits 2j..2j+1 of qs[32h + l] and high bit
// 4h + j of hmask[l]; q = low + 4 high - 4 in -4..3. Sub-block s (16
// weights) has a 6-bit scale (used as sc - 32): low 4 bits in scale byte
// s mod 8 (low nibble for s < 8, high for s >= 8), top 2 bits at 2 (s / 4) of
// scale byte 8 + s mod 4. Lane `sub` (half h = sub / 4, k = sub % 4) takes
// weights 128h + 32j + 8k + i (j < 4, i < 8): qs[32h + 8k ..] and hmask[8k ..]
// (8 bytes each), one sub-block per j.
struct FmtQ3K {
  static constexpr int BE = 256, BB = 110, LPB = 8;
  struct Raw { uint2 q, hm; uint32_t sc[3]; uint32_t dbits; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int sub) {
    const int h = sub >> 2, k = sub & 3;
    r.q = load8_unaligned(blk + 32 + 32 * h + 8 * k);
    r.hm = load8_unaligned(blk + 8 * k);
    const uint2 s01 = load8_unaligned(blk + 96);
    r.sc[0] = s01.x; r.sc[1] = s01.y;
    const uint2 s2d = load8_unaligned(blk + 102);  // bytes 102..109: scale bytes 8..11, d
    r.sc[2] = (s2d.x >> 16) | (s2d.y << 16);
    r.dbits = s2d.y >> 16;
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int sub) {
    const int h = sub >> 2, k = sub & 3;
    const int8_t* ab = a.qs + b * 256 + 128 * h + 8 * k;
    int S = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // q + 4 per byte: low 2 bits | high bit << 2, then - 4 without carries
      const uint32_t hb = 4 * h + j;
      uint32_t w0 = ((r.q.x >> (2 * j)) & 0x03030303u) | (((r.hm.x >> hb) & 0x01010101u) << 2);
      uint32_t w1 = ((r.q.y >> (2 * j)) & 0x03030303u) | (((r.hm.y >> hb) & 0x01010101u) << 2);
      w0 = ((w0 | 0x80808080u) - 0x04040404u) ^ 0x80808080u;
      w1 = ((w1 | 0x80808080u) - 0x04040404u) ^ 0x80808080u;
      const int2 av = *reinterpret_cast<const int2*>(ab + 32 * j);
      int dot = sdot4(static_cast<int>(w0), av.x, 0);
      dot = sdot4(static_cast<int>(w1), av.y, dot);
      const int s = 8 * h + 2 * j + (k >> 1);  // sub-block
      const uint32_t lw = r.sc[(s & 7) >> 2];
      const int lo = ((lw >> (8 * (s & 3))) >> (s >= 8 ? 4 : 0)) & 15;
      const int hi = (r.sc[2] >> (8 * (s & 3) + 2 * (s >> 2))) & 3;
      S += ((lo | (hi << 4)) - 32) * dot;
    }
    return make_int2(sum8(S), 0);
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    return d8 * half_bits_to_f32(r.dbits) * static_cast<float>(p.x);
  }
};

// Bits 0..3 of v spread to bit 0 of bytes 0..3 (the four shifted copies of
// the 4-bit value do not overlap, so the product is a plain OR of them).
__device__ __forceinline__ uint32_t spread4(uint32_t v) {
  return ((v & 0xFu) * 0x00204081u) & 0x01010101u;
}

// Q4_0 (18 B: fp16 d, 16 bytes of nibbles; byte j = element j low, j + 16
// high; w = d (q - 8)) and Q5_1 (24 B: fp16 d, fp16 m, 32-bit qh whose bit j is
// element j's fifth bit, 16 nibble bytes; w = d q + m), against q8 activations
// in blocks of 32 (int8 quants, one scale per block). One lane per block.
struct FmtQ40 {
  static constexpr int BE = 32, BB = 18, LPB = 1;
  // Five dwords from the aligned one holding byte 0 (blocks are 2-byte
  // aligned, sh = 0 or 2): each starts inside the block.
  struct Raw { uint32_t w[5]; uint32_t sh; };
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(blk);
    const uint8_t* p = reinterpret_cast<const uint8_t*>(a & ~static_cast<uintptr_t>(3));
    r.sh = static_cast<uint32_t>(a & 3);
#pragma unroll
    for (int i = 0; i < 5; ++i) r.w[i] = ld_nt4(p + 4 * i);
  }
  // nibble bytes 4i..4i+3 (block bytes 2 + 4i ..)
  __device__ static __forceinline__ uint32_t nib(const Raw& r, int i) {
    return r.sh == 2 ? r.w[i + 1] : __builtin_amdgcn_alignbyte(r.w[i + 1], r.w[i], 2);
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int) {
    const int4* ax = reinterpret_cast<const int4*>(a.qs + b * 32);
    const int4 alo = ax[0], ahi = ax[1];
    const int al[4] = {alo.x, alo.y, alo.z, alo.w}, ah[4] = {ahi.x, ahi.y, ahi.z, ahi.w};
    int S = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t nb = nib(r, i);
      uint32_t lo = nb & 0x0F0F0F0Fu, hi = (nb >> 4) & 0x0F0F0F0Fu;
      lo = ((lo | 0x80808080u) - 0x08080808u) ^ 0x80808080u;  // q - 8 per byte
      hi = ((hi | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
      S = sdot4(static_cast<int>(lo), al[i], S);
      S = sdot4(static_cast<int>(hi), ah[i], S);
    }
    return make_int2(S, 0);
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    return d8 * half_bits_to_f32((r.w[0] >> (8 * r.sh)) & 0xFFFF) * static_cast<float>(p.x);
  }
};

struct FmtQ51 {
  static constexpr int BE = 32, BB = 24, LPB = 1;
  struct Raw { uint32_t dm, qh, q[4]; };  // blocks are 4-byte aligned
  __device__ static __forceinline__ void load(Raw& r, const uint8_t* blk, int) {
    const uint2 a = make_uint2(ld_nt4(blk), ld_nt4(blk + 4));
    r.dm = a.x;
    r.qh = a.y;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = ld_nt4(blk + 8 + 4 * i);
  }
  __device__ static __forceinline__ int2 partials(const Raw& r, const ActView& a, int b, int) {
    const int4* ax = reinterpret_cast<const int4*>(a.qs + b * 32);
    const int4 alo = ax[0], ahi = ax[1];
    const int al[4] = {alo.x, alo.y, alo.z, alo.w}, ah[4] = {ahi.x, ahi.y, ahi.z, ahi.w};
    int S1 = 0, S2 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (r.q[i] & 0x0F0F0F0Fu) | (spread4(r.qh >> (4 * i)) << 4);
      const uint32_t hi = ((r.q[i] >> 4) & 0x0F0F0F0Fu) | (spread4(r.qh >> (16 + 4 * i)) << 4);
      S1 = sdot4(static_cast<int>(lo), al[i], S1);
      S1 = sdot4(static_cast<int>(hi), ah[i], S1);
      S2 = sdot4(0x01010101, al[i], S2);
      S2 = sdot4(0x01010101, ah[i], S2);
    }
    return make_int2(S1, S2);
  }
  __device__ static __forceinline__ float value(const Raw& r, int2 p, float d8) {
    const float d = half_bits_to_f32(r.dm & 0xFFFF), m = half_bits_to_f32(r.dm >> 16);
    return d8 * (d * static_cast<float>(p.x) + m * static_cast<float>(p.y));
  }
};

template <int FMT> struct FmtOf;
template <> struct FmtOf<FMT_Q4_K> { using T = FmtQ4K; };
template <> struct FmtOf<FMT_Q6_K> { using T = FmtQ6K; };
template <> struct FmtOf<FMT_MXFP4> { using T = FmtMXFP4; };
template <> struct FmtOf<FMT_Q5_K> { using T = FmtQ5K; };
template <> struct FmtOf<FMT_Q2_K> { using T = FmtQ2K; };
template <> struct FmtOf<FMT_Q3_K> { using T = FmtQ3K; };
template <> struct FmtOf<FMT_Q4_0> { using T = FmtQ40; };
template <> struct FmtOf<FMT_Q5_1> { using T = FmtQ51; };

// ------------------------------------------------------- MXFP4 decode GEMV
// A 17-byte block has no fixed alignment, so one lane per block would need five
// dword loads spread over 17-byte steps; the memory pipeline then spends ~24
// cycles per such load for 256 useful bytes. Instead a wave reads two rows at a
// time as coalesced 16-byte pieces (piece j = lane + 64 m of the pair: row 0's
// npc pieces, then row 1's), realigns them through its own LDS scratch, and
// every lane dots the blocks it owns (b = lane + 64 i) against activation pairs
// it keeps in registers.

__host__ __device__ inline int mx_row_pieces(int nb) { return (17 * nb + 15) / 16; }
// Per-wave scratch: two rows of pieces plus the bytes that the five-dword
// window of a row's last block may reach past them.
__host__ __device__ inline int mx_scratch_bytes(int nb) { return 32 * mx_row_pieces(nb) + 16; }

template <int NBL>
struct MxAct {
  half2_t ap[NBL][16];
  float d[NBL];
};

// Rows of 65..96 blocks: the 2 (nb - 64) tail blocks of a row pair (blocks
// 64.. of row 0, then of row 1) fold onto lanes 0 .. 2 (nb - 64) - 1, so a
// lane dots three blocks per pair instead of four. Its second activation
// block is then 64 + lane mod (nb - 64).
__device__ __forceinline__ bool mx_fold(int nb) { return nb > 64 && nb <= 96; }

// The lane's blocks of one activation vector from its LDS image (ActView layout).
template <int NBL>
__device__ __forceinline__ void mx_act_load(MxAct<NBL>& A, const half2_t* lap, const float* ld,
                                            int nb, int lane) {
  const int tail = nb - 64;
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int b = (NBL == 2 && i == 1 && mx_fold(nb)) ? 64 + (lane < tail ? lane : lane - tail)
                                                      : lane + 64 * i;
    const uint4* p = reinterpret_cast<const uint4*>(lap + min(b, nb - 1) * kApPitch);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = p[c];
      A.ap[i][4 * c] = __builtin_bit_cast(half2_t, v.x);
      A.ap[i][4 * c + 1] = __builtin_bit_cast(half2_t, v.y);
      A.ap[i][4 * c + 2] = __builtin_bit_cast(half2_t, v.z);
      A.ap[i][4 * c + 3] = __builtin_bit_cast(half2_t, v.w);
    }
    A.d[i] = b < nb ? ld[b] : 0.0f;
  }
}

// Dot of one block's 16 nibble bytes (five dwords w from the aligned dword
// holding the first one, at byte offset sh) with its 16 activation pairs;
// exact as in FmtMXFP4::dot.
__device__ __forceinline__ float mx_dot_regs(const uint32_t (&w)[5], uint32_t sh,
                                             const half2_t (&ap)[16]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t qw = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 0),
                                 ap[4 * i], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 1),
                                 ap[4 * i + 1], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 2),
                                 ap[4 * i + 2], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 3),
                                 ap[4 * i + 3], acc, false);
  }
  return acc;
}

// One row pair: the lane's NL pieces go to the wave's scratch, then every
// block the lane owns in either row is realigned from the scratch and dotted
// with its activation pairs; f(row, b, i, dot, e) receives each block's exact
// dot (sum of e2m1 value times activation quant, a multiple of 0.5) and scale
// byte e, in a fixed order: for the lane's activation block i, row 0 then row 1.
template <int NL, int NBL, class Fn>
__device__ __forceinline__ void mx_pair_blocks(const uint4 (&pc)[NL], uint8_t* scr, int nb,
                                               const MxAct<NBL>& A, int lane, Fn&& f) {
  const int npc = mx_row_pieces(nb);
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    const int j = lane + 64 * m;
    if (j < 2 * npc) reinterpret_cast<uint4*>(scr)[j] = pc[m];
  }
  // LDS operations of one wave complete in order: the fences only keep the
  // compiler from moving the reads above the writes (and the next pair's
  // writes above these reads)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  auto block = [&](int row, int b, int i) {
    const uint32_t o = static_cast<uint32_t>(row * 16 * npc + 17 * b);  // scale byte
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(scr + ((o + 1) & ~3u));
    uint32_t w[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) w[k] = wp[k];
    const int e = scr[o];
    f(row, b, i, mx_dot_regs(w, (o + 1) & 3u, A.ap[i]), e);
  };
  if (NBL == 2 && mx_fold(nb)) {  // wave-uniform
    block(0, lane, 0);
    block(1, lane, 0);
    const int tail = nb - 64;
    if (lane < 2 * tail) {
      const int row = lane < tail ? 0 : 1;
      block(row, 64 + lane - row * tail, NBL - 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int b = lane + 64 * i;
      if (b < nb) {
        block(0, b, i);
        block(1, b, i);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The two row sums of a row pair (every lane): block values d8 * 2^(e-127) *
// dot summed per lane, then over the wave in a fixed order.
template <int NL, int NBL>
__device__ __forceinline__ float2 mx_pair(const uint4 (&pc)[NL], uint8_t* scr, int nb,
                                          const MxAct<NBL>& A, int lane) {
  float s0 = 0.0f, s1 = 0.0f;
  mx_pair_blocks<NL, NBL>(pc, scr, nb, A, lane, [&](int row, int, int i, float dot, int e) {
    float v = A.d[i] * __builtin_ldexpf(dot, e - 127);
    // the product is rounded on its own, never fused into the sum below, so
    // that every row layout (and every unrolled form) rounds the same way
    asm volatile("" : "+v"(v));
    // selects, not a branch: with a per-lane row (folded tail blocks) a branch
    // made the compiler keep {s0, s1} in scratch memory
    const bool r0 = row == 0;
    s0 += r0 ? v : 0.0f;
    s1 += r0 ? 0.0f : v;
  });
  return make_float2(wave_sum(s0), wave_sum(s1));
}

// ------------------------------------------ MXFP4 rows in the MX16 order
// A row of nb blocks stored in the MX16 order (moe_layout MX16): the 16 nibble
// bytes of block b at byte 16 b, the scale bytes of all blocks after them
// (block b's at byte 16 nb + b). Every field is aligned, so a lane loads each
// block it owns as one 16-byte piece straight into registers, and its scale
// byte from its row's scale run, loaded as one dword per lane and handed
// around the wave: no realignment through LDS.
//
// The blocks of a row pair that a lane owns, slot j < NS, are those of
// mx_pair_blocks in the same order (for activation block i, row 0 then row 1);
// NS = 3 for rows of 65..96 blocks (block lane of both rows, then one folded
// tail block), 2 NBL otherwise.
struct Mx16Slot {
  int row, b, i;
  bool ok;
};
template <int NS>
__device__ __forceinline__ Mx16Slot mx16_slot(int j, int nb, int lane) {
  if constexpr (NS == 3) {
    if (j < 2) return Mx16Slot{j, lane, 0, true};
    const int tail = nb - 64, row = lane < tail ? 0 : 1;
    return Mx16Slot{row, 64 + lane - row * tail, 1, lane < 2 * tail};
  }
  const int b = lane + 64 * (j >> 1);
  return Mx16Slot{j & 1, b, j >> 1, b < nb};
}

template <int NS>
struct Mx16Unit {
  uint4 q[NS];
  // scale runs of the two rows, one dword per lane: rows of up to 128 blocks
  // (32 dwords) share one register (lane 32 row + dword); longer rows (NS =
  // 8) take one register per row
  uint32_t sd[NS == 8 ? 2 : 1];
};

// The loads of one row pair: rows r0 and r1 (ok0 / ok1: the row exists);
// absent blocks and lanes past a scale run read the dummy line.
template <int NS>
__device__ __forceinline__ void mx16_issue(Mx16Unit<NS>& u, const uint8_t* r0, const uint8_t* r1,
                                           bool ok0, bool ok1, int nb, int lane,
                                           const uint8_t* dummy) {
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const Mx16Slot sl = mx16_slot<NS>(j, nb, lane);
    const bool v = sl.ok && (sl.row ? ok1 : ok0);
    const uint8_t* rb = sl.row ? r1 : r0;
    u.q[j] = ld_nt16(v ? rb + 16 * sl.b : dummy);
  }
  const int nd = (nb + 3) >> 2;  // dwords of a scale run
  if constexpr (NS == 8) {
    u.sd[0] = ld_nt4(ok0 && lane < nd ? r0 + 16 * nb + 4 * lane : dummy);
    u.sd[1] = ld_nt4(ok1 && lane < nd ? r1 + 16 * nb + 4 * lane : dummy);
  } else {
    const int row = lane >> 5, dw = lane & 31;
    const bool ok = (row ? ok1 : ok0) && dw < nd;
    u.sd[0] = ld_nt4(ok ? (row ? r1 : r0) + 16 * nb + 4 * dw : dummy);
  }
}

// Scale byte of slot j's block, from the lane that loaded its dword (all lanes
// take part in the exchange).
template <int NS>
__device__ __forceinline__ int mx16_scale(const Mx16Unit<NS>& u, const Mx16Slot& sl) {
  const int src = NS == 8 ? sl.b >> 2 : 32 * sl.row + (sl.b >> 2);
  const uint32_t reg = NS == 8 ? u.sd[sl.row] : u.sd[0];
  const uint32_t w = static_cast<uint32_t>(
      __builtin_amdgcn_ds_bpermute(4 * (src & 63), static_cast<int>(reg)));
  return static_cast<int>((w >> (8 * (sl.b & 3))) & 0xFFu);
}

// Dot of one block's 16 nibble bytes with its 16 activation pairs: the
// operations of mx_dot_regs on the same bytes, so the same exact value.
__device__ __forceinline__ float mx16_dot(const uint4& q, const half2_t (&ap)[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0),
                                 ap[4 * i], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1),
                                 ap[4 * i + 1], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2),
                                 ap[4 * i + 2], acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3),
                                 ap[4 * i + 3], acc, false);
  }
  return acc;
}

// f(row, b, i, dot, e) for every block the lane owns, in slot order.
template <int NS, int NBL, class Fn>
__device__ __forceinline__ void mx16_pair_blocks(const Mx16Unit<NS>& u, const MxAct<NBL>& A,
                                                 int nb, int lane, Fn&& f) {
  int e[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) e[j] = mx16_scale<NS>(u, mx16_slot<NS>(j, nb, lane));
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const Mx16Slot sl = mx16_slot<NS>(j, nb, lane);
    if (sl.ok) f(sl.row, sl.b, sl.i, mx16_dot(u.q[j], A.ap[sl.i]), e[j]);
  }
}

// The two row sums of a row pair, summed as mx_pair sums them (products and
// sums rounded one by one in both).
template <int NS, int NBL>
__device__ __forceinline__ float2 mx16_pair(const Mx16Unit<NS>& u, const MxAct<NBL>& A, int nb,
                                            int lane) {
  float s0 = 0.0f, s1 = 0.0f;
  mx16_pair_blocks<NS, NBL>(u, A, nb, lane, [&](int row, int, int i, float dot, int e) {
    float v = A.d[i] * __builtin_ldexpf(dot, e - 127);
    asm volatile("" : "+v"(v));  // rounded on its own, as in mx_pair
    const bool r0 = row == 0;
    s0 += r0 ? v : 0.0f;
    s1 += r0 ? 0.0f : v;
  });
  return make_float2(wave_sum(s0), wave_sum(s1));
}

// fp32 value of one block for the lane's share (all LPB lanes get the value).
template <class F>
__device__ __forceinline__ float block_value(const typename F::Raw& r, const ActView& a, int b,
                                             int sub) {
  if constexpr (std::is_same<F, FmtMXFP4>::value) {
    return F::value_from_dot(r, F::dot(r, a, b), a.d[b]);
  } else {
    return F::value(r, F::partials(r, a, b, sub), a.d[b]);
  }
}

// Activation layouts in LDS: q8_K (int8, scale per 256, 16-element sums),
// fp16 pairs of q8_32 (MXFP4 rows) and int8 q8_32 (Q4_0 and Q5_1 rows).
enum { ACT_Q8K = 0, ACT_PAIRS = 1, ACT_I8_32 = 2 };
template <int FMT>
struct ActMode {
  static constexpr int v = FMT == FMT_MXFP4 ? ACT_PAIRS
                           : (FMT == FMT_Q4_0 || FMT == FMT_Q5_1) ? ACT_I8_32 : ACT_Q8K;
};

// Stage q8 activations (global, one token) into LDS in the layout the format reads.
template <int MODE>
__device__ __forceinline__ void stage_act(const int8_t* qs, const float* d, const int16_t* bs,
                                          int K, int8_t* lqs, float* ld, int16_t* lbs,
                                          half2_t* lap) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if constexpr (MODE == ACT_Q8K) {
    for (int i = tid; i < K / 16; i += nt) {
      reinterpret_cast<int4*>(lqs)[i] = reinterpret_cast<const int4*>(qs)[i];
      lbs[i] = bs[i];
    }
    for (int i = tid; i < K / 256; i += nt) ld[i] = d[i];
  } else if constexpr (MODE == ACT_I8_32) {
    for (int i = tid; i < K / 16; i += nt)
      reinterpret_cast<int4*>(lqs)[i] = reinterpret_cast<const int4*>(qs)[i];
    for (int i = tid; i < K / 32; i += nt) ld[i] = d[i];
  } else {
    for (int i = tid; i < K / 2; i += nt) {  // block-major, padded (see ActView)
      const int b = i / 16, ii = i % 16;
      lap[b * kApPitch + ii] = half2_t{static_cast<_Float16>(qs[32 * b + ii]),
                                       static_cast<_Float16>(qs[32 * b + 16 + ii])};
    }
    for (int i = tid; i < K / 32; i += nt) ld[i] = d[i];
  }
}

__device__ __forceinline__ float act_fn(int act, float alpha, float limit, float g, float u) {
  if (act == 0) return g / (1.0f + __expf(-g)) * u;
  if (act >= ACT_PRE_GATE) return act == ACT_PRE_GATE ? g : u;  // pre-activation export
  const float gc = fminf(g, limit);
  const float uc = fminf(fmaxf(u, -limit), limit);
  return gc / (1.0f + __expf(-alpha * gc)) * (uc + 1.0f);
}

// Order-preserving key: larger float -> larger key; -0 and +0 share a key.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  // 0 is the identity of the unsigned max, so lanes without a DPP source may
  // read 0 (bound_ctrl) and the move folds into one v_max_u32_dpp per step.
#define MOE_DPP_UMAX(CTRL, RM) \
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, RM, 0xF, true)))
  MOE_DPP_UMAX(0x111, 0xF);
  MOE_DPP_UMAX(0x112, 0xF);
  MOE_DPP_UMAX(0x114, 0xF);
  MOE_DPP_UMAX(0x118, 0xF);
  MOE_DPP_UMAX(0x142, 0xA);
  MOE_DPP_UMAX(0x143, 0xC);
#undef MOE_DPP_UMAX
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Per-wave LDS scratch of the candidate ranking below (workgroups of at most
// four waves): up to 64 composite keys and their ranks.
struct TopkLds {
  uint64_t* cand;
  int* rank;
};
__device__ __forceinline__ TopkLds topk_lds() {
  __shared__ __align__(16) uint64_t cand[4][64];
  __shared__ int rank[4][64];
  const int w = (threadIdx.x >> 6) & 3;
  return TopkLds{cand[w], rank[w]};
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One-pass ranking of the keys that can be among the 8 largest (keys as in
// topk_select: expert e = lane + 64 i in register i, 0 = absent).
//
// The lanes form 8 groups of 8; the maxima of the groups are keys of 8
// different experts, so at least 8 keys reach tau, the smallest group maximum,
// and so does every key among the 8 largest. A key that outranks a candidate
// (a present key >= tau) is a candidate itself, so a candidate's rank among the
// candidates is its rank among all keys. The candidates are written to LDS as
// (key << 32 | ~expert): distinct, and ordered as (key descending, expert
// ascending). Lane l < C then counts the candidates above cand[l]; every rank
// comes out of one pass instead of one wave reduction per rank.
//
// Returns C, the number of candidates (wave-uniform), or 0 when more than 64
// keys reach tau (equal keys at the threshold); nothing is ranked then. For
// C > 0: lane l < C holds the rank r of candidate mine = cand[l]; pos[i] is
// the list position of register i's key, or -1 when it is not a candidate.
template <int NC>
__device__ __forceinline__ int topk_rank8(const uint32_t (&key)[NC], uint64_t* cand, int& r,
                                          uint64_t& mine, int (&pos)[NC]) {
  const int lane = threadIdx.x & 63;
  uint32_t m = key[0];
#pragma unroll
  for (int i = 1; i < NC; ++i) m = max(m, key[i]);
  // maxima over 8 consecutive lanes (row shifts by 1, 2, 4 within rows of 16;
  // lanes without a source read 0, the identity of the unsigned max): lane
  // 8 g + 7 then holds group g's maximum
  m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x111, 0xF, 0xF, true)));
  m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x112, 0xF, 0xF, true)));
  m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x114, 0xF, 0xF, true)));
  uint32_t tau = 0xFFFFFFFFu;
#pragma unroll
  for (int g = 0; g < 8; ++g)
    tau = min(tau, static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m), 8 * g + 7)));
  const uint32_t th = max(tau, 1u);  // a group of absent keys only: every present key
  int C = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const bool c = key[i] >= th;
    const unsigned long long b = __builtin_amdgcn_ballot_w64(c);
    const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(b >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
    pos[i] = c ? C + below : -1;
    C += __builtin_popcountll(b);
  }
  if (C > 64) return 0;  // wave-uniform
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (pos[i] >= 0)
      cand[pos[i]] = (static_cast<uint64_t>(key[i]) << 32) | static_cast<uint32_t>(~(lane + 64 * i));
  if (lane >= C) cand[lane] = 0;  // below every candidate
  wave_lds_sync();
  mine = cand[lane];
  int cnt = 0;
  for (int j = 0; j < C; j += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cand[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) cnt += v[u] > mine ? 1 : 0;
  }
  r = cnt;
  return C;
}

// Top-k selection over order-preserving keys, expert e = lane + 64 i held in
// register i of every lane. key 0 marks an absent candidate (every real key
// is above it). On return rank[i] is the rank (0 = first) of that candidate,
// or -1 when it is not among the k selected. Rank order is key descending,
// index ascending.
//
// k <= 8 and E > 64: the one-pass candidate ranking (topk_rank8; for E <= 64
// every key is a candidate, and the gpt-oss shape, E = 32 and k = 4, measured
// slower with it than with the rounds). Otherwise, and when more than 64 keys
// reach its threshold, rounds of one wave reduction each.
// Their fast path: k rounds of one 32-bit wave max each; every candidate equal
// to the round's maximum takes rank r and leaves. That is exact when every
// round's maximum is unique, which holds exactly when k candidates end up
// ranked (each round ranks at least one). Otherwise (equal keys) the exact
// path reruns the selection with the lowest index taken first among equal
// keys: per round the lowest hit lane of each register's ballot gives a
// candidate index, and the smallest of those wins.
template <int NC>
__device__ __forceinline__ void topk_select(const uint32_t (&key0)[NC], int E, int k,
                                            int (&rank)[NC]) {
  const int lane = threadIdx.x & 63;
  if (E > 64 && k <= 8) {  // one-pass candidate ranking (wave-uniform branches)
    const TopkLds s = topk_lds();
    int r, pos[NC];
    uint64_t mine;
    if (topk_rank8<NC>(key0, s.cand, r, mine, pos) > 0) {
      s.rank[lane] = r;  // lanes past the candidates store a rank nobody reads
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int rr = s.rank[pos[i] < 0 ? 0 : pos[i]];
        rank[i] = pos[i] >= 0 && rr < k ? rr : -1;
      }
      return;
    }
  }
  uint32_t key[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) { key[i] = key0[i]; rank[i] = -1; }
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < NC; ++i) best = max(best, key[i]);
    const uint32_t kmax = wave_max_u32(best);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bool hit = key[i] == kmax;
      rank[i] = hit ? r : rank[i];
      key[i] = hit ? 0u : key[i];
    }
  }
  int n = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(rank[i] >= 0));
  if (n == k) return;  // wave-uniform
#pragma unroll
  for (int i = 0; i < NC; ++i) { key[i] = key0[i]; rank[i] = -1; }
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < NC; ++i) best = max(best, key[i]);
    const uint32_t kmax = wave_max_u32(best);
    // lowest hit lane of register i is candidate 64 i + lane; no hit leaves
    // all ones, above every candidate
    uint32_t e = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(key[i] == kmax);
      const uint32_t c = hit ? static_cast<uint32_t>(__builtin_ctzll(hit)) + 64u * i : 0xFFFFFFFFu;
      e = min(e, c);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bool win = static_cast<uint32_t>(lane + 64 * i) == e;
      rank[i] = win ? r : rank[i];
      key[i] = win ? 0u : key[i];
    }
  }
}

// Selection keys of one wave's candidates (expert e = lane + 64 i in register
// i): key = order-preserving bits of logit (+ selection bias, one fp32 add),
// 0 for e >= E; lg[i] of e >= E becomes -inf.
template <int NC>
__device__ __forceinline__ void topk_keys(float (&lg)[NC], const float* sel_bias, int E,
                                          uint32_t (&key)[NC]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int e = lane + 64 * i;
    const bool valid = e < E;
    const float sb = sel_bias ? sel_bias[min(e, E - 1)] : 0.0f;
    key[i] = valid ? float_key(sel_bias ? lg[i] + sb : lg[i]) : 0u;
    lg[i] = valid ? lg[i] : -INFINITY;
  }
}

// One exact selection round: the largest key, lowest index among equal keys;
// returns its expert index (wave-uniform) and removes it from the candidates.
template <int NC>
__device__ __forceinline__ int topk_round(uint32_t (&key)[NC]) {
  const int lane = threadIdx.x & 63;
  uint32_t best = key[0];
#pragma unroll
  for (int i = 1; i < NC; ++i) best = max(best, key[i]);
  const uint32_t kmax = wave_max_u32(best);
  uint32_t e = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(key[i] == kmax);
    e = min(e, hit ? static_cast<uint32_t>(__builtin_ctzll(hit)) + 64u * i : 0xFFFFFFFFu);
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) key[i] = static_cast<uint32_t>(lane + 64 * i) == e ? 0u : key[i];
  return static_cast<int>(e);
}

// Expert index of rank n (0-based; n < the number of candidates), exact.
// n < 8 and E > 64: the one-pass candidate ranking (topk_rank8). Otherwise,
// and when more than 64 keys reach its threshold, rounds. Their fast path: n + 1
// rounds of one wave max each, every candidate equal to the
// round's maximum leaving; the rank-n expert is the one equal to the last
// maximum. That is exact when every round's maximum is unique; the ballot
// counts that check it sit off the dependent chain. Otherwise the exact
// rounds (lowest index first among equal keys) run from the original keys.
template <int NC>
__device__ __forceinline__ int topk_nth(const uint32_t (&key0)[NC], int E, int n) {
  if (E > 64 && n < 8) {  // one-pass candidate ranking (wave-uniform branches)
    const int lane = threadIdx.x & 63;
    const TopkLds s = topk_lds();
    int r, pos[NC];
    uint64_t mine;
    const int C = topk_rank8<NC>(key0, s.cand, r, mine, pos);
    if (C > 0) {
      // ranks 0..C-1 are held once each, and n < 8 <= C or n < E = C
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < C && r == n);
      const int l = static_cast<int>(__builtin_ctzll(hit));
      return static_cast<int>(~static_cast<uint32_t>(
          __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(mine)), l)));
    }
  }
  uint32_t key[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) key[i] = key0[i];
  uint32_t kmax = 0;
  int ties = 0;
  for (int r = 0; r <= n; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < NC; ++i) best = max(best, key[i]);
    kmax = wave_max_u32(best);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bool hit = key[i] == kmax;
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(hit));
      key[i] = hit ? 0u : key[i];
    }
    ties |= cnt != 1;
  }
  if (!ties) {  // wave-uniform
    int e = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(key0[i] == kmax);
      if (hit) e = min(e, static_cast<int>(__builtin_ctzll(hit)) + 64 * i);
    }
    return e;
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) key[i] = key0[i];
  int e = 0;
  for (int r = 0; r <= n; ++r) e = topk_round<NC>(key);
  return e;
}

// Routing weights of the selected experts: lane r < k holds rank r's expert
// my_id; lg as left by topk_keys. Softmax over the selected (norm_topk) or
// over all E, or sigmoid (normalized over the selected when norm_topk), times
// route_scale. Lane r < k writes w_out[r].
template <int NC>
__device__ __forceinline__ void topk_weights(const float (&lg)[NC], int my_id, int E, int k,
                                             int router, int norm_topk, float route_scale,
                                             float* w_out) {
  const int lane = threadIdx.x & 63;
  const int my_reg = my_id >> 6, my_lane = my_id & 63;
  float my_l = -INFINITY;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const float v = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * my_lane, __float_as_int(lg[i])));
    my_l = my_reg == i ? v : my_l;
  }
  if (lane >= k) my_l = -INFINITY;
  float w;
  if (router == 0) {
    float mx, z;
    if (norm_topk) {
      mx = wave_max(my_l);
      const float ex = lane < k ? expf(my_l - mx) : 0.0f;
      z = wave_sum(ex);
      w = ex / z;
    } else {
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < NC; ++i) lm = fmaxf(lm, lg[i]);
      mx = wave_max(lm);
      float zz = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; ++i) if (lane + 64 * i < E) zz += expf(lg[i] - mx);
      z = wave_sum(zz);
      w = lane < k ? expf(my_l - mx) / z : 0.0f;
    }
  } else {
    const float sg = lane < k ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
    w = norm_topk ? sg / wave_sum(sg) : sg;
  }
  if (lane < k) w_out[lane] = w * route_scale;
}

// Top-k of one token by one wave (all 64 lanes must call it). Selection key =
// logit (+ selection bias, one fp32 add); rank order as in topk_select.
// Weights come from the unbiased logits: softmax over the selected
// (norm_topk) or over all E, or sigmoid (normalized over the selected when
// norm_topk), times route_scale. Rank r goes to ids_out[r] (written by the
// lane that holds that expert) and w_out[r] (lane r); global or LDS.
// wave_topk_regs takes the logits already in registers (lg[i] = logit of expert
// lane + 64 i; lanes past E may hold anything). NC candidates per lane,
// E <= 64 NC.
template <int NC>
__device__ __forceinline__ void wave_topk_regs(float (&lg)[NC], const float* sel_bias, int E,
                                               int k, int router, int norm_topk,
                                               float route_scale, int* ids_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  float sb[NC];
  if (sel_bias) {
#pragma unroll
    for (int i = 0; i < NC; ++i) sb[i] = sel_bias[min(lane + 64 * i, E - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < NC; ++i) sb[i] = 0.0f;
  }
  uint32_t key[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const bool valid = lane + 64 * i < E;
    key[i] = valid ? float_key(sel_bias ? lg[i] + sb[i] : lg[i]) : 0u;
    lg[i] = valid ? lg[i] : -INFINITY;
  }
  int rank[NC];
  topk_select<NC>(key, E, k, rank);
  // ids and the selected logits in rank order; lane r < k then holds rank r
  __shared__ float s_rank_l[16][16];
  float* rl = s_rank_l[(threadIdx.x >> 6) & 15];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (rank[i] >= 0) {
      ids_out[rank[i]] = lane + 64 * i;
      rl[rank[i]] = lg[i];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float my_l = lane < k ? rl[lane] : -INFINITY;
  float w;
  if (router == 0) {
    float mx, z;
    if (norm_topk) {
      mx = wave_max(my_l);
      const float ex = lane < k ? expf(my_l - mx) : 0.0f;
      z = wave_sum(ex);
      w = ex / z;
    } else {
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < NC; ++i) lm = fmaxf(lm, lg[i]);
      mx = wave_max(lm);
      float zz = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; ++i) if (lane + 64 * i < E) zz += expf(lg[i] - mx);
      z = wave_sum(zz);
      w = lane < k ? expf(my_l - mx) / z : 0.0f;
    }
  } else {
    const float sg = lane < k ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
    w = norm_topk ? sg / wave_sum(sg) : sg;
  }
  if (lane < k) w_out[lane] = w * route_scale;
}

template <int NC>
__device__ __forceinline__ void wave_topk(const float* logits, const float* sel_bias, int E,
                                          int k, int router, int norm_topk, float route_scale,
                                          int* ids_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  float lg[NC];
  // all loads issued before any use (clamped indices, masked afterwards)
#pragma unroll
  for (int i = 0; i < NC; ++i) lg[i] = logits[min(lane + 64 * i, E - 1)];
  wave_topk_regs<NC>(lg, sel_bias, E, k, router, norm_topk, route_scale, ids_out, w_out);
}

}  // namespace dev
}  // namespace moe
