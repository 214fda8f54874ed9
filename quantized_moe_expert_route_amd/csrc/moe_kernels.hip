// HIP kernels of the routed-expert MoE FFN layer for gfx950 (MI355X).
//
// Path (one layer, T tokens):
//   k_quant        x -> q8 blocks (fp32 recipe, bit-exact with the definition)
//   k_router       router GEMV with fp64 accumulation; for small T the last
//                  workgroup to finish also runs top-k and the routing weights
//   k_topk         top-k + weights, one wave per token (larger T)
//   k_gateup_gemv  per (token, slot) pair: gate/up rows of the selected
//                  expert against q8(x), SwiGLU epilogue -> h (fp32)
//   k_down_gemv    per token: re-quantizes the h of its slots to q8, down rows,
//                  routing-weighted sum in a fixed order (+ shared expert) -> y
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
// activation quants per block, rescaled per block in fp32 — the integer-dot
// numerics the Pulsar README describes for its q8_K/q8_0 activations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

namespace {


typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load: expert weights are read once per call.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float load_x(const void* x, int dtype, size_t i) {
  return dtype == 0 ? static_cast<const float*>(x)[i]
                    : bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
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
  constexpr int G = B / 4;  // lanes per block
#pragma unroll
  for (int o = 1; o < G; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
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
    int sm = q[0] + q[1] + q[2] + q[3];
    sm += __shfl_xor(sm, 1);
    sm += __shfl_xor(sm, 2);
    if (valid && (lane & 3) == 0) bs[lane >> 2] = static_cast<int16_t>(sm);
  }
}

// B = 32 quantization stored as fp16 pairs (a[i], a[i+16]) per block, the layout
// the MXFP4 dot reads: ap gets 128 pairs for the 256-value piece.
__device__ __forceinline__ void quant_wave_pairs(const float v[4], bool valid, int lane,
                                                 half2_t* ap, float* d) {
  int q[4];
  const float dv = quant_wave_q<32>(v, q);
  int o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __shfl_down(q[i], 4);  // partner 16 elements ahead
  const int bl = lane >> 3, off = 4 * (lane & 7);
  if (valid && off < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ap[16 * bl + off + i] = half2_t{static_cast<_Float16>(q[i]), static_cast<_Float16>(o[i])};
  }
  if (valid && (lane & 7) == 0) d[bl] = dv;
}

// Activations of one row vector as the dot routines read them (LDS).
struct ActView {
  const int8_t* qs;     // [K] (Q8_K)
  const float* d;       // [K / B]
  const int16_t* bs;    // [K / 16] (Q8_K)
  const half2_t* ap;    // [K / 2] fp16 pairs (Q8_32): block b, i < 16: (a[32b+i], a[32b+16+i])
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
    // 6-bit scales/mins of the 8 sub-blocks as bytes: sub-blocks 0..3 sit in the
    // low 6 bits of scale bytes 0..3 (sc) and 4..7 (m); 4..7 take their low 4
    // bits from bytes 8..11 and their top 2 bits from bits 6..7 of bytes 0..7.
    const uint32_t s0 = r.hdr.y, s1 = r.hdr.z, s2 = r.hdr.w;
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
  const uint32_t* w = reinterpret_cast<const uint32_t*>(a & ~static_cast<uintptr_t>(3));
  const uint32_t* w_last = reinterpret_cast<const uint32_t*>((a + 7) & ~static_cast<uintptr_t>(3));
  const uint32_t sh = static_cast<uint32_t>(a & 3);
  const uint32_t w0 = __builtin_nontemporal_load(w), w1 = __builtin_nontemporal_load(w + 1),
                 w2 = __builtin_nontemporal_load(w_last);
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}

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
    r.dbits = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(blk + 208));
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
    const uint32_t* p = reinterpret_cast<const uint32_t*>(a & ~static_cast<uintptr_t>(3));
    r.sh = static_cast<uint32_t>(a & 3);
#pragma unroll
    for (int i = 0; i < 5; ++i) r.w[i] = __builtin_nontemporal_load(p + i);
  }
  __device__ static __forceinline__ uint32_t scale_byte(const Raw& r) {
    return (r.w[0] >> (8 * r.sh)) & 0xFF;
  }
  // Exact: e2m1 values and int8 activations are exact in fp16, products exact in
  // fp32 and every partial sum is a multiple of 0.5 below 2^23.
  __device__ static __forceinline__ float dot(const Raw& r, const ActView& a, int b) {
    const half2_t* ap = a.ap + 16 * b;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qw = r.sh == 3 ? r.w[i + 1]
                                    : __builtin_amdgcn_alignbyte(r.w[i + 1], r.w[i], r.sh + 1);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 0),
                                   ap[4 * i + 0], acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 1),
                                   ap[4 * i + 1], acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 2),
                                   ap[4 * i + 2], acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw, 1.0f, 3),
                                   ap[4 * i + 3], acc, false);
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

template <int FMT> struct FmtOf;
template <> struct FmtOf<FMT_Q4_K> { using T = FmtQ4K; };
template <> struct FmtOf<FMT_Q6_K> { using T = FmtQ6K; };
template <> struct FmtOf<FMT_MXFP4> { using T = FmtMXFP4; };

// fp32 value of one block for the lane's share (all LPB lanes get the value).
template <class F>
__device__ __forceinline__ float block_value(const typename F::Raw& r, const ActView& a, int b,
                                             int sub) {
  if constexpr (F::LPB == 1) {
    return F::value_from_dot(r, F::dot(r, a, b), a.d[b]);
  } else {
    return F::value(r, F::partials(r, a, b, sub), a.d[b]);
  }
}

// Stage q8 activations (global, one token) into LDS in the layout the format reads.
template <int AFMT_MX>
__device__ __forceinline__ void stage_act(const int8_t* qs, const float* d, const int16_t* bs,
                                          int K, int8_t* lqs, float* ld, int16_t* lbs,
                                          half2_t* lap) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if constexpr (!AFMT_MX) {
    for (int i = tid; i < K / 16; i += nt) {
      reinterpret_cast<int4*>(lqs)[i] = reinterpret_cast<const int4*>(qs)[i];
      lbs[i] = bs[i];
    }
    for (int i = tid; i < K / 256; i += nt) ld[i] = d[i];
  } else {
    for (int i = tid; i < K / 2; i += nt) {
      const int b = i / 16, ii = i % 16;
      lap[i] = half2_t{static_cast<_Float16>(qs[32 * b + ii]),
                       static_cast<_Float16>(qs[32 * b + 16 + ii])};
    }
    for (int i = tid; i < K / 32; i += nt) ld[i] = d[i];
  }
}

__device__ __forceinline__ float act_fn(int act, float alpha, float limit, float g, float u) {
  if (act == 0) return g / (1.0f + __expf(-g)) * u;
  const float gc = fminf(g, limit);
  const float uc = fminf(fmaxf(u, -limit), limit);
  return gc / (1.0f + __expf(-alpha * gc)) * (uc + 1.0f);
}

// ================================================================== kernels

// x [T, H] -> q8. grid (ceil(H / 256), T), block 64. Also zeroes n_zero words.
template <int B>
__global__ __launch_bounds__(64) void k_quant(const void* x, int dtype, int H, int8_t* qs,
                                              float* d, int16_t* bs, uint32_t* zero_words,
                                              int n_zero) {
  const int lane = threadIdx.x, t = blockIdx.y;
  if (blockIdx.x == 0 && t == 0 && lane < n_zero) zero_words[lane] = 0;
  const int e0 = blockIdx.x * 256 + 4 * lane;
  const bool valid = e0 < H;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = valid ? load_x(x, dtype, static_cast<size_t>(t) * H + e0 + i) : 0.0f;
  const size_t base = static_cast<size_t>(t) * H + blockIdx.x * 256;
  quant_wave<B>(v, valid, lane, qs + base, d + base / B, bs ? bs + base / 16 : nullptr);
}

// Shared-expert gate sigmoid(v . x) per token, fp64 dot. grid T, block 256.
__global__ __launch_bounds__(256) void k_shared_gate(KArgs a) {
  __shared__ double red[4];
  const int t = blockIdx.x;
  double acc = 0.0;
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

// Order-preserving key: larger float -> larger key; -0 and +0 share a key.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wave: rank order (key desc, index asc), then weights
// in fp64 from the unbiased logits.
__device__ void topk_token(const KArgs& a, int t, const float* logits) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  constexpr int kMaxPer = (1024 + 63) / 64;
  unsigned long long cand[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      float key = logits[e];
      if (a.sel_bias) key = key + a.sel_bias[e];
      cand[i] = (static_cast<unsigned long long>(float_key(key)) << 32) |
                static_cast<uint32_t>(0xFFFFFFFFu - e);
    } else {
      cand[i] = 0;
    }
  }
  int my_ids[16];
  double wv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    my_ids[r] = 0;
    wv[r] = 0.0;
    if (r < k) {
      unsigned long long best = 0;
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i) best = cand[i] > best ? cand[i] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
      my_ids[r] = e;
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i)
        if (lane + 64 * i == e) cand[i] = 0;
    }
  }
  // weights (fp64) from the unbiased logits of the selected experts
  if (a.router == 0) {
    double mx = -INFINITY, z = 0.0;
    if (a.norm_topk) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < k) mx = fmax(mx, static_cast<double>(logits[my_ids[r]]));
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < k) z += exp(static_cast<double>(logits[my_ids[r]]) - mx);
    } else {
      for (int e = lane; e < E; e += 64) mx = fmax(mx, static_cast<double>(logits[e]));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
      for (int e = lane; e < E; e += 64) z += exp(static_cast<double>(logits[e]) - mx);
      z = wave_sum_d(z);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r < k) wv[r] = exp(static_cast<double>(logits[my_ids[r]]) - mx) / z;
  } else {
    double z = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r < k) {
        wv[r] = 1.0 / (1.0 + exp(-static_cast<double>(logits[my_ids[r]])));
        z += wv[r];
      }
    if (a.norm_topk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) wv[r] /= z;
    }
  }
  int id = 0;
  double wl = 0.0;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (r == lane) { id = my_ids[r]; wl = wv[r]; }
  if (lane < k) {
    a.ids[t * k + lane] = id;
    a.w[t * k + lane] = static_cast<float>(wl * static_cast<double>(a.route_scale));
  }
}

// Router logits. grid (E + has_gate_vec, ceil(T / TT)), block 64 (one wave per
// expert row and token group). Row E (if present) is the shared-expert gate.
// fuse_topk: the last wave to finish (atomic ticket on counters[0]) runs top-k.
template <int TT>
__global__ __launch_bounds__(64) void k_router(KArgs a, int fuse_topk) {
  const int lane = threadIdx.x, e = blockIdx.x, t0 = blockIdx.y * TT;
  const float* wrow = e < a.E ? a.w_router + static_cast<size_t>(e) * a.H : a.sh_gate_vec;
  double acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0;
  for (int h = 4 * lane; h < a.H; h += 256) {
    const float4 wv = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      if (t0 + i < a.T) {
        const size_t xo = static_cast<size_t>(t0 + i) * a.H + h;
        float xv[4];
        if (a.x_dtype == 0) {
          const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + xo);
          xv[0] = f.x; xv[1] = f.y; xv[2] = f.z; xv[3] = f.w;
        } else {
          const uint2 bb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + xo);
          xv[0] = bf16_bits_to_f32(bb.x & 0xFFFF); xv[1] = bf16_bits_to_f32(bb.x >> 16);
          xv[2] = bf16_bits_to_f32(bb.y & 0xFFFF); xv[3] = bf16_bits_to_f32(bb.y >> 16);
        }
        acc[i] = fma(static_cast<double>(wv.x), static_cast<double>(xv[0]), acc[i]);
        acc[i] = fma(static_cast<double>(wv.y), static_cast<double>(xv[1]), acc[i]);
        acc[i] = fma(static_cast<double>(wv.z), static_cast<double>(xv[2]), acc[i]);
        acc[i] = fma(static_cast<double>(wv.w), static_cast<double>(xv[3]), acc[i]);
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
  if (!fuse_topk) return;
  __shared__ int last;
  __threadfence();
  if (lane == 0) {
    const uint32_t n = gridDim.x * gridDim.y;
    last = atomicAdd(&a.counters[0], 1u) == n - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int t = 0; t < a.T; ++t) topk_token(a, t, a.logits + static_cast<size_t>(t) * a.E);
  if (lane == 0) a.counters[0] = 0;
}

// Top-k for many tokens: one wave per token. grid ceil(T / 4), block 256.
__global__ __launch_bounds__(256) void k_topk(KArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < a.T) topk_token(a, t, a.logits + static_cast<size_t>(t) * a.E);
}

// -------------------------------------------------------------- GEMV gate/up
// grid (ceil(F / R), P), block 256. Pair p < T*k: token p / k, slot p % k;
// p >= T*k: shared expert of token p - T*k. Tasks (m in {gate, up}, row, block)
// are spread over lane groups; each group's block values go to LDS and one
// thread per row sums them in block order.
template <int FMT, int TPG>
__global__ __launch_bounds__(256) void k_gateup_gemv(KArgs a, int R) {
  using F = typename FmtOf<FMT>::T;
  constexpr bool MX = FMT == FMT_MXFP4;
  extern __shared__ __align__(16) unsigned char smem[];
  const int p = blockIdx.y, row0 = blockIdx.x * R;
  const int Tk = a.T * a.k;
  const uint8_t* gbase;
  const uint8_t* ubase;
  const float* bg = nullptr;
  const float* bu = nullptr;
  int t;
  if (p < Tk) {
    t = p / a.k;
    const int e = a.ids[p];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(a.E)) return;  // invalid id: no-op
    gbase = static_cast<const uint8_t*>(a.gate[e]);
    if (gbase == nullptr) return;  // expert not present: the slot contributes nothing
    ubase = static_cast<const uint8_t*>(a.up[e]);
    if (a.b_gate) { bg = a.b_gate[e]; bu = a.b_up[e]; }
  } else {
    t = p - Tk;
    gbase = static_cast<const uint8_t*>(a.sh_gate);
    ubase = static_cast<const uint8_t*>(a.sh_up);
  }
  const int K = a.H, nb = K / F::BE;
  // LDS: activations, then block values [2][R][nb]
  int8_t* lqs = reinterpret_cast<int8_t*>(smem);
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  const int act_bytes = MX ? K * 2 : K;
  float* ld = reinterpret_cast<float*>(smem + act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + act_bytes + 4 * (K / 32));
  float* vals = reinterpret_cast<float*>(smem + act_bytes + 4 * (K / 32) + 2 * (K / 16));
  {
    const int Bx = MX ? 32 : 256;
    stage_act<MX>(a.xqs + static_cast<size_t>(t) * K, a.xd + static_cast<size_t>(t) * (K / Bx),
                  MX ? nullptr : a.xbs + static_cast<size_t>(t) * (K / 16), K, lqs, ld, lbs, lap);
  }
  ActView av{lqs, ld, lbs, lap};
  const int G = 256 / F::LPB;
  const int grp = threadIdx.x / F::LPB, sub = threadIdx.x % F::LPB;
  const int total = 2 * R * nb;
  typename F::Raw raw[TPG];
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int task = grp + G * i;
    const int m = task / (R * nb), r = (task / nb) % R, b = task % nb;
    const int row = row0 + r;
    if (task < total && row < a.F) {
      const uint8_t* base = m ? ubase : gbase;
      const size_t stride = m ? a.stride_up : a.stride_gate;
      F::load(raw[i], base + static_cast<size_t>(row) * stride + static_cast<size_t>(b) * F::BB, sub);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int task = grp + G * i;
    const int m = task / (R * nb), r = (task / nb) % R, b = task % nb;
    if (task < total && row0 + r < a.F) {
      const float v = block_value<F>(raw[i], av, b, sub);
      if (sub == 0) vals[(m * R + r) * nb + b] = v;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 256) {
    const int row = row0 + r;
    if (row >= a.F) break;
    float g = 0.0f, u = 0.0f;
    for (int b = 0; b < nb; ++b) g += vals[r * nb + b];
    for (int b = 0; b < nb; ++b) u += vals[(R + r) * nb + b];
    if (bg) { g += bg[row]; u += bu[row]; }
    a.h[static_cast<size_t>(p) * a.F + row] = act_fn(a.act, a.act_alpha, a.act_limit, g, u);
  }
}

// ---------------------------------------------------------------- GEMV down
// grid (ceil(H / R), T), block 256. For each present slot of token t (and the
// shared expert): q8(h) into LDS, down rows [row0, row0 + R), then
// y = sum_slot w * (o + b_down) + shw * o_shared in slot order.
template <int FMT, int TPG>
__global__ __launch_bounds__(256) void k_down_gemv(KArgs a, int R) {
  using F = typename FmtOf<FMT>::T;
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int B = MX ? 32 : 256;
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = blockIdx.y, row0 = blockIdx.x * R;
  const int K = a.F, nb = K / F::BE;
  const int ns = a.k + a.has_shared;
  // per-slot activations: qs [ns][K] (or fp16 pairs [ns][K/2]), d [ns][K/32], bs [ns][K/16]
  const int act_bytes = MX ? K * 2 : K;
  unsigned char* p_act = smem;
  float* ld = reinterpret_cast<float*>(smem + ns * act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + ns * act_bytes + ns * 4 * (K / 32));
  float* vals = reinterpret_cast<float*>(smem + ns * act_bytes + ns * 4 * (K / 32) +
                                         ns * 2 * (K / 16));
  __shared__ const uint8_t* dptr[17];
  __shared__ const float* dbias[17];
  __shared__ float wslot[17];
  if (threadIdx.x < ns) {
    const int s = threadIdx.x;
    if (s < a.k) {
      const int e = a.ids[t * a.k + s];
      const bool ok = static_cast<unsigned>(e) < static_cast<unsigned>(a.E) && a.gate[e];
      dptr[s] = ok ? static_cast<const uint8_t*>(a.down[e]) : nullptr;
      dbias[s] = (ok && a.b_down) ? a.b_down[e] : nullptr;
      wslot[s] = a.w[t * a.k + s];
    } else {
      dptr[s] = static_cast<const uint8_t*>(a.sh_down);
      dbias[s] = nullptr;
      wslot[s] = a.sh_gate_vec ? a.shw[t] : 1.0f;
    }
  }
  __syncthreads();
  const int G = 256 / F::LPB;
  const int grp = threadIdx.x / F::LPB, sub = threadIdx.x % F::LPB;
  const int total = ns * R * nb;
  typename F::Raw raw[TPG];
  // issue the weight loads first; they do not depend on h
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int task = grp + G * i;
    const int s = task / (R * nb), r = (task / nb) % R, b = task % nb;
    if (task < total && row0 + r < a.H && dptr[s] != nullptr)
      F::load(raw[i], dptr[s] + static_cast<size_t>(row0 + r) * a.stride_down +
                          static_cast<size_t>(b) * F::BB, sub);
  }
  // q8 of h for every present slot: waves take 256-value pieces
  {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pieces = (K + 255) / 256;
    for (int job = wave; job < ns * pieces; job += 4) {
      const int s = job / pieces, pc = job % pieces;
      if (dptr[s] == nullptr) continue;
      const int pair = s < a.k ? t * a.k + s : a.T * a.k + t;
      const float* hsrc = a.h + static_cast<size_t>(pair) * K;
      const int e0 = pc * 256 + 4 * lane;
      const bool valid = e0 < K;
      float v[4];
      if (valid) {
        const float4 f = *reinterpret_cast<const float4*>(hsrc + e0);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
        v[0] = v[1] = v[2] = v[3] = 0.0f;
      }
      if constexpr (!MX) {
        quant_wave<B>(v, valid, lane, reinterpret_cast<int8_t*>(p_act + s * act_bytes) + pc * 256,
                      ld + s * (K / 32) + pc, lbs + s * (K / 16) + pc * 16);
      } else {
        quant_wave_pairs(v, valid, lane, reinterpret_cast<half2_t*>(p_act + s * act_bytes) + pc * 128,
                         ld + s * (K / 32) + pc * 8);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int task = grp + G * i;
    const int s = task / (R * nb), r = (task / nb) % R, b = task % nb;
    if (task < total && row0 + r < a.H && dptr[s] != nullptr) {
      ActView av{reinterpret_cast<const int8_t*>(p_act + s * act_bytes), ld + s * (K / 32),
                 lbs + s * (K / 16), reinterpret_cast<const half2_t*>(p_act + s * act_bytes)};
      const float v = block_value<F>(raw[i], av, b, sub);
      if (sub == 0) vals[(s * R + r) * nb + b] = v;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 256) {
    const int row = row0 + r;
    if (row >= a.H) break;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) {
      if (dptr[s] == nullptr) continue;
      float o = 0.0f;
      for (int b = 0; b < nb; ++b) o += vals[(s * R + r) * nb + b];
      if (dbias[s]) o += dbias[s][row];
      acc += wslot[s] * o;
    }
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
  const int act_bytes = MX ? K * 2 : K;
  int8_t* lqs = reinterpret_cast<int8_t*>(smem);
  half2_t* lap = reinterpret_cast<half2_t*>(smem);
  float* ld = reinterpret_cast<float*>(smem + act_bytes);
  int16_t* lbs = reinterpret_cast<int16_t*>(smem + act_bytes + 4 * (K / 32));
  stage_act<MX>(qs, d, bs, K, lqs, ld, lbs, lap);
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

// ids/w copies for the caller. grid 1, block 256.
__global__ void k_copy_routing(const int32_t* ids, const float* w, int n, int32_t* ids_out,
                               float* w_out) {
  for (int i = threadIdx.x; i < n; i += 256) {
    if (ids_out) ids_out[i] = ids[i];
    if (w_out) w_out[i] = w[i];
  }
}

// Rows per workgroup and tasks per lane group for a GEMV launch: aim for
// >= 2 workgroups per CU while keeping every lane group busy.
struct GemvShape { int R, tpg; };
GemvShape gemv_shape(int rows_total, int nmat, int nb, int lpb, int grid_y, int tpg_max) {
  const int G = 256 / lpb;
  int R = (G * tpg_max) / (nmat * nb);
  if (R < 1) R = 1;
  if (R > rows_total) R = rows_total;
  while (R > 1 && static_cast<long>((rows_total + R - 1) / R) * grid_y < 512) R = (R + 1) / 2;
  const int tpg = (nmat * R * nb + G - 1) / G;
  return {R, tpg};
}

int tpg_bucket(int tpg) { return tpg <= 1 ? 1 : tpg <= 2 ? 2 : tpg <= 4 ? 4 : 8; }

template <int FMT>
size_t gateup_lds(const KArgs& a, GemvShape* out) {
  using F = typename FmtOf<FMT>::T;
  const int P = a.T * a.k + a.T * a.has_shared;
  const int nb = a.H / F::BE;
  const int tpg_max = FMT == FMT_Q6_K ? 4 : 8;
  GemvShape sh = gemv_shape(a.F, 2, nb, F::LPB, P, tpg_max);
  if (out) *out = sh;
  const bool MX = FMT == FMT_MXFP4;
  return (MX ? 2 * a.H : a.H) + 4 * (a.H / 32) + 2 * (a.H / 16) +
         4 * static_cast<size_t>(2 * sh.R * nb);
}

template <int FMT>
size_t down_lds(const KArgs& a, GemvShape* out) {
  using F = typename FmtOf<FMT>::T;
  const int ns = a.k + a.has_shared;
  const int nb = a.F / F::BE;
  const int tpg_max = FMT == FMT_Q6_K ? 4 : 8;
  GemvShape sh = gemv_shape(a.H, ns, nb, F::LPB, a.T, tpg_max);
  if (out) *out = sh;
  const bool MX = FMT == FMT_MXFP4;
  return ns * ((MX ? 2 * a.F : a.F) + 4 * (a.F / 32) + 2 * (a.F / 16)) +
         4 * static_cast<size_t>(ns * sh.R * nb);
}

template <int FMT>
hipError_t gateup_dispatch(const KArgs& a, hipStream_t s) {
  using F = typename FmtOf<FMT>::T;
  const int P = a.T * a.k + a.T * a.has_shared;
  GemvShape sh;
  const size_t lds = gateup_lds<FMT>(a, &sh);
  const int tpg = tpg_bucket(sh.tpg);
  (void)sizeof(F);
  dim3 grid((a.F + sh.R - 1) / sh.R, P);
  switch (tpg) {
    case 1: hipLaunchKernelGGL((k_gateup_gemv<FMT, 1>), grid, 256, lds, s, a, sh.R); break;
    case 2: hipLaunchKernelGGL((k_gateup_gemv<FMT, 2>), grid, 256, lds, s, a, sh.R); break;
    case 4: hipLaunchKernelGGL((k_gateup_gemv<FMT, 4>), grid, 256, lds, s, a, sh.R); break;
    default: hipLaunchKernelGGL((k_gateup_gemv<FMT, 8>), grid, 256, lds, s, a, sh.R); break;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t down_dispatch(const KArgs& a, hipStream_t s) {
  GemvShape sh;
  const size_t lds = down_lds<FMT>(a, &sh);
  const int tpg = tpg_bucket(sh.tpg);
  dim3 grid((a.H + sh.R - 1) / sh.R, a.T);
  switch (tpg) {
    case 1: hipLaunchKernelGGL((k_down_gemv<FMT, 1>), grid, 256, lds, s, a, sh.R); break;
    case 2: hipLaunchKernelGGL((k_down_gemv<FMT, 2>), grid, 256, lds, s, a, sh.R); break;
    case 4: hipLaunchKernelGGL((k_down_gemv<FMT, 4>), grid, 256, lds, s, a, sh.R); break;
    default: hipLaunchKernelGGL((k_down_gemv<FMT, 8>), grid, 256, lds, s, a, sh.R); break;
  }
  return hipGetLastError();
}

}  // namespace

bool gemv_fits(const KArgs& a) {
  size_t g = a.fmt_gu == FMT_Q4_K ? gateup_lds<FMT_Q4_K>(a, nullptr)
           : a.fmt_gu == FMT_Q6_K ? gateup_lds<FMT_Q6_K>(a, nullptr)
                                  : gateup_lds<FMT_MXFP4>(a, nullptr);
  size_t d = a.fmt_d == FMT_Q4_K ? down_lds<FMT_Q4_K>(a, nullptr)
           : a.fmt_d == FMT_Q6_K ? down_lds<FMT_Q6_K>(a, nullptr)
                                 : down_lds<FMT_MXFP4>(a, nullptr);
  return g <= kMaxLds && d <= kMaxLds;
}

hipError_t launch_quant(const void* x, int dtype, int T, int H, int B, int8_t* qs, float* d,
                        int16_t* bs, uint32_t* zero_words, int n_zero, hipStream_t s) {
  dim3 grid((H + 255) / 256, T);
  if (B == 256)
    hipLaunchKernelGGL(k_quant<256>, grid, 64, 0, s, x, dtype, H, qs, d, bs, zero_words, n_zero);
  else
    hipLaunchKernelGGL(k_quant<32>, grid, 64, 0, s, x, dtype, H, qs, d, nullptr, zero_words,
                       n_zero);
  return hipGetLastError();
}

hipError_t launch_shared_gate(const KArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gate, dim3(a.T), 256, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_router(const KArgs& a, bool fuse_topk, hipStream_t s) {
  constexpr int TT = 8;
  dim3 grid(a.E + (a.sh_gate_vec ? 1 : 0), (a.T + TT - 1) / TT);
  hipLaunchKernelGGL(k_router<TT>, grid, 64, 0, s, a, fuse_topk ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_topk(const KArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((a.T + 3) / 4), 256, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup_gemv(const KArgs& a, hipStream_t s) {
  switch (a.fmt_gu) {
    case FMT_Q4_K: return gateup_dispatch<FMT_Q4_K>(a, s);
    case FMT_Q6_K: return gateup_dispatch<FMT_Q6_K>(a, s);
    default: return gateup_dispatch<FMT_MXFP4>(a, s);
  }
}

hipError_t launch_down_gemv(const KArgs& a, hipStream_t s) {
  switch (a.fmt_d) {
    case FMT_Q4_K: return down_dispatch<FMT_Q4_K>(a, s);
    case FMT_Q6_K: return down_dispatch<FMT_Q6_K>(a, s);
    default: return down_dispatch<FMT_MXFP4>(a, s);
  }
}

hipError_t launch_copy_routing(const KArgs& a, int32_t* ids_out, float* w_out, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_routing, dim3(1), 256, 0, s, a.ids, a.w, a.T * a.k, ids_out, w_out);
  return hipGetLastError();
}

hipError_t launch_block_dots(int fmt, const void* rows, int n_rows, int K, size_t stride,
                             const int8_t* qs, const float* d, const int16_t* bs, int32_t* out,
                             hipStream_t s) {
  const uint8_t* r = static_cast<const uint8_t*>(rows);
  const size_t lds = (fmt == FMT_MXFP4 ? 2 * K : K) + 4 * (K / 32) + 2 * (K / 16);
  switch (fmt) {
    case FMT_Q4_K:
      hipLaunchKernelGGL(k_block_dots<FMT_Q4_K>, dim3(n_rows), 256, lds, s, r, K, stride, qs, d,
                         bs, out);
      break;
    case FMT_Q6_K:
      hipLaunchKernelGGL(k_block_dots<FMT_Q6_K>, dim3(n_rows), 256, lds, s, r, K, stride, qs, d,
                         bs, out);
      break;
    default:
      hipLaunchKernelGGL(k_block_dots<FMT_MXFP4>, dim3(n_rows), 256, lds, s, r, K, stride, qs, d,
                         bs, out);
      break;
  }
  return hipGetLastError();
}

// Grouped path entry points land with the MFMA kernels.
hipError_t launch_bucket(const KArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gateup_grouped(const KArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_hquant(const KArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_down_grouped(const KArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_combine(const KArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
