// C ABI of the routed-expert MoE FFN layer: argument validation, workspace
// layout, path choice and the launch sequence. All device work is enqueued on
// the caller's stream; nothing here allocates or synchronizes.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "moe_internal.h"

// Device scratch of moe_layer_forward_noalloc: each GPU the library runs on
// holds its own copy from the moment the code object is loaded on it until the
// process ends. Host code never passes this name to a kernel: it stands for a
// host-side shadow; the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {

namespace {


bool known_fmt(int fmt) { return fmt >= MOE_WFMT_Q4_K && fmt <= MOE_WFMT_Q5_1; }
int block_elems(int fmt) { return act32(fmt) ? 32 : 256; }
size_t block_bytes(int fmt) {
  switch (fmt) {
    case FMT_Q4_K: return 144;
    case FMT_Q6_K: return 210;
    case FMT_MXFP4: return 17;
    case FMT_Q5_K: return 176;
    case FMT_Q2_K: return 84;
    case FMT_Q3_K: return 110;
    case FMT_Q4_0: return 18;
    default: return 24;  // Q5_1
  }
}
// q8 format of the activations that rows of a weight format consume
int act_fmt(int fmt) { return act32(fmt) ? MOE_AFMT_Q8_32 : MOE_AFMT_Q8_K; }
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
KArgs make_args(const moe_layer_desc* d, int T);

moe_status validate_desc(const moe_layer_desc* d) {
  if (!d) return MOE_EINVAL;
  const int H = d->hidden, F = d->ffn, E = d->n_expert, k = d->top_k;
  if (H <= 0 || F <= 0) return MOE_EINVAL;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (k < 1 || k > E || k > MOE_MAX_TOPK) return MOE_EINVAL;
  if (d->router != MOE_ROUTER_SOFTMAX && d->router != MOE_ROUTER_SIGMOID) return MOE_EINVAL;
  if (d->norm_topk != 0 && d->norm_topk != 1) return MOE_EINVAL;
  if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_SWIGLU_OAI) return MOE_EINVAL;
  if (d->path != MOE_PATH_AUTO && d->path != MOE_PATH_GEMV && d->path != MOE_PATH_GROUPED)
    return MOE_EINVAL;
  if (d->act_quant != MOE_ACTQ_Q8 && d->act_quant != MOE_ACTQ_MXFP8) return MOE_EINVAL;
  if (d->layout != MOE_LAYOUT_ROWS && d->layout != MOE_LAYOUT_TILE64 &&
      d->layout != MOE_LAYOUT_MX16)
    return MOE_EINVAL;
  for (int f : {d->fmt_gate, d->fmt_up, d->fmt_down})
    if (!known_fmt(f)) return MOE_EINVAL;
  if (d->fmt_gate != d->fmt_up) return MOE_EUNSUPPORTED;
  // MXFP8 activations: MXFP4 experts on the block-scaled MFMA path only
  if (d->act_quant == MOE_ACTQ_MXFP8 &&
      (d->fmt_gate != MOE_WFMT_MXFP4 || d->fmt_down != MOE_WFMT_MXFP4 || d->path == MOE_PATH_GEMV))
    return MOE_EUNSUPPORTED;
  if (H % block_elems(d->fmt_gate) != 0 || H % 32 != 0) return MOE_EINVAL;
  if (F % block_elems(d->fmt_down) != 0 || F % 32 != 0) return MOE_EINVAL;
  const size_t rb_gu = static_cast<size_t>(H / block_elems(d->fmt_gate)) * block_bytes(d->fmt_gate);
  const size_t rb_d = static_cast<size_t>(F / block_elems(d->fmt_down)) * block_bytes(d->fmt_down);
  if (d->stride_gate < rb_gu || d->stride_gate % 16) return MOE_EINVAL;
  if (d->stride_up < rb_gu || d->stride_up % 16) return MOE_EINVAL;
  if (d->stride_down < rb_d || d->stride_down % 16) return MOE_EINVAL;
  if (!d->w_router || !aligned(d->w_router, 16)) return MOE_EINVAL;
  if (!d->gate || !d->up || !d->down) return MOE_EINVAL;
  if (!aligned(d->gate, 8) || !aligned(d->up, 8) || !aligned(d->down, 8)) return MOE_EINVAL;
  if ((d->b_gate == nullptr) != (d->b_up == nullptr)) return MOE_EINVAL;
  if (d->sel_bias && !aligned(d->sel_bias, 4)) return MOE_EINVAL;
  const int nsh = (d->sh_gate != nullptr) + (d->sh_up != nullptr) + (d->sh_down != nullptr);
  if (nsh != 0 && nsh != 3) return MOE_EINVAL;
  if (nsh == 3 && (!aligned(d->sh_gate, 16) || !aligned(d->sh_up, 16) || !aligned(d->sh_down, 16)))
    return MOE_EINVAL;
  if (d->sh_gate_vec && (nsh == 0 || !aligned(d->sh_gate_vec, 16))) return MOE_EINVAL;
  if (!(d->act_limit > 0.0f) && d->act == MOE_ACT_SWIGLU_OAI) return MOE_EINVAL;
  // 64-row tiles: read by the grouped Q4_K / Q6_K ring kernels only
  if (d->layout == MOE_LAYOUT_TILE64 &&
      (d->fmt_gate != MOE_WFMT_Q4_K ||
       (d->fmt_down != MOE_WFMT_Q4_K && d->fmt_down != MOE_WFMT_Q6_K) || d->b_gate || d->b_down ||
       d->act_quant != MOE_ACTQ_Q8 || d->path == MOE_PATH_GEMV))
    return MOE_EUNSUPPORTED;
  // MX16 rows: read by the per-pair MXFP4 kernels only, whose row plans cover
  // up to 256 blocks per row within the LDS budget
  if (d->layout == MOE_LAYOUT_MX16) {
    if (d->fmt_gate != MOE_WFMT_MXFP4 || d->fmt_down != MOE_WFMT_MXFP4 ||
        d->act_quant != MOE_ACTQ_Q8 || d->path == MOE_PATH_GROUPED)
      return MOE_EUNSUPPORTED;
    if (!mx16_fits(make_args(d, 1))) return MOE_EUNSUPPORTED;
    if (d->stride_gate < mx16_row_bytes(H / 32) || d->stride_up < mx16_row_bytes(H / 32) ||
        d->stride_down < mx16_row_bytes(F / 32))
      return MOE_EINVAL;
  }
  return MOE_OK;
}

moe_status validate_x(const void* x, moe_dtype dtype) {
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_EINVAL;
  if (!x || !aligned(x, 16)) return MOE_EINVAL;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

KArgs make_args(const moe_layer_desc* d, int T) {
  KArgs a;
  memset(&a, 0, sizeof a);
  a.H = d->hidden; a.F = d->ffn; a.E = d->n_expert; a.k = d->top_k; a.T = T;
  a.router = d->router; a.norm_topk = d->norm_topk; a.route_scale = d->route_scale;
  a.w_router = d->w_router; a.sel_bias = d->sel_bias;
  a.fmt_gu = d->fmt_gate; a.fmt_d = d->fmt_down;
  a.stride_gate = d->stride_gate; a.stride_up = d->stride_up; a.stride_down = d->stride_down;
  a.gate = d->gate; a.up = d->up; a.down = d->down;
  a.b_gate = d->b_gate; a.b_up = d->b_up; a.b_down = d->b_down;
  a.act = d->act; a.act_alpha = d->act_alpha; a.act_limit = d->act_limit;
  a.sh_gate = d->sh_gate; a.sh_up = d->sh_up; a.sh_down = d->sh_down;
  a.sh_gate_vec = d->sh_gate_vec;
  a.has_shared = d->sh_gate != nullptr;
  a.mx8 = d->act_quant == MOE_ACTQ_MXFP8;
  a.tiled = d->layout == MOE_LAYOUT_TILE64;
  a.mx16 = d->layout == MOE_LAYOUT_MX16;
  return a;
}

void bind_ws(KArgs& a, const WsLayout& L, void* ws) {
  unsigned char* b = static_cast<unsigned char*>(ws);
  a.counters = reinterpret_cast<uint32_t*>(b + L.counters);
  a.xqs = reinterpret_cast<int8_t*>(b + L.xqs);
  a.xd = reinterpret_cast<float*>(b + L.xd);
  a.xbs = reinterpret_cast<int16_t*>(b + L.xbs);
  a.logits = reinterpret_cast<float*>(b + L.logits);
  a.ids = reinterpret_cast<int32_t*>(b + L.ids);
  a.w = reinterpret_cast<float*>(b + L.w);
  a.shw = reinterpret_cast<float*>(b + L.shw);
  a.slots = reinterpret_cast<SlotRef*>(b + L.slots);
  a.h = reinterpret_cast<float*>(b + L.h);
  a.hqs = reinterpret_cast<int8_t*>(b + L.hqs);
  a.hd = reinterpret_cast<float*>(b + L.hd);
  a.hbs = reinterpret_cast<int16_t*>(b + L.hbs);
  a.rpart = reinterpret_cast<double*>(b + L.rpart);
  a.plist = reinterpret_cast<int2*>(b + L.plist);
  a.present = reinterpret_cast<int32_t*>(b + L.present);
  a.tiles = reinterpret_cast<GTile*>(b + L.tiles);
  a.part = reinterpret_cast<float*>(b + L.part);
  a.xe = L.xe ? b + L.xe : nullptr;
  a.he = L.he ? b + L.he : nullptr;
}

// Per-kernel (start, stop) event pairs of moe_layer_forward_timed.
struct Stages {
  hipEvent_t* ev;
  int n;
  int i;
  Ev next() {
    Ev e;
    if (ev && 2 * i + 1 < n) {
      e.start = ev[2 * i];
      e.stop = ev[2 * i + 1];
    }
    ++i;
    return e;
  }
};

}  // namespace

// Dispatch rule between the two expert-FFN paths (MOE_PATH_AUTO). The
// per-(token, slot) GEMV path (moe_kernels.hip) streams every pair's expert
// rows; the expert-grouped path (moe_grouped.hip) reads each selected expert's
// rows once per 16 tokens routed to it through LDS-ring int8-MFMA tiles, at
// the cost of seven launches. Measured on one MI355X (us per forward, GEMV /
// grouped):
//   Qwen3.6 shape, 1.77 MB experts, 8 + 1 slots, random routing: T = 1: 15.5 /
//     42.6, T = 8: 52.2 / 59.5, T = 10: 63.6 / 70.3, T = 12: 74.5 / 72.6,
//     T = 16: 92.7 / 84.0;
//   DeepSeek-V4-Flash shape, 16.3 MB experts, 6 + 1 slots, Zipf routing:
//     T = 1: 74.5 / 66.0, T = 2: 138.7 / 84.3, T = 16: 1010 / 168;
//   Kimi-K2 shape, 24.8 MB experts, 8 + 1 slots: T = 1: 123 / 100.
// So: grouped once the per-pair bytes T (k + shared) expert_bytes reach 160 MB
// (the small-expert crossover lies between 159 and 191 MB), and at every T for
// experts of 8 MB or more (the per-pair kernels stream such rows more slowly
// than the tiles, even for one token). Layers with a matrix in a format without
// tile kernels (MXFP4, Q5_K, Q2_K) take the GEMV path.
constexpr double kGroupedMinPairBytes = 160e6;
constexpr double kGroupedMinExpertBytes = 8e6;

static size_t expert_block_bytes(const moe_layer_desc* d) {
  const size_t gu = static_cast<size_t>(d->hidden / block_elems(d->fmt_gate)) * block_bytes(d->fmt_gate);
  const size_t dn = static_cast<size_t>(d->ffn / block_elems(d->fmt_down)) * block_bytes(d->fmt_down);
  return 2 * static_cast<size_t>(d->ffn) * gu + static_cast<size_t>(d->hidden) * dn;
}

bool use_grouped(const moe_layer_desc* d, int T) {
  if (d->act_quant == MOE_ACTQ_MXFP8) return T >= 1;  // block-scaled MFMA tiles at every T
  if (d->layout == MOE_LAYOUT_TILE64) return T >= 1;  // only the ring kernels read tiles
  auto tiled = [](int f) { return f == FMT_Q4_K || f == FMT_Q6_K; };
  if (!tiled(d->fmt_gate) || !tiled(d->fmt_down) || T < 1) return false;
  if (d->path == MOE_PATH_GEMV) return false;
  if (d->path == MOE_PATH_GROUPED) return true;
  // per-pair shapes past the GEMV kernels' LDS budget or task plans: the tiles
  if (!gemv_fits(make_args(d, T))) return true;
  const double eb = static_cast<double>(expert_block_bytes(d));
  if (eb >= kGroupedMinExpertBytes) return true;
  const int slots = d->top_k + (d->sh_gate != nullptr ? 1 : 0);
  return static_cast<double>(T) * slots * eb >= kGroupedMinPairBytes;
}

WsLayout ws_layout(int H, int F, int E, int k, int T, int has_shared, bool grouped, bool mx8) {
  WsLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t P = static_cast<size_t>(T) * k + static_cast<size_t>(T) * has_shared;
  L.counters = take(4 * (P > 64 ? P : 64));
  L.xqs = take(static_cast<size_t>(T) * H);
  L.xd = take(static_cast<size_t>(T) * (H / 32) * 4);
  L.xbs = take(static_cast<size_t>(T) * (H / 16) * 2);
  L.logits = take(static_cast<size_t>(T) * E * 4);
  L.ids = take(static_cast<size_t>(T) * k * 4);
  L.w = take(static_cast<size_t>(T) * k * 4);
  L.shw = take(static_cast<size_t>(T) * 4);
  L.slots = take(static_cast<size_t>(T) * k * sizeof(SlotRef));
  L.h = take(P * F * 4);
  if (grouped) {
    const RouterSplit rs = router_split(T, E, H);
    L.hqs = take(P * F);
    L.hd = take(P * (F / 256) * 4);
    L.hbs = take(P * (F / 16) * 2);
    L.rpart = take(static_cast<size_t>(rs.ks) * T * (E + 1) * 8);
    L.plist = take(P * 8);
    L.present = take(P * 4);
    L.tiles = take(static_cast<size_t>(max_tiles(T, k, E, has_shared)) * sizeof(GTile));
    L.part = take(P * H * 4);
    L.xe = mx8 ? take(static_cast<size_t>(T) * mx8_pitch(H)) : 0;
    L.he = mx8 ? take(P * mx8_pitch(F)) : 0;
  } else {
    // q8 of h for an MXFP4 down, quantized once per pair: fp16 pairs + scales
    L.hqs = take(P * (F / 32) * 80);  // 80 bytes per 32-value block (kApPitch pairs)
    L.hd = take(P * (F / 32) * 4);
    L.hbs = 0;
    L.rpart = L.plist = L.present = L.tiles = L.part = L.xe = L.he = 0;
  }
  L.total = off;
  return L;
}

static WsLayout ws_of(const moe_layer_desc* d, int T, bool grouped) {
  return ws_layout(d->hidden, d->ffn, d->n_expert, d->top_k, T, d->sh_gate != nullptr, grouped,
                   d->act_quant == MOE_ACTQ_MXFP8);
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported combination";
    case MOE_ENOWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t moe_workspace_size(const moe_layer_desc* desc, int T) {
  if (validate_desc(desc) != MOE_OK || T < 0 || T > kMaxTokens) return 0;
  const bool g = use_grouped(desc, T);
  return ws_of(desc, T, g).total;
}

moe_status moe_quantize_act_q8k(const void* x, moe_dtype dtype, int T, int H, moe_afmt fmt,
                                moe_qact* out, hipStream_t stream) {
  if (validate_x(x, dtype) != MOE_OK || !out) return MOE_EINVAL;
  if (fmt == MOE_AFMT_MXFP8) {
    if (T < 0 || H <= 0 || H % 32 != 0) return MOE_EINVAL;
    if (!out->qs || !out->scales || !aligned(out->qs, 16) || !aligned(out->scales, 16))
      return MOE_EINVAL;
    out->fmt = fmt;
    out->T = T;
    out->H = H;
    if (T == 0) return MOE_OK;
    return hip_status(launch_quant_mx8(x, dtype, T, H, reinterpret_cast<uint8_t*>(out->qs),
                                       out->scales, stream, Ev{}));
  }
  if (fmt != MOE_AFMT_Q8_K && fmt != MOE_AFMT_Q8_32) return MOE_EINVAL;
  const int B = fmt == MOE_AFMT_Q8_K ? 256 : 32;
  if (T < 0 || H <= 0 || H % B != 0) return MOE_EINVAL;
  if (!out->qs || !out->d || !aligned(out->qs, 16) || !aligned(out->d, 4)) return MOE_EINVAL;
  if (fmt == MOE_AFMT_Q8_K && (!out->bsums || !aligned(out->bsums, 4))) return MOE_EINVAL;
  out->fmt = fmt;
  out->T = T;
  out->H = H;
  if (T == 0) return MOE_OK;
  return hip_status(launch_quant(x, dtype, T, H, B, out->qs, out->d,
                                 fmt == MOE_AFMT_Q8_K ? out->bsums : nullptr, stream));
}

moe_status moe_route_topk(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                          int32_t* ids, float* w, float* logits, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st != MOE_OK) return st;
  if (validate_x(x, dtype) != MOE_OK) return MOE_EINVAL;
  if (T < 0 || T > kMaxTokens || !ids || !w) return MOE_EINVAL;
  if (!aligned(ids, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4))) return MOE_EINVAL;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  const bool g = use_grouped(desc, T);
  const WsLayout L = ws_of(desc, T, g);
  if (ws_bytes < L.total) return MOE_ENOWORKSPACE;
  if (T == 0) return MOE_OK;
  KArgs a = make_args(desc, T);
  bind_ws(a, L, ws);
  a.x = x; a.x_dtype = dtype;
  a.ids = ids; a.w = w;
  if (logits) a.logits = logits;
  a.sh_gate_vec = nullptr;  // the shared gate is not part of routing
  hipError_t e;
  if (g) {
    const RouterSplit rs = router_split(T, desc->n_expert, desc->hidden);
    e = launch_router_grouped(a, false, rs, stream, Ev{});
    if (e == hipSuccess) e = launch_topk_sum(a, rs, stream, Ev{});
  } else {
    e = launch_router(a, false, 0, stream, Ev{});
    if (e == hipSuccess) e = launch_topk(a, stream);
  }
  return hip_status(e);
}

// Host-side check that the chosen path's launch shapes fit, before anything is enqueued.
static bool path_fits(const KArgs& a, bool grouped) { return grouped || gemv_fits(a); }

// Expert part of the layer. GEMV path: per-pair gate/up (+ top-k unless routing
// is given), then per-token down + combine. Grouped path (routing already in
// a.ids / a.w): bucketing, tile gate/up, q8 of h, tile down, combine.
static moe_status expert_ffn_impl(KArgs& a, bool grouped, bool routing_given, hipStream_t stream,
                                  Stages& st) {
  hipError_t e;
  if (grouped && a.mx8) {
    const int mt = max_tiles(a.T, a.k, a.E, a.has_shared);
    e = launch_bucket(a, stream, st.next());
    if (e == hipSuccess) e = launch_gateup_mx(a, mt, stream, st.next());
    if (e == hipSuccess) e = launch_hquant_mx8(a, stream, st.next());
    if (e == hipSuccess) e = launch_down_mx(a, mt, stream, st.next());
    if (e == hipSuccess) e = launch_combine(a, stream, st.next());
  } else if (grouped) {
    e = launch_bucket(a, stream, st.next());
    if (e == hipSuccess) e = launch_gateup_grouped(a, stream, st.next());
    if (e == hipSuccess) e = launch_hquant(a, stream, st.next());
    if (e == hipSuccess) e = launch_down_grouped(a, stream, st.next());
    if (e == hipSuccess) e = launch_combine(a, stream, st.next());
  } else {
    e = launch_gateup(a, routing_given, stream, st.next());
    if (e == hipSuccess && gemv_hquant(a.fmt_d, a.F, a.k, a.has_shared, a.mx16)) e = launch_hquant_pairs(a, stream, st.next());
    if (e == hipSuccess) e = launch_down(a, stream, st.next());
  }
  return hip_status(e);
}

// Quantized x as the layer's gate/up rows consume it, for T tokens.
static bool qact_ok(const moe_layer_desc* desc, const moe_qact* xq, int T) {
  if (desc->act_quant == MOE_ACTQ_MXFP8)
    return xq->fmt == MOE_AFMT_MXFP8 && xq->T >= T && xq->H == desc->hidden && xq->qs &&
           xq->scales && aligned(xq->qs, 16) && aligned(xq->scales, 16);
  const int want_afmt = act_fmt(desc->fmt_gate);
  if (xq->fmt != want_afmt || xq->T < T || xq->H != desc->hidden) return false;
  if (!xq->qs || !xq->d || !aligned(xq->qs, 16) || !aligned(xq->d, 4)) return false;
  if (want_afmt == MOE_AFMT_Q8_K && (!xq->bsums || !aligned(xq->bsums, 4))) return false;
  return true;
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_qact* xq, const void* x,
                          moe_dtype dtype, int T, const int32_t* ids, const float* w, float* y,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0 || T > kMaxTokens || !xq || !ids || !w || !y) return MOE_EINVAL;
  if (!qact_ok(desc, xq, T)) return MOE_EINVAL;
  if (desc->sh_gate_vec && validate_x(x, dtype) != MOE_OK) return MOE_EINVAL;
  if (!aligned(ids, 4) || !aligned(w, 4) || !aligned(y, 16)) return MOE_EINVAL;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  const bool g = use_grouped(desc, T);
  const WsLayout L = ws_of(desc, T, g);
  if (ws_bytes < L.total) return MOE_ENOWORKSPACE;
  if (T == 0) return MOE_OK;
  KArgs a = make_args(desc, T);
  bind_ws(a, L, ws);
  a.x = x; a.x_dtype = dtype;
  a.xqs = xq->qs; a.xd = xq->d; a.xbs = xq->bsums;
  if (a.mx8) a.xe = xq->scales;
  a.ids = const_cast<int32_t*>(ids);
  a.w = const_cast<float*>(w);
  a.y = y;
  if (!path_fits(a, g)) return MOE_EUNSUPPORTED;
  if (desc->sh_gate_vec && launch_shared_gate(a, stream) != hipSuccess) return MOE_EHIP;
  Stages stg{nullptr, 0, 0};
  return expert_ffn_impl(a, g, true, stream, stg);
}

// Argument checks of a layer call (everything but the workspace), and the path
// and workspace layout it takes.
static moe_status check_forward(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                                float* y, int32_t* ids_out, float* w_out, hipEvent_t* events,
                                int n_events, bool* grouped, WsLayout* L) {
  moe_status st = validate_desc(desc);
  if (st != MOE_OK) return st;
  if (validate_x(x, dtype) != MOE_OK) return MOE_EINVAL;
  if (T < 0 || T > kMaxTokens || !y || !aligned(y, 16)) return MOE_EINVAL;
  if ((ids_out && !aligned(ids_out, 4)) || (w_out && !aligned(w_out, 4))) return MOE_EINVAL;
  if (events && n_events < 0) return MOE_EINVAL;
  *grouped = use_grouped(desc, T);
  *L = ws_of(desc, T, *grouped);
  return MOE_OK;
}

// The layer's launch sequence on a checked call with its workspace bound.
static moe_status run_forward(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                              float* y, int32_t* ids_out, float* w_out, void* ws, bool g,
                              const WsLayout& L, hipStream_t stream, hipEvent_t* events,
                              int n_events) {
  if (T == 0) return MOE_OK;
  KArgs a = make_args(desc, T);
  bind_ws(a, L, ws);
  a.x = x; a.x_dtype = dtype;
  a.y = y;
  if (ids_out) a.ids = ids_out;
  if (w_out) a.w = w_out;
  if (!path_fits(a, g)) return MOE_EUNSUPPORTED;
  Stages stg{events, n_events, 0};
  if (g) {
    const RouterSplit rs = router_split(T, desc->n_expert, desc->hidden);
    hipError_t e = launch_router_grouped(a, true, rs, stream, stg.next());
    if (e == hipSuccess) e = launch_topk_sum(a, rs, stream, stg.next());
    if (e != hipSuccess) return MOE_EHIP;
    return expert_ffn_impl(a, true, false, stream, stg);
  }
  hipError_t e = launch_router(a, true, 0, stream, stg.next());
  if (e != hipSuccess) return MOE_EHIP;
  return expert_ffn_impl(a, false, false, stream, stg);
}

static moe_status layer_forward(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                                float* y, int32_t* ids_out, float* w_out, void* ws,
                                size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                                int n_events) {
  bool g;
  WsLayout L;
  moe_status st = check_forward(desc, x, dtype, T, y, ids_out, w_out, events, n_events, &g, &L);
  if (st != MOE_OK) return st;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  if (ws_bytes < L.total) return MOE_ENOWORKSPACE;
  return run_forward(desc, x, dtype, T, y, ids_out, w_out, ws, g, L, stream, events, n_events);
}

// Per-device address of `scratch`, looked up once per device with that device
// current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

static void* scratch_ptr(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

moe_status moe_layer_forward(const moe_layer_desc* desc, const void* x, moe_dtype dtype, int T,
                             float* y, int32_t* ids_out, float* w_out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  return layer_forward(desc, x, dtype, T, y, ids_out, w_out, ws, ws_bytes, stream, nullptr, 0);
}

moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* x, moe_dtype dtype,
                                     int T, float* y, int32_t* ids_out, float* w_out,
                                     hipStream_t stream) {
  bool g;
  WsLayout L;
  moe_status st = check_forward(desc, x, dtype, T, y, ids_out, w_out, nullptr, 0, &g, &L);
  if (st != MOE_OK) return st;
  if (L.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOWORKSPACE;
  if (T == 0) return MOE_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  void* ws = scratch_ptr(dev);
  if (!ws) return MOE_EHIP;
  return run_forward(desc, x, dtype, T, y, ids_out, w_out, ws, g, L, stream, nullptr, 0);
}

moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const void* x, moe_dtype dtype,
                                   int T, float* y, int32_t* ids_out, float* w_out, void* ws,
                                   size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                                   int n_events) {
  return layer_forward(desc, x, dtype, T, y, ids_out, w_out, ws, ws_bytes, stream, events,
                       n_events);
}

int moe_layer_stage_count(const moe_layer_desc* desc, int T) {
  if (validate_desc(desc) != MOE_OK || T <= 0 || T > kMaxTokens) return 0;
  if (use_grouped(desc, T)) return 7;
  return gemv_hquant(desc->fmt_down, desc->ffn, desc->top_k, desc->sh_gate != nullptr,
                     desc->layout == MOE_LAYOUT_MX16) ? 4 : 3;
}

const char* moe_layer_stage_name(const moe_layer_desc* desc, int T, int stage) {
  static const char* gemv[] = {"router", "gateup", "down"};
  static const char* gemv_hq[] = {"router", "gateup", "hquant", "down"};
  static const char* grouped[] = {"router", "topk", "bucket", "gateup", "hquant", "down",
                                  "combine"};
  const int n = moe_layer_stage_count(desc, T);
  if (stage < 0 || stage >= n) return nullptr;
  return n == 7 ? grouped[stage] : n == 4 ? gemv_hq[stage] : gemv[stage];
}

moe_status moe_repack_tile64(moe_wfmt fmt, const void* src, size_t src_stride, int n_rows, int K,
                             void* dst, hipStream_t stream) {
  if (fmt != MOE_WFMT_Q4_K && fmt != MOE_WFMT_Q6_K) return MOE_EINVAL;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return MOE_EINVAL;
  if (n_rows <= 0 || n_rows % 64 || K <= 0 || K % 256) return MOE_EINVAL;
  const int nb = K / 256;
  const size_t BB = block_bytes(fmt), row = static_cast<size_t>(nb) * BB;
  if (src_stride < row || src_stride % 2) return MOE_EINVAL;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + (static_cast<size_t>(n_rows) - 1) * src_stride + row;
  const uintptr_t d1 = d0 + static_cast<size_t>(n_rows) * row;
  if (s0 < d1 && d0 < s1) return MOE_EINVAL;  // overlapping buffers
  return hip_status(launch_repack_tile64(static_cast<const uint8_t*>(src), src_stride, n_rows, nb,
                                         static_cast<int>(BB), static_cast<uint8_t*>(dst), stream));
}

moe_status moe_repack_mx16(const void* src, size_t src_stride, int n_rows, int K, void* dst,
                           size_t dst_stride, hipStream_t stream) {
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return MOE_EINVAL;
  if (n_rows <= 0 || K <= 0 || K % 32) return MOE_EINVAL;
  const int nb = K / 32;
  if (src_stride < 17 * static_cast<size_t>(nb)) return MOE_EINVAL;
  if (dst_stride < mx16_row_bytes(nb) || dst_stride % 16) return MOE_EINVAL;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + (static_cast<size_t>(n_rows) - 1) * src_stride + 17 * static_cast<size_t>(nb);
  const uintptr_t d1 = d0 + (static_cast<size_t>(n_rows) - 1) * dst_stride + mx16_row_bytes(nb);
  if (s0 < d1 && d0 < s1) return MOE_EINVAL;  // overlapping buffers
  return hip_status(launch_repack_mx16(static_cast<const uint8_t*>(src), src_stride, n_rows, nb,
                                       static_cast<uint8_t*>(dst), dst_stride, stream));
}

moe_status moe_test_block_dots_mx16(const void* rows, int n_rows, int K, size_t stride,
                                    const moe_qact* xq, int token, int32_t* out,
                                    hipStream_t stream) {
  if (!rows || !aligned(rows, 16) || !out || !xq || n_rows < 0 || K <= 0 || K % 32) return MOE_EINVAL;
  if (K / 32 > 256) return MOE_EUNSUPPORTED;
  if (stride < mx16_row_bytes(K / 32) || stride % 16) return MOE_EINVAL;
  if (xq->fmt != MOE_AFMT_Q8_32 || xq->H != K || token < 0 || token >= xq->T) return MOE_EINVAL;
  if (!xq->qs || !xq->d) return MOE_EINVAL;
  if (n_rows == 0) return MOE_OK;
  return hip_status(launch_block_dots_mx16(rows, n_rows, K, stride,
                                           xq->qs + static_cast<size_t>(token) * K,
                                           xq->d + static_cast<size_t>(token) * (K / 32), out,
                                           stream));
}

moe_status moe_test_block_dots(moe_wfmt fmt, const void* rows, int n_rows, int K, size_t stride,
                               const moe_qact* xq, int token, int32_t* out, hipStream_t stream) {
  if (!known_fmt(fmt)) return MOE_EINVAL;
  if (!rows || !aligned(rows, 16) || !out || !xq || n_rows < 0 || K <= 0) return MOE_EINVAL;
  if (K % block_elems(fmt) != 0) return MOE_EINVAL;
  const size_t rb = static_cast<size_t>(K / block_elems(fmt)) * block_bytes(fmt);
  if (stride < rb || stride % 16) return MOE_EINVAL;
  const int want = act_fmt(fmt);
  if (xq->fmt != want || xq->H != K || token < 0 || token >= xq->T) return MOE_EINVAL;
  if (!xq->qs || !xq->d || (want == MOE_AFMT_Q8_K && !xq->bsums)) return MOE_EINVAL;
  if (n_rows == 0) return MOE_OK;
  const int B = want == MOE_AFMT_Q8_K ? 256 : 32;
  return hip_status(launch_block_dots(
      fmt, rows, n_rows, K, stride, xq->qs + static_cast<size_t>(token) * K,
      xq->d + static_cast<size_t>(token) * (K / B),
      want == MOE_AFMT_Q8_K ? xq->bsums + static_cast<size_t>(token) * (K / 16) : nullptr, out,
      stream));
}

moe_status moe_test_tile_dots(int mode, const void* rows, int n_rows, int K, size_t stride,
                              const moe_qact* xq, int n_tok, int32_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (mode < 0 || mode > 2) return MOE_EINVAL;
  const int fmt = mode == 2 ? FMT_Q6_K : FMT_Q4_K;
  if (!rows || !aligned(rows, 16) || !out || !aligned(out, 4) || !xq) return MOE_EINVAL;
  if (n_tok < 1 || n_tok > 16 || n_rows <= 0 || K <= 0 || K % 256 != 0) return MOE_EINVAL;
  if (n_rows % (mode == 1 ? 128 : 64) != 0) return MOE_EINVAL;
  const size_t rb = static_cast<size_t>(K / 256) * block_bytes(fmt);
  if (stride < rb || stride % 16) return MOE_EINVAL;
  if (xq->fmt != MOE_AFMT_Q8_K || xq->H != K || xq->T < n_tok) return MOE_EINVAL;
  if (!xq->qs || !xq->d || !xq->bsums || !aligned(xq->qs, 16) || !aligned(xq->d, 4) ||
      !aligned(xq->bsums, 16))
    return MOE_EINVAL;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  if (ws_bytes < tile_dots_ws(mode, n_rows, K, n_tok)) return MOE_ENOWORKSPACE;
  return hip_status(launch_tile_dots(mode, rows, n_rows, K, stride, xq->qs, xq->d, xq->bsums,
                                     n_tok, out, ws, stream));
}

size_t moe_test_tile_dots_ws(int mode, int n_rows, int K, int n_tok) {
  if (mode < 0 || mode > 2 || n_rows <= 0 || n_tok < 1 || n_tok > 16) return 0;
  return tile_dots_ws(mode, n_rows, K, n_tok);
}

moe_status moe_test_preact(const moe_layer_desc* desc, const moe_qact* xq, int T,
                           const int32_t* ids, int which, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st != MOE_OK) return st;
  if (which != 0 && which != 1) return MOE_EINVAL;
  if (T < 0 || T > kMaxTokens || !xq || !ids || !out) return MOE_EINVAL;
  if (!qact_ok(desc, xq, T)) return MOE_EINVAL;
  if (!aligned(ids, 4) || !aligned(out, 16)) return MOE_EINVAL;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  const bool g = use_grouped(desc, T);
  const WsLayout L = ws_of(desc, T, g);
  if (ws_bytes < L.total) return MOE_ENOWORKSPACE;
  if (T == 0) return MOE_OK;
  KArgs a = make_args(desc, T);
  bind_ws(a, L, ws);
  a.xqs = xq->qs; a.xd = xq->d; a.xbs = xq->bsums;
  if (a.mx8) a.xe = xq->scales;
  a.ids = const_cast<int32_t*>(ids);
  a.h = out;
  a.act = which ? ACT_PRE_UP : ACT_PRE_GATE;
  if (!path_fits(a, g)) return MOE_EUNSUPPORTED;
  hipError_t e;
  if (g) {
    e = launch_bucket(a, stream, Ev{});
    if (e == hipSuccess)
      e = a.mx8 ? launch_gateup_mx(a, max_tiles(a.T, a.k, a.E, a.has_shared), stream, Ev{})
                : launch_gateup_grouped(a, stream, Ev{});
  } else {
    e = launch_gateup(a, true, stream, Ev{});
  }
  return hip_status(e);
}

moe_status moe_probe_read_wall(const void* buf, size_t bytes, int nwg, uint32_t* sink,
                               hipStream_t stream) {
  if (!buf || !aligned(buf, 16) || bytes % 16 || !sink || !aligned(sink, 4)) return MOE_EINVAL;
  if (nwg < 1 || nwg > (1 << 20)) return MOE_EINVAL;
  if (bytes == 0) return MOE_OK;
  return hip_status(launch_read_wall(buf, bytes, sink, nwg, stream));
}

moe_status moe_probe_empty_chain(int n, hipStream_t stream) {
  if (n < 1 || n > 4096) return MOE_EINVAL;
  return hip_status(launch_empty_chain(n, stream));
}

moe_status moe_probe_mfma_i8(int k64, int iters, int nwg, int32_t* sink, hipStream_t stream) {
  if ((k64 != 0 && k64 != 1) || iters < 0 || nwg < 1 || nwg > (1 << 20) || !sink ||
      !aligned(sink, 4))
    return MOE_EINVAL;
  return hip_status(launch_mfma_i8(k64, iters, nwg, sink, stream));
}

}  // extern "C"
