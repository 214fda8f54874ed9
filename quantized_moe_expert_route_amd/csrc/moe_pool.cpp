// Expert pool: pinned host tier, device slot arena, per-layer pointer tables
// and the copy-stream ordering around the slot policy (moe_pool_policy.h).
//
// Ordering. Every resolve is an epoch. Its copies run on the pool's copy
// stream after an event recorded on the compute stream at the call, so they
// start only once the kernels enqueued before it (the previous epochs, the
// only ones that may read the slots the policy hands out) are done; the
// compute stream then waits for an event recorded after the copies. Prefetch
// copies follow the same rule; the next resolve's event covers them too.
// The layer's table is rewritten with an async copy on the compute stream
// from a ring of pinned mirrors, each reused once its previous copy is done.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/moe_pool.h"
#include "moe_pool_policy.h"

using moe::PoolPolicy;

namespace {

constexpr int kMirrors = 8;

size_t pitch_of(size_t slab) { return (slab + 255) & ~static_cast<size_t>(255); }

bool config_ok(const moe_pool_config* c) {
  if (!c || c->n_layers < 1 || c->n_experts < 1 || c->slab_bytes == 0) return false;
  if (c->up_offset % 16 || c->down_offset % 16) return false;
  if (c->up_offset >= c->slab_bytes || c->down_offset >= c->slab_bytes) return false;
  if (c->n_slots < 1 || c->n_transient < 1 || c->n_transient > c->n_slots) return false;
  if (static_cast<int64_t>(c->n_layers) * c->n_experts > (int64_t{1} << 30)) return false;
  return true;
}

}  // namespace

struct moe_pool {
  moe_pool_config cfg;
  PoolPolicy policy;
  size_t pitch = 0;
  uint8_t* host = nullptr;   // pinned [L E] slabs
  uint8_t* arena = nullptr;  // device [n_slots] slabs
  void** dtab = nullptr;     // device [L][3][E] pointers
  void** mirror[kMirrors] = {};
  hipEvent_t mirror_ev[kMirrors] = {};
  int next_mirror = 0;
  hipStream_t copy = nullptr;
  hipEvent_t ev_compute = nullptr, ev_copy = nullptr;
  int32_t* ids_host = nullptr;  // pinned, for moe_pool_layer_step
  size_t ids_host_n = 0;
  int64_t bytes_h2d = 0;
  std::vector<PoolPolicy::Place> places;

  explicit moe_pool(const moe_pool_config& c)
      : cfg(c), policy(c.n_layers, c.n_experts, c.n_slots, c.n_transient) {}

  // copies of the placements that need one, ordered after the stream's work so far
  hipError_t copy_in(hipStream_t stream) {
    hipError_t e = hipEventRecord(ev_compute, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(copy, ev_compute, 0);
    for (const auto& p : places) {
      if (e != hipSuccess) break;
      if (!p.copy) continue;
      e = hipMemcpyAsync(arena + static_cast<size_t>(p.slot) * pitch,
                         host + static_cast<size_t>(p.key) * pitch, cfg.slab_bytes,
                         hipMemcpyHostToDevice, copy);
      bytes_h2d += static_cast<int64_t>(cfg.slab_bytes);
    }
    return e;
  }
};

extern "C" {

moe_status moe_pool_create(const moe_pool_config* cfg, moe_pool** out) {
  if (!out || !config_ok(cfg)) return MOE_EINVAL;
  *out = nullptr;
  moe_pool* p = new (std::nothrow) moe_pool(*cfg);
  if (!p) return MOE_EHIP;
  p->pitch = pitch_of(cfg->slab_bytes);
  const size_t n_host = static_cast<size_t>(cfg->n_layers) * cfg->n_experts;
  const size_t tab = static_cast<size_t>(3) * cfg->n_experts * sizeof(void*);
  bool ok = hipHostMalloc(reinterpret_cast<void**>(&p->host), n_host * p->pitch,
                          hipHostMallocDefault) == hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&p->arena),
                       static_cast<size_t>(cfg->n_slots) * p->pitch) == hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&p->dtab), tab * cfg->n_layers) == hipSuccess;
  ok = ok && hipMemset(p->dtab, 0, tab * cfg->n_layers) == hipSuccess;
  for (int i = 0; ok && i < kMirrors; ++i) {
    ok = hipHostMalloc(reinterpret_cast<void**>(&p->mirror[i]), tab, hipHostMallocDefault) ==
             hipSuccess &&
         hipEventCreateWithFlags(&p->mirror_ev[i], hipEventDisableTiming) == hipSuccess;
  }
  p->ids_host_n = static_cast<size_t>(2048) * MOE_MAX_TOPK;  // tokens x slots of one step
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&p->ids_host), p->ids_host_n * 4,
                           hipHostMallocDefault) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&p->copy, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_compute, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_copy, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;  // the table memset is done
  if (!ok) {
    moe_pool_destroy(p);
    return MOE_EHIP;
  }
  *out = p;
  return MOE_OK;
}

void moe_pool_destroy(moe_pool* p) {
  if (!p) return;
  if (p->copy) (void)hipStreamSynchronize(p->copy);
  for (int i = 0; i < kMirrors; ++i) {
    if (p->mirror_ev[i]) {
      (void)hipEventSynchronize(p->mirror_ev[i]);
      (void)hipEventDestroy(p->mirror_ev[i]);
    }
    if (p->mirror[i]) (void)hipHostFree(p->mirror[i]);
  }
  if (p->ev_compute) (void)hipEventDestroy(p->ev_compute);
  if (p->ev_copy) (void)hipEventDestroy(p->ev_copy);
  if (p->copy) (void)hipStreamDestroy(p->copy);
  if (p->ids_host) (void)hipHostFree(p->ids_host);
  if (p->dtab) (void)hipFree(p->dtab);
  if (p->arena) (void)hipFree(p->arena);
  if (p->host) (void)hipHostFree(p->host);
  delete p;
}

uint8_t* moe_pool_host_slab(moe_pool* p, int layer, int expert) {
  if (!p || layer < 0 || layer >= p->cfg.n_layers || expert < 0 || expert >= p->cfg.n_experts)
    return nullptr;
  return p->host + (static_cast<size_t>(layer) * p->cfg.n_experts + expert) * p->pitch;
}

moe_status moe_pool_layer_tables(moe_pool* p, int layer, const void* const** gate,
                                 const void* const** up, const void* const** down) {
  if (!p || layer < 0 || layer >= p->cfg.n_layers || !gate || !up || !down) return MOE_EINVAL;
  void** t = p->dtab + static_cast<size_t>(layer) * 3 * p->cfg.n_experts;
  *gate = t;
  *up = t + p->cfg.n_experts;
  *down = t + 2 * p->cfg.n_experts;
  return MOE_OK;
}

moe_status moe_pool_resolve(moe_pool* p, int layer, const int32_t* ids, int n,
                            hipStream_t stream) {
  if (!p || layer < 0 || layer >= p->cfg.n_layers || n < 0 || (n > 0 && !ids)) return MOE_EINVAL;
  if (!p->policy.resolve(layer, ids, n, &p->places)) return MOE_ENOWORKSPACE;
  hipError_t e = p->copy_in(stream);
  // every copy issued so far (this call's and earlier prefetches) before the
  // stream's next work
  if (e == hipSuccess) e = hipEventRecord(p->ev_copy, p->copy);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, p->ev_copy, 0);
  if (e != hipSuccess) return MOE_EHIP;
  // the layer's table: requested experts -> their slots, every other entry NULL
  const int E = p->cfg.n_experts;
  const int m = p->next_mirror;
  p->next_mirror = (m + 1) % kMirrors;
  if (hipEventSynchronize(p->mirror_ev[m]) != hipSuccess) return MOE_EHIP;
  void** h = p->mirror[m];
  memset(h, 0, static_cast<size_t>(3) * E * sizeof(void*));
  for (const auto& pl : p->places) {
    const int ex = pl.key - layer * E;
    uint8_t* base = p->arena + static_cast<size_t>(pl.slot) * p->pitch;
    h[ex] = base;
    h[E + ex] = base + p->cfg.up_offset;
    h[2 * E + ex] = base + p->cfg.down_offset;
  }
  e = hipMemcpyAsync(p->dtab + static_cast<size_t>(layer) * 3 * E, h,
                     static_cast<size_t>(3) * E * sizeof(void*), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipEventRecord(p->mirror_ev[m], stream);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_pool_prefetch(moe_pool* p, int layer, const int32_t* ids, int n,
                             hipStream_t stream) {
  if (!p || layer < 0 || layer >= p->cfg.n_layers || n < 0 || (n > 0 && !ids)) return MOE_EINVAL;
  p->policy.prefetch(layer, ids, n, &p->places);
  if (p->places.empty()) return MOE_OK;
  return p->copy_in(stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_pool_get_stats(const moe_pool* p, moe_pool_stats* out) {
  if (!p || !out) return MOE_EINVAL;
  const PoolPolicy::Stats& s = p->policy.stats();
  *out = moe_pool_stats{s.epochs,          s.requests,   s.hits_resident,  s.hits_transient,
                        s.admitted,        s.transient_loads, s.promotions, s.evictions,
                        s.prefetch_loads,  s.prefetch_hits,   p->bytes_h2d};
  return MOE_OK;
}

// Step scratch: the layer's workspace, then q8 of x, then the predicted ids
// and weights of the next layer.
struct StepWs { size_t layer, qs, d, bs, pids, pw, total; };
static StepWs step_ws(const moe_layer_desc* d, int T) {
  StepWs w{};
  const size_t lw = moe_workspace_size(d, T);
  if (lw == 0) return w;
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  const size_t H = static_cast<size_t>(d->hidden), t = static_cast<size_t>(T);
  w.layer = 0;
  w.qs = up(lw);
  w.d = up(w.qs + t * H);
  // q8 scales, or MXFP8 scale rows (16 ceil(H / 512) bytes each)
  const size_t d_bytes = t * (H / 32) * 4, e_bytes = t * 16 * ((H / 32 + 15) / 16);
  w.bs = up(w.d + (d_bytes > e_bytes ? d_bytes : e_bytes));
  w.pids = up(w.bs + t * (H / 16) * 2 + 16);
  w.pw = up(w.pids + t * d->top_k * 4);
  w.total = up(w.pw + t * d->top_k * 4);
  return w;
}

size_t moe_pool_step_workspace(const moe_layer_desc* desc, int T) {
  if (T < 1) return 0;
  return step_ws(desc, T).total;
}

moe_status moe_pool_layer_step(moe_pool* p, int layer, const moe_layer_desc* desc,
                               const moe_layer_desc* next_desc, const void* x, moe_dtype dtype,
                               int T, int32_t* ids, float* w, float* y, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!p || !desc || layer < 0 || layer >= p->cfg.n_layers || T < 1 || !ws) return MOE_EINVAL;
  if (desc->n_expert != p->cfg.n_experts) return MOE_EINVAL;
  if (next_desc && (layer + 1 >= p->cfg.n_layers || next_desc->n_expert != p->cfg.n_experts ||
                    next_desc->top_k != desc->top_k || next_desc->hidden != desc->hidden))
    return MOE_EINVAL;
  const StepWs sw = step_ws(desc, T);
  if (sw.total == 0) return MOE_EINVAL;
  if (ws_bytes < sw.total) return MOE_ENOWORKSPACE;
  const size_t nk = static_cast<size_t>(T) * desc->top_k;
  if (nk > p->ids_host_n) return MOE_EINVAL;
  const size_t lw = moe_workspace_size(desc, T);
  uint8_t* b = static_cast<uint8_t*>(ws);
  moe_status st = moe_route_topk(desc, x, dtype, T, ids, w, nullptr, b, lw, stream);
  if (st != MOE_OK) return st;
  if (hipMemcpyAsync(p->ids_host, ids, nk * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_EHIP;
  st = moe_pool_resolve(p, layer, p->ids_host, static_cast<int>(nk), stream);
  if (st != MOE_OK) return st;
  if (next_desc) {
    int32_t* pids = reinterpret_cast<int32_t*>(b + sw.pids);
    float* pw = reinterpret_cast<float*>(b + sw.pw);
    const size_t nlw = moe_workspace_size(next_desc, T);
    if (nlw == 0 || nlw > lw) return MOE_EINVAL;  // routing the next layer reuses this scratch
    st = moe_route_topk(next_desc, x, dtype, T, pids, pw, nullptr, b, lw, stream);
    if (st != MOE_OK) return st;
    if (hipMemcpyAsync(p->ids_host, pids, nk * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return MOE_EHIP;
    st = moe_pool_prefetch(p, layer + 1, p->ids_host, static_cast<int>(nk), stream);
    if (st != MOE_OK) return st;
  }
  moe_qact q{};
  q.qs = reinterpret_cast<int8_t*>(b + sw.qs);
  q.d = reinterpret_cast<float*>(b + sw.d);
  q.bsums = reinterpret_cast<int16_t*>(b + sw.bs);
  const bool mx8 = desc->act_quant == MOE_ACTQ_MXFP8;
  const bool q32 = desc->fmt_gate == MOE_WFMT_MXFP4 || desc->fmt_gate == MOE_WFMT_Q4_0 ||
                   desc->fmt_gate == MOE_WFMT_Q5_1;
  const moe_afmt af = mx8 ? MOE_AFMT_MXFP8 : (q32 ? MOE_AFMT_Q8_32 : MOE_AFMT_Q8_K);
  if (mx8) {
    q.scales = reinterpret_cast<uint8_t*>(b + sw.d);  // [T, 16 ceil(H / 512)]
    q.d = nullptr;
    q.bsums = nullptr;
  } else if (af == MOE_AFMT_Q8_32) {
    q.bsums = nullptr;
  }
  st = moe_quantize_act_q8k(x, dtype, T, desc->hidden, af, &q, stream);
  if (st != MOE_OK) return st;
  return moe_expert_ffn(desc, &q, x, dtype, T, ids, w, y, b, lw, stream);
}

moe_status moe_pool_policy_trace(const moe_pool_config* cfg, int n_ops, const int32_t* kind,
                                 const int32_t* layer, const int32_t* off, const int32_t* ids,
                                 int32_t* out, int32_t* n_out, int64_t* stats) {
  if (!config_ok(cfg) || n_ops < 0 || (n_ops > 0 && (!kind || !layer || !off || !n_out)) ||
      !stats)
    return MOE_EINVAL;
  PoolPolicy pol(cfg->n_layers, cfg->n_experts, cfg->n_slots, cfg->n_transient);
  std::vector<PoolPolicy::Place> pl;
  size_t w = 0;
  for (int i = 0; i < n_ops; ++i) {
    const int n = off[i + 1] - off[i];
    if (n < 0 || (n > 0 && !ids) || (kind[i] != 0 && kind[i] != 1)) return MOE_EINVAL;
    const int32_t* v = ids + off[i];
    if (kind[i] == 0) {
      if (!pol.resolve(layer[i], v, n, &pl)) {
        n_out[i] = -1;
        continue;
      }
    } else {
      pol.prefetch(layer[i], v, n, &pl);
    }
    n_out[i] = static_cast<int32_t>(pl.size());
    for (const auto& q : pl) {
      if (out) {
        out[3 * w] = q.key;
        out[3 * w + 1] = q.slot;
        out[3 * w + 2] = q.copy ? 1 : 0;
      }
      ++w;
    }
  }
  const PoolPolicy::Stats& s = pol.stats();
  const int64_t v[10] = {s.epochs,   s.requests,  s.hits_resident, s.hits_transient,
                         s.admitted, s.transient_loads, s.promotions, s.evictions,
                         s.prefetch_loads, s.prefetch_hits};
  memcpy(stats, v, sizeof v);
  return MOE_OK;
}

}  // extern "C"
