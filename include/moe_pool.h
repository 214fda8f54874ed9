/*
 * moe_pool — an expert pool larger than the device memory it is given: every
 * expert of every layer lives in a pinned host tier, a fixed arena of device
 * slots holds a hot set (touch-count admission) plus transient slots, and
 * each layer step resolves its routed experts into slots before the expert
 * kernels run. Sources: Pulsar README, MoE expert-resolve list (VRAM hot-set
 * cache with touch-count admission; host tier; next-layer prefetch by running
 * the next layer's router on the current layer's input; the MoE kernels get
 * explicit per-expert device pointers resolved before launch) and the
 * article on running Kimi K3 on one DGX Spark (experts streamed from a tier
 * below device memory).
 *
 * Usage per layer step (one host thread per pool; one compute stream):
 *   moe_route_topk(...)                -> ids on the device, copied to the host
 *   moe_pool_resolve(pool, l, ids, n, stream)
 *   moe_expert_ffn(desc with moe_pool_layer_tables(pool, l, ...), ...)
 *   optionally moe_pool_prefetch(pool, l + 1, predicted ids, n, stream)
 * The pool orders the stream's later work after its copies, and its copies
 * after the stream's earlier work, with events (default-priority streams).
 */
#ifndef MOE_POOL_H
#define MOE_POOL_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_pool moe_pool;

/* n_layers x n_experts experts of slab_bytes each (one expert's gate, up and
 * down matrices, laid out by the caller; up and down start at up_offset and
 * down_offset, multiples of 16). n_slots device slots, of which n_transient
 * are kept for requested experts that are not admitted to the hot set
 * (n_transient >= the unique experts of any one resolve call, >= 1). */
typedef struct {
  int32_t n_layers;
  int32_t n_experts;
  size_t slab_bytes;
  size_t up_offset;
  size_t down_offset;
  int32_t n_slots;
  int32_t n_transient;
} moe_pool_config;

typedef struct {
  int64_t epochs, requests, hits_resident, hits_transient, admitted, transient_loads,
      promotions, evictions, prefetch_loads, prefetch_hits, bytes_h2d;
} moe_pool_stats;

/* Allocates the pinned host tier (n_layers * n_experts slabs), the device
 * arena (n_slots slabs), per-layer device pointer tables and a copy stream on
 * the current device. Errors: MOE_EINVAL (bad config), MOE_EHIP (allocation). */
MOE_API moe_status moe_pool_create(const moe_pool_config* cfg, moe_pool** out);
/* Waits for the pool's copies, then frees everything it allocated. */
MOE_API void moe_pool_destroy(moe_pool* pool);
/* Host (pinned) slab of one expert, for the caller to fill before use; NULL
 * for an index out of range. Bytes are read by later copies only. */
MOE_API uint8_t* moe_pool_host_slab(moe_pool* pool, int layer, int expert);
/* Device arrays of n_experts pointers (gate, up, down) for a layer's
 * moe_layer_desc. After a resolve for that layer they point to the slots of
 * its requested experts and are NULL for every other expert ("not present"). */
MOE_API moe_status moe_pool_layer_tables(moe_pool* pool, int layer, const void* const** gate,
                                         const void* const** up, const void* const** down);
/* Resolves n host-side expert ids of a layer (duplicates and ids outside
 * [0, n_experts) ignored) into device slots: hits keep their slot, misses are
 * copied from the host tier (admitted to the hot set or loaded as transient),
 * and the layer's tables are rewritten on `stream`; work enqueued on `stream`
 * afterwards sees every copied expert. Errors: MOE_EINVAL, MOE_ENOWORKSPACE
 * (more unique experts than slots not in use this step; nothing changed),
 * MOE_EHIP. */
MOE_API moe_status moe_pool_resolve(moe_pool* pool, int layer, const int32_t* ids, int n,
                                    hipStream_t stream);
/* Starts copies of predicted experts of a layer that would be admitted (or fit
 * a free or reusable transient slot) without waiting for them; the next
 * resolve of that layer finds them as hits. Touch counts are not changed. */
MOE_API moe_status moe_pool_prefetch(moe_pool* pool, int layer, const int32_t* ids, int n,
                                     hipStream_t stream);
MOE_API moe_status moe_pool_get_stats(const moe_pool* pool, moe_pool_stats* out);

/* One layer step of a pool-backed stack, natively: routes x [T, H] with
 * `desc` into ids / w (device [T, k]), copies the ids to the host, resolves
 * them into `layer`'s tables; if next_desc is not NULL, routes x with the next
 * layer's router and prefetches the predicted experts into layer + 1 (the
 * next layer's input is not known yet: its router on this input is the
 * prediction, as in the Pulsar README's resolve list); then quantizes x and
 * runs the expert FFN into y [T, H]. desc's gate/up/down must be this pool's
 * tables of `layer` (next_desc's those of layer + 1). ws: device scratch of
 * moe_pool_step_workspace(desc, T) bytes, 256-byte aligned. The call waits for
 * the routing (host round trip) and returns with the FFN enqueued on stream.
 * Errors: those of the calls it makes. */
MOE_API moe_status moe_pool_layer_step(moe_pool* pool, int layer, const moe_layer_desc* desc,
                                       const moe_layer_desc* next_desc, const void* x,
                                       moe_dtype dtype, int T, int32_t* ids, float* w, float* y,
                                       void* ws, size_t ws_bytes, hipStream_t stream);
/* Workspace of moe_pool_layer_step (0 for an invalid descriptor or T). */
MOE_API size_t moe_pool_step_workspace(const moe_layer_desc* desc, int T);

/* Test export (host only, no device work): the slot policy of a pool with
 * this config run over n_ops operations. Operation i is a resolve (kind[i] =
 * 0) or a prefetch (kind[i] = 1) of layer[i] with ids[off[i] .. off[i + 1]).
 * Placements (key = layer * n_experts + expert, slot, copy flag) are written
 * as int32 triples to `out` in order, n_out[i] = the op's count (-1 for a
 * resolve that found no slot); stats (10 counters, moe_pool_stats order
 * without bytes_h2d) after the last op. Errors: MOE_EINVAL. */
MOE_API moe_status moe_pool_policy_trace(const moe_pool_config* cfg, int n_ops,
                                         const int32_t* kind, const int32_t* layer,
                                         const int32_t* off, const int32_t* ids, int32_t* out,
                                         int32_t* n_out, int64_t* stats);

#ifdef __cplusplus
}
#endif
#endif
