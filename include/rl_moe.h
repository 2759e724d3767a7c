/*
 * rl_moe.h -- C ABI of the routed mixture-of-experts FFN for AMD MI355X.
 *
 * One MoE layer of a Qwen3-Next-style decoder: router GEMV, softmax top-k
 * selection, residency lookup with a per-layer early-out flag, block-quantised
 * SwiGLU experts (gate/up, down) and a weighted sum of each token's experts in
 * router rank order.  Two forms: single-token decode and chunked prefill over
 * (expert, token) pairs sorted by expert.
 *
 * Sources (the Red Lite development notes):
 *   dev21  "Red Lite dev21 - GPU-routed decode (full residency)", "What changed":
 *          selection rule, renormalised weights, residency table, slot table,
 *          per-layer miss count.
 *   dev23  "Red Lite dev23 - per-layer early-out and pre-gated expert prefetch",
 *          "What changed": every kernel of the layer returns at once when the
 *          early-out flag is set.
 *   dev20  "Red Lite dev20 - batched prompt ingestion", "What changed": chunks,
 *          plans of at most 512 distinct experts split into consecutive token
 *          groups past the cap, pairs sorted by expert, per-token sum in router
 *          selection order.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *     and owns every buffer and keeps it alive until the work queued on
 *     `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call of the
 *     layer API only enqueues work on it: no allocation, no free, no
 *     synchronisation.  The exceptions are the host objects at the end: the
 *     expert cache (rl_cache_*, host memory only, no stream) and the decode
 *     driver (rl_driver_*, which allocates at creation and waits for its
 *     stream at the end of each token).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative return code means nothing was enqueued.  RL_E_DEVICE means a
 *     launch failed (hipGetLastError) and the queued state is unspecified.
 *   - The early-out flag is data, not an error.
 *   - Calls on different streams must not share outputs or scratch.
 *   - NaN or infinite inputs give unspecified (but in-bounds) results.
 *
 * Block format of an expert tensor (the workload's 2- and 3-bit format).
 *   The R x C elements, row-major and flattened, form blocks of 256 values;
 *   group g = 0..7 of a block holds 32 consecutive values.  Weight =
 *   d * (2s+1)/16 * level(c): level = c - 1.5 (2-bit code c), or (c - 3.5)/2
 *   (3-bit code).  Byte planes, each at a 256-byte aligned offset, in order:
 *     Q   nb*64 B  low code bits: element j of block b at byte 64b + j/4,
 *                  bits 2(j%4), 2(j%4)+1
 *     Hb  nb*32 B  (3-bit only) code bit 2: byte 32b + j/8, bit j%8
 *     S   nb*4  B  group scale s of group g: byte 4b + g/2, low nibble if g even
 *     D   nb*2  B  block scale d, IEEE binary16 little endian, at byte 2b
 *   and the tensor size is rounded up to 256 bytes (rl_tensor_bytes).
 *   An expert slot is gate [F x H], up [F x H], down [H x F] back to back;
 *   slot s of the pool starts at byte s * rl_slot_bytes().
 */
#ifndef RL_MOE_H
#define RL_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one MoE layer (host struct).
 * Supported: hidden in {256, 512, 1024, 2048}; width a power of two in
 * [32, 2048]; 1 <= top_k <= min(n_experts, 32); 1 <= n_experts <= 1024;
 * n_layers >= 1; qbits in {2, 3}; n_slots >= 0 (slots in the pool);
 * flags 0 or RL_STICKY_EARLY_OUT.
 *
 * RL_STICKY_EARLY_OUT (decode calls only: moe_decode_layer, rl_decode_stage;
 * rl_route, moe_prefill_chunk and rl_prefill_stage return RL_E_INVAL): the
 * notes' single early-out flag shared by every kernel of a token ("Red Lite
 * dev23 - per-layer early-out", "What changed": every decode kernel takes
 * the flag and returns at once when it is set).  A call whose *early_out is
 * already nonzero does nothing at all (no output, miss_count left as it
 * was); a call that misses sets *early_out = 1; nothing ever clears it, so
 * the caller zeroes it before a token (or a resumed part of one).  Without
 * the flag bit, each call overwrites *early_out with its own miss state. */
typedef struct rl_moe_desc {
  int32_t hidden;     /* H */
  int32_t n_experts;  /* E */
  int32_t top_k;      /* k */
  int32_t width;      /* F, expert intermediate width */
  int32_t n_layers;   /* rows of the residency table */
  int32_t qbits;      /* 2 or 3 */
  int32_t n_slots;    /* slots in slot_pool; table entries >= n_slots miss */
  int32_t flags;      /* 0 or RL_STICKY_EARLY_OUT */
} rl_moe_desc;

enum { RL_STICKY_EARLY_OUT = 1 };

enum {
  RL_OK = 0,
  RL_E_INVAL = -1,    /* null required pointer or misaligned buffer */
  RL_E_SHAPE = -2,    /* unsupported layer shape in the descriptor */
  RL_E_RANGE = -3,    /* layer, n_tokens or plan_cap out of range */
  RL_E_SCRATCH = -4,  /* scratch smaller than the size query returns */
  RL_E_DEVICE = -5,   /* a kernel launch failed */
  RL_E_STATE = -6     /* a decode driver's token failed an internal check */
};

/* Routing results of one call (host struct of device pointers).
 * The notes' rl_route writes the slot table and weights the expert kernels
 * read and a per-layer miss count (dev21, "What changed"). */
typedef struct rl_route_out {
  int32_t*  ids;        /* [T][k] expert ids in router rank order           */
  float*    weights;    /* [T][k] softmax weights renormalised over the k   */
  int32_t*  slots;      /* [T][k] residency[layer][id], -1 = not resident   */
  uint32_t* miss_count; /* [1] selections with slot -1, over the T tokens  */
  uint32_t* early_out;  /* [1] 1 when miss_count > 0, else 0 (overwritten;  */
                        /* raised only, with RL_STICKY_EARLY_OUT)          */
  float*    logits;     /* [T][E] router logits, or NULL = not stored       */
} rl_route_out;

/* Bytes of one expert tensor (F x H elements) and of one slot (3 tensors). */
int64_t rl_tensor_bytes(const rl_moe_desc* d);
int64_t rl_slot_bytes(const rl_moe_desc* d);

/* Scratch sizes in bytes (negative = error code for a bad descriptor).
 * Scratch must be 256-byte aligned; its contents need no initialisation and
 * are overwritten by every call (except where a stage entry point below
 * reads what an earlier stage left there). */
int64_t rl_route_scratch_bytes(const rl_moe_desc* d, int32_t n_tokens);
int64_t rl_decode_scratch_bytes(const rl_moe_desc* d);
int64_t rl_prefill_scratch_bytes(const rl_moe_desc* d, int32_t max_tokens);

/* Where moe_prefill_chunk keeps its plan inside scratch (byte offsets from
 * the scratch base), so that callers and tests can read it after the call.
 * The offsets depend on the call's token count: pass the n_tokens of the
 * moe_prefill_chunk call as max_tokens here.
 * All arrays are int32; they are written only when early_out is 0.
 *   n_groups            [1]
 *   group_bounds        [n_groups+1] token boundaries of the token groups
 *   n_buckets           [1]   distinct (group, expert) buckets
 *   group_bucket_start  [n_groups+1] first bucket of each group
 *   bucket_expert       [n_buckets]  expert id of each bucket (ascending
 *                                    inside a group)
 *   bucket_start        [n_buckets+1] offsets into pairs
 *   pairs               [T*k] pair ids p = t*k + r, per group sorted by
 *                                    expert, then by p (stable) */
typedef struct rl_prefill_layout {
  int64_t n_groups, group_bounds, n_buckets, group_bucket_start,
          bucket_expert, bucket_start, pairs, total;
} rl_prefill_layout;
int rl_prefill_plan_layout(const rl_moe_desc* d, int32_t max_tokens,
                           rl_prefill_layout* out /* (host) */);

const char* rl_strerror(int code);

/* Router, softmax top-k, renormalised weights and residency lookup for
 * n_tokens tokens of layer `layer` (dev21 "What changed"; dev23 "What
 * changed" for the flag).
 *   x          [T][H] float32 activations
 *   router_w   [E][H] float32
 *   router_bias[E] float32 or NULL
 *   residency  [L][E] int32 slot indices; -1 = not resident.  Entries outside
 *              [-1, n_slots) are treated as not resident.
 *   out        (host) struct of device pointers; ids, weights, slots,
 *              miss_count, early_out required, logits optional.
 * Logits accumulate in float64 and round once to float32; experts are taken
 * by logit, largest first, ties to the lower index (-0 == +0); weights are
 * exp(l_r - l_0) / sum_j exp(l_j - l_0) over the k taken, summed in rank
 * order.  The flag is overwritten on every call. */
int rl_route(const rl_moe_desc* d, int32_t layer, int32_t n_tokens,
             const float* x, const float* router_w, const float* router_bias,
             const int32_t* residency, const rl_route_out* out,
             void* scratch, int64_t scratch_bytes, void* stream);

/* One single-token decode step of layer `layer`: rl_route for the token, then
 * the k experts' gate/up GEMVs with SwiGLU, the down GEMVs, and
 *   y = sum_{r=0..k-1} w_r * (W_down[slot_r] h_r)
 * accumulated in rank order (fused multiply-add from 0).  When the router
 * raises the flag every expert kernel returns at once and y is NOT written
 * (dev23 "What changed").
 *   x [H] float32; slot_pool: n_slots slots of rl_slot_bytes bytes;
 *   route: where the routing results go (as for rl_route);
 *   scratch: rl_decode_scratch_bytes bytes; y [H] float32. */
int moe_decode_layer(const rl_moe_desc* d, int32_t layer, const float* x,
                     const float* router_w, const float* router_bias,
                     const int32_t* residency, const void* slot_pool,
                     const rl_route_out* route, void* scratch,
                     int64_t scratch_bytes, float* y, void* stream);

/* moe_decode_layer preceded by the step between two layers of a stack (a
 * pre-norm decoder: each layer's input is the RMSNorm of the residual
 * stream, and the layer's output is added to the stream), with that step
 * done inside the layer's first kernel instead of a launch of its own:
 *   r = x_prev + y_prev, or x_prev when y_prev is NULL or *flag_prev is set
 *       (the previous layer stopped: its y is not valid), in float32;
 *   a = r / sqrt(mean(r^2) + eps), mean of squares in float64;
 *   then moe_decode_layer(d, layer, a, ...).
 * x_prev, y_prev [H] float32 (y_prev may be NULL); flag_prev: the previous
 * layer's early-out word (may be NULL: never set); x_out [H] receives r (NULL:
 * not written); a_out [H] receives a (required).  The results are bit-identical
 * to rl_residual_rmsnorm (or rl_rmsnorm when y_prev is NULL) followed by
 * moe_decode_layer on a_out.  The hidden floats of x_out and of a_out must
 * not share a byte with each other, x_prev or y_prev (RL_E_INVAL; nothing is
 * enqueued); eps must be finite and >= 0 (RL_E_RANGE).
 * With RL_STICKY_EARLY_OUT and the shared flag set, r and a are still
 * written and the layer does nothing else. */
int moe_decode_layer_after(const rl_moe_desc* d, int32_t layer, const float* x_prev,
                           const float* y_prev, const uint32_t* flag_prev, float eps,
                           float* x_out, float* a_out, const float* router_w,
                           const float* router_bias, const int32_t* residency,
                           const void* slot_pool, const rl_route_out* route, void* scratch,
                           int64_t scratch_bytes, float* y, void* stream);

/* moe_decode_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call and results without the scratch arguments.  The
 * scratch lives in a fixed device array of RL_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per GPU, held until the process ends; the call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Layers whose rl_decode_scratch_bytes exceeds that size return
 * RL_E_SCRATCH with nothing enqueued (the hidden-2048, 512-expert, top-10,
 * width-512 layer needs 22,528 bytes).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap in time on one GPU -- on different
 * streams, or from several host threads -- race and give undefined results;
 * serialise them (one stream, or events).  The first call on a device looks
 * up the array's address on it (RL_E_DEVICE if that fails); the other errors
 * are those of moe_decode_layer and come before any device call. */
#define RL_NOALLOC_SCRATCH_BYTES 65536
int moe_decode_layer_noalloc(const rl_moe_desc* d, int32_t layer, const float* x,
                             const float* router_w, const float* router_bias,
                             const int32_t* residency, const void* slot_pool,
                             const rl_route_out* route, float* y, void* stream);

/* One prefill chunk of n_tokens tokens through layer `layer` (dev20 "What
 * changed"): route every token, build the chunk's plan -- consecutive token
 * groups whose union of selected experts stays within plan_cap (a token
 * joins the current group unless the union would exceed the cap), and per
 * group the (expert, token) pairs sorted by expert -- run the batched
 * gate/up and down projections over the pairs and sum each token's k expert
 * outputs in rank order.  One miss anywhere in the chunk raises the chunk's
 * flag; then nothing after routing runs and y is NOT written.
 *   x [T][H]; y [T][H] float32; plan_cap >= top_k;
 *   scratch: rl_prefill_scratch_bytes(d, max_tokens) with max_tokens >= T. */
int moe_prefill_chunk(const rl_moe_desc* d, int32_t layer, int32_t n_tokens,
                      int32_t plan_cap, const float* x, const float* router_w,
                      const float* router_bias, const int32_t* residency,
                      const void* slot_pool, const rl_route_out* route,
                      void* scratch, int64_t scratch_bytes, float* y,
                      void* stream);

/* Stage entry points, for tests and benchmarks: each enqueues the kernels of
 * one step of a path above, with the same arguments and scratch layout.
 *   rl_decode_stage: stage 0 = router GEMV into scratch; stage 1 = softmax
 *     top-k, lookup and flag (written to `route`) then the gate/up GEMVs +
 *     SwiGLU of the k selected experts into scratch; stage 2 = down GEMVs +
 *     rank-ordered sum into y.  Each stage needs the previous ones in the same
 *     scratch.  Same early-out behaviour as moe_decode_layer.
 *   rl_prefill_stage: stage 0 = plan (needs `route` filled by rl_route for
 *     the n_tokens tokens of x), 1 = batched gate/up, 2 = batched down,
 *     3 = per-token ordered sum into y; each stage needs the previous ones in
 *     the same scratch (sized for n_tokens).
 * Sources as for moe_decode_layer (dev21, dev23) and moe_prefill_chunk (dev20). */
int rl_decode_stage(const rl_moe_desc* d, int32_t stage, int32_t layer,
                    const float* x, const float* router_w,
                    const float* router_bias, const int32_t* residency,
                    const void* slot_pool, const rl_route_out* route,
                    void* scratch, int64_t scratch_bytes, float* y, void* stream);
int rl_prefill_stage(const rl_moe_desc* d, int32_t stage, int32_t layer,
                     int32_t n_tokens, int32_t plan_cap, const float* x,
                     const int32_t* residency, const void* slot_pool,
                     const rl_route_out* route, void* scratch,
                     int64_t scratch_bytes, float* y, void* stream);

/* Helpers for stacks of layers (not part of the MoE layer itself).
 * rl_rmsnorm: out[t] = x[t] / sqrt(mean(x[t]^2) + eps), no weight.
 * rl_residual_add: x[t] += y[t], skipped entirely when *early_out != 0
 * (early_out may be NULL = always add).  hidden must be a multiple of 256;
 * the norms take x, out (and y, x_out, a_out below) 16-byte aligned (else
 * RL_E_INVAL) and accumulate the mean of squares in float64 in a fixed order,
 * the same in rl_rmsnorm, rl_residual_rmsnorm and moe_decode_layer_after. */
int rl_rmsnorm(int32_t n_tokens, int32_t hidden, const float* x, float* out,
               float eps, void* stream);
int rl_residual_add(int32_t n_tokens, int32_t hidden, float* x, const float* y,
                    const uint32_t* early_out, void* stream);
/* rl_residual_rmsnorm: the step between two layers in one launch:
 * x_out[t] = x[t] + y[t] (x_out[t] = x[t] when *early_out != 0; early_out
 * may be NULL = always add), then a_out[t] = rl_rmsnorm of x_out[t].  x_out
 * must not overlap x or y.  hidden: a multiple of 256, at most 2048. */
int rl_residual_rmsnorm(int32_t n_tokens, int32_t hidden, const float* x, const float* y,
                        const uint32_t* early_out, float* x_out, float* a_out, float eps,
                        void* stream);

/* ---------------------------------------------------------------------------
 * Expert cache (host memory and host code only; no device calls).
 * A bounded pool of n_slots expert slots serves n_layers x n_experts keys.
 * The cache decides which slot a missing expert is loaded into and which
 * resident expert that evicts; the caller copies the expert's bytes into the
 * slot and mirrors the cache's table into the device residency table
 * ("Red Lite dev21 - GPU-routed decode", "What changed": the residency table
 * is maintained on every LRU commit and abort, and a reservation reports the
 * key a miss evicts).  Least recently used replacement; all hits of a
 * selection are reserved before any victim is chosen, so a selection never
 * evicts one of its own experts ("Red Lite dev20 - batched prompt
 * ingestion", the LRU fix).  Every load into a slot bumps that slot's load
 * generation ("Red Lite dev23", "What changed", per-slot load generations):
 * a caller that recorded generations when it planned work on some slots can
 * tell whether any of them was reloaded since.  One reservation may be open
 * at a time; the cache is not thread-safe.  Keys are layer * n_experts +
 * expert.
 *
 * rl_cache_create: NULL if a count is < 1, n_layers * n_experts > 2^30 or
 *   memory runs out.  All slots start free (used before any eviction).
 * rl_cache_insert: make (layer, expert) resident in a free slot (for seeding
 *   from an initial residency table); RL_E_INVAL if the key is resident, the
 *   slot is taken or a reservation is open; RL_E_RANGE for bad indices.
 * rl_cache_lookup: the key's slot, or -1.
 * rl_cache_reserve: the k ids (host array) of one layer's selection; writes
 *   per id its slot, load[i] = 1 if the caller must copy the expert into that
 *   slot, evicted[i] = the key the load displaces (-1: the slot was free or
 *   no load), and (if gens != NULL) the slot's load generation.  Returns the
 *   number of loads (>= 0), RL_E_RANGE (bad layer/id, k < 1, or more misses
 *   than slots outside the selection: the cache is then unchanged) or
 *   RL_E_INVAL (NULL pointer, or a reservation already open).
 * rl_cache_reserve_excluding: rl_cache_reserve that takes no victim from a
 *   slot holding an expert of exclude_layer (-1: none excluded), for loads
 *   queued while that layer may still be running: its kernels read only its
 *   own experts' slots.  Returns RL_E_RANGE (cache unchanged, counted as an
 *   abort) when too few slots qualify (decided before anything changes).
 * rl_cache_touch: the resident ones of a layer's k ids become the most
 *   recently used (the first id most recent), as after the device used them
 *   without any load; returns how many were resident, RL_E_RANGE for a bad
 *   layer or id (ids before it may have been touched), RL_E_INVAL while a
 *   reservation is open.
 * rl_cache_commit: the reservation's slots become the most recently used
 *   (the first id most recent) and the reservation closes.
 * rl_cache_abort: keys return to the slots they held before the reservation
 *   (load generations stay bumped) and the reservation closes.
 * rl_cache_generation: load generation of a slot (0 for a bad slot).
 * rl_cache_table: writes the [n_layers x n_experts] int32 table of slots
 *   (-1 = not resident) into a host array, for the device residency table.
 * rl_cache_stats: out[5] = reservations, hits, misses (= loads), evictions,
 *   aborted reservations. */
typedef struct rl_cache rl_cache;
rl_cache* rl_cache_create(int32_t n_slots, int32_t n_layers, int32_t n_experts);
void rl_cache_destroy(rl_cache* c);
int rl_cache_insert(rl_cache* c, int32_t layer, int32_t expert, int32_t slot);
int32_t rl_cache_lookup(const rl_cache* c, int32_t layer, int32_t expert);
int rl_cache_reserve(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k, int32_t* slots,
                     int32_t* load, int32_t* evicted, uint32_t* gens);
int rl_cache_reserve_excluding(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k,
                               int32_t exclude_layer, int32_t* slots, int32_t* load,
                               int32_t* evicted, uint32_t* gens);
int rl_cache_touch(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k);
int rl_cache_commit(rl_cache* c);
int rl_cache_abort(rl_cache* c);
uint32_t rl_cache_generation(const rl_cache* c, int32_t slot);
int rl_cache_table(const rl_cache* c, int32_t* table);
int rl_cache_stats(const rl_cache* c, int64_t* out);

/* ---------------------------------------------------------------------------
 * Decode driver: single tokens through all n_layers layers of a model whose
 * slot pool holds only part of its experts, with miss service and resume
 * ("Red Lite dev23 - per-layer early-out and pre-gated expert prefetch",
 * "What changed": the first layer f that selects a non-resident expert
 * stops the token there; f's missing experts are loaded, f runs again and
 * the token resumes at f + 1; a token with more than a few early-outs sends
 * the next tokens to a layer-by-layer path, a token without loads sends them
 * back; optionally the next layer's router on the current layer's input
 * predicts its selection and the predicted experts are loaded ahead of it).
 * Host code driving the library's own calls: per layer moe_decode_layer on
 * a_l = rmsnorm(x_l), then rl_residual_rmsnorm (x_{l+1} = x_l + y_l, or x_l
 * when the layer's flag is set), replayed as HIP graphs captured at creation.
 * A layer's misses are copied from the host store into the slots the cache
 * picks by one gather launch that reads the store through its device
 * address and also writes the changed residency entries (one hipMemcpyAsync
 * per expert plus an entry copy when the store has no device address);
 * after a token every layer's selection is touched in the cache ("Red Lite
 * dev21", "What changed", LRU stamps refreshed after the token).  With
 * prefetch, layer l's graph also runs layer l+2's router on layer l+1's
 * input (in the step between the layers), the host takes the top k of those
 * logits, reserves the experts (no victim among layer l+1's slots), and
 * their gather is queued right behind layer l+1's graph, so the copies run
 * while the host reads layer l+1's flags and relaunches.
 *
 * rl_driver_config (host struct; the pointers stay owned by the caller and
 * must outlive the driver):
 *   desc             layer shape, n_layers >= 1, top_k <= 32; flags may hold
 *                    RL_STICKY_EARLY_OUT (one shared flag word per token)
 *   router_w         [n_layers] device pointers, each [E x H] float32
 *   router_bias      [n_layers] device pointers ([E] float32) or NULL entries;
 *                    NULL = no bias anywhere
 *   residency        device [n_layers x E] int32; overwritten at creation with
 *                    the cache's table and kept equal to it afterwards
 *   slot_pool        device pool of desc->n_slots slots (rl_slot_bytes each)
 *   host_store       pinned host memory (hipHostMalloc or equivalent) holding
 *                    every expert: row layer * E + expert, rl_slot_bytes each
 *   cache            an rl_cache over the same slots, seeded with the pool's
 *                    resident experts; the driver reserves, commits and
 *                    touches it and no one else may use it meanwhile
 *   x                device [(n_layers + 1) x H] float32: after a token, x[l]
 *                    is layer l's input and x[n_layers] the output
 *   early_out_limit  >= 0: a token with more early-outs than this sends the
 *                    next tokens to the layer-by-layer path
 *   prefetch         nonzero: predict and load the next layer's experts on
 *                    the layer-by-layer path (needs a host_store with a
 *                    device address: rl_driver_create returns NULL otherwise)
 *   eps              RMSNorm epsilon
 * rl_driver_create: allocates its device and pinned buffers, captures its
 *   graphs on `stream` (a hipStream_t) and runs one layer eagerly; NULL on a
 *   bad argument or a failed allocation, capture or launch.  All later
 *   calls use the same stream.
 * rl_driver_token: x0 device [H] float32; runs the token and returns after
 *   the stream has drained.  RL_E_RANGE if the cache cannot hold one layer's
 *   selection, RL_E_DEVICE on a failed launch or copy, RL_E_STATE if a
 *   serviced layer still missed or one of its slots was reloaded meanwhile.
 *   After any error the driver refuses further tokens (RL_E_STATE).
 * rl_driver_stats: out[8] = tokens, early-outs, loads on the critical path,
 *   tokens on the layer-by-layer path, evictions, predictions, predicted
 *   experts that the layer then selected, prefetched loads.
 * rl_driver_destroy: waits for the stream and frees the driver. */
typedef struct rl_driver_config {
  const rl_moe_desc* desc;
  const float* const* router_w;
  const float* const* router_bias;
  int32_t* residency;
  void* slot_pool;
  const void* host_store;
  rl_cache* cache;
  float* x;
  int32_t early_out_limit;
  int32_t prefetch;
  float eps;
} rl_driver_config;

typedef struct rl_decode_driver rl_decode_driver;
rl_decode_driver* rl_driver_create(const rl_driver_config* config, void* stream);
int rl_driver_token(rl_decode_driver* driver, const float* x0);
int rl_driver_stats(const rl_decode_driver* driver, int64_t* out);
void rl_driver_destroy(rl_decode_driver* driver);

/* Measurement helper (not part of the MoE layer): reads `bytes` bytes of the
 * device buffer `buf` once, in 16-byte words, with a grid of eight blocks
 * per compute unit, so that the time of the launch gives the HBM read rate
 * this device reaches with plain streaming loads.  `sink` is a device word
 * that is written only in the (practically never taken) case that the
 * folded data equal a fixed constant.  bytes must be a positive multiple of
 * 16 (RL_E_RANGE); NULL pointers give RL_E_INVAL. */
int rl_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RL_MOE_H */
