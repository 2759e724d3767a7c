// C ABI of librlmoe: host-side validation, scratch layout, launch sequences.
// Nothing here allocates, frees or synchronises; every call only enqueues
// kernels on the caller's stream after all of its checks have passed.
#include <hip/hip_runtime.h>

#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_moe.h"

using namespace rl;

namespace {

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int check_desc(const rl_moe_desc* d) {
  if (!d) return RL_E_INVAL;
  const bool ok_h = d->hidden == 256 || d->hidden == 512 || d->hidden == 1024 || d->hidden == 2048;
  const bool ok_f = pow2(d->width) && d->width >= 32 && d->width <= 2048;
  const bool ok_e = d->n_experts >= 1 && d->n_experts <= 1024;
  const bool ok_k = d->top_k >= 1 && d->top_k <= 32 && d->top_k <= d->n_experts;
  const bool ok_q = d->qbits == 2 || d->qbits == 3;
  if (!(ok_h && ok_f && ok_e && ok_k && ok_q && d->n_layers >= 1 && d->n_slots >= 0))
    return RL_E_SHAPE;
  if (d->flags != 0 && d->flags != RL_STICKY_EARLY_OUT) return RL_E_INVAL;
  return RL_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t a256(int64_t n) { return up256(n); }

// [p, p + bytes) and [q, q + bytes) share a byte (false when either is NULL).
bool overlap(const void* p, const void* q, int64_t bytes) {
  if (!p || !q) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + uintptr_t(bytes) && b < a + uintptr_t(bytes);
}

// --- decode / route scratch: logits [T*E] f32, h [k*F] f32
struct DecodeLayout {
  int64_t logits, hbuf, total;
};
DecodeLayout decode_layout(const rl_moe_desc* d, int T) {
  DecodeLayout l;
  int64_t off = 0;
  l.logits = off;
  off = a256(off + int64_t(T) * d->n_experts * 4);
  l.hbuf = off;
  off = a256(off + int64_t(d->top_k) * d->width * 4);
  l.total = off;
  return l;
}

// --- prefill scratch: logits, the documented plan, internal plan arrays,
// pair intermediates.
struct PrefillLayout {
  rl_prefill_layout pub;
  int64_t logits, counts, offs, bucket_slot, tile_start, tile_bucket, n_tiles, hbuf, ebuf, xq, xe, hq, he,
      total;
};
PrefillLayout prefill_layout(const rl_moe_desc* d, int T) {
  PrefillLayout l;
  const int64_t E = d->n_experts, k = d->top_k, P = int64_t(T) * k;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off = a256(off + bytes);
    return at;
  };
  l.logits = take(int64_t(T) * E * 4);
  l.pub.n_groups = take(4);
  l.pub.group_bounds = take((int64_t(T) + 1) * 4);
  l.pub.n_buckets = take(4);
  l.pub.group_bucket_start = take((int64_t(T) + 1) * 4);
  l.pub.bucket_expert = take(P * 4);
  l.pub.bucket_start = take((P + 1) * 4);
  l.pub.pairs = take(P * 4);
  l.counts = take(int64_t(T) * E * 4);
  l.offs = take(int64_t(T) * E * 4);
  l.bucket_slot = take(P * 4);
  l.tile_start = take((P + 1) * 4);
  l.tile_bucket = take(P * 4);
  l.n_tiles = take(4);
  l.hbuf = take(P * d->width * 4);
  l.ebuf = take(P * d->hidden * 4);
  l.xq = take(int64_t(T) * d->hidden * 4);
  l.xe = take(int64_t(T) * (d->hidden / 256) * 4);
  l.hq = take(P * d->width * 4);
  l.he = take(P * ((d->width + 255) / 256) * 4);
  l.total = off;
  l.pub.total = off;
  return l;
}

int check_route_out(const rl_route_out* o) {
  if (!o || !o->ids || !o->weights || !o->slots || !o->miss_count || !o->early_out)
    return RL_E_INVAL;
  return RL_OK;
}

int check_common(const rl_moe_desc* d, int32_t layer, const float* x, const float* router_w,
                 const int32_t* residency, const rl_route_out* out, const void* scratch) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!x || !router_w || !residency || !scratch) return RL_E_INVAL;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(scratch, 256)) return RL_E_INVAL;
  rc = check_route_out(out);
  if (rc) return rc;
  if (layer < 0 || layer >= d->n_layers) return RL_E_RANGE;
  return RL_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? RL_OK : RL_E_DEVICE; }

RouteArgs route_args(const rl_moe_desc* d, int32_t layer, int32_t T, const float* x,
                     const float* router_w, const float* bias, const int32_t* residency,
                     const rl_route_out* out, float* logits) {
  RouteArgs a;
  a.x = x;
  a.W = router_w;
  a.bias = bias;
  a.T = T;
  a.E = d->n_experts;
  a.H = d->hidden;
  a.k = d->top_k;
  a.layer = layer;
  a.n_slots = d->n_slots;
  a.residency = residency;
  a.logits = logits;
  a.logits_out = out->logits;
  a.ids = out->ids;
  a.weights = out->weights;
  a.slots = out->slots;
  a.miss_count = out->miss_count;
  a.early_out = out->early_out;
  return a;
}

DecodeArgs decode_args(const rl_moe_desc* d, int32_t layer, const float* x, const float* router_w,
                       const float* bias, const int32_t* residency, const void* slot_pool,
                       const rl_route_out* route, uint8_t* s, const DecodeLayout& l, float* y) {
  DecodeArgs da;
  da.pool = make_pool_view(slot_pool, d->hidden, d->width, d->qbits);
  da.H = d->hidden;
  da.F = d->width;
  da.E = d->n_experts;
  da.k = d->top_k;
  da.qbits = d->qbits;
  da.layer = layer;
  da.n_slots = d->n_slots;
  da.x = x;
  da.W = router_w;
  da.bias = bias;
  da.residency = residency;
  da.logits = reinterpret_cast<float*>(s + l.logits);
  da.logits_out = route->logits;
  da.ids = route->ids;
  da.weights = route->weights;
  da.slots = route->slots;
  da.miss_count = route->miss_count;
  da.early_out = route->early_out;
  da.hbuf = reinterpret_cast<float*>(s + l.hbuf);
  da.y = y;
  da.mfma = d->width % 256 == 0;
  da.sticky = (d->flags & RL_STICKY_EARLY_OUT) != 0;
  return da;
}

PrefillArgs prefill_args(const rl_moe_desc* d, int32_t layer, int32_t n_tokens, int32_t plan_cap,
                         const float* x, const int32_t* residency, const void* slot_pool,
                         const rl_route_out* route, uint8_t* s, const PrefillLayout& l,
                         float* y) {
  PrefillArgs a;
  a.pool = make_pool_view(slot_pool, d->hidden, d->width, d->qbits);
  a.T = n_tokens;
  a.H = d->hidden;
  a.F = d->width;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.qbits = d->qbits;
  a.plan_cap = plan_cap;
  a.layer = layer;
  a.x = x;
  a.residency = residency;
  a.ids = route->ids;
  a.slots = route->slots;
  a.weights = route->weights;
  a.early_out = route->early_out;
  auto i32 = [&](int64_t off) { return reinterpret_cast<int32_t*>(s + off); };
  a.plan.n_groups = i32(l.pub.n_groups);
  a.plan.group_bounds = i32(l.pub.group_bounds);
  a.plan.n_buckets = i32(l.pub.n_buckets);
  a.plan.group_bucket_start = i32(l.pub.group_bucket_start);
  a.plan.bucket_expert = i32(l.pub.bucket_expert);
  a.plan.bucket_start = i32(l.pub.bucket_start);
  a.plan.pairs = i32(l.pub.pairs);
  a.plan.counts = i32(l.counts);
  a.plan.offs = i32(l.offs);
  a.plan.bucket_slot = i32(l.bucket_slot);
  a.plan.tile_start = i32(l.tile_start);
  a.plan.tile_bucket = i32(l.tile_bucket);
  a.plan.n_tiles = i32(l.n_tiles);
  a.hbuf = reinterpret_cast<float*>(s + l.hbuf);
  a.ebuf = reinterpret_cast<float*>(s + l.ebuf);
  a.xq = s + l.xq;
  a.xe = i32(l.xe);
  a.hq = s + l.hq;
  a.he = i32(l.he);
  a.mfma = d->width % 256 == 0;
  a.tile_tokens = a.mfma ? 16 : 8;   // tokens per matrix-core pass / VALU tile
  a.y = y;
  a.n_slots = d->n_slots;
  return a;
}

}  // namespace

// The argument checks of moe_decode_layer (everything but the scratch size).
int rl::decode_layer_check(const rl_moe_desc* d, int32_t layer, const float* x,
                           const float* router_w, const int32_t* residency, const void* slot_pool,
                           const rl_route_out* route, const void* scratch, const float* y) {
  const int rc = check_common(d, layer, x, router_w, residency, route, scratch);
  if (rc) return rc;
  if (!slot_pool || !y || !aligned(slot_pool, 256) || !aligned(y, 16)) return RL_E_INVAL;
  return RL_OK;
}

extern "C" {

int64_t rl_tensor_bytes(const rl_moe_desc* d) {
  const int rc = check_desc(d);
  if (rc) return rc;
  return tensor_layout(int64_t(d->hidden) * d->width, d->qbits).total;
}

int64_t rl_slot_bytes(const rl_moe_desc* d) {
  const int64_t t = rl_tensor_bytes(d);
  return t < 0 ? t : 3 * t;
}

int64_t rl_route_scratch_bytes(const rl_moe_desc* d, int32_t n_tokens) {
  const int rc = check_desc(d);
  if (rc) return rc;
  if (n_tokens < 1) return RL_E_RANGE;
  return decode_layout(d, n_tokens).total;
}

int64_t rl_decode_scratch_bytes(const rl_moe_desc* d) {
  const int rc = check_desc(d);
  if (rc) return rc;
  return decode_layout(d, 1).total;
}

int64_t rl_prefill_scratch_bytes(const rl_moe_desc* d, int32_t max_tokens) {
  const int rc = check_desc(d);
  if (rc) return rc;
  if (max_tokens < 1) return RL_E_RANGE;
  return prefill_layout(d, max_tokens).total;
}

int rl_prefill_plan_layout(const rl_moe_desc* d, int32_t max_tokens, rl_prefill_layout* out) {
  const int rc = check_desc(d);
  if (rc) return rc;
  if (!out) return RL_E_INVAL;
  if (max_tokens < 1) return RL_E_RANGE;
  *out = prefill_layout(d, max_tokens).pub;
  return RL_OK;
}

const char* rl_strerror(int code) {
  switch (code) {
    case RL_OK: return "ok";
    case RL_E_INVAL: return "null or misaligned pointer";
    case RL_E_SHAPE: return "unsupported layer shape";
    case RL_E_RANGE: return "layer, token count or plan cap out of range";
    case RL_E_SCRATCH: return "scratch buffer too small";
    case RL_E_DEVICE: return "kernel launch failed";
    case RL_E_STATE: return "decode driver check failed";
    default: return "unknown error";
  }
}

int rl_route(const rl_moe_desc* d, int32_t layer, int32_t n_tokens, const float* x,
             const float* router_w, const float* router_bias, const int32_t* residency,
             const rl_route_out* out, void* scratch, int64_t scratch_bytes, void* stream) {
  int rc = check_common(d, layer, x, router_w, residency, out, scratch);
  if (rc) return rc;
  if (d->flags & RL_STICKY_EARLY_OUT) return RL_E_INVAL;   // decode calls only
  if (n_tokens < 1) return RL_E_RANGE;
  const DecodeLayout l = decode_layout(d, n_tokens);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  uint8_t* s = static_cast<uint8_t*>(scratch);
  const RouteArgs a = route_args(d, layer, n_tokens, x, router_w, router_bias, residency, out,
                                 reinterpret_cast<float*>(s + l.logits));
  launch_route(a, static_cast<hipStream_t>(stream));
  return launch_status();
}

int moe_decode_layer(const rl_moe_desc* d, int32_t layer, const float* x, const float* router_w,
                     const float* router_bias, const int32_t* residency, const void* slot_pool,
                     const rl_route_out* route, void* scratch, int64_t scratch_bytes, float* y,
                     void* stream) {
  const int rc = rl::decode_layer_check(d, layer, x, router_w, residency, slot_pool, route,
                                        scratch, y);
  if (rc) return rc;
  const DecodeLayout l = decode_layout(d, 1);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  uint8_t* s = static_cast<uint8_t*>(scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DecodeArgs da = decode_args(d, layer, x, router_w, router_bias, residency, slot_pool,
                                    route, s, l, y);
  launch_decode_router(da, st);
  launch_decode_gateup(da, st);
  launch_decode_down_sum(da, st);
  return launch_status();
}

int moe_decode_layer_after(const rl_moe_desc* d, int32_t layer, const float* x_prev,
                           const float* y_prev, const uint32_t* flag_prev, float eps,
                           float* x_out, float* a_out, const float* router_w,
                           const float* router_bias, const int32_t* residency,
                           const void* slot_pool, const rl_route_out* route, void* scratch,
                           int64_t scratch_bytes, float* y, void* stream) {
  int rc = check_common(d, layer, x_prev, router_w, residency, route, scratch);
  if (rc) return rc;
  if (!slot_pool || !y || !a_out || !aligned(slot_pool, 256) || !aligned(y, 16) ||
      !aligned(a_out, 16) || (y_prev && !aligned(y_prev, 16)) || (x_out && !aligned(x_out, 16)))
    return RL_E_INVAL;
  // the router's blocks read x_prev and y_prev while block 0 writes x_out and
  // a_out: no byte of an output may lie in another vector
  const int64_t vb = int64_t(d->hidden) * 4;
  if (overlap(x_out, a_out, vb) || overlap(x_out, x_prev, vb) || overlap(x_out, y_prev, vb) ||
      overlap(a_out, x_prev, vb) || overlap(a_out, y_prev, vb))
    return RL_E_INVAL;
  if (!(eps >= 0.f) || !(eps < 3.0e38f)) return RL_E_RANGE;
  const DecodeLayout l = decode_layout(d, 1);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  uint8_t* s = static_cast<uint8_t*>(scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeArgs da = decode_args(d, layer, a_out, router_w, router_bias, residency, slot_pool, route,
                              s, l, y);
  da.x_prev = x_prev;
  da.y_prev = y_prev;
  da.flag_prev = flag_prev;
  da.x_out = x_out;
  da.a_out = a_out;
  da.eps = eps;
  launch_decode_router(da, st);
  launch_decode_gateup(da, st);
  launch_decode_down_sum(da, st);
  return launch_status();
}

int moe_prefill_chunk(const rl_moe_desc* d, int32_t layer, int32_t n_tokens, int32_t plan_cap,
                      const float* x, const float* router_w, const float* router_bias,
                      const int32_t* residency, const void* slot_pool, const rl_route_out* route,
                      void* scratch, int64_t scratch_bytes, float* y, void* stream) {
  int rc = check_common(d, layer, x, router_w, residency, route, scratch);
  if (rc) return rc;
  if (!slot_pool || !y || !aligned(slot_pool, 256) || !aligned(y, 16)) return RL_E_INVAL;
  if (d->flags & RL_STICKY_EARLY_OUT) return RL_E_INVAL;   // decode calls only
  if (n_tokens < 1 || plan_cap < d->top_k) return RL_E_RANGE;
  const PrefillLayout l = prefill_layout(d, n_tokens);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  uint8_t* s = static_cast<uint8_t*>(scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RouteArgs ra = route_args(d, layer, n_tokens, x, router_w, router_bias, residency, route,
                                  reinterpret_cast<float*>(s + l.logits));
  launch_route(ra, st);
  const PrefillArgs a = prefill_args(d, layer, n_tokens, plan_cap, x, residency, slot_pool, route,
                                     s, l, y);
  launch_prefill_plan(a, st);
  launch_prefill_gateup(a, st);
  launch_prefill_down(a, st);
  launch_prefill_sum(a, st);
  return launch_status();
}

int rl_decode_stage(const rl_moe_desc* d, int32_t stage, int32_t layer, const float* x,
                    const float* router_w, const float* router_bias, const int32_t* residency,
                    const void* slot_pool, const rl_route_out* route, void* scratch,
                    int64_t scratch_bytes, float* y, void* stream) {
  int rc = check_common(d, layer, x, router_w, residency, route, scratch);
  if (rc) return rc;
  if (!slot_pool || !aligned(slot_pool, 256)) return RL_E_INVAL;
  if (stage == 2 && (!y || !aligned(y, 16))) return RL_E_INVAL;
  if (stage < 0 || stage > 2) return RL_E_RANGE;
  const DecodeLayout l = decode_layout(d, 1);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  const DecodeArgs da = decode_args(d, layer, x, router_w, router_bias, residency, slot_pool,
                                    route, static_cast<uint8_t*>(scratch), l, y);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (stage == 0)
    launch_decode_router(da, st);
  else if (stage == 1)
    launch_decode_gateup(da, st);
  else
    launch_decode_down_sum(da, st);
  return launch_status();
}

int rl_prefill_stage(const rl_moe_desc* d, int32_t stage, int32_t layer, int32_t n_tokens,
                     int32_t plan_cap, const float* x, const int32_t* residency,
                     const void* slot_pool, const rl_route_out* route, void* scratch,
                     int64_t scratch_bytes, float* y, void* stream) {
  if (d && (d->flags & RL_STICKY_EARLY_OUT)) return RL_E_INVAL;   // decode calls only
  int rc = check_desc(d);
  if (rc) return rc;
  rc = check_route_out(route);
  if (rc) return rc;
  if (!x || !residency || !slot_pool || !scratch || !y) return RL_E_INVAL;
  if (!aligned(x, 16) || !aligned(slot_pool, 256) || !aligned(scratch, 256) || !aligned(y, 16))
    return RL_E_INVAL;
  if (stage < 0 || stage > 3 || layer < 0 || layer >= d->n_layers || n_tokens < 1 ||
      plan_cap < d->top_k)
    return RL_E_RANGE;
  const PrefillLayout l = prefill_layout(d, n_tokens);
  if (scratch_bytes < l.total) return RL_E_SCRATCH;
  const PrefillArgs a = prefill_args(d, layer, n_tokens, plan_cap, x, residency, slot_pool, route,
                                     static_cast<uint8_t*>(scratch), l, y);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (stage) {
    case 0: launch_prefill_plan(a, st); break;
    case 1: launch_prefill_gateup(a, st); break;
    case 2: launch_prefill_down(a, st); break;
    default: launch_prefill_sum(a, st); break;
  }
  return launch_status();
}

int rl_rmsnorm(int32_t n_tokens, int32_t hidden, const float* x, float* out, float eps,
               void* stream) {
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return RL_E_INVAL;
  if (n_tokens < 1 || hidden < 256 || hidden % 256) return RL_E_RANGE;
  launch_rmsnorm(n_tokens, hidden, x, out, eps, static_cast<hipStream_t>(stream));
  return launch_status();
}

int rl_residual_add(int32_t n_tokens, int32_t hidden, float* x, const float* y,
                    const uint32_t* early_out, void* stream) {
  if (!x || !y) return RL_E_INVAL;
  if (n_tokens < 1 || hidden < 256 || hidden % 256) return RL_E_RANGE;
  launch_residual_add(n_tokens, hidden, x, y, early_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

int rl_residual_rmsnorm(int32_t n_tokens, int32_t hidden, const float* x, const float* y,
                        const uint32_t* early_out, float* x_out, float* a_out, float eps,
                        void* stream) {
  if (!x || !y || !x_out || !a_out || !aligned(x, 16) || !aligned(y, 16) || !aligned(x_out, 16) ||
      !aligned(a_out, 16))
    return RL_E_INVAL;
  if (n_tokens < 1 || hidden < 256 || hidden > 2048 || hidden % 256) return RL_E_RANGE;
  launch_residual_rmsnorm(n_tokens, hidden, x, y, early_out, x_out, a_out, eps,
                          static_cast<hipStream_t>(stream));
  return launch_status();
}

int rl_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return RL_E_INVAL;
  if (bytes < 16 || bytes % 16) return RL_E_RANGE;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    return RL_E_DEVICE;
  launch_stream_read(buf, bytes, sink, n_cu, static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"
