// Host-side decode driver: one token at a time through L MoE layers whose
// expert pool holds only part of the experts (host code; the kernels are the
// library's own decode, route and norm launches, replayed as HIP graphs).
//
// Per token ("Red Lite dev23 - per-layer early-out and pre-gated expert
// prefetch", "What changed"):
//  - a layer whose selection names a non-resident expert raises its flag and
//    every later kernel of that layer returns at once; the layers before the
//    first flagged layer f are complete;
//  - the host loads f's missing experts into slots the expert cache picks
//    (least recently used, hits reserved first: "Red Lite dev20", LRU fix),
//    mirrors the cache's table into the device residency table, runs layer f
//    again and resumes at f + 1;
//  - policy: on the early-out path the rest of the token is one graph
//    launch and the flags are read afterwards; a token with more than
//    `early_out_limit` early-outs sends the following tokens to the
//    synchronous path (one launch and one wait per layer, a miss serviced as
//    soon as its layer shows it), and a token that needed no load sends them
//    back;
//  - pre-gated prefetch (synchronous path, optional): layer m's router on
//    layer m-1's input predicts m's selection.  Layer l's graph ends with
//    a_{l+1}, so it also runs layer l+2's router on it and copies the
//    prediction out with the flags: after the one wait per layer the host
//    reserves the predicted experts with no victim among layer l+1's slots
//    (rl_cache_reserve_excluding: a layer reads only its own experts' slots)
//    and keeps their loads (store rows, slots, table entries).  Right after
//    layer l+1's graph, behind the event the host waits on, one gather launch
//    copies them from the store (through its device address): the copies
//    run while the host wakes, reads the flags and launches the next graph,
//    time in which the device would otherwise be idle, and the stream orders
//    them before layer l+2 and before any miss service.  Layer 1's
//    prediction is made from a_0 before layer 0;
//  - after the token every layer's selection becomes the most recently used
//    ("Red Lite dev21 - GPU-routed decode", "What changed": LRU stamps
//    refreshed after the token).
// The layers after an early-out run on an unfinished input; their results are
// overwritten when the token resumes, so every layer's output equals that of a
// fully resident stack.
//
// Graphs (captured once at creation): suffix[l] = layers l .. L-1, single[l]
// = layer l; with prefetch, single_pf[l] = layer l then the prediction for
// l+2 (l+2 < L) and first_pf = the prediction for layer 1 alone.  Each ends
// by copying the flags, miss counts, selected ids and predicted ids into
// pinned host mirrors, so one wait after a launch gives the host all it reads.
// A layer = moe_decode_layer(a_l) -> y_l, then rl_residual_rmsnorm(x_l, y_l,
// flag) -> x_{l+1}, a_{l+1}; the token starts with x_0 = x0, a_0 = rmsnorm(x0).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "rl_kernels.h"
#include "rl_moe.h"

struct rl_decode_driver {
  rl_moe_desc d;          // as given (flags may hold RL_STICKY_EARLY_OUT)
  int L = 0, E = 0, H = 0, k = 0;
  bool sticky = false, prefetch = false, sync_path = false;
  int limit = 0;
  float eps = 0.f;
  hipStream_t st = nullptr;
  hipEvent_t ev_done = nullptr;
  std::vector<const float*> W, bias;
  int32_t* residency = nullptr;
  uint8_t* pool = nullptr;
  const uint8_t* store = nullptr;
  const void* store_dev = nullptr;    // the store's device address (gather launches), or NULL
  int64_t slot_bytes = 0;
  rl_cache* cache = nullptr;
  float* x = nullptr;     // caller's [(L+1) x H]
  // device buffers (one allocation)
  void* dev = nullptr;
  float *a = nullptr, *y = nullptr;
  int32_t *ids = nullptr, *slots = nullptr;
  float *wts = nullptr, *plogits = nullptr;   // plogits: the prediction's router logits [E]
  uint32_t *miss = nullptr, *flags = nullptr, *pflag = nullptr;
  uint8_t* scratch = nullptr;
  int64_t scratch_bytes = 0;
  // pinned host mirrors and the host copy of the residency table
  void* host = nullptr;
  uint32_t *h_flags = nullptr, *h_miss = nullptr;
  int32_t *h_ids = nullptr, *h_table = nullptr;
  float* h_plogits = nullptr;
  int32_t *h_pairs = nullptr, *d_pairs = nullptr;   // changed table entries (key, slot)
  rl::ExpertLoads pf;                 // prefetch loads for the next gather launch
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> suffix, single, single_pf;
  hipGraphExec_t first_pf = nullptr;
  // tokens, early_outs, loads, sync_tokens, evictions, predictions,
  // predicted_selected, prefetch_loads
  int64_t stats[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool broken = false;
};

namespace {

rl_route_out layer_route(const rl_decode_driver* v, int l) {
  rl_route_out o;
  o.ids = v->ids + l * v->k;
  o.weights = v->wts + l * v->k;
  o.slots = v->slots + l * v->k;
  o.miss_count = v->miss + l;
  o.early_out = v->flags + (v->sticky ? 0 : l);
  o.logits = nullptr;
  return o;
}

// Layer l, then the step to layer l+1 (x_{l+1}, a_{l+1}).  With predict that
// step is the library's fused residual + norm + router kernel run with layer
// l+2's router: a_{l+1} bit for bit as rl_residual_rmsnorm gives it, and the
// prediction's logits as the router GEMV gives them, in one launch.
int run_layer(rl_decode_driver* v, int l, bool predict) {
  const rl_route_out o = layer_route(v, l);
  const int64_t H = v->H;
  int rc = moe_decode_layer(&v->d, l, v->a + l * H, v->W[l], v->bias[l], v->residency, v->pool, &o,
                            v->scratch, v->scratch_bytes, v->y + l * H, v->st);
  if (rc) return rc;
  if (!predict)
    return rl_residual_rmsnorm(1, v->H, v->x + l * H, v->y + l * H, o.early_out,
                               v->x + (l + 1) * H, v->a + (l + 1) * H, v->eps, v->st);
  rl::DecodeArgs a{};
  a.x_prev = v->x + l * H;
  a.y_prev = v->y + l * H;
  a.flag_prev = o.early_out;
  a.x_out = v->x + (l + 1) * H;
  a.a_out = v->a + (l + 1) * H;
  a.eps = v->eps;
  a.W = v->W[l + 2];
  a.bias = v->bias[l + 2];
  a.E = v->E;
  a.H = v->H;
  a.logits = v->plogits;
  a.early_out = v->pflag;               // not read: no sticky flag here
  a.sticky = false;
  rl::launch_decode_router(a, v->st);
  return hipGetLastError() == hipSuccess ? RL_OK : RL_E_DEVICE;
}

// layer l+1's router on a_l alone (a token's first prediction)
int run_predict(rl_decode_driver* v, int l) {
  rl::DecodeArgs a{};
  a.x = v->a + int64_t(l) * v->H;
  a.W = v->W[l + 1];
  a.bias = v->bias[l + 1];
  a.E = v->E;
  a.H = v->H;
  a.logits = v->plogits;
  a.early_out = v->pflag;
  a.sticky = false;
  rl::launch_decode_router(a, v->st);
  return hipGetLastError() == hipSuccess ? RL_OK : RL_E_DEVICE;
}

// The first k experts of the order (logit descending, index ascending) on the
// host, with the routing kernels' key (-0 as +0, a total order on the bits).
void host_topk(const float* lg, int E, int k, int32_t* ids) {
  std::vector<uint32_t> key(E);
  for (int e = 0; e < E; ++e) {
    const float f = lg[e] + 0.0f;
    uint32_t u;
    std::memcpy(&u, &f, sizeof(u));
    key[e] = u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
  }
  std::vector<int32_t> idx(E);
  for (int e = 0; e < E; ++e) idx[e] = e;
  std::partial_sort(idx.begin(), idx.begin() + k, idx.end(), [&](int32_t a, int32_t b) {
    return key[a] > key[b] || (key[a] == key[b] && a < b);
  });
  for (int i = 0; i < k; ++i) ids[i] = idx[i];
}

// flags [L], miss counts [L], ids [L x k] and the prediction's logits [E] sit
// back to back on the device and in the pinned mirror: one copy moves them all
int run_mirror(rl_decode_driver* v) {
  const size_t n = sizeof(int32_t) * (2 * v->L + v->L * v->k) + sizeof(float) * v->E;
  return hipMemcpyAsync(v->h_flags, v->flags, n, hipMemcpyDeviceToHost, v->st) == hipSuccess
             ? RL_OK
             : RL_E_DEVICE;
}

// Layers l0 .. l1-1, with (predict) layer l1+1's router on a_{l1}, then the
// mirror copy.
int run_body(rl_decode_driver* v, int l0, int l1, bool predict) {
  int rc = RL_OK;
  for (int l = l0; l < l1 && !rc; ++l) rc = run_layer(v, l, predict && l == l1 - 1);
  if (!rc && predict && l0 == l1) rc = run_predict(v, l1);
  return rc ? rc : run_mirror(v);
}

int capture(rl_decode_driver* v, int l0, int l1, bool predict, hipGraphExec_t* out) {
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(v->st, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return RL_E_DEVICE;
  const int rc = run_body(v, l0, l1, predict);
  const hipError_t e = hipStreamEndCapture(v->st, &g);
  if (rc || e != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    return rc ? rc : RL_E_DEVICE;
  }
  v->graphs.push_back(g);
  return hipGraphInstantiate(out, g, nullptr, nullptr, 0) == hipSuccess ? RL_OK : RL_E_DEVICE;
}

// Waits for an event by polling it: the host learns a layer's flags a few
// microseconds after the device is done, where a blocking wait sleeps and is
// woken tens of microseconds later.  Every token waits once per layer (and
// once more per layer with prefetch), so the wake-up latency would be paid
// dozens of times per token.
int spin_wait(hipEvent_t e) {
  for (;;) {
    const hipError_t r = hipEventQuery(e);
    if (r == hipSuccess) return RL_OK;
    if (r != hipErrorNotReady) return RL_E_DEVICE;
  }
}

// Everything queued on the main stream so far is done.
int wait_main(rl_decode_driver* v) {
  if (hipEventRecord(v->ev_done, v->st) != hipSuccess) return RL_E_DEVICE;
  return spin_wait(v->ev_done);
}

int launch_wait(rl_decode_driver* v, hipGraphExec_t g) {
  if (hipGraphLaunch(g, v->st) != hipSuccess) return RL_E_DEVICE;
  return wait_main(v);
}

int clear_flags(rl_decode_driver* v, int miss_from) {
  if (!v->sticky) return RL_OK;
  hipError_t e = hipMemsetAsync(v->flags, 0, sizeof(uint32_t), v->st);
  if (e == hipSuccess && miss_from < v->L)
    e = hipMemsetAsync(v->miss + miss_from, 0, sizeof(uint32_t) * (v->L - miss_from), v->st);
  return e == hipSuccess ? RL_OK : RL_E_DEVICE;
}

// Sends the n changed table entries staged in hp to the device table (dp; one
// copy and one scatter launch on stream s).  The staging stays unchanged until
// the copy has run: every load is followed by a wait on the stream.
int put_entries(rl_decode_driver* v, const int32_t* hp, int32_t* dp, int n, hipStream_t s) {
  if (n == 0) return RL_OK;
  if (hipMemcpyAsync(dp, hp, sizeof(int32_t) * 2 * n, hipMemcpyHostToDevice, s) != hipSuccess)
    return RL_E_DEVICE;
  rl::launch_table_scatter(v->residency, dp, n, s);
  return hipGetLastError() == hipSuccess ? RL_OK : RL_E_DEVICE;
}

// Reserves layer's selection in the cache (no victim among exclude_layer's
// experts when >= 0) and, with list NULL, queues on stream s the copies of
// its missing experts from the host store and the table entries that change
// (through the gather kernel, or memcpys and hp/dp staging); with a list,
// writes them there for a later gather launch instead.  Returns the number
// of loads (>= 0) or an error; slots and gens receive the selection's slots
// and their load generations.
int load_layer(rl_decode_driver* v, int layer, const int32_t* sel, int32_t* slots, uint32_t* gens,
               int exclude_layer, hipStream_t s, int32_t* hp, int32_t* dp,
               rl::ExpertLoads* list = nullptr) {
  const int k = v->k;
  int32_t load[32], evicted[32];
  const int n = rl_cache_reserve_excluding(v->cache, layer, sel, k, exclude_layer, slots, load,
                                           evicted, gens);
  if (n < 0) return n;
  int np = 0;
  rl::ExpertLoads ld;
  for (int i = 0; i < k; ++i) {
    if (!load[i]) continue;
    const int64_t key = int64_t(layer) * v->E + sel[i];
    if (v->store_dev) {                      // copied by the gather launch below
      ld.src_row[ld.n] = key;
      ld.dst_slot[ld.n] = slots[i];
      ld.n += 1;
    } else if (hipMemcpyAsync(v->pool + int64_t(slots[i]) * v->slot_bytes,
                              v->store + key * v->slot_bytes, v->slot_bytes,
                              hipMemcpyHostToDevice, s) != hipSuccess) {
      rl_cache_abort(v->cache);
      return RL_E_DEVICE;
    }
    v->h_table[key] = slots[i];
    hp[2 * np] = int32_t(key);
    hp[2 * np + 1] = slots[i];
    np += 1;
    if (evicted[i] >= 0) {
      v->h_table[evicted[i]] = -1;
      hp[2 * np] = evicted[i];
      hp[2 * np + 1] = -1;
      np += 1;
      v->stats[4] += 1;
    }
  }
  int rc = RL_OK;
  if (list) {                                // a later gather launch does it
    ld.n_pairs = np;
    for (int j = 0; j < 2 * np; ++j) ld.pairs[j] = hp[j];
    *list = ld;
  } else if (v->store_dev) {                 // copies and table entries in one launch
    ld.n_pairs = np;
    for (int j = 0; j < 2 * np; ++j) ld.pairs[j] = hp[j];
    rl::launch_expert_gather(v->store_dev, v->pool, v->slot_bytes, ld, v->residency, s);
    rc = hipGetLastError() == hipSuccess ? RL_OK : RL_E_DEVICE;
  } else {
    rc = put_entries(v, hp, dp, np, s);
  }
  if (rc) {
    rl_cache_abort(v->cache);
    return rc;
  }
  rl_cache_commit(v->cache);
  return n;
}

// The predicted experts of layer (layer - 1 runs next): reserved with no
// victim among layer - 1's slots, their loads kept in v->pf for the gather
// launched behind layer - 1's graph; a reservation refused for want of such
// slots loads nothing.  Returns the loads or an error.
int prefetch_layer(rl_decode_driver* v, int layer, const int32_t* sel) {
  int32_t slots[32], pairs[4 * 32];
  uint32_t gens[32];
  const int n = load_layer(v, layer, sel, slots, gens, layer - 1, v->st, pairs, nullptr, &v->pf);
  return n == RL_E_RANGE ? 0 : n;
}

// Loads layer f's missing experts and runs layer f again (graph g: single[f],
// or single_pf[f], which recomputes the prediction from the finished
// a_{f+1}); afterwards its flag must be clear and no slot it used may have
// been reloaded.
int service(rl_decode_driver* v, int f, hipGraphExec_t g) {
  int32_t sel[32], slots[32];
  uint32_t gens[32];
  for (int i = 0; i < v->k; ++i) sel[i] = v->h_ids[f * v->k + i];
  const int n = load_layer(v, f, sel, slots, gens, -1, v->st, v->h_pairs, v->d_pairs);
  if (n < 0) return n;
  v->stats[2] += n;
  int rc = clear_flags(v, v->L);
  if (!rc) rc = launch_wait(v, g);
  if (rc) return rc;
  if (v->h_flags[v->sticky ? 0 : f] != 0) return RL_E_STATE;
  for (int i = 0; i < v->k; ++i)
    if (rl_cache_generation(v->cache, slots[i]) != gens[i]) return RL_E_STATE;
  return RL_OK;
}

int token(rl_decode_driver* v, const float* x0) {
  const int L = v->L, k = v->k;
  if (hipMemcpyAsync(v->x, x0, sizeof(float) * v->H, hipMemcpyDeviceToDevice, v->st) !=
      hipSuccess)
    return RL_E_DEVICE;
  int rc = rl_rmsnorm(1, v->H, v->x, v->a, v->eps, v->st);
  if (rc) return rc;
  const bool sync = v->sync_path;
  int n_eo = 0, l = 0;
  std::vector<std::pair<int, std::vector<int32_t>>> predicted;
  while (l < L) {
    if (!sync) {
      if ((rc = clear_flags(v, l)) || (rc = launch_wait(v, v->suffix[l]))) return rc;
      int f = -1;
      if (v->sticky) {
        if (v->h_flags[0] == 0) break;
        for (int j = l; j < L && f < 0; ++j)
          if (v->h_miss[j]) f = j;
        if (f < 0) return RL_E_STATE;          // a raised flag without a miss
      } else {
        for (int j = l; j < L && f < 0; ++j)
          if (v->h_flags[j]) f = j;
        if (f < 0) break;
      }
      n_eo += 1;
      if ((rc = service(v, f, v->single[f]))) return rc;
      l = f + 1;
    } else {
      // the predicted experts of layer m, copied behind layer m-1's graph
      auto prefetch = [&](int m) {
        std::vector<int32_t> p(k);
        host_topk(v->h_plogits, v->E, k, p.data());
        const int n = prefetch_layer(v, m, p.data());
        if (n < 0) return n;
        v->stats[7] += n;
        predicted.emplace_back(m, std::move(p));
        return int(RL_OK);
      };
      if (l == 0 && v->prefetch && L > 1) {    // layer 1's prediction, from a_0
        if ((rc = launch_wait(v, v->first_pf)) || (rc = prefetch(1))) return rc;
      }
      const bool predict = v->prefetch && l + 2 < L;
      hipGraphExec_t g = predict ? v->single_pf[l] : v->single[l];
      if ((rc = clear_flags(v, L))) return rc;
      if (hipGraphLaunch(g, v->st) != hipSuccess ||
          hipEventRecord(v->ev_done, v->st) != hipSuccess)
        return RL_E_DEVICE;
      if (v->pf.n > 0 || v->pf.n_pairs > 0) {  // layer l+1's predicted experts
        rl::launch_expert_gather(v->store_dev, v->pool, v->slot_bytes, v->pf, v->residency,
                                 v->st);
        v->pf.n = v->pf.n_pairs = 0;
        if (hipGetLastError() != hipSuccess) return RL_E_DEVICE;
      }
      if ((rc = spin_wait(v->ev_done))) return rc;
      if (v->h_flags[v->sticky ? 0 : l] != 0) {
        n_eo += 1;
        if ((rc = service(v, l, g))) return rc;
      }
      if (predict && (rc = prefetch(l + 2))) return rc;
      l += 1;
    }
  }
  // the mirror holds every layer's last selection (the last launch copied it)
  for (int layer = 0; layer < L; ++layer) {
    rc = rl_cache_touch(v->cache, layer, v->h_ids + layer * k, k);
    if (rc < 0) return rc;
  }
  for (const auto& pr : predicted) {
    v->stats[5] += 1;
    const int32_t* got = v->h_ids + pr.first * k;
    for (int i = 0; i < k; ++i) {
      bool dup = false;                        // count each predicted expert once
      for (int j = 0; j < i && !dup; ++j) dup = pr.second[j] == pr.second[i];
      if (dup) continue;
      if (std::find(got, got + k, pr.second[i]) != got + k) v->stats[6] += 1;
    }
  }
  v->stats[0] += 1;
  v->stats[1] += n_eo;
  v->stats[3] += sync ? 1 : 0;
  if (n_eo > v->limit)
    v->sync_path = true;
  else if (n_eo == 0)
    v->sync_path = false;
  return RL_OK;
}

void release(rl_decode_driver* v) {
  for (auto g : v->suffix)
    if (g) (void)hipGraphExecDestroy(g);
  for (auto g : v->single)
    if (g) (void)hipGraphExecDestroy(g);
  for (auto g : v->single_pf)
    if (g) (void)hipGraphExecDestroy(g);
  if (v->first_pf) (void)hipGraphExecDestroy(v->first_pf);
  if (v->ev_done) (void)hipEventDestroy(v->ev_done);

  for (auto g : v->graphs) (void)hipGraphDestroy(g);
  if (v->dev) (void)hipFree(v->dev);
  if (v->host) (void)hipHostFree(v->host);
  delete v;
}

}  // namespace

extern "C" {

rl_decode_driver* rl_driver_create(const rl_driver_config* c, void* stream) {
  if (!c || !c->desc || !c->router_w || !c->residency || !c->slot_pool || !c->host_store ||
      !c->cache || !c->x)
    return nullptr;
  const rl_moe_desc* d = c->desc;
  if (rl_decode_scratch_bytes(d) < 0 || d->top_k > 32 || c->early_out_limit < 0) return nullptr;
  const int L = d->n_layers;
  for (int l = 0; l < L; ++l)
    if (!c->router_w[l]) return nullptr;
  rl_decode_driver* v = new (std::nothrow) rl_decode_driver;
  if (!v) return nullptr;
  v->d = *d;
  v->L = L;
  v->E = d->n_experts;
  v->H = d->hidden;
  v->k = d->top_k;
  v->sticky = (d->flags & RL_STICKY_EARLY_OUT) != 0;
  v->prefetch = c->prefetch != 0 && L > 1;
  v->limit = c->early_out_limit;
  v->eps = c->eps;
  v->st = static_cast<hipStream_t>(stream);
  v->W.assign(c->router_w, c->router_w + L);
  v->bias.assign(L, nullptr);
  if (c->router_bias)
    for (int l = 0; l < L; ++l) v->bias[l] = c->router_bias[l];
  v->residency = c->residency;
  v->pool = static_cast<uint8_t*>(c->slot_pool);
  v->store = static_cast<const uint8_t*>(c->host_store);
  v->slot_bytes = rl_slot_bytes(d);
  {
    // loads go through the gather kernel when the store has a device address
    // (pinned by hipHostMalloc); else one hipMemcpyAsync per expert
    void* p = nullptr;
    if (v->slot_bytes % 16 == 0 &&
        hipHostGetDevicePointer(&p, const_cast<void*>(c->host_store), 0) == hipSuccess)
      v->store_dev = p;
    (void)hipGetLastError();
  }
  v->cache = c->cache;
  v->x = c->x;
  const int64_t H = v->H, k = v->k;
  v->scratch_bytes = rl_decode_scratch_bytes(d);
  // one device allocation, every part 256-byte aligned
  auto up = [](int64_t n) { return (n + 255) & ~int64_t(255); };
  // flags, miss, ids, prediction logits contiguous (one mirror copy)
  const int64_t o_a = 0, o_y = o_a + up(4 * (L + 1) * H), o_flags = o_y + up(4 * L * H),
                o_miss = o_flags + 4 * L, o_ids = o_miss + 4 * L, o_plog = o_ids + 4 * L * k,
                o_slots = o_flags + up(4 * (2 * L + L * k) + 4 * int64_t(v->E)),
                o_wts = o_slots + up(4 * L * k), o_pflag = o_wts + up(4 * L * k),
                o_pairs = o_pflag + 256, o_scr = o_pairs + up(4 * 4 * k),
                dev_bytes = o_scr + up(v->scratch_bytes);
  const int64_t h_flags = 0, h_miss = h_flags + 4 * L, h_ids = h_miss + 4 * L,
                h_plog = h_ids + 4 * L * k, h_pairs = up(h_plog + 4 * int64_t(v->E)),
                h_table = h_pairs + up(4 * 4 * k),
                host_bytes = h_table + up(4 * int64_t(L) * v->E);
  if (hipMalloc(&v->dev, dev_bytes) != hipSuccess) v->dev = nullptr;
  if (hipHostMalloc(&v->host, host_bytes, hipHostMallocDefault) != hipSuccess) v->host = nullptr;
  if (hipEventCreateWithFlags(&v->ev_done, hipEventDisableTiming) != hipSuccess) {
    v->ev_done = nullptr;
    release(v);
    return nullptr;
  }
  if (!v->dev || !v->host) {
    release(v);
    return nullptr;
  }
  uint8_t* b = static_cast<uint8_t*>(v->dev);
  v->a = reinterpret_cast<float*>(b + o_a);
  v->y = reinterpret_cast<float*>(b + o_y);
  v->ids = reinterpret_cast<int32_t*>(b + o_ids);
  v->slots = reinterpret_cast<int32_t*>(b + o_slots);
  v->wts = reinterpret_cast<float*>(b + o_wts);
  v->miss = reinterpret_cast<uint32_t*>(b + o_miss);
  v->flags = reinterpret_cast<uint32_t*>(b + o_flags);
  v->plogits = reinterpret_cast<float*>(b + o_plog);
  v->pflag = reinterpret_cast<uint32_t*>(b + o_pflag);
  v->d_pairs = reinterpret_cast<int32_t*>(b + o_pairs);
  v->scratch = b + o_scr;
  uint8_t* hb = static_cast<uint8_t*>(v->host);
  v->h_flags = reinterpret_cast<uint32_t*>(hb + h_flags);
  v->h_miss = reinterpret_cast<uint32_t*>(hb + h_miss);
  v->h_ids = reinterpret_cast<int32_t*>(hb + h_ids);
  v->h_plogits = reinterpret_cast<float*>(hb + h_plog);
  v->h_pairs = reinterpret_cast<int32_t*>(hb + h_pairs);
  if (v->prefetch && !v->store_dev) {   // prefetch copies through the gather launch
    release(v);
    return nullptr;
  }
  v->h_table = reinterpret_cast<int32_t*>(hb + h_table);
  int rc = rl_cache_table(v->cache, v->h_table);
  // the device table starts as the cache's table
  if (!rc && hipMemcpyAsync(v->residency, v->h_table, 4 * int64_t(L) * v->E,
                            hipMemcpyHostToDevice, v->st) != hipSuccess)
    rc = RL_E_DEVICE;
  if (!rc && hipMemsetAsync(v->dev, 0, dev_bytes, v->st) != hipSuccess) rc = RL_E_DEVICE;
  // one eager layer (and prediction) before any capture
  if (!rc && v->prefetch) rc = run_body(v, 0, 0, true);
  if (!rc) rc = run_body(v, 0, 1, false);
  if (!rc && hipStreamSynchronize(v->st) != hipSuccess) rc = RL_E_DEVICE;
  v->suffix.assign(L, nullptr);
  v->single.assign(L, nullptr);
  v->single_pf.assign(L, nullptr);
  if (!rc && v->prefetch) rc = capture(v, 0, 0, true, &v->first_pf);
  for (int l = 0; l < L && !rc; ++l) {
    rc = capture(v, l, L, false, &v->suffix[l]);
    if (!rc) rc = capture(v, l, l + 1, false, &v->single[l]);
    if (!rc && v->prefetch && l + 2 < L) rc = capture(v, l, l + 1, true, &v->single_pf[l]);
  }
  if (rc) {
    release(v);
    return nullptr;
  }
  return v;
}

int rl_driver_token(rl_decode_driver* v, const float* x0) {
  if (!v || !x0) return RL_E_INVAL;
  if (v->broken) return RL_E_STATE;
  const int rc = token(v, x0);
  if (rc) v->broken = true;   // an interrupted token leaves cache and pool out of step
  return rc;
}

int rl_driver_stats(const rl_decode_driver* v, int64_t* out) {
  if (!v || !out) return RL_E_INVAL;
  for (int i = 0; i < 8; ++i) out[i] = v->stats[i];
  return RL_OK;
}

void rl_driver_destroy(rl_decode_driver* v) {
  if (!v) return;
  (void)hipStreamSynchronize(v->st);
  release(v);
}

}  // extern "C"
