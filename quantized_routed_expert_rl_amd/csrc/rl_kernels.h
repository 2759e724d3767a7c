// Launch interfaces between the C ABI (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rl_common.h"

namespace rl {

struct RouteArgs {
  const float* x;
  const float* W;
  const float* bias;
  int T, E, H, k, layer, n_slots;
  const int32_t* residency;
  float* logits;       // [T][E] scratch
  float* logits_out;   // optional copy for the caller
  int32_t* ids;
  float* weights;
  int32_t* slots;
  uint32_t* miss_count;
  uint32_t* early_out;
};
void launch_route(const RouteArgs& a, hipStream_t st);

struct DecodeArgs {
  PoolView pool;
  int H, F, E, k, qbits, layer, n_slots;
  const float* x;
  const float* W;
  const float* bias;
  const int32_t* residency;
  float* logits;        // [E] scratch
  float* logits_out;    // optional copy for the caller
  int32_t* ids;         // route outputs
  float* weights;
  int32_t* slots;
  uint32_t* miss_count;
  uint32_t* early_out;
  float* hbuf;          // [k][F] scratch
  float* y;
  bool mfma;            // int8 matrix-core expert kernels (F % 256 == 0)
  bool sticky;          // early_out shared and only raised: a set flag stops the call
  // the step before the layer, folded into the router kernel (a_out NULL:
  // none, x is the layer input): r = x_prev + y_prev (x_prev alone when
  // y_prev is NULL or *flag_prev is set), written to x_out when not NULL;
  // x = a_out = rmsnorm(r) with epsilon eps
  const float* x_prev = nullptr;
  const float* y_prev = nullptr;
  const uint32_t* flag_prev = nullptr;
  float* x_out = nullptr;
  float* a_out = nullptr;
  float eps = 0.f;
  // words the router kernel zeroes first (a one-token rl_route's miss count
  // and flag, which its top-k kernel then accumulates), or NULL
  uint32_t* clear_miss = nullptr;
  uint32_t* clear_flag = nullptr;
};
void launch_decode_router(const DecodeArgs& a, hipStream_t st);
void launch_decode_gateup(const DecodeArgs& a, hipStream_t st);
void launch_decode_down_sum(const DecodeArgs& a, hipStream_t st);
void launch_decode_gateup_mfma(const DecodeArgs& a, hipStream_t st);
void launch_decode_down_sum_mfma(const DecodeArgs& a, hipStream_t st);

// Plan of a prefill chunk inside scratch (see rl_prefill_layout).
struct PlanPtrs {
  int32_t* n_groups;
  int32_t* group_bounds;
  int32_t* n_buckets;
  int32_t* group_bucket_start;
  int32_t* bucket_expert;
  int32_t* bucket_start;
  int32_t* pairs;
  // internal
  int32_t* counts;        // [max_groups*E]
  int32_t* offs;          // [max_groups*E]
  int32_t* bucket_slot;   // [T*k]
  int32_t* tile_start;    // [T*k+1] token tiles before each bucket
  int32_t* tile_bucket;   // [T*k] bucket of each token tile
  int32_t* n_tiles;       // [1]
};

struct PrefillArgs {
  PoolView pool;
  int T, H, F, E, k, qbits, plan_cap, layer;
  const float* x;
  const int32_t* residency;
  const int32_t* ids;
  const int32_t* slots;
  const float* weights;
  const uint32_t* early_out;
  PlanPtrs plan;
  bool mfma;        // int8 matrix-core path (F % 256 == 0)
  int tile_tokens;  // tokens per token tile of a bucket
  float* hbuf;      // [T*k][F], rows in sorted pair order
  float* ebuf;      // [T*k][H], rows by pair id p = t*k + r
  uint8_t* xq;      // [T][H*4] digit operands of x (MFMA path)
  int32_t* xe;      // [T][H/256] exponents of x
  uint8_t* hq;      // [T*k][F*4] digit operands of h (MFMA path)
  int32_t* he;      // [T*k][F/256] exponents of h
  float* y;
  int n_slots = 0;
};
void launch_prefill_plan(const PrefillArgs& a, hipStream_t st);
void launch_prefill_gateup(const PrefillArgs& a, hipStream_t st);
void launch_prefill_down(const PrefillArgs& a, hipStream_t st);
void launch_prefill_sum(const PrefillArgs& a, hipStream_t st);
void launch_quantize_x(const PrefillArgs& a, hipStream_t st);
void launch_quantize_h(const PrefillArgs& a, hipStream_t st);
void launch_prefill_gateup_mfma(const PrefillArgs& a, hipStream_t st);
void launch_prefill_down_mfma(const PrefillArgs& a, hipStream_t st);

// Compute units of the current device (cached per device; util.hip).
int device_cu_count();

// moe_decode_layer's argument checks, scratch size aside (abi.hip).
int decode_layer_check(const rl_moe_desc* d, int32_t layer, const float* x, const float* router_w,
                       const int32_t* residency, const void* slot_pool, const rl_route_out* route,
                       const void* scratch, const float* y);

void launch_rmsnorm(int T, int H, const float* x, float* out, float eps, hipStream_t st);
void launch_residual_rmsnorm(int T, int H, const float* x, const float* y,
                             const uint32_t* early_out, float* x_out, float* a_out, float eps,
                             hipStream_t st);
void launch_residual_add(int T, int H, float* x, const float* y, const uint32_t* early_out,
                         hipStream_t st);
void launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int n_cu, hipStream_t st);
void launch_table_scatter(int32_t* table, const int32_t* pairs, int n, hipStream_t st);

// One layer's expert loads (k <= 32), passed by value to the gather kernel:
// expert i goes from host-store row src_row[i] to pool slot dst_slot[i];
// pairs[2j], pairs[2j+1] = (key, slot) residency entries to write, j < n_pairs.
struct ExpertLoads {
  int32_t n = 0, n_pairs = 0;
  int64_t src_row[32];
  int32_t dst_slot[32];
  int32_t pairs[128];
};
// store_dev: the device address of the pinned host store; slot_bytes % 16 == 0.
void launch_expert_gather(const void* store_dev, void* pool, int64_t slot_bytes,
                          const ExpertLoads& ld, int32_t* table, hipStream_t st);


}  // namespace rl
