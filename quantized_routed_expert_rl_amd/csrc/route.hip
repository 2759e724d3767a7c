// Router GEMV/GEMM, softmax top-k, renormalised weights and residency lookup
// ("Red Lite dev21 - GPU-routed decode", "What changed": candidates ordered
// by logit, ties to the lower index, weights renormalised over the selected
// experts, expert lookups in the residency table, per-layer miss count;
// "Red Lite dev23", "What changed": the router raises the early-out flag).
//
// Logits accumulate in float64: every float32 product is exact in float64,
// so the logit is the float32 rounding of a float64 sum whatever the order
// of the partial sums, and the selected ids do not depend on the launch
// shape.
#include "rl_common.h"
#include "rl_kernels.h"

namespace rl {

// ------------------------------------------------------------ selection
// Top-k of E logits by one wave (lane l owns experts l + 64*i, i < N).
// Each lane sorts its N candidates once (largest key first; equal keys keep
// the lower index first), then k rounds take the best lane head: a DPP max
// over the 64 heads, and on an exact tie the lowest expert index.
// Writes sel_ids[r], sel_key[r] (float32 logit) for r < k into LDS arrays.
template <int N>
__device__ void wave_topk(const float* __restrict__ lg, int E, int k,
                          uint32_t* s_key, int* s_idx, int* sel_ids, float* sel_lg) {
  const int lane = threadIdx.x & 63;
  uint32_t key[N];
  int idx[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? float_key(lg[e]) : 0u;
    idx[i] = e;
  }
  // bubble network, stable: swap only when the later key is strictly larger
#pragma unroll
  for (int a = 0; a < N; ++a) {
#pragma unroll
    for (int i = 0; i + 1 < N - a; ++i) {
      const bool sw = key[i + 1] > key[i];
      const uint32_t k0 = key[i], k1 = key[i + 1];
      const int i0 = idx[i], i1 = idx[i + 1];
      key[i] = sw ? k1 : k0;
      key[i + 1] = sw ? k0 : k1;
      idx[i] = sw ? i1 : i0;
      idx[i + 1] = sw ? i0 : i1;
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    s_key[lane * N + i] = key[i];
    s_idx[lane * N + i] = idx[i];
  }
  int ptr = 0;
  uint32_t hk = key[0];
  int hi = idx[0];
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(hk);
    const unsigned long long tie = __ballot(hk == m);
    int win;
    if (__popcll(tie) == 1) {
      win = __ffsll(tie) - 1;
    } else {
      const uint32_t mi = wave_min_u32(hk == m ? uint32_t(hi) : 0xffffffffu);
      win = __ffsll(__ballot(hk == m && uint32_t(hi) == mi)) - 1;
    }
    const int e = __builtin_amdgcn_readlane(hi, win);
    if (lane == 0) {
      sel_ids[r] = e;
      sel_lg[r] = lg[e];
    }
    if (lane == win) {
      ++ptr;
      hk = ptr < N ? s_key[lane * N + ptr] : 0u;
      hi = ptr < N ? s_idx[lane * N + ptr] : 0x7fffffff;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Weights, slots and miss count of one token from the selection in LDS.
// Returns the token's miss count (in every lane).
__device__ int finish_token(const int* sel_ids, const float* sel_lg, int k, int E,
                            int layer, int n_slots, const int32_t* __restrict__ residency,
                            int32_t* ids, float* weights, int32_t* slots) {
  const int lane = threadIdx.x & 63;
  double a = 0.0;
  if (lane < k) a = exp(double(sel_lg[lane]) - double(sel_lg[0]));
  double total = 0.0;
  for (int r = 0; r < k; ++r) {  // rank order
    const double ar = __shfl(a, r, kWave);
    total += ar;
  }
  int slot = -1;
  if (lane < k) {
    const int e = min(max(sel_ids[lane], 0), E - 1);   // in bounds even for NaN logits
    const int v = residency[int64_t(layer) * E + e];
    slot = (v >= 0 && v < n_slots) ? v : -1;
    ids[lane] = e;
    weights[lane] = float(a / total);
    slots[lane] = slot;
  }
  return __popcll(__ballot(lane < k && slot < 0));
}

// ----------------------------------------------------- decode: T = 1
// Router GEMV over E rows (rows e = block + grid*i), then the last block to
// finish performs the selection.  One wave per block.
template <int N, int NM>
__global__ __launch_bounds__(64) void route_gemv_topk_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
    int E, int H, int k, int layer, int n_slots, const int32_t* __restrict__ residency,
    float* __restrict__ logits, float* __restrict__ logits_out, uint32_t* counter,
    int32_t* ids, float* weights, int32_t* slots, uint32_t* miss_count, uint32_t* early_out) {
  const int lane = threadIdx.x;
  // lane holds x[256m + 4 lane + q], m < NM (H = 256*NM)
  float xv[NM * 4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float4 v = *reinterpret_cast<const float4*>(x + 256 * m + 4 * lane);
    xv[4 * m + 0] = v.x;
    xv[4 * m + 1] = v.y;
    xv[4 * m + 2] = v.z;
    xv[4 * m + 3] = v.w;
  }
  for (int e = blockIdx.x; e < E; e += gridDim.x) {
    const float* row = W + int64_t(e) * H;
    float4 wv[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) wv[m] = *reinterpret_cast<const float4*>(row + 256 * m + 4 * lane);
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      acc = fma(double(wv[m].x), double(xv[4 * m + 0]), acc);
      acc = fma(double(wv[m].y), double(xv[4 * m + 1]), acc);
      acc = fma(double(wv[m].z), double(xv[4 * m + 2]), acc);
      acc = fma(double(wv[m].w), double(xv[4 * m + 3]), acc);
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) {
      if (bias) acc += double(bias[e]);
      const float l = float(acc);
      logits[e] = l;
      if (logits_out) logits_out[e] = l;
    }
  }
  // last block to arrive selects
  __shared__ int s_last;
  __threadfence();
  if (lane == 0) s_last = (atomicAdd(counter, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  __shared__ uint32_t s_key[64 * N];
  __shared__ int s_idx[64 * N];
  __shared__ int sel_ids[32];
  __shared__ float sel_lg[32];
  wave_topk<N>(logits, E, k, s_key, s_idx, sel_ids, sel_lg);
  const int miss = finish_token(sel_ids, sel_lg, k, E, layer, n_slots, residency, ids, weights, slots);
  if (lane == 0) {
    *miss_count = uint32_t(miss);
    *early_out = miss > 0 ? 1u : 0u;
    *counter = 0u;  // ready for the next call
  }
}

// ------------------------------------------------------- T > 1: GEMM
// logits[t][e] = fl32(sum_i W[e][i] x[t][i] + b[e]) on the float64 matrix
// cores (v_mfma_f64_16x16x4f64; A lane l: row l%16, K index l/16; B lane l:
// column l%16, K index l/16; output lane l, v: row l/16 + 4v, column l%16).
// Block = 32 tokens x 32 experts, one 16x16 tile per wave over all of K.
// Inside each 16-value chunk c, MFMA step 4c+i of lane quad kq takes K index
// 16c + 4kq + i for both operands, so each lane reads float4s.
typedef double v4d __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void route_gemm_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
    int T, int E, int H, float* __restrict__ logits, float* __restrict__ logits_out,
    uint32_t* miss_count, uint32_t* early_out) {
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 32 + (wv >> 1) * 16, e0 = blockIdx.x * 32 + (wv & 1) * 16;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    *miss_count = 0u;
    *early_out = 0u;
  }
  const int r = l & 15, kq = l >> 4;
  const int ta = t0 + r, eb = e0 + r;
  const bool va = ta < T, vb = eb < E;
  const float* xa = x + int64_t(va ? ta : 0) * H + 4 * kq;
  const float* wb = W + int64_t(vb ? eb : 0) * H + 4 * kq;
  // four independent accumulation chains (one per 16-value chunk of each
  // 64-value step) keep the matrix core busy; summed in float64 at the end
  v4d acc4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc4[u] = v4d{0.0, 0.0, 0.0, 0.0};
  for (int c = 0; c < H; c += 64) {
    float4 av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = va ? *reinterpret_cast<const float4*>(xa + c + 16 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
      bv[u] = vb ? *reinterpret_cast<const float4*>(wb + c + 16 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc4[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(av[u].x), double(bv[u].x), acc4[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc4[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(av[u].y), double(bv[u].y), acc4[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc4[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(av[u].z), double(bv[u].z), acc4[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc4[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(av[u].w), double(bv[u].w), acc4[u], 0, 0, 0);
  }
  const v4d acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + kq + 4 * v, e = e0 + r;
    if (t < T && e < E) {
      double s = acc[v];
      if (bias) s += double(bias[e]);
      const float lg = float(s);
      logits[int64_t(t) * E + e] = lg;
      if (logits_out) logits_out[int64_t(t) * E + e] = lg;
    }
  }
}

// One wave per token: selection, weights, lookup; misses summed atomically.
template <int N>
__global__ __launch_bounds__(64) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int layer, int n_slots,
    const int32_t* __restrict__ residency, int32_t* ids, float* weights, int32_t* slots,
    uint32_t* miss_count, uint32_t* early_out) {
  __shared__ uint32_t s_key[64 * N];
  __shared__ int s_idx[64 * N];
  __shared__ int sel_ids[32];
  __shared__ float sel_lg[32];
  const int t = blockIdx.x;
  wave_topk<N>(logits + int64_t(t) * E, E, k, s_key, s_idx, sel_ids, sel_lg);
  const int miss = finish_token(sel_ids, sel_lg, k, E, layer, n_slots, residency,
                                ids + int64_t(t) * k, weights + int64_t(t) * k,
                                slots + int64_t(t) * k);
  if ((threadIdx.x & 63) == 0 && miss > 0) {
    atomicAdd(miss_count, uint32_t(miss));
    atomicOr(early_out, 1u);
  }
}

// ------------------------------------------------------------ launchers
template <int N>
static void launch_gemv_n(const RouteArgs& a, hipStream_t st) {
  const int grid = a.E < 256 ? a.E : 256;
  switch (a.H) {
#define RL_CASE(NM)                                                                        \
  case 256 * NM:                                                                           \
    route_gemv_topk_kernel<N, NM><<<grid, 64, 0, st>>>(                                   \
        a.x, a.W, a.bias, a.E, a.H, a.k, a.layer, a.n_slots, a.residency, a.logits,        \
        a.logits_out, a.counter, a.ids, a.weights, a.slots, a.miss_count, a.early_out);    \
    break;
    RL_CASE(1) RL_CASE(2) RL_CASE(4) RL_CASE(8)
#undef RL_CASE
  }
}

template <int N>
static void launch_topk_n(const RouteArgs& a, hipStream_t st) {
  route_topk_kernel<N><<<a.T, 64, 0, st>>>(a.logits, a.T, a.E, a.k, a.layer, a.n_slots,
                                           a.residency, a.ids, a.weights, a.slots,
                                           a.miss_count, a.early_out);
}

static int cand_per_lane(int E) {
  int n = 1;
  while (64 * n < E) n <<= 1;
  return n;
}

void launch_route(const RouteArgs& a, hipStream_t st) {
  const int n = cand_per_lane(a.E);
  if (a.T == 1 && a.counter) {   // one token: GEMV, last block selects
    switch (n) {
      case 1: launch_gemv_n<1>(a, st); break;
      case 2: launch_gemv_n<2>(a, st); break;
      case 4: launch_gemv_n<4>(a, st); break;
      case 8: launch_gemv_n<8>(a, st); break;
      default: launch_gemv_n<16>(a, st); break;
    }
    return;
  }
  dim3 grid((a.E + 31) / 32, (a.T + 31) / 32);
  route_gemm_kernel<<<grid, 256, 0, st>>>(a.x, a.W, a.bias, a.T, a.E, a.H, a.logits,
                                          a.logits_out, a.miss_count, a.early_out);
  switch (n) {
    case 1: launch_topk_n<1>(a, st); break;
    case 2: launch_topk_n<2>(a, st); break;
    case 4: launch_topk_n<4>(a, st); break;
    case 8: launch_topk_n<8>(a, st); break;
    default: launch_topk_n<16>(a, st); break;
  }
}

}  // namespace rl
