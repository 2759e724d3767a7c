// Single-token decode of one MoE layer in three kernels:
//   1. router GEMV (float64 accumulation) -> logits;
//   2. softmax top-k + residency lookup, redone by every block of the
//      gate/up kernel (no cross-block hand-off), then the gate/up GEMVs of
//      the selected experts with SwiGLU;
//   3. down GEMVs fused with the rank-ordered weighted sum.
// Sources: "Red Lite dev21 - GPU-routed decode", "What changed" (the router
// writes the slot table and weights that the expert kernels read, and a
// per-layer miss count); "Red Lite dev23", "What changed" (with the flag set
// every expert kernel returns at once); "Red Lite dev20", "What changed" (a
// token's experts are summed in router selection order).
//
// Lane mapping of the expert GEMVs.  A lane owns one 32-value group of a row:
// 8 bytes of codes, one group scale, one block scale, and the 32 matching
// activations held in registers.  A row of C values spans C/32 lanes (the
// notes found 8 lanes of 64 values best for the 512-column down rows on a
// 32-wide SIMD, "Red Lite dev38", "Changes"; on a 64-wide wave the same 8
// bytes per lane gives 16 lanes of 32 values), and a DPP sum over those lanes
// finishes the row.  Every load a wave needs is issued before it computes.
#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_select.h"

namespace rl {

int cand_per_lane(int E);

__device__ inline void load_act32(const float* __restrict__ src, float* xv, float& xsum) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
    xv[4 * q + 0] = v.x;
    xv[4 * q + 1] = v.y;
    xv[4 * q + 2] = v.z;
    xv[4 * q + 3] = v.w;
  }
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 32; ++n) s += xv[n];
  xsum = s;
}

// ------------------------------------------------------------ 1. router
// Block = one wave over up to RPB rows e = blockIdx*rows .. +rows-1; all row
// loads are issued before any arithmetic.  H = 256*NM.
template <int RPB, int NM>
__global__ __launch_bounds__(64) void decode_router_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
    int E, int H, int rows, float* __restrict__ logits, float* __restrict__ logits_out,
    const uint32_t* __restrict__ early_out, int sticky, uint32_t* clear0, uint32_t* clear1) {
  const int lane = threadIdx.x;
  if (blockIdx.x == 0 && lane == 0) {   // a one-token rl_route's miss count and flag
    if (clear0) *clear0 = 0u;
    if (clear1) *clear1 = 0u;
  }
  if (sticky && *early_out) return;
  const int e0 = blockIdx.x * rows;
  float4 xv[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) xv[m] = *reinterpret_cast<const float4*>(x + 256 * m + 4 * lane);
  float4 wv[RPB][NM];
#pragma unroll
  for (int rr = 0; rr < RPB; ++rr) {
    const int e = e0 + rr < E && rr < rows ? e0 + rr : e0;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      wv[rr][m] = *reinterpret_cast<const float4*>(W + int64_t(e) * H + 256 * m + 4 * lane);
  }
#pragma unroll
  for (int rr = 0; rr < RPB; ++rr) {
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      acc = fma(double(wv[rr][m].x), double(xv[m].x), acc);
      acc = fma(double(wv[rr][m].y), double(xv[m].y), acc);
      acc = fma(double(wv[rr][m].z), double(xv[m].z), acc);
      acc = fma(double(wv[rr][m].w), double(xv[m].w), acc);
    }
    acc = wave_sum_f64(acc);
    const int e = e0 + rr;
    if (lane == 0 && rr < rows && e < E) {
      if (bias) acc += double(bias[e]);
      const float l = float(acc);
      logits[e] = l;
      if (logits_out) logits_out[e] = l;
    }
  }
}

// The step between two layers of a stack folded into the router: each block
// (one wave) rebuilds r = x_prev + y_prev (x_prev when there is no y_prev or
// the previous layer's flag is set) and a = rmsnorm(r) in the order of the
// 256-thread norm kernels: there thread t owns the 4-value chunks at
// 4t + 1024u and chains their float64 squares in (u, component) order; here
// lane l holds the chunks 256m + 4l of the router's operand layout, which are
// those of threads l + 64w with m = w + 4u, so chain w runs over m = w, w + 4,
// ..., the same butterfly sum gives each wave's total and the four totals
// are added in w order: a is bit-identical to rl_residual_rmsnorm's.  Block
// 0 writes r and a; every block then computes its router row as
// decode_router_kernel does, from the same registers.
template <int NM>
__global__ __launch_bounds__(64) void decode_router_residual_kernel(
    const float* __restrict__ x_prev, const float* __restrict__ y_prev,
    const uint32_t* __restrict__ flag_prev, float* __restrict__ x_out, float* __restrict__ a_out,
    float eps, const float* __restrict__ W, const float* __restrict__ bias, int E, int H,
    float* __restrict__ logits, float* __restrict__ logits_out,
    const uint32_t* __restrict__ early_out, int sticky) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  if (e > 0 && sticky && *early_out) return;      // block 0 still writes r and a
  float4 wv[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
    wv[m] = *reinterpret_cast<const float4*>(W + int64_t(e) * H + 256 * m + 4 * lane);
  const bool skip = !y_prev || (flag_prev && *flag_prev);
  float4 xv[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int i = 256 * m + 4 * lane;
    const float4 xp = *reinterpret_cast<const float4*>(x_prev + i);
    if (skip) {
      xv[m] = xp;
    } else {
      const float4 yp = *reinterpret_cast<const float4*>(y_prev + i);
      xv[m] = make_float4(xp.x + yp.x, xp.y + yp.y, xp.z + yp.z, xp.w + yp.w);
    }
  }
  double tot[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    double s = 0.0;
#pragma unroll
    for (int m = w; m < NM; m += 4) s = chunk_sq(xv[m], s);
    tot[w] = wave_sum_f64(s);
  }
  const double inv = 1.0 / sqrt((tot[0] + tot[1] + tot[2] + tot[3]) / H + double(eps));
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int i = 256 * m + 4 * lane;
    const float4 av = chunk_scale(xv[m], inv);
    if (e == 0) {
      if (x_out) *reinterpret_cast<float4*>(x_out + i) = xv[m];
      *reinterpret_cast<float4*>(a_out + i) = av;
    }
    xv[m] = av;
  }
  if (sticky && *early_out) return;
  double acc = 0.0;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    acc = fma(double(wv[m].x), double(xv[m].x), acc);
    acc = fma(double(wv[m].y), double(xv[m].y), acc);
    acc = fma(double(wv[m].z), double(xv[m].z), acc);
    acc = fma(double(wv[m].w), double(xv[m].w), acc);
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) {
    if (bias) acc += double(bias[e]);
    const float l = float(acc);
    logits[e] = l;
    if (logits_out) logits_out[e] = l;
  }
}

// -------------------------------------------------- 2. top-k + gate/up
// Block = (expert rank r, 16 rows j); wave w takes rows j0+4w .. +3 of gate
// and of up.  Wave 0 selects the experts while the other waves load x;
// block 0 publishes the routing results.
template <int N, int QBITS, int LPR>
__global__ __launch_bounds__(256) void decode_topk_gateup_kernel(
    PoolView pv, int H, int F, int E, int k, int layer, int n_slots,
    const float* __restrict__ x, const float* __restrict__ logits,
    const int32_t* __restrict__ residency, int32_t* ids, float* weights, int32_t* slots,
    uint32_t* miss_count, uint32_t* early_out, float* __restrict__ hbuf, int sticky) {
  if (sticky && *early_out) return;
  constexpr int RPI = 64 / LPR;     // rows per wave iteration
  constexpr int JW = 4;             // j values per wave
  constexpr int NIT = 2 * JW / RPI > 0 ? 2 * JW / RPI : 1;
  __shared__ __align__(16) TopkLds s_tk;
  __shared__ int sel_ids[32];
  __shared__ float sel_lg[32];
  __shared__ int sel_res[32];
  __shared__ int s_ids[32];
  __shared__ float s_w[32];
  __shared__ int s_slot[32];
  __shared__ int s_miss;
  __shared__ float s_row[4][2 * JW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = lane % LPR, rs = lane / LPR;
  float xv[32], xsum;
  load_act32(x + 32 * seg, xv, xsum);
  if (wv == 0) {
    wave_topk<N>(logits, E, k, residency + int64_t(layer) * E, s_tk, sel_ids, sel_lg, sel_res);
    const int miss = finish_token(sel_ids, sel_lg, sel_res, k, E, n_slots, s_ids, s_w, s_slot);
    if (lane == 0) s_miss = miss;
    if (blockIdx.x == 0) {
      if (lane < k) {
        ids[lane] = s_ids[lane];
        weights[lane] = s_w[lane];
        slots[lane] = s_slot[lane];
      }
      if (lane == 0) {
        *miss_count = uint32_t(miss);
        if (!sticky || miss > 0) *early_out = miss > 0 ? 1u : 0u;
      }
    }
  }
  __syncthreads();
  if (s_miss) return;                  // early-out: nothing downstream runs
  const int per_expert = F / 16;
  const int r = blockIdx.x / per_expert;
  const int j0 = (blockIdx.x % per_expert) * 16 + JW * wv;
  const int slot = s_slot[r];
  const uint8_t* gate = tensor_base(pv, slot, 0);
  const uint8_t* up = tensor_base(pv, slot, 1);
  Group32 g[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int rl_ = it * RPI + rs;
    const uint8_t* t = rl_ < JW ? gate : up;
    g[it] = load_group<QBITS>(t, pv, int64_t(j0 + (rl_ % JW)) * H + 32 * seg);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float p = group_dot<QBITS>(g[it], xv, xsum);
    p = group_sum_last<LPR>(p);
    if (seg == LPR - 1 && it * RPI + rs < 2 * JW) s_row[wv][it * RPI + rs] = p;
  }
  __syncthreads();
  if (lane < JW) {
    const float gg = s_row[wv][lane], uu = s_row[wv][JW + lane];
    hbuf[int64_t(r) * F + j0 + lane] = silu_mul(gg, uu);
  }
}

// ------------------------------------------------- 3. down + ordered sum
// Block = RB output rows i for all k experts, one wave per expert (up to 16
// waves; more experts loop).  e_r[i] goes to LDS, then
// y[i] = fma(w_r, e_r[i], acc) for r = 0..k-1.
template <int QBITS, int LPR>
__global__ __launch_bounds__(1024) void decode_down_sum_kernel(
    PoolView pv, int H, int F, int k, int RB, const int32_t* __restrict__ slots,
    const float* __restrict__ weights, const float* __restrict__ hbuf,
    const uint32_t* __restrict__ early_out, float* __restrict__ y) {
  constexpr int RPI = 64 / LPR;
  extern __shared__ float s_e[];   // [k][RB]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int i0 = blockIdx.x * RB;
  const int seg = lane % LPR, rs = lane / LPR;
  const int nit = RB / RPI;        // 1..4
  // the flag, the first expert's slot and h are loaded together; only the
  // code loads (whose addresses need a valid slot) wait for the flag
  const uint32_t flag = *early_out;
  int slot_next = slots[wv < k ? wv : 0];
  if (flag) return;
  for (int r = wv; r < k; r += nw) {
    float xv[32], xsum;
    load_act32(hbuf + int64_t(r) * F + 32 * seg, xv, xsum);
    const int slot = slot_next;
    if (r + nw < k) slot_next = slots[r + nw];
    const uint8_t* down = tensor_base(pv, slot, 2);
    Group32 g[4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
      g[it] = load_group<QBITS>(down, pv, int64_t(i0 + (it < nit ? it : 0) * RPI + rs) * F + 32 * seg);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (it < nit) {
        float p = group_dot<QBITS>(g[it], xv, xsum);
        p = group_sum_last<LPR>(p);
        if (seg == LPR - 1) s_e[r * RB + it * RPI + rs] = p;
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RB; t += blockDim.x) {
    float acc = 0.f;
    for (int r = 0; r < k; ++r) acc = fmaf(weights[r], s_e[r * RB + t], acc);
    y[i0 + t] = acc;
  }
}

// ------------------------------------------------------------ launchers
template <int RPB>
static void router_rpb(const DecodeArgs& a, int rows, hipStream_t st) {
  const int grid = (a.E + rows - 1) / rows;
  switch (a.H) {
#define RL_CASE(NM)                                                                   \
  case 256 * NM:                                                                      \
    decode_router_kernel<RPB, NM><<<grid, 64, 0, st>>>(a.x, a.W, a.bias, a.E, a.H,    \
                                                       rows, a.logits, a.logits_out,  \
                                                       a.early_out, int(a.sticky),    \
                                                       a.clear_miss, a.clear_flag);   \
    break;
    RL_CASE(1) RL_CASE(2) RL_CASE(4) RL_CASE(8)
#undef RL_CASE
  }
}

// One row per single-wave block (E <= 1024 blocks): with two rows per wave
// the token took 0.1 us longer at E = 512.
void launch_decode_router(const DecodeArgs& a, hipStream_t st) {
  if (!a.a_out) {
    router_rpb<1>(a, 1, st);
    return;
  }
  switch (a.H) {
#define RL_CASE(NM)                                                                            \
  case 256 * NM:                                                                               \
    decode_router_residual_kernel<NM><<<a.E, 64, 0, st>>>(                                     \
        a.x_prev, a.y_prev, a.flag_prev, a.x_out, a.a_out, a.eps, a.W, a.bias, a.E, a.H,       \
        a.logits, a.logits_out, a.early_out, int(a.sticky));                                   \
    break;
    RL_CASE(1) RL_CASE(2) RL_CASE(4) RL_CASE(8)
#undef RL_CASE
  }
}

template <int N, int QBITS, int LPR>
static void gateup_l(const DecodeArgs& a, hipStream_t st) {
  decode_topk_gateup_kernel<N, QBITS, LPR><<<a.k * (a.F / 16), 256, 0, st>>>(
      a.pool, a.H, a.F, a.E, a.k, a.layer, a.n_slots, a.x, a.logits, a.residency, a.ids,
      a.weights, a.slots, a.miss_count, a.early_out, a.hbuf, int(a.sticky));
}

template <int N, int QBITS>
static void gateup_h(const DecodeArgs& a, hipStream_t st) {
  switch (a.H / 32) {
    case 8: gateup_l<N, QBITS, 8>(a, st); break;
    case 16: gateup_l<N, QBITS, 16>(a, st); break;
    case 32: gateup_l<N, QBITS, 32>(a, st); break;
    default: gateup_l<N, QBITS, 64>(a, st); break;
  }
}

template <int N>
static void gateup_n(const DecodeArgs& a, hipStream_t st) {
  if (a.qbits == 3) gateup_h<N, 3>(a, st); else gateup_h<N, 2>(a, st);
}

void launch_decode_gateup(const DecodeArgs& a, hipStream_t st) {
  if (a.mfma) {
    launch_decode_gateup_mfma(a, st);
    return;
  }
  switch (cand_per_lane(a.E)) {
    case 1: gateup_n<1>(a, st); break;
    case 2: gateup_n<2>(a, st); break;
    case 4: gateup_n<4>(a, st); break;
    case 8: gateup_n<8>(a, st); break;
    default: gateup_n<16>(a, st); break;
  }
}

template <int QBITS, int LPR>
static void launch_down(const DecodeArgs& a, hipStream_t st) {
  constexpr int RPI = 64 / LPR;
  // RB rows per block: a multiple of RPI, at most 4*RPI (the kernel's
  // per-wave iteration limit), grown towards about 256 blocks
  int RB = RPI > (8 < 4 * RPI ? 8 : 4 * RPI) ? RPI : (8 < 4 * RPI ? 8 : 4 * RPI);
  while (RB * 256 < a.H && 2 * RB <= 4 * RPI) RB <<= 1;
  const int waves = a.k < 16 ? a.k : 16;
  const size_t lds = size_t(a.k) * RB * sizeof(float);
  decode_down_sum_kernel<QBITS, LPR><<<a.H / RB, 64 * waves, lds, st>>>(
      a.pool, a.H, a.F, a.k, RB, a.slots, a.weights, a.hbuf, a.early_out, a.y);
}

template <int QBITS>
static void down_q(const DecodeArgs& a, hipStream_t st) {
  switch (a.F / 32) {
    case 1: launch_down<QBITS, 1>(a, st); break;
    case 2: launch_down<QBITS, 2>(a, st); break;
    case 4: launch_down<QBITS, 4>(a, st); break;
    case 8: launch_down<QBITS, 8>(a, st); break;
    case 16: launch_down<QBITS, 16>(a, st); break;
    case 32: launch_down<QBITS, 32>(a, st); break;
    default: launch_down<QBITS, 64>(a, st); break;
  }
}

void launch_decode_down_sum(const DecodeArgs& a, hipStream_t st) {
  if (a.mfma) {
    launch_decode_down_sum_mfma(a, st);
    return;
  }
  if (a.qbits == 3) down_q<3>(a, st); else down_q<2>(a, st);
}

}  // namespace rl
