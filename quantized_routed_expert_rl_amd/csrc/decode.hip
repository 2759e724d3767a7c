// Single-token expert kernels: gate/up GEMVs with SwiGLU, then the down
// GEMVs fused with the rank-ordered weighted sum ("Red Lite dev21",
// "What changed": the expert kernels read the slot table and weights the
// router wrote; "Red Lite dev23", "What changed": each returns at once when
// the early-out flag is set; "Red Lite dev20", "What changed": a token's
// experts are summed in router selection order).
//
// Lane mapping.  A lane owns one 32-value group of a row: 8 bytes of codes,
// one group scale, one block scale, and the 32 matching activations held in
// registers for every row the wave visits.  A row of C values is C/32 lanes
// (the notes found 8 lanes of 64 values best for the 512-column down rows on
// a 32-wide SIMD, "Red Lite dev38", "Changes"; on a 64-wide wave the same
// byte count per lane gives 16 lanes of 32 values), and a butterfly over
// those lanes finishes the row.
#include "rl_common.h"
#include "rl_kernels.h"

namespace rl {

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

// Each wave computes JW consecutive rows j of one expert for both gate and
// up (2*JW rows), then h_j = silu(g_j) * u_j.
template <int QBITS, int LPR>
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    PoolView pv, int H, int F, int k, const float* __restrict__ x,
    const int32_t* __restrict__ slots, const uint32_t* __restrict__ early_out,
    float* __restrict__ hbuf) {
  if (*early_out) return;
  constexpr int RPI = 64 / LPR;     // rows per wave iteration
  constexpr int JW = 4;             // j values per wave
  constexpr int NIT = 2 * JW / RPI > 0 ? 2 * JW / RPI : 1;
  __shared__ float s_row[4][2 * JW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + wv;
  const int per_expert = F / JW;
  const bool active = gw < k * per_expert;
  const int r = gw / per_expert;
  const int j0 = (gw % per_expert) * JW;
  const int seg = lane % LPR, rs = lane / LPR;
  if (active) {
    float xv[32], xsum;
    load_act32(x + 32 * seg, xv, xsum);
    const int slot = slots[r];
    const uint8_t* gate = tensor_base(pv, slot, 0);
    const uint8_t* up = tensor_base(pv, slot, 1);
    Group32 g[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rl_ = it * RPI + rs;
      const uint8_t* t = rl_ < JW ? gate : up;
      const int j = j0 + (rl_ % JW);
      g[it] = load_group<QBITS>(t, pv, int64_t(j) * H + 32 * seg);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float p = group_dot<QBITS>(g[it], xv, xsum);
      p = wave_sum_width(p, LPR);
      if (seg == 0 && it * RPI + rs < 2 * JW) s_row[wv][it * RPI + rs] = p;
    }
  }
  __syncthreads();
  if (active && lane < JW) {
    const float gg = s_row[wv][lane], uu = s_row[wv][JW + lane];
    hbuf[int64_t(r) * F + j0 + lane] = silu_mul(gg, uu);
  }
}

// Block = RB output rows i for all k experts; wave w takes experts w, w+4...
// e_r[i] goes to LDS, then y[i] = fma(w_r, e_r[i], acc) for r = 0..k-1.
template <int QBITS, int LPR>
__global__ __launch_bounds__(256) void decode_down_sum_kernel(
    PoolView pv, int H, int F, int k, int RB, const int32_t* __restrict__ slots,
    const float* __restrict__ weights, const float* __restrict__ hbuf,
    const uint32_t* __restrict__ early_out, float* __restrict__ y) {
  if (*early_out) return;
  constexpr int RPI = 64 / LPR;
  extern __shared__ float s_e[];   // [k][RB]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i0 = blockIdx.x * RB;
  const int seg = lane % LPR, rs = lane / LPR;
  const int nit = RB / RPI;
  for (int r = wv; r < k; r += 4) {
    float xv[32], xsum;
    load_act32(hbuf + int64_t(r) * F + 32 * seg, xv, xsum);
    const uint8_t* down = tensor_base(pv, slots[r], 2);
    for (int it0 = 0; it0 < nit; it0 += 2) {
      Group32 g[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = it0 + u < nit ? it0 + u : it0;
        g[u] = load_group<QBITS>(down, pv, int64_t(i0 + it * RPI + rs) * F + 32 * seg);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (it0 + u < nit) {
          float p = group_dot<QBITS>(g[u], xv, xsum);
          p = wave_sum_width(p, LPR);
          if (seg == 0) s_e[r * RB + (it0 + u) * RPI + rs] = p;
        }
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RB; t += 256) {
    float acc = 0.f;
    for (int r = 0; r < k; ++r) acc = fmaf(weights[r], s_e[r * RB + t], acc);
    y[i0 + t] = acc;
  }
}

template <int QBITS, int LPR>
static void launch_gateup(const DecodeArgs& a, hipStream_t st) {
  const int waves = a.k * (a.F / 4);
  decode_gateup_kernel<QBITS, LPR><<<(waves + 3) / 4, 256, 0, st>>>(
      a.pool, a.H, a.F, a.k, a.x, a.slots, a.early_out, a.hbuf);
}

template <int QBITS, int LPR>
static void launch_down(const DecodeArgs& a, hipStream_t st) {
  constexpr int RPI = 64 / LPR;
  int RB = RPI > 8 ? RPI : 8;
  while (RB * 256 < a.H && RB < 64) RB <<= 1;   // about 256 blocks or fewer
  if (RB > a.H) RB = a.H;
  const size_t lds = size_t(a.k) * RB * sizeof(float);
  decode_down_sum_kernel<QBITS, LPR><<<a.H / RB, 256, lds, st>>>(
      a.pool, a.H, a.F, a.k, RB, a.slots, a.weights, a.hbuf, a.early_out, a.y);
}

template <int QBITS>
static void gateup_q(const DecodeArgs& a, hipStream_t st) {
  switch (a.H / 32) {
    case 8: launch_gateup<QBITS, 8>(a, st); break;
    case 16: launch_gateup<QBITS, 16>(a, st); break;
    case 32: launch_gateup<QBITS, 32>(a, st); break;
    default: launch_gateup<QBITS, 64>(a, st); break;
  }
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

void launch_decode_gateup(const DecodeArgs& a, hipStream_t st) {
  if (a.qbits == 3) gateup_q<3>(a, st); else gateup_q<2>(a, st);
}

void launch_decode_down_sum(const DecodeArgs& a, hipStream_t st) {
  if (a.qbits == 3) down_q<3>(a, st); else down_q<2>(a, st);
}

}  // namespace rl
