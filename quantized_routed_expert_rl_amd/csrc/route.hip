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
#include "rl_select.h"

namespace rl {

// ------------------------------------------------------- T > 1: GEMM
// logits[t][e] = fl32(sum_i W[e][i] x[t][i] + b[e]) on the float64 matrix
// cores (v_mfma_f64_16x16x4f64; A lane l: row l%16, K index l/16; B lane l:
// column l%16, K index l/16; output lane l, v: row l/16 + 4v, column l%16).
// Block = 32 tokens x 32 experts, one 16x16 tile per wave pair: waves w and
// w + 4 take the two halves of K, so two waves share each SIMD and hide each
// other's LDS and memory latency, and the halves are added in float64 at the
// end.  Each half runs in 64-value chunks staged through LDS (double buffer;
// a chunk's float4 loads are issued two chunks before it is staged), so each
// x and W value is read from memory once per block.  Inside each 16-value
// group g of a chunk, MFMA step 4g+i of lane quad kq takes K index
// 16g + 4kq + i for both operands: one float4 LDS read per lane per group.
// A chunk's operands are read into one of two register sets right after the
// barrier that publishes it, while the previous chunk's MFMAs still run, so
// the matrix core does not wait for LDS after each barrier.  Four
// accumulation chains (one per group) keep it busy; summed in float64 at the
// end.
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kRgStride = 68;   // floats per staged row: 64 + 4 keeps float4 reads conflict-free

__global__ __launch_bounds__(512) void route_gemm_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
    int T, int E, int H, float* __restrict__ logits, float* __restrict__ logits_out,
    uint32_t* miss_count, uint32_t* early_out) {
  __shared__ __align__(16) float s_a[2][2][32 * kRgStride];   // [K half][buffer] tokens
  __shared__ __align__(16) float s_b[2][2][32 * kRgStride];   // [K half][buffer] experts
  __shared__ v4d s_part[4][64];                               // upper half's sums
  const int tid = threadIdx.x, l = tid & 63, wv = (tid >> 6) & 3, kh = tid >> 8;
  const int tb = blockIdx.y * 32, eb = blockIdx.x * 32;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    *miss_count = 0u;
    *early_out = 0u;
  }
  // staging: thread copies row (tid%256)/8, floats 8*(tid%8) .. +7 of its
  // half's chunk for both operands (two float4 each)
  const int st = tid & 255, sr = st >> 3, sc = 8 * (st & 7);
  const int nch = H / 128;                                     // chunks per K half
  const int k0 = kh * (H / 2);
  const bool va = tb + sr < T, vb = eb + sr < E;
  const float* ga = x + int64_t(va ? tb + sr : 0) * H + k0 + sc;
  const float* gb = W + int64_t(vb ? eb + sr : 0) * H + k0 + sc;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  // two chunks in flight in registers: a chunk's loads are issued two chunks
  // before it is staged, since one chunk of MFMAs is shorter than a load's
  // round trip
  float4 pa0, pa1, pb0, pb1, qa0, qa1, qb0, qb1;
  auto fetch = [&](int c, float4& a0, float4& a1, float4& b0, float4& b1)
      __attribute__((always_inline)) {
    const int off = c * 64;
    a0 = va ? *reinterpret_cast<const float4*>(ga + off) : z4;
    a1 = va ? *reinterpret_cast<const float4*>(ga + off + 4) : z4;
    b0 = vb ? *reinterpret_cast<const float4*>(gb + off) : z4;
    b1 = vb ? *reinterpret_cast<const float4*>(gb + off + 4) : z4;
  };
  fetch(0, pa0, pa1, pb0, pb1);
  fetch(1, qa0, qa1, qb0, qb1);
  const int r = l & 15, kq = l >> 4;
  const int ra = (wv >> 1) * 16 + r, rb = (wv & 1) * 16 + r;   // staged rows this lane reads
  v4d acc4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc4[u] = v4d{0.0, 0.0, 0.0, 0.0};
  auto stage = [&](int ch, const float4& a0, const float4& a1, const float4& b0, const float4& b1)
      __attribute__((always_inline)) {
    float* sa = s_a[kh][ch & 1];
    float* sb = s_b[kh][ch & 1];
    *reinterpret_cast<float4*>(&sa[sr * kRgStride + sc]) = a0;
    *reinterpret_cast<float4*>(&sa[sr * kRgStride + sc + 4]) = a1;
    *reinterpret_cast<float4*>(&sb[sr * kRgStride + sc]) = b0;
    *reinterpret_cast<float4*>(&sb[sr * kRgStride + sc + 4]) = b1;
  };
  // operand registers of one chunk: group g of A and B
  float4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3, ya0, ya1, ya2, ya3, yb0, yb1, yb2, yb3;
  auto readop = [&](int ch, float4& a0, float4& a1, float4& a2, float4& a3, float4& b0, float4& b1,
                    float4& b2, float4& b3) __attribute__((always_inline)) {
    const float* sa = s_a[kh][ch & 1] + ra * kRgStride + 4 * kq;
    const float* sb = s_b[kh][ch & 1] + rb * kRgStride + 4 * kq;
    a0 = *reinterpret_cast<const float4*>(sa);
    a1 = *reinterpret_cast<const float4*>(sa + 16);
    a2 = *reinterpret_cast<const float4*>(sa + 32);
    a3 = *reinterpret_cast<const float4*>(sa + 48);
    b0 = *reinterpret_cast<const float4*>(sb);
    b1 = *reinterpret_cast<const float4*>(sb + 16);
    b2 = *reinterpret_cast<const float4*>(sb + 32);
    b3 = *reinterpret_cast<const float4*>(sb + 48);
  };
  auto mma = [&](const float4& a0, const float4& a1, const float4& a2, const float4& a3,
                 const float4& b0, const float4& b1, const float4& b2, const float4& b3)
      __attribute__((always_inline)) {
#define RG_STEP(c)                                                                                  \
    acc4[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a0.c), double(b0.c), acc4[0], 0, 0, 0); \
    acc4[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a1.c), double(b1.c), acc4[1], 0, 0, 0); \
    acc4[2] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a2.c), double(b2.c), acc4[2], 0, 0, 0); \
    acc4[3] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a3.c), double(b3.c), acc4[3], 0, 0, 0);
    RG_STEP(x) RG_STEP(y) RG_STEP(z) RG_STEP(w)
#undef RG_STEP
  };
  // chunk ch's MFMAs are issued around the barrier that publishes chunk
  // ch+1, and chunk ch+1's operands are read while they run.  nch = H/128 is
  // even (H is a multiple of 256), so the register sets alternate in a fixed
  // order.
  stage(0, pa0, pa1, pb0, pb1);
  if (2 < nch) fetch(2, pa0, pa1, pb0, pb1);
  __syncthreads();
  readop(0, xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
  for (int ch = 0; ch < nch; ch += 2) {
    // even chunk ch: operands in x; chunk ch+1's staged values in q
    stage(ch + 1, qa0, qa1, qb0, qb1);
    if (ch + 3 < nch) fetch(ch + 3, qa0, qa1, qb0, qb1);
    mma(xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
    __syncthreads();
    readop(ch + 1, ya0, ya1, ya2, ya3, yb0, yb1, yb2, yb3);
    // odd chunk ch+1: operands in y; chunk ch+2's staged values in p
    if (ch + 2 < nch) {
      stage(ch + 2, pa0, pa1, pb0, pb1);
      if (ch + 4 < nch) fetch(ch + 4, pa0, pa1, pb0, pb1);
    }
    mma(ya0, ya1, ya2, ya3, yb0, yb1, yb2, yb3);
    __syncthreads();
    if (ch + 2 < nch) readop(ch + 2, xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
  }
  v4d acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  if (kh == 1) s_part[wv][l] = acc;
  __syncthreads();
  if (kh == 1) return;
  acc += s_part[wv][l];
  const int t0 = tb + (wv >> 1) * 16, e0 = eb + (wv & 1) * 16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + kq + 4 * v, e = e0 + r;
    if (t < T && e < E) {
      double sum = v == 0 ? acc.x : v == 1 ? acc.y : v == 2 ? acc.z : acc.w;
      if (bias) sum += double(bias[e]);
      const float lg = float(sum);
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
  __shared__ __align__(16) TopkLds s_tk;
  __shared__ int sel_ids[32];
  __shared__ float sel_lg[32];
  __shared__ int sel_res[32];
  const int t = blockIdx.x;
  wave_topk<N>(logits + int64_t(t) * E, E, k, residency + int64_t(layer) * E, s_tk, sel_ids,
               sel_lg, sel_res);
  const int miss = finish_token(sel_ids, sel_lg, sel_res, k, E, n_slots, ids + int64_t(t) * k,
                                weights + int64_t(t) * k, slots + int64_t(t) * k);
  if ((threadIdx.x & 63) == 0 && miss > 0) {
    atomicAdd(miss_count, uint32_t(miss));
    atomicOr(early_out, 1u);
  }
}

// ------------------------------------------------------------ launchers
template <int N>
static void launch_topk_n(const RouteArgs& a, hipStream_t st) {
  route_topk_kernel<N><<<a.T, 64, 0, st>>>(a.logits, a.T, a.E, a.k, a.layer, a.n_slots,
                                           a.residency, a.ids, a.weights, a.slots,
                                           a.miss_count, a.early_out);
}

int cand_per_lane(int E) {
  int n = 1;
  while (64 * n < E) n <<= 1;
  return n;
}

// One token: the decode router GEMV (one wave per row, float64 sums, 4 us at
// E = 512, H = 2048) instead of the GEMM, whose 32-token tiles would be 1/32
// used (26 us).
void launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.T == 1) {
    DecodeArgs da;
    da.x = a.x;
    da.W = a.W;
    da.bias = a.bias;
    da.E = a.E;
    da.H = a.H;
    da.logits = a.logits;
    da.logits_out = a.logits_out;
    da.early_out = a.early_out;
    da.sticky = false;
    da.clear_miss = a.miss_count;
    da.clear_flag = a.early_out;
    launch_decode_router(da, st);
  } else {
    dim3 grid((a.E + 31) / 32, (a.T + 31) / 32);
    route_gemm_kernel<<<grid, 512, 0, st>>>(a.x, a.W, a.bias, a.T, a.E, a.H, a.logits,
                                            a.logits_out, a.miss_count, a.early_out);
  }
  switch (cand_per_lane(a.E)) {
    case 1: launch_topk_n<1>(a, st); break;
    case 2: launch_topk_n<2>(a, st); break;
    case 4: launch_topk_n<4>(a, st); break;
    case 8: launch_topk_n<8>(a, st); break;
    default: launch_topk_n<16>(a, st); break;
  }
}

}  // namespace rl
