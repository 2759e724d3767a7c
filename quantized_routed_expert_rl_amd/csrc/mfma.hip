// Batched expert projections on the int8 matrix cores of gfx950
// (v_mfma_i32_16x16x64_i8), for 2-bit and 3-bit block weights when both
// expert dimensions are multiples of 256 ("Red Lite dev20 - batched prompt
// ingestion", "What changed": batched gate/up and down over (expert, token)
// pairs sorted by expert).
//
// The int8 operands and their exactness are described in rl_mfma.h; columns
// of the B operand are 4 * token + digit.
#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_mfma.h"

namespace rl {

constexpr int kMT = 12;   // tokens per token tile: 3 column tiles of 4 tokens x 4 digits

// --------------------------------------------------------------- digits
// Rows of K float32 values -> operand-ready digit bytes.  Row r goes to
// q + r*K*4; the 16-byte chunk of (block kb, quad qq, digit d) starts at
// ((kb*4 + qq)*4 + d)*64 and holds MFMA m's 16 bytes at m*16.  Exponents:
// ex[r*(K/256) + kb].  PER_ROW: one exponent for the whole row.
// Each thread takes 16 consecutive values.
template <bool PER_ROW>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const float* __restrict__ src, int R, int K, uint8_t* __restrict__ q,
    int32_t* __restrict__ ex, const uint32_t* __restrict__ early_out) {
  if (*early_out) return;
  __shared__ uint32_t s_max[16];
  const int lpr = K / 16;                       // threads per row (<= 256)
  const int rpb = 256 / lpr;                    // rows per block
  const int tid = threadIdx.x;
  const int r = blockIdx.x * rpb + tid / lpr;
  const int lr = tid % lpr;
  const bool active = (tid / lpr) < rpb && r < R;
  const int k0 = 16 * lr;
  float v[16];
  float amax = 0.f;
  if (active) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 f = *reinterpret_cast<const float4*>(src + int64_t(r) * K + k0 + 4 * u);
      v[4 * u + 0] = f.x;
      v[4 * u + 1] = f.y;
      v[4 * u + 2] = f.z;
      v[4 * u + 3] = f.w;
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) amax = fmaxf(amax, fabsf(v[n]));
  } else {
#pragma unroll
    for (int n = 0; n < 16; ++n) v[n] = 0.f;
  }
  // group: the row (PER_ROW) or the row's 256-value block
  const int grp = PER_ROW ? (tid / lpr) : (tid / 16);
  if (tid < 16) s_max[tid] = 0u;
  __syncthreads();
  if (active) atomicMax(&s_max[grp], __float_as_uint(amax));
  __syncthreads();
  if (!active) return;
  const int e = scale_exp(__uint_as_float(s_max[grp]));
  uint4 ch[4];
  digit_chunks(v, e, ch);
  const int kb = k0 >> 8, qq = (k0 & 255) >> 6, mm = (k0 & 63) >> 4;
  uint8_t* row = q + int64_t(r) * K * 4 + kb * 1024;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    *reinterpret_cast<uint4*>(row + digit_chunk_offset(qq, d, mm)) = ch[d];
  if ((k0 & 255) == 0) ex[int64_t(r) * (K >> 8) + kb] = e;
}

// -------------------------------------------------- batched projections
// One kernel for both projections.  Work item = (token tile of <= 12 tokens
// of one bucket, 128 rows j of gate and up) or (token tile, 256 rows i of
// down).  Block = 8 waves over the same token tile; wave w owns two 16-row
// tiles: gate and up of rows j0+16w (gate/up), or rows i0+32w and i0+32w+16
// (down).  K runs over 256-value blocks: the tile's digit operands for block
// kb+1 are copied to LDS (double buffer) and the wave's codes for kb+1 are
// loaded while block kb computes.  The three 4-token column tiles give three
// independent MFMA chains per row tile, issued interleaved.
constexpr int kProjWaves = 8;

template <bool GATEUP, int QBITS>
__global__ __launch_bounds__(512) void prefill_proj_mfma_kernel(
    PoolView pv, int H, int F, int k, const uint8_t* __restrict__ aq,
    const int32_t* __restrict__ ae, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_tiles_p, const int32_t* __restrict__ tile_bucket,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ bucket_start,
    const int32_t* __restrict__ bucket_slot, const int32_t* __restrict__ pairs,
    float* __restrict__ out) {
  if (*early_out) return;
  __shared__ __align__(16) uint8_t s_b[2][kMT * 1024];
  __shared__ int s_row[kMT];            // operand row of each token slot
  __shared__ __align__(16) float s_rs[kProjWaves][2][16];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int row = l & 15, q = l >> 4, tk = (l & 15) >> 2, dj = l & 3;
  const int K = GATEUP ? H : F;          // reduction length
  const int NR = GATEUP ? F : H;         // output rows
  const int KB = K / 256;
  const int rows_per_item = GATEUP ? 128 : 256;
  const int nri = NR / rows_per_item;
  const int ntiles = *n_tiles_p;
  for (int item = blockIdx.x; item < ntiles * nri; item += gridDim.x) {
    const int tile = item / nri, ri = item % nri;
    const int b = tile_bucket[tile];
    const int pos0 = bucket_start[b] + (tile - tile_start[b]) * kMT;
    const int rem = bucket_start[b + 1] - pos0;
    const int nt = rem < kMT ? rem : kMT;
    const int slot = bucket_slot[b];
    __syncthreads();                     // previous item done with s_b, s_row
    if (tid < nt) s_row[tid] = GATEUP ? pairs[pos0 + tid] / k : pos0 + tid;
    __syncthreads();
    const uint8_t* t0p = tensor_base(pv, slot, GATEUP ? 0 : 2);
    const uint8_t* t1p = tensor_base(pv, slot, GATEUP ? 1 : 2);
    const int r00 = GATEUP ? ri * 128 + 16 * w : ri * 256 + 32 * w;
    const int r01 = GATEUP ? r00 : r00 + 16;
    const int64_t blk0 = int64_t(r00 + row) * KB, blk1 = int64_t(r01 + row) * KB;
    bool tok_ok[3];
    int orow[3];
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
      tok_ok[ct] = 4 * ct + tk < nt;
      orow[ct] = s_row[tok_ok[ct] ? 4 * ct + tk : 0];
    }
    // operand copy: 12 slots x 1 KB = 768 chunks of 16 B; thread takes chunk
    // tid and tid+512 (the second only for tid < 256); empty slots get zeros
    const int c0 = tid, c1 = tid + 512;
    const uint32_t m0 = c0 < nt * 64 ? ~0u : 0u;
    const uint32_t m1 = (c1 < 768 && c1 < nt * 64) ? ~0u : 0u;
    const uint8_t* src0 = aq + int64_t(s_row[m0 ? (c0 >> 6) : 0]) * K * 4 + (c0 & 63) * 16;
    const uint8_t* src1 = aq + int64_t(s_row[m1 ? (c1 >> 6) : 0]) * K * 4 + (c1 & 63) * 16;
    float acc[2][3][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][ct][v] = 0.f;
    uint4 cr0, cr1;
    TileCodes ta0, ta1, tb0, tb1;        // double-buffered codes of the two tiles
    cr0 = *reinterpret_cast<const uint4*>(src0);
    cr1 = *reinterpret_cast<const uint4*>(src1);
    ta0 = load_tile<QBITS>(t0p, pv, blk0, q);
    ta1 = load_tile<QBITS>(t1p, pv, blk1, q);
    *reinterpret_cast<uint4*>(&s_b[0][c0 * 16]) =
        make_uint4(cr0.x & m0, cr0.y & m0, cr0.z & m0, cr0.w & m0);
    if (c1 < 768)
      *reinterpret_cast<uint4*>(&s_b[0][c1 * 16]) =
          make_uint4(cr1.x & m1, cr1.y & m1, cr1.z & m1, cr1.w & m1);
    __syncthreads();
    for (int kb = 0; kb < KB; ++kb) {
      const int buf = kb & 1;
      const bool more = kb + 1 < KB;
      if (more) {
        cr0 = *reinterpret_cast<const uint4*>(src0 + (kb + 1) * 1024);
        cr1 = *reinterpret_cast<const uint4*>(src1 + (kb + 1) * 1024);
        tb0 = load_tile<QBITS>(t0p, pv, blk0 + kb + 1, q);
        tb1 = load_tile<QBITS>(t1p, pv, blk1 + kb + 1, q);
      }
      // d/32 of output rows 4q+v of both tiles, through LDS
      if (q == 0) {
        s_rs[w][0][row] = tile_dq<QBITS>(ta0);
        s_rs[w][1][row] = tile_dq<QBITS>(ta1);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const float4 ds0 = *reinterpret_cast<const float4*>(&s_rs[w][0][4 * q]);
      const float4 ds1 = *reinterpret_cast<const float4*>(&s_rs[w][1][4 * q]);
      v4i A0[4], A1[4], G0[4], G1[4];
      dequant_tile(ta0, A0);
      dequant_tile(ta1, A1);
      if (QBITS == 3) {                  // third-bit operands
        dequant_tile_hi(ta0, G0);
        dequant_tile_hi(ta1, G1);
      }
      v4i D0[3], D1[3];
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        D0[ct] = v4i{0, 0, 0, 0};
        D1[ct] = v4i{0, 0, 0, 0};
      }
      const uint8_t* bb = &s_b[buf][tk * 1024 + q * 256 + dj * 64];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v4i Bm[3];
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
          const int4 v = *reinterpret_cast<const int4*>(bb + ct * 4096 + m * 16);
          Bm[ct] = v4i{v.x, v.y, v.z, v.w};
        }
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
          D0[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[m], Bm[ct], D0[ct], 0, 0, 0);
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
          D1[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[m], Bm[ct], D1[ct], 0, 0, 0);
        if (QBITS == 3) {
#pragma unroll
          for (int ct = 0; ct < 3; ++ct)
            D0[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(G0[m], Bm[ct], D0[ct], 0, 0, 0);
#pragma unroll
          for (int ct = 0; ct < 3; ++ct)
            D1[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(G1[m], Bm[ct], D1[ct], 0, 0, 0);
        }
      }
      float f[3] = {1.f, 1.f, 1.f};
      if (!GATEUP) {
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) f[ct] = ldexpf(1.f, 8 * (3 - dj) - ae[int64_t(orow[ct]) * KB + kb]);
      }
      const float s0[4] = {ds0.x, ds0.y, ds0.z, ds0.w}, s1[4] = {ds1.x, ds1.y, ds1.z, ds1.w};
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[0][ct][v] = fmaf(s0[v] * f[ct], float(D0[ct][v]), acc[0][ct][v]);
          acc[1][ct][v] = fmaf(s1[v] * f[ct], float(D1[ct][v]), acc[1][ct][v]);
        }
      if (more) {
        *reinterpret_cast<uint4*>(&s_b[buf ^ 1][c0 * 16]) =
            make_uint4(cr0.x & m0, cr0.y & m0, cr0.z & m0, cr0.w & m0);
        if (c1 < 768)
          *reinterpret_cast<uint4*>(&s_b[buf ^ 1][c1 * 16]) =
              make_uint4(cr1.x & m1, cr1.y & m1, cr1.z & m1, cr1.w & m1);
        ta0 = tb0;
        ta1 = tb1;
      }
      __syncthreads();
    }
    // combine each token's 4 digit columns; store
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
      const int n = 4 * ct + tk;
      if (GATEUP) {
        const float fx = ldexpf(1.f, 8 * (3 - dj) - (tok_ok[ct] ? ae[int64_t(orow[ct]) * KB] : 0));
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float g = acc[0][ct][v] * fx, u = acc[1][ct][v] * fx;
          g += __shfl_xor(g, 1, kWave);
          g += __shfl_xor(g, 2, kWave);
          u += __shfl_xor(u, 1, kWave);
          u += __shfl_xor(u, 2, kWave);
          h[v] = silu_mul(g, u);
        }
        if (dj == 0 && tok_ok[ct])
          *reinterpret_cast<float4*>(out + int64_t(pos0 + n) * F + r00 + 4 * q) =
              make_float4(h[0], h[1], h[2], h[3]);
      } else {
        const int p = tok_ok[ct] ? pairs[pos0 + n] : 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float e[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float sv = acc[u][ct][v];
            sv += __shfl_xor(sv, 1, kWave);
            sv += __shfl_xor(sv, 2, kWave);
            e[v] = sv;
          }
          if (dj == 0 && tok_ok[ct])
            *reinterpret_cast<float4*>(out + int64_t(p) * H + (u ? r01 : r00) + 4 * q) =
                make_float4(e[0], e[1], e[2], e[3]);
        }
      }
    }
  }
}

// ------------------------------------------------------------ launchers
void launch_quantize_x(const PrefillArgs& a, hipStream_t st) {
  const int rpb = 256 / (a.H / 16);
  quantize_rows_kernel<true><<<(a.T + rpb - 1) / rpb, 256, 0, st>>>(a.x, a.T, a.H, a.xq, a.xe,
                                                                     a.early_out);
}

void launch_quantize_h(const PrefillArgs& a, hipStream_t st) {
  const int rpb = 256 / (a.F / 16);
  const int R = a.T * a.k;
  quantize_rows_kernel<false><<<(R + rpb - 1) / rpb, 256, 0, st>>>(a.hbuf, R, a.F, a.hq, a.he,
                                                                    a.early_out);
}

void launch_prefill_gateup_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  auto kern = a.qbits == 3 ? prefill_proj_mfma_kernel<true, 3> : prefill_proj_mfma_kernel<true, 2>;
  kern<<<512, 512, 0, st>>>(
      a.pool, a.H, a.F, a.k, a.xq, a.xe, a.early_out, p.n_tiles, p.tile_bucket, p.tile_start,
      p.bucket_start, p.bucket_slot, p.pairs, a.hbuf);
}

void launch_prefill_down_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  auto kern = a.qbits == 3 ? prefill_proj_mfma_kernel<false, 3> : prefill_proj_mfma_kernel<false, 2>;
  kern<<<512, 512, 0, st>>>(
      a.pool, a.H, a.F, a.k, a.hq, a.he, a.early_out, p.n_tiles, p.tile_bucket, p.tile_start,
      p.bucket_start, p.bucket_slot, p.pairs, a.ebuf);
}

}  // namespace rl
