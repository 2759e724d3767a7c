// Batched expert projections on the int8 matrix cores of gfx950
// (v_mfma_i32_16x16x64_i8), for the 2-bit block format when both expert
// dimensions are multiples of 256 ("Red Lite dev20 - batched prompt
// ingestion", "What changed": batched gate/up and down over (expert, token)
// pairs sorted by expert).
//
// Exactness.  A 2-bit weight is d * q / 32 with the integer q = (2s+1)(2c-3)
// in [-93, 93]: an int8, turned out of the code bits by one byte permute
// against a 4-entry table per group.  An activation row is scaled by a power
// of two 2^e (per row, or per 256-value block) so that |x * 2^e| < 2^30,
// rounded to the integer X, and X is written as four balanced base-256 digits
// in [-128, 127].  Each MFMA then sums int8 * int8 products exactly in int32
// over one 256-value block (|sum| < 2^22), and the block's int32 result is
// scaled by d/32 and 2^(8*(3-digit) - e) into a float32 accumulator.  Values
// with |x| >= 2^-7 max|x| are represented exactly; the rest lose nothing
// above 2^-31 max|x|.
//
// Operand layout (checked on the device): A lane l holds row l%16 and the 16
// bytes of K-slice l/16; B lane l holds column l%16 and the same K-slice; the
// output lane l holds rows 4*(l/16)+v, v < 4, of column l%16.  Inside a
// 256-value block, lane quad q and MFMA m cover K = 64q + 16m + [0, 16), and
// byte i of dword jj of the operand is K offset 4i + jj (the order in which
// (codes >> 2jj) & 0x03030303 exposes four codes).  Columns are
// 4 * token + digit.
#include "rl_common.h"
#include "rl_kernels.h"

namespace rl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMT = 12;   // tokens per token tile: 3 column tiles of 4 tokens x 4 digits

// --------------------------------------------------------------- digits
// e with max * 2^e < 2^30 (0 for a zero or non-finite max).
__device__ inline int scale_exp(float amax) {
  if (!(amax > 0.f) || !(amax < 3.0e38f)) return 0;
  int E;
  frexpf(amax, &E);
  return 30 - E;
}

// Balanced base-256 digits of X (|X| <= 2^30): digit d (0 = most significant)
// in byte 3-d, as a two's complement int8.
__device__ inline uint32_t digits_of(int X) { return (uint32_t(X) + 0x80808080u) ^ 0x80808080u; }

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
  uint32_t Z[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) Z[n] = digits_of(int(rintf(ldexpf(v[n], e))));
  const int kb = k0 >> 8, qq = (k0 & 255) >> 6, mm = (k0 & 63) >> 4;
  uint8_t* row = q + int64_t(r) * K * 4;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t b = 3 - d;   // byte of digit d in Z
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // bytes i = 0..3 <- Z[4i + jj] byte b
      const uint32_t lo = __builtin_amdgcn_perm(Z[4 + jj], Z[jj], b | ((b + 4) << 8));
      const uint32_t hi = __builtin_amdgcn_perm(Z[12 + jj], Z[8 + jj], b | ((b + 4) << 8));
      w[jj] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    *reinterpret_cast<uint4*>(row + ((kb * 4 + qq) * 4 + d) * 64 + mm * 16) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
  if ((k0 & 255) == 0) ex[int64_t(r) * (K >> 8) + kb] = e;
}

// ------------------------------------------------------------- weights
// Byte table of q = (2s+1)(2c-3) for c = 0..3: {-3m, -m, m, 3m}, m = 2s+1.
__device__ inline uint32_t lut2(uint32_t s) {
  const uint32_t m = 2u * s + 1u;
  return ((0x10100u - 259u * m) & 0xffffu) | ((m * 0x0301u) << 16);
}

__device__ inline v4i dequant_dword(uint32_t w, uint32_t lut) {
  v4i a;
  a.x = int(__builtin_amdgcn_perm(lut, lut, w & 0x03030303u));
  a.y = int(__builtin_amdgcn_perm(lut, lut, (w >> 2) & 0x03030303u));
  a.z = int(__builtin_amdgcn_perm(lut, lut, (w >> 4) & 0x03030303u));
  a.w = int(__builtin_amdgcn_perm(lut, lut, (w >> 6) & 0x03030303u));
  return a;
}

// One lane's share of a 16-row x 256-column block tile of a tensor.
struct TileCodes {
  uint4 c;       // 64 codes: K = 64q .. 64q+63 of the block, row l%16
  uint32_t s;    // group scales of groups 2q (low nibble) and 2q+1
  float dq;      // d / 32 of the lane's row
};

__device__ inline TileCodes load_tile(const uint8_t* t, const PoolView& p, int64_t blk, int q) {
  TileCodes r;
  r.c = *reinterpret_cast<const uint4*>(t + p.q + 64 * blk + 16 * q);
  r.s = t[p.s + 4 * blk + q];
  r.dq = half_bits_to_float(*reinterpret_cast<const uint16_t*>(t + p.d + 2 * blk)) * (1.f / 32.f);
  return r;
}

__device__ inline void dequant_tile(const TileCodes& tc, v4i A[4]) {
  const uint32_t l0 = lut2(tc.s & 15u), l1 = lut2(tc.s >> 4);
  A[0] = dequant_dword(tc.c.x, l0);
  A[1] = dequant_dword(tc.c.y, l0);
  A[2] = dequant_dword(tc.c.z, l1);
  A[3] = dequant_dword(tc.c.w, l1);
}

// d/32 of the output rows 4*(l/16)+v, fetched from the lanes that own them.
__device__ inline void out_row_scales(float dq, float dsc[4]) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < 4; ++v) dsc[v] = __shfl(dq, 4 * (l >> 4) + v, kWave);
}

__device__ inline v4i mfma4(const v4i A[4], const v4i B[4]) {
  v4i D = {0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 4; ++m) D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[m], B[m], D, 0, 0, 0);
  return D;
}

__device__ inline void load_b(const uint8_t* rowq, int kb, int q, int dj, v4i B[4]) {
  const int4* p = reinterpret_cast<const int4*>(rowq + ((kb * 4 + q) * 4 + dj) * 64);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int4 v = p[m];
    B[m] = v4i{v.x, v.y, v.z, v.w};
  }
}

__device__ inline int tile_bucket_m(const int32_t* tile_start, int nb, int tile) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------ gate / up
// Work item = (token tile of <= 12 tokens of one bucket, 64 rows j).  One
// wave per item: four 16-row tiles of gate and of up over all H/256 blocks;
// then h = silu(g) * u for the item's rows and tokens.
__global__ __launch_bounds__(64) void prefill_gateup_mfma_kernel(
    PoolView pv, int H, int F, int k, const uint8_t* __restrict__ xq,
    const int32_t* __restrict__ xe, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_buckets_p, const int32_t* __restrict__ n_tiles_p,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ bucket_start,
    const int32_t* __restrict__ bucket_slot, const int32_t* __restrict__ pairs,
    float* __restrict__ hbuf) {
  if (*early_out) return;
  const int l = threadIdx.x;
  const int row = l & 15, q = l >> 4, tk = (l & 15) >> 2, dj = l & 3;
  const int nb = *n_buckets_p, ntiles = *n_tiles_p;
  const int njr = F / 64, HB = H / 256;
  for (int item = blockIdx.x; item < ntiles * njr; item += gridDim.x) {
    const int tile = item / njr, jr = item % njr;
    const int b = tile_bucket_m(tile_start, nb, tile);
    const int pos0 = bucket_start[b] + (tile - tile_start[b]) * kMT;
    const int rem = bucket_start[b + 1] - pos0;
    const int nt = rem < kMT ? rem : kMT;
    const int nct = (nt + 3) >> 2;
    const int slot = bucket_slot[b];
    const uint8_t* tens[2] = {tensor_base(pv, slot, 0), tensor_base(pv, slot, 1)};
    const uint8_t* xrow[3];
    float fct[3];
    bool tok_ok[3];
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
      const int n = 4 * ct + tk;
      tok_ok[ct] = n < nt;
      const int t = tok_ok[ct] ? pairs[pos0 + n] / k : 0;
      xrow[ct] = xq + int64_t(t) * H * 4;
      fct[ct] = ldexpf(1.f, 8 * (3 - dj) - (tok_ok[ct] ? xe[int64_t(t) * HB] : 0));
    }
    float acc[2][4][3][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[a][rt][ct][v] = 0.f;
    for (int kb = 0; kb < HB; ++kb) {
      TileCodes tc[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          tc[a][rt] = load_tile(tens[a], pv, int64_t(jr * 64 + rt * 16 + row) * HB + kb, q);
      v4i B[3][4];
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        if (ct < nct && tok_ok[ct]) {
          load_b(xrow[ct], kb, q, dj, B[ct]);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) B[ct][m] = v4i{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          v4i A[4];
          dequant_tile(tc[a][rt], A);
          float dsc[4];
          out_row_scales(tc[a][rt].dq, dsc);
#pragma unroll
          for (int ct = 0; ct < 3; ++ct) {
            if (ct < nct) {
              const v4i D = mfma4(A, B[ct]);
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[a][rt][ct][v] = fmaf(dsc[v], float(D[v]), acc[a][rt][ct][v]);
            }
          }
        }
      }
    }
    // combine the 4 digit columns of each token and apply SwiGLU
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        if (ct < nct) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float g = acc[0][rt][ct][v] * fct[ct];
            float u = acc[1][rt][ct][v] * fct[ct];
            g += __shfl_xor(g, 1, kWave);
            g += __shfl_xor(g, 2, kWave);
            u += __shfl_xor(u, 1, kWave);
            u += __shfl_xor(u, 2, kWave);
            h[v] = silu_mul(g, u);
          }
          if (dj == 0 && tok_ok[ct]) {
            const int n = 4 * ct + tk;
            *reinterpret_cast<float4*>(hbuf + int64_t(pos0 + n) * F + jr * 64 + rt * 16 + 4 * q) =
                make_float4(h[0], h[1], h[2], h[3]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Work item = (token tile, 64 rows i).  B = the tile's h rows as digits with
// one exponent per (pair, 256-value block).  Output rows go to ebuf row p.
__global__ __launch_bounds__(64) void prefill_down_mfma_kernel(
    PoolView pv, int H, int F, const uint8_t* __restrict__ hq, const int32_t* __restrict__ he,
    const uint32_t* __restrict__ early_out, const int32_t* __restrict__ n_buckets_p,
    const int32_t* __restrict__ n_tiles_p, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ bucket_start, const int32_t* __restrict__ bucket_slot,
    const int32_t* __restrict__ pairs, float* __restrict__ ebuf) {
  if (*early_out) return;
  const int l = threadIdx.x;
  const int row = l & 15, q = l >> 4, tk = (l & 15) >> 2, dj = l & 3;
  const int nb = *n_buckets_p, ntiles = *n_tiles_p;
  const int nir = H / 64, FB = F / 256;
  for (int item = blockIdx.x; item < ntiles * nir; item += gridDim.x) {
    const int tile = item / nir, ir = item % nir;
    const int b = tile_bucket_m(tile_start, nb, tile);
    const int pos0 = bucket_start[b] + (tile - tile_start[b]) * kMT;
    const int rem = bucket_start[b + 1] - pos0;
    const int nt = rem < kMT ? rem : kMT;
    const int nct = (nt + 3) >> 2;
    const uint8_t* down = tensor_base(pv, bucket_slot[b], 2);
    bool tok_ok[3];
    int pos[3];
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
      const int n = 4 * ct + tk;
      tok_ok[ct] = n < nt;
      pos[ct] = tok_ok[ct] ? pos0 + n : pos0;
    }
    float acc[4][3][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rt][ct][v] = 0.f;
    for (int kb = 0; kb < FB; ++kb) {
      TileCodes tc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        tc[rt] = load_tile(down, pv, int64_t(ir * 64 + rt * 16 + row) * FB + kb, q);
      v4i B[3][4];
      float fct[3];
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        if (ct < nct && tok_ok[ct]) {
          load_b(hq + int64_t(pos[ct]) * F * 4, kb, q, dj, B[ct]);
          fct[ct] = ldexpf(1.f, 8 * (3 - dj) - he[int64_t(pos[ct]) * FB + kb]);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) B[ct][m] = v4i{0, 0, 0, 0};
          fct[ct] = 0.f;
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        v4i A[4];
        dequant_tile(tc[rt], A);
        float dsc[4];
        out_row_scales(tc[rt].dq, dsc);
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
          if (ct < nct) {
            const v4i D = mfma4(A, B[ct]);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[rt][ct][v] = fmaf(dsc[v] * fct[ct], float(D[v]), acc[rt][ct][v]);
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        if (ct < nct) {
          float e[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float s = acc[rt][ct][v];
            s += __shfl_xor(s, 1, kWave);
            s += __shfl_xor(s, 2, kWave);
            e[v] = s;
          }
          if (dj == 0 && tok_ok[ct]) {
            const int p = pairs[pos[ct]];
            *reinterpret_cast<float4*>(ebuf + int64_t(p) * H + ir * 64 + rt * 16 + 4 * q) =
                make_float4(e[0], e[1], e[2], e[3]);
          }
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

void launch_prefill_gateup_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  prefill_gateup_mfma_kernel<<<2048, 64, 0, st>>>(
      a.pool, a.H, a.F, a.k, a.xq, a.xe, a.early_out, p.n_buckets, p.n_tiles, p.tile_start,
      p.bucket_start, p.bucket_slot, p.pairs, a.hbuf);
}

void launch_quantize_h(const PrefillArgs& a, hipStream_t st) {
  const int rpb = 256 / (a.F / 16);
  const int R = a.T * a.k;
  quantize_rows_kernel<false><<<(R + rpb - 1) / rpb, 256, 0, st>>>(a.hbuf, R, a.F, a.hq, a.he,
                                                                    a.early_out);
}

void launch_prefill_down_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  prefill_down_mfma_kernel<<<2048, 64, 0, st>>>(
      a.pool, a.H, a.F, a.hq, a.he, a.early_out, p.n_buckets, p.n_tiles, p.tile_start,
      p.bucket_start, p.bucket_slot, p.pairs, a.ebuf);
}

}  // namespace rl
