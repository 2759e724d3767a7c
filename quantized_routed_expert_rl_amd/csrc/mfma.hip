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

__device__ inline void wave_lds_sync32() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

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

// ------------------------------------ batched projections, 32x32 tiles
// v_mfma_i32_32x32x32_i8 (checked on the device): A lane l holds row l%32
// and 16 bytes of K-half l/32, B lane l column l%32 and the same K-half,
// pairing byte for byte; output lane l, v is row 8(v/4) + 4(l/32) + v%4,
// column l%32.  A 256-value block takes 8 MFMAs; MFMA n pairs the 16-value
// runs n (half 0) and 8 + n (half 1), so a lane's codes for a block are 32
// contiguous bytes of its row.  Columns are 4 * token + digit: 8 tokens per
// column tile, kCT column tiles per pass, so each dequantised weight serves
// 8 * kCT tokens.
//
// One 32-row tile per wave.  Gate/up: rows 0-15 are gate rows j0 .. j0+15
// and rows 16-31 the up rows of the same j, so output registers v and v + 8
// of a lane hold gate and up of one (j, token) and SwiGLU stays in the lane.
// Work item = (bucket, pass of 8 * kCT of its tokens) over all rows: 8 waves
// share the pass's operands and each sweeps every eighth 32-row tile.  The
// item first copies its tokens' digit operands for every K-block from
// memory straight into LDS (global_load_lds, no registers), then runs
// without a block barrier while each wave keeps a ring of its next code
// blocks in flight across tile boundaries.
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kCT = 2;             // column tiles per pass
constexpr int kPassTok = 8 * kCT;  // tokens per pass
constexpr int kTokStride = 1040;   // LDS bytes per staged token: 1024 + 16 spreads the banks

struct RowCodes {                  // one lane's share of a row's 256-value block
  uint4 lo, hi;                    // runs 8h .. 8h+7 (16 codes, 4 bytes each)
  uint32_t s;                      // group scales of groups 4h .. 4h+3 (16 bits)
  uint32_t dh;                     // block scale d (binary16 bits)
  uint4 hb;                        // third code bit of the 128 codes (3-bit only)
};

template <int QBITS>
__device__ inline RowCodes load_row_codes(const uint8_t* t, const PoolView& p, int64_t blk,
                                          int h) {
  RowCodes r;
  r.lo = *reinterpret_cast<const uint4*>(t + p.q + 64 * blk + 32 * h);
  r.hi = *reinterpret_cast<const uint4*>(t + p.q + 64 * blk + 32 * h + 16);
  r.s = *reinterpret_cast<const uint16_t*>(t + p.s + 4 * blk + 2 * h);
  r.dh = *reinterpret_cast<const uint16_t*>(t + p.d + 2 * blk);
  r.hb = make_uint4(0u, 0u, 0u, 0u);
  if (QBITS == 3) r.hb = *reinterpret_cast<const uint4*>(t + p.hb + 32 * blk + 16 * h);
  return r;
}

template <int QP>
__device__ inline float quad_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), QP, 0xf, 0xf, false));
}

__device__ inline uint32_t sel_u4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Byte tables of the lane's four groups 4h .. 4h+3 (MFMA n uses n/2).
template <int QBITS>
struct RowLuts {
  uint32_t lo[4], hi[4];
};

template <int QBITS>
__device__ inline RowLuts<QBITS> row_luts(const RowCodes& rc) {
  RowLuts<QBITS> t;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t sg = (rc.s >> (4 * g)) & 15u;
    t.lo[g] = lut2(sg);
    t.hi[g] = QBITS == 3 ? lut_hi(sg) : 0u;
  }
  return t;
}

// A operand of MFMA n (run 8h + n of the lane's row): the low-bit integers,
// and for 3-bit codes the third-bit integers in G.
template <int QBITS>
__device__ inline void row_operand(const RowCodes& rc, const RowLuts<QBITS>& t, int n, v4i& A,
                                   v4i& G) {
  A = dequant_dword(n < 4 ? sel_u4(rc.lo, n) : sel_u4(rc.hi, n - 4), t.lo[n >> 1]);
  if (QBITS == 3) {
    const uint32_t bits = (sel_u4(rc.hb, n >> 1) >> (16 * (n & 1))) & 0xffffu;
    G = dequant_hi16(bits, t.hi[n >> 1]);
  }
}

template <bool GATEUP, int QBITS>
__global__ __launch_bounds__(512) void prefill_expert32_kernel(
    PoolView pv, int H, int F, int k, const uint8_t* __restrict__ aq,
    const int32_t* __restrict__ ae, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_items_p, const int32_t* __restrict__ tile_bucket,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ bucket_start,
    const int32_t* __restrict__ bucket_slot, const int32_t* __restrict__ pairs,
    float* __restrict__ out) {
  if (*early_out) return;
  // the pass's digit operands for every K-block: token t's block kb at
  // t * tstride + kb * 1024, tstride = KB*1024 + 144 (= 9 mod 16 in 16-byte
  // units, so the 16 lanes of a read hit 16 different bank groups)
  __shared__ __align__(16) uint8_t s_b[kPassTok * (8 * 1024 + 144)];
  __shared__ int s_src[kPassTok];     // operand row of each pass token (-1: none)
  __shared__ int s_dst[kPassTok];     // output row
  __shared__ int s_e[kPassTok * 8];   // exponent of (token, K-block)
  __shared__ __align__(16) float s_rs[8][32];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int K = GATEUP ? H : F;
  const int NR = GATEUP ? F : H;
  const int KB = K / 256, kbs = __builtin_ctz(KB);
  const int tstride = KB * 1024 + 144;
  const int NTI = GATEUP ? NR / 16 : NR / 32;     // 32-row tiles per item
  const int NQ = (NTI / 8) * KB;                   // (tile, K-block) steps of a wave
  const int h = l >> 5, lr = l & 31;               // A: row lr of the tile, K-half h
  const int tcol = lr >> 2, dcol = l & 3;          // B/D: token and digit of column lr
  constexpr int NPF = QBITS == 3 ? 2 : 4;          // code blocks in flight
  const int n_items = *n_items_p;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int b = tile_bucket[item];
    const int p0 = bucket_start[b], n = bucket_start[b + 1] - p0;
    const int c0 = (item - tile_start[b]) * kPassTok;
    const int nt = n - c0 < kPassTok ? n - c0 : kPassTok;
    const int slot = bucket_slot[b];
    // the wave's A stream: step q = (tile i = q >> kbs, K-block q & (KB-1));
    // tile i is row tile w + 8i: gate/up rows 16(w+8i) .. +15 of gate (lanes
    // lr < 16) and of up (lr >= 16); down rows 32(w+8i) + lr
    const uint8_t* tA = tensor_base(pv, slot, GATEUP ? (lr < 16 ? 0 : 1) : 2);
    auto blk_of = [&](int q) {
      const int tt = w + 8 * (q >> kbs);
      const int row = GATEUP ? 16 * tt + (lr & 15) : 32 * tt + lr;
      return int64_t(row) * KB + (q & (KB - 1));
    };
    __syncthreads();                       // the previous item is done with LDS
    if (tid < kPassTok) {
      const int pos = p0 + c0 + tid;
      s_src[tid] = tid < nt ? (GATEUP ? pairs[pos] / k : pos) : -1;
      s_dst[tid] = tid < nt ? (GATEUP ? pos : pairs[pos]) : -1;
    }
    RowCodes pf[NPF];                      // a ring of code blocks in flight
#pragma unroll
    for (int i = 0; i < NPF; ++i)
      if (i < NQ) pf[i] = load_row_codes<QBITS>(tA, pv, blk_of(i), h);
    __syncthreads();
    // operands straight from memory to LDS: wave w copies tokens
    // kPassTok/8 * w .. +kPassTok/8 - 1, one 1 KiB K-block per instruction;
    // absent tokens are skipped (their columns are never stored)
    constexpr int TPW = kPassTok / 8;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = TPW * w + u;
      const int src = __builtin_amdgcn_readfirstlane(s_src[t]);
      if (src >= 0) {
        const uint8_t* g = aq + int64_t(src) * KB * 1024 + 16 * l;
        uint8_t* d = &s_b[t * tstride];
        for (int kb = 0; kb < KB; ++kb)
          __builtin_amdgcn_global_load_lds(g + kb * 1024, d + kb * 1024, 16, 0, 0);
      }
      if (l < KB) s_e[t * 8 + l] = src >= 0 ? ae[int64_t(src) * KB + l] : 0;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float acc[kCT][16];
    for (int q0 = 0; q0 < NQ; q0 += NPF)
#pragma unroll
    for (int ip = 0; ip < NPF; ++ip) {
      const int q = q0 + ip;
      if (q >= NQ) break;
      const int kb = q & (KB - 1);
      const RowCodes ca = pf[ip];
      if (q + NPF < NQ) pf[ip] = load_row_codes<QBITS>(tA, pv, blk_of(q + NPF), h);
      if (kb == 0) {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ct][v] = 0.f;
      }
      if (h == 0) s_rs[w][lr] = dh_dq<QBITS>(ca.dh);   // row scales through LDS
      wave_lds_sync32();
      const RowLuts<QBITS> luts = row_luts<QBITS>(ca);
      v16i D[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) D[ct] = v16i{};
      // B operands read one MFMA step ahead, so no MFMA waits on its own LDS
      // read.  Chunk of run 8h + nn, digit dcol: 512h + 64dcol + 256(nn/4) +
      // 16(nn%4) bytes into the token's K-block.
      const uint8_t* bbase = &s_b[tcol * tstride + kb * 1024 + 512 * h + 64 * dcol];
      auto bread = [&](int nn, int ct) {
        const int4 v = *reinterpret_cast<const int4*>(bbase + 8 * ct * tstride +
                                                      256 * (nn >> 2) + 16 * (nn & 3));
        return v4i{v.x, v.y, v.z, v.w};
      };
      v4i Bc[2][kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) Bc[0][ct] = bread(0, ct);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        if (nn < 7) {
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) Bc[(nn + 1) & 1][ct] = bread(nn + 1, ct);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's MFMAs
        v4i A, G;
        row_operand<QBITS>(ca, luts, nn, A, G);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          D[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bc[nn & 1][ct], D[ct], 0, 0, 0);
          if (QBITS == 3)
            D[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(G, Bc[nn & 1][ct], D[ct], 0, 0, 0);
        }
      }
      // row factor d/32 (or d/64); the column factor 2^(8(3-digit) - e) is one
      // per token (a row exponent) and applied when the tile is done
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 f = *reinterpret_cast<const float4*>(&s_rs[w][8 * g + 4 * h]);
        const float rv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[ct][4 * g + j] = fmaf(float(D[ct][4 * g + j]), rv[j], acc[ct][4 * g + j]);
      }
      wave_lds_sync32();                   // row scales read before the next step's
      if (kb == KB - 1) {
        // tile done: combine each token's four digit columns (lanes
        // 4*tcol .. +3) and store
        const int tt = w + 8 * (q >> kbs);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          const int dst = s_dst[8 * ct + tcol];
          const float cs = ldexpf(1.f, 8 * (3 - dcol) - s_e[(8 * ct + tcol) * 8]);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = acc[ct][v] * cs;
            x += quad_swap<0xb1>(x);          // quad_perm [1,0,3,2]
            x += quad_swap<0x4e>(x);          // quad_perm [2,3,0,1]
            acc[ct][v] = x;
          }
          if (dcol == 0 && dst >= 0) {
            if (GATEUP) {                  // rows R = 8g + 4h + j < 16: gate; R + 16: up
              const int j0 = 16 * tt;
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                float4 hv;
                hv.x = silu_mul(acc[ct][4 * g + 0], acc[ct][4 * g + 8]);
                hv.y = silu_mul(acc[ct][4 * g + 1], acc[ct][4 * g + 9]);
                hv.z = silu_mul(acc[ct][4 * g + 2], acc[ct][4 * g + 10]);
                hv.w = silu_mul(acc[ct][4 * g + 3], acc[ct][4 * g + 11]);
                *reinterpret_cast<float4*>(out + int64_t(dst) * F + j0 + 8 * g + 4 * h) = hv;
              }
            } else {
              const int i0 = 32 * tt;
#pragma unroll
              for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(out + int64_t(dst) * H + i0 + 8 * g + 4 * h) =
                    make_float4(acc[ct][4 * g], acc[ct][4 * g + 1], acc[ct][4 * g + 2],
                                acc[ct][4 * g + 3]);
            }
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

void launch_quantize_h(const PrefillArgs& a, hipStream_t st) {
  const int rpb = 256 / (a.F / 16);
  const int R = a.T * a.k;
  quantize_rows_kernel<true><<<(R + rpb - 1) / rpb, 256, 0, st>>>(a.hbuf, R, a.F, a.hq, a.he,
                                                                   a.early_out);
}

void launch_prefill_gateup_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  auto kern = a.qbits == 3 ? prefill_expert32_kernel<true, 3> : prefill_expert32_kernel<true, 2>;
  kern<<<1024, 512, 0, st>>>(a.pool, a.H, a.F, a.k, a.xq, a.xe, a.early_out, p.n_tiles,
                             p.tile_bucket, p.tile_start, p.bucket_start, p.bucket_slot,
                             p.pairs, a.hbuf);
}

void launch_prefill_down_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  auto kern = a.qbits == 3 ? prefill_expert32_kernel<false, 3> : prefill_expert32_kernel<false, 2>;
  kern<<<1024, 512, 0, st>>>(a.pool, a.H, a.F, a.k, a.hq, a.he, a.early_out, p.n_tiles,
                             p.tile_bucket, p.tile_start, p.bucket_start, p.bucket_slot,
                             p.pairs, a.ebuf);
}

}  // namespace rl
