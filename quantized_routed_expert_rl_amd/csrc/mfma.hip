// Batched expert projections on the int8 matrix cores of gfx950
// (v_mfma_i32_16x16x64_i8), for 2-bit and 3-bit block weights when both
// expert dimensions are multiples of 256 ("Red Lite dev20 - batched prompt
// ingestion", "What changed": batched gate/up and down over (expert, token)
// pairs sorted by expert).
//
// The int8 operands and their exactness are described in rl_mfma.h; columns
// of the B operand are 4 * token + digit.
#include <atomic>
#include <type_traits>

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
// contiguous bytes of one weight row.
//
// A = activation digits, row 4 * token + digit (8 tokens per MFMA, kCT
// MFMAs per pass); B = dequantised weights, column = one of a tile's 32
// weight rows.  A lane's outputs are then its own weight row for tokens
// 2m + l/32 (m < 4), with the four digits of each token in registers
// 4m .. 4m+3: digits combine inside the lane, and the row's block scale d is
// the lane's own, so scaling needs nothing from other lanes.  Gate/up tiles
// hold gate rows j0 .. j0+15 in columns 0-15 and the up rows of the same j in
// columns 16-31; lanes l and l^16 trade half of their tokens for SwiGLU.
//
// Work: item = (bucket, pass of kPassTok of its tokens) over all rows;
// round = 8 tiles of one item, one per wave.  The rounds of all items are
// split evenly over the blocks (one per compute unit), each taking a
// contiguous range, so no compute unit idles while another still has whole
// items queued.  When its range enters a new item, the block copies the
// pass's digit operands for every K-block straight into LDS
// (global_load_lds, no registers); in between, each wave streams its tiles'
// codes through a ring of blocks in flight that runs across tile and item
// boundaries.
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kCT = 2;             // MFMAs (8 tokens each) per pass
constexpr int kPassTok = 8 * kCT;  // tokens per pass

// Whole dwords only: a sub-dword load is widened right after it is issued,
// which would make the wave wait for it there and empty the ring of loads in
// flight.  The halves are picked when the block is used.
struct RowCodes {                  // one lane's share of a row's 256-value block
  uint4 lo, hi;                    // runs 8h .. 8h+7 (16 codes, 4 bytes each)
  uint32_t s;                      // the block's eight group scales (lane uses half h)
  uint32_t dh;                     // d of blocks 2(blk/2) and 2(blk/2)+1 (binary16 bits)
  uint4 hb;                        // third code bit of the 128 codes (3-bit only)
};

// Buffer loads of a lane's block: the slot's buffer descriptor lives in
// scalar registers (one per item: gate/up tiles read two tensors of the slot,
// so the descriptor covers the slot and the lane's tensor is part of its
// offset), the lane's part of each address (its tensor, row and half) is a
// per-lane offset fixed for the whole kernel, and the block index's
// wave-uniform part is a scalar offset, so no per-lane address arithmetic
// runs per step.  Block blk = bu + bl: bu (uniform) = ROWS*tile*KB + kb,
// bl (lane) = rowoff*KB; bu + bl is even whenever bl is odd (KB = 1, where
// bu = ROWS*tile is even), so blk/2 = bu/2 + bl/2 for the d plane.
struct LaneOffsets {
  int q, s, d, hb;                 // per-lane byte offsets inside the tensor
};

__device__ inline LaneOffsets lane_offsets(const PoolView& p, int which, int bl, int h) {
  const int t = which * int(p.tensor_bytes);
  LaneOffsets o;
  o.q = t + int(p.q) + 64 * bl + 32 * h;
  o.s = t + int(p.s) + 4 * bl;
  o.d = t + int(p.d) + 4 * (bl >> 1);
  o.hb = t + int(p.hb) + 32 * bl + 16 * h;
  return o;
}

template <int QBITS>
__device__ inline RowCodes load_row_codes(__amdgpu_buffer_rsrc_t t, const LaneOffsets& o, int bu) {
  RowCodes r;
  r.lo = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t, o.q, 64 * bu, 0));
  r.hi = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t, o.q, 64 * bu + 16, 0));
  r.s = __builtin_amdgcn_raw_buffer_load_b32(t, o.s, 4 * bu, 0);
  r.dh = __builtin_amdgcn_raw_buffer_load_b32(t, o.d, 4 * (bu >> 1), 0);
  r.hb = make_uint4(0u, 0u, 0u, 0u);
  if (QBITS == 3)
    r.hb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t, o.hb, 32 * bu, 0));
  return r;
}

__device__ inline uint32_t sel_u4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Byte tables of the lane's four groups 4h .. 4h+3 (MFMA n uses n/2).
template <int QBITS>
struct RowLuts {
  uint32_t lo[4], hi[4];
};

// The four tables of groups 4h .. 4h+3 at once, byte-parallel: bytes
// m_g = 2 s_g + 1 (<= 31) and 3 m_g (<= 93) never carry, and the byte-wise
// negation of M is 0x01010100 - M (mod 2^32) since every byte is nonzero.
// ssel picks the lane's two scale bytes: 0x01010000 (h = 0), 0x03030202.
template <int QBITS>
__device__ inline RowLuts<QBITS> row_luts(const RowCodes& rc, uint32_t ssel) {
  RowLuts<QBITS> t;
  const uint32_t y = __builtin_amdgcn_perm(rc.s, rc.s, ssel);          // bytes s01 s01 s23 s23
  const uint32_t x = (y & 0x000f000fu) | ((y >> 4) & 0x0f000f00u);    // bytes s0 s1 s2 s3
  const uint32_t M = (x << 1) | 0x01010101u;
  const uint32_t M3 = M + (M << 1);
  const uint32_t nM = 0x01010100u - M, nM3 = 0x01010100u - M3;
  const uint32_t a01 = __builtin_amdgcn_perm(nM, nM3, 0x05010400u);    // -3m0 -m0 -3m1 -m1
  const uint32_t a23 = __builtin_amdgcn_perm(nM, nM3, 0x07030602u);
  const uint32_t b01 = __builtin_amdgcn_perm(M3, M, 0x05010400u);      // m0 3m0 m1 3m1
  const uint32_t b23 = __builtin_amdgcn_perm(M3, M, 0x07030602u);
  t.lo[0] = __builtin_amdgcn_perm(b01, a01, 0x05040100u);              // -3m -m m 3m
  t.lo[1] = __builtin_amdgcn_perm(b01, a01, 0x07060302u);
  t.lo[2] = __builtin_amdgcn_perm(b23, a23, 0x05040100u);
  t.lo[3] = __builtin_amdgcn_perm(b23, a23, 0x07060302u);
  if (QBITS == 3) {
    const uint32_t M4 = M << 2, nM4 = 0x01010100u - M4;                // 4m <= 124
#pragma unroll
    for (int g = 0; g < 4; ++g)                                         // -4m 4m
      t.hi[g] = __builtin_amdgcn_perm(M4, nM4, uint32_t(g) | (uint32_t(4 + g) << 8));
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) t.hi[g] = 0u;
  }
  return t;
}

// Weight operand of MFMA n (run 8h + n of the lane's row): the low-bit
// integers, and for 3-bit codes the third-bit integers in G.
template <int QBITS>
__device__ inline void row_operand(const RowCodes& rc, const RowLuts<QBITS>& t, int n, v4i& W,
                                   v4i& G) {
  W = dequant_dword(n < 4 ? sel_u4(rc.lo, n) : sel_u4(rc.hi, n - 4), t.lo[n >> 1]);
  if (QBITS == 3) {
    const uint32_t bits = (sel_u4(rc.hb, n >> 1) >> (16 * (n & 1))) & 0xffffu;
    G = dequant_hi16(bits, t.hi[n >> 1]);
  }
}

template <bool GATEUP, int QBITS>
__global__ __launch_bounds__(512) void prefill_expert_kernel(
    PoolView pv, int H, int F, int k, const uint8_t* __restrict__ aq,
    const int32_t* __restrict__ ae, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_items_p, const int32_t* __restrict__ item_bucket,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ bucket_start,
    const int32_t* __restrict__ bucket_slot, const int32_t* __restrict__ pairs,
    float* __restrict__ out) {
  if (*early_out) return;
  // the pass's digit operands for every K-block: token t's block kb at
  // t * tstride + kb * 1024, tstride = KB*1024 + 144 (= 9 mod 16 in 16-byte
  // units, so the 16 lanes of a read hit 16 different bank groups)
  __shared__ __align__(16) uint8_t s_b[kPassTok * (8 * 1024 + 144)];
  __shared__ int s_src[kPassTok];     // operand row of each pass token (-1: none)
  __shared__ int s_dst[kPassTok];     // output row
  __shared__ float s_cs[kPassTok];    // 2^-e of the token's operand row
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = GATEUP ? H : F;
  const int NR = GATEUP ? F : H;
  const int KB = K / 256, kbs = __builtin_ctz(KB);
  const int tstride = KB * 1024 + 144;
  const int NTI = GATEUP ? NR / 16 : NR / 32;     // 32-row tiles per item
  const int RPI = NTI / 8;                         // rounds per item
  const int h = l >> 5, c = l & 31;
  constexpr int NPF = QBITS == 3 ? 2 : 4;          // code blocks in flight
  const int n_items = *n_items_p;
  const int64_t R = int64_t(n_items) * RPI;
  const int r0 = int(R * blockIdx.x / gridDim.x);
  const int r1 = int(R * (blockIdx.x + 1) / gridDim.x);
  if (r0 >= r1) return;
  const int NQ = (r1 - r0) * KB;                   // (round, K-block) steps

  // The wave's code stream: round r's tile is (r % RPI) * 8 + w of item
  // r / RPI; the lane's row in it is 16 * tile + c%16 of gate (c < 16) or
  // up (c >= 16), or 32 * tile + c of down.
  const int which = GATEUP ? (c < 16 ? 0 : 1) : 2;
  const int rowoff = GATEUP ? (c & 15) : c;
  constexpr int ROWS = GATEUP ? 16 : 32;
  const uint32_t ssel = h ? 0x03030202u : 0x01010000u;
  // Past the end of the range the stream keeps loading its last block, so
  // every ring slot is refilled at every step (no data-dependent refills,
  // which would make the compiler copy the ring and wait for it).
  int s_item = r0 / RPI, s_tile = (r0 - s_item * RPI) * 8 + w, s_kb = 0, s_left = NQ;
  // the item's tensor in its bucket's pool slot
  // the item's pool slot as a buffer descriptor (reads past the slot's end
  // return 0)
  auto item_tensor = [&](int it) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(tensor_base(pv, bucket_slot[item_bucket[it]], 0)), 0,
        int(pv.slot_bytes), 0x00020000);
  };
  __amdgpu_buffer_rsrc_t s_t = item_tensor(s_item);
  const LaneOffsets lo = lane_offsets(pv, which, rowoff * KB, h);
  auto next_codes = [&]() {
    const RowCodes rc = load_row_codes<QBITS>(s_t, lo, ROWS * s_tile * KB + s_kb);
    if (--s_left <= 0) return rc;
    if (++s_kb == KB) {
      s_kb = 0;
      s_tile += 8;
      if (s_tile >= NTI) {
        s_tile -= NTI;
        if (++s_item < n_items) s_t = item_tensor(s_item);
      }
    }
    return rc;
  };
  // A ring of NPF code blocks in flight in NPF + 1 slots: step ip uses slot
  // ip and refills slot ip - 1, the one the previous step finished with, so
  // no load targets a register that is still being read and the unrolled
  // loop keeps every slot in fixed registers.
  constexpr int NS = NPF + 1;
  RowCodes pf[NS];
#pragma unroll
  for (int i = 0; i < NPF; ++i) pf[i] = next_codes();

  int staged = -1;                       // item whose operands are in LDS
  int item = 0, tile = 0;                // the current round's item and this wave's tile
  bool two = true;                       // the pass has more than 8 tokens (both MFMA groups)
  float acc[kCT][4];
  for (int q0 = 0; q0 < NQ; q0 += NS)
#pragma unroll
  for (int ip = 0; ip < NS; ++ip) {
    const int q = q0 + ip;
    const RowCodes& ca = pf[ip];
    pf[(ip + NPF) % NS] = next_codes();  // on every path, so the ring stays in place
    if (q >= NQ) continue;
    const int kb = q & (KB - 1);
    if (kb == 0) {
      const int r = r0 + (q >> kbs);
      item = r / RPI;
      tile = (r - item * RPI) * 8 + w;
      if (item != staged) {
        // every wave reaches this step together (same rounds, same K-blocks)
        __syncthreads();                 // the previous item's operands are no longer read
        const int b = item_bucket[item];
        const int p0 = bucket_start[b], n = bucket_start[b + 1] - p0;
        const int c0 = (item - item_start[b]) * kPassTok;
        const int nt = n - c0 < kPassTok ? n - c0 : kPassTok;
        two = nt > 8;
        if (tid < kPassTok) {
          const int pos = p0 + c0 + tid;
          const int src = tid < nt ? (GATEUP ? pairs[pos] / k : pos) : -1;
          s_src[tid] = src;
          s_dst[tid] = tid < nt ? (GATEUP ? pos : pairs[pos]) : -1;
          s_cs[tid] = src >= 0 ? ldexpf(1.f, -ae[int64_t(src) * KB]) : 0.f;
        }
        __syncthreads();
        // wave w copies tokens TPW*w .. TPW*w + TPW-1, one 1 KiB K-block per
        // instruction; absent tokens are skipped (their rows are never stored)
        constexpr int TPW = kPassTok / 8;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int t = TPW * w + u;
          const int src = __builtin_amdgcn_readfirstlane(s_src[t]);
          if (src >= 0) {
            const uint8_t* g = aq + int64_t(src) * KB * 1024 + 16 * l;
            uint8_t* d = &s_b[t * tstride];
            for (int j = 0; j < KB; ++j)
              __builtin_amdgcn_global_load_lds(g + j * 1024, d + j * 1024, 16, 0, 0);
          }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        staged = item;
      }
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[ct][m] = 0.f;
    }
    // one step for kc groups of 8 tokens: with 3-bit codes, passes of at most
    // 8 tokens skip the second group's MFMAs, scaling and digit reads (with
    // 2-bit codes the second copy of the step costs more than it saves:
    // measured, 5 % slower)
    auto step = [&](auto kc_tag) __attribute__((always_inline)) {
    constexpr int kc = decltype(kc_tag)::value;
    const RowLuts<QBITS> luts = row_luts<QBITS>(ca, ssel);
    // the lane's row's block factor: half (block parity) of the d dword
    const float rs = dh_dq<QBITS>((KB == 1 ? rowoff & 1 : kb & 1) ? ca.dh >> 16 : ca.dh & 0xffffu);
    v16i D[kc];
#pragma unroll
    for (int ct = 0; ct < kc; ++ct) D[ct] = v16i{};
    // digit operands read one MFMA step ahead, so no MFMA waits on its own
    // LDS read.  Chunk of token c/4, digit c%4, run 8h + nn: 512h + 64(c%4) +
    // 256(nn/4) + 16(nn%4) bytes into the token's K-block.
    const uint8_t* abase = &s_b[(c >> 2) * tstride + kb * 1024 + 512 * h + 64 * (c & 3)];
    auto aread = [&](int nn, int ct) {
      const int4 v = *reinterpret_cast<const int4*>(abase + 8 * ct * tstride +
                                                    256 * (nn >> 2) + 16 * (nn & 3));
      return v4i{v.x, v.y, v.z, v.w};
    };
    v4i Ad[2][kc];
#pragma unroll
    for (int ct = 0; ct < kc; ++ct) Ad[0][ct] = aread(0, ct);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      if (nn < 7) {
#pragma unroll
        for (int ct = 0; ct < kc; ++ct) Ad[(nn + 1) & 1][ct] = aread(nn + 1, ct);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's MFMAs
      v4i W, G;
      row_operand<QBITS>(ca, luts, nn, W, G);
#pragma unroll
      for (int ct = 0; ct < kc; ++ct) {
        D[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Ad[nn & 1][ct], W, D[ct], 0, 0, 0);
        if (QBITS == 3)
          D[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Ad[nn & 1][ct], G, D[ct], 0, 0, 0);
      }
    }
    // X = 2^24 D0 + 2^16 D1 + 2^8 D2 + D3 (digit 0 most significant): the
    // pairs 256 D0 + D1 and 256 D2 + D3 stay below 2^31, so each token takes
    // two conversions and one scaled add per block
#pragma unroll
    for (int ct = 0; ct < kc; ++ct)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int hi = D[ct][4 * m] * 256 + D[ct][4 * m + 1];
        const int lo = D[ct][4 * m + 2] * 256 + D[ct][4 * m + 3];
        acc[ct][m] = fmaf(fmaf(float(hi), 65536.f, float(lo)), rs, acc[ct][m]);
      }
    if (kb == KB - 1) {
      // tile done: the lane holds row c of the tile for tokens 8ct + 2m + h.
      // Every LDS read of the token tables and every lane exchange is issued
      // before any result is used, and SwiGLU picks its operands by select,
      // so the tile's end costs two LDS round trips instead of two per output.
      float v[kc][4];
      int dst[kc][4];
#pragma unroll
      for (int ct = 0; ct < kc; ++ct)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v[ct][m] = acc[ct][m] * s_cs[8 * ct + 2 * m + h];
          dst[ct][m] = s_dst[8 * ct + 2 * m + h];
        }
      if (GATEUP) {
        // gate lanes (c < 16) finish tokens m = 0, 1 and up lanes m = 2, 3
        const bool gl = c < 16;
        const int j = 16 * tile + (c & 15);
        float other[kc][2];
#pragma unroll
        for (int ct = 0; ct < kc; ++ct)
#pragma unroll
          for (int i = 0; i < 2; ++i) other[ct][i] = __shfl_xor(gl ? v[ct][2 + i] : v[ct][i], 16);
#pragma unroll
        for (int ct = 0; ct < kc; ++ct)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float g = gl ? v[ct][i] : other[ct][i];
            const float u = gl ? other[ct][i] : v[ct][2 + i];
            const float hv = silu_mul(g, u);
            const int d = gl ? dst[ct][i] : dst[ct][2 + i];
            if (d >= 0) out[int64_t(d) * F + j] = hv;
          }
      } else {
        const int i0 = 32 * tile + c;
#pragma unroll
        for (int ct = 0; ct < kc; ++ct)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (dst[ct][m] >= 0) out[int64_t(dst[ct][m]) * H + i0] = v[ct][m];
      }
    }
    };
    if (QBITS == 2 || two)
      step(std::integral_constant<int, 2>{});
    else
      step(std::integral_constant<int, 1>{});
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
  auto kern = a.qbits == 3 ? prefill_expert_kernel<true, 3> : prefill_expert_kernel<true, 2>;
  kern<<<device_cu_count(), 512, 0, st>>>(a.pool, a.H, a.F, a.k, a.xq, a.xe, a.early_out, p.n_tiles,
                                   p.tile_bucket, p.tile_start, p.bucket_start, p.bucket_slot,
                                   p.pairs, a.hbuf);
}

void launch_prefill_down_mfma(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  auto kern = a.qbits == 3 ? prefill_expert_kernel<false, 3> : prefill_expert_kernel<false, 2>;
  kern<<<device_cu_count(), 512, 0, st>>>(a.pool, a.H, a.F, a.k, a.hq, a.he, a.early_out, p.n_tiles,
                                   p.tile_bucket, p.tile_start, p.bucket_start, p.bucket_slot,
                                   p.pairs, a.ebuf);
}

}  // namespace rl
