// Exact int8 operands for the gfx950 matrix cores (v_mfma_i32_16x16x64_i8),
// shared by the decode and prefill expert kernels.
//
// Weights.  A 2-bit weight is d * q / 32 with the integer q = (2s+1)(2c-3) in
// [-93, 93]: an int8, turned out of the code bits by one byte permute against
// a 4-entry table per 32-value group.  A 3-bit weight is d * q3 / 64 with
// q3 = (2s+1)(2c-7), c = c01 + 4*b2, which reaches 217; it is split exactly as
// q3 = (2s+1)(2c01-3) + 4(2s+1)(2b2-1): the 2-bit integer of the low code
// bits plus a second int8 in [-124, 124] from the third bit, each its own
// MFMA into the same int32 accumulator (|sum| over a block < 2^23).
//
// Activations.  A run of values sharing one scale (a row, or a 256-value
// block) is multiplied by a power of two 2^e so that |x * 2^e| < 2^30,
// rounded to the integer X, and X is written as four balanced base-256 digits
// in [-128, 127].  Products of int8 weights and digits summed over one
// 256-value block stay below 2^22 in magnitude, so the int32 result is exact
// and is scaled once by d/32 and 2^(8*(3-digit) - e).  Values with
// |x| >= 2^-7 * max|x| are represented exactly; the rest lose nothing above
// 2^-31 * max|x|.
//
// Operand layout (checked on the device): A lane l holds row l%16 and the 16
// bytes of K-slice l/16; B lane l holds column l%16 and the same K-slice; the
// output lane l holds rows 4*(l/16)+v, v < 4, of column l%16.  Inside a
// 256-value block, lane quad q and MFMA m cover K = 64q + 16m + [0, 16), and
// byte i of dword jj of the operand is K offset 4i + jj (the order in which
// (codes >> 2jj) & 0x03030303 exposes four codes).  A block's digit operands
// are 1024 bytes: one 16-byte chunk per (quad, digit, MFMA), placed by
// digit_chunk_offset.
#pragma once

#include "rl_common.h"

namespace rl {

typedef int v4i __attribute__((ext_vector_type(4)));

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

// Byte offset, inside one 256-value block's 1024 bytes of digit operands, of
// the 16-byte chunk of (quad q, digit d, MFMA m).
__host__ __device__ constexpr int digit_chunk_offset(int q, int d, int m) {
  return ((q * 4 + d) * 4 + m) * 16;
}

// 16 consecutive values v (K = 64q + 16m + [0, 16) of a block) scaled by 2^e
// -> the four 16-byte digit chunks of (q, m): chunk[d] for digit d.
__device__ inline void digit_chunks(const float* v, int e, uint4* chunk) {
  uint32_t Z[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) Z[n] = digits_of(int(rintf(ldexpf(v[n], e))));
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
    chunk[d] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Byte table of q = (2s+1)(2c-3) for c = 0..3: {-3m, -m, m, 3m}, m = 2s+1.
__device__ inline uint32_t lut2(uint32_t s) {
  const uint32_t m = 2u * s + 1u;
  return ((0x10100u - __umul24(259u, m)) & 0xffffu) | (__umul24(m, 0x0301u) << 16);
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
// Raw bytes only: nothing is computed from a load when it is issued, so a
// prefetched tile does not make the wave wait.
struct TileCodes {
  uint4 c;       // 64 codes (low two bits): K = 64q .. 64q+63 of the block
  uint32_t s;    // group scales of groups 2q (low nibble) and 2q+1
  uint32_t dh;   // block scale d, binary16 bits
  uint2 hb;      // third code bit of the 64 codes (3-bit only)
};

template <int QBITS>
__device__ inline TileCodes load_tile(const uint8_t* t, const PoolView& p, int64_t blk, int q) {
  TileCodes r;
  r.c = *reinterpret_cast<const uint4*>(t + p.q + 64 * blk + 16 * q);
  r.s = t[p.s + 4 * blk + q];
  r.dh = *reinterpret_cast<const uint16_t*>(t + p.d + 2 * blk);
  r.hb = make_uint2(0u, 0u);
  if (QBITS == 3) r.hb = *reinterpret_cast<const uint2*>(t + p.hb + 32 * blk + 8 * q);
  return r;
}

// d/32 (2-bit) or d/64 (3-bit): the factor of the block's integer sums.
template <int QBITS>
__device__ inline float dh_dq(uint32_t dh) {
  return half_bits_to_float(uint16_t(dh)) * (QBITS == 3 ? 1.f / 64.f : 1.f / 32.f);
}
template <int QBITS>
__device__ inline float tile_dq(const TileCodes& t) { return dh_dq<QBITS>(t.dh); }

__device__ inline void dequant_tile(const TileCodes& tc, v4i A[4]) {
  const uint32_t l0 = lut2(tc.s & 15u), l1 = lut2(tc.s >> 4);
  A[0] = dequant_dword(tc.c.x, l0);
  A[1] = dequant_dword(tc.c.y, l0);
  A[2] = dequant_dword(tc.c.z, l1);
  A[3] = dequant_dword(tc.c.w, l1);
}

// Byte table of the third-bit term 4(2s+1)(2b-1) for b = 0, 1.
__device__ inline uint32_t lut_hi(uint32_t s) {
  const uint32_t m4 = 4u * (2u * s + 1u);
  return ((0x100u - m4) & 0xffu) | (m4 << 8);
}

// Third-bit operand of MFMA m from 16 bits x16 (code 16m + n at bit n):
// dword jj byte i <- bit 4i + jj, mapped through lut.
__device__ inline v4i dequant_hi16(uint32_t x16, uint32_t lut) {
  v4i a;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t x = x16 >> jj;
    const uint32_t w = __builtin_amdgcn_perm(x, x, 0x01010000u);   // bytes x0 x0 x1 x1
    const uint32_t sel = ((w >> 4) & 0x01000100u) | (w & 0x00010001u);
    a[jj] = int(__builtin_amdgcn_perm(lut, lut, sel));
  }
  return a;
}

__device__ inline void dequant_tile_hi(const TileCodes& tc, v4i A[4]) {
  const uint32_t l0 = lut_hi(tc.s & 15u), l1 = lut_hi(tc.s >> 4);
  A[0] = dequant_hi16(tc.hb.x & 0xffffu, l0);
  A[1] = dequant_hi16(tc.hb.x >> 16, l0);
  A[2] = dequant_hi16(tc.hb.y & 0xffffu, l1);
  A[3] = dequant_hi16(tc.hb.y >> 16, l1);
}

// Four chained MFMAs over one 256-value block: D = sum_m A[m] * B[m].
__device__ inline v4i mfma4(const v4i A[4], const v4i B[4]) {
  v4i D = {0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 4; ++m) D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[m], B[m], D, 0, 0, 0);
  return D;
}

// The block's integer sums for QBITS-bit codes: D += A * B over the low
// code bits and, for 3-bit codes, the third-bit term.
template <int QBITS>
__device__ inline v4i tile_mfma(const TileCodes& tc, const v4i B[4]) {
  v4i A[4];
  dequant_tile(tc, A);
  v4i D = mfma4(A, B);
  if (QBITS == 3) {
    dequant_tile_hi(tc, A);
#pragma unroll
    for (int m = 0; m < 4; ++m) D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[m], B[m], D, 0, 0, 0);
  }
  return D;
}

}  // namespace rl
