// Internal helpers shared by the gfx950 kernels of librlmoe (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rl_moe.h"

namespace rl {

constexpr int kWave = 64;

// ---------------------------------------------------------------- format
// Plane offsets of one block-format tensor (see rl_moe.h for the format).
struct TensorLayout {
  int64_t nb, q, hb, s, d, total;
};

__host__ __device__ inline int64_t up256(int64_t n) { return (n + 255) & ~int64_t(255); }

__host__ __device__ inline TensorLayout tensor_layout(int64_t n_elems, int qbits) {
  TensorLayout t;
  t.nb = n_elems >> 8;
  t.q = 0;
  int64_t end = t.nb * 64;
  t.hb = 0;
  if (qbits == 3) {
    t.hb = up256(end);
    end = t.hb + t.nb * 32;
  }
  t.s = up256(end);
  t.d = up256(t.s + t.nb * 4);
  t.total = up256(t.d + t.nb * 2);
  return t;
}

// Device-side view of the slot pool: slot s starts at base + s*slot_bytes;
// inside a slot, gate at 0, up at tensor bytes, down at twice that.
struct PoolView {
  const uint8_t* base;
  int64_t slot_bytes;
  int64_t tensor_bytes;
  int64_t q, hb, s, d;   // plane offsets inside one tensor
};

inline PoolView make_pool_view(const void* pool, int hidden, int width, int qbits) {
  TensorLayout t = tensor_layout(int64_t(hidden) * width, qbits);
  PoolView v;
  v.base = static_cast<const uint8_t*>(pool);
  v.tensor_bytes = t.total;
  v.slot_bytes = 3 * t.total;
  v.q = t.q;
  v.hb = t.hb;
  v.s = t.s;
  v.d = t.d;
  return v;
}

// Base of tensor `which` (0 gate, 1 up, 2 down) of slot `slot`.
__device__ inline const uint8_t* tensor_base(const PoolView& p, int slot, int which) {
  return p.base + int64_t(slot) * p.slot_bytes + int64_t(which) * p.tensor_bytes;
}

// One 32-value group of a tensor, ready for a dot product with 32
// activations: codes (low bits, 64 bits), third bit plane (3-bit only),
// group scale factor (2s+1)/16 * d.
struct Group32 {
  uint32_t c0, c1;   // low two bits of 32 codes: code n at bits 2n of c0:c1
  uint32_t hi;       // bit 2 of code n at bit n (3-bit only)
  float scale;       // d * (2s+1) / 16
};

__device__ inline float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Load group at flat element index `flat` (a multiple of 32) of a tensor.
template <int QBITS>
__device__ inline Group32 load_group(const uint8_t* t, const PoolView& p, int64_t flat) {
  Group32 g;
  const int64_t b = flat >> 8;
  const int j = int(flat & 255);
  const uint2 c = *reinterpret_cast<const uint2*>(t + p.q + 64 * b + (j >> 2));
  g.c0 = c.x;
  g.c1 = c.y;
  g.hi = 0;
  if (QBITS == 3) g.hi = *reinterpret_cast<const uint32_t*>(t + p.hb + 32 * b + (j >> 3));
  const int grp = j >> 5;
  const uint32_t sb = t[p.s + 4 * b + (grp >> 1)];
  const uint32_t s = (grp & 1) ? (sb >> 4) : (sb & 15u);
  const uint16_t dh = *reinterpret_cast<const uint16_t*>(t + p.d + 2 * b);
  g.scale = half_bits_to_float(dh) * float(2 * s + 1) * (1.0f / 16.0f);
  return g;
}

// sum_{n<32} level(c_n) * xv[n] * scale for one group; xsum = sum_n xv[n].
// level(c) = c - 1.5 (2-bit) or (c - 3.5)/2 (3-bit); the offset term is
// applied once per group through xsum.
template <int QBITS>
__device__ inline float group_dot(const Group32& g, const float* xv, float xsum) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t dw = w ? g.c1 : g.c0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t t = (dw >> (2 * jj)) & 0x03030303u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = fmaf(float((t >> (8 * i)) & 0xffu), xv[16 * w + 4 * i + jj], acc);
    }
  }
  if (QBITS == 3) {
    float acch = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t t = (g.hi >> jj) & 0x01010101u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acch = fmaf(float((t >> (8 * i)) & 0xffu), xv[8 * i + jj], acch);
    }
    return g.scale * 0.5f * fmaf(4.f, acch, acc - 3.5f * xsum);
  }
  return g.scale * (acc - 1.5f * xsum);
}

// ---------------------------------------------------------- wave helpers
__device__ inline float wave_sum_width(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Float64 sum of squares of a 4-value chunk added to s in component order,
// and the chunk scaled by inv and rounded to float32 (the RMSNorms).
__device__ inline double chunk_sq(const float4& f, double s) {
  s = fma(double(f.x), double(f.x), s);
  s = fma(double(f.y), double(f.y), s);
  s = fma(double(f.z), double(f.z), s);
  return fma(double(f.w), double(f.w), s);
}

__device__ inline float4 chunk_scale(const float4& f, double inv) {
  return make_float4(float(double(f.x) * inv), float(double(f.y) * inv), float(double(f.z) * inv),
                     float(double(f.w) * inv));
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP max/min over the 64 lanes; the result is returned in every lane.
// row_shr 1, 2, 4, 8 leave each row's extreme in its lane 15; row_bcast 15
// and 31 carry it to lane 63.  Lanes without a DPP source keep their value.
template <int CTRL, int ROWMASK, bool MAX>
__device__ inline uint32_t dpp_step(uint32_t x) {
  const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), CTRL, ROWMASK, 0xf, false));
  return MAX ? (o > x ? o : x) : (o < x ? o : x);
}

template <bool MAX>
__device__ inline uint32_t wave_reduce_u32(uint32_t v) {
  v = dpp_step<0x111, 0xf, MAX>(v);  // row_shr:1
  v = dpp_step<0x112, 0xf, MAX>(v);  // row_shr:2
  v = dpp_step<0x114, 0xf, MAX>(v);  // row_shr:4
  v = dpp_step<0x118, 0xf, MAX>(v);  // row_shr:8
  v = dpp_step<0x142, 0xa, MAX>(v);  // row_bcast:15
  v = dpp_step<0x143, 0xc, MAX>(v);  // row_bcast:31
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

__device__ inline uint32_t wave_max_u32(uint32_t v) { return wave_reduce_u32<true>(v); }
__device__ inline uint32_t wave_min_u32(uint32_t v) { return wave_reduce_u32<false>(v); }

// DPP sum over groups of W consecutive lanes (W = 1..64, a power of two);
// the group's total lands in its last lane (other lanes hold partial sums).
// Lanes without a DPP source contribute 0 (bound_ctrl).
template <int CTRL, int ROWMASK>
__device__ inline float dpp_add(float x) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf, true);
  return x + __int_as_float(o);
}

template <int W>
__device__ inline float group_sum_last(float v) {
  if (W >= 2) v = dpp_add<0x111, 0xf>(v);   // row_shr:1
  if (W >= 4) v = dpp_add<0x112, 0xf>(v);   // row_shr:2
  if (W >= 8) v = dpp_add<0x114, 0xf>(v);   // row_shr:4
  if (W >= 16) v = dpp_add<0x118, 0xf>(v);  // row_shr:8
  if (W >= 32) v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
  if (W >= 64) v = dpp_add<0x143, 0xc>(v);  // row_bcast:31
  return v;
}

// Order-preserving map of a float32 to uint32 (larger float -> larger key):
// negative floats have all bits flipped, others only the sign bit.  Adding
// +0 first turns -0 into +0 (round to nearest), so the two compare equal.
__device__ inline uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}

// Inverse of float_key (a -0 comes back as +0).
__device__ inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// silu(g) * u = g / (1 + e^-g) * u with the hardware exponential and
// reciprocal (about 1 ulp each; far inside the float32 tolerance).
__device__ inline float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

}  // namespace rl
