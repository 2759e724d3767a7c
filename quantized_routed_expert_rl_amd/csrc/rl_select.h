// Softmax top-k selection by one wave, shared by the router kernels
// ("Red Lite dev21 - GPU-routed decode", "What changed": candidates ordered by
// logit, ties to the lower index; weights renormalised over the selected
// experts; expert lookups in the residency table).
#pragma once

#include "rl_common.h"

namespace rl {

// ------------------------------------------------------------ selection
// LDS of one selecting wave.
struct TopkLds {
  uint32_t gm[64];              // group maxima
  unsigned long long ck[128];   // candidates: key << 32 | (0xffff - expert); 64.. unused slots
  int cr[128];                  // the candidates' residency entries
};

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int CTRL, int ROWMASK>
__device__ inline int dpp_add_i32(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWMASK, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ inline int wave_incl_scan(int v) {
  v = dpp_add_i32<0x111, 0xf>(v);   // row_shr:1
  v = dpp_add_i32<0x112, 0xf>(v);   // row_shr:2
  v = dpp_add_i32<0x114, 0xf>(v);   // row_shr:4
  v = dpp_add_i32<0x118, 0xf>(v);   // row_shr:8
  v = dpp_add_i32<0x142, 0xa>(v);   // row_bcast:15
  v = dpp_add_i32<0x143, 0xc>(v);   // row_bcast:31
  return v;
}

template <int QP>
__device__ inline uint32_t quad_max(uint32_t x) {
  const uint32_t o = uint32_t(__builtin_amdgcn_mov_dpp(int(x), QP, 0xf, 0xf, false));
  return o > x ? o : x;
}

// 1 if a > b for 31-bit values, from the sign of the difference (no compare
// mask, so no trip through a condition register).
__device__ inline int gt31(uint32_t a, uint32_t b) { return int((b - a) >> 31); }

// Top-k of E logits by one wave (lane l owns experts N*l .. N*l + N-1), as
// the unique first k of the order (logit descending, expert index
// ascending).  A single wave issues one instruction per 4 cycles and pays
// for every trip between its vector and scalar units and through condition
// registers, so each step is a short run of independent vector arithmetic:
//  1. A threshold t from group maxima (groups of 4 lanes when k <= 16, else
//     single lanes): t is the smallest group maximum with fewer than k
//     group maxima above it, comparing keys shifted right by one bit.  The
//     shift can only merge keys, which only lowers t; at least k groups
//     have a maximum >= t, so every one of the top k keys is >= t.
//  2. The keys >= t (usually 10-20) are written to LDS at positions from a
//     prefix sum of the per-lane counts.  If there are more than 64 (heavy
//     ties), t becomes the exact k-th largest key (bisection over all keys)
//     and only the first keys equal to t in index order are kept.
//  3. Each candidate's rank = number of candidates before it in the order,
//     one 64-bit compare each; ranks < k give sel_ids[rank], sel_lg[rank]
//     and, when a residency row res_row is given, sel_res[rank] =
//     res_row[expert] (loaded with the logits, so no lookup follows).
// Keys of experts >= E are 0 and never taken (t >= 1).
template <int N>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lg, int E, int k,
                                          const int32_t* __restrict__ res_row, TopkLds& s,
                                          int* sel_ids, float* sel_lg, int* sel_res) {
  const int lane = threadIdx.x & 63;
  uint32_t key[N];
  int res[N];
  const bool vec = N >= 4 && (E & 3) == 0 && (reinterpret_cast<uintptr_t>(lg) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(res_row) & 15) == 0;
  if (vec) {                          // whole 16-byte chunks are in or out of range
#pragma unroll
    for (int c = 0; c < (N >= 4 ? N / 4 : 1); ++c) {
      const int e0 = N * lane + 4 * c;
      const bool in = e0 + 4 <= E;
      const float4 v = *reinterpret_cast<const float4*>(lg + (in ? e0 : 0));
      int4 rv = make_int4(0, 0, 0, 0);
      if (res_row) rv = *reinterpret_cast<const int4*>(res_row + (in ? e0 : 0));
      const float f[4] = {v.x, v.y, v.z, v.w};
      const int rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (4 * c + u < N) {
          key[4 * c + u] = in ? float_key(f[u]) : 0u;
          res[4 * c + u] = rr[u];
        }
      }
    }
  } else {
    float lv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = N * lane + i < E ? N * lane + i : 0;
      lv[i] = lg[e];
      res[i] = res_row ? res_row[e] : 0;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) key[i] = N * lane + i < E ? float_key(lv[i]) : 0u;
  }
  uint32_t gmax = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) gmax = key[i] > gmax ? key[i] : gmax;
  // 1. threshold
  uint32_t t;
  if (k <= 16) {
    gmax = quad_max<0xb1>(gmax);      // quad_perm [1,0,3,2]
    gmax = quad_max<0x4e>(gmax);      // quad_perm [2,3,0,1]
    if ((lane & 3) == 0) s.gm[lane >> 2] = gmax;
    wave_lds_sync();
    const uint32_t mine = gmax >> 1;
    int gt = 0;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&s.gm[j]);
      gt += gt31(q.x >> 1, mine) + gt31(q.y >> 1, mine) + gt31(q.z >> 1, mine) +
            gt31(q.w >> 1, mine);
    }
    t = wave_min_u32(gt < k ? gmax : 0xffffffffu);
  } else {
    s.gm[lane] = gmax;
    wave_lds_sync();
    const uint32_t mine = gmax >> 1;
    int gt = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&s.gm[j]);
      gt += gt31(q.x >> 1, mine) + gt31(q.y >> 1, mine) + gt31(q.z >> 1, mine) +
            gt31(q.w >> 1, mine);
    }
    t = wave_min_u32(gt < k ? gmax : 0xffffffffu);
  }
  t = t > 1u ? t : 1u;
  // 2. candidates
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) cnt += key[i] >= t ? 1 : 0;
  int incl = wave_incl_scan(cnt);
  int C = __builtin_amdgcn_readlane(incl, 63);
  int n_take_eq = 1 << 30;            // keys equal to t that may be taken
  int eq_before = 0;                  // keys equal to t in lanes below this one
  if (C > 64) {                       // heavy ties: exact k-th largest key
    t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) c += key[i] >= cand ? 1 : 0;
      if (__builtin_amdgcn_readlane(wave_incl_scan(c), 63) >= k) t = cand;
    }
    t = t > 1u ? t : 1u;
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      ngt += key[i] > t ? 1 : 0;
      neq += key[i] == t ? 1 : 0;
    }
    n_take_eq = k - __builtin_amdgcn_readlane(wave_incl_scan(ngt), 63);
    const int eq0 = wave_incl_scan(neq) - neq;
    eq_before = eq0;
    cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool take = key[i] > t || (key[i] == t && eq_before < n_take_eq);
      eq_before += key[i] == t ? 1 : 0;
      cnt += take ? 1 : 0;
    }
    incl = wave_incl_scan(cnt);
    C = __builtin_amdgcn_readlane(incl, 63);
    eq_before = eq0;
  }
  // branch-free writes: a key that is not taken goes to this lane's unused slot
  int pos = incl - cnt;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool take = key[i] > t || (key[i] == t && eq_before < n_take_eq);
    eq_before += key[i] == t ? 1 : 0;
    const int at = take ? pos : 64 + lane;
    s.ck[at] = (static_cast<unsigned long long>(key[i]) << 32) |
               static_cast<unsigned long long>(0xffffu - unsigned(N * lane + i));
    s.cr[at] = res[i];
    pos += take ? 1 : 0;
  }
  const int Cpad = (C + 7) & ~7;
  if (lane >= C && lane < Cpad) s.ck[lane] = 0ull;   // padding never outranks a candidate
  wave_lds_sync();
  // 3. ranks
  const unsigned long long mine = s.ck[lane];
  const int mres = s.cr[lane];
  int rank = 0;
  for (int j0 = 0; j0 < C; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(&s.ck[j0 + 2 * u]);
      rank += (v.x > mine) + (v.y > mine);
    }
  }
  if (lane < C && rank < k) {
    sel_ids[rank] = int(0xffffu - unsigned(mine & 0xffffu));
    sel_lg[rank] = key_float(uint32_t(mine >> 32));   // the key holds the logit exactly
    if (sel_res) sel_res[rank] = mres;
  }
  wave_lds_sync();
}

// Slot of a selected expert from its residency entry: entries outside
// [0, n_slots) mean not resident (-1).
__device__ inline int slot_of(int v, int n_slots) { return (v >= 0 && v < n_slots) ? v : -1; }

// Renormalised softmax weight of the lane's rank (lanes < k) from the
// selected logits in LDS, sel_lg[0] the largest: exp(l_r - l_0) over their
// sum in rank order, in float64.  Every block that needs the weights calls
// this, so they agree bit for bit.
__device__ __forceinline__ float selected_weight(const float* sel_lg, int k) {
  const int lane = threadIdx.x & 63;
  double a = 0.0;
  if (lane < k) a = exp(double(sel_lg[lane]) - double(sel_lg[0]));
  double total = 0.0;
  for (int r = 0; r < k; ++r) {  // rank order, summed in scalar registers
    const long long bits = __double_as_longlong(a);
    const int lo = __builtin_amdgcn_readlane(int(bits & 0xffffffffll), r);
    const int hi = __builtin_amdgcn_readlane(int(bits >> 32), r);
    total += __longlong_as_double((static_cast<long long>(hi) << 32) |
                                  static_cast<unsigned int>(lo));
  }
  return float(a / total);
}

// Weights, slots and miss count of one token from the selection in LDS
// (sel_res: the selected experts' residency entries).  Returns the token's
// miss count (in every lane).
__device__ __forceinline__ int finish_token(const int* sel_ids, const float* sel_lg, const int* sel_res,
                                   int k, int E, int n_slots, int32_t* ids, float* weights,
                                   int32_t* slots) {
  const int lane = threadIdx.x & 63;
  const float w = selected_weight(sel_lg, k);
  int slot = -1;
  if (lane < k) {
    const int e = min(max(sel_ids[lane], 0), E - 1);   // in bounds even for NaN logits
    slot = slot_of(sel_res[lane], n_slots);
    ids[lane] = e;
    weights[lane] = w;
    slots[lane] = slot;
  }
  return __popcll(__ballot(lane < k && slot < 0));
}

}  // namespace rl
