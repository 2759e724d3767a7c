// Softmax top-k selection by one wave, shared by the router kernels
// ("Red Lite dev21 - GPU-routed decode", "What changed": candidates ordered by
// logit, ties to the lower index; weights renormalised over the selected
// experts; expert lookups in the residency table).
#pragma once

#include "rl_common.h"

namespace rl {

// ------------------------------------------------------------ selection
// Top-k of E logits by one wave (lane l owns experts l + 64*i, i < N), as
// the unique first k of the order (logit descending, expert index ascending).
// A single wave issues one instruction per 4 cycles, so the serial part is
// kept to a few hundred instructions:
//  1. Each lane's largest key; t = the k-th largest of those 64 lane maxima
//     (bisection over 32 bits, one ballot per step, early exit).  k lanes
//     hold a key >= t, so every one of the top k keys is >= t.
//  2. The keys >= t (usually 10-20) are compacted into LDS; if more than 64
//     (heavy ties), t becomes the exact k-th largest key by bisection over
//     all keys and only the k first in index order among keys equal to t
//     are kept.
//  3. Each candidate's rank = number of candidates before it in the order;
//     ranks < k give sel_ids[rank], sel_lg[rank] in LDS.
// s_key / s_idx: LDS scratch of at least 64 entries each, 16-byte aligned.
template <int N>
__device__ inline void wave_topk(const float* __restrict__ lg, int E, int k,
                                 uint32_t* s_key, int* s_idx, int* sel_ids, float* sel_lg) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  float lv[N];
#pragma unroll
  for (int i = 0; i < N; ++i) lv[i] = lg[lane + 64 * i < E ? lane + 64 * i : 0];
  uint32_t key[N];
  uint32_t lmax = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    key[i] = lane + 64 * i < E ? float_key(lv[i]) : 0u;
    lmax = key[i] > lmax ? key[i] : lmax;
  }
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    const int cnt = __popcll(__ballot(lmax >= cand));
    if (cnt >= k) {
      t = cand;
      if (cnt == k) break;
    }
  }
  int n_cand = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) n_cand += __popcll(__ballot(key[i] >= t));
  int n_take_eq = 1 << 30;           // keys equal to t that may be taken
  if (n_cand > 64) {                 // heavy ties: exact k-th largest key
    t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) cnt += __popcll(__ballot(key[i] >= cand));
      if (cnt >= k) t = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) n_gt += __popcll(__ballot(key[i] > t));
    n_take_eq = k - n_gt;
  }
  int pos_base = 0, eq_base = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const unsigned long long eqm = __ballot(key[i] == t);
    const int eq_rank = eq_base + __popcll(eqm & below);
    const bool take = key[i] > t || (key[i] == t && eq_rank < n_take_eq);
    const unsigned long long tm = __ballot(take);
    if (take) {
      const int pos = pos_base + __popcll(tm & below);
      s_key[pos] = key[i];
      s_idx[pos] = lane + 64 * i;
    }
    pos_base += __popcll(tm);
    eq_base += __popcll(eqm);
  }
  const int C = pos_base;            // candidates in LDS, k <= C <= 64
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const uint32_t mk = s_key[lane];
  const int mi = s_idx[lane];
  int rank = 0;
  for (int j0 = 0; j0 < C; j0 += 16) {   // 16 candidates per batch of vector LDS reads
    uint4 kq[4];
    int4 iq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kq[u] = *reinterpret_cast<const uint4*>(s_key + j0 + 4 * u);
      iq[u] = *reinterpret_cast<const int4*>(s_idx + j0 + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t kv[4] = {kq[u].x, kq[u].y, kq[u].z, kq[u].w};
      const int iv[4] = {iq[u].x, iq[u].y, iq[u].z, iq[u].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool valid = j0 + 4 * u + v < C;
        rank += (valid && (kv[v] > mk || (kv[v] == mk && iv[v] < mi))) ? 1 : 0;
      }
    }
  }
  if (lane < C && rank < k) {
    sel_ids[rank] = mi;
    sel_lg[rank] = key_float(mk);   // the key holds the logit exactly
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Weights, slots and miss count of one token from the selection in LDS.
// Returns the token's miss count (in every lane).
__device__ inline int finish_token(const int* sel_ids, const float* sel_lg, int k, int E,
                                   int n_slots, const int32_t* res_row, int32_t* ids,
                                   float* weights, int32_t* slots) {
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
  int slot = -1;
  if (lane < k) {
    const int e = min(max(sel_ids[lane], 0), E - 1);   // in bounds even for NaN logits
    const int v = res_row[e];
    slot = (v >= 0 && v < n_slots) ? v : -1;
    ids[lane] = e;
    weights[lane] = float(a / total);
    slots[lane] = slot;
  }
  return __popcll(__ballot(lane < k && slot < 0));
}


}  // namespace rl
