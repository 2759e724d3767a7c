// Prefill chunk after routing ("Red Lite dev20 - batched prompt ingestion",
// "What changed"): the chunk's plan (consecutive token groups whose union of
// selected experts stays within the plan cap; per group the (expert, token)
// pairs sorted by expert), the batched gate/up and down projections over the
// pairs, and the per-token sum of the k expert outputs in router selection
// order.  Every kernel returns at once when the chunk's early-out flag is set
// ("Red Lite dev23", "What changed").
#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_select.h"

namespace rl {

constexpr int kTileTokens = 8;   // tokens of one bucket per VALU work item

// ----------------------------------------------------------------- plan
// Greedy consecutive token groups, one wave.  A token joins the current
// group unless the union of selected experts would exceed plan_cap.
__global__ __launch_bounds__(64) void plan_groups_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int plan_cap,
    const uint32_t* __restrict__ early_out, int32_t* n_groups, int32_t* group_bounds) {
  if (*early_out) return;
  const int lane = threadIdx.x;
  if (plan_cap >= E) {   // a union never exceeds E distinct experts
    if (lane == 0) {
      *n_groups = 1;
      group_bounds[0] = 0;
      group_bounds[1] = T;
    }
    return;
  }
  __shared__ uint32_t bits[32];   // E <= 1024
  if (lane < 32) bits[lane] = 0u;
  __syncthreads();
  if (lane == 0) group_bounds[0] = 0;
  int ng = 0, start = 0, ucount = 0;
  for (int t = 0; t < T; ++t) {
    const int e = lane < k ? ids[int64_t(t) * k + lane] : 0;
    const bool in = lane < k && ((bits[e >> 5] >> (e & 31)) & 1u);
    int nnew = __popcll(__ballot(lane < k && !in));
    if (t > start && ucount + nnew > plan_cap) {
      ++ng;
      if (lane == 0) group_bounds[ng] = t;
      start = t;
      __syncthreads();
      if (lane < 32) bits[lane] = 0u;
      ucount = 0;
      nnew = k;
    }
    __syncthreads();
    if (lane < k) atomicOr(&bits[e >> 5], 1u << (e & 31));
    __syncthreads();
    ucount += nnew;
  }
  if (lane == 0) {
    group_bounds[ng + 1] = T;
    *n_groups = ng + 1;
  }
}

// One wave per expert walks the pairs of each group in order, 16 experts per
// block; the pairs' expert ids are staged in LDS kPairChunk at a time, so
// each id is read from memory once per block.  COUNT mode stores the number
// of pairs of (group, expert); SCATTER mode writes each matching pair id at
// offs[(group, expert)] + its rank among the matches (so the order inside a
// bucket is the pair order: stable).
constexpr int kPairChunk = 8192;

template <bool SCATTER>
__global__ __launch_bounds__(1024) void plan_pairs_kernel(
    const int32_t* __restrict__ ids, int k, int E, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_groups, const int32_t* __restrict__ group_bounds,
    int32_t* __restrict__ counts, const int32_t* __restrict__ offs, int32_t* __restrict__ pairs) {
  if (*early_out) return;
  __shared__ int s_ids[kPairChunk];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 16 + wv;
  const bool live = e < E;
  const unsigned long long below = (1ull << lane) - 1ull;
  const int ng = *n_groups;
  for (int g = 0; g < ng; ++g) {
    const int p0 = group_bounds[g] * k, p1 = group_bounds[g + 1] * k;
    int run = (SCATTER && live) ? offs[int64_t(g) * E + e] : 0;
    for (int c0 = p0; c0 < p1; c0 += kPairChunk) {
      const int cn = p1 - c0 < kPairChunk ? p1 - c0 : kPairChunk;
      __syncthreads();                     // the previous chunk has been scanned
      for (int i = threadIdx.x; i < cn; i += blockDim.x) s_ids[i] = ids[c0 + i];
      __syncthreads();
      if (live) {
        for (int base = 0; base < cn; base += 64) {
          const int i = base + lane;
          const bool m = i < cn && s_ids[i < cn ? i : 0] == e;
          const unsigned long long mask = __ballot(m);
          if (SCATTER && m) pairs[run + __popcll(mask & below)] = c0 + i;
          run += __popcll(mask);
        }
      }
    }
    if (!SCATTER && live && lane == 0) counts[int64_t(g) * E + e] = run;
  }
}

// Exclusive scan of three ints over a block of exactly 1024 threads; the
// block totals come back in tot[].  Every thread reaches every barrier.
__device__ inline void block_scan3(int v[3], int tot[3]) {
  __shared__ int s_w[16][3];
  __shared__ int s_tot[3];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int x = v[c];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    inc[c] = x;
    if (lane == 63) s_w[wv][c] = x;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = s_w[w][threadIdx.x];
      s_w[w][threadIdx.x] = run;
      run += t;
    }
    s_tot[threadIdx.x] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    v[c] = s_w[wv][c] + inc[c] - v[c];
    tot[c] = s_tot[c];
  }
  __syncthreads();
}

__device__ inline int v2_tiles(int c, int tile_tokens) { return (c + tile_tokens - 1) / tile_tokens; }

// Offsets of every (group, expert) run of pairs, the bucket list, each
// bucket's slot and its first token tile.
__global__ __launch_bounds__(1024) void plan_scan_kernel(
    int E, int layer, const int32_t* __restrict__ residency,
    const uint32_t* __restrict__ early_out, const int32_t* __restrict__ n_groups,
    const int32_t* __restrict__ counts, int32_t* offs, int32_t* n_buckets,
    int32_t* group_bucket_start, int32_t* bucket_expert, int32_t* bucket_start,
    int32_t* bucket_slot, int32_t* tile_start, int32_t* n_tiles, int32_t* tile_bucket,
    int tile_tokens) {
  if (*early_out) return;
  const int ng = *n_groups;
  const int n = ng * E;
  int carry[3] = {0, 0, 0};   // pairs, buckets, tiles
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int c = i < n ? counts[i] : 0;
    int v[3] = {c, c > 0 ? 1 : 0, (c + tile_tokens - 1) / tile_tokens};
    int tot[3];
    block_scan3(v, tot);
    if (i < n) {
      const int e = i % E;
      offs[i] = carry[0] + v[0];
      if (e == 0) group_bucket_start[i / E] = carry[1] + v[1];
      if (c > 0) {
        const int b = carry[1] + v[1];
        bucket_expert[b] = e;
        bucket_start[b] = carry[0] + v[0];
        bucket_slot[b] = residency[int64_t(layer) * E + e];
        tile_start[b] = carry[2] + v[2];
        for (int u = 0; u < v2_tiles(c, tile_tokens); ++u) tile_bucket[carry[2] + v[2] + u] = b;
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) carry[q] += tot[q];
  }
  if (threadIdx.x == 0) {
    *n_buckets = carry[1];
    bucket_start[carry[1]] = carry[0];
    tile_start[carry[1]] = carry[2];
    *n_tiles = carry[2];
    group_bucket_start[ng] = carry[1];
  }
}

// The whole plan in one block when the chunk forms a single token group
// (plan_cap >= E) and its pairs fit in LDS.  The pairs are cut into 16
// consecutive segments, one per wave; per-(segment, expert) counts give each
// wave its base inside every expert's run, and a wave walks its segment 64
// pairs at a time, ranking each pair among the equal experts before it in
// the batch, so every bucket holds its pairs in pair order (stable), exactly
// as the per-expert scan above.
constexpr int kFusedMaxPairs = 16384;
constexpr int kFusedMaxExperts = 1024;

__global__ __launch_bounds__(1024) void plan_fused_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int layer,
    const int32_t* __restrict__ residency, const uint32_t* __restrict__ early_out, PlanPtrs p,
    int tile_tokens) {
  if (*early_out) return;
  __shared__ int s_ids[kFusedMaxPairs];
  __shared__ int s_cnt[16][kFusedMaxExperts];   // per (segment, expert): count, then base
  __shared__ int s_off[kFusedMaxExperts];       // start of each expert's run
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int P = T * k;
  const int seg = ((P + 15) / 16 + 63) & ~63;   // pairs per segment, whole batches
  for (int i = tid; i < P; i += 1024) s_ids[i] = ids[i];
  for (int i = tid; i < 16 * kFusedMaxExperts; i += 1024) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const int s0 = wv * seg, s1 = min(P, s0 + seg);
  for (int i = s0 + lane; i < s1; i += 64) atomicAdd(&s_cnt[wv][s_ids[i]], 1);
  __syncthreads();
  // per expert: total count and each segment's base inside the expert's run
  int total = 0;
  if (tid < E) {
    for (int w = 0; w < 16; ++w) {
      const int c = s_cnt[w][tid];
      s_cnt[w][tid] = total;
      total += c;
    }
  }
  int v[3] = {total, total > 0 ? 1 : 0, (total + tile_tokens - 1) / tile_tokens};
  int tot[3];
  block_scan3(v, tot);
  if (tid < E) {
    p.counts[tid] = total;
    p.offs[tid] = v[0];
    s_off[tid] = v[0];
    if (total > 0) {
      const int b = v[1];
      p.bucket_expert[b] = tid;
      p.bucket_start[b] = v[0];
      p.bucket_slot[b] = residency[int64_t(layer) * E + tid];
      p.tile_start[b] = v[2];
      for (int u = 0; u < (total + tile_tokens - 1) / tile_tokens; ++u) p.tile_bucket[v[2] + u] = b;
    }
  }
  if (tid == 0) {
    *p.n_groups = 1;
    p.group_bounds[0] = 0;
    p.group_bounds[1] = T;
    *p.n_buckets = tot[1];
    p.group_bucket_start[0] = 0;
    p.group_bucket_start[1] = tot[1];
    p.bucket_start[tot[1]] = tot[0];
    p.tile_start[tot[1]] = tot[2];
    *p.n_tiles = tot[2];
  }
  __syncthreads();
  // stable scatter, wave wv over its segment in order.  Per batch the high
  // half of s_cnt[wv][e] counts the batch's pairs of expert e (LDS adds, so
  // the count is exact whatever order the lanes are served in); a pair whose
  // expert is unique in the batch has rank 0, and only repeated experts are
  // ranked by ballots, one distinct expert per round.
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int b0 = s0; b0 < s1; b0 += 64) {
    const int i = b0 + lane;
    const bool live = i < s1;
    const int e = live ? s_ids[i] : 0;
    if (live) atomicAdd(&s_cnt[wv][e], 1 << 16);
    wave_lds_sync();
    const int cb = live ? s_cnt[wv][e] : 0;
    const int cnt = cb >> 16, base = cb & 0xffff;
    int rank = 0;
    unsigned long long todo = __ballot(cnt > 1);
    while (todo) {
      const int e0 = __builtin_amdgcn_readlane(e, __builtin_ctzll(todo));
      const unsigned long long m = __ballot(live && e == e0);
      if (live && e == e0) rank = __popcll(m & below);
      todo &= ~m;
    }
    if (live) p.pairs[s_off[e] + base + rank] = i;
    wave_lds_sync();
    if (live && rank == cnt - 1) s_cnt[wv][e] = base + cnt;   // the batch's last pair of e
    wave_lds_sync();
  }
}

// ---------------------------------------------------- batched experts
// Bucket of a token tile: last b with tile_start[b] <= tile.
__device__ inline int find_tile_bucket(const int32_t* tile_start, int nb, int tile) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Decode one lane's 32 weights of a group to float32 (exact values).
template <int QBITS>
__device__ inline void group_weights(const Group32& g, float* w) {
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    const uint32_t dw = n < 16 ? g.c0 : g.c1;
    uint32_t c = (dw >> (2 * (n & 15))) & 3u;
    if (QBITS == 3) {
      c |= ((g.hi >> n) & 1u) << 2;
      w[n] = g.scale * 0.5f * (float(c) - 3.5f);
    } else {
      w[n] = g.scale * (float(c) - 1.5f);
    }
  }
}

// Gate/up for one token tile of one bucket, all F rows j.  Activations of
// the tile's tokens staged in LDS; each lane decodes its group's 32 weights
// once per row and applies them to every token of the tile.
template <int QBITS, int LPR>
__global__ __launch_bounds__(256) void prefill_gateup_kernel(
    PoolView pv, int H, int F, int k, const float* __restrict__ x,
    const uint32_t* __restrict__ early_out, const int32_t* __restrict__ n_buckets_p,
    const int32_t* __restrict__ n_tiles_p, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ bucket_start, const int32_t* __restrict__ bucket_slot,
    const int32_t* __restrict__ pairs, float* __restrict__ hbuf) {
  if (*early_out) return;
  constexpr int RPI = 64 / LPR;
  extern __shared__ float xs[];          // [kTileTokens][H]
  __shared__ float s_gu[4][2][RPI][kTileTokens];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int seg = lane % LPR, rs = lane / LPR;
  const int nb = *n_buckets_p, ntiles = *n_tiles_p;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int b = find_tile_bucket(tile_start, nb, tile);
    const int pos0 = bucket_start[b] + (tile - tile_start[b]) * kTileTokens;
    const int pend = bucket_start[b + 1];
    const int nt = pend - pos0 < kTileTokens ? pend - pos0 : kTileTokens;
    const int slot = bucket_slot[b];
    __syncthreads();
    for (int q = threadIdx.x; q < nt * (H / 4); q += 256) {
      const int n = q / (H / 4), c = q % (H / 4);
      const int t = pairs[pos0 + n] / k;
      reinterpret_cast<float4*>(xs)[n * (H / 4) + c] =
          reinterpret_cast<const float4*>(x + int64_t(t) * H)[c];
    }
    __syncthreads();
    const uint8_t* gate = tensor_base(pv, slot, 0);
    const uint8_t* up = tensor_base(pv, slot, 1);
    // wave iteration: RPI consecutive j, gate and up
    for (int jb = wv * RPI; jb < F; jb += 4 * RPI) {
      const int j = jb + rs;
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const Group32 g = load_group<QBITS>(which ? up : gate, pv, int64_t(j) * H + 32 * seg);
        float w[32];
        group_weights<QBITS>(g, w);
        for (int n = 0; n < nt; ++n) {
          const float* xr = xs + n * H + 32 * seg;
          float acc = 0.f;
#pragma unroll
          for (int q = 0; q < 32; ++q) acc = fmaf(w[q], xr[q], acc);
          acc = wave_sum_width(acc, LPR);
          if (seg == 0) s_gu[wv][which][rs][n] = acc;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      for (int q = lane; q < RPI * nt; q += 64) {
        const int rr = q / nt, n = q % nt;
        hbuf[int64_t(pos0 + n) * F + jb + rr] =
            silu_mul(s_gu[wv][0][rr][n], s_gu[wv][1][rr][n]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
}

// Down projection for one token tile of one bucket and a range of 256 rows
// i; results go to ebuf row p (the pair id), so each token's k outputs are
// adjacent for the ordered sum.
template <int QBITS, int LPR>
__global__ __launch_bounds__(256) void prefill_down_kernel(
    PoolView pv, int H, int F, const uint32_t* __restrict__ early_out,
    const int32_t* __restrict__ n_buckets_p, const int32_t* __restrict__ n_tiles_p,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ bucket_start,
    const int32_t* __restrict__ bucket_slot, const int32_t* __restrict__ pairs,
    const float* __restrict__ hbuf, float* __restrict__ ebuf) {
  if (*early_out) return;
  constexpr int RPI = 64 / LPR;
  constexpr int ROWS = 256;
  extern __shared__ float hs[];          // [kTileTokens][F]
  __shared__ float s_e[4][RPI][kTileTokens];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int seg = lane % LPR, rs = lane / LPR;
  const int nb = *n_buckets_p, ntiles = *n_tiles_p;
  const int nrt = (H + ROWS - 1) / ROWS;
  for (int item = blockIdx.x; item < ntiles * nrt; item += gridDim.x) {
    const int tile = item / nrt, rt = item % nrt;
    const int b = find_tile_bucket(tile_start, nb, tile);
    const int pos0 = bucket_start[b] + (tile - tile_start[b]) * kTileTokens;
    const int pend = bucket_start[b + 1];
    const int nt = pend - pos0 < kTileTokens ? pend - pos0 : kTileTokens;
    const int slot = bucket_slot[b];
    __syncthreads();
    for (int q = threadIdx.x; q < nt * (F / 4); q += 256) {
      const int n = q / (F / 4), c = q % (F / 4);
      reinterpret_cast<float4*>(hs)[n * (F / 4) + c] =
          reinterpret_cast<const float4*>(hbuf + int64_t(pos0 + n) * F)[c];
    }
    __syncthreads();
    const uint8_t* down = tensor_base(pv, slot, 2);
    const int i_end = (rt + 1) * ROWS < H ? (rt + 1) * ROWS : H;
    for (int ib = rt * ROWS + wv * RPI; ib < i_end; ib += 4 * RPI) {
      const int i = ib + rs;
      const Group32 g = load_group<QBITS>(down, pv, int64_t(i) * F + 32 * seg);
      float w[32];
      group_weights<QBITS>(g, w);
      for (int n = 0; n < nt; ++n) {
        const float* hr = hs + n * F + 32 * seg;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 32; ++q) acc = fmaf(w[q], hr[q], acc);
        acc = wave_sum_width(acc, LPR);
        if (seg == 0) s_e[wv][rs][n] = acc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      for (int q = lane; q < RPI * nt; q += 64) {
        const int rr = q / nt, n = q % nt;
        ebuf[int64_t(pairs[pos0 + n]) * H + ib + rr] = s_e[wv][rr][n];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
}

// y[t][i] = sum_r w[t][r] * ebuf[t*k + r][i], fused multiply-add from 0 in
// rank order.
__global__ __launch_bounds__(256) void prefill_sum_kernel(
    int H, int k, const float* __restrict__ weights, const float* __restrict__ ebuf,
    const uint32_t* __restrict__ early_out, float* __restrict__ y) {
  if (*early_out) return;
  const int t = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  float acc = 0.f;
  for (int r = 0; r < k; ++r)
    acc = fmaf(weights[int64_t(t) * k + r], ebuf[(int64_t(t) * k + r) * H + i], acc);
  y[int64_t(t) * H + i] = acc;
}

// ------------------------------------------------------------ launchers
void launch_prefill_plan(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  if (a.plan_cap >= a.E && a.T * a.k <= kFusedMaxPairs && a.E <= kFusedMaxExperts) {
    plan_fused_kernel<<<1, 1024, 0, st>>>(a.ids, a.T, a.k, a.E, a.layer, a.residency,
                                          a.early_out, p, a.tile_tokens);
    return;
  }
  plan_groups_kernel<<<1, 64, 0, st>>>(a.ids, a.T, a.k, a.E, a.plan_cap, a.early_out,
                                       p.n_groups, p.group_bounds);
  const int blocks = (a.E + 15) / 16;
  plan_pairs_kernel<false><<<blocks, 1024, 0, st>>>(a.ids, a.k, a.E, a.early_out, p.n_groups,
                                                   p.group_bounds, p.counts, nullptr, nullptr);
  plan_scan_kernel<<<1, 1024, 0, st>>>(a.E, a.layer, a.residency, a.early_out, p.n_groups,
                                       p.counts, p.offs, p.n_buckets, p.group_bucket_start,
                                       p.bucket_expert, p.bucket_start, p.bucket_slot,
                                       p.tile_start, p.n_tiles, p.tile_bucket, a.tile_tokens);
  plan_pairs_kernel<true><<<blocks, 1024, 0, st>>>(a.ids, a.k, a.E, a.early_out, p.n_groups,
                                                  p.group_bounds, nullptr, p.offs, p.pairs);
}

template <int QBITS, int LPR>
static void launch_gateup_q(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  const size_t lds = size_t(kTileTokens) * a.H * sizeof(float);
  prefill_gateup_kernel<QBITS, LPR><<<1024, 256, lds, st>>>(
      a.pool, a.H, a.F, a.k, a.x, a.early_out, p.n_buckets, p.n_tiles, p.tile_start,
      p.bucket_start, p.bucket_slot, p.pairs, a.hbuf);
}

template <int QBITS, int LPR>
static void launch_down_q(const PrefillArgs& a, hipStream_t st) {
  const PlanPtrs& p = a.plan;
  const size_t lds = size_t(kTileTokens) * a.F * sizeof(float);
  prefill_down_kernel<QBITS, LPR><<<2048, 256, lds, st>>>(
      a.pool, a.H, a.F, a.early_out, p.n_buckets, p.n_tiles, p.tile_start, p.bucket_start,
      p.bucket_slot, p.pairs, a.hbuf, a.ebuf);
}

template <int QBITS>
static void gateup_q(const PrefillArgs& a, hipStream_t st) {
  switch (a.H / 32) {
    case 8: launch_gateup_q<QBITS, 8>(a, st); break;
    case 16: launch_gateup_q<QBITS, 16>(a, st); break;
    case 32: launch_gateup_q<QBITS, 32>(a, st); break;
    default: launch_gateup_q<QBITS, 64>(a, st); break;
  }
}

template <int QBITS>
static void down_q(const PrefillArgs& a, hipStream_t st) {
  switch (a.F / 32) {
    case 1: launch_down_q<QBITS, 1>(a, st); break;
    case 2: launch_down_q<QBITS, 2>(a, st); break;
    case 4: launch_down_q<QBITS, 4>(a, st); break;
    case 8: launch_down_q<QBITS, 8>(a, st); break;
    case 16: launch_down_q<QBITS, 16>(a, st); break;
    case 32: launch_down_q<QBITS, 32>(a, st); break;
    default: launch_down_q<QBITS, 64>(a, st); break;
  }
}

void launch_prefill_gateup(const PrefillArgs& a, hipStream_t st) {
  if (a.mfma) {
    launch_quantize_x(a, st);
    launch_prefill_gateup_mfma(a, st);
  } else if (a.qbits == 3) {
    gateup_q<3>(a, st);
  } else {
    gateup_q<2>(a, st);
  }
}

void launch_prefill_down(const PrefillArgs& a, hipStream_t st) {
  if (a.mfma) {
    launch_quantize_h(a, st);
    launch_prefill_down_mfma(a, st);
  } else if (a.qbits == 3) {
    down_q<3>(a, st);
  } else {
    down_q<2>(a, st);
  }
}

void launch_prefill_sum(const PrefillArgs& a, hipStream_t st) {
  dim3 grid(a.H / 256, a.T);
  prefill_sum_kernel<<<grid, 256, 0, st>>>(a.H, a.k, a.weights, a.ebuf, a.early_out, a.y);
}

}  // namespace rl
