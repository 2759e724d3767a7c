// Single-token decode expert GEMVs on the int8 matrix cores of gfx950, for
// 2-bit and 3-bit block weights when the expert width is a multiple of 256
// (the operands are described in rl_mfma.h).  Same three-kernel structure and
// routing rules as decode.hip ("Red Lite dev21 - GPU-routed decode", "What
// changed"; "Red Lite dev23", "What changed": with the flag set every expert
// kernel returns at once; "Red Lite dev20", "What changed": a token's experts
// are summed in router selection order).
//
// Diagonal tiles.  A GEMV has one activation vector, so of the 16 columns of
// an MFMA only the 4 digit columns would carry data.  Instead a 16-row A tile
// holds RPT = 16/BPT output rows times BPT 256-value K-blocks (A row
// rho = BPT*i + beta), and B column c = 4*beta' + digit holds the digits of
// K-block beta'.  Output entry (rho, c) is wanted when beta == beta', i.e.
// the diagonal 4x4 blocks; the rest is discarded.  Output lane l holds rows
// 4*(l/16) + v, so every wanted entry of output row i sits in the 16-lane
// group l/16 = BPT*i/4, and one DPP sum over that group finishes the row.
#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_mfma.h"
#include "rl_select.h"

namespace rl {

int cand_per_lane(int E);

__device__ inline int sel4(const v4i& D, int v) {
  return v == 0 ? D.x : v == 1 ? D.y : v == 2 ? D.z : D.w;
}

// B operand of tile half h (K-blocks BPT*h .. BPT*h + BPT - 1) from the
// digit operands of a vector (KB blocks of 1024 bytes in LDS).  Columns of
// blocks beta' >= BPT are zero.
template <int BPT>
__device__ inline void load_b_diag(const uint8_t* xq, int h, int lane, v4i B[4]) {
  const int c = lane & 15, beta = c >> 2, d = c & 3, q = lane >> 4;
  const bool ok = beta < BPT;
  const uint8_t* base = xq + ((ok ? beta : 0) + BPT * h) * 1024;
  const int msk = ok ? -1 : 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int4 v = *reinterpret_cast<const int4*>(base + digit_chunk_offset(q, d, m));
    B[m] = v4i{v.x & msk, v.y & msk, v.z & msk, v.w & msk};
  }
}

// Adds the wanted entries of one tile half's int32 result D, scaled to
// float, into acc[il] (output row 4*(lane/16)/BPT + il of the tile).
// dh: the lane's block scale bits from its A tile; xe: exponents of the
// vector's K-blocks.
template <int BPT, int QBITS>
__device__ inline void diag_accumulate(const v4i& D, uint32_t dh, const int* xe, int h, int lane,
                                       float* acc) {
  constexpr int RG = 4 / BPT;
  const int g = lane >> 4, c = lane & 15, bc = c >> 2, dc = c & 3;
  const bool useful = bc < BPT;
  const int b = useful ? bc : 0;
  const int sh = 8 * (3 - dc) - xe[b + BPT * h];
#pragma unroll
  for (int il = 0; il < RG; ++il) {
    const int v = BPT * il + b;
    // block scale of A row 4g + v, held by A lane 4g + v (quad 0)
    const float dq = dh_dq<QBITS>(uint32_t(__shfl(int(dh), 4 * g + v, kWave)));
    const float t = float(sel4(D, v)) * ldexpf(dq, sh);
    acc[il] += useful ? t : 0.f;
  }
}

// Max over the 16 lanes of each DPP row, in every lane of the row (row_ror
// by 1, 2, 4 and 8).
template <int CTRL>
__device__ inline float row_ror_max(float x) {
  const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
  return fmaxf(x, o);
}
__device__ inline float row_max16(float x) {
  x = row_ror_max<0x121>(x);   // row_ror:1
  x = row_ror_max<0x122>(x);   // row_ror:2
  x = row_ror_max<0x124>(x);   // row_ror:4
  x = row_ror_max<0x128>(x);   // row_ror:8
  return x;
}

// One 16-value run of a vector (K = 16*run .. +15), loaded (lanes past the
// end load run 0 and are ignored).
__device__ __forceinline__ void load_run(const float* __restrict__ src, int run, bool act,
                                         float* v) {
  const int k0 = 16 * (act ? run : 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 f = *reinterpret_cast<const float4*>(src + k0 + 4 * u);
    v[4 * u + 0] = f.x;
    v[4 * u + 1] = f.y;
    v[4 * u + 2] = f.z;
    v[4 * u + 3] = f.w;
  }
}

// A loaded run -> its four digit chunks in LDS, with one exponent per
// 256-value block.  The 16 runs of a block must sit in one DPP row (16
// consecutive lanes starting at a multiple of 16), all of which call this.
__device__ __forceinline__ void quantize_loaded(const float* v, int run, bool act, uint8_t* xq,
                                                int* xe) {
  float amax = 0.f;
#pragma unroll
  for (int n = 0; n < 16; ++n) amax = fmaxf(amax, fabsf(v[n]));
  amax = row_max16(act ? amax : 0.f);
  const int e = scale_exp(amax);
  if (act) {
    uint4 ch[4];
    digit_chunks(v, e, ch);
    const int k0 = 16 * run;
    const int kb = k0 >> 8, qq = (k0 & 255) >> 6, mm = (k0 & 63) >> 4;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      *reinterpret_cast<uint4*>(xq + kb * 1024 + digit_chunk_offset(qq, d, mm)) = ch[d];
    if ((k0 & 255) == 0) xe[kb] = e;
  }
}

// -------------------------------------------------- top-k + gate/up
// Grid: k * F/(4*RPT) work blocks + 1 publisher block, 4 waves each.
// Every block selects the experts (wave 0, which loads the residency entries
// of its experts with their logits) while waves 1-2 turn x into digit
// operands in LDS; one barrier joins them.  The publisher computes the
// renormalised weights and writes ids, weights, slots, the miss count and
// the flag; a work block only needs its slots.  Work block = (rank r, 4*RPT rows j); wave w takes
// RPT rows of gate and up over all KB = H/256 K-blocks: 2*NH diagonal tiles.
template <int N, int KB, int QBITS, int NW>
__global__ __launch_bounds__(64 * NW) void decode_topk_gateup_mfma_kernel(
    PoolView pv, int H, int F, int E, int k, int layer, int n_slots,
    const float* __restrict__ x, const float* __restrict__ logits,
    const int32_t* __restrict__ residency, int32_t* ids, float* weights, int32_t* slots,
    uint32_t* miss_count, uint32_t* early_out, float* __restrict__ hbuf, int sticky) {
  if (sticky && *early_out) return;      // a set shared flag stops the whole call
  constexpr int BPT = KB < 4 ? KB : 4;   // K-blocks per tile
  constexpr int RPT = 16 / BPT;          // output rows per tile
  constexpr int NH = KB / BPT;           // tiles per tensor
  constexpr int RG = 4 / BPT;            // output rows per 16-lane group
  __shared__ __align__(16) TopkLds s_tk;
  __shared__ int sel_ids[32];
  __shared__ float sel_lg[32];
  __shared__ int sel_res[32];
  __shared__ int s_slot[32];
  __shared__ int s_miss;
  __shared__ __align__(16) uint8_t s_xq[KB * 1024];
  __shared__ int s_xe[KB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool publisher = blockIdx.x == gridDim.x - 1;
  if (wv == 0) {
    wave_topk<N>(logits, E, k, residency + int64_t(layer) * E, s_tk, sel_ids, sel_lg, sel_res);
    if (publisher) {
      const int miss = finish_token(sel_ids, sel_lg, sel_res, k, E, n_slots, ids, weights, slots);
      if (lane == 0) {
        *miss_count = uint32_t(miss);
        if (!sticky || miss > 0) *early_out = miss > 0 ? 1u : 0u;   // sticky: only raised
      }
    } else {
      const int slot = lane < k ? slot_of(sel_res[lane], n_slots) : 0;
      if (lane < k) s_slot[lane] = slot;
      const int miss = __popcll(__ballot(slot < 0));
      if (lane == 0) s_miss = miss;
    }
  } else if (!publisher) {
    // H/16 <= 128 runs over waves 1-2 (wave 1 alone takes two per lane when
    // the block has two waves); a wave's runs are all below 128 or all above
    for (int run = tid - 64; run < 128; run += 64 * (NW > 2 ? 2 : 1)) {
      float v[16];
      load_run(x, run, run < H / 16, v);
      quantize_loaded(v, run, run < H / 16, s_xq, s_xe);
    }
  }
  if (publisher) return;
  __syncthreads();
  if (s_miss) return;                    // early-out: nothing downstream runs
  const int jpb = NW * RPT;
  const int bpr = F / jpb;
  const int r = blockIdx.x / bpr;
  const int j0 = (blockIdx.x % bpr) * jpb + wv * RPT;
  const int slot = s_slot[r];
  const uint8_t* tg = tensor_base(pv, slot, 0);
  const uint8_t* tu = tensor_base(pv, slot, 1);
  const int rho = lane & 15, q = lane >> 4;
  const int64_t blk = int64_t(j0 + rho / BPT) * KB + rho % BPT;
  TileCodes cg[NH], cu[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    cg[h] = load_tile<QBITS>(tg, pv, blk + BPT * h, q);
    cu[h] = load_tile<QBITS>(tu, pv, blk + BPT * h, q);
  }
  float ag[RG], au[RG];
#pragma unroll
  for (int il = 0; il < RG; ++il) ag[il] = au[il] = 0.f;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    v4i B[4];
    load_b_diag<BPT>(s_xq, h, lane, B);
    const v4i Dg = tile_mfma<QBITS>(cg[h], B);
    const v4i Du = tile_mfma<QBITS>(cu[h], B);
    diag_accumulate<BPT, QBITS>(Dg, cg[h].dh, s_xe, h, lane, ag);
    diag_accumulate<BPT, QBITS>(Du, cu[h].dh, s_xe, h, lane, au);
  }
#pragma unroll
  for (int il = 0; il < RG; ++il) {
    ag[il] = group_sum_last<16>(ag[il]);
    au[il] = group_sum_last<16>(au[il]);
  }
  if ((lane & 15) == 15) {
    const int g = lane >> 4;
#pragma unroll
    for (int il = 0; il < RG; ++il)
      hbuf[int64_t(r) * F + j0 + g * RG + il] = silu_mul(ag[il], au[il]);
  }
}

// ------------------------------------------------- down + ordered sum
// Byte offset of the staged h rows in the down kernel's dynamic LDS, after
// the digits (nw * KBD KiB), exponents (nw * KBD ints) and e (k * RPT floats),
// rounded up to 16 bytes.
__host__ __device__ constexpr int decode_down_hf_offset(int nw, int KBD, int k) {
  return (nw * KBD * 1024 + nw * KBD * 4 + k * (16 / (KBD < 4 ? KBD : 4)) * 4 + 15) & ~15;
}

// Block = RPT output rows i for all k experts; one wave per expert (up to
// the wave count; more experts loop).  A wave turns h_r into digit operands
// in its own LDS region while its down codes load, runs NH diagonal tiles,
// and leaves e_r[i] in LDS; then y[i] = fma(w_r, e_r[i], acc), r = 0..k-1.
// Dynamic LDS: nw * (KBD*1024 + KBD*4) + k*RPT*4 bytes, then nw staged h rows.
template <int KBD, int QBITS>
__global__ __launch_bounds__(1024) void decode_down_sum_mfma_kernel(
    PoolView pv, int H, int F, int k, const int32_t* __restrict__ slots,
    const float* __restrict__ weights, const float* __restrict__ hbuf,
    const uint32_t* __restrict__ early_out, float* __restrict__ y) {
  constexpr int BPT = KBD < 4 ? KBD : 4;
  constexpr int RPT = 16 / BPT;
  constexpr int NH = KBD / BPT;
  constexpr int RG = 4 / BPT;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint8_t* s_hq = s_dyn + wv * KBD * 1024;
  int* s_he = reinterpret_cast<int*>(s_dyn + nw * KBD * 1024) + wv * KBD;
  float* s_e = reinterpret_cast<float*>(s_dyn + nw * KBD * 1024 + nw * KBD * 4);
  uint8_t* s_hf = s_dyn + decode_down_hf_offset(nw, KBD, k) + wv * KBD * 1024;   // h_r (F floats)
  // The first expert's h_r and the k slots are copied straight into LDS
  // (global_load_lds, stores the compiler keeps in place) before the flag is
  // looked at: all of these addresses are valid either way, so the flag's
  // latency overlaps theirs.  Only the code loads, whose addresses need a
  // resident slot, wait for the flag; h_r's quantisation then overlaps them
  // (loads complete in issue order).
  constexpr int NU = (16 * KBD + 63) / 64;   // runs of 16 values per lane
  const uint32_t flag = *early_out;
  __shared__ int s_sl[16][64];           // each wave's copy of the k slots (k <= 32)
  {
    const uint8_t* g = reinterpret_cast<const uint8_t*>(hbuf + int64_t(wv < k ? wv : 0) * F) + 16 * lane;
#pragma unroll
    for (int c = 0; c < KBD; ++c) __builtin_amdgcn_global_load_lds(g + c * 1024, s_hf + c * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(slots + (lane < k ? lane : 0), &s_sl[wv][0], 4, 0, 0);
  }
  if (flag) return;
  const int i0 = blockIdx.x * RPT;
  const int rho = lane & 15, q = lane >> 4;
  const int64_t blk = int64_t(i0 + rho / BPT) * KBD + rho % BPT;
  for (int r = wv; r < k; r += nw) {
    if (r != wv) {
      // a later expert (more experts than waves): its h_r into the wave's
      // staging region, whose previous contents were read an iteration ago
      const uint8_t* g = reinterpret_cast<const uint8_t*>(hbuf + int64_t(r) * F) + 16 * lane;
#pragma unroll
      for (int c = 0; c < KBD; ++c) __builtin_amdgcn_global_load_lds(g + c * 1024, s_hf + c * 1024, 16, 0, 0);
    }
    // h_r always comes from LDS, so the only global loads in flight while it
    // is quantised below are this expert's code loads: the quantisation
    // overlaps them instead of waiting for them at a join of two paths
    __builtin_amdgcn_s_waitcnt(0);       // the copy into LDS has landed
    wave_lds_sync();
    float v[NU][16];
    const float* hf = reinterpret_cast<const float*>(s_hf);
#pragma unroll
    for (int u = 0; u < NU; ++u) load_run(hf, lane + 64 * u, lane + 64 * u < 16 * KBD, v[u]);
    const int slot = s_sl[wv][r];
    const uint8_t* td = tensor_base(pv, slot, 2);
    TileCodes cd[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) cd[h] = load_tile<QBITS>(td, pv, blk + BPT * h, q);
#pragma unroll
    for (int u = 0; u < NU; ++u)
      quantize_loaded(v[u], lane + 64 * u, lane + 64 * u < 16 * KBD, s_hq, s_he);
    wave_lds_sync();
    float acc[RG];
#pragma unroll
    for (int il = 0; il < RG; ++il) acc[il] = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      v4i B[4];
      load_b_diag<BPT>(s_hq, h, lane, B);
      const v4i D = tile_mfma<QBITS>(cd[h], B);
      diag_accumulate<BPT, QBITS>(D, cd[h].dh, s_he, h, lane, acc);
    }
#pragma unroll
    for (int il = 0; il < RG; ++il) acc[il] = group_sum_last<16>(acc[il]);
    if ((lane & 15) == 15) {
      const int g = lane >> 4;
#pragma unroll
      for (int il = 0; il < RG; ++il) s_e[r * RPT + g * RG + il] = acc[il];
    }
    wave_lds_sync();                     // digit region reused by the next expert
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RPT; t += blockDim.x) {
    float a = 0.f;
    for (int r = 0; r < k; ++r) a = fmaf(weights[r], s_e[r * RPT + t], a);
    y[i0 + t] = a;
  }
}

// ------------------------------------------------------------ launchers
// Waves per gate/up block (4 rows each at H = 2048).  At the real shape four
// waves give 321 blocks on 256 compute units; two waves (641 blocks) and
// sixteen (81) were slower, eight (161) the same (measured per launch: 6.32,
// 7.07 and 6.05 against 5.97 us).
constexpr int kGateupWaves = 4;

template <int N, int KB, int QBITS>
static void gateup_mfma(const DecodeArgs& a, hipStream_t st) {
  constexpr int BPT = KB < 4 ? KB : 4;
  const int blocks = a.k * (a.F / (kGateupWaves * (16 / BPT))) + 1;
  decode_topk_gateup_mfma_kernel<N, KB, QBITS, kGateupWaves><<<blocks, 64 * kGateupWaves, 0, st>>>(
      a.pool, a.H, a.F, a.E, a.k, a.layer, a.n_slots, a.x, a.logits, a.residency, a.ids,
      a.weights, a.slots, a.miss_count, a.early_out, a.hbuf, int(a.sticky));
}

template <int N, int QBITS>
static void gateup_mfma_h(const DecodeArgs& a, hipStream_t st) {
  switch (a.H / 256) {
    case 1: gateup_mfma<N, 1, QBITS>(a, st); break;
    case 2: gateup_mfma<N, 2, QBITS>(a, st); break;
    case 4: gateup_mfma<N, 4, QBITS>(a, st); break;
    default: gateup_mfma<N, 8, QBITS>(a, st); break;
  }
}

template <int N>
static void gateup_mfma_n(const DecodeArgs& a, hipStream_t st) {
  if (a.qbits == 3) gateup_mfma_h<N, 3>(a, st); else gateup_mfma_h<N, 2>(a, st);
}

void launch_decode_gateup_mfma(const DecodeArgs& a, hipStream_t st) {
  switch (cand_per_lane(a.E)) {
    case 1: gateup_mfma_n<1>(a, st); break;
    case 2: gateup_mfma_n<2>(a, st); break;
    case 4: gateup_mfma_n<4>(a, st); break;
    case 8: gateup_mfma_n<8>(a, st); break;
    default: gateup_mfma_n<16>(a, st); break;
  }
}

// Waves per down block: one per expert, at most 16, and few enough that the
// digit regions fit in 64 KiB of LDS.
int decode_down_mfma_waves(int k, int F) {
  const int kbd = F / 256;
  int nw = k < 16 ? k : 16;
  const int cap = (60 * 1024) / (kbd * 2052);   // digits, exponents and staged h per wave
  return nw < cap ? nw : cap;
}

template <int KBD, int QBITS>
static void down_mfma(const DecodeArgs& a, hipStream_t st) {
  constexpr int BPT = KBD < 4 ? KBD : 4;
  constexpr int RPT = 16 / BPT;
  const int nw = decode_down_mfma_waves(a.k, a.F);
  const size_t lds = size_t(decode_down_hf_offset(nw, KBD, a.k)) + size_t(nw) * KBD * 1024;
  decode_down_sum_mfma_kernel<KBD, QBITS><<<a.H / RPT, 64 * nw, lds, st>>>(
      a.pool, a.H, a.F, a.k, a.slots, a.weights, a.hbuf, a.early_out, a.y);
}

void launch_decode_down_sum_mfma(const DecodeArgs& a, hipStream_t st) {
  switch (a.F / 256) {
    case 1: a.qbits == 3 ? down_mfma<1, 3>(a, st) : down_mfma<1, 2>(a, st); break;
    case 2: a.qbits == 3 ? down_mfma<2, 3>(a, st) : down_mfma<2, 2>(a, st); break;
    case 4: a.qbits == 3 ? down_mfma<4, 3>(a, st) : down_mfma<4, 2>(a, st); break;
    default: a.qbits == 3 ? down_mfma<8, 3>(a, st) : down_mfma<8, 2>(a, st); break;
  }
}

}  // namespace rl
