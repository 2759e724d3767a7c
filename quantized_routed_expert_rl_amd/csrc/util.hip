// Helpers for stacks of MoE layers: weightless RMSNorm before each layer and
// the residual add after it, skipped when the layer's early-out flag is set.
// They are not part of the MoE layer; they let a stack of layers run on the
// device without host round trips.
#include <atomic>

#include "rl_common.h"
#include "rl_kernels.h"

namespace rl {

// Compute units of the current device, queried once per device.  Calls from
// several host threads may query at the same time; they store the same value.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// 1 / sqrt(mean(v^2) + eps) of one token's row, from each thread's float64
// sum of squares, in every thread of the 256-thread block.
__device__ inline double block_inv_rms(double s, int H, float eps) {
  s = wave_sum_f64(s);
  __shared__ double s_w[4];
  __shared__ double s_inv;
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) s_inv = 1.0 / sqrt((s_w[0] + s_w[1] + s_w[2] + s_w[3]) / H + double(eps));
  __syncthreads();
  return s_inv;
}

// Element order of the norms: thread t of the 256-thread block owns the
// 4-value chunks at 4t + 1024u and chains their float64 squares in
// (u, component) order (chunk_sq); the four waves' sums are added in order.
// decode_router_residual_kernel repeats this order in one wave (lane l
// standing for threads l + 64w), so the three norms give the same bits.
// One block per token: out = x / sqrt(mean(x^2) + eps), the mean of squares
// accumulated in float64.
__global__ __launch_bounds__(256) void rmsnorm_kernel(int H, const float* __restrict__ x,
                                                      float* __restrict__ out, float eps) {
  const int64_t base = int64_t(blockIdx.x) * H;
  double s = 0.0;
  for (int i = 4 * threadIdx.x; i < H; i += 1024)
    s = chunk_sq(*reinterpret_cast<const float4*>(x + base + i), s);
  const double inv = block_inv_rms(s, H, eps);
  for (int i = 4 * threadIdx.x; i < H; i += 1024)
    *reinterpret_cast<float4*>(out + base + i) =
        chunk_scale(*reinterpret_cast<const float4*>(x + base + i), inv);
}

// The step between two layers of a stack in one launch, one block per token:
// x_out = x + y (x_out = x when the layer's flag is set), then
// a_out = rmsnorm(x_out), each thread keeping its own elements in registers.
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(
    int H, const float* __restrict__ x, const float* __restrict__ y,
    const uint32_t* __restrict__ early_out, float* __restrict__ x_out, float* __restrict__ a_out,
    float eps) {
  const int64_t base = int64_t(blockIdx.x) * H;
  const bool skip = early_out && *early_out;
  float4 v[2];
  double s = 0.0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {                  // H <= 2048
    const int i = 4 * threadIdx.x + 1024 * u;
    if (i < H) {
      const float4 xv = *reinterpret_cast<const float4*>(x + base + i);
      if (skip) {
        v[u] = xv;
      } else {
        const float4 yv = *reinterpret_cast<const float4*>(y + base + i);
        v[u] = make_float4(xv.x + yv.x, xv.y + yv.y, xv.z + yv.z, xv.w + yv.w);
      }
      *reinterpret_cast<float4*>(x_out + base + i) = v[u];
      s = chunk_sq(v[u], s);
    }
  }
  const double inv = block_inv_rms(s, H, eps);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 4 * threadIdx.x + 1024 * u;
    if (i < H) *reinterpret_cast<float4*>(a_out + base + i) = chunk_scale(v[u], inv);
  }
}

__global__ __launch_bounds__(256) void residual_add_kernel(int64_t n, float* __restrict__ x,
                                                           const float* __restrict__ y,
                                                           const uint32_t* __restrict__ early_out) {
  if (early_out && *early_out) return;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    x[i] = x[i] + y[i];
}

void launch_rmsnorm(int T, int H, const float* x, float* out, float eps, hipStream_t st) {
  rmsnorm_kernel<<<T, 256, 0, st>>>(H, x, out, eps);
}

void launch_residual_rmsnorm(int T, int H, const float* x, const float* y,
                             const uint32_t* early_out, float* x_out, float* a_out, float eps,
                             hipStream_t st) {
  residual_rmsnorm_kernel<<<T, 256, 0, st>>>(H, x, y, early_out, x_out, a_out, eps);
}

void launch_residual_add(int T, int H, float* x, const float* y, const uint32_t* early_out,
                         hipStream_t st) {
  const int64_t n = int64_t(T) * H;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  residual_add_kernel<<<int(blocks), 256, 0, st>>>(n, x, y, early_out);
}

// A plain streaming read: every 16-byte word of buf once, four loads in
// flight per thread, folded so the loads cannot be dropped; sink is written
// only if the fold hits a value it never takes in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= (a.x ^ b.y ^ c.z ^ d.w) + (a.w ^ b.z ^ c.y ^ d.x);
  }
  for (; i < n; i += stride) acc ^= buf[i].x ^ buf[i].w;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// table[pairs[2i]] = pairs[2i+1] for i < n (residency entries that a load
// or an eviction changed; keys are distinct).
__global__ __launch_bounds__(64) void table_scatter_kernel(int32_t* __restrict__ table,
                                                           const int32_t* __restrict__ pairs,
                                                           int n) {
  for (int i = threadIdx.x; i < n; i += 64) table[pairs[2 * i]] = pairs[2 * i + 1];
}

void launch_table_scatter(int32_t* table, const int32_t* pairs, int n, hipStream_t st) {
  table_scatter_kernel<<<1, 64, 0, st>>>(table, pairs, n);
}

// One layer's expert loads in one launch: expert e (blockIdx.y) is copied
// from row src_row[e] of the host store, read through its device address
// (pinned host memory, over PCIe), into pool slot dst_slot[e]; block (0, 0)
// also writes the residency entries the loads change.  Every block keeps
// four 16-byte reads in flight per thread.
__global__ __launch_bounds__(256) void expert_gather_kernel(const uint4* __restrict__ store,
                                                            uint4* __restrict__ pool,
                                                            int64_t slot_vecs, ExpertLoads ld,
                                                            int32_t* __restrict__ table) {
  const int e = blockIdx.y;
  const uint4* src = store + ld.src_row[e] * slot_vecs;
  uint4* dst = pool + int64_t(ld.dst_slot[e]) * slot_vecs;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i0 = int64_t(blockIdx.x) * 256 + threadIdx.x; i0 < slot_vecs; i0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * stride < slot_vecs) v[u] = src[i0 + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * stride < slot_vecs) dst[i0 + u * stride] = v[u];
  }
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < ld.n_pairs; i += 256) table[ld.pairs[2 * i]] = ld.pairs[2 * i + 1];
}

void launch_expert_gather(const void* store_dev, void* pool, int64_t slot_bytes,
                          const ExpertLoads& ld, int32_t* table, hipStream_t st) {
  if (ld.n <= 0 && ld.n_pairs <= 0) return;
  const dim3 grid(64, ld.n > 0 ? ld.n : 1);
  ExpertLoads a = ld;
  if (a.n <= 0) {                      // entries only: one block, no copy
    a.src_row[0] = 0;
    a.dst_slot[0] = 0;
    expert_gather_kernel<<<dim3(1, 1), 256, 0, st>>>(static_cast<const uint4*>(store_dev),
                                                      static_cast<uint4*>(pool), 0, a, table);
    return;
  }
  expert_gather_kernel<<<grid, 256, 0, st>>>(static_cast<const uint4*>(store_dev),
                                             static_cast<uint4*>(pool), slot_bytes / 16, a, table);
}

void launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int n_cu, hipStream_t st) {
  stream_read_kernel<<<8 * n_cu, 256, 0, st>>>(static_cast<const uint4*>(buf), bytes / 16, sink);
}

}  // namespace rl
