// Measurement kernels: the two ceilings the attention kernels are compared with on the
// same GPU and in the same run. They compute nothing of the attention method.
//
//  * stream_read_kernel: reads a device buffer once with 16-byte loads (each workgroup a
//    contiguous slab, 8 loads per thread in flight) and folds the bytes into one word
//    per wave, so no load can be elided. Timed on a buffer of the decode's size
//    read in rotation over several copies, it is the measured HBM ceiling of a 68 MB
//    one-pass read (launch, ramp-up and tail included); on a large buffer it is the
//    sustained read bandwidth.
//  * page_gather_kernel: the decode's reads without its arithmetic: for every page of a
//    block table, the 4 KB of K codes and the 4 KB of V codes of one KV head and its 16 +
//    16 scales, one workgroup per (run of pages, KV head), 16-byte loads with 4 pages
//    (8 loads per thread) in flight, folded like the streaming read. Timed over the
//    decode's cache copies, it is the measured ceiling of the decode's own access pattern
//    (scattered 4 KB pages instead of one contiguous buffer).
//  * mfma_i8_kernel: a loop of v_mfma_i32_16x16x64_i8 on register operands, 8
//    independent accumulator chains per wave and two waves per SIMD, so the matrix core
//    never waits on a result: the measured int8 MFMA ceiling, and a kernel whose MFMA
//    count is known exactly (for calibrating the MFMA-busy counters).
#include "common.hpp"
#include "int8attn.h"
#include "launch.hpp"

namespace i8a {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kMfmaThreads = 512;   // 8 waves: two per SIMD
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(
    const uint4* __restrict__ src, unsigned long long n16, uint32_t* __restrict__ sink) {
  const unsigned long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const unsigned long long b = (unsigned long long)blockIdx.x * per;
  const unsigned long long e = min(n16, b + per);
  uint32_t acc = 0u;
  unsigned long long i = b + threadIdx.x;
  for (; i + (kReadUnroll - 1) * kReadThreads < e; i += kReadUnroll * kReadThreads) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + (unsigned long long)u * kReadThreads];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += kReadThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the wave; one plain store per wave (sink holds 4 words per workgroup)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

constexpr int kGatherThreads = 256;  // 16 bytes each: one 4 KB page per load round
constexpr int kGatherUnroll = 4;     // pages in flight per thread (K and V: 8 loads)

__global__ __launch_bounds__(kGatherThreads) void page_gather_kernel(
    const int8_t* __restrict__ k_cache, const int8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, int n_blocks, int n_kv_heads, int num_pages,
    int pages_per_wg, uint32_t* __restrict__ sink) {
  const int g = blockIdx.y, tid = threadIdx.x;
  const int b0 = blockIdx.x * pages_per_wg, b1 = min(n_blocks, b0 + pages_per_wg);
  uint32_t acc = 0u;
  for (int b = b0; b < b1; b += kGatherUnroll) {
    uint4 kv[2 * kGatherUnroll];
    float sc[2 * kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      kv[2 * u] = kv[2 * u + 1] = make_uint4(0u, 0u, 0u, 0u);
      sc[2 * u] = sc[2 * u + 1] = 0.f;
      if (b + u < b1) {  // (uniform) every page of the run is read once
        const int pr = block_table[b + u];
        const int p = (uint32_t)pr < (uint32_t)num_pages ? pr : 0;  // (out-of-pool: page 0)
        const size_t base = ((size_t)p * n_kv_heads + g) * kBlockBytes + (size_t)tid * 16;
        kv[2 * u] = *reinterpret_cast<const uint4*>(k_cache + base);
        kv[2 * u + 1] = *reinterpret_cast<const uint4*>(v_cache + base);
        if (tid < 16) {
          const size_t si = ((size_t)p * n_kv_heads + g) * kPage + tid;
          sc[2 * u] = k_scale[si];
          sc[2 * u + 1] = v_scale[si];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2 * kGatherUnroll; ++u)
      acc ^= kv[u].x ^ kv[u].y ^ kv[u].z ^ kv[u].w ^ __float_as_uint(sc[u]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if ((tid & 63) == 0)
    sink[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * (kGatherThreads / 64) + (tid >> 6)] = acc;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_i8_kernel(int iters, int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operands that the compiler cannot fold (they depend on the lane and the launch)
  v4i a = {lane * 3 + 1, lane ^ 0x55, (int)blockIdx.x, lane - 7};
  v4i b = {lane + 5, (int)threadIdx.x, lane * 11, 0x01020304};
  v4i acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = v4i{c, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
  }
  int r = 0;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) r ^= acc[c][0] ^ acc[c][1] ^ acc[c][2] ^ acc[c][3];
  if (r == 0x7fffffff) sink[blockIdx.x] = r;  // keeps the chains live; practically never stored
}

}  // namespace i8a

using namespace i8a;

extern "C" {

int int8attn_ceiling_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_workgroups,
                                 void* stream) {
  if (bytes == 0 || bytes % 16 != 0 || n_workgroups <= 0 || !src || !sink ||
      ((uintptr_t)src & 15u) != 0)
    return set_error(I8A_EINVAL, "ceiling_stream_read: %zu bytes (a positive multiple of 16, "
                     "16-byte aligned), %d workgroups", bytes, n_workgroups);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_workgroups), dim3(kReadThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(src),
                     (unsigned long long)(bytes / 16), sink);
  return check_launch("ceiling_stream_read");
}

int int8attn_ceiling_page_gather(const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, int n_blocks, int n_kv_heads,
                                 int num_pages, int pages_per_workgroup, uint32_t* sink,
                                 void* stream) {
  if (!k_cache || !v_cache || !k_scale || !v_scale || !block_table || !sink || n_blocks <= 0 ||
      n_kv_heads <= 0 || num_pages <= 0 || pages_per_workgroup <= 0)
    return set_error(I8A_EINVAL, "ceiling_page_gather: %d blocks, %d KV heads, %d pages, %d pages "
                     "per workgroup", n_blocks, n_kv_heads, num_pages, pages_per_workgroup);
  const int nx = (n_blocks + pages_per_workgroup - 1) / pages_per_workgroup;
  hipLaunchKernelGGL(page_gather_kernel, dim3((unsigned)nx, (unsigned)n_kv_heads),
                     dim3(kGatherThreads), 0, (hipStream_t)stream, k_cache, v_cache, k_scale,
                     v_scale, block_table, n_blocks, n_kv_heads, num_pages, pages_per_workgroup,
                     sink);
  return check_launch("ceiling_page_gather");
}

int int8attn_ceiling_mfma_i8(int n_workgroups, int iters, int32_t* sink, void* stream) {
  if (n_workgroups <= 0 || iters <= 0 || !sink)
    return set_error(I8A_EINVAL, "ceiling_mfma_i8: %d workgroups, %d iterations", n_workgroups, iters);
  hipLaunchKernelGGL(mfma_i8_kernel, dim3((unsigned)n_workgroups), dim3(kMfmaThreads), 0,
                     (hipStream_t)stream, iters, sink);
  return check_launch("ceiling_mfma_i8");
}

int64_t int8attn_ceiling_mfma_i8_count(int n_workgroups, int iters) {
  if (n_workgroups <= 0 || iters <= 0) return 0;
  return (int64_t)n_workgroups * (kMfmaThreads / 64) * kMfmaChains * iters;
}

}  // extern "C"
