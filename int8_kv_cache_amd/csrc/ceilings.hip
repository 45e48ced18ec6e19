// Measurement kernels: the two ceilings the attention kernels are compared with on the
// same GPU and in the same run. They compute nothing of the attention method.
//
//  * stream_read_kernel: reads a device buffer once with 16-byte loads (each workgroup a
//    contiguous slab, 8 loads per thread in flight) and folds the bytes into one word
//    per wave, so no load can be elided. Timed on a buffer of the decode's size
//    read in rotation over several copies, it is the measured HBM ceiling of a 68 MB
//    one-pass read (launch, ramp-up and tail included); on a large buffer it is the
//    sustained read bandwidth.
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
