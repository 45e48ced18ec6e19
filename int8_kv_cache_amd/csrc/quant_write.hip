// kv_quant_write and q_quant kernels: per-row absmax/127 int8 quantization of new K/V
// rows written straight into the paged cache, and of bf16 query rows.
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.1 rule, §2.2 fused producer:
// absmax, scale, quantize, paged INT8 write and scale write in one kernel.)
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

template <int IN_BF16>
__device__ __forceinline__ void load_row4(const void* base, size_t row, int lane, float* x) {
  if (IN_BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(
        static_cast<const uint16_t*>(base) + row * kHeadDim + lane * 4);
    x[0] = bf16_to_f32(w.x & 0xffffu); x[1] = bf16_to_f32(w.x >> 16);
    x[2] = bf16_to_f32(w.y & 0xffffu); x[3] = bf16_to_f32(w.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(
        static_cast<const float*>(base) + row * kHeadDim + lane * 4);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
}

// One wave per (token, kv head); 4 waves per block. The wave quantizes that token's K
// row and V row (independently) and scatters codes and scales into the page layout.
template <int IN_BF16>
__global__ __launch_bounds__(256) void kv_quant_write_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int n_rows, int n_kv_heads,
    const int32_t* __restrict__ slots, int8_t* __restrict__ k_cache,
    int8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    long long n_slots) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // = token * H + head
  if (row >= n_rows) return;                            // whole wave
  const int tok = row / n_kv_heads, head = row - tok * n_kv_heads;
  const int slot = slots[tok];
  if (slot < 0 || (long long)slot >= n_slots) return;   // skipped token (whole wave)

  float kx[4], vx[4];
  load_row4<IN_BF16>(k, (size_t)row, lane, kx);
  load_row4<IN_BF16>(v, (size_t)row, lane, vx);
  float ks, vs;
  const uint32_t kq = quantize4(kx[0], kx[1], kx[2], kx[3], &ks);
  const uint32_t vq = quantize4(vx[0], vx[1], vx[2], vx[3], &vs);

  const int page = slot >> 4, o = slot & 15;
  const size_t blk = ((size_t)page * n_kv_heads + head) * kBlockBytes;
  // K: dims 4l..4l+3 sit in chunk l/4 at byte (l%4)*4 of token o's 16-byte run.
  *reinterpret_cast<uint32_t*>(k_cache + blk + (lane >> 2) * 256 + o * 16 + (lane & 3) * 4) = kq;
  // V: dim d = 4l + j sits at byte d*16 + o (dim-major, the 16 tokens of a dim adjacent).
  int8_t* vb = v_cache + blk + lane * 64 + o;
#pragma unroll
  for (int j = 0; j < 4; ++j) vb[j * 16] = (int8_t)(vq >> (8 * j));
  if (lane == 0) {
    const size_t si = ((size_t)page * n_kv_heads + head) * kPage + o;
    k_scale[si] = ks;
    v_scale[si] = vs;
  }
}

// One wave per bf16 query row of 256; codes are written row-major.
__global__ __launch_bounds__(256) void q_quant_kernel(const uint16_t* __restrict__ q, int n_rows,
                                                      int8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  float x[4];
  load_row4<1>(q, (size_t)row, lane, x);
  float s;
  const uint32_t c = quantize4(x[0], x[1], x[2], x[3], &s);
  *reinterpret_cast<uint32_t*>(codes + (size_t)row * kHeadDim + lane * 4) = c;
  if (lane == 0) scales[row] = s;
}

int launch_kv_quant_write(const void* k, const void* v, int in_bf16, int n_tokens, int n_kv_heads,
                          const int32_t* slots, int8_t* k_cache, int8_t* v_cache, float* k_scale,
                          float* v_scale, int num_pages, hipStream_t stream) {
  const int rows = n_tokens * n_kv_heads;
  const dim3 grid((rows + 3) / 4), block(256);
  const long long n_slots = (long long)num_pages * kPage;
  if (in_bf16)
    hipLaunchKernelGGL(kv_quant_write_kernel<1>, grid, block, 0, stream, k, v, rows, n_kv_heads,
                       slots, k_cache, v_cache, k_scale, v_scale, n_slots);
  else
    hipLaunchKernelGGL(kv_quant_write_kernel<0>, grid, block, 0, stream, k, v, rows, n_kv_heads,
                       slots, k_cache, v_cache, k_scale, v_scale, n_slots);
  return check_launch("kv_quant_write");
}

int launch_q_quant(const uint16_t* q, int n_rows, int8_t* codes, float* scales,
                   hipStream_t stream) {
  hipLaunchKernelGGL(q_quant_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, q, n_rows,
                     codes, scales);
  return check_launch("q_quant");
}

}  // namespace i8a
