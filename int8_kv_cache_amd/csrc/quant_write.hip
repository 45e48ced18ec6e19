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

// Workgroup = (16 consecutive tokens, KV head): wave w quantizes the K and V rows of
// tokens 4w..4w+3 of the group (row loads issued before anything waits). When the 16
// tokens fill one whole page in order (slots s0..s0+15, s0 % 16 == 0, the common case of
// prefill chunks and bulk fills) the workgroup assembles the page's dim-major V block
// in LDS and writes K, V and the scales as whole 16-byte runs; otherwise every token is
// scattered to its own slot.
template <int IN_BF16>
__global__ __launch_bounds__(256) void kv_quant_write_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int n_tokens, int n_kv_heads,
    const int32_t* __restrict__ slots, int8_t* __restrict__ k_cache,
    int8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    long long n_slots) {
  const int grp = blockIdx.x, head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tok0 = grp * 16;
  __shared__ int s_run;
  __shared__ __align__(16) uint32_t s_v[kBlockBytes / 4];  // V block [dim][token]
  __shared__ float s_sc[2][16];

  if (w == 0) {  // page-run test on the group's 16 slots (lanes 16..63 repeat 0..15)
    const int t = tok0 + (lane & 15);
    const int sl = t < n_tokens ? slots[t] : -1;
    const int s0 = __shfl(sl, 0);
    const bool ok = t < n_tokens && sl == s0 + (lane & 15) && (s0 & 15) == 0 && s0 >= 0 &&
                    (long long)s0 + 15 < n_slots;
    const bool all = __all(ok);
    if (lane == 0) s_run = all ? 1 : 0;
  }
  float kx[4][4], vx[4][4];
  int myslot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(tok0 + 4 * w + i, n_tokens - 1);
    const size_t row = (size_t)t * n_kv_heads + head;
    load_row4<IN_BF16>(k, row, lane, kx[i]);
    load_row4<IN_BF16>(v, row, lane, vx[i]);
    myslot[i] = tok0 + 4 * w + i < n_tokens ? slots[tok0 + 4 * w + i] : -1;
  }
  uint32_t kq[4], vq[4];
  float ks[4], vs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kq[i] = quantize4(kx[i][0], kx[i][1], kx[i][2], kx[i][3], &ks[i]);
    vq[i] = quantize4(vx[i][0], vx[i][1], vx[i][2], vx[i][3], &vs[i]);
  }
  __syncthreads();
  if (s_run) {
    const int page = __shfl(myslot[0], 0) >> 4;  // slot s0 + 4w, same page for every wave
    const size_t blk = ((size_t)page * n_kv_heads + head) * kBlockBytes;
    // K: token 4w + i, dims 4l..4l+3 -> chunk l/4, byte (l%4)*4 of the token's 16-byte run.
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint32_t*>(k_cache + blk + (lane >> 2) * 256 + (4 * w + i) * 16 +
                                   (lane & 3) * 4) = kq[i];
    // V: dim 4l + j gets the 4 bytes of tokens 4w..4w+3 in one LDS dword.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = __builtin_amdgcn_perm(vq[1], vq[0], 0x0c0c0400u + j * 0x00000101u);
      const uint32_t hi = __builtin_amdgcn_perm(vq[3], vq[2], 0x0c0c0400u + j * 0x00000101u);
      s_v[(4 * lane + j) * 4 + w] = (lo & 0xffffu) | (hi << 16);
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_sc[0][4 * w + i] = ks[i];
        s_sc[1][4 * w + i] = vs[i];
      }
    }
    __syncthreads();
    *reinterpret_cast<uint4*>(v_cache + blk + tid * 16) = reinterpret_cast<const uint4*>(s_v)[tid];
    if (tid < 32) {
      const size_t si = ((size_t)page * n_kv_heads + head) * kPage + (tid & 15);
      (tid < 16 ? k_scale : v_scale)[si] = s_sc[tid >> 4][tid & 15];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = myslot[i];
      if (slot < 0 || (long long)slot >= n_slots) continue;  // skipped token (whole wave)
      const int page = slot >> 4, o = slot & 15;
      const size_t blk = ((size_t)page * n_kv_heads + head) * kBlockBytes;
      *reinterpret_cast<uint32_t*>(k_cache + blk + (lane >> 2) * 256 + o * 16 + (lane & 3) * 4) = kq[i];
      // V: dim d = 4l + j sits at byte d*16 + o.
      int8_t* vb = v_cache + blk + lane * 64 + o;
#pragma unroll
      for (int j = 0; j < 4; ++j) vb[j * 16] = (int8_t)(vq[i] >> (8 * j));
      if (lane == 0) {
        const size_t si = ((size_t)page * n_kv_heads + head) * kPage + o;
        k_scale[si] = ks[i];
        v_scale[si] = vs[i];
      }
    }
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
  const dim3 grid((n_tokens + 15) / 16, n_kv_heads), block(256);
  const long long n_slots = (long long)num_pages * kPage;
  if (in_bf16)
    hipLaunchKernelGGL(kv_quant_write_kernel<1>, grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots);
  else
    hipLaunchKernelGGL(kv_quant_write_kernel<0>, grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots);
  return check_launch("kv_quant_write");
}

int launch_q_quant(const uint16_t* q, int n_rows, int8_t* codes, float* scales,
                   hipStream_t stream) {
  hipLaunchKernelGGL(q_quant_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, q, n_rows,
                     codes, scales);
  return check_launch("q_quant");
}

}  // namespace i8a
