// kv_quant_write, kv_produce and q_quant kernels: per-row absmax/127 int8 quantization
// of new K/V rows written straight into the paged cache (kv_produce first rotates K and
// Q by RoPE and also quantizes Q), and of bf16 query rows.
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.1 rule, §2.2 fused producer:
// read Q/K/V, RoPE on Q/K, absmax, scale, quantize, paged INT8 write and scale write in
// one kernel, with no high-precision Q/K written back.)
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

// RoPE on one row held 4 dims per lane (lane l: dims 4l..4l+3). Pair (i, i + rd/2) of
// the first rd dims turns by the angle whose cos and sin are cs[i] and cs[rd/2 + i]; rd is
// a multiple of 8, so a lane's 4 dims are all rotated or all passed through and all in
// one half. Every product and sum is rounded on its own (no contraction into fma), the
// fp32 rule the results are defined by.
__device__ __forceinline__ float rot_second(float b, float c, float a, float s) {
#pragma clang fp contract(off)
  return b * c + a * s;
}
// The cos/sin of one token for this lane's 4 dims (loaded once, used for K and every
// query row of the token), and the lane holding the partner dims.
struct RopeLane {
  float cc[4], ss[4];
  int partner;
  bool in, first;
};
__device__ __forceinline__ RopeLane rope_lane(const float* __restrict__ cs, int rd, int lane) {
  RopeLane r;
  const int half = rd >> 1;
  const int d0 = lane * 4;
  r.in = d0 < rd;
  r.first = d0 < half;
  r.partner = r.in ? (r.first ? lane + (half >> 2) : lane - (half >> 2)) : lane;
  if (r.in) {
    const int i0 = r.first ? d0 : d0 - half;
    const float4 c = *reinterpret_cast<const float4*>(cs + i0);
    const float4 sn = *reinterpret_cast<const float4*>(cs + half + i0);
    r.cc[0] = c.x; r.cc[1] = c.y; r.cc[2] = c.z; r.cc[3] = c.w;
    // The first half turns by -sin: a c - b s = a c + b (-s), the same rounding.
    const float sg = r.first ? -1.0f : 1.0f;
    r.ss[0] = sg * sn.x; r.ss[1] = sg * sn.y; r.ss[2] = sg * sn.z; r.ss[3] = sg * sn.w;
  }
  return r;
}
__device__ __forceinline__ void rope4(float* x, const RopeLane& r) {
  float y[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = __shfl(x[j], r.partner);
  if (r.in) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = rot_second(x[j], r.cc[j], y[j], r.ss[j]);
  }
}

// Workgroup = (16 consecutive tokens, KV head) of 16 / TPW waves: wave w quantizes the K
// and V rows of tokens TPW w .. TPW w + TPW - 1 of the group (row loads issued before
// anything waits). kv_quant_write runs 2 tokens per wave, kv_produce (with 6 query rows per
// token) 1, so that more waves hide the load and reduction latencies. When the 16
// tokens fill one whole page in order (slots s0..s0+15, s0 % 16 == 0, the common case of
// prefill chunks and bulk fills) the workgroup assembles the page's dim-major V block
// in LDS and writes K, V and the scales as whole 16-byte runs; otherwise every token is
// scattered to its own slot.
// With PRODUCE (kv_produce) the K rows are rotated by their token's position first, and
// the workgroup also rotates and quantizes the query rows of the KV head's group for its
// 16 tokens (each wave: its tokens, all 6 heads), codes row-major into q_codes. PRODUCE = 2
// is the common case compiled on its own (rotation, query codes, no bf16 copies): without
// the per-row tests of those options the six query rows are straight-line code.
struct Produce {
  const void* q;
  const int32_t* positions;
  const float* cos_sin;
  int rotary_dim, max_pos, n_q_heads;
  int8_t* q_codes;
  float* q_scales;
  uint16_t* q_rot;  // rotated Q / K rows rounded to bf16 (a chunk with no history)
  uint16_t* k_rot;
};

__device__ __forceinline__ uint32_t bf16_bits(float x) {  // nearest, ties to even; finite x
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, const float* x) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_bits(x[0]) | (bf16_bits(x[1]) << 16),
                                              bf16_bits(x[2]) | (bf16_bits(x[3]) << 16));
}

constexpr int kWriteTpw = 2;    // tokens per wave of kv_quant_write
constexpr int kProduceTpw = 1;  // tokens per wave of kv_produce

template <int IN_BF16, int PRODUCE, int TPW>
__global__ __launch_bounds__(64 * 16 / TPW) void kv_quant_write_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int n_tokens, int n_kv_heads,
    const int32_t* __restrict__ slots, int8_t* __restrict__ k_cache,
    int8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    long long n_slots, Produce pr) {
  const int grp = blockIdx.x, head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar row arithmetic
  const int tok0 = grp * 16;
  __shared__ int s_run;
  __shared__ __align__(16) uint32_t s_v[kBlockBytes / 4];  // V block [dim][token]
  __shared__ float s_sc[2][16];

  // Positions first, so that the RoPE rows they address can be requested right after the
  // K/V rows: the rotation of K waits for them, and for every load issued before them.
  // Only the load is here, its first use (the clamp) comes after the row loads; the load is
  // unconditional (no rotation: a slot is read instead, unused) so that it shares a block
  // with the row loads and the compiler does not wait for it before issuing them.
  int posn[PRODUCE ? TPW : 1];
  if (PRODUCE) {
    const int32_t* ppos = (PRODUCE == 2 || pr.rotary_dim > 0) ? pr.positions : slots;
#pragma unroll
    for (int i = 0; i < TPW; ++i) posn[PRODUCE ? i : 0] = ppos[min(tok0 + TPW * w + i, n_tokens - 1)];
  }
  float kx[TPW][4], vx[TPW][4];
  int myslot[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = min(tok0 + TPW * w + i, n_tokens - 1);
    const size_t row = (size_t)t * n_kv_heads + head;
    load_row4<IN_BF16>(k, row, lane, kx[i]);
    load_row4<IN_BF16>(v, row, lane, vx[i]);
    myslot[i] = tok0 + TPW * w + i < n_tokens ? slots[tok0 + TPW * w + i] : -1;
  }
  // The RoPE rows of the tokens, ahead of the query rows in the load order.
  RopeLane rl[PRODUCE ? TPW : 1];
  if (PRODUCE == 2 || (PRODUCE && pr.rotary_dim > 0)) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int pos = min(max(posn[PRODUCE ? i : 0], 0), pr.max_pos - 1);  // clamped: memory-safe
      rl[PRODUCE ? i : 0] = rope_lane(pr.cos_sin + (size_t)pos * pr.rotary_dim, pr.rotary_dim, lane);
    }
  }
  // Query rows of the group for this wave's tokens, loaded with the K/V rows (one round
  // trip); tokens past the batch re-read the last one and are not stored.
  float qx[PRODUCE ? TPW : 1][kGroup][4];
  const bool want_q = PRODUCE == 2 || (PRODUCE && (pr.q_codes != nullptr || pr.q_rot != nullptr));
  if (want_q) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = min(tok0 + TPW * w + i, n_tokens - 1);
#pragma unroll
      for (int hh = 0; hh < kGroup; ++hh)
        load_row4<IN_BF16>(pr.q, (size_t)t * pr.n_q_heads + head * kGroup + hh, lane,
                           qx[PRODUCE ? i : 0][hh]);
    }
  }
  // The group's 16 slots for the page-run test (wave 0), consumed only before the writes.
  int sl_run = -1;
  if (w == 0) {
    const int t = tok0 + (lane & 15);
    sl_run = t < n_tokens ? slots[t] : -1;
  }
  if (PRODUCE == 2 || (PRODUCE && pr.rotary_dim > 0)) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) rope4(kx[i], rl[PRODUCE ? i : 0]);
  }
  if (PRODUCE == 1 && pr.k_rot != nullptr) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = tok0 + TPW * w + i;
      if (t < n_tokens) store_bf16x4(pr.k_rot + ((size_t)t * n_kv_heads + head) * kHeadDim + lane * 4, kx[i]);
    }
  }
  uint32_t kq[TPW], vq[TPW];
  float ks[TPW], vs[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    kq[i] = quantize4(kx[i][0], kx[i][1], kx[i][2], kx[i][3], &ks[i]);
    vq[i] = quantize4(vx[i][0], vx[i][1], vx[i][2], vx[i][3], &vs[i]);
  }
  if (want_q) {
    // The group's query rows of this wave's tokens: rotate, quantize, store.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = tok0 + TPW * w + i;
      if (t >= n_tokens) break;  // whole wave
      // The group's 6 rows are consecutive: one base per token, the rows at fixed offsets.
      const size_t row0 = (size_t)t * pr.n_q_heads + head * kGroup;
#pragma unroll
      for (int hh = 0; hh < kGroup; ++hh) {
        float* xr = qx[PRODUCE ? i : 0][hh];
        if (PRODUCE == 2 || pr.rotary_dim > 0) rope4(xr, rl[PRODUCE ? i : 0]);
        if (PRODUCE == 1 && pr.q_rot != nullptr) store_bf16x4(pr.q_rot + row0 * kHeadDim + lane * 4 + hh * kHeadDim, xr);
        if (PRODUCE == 2 || pr.q_codes != nullptr) {
          float sc;
          const uint32_t c = quantize4(xr[0], xr[1], xr[2], xr[3], &sc);
          *reinterpret_cast<uint32_t*>(pr.q_codes + row0 * kHeadDim + lane * 4 + hh * kHeadDim) = c;
          if (lane == 0) pr.q_scales[row0 + hh] = sc;
        }
      }
    }
  }
  if (w == 0) {  // page-run test on the group's 16 slots (lanes 16..63 repeat 0..15)
    const int t = tok0 + (lane & 15);
    const int s0_run = __shfl(sl_run, 0);
    const bool ok = t < n_tokens && sl_run == s0_run + (lane & 15) && (s0_run & 15) == 0 &&
                    s0_run >= 0 && (long long)s0_run + 15 < n_slots;
    const bool all = __all(ok);
    if (lane == 0) s_run = all ? 1 : 0;
  }
  __syncthreads();
  if (s_run) {
    const int page = __shfl(myslot[0], 0) >> 4;  // slot s0 + TPW w, same page for every wave
    const size_t blk = ((size_t)page * n_kv_heads + head) * kBlockBytes;
    // K: token TPW w + i, dims 4l..4l+3 -> chunk l/4, byte (l%4)*4 of the token's 16-byte run.
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      *reinterpret_cast<uint32_t*>(k_cache + blk + (lane >> 2) * 256 + (TPW * w + i) * 16 +
                                   (lane & 3) * 4) = kq[i];
    // V: dim 4l + j gets the TPW bytes of tokens TPW w .. TPW w + TPW - 1.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (TPW == 4) {
        const uint32_t lo = __builtin_amdgcn_perm(vq[1], vq[0], 0x0c0c0400u + j * 0x00000101u);
        const uint32_t hi = __builtin_amdgcn_perm(vq[3 % TPW], vq[2 % TPW], 0x0c0c0400u + j * 0x00000101u);
        s_v[(4 * lane + j) * 4 + w] = (lo & 0xffffu) | (hi << 16);
      } else if (TPW == 2) {
        const uint32_t lo = __builtin_amdgcn_perm(vq[1 % TPW], vq[0], 0x0c0c0400u + j * 0x00000101u);
        reinterpret_cast<uint16_t*>(s_v)[(4 * lane + j) * 8 + w] = (uint16_t)lo;
      } else {
        reinterpret_cast<uint8_t*>(s_v)[(4 * lane + j) * 16 + w] = (uint8_t)(vq[0] >> (8 * j));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        s_sc[0][TPW * w + i] = ks[i];
        s_sc[1][TPW * w + i] = vs[i];
      }
    }
    __syncthreads();
    if (tid < kBlockBytes / 16)
      *reinterpret_cast<uint4*>(v_cache + blk + tid * 16) = reinterpret_cast<const uint4*>(s_v)[tid];
    if (tid < 32) {
      const size_t si = ((size_t)page * n_kv_heads + head) * kPage + (tid & 15);
      (tid < 16 ? k_scale : v_scale)[si] = s_sc[tid >> 4][tid & 15];
    }
  } else {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
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
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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
  const dim3 grid((n_tokens + 15) / 16, n_kv_heads), block(64 * 16 / kWriteTpw);
  const long long n_slots = (long long)num_pages * kPage;
  const Produce none{nullptr, nullptr, nullptr, 0, 1, 0, nullptr, nullptr, nullptr, nullptr};
  if (in_bf16)
    hipLaunchKernelGGL((kv_quant_write_kernel<1, 0, kWriteTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, none);
  else
    hipLaunchKernelGGL((kv_quant_write_kernel<0, 0, kWriteTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, none);
  return check_launch("kv_quant_write");
}

int launch_kv_produce(const void* q, const void* k, const void* v, int in_bf16, int n_tokens,
                      int n_q_heads, int n_kv_heads, const int32_t* positions, const float* cos_sin,
                      int rotary_dim, int max_pos, const int32_t* slots, int8_t* k_cache,
                      int8_t* v_cache, float* k_scale, float* v_scale, int num_pages,
                      int8_t* q_codes, float* q_scales, uint16_t* q_rot, uint16_t* k_rot,
                      hipStream_t stream) {
  const dim3 grid((n_tokens + 15) / 16, n_kv_heads), block(64 * 16 / kProduceTpw);
  const long long n_slots = (long long)num_pages * kPage;
  const Produce pr{q, positions, cos_sin, rotary_dim, max_pos, n_q_heads, q_codes, q_scales,
                   q_rot, k_rot};
  // The common case (rotation, int8 query codes, no bf16 copies) has its own instance
  // with those tests compiled away.
  const bool common = rotary_dim > 0 && q_codes != nullptr && q_rot == nullptr && k_rot == nullptr;
  if (in_bf16 && common)
    hipLaunchKernelGGL((kv_quant_write_kernel<1, 2, kProduceTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, pr);
  else if (in_bf16)
    hipLaunchKernelGGL((kv_quant_write_kernel<1, 1, kProduceTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, pr);
  else if (common)
    hipLaunchKernelGGL((kv_quant_write_kernel<0, 2, kProduceTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, pr);
  else
    hipLaunchKernelGGL((kv_quant_write_kernel<0, 1, kProduceTpw>), grid, block, 0, stream, k, v, n_tokens,
                       n_kv_heads, slots, k_cache, v_cache, k_scale, v_scale, n_slots, pr);
  return check_launch("kv_produce");
}

int launch_q_quant(const uint16_t* q, int n_rows, int8_t* codes, float* scales,
                   hipStream_t stream) {
  hipLaunchKernelGGL(q_quant_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, q, n_rows,
                     codes, scales);
  return check_launch("q_quant");
}

}  // namespace i8a
