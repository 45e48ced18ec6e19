// Decode attention over the paged INT8 KV cache: split-K over 512-row partitions
// (stage 1) and a log-sum-exp merge of the partial states (stage 2).
//
// ("dot4-flash-attention" README route table: split-K stage 1 distributes K rows over
// workgroups in 512-row splits, stage 2 merges; "INT8 KV and INT8 MMAC attention on a
// gfx936 DCU" §3.3: paged INT8 K/V read directly, INT8 query and query scale, scales
// restored after the integer accumulation, partitions merged; §1.3 score formula.)
//
// Stage 1 workgroup = (partition j, KV head g, sequence s), 8 waves. Wave w owns the
// 64 tokens [64w, 64w+64) of the partition (4 pages). Per wave:
//  * QK on the int8 matrix cores as S^T = K . Q^T (v_mfma_i32_16x16x64_i8): the 16
//    accumulator rows are 16 tokens of one page, the 16 columns are the 6 query heads
//    of the group, repeated once (columns 6..11), then 4 zero columns. Each K operand
//    load is one contiguous 1 KB per wave thanks to the K page layout.
//  * scores s = qk * sQ * sK * sm_scale * log2(e) (exp2 domain), fp32 softmax over the
//    64 tokens with column max/sum over the 4 lanes of a column.
//  * PV in fp32-equivalent precision: w = p * (sV / max(sV)) lies in [0, 1]; columns 0..5
//    carry fp16(w) and columns 6..11 carry fp16(w - fp16(w)), so hi + lo keeps 22
//    significant bits; V codes are exact in fp16. v_mfma_f32_16x16x32_f16 computes
//    out^T = V^T . P^T with fp32 accumulation; the two halves are summed with a DPP
//    row shift. The wave's softmax state goes to LDS and the 8 states of the partition
//    are merged into one partial (m, l, o[256]) per query head.
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

constexpr int kPart = 512;
constexpr int kDecWaves = 8;

__device__ __forceinline__ float from_lane_plus6(float v) {
  // DPP row_shl:6 -- lane i of each 16-lane row reads lane i + 6 of the same row.
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x106, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t comp(const uint4& a, int u) {
  return u == 0 ? a.x : (u == 1 ? a.y : (u == 2 ? a.z : a.w));
}

__global__ __launch_bounds__(512, 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int num_pages, int n_q_heads,
    int n_kv_heads, float qk_scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int max_parts) {
  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int ctx = ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
  const int tok0 = j * kPart;
  if (tok0 >= ctx) return;  // whole workgroup: this partition is past the context
  const int n_tok = min(kPart, ctx - tok0);

  __shared__ int s_pages[kPart / kPage];
  __shared__ __align__(16) int8_t s_q[kGroup][kHeadDim];
  __shared__ float s_qs[kGroup];
  __shared__ __align__(16) float s_ks[kPart];
  __shared__ __align__(16) float s_vs[kPart];
  __shared__ float s_m[kDecWaves][kGroup], s_l[kDecWaves][kGroup];
  __shared__ __align__(16) float s_o[kDecWaves][kGroup][kHeadDim];

  // Block table of the partition -> LDS; query rows of the group -> int8 in LDS.
  if (tid < kPart / kPage) {
    const int blk = (tok0 >> 4) + tid;
    int p = 0;
    if (blk * kPage < ctx) {
      p = block_table[(size_t)s * max_blocks + blk];
      if (p < 0 || p >= num_pages) p = 0;
    }
    s_pages[tid] = p;
  }
  if (w < kGroup) {
    const size_t row = (size_t)s * n_q_heads + g * kGroup + w;
    const uint2 qw = *reinterpret_cast<const uint2*>(q + row * kHeadDim + lane * 4);
    float sc;
    const uint32_t c = quantize4(bf16_to_f32(qw.x & 0xffffu), bf16_to_f32(qw.x >> 16),
                                 bf16_to_f32(qw.y & 0xffffu), bf16_to_f32(qw.y >> 16), &sc);
    *reinterpret_cast<uint32_t*>(&s_q[w][lane * 4]) = c;
    if (lane == 0) s_qs[w] = sc;
  }
  __syncthreads();

  // Issue this wave's K and V loads (4 pages x 4 KB each), then the token scales.
  const int wtok0 = w * 64;
  const int nvalid = min(64, n_tok - wtok0);  // <= 0: wave has no tokens
  uint4 kA[4][4], vA[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (wtok0 + 16 * t < n_tok) {
      const size_t base = ((size_t)s_pages[4 * w + t] * n_kv_heads + g) * kBlockBytes + lane * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) kA[t][u] = *reinterpret_cast<const uint4*>(k_cache + base + u * 1024);
#pragma unroll
      for (int u = 0; u < 4; ++u) vA[t][u] = *reinterpret_cast<const uint4*>(v_cache + base + u * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) { kA[t][u] = make_uint4(0, 0, 0, 0); vA[t][u] = make_uint4(0, 0, 0, 0); }
    }
  }
  {
    float a = 0.f, b = 0.f;
    if (tid < n_tok) {
      const size_t si = ((size_t)s_pages[tid >> 4] * n_kv_heads + g) * kPage + (tid & 15);
      a = k_scale[si];
      b = v_scale[si];
    }
    s_ks[tid] = a;
    s_vs[tid] = b;
  }
  __syncthreads();

  const int n = lane & 15, gq = lane >> 4;
  if (nvalid > 0) {
    const int col_head = n < 2 * kGroup ? (n < kGroup ? n : n - kGroup) : -1;
    v4i qB[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qB[u] = col_head >= 0 ? *reinterpret_cast<const v4i*>(&s_q[col_head][u * 64 + gq * 16])
                            : v4i{0, 0, 0, 0};
    v4i S[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      S[t] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        S[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, kA[t][u]), qB[u], S[t],
                                                     0, 0, 0);
    }
    const float rs = col_head >= 0 ? s_qs[col_head] * qk_scale_log2 : 0.f;
    float x[16], sv[16];
    float mx = -INFINITY, svm = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 kk = *reinterpret_cast<const float4*>(&s_ks[wtok0 + 16 * t + 4 * gq]);
      const float4 vv = *reinterpret_cast<const float4*>(&s_vs[wtok0 + 16 * t + 4 * gq]);
      const float kv4[4] = {kk.x, kk.y, kk.z, kk.w}, vv4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * t + 4 * gq + i < nvalid;
        const float xv = ok ? (float)S[t][i] * kv4[i] * rs : -INFINITY;
        x[4 * t + i] = xv;
        sv[4 * t + i] = ok ? vv4[i] : 0.f;
        mx = fmaxf(mx, xv);
        svm = fmaxf(svm, sv[4 * t + i]);
      }
    }
    mx = col_max(mx);
    svm = col_max(svm);
    float lsum = 0.f;
    v8h B0, B1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2f(x[e] - mx);
      lsum += p;
      // sv / svm is a true division so that the largest-scale token gets exactly 1
      // (a one-token context then returns fl32(code * scale) exactly).
      const float wv = svm > 0.f ? p * (sv[e] / svm) : 0.f;
      const _Float16 hi = (_Float16)wv;
      const _Float16 val = n < kGroup ? hi : (n < 2 * kGroup ? (_Float16)(wv - (float)hi) : (_Float16)0.f);
      if (e < 8) B0[e] = val; else B1[e - 8] = val;
    }
    lsum = col_sum(lsum);

#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const int q4 = dt >> 2, u = dt & 3;
      const v8h A0 = i8x8_to_f16(comp(vA[0][q4], u), comp(vA[1][q4], u));
      const v8h A1 = i8x8_to_f16(comp(vA[2][q4], u), comp(vA[3][q4], u));
      v4f O = {0.f, 0.f, 0.f, 0.f};
      O = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B0, O, 0, 0, 0);
      O = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B1, O, 0, 0, 0);
      float4 r;
      r.x = (O[0] + from_lane_plus6(O[0])) * svm;
      r.y = (O[1] + from_lane_plus6(O[1])) * svm;
      r.z = (O[2] + from_lane_plus6(O[2])) * svm;
      r.w = (O[3] + from_lane_plus6(O[3])) * svm;
      if (n < kGroup) *reinterpret_cast<float4*>(&s_o[w][n][16 * dt + 4 * gq]) = r;
    }
    if (gq == 0 && n < kGroup) {
      s_m[w][n] = mx;
      s_l[w][n] = lsum;
    }
  } else if (lane < kGroup) {
    s_m[w][lane] = -INFINITY;
    s_l[w][lane] = 0.f;
  }
  __syncthreads();

  // Merge the 8 wave states of this partition and write its partial.
  for (int idx = tid; idx < kGroup * kHeadDim; idx += kDecWaves * 64) {
    const int h = idx >> 8, d = idx & 255;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float mw = s_m[ww][h];
      if (mw != -INFINITY) {
        const float a = exp2f(mw - M);
        L += a * s_l[ww][h];
        O += a * s_o[ww][h][d];
      }
    }
    const size_t pi = ((size_t)s * n_q_heads + g * kGroup + h) * max_parts + j;
    ws_o[pi * kHeadDim + d] = O;
    if (d == 0) {
      ws_m[pi] = M;
      ws_l[pi] = L;
    }
  }
}

// Stage 2: one workgroup per (q head, sequence), one thread per output dim.
// out = sum_j o_j 2^(m_j - M) / sum_j l_j 2^(m_j - M), M = max_j m_j.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l, const float* __restrict__ ws_o,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int n_q_heads, int max_parts,
    float* __restrict__ out) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int lane = d & 63, wv = d >> 6;
  int ctx = ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
  const int P = (ctx + kPart - 1) / kPart;
  float* o = out + ((size_t)s * n_q_heads + h) * kHeadDim;
  if (P == 0) {
    o[d] = 0.f;
    return;
  }
  const size_t base = ((size_t)s * n_q_heads + h) * max_parts;
  __shared__ float s_red[4];
  __shared__ float s_a[256], s_al[256];
  float m = -INFINITY;
  for (int jj = d; jj < P; jj += 256) m = fmaxf(m, ws_m[base + jj]);
  m = wave_max(m);
  if (lane == 0) s_red[wv] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float L = 0.f, O0 = 0.f, O1 = 0.f, O2 = 0.f, O3 = 0.f;
  for (int c0 = 0; c0 < P; c0 += 256) {
    const int jj = c0 + d;
    float a = 0.f, al = 0.f;
    if (jj < P) {
      a = exp2f(ws_m[base + jj] - M);
      al = a * ws_l[base + jj];
    }
    s_a[d] = a;
    s_al[d] = al;
    __syncthreads();
    const int cnt = min(256, P - c0);
    const float* op = ws_o + (base + c0) * kHeadDim + d;
    int k = 0;
    for (; k + 4 <= cnt; k += 4) {
      O0 += s_a[k] * op[(size_t)k * kHeadDim];
      O1 += s_a[k + 1] * op[(size_t)(k + 1) * kHeadDim];
      O2 += s_a[k + 2] * op[(size_t)(k + 2) * kHeadDim];
      O3 += s_a[k + 3] * op[(size_t)(k + 3) * kHeadDim];
      L += (s_al[k] + s_al[k + 1]) + (s_al[k + 2] + s_al[k + 3]);
    }
    for (; k < cnt; ++k) {
      O0 += s_a[k] * op[(size_t)k * kHeadDim];
      L += s_al[k];
    }
    __syncthreads();
  }
  o[d] = ((O0 + O1) + (O2 + O3)) / L;
}

int launch_decode(const uint16_t* q, const int8_t* k_cache, const int8_t* v_cache,
                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                  int max_blocks, const int32_t* ctx_lens, int num_seqs, int max_ctx,
                  int num_pages, int n_q_heads, int n_kv_heads, float sm_scale, float* out,
                  float* ws, int max_parts, hipStream_t stream) {
  const size_t np = (size_t)num_seqs * n_q_heads * max_parts;
  float* ws_m = ws;
  float* ws_l = ws + np;
  float* ws_o = ws + 2 * np;
  const long long cap = (long long)max_blocks * kPage;
  const int ctx_cap = (int)(cap < max_ctx ? cap : max_ctx);
  hipLaunchKernelGGL(decode_split_kernel, dim3(max_parts, n_kv_heads, num_seqs), dim3(512), 0,
                     stream, q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks,
                     ctx_lens, ctx_cap, num_pages, n_q_heads, n_kv_heads, sm_scale * kLog2e, ws_m,
                     ws_l, ws_o, max_parts);
  int rc = check_launch("attn_decode stage 1");
  if (rc) return rc;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(n_q_heads, num_seqs), dim3(256), 0, stream, ws_m,
                     ws_l, ws_o, ctx_lens, ctx_cap, n_q_heads, max_parts, out);
  return check_launch("attn_decode stage 2");
}

}  // namespace i8a
