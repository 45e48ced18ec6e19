// Decode attention over the paged INT8 KV cache: split-K over 512-row partitions
// (stage 1) and a log-sum-exp merge of the partial states (stage 2).
//
// ("dot4-flash-attention" README route table: split-K stage 1 distributes K rows over
// workgroups in 512-row splits, stage 2 merges; "INT8 KV and INT8 MMAC attention on a
// gfx936 DCU" §3.3: paged INT8 K/V read directly, INT8 query and query scale, scales
// restored after the integer accumulation, partitions merged; §1.3 score formula.)
//
// Stage 1 workgroup = (partition j, KV head g, sequence s), 8 waves. Wave w owns the 64
// tokens [64w, 64w+64) of the partition (4 pages) and walks them page by page with an
// online softmax, issuing loads two pages ahead of the page it computes. Per page:
//  * QK on the int8 matrix cores as S^T = K . Q^T (v_mfma_i32_16x16x64_i8): the 16
//    accumulator rows are the 16 tokens of the page, the 16 columns are the 6 query
//    heads of the group, repeated once (columns 6..11), then 4 zero columns. Each K
//    operand load is one contiguous 1 KB per wave thanks to the K page layout.
//  * scores s = qk * sQ * sK * sm_scale * log2(e) (exp2 domain), column max/sum over
//    the 4 lanes that share a column.
//  * PV in fp32-equivalent precision: w = p * (sV / max(sV)); columns 0..5 carry fp16(w)
//    and columns 6..11 carry fp16(w - fp16(w)) (22 significant bits in all); V codes
//    are exact in fp16. v_mfma_f32_16x16x16_f16 computes out^T = V^T . P^T with fp32
//    accumulation; the halves are summed with a DPP row shift.
// The 8 wave states are merged into one partial (m, l, o[256]) per query head.
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

constexpr int kPart = 512;
constexpr int kDecWaves = 8;
constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ float from_lane_plus6(float v) {
  // DPP row_shl:6 -- lane i of each 16-lane row reads lane i + 6 of the same row.
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x106, 0xF, 0xF, true));
}

// Q8: the query arrives as int8 codes [S][Hq][D] with fp32 scales [S][Hq] (kv_produce's
// output) instead of bf16 rows to quantize.
template <int Q8>
__global__ __launch_bounds__(512, 1) void decode_split_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scales,
    const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int num_pages, int n_q_heads,
    int n_kv_heads, float qk_scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int max_parts, float* __restrict__ out) {
  // out != nullptr: a single partition per sequence, so the workgroup writes the
  // normalized output itself and no merge stage runs.
  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The context length and this wave's 4 page ids are fetched together (one round
  // trip); the table index is clamped so the fetch is safe before ctx is known.
  const int32_t* trow = block_table + (size_t)s * max_blocks;
  const int blk0 = j * (kPart / kPage) + 4 * w;
  int pr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pr[t] = trow[min(blk0 + t, max_blocks - 1)];
  int ctx = ctx_lens[s];
  // Consume all five scalar loads here so that none of them is sunk past the branch
  // below (which would cost a second memory round trip before the K/V loads).
  asm volatile("" ::"s"(ctx), "s"(pr[0]), "s"(pr[1]), "s"(pr[2]), "s"(pr[3]));
  ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
  const int tok0 = j * kPart;
  if (tok0 >= ctx) {  // whole workgroup: this partition is past the context
    if (out != nullptr)  // no key at all: zeros
      for (int i = tid; i < kGroup * kHeadDim; i += 512)
        out[((size_t)s * n_q_heads + g * kGroup) * kHeadDim + i] = 0.f;
    return;
  }
  const int n_tok = min(kPart, ctx - tok0);

  __shared__ __align__(16) int8_t s_q[kGroup][kHeadDim];
  __shared__ float s_qs[kGroup];
  __shared__ __align__(16) float s_ks[kPart];
  __shared__ __align__(16) float s_vs[kPart];
  __shared__ float s_m[kDecWaves][kGroup], s_l[kDecWaves][kGroup], s_f[kDecWaves];
  __shared__ __align__(16) float s_o[kDecWaves][kGroup][kHeadDim + 4];  // rows padded by 16 B
  __shared__ __align__(16) float4 s_junk[64];  // sink for the stores of unused columns
  __shared__ uint32_t s_bias;  // 0x80808080, read back after the barrier (see i8x4_to_f16)

  // Wave w owns tokens [64w, 64w+64) of the partition: pages 4w..4w+3 (wave-uniform page
  // ids in scalar registers). Loads are issued in the order they are consumed (vmcnt
  // order): query row and token scales, pages 0 and 1; the barrier then only waits for
  // the query and the scales; pages 2 and 3 are issued two steps ahead of the page
  // being computed, so each wave keeps about two pages (16 KB) in flight.
  // A page past the context reads page 0 and its tokens are masked; waves 6 and 7
  // re-read query row 5.
  const int wtok0 = w * 64;
  const int nvalid = min(64, n_tok - wtok0);  // <= 0: the wave has no tokens
  int pg[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    pg[t] = (16 * t < nvalid && pr[t] >= 0 && pr[t] < num_pages) ? pr[t] : 0;
  const size_t qrow = (size_t)s * n_q_heads + g * kGroup + min(w, kGroup - 1);
  uint2 qw = make_uint2(0u, 0u);
  uint32_t qc = 0u;
  float qsc = 0.f;
  if (Q8) {
    qc = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(q) + qrow * kHeadDim + lane * 4);
    qsc = q_scales[qrow];
  } else {
    qw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + qrow * kHeadDim + lane * 4);
  }
  const int pl = (lane >> 4) == 0 ? pg[0] : (lane >> 4) == 1 ? pg[1] : (lane >> 4) == 2 ? pg[2] : pg[3];
  const size_t si = ((size_t)pl * n_kv_heads + g) * kPage + (lane & 15);
  const float sk_l = k_scale[si];
  const float sv_l = v_scale[si];
  // K and V: four 1 KB wave loads per page each (lane l reads bytes 16l.. of each KB).
  // V lane (n, gq) thus receives all 16 tokens of dim 16(4q + gq) + n for q = 0..3; a 4x4
  // transpose over the lanes of its column (gfx950 lane swaps) gives it the A operand of
  // every dim tile: tokens 4gq..4gq+3 of dim 16dt + n.
  uint4 kA[4][4];
  uint4 vL[4][4];
  auto issue_page = [&](int t) {
    const size_t blk = ((size_t)pg[t] * n_kv_heads + g) * kBlockBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kA[t][u] = *reinterpret_cast<const uint4*>(k_cache + blk + lane * 16 + u * 1024);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vL[t][u] = *reinterpret_cast<const uint4*>(v_cache + blk + lane * 16 + u * 1024);
  };
  __builtin_amdgcn_sched_barrier(0);
  issue_page(0);
  issue_page(1);
  __builtin_amdgcn_sched_barrier(0);

  // Quantize the group's query rows (waves 0..5) and stage them with the scales in LDS.
  if (w < kGroup) {
    float sc = qsc;
    const uint32_t c = Q8 ? qc
                          : quantize4(bf16_to_f32(qw.x & 0xffffu), bf16_to_f32(qw.x >> 16),
                                      bf16_to_f32(qw.y & 0xffffu), bf16_to_f32(qw.y >> 16), &sc);
    *reinterpret_cast<uint32_t*>(&s_q[w][lane * 4]) = c;
    if (lane == 0) s_qs[w] = sc;
  }
  s_ks[wtok0 + lane] = sk_l;
  s_vs[wtok0 + lane] = sv_l;
  if (tid == 0) s_bias = 0x80808080u;
  lds_barrier();
  const uint32_t bias = s_bias;

  const int n = lane & 15, gq = lane >> 4;
  if (nvalid > 0) {
    const int col_head = n < 2 * kGroup ? (n < kGroup ? n : n - kGroup) : 0;
    const float col_on = n < 2 * kGroup ? 1.f : 0.f;   // columns 12..15 carry nothing
    v4i qB[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) qB[u] = *reinterpret_cast<const v4i*>(&s_q[col_head][u * 64 + gq * 16]);
    const float rs = s_qs[col_head] * qk_scale_log2;
    // Scales of this lane's 16 tokens (16t + 4gq + i); masked tokens get sV = 0.
    float kk[16], rv[16];
    float svm = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 a = *reinterpret_cast<const float4*>(&s_ks[wtok0 + 16 * t + 4 * gq]);
      const float4 b = *reinterpret_cast<const float4*>(&s_vs[wtok0 + 16 * t + 4 * gq]);
      kk[4 * t] = a.x; kk[4 * t + 1] = a.y; kk[4 * t + 2] = a.z; kk[4 * t + 3] = a.w;
      rv[4 * t] = b.x; rv[4 * t + 1] = b.y; rv[4 * t + 2] = b.z; rv[4 * t + 3] = b.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (16 * t + 4 * gq + i >= nvalid) rv[4 * t + i] = 0.f;
        svm = fmaxf(svm, rv[4 * t + i]);
      }
    }
    svm = col_max(svm);  // max V scale over the wave's 64 tokens (same in every lane)
    const float inv = svm > 0.f ? 1.0f / svm : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)  // the largest-scale token gets exactly 1
      rv[e] = (rv[e] == svm ? 1.0f : rv[e] * inv) * col_on;

    // Online softmax over the 4 pages. The reference max m_run only moves when a page
    // max exceeds it by more than 2^8 (lazy rescale), so p <= 256 and w <= 256.
    float m_run = -INFINITY, l_run = 0.f;
    v4f O[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) O[dt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 2 < 4) {
        __builtin_amdgcn_sched_barrier(0);
        issue_page(t + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      v4i S = v4i{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        S = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, kA[t][u]), qB[u], S, 0, 0, 0);
      float x[4];
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * t + 4 * gq + i < nvalid;
        x[i] = ok ? (float)S[i] * kk[4 * t + i] * rs : -INFINITY;
        bm = fmaxf(bm, x[i]);
      }
      bm = col_max(bm);
      if (__any(bm > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, bm);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) O[dt] *= alpha;
        m_run = m_new;
      }
      v4h B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i] - m_run);
        l_run += p;
        const float wv = p * rv[4 * t + i];
        // columns 0..5: fp16(w); columns 6..11: fp16(w - fp16(w))
        const float base = n >= kGroup ? (float)(_Float16)wv : 0.f;
        B[i] = (_Float16)(wv - base);
      }
      // Lane (n, gq) loaded dim 16(4q + gq) + n, all 16 tokens; transpose the 4x4 dwords
      // over the lanes {n, n+16, n+32, n+48} so that it holds tokens 4gq..4gq+3 of dims
      // 16(4q + c) + n, c = 0..3.
      uint32_t vA[16];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint32_t r0 = vL[t][qq].x, r1 = vL[t][qq].y, r2 = vL[t][qq].z, r3 = vL[t][qq].w;
        auto p = __builtin_amdgcn_permlane32_swap(r0, r2, false, false); r0 = p[0]; r2 = p[1];
        p = __builtin_amdgcn_permlane32_swap(r1, r3, false, false); r1 = p[0]; r3 = p[1];
        p = __builtin_amdgcn_permlane16_swap(r0, r1, false, false); r0 = p[0]; r1 = p[1];
        p = __builtin_amdgcn_permlane16_swap(r2, r3, false, false); r2 = p[0]; r3 = p[1];
        vA[4 * qq] = r0; vA[4 * qq + 1] = r1; vA[4 * qq + 2] = r2; vA[4 * qq + 3] = r3;
      }
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        h2 lo, hi;
        i8x4_to_f16(vA[dt], &lo, &hi, bias);
        const v4h A = {lo[0], lo[1], hi[0], hi[1]};
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, B, O[dt], 0, 0, 0);
      }
    }
    l_run = col_sum(l_run);
    // hi + lo columns; lanes of the unused columns store into s_junk.
    float4* dst = n < kGroup ? reinterpret_cast<float4*>(&s_o[w][n][4 * gq]) : &s_junk[lane];
    const int stride = n < kGroup ? 4 : 0;  // float4 units between dim tiles
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      float4 r;
      r.x = O[dt][0] + from_lane_plus6(O[dt][0]);
      r.y = O[dt][1] + from_lane_plus6(O[dt][1]);
      r.z = O[dt][2] + from_lane_plus6(O[dt][2]);
      r.w = O[dt][3] + from_lane_plus6(O[dt][3]);
      dst[dt * stride] = r;
    }
    if (gq == 0 && n < kGroup) {
      s_m[w][n] = m_run;
      s_l[w][n] = l_run;
    }
    if (lane == 0) s_f[w] = svm;
  } else {
    // No tokens: an empty state (its weight in the merge below is exp2(-inf) = 0).
#pragma unroll
    for (int r = 0; r < kGroup; ++r)
      reinterpret_cast<float4*>(&s_o[w][r][0])[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < kGroup) {
      s_m[w][lane] = -INFINITY;
      s_l[w][lane] = 0.f;
    }
    if (lane == 0) s_f[w] = 0.f;
  }
  lds_barrier();

  // Merge the 8 wave states of this partition: wave h < 6 merges query head h, lane l
  // dims 4l..4l+3. A wave's stored output is in units of its max V scale (s_f).
  if (w < kGroup) {
    const int h = w;
    float mw[kDecWaves];
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      mw[ww] = s_m[ww][h];
      M = fmaxf(M, mw[ww]);
    }
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float a = __builtin_amdgcn_exp2f(mw[ww] - M);
      L += a * s_l[ww][h];
      const float af = a * s_f[ww];
      const float4 ov = *reinterpret_cast<const float4*>(&s_o[ww][h][4 * lane]);
      acc.x += af * ov.x; acc.y += af * ov.y; acc.z += af * ov.z; acc.w += af * ov.w;
    }
    if (out != nullptr) {
      *reinterpret_cast<float4*>(&out[((size_t)s * n_q_heads + g * kGroup + h) * kHeadDim + 4 * lane]) =
          make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
      return;
    }
    const size_t pi = ((size_t)s * n_q_heads + g * kGroup + h) * max_parts + j;
    *reinterpret_cast<float4*>(&ws_o[pi * kHeadDim + 4 * lane]) = acc;
    if (lane == 0) {
      ws_m[pi] = M;
      ws_l[pi] = L;
    }
  }
}

// Stage 2: one wave per (64-dim chunk, q head, query row), online log-sum-exp over the
// partitions in chunks of 64: lane j holds m_j and l_j, every lane loads o_j[d] of all
// 64 partitions of the chunk up front. The first chunk is loaded together with the
// context length (indices clamped to the workspace), so a call with at most 64
// partitions costs one memory round trip. Query row z is query i = z % nq of sequence
// s = z / nq and sees ctx - nq + i + 1 keys (nq = 1: one row per sequence).
// out = sum_j o_j 2^(m_j - M) / sum_j l_j 2^(m_j - M), M = max_j m_j.
// KIND only names the instantiation (0: after the one-row split kernel, 1: after the
// int8 matrix-core split kernel) so that profiles tell the two apart.
template <int KIND>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l, const float* __restrict__ ws_o,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int n_q_heads, int max_parts, int nq,
    int part_rows, float* __restrict__ out) {
  const int c = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const int s = z / nq, qi = z - s * nq;
  const int lane = threadIdx.x;
  const int d = c * 64 + lane;
  const size_t base = ((size_t)z * n_q_heads + h) * max_parts;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  const float* po = ws_o + base * kHeadDim + d;
  float mj0, lj0, oj[64];
  auto load_chunk = [&](int j0, int cnt) {
    const int jl = j0 + min(lane, cnt - 1);
    mj0 = pm[jl];
    lj0 = pl[jl];
#pragma unroll
    for (int i = 0; i < 64; ++i) oj[i] = po[(size_t)(j0 + min(i, cnt - 1)) * kHeadDim];
  };
  int ctx = ctx_lens != nullptr ? ctx_lens[s] : ctx_cap;  // (null: one sequence of ctx_cap)
  load_chunk(0, min(64, max_parts));
  ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
  const int keys = max(0, ctx - nq + qi + 1);  // keys this query row sees
  const int P = (keys + part_rows - 1) / part_rows;
  float* o = out + ((size_t)z * n_q_heads + h) * kHeadDim;
  if (P == 0) {
    o[d] = 0.f;
    return;
  }
  __shared__ __align__(16) float s_a[64];  // the chunk's partition weights, broadcast
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int j0 = 0; j0 < P; j0 += 64) {
    const int cnt = min(64, P - j0);
    if (j0 > 0) {
      __syncthreads();  // the previous chunk's weights have been read
      load_chunk(j0, cnt);
    }
    const float mj = lane < cnt ? mj0 : -INFINITY;
    const float cm = fmaxf(M, wave_max(mj));
    const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - cm);
    const float a = lane < cnt ? __builtin_amdgcn_exp2f(mj - cm) : 0.f;
    L = L * r + wave_sum(a * (lane < cnt ? lj0 : 0.f));
    s_a[lane] = a;
    __syncthreads();
    float sacc = 0.f;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&s_a[i]);
      sacc = fmaf(w4.x, i + 0 < cnt ? oj[i + 0] : 0.f, sacc);
      sacc = fmaf(w4.y, i + 1 < cnt ? oj[i + 1] : 0.f, sacc);
      sacc = fmaf(w4.z, i + 2 < cnt ? oj[i + 2] : 0.f, sacc);
      sacc = fmaf(w4.w, i + 3 < cnt ? oj[i + 3] : 0.f, sacc);
    }
    acc = acc * r + sacc;
    M = cm;
  }
  o[d] = acc / L;
}

int launch_decode(const void* q, const float* q_scales, const int8_t* k_cache, const int8_t* v_cache,
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
  if (q_scales != nullptr)
    hipLaunchKernelGGL(decode_split_kernel<1>, dim3(max_parts, n_kv_heads, num_seqs), dim3(512), 0,
                       stream, q, q_scales, k_cache, v_cache, k_scale, v_scale, block_table,
                       max_blocks, ctx_lens, ctx_cap, num_pages, n_q_heads, n_kv_heads,
                       sm_scale * kLog2e, ws_m, ws_l, ws_o, max_parts, max_parts == 1 ? out : nullptr);
  else
    hipLaunchKernelGGL(decode_split_kernel<0>, dim3(max_parts, n_kv_heads, num_seqs), dim3(512), 0,
                       stream, q, q_scales, k_cache, v_cache, k_scale, v_scale, block_table,
                       max_blocks, ctx_lens, ctx_cap, num_pages, n_q_heads, n_kv_heads,
                       sm_scale * kLog2e, ws_m, ws_l, ws_o, max_parts, max_parts == 1 ? out : nullptr);
  int rc = check_launch("attn_decode stage 1");
  if (rc || max_parts == 1) return rc;
  hipLaunchKernelGGL(decode_merge_kernel<0>, dim3(kHeadDim / 64, n_q_heads, num_seqs), dim3(64), 0,
                     stream, ws_m, ws_l, ws_o, ctx_lens, ctx_cap, n_q_heads, max_parts, 1, kPart, out);
  return check_launch("attn_decode stage 2");
}

int launch_verify(const void* q, const float* q_scales, int nq, const int8_t* k_cache,
                  const int8_t* v_cache,
                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                  int max_blocks, const int32_t* ctx_lens, int num_seqs, int max_ctx,
                  int num_pages, int n_q_heads, int n_kv_heads, float sm_scale, float* out,
                  float* ws, int max_parts, hipStream_t stream) {
  if (nq == 1)  // one row: the one-row kernel (route by live rows)
    return launch_decode(q, q_scales, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks,
                         ctx_lens, num_seqs, max_ctx, num_pages, n_q_heads, n_kv_heads, sm_scale,
                         out, ws, max_parts, stream);
  // several rows: one read of the K/V for all of them, the weighted sum of V on the int8
  // matrix cores with three digit planes per weight
  return launch_decode_i8pv(3, kPart, q, q_scales, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                            max_blocks, ctx_lens, num_seqs, max_ctx, num_pages, n_q_heads,
                            n_kv_heads, sm_scale, out, ws, stream);
}

int launch_merge(const float* ws_m, const float* ws_l, const float* ws_o, const int32_t* ctx_lens,
                 int ctx_cap, int num_seqs, int nq, int n_q_heads, int max_parts, int part_rows,
                 float* out, hipStream_t stream) {
  hipLaunchKernelGGL(decode_merge_kernel<1>, dim3(kHeadDim / 64, n_q_heads, num_seqs * nq), dim3(64),
                     0, stream, ws_m, ws_l, ws_o, ctx_lens, ctx_cap, n_q_heads, max_parts, nq,
                     part_rows, out);
  return check_launch("decode merge");
}

// Merge for many query rows with few partitions each (the chunk routes' key partitions):
// one wave per (row, query head), lane l owning dims 4l..4l+3, so each partition's
// output row is one coalesced 1 KB load; the workgroup holds 4 such pairs. Same
// combination as decode_merge_kernel: M = max m_j, out = sum_j 2^(m_j - M) o_j /
// sum_j 2^(m_j - M) l_j over the partitions j that hold a key of the row.
__global__ __launch_bounds__(256) void merge_rows_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l, const float* __restrict__ ws_o,
    int ctx, int n_q_heads, int n_parts, int nq, int part_rows, float* __restrict__ out,
    long long n_pairs) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long pair = (long long)blockIdx.x * 4 + w;
  if (pair >= n_pairs) return;  // whole wave
  const int qi = (int)(pair / n_q_heads);
  const int keys = max(0, ctx - nq + qi + 1);  // keys this query row sees
  const int P = min(n_parts, (keys + part_rows - 1) / part_rows);
  const size_t base = (size_t)pair * n_parts;
  float4* o = reinterpret_cast<float4*>(out + (size_t)pair * kHeadDim) + lane;
  if (P == 0) {
    *o = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  float M = -INFINITY;
  for (int j = 0; j < P; ++j) M = fmaxf(M, ws_m[base + j]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* src = reinterpret_cast<const float4*>(ws_o + base * kHeadDim) + lane;
#pragma unroll 4
  for (int j = 0; j < P; ++j) {
    const float a = __builtin_amdgcn_exp2f(ws_m[base + j] - M);
    const float4 v = src[(size_t)j * (kHeadDim / 4)];
    L = fmaf(a, ws_l[base + j], L);
    acc.x = fmaf(a, v.x, acc.x);
    acc.y = fmaf(a, v.y, acc.y);
    acc.z = fmaf(a, v.z, acc.z);
    acc.w = fmaf(a, v.w, acc.w);
  }
  const float il = 1.0f / L;
  *o = make_float4(acc.x * il, acc.y * il, acc.z * il, acc.w * il);
}

int launch_merge_rows(const float* ws_m, const float* ws_l, const float* ws_o, int ctx, int nq,
                      int n_q_heads, int n_parts, int part_rows, float* out, hipStream_t stream) {
  const long long n_pairs = (long long)nq * n_q_heads;
  hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)((n_pairs + 3) / 4)), dim3(256), 0, stream,
                     ws_m, ws_l, ws_o, ctx, n_q_heads, n_parts, nq, part_rows, out, n_pairs);
  return check_launch("merge rows");
}

}  // namespace i8a
