// Prefill / verify chunk attention over the paged INT8 KV cache in one pass.
//
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.2: INT8 Q, history and current
// INT8 K/V in one online-softmax pass with INT8 QK and INT8 PV; §3.3 and §1.3: the V
// scale is folded into the softmax weight, the weight block is quantized with scale =
// block absmax / 127 and the int8 product is scaled back by it; §4.2: more query rows
// per K/V tile. "#3381 prompt QSA attention without the decode kernel's split and
// merge", Approach: one workgroup walks all chunks with an online softmax, each chunk
// summed from zero and folded in. "dot4-flash-attention" README recthist: prefix keys
// need no mask, only the causal tail does.)
//
// Workgroup = (block of 16*kPfNT query tokens, KV head g), 6 waves; wave w is query
// head 6g + w and owns kPfNT 16-token column tiles. The K/V of each 64-key block (4 pages) is
// staged in LDS (double buffered) and shared by the 6 waves. Per wave and key block:
//  * S^T = K . Q^T on v_mfma_i32_16x16x64_i8 (rows: 16 keys of one page, columns: 16
//    query tokens), so every lane holds 16 scores of one query row;
//  * scores in the exp2 domain, online max with a lazy rescale (the reference max only
//    moves when a block max exceeds it by more than 2^8, which keeps p <= 256);
//  * w = p * sV, per (row, block) scale s_b = max w / 127, codes rint(w / s_b) in
//    [0, 127]; the denominator sums the unquantized p;
//  * out^T += s_b * (V^T . P^T) on v_mfma_i32_16x16x64_i8, int32 exact per block.
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

constexpr int kPfNT = 1;         // 16-token column tiles per wave
constexpr int kPfBQ = 16 * kPfNT; // query tokens per workgroup
constexpr int kPfWaves = kGroup; // one wave per query head of the group
constexpr int kPfThreads = kPfWaves * 64;
constexpr float kLazyRescale = 8.0f;  // log2 units

struct LoadCtx {
  const int8_t* k_cache;
  const int8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  int n_table, num_pages, n_kv_heads, g, tid;
};

__device__ __forceinline__ int page_of(const LoadCtx& c, int kb, int t) {
  const int pi = kb * 4 + t;
  const int p = pi < c.n_table ? c.block_table[pi] : 0;
  return (p < 0 || p >= c.num_pages) ? 0 : p;
}

// Chunk ch (0..2047) of a 64-key block: K (ch < 1024) or V, page t = (ch >> 8) & 3,
// 16-byte offset (ch & 255) * 16 inside that page's 4 KB block.
__device__ __forceinline__ uint4 load_chunk(const LoadCtx& c, int kb, int ch) {
  const int kv = ch >> 10, t = (ch >> 8) & 3, off = (ch & 255) * 16;
  const size_t base = ((size_t)page_of(c, kb, t) * c.n_kv_heads + c.g) * kBlockBytes + off;
  return *reinterpret_cast<const uint4*>((kv ? c.v_cache : c.k_cache) + base);
}

__device__ __forceinline__ void store_chunk(int8_t (*s_kv)[4 * kBlockBytes], int ch, uint4 v) {
  const int kv = ch >> 10, t = (ch >> 8) & 3, off = (ch & 255) * 16;
  *reinterpret_cast<uint4*>(&s_kv[kv][t * kBlockBytes + off]) = v;
}

__device__ __forceinline__ void issue_block(const LoadCtx& c, int kb, uint4& r0, uint4& r1,
                                            uint4& r2, uint4& r3, uint4& r4, uint4& r5,
                                            float& scv) {
  const int T = kPfThreads;
  r0 = load_chunk(c, kb, c.tid);
  r1 = load_chunk(c, kb, c.tid + T);
  r2 = load_chunk(c, kb, c.tid + 2 * T);
  r3 = load_chunk(c, kb, c.tid + 3 * T);
  r4 = load_chunk(c, kb, c.tid + 4 * T);
  if (c.tid + 5 * T < 2048) r5 = load_chunk(c, kb, c.tid + 5 * T);
  if (c.tid < 128) {
    const int kv = c.tid >> 6, key = c.tid & 63;
    const size_t si = ((size_t)page_of(c, kb, key >> 4) * c.n_kv_heads + c.g) * kPage + (key & 15);
    scv = (kv ? c.v_scale : c.k_scale)[si];
  }
}

__device__ __forceinline__ void commit_block(int8_t (*s_kv)[4 * kBlockBytes], float (*s_sc)[64],
                                             int tid, uint4 r0, uint4 r1, uint4 r2, uint4 r3,
                                             uint4 r4, uint4 r5, float scv) {
  const int T = kPfThreads;
  store_chunk(s_kv, tid, r0);
  store_chunk(s_kv, tid + T, r1);
  store_chunk(s_kv, tid + 2 * T, r2);
  store_chunk(s_kv, tid + 3 * T, r3);
  store_chunk(s_kv, tid + 4 * T, r4);
  if (tid + 5 * T < 2048) store_chunk(s_kv, tid + 5 * T, r5);
  if (tid < 128) s_sc[tid >> 6][tid & 63] = scv;
}

__global__ __launch_bounds__(kPfThreads, 1) void prefill_chunk_kernel(
    const uint16_t* __restrict__ q, int n_new, const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int ctx,
    int causal, int num_pages, int n_q_heads, int n_kv_heads, float qk_scale_log2,
    float* __restrict__ out) {
  const int qb = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = g * kGroup + w;
  const int n = lane & 15, gq = lane >> 4;
  const int t0 = qb * kPfBQ;
  const int nq = min(kPfBQ, n_new - t0);
  const int pos0 = ctx - n_new;
  const int kend = causal ? pos0 + t0 + nq : ctx;   // keys [0, kend) are needed
  const int nkb = (kend + 63) >> 6;
  const int kfull = causal ? pos0 + t0 + 1 : ctx;   // keys < kfull are seen by every row
  const int n_table = (ctx + kPage - 1) / kPage;

  __shared__ __align__(16) int8_t s_kv[2][2][4 * kBlockBytes];    // [buffer][K,V][4 pages]
  __shared__ __align__(16) float s_sc[2][2][64];                  // [buffer][K,V][key]
  __shared__ __align__(16) int8_t s_q[kPfWaves][kPfBQ][kHeadDim]; // query codes
  __shared__ float s_qs[kPfWaves][kPfBQ];

  // ---- quantize this wave's query rows into LDS (rows past the chunk are zero).
  for (int r = 0; r < kPfBQ; ++r) {
    uint32_t c = 0u;
    float sc = 0.f;
    if (r < nq) {
      const uint2 qw = *reinterpret_cast<const uint2*>(
          q + ((size_t)(t0 + r) * n_q_heads + h) * kHeadDim + lane * 4);
      c = quantize4(bf16_to_f32(qw.x & 0xffffu), bf16_to_f32(qw.x >> 16),
                    bf16_to_f32(qw.y & 0xffffu), bf16_to_f32(qw.y >> 16), &sc);
    }
    *reinterpret_cast<uint32_t*>(&s_q[w][r][lane * 4]) = c;
    if (lane == 0) s_qs[w][r] = sc;
  }
  __syncthreads();
  float rs[kPfNT];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) rs[nt] = s_qs[w][16 * nt + n] * qk_scale_log2;

  // ---- K/V block loader: 2048 chunks of 16 B (K then V, page-major) + 128 scales.
  uint4 r0, r1, r2, r3, r4, r5;
  float scv = 0.f;
  const LoadCtx lc{k_cache, v_cache, k_scale, v_scale, block_table, n_table, num_pages, n_kv_heads,
                   g, tid};
  float m_run[kPfNT], l_part[kPfNT];
  v4f acc[kPfNT][16];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    m_run[nt] = -INFINITY;
    l_part[nt] = 0.f;
  }
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) acc[nt][dt] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nkb > 0) {
    issue_block(lc, 0, r0, r1, r2, r3, r4, r5, scv);
    commit_block(s_kv[0], s_sc[0], tid, r0, r1, r2, r3, r4, r5, scv);
  }
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) issue_block(lc, kb + 1, r0, r1, r2, r3, r4, r5, scv);
    const int8_t* sK = s_kv[buf][0];
    const int8_t* sV = s_kv[buf][1];

    // QK: S[nt][t] = K(page t) . Q^T(column tile nt)
    v4i S[kPfNT][4];
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt)
#pragma unroll
      for (int t = 0; t < 4; ++t) S[nt][t] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v4i b[kPfNT];
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt)
        b[nt] = *reinterpret_cast<const v4i*>(&s_q[w][16 * nt + n][gq * 16 + u * 64]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i a = *reinterpret_cast<const v4i*>(sK + t * kBlockBytes + u * 1024 + lane * 16);
#pragma unroll
        for (int nt = 0; nt < kPfNT; ++nt)
          S[nt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[nt], S[nt][t], 0, 0, 0);
      }
    }
    const int key0 = kb * 64;
    const bool need_mask = (key0 + 64 > kfull) || (key0 + 64 > ctx);

    v4i Pb[kPfNT];
    float sb[kPfNT];
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt) {
      const int qpos = pos0 + t0 + 16 * nt + n;
      const int lim = causal ? min(qpos + 1, ctx) : ctx;  // keys < lim are visible
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 16 * (e >> 2) + 4 * gq + (e & 3);
        const float ksc = s_sc[buf][0][16 * (e >> 2) + 4 * gq + (e & 3)];
        float xv = (float)S[nt][e >> 2][e & 3] * ksc * rs[nt];
        if (need_mask && key >= lim) xv = -INFINITY;
        x[e] = xv;
        bm = fmaxf(bm, xv);
      }
      bm = col_max(bm);
      const bool up = bm > m_run[nt] + kLazyRescale;
      if (__any(up)) {
        const float mn = up ? bm : m_run[nt];
        const float alpha = (m_run[nt] == -INFINITY) ? 0.f : exp2f(m_run[nt] - mn);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) acc[nt][dt] *= alpha;
        l_part[nt] *= alpha;
        m_run[nt] = mn;
      }
      const float mref = m_run[nt];
      float ls = 0.f, wm = 0.f;
      float wv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool live = x[e] != -INFINITY;
        const float p = live ? exp2f(x[e] - mref) : 0.f;
        ls += p;
        const float vsc = s_sc[buf][1][16 * (e >> 2) + 4 * gq + (e & 3)];
        wv[e] = live ? p * vsc : 0.f;
        wm = fmaxf(wm, wv[e]);
      }
      l_part[nt] += ls;
      wm = col_max(wm);
      const float inv = wm > 0.f ? 127.0f / wm : 0.f;
      sb[nt] = wm * (1.0f / 127.0f);
      v4i pb;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t d = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t c = (uint32_t)rintf(fminf(wv[4 * t + i] * inv, 127.0f));
          d |= c << (8 * i);
        }
        pb[t] = (int)d;
      }
      Pb[nt] = pb;
    }

    // PV: out^T(dim tile dt) += s_b * V^T(dt) . P^T
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint4 vl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vl[t] = *reinterpret_cast<const uint4*>(sV + t * kBlockBytes + q4 * 1024 + lane * 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dt = q4 * 4 + u;
        const v4i a = {(int)(u == 0 ? vl[0].x : u == 1 ? vl[0].y : u == 2 ? vl[0].z : vl[0].w),
                       (int)(u == 0 ? vl[1].x : u == 1 ? vl[1].y : u == 2 ? vl[1].z : vl[1].w),
                       (int)(u == 0 ? vl[2].x : u == 1 ? vl[2].y : u == 2 ? vl[2].z : vl[2].w),
                       (int)(u == 0 ? vl[3].x : u == 1 ? vl[3].y : u == 2 ? vl[3].z : vl[3].w)};
#pragma unroll
        for (int nt = 0; nt < kPfNT; ++nt) {
          const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, Pb[nt], v4i{0, 0, 0, 0}, 0, 0, 0);
          acc[nt][dt][0] += sb[nt] * (float)r[0];
          acc[nt][dt][1] += sb[nt] * (float)r[1];
          acc[nt][dt][2] += sb[nt] * (float)r[2];
          acc[nt][dt][3] += sb[nt] * (float)r[3];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kb + 1 < nkb) commit_block(s_kv[buf ^ 1], s_sc[buf ^ 1], tid, r0, r1, r2, r3, r4, r5, scv);
    __syncthreads();
  }

  // ---- normalise and store: lane (n, gq) holds dims 16*dt + 4*gq + i of its row.
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const float l = col_sum(l_part[nt]);
    const int r = 16 * nt + n;
    if (r < nq) {
      const float il = 1.0f / l;
      float* o = out + ((size_t)(t0 + r) * n_q_heads + h) * kHeadDim + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        float4 v;
        v.x = acc[nt][dt][0] * il; v.y = acc[nt][dt][1] * il;
        v.z = acc[nt][dt][2] * il; v.w = acc[nt][dt][3] * il;
        *reinterpret_cast<float4*>(o + 16 * dt) = v;
      }
    }
  }
}

int launch_prefill(const uint16_t* q, int n_new, const int8_t* k_cache, const int8_t* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int ctx, int causal, int num_pages, int n_q_heads, int n_kv_heads,
                   float sm_scale, float* out, hipStream_t stream) {
  const dim3 grid((n_new + kPfBQ - 1) / kPfBQ, n_kv_heads);
  hipLaunchKernelGGL(prefill_chunk_kernel, grid, dim3(kPfThreads), 0, stream, q, n_new, k_cache,
                     v_cache, k_scale, v_scale, block_table, ctx, causal, num_pages, n_q_heads,
                     n_kv_heads, sm_scale * kLog2e, out);
  return check_launch("attn_prefill_chunk");
}

}  // namespace i8a
