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
// Workgroup = (32 query tokens, KV head g): 12 waves = the 6 query heads of the group x
// two 16-token column tiles, i.e. 192 query rows that share every K/V byte staged in
// LDS. The K/V of each 64-key block (4 pages, 32 KB) is double buffered in LDS and
// moved by direct global->LDS loads issued one block ahead; one LDS-only barrier per
// block hands the buffers over.
// Per wave and key block:
//  * S^T = K . Q^T on v_mfma_i32_16x16x64_i8, 4 tiles t of 16 keys x 16 query tokens.
//    Row r of tile t is token 4t + r%4 of page r/4, so lane group gq (lanes 16gq..)
//    ends up holding all 16 tokens of page gq for one query row: its P codes, in token
//    order, are then exactly the B operand that meets page gq's dim-major V bytes;
//  * x = qk * sK * (sQ * sm_scale * log2 e), online max with a lazy rescale (the
//    reference max only moves when a block max exceeds it by more than 2^8, so
//    p <= 256);
//  * w = p * sV, per (row, block) s_b = max w / 127, codes rint(w / s_b) in [0, 127]
//    (v_cvt_pk_u8_f32 converts and packs); the denominator sums the unquantized p;
//  * out^T += s_b * (V^T . P^T) on v_mfma_i32_16x16x64_i8, exact in int32 per block.
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

constexpr int kPfTok = 32;                 // query tokens per workgroup
constexpr int kPfWaves = 2 * kGroup;       // (head, 16-token half) per wave
constexpr int kPfThreads = kPfWaves * 64;  // 768
constexpr int kPfChunks = 2048;            // 16-byte chunks of one 64-key K+V block
constexpr int kPfPerThread = (kPfChunks + kPfThreads - 1) / kPfThreads;  // 3
constexpr float kLazyRescale = 8.0f;       // log2 units
constexpr int kQStride = kHeadDim + 16;    // padded LDS row of query codes (no bank conflicts)
constexpr int kPfPage = kBlockBytes + 64;  // LDS stride of a staged page: the 4 pages of a
                                           // block start on different banks

// Moves one 64-key block (4 pages of K and of V, 32 KB) of KV head g into an LDS buffer
// with direct global->LDS loads (global_load_lds_dwordx4: lane i of a wave lands at
// LDS base + 16 i), 1 KB per wave instruction: chunk c (0..2047) is K (c < 1024) or V,
// page t = (c >> 8) & 3, bytes (c & 255) * 16 of that page's 4 KB block, stored at
// t * kPfPage + (c & 255) * 16. The 128 token scales go through one register per thread
// so that slots past the context can be zeroed on the way.
struct BlockLoader {
  const int8_t* k_cache;
  const int8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  int n_table, num_pages, n_kv_heads, g, ctx, tid, w, lane;

  __device__ __forceinline__ int page(int kb, int t) const {
    const int pi = kb * 4 + t;
    const int p = pi < n_table ? block_table[pi] : 0;
    return (p < 0 || p >= num_pages) ? 0 : p;
  }
  __device__ __forceinline__ void issue(int kb, int8_t (*kv_lds)[4 * kPfPage], float& sc) const {
#pragma unroll
    for (int it = 0; it < kPfPerThread; ++it) {
      const int c0 = 64 * w + kPfThreads * it;  // first chunk of this wave's instruction
      if (c0 < kPfChunks) {
        const int kv = c0 >> 10, t = (c0 >> 8) & 3, off = (c0 & 255) * 16 + lane * 16;
        const int8_t* src = (kv ? v_cache : k_cache) +
                            ((size_t)page(kb, t) * n_kv_heads + g) * kBlockBytes + off;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)&kv_lds[kv][t * kPfPage + (c0 & 255) * 16],
            16, 0, 0);
      }
    }
    if (tid < 128) {
      const int kv = tid >> 6, key = tid & 63;
      const size_t si = ((size_t)page(kb, key >> 4) * n_kv_heads + g) * kPage + (key & 15);
      sc = (kv ? v_scale : k_scale)[si];
    }
  }
  // Call after the loads of `issue` have completed (vmcnt(0)).
  __device__ __forceinline__ void put_scales(int kb, float (*sc_lds)[64], float sc) const {
    if (tid < 128) sc_lds[tid >> 6][tid & 63] = kb * 64 + (tid & 63) < ctx ? sc : 0.f;
  }
};

__global__ __launch_bounds__(kPfThreads, 1) void prefill_chunk_kernel(
    const uint16_t* __restrict__ q, int n_new, const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int ctx,
    int causal, int num_pages, int n_q_heads, int n_kv_heads, float qk_scale_log2,
    float* __restrict__ out) {
  const int qb = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = w >> 1, half = w & 1;  // head within the group, 16-token half
  const int h = g * kGroup + hl;
  const int n = lane & 15, gq = lane >> 4;
  const int t0 = qb * kPfTok;
  const int nq = min(kPfTok, n_new - t0);
  const int pos0 = ctx - n_new;
  const int kend = causal ? pos0 + t0 + nq : ctx;  // keys [0, kend) are needed
  const int nkb = (kend + 63) >> 6;
  const int kfull = causal ? pos0 + t0 + 1 : ctx;  // keys < kfull are seen by every row
  const int my_tok = t0 + 16 * half + n;            // this lane's query token
  const int lim = causal ? min(pos0 + my_tok + 1, ctx) : ctx;  // keys < lim are visible

  __shared__ __align__(16) int8_t s_kv[2][2][4 * kPfPage];       // [buffer][K,V][4 pages]
  __shared__ __align__(16) float s_sc[2][2][64];                 // [buffer][K,V][key]
  __shared__ __align__(16) int8_t s_q[kGroup * kPfTok][kQStride];  // query codes
  __shared__ float s_qs[kGroup][kPfTok];

  const BlockLoader ld{k_cache, v_cache, k_scale, v_scale, block_table, (ctx + kPage - 1) / kPage,
                       num_pages, n_kv_heads, g, ctx, tid, w, lane};
  float sc_next = 0.f;
  if (nkb > 0) ld.issue(0, s_kv[0], sc_next);  // first block in flight during the Q work

  // ---- quantize this wave's 16 query rows (head h); rows past the chunk are zero.
  int8_t* qrows = &s_q[hl * kPfTok + 16 * half][0];
  {
    uint2 qw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = min(t0 + 16 * half + r, n_new - 1);
      qw[r] = *reinterpret_cast<const uint2*>(q + ((size_t)tok * n_q_heads + h) * kHeadDim + lane * 4);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sc;
      uint32_t c = quantize4(bf16_to_f32(qw[r].x & 0xffffu), bf16_to_f32(qw[r].x >> 16),
                             bf16_to_f32(qw[r].y & 0xffffu), bf16_to_f32(qw[r].y >> 16), &sc);
      const bool live = 16 * half + r < nq;
      *reinterpret_cast<uint32_t*>(qrows + r * kQStride + lane * 4) = live ? c : 0u;
      if (lane == 0) s_qs[hl][16 * half + r] = live ? sc : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (nkb > 0) ld.put_scales(0, s_sc[0], sc_next);
  lds_barrier();
  const int8_t* qcol = qrows + n * kQStride + gq * 16;  // this lane's B-operand bytes
  // A-operand bytes: QK row n = token 4t + n%4 of page n/4 (dims 64u + 16gq..),
  // PV row n of dim tile dt = dim 16dt + n of page gq (its 16 tokens).
  const int koff = (n >> 2) * kPfPage + gq * 256 + (n & 3) * 16;
  const int voff = gq * kPfPage + n * 16;
  // rs > 0 keeps max(x) = rs * max(y) and exp2(fma(y, rs, -m)) = 0 for masked y = -inf.
  const float rs = fmaxf(s_qs[hl][16 * half + n] * qk_scale_log2, 1e-30f);

  float m_run = -INFINITY, l_part = 0.f;
  v4f acc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) ld.issue(kb + 1, s_kv[buf ^ 1], sc_next);
    const int8_t* sK = s_kv[buf][0];
    const int8_t* sV = s_kv[buf][1];

    // QK: S[t] rows = tokens 4t..4t+3 of each of the 4 pages
    v4i S[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const v4i b = *reinterpret_cast<const v4i*>(qcol + u * 64);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i a = *reinterpret_cast<const v4i*>(sK + koff + u * 1024 + t * 64);
        S[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, S[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // bound the operand registers in flight
    }
    // y = qk * sK (key 16gq + 4t + i of the block), masked on diagonal / tail blocks only.
    const int key0 = kb * 64;
    const bool need_mask = (key0 + 64 > kfull) || (key0 + 64 > ctx);
    float y[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 sk = *reinterpret_cast<const float4*>(&s_sc[buf][0][16 * gq + 4 * t]);
      y[4 * t] = (float)S[t][0] * sk.x;
      y[4 * t + 1] = (float)S[t][1] * sk.y;
      y[4 * t + 2] = (float)S[t][2] * sk.z;
      y[4 * t + 3] = (float)S[t][3] * sk.w;
    }
    if (need_mask) {  // diagonal or context-tail block (wave-uniform)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 16 * gq + e >= lim) y[e] = -INFINITY;
    }
    float ymax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) ymax = fmaxf(ymax, y[e]);
    const float xmax = ymax * rs;
    if (__any(xmax > m_run + kLazyRescale)) {
      const float m_new = fmaxf(m_run, col_max(xmax));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) acc[dt] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
    const float nm = -m_run;
    float wm = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 sv = *reinterpret_cast<const float4*>(&s_sc[buf][1][16 * gq + 4 * t]);
      const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(y[4 * t + i], rs, nm));
        l_part += p;
        const float wv = p * svv[i];
        y[4 * t + i] = wv;
        wm = fmaxf(wm, wv);
      }
    }
    wm = col_max(wm);
    const float inv = wm > 0.f ? 127.0f / wm : 0.f;
    const float sb = wm * (1.0f / 127.0f);
    v4i Pb;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t d = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * t + i] * inv, i, d);
      Pb[t] = (int)d;
    }

    // PV: out^T(dim tile dt) += s_b * V^T(dt) . P^T; the A operand of lane (n, gq) is
    // the 16 token codes of dim 16dt + n in page gq, one 16-byte LDS read.
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dt = q4 * 4 + u;
        const v4i a = *reinterpret_cast<const v4i*>(sV + voff + dt * 256);
        const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, Pb, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dt][i] = fmaf((float)r[i], sb, acc[dt][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kb + 1 < nkb) {
      __builtin_amdgcn_s_waitcnt(0);  // the next block has landed in LDS
      ld.put_scales(kb + 1, s_sc[buf ^ 1], sc_next);
    }
    lds_barrier();
  }

  // ---- normalise and store: lane (n, gq) holds dims 16*dt + 4*gq + i of its row.
  const float l = col_sum(l_part);
  if (my_tok < t0 + nq) {
    const float il = 1.0f / l;
    float* o = out + ((size_t)my_tok * n_q_heads + h) * kHeadDim + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      float4 v;
      v.x = acc[dt][0] * il; v.y = acc[dt][1] * il;
      v.z = acc[dt][2] * il; v.w = acc[dt][3] * il;
      *reinterpret_cast<float4*>(o + 16 * dt) = v;
    }
  }
}

int launch_prefill(const uint16_t* q, int n_new, const int8_t* k_cache, const int8_t* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int ctx, int causal, int num_pages, int n_q_heads, int n_kv_heads,
                   float sm_scale, float* out, hipStream_t stream) {
  const dim3 grid((n_new + kPfTok - 1) / kPfTok, n_kv_heads);
  hipLaunchKernelGGL(prefill_chunk_kernel, grid, dim3(kPfThreads), 0, stream, q, n_new, k_cache,
                     v_cache, k_scale, v_scale, block_table, ctx, causal, num_pages, n_q_heads,
                     n_kv_heads, sm_scale * kLog2e, out);
  return check_launch("attn_prefill_chunk");
}

}  // namespace i8a
