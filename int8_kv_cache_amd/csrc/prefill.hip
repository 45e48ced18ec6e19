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
// LDS. The K/V of each 64-key block (4 pages, 32 KB) is double buffered in LDS (two
// distinct LDS variables, loop unrolled by two) and moved by direct global->LDS loads
// issued one block ahead; one LDS-only barrier per block hands the buffers over.
// Per wave and key block:
//  * S^T = K . Q^T on v_mfma_i32_16x16x64_i8, 4 tiles t of 16 keys x 16 query tokens.
//    Row r of tile t is token 4t + r%4 of page r/4, so lane group gq (lanes 16gq..)
//    ends up holding all 16 tokens of page gq for one query row: its P codes, in token
//    order, are then exactly the B operand that meets page gq's dim-major V bytes;
//  * x = qk * sK * (sQ * sm_scale * log2 e), online softmax with a lazy rescale: the
//    weights p = 2^(x - m) are taken against the running reference max m as it stands,
//    and only when a lane's block sum of them passes 2^8 (or the row has no m yet) is
//    the block redone with its max, m moving only if that max exceeds it by more than
//    2^8; so p <= 256, and the common block takes no max of the scores at all;
//  * w = p * sV, per (row, block) s_b = max w / 127, codes rint(w / s_b) in [0, 127]
//    (one fma onto 1.5 * 2^23 rounds each to an integer in the low mantissa bits, two
//    byte permutes pack four); the denominator sums the unquantized p;
//  * out^T += s_b * (V^T . P^T) on v_mfma_i32_16x16x64_i8, exact in int32 per block.
//    The product is accumulated onto the bit pattern of 1.5 * 2^23 (|V^T . P^T| <=
//    64 * 127 * 127 < 2^22), so read as fp32 it is 1.5 * 2^23 + the exact integer and
//    one fma folds it in; the offsets s_b * 1.5 * 2^23 are summed per row and taken
//    out every 8 blocks and at the end.
#include "common.hpp"
#include "int8attn.h"
#include "launch.hpp"

namespace i8a {

constexpr int kPfTok = 32;                 // query tokens per workgroup
constexpr int kPfWaves = 2 * kGroup;       // (head, 16-token half) per wave
constexpr int kPfThreads = kPfWaves * 64;  // 768
constexpr float kLazyRescale = 8.0f;       // log2 units
constexpr float kMagicF = 12582912.0f;   // 1.5 * 2^23
constexpr v4i kMagic4 = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};  // its bits
constexpr int kFlushBlocks = 8;           // blocks between removals of the offsets
constexpr int kXcds = 8;                   // XCDs of an MI355X
constexpr int kQStride = kHeadDim + 32;    // padded LDS row of query codes (no bank conflicts)
constexpr int kPfPage = kBlockBytes + 64;  // LDS stride of a staged K page: the 4 pages of a
                                           // block start on different banks (V pages are
                                           // read one page per lane group and need none)

// Moves one 64-key block (4 pages of K and of V, 32 KB, and their 128 token scales) of
// KV head g into an LDS buffer with direct global->LDS loads. Wave w moves page t = w % 4
// of the block: waves 0-3 its 4 KB of K codes, waves 4-7 its 4 KB of V codes (four 1 KB
// wave loads, global_load_lds_dwordx4: lane i lands at LDS base + 16 i), waves 8-11 its 16
// K and 16 V scales (global_load_lds_dword on lanes 0-15). So every wave resolves one
// page id per block (one scalar load, fetched a block ahead) and the work of issuing is
// spread over all twelve waves. K page t lands at t * kPfPage, V page t at t * 4096.
// Nothing waits here: the loads land while the previous block is computed and are waited
// for once, before the barrier.
struct BlockLoader {
  const int8_t* k_cache;
  const int8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  int n_table, num_pages, n_kv_heads, g, w, lane;

  // This wave's raw table entry for block kb. The index is clamped to the table, so a
  // block past the context reads the sequence's last page, whose keys are masked.
  __device__ __forceinline__ int page(int kb) const {
    return block_table[min(kb * 4 + (w & 3), n_table - 1)];
  }
  // An entry outside the pool reads page 0 instead: memory-safe but wrong when it lies
  // inside the context (int8attn_check_block_table reports such tables).
  __device__ __forceinline__ void issue(int p_raw, int8_t (*kv_lds)[4 * kPfPage],
                                        float (*sc_lds)[64]) const {
    const int t = w & 3;
    const int p = (uint32_t)p_raw < (uint32_t)num_pages ? p_raw : 0;
    if (w < 8) {
      const int kv = w >> 2;
      const int8_t* src = (kv ? v_cache : k_cache) + ((size_t)p * n_kv_heads + g) * kBlockBytes;
      int8_t* dst = &kv_lds[kv][t * (kv ? kBlockBytes : kPfPage)];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint32_t lo = lane * 16 + qq * 1024;
        asm volatile("" : "+v"(lo));  // keeps (scalar base, 32-bit lane offset) addressing
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(src + lo),
            (__attribute__((address_space(3))) void*)(dst + qq * 1024), 16, 0, 0);
      }
    } else if (lane < 16) {
      // 32-bit element index: the launcher checks num_pages * n_kv_heads * 16 < 2^32.
      const uint32_t off = ((uint32_t)p * (uint32_t)n_kv_heads + (uint32_t)g) * kPage;
      uint32_t lo = lane;
      asm volatile("" : "+v"(lo));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(k_scale + off + lo),
                                       (__attribute__((address_space(3))) void*)&sc_lds[0][16 * t],
                                       4, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(v_scale + off + lo),
                                       (__attribute__((address_space(3))) void*)&sc_lds[1][16 * t],
                                       4, 0, 0);
    }
  }
};

// Per-lane constants of a wave's 16 query rows.
struct RowCtx {
  const int8_t* qcol;  // this lane's B-operand bytes of the query codes (LDS)
  int koff, voff;      // A-operand byte offsets in a staged K / V block
  int gq, lim, kfull, ctx;
  float rs;            // sQ * sm_scale * log2(e), > 0
  v4i qB[4];           // the query operand, held for the whole loop
};

// Running softmax state of one lane: its query row's max and partial sum, 64 of the
// row's fp32 output accumulators (dims 16 dt + 4 gq + i), and the offset they carry.
struct RowState {
  float m_run, l_part, corr;
  v4f acc[16];
};

// One 64-key block: reads the staged block (sK/sV/sSk/sSv) and first issues the loads
// of the next one into the other buffer (nKV/nSc). The two buffers are distinct LDS
// variables, so the compiler can tell the in-flight direct-to-LDS writes from the reads
// of this block and need not wait for them before reading.
// GUARD: a row may meet blocks before its first visible key (a key partition that
// starts past the row's last key); its state then stays empty instead of taking NaNs.
// Without key partitions every row sees key 0 in its first block.
template <int GUARD>
__device__ __forceinline__ void block_step(
    int kb, int nkb, const BlockLoader& ld, int& pg_next, const RowCtx& rc,
    RowState& st, const int8_t* sK, const int8_t* sV, const float* sSk, const float* sSv,
    int8_t (*nKV)[4 * kPfPage], float (*nSc)[64]) {
  // QK: S[t] rows = tokens 4t..4t+3 of each of the 4 pages. The operands of group u+1
  // are read while the products of group u run.
  v4i S[4];
  auto qk = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] = v4i{0, 0, 0, 0};
    v4i ka[4], qa;
#pragma unroll
    for (int t = 0; t < 4; ++t) ka[t] = *reinterpret_cast<const v4i*>(sK + rc.koff + t * 64);
    qa = rc.qB[0];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v4i kn[4], qn;
      if (u < 3) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kn[t] = *reinterpret_cast<const v4i*>(sK + rc.koff + (u + 1) * 1024 + t * 64);
        qn = rc.qB[u + 1];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) S[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka[t], qa, S[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (u < 3) {
#pragma unroll
        for (int t = 0; t < 4; ++t) ka[t] = kn[t];
        qa = qn;
      }
    }
  };
  qk();
  // The next block's loads go out once this block's query reads are issued.
  if (kb + 1 < nkb) {
    ld.issue(pg_next, nKV, nSc);
    pg_next = ld.page(kb + 2);
  }
  // y = qk * sK (key 16gq + 4t + i of the block), masked on diagonal / tail blocks only.
  const int key0 = kb * 64;
  const bool need_mask = (key0 + 64 > rc.kfull) || (key0 + 64 > rc.ctx);
  float y[16], sv[16];
  auto scores = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 sk = *reinterpret_cast<const float4*>(&sSk[16 * rc.gq + 4 * t]);
      const float4 vs = *reinterpret_cast<const float4*>(&sSv[16 * rc.gq + 4 * t]);
      y[4 * t] = (float)S[t][0] * sk.x;
      y[4 * t + 1] = (float)S[t][1] * sk.y;
      y[4 * t + 2] = (float)S[t][2] * sk.z;
      y[4 * t + 3] = (float)S[t][3] * sk.w;
      sv[4 * t] = vs.x; sv[4 * t + 1] = vs.y; sv[4 * t + 2] = vs.z; sv[4 * t + 3] = vs.w;
    }
    if (need_mask) {  // diagonal or context-tail block (wave-uniform)
      // Masked keys (including slots past the context, whose scales are not data) get
      // y = -inf and sV = 0, so their weight is exactly 0.
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 16 * rc.gq + e >= rc.lim) {
          y[e] = -INFINITY;
          sv[e] = 0.f;
        }
    }
  };
  scores();
  // Weights against the running max as it stands: no block max is taken on this path.
  // The lane's sum of the block's weights then shows whether a score passed the running
  // max by more than the lazy window (a weight above 2^8 makes the sum exceed it; a row
  // with no reference max yet gives a non-finite sum): only then is the block redone on
  // the exact path, with the block max and the rescale. Both paths produce the same
  // weights whenever no rescale is due, so the result does not depend on the path.
  float wm = 0.f, lb = 0.f;
  bool exact = __any(st.m_run == -INFINITY);
  if (!exact) {
    const float nm0 = -st.m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(y[e], rc.rs, nm0));
      lb += p;
      y[e] = p * sv[e];
      wm = fmaxf(wm, y[e]);
    }
    exact = __any(!(lb <= (float)(1 << (int)kLazyRescale)));
  }
  if (exact) {  // first block of a row, or a score beyond the lazy window: recompute
    qk();
    scores();
    float ymax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) ymax = fmaxf(ymax, y[e]);
    const float xmax = ymax * rc.rs;
    if (__any(xmax > st.m_run + kLazyRescale)) {
      const float m_new = fmaxf(st.m_run, col_max(xmax));
      const float alpha = (GUARD && m_new == st.m_run) ? 1.0f : __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) st.acc[dt] *= alpha;
      st.l_part *= alpha;
      st.corr *= alpha;
      st.m_run = m_new;
    }
    const float nm = (GUARD && st.m_run == -INFINITY) ? 0.f : -st.m_run;
    wm = 0.f;
    lb = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(y[e], rc.rs, nm));
      lb += p;
      y[e] = p * sv[e];
      wm = fmaxf(wm, y[e]);
    }
  }
  st.l_part += lb;
  wm = __uint_as_float(col_max_u(__float_as_uint(wm)));  // wm >= 0: integer order
  // 127 / wm via the hardware reciprocal (about 1 ulp): a code can move only at an
  // exact rounding tie, and w * inv stays below 127.5, so codes never exceed 127.
  // fma(w, inv, 1.5 * 2^23) lies in [2^23, 2^24), where the fp32 spacing is 1, so its
  // single rounding (to nearest even) leaves rint(w * inv) in the low byte.
  const float inv = wm > 0.f ? 127.0f * __builtin_amdgcn_rcpf(wm) : 0.f;
  const float sb = wm * (1.0f / 127.0f);
  v4i Pb;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(fmaf(y[4 * t + i], inv, kMagicF));
    const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);  // [r0.b0, r1.b0, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(r[3], r[2], 0x04000c0cu);  // [0, 0, r2.b0, r3.b0]
    Pb[t] = (int)(lo | hi);
  }

  // PV: out^T(dim tile dt) += s_b * V^T(dt) . P^T; the A operand of lane (n, gq) is
  // the 16 token codes of dim 16dt + n in page gq, one 16-byte LDS read. The operands of
  // group q4+1 are read while the products of group q4 run; each group's fold follows
  // its 4 products.
  v4i va[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) va[u] = *reinterpret_cast<const v4i*>(sV + rc.voff + u * 256);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    v4i vn[4];
    if (q4 < 3) {
#pragma unroll
      for (int u = 0; u < 4; ++u) vn[u] = *reinterpret_cast<const v4i*>(sV + rc.voff + ((q4 + 1) * 4 + u) * 256);
    }
    v4i r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(va[u], Pb, kMagic4, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[q4 * 4 + u][i] = fmaf(__int_as_float(r[u][i]), sb, st.acc[q4 * 4 + u][i]);
    __builtin_amdgcn_sched_barrier(0);
    if (q4 < 3) {
#pragma unroll
      for (int u = 0; u < 4; ++u) va[u] = vn[u];
    }
  }
  st.corr = fmaf(sb, kMagicF, st.corr);
  if ((kb & (kFlushBlocks - 1)) == kFlushBlocks - 1) {  // bounds the offset carried
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.acc[dt] -= st.corr;
    st.corr = 0.f;
  }
  // Pin the fold and the row sum of this block before the barrier (left alone, the
  // compiler sinks them past it and keeps the 16 raw products live across).
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) asm volatile("" : "+v"(st.acc[dt]));
  asm volatile("" : "+v"(st.l_part), "+v"(st.corr));
  if (kb + 1 < nkb) __builtin_amdgcn_s_waitcnt(0);  // the next block has landed in LDS
  lds_barrier();
}

// Q8: the query arrives as int8 codes with fp32 scales (kv_produce's output) instead of
// bf16 rows to quantize.
// SPLIT: the keys are cut into partitions of part_blocks 64-key blocks, one workgroup per
// (KV head, partition, query block); each writes the partial softmax state (max, sum,
// unnormalised output) of its rows over its partition, and the row merge kernel
// (merge_rows_kernel) combines them.
struct SplitOut {
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int part_blocks;  // 64-key blocks per partition
  int n_parts;
};

template <int Q8, int SPLIT>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_chunk_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scales, int n_new,
    const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int ctx,
    int causal, int num_pages, int n_q_heads, int n_kv_heads, float qk_scale_log2,
    float* __restrict__ out, int n_qb, int xcd_per_head, SplitOut sp) {
  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs (linear id
  // mod 8), so give each KV head its own XCDs (8 / H of them when H divides 8). Each
  // XCD's L2 then streams the K/V of one head instead of all of them.
  int qb, g, part = 0;
  if (SPLIT) {
    // Work items (KV head, partition, query block), query block fastest, dealt to the
    // XCDs in 8 contiguous runs: the query blocks that read one partition share an L2.
    const int total = n_kv_heads * sp.n_parts * n_qb;
    const int per = (total + kXcds - 1) / kXcds;
    const int L = blockIdx.x, wi = (L % kXcds) * per + L / kXcds;
    if (wi >= total) return;  // padding workgroup (whole block)
    qb = wi % n_qb;
    part = (wi / n_qb) % sp.n_parts;
    g = wi / (n_qb * sp.n_parts);
  } else {
    const int L = blockIdx.x, xcd = L % kXcds, slot = L / kXcds;
    if (xcd_per_head > 0) {
      g = xcd / xcd_per_head;
      qb = slot * xcd_per_head + xcd % xcd_per_head;
    } else {
      g = L / n_qb;
      qb = L % n_qb;
    }
    if (qb >= n_qb || g >= n_kv_heads) return;  // padding workgroup (whole block)
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = w >> 1, half = w & 1;  // head within the group, 16-token half
  const int h = g * kGroup + hl;
  const int n = lane & 15, gq = lane >> 4;
  const int t0 = qb * kPfTok;
  const int nq = min(kPfTok, n_new - t0);
  const int pos0 = ctx - n_new;
  const int kend = causal ? pos0 + t0 + nq : ctx;  // keys [0, kend) are needed
  // 64-key blocks [kb0, nkb) of this workgroup: all of them, or one partition's
  const int kb0 = SPLIT ? part * sp.part_blocks : 0;
  const int nkb = SPLIT ? min((kend + 63) >> 6, kb0 + sp.part_blocks) : (kend + 63) >> 6;
  if (SPLIT && kb0 >= nkb) return;  // no row of this tile reaches the partition (whole block)
  const int my_tok = t0 + 16 * half + n;            // this lane's query token

  // Two K/V buffers and two scale buffers, each its own LDS variable.
  __shared__ __align__(16) int8_t s_kv0[2][4 * kPfPage];  // [K,V][4 pages]
  __shared__ __align__(16) int8_t s_kv1[2][4 * kPfPage];
  __shared__ __align__(16) float s_sc0[2][64];            // [K,V][key]
  __shared__ __align__(16) float s_sc1[2][64];
  __shared__ __align__(16) int8_t s_q[kGroup * kPfTok][kQStride];  // query codes
  __shared__ float s_qs[kGroup][kPfTok];

  const BlockLoader ld{k_cache, v_cache, k_scale, v_scale, block_table, (ctx + kPage - 1) / kPage,
                       num_pages, n_kv_heads, g, w, lane};
  int pg_next = ld.page(kb0);
  if (nkb > kb0) ld.issue(pg_next, s_kv0, s_sc0);  // first block in flight during the Q work
  pg_next = ld.page(kb0 + 1);

  // ---- quantize this wave's 16 query rows (head h); rows past the chunk are zero.
  int8_t* qrows = &s_q[hl * kPfTok + 16 * half][0];
  {
    uint2 qw[16];
    float qsc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = min(t0 + 16 * half + r, n_new - 1);
      const size_t row = (size_t)tok * n_q_heads + h;
      if (Q8) {
        qw[r].x = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(q) + row * kHeadDim + lane * 4);
        qsc[r] = q_scales[row];
      } else {
        qw[r] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + row * kHeadDim + lane * 4);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sc = qsc[r];
      uint32_t c = Q8 ? qw[r].x
                      : quantize4(bf16_to_f32(qw[r].x & 0xffffu), bf16_to_f32(qw[r].x >> 16),
                                  bf16_to_f32(qw[r].y & 0xffffu), bf16_to_f32(qw[r].y >> 16), &sc);
      const bool live = 16 * half + r < nq;
      *reinterpret_cast<uint32_t*>(qrows + r * kQStride + lane * 4) = live ? c : 0u;
      if (lane == 0) s_qs[hl][16 * half + r] = live ? sc : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  RowCtx rc;
  rc.qcol = qrows + n * kQStride + gq * 16;
  // A-operand bytes: QK row n = token 4t + n%4 of page n/4 (dims 64u + 16gq..),
  // PV row n of dim tile dt = dim 16dt + n of page gq (its 16 tokens).
  rc.koff = (n >> 2) * kPfPage + gq * 256 + (n & 3) * 16;
  rc.voff = gq * kBlockBytes + n * 16;
  rc.gq = gq;
  rc.lim = causal ? min(pos0 + my_tok + 1, ctx) : ctx;  // keys < lim are visible
  rc.kfull = causal ? pos0 + t0 + 1 : ctx;              // keys < kfull are seen by every row
  rc.ctx = ctx;
  // rs > 0 keeps max(x) = rs * max(y) and exp2(fma(y, rs, -m)) = 0 for masked y = -inf.
  rc.rs = fmaxf(s_qs[hl][16 * half + n] * qk_scale_log2, 1e-30f);
#pragma unroll
  for (int u = 0; u < 4; ++u) rc.qB[u] = *reinterpret_cast<const v4i*>(rc.qcol + u * 64);

  RowState st;
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  st.corr = 0.f;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) st.acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb = kb0; kb < nkb; kb += 2) {
    block_step<SPLIT>(kb, nkb, ld, pg_next, rc, st, s_kv0[0], s_kv0[1], s_sc0[0], s_sc0[1], s_kv1,
                      s_sc1);
    if (kb + 1 < nkb)
      block_step<SPLIT>(kb + 1, nkb, ld, pg_next, rc, st, s_kv1[0], s_kv1[1], s_sc1[0], s_sc1[1], s_kv0,
                        s_sc0);
  }

  // ---- normalise and store: lane (n, gq) holds dims 16*dt + 4*gq + i of its row.
  const float l = col_sum(st.l_part);
  if (SPLIT) {  // the partial state over this partition (rows without a key in it are
                // never read by the merge)
    if (my_tok < t0 + nq) {
      const size_t pi = ((size_t)my_tok * n_q_heads + h) * sp.n_parts + part;
      float* o = sp.ws_o + pi * kHeadDim + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        float4 v;
        v.x = st.acc[dt][0] - st.corr; v.y = st.acc[dt][1] - st.corr;
        v.z = st.acc[dt][2] - st.corr; v.w = st.acc[dt][3] - st.corr;
        *reinterpret_cast<float4*>(o + 16 * dt) = v;
      }
      if (gq == 0) {
        sp.ws_m[pi] = st.m_run;
        sp.ws_l[pi] = l;
      }
    }
    return;
  }
  if (my_tok < t0 + nq) {
    const float il = 1.0f / l;
    float* o = out + ((size_t)my_tok * n_q_heads + h) * kHeadDim + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      float4 v;
      v.x = (st.acc[dt][0] - st.corr) * il; v.y = (st.acc[dt][1] - st.corr) * il;
      v.z = (st.acc[dt][2] - st.corr) * il; v.w = (st.acc[dt][3] - st.corr) * il;
      *reinterpret_cast<float4*>(o + 16 * dt) = v;
    }
  }
}

// Bytes of the partial states of np (row, head, partition) triples: o[256], m and l in
// fp32, rounded up to 256.
static size_t split_state_bytes(size_t np) {
  return ((2 * np + np * kHeadDim) * sizeof(float) + 255) / 256 * 256;
}

int launch_prefill(const void* q, const float* q_scales, int n_new, const int8_t* k_cache,
                   const int8_t* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int ctx, int causal, int num_pages, int n_q_heads, int n_kv_heads,
                   float sm_scale, float* out, float* ws, size_t ws_bytes, hipStream_t stream) {
  const int n_qb = (n_new + kPfTok - 1) / kPfTok;
  // Heads spread over the XCDs when the head count divides their number; otherwise the
  // plain (head-major) order.
  const int xcd_per_head = (n_kv_heads <= kXcds && kXcds % n_kv_heads == 0) ? kXcds / n_kv_heads : 0;
  const long long n_wg = xcd_per_head > 0
                             ? (long long)kXcds * ((n_qb + xcd_per_head - 1) / xcd_per_head)
                             : (long long)n_qb * n_kv_heads;
  SplitOut sp{nullptr, nullptr, nullptr, 0, 1};
  const int n_parts = ws != nullptr ? prefill_split_parts(n_new, ctx, causal, n_kv_heads, &sp.part_blocks) : 1;
  if (n_parts > 1) {
    const size_t np = (size_t)n_new * n_q_heads * n_parts;
    if (ws_bytes < prefill_split_ws_bytes(n_new, ctx, causal, n_q_heads, n_kv_heads))
      return set_error(I8A_EWORKSPACE, "attn_prefill_chunk_split: workspace too small");
    sp.ws_o = ws;  // [row][head][partition][256], then m and l
    sp.ws_m = ws + np * kHeadDim;
    sp.ws_l = sp.ws_m + np;
    sp.n_parts = n_parts;
    if (q_scales == nullptr) {
      // bf16 rows: quantized once here (bit for bit the in-kernel quantizer) instead of by
      // every partition's workgroup; the int8 codes and scales follow the partial states.
      const size_t rows = (size_t)n_new * n_q_heads;
      int8_t* codes = reinterpret_cast<int8_t*>(ws) + split_state_bytes(np);
      float* scales = reinterpret_cast<float*>(codes + (rows * kHeadDim + 255) / 256 * 256);
      int rc = launch_q_quant(static_cast<const uint16_t*>(q), (int)rows, codes, scales, stream);
      if (rc) return rc;
      q = codes;
      q_scales = scales;
    }
  }
  const dim3 grid(n_parts > 1 ? (unsigned)(kXcds * ((n_qb * n_kv_heads * n_parts + kXcds - 1) / kXcds))
                              : (unsigned)n_wg);
  const float qs = sm_scale * kLog2e;
#define PF_ARGS q, q_scales, n_new, k_cache, v_cache, k_scale, v_scale, block_table, ctx, causal, \
                num_pages, n_q_heads, n_kv_heads, qs, out, n_qb, xcd_per_head, sp
  if (n_parts > 1) {  // (the query is int8 codes by now)
    hipLaunchKernelGGL((prefill_chunk_kernel<1, 1>), grid, dim3(kPfThreads), 0, stream, PF_ARGS);
  } else {
    if (q_scales != nullptr)
      hipLaunchKernelGGL((prefill_chunk_kernel<1, 0>), grid, dim3(kPfThreads), 0, stream, PF_ARGS);
    else
      hipLaunchKernelGGL((prefill_chunk_kernel<0, 0>), grid, dim3(kPfThreads), 0, stream, PF_ARGS);
  }
#undef PF_ARGS
  int rc = check_launch("attn_prefill_chunk");
  if (rc || n_parts == 1) return rc;
  // Query row t of the chunk sees ctx - n_new + t + 1 keys: the merge of nq = n_new rows.
  return launch_merge_rows(sp.ws_m, sp.ws_l, sp.ws_o, ctx, n_new, n_q_heads, n_parts,
                           sp.part_blocks * 64, out, stream);
}

// Partitions for a chunk whose single pass would leave most CUs idle: causal chunks with
// fewer than 128 (query block, KV head) workgroups are cut into partitions of whole
// 64-key blocks so that about 256 workgroups run. Returns 1 for the single pass.
int prefill_split_parts(int n_new, int ctx, int causal, int n_kv_heads, int* part_blocks) {
  const long long n_wg = (long long)((n_new + kPfTok - 1) / kPfTok) * n_kv_heads;
  const int nkb = (int)(((long long)ctx + 63) / 64);
  *part_blocks = nkb;
  if (!causal || n_wg <= 0 || n_wg >= 128 || nkb < 2) return 1;
  int parts = (int)((256 + n_wg - 1) / n_wg);
  parts = parts < nkb ? parts : nkb;
  const int pb = (nkb + parts - 1) / parts;
  *part_blocks = pb;
  return (nkb + pb - 1) / pb;
}

size_t prefill_split_ws_bytes(int n_new, int ctx, int causal, int n_q_heads, int n_kv_heads) {
  int pb;
  const int parts = prefill_split_parts(n_new, ctx, causal, n_kv_heads, &pb);
  if (parts <= 1) return 0;
  const size_t rows = (size_t)n_new * n_q_heads;
  return split_state_bytes(rows * parts) + (rows * kHeadDim + 255) / 256 * 256 +
         (rows * sizeof(float) + 255) / 256 * 256;
}

}  // namespace i8a
