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
constexpr int kFlatMinSeqs = 16;       // batches of this size and up to kFlatMaxSeqs take
constexpr int kFlatMaxSeqs = 4096;     // the flattened grid
constexpr int kFlatWorkgroups = 256;  // one per CU (the split kernel fits one per CU)
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
#include "decode_item.inc"
}

// A batch of sequences of unequal lengths. The (partition, head, sequence) grid would
// hold a workgroup for every partition up to the longest context, most of them past
// their own sequence's end, and with one workgroup per CU each of those still occupies
// a CU for its launch and first memory round trip. Instead every workgroup lists the
// real work items -- sequence s has max(1, ceil(ctx_s / 512)) partitions, prefix sums
// in LDS -- and takes items blockIdx.x, blockIdx.x + gridDim.x, ... (a sequence with no
// key still gets its one item, which writes its zeros or an empty partial).
template <int Q8>
__global__ __launch_bounds__(512, 1) void decode_split_flat_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scales,
    const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int num_pages, int n_q_heads,
    int n_kv_heads, float qk_scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int max_parts, float* __restrict__ out, int num_seqs) {
  const int tid0 = threadIdx.x;
  const int w0 = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  __shared__ int s_pref[kFlatMaxSeqs + 1];
  if (w0 == 0) {
    const int ln = tid0;
    const int per = (num_seqs + 63) / 64;  // sequences per lane
    const int i0 = min(ln * per, num_seqs), i1 = min(i0 + per, num_seqs);
    int local = 0;
    for (int i = i0; i < i1; ++i) {
      const int c = min(max(ctx_lens[i], 0), ctx_cap);
      local += max(1, (c + kPart - 1) / kPart);
    }
    int incl = local;  // inclusive scan over the 64 lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (ln >= d) incl += v;
    }
    int run = incl - local;
    for (int i = i0; i < i1; ++i) {
      s_pref[i] = run;
      const int c = min(max(ctx_lens[i], 0), ctx_cap);
      run += max(1, (c + kPart - 1) / kPart);
    }
    if (ln == 63) s_pref[num_seqs] = incl;
  }
  lds_barrier();
  const int n_items = s_pref[num_seqs] * n_kv_heads;
  auto item = [&](const int j, const int g, const int s) {
    // (the thread index goes through an opaque copy, so that the values derived from it
    // are recomputed per item instead of held in registers across the loop)
    int tid_item = tid0;
    asm volatile("" : "+v"(tid_item));
    const int tid = tid_item, lane = tid & 63;
    const int w = w0;
#include "decode_item.inc"
  };
  const int stride = (num_seqs + 63) / 64;  // <= 64 for kFlatMaxSeqs sequences
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int pidx = it / n_kv_heads, g = it - pidx * n_kv_heads;
    // The sequence s with s_pref[s] <= pidx < s_pref[s + 1], in two wave-wide steps (the
    // prefix is strictly increasing, so the lanes that pass form a prefix of the wave):
    // first among every stride-th sequence, then among the stride that follow.
    const int ln = tid0 & 63;
    const unsigned long long m1 = __ballot(s_pref[min(ln * stride, num_seqs)] <= pidx);
    const int lo = (63 - __builtin_clzll(m1)) * stride;
    const unsigned long long m2 = __ballot(s_pref[min(lo + ln, num_seqs)] <= pidx);
    const int sq = __builtin_amdgcn_readfirstlane(lo + 63 - __builtin_clzll(m2));
    item(pidx - s_pref[sq], g, sq);
    lds_barrier();  // this item's LDS reads are done before the next item's writes
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
  __shared__ __align__(16) float s_a[64];  // the chunk's partition weights, broadcast
  float M = -INFINITY, L = 0.f, acc = 0.f;
  // The first chunk is merged whatever P is (P = 0: every weight 0, output 0 below): with
  // no exit before it, its loads are issued together with the context length's instead of
  // after it.
  for (int j0 = 0; j0 == 0 || j0 < P; j0 += 64) {
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
  o[d] = P > 0 ? acc / L : 0.f;
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
  // Batches of kFlatMinSeqs..kFlatMaxSeqs sequences: the flattened grid of real work
  // items, one workgroup per CU; otherwise the (partition, head, sequence) grid. (The
  // flattened loop costs ~1 us more per item than a fresh workgroup, so it wins where
  // the grid would hold many partitions past their sequence's end -- unequal lengths --
  // and loses a few percent on batches of equal lengths; small batches keep the grid.)
  const bool flat = num_seqs >= kFlatMinSeqs && num_seqs <= kFlatMaxSeqs;
  const long long items_max = (long long)num_seqs * max_parts * n_kv_heads;
  const dim3 grid = flat ? dim3((unsigned)(items_max < kFlatWorkgroups ? items_max : kFlatWorkgroups))
                         : dim3(max_parts, n_kv_heads, num_seqs);
#define DEC_ARGS q, q_scales, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, ctx_lens, \
                 ctx_cap, num_pages, n_q_heads, n_kv_heads, sm_scale * kLog2e, ws_m, ws_l, ws_o,   \
                 max_parts, max_parts == 1 ? out : nullptr
  if (q_scales != nullptr) {
    if (flat)
      hipLaunchKernelGGL(decode_split_flat_kernel<1>, grid, dim3(512), 0, stream, DEC_ARGS, num_seqs);
    else
      hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(512), 0, stream, DEC_ARGS);
  } else {
    if (flat)
      hipLaunchKernelGGL(decode_split_flat_kernel<0>, grid, dim3(512), 0, stream, DEC_ARGS, num_seqs);
    else
      hipLaunchKernelGGL(decode_split_kernel<0>, grid, dim3(512), 0, stream, DEC_ARGS);
  }
#undef DEC_ARGS
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
