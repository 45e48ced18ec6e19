// Split-K decode over the paged INT8 KV cache with the weighted sum of V on the int8
// matrix cores, for 1..8 query rows per sequence.
//
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.3: the decode kernel reads the
// paged INT8 K/V directly and runs INT8 QK and INT8 PV, the V scale folded into the
// softmax weight and the weights quantized per block with scale = block absmax / 127;
// 256-token partitions. "dot4-flash-attention" README route table: split-K stage 1 over
// row splits, stage 2 merge; next steps: split-K for small query batches. vLLM docs
// page, "The selection law": the number of KV segments is a power of two derived from a
// workgroup-count target over (kv heads x query rows), with a floor on keys per
// segment.)
//
// Workgroup = (partition j of 64 * WAVES keys, KV head g, sequence s). Wave w owns the
// aligned 64-key block [64w, 64w+64) of the partition (4 pages) and loads its K and V
// codes once into registers. The 6 * nq query rows of the group, r = 6 i + head, are
// taken in tiles of 16 (the matrix-core columns):
//  * QK as S^T = K . Q^T on v_mfma_i32_16x16x64_i8, one accumulator per page; lane
//    (n, gq) then holds tokens 4gq..4gq+3 of every page for query row n;
//  * one softmax over the block (the wave's whole share of the partition, so no
//    running rescale): x = qk * sK * sQ * sm_scale * log2 e, p = 2^(x - max),
//    w = p * sV / max sV, block scale s_b = max w / 127;
//  * the weights w / s_b in [0, 127] as DIG int8 digit planes:
//      DIG = 1: c = rint(w / s_b), the int8-P path (one plane);
//      DIG = 3: U = rint(2^14 w / s_b) split into 7-bit digits d0 d1 d2, so that
//               w / s_b = (2^14 d0 + 2^7 d1 + d2) / 2^14 to 2^-15 (fp32-class path);
//  * PV as out^T = V^T . P^T on v_mfma_i32_16x16x64_i8 with K = the 64 keys of the
//    block (key 16 kg + 4 t + i = token 4 kg + i of page t): the A operand of lane
//    (m, kg) is 4 dwords, tokens 4kg..4kg+3 of dim 16 dt + m from each page, which a
//    4x4 lane transpose of the loaded V dwords provides; the B operand of lane (n, kg)
//    is exactly the 16 codes that lane computed. The planes' int32 products are
//    combined as (2^7 X0 + X1) + X2 / 2^7 (the first two exact in int32 by chaining
//    the accumulator); the third plane and the single plane are read back through the
//    exponent-offset trick (accumulator started at the bits of 1.5 * 2^23).
// The wave states (max, sum, output in units of the block scale) are merged in LDS per
// tile into one partial per (query row, partition); the partials are merged by the
// log-sum-exp stage of the one-row decode.
#include "common.hpp"
#include "launch.hpp"

namespace i8a {

namespace {

constexpr int kRowTile = 16;            // query rows per matrix-core column tile
constexpr int kMaxQRows = kGroup * 8;   // 6 heads x at most 8 query rows
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23
constexpr int kMagicBits = 0x4B400000;  // its bits
constexpr int kFlatMinSeqs = 16;        // batches of kFlatMinSeqs..kFlatMaxSeqs sequences with
constexpr int kFlatMaxSeqs = 1024;      // 512-key partitions take the flattened grid (the
                                        // prefix sums share the LDS with ~151 KB of tiles)
constexpr int kFlatWorkgroups = 256;    // one per CU

// Four bytes, byte k of the result = byte `b` of x_k (x_k = register k).
__device__ __forceinline__ uint32_t pack_byte(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x0c0c0400u);  // [x0.b0, x1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(x3, x2, 0x04000c0cu);  // [0, 0, x2.b0, x3.b0]
  return lo | hi;
}

// Q8: the query arrives as int8 codes with fp32 scales (kv_produce's output).
template <int DIG, int WAVES, int Q8>
__global__ __launch_bounds__(WAVES * 64, 1) void split_i8pv_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scales, int nq,
    const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int num_pages, int n_q_heads,
    int n_kv_heads, float qk_scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int max_parts, float* __restrict__ out) {
  // out != nullptr: a single partition per sequence, so the workgroup writes the
  // normalized output itself and no merge stage runs.
  constexpr int kKeys = WAVES * 64;  // keys per partition
  constexpr int kRowsPerWave = (kMaxQRows + WAVES - 1) / WAVES;
  // Value the stored outputs carry on top of the product (the offset of the trick).
  constexpr float kOffset = DIG == 1 ? kMagicF : kMagicF / 128.0f;
  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = WAVES == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
#include "decode_i8pv_item.inc"
}

// Batches of 16+ sequences with 512-key partitions: the flattened grid of real work items,
// as decode_split_flat_kernel does for the one-row decode (sequence s has max(1,
// ceil(ctx_s / 512)) partitions; prefix sums in LDS; items blockIdx.x, + gridDim.x, ...).
template <int DIG, int Q8>
__global__ __launch_bounds__(512, 1) void split_i8pv_flat_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scales, int nq,
    const int8_t* __restrict__ k_cache,
    const int8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ ctx_lens, int ctx_cap, int num_pages, int n_q_heads,
    int n_kv_heads, float qk_scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int max_parts, float* __restrict__ out, int num_seqs) {
  constexpr int WAVES = 8;
  constexpr int kKeys = WAVES * 64;
  constexpr int kRowsPerWave = (kMaxQRows + WAVES - 1) / WAVES;
  constexpr float kOffset = DIG == 1 ? kMagicF : kMagicF / 128.0f;
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
      local += max(1, (c + kKeys - 1) / kKeys);
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
      run += max(1, (c + kKeys - 1) / kKeys);
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
    // (likewise the wave index, so that the per-row conditions derived from it are
    // recomputed per item as scalar compares instead of flags kept, and spilled, across it)
    int w_item = w0;
    asm volatile("" : "+s"(w_item));
    const int w = w_item;
#include "decode_i8pv_item.inc"
  };
  const int stride = (num_seqs + 63) / 64;  // <= 16 for kFlatMaxSeqs sequences
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int pidx = it / n_kv_heads, g = it - pidx * n_kv_heads;
    // the sequence s with s_pref[s] <= pidx < s_pref[s + 1], by two wave-wide ballots
    const int ln = tid0 & 63;
    const unsigned long long m1 = __ballot(s_pref[min(ln * stride, num_seqs)] <= pidx);
    const int lo = (63 - __builtin_clzll(m1)) * stride;
    const unsigned long long m2 = __ballot(s_pref[min(lo + ln, num_seqs)] <= pidx);
    const int sq = __builtin_amdgcn_readfirstlane(lo + 63 - __builtin_clzll(m2));
    item(pidx - s_pref[sq], g, sq);
    lds_barrier();  // this item's LDS reads are done before the next item's writes
  }
}

template <int DIG, int WAVES>
int launch_split(const void* q, const float* q_scales, int nq, const int8_t* k_cache, const int8_t* v_cache,
                 const float* k_scale, const float* v_scale, const int32_t* block_table,
                 int max_blocks, const int32_t* ctx_lens, int ctx_cap, int num_seqs,
                 int num_pages, int n_q_heads, int n_kv_heads, float qk_scale_log2, float* ws_m,
                 float* ws_l, float* ws_o, int max_parts, float* out, hipStream_t stream) {
  if (WAVES == 8 && num_seqs >= kFlatMinSeqs && num_seqs <= kFlatMaxSeqs) {
    const long long items_max = (long long)num_seqs * max_parts * n_kv_heads;
    const dim3 grid((unsigned)(items_max < kFlatWorkgroups ? items_max : kFlatWorkgroups));
    if (q_scales != nullptr)
      hipLaunchKernelGGL((split_i8pv_flat_kernel<DIG, 1>), grid, dim3(512), 0, stream, q, q_scales,
                         nq, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, ctx_lens,
                         ctx_cap, num_pages, n_q_heads, n_kv_heads, qk_scale_log2, ws_m, ws_l, ws_o,
                         max_parts, out, num_seqs);
    else
      hipLaunchKernelGGL((split_i8pv_flat_kernel<DIG, 0>), grid, dim3(512), 0, stream, q, q_scales,
                         nq, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, ctx_lens,
                         ctx_cap, num_pages, n_q_heads, n_kv_heads, qk_scale_log2, ws_m, ws_l, ws_o,
                         max_parts, out, num_seqs);
    return check_launch("int8-PV decode stage 1");
  }
  if (q_scales != nullptr)
    hipLaunchKernelGGL((split_i8pv_kernel<DIG, WAVES, 1>), dim3(max_parts, n_kv_heads, num_seqs),
                       dim3(WAVES * 64), 0, stream, q, q_scales, nq, k_cache, v_cache, k_scale,
                       v_scale, block_table, max_blocks, ctx_lens, ctx_cap, num_pages, n_q_heads,
                       n_kv_heads, qk_scale_log2, ws_m, ws_l, ws_o, max_parts, out);
  else
    hipLaunchKernelGGL((split_i8pv_kernel<DIG, WAVES, 0>), dim3(max_parts, n_kv_heads, num_seqs),
                       dim3(WAVES * 64), 0, stream, q, q_scales, nq, k_cache, v_cache, k_scale,
                       v_scale, block_table, max_blocks, ctx_lens, ctx_cap, num_pages, n_q_heads,
                       n_kv_heads, qk_scale_log2, ws_m, ws_l, ws_o, max_parts, out);
  return check_launch("int8-PV decode stage 1");
}

}  // namespace

int launch_decode_i8pv(int digits, int part_rows, const void* q, const float* q_scales, int nq,
                       const int8_t* k_cache,
                       const int8_t* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int max_blocks, const int32_t* ctx_lens,
                       int num_seqs, int max_ctx, int num_pages, int n_q_heads, int n_kv_heads,
                       float sm_scale, float* out, float* ws, hipStream_t stream) {
  const int max_parts = (max_ctx + part_rows - 1) / part_rows;
  const size_t np = (size_t)num_seqs * nq * n_q_heads * max_parts;
  float* ws_m = ws;
  float* ws_l = ws + np;
  float* ws_o = ws + 2 * np;
  const long long cap = (long long)max_blocks * kPage;
  const int ctx_cap = (int)(cap < max_ctx ? cap : max_ctx);
  const float qs = sm_scale * kLog2e;
  float* direct = max_parts == 1 ? out : nullptr;  // one partition: no merge stage
  int rc;
#define I8PV_ARGS q, q_scales, nq, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, ctx_lens, \
                  ctx_cap, num_seqs, num_pages, n_q_heads, n_kv_heads, qs, ws_m, ws_l, ws_o,   \
                  max_parts, direct, stream
  if (digits == 1) {
    switch (part_rows) {
      case 64: rc = launch_split<1, 1>(I8PV_ARGS); break;
      case 128: rc = launch_split<1, 2>(I8PV_ARGS); break;
      case 256: rc = launch_split<1, 4>(I8PV_ARGS); break;
      default: rc = launch_split<1, 8>(I8PV_ARGS); break;
    }
  } else {
    switch (part_rows) {
      case 64: rc = launch_split<3, 1>(I8PV_ARGS); break;
      case 128: rc = launch_split<3, 2>(I8PV_ARGS); break;
      case 256: rc = launch_split<3, 4>(I8PV_ARGS); break;
      default: rc = launch_split<3, 8>(I8PV_ARGS); break;
    }
  }
#undef I8PV_ARGS
  if (rc || direct != nullptr) return rc;
  return launch_merge(ws_m, ws_l, ws_o, ctx_lens, ctx_cap, num_seqs, nq, n_q_heads, max_parts,
                      part_rows, out, stream);
}

}  // namespace i8a
