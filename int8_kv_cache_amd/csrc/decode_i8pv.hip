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
  const int32_t* trow = block_table + (size_t)s * max_blocks;
  const int blk0 = j * (kKeys / kPage) + 4 * w;
  int pr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pr[t] = trow[min(blk0 + t, max_blocks - 1)];
  int ctx = ctx_lens != nullptr ? ctx_lens[s] : ctx_cap;  // (null: one sequence of ctx_cap)
  asm volatile("" ::"s"(ctx), "s"(pr[0]), "s"(pr[1]), "s"(pr[2]), "s"(pr[3]));
  ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
  const int tok0 = j * kKeys;
  const int n_rows = kGroup * nq;
  if (tok0 >= ctx) {  // whole workgroup: this partition is past the context
    if (out != nullptr)  // no key at all: zeros
      for (int r = 0; r < n_rows; ++r) {
        const int qi = r / kGroup;
        float* o = out + (((size_t)s * nq + qi) * n_q_heads + g * kGroup + (r - kGroup * qi)) * kHeadDim;
        for (int i = tid; i < kHeadDim; i += WAVES * 64) o[i] = 0.f;
      }
    return;
  }
  const int n_tok = min(kKeys, ctx - tok0);
  const int n_tiles = (n_rows + kRowTile - 1) / kRowTile;

  __shared__ __align__(16) int8_t s_q[kMaxQRows][kHeadDim];
  __shared__ float s_qs[kMaxQRows];
  __shared__ __align__(16) float s_ks[kKeys];
  __shared__ __align__(16) float s_vs[kKeys];
  __shared__ float s_f[WAVES];                               // the wave's max V scale
  __shared__ float s_m[WAVES][kRowTile], s_l[WAVES][kRowTile], s_c[WAVES][kRowTile];
  // Rows padded by 16 bytes: the 16 rows a wave writes at one dim range fall on
  // different banks.
  __shared__ __align__(16) float s_o[WAVES][kRowTile][kHeadDim + 4];

  const int wtok0 = w * 64;
  const int nvalid = min(64, n_tok - wtok0);  // tokens of the block inside the context
  int pg[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    pg[t] = (16 * t < nvalid && pr[t] >= 0 && pr[t] < num_pages) ? pr[t] : 0;
  // This wave quantizes query rows w, w + WAVES, ... (my_rows of them).
  const int my_rows = n_rows > w ? (n_rows - w + WAVES - 1) / WAVES : 0;
  uint2 qw[kRowsPerWave];
  float qsc[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    if (k < my_rows) {
      const int r = w + WAVES * k;
      const int qi = r / kGroup;
      const size_t row = ((size_t)s * nq + qi) * n_q_heads + g * kGroup + (r - kGroup * qi);
      if (Q8) {
        qw[k].x = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(q) + row * kHeadDim + lane * 4);
        qsc[k] = q_scales[row];
      } else {
        qw[k] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + row * kHeadDim + lane * 4);
      }
    }
  }
  const int pl = (lane >> 4) == 0 ? pg[0] : (lane >> 4) == 1 ? pg[1] : (lane >> 4) == 2 ? pg[2] : pg[3];
  const size_t si = ((size_t)pl * n_kv_heads + g) * kPage + (lane & 15);
  const float sk_l = k_scale[si];
  const float sv_l = v_scale[si];
  // K and V of page t: four 1 KB wave loads each (lane l reads bytes 16 l of each KB).
  uint4 kA[4][4];
  uint4 vA[4][4];
  auto issue_page = [&](int t) {
    const size_t blk = ((size_t)pg[t] * n_kv_heads + g) * kBlockBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kA[t][u] = *reinterpret_cast<const uint4*>(k_cache + blk + lane * 16 + u * 1024);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vA[t][u] = *reinterpret_cast<const uint4*>(v_cache + blk + lane * 16 + u * 1024);
  };
  __builtin_amdgcn_sched_barrier(0);
  issue_page(0);
  issue_page(1);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    if (k < my_rows) {
      const int r = w + WAVES * k;
      float sc = qsc[k];
      const uint32_t c = Q8 ? qw[k].x
                            : quantize4(bf16_to_f32(qw[k].x & 0xffffu), bf16_to_f32(qw[k].x >> 16),
                                        bf16_to_f32(qw[k].y & 0xffffu), bf16_to_f32(qw[k].y >> 16), &sc);
      *reinterpret_cast<uint32_t*>(&s_q[r][lane * 4]) = c;
      if (lane == 0) s_qs[r] = sc;
    }
  }
  // Token scales, lane = token wtok0 + lane; the V scale in units of the wave's largest
  // one, tokens past the context 0.
  {
    const float sv = lane < nvalid ? sv_l : 0.f;
    const float svm = wave_max(sv);
    const float inv = svm > 0.f ? 1.0f / svm : 0.f;
    s_ks[wtok0 + lane] = sk_l;
    s_vs[wtok0 + lane] = sv == svm ? (svm > 0.f ? 1.0f : 0.f) : sv * inv;
    if (lane == 0) s_f[w] = svm;
  }
  lds_barrier();

  const int n = lane & 15, gq = lane >> 4;
  for (int c = 0; c < n_tiles; ++c) {
    if (nvalid > 0) {
      if (c == 0) {
        __builtin_amdgcn_sched_barrier(0);
        issue_page(2);
        issue_page(3);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int r = c * kRowTile + n;
      const bool on = r < n_rows;
      const int rq = on ? r : 0;
      const int qi = rq / kGroup;
      // Tokens of this block that the column's query row sees: index e (0..63) < lim.
      const int lim = on ? ctx - nq + qi + 1 - tok0 - wtok0 : 0;
      const int8_t* qcol = &s_q[rq][gq * 16];
      const float rs = s_qs[rq] * qk_scale_log2;
      v4i S[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        S[t] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          S[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, kA[t][u]),
                                                       *reinterpret_cast<const v4i*>(qcol + u * 64),
                                                       S[t], 0, 0, 0);
      }
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 kk = *reinterpret_cast<const float4*>(&s_ks[wtok0 + 16 * t + 4 * gq]);
        const float kks[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[4 * t + i] = 16 * t + 4 * gq + i < lim ? (float)S[t][i] * kks[i] * rs : -INFINITY;
          bm = fmaxf(bm, x[4 * t + i]);
        }
      }
      bm = col_max(bm);
      const float mu = bm == -INFINITY ? 0.f : bm;  // a row with no visible key: weights 0
      float lsum = 0.f, wm = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 rv = *reinterpret_cast<const float4*>(&s_vs[wtok0 + 16 * t + 4 * gq]);
        const float rvs[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(x[4 * t + i] - mu);
          lsum += p;
          x[4 * t + i] = p * rvs[i];
          wm = fmaxf(wm, x[4 * t + i]);
        }
      }
      const float l = col_sum(lsum);
      wm = col_max(wm);
      if (c == 0) {
        // Lane (n, gq) loaded dim 16(4u + gq) + n of each page (all 16 tokens); after a
        // 4x4 dword transpose over {n, n+16, n+32, n+48} it holds tokens 4gq..4gq+3 of
        // dim 16(4u + e) + n in dword e.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            uint32_t r0 = vA[t][u].x, r1 = vA[t][u].y, r2 = vA[t][u].z, r3 = vA[t][u].w;
            auto pp = __builtin_amdgcn_permlane32_swap(r0, r2, false, false); r0 = pp[0]; r2 = pp[1];
            pp = __builtin_amdgcn_permlane32_swap(r1, r3, false, false); r1 = pp[0]; r3 = pp[1];
            pp = __builtin_amdgcn_permlane16_swap(r0, r1, false, false); r0 = pp[0]; r1 = pp[1];
            pp = __builtin_amdgcn_permlane16_swap(r2, r3, false, false); r2 = pp[0]; r3 = pp[1];
            vA[t][u] = make_uint4(r0, r1, r2, r3);
          }
      }
      // 127 / wm via the hardware reciprocal (about 1 ulp), as in the prefill kernel.
      const float inv = wm > 0.f ? 127.0f * __builtin_amdgcn_rcpf(wm) : 0.f;
      const float sb = wm * (1.0f / 127.0f);
      float4* dst = reinterpret_cast<float4*>(&s_o[w][n][4 * gq]);
      auto vop = [&](int dt) {  // A operand of dim tile dt: one dword per page
        const int u = dt >> 2, e = dt & 3;
        auto pick = [&](const uint4& v) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; };
        return v4i{(int)pick(vA[0][u]), (int)pick(vA[1][u]), (int)pick(vA[2][u]), (int)pick(vA[3][u])};
      };
      const v4i kMag = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
      if constexpr (DIG == 1) {
        v4i P;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t d = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_cvt_pk_u8_f32(x[4 * t + i] * inv, i, d);
          P[t] = (int)d;
        }
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          const v4i X = __builtin_amdgcn_mfma_i32_16x16x64_i8(vop(dt), P, kMag, 0, 0, 0);
          dst[dt * 4] = make_float4(__int_as_float(X[0]), __int_as_float(X[1]),
                                    __int_as_float(X[2]), __int_as_float(X[3]));
        }
      } else {
        // U = rint(2^14 * w / s_b) < 2^21 sits in the low bits of fl(w * sc + 1.5 * 2^23).
        const float sc = inv * 16384.0f;
        v4i P0, P1, P2;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t F[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) F[i] = __float_as_uint(fmaf(x[4 * t + i], sc, kMagicF));
          P2[t] = (int)(pack_byte(F[0], F[1], F[2], F[3]) & 0x7f7f7f7fu);
          P1[t] = (int)(pack_byte(F[0] >> 7, F[1] >> 7, F[2] >> 7, F[3] >> 7) & 0x7f7f7f7fu);
          P0[t] = (int)pack_byte(F[0] >> 14, F[1] >> 14, F[2] >> 14, F[3] >> 14);
        }
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          const v4i A = vop(dt);
          const v4i X0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, P0, v4i{0, 0, 0, 0}, 0, 0, 0);
          const v4i Z = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, P1, X0 << 7, 0, 0, 0);
          const v4i X2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, P2, kMag, 0, 0, 0);
          float4 o;
          o.x = fmaf(__int_as_float(X2[0]), 1.0f / 128.0f, (float)Z[0]);
          o.y = fmaf(__int_as_float(X2[1]), 1.0f / 128.0f, (float)Z[1]);
          o.z = fmaf(__int_as_float(X2[2]), 1.0f / 128.0f, (float)Z[2]);
          o.w = fmaf(__int_as_float(X2[3]), 1.0f / 128.0f, (float)Z[3]);
          dst[dt * 4] = o;
        }
      }
      if (gq == 0) {
        s_m[w][n] = bm;
        s_l[w][n] = l;
        s_c[w][n] = DIG == 1 ? sb : sb * (1.0f / 128.0f);
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRowTile; ++r)
        reinterpret_cast<float4*>(&s_o[w][r][0])[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (lane < kRowTile) {
        s_m[w][lane] = -INFINITY;
        s_l[w][lane] = 0.f;
        s_c[w][lane] = 0.f;
      }
    }
    lds_barrier();
    // Merge the wave states of the tile: wave w takes rows w, w + WAVES, ...; lane l
    // dims 4l..4l+3.
    for (int rr = w; rr < kRowTile; rr += WAVES) {
      const int row = c * kRowTile + rr;
      if (row >= n_rows) break;
      float mw[WAVES];
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        mw[ww] = s_m[ww][rr];
        M = fmaxf(M, mw[ww]);
      }
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M > -INFINITY) {  // else no key of the partition is visible to this row
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) {
          const float a = __builtin_amdgcn_exp2f(mw[ww] - M);
          L += a * s_l[ww][rr];
          const float f = a * s_f[ww] * s_c[ww][rr];
          const float4 ov = *reinterpret_cast<const float4*>(&s_o[ww][rr][4 * lane]);
          acc.x = fmaf(f, ov.x - kOffset, acc.x);
          acc.y = fmaf(f, ov.y - kOffset, acc.y);
          acc.z = fmaf(f, ov.z - kOffset, acc.z);
          acc.w = fmaf(f, ov.w - kOffset, acc.w);
        }
      }
      const int qi = row / kGroup;
      const size_t hrow = ((size_t)s * nq + qi) * n_q_heads + g * kGroup + (row - kGroup * qi);
      if (out != nullptr) {
        *reinterpret_cast<float4*>(&out[hrow * kHeadDim + 4 * lane]) =
            M > -INFINITY ? make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        continue;
      }
      const size_t pi = hrow * max_parts + j;
      *reinterpret_cast<float4*>(&ws_o[pi * kHeadDim + 4 * lane]) = acc;
      if (lane == 0) {
        ws_m[pi] = M;
        ws_l[pi] = L;
      }
    }
    lds_barrier();  // the next tile rewrites the wave states
  }
}

template <int DIG, int WAVES>
int launch_split(const void* q, const float* q_scales, int nq, const int8_t* k_cache, const int8_t* v_cache,
                 const float* k_scale, const float* v_scale, const int32_t* block_table,
                 int max_blocks, const int32_t* ctx_lens, int ctx_cap, int num_seqs,
                 int num_pages, int n_q_heads, int n_kv_heads, float qk_scale_log2, float* ws_m,
                 float* ws_l, float* ws_o, int max_parts, float* out, hipStream_t stream) {
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
