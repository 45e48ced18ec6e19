// High-precision attention of a prefill chunk with no history, over its own bf16 rows.
//
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.1: the first prefill chunk has
// no KV history to read, so it keeps a high-precision attention while the fused producer
// writes its K/V as int8 for the later chunks and the decode; §3.2: from the point where
// a history exists the chunk runs the int8 path.)
//
// Workgroup = (32 query tokens, KV head g): 12 waves = the 6 query heads of the group x
// two 16-token halves, every K/V byte staged once in LDS for 192 query rows. Per 64-key
// block (double buffered; the next block's K and V move by direct global->LDS buffer loads
// while the current one is computed):
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 sums): tile t
//    holds keys 16t..16t+15 of the block; the query operands stay in registers, and the
//    K operands of the next 32-dim group are read while the current group's products run;
//  * online softmax in the exp2 domain with the lazy rescale (the reference max moves
//    only when a block max exceeds it by more than 2^8);
//  * out^T += V^T . P^T on v_mfma_f32_16x16x32_bf16 with P carried as two bf16 terms,
//    hi = bf16(p) and lo = bf16(p - hi) (16 significant bits; gfx950's packed fp32 -> bf16
//    conversion rounds two values to nearest even per instruction), and fp32 accumulation, so
//    the weighted sum keeps fp32-class precision. The 32 keys of one product are the 4
//    consecutive keys that each lane already holds from two tiles (key index 8 kg + j =
//    key 16(2h + j/4) + 4 kg + j%4), so P needs no lane movement; V is staged as key rows
//    by direct-to-LDS loads and read with gfx950's transposing LDS read (ds_read_b64_tr_b16),
//    two per operand, one dim tile ahead of the products;
//  * the row's weight sum on the matrix core as well: ones . P^T over the same hi and lo
//    terms, so the sum and the weighted values see the same weights.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace i8a {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kCbTok = 32;                  // query tokens per workgroup
constexpr int kCbWaves = 2 * kGroup;        // (head, 16-token half) per wave
constexpr int kCbThreads = kCbWaves * 64;   // 768
constexpr int kKBytes = 32 * 64 * 16;       // staged K block: [dim chunk of 8][key][8 dims]
constexpr int kVBytes = 64 * kHeadDim * 2;   // staged V block: [key][256 dims], swizzled
constexpr float kLazyRescale = 8.0f;

struct Block {
  int8_t* k;   // staged K block (kKBytes)
  int8_t* v;   // staged V block (kVBytes)
};

// Loads of key block kb by direct-to-LDS buffer loads (dword x4): K as instruction c =
// dim chunk c of 8 dims, lane = key; V as key rows, two keys per instruction. The
// block's address and bound are scalar: the resource starts at key 64 kb of head g and
// ends after the chunk's last key row, so the rows past the chunk read as zeros (their
// weights are 0). Each lane keeps one offset per operand.
struct Loader {
  const uint16_t* k;
  const uint16_t* v;
  int n, n_kv_heads, g, w;
  uint32_t rstride;  // bytes per key row (all KV heads)
  uint32_t k_vo;     // key = lane
  uint32_t v_vo;     // key 2i + half (the 2i rows go in the scalar offset), swizzled chunk

  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t* base, int kb) const {
    const char* p = reinterpret_cast<const char*>(base) +
                    ((size_t)kb * 64 * n_kv_heads + g) * (kHeadDim * 2);
    const uint32_t rows = (uint32_t)min(n - kb * 64, 64);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0,
                                             (int)((rows - 1) * rstride + kHeadDim * 2),
                                             0x00020000);
  }
  __device__ __forceinline__ void issue_k(int kb, int8_t* k_lds) const {
    const __amdgpu_buffer_rsrc_t r = rsrc(k, kb);
    for (int c = w; c < 32; c += kCbWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(k_lds + c * 1024), 16, k_vo, c * 16, 0, 0);
  }
  // V rows (512 B per key), instruction i = keys 2i, 2i+1. The 16-byte chunks of key row
  // r are stored XOR-ed with (r & 7) << 1: LDS chunk c of row r holds dims
  // 8 (c ^ ((r & 7) << 1)) .. +7, so the transposed reads of 16 rows at one dim range
  // spread over all banks. A wave's instructions i = w + 12 j all have r & 7 = (2w + half) & 7.
  __device__ __forceinline__ void issue_v(int kb, int8_t* v_lds) const {
    const __amdgpu_buffer_rsrc_t r = rsrc(v, kb);
    for (int i = w; i < 32; i += kCbWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(v_lds + i * 1024), 16, v_vo,
          2 * i * rstride, 0, 0);
  }
};

// l: the row's weight sum, formed on the matrix core as ones . P^T (every element of a
// lane's l holds the sum of its query row).
struct RowState {
  float m_run;
  v4f l;
  v4f acc[16];
};

// One 64-key block: QK, softmax, PV from the staged block `cur`; the loads of block kb+1
// into `nxt` go out first.
__device__ __forceinline__ void block_step(int kb, int nkb, const Loader& ld, const v8bf* qop,
                                           int my_tok, int first_tok, bool causal, int n,
                                           float qk_scale_log2,
                                           int gq, int nn, int vbase, RowState& st,
                                           Block cur, Block nxt) {
  const bool more = kb + 1 < nkb;
  if (more) {
    ld.issue_v(kb + 1, nxt.v);
    ld.issue_k(kb + 1, nxt.k);
  }
  // S^T tile t: rows = keys 16t..16t+15 (lane (m, kg) reads key 16t + m, dims 32u + 8kg..).
  // Dim group u feeds the 4 tiles' independent accumulations; the operands of group u + 1
  // are read while the products of group u run.
  v4f S[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) S[t] = v4f{0.f, 0.f, 0.f, 0.f};
  {
    const int8_t* kp = cur.k + gq * 1024 + nn * 16;
    v8bf ka[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ka[t] = *reinterpret_cast<const v8bf*>(kp + t * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v8bf kn[4];
      if (u < 7) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kn[t] = *reinterpret_cast<const v8bf*>(kp + (u + 1) * 4096 + t * 256);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) S[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t], qop[u], S[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (u < 7) {
#pragma unroll
        for (int t = 0; t < 4; ++t) ka[t] = kn[t];
      }
    }
  }
  // Lane (nn, gq) holds keys 64kb + 16t + 4gq + i of its query row. Only blocks that
  // reach past the chunk or past the workgroup's first row need the mask.
  const int key0 = kb * 64;
  float x[16];
  float bmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = S[e >> 2][e & 3];
  if (key0 + 64 > n || (causal && key0 + 63 > first_tok)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * t + 4 * gq + i;
        if (!(key < n && (!causal || key <= my_tok))) x[4 * t + i] = -INFINITY;
      }
  }
  // The scale c > 0 goes into the exponent's fma: max(c s) = c max(s), and a masked
  // s = -inf gives exp2(-inf) = 0.
#pragma unroll
  for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, x[e]);
  bmax = col_max(bmax) * qk_scale_log2;
  if (__any(bmax > st.m_run + kLazyRescale)) {
    const float m_new = fmaxf(st.m_run, bmax);
    const float alpha = m_new == st.m_run ? 1.0f : __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.acc[dt] *= alpha;
    st.l *= alpha;
    st.m_run = m_new;
  }
  const float nmu = st.m_run == -INFINITY ? 0.f : -st.m_run;
  // B operands of the two 32-key halves: h holds tiles 2h and 2h + 1 (elements 8h..8h+7).
  // hi = bf16(p) and lo = bf16(p - hi), both rounded to nearest even by the hardware
  // conversion (two values per instruction).
  uint4 ph[2], pl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(x[8 * h + 2 * j2], qk_scale_log2, nmu));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(x[8 * h + 2 * j2 + 1], qk_scale_log2, nmu));
      const bf2 hi = {(__bf16)p0, (__bf16)p1};
      hw[j2] = __builtin_bit_cast(uint32_t, hi);
      const bf2 lo = {(__bf16)(p0 - __uint_as_float(hw[j2] << 16)),
                      (__bf16)(p1 - __uint_as_float(hw[j2] & 0xffff0000u))};
      lw[j2] = __builtin_bit_cast(uint32_t, lo);
    }
    ph[h] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    pl[h] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  // out^T(dt) += V^T(dt) . P^T: lane (nn, gq) needs dim 16dt + nn of keys 32h + 4gq..+3
  // and 32h + 16 + 4gq..+3 (tiles 2h and 2h + 1). Two transposed 8-byte reads give them:
  // within each 16-lane group, lane s addresses 4 dims (16dt + 4(s & 3)..) of key row
  // 32h (+16) + 4gq + s/4, and lane nn receives element nn & 3 of lanes nn/4 + 4k.
  // The operands of dim tile dt + 1 are read while the 4 products of tile dt run.
  int vb = vbase;
  asm volatile("" : "+v"(vb));  // the 8 offsets vb ^ 32dt are formed here, not kept live
  auto vop = [&](int dt, int h) {
    const int8_t* p0 = cur.v + (vb ^ ((dt & 7) << 5)) + (dt >> 3) * 256 + 32 * h * 512;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p0 + 16 * 512));
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  v8bf va[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) va[h] = vop(0, h);
  {
    const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(v8bf, ph[h]), st.l, 0, 0, 0);
      st.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(v8bf, pl[h]), st.l, 0, 0, 0);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    v8bf vn[2];
    if (dt < 15) {
#pragma unroll
      for (int h = 0; h < 2; ++h) vn[h] = vop(dt + 1, h);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[h], __builtin_bit_cast(v8bf, ph[h]),
                                                           st.acc[dt], 0, 0, 0);
      st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[h], __builtin_bit_cast(v8bf, pl[h]),
                                                           st.acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (dt < 15) {
#pragma unroll
      for (int h = 0; h < 2; ++h) va[h] = vn[h];
    }
  }
  if (more) __builtin_amdgcn_s_waitcnt(0);  // the next K/V block has landed in LDS
  lds_barrier();
}

// Key partitions of a causal chunk (SPLIT): partition p holds the 64-key blocks
// [p * part_blocks, (p + 1) * part_blocks). The boundary part_blocks * 64 = row0 is a
// multiple of 64, so a 32-token tile lies wholly below it (its rows see one partition and
// it writes its outputs) or wholly at or above it (every row sees at least two partitions:
// the tile writes partial states for rows row0.., which the merge kernel combines).
struct ChunkSplit {
  float* ws_o;  // [row - row0][head][partition][256] unnormalised outputs
  float* ws_m;  // running max (exp2 domain)
  float* ws_l;  // sum of the weights
  int part_blocks, n_parts, row0;
};

template <int SPLIT>
__global__ __launch_bounds__(kCbThreads, 1) void chunk_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int n, int causal, int n_q_heads, int n_kv_heads,
    float qk_scale_log2, float* __restrict__ out, int n_qb, int xcd_per_head, ChunkSplit sp) {
  int qb, g, part = 0;
  if (SPLIT) {
    // grid x = (query tile, KV head), the tiles with the most keys first and the heads
    // interleaved; grid y = the partition (partitions past a tile's keys exit at once).
    const int x = blockIdx.x;
    g = x % n_kv_heads;
    qb = n_qb - 1 - x / n_kv_heads;
    part = blockIdx.y;
  } else {  // XCD-aware order as in the int8 chunk kernel: each KV head on its own XCDs
    const int L = blockIdx.x, xcd = L % 8, slot = L / 8;
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
  const int hl = w >> 1, half = w & 1;
  const int h = g * kGroup + hl;
  const int nn = lane & 15, gq = lane >> 4;
  const int t0 = qb * kCbTok;
  const int my_tok = t0 + 16 * half + nn;
  const int last_tok = min(t0 + kCbTok, n) - 1;
  const int kend = causal ? last_tok + 1 : n;
  // 64-key blocks [kb0, nkb) of this workgroup
  const int nkb_tile = (kend + 63) >> 6;
  const int kb0 = SPLIT ? part * sp.part_blocks : 0;
  const int nkb = SPLIT ? min(nkb_tile, kb0 + sp.part_blocks) : nkb_tile;
  if (SPLIT && kb0 >= nkb) return;  // the tile's keys end before this partition

  // Four distinct LDS variables, so that the compiler can tell the in-flight direct-to-LDS
  // writes of one buffer from the reads of the other and need not wait for them. The V
  // buffers carry the names that sort first: the compiler lays the kernel's LDS variables
  // out in name order, which puts them in the low 64 KB, where every transposed V read
  // reaches its buffer through the instruction's 16-bit offset field (an add per read
  // otherwise).
  __shared__ __align__(16) int8_t sv0[kVBytes];
  __shared__ __align__(16) int8_t sv1[kVBytes];
  __shared__ __align__(16) int8_t s_k0[kKBytes];
  __shared__ __align__(16) int8_t s_k1[kKBytes];

  const uint32_t rstride = (uint32_t)n_kv_heads * (kHeadDim * 2);
  const int vh = lane >> 5;
  const Loader ld{k, v, n, n_kv_heads, g, w, rstride, (uint32_t)lane * rstride,
                  vh * rstride + 16 * ((lane & 31) ^ (((2 * w + vh) & 7) << 1))};
  {
    ld.issue_v(kb0, sv0);
    ld.issue_k(kb0, s_k0);
    // Query operands: lane (nn, gq) holds dims 32u + 8gq..+7 of its row (rows past the
    // chunk re-read the last one; their outputs are not stored).
    v8bf qop[8];
    const size_t qrow = ((size_t)min(my_tok, n - 1) * n_q_heads + h) * kHeadDim;
#pragma unroll
    for (int u = 0; u < 8; ++u) qop[u] = *reinterpret_cast<const v8bf*>(q + qrow + 32 * u + 8 * gq);
    // Byte offset of this lane's transposed V reads for dim tile dt (0..7; tiles 8..15
    // add 256): key row r = 4gq + nn/4 (+32h, +16 as immediates), dims 16dt + 4(nn & 3),
    // 16-byte chunk 2dt + (nn & 3)/2 stored at chunk (2dt + (nn & 3)/2) ^ 2(r & 7), i.e.
    // vbase ^ 32dt with vbase the offset for dt = 0.
    const int vbase = [&] {
      const int r = 4 * gq + (nn >> 2);
      return r * 512 + (r & 7) * 32 + ((nn & 3) >> 1) * 16 + (nn & 1) * 8;
    }();
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();

    RowState st;
    st.m_run = -INFINITY;
    st.l = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    const Block b0{s_k0, sv0}, b1{s_k1, sv1};
    for (int kb = kb0; kb < nkb; kb += 2) {
      block_step(kb, nkb, ld, qop, my_tok, t0, causal != 0, n, qk_scale_log2, gq, nn, vbase, st,
                 b0, b1);
      if (kb + 1 < nkb)
        block_step(kb + 1, nkb, ld, qop, my_tok, t0, causal != 0, n, qk_scale_log2, gq, nn, vbase,
                   st, b1, b0);
    }
    const float l = st.l[0];
    if (SPLIT && nkb_tile > sp.part_blocks) {  // a tile at or above row0: partial state
      if (my_tok < n) {
        const size_t pi = ((size_t)(my_tok - sp.row0) * n_q_heads + h) * sp.n_parts + part;
        float* o = sp.ws_o + pi * kHeadDim + 4 * gq;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
          *reinterpret_cast<float4*>(o + 16 * dt) =
              make_float4(st.acc[dt][0], st.acc[dt][1], st.acc[dt][2], st.acc[dt][3]);
        if (gq == 0) {
          sp.ws_m[pi] = st.m_run;
          sp.ws_l[pi] = l;
        }
      }
    } else if (my_tok < n) {
      const float il = 1.0f / l;
      float* o = out + ((size_t)my_tok * n_q_heads + h) * kHeadDim + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        *reinterpret_cast<float4*>(o + 16 * dt) =
            make_float4(st.acc[dt][0] * il, st.acc[dt][1] * il, st.acc[dt][2] * il, st.acc[dt][3] * il);
    }
  }
}

}  // namespace

// Partitions for a causal chunk: part_blocks = 1.2 x the 64-key blocks of all (tile, KV
// head) pairs spread over the 256 CUs (at least 4); 1 (the one pass) when no tile reaches
// past one partition. Every row past the first partition costs two partial states written
// and a merge that reads them, so partitions somewhat above the average win: on 2,048
// rows (24 / 4 heads), 17 blocks (the average) took 0.112 ms, 20 blocks 0.103 ms, 24
// blocks 0.111 ms, the one pass 0.127 ms.
int chunk_bf16_split_parts(int n, int causal, int n_kv_heads, int* part_blocks) {
  const long long n_qb = (n + kCbTok - 1) / kCbTok;
  const int nkb_max = (int)(((long long)n + 63) / 64);
  *part_blocks = nkb_max;
  if (!causal || n <= 0) return 1;
  long long total = 0;  // sum over tiles of their 64-key blocks, per KV head
  for (long long t = 0; t < n_qb; ++t) total += (std::min<long long>(t * kCbTok + kCbTok, n) + 63) / 64;
  const long long per_cu = (total * n_kv_heads + 255) / 256;
  const int pb = (int)std::max<long long>(4, per_cu * 6 / 5);
  if (pb >= nkb_max) return 1;
  *part_blocks = pb;
  return (nkb_max + pb - 1) / pb;
}

size_t chunk_bf16_ws_bytes(int n, int causal, int n_q_heads, int n_kv_heads) {
  int pb;
  const int parts = chunk_bf16_split_parts(n, causal, n_kv_heads, &pb);
  if (parts <= 1) return 0;
  const size_t np = (size_t)(n - pb * 64) * n_q_heads * parts;
  return ((np * kHeadDim + 2 * np) * sizeof(float) + 255) / 256 * 256;
}

int launch_chunk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int causal,
                      int n_q_heads, int n_kv_heads, float sm_scale, float* out, float* ws,
                      hipStream_t stream) {
  const int n_qb = (n + kCbTok - 1) / kCbTok;
  // The kernels need a scale > 0 (it multiplies the block max); sm_scale = 0 runs as 1e-30,
  // which gives the same uniform weights in fp32.
  ChunkSplit sp{nullptr, nullptr, nullptr, 0, 1, 0};
  const int n_parts = ws != nullptr ? chunk_bf16_split_parts(n, causal, n_kv_heads, &sp.part_blocks) : 1;
  if (n_parts > 1) {
    sp.n_parts = n_parts;
    sp.row0 = sp.part_blocks * 64;
    const size_t np = (size_t)(n - sp.row0) * n_q_heads * n_parts;
    sp.ws_o = ws;
    sp.ws_m = ws + np * kHeadDim;
    sp.ws_l = sp.ws_m + np;
    hipLaunchKernelGGL(chunk_bf16_kernel<1>, dim3((unsigned)(n_qb * n_kv_heads), (unsigned)n_parts),
                       dim3(kCbThreads), 0, stream, q, k, v, n, causal, n_q_heads, n_kv_heads,
                       fmaxf(sm_scale * kLog2e, 1e-30f), out, n_qb, 0, sp);
    int rc = check_launch("attn_chunk_bf16");
    if (rc) return rc;
    // rows row0.. : n - row0 rows at the tail of an n-key sequence (row t sees t + 1 keys)
    return launch_merge_rows(sp.ws_m, sp.ws_l, sp.ws_o, n, n - sp.row0, n_q_heads, n_parts,
                             sp.row0, out + (size_t)sp.row0 * n_q_heads * kHeadDim, stream);
  }
  const int xcd_per_head = (n_kv_heads <= 8 && 8 % n_kv_heads == 0) ? 8 / n_kv_heads : 0;
  const long long n_wg = xcd_per_head > 0 ? 8LL * ((n_qb + xcd_per_head - 1) / xcd_per_head)
                                          : (long long)n_qb * n_kv_heads;
  hipLaunchKernelGGL(chunk_bf16_kernel<0>, dim3((unsigned)n_wg), dim3(kCbThreads), 0, stream, q, k,
                     v, n, causal, n_q_heads, n_kv_heads, fmaxf(sm_scale * kLog2e, 1e-30f), out, n_qb,
                     xcd_per_head, sp);
  return check_launch("attn_chunk_bf16");
}

}  // namespace i8a
