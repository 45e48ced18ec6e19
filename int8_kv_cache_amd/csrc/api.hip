// extern "C" entry points: argument validation, workspace sizing, launch, error codes.
// Nothing here allocates device memory or synchronizes; every check happens before
// anything is enqueued, so an error leaves every output untouched. (The opt-in metadata
// checks at the end work on host arrays and use host memory only.)
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>
#include <vector>

#include "int8attn.h"
#include "launch.hpp"

namespace i8a {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(I8A_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return I8A_OK;
}

// The softmax scale must be finite and not negative: the chunk kernel bounds its running
// max through the scale's sign, so a negative scale is refused on every route alike.
static int check_sm_scale(const char* who, float sm_scale) {
  if (!isfinite(sm_scale) || sm_scale < 0.0f)
    return set_error(I8A_EINVAL, "%s: sm_scale %g (must be finite and >= 0)", who, (double)sm_scale);
  return I8A_OK;
}

static int check_heads(int n_q_heads, int n_kv_heads, int head_dim) {
  if (n_q_heads <= 0 || n_kv_heads <= 0) return set_error(I8A_EINVAL, "head counts must be > 0");
  // The merge kernels put the query heads on grid.y (at most 65535).
  if (n_q_heads > 65535) return set_error(I8A_EINVAL, "n_q_heads %d > 65535", n_q_heads);
  if (head_dim != 256) return set_error(I8A_EUNSUPPORTED, "head_dim %d unsupported (v1: 256)", head_dim);
  if (n_kv_heads > 65535 / 6 || n_q_heads != 6 * n_kv_heads)
    return set_error(I8A_EUNSUPPORTED, "n_q_heads %d / n_kv_heads %d: v1 supports GQA groups of 6",
                     n_q_heads, n_kv_heads);
  return I8A_OK;
}

static size_t decode_ws_bytes(long long num_seqs, long long max_ctx, long long n_q_heads) {
  const long long parts = (max_ctx + 511) / 512;
  const long long floats = num_seqs * n_q_heads * parts * (2 + 256);
  return (size_t)((floats * 4 + 255) / 256 * 256);
}

// Keys per split-K partition of the int8-PV decode when the caller passes 0. The vLLM
// docs page's selection law picks a power-of-two segment count from a workgroup-count
// target over (KV heads x rows) with a floor on keys per segment; in this kernel every
// wave owns one 64-key block whatever the partition size, so smaller partitions add
// partials (merge work) without adding waves, and only help by spreading a short grid
// over more CUs. Hence: a context that fits one partition takes 512 keys (one
// partition, no merge stage); otherwise halve from 512 while sequences x KV heads x
// partitions stays under 64 workgroups, down to 128 keys.
static int partition_law(long long num_seqs, long long max_ctx, long long n_kv_heads) {
  constexpr long long kTargetWorkgroups = 64;
  if (max_ctx <= 512) return 512;
  int p = 512;
  while (p > 128 && num_seqs * n_kv_heads * ((max_ctx + p - 1) / p) < kTargetWorkgroups) p >>= 1;
  return p;
}

static size_t partials_bytes(long long rows, long long max_ctx, long long n_q_heads, int part) {
  const long long parts = (max_ctx + part - 1) / part;
  const long long floats = rows * n_q_heads * parts * (2 + 256);
  return (size_t)((floats * 4 + 255) / 256 * 256);
}

}  // namespace i8a

using namespace i8a;

extern "C" {

const char* int8attn_last_error(void) { return g_last_error.c_str(); }

int int8attn_version(void) { return (1 << 16) | 0; }

int kv_quant_write(const void* k, const void* v, int in_dtype, int n_tokens, int n_kv_heads,
                   int head_dim, const int32_t* slot_mapping, int8_t* k_cache, int8_t* v_cache,
                   float* k_scale, float* v_scale, int num_pages, void* stream) {
  if (in_dtype != I8A_DTYPE_F32 && in_dtype != I8A_DTYPE_BF16)
    return set_error(I8A_EINVAL, "kv_quant_write: in_dtype %d", in_dtype);
  if (n_tokens < 0 || n_kv_heads <= 0 || num_pages <= 0)
    return set_error(I8A_EINVAL, "kv_quant_write: n_tokens %d, n_kv_heads %d, num_pages %d",
                     n_tokens, n_kv_heads, num_pages);
  if (head_dim != 256)
    return set_error(I8A_EUNSUPPORTED, "kv_quant_write: head_dim %d unsupported (v1: 256)", head_dim);
  if ((long long)n_tokens * n_kv_heads > 2147483000LL)
    return set_error(I8A_EINVAL, "kv_quant_write: too many rows");
  if (n_tokens == 0) return I8A_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return set_error(I8A_EINVAL, "kv_quant_write: null pointer");
  return launch_kv_quant_write(k, v, in_dtype == I8A_DTYPE_BF16, n_tokens, n_kv_heads,
                               slot_mapping, k_cache, v_cache, k_scale, v_scale, num_pages,
                               (hipStream_t)stream);
}

int kv_produce(const void* q, const void* k, const void* v, int in_dtype, int n_tokens,
               int n_q_heads, int n_kv_heads, int head_dim, const int32_t* positions,
               const float* cos_sin, int rotary_dim, int max_position,
               const int32_t* slot_mapping, int8_t* k_cache, int8_t* v_cache, float* k_scale,
               float* v_scale, int num_pages, int8_t* q_codes, float* q_scales, uint16_t* q_rot,
               uint16_t* k_rot, void* stream) {
  if (in_dtype != I8A_DTYPE_F32 && in_dtype != I8A_DTYPE_BF16)
    return set_error(I8A_EINVAL, "kv_produce: in_dtype %d", in_dtype);
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (n_tokens < 0 || num_pages <= 0 || (long long)n_tokens * n_q_heads > 2147483000LL)
    return set_error(I8A_EINVAL, "kv_produce: n_tokens %d, num_pages %d", n_tokens, num_pages);
  if (rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 8 != 0)
    return set_error(I8A_EINVAL, "kv_produce: rotary_dim %d (0..256, a multiple of 8)", rotary_dim);
  if (rotary_dim > 0 && (max_position <= 0 || !cos_sin || !positions))
    return set_error(I8A_EINVAL, "kv_produce: RoPE needs positions, cos_sin and max_position > 0");
  if ((q_codes == nullptr) != (q_scales == nullptr) ||
      ((q_codes != nullptr || q_rot != nullptr) != (q != nullptr)))
    return set_error(I8A_EINVAL, "kv_produce: q goes with q_codes + q_scales and/or q_rot");
  if (n_tokens == 0) return I8A_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return set_error(I8A_EINVAL, "kv_produce: null pointer");
  if (rotary_dim > 0 && ((uintptr_t)cos_sin & 15u) != 0)
    return set_error(I8A_EINVAL, "kv_produce: cos_sin not 16-byte aligned");
  return launch_kv_produce(q, k, v, in_dtype == I8A_DTYPE_BF16, n_tokens, n_q_heads, n_kv_heads,
                           positions, cos_sin, rotary_dim, max_position > 0 ? max_position : 1,
                           slot_mapping, k_cache, v_cache, k_scale, v_scale, num_pages, q_codes,
                           q_scales, q_rot, k_rot, (hipStream_t)stream);
}

size_t attn_chunk_bf16_workspace_bytes(int n, int causal, int n_q_heads, int n_kv_heads,
                                       int head_dim) {
  if (n <= 0 || (causal != 0 && causal != 1) || head_dim != 256 || n_kv_heads <= 0 ||
      n_kv_heads > 65535 / 6 || n_q_heads != 6 * n_kv_heads || (long long)n * n_q_heads > 2147483000LL)
    return 0;
  return chunk_bf16_ws_bytes(n, causal, n_q_heads, n_kv_heads);
}

int attn_chunk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int causal,
                    int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (n < 0 || (causal != 0 && causal != 1) || (long long)n * n_q_heads > 2147483000LL)
    return set_error(I8A_EINVAL, "attn_chunk_bf16: n %d, causal %d", n, causal);
  if ((rc = check_sm_scale("attn_chunk_bf16", sm_scale))) return rc;
  size_t need = 0;
  if (workspace != nullptr) {
    if (((uintptr_t)workspace & 15u) != 0)
      return set_error(I8A_EINVAL, "attn_chunk_bf16: workspace not 16-byte aligned");
    need = n > 0 ? chunk_bf16_ws_bytes(n, causal, n_q_heads, n_kv_heads) : 0;
    if (workspace_bytes < need)
      return set_error(I8A_EWORKSPACE, "attn_chunk_bf16: workspace %zu bytes < %zu needed",
                       workspace_bytes, need);
  }
  if (n == 0) return I8A_OK;
  if (!q || !k || !v || !out) return set_error(I8A_EINVAL, "attn_chunk_bf16: null pointer");
  return launch_chunk_bf16(q, k, v, n, causal, n_q_heads, n_kv_heads, sm_scale, out,
                           need > 0 ? static_cast<float*>(workspace) : nullptr,
                           (hipStream_t)stream);
}

// The int8 route's Q codes and scales, rounded up to 256 bytes; its split-route scratch
// follows them.
static size_t step_q8_bytes(int n_new, int n_q_heads) {
  return ((size_t)n_new * n_q_heads * (256 + 4) + 255) / 256 * 256;
}

size_t prefill_step_workspace_bytes(int n_new, int context_len, int n_q_heads, int n_kv_heads,
                                    int head_dim) {
  if (n_new <= 0 || context_len < n_new || context_len > 2147483000 - 64 || n_q_heads <= 0 ||
      n_kv_heads <= 0 || n_kv_heads > 65535 / 6 || head_dim != 256 || n_q_heads != 6 * n_kv_heads)
    return 0;
  if (context_len == n_new) {  // bf16 route: the rotated Q and K rows, then the split scratch
    const size_t rot = (size_t)n_new * (n_q_heads + n_kv_heads) * head_dim * 2;
    return (rot + 255) / 256 * 256 +
           attn_chunk_bf16_workspace_bytes(n_new, 1, n_q_heads, n_kv_heads, head_dim);
  }
  return step_q8_bytes(n_new, n_q_heads) +
         attn_prefill_chunk_split_workspace_bytes(n_new, context_len, 1, n_q_heads, n_kv_heads,
                                                  head_dim);
}

int prefill_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n_new,
                 const int32_t* positions, const float* cos_sin, int rotary_dim, int max_position,
                 const int32_t* slot_mapping, int8_t* k_cache, int8_t* v_cache, float* k_scale,
                 float* v_scale, int num_pages, const int32_t* block_table, int context_len,
                 int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (n_new < 0 || context_len < n_new || context_len < 1)
    return set_error(I8A_EINVAL, "prefill_step: n_new %d, context_len %d", n_new, context_len);
  // (checked before the producer runs, so that a refused call enqueues nothing)
  if ((rc = check_sm_scale("prefill_step", sm_scale))) return rc;
  if (n_new == 0) return I8A_OK;
  if (!out || (context_len > n_new && !block_table))
    return set_error(I8A_EINVAL, "prefill_step: null out or block_table");
  if ((long long)num_pages * n_kv_heads * 16 >= (1ll << 32))
    return set_error(I8A_EUNSUPPORTED, "prefill_step: num_pages %d x %d heads exceeds the scale index range",
                     num_pages, n_kv_heads);
  if (!workspace || ((uintptr_t)workspace & 255u) != 0)
    return set_error(I8A_EINVAL, "prefill_step: workspace null or not 256-byte aligned");
  const size_t need = prefill_step_workspace_bytes(n_new, context_len, n_q_heads, n_kv_heads, head_dim);
  if (workspace_bytes < need)
    return set_error(I8A_EWORKSPACE, "prefill_step: workspace %zu bytes < %zu needed", workspace_bytes, need);
  char* ws = static_cast<char*>(workspace);
  if (context_len == n_new) {
    // No history: high-precision attention over the chunk's rotated bf16 rows; the
    // producer still writes the int8 K/V for the later chunks and the decode.
    uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws);
    uint16_t* k_rot = q_rot + (size_t)n_new * n_q_heads * head_dim;
    rc = kv_produce(q, k, v, I8A_DTYPE_BF16, n_new, n_q_heads, n_kv_heads, head_dim, positions,
                    cos_sin, rotary_dim, max_position, slot_mapping, k_cache, v_cache, k_scale,
                    v_scale, num_pages, nullptr, nullptr, q_rot, k_rot, stream);
    if (rc) return rc;
    const size_t rot = ((size_t)n_new * (n_q_heads + n_kv_heads) * head_dim * 2 + 255) / 256 * 256;
    return attn_chunk_bf16(q_rot, k_rot, v, n_new, 1, n_q_heads, n_kv_heads, head_dim, sm_scale,
                           out, ws + rot, workspace_bytes - rot, stream);
  }
  // A history exists (in the int8 cache only): the int8 chunk path with the producer's Q,
  // split over key partitions when the chunk is short.
  int8_t* q_codes = reinterpret_cast<int8_t*>(ws);
  float* q_scales = reinterpret_cast<float*>(ws + (size_t)n_new * n_q_heads * head_dim);
  rc = kv_produce(q, k, v, I8A_DTYPE_BF16, n_new, n_q_heads, n_kv_heads, head_dim, positions,
                  cos_sin, rotary_dim, max_position, slot_mapping, k_cache, v_cache, k_scale,
                  v_scale, num_pages, q_codes, q_scales, nullptr, nullptr, stream);
  if (rc) return rc;
  const size_t q8 = step_q8_bytes(n_new, n_q_heads);
  return attn_prefill_chunk_split_q8(q_codes, q_scales, n_new, k_cache, v_cache, k_scale, v_scale,
                                     block_table, context_len, 1, num_pages, n_q_heads,
                                     n_kv_heads, head_dim, sm_scale, out, ws + q8,
                                     workspace_bytes - q8, stream);
}

int q_quant(const uint16_t* q_bf16, int n_rows, int head_dim, int8_t* codes, float* scales,
            void* stream) {
  if (n_rows < 0 || n_rows > 2147483000) return set_error(I8A_EINVAL, "q_quant: n_rows %d", n_rows);
  if (head_dim != 256) return set_error(I8A_EUNSUPPORTED, "q_quant: head_dim %d unsupported", head_dim);
  if (n_rows == 0) return I8A_OK;
  if (!q_bf16 || !codes || !scales) return set_error(I8A_EINVAL, "q_quant: null pointer");
  return launch_q_quant(q_bf16, n_rows, codes, scales, (hipStream_t)stream);
}

size_t attn_decode_workspace_bytes(int num_seqs, int max_context_len, int n_q_heads, int head_dim) {
  if (num_seqs <= 0 || max_context_len <= 0 || n_q_heads <= 0 || head_dim != 256) return 0;
  return decode_ws_bytes(num_seqs, max_context_len, n_q_heads);
}

// The attention entry points take the query either as bf16 rows (quantized inside) or,
// in their *_q8 forms, as int8 codes with fp32 scales (kv_produce's output): q_scales
// is null for the former.
static int decode_impl(const void* q, const float* q_scales, const int8_t* k_cache,
                       const int8_t* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int max_blocks_per_seq,
                       const int32_t* context_lens, int num_seqs, int max_context_len,
                       int num_pages, int n_q_heads, int n_kv_heads, int head_dim, float sm_scale,
                       float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (num_seqs < 0 || num_seqs > 65535) return set_error(I8A_EINVAL, "attn_decode: num_seqs %d", num_seqs);
  if (num_seqs == 0) return I8A_OK;
  if (max_context_len <= 0 || max_blocks_per_seq <= 0 || num_pages <= 0)
    return set_error(I8A_EINVAL, "attn_decode: max_context_len %d, max_blocks_per_seq %d, num_pages %d",
                     max_context_len, max_blocks_per_seq, num_pages);
  if ((rc = check_sm_scale("attn_decode", sm_scale))) return rc;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !context_lens || !out ||
      !workspace)
    return set_error(I8A_EINVAL, "attn_decode: null pointer");
  if (((uintptr_t)workspace & 15u) != 0) return set_error(I8A_EINVAL, "attn_decode: workspace not 16-byte aligned");
  const size_t need = decode_ws_bytes(num_seqs, max_context_len, n_q_heads);
  if (workspace_bytes < need)
    return set_error(I8A_EWORKSPACE, "attn_decode: workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int max_parts = (max_context_len + 511) / 512;
  return launch_decode(q, q_scales, k_cache, v_cache, k_scale, v_scale, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                       n_q_heads, n_kv_heads, sm_scale, out, (float*)workspace, max_parts,
                       (hipStream_t)stream);
}

int attn_decode(const uint16_t* q, const int8_t* k_cache, const int8_t* v_cache,
                const float* k_scale, const float* v_scale, const int32_t* block_table,
                int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                int max_context_len, int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  return decode_impl(q, nullptr, k_cache, v_cache, k_scale, v_scale, block_table,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                     n_q_heads, n_kv_heads, head_dim, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

int attn_decode_q8(const int8_t* q_codes, const float* q_scales, const int8_t* k_cache,
                   const int8_t* v_cache, const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks_per_seq,
                   const int32_t* context_lens, int num_seqs, int max_context_len, int num_pages,
                   int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_scales && num_seqs > 0) return set_error(I8A_EINVAL, "attn_decode_q8: null q_scales");
  return decode_impl(q_codes, q_scales, k_cache, v_cache, k_scale, v_scale, block_table,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                     n_q_heads, n_kv_heads, head_dim, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

size_t attn_verify_workspace_bytes(int num_seqs, int nq, int max_context_len, int n_q_heads,
                                   int head_dim) {
  if (num_seqs <= 0 || nq < 1 || nq > 8 || max_context_len <= 0 || n_q_heads <= 0 || head_dim != 256)
    return 0;
  return decode_ws_bytes((long long)num_seqs * nq, max_context_len, n_q_heads);
}

static int verify_impl(const void* q, const float* q_scales, int nq, const int8_t* k_cache,
                       const int8_t* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int max_blocks_per_seq,
                       const int32_t* context_lens, int num_seqs, int max_context_len,
                       int num_pages, int n_q_heads, int n_kv_heads, int head_dim, float sm_scale,
                       float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (nq < 1 || nq > 8) return set_error(I8A_EINVAL, "attn_verify: nq %d outside 1..8", nq);
  if (num_seqs < 0 || (long long)num_seqs * nq > 65535)
    return set_error(I8A_EINVAL, "attn_verify: num_seqs %d x nq %d", num_seqs, nq);
  if (num_seqs == 0) return I8A_OK;
  if (max_context_len <= 0 || max_blocks_per_seq <= 0 || num_pages <= 0)
    return set_error(I8A_EINVAL, "attn_verify: max_context_len %d, max_blocks_per_seq %d, num_pages %d",
                     max_context_len, max_blocks_per_seq, num_pages);
  if ((rc = check_sm_scale("attn_verify", sm_scale))) return rc;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !context_lens || !out ||
      !workspace)
    return set_error(I8A_EINVAL, "attn_verify: null pointer");
  if (((uintptr_t)workspace & 15u) != 0) return set_error(I8A_EINVAL, "attn_verify: workspace not 16-byte aligned");
  const size_t need = decode_ws_bytes((long long)num_seqs * nq, max_context_len, n_q_heads);
  if (workspace_bytes < need)
    return set_error(I8A_EWORKSPACE, "attn_verify: workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int max_parts = (max_context_len + 511) / 512;
  return launch_verify(q, q_scales, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                       n_q_heads, n_kv_heads, sm_scale, out, (float*)workspace, max_parts,
                       (hipStream_t)stream);
}

int attn_verify(const uint16_t* q, int nq, const int8_t* k_cache, const int8_t* v_cache,
                const float* k_scale, const float* v_scale, const int32_t* block_table,
                int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                int max_context_len, int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  return verify_impl(q, nullptr, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                     n_q_heads, n_kv_heads, head_dim, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

int attn_verify_q8(const int8_t* q_codes, const float* q_scales, int nq, const int8_t* k_cache,
                   const int8_t* v_cache, const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks_per_seq,
                   const int32_t* context_lens, int num_seqs, int max_context_len, int num_pages,
                   int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_scales && num_seqs > 0) return set_error(I8A_EINVAL, "attn_verify_q8: null q_scales");
  return verify_impl(q_codes, q_scales, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                     n_q_heads, n_kv_heads, head_dim, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

int attn_decode_partition_rows(int num_seqs, int max_context_len, int n_kv_heads) {
  if (num_seqs <= 0 || max_context_len <= 0 || n_kv_heads <= 0) return 0;
  return partition_law(num_seqs, max_context_len, n_kv_heads);
}

static int resolve_partition(int partition_rows, int num_seqs, int max_context_len, int n_kv_heads) {
  if (partition_rows == 0) return partition_law(num_seqs, max_context_len, n_kv_heads);
  if (partition_rows == 64 || partition_rows == 128 || partition_rows == 256 || partition_rows == 512)
    return partition_rows;
  return -1;
}

size_t attn_decode_int8p_workspace_bytes(int num_seqs, int nq, int max_context_len, int n_q_heads,
                                         int n_kv_heads, int head_dim, int partition_rows) {
  if (num_seqs <= 0 || nq < 1 || nq > 8 || max_context_len <= 0 || n_q_heads <= 0 ||
      n_kv_heads <= 0 || head_dim != 256)
    return 0;
  const int part = resolve_partition(partition_rows, num_seqs, max_context_len, n_kv_heads);
  if (part < 0) return 0;
  return partials_bytes((long long)num_seqs * nq, max_context_len, n_q_heads, part);
}

static int int8p_impl(const void* q, const float* q_scales, int nq, const int8_t* k_cache,
                      const int8_t* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int max_context_len,
                      int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                      int partition_rows, float sm_scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (nq < 1 || nq > 8) return set_error(I8A_EINVAL, "attn_decode_int8p: nq %d outside 1..8", nq);
  if (num_seqs < 0 || (long long)num_seqs * nq > 65535)
    return set_error(I8A_EINVAL, "attn_decode_int8p: num_seqs %d x nq %d", num_seqs, nq);
  if (num_seqs == 0) return I8A_OK;
  if (max_context_len <= 0 || max_blocks_per_seq <= 0 || num_pages <= 0)
    return set_error(I8A_EINVAL, "attn_decode_int8p: max_context_len %d, max_blocks_per_seq %d, num_pages %d",
                     max_context_len, max_blocks_per_seq, num_pages);
  const int part = resolve_partition(partition_rows, num_seqs, max_context_len, n_kv_heads);
  if (part < 0)
    return set_error(I8A_EINVAL, "attn_decode_int8p: partition_rows %d (0, 64, 128, 256 or 512)",
                     partition_rows);
  if ((rc = check_sm_scale("attn_decode_int8p", sm_scale))) return rc;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !context_lens || !out ||
      !workspace)
    return set_error(I8A_EINVAL, "attn_decode_int8p: null pointer");
  if (((uintptr_t)workspace & 15u) != 0)
    return set_error(I8A_EINVAL, "attn_decode_int8p: workspace not 16-byte aligned");
  const size_t need = partials_bytes((long long)num_seqs * nq, max_context_len, n_q_heads, part);
  if (workspace_bytes < need)
    return set_error(I8A_EWORKSPACE, "attn_decode_int8p: workspace %zu bytes < %zu needed",
                     workspace_bytes, need);
  return launch_decode_i8pv(1, part, q, q_scales, nq, k_cache, v_cache, k_scale, v_scale,
                            block_table, max_blocks_per_seq, context_lens, num_seqs,
                            max_context_len, num_pages, n_q_heads, n_kv_heads, sm_scale, out,
                            (float*)workspace, (hipStream_t)stream);
}

int attn_decode_int8p(const uint16_t* q, int nq, const int8_t* k_cache, const int8_t* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                      int max_context_len, int num_pages, int n_q_heads, int n_kv_heads,
                      int head_dim, int partition_rows, float sm_scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return int8p_impl(q, nullptr, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                    max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                    n_q_heads, n_kv_heads, head_dim, partition_rows, sm_scale, out, workspace,
                    workspace_bytes, stream);
}

int attn_decode_int8p_q8(const int8_t* q_codes, const float* q_scales, int nq,
                         const int8_t* k_cache, const int8_t* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                         int partition_rows, float sm_scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!q_scales && num_seqs > 0) return set_error(I8A_EINVAL, "attn_decode_int8p_q8: null q_scales");
  return int8p_impl(q_codes, q_scales, nq, k_cache, v_cache, k_scale, v_scale, block_table,
                    max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_pages,
                    n_q_heads, n_kv_heads, head_dim, partition_rows, sm_scale, out, workspace,
                    workspace_bytes, stream);
}

// The split route of a chunk: 0 the one pass, 1 key partitions of the chunk kernel, 2 the
// int8-P decode kernel (chunks of at most 8 rows: the same weight rule, one workgroup per
// (KV head, key partition) for all the rows). Causal chunks only.
static int split_route(int n_new, int context_len, int causal, int n_kv_heads) {
  if (!causal || n_new <= 0) return 0;
  if (n_new <= 8) return 2;
  int pb;
  return prefill_split_parts(n_new, context_len, causal, n_kv_heads, &pb) > 1 ? 1 : 0;
}

static size_t split_ws_bytes(int n_new, int context_len, int causal, int n_q_heads, int n_kv_heads) {
  switch (split_route(n_new, context_len, causal, n_kv_heads)) {
    case 1: return prefill_split_ws_bytes(n_new, context_len, causal, n_q_heads, n_kv_heads);
    case 2: return partials_bytes(n_new, context_len, n_q_heads, partition_law(1, context_len, n_kv_heads));
    default: return 0;
  }
}

static int prefill_impl(const void* q, const float* q_scales, int n_new, const int8_t* k_cache,
                        const int8_t* v_cache, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int context_len, int causal, int num_pages,
                        int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                        int split, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (rc) return rc;
  if (n_new < 0 || context_len < 1 || n_new > context_len || num_pages <= 0 ||
      (causal != 0 && causal != 1))
    return set_error(I8A_EINVAL, "attn_prefill_chunk: n_new %d, context_len %d, num_pages %d, causal %d",
                     n_new, context_len, num_pages, causal);
  if (context_len > 2147483000 - 64) return set_error(I8A_EINVAL, "attn_prefill_chunk: context too long");
  size_t need = 0;
  if (split) {
    need = split_ws_bytes(n_new, context_len, causal, n_q_heads, n_kv_heads);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 15u) != 0))
      return set_error(I8A_EINVAL, "attn_prefill_chunk_split: workspace null or not 16-byte aligned");
    if (workspace_bytes < need)
      return set_error(I8A_EWORKSPACE, "attn_prefill_chunk_split: workspace %zu bytes < %zu needed",
                       workspace_bytes, need);
  }
  if ((long long)num_pages * n_kv_heads * 16 >= (1ll << 32))
    return set_error(I8A_EUNSUPPORTED, "attn_prefill_chunk: num_pages %d x %d heads exceeds the scale index range",
                     num_pages, n_kv_heads);
  if ((rc = check_sm_scale("attn_prefill_chunk", sm_scale))) return rc;
  if (n_new == 0) return I8A_OK;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !out)
    return set_error(I8A_EINVAL, "attn_prefill_chunk: null pointer");
  if (split && split_route(n_new, context_len, causal, n_kv_heads) == 2)
    return launch_decode_i8pv(1, partition_law(1, context_len, n_kv_heads), q, q_scales, n_new,
                              k_cache, v_cache, k_scale, v_scale, block_table,
                              (context_len + 15) / 16, nullptr, 1, context_len, num_pages,
                              n_q_heads, n_kv_heads, sm_scale, out, static_cast<float*>(workspace),
                              (hipStream_t)stream);
  return launch_prefill(q, q_scales, n_new, k_cache, v_cache, k_scale, v_scale, block_table,
                        context_len, causal, num_pages, n_q_heads, n_kv_heads, sm_scale, out,
                        need > 0 ? static_cast<float*>(workspace) : nullptr, workspace_bytes,
                        (hipStream_t)stream);
}

int attn_prefill_chunk(const uint16_t* q, int n_new, const int8_t* k_cache, const int8_t* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       int context_len, int causal, int num_pages, int n_q_heads, int n_kv_heads,
                       int head_dim, float sm_scale, float* out, void* stream) {
  return prefill_impl(q, nullptr, n_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_len, causal, num_pages, n_q_heads, n_kv_heads, head_dim, sm_scale,
                      out, 0, nullptr, 0, stream);
}

int attn_prefill_chunk_q8(const int8_t* q_codes, const float* q_scales, int n_new,
                          const int8_t* k_cache, const int8_t* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* block_table, int context_len,
                          int causal, int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                          float sm_scale, float* out, void* stream) {
  if (!q_scales && n_new > 0) return set_error(I8A_EINVAL, "attn_prefill_chunk_q8: null q_scales");
  return prefill_impl(q_codes, q_scales, n_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_len, causal, num_pages, n_q_heads, n_kv_heads, head_dim, sm_scale,
                      out, 0, nullptr, 0, stream);
}

size_t attn_prefill_chunk_split_workspace_bytes(int n_new, int context_len, int causal,
                                                int n_q_heads, int n_kv_heads, int head_dim) {
  if (n_new <= 0 || context_len < n_new || context_len > 2147483000 - 64 ||
      (causal != 0 && causal != 1) || head_dim != 256 || n_kv_heads <= 0 ||
      n_kv_heads > 65535 / 6 || n_q_heads != n_kv_heads * 6)
    return 0;
  return split_ws_bytes(n_new, context_len, causal, n_q_heads, n_kv_heads);
}

int attn_prefill_chunk_split(const uint16_t* q, int n_new, const int8_t* k_cache,
                             const int8_t* v_cache, const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int context_len, int causal,
                             int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                             float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return prefill_impl(q, nullptr, n_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_len, causal, num_pages, n_q_heads, n_kv_heads, head_dim, sm_scale,
                      out, 1, workspace, workspace_bytes, stream);
}

int attn_prefill_chunk_split_q8(const int8_t* q_codes, const float* q_scales, int n_new,
                                const int8_t* k_cache, const int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int context_len, int causal,
                                int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                                float sm_scale, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!q_scales && n_new > 0)
    return set_error(I8A_EINVAL, "attn_prefill_chunk_split_q8: null q_scales");
  return prefill_impl(q_codes, q_scales, n_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_len, causal, num_pages, n_q_heads, n_kv_heads, head_dim, sm_scale,
                      out, 1, workspace, workspace_bytes, stream);
}

// Opt-in checks of the paging metadata on host copies. The kernels map an entry outside
// the pool to page 0 (memory-safe, result unspecified) and the writers skip slots outside
// the pool; these calls turn such entries into an error that names the first offender.
int int8attn_check_block_table(const int32_t* block_table, int num_seqs, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len, int num_pages) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_pages <= 0)
    return set_error(I8A_EINVAL, "check_block_table: num_seqs %d, max_blocks_per_seq %d, "
                     "max_context_len %d, num_pages %d", num_seqs, max_blocks_per_seq,
                     max_context_len, num_pages);
  if (num_seqs > 0 && !block_table) return set_error(I8A_EINVAL, "check_block_table: null table");
  const long long cap = (long long)max_blocks_per_seq * 16;
  for (int s = 0; s < num_seqs; ++s) {
    const int ctx = context_lens ? context_lens[s] : max_context_len;
    if (ctx < 0 || ctx > max_context_len || ctx > cap)
      return set_error(I8A_EINVAL, "check_block_table: sequence %d has context %d (0 .. min(%d, "
                       "16 x %d blocks))", s, ctx, max_context_len, max_blocks_per_seq);
    const int32_t* row = block_table + (size_t)s * max_blocks_per_seq;
    for (int b = 0; b < (ctx + 15) / 16; ++b)
      if (row[b] < 0 || row[b] >= num_pages)
        return set_error(I8A_EINVAL, "check_block_table: sequence %d block %d (tokens %d..%d) "
                         "names page %d outside the pool of %d pages", s, b, 16 * b,
                         ctx < 16 * b + 16 ? ctx - 1 : 16 * b + 15, (int)row[b], num_pages);
  }
  return I8A_OK;
}

int int8attn_check_slots(const int32_t* slot_mapping, int n_tokens, int num_pages) {
  if (n_tokens < 0 || num_pages <= 0 || (long long)num_pages * 16 > 2147483647LL)
    return set_error(I8A_EINVAL, "check_slots: n_tokens %d, num_pages %d", n_tokens, num_pages);
  if (n_tokens > 0 && !slot_mapping) return set_error(I8A_EINVAL, "check_slots: null slot_mapping");
  const int n_slots = num_pages * 16;
  std::vector<int32_t> seen;
  seen.reserve(n_tokens);
  for (int t = 0; t < n_tokens; ++t) {
    const int32_t sl = slot_mapping[t];
    if (sl >= n_slots)
      return set_error(I8A_EINVAL, "check_slots: token %d has slot %d outside the pool of %d slots",
                       t, (int)sl, n_slots);
    if (sl >= 0) seen.push_back(sl);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i] == seen[i - 1])
      return set_error(I8A_EINVAL, "check_slots: slot %d is named by two tokens", (int)seen[i]);
  return I8A_OK;
}

}  // extern "C"
