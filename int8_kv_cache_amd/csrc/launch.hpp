// Host-side launch helpers and error plumbing shared by the kernel files and api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8a {

// Records a thread-local message for int8attn_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...);
// hipGetLastError() after a launch: I8A_OK or I8A_ELAUNCH with the runtime's message.
int check_launch(const char* what);

int launch_kv_quant_write(const void* k, const void* v, int in_bf16, int n_tokens, int n_kv_heads,
                          const int32_t* slots, int8_t* k_cache, int8_t* v_cache, float* k_scale,
                          float* v_scale, int num_pages, hipStream_t stream);
int launch_kv_produce(const void* q, const void* k, const void* v, int in_bf16, int n_tokens,
                      int n_q_heads, int n_kv_heads, const int32_t* positions, const float* cos_sin,
                      int rotary_dim, int max_pos, const int32_t* slots, int8_t* k_cache,
                      int8_t* v_cache, float* k_scale, float* v_scale, int num_pages,
                      int8_t* q_codes, float* q_scales, uint16_t* q_rot, uint16_t* k_rot,
                      hipStream_t stream);
// ws == nullptr: the one pass; otherwise causal chunks whose tiles reach past one key
// partition run split (chunk_bf16_ws_bytes of scratch) and merged.
int launch_chunk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int causal,
                      int n_q_heads, int n_kv_heads, float sm_scale, float* out, float* ws,
                      hipStream_t stream);
int chunk_bf16_split_parts(int n, int causal, int n_kv_heads, int* part_blocks);
size_t chunk_bf16_ws_bytes(int n, int causal, int n_q_heads, int n_kv_heads);
int launch_q_quant(const uint16_t* q, int n_rows, int8_t* codes, float* scales,
                   hipStream_t stream);
// q: bf16 rows to quantize (q_scales == nullptr) or int8 codes with q_scales (kv_produce).
int launch_decode(const void* q, const float* q_scales, const int8_t* k_cache, const int8_t* v_cache,
                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                  int max_blocks, const int32_t* ctx_lens, int num_seqs, int max_ctx,
                  int num_pages, int n_q_heads, int n_kv_heads, float sm_scale, float* out,
                  float* ws, int max_parts, hipStream_t stream);
int launch_verify(const void* q, const float* q_scales, int nq, const int8_t* k_cache,
                  const int8_t* v_cache,
                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                  int max_blocks, const int32_t* ctx_lens, int num_seqs, int max_ctx,
                  int num_pages, int n_q_heads, int n_kv_heads, float sm_scale, float* out,
                  float* ws, int max_parts, hipStream_t stream);
// ctx_lens == nullptr (here and in launch_decode_i8pv): one sequence of ctx_cap keys.
int launch_merge(const float* ws_m, const float* ws_l, const float* ws_o, const int32_t* ctx_lens,
                 int ctx_cap, int num_seqs, int nq, int n_q_heads, int max_parts, int part_rows,
                 float* out, hipStream_t stream);
// One sequence's nq query rows at the tail of ctx keys, each with the partial states of
// up to n_parts key partitions of part_rows keys: [row][head][partition] (m, l, o[256]).
int launch_merge_rows(const float* ws_m, const float* ws_l, const float* ws_o, int ctx, int nq,
                      int n_q_heads, int n_parts, int part_rows, float* out, hipStream_t stream);
int launch_decode_i8pv(int digits, int part_rows, const void* q, const float* q_scales, int nq,
                       const int8_t* k_cache,
                       const int8_t* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int max_blocks, const int32_t* ctx_lens,
                       int num_seqs, int max_ctx, int num_pages, int n_q_heads, int n_kv_heads,
                       float sm_scale, float* out, float* ws, hipStream_t stream);
int launch_prefill(const void* q, const float* q_scales, int n_new, const int8_t* k_cache,
                   const int8_t* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int ctx, int causal, int num_pages, int n_q_heads, int n_kv_heads,
                   float sm_scale, float* out, float* ws, size_t ws_bytes, hipStream_t stream);
// Key partitions of the split route for a chunk (1: the single pass); *part_blocks gets
// the 64-key blocks per partition.
int prefill_split_parts(int n_new, int ctx, int causal, int n_kv_heads, int* part_blocks);
// Workspace bytes of the split route (0 when the chunk takes the single pass).
size_t prefill_split_ws_bytes(int n_new, int ctx, int causal, int n_q_heads, int n_kv_heads);

}  // namespace i8a
