/* int8attn.h -- C ABI of the MI355X (gfx950) INT8-KV paged attention library.
 *
 * Attention reads a paged cache of int8 K/V codes with one fp32 absmax scale per
 * (token, KV head) directly; no dequantized K/V tensor ever exists.
 *
 * Sources (cited by page title and section):
 *  [DCU]   "INT8 KV and INT8 MMAC attention on a gfx936 DCU" (gfx936 DCU上实现INT8 KV与
 *          INT8 MMAC Attention推理优化, sourcefind forum article)
 *  [DOT4]  "dot4-flash-attention" (GitHub README)
 *  [QSA]   "#3381 prompt QSA attention without the decode kernel's split and merge"
 *          (strata engine pull request)
 *  [R4D]   "ROCm/RDNA4 (gfx1201) vLLM: native HIP kernels, baked-in quantizers and
 *          tuner" (vLLM docs page, kernel-lessons part)
 *
 * ---------------------------------------------------------------------------
 * Conventions common to every entry point
 *  - Every pointer argument except `stream` is a DEVICE pointer (hipMalloc'd or
 *    torch-owned GPU memory). The caller owns every buffer; the library keeps no
 *    reference after the call returns and allocates nothing (attn_decode_noalloc's
 *    fixed scratch array is part of the library's own device image).
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *    Work is enqueued asynchronously; no call synchronizes. A call enqueues only kernel
 *    launches (no memset, copy or host callback), so it may be captured into a HIP
 *    graph; every replay recomputes the outputs from the inputs it then finds, bit for
 *    bit as an eager call does (no kernel uses atomics or timing-dependent orders).
 *  - Return value: I8A_OK (0) on success, a negative I8A_E* code on error. On an
 *    argument error nothing is enqueued and no output is touched. The message of the
 *    last error on the calling thread is available from int8attn_last_error().
 *  - Thread-safe: no global mutable state except the thread-local error message.
 *  - v1 shape contract: head_dim == 256, page size 16 tokens, n_q_heads ==
 *    6 * n_kv_heads (GQA groups of 6, query head h reads KV head h / 6) [DOT4 contract
 *    "D=256, GQA required"; DCU §1.1 geometry 24 q heads over 4 KV heads]. Any other
 *    shape returns I8A_EUNSUPPORTED.
 *  - Inputs must be finite. Contexts are >= 1 token.
 *
 * ---------------------------------------------------------------------------
 * Paged cache layout (the contract between the writer and the readers)
 *  A page holds 16 consecutive tokens of one sequence; slot = page * 16 + offset.
 *  Each (page p, KV head h) owns one contiguous 4096-byte block of K codes, one of V
 *  codes, and 16 fp32 scales of each. With H = n_kv_heads, the element (p, h, token
 *  offset o in 0..15, dim d in 0..255) lives at:
 *
 *    k_cache byte  ((p*H + h)*16 + d/16)*256 + o*16 + d%16
 *        = [page][head][d/16][o][d%16]: 16 dims of one token are one 16-byte run
 *          [DCU §2.3 chooses the same K blocking, [blocks, 4, 16, block_size, 16]].
 *    v_cache byte  (p*H + h)*4096 + d*16 + o
 *        = [page][head][d][o]: the 16 tokens of one dim are one 16-byte run, which is
 *          exactly one lane's operand bytes of the PV matrix product [DCU §2.3 keeps V
 *          token-contiguous per output dim, [blocks, 4, 256, block_size]].
 *    k_scale / v_scale float  (p*H + h)*16 + o      [DCU §2.3: FP32 scales apart from
 *          the codes]
 *
 *  Per token and per layer this is 2*4*256 + 2*4*4 = 2080 bytes at H = 4 [DCU §1.1].
 *  The library never reads a slot that no table entry covers with a valid position.
 *
 * Quantization rule (bit-exact contract) [DCU §2.1]
 *  For one row x of 256 values (one token of one K, V or Q head), in IEEE fp32:
 *    amax  = max |x_i|
 *    scale = amax / 127           (correctly rounded fp32 division)
 *    code  = clamp(rint(x_i / scale), -127, 127)   (x_i / scale correctly rounded,
 *                                                    rint = round half to even)
 *  If scale == 0 (amax == 0, or amax/127 underflows) the codes are all 0 and the
 *  stored scale is 0.0. Dequantized value = code * scale.
 */
#ifndef INT8ATTN_H
#define INT8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I8A_OK            0
#define I8A_EINVAL       -1  /* null pointer, negative or zero size, bad dtype flag    */
#define I8A_EUNSUPPORTED -2  /* shape outside the v1 contract (head_dim, GQA group)    */
#define I8A_EWORKSPACE   -3  /* decode workspace too small                             */
#define I8A_ELAUNCH      -4  /* the HIP runtime reported an error at launch            */

#define I8A_DTYPE_F32  0
#define I8A_DTYPE_BF16 1

/* Message of the last error returned on this thread ("" if none). The pointer stays
 * valid until the next call on the same thread. */
const char* int8attn_last_error(void);

/* Library version, (major << 16) | minor. */
int int8attn_version(void);

/* kv_quant_write -- quantize new K and V rows and write them into the paged cache.
 * [DCU §2.1 rule; §2.2 fused producer: absmax, scale, quantize, paged INT8 write and
 *  scale write in one kernel; DOT4 "K packing" at cache-write time.]
 *
 *  k, v          input rows [n_tokens][n_kv_heads][head_dim], fp32 or bf16 (in_dtype),
 *                row-major and contiguous. K and V rows are quantized independently.
 *  slot_mapping  int32 [n_tokens]: destination slot of each token. A slot < 0 or
 *                >= num_pages*16 skips that token (nothing is written for it). Two
 *                tokens with the same slot: unspecified which one wins.
 *  k_cache, v_cache   int8 [num_pages * n_kv_heads * 4096] in the layout above.
 *  k_scale, v_scale   fp32 [num_pages * n_kv_heads * 16].
 *  Only the slots named by slot_mapping are written; everything else is untouched.
 *  n_tokens == 0 is a no-op returning I8A_OK. */
int kv_quant_write(const void* k, const void* v, int in_dtype,
                   int n_tokens, int n_kv_heads, int head_dim,
                   const int32_t* slot_mapping,
                   int8_t* k_cache, int8_t* v_cache,
                   float* k_scale, float* v_scale,
                   int num_pages, void* stream);

/* kv_produce -- the fused producer: RoPE on the new Q and K rows, then Q, K and V
 * quantized with the kv_quant_write rule, K/V codes and scales written into the paged
 * cache and Q kept as int8 codes + scales, in one launch.
 * [DCU §2.2: read Q/K/V, apply RoPE to Q/K, reduce each row's absmax, compute the scale
 *  and quantize, write the K/V codes and scales into the paged cache, and skip writing
 *  back high-precision Q/K; the query is quantized once and reused by every partition.]
 *
 *  q             [n_tokens][n_q_heads][head_dim] (fp32 or bf16 as in_dtype), or NULL
 *                together with q_codes and q_scales (K/V only).
 *  k, v, slot_mapping, caches, num_pages: as for kv_quant_write.
 *  positions     int32 [n_tokens]: the position of each token (the RoPE angle index);
 *                values outside [0, max_position) are clamped into it (memory-safe,
 *                result unspecified).
 *  cos_sin       fp32 [max_position][rotary_dim], 16-byte aligned: row p holds the cos of
 *                pairs 0..rotary_dim/2-1, then their sin. The frequencies, base and any
 *                scaling of the caller's RoPE live in this table.
 *  rotary_dim    0 (no rotation) or a multiple of 8 up to head_dim: pair (i, i +
 *                rotary_dim/2), i < rotary_dim/2, of each Q and K row turns by row p of
 *                the table; dims >= rotary_dim pass through. In fp32 with every product
 *                and sum rounded on its own: x_i' = x_i c - x_j s, x_j' = x_j c + x_i s.
 *  q_codes       int8 [n_tokens][n_q_heads][head_dim] and q_scales fp32
 *                [n_tokens][n_q_heads]: the rotated Q rows quantized (the *_q8 attention
 *                entry points take them as they are); both NULL: not produced.
 *  q_rot, k_rot  bf16 [n_tokens][n_q_heads][head_dim] / [n_tokens][n_kv_heads][head_dim]:
 *                the rotated Q and K rows rounded to bf16 (nearest, ties to even), for the
 *                high-precision attention of a chunk with no history [DCU §3.1]; NULL: not
 *                written. q must be given when q_codes or q_rot is.
 *  V rows are not rotated. Codes, scales and bf16 rows are bit-exact functions of the
 *  inputs and the table. */
int kv_produce(const void* q, const void* k, const void* v, int in_dtype,
               int n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
               const int32_t* positions, const float* cos_sin, int rotary_dim,
               int max_position, const int32_t* slot_mapping,
               int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
               int num_pages, int8_t* q_codes, float* q_scales,
               uint16_t* q_rot, uint16_t* k_rot, void* stream);

/* attn_chunk_bf16 -- high-precision causal (or full) attention of a chunk over its own
 * rows: q [n][n_q_heads][head_dim], k, v [n][n_kv_heads][head_dim], all bf16 and
 * contiguous; query t sees keys 0..t (causal) or all n.
 * [DCU §3.1: the first prefill chunk has no history and keeps a high-precision attention
 *  while the producer writes its K/V as int8.]
 *  Scores are bf16 x bf16 products summed in fp32; the softmax runs in fp32; the weights
 *  multiply V as two bf16 terms (16 significant bits) with fp32 accumulation, so the
 *  output meets the fp32-class bound (1e-4 * max|V|) against exact attention on the
 *  same bf16 rows.
 *  out           fp32 [n][n_q_heads][head_dim]. n == 0 is a no-op.
 *  workspace     NULL: one pass, one workgroup per 32 query rows and KV head (the
 *                causal tiles then run 1 .. n/64 key blocks each, and the longest sets
 *                the time). Otherwise device scratch, 16-byte aligned, of at least
 *                attn_chunk_bf16_workspace_bytes(...) bytes (contents on entry do not
 *                matter): a causal chunk whose tiles reach past one key partition is
 *                cut into partitions of the average work per CU, the tiles with most
 *                keys first, and the rows past the first partition are merged by a
 *                second kernel (log-sum-exp merge of the partial states, as in the
 *                decode [DCU §3.3]). The two routes differ only by the merge's
 *                rounding, within the same bound. A smaller workspace_bytes returns
 *                I8A_EWORKSPACE. */
size_t attn_chunk_bf16_workspace_bytes(int n, int causal, int n_q_heads, int n_kv_heads,
                                       int head_dim);
int attn_chunk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n,
                    int causal, int n_q_heads, int n_kv_heads, int head_dim,
                    float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of scratch prefill_step needs for a chunk of n_new rows ending at context_len:
 * without history (context_len == n_new) the rotated bf16 Q and K rows
 * (n_new * (n_q_heads + n_kv_heads) * head_dim * 2, rounded up to 256) plus
 * attn_chunk_bf16_workspace_bytes(n_new, 1, ...); with history the
 * int8 Q codes with scales (n_new * n_q_heads * (head_dim + 4), rounded up to 256) plus
 * attn_prefill_chunk_split_workspace_bytes(n_new, context_len, 1, ...). 0 for invalid
 * arguments. */
size_t prefill_step_workspace_bytes(int n_new, int context_len, int n_q_heads, int n_kv_heads,
                                    int head_dim);

/* prefill_step -- one prefill chunk end to end, routed by its history [DCU §3.1, §3.2]:
 * the producer (RoPE, quantization, paged K/V write) runs first, then
 *  - context_len == n_new (no history): attn_chunk_bf16 on the rotated bf16 rows;
 *  - otherwise: attn_prefill_chunk_split_q8 on the int8 cache with the producer's Q
 *    codes (the history exists only as int8; short chunks split over key partitions,
 *    the others in one pass).
 *  q, k, v       bf16 [n_new][heads][head_dim] as projected (before RoPE).
 *  positions, cos_sin, rotary_dim, max_position, slot_mapping, caches: as for kv_produce.
 *  block_table, context_len: as for attn_prefill_chunk (context_len counts the chunk).
 *  workspace     >= prefill_step_workspace_bytes(...), 256-byte aligned.
 *  out           fp32 [n_new][n_q_heads][head_dim]. */
int prefill_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n_new,
                 const int32_t* positions, const float* cos_sin, int rotary_dim,
                 int max_position, const int32_t* slot_mapping,
                 int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                 int num_pages, const int32_t* block_table, int context_len,
                 int n_q_heads, int n_kv_heads, int head_dim, float sm_scale, float* out,
                 void* workspace, size_t workspace_bytes, void* stream);

/* q_quant -- quantize bf16 query rows with the same rule [DCU §2.2: the query is
 * quantized once per token and head]. The attention entry points do this internally
 * with the same device routine; this entry exposes it for inspection.
 *  q_bf16  [n_rows][head_dim] bf16 bits (row = one (token, q head));
 *  codes   int8 [n_rows][head_dim];  scales fp32 [n_rows]. */
int q_quant(const uint16_t* q_bf16, int n_rows, int head_dim,
            int8_t* codes, float* scales, void* stream);

/* Bytes of scratch attn_decode needs for this batch shape: the per-partition partial
 * softmax states, num_seqs * n_q_heads * ceil(max_context_len/512) * (2 + head_dim)
 * floats, rounded up to 256 bytes. Sizing for the largest max_context_len lets smaller
 * calls reuse one buffer (their partials pack into a prefix). Returns 0 for invalid
 * arguments. */
size_t attn_decode_workspace_bytes(int num_seqs, int max_context_len,
                                   int n_q_heads, int head_dim);

/* attn_decode -- one new query token per sequence against its paged INT8 K/V.
 * [DOT4 route table: split-K stage 1 over 512-row splits + stage 2 merge; DCU §3.3:
 *  paged INT8 K/V, per-token scales, INT8 query + query scale, block table, partitions
 *  then a merge of softmax states and outputs; DCU §1.3 score formula.]
 *
 *  Stage 1: for every (sequence, KV head, 512-row partition) the query rows of the
 *  group are quantized (q_quant rule), scores = int8(Q).int8(K) * sQ * sK * sm_scale
 *  (exact int32 dot, scales applied after accumulation), an fp32 softmax over the
 *  partition, and the weighted sum of V in fp32 precision; the partial state
 *  (max, sum, unnormalised output) goes to `workspace`.
 *  Stage 2: partials are merged per (sequence, q head) by log-sum-exp.
 *
 *  q             bf16 [num_seqs][n_q_heads][head_dim]
 *  block_table   int32 [num_seqs][max_blocks_per_seq]: page of each 16-token block
 *  context_lens  int32 [num_seqs]: keys 0..ctx-1 are visible (the new token's K/V row
 *                must already be written). Values are clamped on the device to
 *                [0, min(max_context_len, 16*max_blocks_per_seq)]; a sequence with 0
 *                keys produces zeros.
 *  max_context_len   >= every context_lens[s] (sets the launch grid).
 *  num_pages     pool size; a table entry outside [0, num_pages) reads page 0 instead
 *                (memory-safe, result unspecified; int8attn_check_block_table reports
 *                such entries).
 *  sm_scale      softmax scale, normally 1/sqrt(head_dim) = 1/16 [DCU §1.3]; every
 *                attention entry point refuses a scale that is negative or not finite
 *                (I8A_EINVAL).
 *  out           fp32 [num_seqs][n_q_heads][head_dim], fully overwritten.
 *  workspace     >= attn_decode_workspace_bytes(...) bytes, device memory, contents
 *                undefined after the call. Calls sharing one workspace must be ordered
 *                on one stream. */
int attn_decode(const uint16_t* q,
                const int8_t* k_cache, const int8_t* v_cache,
                const float* k_scale, const float* v_scale,
                const int32_t* block_table, int max_blocks_per_seq,
                const int32_t* context_lens, int num_seqs, int max_context_len,
                int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                float sm_scale, float* out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch attn_verify needs: num_seqs * nq * n_q_heads *
 * ceil(max_context_len/512) * (2 + head_dim) floats, rounded up to 256 bytes (nq = 1:
 * the same as attn_decode_workspace_bytes). Returns 0 for invalid arguments. */
size_t attn_verify_workspace_bytes(int num_seqs, int nq, int max_context_len,
                                   int n_q_heads, int head_dim);

/* attn_verify -- nq (1..8) new query rows per sequence against its paged INT8 K/V
 * (speculative / multi-token verify, small-batch decode).
 * [DOT4 README: the MTP verify step runs a few query rows and the next steps extend
 *  split-K decode to such small query batches; R4D "Row shape routing": verify rows go
 *  to a multi-row kernel that reads each K/V tile once for all rows, one row to the
 *  one-row kernel; causal rule of a chunk as in attn_prefill_chunk.]
 *
 *  Same two stages and the same 512-row partitions as attn_decode; each (sequence, KV
 *  head, partition) workgroup reads its K/V once for all 6 * nq query rows of the group.
 *  nq == 1 runs the attn_decode kernels (identical results). For nq >= 2 the weighted
 *  sum of V runs on the int8 matrix cores with each weight w / s_b (s_b = block max /
 *  127, aligned 64-key blocks) carried as three 7-bit digit planes, i.e. to 2^-15 of
 *  s_b, which keeps the fp32-class bound of attn_decode.
 *  q             bf16 [num_seqs][nq][n_q_heads][head_dim]; query i of sequence s sits
 *                at position ctx_s - nq + i and sees keys 0 .. ctx_s - nq + i (its own
 *                and the earlier new rows' K/V must already be written).
 *  context_lens  int32 [num_seqs], clamped like attn_decode's; a query row with no
 *                visible key (ctx_s < nq) produces zeros.
 *  out           fp32 [num_seqs][nq][n_q_heads][head_dim], fully overwritten.
 *  workspace     >= attn_verify_workspace_bytes(...) bytes.
 *  Other arguments as for attn_decode. nq outside 1..8 or num_seqs * nq > 65535
 *  returns I8A_EINVAL. */
int attn_verify(const uint16_t* q, int nq,
                const int8_t* k_cache, const int8_t* v_cache,
                const float* k_scale, const float* v_scale,
                const int32_t* block_table, int max_blocks_per_seq,
                const int32_t* context_lens, int num_seqs, int max_context_len,
                int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                float sm_scale, float* out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Keys per split-K partition that attn_decode_int8p uses when passed partition_rows = 0:
 * 512 when max_context_len <= 512 (one partition: the workgroup writes the output and no
 * merge stage runs); otherwise the largest of 512, 256, 128 for which num_seqs *
 * n_kv_heads * ceil(max_context_len / partition) reaches 64 workgroups, else 128
 * [R4D "The selection law": a power-of-two segment count from a workgroup-count target
 * over (KV heads x rows), with a floor on keys per segment; DCU §3.3: 256-token decode
 * partitions]. Returns 0 for invalid arguments. */
int attn_decode_partition_rows(int num_seqs, int max_context_len, int n_kv_heads);

/* Bytes of scratch attn_decode_int8p needs: num_seqs * nq * n_q_heads *
 * ceil(max_context_len / partition) * (2 + head_dim) floats, rounded up to 256 bytes,
 * with the partition resolved as attn_decode_int8p resolves it. 0 for invalid
 * arguments. */
size_t attn_decode_int8p_workspace_bytes(int num_seqs, int nq, int max_context_len,
                                         int n_q_heads, int n_kv_heads, int head_dim,
                                         int partition_rows);

/* attn_decode_int8p -- decode / verify with int8 softmax weights: the int8-P variant of
 * attn_verify (nq = 1: decode).
 * [DCU §3.3: the decode kernel's INT8 PV, the V scale folded into the weight, weights
 *  quantized per block with scale = block absmax / 127 and the block's int8 product
 *  scaled back by it; 256-token partitions; R4D "The selection law".]
 *
 *  As attn_verify, except: the weights p * sV of each query row and aligned 64-key
 *  block are carried as int8 codes rint(w / s_b), s_b = max_block(w) / 127, multiplied
 *  with the V codes on the int8 matrix cores (the same rule as attn_prefill_chunk; the
 *  denominator sums the unquantized weights), and the partition size is
 *  partition_rows keys (64, 128, 256 or 512; 0 = attn_decode_partition_rows). The
 *  codes of a key do not depend on the partition, so neither does the result beyond
 *  rounding.
 *  workspace     >= attn_decode_int8p_workspace_bytes(...) with the same partition_rows.
 *  Other arguments as for attn_verify; a partition_rows value outside the list returns
 *  I8A_EINVAL. */
int attn_decode_int8p(const uint16_t* q, int nq,
                      const int8_t* k_cache, const int8_t* v_cache,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int max_context_len,
                      int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                      int partition_rows, float sm_scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* attn_prefill_chunk -- n_new query tokens at the tail of one sequence, one pass.
 * [DCU §3.2: INT8 Q with history and current INT8 K/V in one online-softmax pass, INT8
 *  QK, INT8 PV; DCU §3.3 and §1.3: the V scale is folded into the softmax weight, the
 *  weight is quantized per block with scale = block absmax / 127 and the block's int8
 *  product is scaled back by it; QSA "Approach": one pass with an online softmax, no
 *  split and no merge; DOT4 recthist: prefix keys unmasked, causal check only on the
 *  tail.]
 *
 *  q             bf16 [n_new][n_q_heads][head_dim]; query t sits at position
 *                context_len - n_new + t.
 *  block_table   int32 [ceil(context_len/16)] pages of this sequence.
 *  context_len   keys 0..context_len-1, including the n_new new rows (already written).
 *  causal        1: query t sees keys 0 .. context_len-n_new+t; 0: all keys.
 *  Weights P are carried as int8 codes per (query row, aligned 64-key block) with
 *  scale = max_k(p_k * sV_k) / 127 and multiplied with the V codes on the int8 matrix
 *  cores; the softmax denominator sums the unquantized weights.
 *  out           fp32 [n_new][n_q_heads][head_dim], fully overwritten.
 *  num_pages * n_kv_heads * 16 must stay below 2^32 (scale index range), else
 *  I8A_EUNSUPPORTED.
 *  n_new == 0 is a no-op returning I8A_OK. */
int attn_prefill_chunk(const uint16_t* q, int n_new,
                       const int8_t* k_cache, const int8_t* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int context_len, int causal,
                       int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                       float sm_scale, float* out, void* stream);

/* attn_prefill_chunk_split -- attn_prefill_chunk with the keys cut into partitions for
 * short causal chunks, whose one-pass grid (one workgroup per 32 query tokens and KV
 * head) would leave most of the GPU idle.
 * [DCU §3.3: key partitions processed by separate workgroups, each keeping its own
 *  running max, sum and output, combined by a log-sum-exp merge as in the decode; DCU
 *  §3.2 and §1.3 for everything inside a partition.]
 *
 *  Arguments as for attn_prefill_chunk, plus:
 *  workspace     device scratch, 16-byte aligned, of at least
 *                attn_prefill_chunk_split_workspace_bytes(...) bytes; its contents on
 *                entry do not matter and are overwritten. Calls that share a workspace
 *                must be ordered (same stream).
 *  The route, for causal chunks:
 *  - n_new <= 8: the int8-P decode kernel (attn_decode_int8p with nq = n_new and its
 *    default partitions; bit for bit its result), which reads each K/V tile once for
 *    all rows of a KV head;
 *  - fewer than 128 (32-token query block, KV head) pairs: the chunk kernel over key
 *    partitions of whole 64-key blocks, about 256 workgroups, then a merge kernel (bf16
 *    queries are first quantized once, as q_quant does);
 *  - otherwise: the one pass of attn_prefill_chunk, bit for bit, with no workspace.
 *  Non-causal chunks always take the one pass. The int8 weight codes are per aligned
 *  64-key block in every route, so the routes differ only by rounding in the merge.
 *  workspace_bytes below the required size returns I8A_EWORKSPACE. */
size_t attn_prefill_chunk_split_workspace_bytes(int n_new, int context_len, int causal,
                                                int n_q_heads, int n_kv_heads, int head_dim);
int attn_prefill_chunk_split(const uint16_t* q, int n_new,
                             const int8_t* k_cache, const int8_t* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int context_len, int causal,
                             int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                             float sm_scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* *_q8 forms: the same computations with the query given as int8 codes and fp32 scales
 * (the format kv_produce writes: q_codes [rows][head_dim], q_scales [rows], rows laid
 * out as the bf16 q of the plain form) instead of bf16 rows that the call quantizes.
 * [DCU §2.2: the query is quantized once by the producer and reused by every
 *  partition.] Given q_codes/q_scales = q_quant(q), each returns bit for bit what the
 * plain form returns for q. q_scales NULL with work to do returns I8A_EINVAL. */
int attn_decode_q8(const int8_t* q_codes, const float* q_scales,
                   const int8_t* k_cache, const int8_t* v_cache,
                   const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks_per_seq,
                   const int32_t* context_lens, int num_seqs, int max_context_len,
                   int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                   float sm_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);
int attn_verify_q8(const int8_t* q_codes, const float* q_scales, int nq,
                   const int8_t* k_cache, const int8_t* v_cache,
                   const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks_per_seq,
                   const int32_t* context_lens, int num_seqs, int max_context_len,
                   int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                   float sm_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);
int attn_decode_int8p_q8(const int8_t* q_codes, const float* q_scales, int nq,
                         const int8_t* k_cache, const int8_t* v_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                         int partition_rows, float sm_scale, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);
int attn_prefill_chunk_q8(const int8_t* q_codes, const float* q_scales, int n_new,
                          const int8_t* k_cache, const int8_t* v_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, int context_len, int causal,
                          int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                          float sm_scale, float* out, void* stream);
int attn_prefill_chunk_split_q8(const int8_t* q_codes, const float* q_scales, int n_new,
                                const int8_t* k_cache, const int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int context_len, int causal,
                                int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                                float sm_scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* attn_decode_noalloc -- attn_decode for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, kernels and results as attn_decode (bit for bit),
 * without workspace/workspace_bytes: the split-K partial states go to a fixed device
 * array inside the library, attn_decode_noalloc_max_bytes() = 32 MiB per GPU (held by
 * each GPU the library runs on until the process ends; its address is looked up once
 * per device at the first call there). Nothing is allocated and nothing needs clearing
 * (every partial that is read was written by the same call).
 *  - A batch whose partials exceed the array (num_seqs * n_q_heads *
 *    ceil(max_context_len/512) * 1032 bytes > 32 MiB, e.g. more than 21 sequences at a
 *    32,768-token context with 24 query heads) returns I8A_EWORKSPACE: use attn_decode.
 *  - `stream` must belong to the current device (else I8A_EINVAL).
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 *    different streams, or from different threads) race and corrupt each other's
 *    partials. Order them on one stream. */
size_t attn_decode_noalloc_max_bytes(void);
int attn_decode_noalloc(const uint16_t* q,
                        const int8_t* k_cache, const int8_t* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int max_blocks_per_seq,
                        const int32_t* context_lens, int num_seqs, int max_context_len,
                        int num_pages, int n_q_heads, int n_kv_heads, int head_dim,
                        float sm_scale, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Opt-in validation of the paging metadata (host arrays).
 * The kernels do not check table entries or slots one by one: an entry outside the
 * pool reads page 0 (memory-safe, but a wrong page's keys enter the result) and a slot
 * outside the pool is skipped by the writers. A caller that wants such mistakes to be
 * errors runs these checks on HOST copies of the arrays before the call (they
 * synchronize with nothing and touch no device memory). [DCU §5.4: a fast kernel that
 * reads the wrong fragment gives plausible but wrong attention; checks that tie every
 * index to the data it names are what catches it.]
 * Both return I8A_OK, or I8A_EINVAL with int8attn_last_error() naming the first
 * offending entry. */

/* int8attn_check_block_table -- for every sequence s (context_lens NULL: one context of
 * max_context_len per sequence, as attn_prefill_chunk's single table row):
 *  - 0 <= context_lens[s] <= max_context_len and <= 16 * max_blocks_per_seq;
 *  - each of the ceil(ctx/16) table entries the sequence uses lies in [0, num_pages).
 * Entries past a sequence's context are not read by the kernels and not checked.
 *  block_table   int32 [num_seqs][max_blocks_per_seq], host memory.
 *  context_lens  int32 [num_seqs], host memory, or NULL. */
int int8attn_check_block_table(const int32_t* block_table, int num_seqs,
                               int max_blocks_per_seq, const int32_t* context_lens,
                               int max_context_len, int num_pages);

/* int8attn_check_slots -- slot_mapping int32 [n_tokens] (host memory) as kv_quant_write
 * and kv_produce take it: a slot >= num_pages * 16 is an error (the writers would skip
 * the token silently), and so is a slot named by two tokens (the writers leave it
 * unspecified which one wins). Negative slots are the documented "skip this token" and
 * pass. */
int int8attn_check_slots(const int32_t* slot_mapping, int n_tokens, int num_pages);

/* ---------------------------------------------------------------------------
 * Measurement kernels (they compute nothing of the attention method): the measured
 * ceilings the attention kernels are reported against, timed on the same GPU in the
 * same run. [R4D "Know your cache regime": a roofline fraction is read against a
 * ceiling measured in the same cache regime; "When the counters read zero, count the
 * ISA": a kernel with a known instruction count calibrates the counters.] */

/* int8attn_ceiling_stream_read -- reads `bytes` (a positive multiple of 16; src 16-byte
 * aligned) once with 16-byte loads, each of n_workgroups workgroups (256 threads) a
 * contiguous slab, and stores a fold of the bytes to sink[4 * n_workgroups] (uint32, one
 * word per wave) so that no load is elided. */
int int8attn_ceiling_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                 int n_workgroups, void* stream);

/* int8attn_ceiling_page_gather -- reads, for each of the first n_blocks entries of the
 * block table (device int32; entries outside [0, num_pages) read page 0), the 4 KB of K
 * codes and the 4 KB of V codes of every KV head and their 16 + 16 scales, from caches laid
 * out as for attn_decode: the decode's access pattern without its arithmetic. One
 * workgroup of 256 threads per (run of pages_per_workgroup pages, KV head); sink (device)
 * receives 4 words per workgroup: 4 * ceil(n_blocks / pages_per_workgroup) * n_kv_heads
 * uint32. Bytes read: n_blocks * (n_kv_heads * (2 * 4096 + 2 * 64) + 4).
 * Errors: I8A_EINVAL for a null pointer or a count <= 0 (nothing enqueued). */
int int8attn_ceiling_page_gather(const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, int n_blocks, int n_kv_heads,
                                 int num_pages, int pages_per_workgroup, uint32_t* sink,
                                 void* stream);

/* int8attn_ceiling_mfma_i8 -- n_workgroups workgroups of 8 waves (two per SIMD), each
 * wave issuing `iters` rounds of 8 independent v_mfma_i32_16x16x64_i8 on register
 * operands: int8attn_ceiling_mfma_i8_count(...) MFMA instructions of 16 x 16 x 64 MACs
 * (32,768 int8 ops each) in all. sink: int32 [n_workgroups] (written only in a case that
 * does not occur; it keeps the results live). */
int int8attn_ceiling_mfma_i8(int n_workgroups, int iters, int32_t* sink, void* stream);
int64_t int8attn_ceiling_mfma_i8_count(int n_workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* INT8ATTN_H */
