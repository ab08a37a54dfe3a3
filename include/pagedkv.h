/*
 * pagedkv.h -- PagedAttention decode and its KV-cache writer on AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * Sources, by page title (sections in brackets):
 *   [TGI] "TGI PagedAttention 深度解析：分块 KV Cache、前缀复用与连续批处理的内存优化"
 *   [L3]  "第三讲：PagedAttention与vLLM——让KV Cache不再'吃'显存"
 *   [CB]  "Continuous Batching与PagedAttention：LLM推理引擎的核心技术"
 *   [VN]  "怎么加快大模型推理 10分钟学懂VLLM内部原理" (vLLM notes)
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *     caller (the host block manager's calls take host pointers); the library
 *     allocates nothing.  Its only state is the block managers a caller
 *     creates and the per-GPU static scratch of
 *     paged_attention_decode_noalloc.
 *   - Work is enqueued on `stream` (0 = the null stream); no call synchronises
 *     and results are visible once the stream reaches that point.
 *   - Tensors are dense and row-major in the order their shape is written.
 *   - Argument errors are found on the host before anything is launched and
 *     are returned as a pkv_status; nothing is enqueued then.  A failed launch
 *     returns PKV_ERR_LAUNCH.  No call aborts or throws.
 *   - Index arrays that live on the device are preconditions, not checked on
 *     the host: see each call.  Kernels never read or write outside the
 *     buffers whose sizes the arguments describe, whatever the index values.
 *   - KV caches have the block layout [num_blocks, num_kv_heads, head_size,
 *     BLOCK_SIZE]: the BLOCK_SIZE tokens of one head of one block are
 *     contiguous, token fastest ([TGI] §4.2, physical layout of the `paged`
 *     backend; [L3] "注意力计算的'分页'实现").  K and V use the same layout.
 *   - BLOCK_SIZE (the `block_size` argument) is 8, 16 or 32 tokens.  16 is the
 *     `paged` backend's and vLLM's default ([TGI] §4.2; [VN] "KV Block") and
 *     the only size of the shared-prefix calls; the pages weigh smaller
 *     blocks (less waste, more table lookups) against larger ones ([TGI]
 *     §4.2, flashinfer uses 1).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                       */
  PKV_ERR_SHAPE = 2,       /* a size is negative, inconsistent or too large    */
  PKV_ERR_DTYPE = 3,       /* dtype combination not accepted                   */
  PKV_ERR_UNSUPPORTED = 4, /* head_size / block_size outside the built set     */
  PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  PKV_ERR_LAUNCH = 6,      /* the HIP runtime refused a kernel launch          */
  PKV_ERR_VALUE = 7,       /* a scalar argument is not finite / not positive   */
  PKV_ERR_ALIGNMENT = 8,   /* a device pointer lacks the required alignment    */
  PKV_ERR_NO_BLOCKS = 9,   /* block manager: the pool has no free block        */
  PKV_ERR_SEQUENCE = 10,   /* block manager: unknown or already used seq id    */
  PKV_ERR_SCRATCH = 11     /* needs more than PKV_NOALLOC_SCRATCH_BYTES        */
} pkv_status;

/* Element types.  PKV_FP8_E4M3 is the OCP 8-bit E4M3 "fn" format: bias 7,
 * 3 mantissa bits, no infinity, S.1111.111 = NaN, largest finite 448. */
typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3
} pkv_dtype;

/* The default (and matrix-core) block size, in tokens. */
#define PKV_BLOCK_SIZE 16
/* Partition length (tokens) used when partition_size = 0 is passed. */
#define PKV_DEFAULT_PARTITION_SIZE 2048
/* Partition lengths are multiples of this many tokens (the kernels' tile). */
#define PKV_PARTITION_QUANTUM 16

/* Human-readable name of a status code (static storage; never NULL). */
const char* pkv_status_string(pkv_status status);

/*
 * reshape_and_cache -- store each new token's key and value in the paged
 * caches at its slot ([TGI] §4.1, the KV write side: `paged_reshape_and_cache`
 * writes new keys/values into the block cache by slot index and has an FP8
 * quantised variant).
 *
 *   key, value      [num_tokens, num_kv_heads, head_size], src_dtype
 *   key_cache,      [num_blocks, num_kv_heads, head_size, block_size],
 *   value_cache       cache_dtype
 *   slot_mapping    [num_tokens] int64; slot = physical_block * block_size +
 *                   offset.  A slot < 0 or >= num_blocks * block_size writes
 *                   nothing.  Two tokens with the same slot: the result is
 *                   one of the two (precondition: slots are distinct).
 *
 * cache_dtype == src_dtype: the element bits are copied unchanged.
 * cache_dtype == PKV_FP8_E4M3 (src F16 or BF16): each element x is stored as
 * E4M3(x / k_scale) (v_scale for values), where x / scale is one correctly
 * rounded float32 division and E4M3() rounds to nearest, ties to even,
 * saturates finite and infinite magnitudes above 448 to 448, keeps the sign of
 * zero and sends NaN to 0x7F with the sign bit of the input.
 * k_scale and v_scale must be finite and > 0 on the FP8 path (ignored
 * otherwise).
 *
 * Sizes: num_tokens in [0, 2^30] (0 is a no-op), num_kv_heads >= 1,
 * head_size >= 1 and a multiple of 8, block_size in {8, 16, 32},
 * num_blocks >= 1, num_kv_heads * ceil(head_size * source element bytes /
 * 256) <= 65535.  key, value and both caches must be 16-byte aligned
 * (PKV_ERR_ALIGNMENT).
 *
 * Runs of a sequence's tokens in order (slots s, s+1, ..., as a prefill or a
 * bulk fill produces) are stored as whole pieces of block rows; tokens with
 * unrelated slots, such as one decode token per sequence, element by element.
 * The result is the same either way.
 */
pkv_status reshape_and_cache(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                             int32_t block_size, int32_t num_blocks, pkv_dtype src_dtype,
                             pkv_dtype cache_dtype, float k_scale, float v_scale,
                             hipStream_t stream);

/*
 * reshape_and_cache_strided -- reshape_and_cache for key / value rows that
 * are not packed, such as the key and value parts of a fused QKV projection
 * output: token t's row [num_kv_heads, head_size] starts at element
 * t * key_row_stride of `key` and t * value_row_stride of `value` (heads and
 * elements within a row stay contiguous).  Strides are in elements, at least
 * num_kv_heads * head_size (PKV_ERR_SHAPE) and multiples of 8
 * (PKV_ERR_ALIGNMENT).  Everything else as for reshape_and_cache, which is
 * this call with packed strides.
 */
pkv_status reshape_and_cache_strided(const void* key, const void* value, void* key_cache,
                                     void* value_cache, const int64_t* slot_mapping,
                                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                                     int32_t block_size, int32_t num_blocks,
                                     int64_t key_row_stride, int64_t value_row_stride,
                                     pkv_dtype src_dtype, pkv_dtype cache_dtype, float k_scale,
                                     float v_scale, hipStream_t stream);

/*
 * paged_attention_decode_workspace_bytes -- size of the float32 scratch that
 * paged_attention_decode needs for the given shapes: 0 when every sequence
 * fits in one partition (max_num_blocks_per_seq * block_size <=
 * partition_size), else num_seqs * num_heads * P * (head_size + 2) * 4 with
 * P = ceil(max_num_blocks_per_seq * block_size / partition_size).
 * partition_size 0 means PKV_DEFAULT_PARTITION_SIZE.  Returns 0 for invalid
 * sizes (the decode call then reports the error).
 */
size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                              int32_t head_size,
                                              int32_t max_num_blocks_per_seq,
                                              int32_t block_size, int32_t partition_size);

/*
 * paged_attention_decode -- one query token per sequence attends over its
 * paged KV cache ([L3] "注意力计算的'分页'实现": walk the logical blocks, read
 * each physical block through the block table, score the query against the
 * key block, softmax over all tokens, weighted sum of values; [TGI] §4.3: the
 * block table is handed to the kernel as `block_tables`).  Long sequences are
 * split into partitions of `partition_size` tokens that are processed in
 * parallel and merged exactly by their log-sum-exp ([TGI] §4.1, V2 with
 * 512-token partitions and a cross-partition reduction).
 *
 *   out            [num_seqs, num_heads, head_size], q_dtype (written)
 *   query          [num_seqs, num_heads, head_size], q_dtype
 *   key_cache,     [num_blocks, num_kv_heads, head_size, block_size], cache_dtype
 *   value_cache
 *   block_tables   [num_seqs, max_num_blocks_per_seq] int32: physical block
 *                  of each logical block.  Entries past a sequence's last
 *                  block are never read.
 *   context_lens   [num_seqs] int32: number of cached tokens L of each
 *                  sequence (the just-written token included).
 *
 * For sequence s and query head h, with kv head h / (num_heads / num_kv_heads)
 * and the L = context_lens[s] tokens t = 0..L-1 found at block
 * block_tables[s][t / block_size], offset t % block_size:
 *     out[s,h,:] = sum_t softmax_t(scale * k_scale * <q[s,h,:], K_t>) * v_scale * V_t
 * where K_t, V_t are the stored values (FP8 codes decoded exactly).  Tokens at
 * positions >= L in the last block never influence the result, whatever bits
 * they hold.  L = 0 gives out = 0.
 * Arithmetic: scores, exponentials, running maxima and sums in float32, one
 * rounding (nearest even) to q_dtype at the end.  On the vector kernel every
 * product and sum is float32.  On the matrix-core kernel (grouped heads, see
 * "Accepted" below) the query and the cached K/V enter the matrix products
 * as their stored 16-bit values (FP8 codes converted exactly), products are
 * exact and sums float32; each softmax weight p enters the P.V product as
 * two 16-bit terms hi + lo (hi = p rounded to q_dtype, lo = p - hi rounded
 * to q_dtype), which keeps about 16 significant bits of p for bf16 and 22
 * for f16 instead of float32's 24.
 *
 * Device preconditions (not checked): 0 <= ceil(L / block_size) <=
 * max_num_blocks_per_seq and the table entries a sequence uses lie in
 * [0, num_blocks).  Defensive behaviour if they do not: L is clamped to
 * max_num_blocks_per_seq * block_size and an entry outside [0, num_blocks)
 * contributes no token (nothing is read).
 *
 * Accepted: head_size in {32, 64, 80, 96, 112, 120, 128, 192, 256};
 * block_size in {8, 16, 32} (grouped heads with 2 <= H / Hk <= 16 and a
 * 16-bit query use the matrix cores, at every block size, for head sizes
 * that are multiples of 16 up to 128 and 192 and 256 with 16-bit caches, 64
 * and 128 with FP8 caches; every other case the vector kernel, which reads
 * each K/V tile once per query head); num_heads a multiple of
 * num_kv_heads; q_dtype in {F32, F16, BF16}; cache_dtype == q_dtype, or
 * cache_dtype == FP8_E4M3 with q_dtype F16 or BF16 (k_scale, v_scale finite
 * and > 0; they are ignored for non-FP8 caches); `scale` finite;
 * partition_size 0 (default) or a positive multiple of PKV_PARTITION_QUANTUM
 * (16); num_seqs >= 0.  PKV_ERR_SHAPE beyond these sizes:
 * max_num_blocks_per_seq <= 2^24; num_seqs * num_heads * P < 2^31 and
 * P * ceil(max_num_blocks_per_seq * block_size / 16) < 2^31, where
 * P = ceil(max_num_blocks_per_seq * block_size / partition_size) is the
 * number of partitions of the longest possible sequence.
 * `workspace` (device, >= paged_attention_decode_workspace_bytes(...) bytes,
 * 4-byte aligned) is needed only when that size is non-zero; the library
 * leaves its contents undefined.  Calls that share a workspace must not run
 * concurrently.
 */
pkv_status paged_attention_decode(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t block_size, int32_t max_num_blocks_per_seq,
                                  int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                  pkv_dtype cache_dtype, float k_scale, float v_scale,
                                  int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * partition results live in a scratch array that the library holds in device
 * memory, PKV_NOALLOC_SCRATCH_BYTES per GPU, from the first call on that GPU
 * until the process ends.  No call allocates: the first call on a GPU (with
 * that GPU current) only looks up the array's address there.
 *
 * Arguments, accepted values, results and errors as for paged_attention_decode
 * with no workspace arguments; the output is bit-identical to that call's.
 * When paged_attention_decode_workspace_bytes(...) for the same shapes exceeds
 * PKV_NOALLOC_SCRATCH_BYTES, the call returns PKV_ERR_SCRATCH and launches
 * nothing (other argument errors are reported first).  `stream` must belong
 * to the current device.  Every call on one GPU uses that GPU's one array:
 * calls that may overlap on one GPU (other streams, other host threads) race
 * and give undefined results; calls on one stream are ordered and safe.  The
 * array needs no clearing: each call writes every entry it reads.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_size, int32_t block_size,
                                          int32_t max_num_blocks_per_seq, int32_t num_blocks,
                                          float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                          float k_scale, float v_scale, int32_t partition_size,
                                          hipStream_t stream);

/*
 * paged_attention_decode_strided -- paged_attention_decode with query and out
 * rows that are not packed (a query taken from a fused QKV projection output,
 * an output written into a wider buffer): sequence s's query row
 * [num_heads, head_size] starts at element s * query_row_stride of `query`,
 * its output row at s * out_row_stride of `out`; heads and elements within a
 * row stay contiguous.  Strides are in elements, at least
 * num_heads * head_size (PKV_ERR_SHAPE: output rows must not overlap) and
 * multiples of 8 (PKV_ERR_ALIGNMENT); query and out must be 16-byte aligned
 * (PKV_ERR_ALIGNMENT).  Output elements between rows are not written.
 * Everything else as for paged_attention_decode.
 */
pkv_status paged_attention_decode_strided(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t max_num_blocks_per_seq, int32_t num_blocks, int64_t query_row_stride,
    int64_t out_row_stride, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_append -- one whole decode step in one call: each
 * sequence's new token is stored into the caches, then every query attends
 * over its sequence including that token.  Sequence s's new key and value
 * rows, key_new / value_new [num_seqs, num_kv_heads, head_size] in q_dtype
 * (device, read only), go to logical position context_lens[s] - 1, i.e. to
 * slot block_tables[s][(L-1) / block_size] * block_size + (L-1) % block_size
 * with L = context_lens[s], exactly as reshape_and_cache would store them
 * (the same bits: a copy, or E4M3 of x / k_scale and x / v_scale); the
 * result equals reshape_and_cache with those slots followed by
 * paged_attention_decode ([TGI] §4.1: the KV write, then paged attention;
 * [L3] "注意力计算的'分页'实现").  No token is stored for a sequence whose
 * context length is outside [1, max_num_blocks_per_seq * block_size] or
 * whose table entry for position L - 1 lies outside the pool.
 *
 * The wave that reads the block holding position L - 1 puts the new token
 * into that block's tile (in registers, or in its LDS stage for E4M3 caches
 * on the matrix cores), writes the whole tile back, and attends over it, so
 * the step touches only whole cache lines and needs one launch (plus the
 * merge) on either kernel.
 *
 * Arguments, accepted values, workspace and errors as for
 * paged_attention_decode; key_cache / value_cache are written.  Calls whose
 * caches overlap must not run concurrently.
 */
pkv_status paged_attention_decode_append(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_append_strided -- paged_attention_decode_append with
 * row strides, as paged_attention_decode_strided, for query and out, and for
 * the new rows: sequence s's key_new / value_new row [num_kv_heads,
 * head_size] starts at element s * key_new_row_stride / s *
 * value_new_row_stride (at least num_kv_heads * head_size, multiples of 8;
 * both pointers 16-byte aligned).  With q, k and v taken from one fused
 * projection output of row length (num_heads + 2 num_kv_heads) * head_size,
 * all three strides are that length.
 */
pkv_status paged_attention_decode_append_strided(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks,
    int64_t query_row_stride, int64_t key_new_row_stride, int64_t value_new_row_stride,
    int64_t out_row_stride, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_shared_prefix_workspace_bytes -- float32 scratch of
 * paged_attention_decode_shared_prefix: num_seqs * num_heads * (R + P) *
 * (head_size + 2) * 4 bytes with R = ceil(max_num_blocks_per_seq / 16) prefix
 * runs and P = ceil(max_num_blocks_per_seq * block_size / partition_size)
 * suffix partitions (partition_size 0 = PKV_DEFAULT_PARTITION_SIZE).  Returns
 * 0 for invalid sizes.
 */
size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                            int32_t head_size,
                                                            int32_t max_num_blocks_per_seq,
                                                            int32_t block_size,
                                                            int32_t partition_size);

/*
 * paged_attention_decode_shared_prefix -- the same result as
 * paged_attention_decode (up to float32 summation order) for a batch whose
 * sequences come in groups that share a common prefix of whole blocks, such
 * as the parallel samples of one prompt ([L3] "共享前缀": the samples' block
 * tables point at the same physical prefix blocks; [TGI] §4: prefix reuse).
 * With 2 <= num_heads / num_kv_heads (= g) <= 16, one launch on the matrix
 * cores: a work-group takes 16 query rows of one group and KV head (16 / g
 * members x their g heads), walks the prefix once for all of them and then
 * each member's own blocks, and writes the final output; the tiles of one
 * group read the prefix through one XCD's L2.  Other g: each prefix K/V tile
 * is read once per group and KV head for all of the group's query rows, each
 * sequence's remaining blocks as in paged_attention_decode, and the partial
 * results are merged by their log-sum-exp.
 *
 * Arguments as for paged_attention_decode, plus
 *   group_starts         [num_groups + 1] int32 (device): the sequences of
 *                        group k are group_starts[k] .. group_starts[k+1]-1
 *   group_prefix_blocks  [num_groups] int32 (device): the first
 *                        group_prefix_blocks[k] entries of every block table
 *                        in group k name the same physical blocks (read from
 *                        the group's first sequence), all of them full
 *   max_group_size       host bound on the number of sequences of a group
 *
 * Device preconditions (not checked): group_starts[0] = 0, non-decreasing,
 * group_starts[num_groups] = num_seqs; every group has at most
 * max_group_size sequences; the shared entries are equal across the group
 * and every member has context_len >= 16 * group_prefix_blocks[k].  A prefix
 * length outside [0, max_num_blocks_per_seq] is clamped to it.  When a
 * precondition fails the output of the affected sequences is unspecified;
 * nothing outside the described buffers is read or written.
 *
 * Accepted: as paged_attention_decode, except block_size 16 and head_size
 * 64 or 128 only (PKV_ERR_UNSUPPORTED otherwise) and q_dtype F16 or BF16 only (PKV_ERR_DTYPE
 * for F32); num_groups in [1, num_seqs] and max_group_size in [1, num_seqs]
 * when num_seqs > 0.  The workspace (>= the size above) is needed only when
 * g is 1 or above 16; with 2 <= g <= 16 it may be NULL and is not touched.
 */
pkv_status paged_attention_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_shared_prefix_append -- one decode step of a
 * shared-prefix batch in one call: each sequence's new token is stored into
 * the caches, then every query attends over its sequence including that
 * token.  key_new / value_new [num_seqs, num_kv_heads, head_size] (q_dtype,
 * read only) go to logical position context_lens[s] - 1 exactly as in
 * paged_attention_decode_append (a copy, or E4M3 of x / k_scale and
 * x / v_scale), and the output is that of
 * paged_attention_decode_shared_prefix over the updated caches ([TGI] §4.1:
 * the KV write, then paged attention; [L3] "共享前缀": new tokens go to each
 * sample's own blocks, never to the shared ones).  No token is stored for a
 * sequence whose position L - 1 lies inside its group's shared prefix (the
 * shared blocks are never written), whose context length is outside
 * [1, max_num_blocks_per_seq * block_size], or whose table entry for L - 1 lies
 * outside the pool.  The wave that reads the block holding L - 1 stores the
 * whole tile with the token in place, so the step touches only whole cache
 * lines.  Arguments and errors as for paged_attention_decode_shared_prefix,
 * which must run on the matrix cores: 2 <= num_heads / num_kv_heads <= 16
 * (PKV_ERR_UNSUPPORTED otherwise); the workspace is not used.
 */
pkv_status paged_attention_decode_shared_prefix_append(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* group_prefix_blocks, int32_t num_groups,
    int32_t max_group_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_kv_gather -- the logical KV of one sequence, read through its block
 * table: k_out[t, h, d] = key_cache[table[t / BS], h, d, t % BS] for t < L
 * (BS = block_size, 8, 16 or 32)
 * (same for V), bits copied unchanged ([L3] "SVG框架图": logical blocks map to
 * scattered physical blocks through the table).  A check of the block
 * indexing; not on the decode path.
 *
 *   k_out, v_out       [L, num_kv_heads, head_size], cache_dtype (written)
 *   block_table_row    [ceil(L / BS)] int32, entries in [0, num_blocks);
 *                      an entry outside that range yields zero bits.
 */
pkv_status paged_kv_gather(void* k_out, void* v_out, const void* key_cache,
                           const void* value_cache, const int32_t* block_table_row,
                           int32_t context_len, int32_t num_kv_heads, int32_t head_size,
                           int32_t block_size, int32_t num_blocks, pkv_dtype cache_dtype,
                           hipStream_t stream);

/*
 * copy_blocks -- the copy step of copy-on-write: for each (src, dst) pair,
 * physical block dst of every layer's key and value cache becomes a bitwise
 * copy of block src ([VN] "Sharing KV Cache": appending to a block that
 * another sequence still references first gives the appending sequence a new
 * block holding a copy; [L3] "共享前缀").  Every KV head and all block_size
 * token slots of the block are copied; nothing else is written.
 *
 *   key_caches,     HOST arrays of num_layers DEVICE pointers, each to a cache
 *   value_caches      [num_blocks, num_kv_heads, head_size, block_size] of
 *                     cache_dtype, 16-byte aligned.  The arrays are read
 *                     during the call only.
 *   block_mapping   [num_pairs, 2] int64 (device): (src, dst) physical ids.
 *                   A pair with either id outside [0, num_blocks) is skipped.
 *
 * Device precondition (not checked): the dst ids are distinct and no dst is
 * also the src of another pair (a copy-on-write destination is a freshly
 * allocated block); otherwise which bytes land is unspecified.
 * Sizes: num_layers >= 0 and num_pairs >= 0 (either 0: a no-op),
 * num_kv_heads >= 1, head_size >= 1, block_size in {8, 16, 32},
 * num_blocks >= 1.  Pointers that are not 16-byte aligned: PKV_ERR_ALIGNMENT.
 */
pkv_status copy_blocks(void* const* key_caches, void* const* value_caches, int32_t num_layers,
                       const int64_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t num_blocks,
                       pkv_dtype cache_dtype, hipStream_t stream);

/*
 * Host block manager -- the bookkeeping half of paged KV caching, on the
 * host ([L3] "核心数据结构：Block Table": a sequence holds
 * ceil(tokens / block_size) physical blocks listed in its block table;
 * [CB] §3.2: allocate, fork (the child shares the parent's blocks and their
 * reference counts go up), free (a block returns to the pool when its count
 * reaches zero); [VN] "Sharing KV Cache", [L3] "共享前缀": a sequence that
 * appends into a block another sequence still references is first moved to
 * a copy of it -- copy-on-write).
 *
 * The manager never touches device memory.  One decode step:
 *   pkv_bm_append_tokens  -> slots of the new tokens + copy-on-write pairs
 *   copy_blocks(pairs), reshape_and_cache(slots)
 *   pkv_bm_build_block_tables -> block_tables / context_lens for the decode
 * Free blocks are handed out lowest id first.  A call that fails changes
 * nothing, except that pkv_bm_append_tokens keeps the appends made before
 * the sequence that failed (*num_done says how many).
 *
 * Prefix cache ([TGI] §5.2-5.3: a trie from prompt tokens to blocks, with a
 * reference count and last access time per node; [VN] "Prefix Caching"):
 * sequences added with their prompt's token ids (pkv_bm_add_sequence_cached)
 * leave their full prompt blocks in a cache when they are freed; a later
 * prompt whose leading full blocks hold the same token ids shares those
 * blocks instead of taking new ones (their KV is already written).  Cached
 * blocks that no sequence references are reclaimed only when the free list
 * is empty, least recently used first (ties: lowest id), leaves of the
 * trie before their parents; every allocation (add, append) may do so.  A manager is not
 * thread-safe: calls on one manager must not overlap.  All pointers of these
 * calls are HOST pointers.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks blocks of block_size tokens (both >= 1). */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);
/* Blocks on the free list (not counting reclaimable cached blocks). */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
/* Blocks held by the prefix cache, referenced by sequences or not. */
int32_t pkv_bm_num_cached_blocks(const pkv_block_manager* bm);

/* New sequence holding num_tokens tokens (>= 0), e.g. a prompt about to be
 * written: ceil(num_tokens / block_size) fresh blocks.  PKV_ERR_SEQUENCE if
 * seq_id is in use, PKV_ERR_NO_BLOCKS if the pool is short. */
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens);

/* New sequence for a prompt given by its token ids tokens[0..num_tokens):
 * its leading full blocks, as far as their token ids match cached blocks
 * block by block from the first and within the first num_tokens - 1 tokens
 * (the last prompt token is always left to compute), are the cached blocks
 * (reference counts up, access time now); the rest are new blocks.
 * *cached_tokens = matched blocks * block_size: the leading tokens whose KV
 * is already in the cache (write only tokens from there on).  When the
 * sequence (or a fork of it) is freed, its full prompt blocks enter the
 * cache.  Errors as for pkv_bm_add_sequence; PKV_ERR_NULL for a null
 * tokens (num_tokens > 0) or cached_tokens. */
pkv_status pkv_bm_add_sequence_cached(pkv_block_manager* bm, int64_t seq_id,
                                      const int64_t* tokens, int64_t num_tokens,
                                      int64_t* cached_tokens);

/* child_id shares all of parent_id's blocks and its token count. */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Drops the sequence; blocks no other sequence references become free, or
 * stay in the prefix cache (a sequence added with its prompt's tokens first
 * enters its full prompt blocks there). */
pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* One new token for each of seq_ids[0..n): slots[i] (block * block_size +
 * offset) is where reshape_and_cache must write it.  A full last block (or
 * none) gets a fresh block; a partially filled last block that another
 * sequence references is copied first: the pair (old, new) is appended to
 * copy_pairs ([n][2], room for n pairs) and *num_copies counts them.  The
 * copies must run (copy_blocks) before the new tokens are written.  Stops at
 * the first sequence that is unknown (PKV_ERR_SEQUENCE) or needs a block the
 * pool does not have (PKV_ERR_NO_BLOCKS); *num_done tokens were appended. */
pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                int64_t* slots, int64_t* copy_pairs, int32_t* num_copies,
                                int32_t* num_done);

/* Block table (capacity entries available; PKV_ERR_SHAPE if too few) and
 * token count of one sequence. */
pkv_status pkv_bm_get_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table,
                                  int32_t capacity, int32_t* num_blocks, int64_t* num_tokens);

/* Slots of tokens first .. first + count - 1 of a sequence (e.g. to write a
 * prompt with reshape_and_cache); PKV_ERR_VALUE outside [0, tokens). */
pkv_status pkv_bm_token_slots(const pkv_block_manager* bm, int64_t seq_id, int64_t first,
                              int32_t count, int64_t* slots);

/* block_tables [n][max_blocks_per_seq] (padded with -1) and context_lens [n]
 * of seq_ids, in the layout paged_attention_decode takes.  PKV_ERR_SHAPE if a
 * sequence has more blocks than max_blocks_per_seq; nothing is written then. */
pkv_status pkv_bm_build_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids,
                                     int32_t n, int32_t max_blocks_per_seq,
                                     int32_t* block_tables, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
