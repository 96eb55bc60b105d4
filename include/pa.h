/*
 * pa.h — C ABI of libpa: paged-KV attention for MI355X (gfx950).
 *
 * Sources (page title, section):
 *   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》
 *   [VF] 《大模型推理：vLLM大模型推理框架（附下载）》
 *   [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》
 *   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》
 *
 * The KV cache is cut into fixed-size blocks of block_size tokens that live
 * anywhere in a pre-allocated pool; a per-sequence block table maps logical
 * block j of a sequence to a physical block ([VE] §3.1; [VI] §2.1).  Token
 * position pos lives in logical block pos / block_size at offset
 * pos % block_size ([VF] §1.1).
 *
 * Storage layout (the ABI; K and V are separate regions of each block,
 * [VI] §2.1):
 *   k_cache  [num_blocks][num_kv_heads][block_size][head_dim]   (token-major)
 *   v_cache  [num_blocks][num_kv_heads][head_dim][block_size]   (dim-major)
 *   Within a block and head, K rows are contiguous per token, V rows are
 *   contiguous per dimension (tokens innermost).
 *
 * Conventions for every device call:
 *   - All pointers are device pointers owned by the caller, 16-byte aligned.
 *     The library never allocates or frees device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Nothing synchronises the host.
 *   - A non-OK status means nothing was enqueued; pa_last_error() gives text.
 *     Faults that happen later on the device surface as HIP errors at the
 *     caller's next synchronisation.
 *   - Supported: head_dim in {64, 128}; block_size in {16, 32, 64, 128};
 *     num_q_heads % num_kv_heads == 0 and group size (Hq/Hkv) <= 16;
 *     dtype bf16 for every call, and fp32 for cache write, block copy and
 *     decode.  Other shapes return PA_ERR_UNSUPPORTED.
 *
 * Host allocator calls touch host memory only and are not thread-safe: one
 * scheduler thread owns an allocator.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* bad pointer, size or value; nothing done      */
    PA_ERR_OUT_OF_BLOCKS = 2, /* the pool cannot supply the blocks asked for   */
    PA_ERR_NOT_FOUND = 3,     /* unknown sequence id                           */
    PA_ERR_UNSUPPORTED = 4,   /* valid arguments with no kernel for them       */
    PA_ERR_DEVICE = 5         /* the HIP runtime refused a launch              */
} pa_status;

typedef enum {
    PA_DTYPE_F32 = 0,
    PA_DTYPE_BF16 = 1,
    /* OCP 8-bit float, E4M3 variant (bias 7, no infinities, NaN = S.1111.111,
     * largest magnitude 448); a cache of such codes has one scale per K or V
     * cache: value = code * scale.  Accepted by the fp8 calls and by the
     * block copies. */
    PA_DTYPE_FP8_E4M3 = 2
} pa_dtype;

/* Text of the last non-OK status returned on this thread ("" if none). */
const char *pa_last_error(void);

/* ------------------------------------------------------------------------ */
/* Device calls                                                               */
/* ------------------------------------------------------------------------ */

/* Cache write: a newly generated token needs only its K/V written into the
 * slot its block table assigns ([VE] §3.1).
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim], dtype.
 *   slot_mapping   [num_tokens] int64 device: slot = block * block_size + offset.
 *                  A negative slot, or one >= num_blocks * block_size, is
 *                  skipped (nothing written for that token).  Slots must be
 *                  distinct: if two tokens name one slot, which of them
 *                  lands is unspecified.
 * Bit-exact copy: no conversion, no arithmetic on the values. */
pa_status pa_cache_write(const void *k_new, const void *v_new,
                         void *k_cache, void *v_cache,
                         const int64_t *slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, void *stream);

/* Copy-on-write copy: before a sequence writes into a block it shares, that
 * whole block (K and V, all heads, all rows) is copied to a private block
 * ([VI] §2.1, COW for shared prefixes).
 *   src_dst  [num_pairs][2] int32 device (src, dst).  Pairs with an id
 *            outside [0, num_blocks) are skipped.  dst blocks must be
 *            distinct from every src and from each other.
 * Must be enqueued before the cache write that targets dst. */
pa_status pa_copy_blocks(void *k_cache, void *v_cache,
                         const int32_t *src_dst, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, void *stream);

/* Reference read stream, for measurement only (no part of attention): reads
 * the `bytes` bytes at `src` once, in 16-byte non-temporal loads spread over
 * a fixed grid, the plain streaming-read rate beside which the decode
 * kernels' HBM rates are reported.  The loads are folded with XOR into one
 * 32-bit word per workgroup, written to sink[0 .. PA_READ_STREAM_SINK_WORDS);
 * the XOR of those words equals the XOR of all 32-bit words of the buffer.
 *   src    device, 16-byte aligned, not written
 *   bytes  a multiple of 16 (0 allowed: the sink words become 0)
 *   sink   device, PA_READ_STREAM_SINK_WORDS words, 4-byte aligned, written
 * Asynchronous on `stream`.  PA_ERR_INVALID_ARG on NULL or misaligned
 * pointers or a size that is not a multiple of 16. */
#define PA_READ_STREAM_SINK_WORDS 32768
pa_status pa_read_stream(const void *src, size_t bytes, uint32_t *sink,
                         void *stream);

/* Partition size (tokens) pa_decode uses when called with partition_size 0:
 * sequences longer than one partition are split and their parts processed
 * independently, then merged ([VF] §1.1: segments of a sequence can be
 * processed independently).  Always a multiple of 32 and of block_size. */
int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t block_size, int32_t max_context_len);

/* Partition size for pa_decode from host copies of the batch's context
 * lengths ([VF] §1.1: any split into independent segments; [VE] §3.3: decode
 * is bound by memory bandwidth, so the split should keep every wave slot
 * streaming).  With 257 .. 1024 (sequence, kv head) pairs the batch runs in
 * about one round of the chip's 2048 wave slots, and the size is 1.2 times
 * the average tokens per slot (the valid lengths' sum times num_kv_heads /
 * 2048), rounded to a multiple of max(128, block_size), at most 4096;
 * otherwise it is pa_decode_default_partition's.  0 on invalid arguments
 * (pa_last_error says which). */
int32_t pa_decode_partition_for_lengths(const int32_t *context_lens, int32_t num_seqs,
                                        int32_t num_kv_heads, int32_t block_size,
                                        int32_t max_context_len);

/* Bytes of device workspace pa_decode needs for the split-K partials with
 * these sizes (partition_size 0 = the default above).  0 when no sequence
 * can span more than one partition; (size_t)-1 on invalid sizes. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len,
                                int32_t partition_size);

/* Paged decode attention ([VE] §3.1 block-table walk; [VE] §3.3 scaling,
 * softmax, weighted sum):
 *   out[s][h][:] = softmax(scale * q[s][h] . K_s^T) V_s
 * where K_s, V_s are the first context_lens[s] tokens of sequence s read
 * through block_tables[s], and query head h reads kv head h / (Hq / Hkv).
 *   out           [num_seqs][num_q_heads][head_dim] fp32.
 *   q             [num_seqs][num_q_heads][head_dim], dtype.
 *   block_tables  [num_seqs][block_table_stride] int32 device.
 *   context_lens  [num_seqs] int32 device; the count includes the token
 *                 being decoded (its K/V already written).  0 gives a zero
 *                 row.  A length < 0, > max_context_len or needing more
 *                 than block_table_stride blocks, and a table entry outside
 *                 [0, num_blocks), make that row NaN; nothing is read out of
 *                 range.
 *   max_context_len  host-known upper bound of context_lens (sizes the grid).
 *   partition_size   tokens per split-K partition: 0 = default, else a
 *                    multiple of 32 and of block_size.
 *   workspace     device scratch of at least pa_decode_workspace_size(...)
 *                 bytes (may be NULL when that is 0).  Its contents on entry
 *                 are irrelevant.  Calls sharing one workspace must be
 *                 ordered on one stream.
 * fp32 output; accumulation in fp32. */
pa_status pa_decode(float *out, const void *q,
                    const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t block_table_stride,
                    const int32_t *context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    float scale, int32_t max_context_len,
                    int32_t partition_size, void *workspace,
                    size_t workspace_bytes, pa_dtype dtype, void *stream);

/* Flags of pa_decode_ex. */
enum {
    /* K/V blocks of this batch are read by more than one sequence (shared
     * prompt prefixes, parallel sampling: [VE] §3.1 KV sharing).  The
     * kernel then loads K/V with the normal cache policy so that sharers
     * running at the same time hit in cache; without the flag K/V are
     * streamed with nontemporal loads, which is faster when every block is
     * read once.  Results are bit-identical either way. */
    PA_DECODE_KV_REUSE = 1,
    /* bf16 caches: run the vector-ALU kernel (per-token dot products with
     * quad exchanges, 16-token steps) instead of the matrix-core one.  A
     * second, independent device implementation of the same definition,
     * kept for comparison and cross-checks; it is slower on this chip.
     * Results agree with the default within fp32 rounding (not bit for
     * bit).  Not available to the grouped and fp8 calls (INVALID_ARG). */
    PA_DECODE_VALU = 2
};

/* pa_decode with flags (a bitwise OR of the PA_DECODE_* values; 0 gives
 * pa_decode).  Unknown flag bits are INVALID_ARG. */
pa_status pa_decode_ex(float *out, const void *q,
                       const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, int32_t block_table_stride,
                       const int32_t *context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       float scale, int32_t max_context_len,
                       int32_t partition_size, void *workspace,
                       size_t workspace_bytes, pa_dtype dtype, uint32_t flags,
                       void *stream);

/* Bytes of the device scratch pa_decode_noalloc keeps per GPU. */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* pa_decode_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops or
 * harnesses that forbid allocation).  The split-K partials go to a device
 * array of PA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from load until the process ends; the call allocates
 * nothing.  A batch whose partials need more (pa_decode_workspace_size) is
 * UNSUPPORTED, and nothing is enqueued.  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, or
 * different host threads without ordering) race on it and must be ordered
 * by the caller.  Nothing in it needs clearing between calls.  Arguments,
 * flags, results and errors otherwise as pa_decode_ex. */
pa_status pa_decode_noalloc(float *out, const void *q,
                            const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, int32_t block_table_stride,
                            const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            float scale, int32_t max_context_len,
                            int32_t partition_size, pa_dtype dtype, uint32_t flags,
                            void *stream);

/* Chunked prefill: one iteration may carry new prompt chunks beside decode
 * rows ([VI] §1, continuous batching mixes requests in different phases).
 * Request r owns query rows cu_q_lens[r] .. cu_q_lens[r+1]-1; its context
 * holds context_lens[r] tokens whose last qlen_r are the chunk itself (their
 * K/V already written with pa_cache_write).  Row i of request r sits at
 * position p = context_lens[r] - qlen_r + i and attends to keys 0..p.
 *   out         [total_q_tokens][num_q_heads][head_dim] fp32.
 *   q           [total_q_tokens][num_q_heads][head_dim] bf16.
 *   cu_q_lens   [num_reqs + 1] int32 device, non-decreasing, cu_q_lens[0]=0,
 *               cu_q_lens[num_reqs] = total_q_tokens.
 *   context_lens [num_reqs] int32 device.
 *   max_q_len, max_context_len  host-known bounds (size the grid).
 * A request whose qlen exceeds its context, exceeds max_q_len, or whose
 * context exceeds max_context_len or its table, or a table entry outside
 * [0, num_blocks), gets NaN rows; nothing is read out of range.  bf16 only.
 * Precision: Q K^T in bf16 with fp32 accumulation; the softmax weights
 * enter P V rounded to fp16 (relative error 2^-11) against V converted to
 * fp16, which is exact for a V element of magnitude in [2^-14, 2^16) and
 * loses bits below 2^-24 for a smaller one (an absolute error under 3e-8
 * per element).  A V element of 2^16 or more, infinite or NaN turns the
 * workgroup's fp32 sums non-finite, and the workgroup recomputes its rows
 * with V in bf16 and the weights split into bf16 high and low parts (error
 * near 2^-16).
 * Non-finite V: an output element (row, head, dim) is NaN exactly when a
 * key its row sees (keys 0..p) holds an infinite or NaN V element in that
 * dim; the definition gives an infinity or a NaN there.  No other output
 * element is affected: a key past a row's position never reaches it. */
pa_status pa_prefill_chunk(float *out, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *block_tables,
                           int32_t block_table_stride,
                           const int32_t *cu_q_lens,
                           const int32_t *context_lens, int32_t num_reqs,
                           int32_t total_q_tokens, int32_t max_q_len,
                           int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           float scale, pa_dtype dtype, void *stream);

/* Paged decode of a batch whose sequences share leading blocks (parallel
 * sampling, forked prompts: [VE] §3.1 KV sharing; [VI] §1 shared prompt
 * prefixes).  The result of pa_decode_ex, but the blocks every member of a
 * group holds in common are read once for the whole group: one wave
 * computes a piece of them for up to 16 / (num_q_heads / num_kv_heads)
 * members at once.
 * Split ([VF] §1.1: segments are processed independently, then merged).
 * Group g's shared region is its first group_shared[g] blocks, T tokens.  A
 * member whose context (L tokens) extends past it, 0 < T < L, is split at
 * T: the region in partitions [i ps, min((i + 1) ps, T)), computed for the
 * group, then the member's own tokens in partitions [T + j ps, min(T + (j +
 * 1) ps, L)).  No member reads a shared block itself, whatever T is.  Other
 * sequences are split as in pa_decode_ex.  With T a multiple of the
 * partition size ps the partitions are pa_decode_ex's and so is the result,
 * bit for bit; otherwise the merge adds the same terms split at other
 * points, and the result differs from pa_decode_ex's by that rounding.
 *   group_offsets  [num_groups + 1] int32 device: group g is the run of
 *                  sequences group_offsets[g] .. group_offsets[g + 1] - 1;
 *                  the first is its leader, whose table is read.
 *   seq_group      [num_seqs] int32 device: the group of each sequence, or
 *                  -1.  A sequence is in group g only if seq_group[s] == g
 *                  and s lies in g's run (and among its first
 *                  max_group_size members); otherwise it is decoded alone.
 *   group_shared   [num_groups] int32 device: leading block-table entries
 *                  (blocks) that every member holds equal to the leader's
 *                  (pa_decode_groups derives them).  A member whose own
 *                  entries differ from the leader's over a shared partition
 *                  gets a NaN row.
 *   num_groups     >= 0 (0: pa_decode_ex).
 *   max_group_size host bound of the group sizes (>= 1 when num_groups > 0).
 *   partition_size 0: pa_decode_default_partition's size; the size
 *                  pa_decode_grouped_partition picks from host copies of the
 *                  group arrays suits a grouped batch better (fewer, longer
 *                  partitions when the groups carry most of the tokens).
 *   workspace      at least pa_decode_grouped_workspace_size(...) bytes.
 * dtype must be BF16 (the fp32 path has no grouped kernel: UNSUPPORTED).
 * Flags and errors as pa_decode_ex. */
pa_status pa_decode_grouped(float *out, const void *q,
                            const void *k_cache, const void *v_cache,
                            const int32_t *block_tables,
                            int32_t block_table_stride,
                            const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale,
                            int32_t max_context_len, int32_t partition_size,
                            const int32_t *group_offsets,
                            const int32_t *seq_group,
                            const int32_t *group_shared, int32_t num_groups,
                            int32_t max_group_size, void *workspace,
                            size_t workspace_bytes, pa_dtype dtype,
                            uint32_t flags, void *stream);

/* Bytes of device workspace pa_decode_grouped (and pa_decode_grouped_fp8)
 * need: the partials of ceil(max_context_len / partition_size) + 1
 * partitions per (sequence, query head) -- one more than pa_decode_ex's, for
 * a member split at its group's shared region -- so never 0 for a batch;
 * (size_t)-1 on invalid sizes. */
size_t pa_decode_grouped_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len,
                                        int32_t partition_size);

/* Partition size for pa_decode_grouped on this batch, from host copies of
 * its lengths and group arrays (the arguments of pa_decode_grouped).  The
 * grouped grid holds a wave per (kv head, group chunk, shared partition)
 * and per (kv head, sequence, own partition), each of which pays a start-up
 * before it streams ([VE] §3.3: decode is bound by memory bandwidth).
 * Starting from pa_decode_default_partition, the size doubles while that
 * grid keeps at least 2048 waves, up to 4096 tokens; with no group sharing
 * anything it is pa_decode_default_partition.  Always a multiple of 32 and
 * of block_size.  0 on invalid arguments (pa_last_error says which). */
int32_t pa_decode_grouped_partition(const int32_t *context_lens,
                                    const int32_t *group_offsets,
                                    const int32_t *seq_group,
                                    const int32_t *group_shared, int32_t num_seqs,
                                    int32_t num_groups, int32_t max_group_size,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t block_size, int32_t max_context_len);

/* Group arrays for pa_decode_grouped from host block tables ([VE] §3.1:
 * sequences forked from one prompt hold its physical blocks).  Host memory
 * only; nothing is enqueued.
 *   block_tables   [num_seqs][block_table_stride] int32 host.
 *   context_lens   [num_seqs] int32 host, >= 0.
 *   seq_group      [num_seqs] int32 host: the caller's grouping, a group id
 *                  in [0, num_groups) or -1 (decoded alone).  Each group's
 *                  members are consecutive, and group ids first appear in
 *                  increasing order from 0, each group non-empty.
 *   group_offsets  [num_groups + 1] out: group g's run starts at
 *                  group_offsets[g] (its first member, the leader) and ends
 *                  where the next group's starts (the last at its last
 *                  member + 1).
 *   group_shared   [num_groups] out: the leading table entries every member
 *                  holds equal to the leader's, counted over the blocks that
 *                  every member's context fills completely.
 *   max_group_size out: the largest member count (0 with no group).
 * INVALID_ARG (nothing written) for a malformed grouping or a negative
 * length. */
pa_status pa_decode_groups(const int32_t *block_tables, int32_t block_table_stride,
                           const int32_t *context_lens, const int32_t *seq_group,
                           int32_t num_seqs, int32_t block_size, int32_t num_groups,
                           int32_t *group_offsets, int32_t *group_shared,
                           int32_t *max_group_size);

/* ------------------------------------------------------------------------ */
/* fp8 KV cache                                                               */
/* ------------------------------------------------------------------------ */
/* The pages name no fp8 format or scale convention; this library's: K and V
 * caches of OCP E4M3 codes (PA_DTYPE_FP8_E4M3, 1 byte per element, the same
 * block layouts as above), each with one fp32 scale: value = code * scale.
 * Halving the bytes per token halves what decode must stream from HBM
 * ([VE] §1 / §3.3: decode is bound by memory bandwidth). */

/* Quantizing cache write: element x of a new row is stored as the nearest
 * E4M3 code of x / scale (binary32 division, correctly rounded; ties to the
 * even code; magnitudes past 448, infinities included, saturate to +-448; a
 * NaN input stores 0x7F).  k_new / v_new [num_tokens][Hkv][D] in in_dtype
 * (F32 or BF16); slots, skipping and errors as pa_cache_write; scales finite
 * and > 0. */
pa_status pa_cache_write_fp8(const void *k_new, const void *v_new, pa_dtype in_dtype,
                             void *k_cache, void *v_cache, const int64_t *slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, float k_scale,
                             float v_scale, void *stream);

/* pa_decode_ex over fp8 caches: q is bf16 [S][Hq][D]; a K code's value is
 * code * k_scale and a V code's code * v_scale.  Codes are widened to bf16
 * exactly; the scales enter in fp32 (k_scale with the softmax scale, v_scale
 * on the output).  Every other argument, the workspace and the error
 * behaviour are those of pa_decode_ex. */
pa_status pa_decode_fp8(float *out, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int32_t block_table_stride,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, float scale, float k_scale, float v_scale,
                        int32_t max_context_len, int32_t partition_size, void *workspace,
                        size_t workspace_bytes, uint32_t flags, void *stream);

/* pa_decode_grouped over fp8 (E4M3) caches with their scales, as
 * pa_decode_fp8; group arguments and workspace as pa_decode_grouped. */
pa_status pa_decode_grouped_fp8(float *out, const void *q,
                                const void *k_cache, const void *v_cache,
                                const int32_t *block_tables,
                                int32_t block_table_stride,
                                const int32_t *context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, float scale, float k_scale,
                                float v_scale, int32_t max_context_len,
                                int32_t partition_size,
                                const int32_t *group_offsets,
                                const int32_t *seq_group,
                                const int32_t *group_shared,
                                int32_t num_groups, int32_t max_group_size,
                                void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream);

/* pa_prefill_chunk over fp8 caches: q is bf16; K codes are widened to bf16
 * and V codes to fp16 exactly when staged, k_scale joins the softmax scale
 * and v_scale the output, in fp32.  A V NaN code (S.1111.111) is treated as
 * a non-finite V element is by pa_prefill_chunk.  Everything else as
 * pa_prefill_chunk. */
pa_status pa_prefill_chunk_fp8(float *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               int32_t block_table_stride, const int32_t *cu_q_lens,
                               const int32_t *context_lens, int32_t num_reqs,
                               int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, float scale, float k_scale,
                               float v_scale, void *stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator                                                       */
/* ------------------------------------------------------------------------ */
/* A fixed pool of num_blocks blocks with a per-block reference count
 * (0 = free, 1 = owned, >1 = shared; the per-block state of [VI] §2.1),
 * a free list used as a stack ([VI] §2.1 allocation pops the free list),
 * and one block table per sequence kept in host memory ([VI] §2.1).
 * A sequence of n tokens holds ceil(n / block_size) blocks ([NV] code
 * example 1); asking for more than the pool has is an error that changes
 * nothing ([NV] code example 1). */

typedef struct pa_allocator pa_allocator;

typedef struct {
    int32_t num_blocks;
    int32_t num_free;
    int32_t num_used;
    int32_t num_shared; /* blocks with refcount > 1 */
    int64_t cow_copies; /* copy-on-write pairs handed out so far */
} pa_allocator_stats_t;

/* free_order: NULL, or a permutation of 0..num_blocks-1 giving the order in
 * which blocks are first handed out (free_order[0] first).  Without it,
 * block 0 first.  *out receives the handle (host memory only). */
pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t *free_order, pa_allocator **out);
void pa_allocator_destroy(pa_allocator *a);

/* New empty sequence.  INVALID_ARG if the id exists. */
pa_status pa_seq_create(pa_allocator *a, int64_t seq_id);

/* Child shares every block of parent (refcount + 1 each) and its length
 * ([VE] §3.1: parallel and speculative sampling share a prefix's blocks). */
pa_status pa_seq_fork(pa_allocator *a, int64_t parent, int64_t child);

/* Append n_tokens positions to a sequence; blocks are taken on demand, one
 * when a position starts a new block ([VE] §3.1).  slots_out[i] receives the
 * slot of position len+i.  If the last block is partly filled and shared, it
 * is first replaced by a fresh private block and (old, new) written to
 * cow_pairs_out (copy-on-write, [VI] §2.1); *n_cow gets the number of pairs
 * (0 or 1).  The caller copies those pairs (pa_copy_blocks) before writing
 * the new slots.  All or nothing: OUT_OF_BLOCKS, or INVALID_ARG when
 * cow_cap is too small, leave every table and count unchanged.
 *   slots_out     [n_tokens] host; cow_pairs_out [cow_cap][2] host. */
pa_status pa_seq_append(pa_allocator *a, int64_t seq_id, int32_t n_tokens,
                        int64_t *slots_out, int32_t *cow_pairs_out,
                        int32_t cow_cap, int32_t *n_cow);

/* Release a finished sequence: each block loses a reference; blocks that
 * reach zero go back on the free list at once ([VE] §3.1), last table entry
 * first, so the sequence's first block is handed out next (registered
 * prefix-cache blocks are queued instead: see the prefix cache below). */
pa_status pa_seq_free(pa_allocator *a, int64_t seq_id);

pa_status pa_seq_length(const pa_allocator *a, int64_t seq_id, int32_t *len);

/* Blocks an append of n_tokens would take now, counting a copy-on-write
 * block (what pa_seq_append checks against the free count). */
pa_status pa_seq_blocks_needed(const pa_allocator *a, int64_t seq_id, int32_t n_tokens,
                               int32_t *blocks);
/* Entries in the sequence's table (host blocks while swapped out). */
pa_status pa_seq_num_blocks(const pa_allocator *a, int64_t seq_id, int32_t *n_blocks);

/* Copy the sequence's block table (physical ids, logical order) to out
 * [cap]; *n_out gets its length.  INVALID_ARG if cap is too small. */
pa_status pa_seq_block_table(const pa_allocator *a, int64_t seq_id,
                             int32_t *out, int32_t cap, int32_t *n_out);

pa_status pa_allocator_stats(const pa_allocator *a, pa_allocator_stats_t *out);
pa_status pa_block_refcount(const pa_allocator *a, int32_t block,
                            int32_t *refcount);

/* One scheduling step for many sequences at once: append n_tokens[i]
 * positions to seq_ids[i] for every i, writing the slots back to back into
 * slots_out (sum of n_tokens entries) and every copy-on-write pair into
 * cow_pairs_out.  All or nothing across the whole batch.  Ids must be
 * distinct. */
pa_status pa_batch_append(pa_allocator *a, int32_t num_seqs,
                          const int64_t *seq_ids, const int32_t *n_tokens,
                          int64_t *slots_out, int32_t *cow_pairs_out,
                          int32_t cow_cap, int32_t *n_cow);

/* Dense block tables and lengths of a batch, ready to copy to the device:
 * tables_out [num_seqs][stride] (entries past a sequence's blocks set to
 * pad_value), context_lens_out [num_seqs].  INVALID_ARG if a table does not
 * fit in stride. */
pa_status pa_batch_tables(const pa_allocator *a, int32_t num_seqs,
                          const int64_t *seq_ids, int32_t *tables_out,
                          int32_t stride, int32_t pad_value,
                          int32_t *context_lens_out);

/* ------------------------------------------------------------------------ */
/* Prefix cache                                                               */
/* ------------------------------------------------------------------------ */
/* Allocation first reuses blocks that can be shared with a request's prefix,
 * then takes free ones; cold blocks leave under an LRU policy ([VI] §2.1,
 * and §3's switch for prompt sharing).  The hit rate is the metric to watch
 * ([NV] practical advice).  The pages fix no key or eviction rule; this
 * library's:
 *  - A block is registered once every position in it was appended with its
 *    token id (pa_seq_append_tokens / pa_batch_append_tokens), along an
 *    unbroken chain from position 0.  Its key is (parent, token ids), parent
 *    being the physical block of the previous logical block (-1 for the
 *    first); since the parent's key names everything before it, a key names
 *    the whole prefix exactly (lookups compare the stored ids, not only a
 *    hash).  A key already registered is not registered again, and that
 *    ends the sequence's chain; so does any append without token ids.
 *  - A registered block whose last reference goes is queued (oldest first)
 *    instead of returning to the free stack, and keeps its contents.
 *  - Taking a block pops the free stack; when it is empty, the oldest queued
 *    block is taken, and its key and its registered descendants' keys are
 *    dropped.  pa_allocator_stats counts stack and queue as free.
 *  - A cached block's contents are those written by the work the caller
 *    enqueued after the append that filled it: reuse it on the same stream,
 *    or after that work. */

typedef struct {
    int64_t queried_blocks;     /* full prompt blocks looked up so far */
    int64_t hit_blocks;         /* of them, found in the cache */
    int32_t cached_blocks;      /* blocks registered now */
    int32_t cached_free_blocks; /* of them, queued with no holder */
} pa_prefix_stats_t;

/* New sequence seq_id for a prompt of n_tokens token ids: its table starts
 * with the cached blocks of the longest registered chain of the prompt's
 * full blocks, at most max_cached_tokens / block_size of them (pass
 * n_tokens - 1 to leave the last position to compute).  Each reused block
 * gains a reference; *n_cached gets the positions covered (a multiple of
 * block_size), which is the new sequence's length.  The caller appends the
 * rest of the prompt with pa_seq_append_tokens.  Counts n_tokens /
 * block_size queried blocks.  INVALID_ARG if the id exists; nothing changes
 * on failure.
 *   tokens [n_tokens] host. */
pa_status pa_seq_create_prefix(pa_allocator *a, int64_t seq_id,
                               const int32_t *tokens, int32_t n_tokens,
                               int32_t max_cached_tokens, int32_t *n_cached);

/* pa_seq_append with the token ids of the new positions: blocks that become
 * full are registered (see above).  tokens [n_tokens] host. */
pa_status pa_seq_append_tokens(pa_allocator *a, int64_t seq_id,
                               const int32_t *tokens, int32_t n_tokens,
                               int64_t *slots_out, int32_t *cow_pairs_out,
                               int32_t cow_cap, int32_t *n_cow);

/* pa_batch_append with token ids: tokens holds sum(n_tokens) ids, the
 * sequences' ids back to back in batch order. */
pa_status pa_batch_append_tokens(pa_allocator *a, int32_t num_seqs,
                                 const int64_t *seq_ids,
                                 const int32_t *n_tokens,
                                 const int32_t *tokens, int64_t *slots_out,
                                 int32_t *cow_pairs_out, int32_t cow_cap,
                                 int32_t *n_cow);

pa_status pa_prefix_cache_stats(const pa_allocator *a, pa_prefix_stats_t *out);

/* Host tier of the prefix cache ([VI] §2.1: cold blocks move to CPU memory
 * under an LRU policy).  Uses the swap space's host pool (set with
 * pa_allocator_set_swap_space), sharing its free host blocks with swapping.
 *
 * Offload: the oldest released registered blocks (the LRU queue, oldest
 * first; queued blocks that lost their key are passed over), up to
 * max_blocks and while host blocks are free, move to host blocks with their
 * keys; their device blocks become free.  pairs_out [cap][2] host gets
 * (device block, host block) per move, *n_pairs their count: copy them
 * device -> host (pa_swap_blocks) before any later cache write or block
 * copy on the device pool, i.e. enqueue the copy first on the same stream.
 * Since blocks are queued children first, a host entry's registered
 * descendants are on the host too. */
pa_status pa_prefix_cache_offload(pa_allocator *a, int32_t max_blocks, int32_t *pairs_out,
                                  int32_t cap, int32_t *n_pairs);

/* pa_seq_create_prefix that also reuses host entries: after the prompt's
 * chain of device hits, each following hit on a host entry takes a free
 * device block (the entry moves back into it, keeping its key, and its host
 * block returns to the host stack) while one is free -- the device hits are
 * held first, so taking blocks never evicts them -- and while pairs_out
 * [cap][2] has room.  pairs_out gets (host block, device block) per reload,
 * *n_pairs their count: copy them host -> device (pa_swap_blocks) before the
 * sequence is decoded.  pa_seq_create_prefix itself stops its chain at a
 * host entry.  Errors as pa_seq_create_prefix. */
pa_status pa_seq_create_prefix_ex(pa_allocator *a, int64_t seq_id, const int32_t *tokens,
                                  int32_t n_tokens, int32_t max_cached_tokens,
                                  int32_t *n_cached, int32_t *pairs_out, int32_t cap,
                                  int32_t *n_pairs);

typedef struct {
    int32_t host_cached_blocks; /* registered entries on the host now */
    int64_t offloaded_blocks;   /* moved to the host so far */
    int64_t reloaded_blocks;    /* brought back by a prompt's hit so far */
} pa_prefix_host_stats_t;

pa_status pa_prefix_host_stats(const pa_allocator *a, pa_prefix_host_stats_t *out);

/* ------------------------------------------------------------------------ */
/* Swap space                                                                 */
/* ------------------------------------------------------------------------ */
/* Preemption moves a request's KV cache out to CPU memory and back in when
 * room returns ([NV] best practice 5); cold blocks migrate to CPU memory
 * ([VI] §2.1); a CPU swap space extends the cache ([VI] §5).  Here a caller-
 * owned host pool (pinned, same block layout as the device pools) holds
 * num_host_blocks blocks; the allocator keeps its own free stack for it
 * (host block 0 handed out first). */

typedef struct {
    int32_t num_host_blocks;
    int32_t num_host_free;
    int32_t swapped_seqs;
    int64_t swap_out_blocks; /* blocks moved out so far */
    int64_t swap_in_blocks;  /* blocks moved in so far */
} pa_swap_stats_t;

/* Size the host pool.  INVALID_ARG while any sequence is swapped out or
 * any prefix-cache entry is on the host. */
pa_status pa_allocator_set_swap_space(pa_allocator *a, int32_t num_host_blocks);

/* Swap a resident sequence out.  Every table entry j, in order, gets a host
 * block; pairs_out[j] = (device block, host block) [cap][2] host, *n_pairs
 * entries.  Then the device blocks lose one reference each, last entry
 * first, as in pa_seq_free (a block shared with other sequences stays theirs;
 * the swapped sequence owns a private host copy).  The caller copies the
 * pairs device -> host (pa_swap_blocks) before any work that may write the
 * released blocks.  The sequence's table then holds host block ids; it
 * cannot be appended to, forked or put in a batch table until swapped in.
 * OUT_OF_BLOCKS (host pool short) or INVALID_ARG (cap too small) change
 * nothing. */
pa_status pa_seq_swap_out(pa_allocator *a, int64_t seq_id, int32_t *pairs_out,
                          int32_t cap, int32_t *n_pairs);

/* Swap a sequence back in: every entry j, in order, gets a fresh device
 * block; pairs_out[j] = (host block, device block); the host blocks return to
 * the host stack, last entry first.  The new blocks are private and not in
 * the prefix cache.  The caller copies the pairs host -> device before the
 * sequence's next use.  OUT_OF_BLOCKS or INVALID_ARG change nothing.
 * pa_seq_free of a swapped sequence returns its host blocks. */
pa_status pa_seq_swap_in(pa_allocator *a, int64_t seq_id, int32_t *pairs_out,
                         int32_t cap, int32_t *n_pairs);

pa_status pa_seq_is_swapped(const pa_allocator *a, int64_t seq_id,
                            int32_t *swapped);
pa_status pa_swap_stats(const pa_allocator *a, pa_swap_stats_t *out);

/* Copy whole blocks between two pools of the same geometry, on the GPU:
 * for each pair i, block src_dst[2i] of (src_k, src_v) goes to block
 * src_dst[2i + 1] of (dst_k, dst_v), K and V regions, all heads.  One pool is
 * normally device memory and the other the pinned host pool (the copy then
 * runs over PCIe); both may be device memory.  Each pool pointer must be
 * device memory or pinned host memory mapped for the device (checked:
 * pageable memory is INVALID_ARG); src_dst [num_pairs][2] int32 must be
 * device-accessible too.  Pairs naming a block outside its pool are skipped.
 * Pools must not overlap. */
pa_status pa_swap_blocks(const void *src_k, const void *src_v, int32_t src_blocks,
                         void *dst_k, void *dst_v, int32_t dst_blocks,
                         const int32_t *src_dst, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void *stream);

/* ------------------------------------------------------------------------ */
/* Continuous-batching scheduler                                              */
/* ------------------------------------------------------------------------ */
/* Requests join the running batch at every step and leave as soon as they
 * finish ([VE] §3.2); one step mixes prompt chunks and decode ([VI] §1); new
 * requests wait in a queue and get blocks when admitted, and finished ones
 * release theirs at once ([VI] §2.2); admission is first-come first-served
 * and a request that cannot get room is preempted by moving its cache to
 * host memory ([NV] best practice 5).  The policy, step by step:
 *   1. Decode set: running requests whose prompt is written, in admission
 *      order, one position each.  While the pool cannot hold those, the most
 *      recently admitted running request is preempted: swapped out if the
 *      host pool holds its blocks, else sent back to the head of the waiting
 *      queue to start over (recompute).
 *   2. The decode positions are appended.
 *   3. The step's token budget (max_batched_tokens minus the decode count)
 *      goes to requests still in their prompt, in admission order:
 *      min(rest of prompt, budget, max_prefill_chunk) positions each while
 *      the pool holds them.
 *   4. Swapped requests return in arrival order while fewer than
 *      max_num_seqs run and the pool holds their blocks (no work that step).
 *   5. Waiting requests are admitted in queue order while fewer than
 *      max_num_seqs run, budget remains and the pool holds their first chunk;
 *      a request given token ids first reuses its cached prompt blocks
 *      (pa_seq_create_prefix, leaving its last position to compute).
 * The step writing a prompt's last chunk yields the request's first token,
 * each decode one more; at max_new tokens the request finishes and its
 * blocks are freed (pa_sched_complete).  Request ids are the allocator's
 * sequence ids.  Host memory only; not thread-safe.
 *
 * Parallel sampling ([VE] §3.1: the outputs drawn from one prompt share its
 * KV blocks, copy-on-write where they diverge): a request added with
 * pa_sched_add_samples asks for n samples.  It runs as one sequence (its own
 * id) until its prompt is written; pa_sched_complete of that step forks
 * samples 2..n from it (pa_seq_fork), each of which already holds its first
 * token.  From then on the request's n sequences decode in the same steps,
 * adjacent in decode_ids (the request's id first, then its sample ids in the
 * order given), and are preempted, swapped back and finished together;
 * their first appends into the shared partial block come with copy-on-write
 * pairs.  max_num_seqs counts sequences, and a request holds n of them from
 * admission on.  Such a decode batch is grouped for pa_decode_grouped by
 * giving each request's run one group id (pa_decode_groups). */

typedef struct pa_sched pa_sched;

/* One step's plan.  The caller provides every array (host memory) with the
 * capacities shown; the step fills them and the counts.  Order of work on
 * the GPU: copy swap_out_pairs device -> host (pa_swap_blocks), then
 * swap_in_pairs host -> device, then cow_pairs (pa_copy_blocks), then write
 * the K/V of the new positions into slots (decode positions first, one per
 * decode entry, then each prefill chunk's positions in order), then run the
 * prefill chunks and the decode batch. */
typedef struct {
    int64_t *decode_ids;      /* [cap_seqs] sequences decoding this step */
    int32_t *decode_lens;     /* [cap_seqs] their context length after the append */
    int64_t *prefill_ids;     /* [cap_seqs] requests writing a prompt chunk */
    int32_t *prefill_starts;  /* [cap_seqs] first position of the chunk */
    int32_t *prefill_lens;    /* [cap_seqs] positions in the chunk */
    int64_t *preempted_ids;   /* [cap_seqs] requests sent back to start over (with
                                 samples: all of them are dropped, to be forked
                                 again) */
    int32_t cap_seqs;         /* >= max_num_seqs */
    int64_t *slots;           /* [cap_slots] slots of the step's new positions */
    int32_t cap_slots;        /* >= max_batched_tokens */
    int32_t *cow_pairs;       /* [cap_cow][2] (src, dst) */
    int32_t cap_cow;          /* >= max_num_seqs */
    int32_t *swap_out_pairs;  /* [cap_swap_pairs][2] (device block, host block) */
    int32_t *swap_in_pairs;   /* [cap_swap_pairs][2] (host block, device block) */
    int32_t cap_swap_pairs;   /* >= the allocator's num_blocks and its number of
                                 host blocks (forked samples swap out a private
                                 copy each of the blocks they share) */
    int32_t n_decode, n_prefill, n_preempted, n_slots, n_cow, n_swap_out, n_swap_in;
} pa_sched_plan_t;

typedef struct {
    int32_t waiting, running, swapped;  /* requests */
    int32_t running_seqs;               /* sequences the running requests hold */
    int64_t finished, swap_preemptions, recompute_preemptions;  /* requests */
    int64_t forked_samples;             /* sample sequences forked so far */
} pa_sched_stats_t;

/* The scheduler borrows the allocator (which must outlive it, and whose swap
 * space, if any, enables preemption by swap).  INVALID_ARG unless all three
 * sizes are >= 1 and max_batched_tokens >= max_num_seqs (a step may decode
 * one position for each of max_num_seqs sequences). */
pa_status pa_sched_create(pa_allocator *a, int32_t max_num_seqs, int32_t max_batched_tokens,
                          int32_t max_prefill_chunk, pa_sched **out);
void pa_sched_destroy(pa_sched *s);
/* Queue a request: n_prompt >= 1 prompt positions, max_new >= 1 tokens to
 * generate; tokens [n_prompt] (host) or NULL (no prefix-cache reuse). */
pa_status pa_sched_add(pa_sched *s, int64_t id, int32_t n_prompt, int32_t max_new,
                       const int32_t *tokens);
/* Queue a request for num_samples >= 1 parallel samples (see above), each
 * generating max_new tokens; sample_ids [num_samples - 1] (host, NULL when
 * num_samples is 1) are the sequence ids of samples 2..n.  INVALID_ARG if
 * num_samples > max_num_seqs (it could never be admitted) or an id repeats
 * or is taken by an earlier request or sample of this scheduler.
 * pa_sched_add is this call with one sample. */
pa_status pa_sched_add_samples(pa_sched *s, int64_t id, int32_t n_prompt, int32_t max_new,
                               const int32_t *tokens, const int64_t *sample_ids,
                               int32_t num_samples);
/* Plan the next step (see above).  INVALID_ARG if the previous plan was not
 * completed or the plan arrays are short; the allocator then is unchanged. */
pa_status pa_sched_step(pa_sched *s, pa_sched_plan_t *plan);
/* The planned step ran: fork the samples of requests whose prompt it wrote,
 * count its tokens and free finished requests, whose sequence ids (the
 * request's, then its samples') go to finished_ids [cap >= running_seqs].
 * A failed fork (a sample id the caller created in the allocator, host
 * memory) undoes this call's forks, returns its status and leaves the plan
 * pending. */
pa_status pa_sched_complete(pa_sched *s, int64_t *finished_ids, int32_t cap,
                            int32_t *n_finished);
pa_status pa_sched_stats(const pa_sched *s, pa_sched_stats_t *out);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
