// launch.h — internal launchers behind the C ABI (host side, no HIP types).
//
// Each launcher enqueues its kernel(s) on `stream` and returns the
// hipError_t of the launch as an int (0 = success).  Arguments have already
// been validated by the C-ABI layer.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Launcher result for a call whose grid would not fit one launch (a 1-D
// grid holds fewer than 2^32 threads); the C-ABI layer reports it as
// PA_ERR_UNSUPPORTED.
constexpr int kLaunchTooLarge = -2;
// Whether `threads` threads fit a 1-D grid of 256-thread workgroups.
inline bool grid_fits(int64_t threads) { return threads >= 0 && threads <= 0xffffffffLL - 255; }

struct DecodeParams {
    float *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws_ml;      // [S][Hq][np_slots][2] (running max in log2 units, sum)
    float *ws_o;       // [S][Hq][np_slots][D] unnormalised partial outputs
    int32_t table_stride;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    int32_t max_context_len;
    int32_t partition_size;
    int32_t np_max;    // ceil(max_context_len / partition_size), >= 1
    int32_t np_slots;  // partitions per sequence the grid and workspace hold:
                       // np_max, one more in a grouped call (decode_split.h)
    float scale_log2;  // scale * log2(e) (times the K scale for an fp8 cache)
    bool kv_reuse;     // keep K/V cached (shared blocks) instead of streaming them
    bool kv_fp8;       // K/V hold OCP E4M3 codes (q stays bf16)
    float v_scale;     // value of a V code = code * v_scale (1 for bf16)
    // Groups of sequences that share leading blocks (null seq_group: none).
    // Sequence s belongs to group g = seq_group[s] when 0 <= g < num_groups,
    // grp_offsets[g] <= s < grp_offsets[g + 1] and s - grp_offsets[g] <
    // grp_cover.  When its context extends past the group's shared region
    // (the first grp_shared[g] blocks) that region's partitions are computed
    // once for the whole group, through the table of sequence grp_offsets[g]
    // (the leader), and its own partitions start where the region ends
    // (decode_split.h).
    const int32_t *seq_group;
    const int32_t *grp_offsets;
    const int32_t *grp_shared;
    int32_t num_groups;
    int32_t grp_cover;    // members per group the group kernel's chunks cover
    int32_t grp_chunks;   // member chunks per group (16 / G members each)
};

struct PrefillParams {
    float *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *cu_q_lens;
    const int32_t *context_lens;
    int32_t table_stride;
    int32_t num_reqs;
    int32_t total_q_tokens;
    int32_t max_q_len;
    int32_t max_context_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    float scale_log2;  // scale * log2(e) (times the K scale for an fp8 cache)
    bool kv_fp8;       // K/V hold OCP E4M3 codes (q stays bf16)
    float v_scale;     // value of a V code = code * v_scale (1 for bf16)
};

// Workspace layout shared by the decode kernels and the split-K reduce:
// np_slots partials per (sequence, query head) row (0 bytes when <= 1).
size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                              int64_t np_slots);
void decode_workspace_split(void *ws, int64_t num_seqs, int64_t num_q_heads, int64_t np_slots,
                            float **ml, float **o);

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                       void *stream);

// Quantizing write into an fp8 (OCP E4M3) cache: code = nearest E4M3 of
// x / scale (binary32 division), saturating at +-448.
int launch_cache_write_fp8(const void *k_new, const void *v_new, pa_dtype in_dtype,
                           void *k_cache, void *v_cache, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, float k_scale,
                           float v_scale, void *stream);

// Plain read stream (bandwidth.hip): one sink word per workgroup of a fixed
// grid of kReadStreamBlocks.  The fastest of a sweep over 8 GiB on one box
// (grids of 2048 to 131072 workgroups, 2 to 8 loads in flight per thread):
// 32768 x 256 threads read 7.07-7.10 TB/s, 8192 x 256 only 6.75-6.77.
constexpr int kReadStreamBlocks = 32768;
int launch_read_stream(const void *src, size_t bytes, uint32_t *sink, void *stream);

int launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, pa_dtype dtype, void *stream);
int launch_swap_blocks(const void *src_k, const void *src_v, int32_t src_blocks, void *dst_k,
                       void *dst_v, int32_t dst_blocks, const int32_t *src_dst,
                       int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, pa_dtype dtype, void *stream);

// bf16 decode on the matrix cores (any group size up to 16).  With groups
// (p.seq_group), the shared partitions are computed by one wave per (kv
// head, group, member chunk, partition) for every member at once, and the
// per-sequence kernel skips them.
int launch_decode_mfma(const DecodeParams &p, void *stream);
// Vector-ALU decode (fp32 or bf16, any group size up to 16).
int launch_decode_valu(const DecodeParams &p, pa_dtype dtype, void *stream);
// Merge split-K partials; a no-op for sequences with one partition.
int launch_decode_reduce(const DecodeParams &p, void *stream);

int launch_prefill(const PrefillParams &p, void *stream);

}  // namespace pa
