// api.cpp — C-ABI device entry points: argument validation, then launch.
//
// Every check runs before anything is enqueued, so a non-OK status means the
// stream is untouched.  Shapes and layouts are documented in pa.h.
#include <cinttypes>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "launch.h"
#include "pa_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_block_size(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128; }
bool valid_dtype(pa_dtype t) { return t == PA_DTYPE_F32 || t == PA_DTYPE_BF16; }
// Element types a block copy can move (it only moves bytes).
bool valid_block_dtype(pa_dtype t) { return valid_dtype(t) || t == PA_DTYPE_FP8_E4M3; }
bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kMaxGroup = 16;
constexpr float kLog2e = 1.4426950408889634f;
// Decode workgroups per launch: a 1-D grid of 64-lane workgroups must stay
// below 2^32 threads.
constexpr int64_t kMaxDecodeItems = (1LL << 26) - 1;

// Common checks of the cache geometry.
pa_status check_geometry(const char *fn, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks) {
    if (num_kv_heads <= 0 || num_blocks <= 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: num_kv_heads=%d num_blocks=%d", fn, num_kv_heads,
                        num_blocks);
    if (!supported_head_dim(head_dim))
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", fn, head_dim);
    if (!supported_block_size(block_size))
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 16, 32, 64, 128)", fn,
                        block_size);
    return PA_OK;
}

// Address at which the GPU reaches memory p: p itself for device memory, the
// mapped address for pinned host memory; nullptr for anything else
// (pageable host memory, which a kernel must never touch).
const void *device_view(const void *p) {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of the failed query
        return nullptr;
    }
    if (at.type == hipMemoryTypeDevice) return p;
    if (at.type == hipMemoryTypeHost && at.devicePointer) return at.devicePointer;
    return nullptr;
}

}  // namespace

extern "C" {

pa_status pa_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                         const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         void *stream) {
    const char *fn = "pa_cache_write";
    if (num_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_tokens %d", fn, num_tokens);
    if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "%s: dtype %d", fn, (int)dtype);
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, num_blocks)) return st;
    if (!k_cache || !v_cache || (num_tokens > 0 && (!k_new || !v_new || !slot_mapping)))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    int rc = pa::launch_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens,
                                    num_kv_heads, head_dim, block_size, num_blocks, dtype, stream);
    if (rc == pa::kLaunchTooLarge)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: too many threads for one launch (%d)", fn, rc);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

pa_status pa_cache_write_fp8(const void *k_new, const void *v_new, pa_dtype in_dtype,
                             void *k_cache, void *v_cache, const int64_t *slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, float k_scale, float v_scale,
                             void *stream) {
    const char *fn = "pa_cache_write_fp8";
    if (num_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_tokens %d", fn, num_tokens);
    if (!valid_dtype(in_dtype))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: input dtype %d", fn, (int)in_dtype);
    if (!valid_scale(k_scale) || !valid_scale(v_scale))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: scales must be finite and > 0", fn);
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, num_blocks)) return st;
    if (!k_cache || !v_cache || (num_tokens > 0 && (!k_new || !v_new || !slot_mapping)))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    int rc = pa::launch_cache_write_fp8(k_new, v_new, in_dtype, k_cache, v_cache, slot_mapping,
                                        num_tokens, num_kv_heads, head_dim, block_size,
                                        num_blocks, k_scale, v_scale, stream);
    if (rc == pa::kLaunchTooLarge)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: too many threads for one launch (%d)", fn, rc);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, pa_dtype dtype, void *stream) {
    const char *fn = "pa_copy_blocks";
    if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_pairs %d", fn, num_pairs);
    if (!valid_block_dtype(dtype))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: dtype %d", fn, (int)dtype);
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, num_blocks)) return st;
    if (!k_cache || !v_cache || (num_pairs > 0 && !src_dst))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src_dst, 4))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    int rc = pa::launch_copy_blocks(k_cache, v_cache, src_dst, num_pairs, num_kv_heads, head_dim,
                                    block_size, num_blocks, dtype, stream);
    if (rc == pa::kLaunchTooLarge)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: too many threads for one launch (%d)", fn, rc);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

pa_status pa_read_stream(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    const char *fn = "pa_read_stream";
    static_assert(PA_READ_STREAM_SINK_WORDS == pa::kReadStreamBlocks, "one sink word per workgroup");
    if (!src || !sink) return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(src, 16) || !aligned(sink, 4))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (bytes % 16 != 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %zu bytes is not a multiple of 16", fn, bytes);
    int rc = pa::launch_read_stream(src, bytes, sink, stream);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

pa_status pa_swap_blocks(const void *src_k, const void *src_v, int32_t src_blocks, void *dst_k,
                         void *dst_v, int32_t dst_blocks, const int32_t *src_dst,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void *stream) {
    const char *fn = "pa_swap_blocks";
    if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_pairs %d", fn, num_pairs);
    if (!valid_block_dtype(dtype))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: dtype %d", fn, (int)dtype);
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, src_blocks)) return st;
    if (dst_blocks <= 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: dst_blocks %d", fn, dst_blocks);
    if (!src_k || !src_v || !dst_k || !dst_v || (num_pairs > 0 && !src_dst))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
        !aligned(src_dst, 4))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (num_pairs == 0) return pa::ok();
    const void *sk = device_view(src_k), *sv = device_view(src_v);
    const void *dk = device_view(dst_k), *dv = device_view(dst_v);
    const void *pr = device_view(src_dst);
    if (!sk || !sv || !dk || !dv || !pr)
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: a pool or the pair list is neither device memory nor pinned host "
                        "memory", fn);
    int rc = pa::launch_swap_blocks(sk, sv, src_blocks, const_cast<void *>(dk),
                                    const_cast<void *>(dv), dst_blocks,
                                    static_cast<const int32_t *>(pr), num_pairs, num_kv_heads,
                                    head_dim, block_size, dtype, stream);
    if (rc == pa::kLaunchTooLarge)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: too many threads for one launch (%d)", fn, rc);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

}  // extern "C"

namespace {

// Workspace bytes of a decode call; grouped: one partition more per row.
size_t workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_context_len,
                      int32_t partition_size, bool grouped) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_context_len < 0 || partition_size < 0)
        return (size_t)-1;
    const int32_t ps = partition_size ? partition_size
                                      : pa::default_partition(num_seqs, num_kv_heads, block_size,
                                                          max_context_len);
    const int64_t np_max = ceil_div(max_context_len > 0 ? max_context_len : 1, ps);
    const int64_t np_slots = grouped ? np_max + 1 : np_max;
    return pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np_slots);
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                int32_t partition_size) {
    return workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, partition_size, false);
}

size_t pa_decode_grouped_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len,
                                        int32_t partition_size) {
    return workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, partition_size, true);
}

pa_status pa_decode(float *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t block_table_stride,
                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    float scale, int32_t max_context_len, int32_t partition_size, void *workspace,
                    size_t workspace_bytes, pa_dtype dtype, void *stream) {
    return pa_decode_ex(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        scale, max_context_len, partition_size, workspace, workspace_bytes,
                        dtype, 0u, stream);
}

}  // extern "C"

namespace {

// Groups of sequences sharing leading blocks (pa_decode_grouped).
struct GroupArgs {
    const int32_t *offsets, *seq_group, *shared;
    int32_t num_groups, max_group_size;
};

// Shared body of the decode entry points.  fp8: the caches hold E4M3 codes
// scaled by k_scale / v_scale and q is bf16 (dtype must be BF16).
pa_status decode_impl(const char *fn, float *out, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, float scale,
                      int32_t max_context_len, int32_t partition_size, void *workspace,
                      size_t workspace_bytes, pa_dtype dtype, uint32_t flags, bool fp8,
                      float k_scale, float v_scale, void *stream,
                      const GroupArgs *grp = nullptr) {
    if (fp8 && (!valid_scale(k_scale) || !valid_scale(v_scale)))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: scales must be finite and > 0", fn);
    if (flags & ~(uint32_t)(PA_DECODE_KV_REUSE | PA_DECODE_VALU))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    const bool valu = (flags & PA_DECODE_VALU) != 0;
    if (valu && (fp8 || grp))
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: PA_DECODE_VALU applies to pa_decode_ex over bf16/fp32 caches only",
                        fn);
    if (num_seqs < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_seqs %d", fn, num_seqs);
    if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "%s: dtype %d", fn, (int)dtype);
    if (grp) {
        if (dtype != PA_DTYPE_BF16)
            return pa::fail(PA_ERR_UNSUPPORTED, "%s: bf16 or fp8 caches only", fn);
        if (grp->num_groups < 0 ||
            (grp->num_groups > 0 && (!grp->offsets || !grp->seq_group || !grp->shared ||
                                     grp->max_group_size < 1)))
            return pa::fail(PA_ERR_INVALID_ARG, "%s: num_groups %d, max_group_size %d, group arrays %s",
                            fn, grp->num_groups, grp->max_group_size,
                            grp->offsets && grp->seq_group && grp->shared ? "set" : "NULL");
        if (!aligned(grp->offsets, 4) || !aligned(grp->seq_group, 4) || !aligned(grp->shared, 4))
            return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned group array", fn);
    }
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, num_blocks)) return st;
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %d not a multiple of num_kv_heads %d",
                        fn, num_q_heads, num_kv_heads);
    if (num_q_heads / num_kv_heads > kMaxGroup)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: group size %d > %d", fn,
                        num_q_heads / num_kv_heads, kMaxGroup);
    if (block_table_stride <= 0 || max_context_len < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: block_table_stride %d max_context_len %d", fn,
                        block_table_stride, max_context_len);
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARG, "%s: scale not finite", fn);
    if (partition_size < 0 ||
        (partition_size > 0 && (partition_size % 32 != 0 || partition_size % block_size != 0)))
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: partition_size %d must be 0 or a multiple of 32 and of block_size %d",
                        fn, partition_size, block_size);
    if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(workspace, 16))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    const int32_t ps = partition_size ? partition_size
                                      : pa::default_partition(num_seqs, num_kv_heads, block_size,
                                                          max_context_len);
    const int64_t np_max = ceil_div(max_context_len > 0 ? max_context_len : 1, ps);
    // a grouped call's members may split at their shared region's end: one
    // partition more per sequence at most
    const bool grouped = grp && grp->num_groups > 0;
    const int64_t np_slots = grouped ? np_max + 1 : np_max;
    const size_t need = pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np_slots);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: workspace %zu bytes, need %zu", fn,
                        workspace ? workspace_bytes : (size_t)0, need);
    if (np_slots * num_kv_heads * (int64_t)num_seqs > kMaxDecodeItems)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: %lld partitions x kv heads x sequences > %lld",
                        fn, (long long)(np_slots * num_kv_heads * (int64_t)num_seqs),
                        (long long)kMaxDecodeItems);
    if (num_seqs == 0) return pa::ok();

    pa::DecodeParams p{};
    p.out = out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.table_stride = block_table_stride;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.num_blocks = num_blocks;
    p.max_context_len = max_context_len;
    p.partition_size = ps;
    p.np_max = (int32_t)np_max;
    p.np_slots = (int32_t)np_slots;
    p.scale_log2 = fp8 ? scale * k_scale * kLog2e : scale * kLog2e;
    p.kv_reuse = (flags & PA_DECODE_KV_REUSE) != 0;
    p.kv_fp8 = fp8;
    p.v_scale = fp8 ? v_scale : 1.f;
    if (need > 0) pa::decode_workspace_split(workspace, num_seqs, num_q_heads, np_slots, &p.ws_ml,
                                             &p.ws_o);
    if (grouped) {
        // one wave serves 16 / G members; chunks cover max_group_size members
        const int64_t mpw = kMaxGroup / (num_q_heads / num_kv_heads);
        const int64_t chunks = (grp->max_group_size + mpw - 1) / mpw;
        const int64_t group_items = np_max * chunks * grp->num_groups * num_kv_heads;
        const int64_t seq_items = np_slots * num_kv_heads * (int64_t)num_seqs;
        if (group_items + seq_items > kMaxDecodeItems)
            return pa::fail(PA_ERR_UNSUPPORTED, "%s: %lld group + %lld sequence work items > %lld",
                            fn, (long long)group_items, (long long)seq_items,
                            (long long)kMaxDecodeItems);
        p.seq_group = grp->seq_group;
        p.grp_offsets = grp->offsets;
        p.grp_shared = grp->shared;
        p.num_groups = grp->num_groups;
        p.grp_chunks = (int32_t)chunks;
        p.grp_cover = (int32_t)(chunks * mpw);
    }
    int rc = dtype == PA_DTYPE_BF16 && !valu ? pa::launch_decode_mfma(p, stream)
                                             : pa::launch_decode_valu(p, dtype, stream);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    rc = pa::launch_decode_reduce(p, stream);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: reduce launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

}  // namespace

extern "C" {

pa_status pa_decode_ex(float *out, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, int32_t block_table_stride,
                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t max_context_len,
                       int32_t partition_size, void *workspace, size_t workspace_bytes,
                       pa_dtype dtype, uint32_t flags, void *stream) {
    return decode_impl("pa_decode", out, q, k_cache, v_cache, block_tables, block_table_stride,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, max_context_len, partition_size, workspace,
                       workspace_bytes, dtype, flags, false, 1.f, 1.f, stream);
}

pa_status pa_decode_grouped(float *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, int32_t block_table_stride,
                            const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t max_context_len,
                            int32_t partition_size, const int32_t *group_offsets,
                            const int32_t *seq_group, const int32_t *group_shared,
                            int32_t num_groups, int32_t max_group_size, void *workspace,
                            size_t workspace_bytes, pa_dtype dtype, uint32_t flags,
                            void *stream) {
    const GroupArgs grp{group_offsets, seq_group, group_shared, num_groups, max_group_size};
    return decode_impl("pa_decode_grouped", out, q, k_cache, v_cache, block_tables,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, max_context_len, partition_size,
                       workspace, workspace_bytes, dtype, flags, false, 1.f, 1.f, stream, &grp);
}

pa_status pa_decode_grouped_fp8(float *out, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                int32_t block_table_stride, const int32_t *context_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                float scale, float k_scale, float v_scale,
                                int32_t max_context_len, int32_t partition_size,
                                const int32_t *group_offsets, const int32_t *seq_group,
                                const int32_t *group_shared, int32_t num_groups,
                                int32_t max_group_size, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream) {
    const GroupArgs grp{group_offsets, seq_group, group_shared, num_groups, max_group_size};
    return decode_impl("pa_decode_grouped_fp8", out, q, k_cache, v_cache, block_tables,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, max_context_len, partition_size,
                       workspace, workspace_bytes, PA_DTYPE_BF16, flags, true, k_scale, v_scale,
                       stream, &grp);
}

pa_status pa_decode_fp8(float *out, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int32_t block_table_stride,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, float scale, float k_scale, float v_scale,
                        int32_t max_context_len, int32_t partition_size, void *workspace,
                        size_t workspace_bytes, uint32_t flags, void *stream) {
    return decode_impl("pa_decode_fp8", out, q, k_cache, v_cache, block_tables,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, max_context_len, partition_size,
                       workspace, workspace_bytes, PA_DTYPE_BF16, flags, true, k_scale, v_scale,
                       stream);
}

}  // extern "C"

namespace {

// Shared body of the prefill entry points (fp8: E4M3 caches with scales).
pa_status prefill_impl(const char *fn, float *out, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_tables,
                       int32_t block_table_stride, const int32_t *cu_q_lens,
                       const int32_t *context_lens, int32_t num_reqs, int32_t total_q_tokens,
                       int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, pa_dtype dtype, bool fp8, float k_scale,
                       float v_scale, void *stream) {
    if (fp8 && (!valid_scale(k_scale) || !valid_scale(v_scale)))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: scales must be finite and > 0", fn);
    if (num_reqs < 0 || total_q_tokens < 0 || max_q_len < 0 || max_context_len < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
    if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "%s: dtype %d", fn, (int)dtype);
    if (dtype != PA_DTYPE_BF16) return pa::fail(PA_ERR_UNSUPPORTED, "%s: bf16 only", fn);
    if (pa_status st = check_geometry(fn, num_kv_heads, head_dim, block_size, num_blocks)) return st;
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %d not a multiple of num_kv_heads %d",
                        fn, num_q_heads, num_kv_heads);
    if (num_q_heads / num_kv_heads > kMaxGroup)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: group size %d > %d", fn,
                        num_q_heads / num_kv_heads, kMaxGroup);
    if (block_table_stride <= 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: block_table_stride %d", fn, block_table_stride);
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARG, "%s: scale not finite", fn);
    if (num_reqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !cu_q_lens ||
                         !context_lens))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(cu_q_lens, 4) || !aligned(context_lens, 4))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (num_reqs == 0 || total_q_tokens == 0 || max_q_len == 0) return pa::ok();
    pa::PrefillParams p{};
    p.out = out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.cu_q_lens = cu_q_lens;
    p.context_lens = context_lens;
    p.table_stride = block_table_stride;
    p.num_reqs = num_reqs;
    p.total_q_tokens = total_q_tokens;
    p.max_q_len = max_q_len;
    p.max_context_len = max_context_len;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.num_blocks = num_blocks;
    p.scale_log2 = fp8 ? scale * k_scale * kLog2e : scale * kLog2e;
    p.kv_fp8 = fp8;
    p.v_scale = fp8 ? v_scale : 1.f;
    int rc = pa::launch_prefill(p, stream);
    if (rc == -1) return pa::fail(PA_ERR_UNSUPPORTED, "%s: no kernel for this shape", fn);
    if (rc) return pa::fail(PA_ERR_DEVICE, "%s: launch failed (hip error %d)", fn, rc);
    return pa::ok();
}

}  // namespace

extern "C" {

pa_status pa_prefill_chunk(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, int32_t block_table_stride,
                           const int32_t *cu_q_lens, const int32_t *context_lens, int32_t num_reqs,
                           int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, float scale, pa_dtype dtype,
                           void *stream) {
    return prefill_impl("pa_prefill_chunk", out, q, k_cache, v_cache, block_tables,
                        block_table_stride, cu_q_lens, context_lens, num_reqs, total_q_tokens,
                        max_q_len, max_context_len, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, dtype, false, 1.f, 1.f, stream);
}

pa_status pa_prefill_chunk_fp8(float *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               int32_t block_table_stride, const int32_t *cu_q_lens,
                               const int32_t *context_lens, int32_t num_reqs,
                               int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, float scale, float k_scale,
                               float v_scale, void *stream) {
    return prefill_impl("pa_prefill_chunk_fp8", out, q, k_cache, v_cache, block_tables,
                        block_table_stride, cu_q_lens, context_lens, num_reqs, total_q_tokens,
                        max_q_len, max_context_len, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, PA_DTYPE_BF16, true, k_scale, v_scale,
                        stream);
}

}  // extern "C"
