// decode_split.h — how a decode call splits each sequence into partitions
// (device side; shared by the partition kernels and the merge).
//
// Source: [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1 — segments of a
// sequence can be processed independently and merged; [VE] 《加速 LLM 推理：
// 深入了解 vLLM 引擎》 §3.1 — sequences forked from one prompt hold its
// physical blocks.
//
// A sequence of L tokens is split into partitions of partition_size (ps)
// tokens, the last one partial.  In a grouped call a member of a group whose
// shared region (the group's first grp_shared blocks, T tokens) ends before
// its context does (0 < T < L) is split at T instead: ceil(T / ps) shared
// partitions [i ps, min((i + 1) ps, T)), computed once for the whole group,
// then its private tokens in partitions [T + j ps, min(T + (j + 1) ps, L)).
// With T a multiple of ps these are the plain partitions.  Partitions are
// numbered in token order; the merge takes them in that order.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace pa {

// Whether a context length can be walked: 0 <= L <= max_context_len and its
// blocks fit the table row.
__device__ __forceinline__ bool bad_length(const DecodeParams &p, int32_t L, int block_size) {
    const int32_t nb = (L + block_size - 1) / block_size;
    return L < 0 || L > p.max_context_len || nb > p.table_stride;
}
__device__ __forceinline__ int32_t num_parts(const DecodeParams &p, int32_t L, bool bad) {
    return bad ? 1 : max(1, (L + p.partition_size - 1) / p.partition_size);
}

// The partitions of one sequence: np in all, the first `shared` of them
// computed by its group (tokens [0, t_shared)); shared = t_shared = 0 for a
// sequence decoded alone.  np <= np_slots always: ceil(T / ps) + ceil((L -
// T) / ps) <= ceil(L / ps) + 1.
struct SeqSplit {
    int32_t np, shared, t_shared;
};

// A shared region of `blocks` blocks, in tokens (64-bit, so a malformed
// count cannot overflow; any region that is not shorter than a member's
// context shares nothing with it).
__device__ __forceinline__ int64_t shared_tokens(const DecodeParams &p, int32_t blocks) {
    return (int64_t)blocks * p.block_size;
}

// Whether sequence s (length L, bad_len from bad_length(), group id gid =
// seq_group[s]; lo, hi the group's run, T its region in tokens) shares the
// region.  The group kernel decides a member's column, the per-sequence
// items their partitions and the merge its partition count with this one
// test, so every partition is computed exactly once.
__device__ __forceinline__ bool member_shares(const DecodeParams &p, int s, int32_t gid,
                                              int32_t lo, int32_t hi, int64_t T, int32_t L,
                                              bool bad_len) {
    return gid >= 0 && gid < p.num_groups && lo >= 0 && s >= lo && s < hi &&
           s - lo < p.grp_cover && !bad_len && T > 0 && T < L;
}
__device__ __forceinline__ SeqSplit split_with(const DecodeParams &p, int32_t L, bool bad_len,
                                               bool shares, int64_t T) {
    SeqSplit r{num_parts(p, L, bad_len), 0, 0};
    if (shares) {
        const int32_t ps = p.partition_size;
        r.t_shared = (int32_t)T;
        r.shared = (r.t_shared + ps - 1) / ps;
        r.np = r.shared + (L - r.t_shared + ps - 1) / ps;
    }
    return r;
}
// The whole lookup, for callers that hold only s, L and gid.
__device__ __forceinline__ SeqSplit seq_split(const DecodeParams &p, int s, int32_t gid,
                                              int32_t L, bool bad_len) {
    if (gid < 0 || gid >= p.num_groups || bad_len) return split_with(p, L, bad_len, false, 0);
    const int32_t lo = p.grp_offsets[gid], hi = p.grp_offsets[gid + 1];
    const int64_t T = shared_tokens(p, p.grp_shared[gid]);
    return split_with(p, L, bad_len, member_shares(p, s, gid, lo, hi, T, L, bad_len), T);
}

}  // namespace pa
