// groups.cpp — host derivation of the group arrays pa_decode_grouped takes.
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — sequences forked from
//        one prompt share its physical blocks through their block tables.
//   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1 — requests
//        with a common prompt prefix share its blocks.
//
// A group is a run of consecutive sequences of the decode batch.  What the
// members share is read off their block tables: the leading entries that
// every member's table holds equal to the leader's (its first member's),
// counted over the blocks every member fills completely.  The decode splits
// that region into partitions of the size it runs with, the last one ending
// where the region ends, and each member's own tokens after it.

#include <cstdint>

#include "pa_internal.h"

extern "C" {

pa_status pa_decode_groups(const int32_t *block_tables, int32_t block_table_stride,
                           const int32_t *context_lens, const int32_t *seq_group,
                           int32_t num_seqs, int32_t block_size, int32_t num_groups,
                           int32_t *group_offsets, int32_t *group_shared,
                           int32_t *max_group_size) {
    const char *fn = "pa_decode_groups";
    if (num_seqs < 0 || num_groups < 0 || block_table_stride <= 0 || block_size <= 0)
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: num_seqs %d num_groups %d block_table_stride %d block_size %d", fn,
                        num_seqs, num_groups, block_table_stride, block_size);
    if (!group_offsets || !max_group_size || (num_groups > 0 && !group_shared) ||
        (num_seqs > 0 && (!block_tables || !context_lens || !seq_group)))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    // Validate the grouping first, so a rejected call writes nothing.
    int32_t expect = 0;  // the next group id to open
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t g = seq_group[s];
        if (g < -1 || g >= num_groups)
            return pa::fail(PA_ERR_INVALID_ARG, "%s: seq_group[%d] = %d outside [-1, %d)", fn, s,
                            g, num_groups);
        if (context_lens[s] < 0)
            return pa::fail(PA_ERR_INVALID_ARG, "%s: context_lens[%d] = %d", fn, s,
                            context_lens[s]);
        if (g < 0) continue;
        if (g == expect) {
            ++expect;  // a group opens
        } else if (g != expect - 1 || seq_group[s - 1] != g) {
            return pa::fail(PA_ERR_INVALID_ARG,
                            "%s: group %d: members must be consecutive and group ids follow "
                            "sequence order", fn, g);
        }
    }
    if (expect != num_groups)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %d groups named, %d declared", fn, expect,
                        num_groups);

    int32_t largest = 0;
    int32_t g = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (seq_group[s] < 0 || seq_group[s] != g) continue;
        // group g is sequences s .. e-1
        int32_t e = s;
        int32_t full = INT32_MAX;  // blocks every member fills completely
        while (e < num_seqs && seq_group[e] == g) {
            const int32_t f = context_lens[e] / block_size;
            full = f < full ? f : full;
            ++e;
        }
        if (full > block_table_stride) full = block_table_stride;
        const int32_t *lead = block_tables + (int64_t)s * block_table_stride;
        int32_t common = full;
        for (int32_t m = s + 1; m < e; ++m) {
            const int32_t *t = block_tables + (int64_t)m * block_table_stride;
            int32_t j = 0;
            while (j < common && t[j] == lead[j]) ++j;
            common = j;
        }
        group_offsets[g] = s;
        group_offsets[g + 1] = e;
        group_shared[g] = common;
        largest = e - s > largest ? e - s : largest;
        ++g;
        s = e - 1;
    }
    if (num_groups == 0) group_offsets[0] = 0;
    *max_group_size = largest;
    return pa::ok();
}

}  // extern "C"
