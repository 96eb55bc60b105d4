// partition.cpp — how many tokens a decode partition holds (host side).
//
// Source: [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1 — segments of
// a sequence are processed independently and merged; [VE] 《加速 LLM 推理：
// 深入了解 vLLM 引擎》 §3.3 — decode is bound by memory bandwidth, so the
// split is chosen to keep the chip's memory pipes busy.
#include <cstdint>

#include "pa_internal.h"

namespace {
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

namespace pa {

// Partition size in tokens: a multiple of 32 (the decode step) and of the
// block size.  Start at 512 and halve while the grid would leave the 256
// compute units short of work (about 8 waves each).  With few (sequence,
// kv head) pairs -- a handful of long contexts -- every wave streams a full
// partition, and longer partitions amortise each wave's start-up (length,
// table slice, first loads) and shrink the merge: grow up to 4096 tokens
// while the grid keeps at least 1024 waves (4 per compute unit).
int32_t default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                          int32_t max_context_len) {
    const int32_t unit = block_size > 32 ? block_size : 32;
    const int64_t max_len = max_context_len > 0 ? max_context_len : 1;
    int32_t ps = 512;
    const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
    while (ps / 2 >= unit && (ps / 2) % unit == 0 && pairs * ceil_div(max_len, ps) < 2048)
        ps /= 2;
    if (pairs <= 256)
        while (ps < 4096 && pairs * ceil_div(max_len, 2 * ps) >= 1024) ps *= 2;
    // Then at most 16 partitions for the longest context, while the grid
    // keeps at least 512 waves: each partition's wave starts with a chain of
    // dependent loads that a longer partition amortises (on one box: the GQA
    // batch of up to 8192 tokens 184.5 -> 178.9 us at 1024, 8 x 32768 196.4
    // -> 189.0 us at 4096; batches of up to 4096 tokens keep 512, where 1024
    // is no faster).
    while (ps < 4096 && max_len >= 16 * (int64_t)ps && pairs * ceil_div(max_len, 2 * ps) >= 512)
        ps *= 2;
    return ps;
}

}  // namespace pa

extern "C" {

int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                    int32_t max_context_len) {
    return pa::default_partition(num_seqs, num_kv_heads, block_size, max_context_len);
}

// From the lengths themselves.  With 257 .. 1024 (sequence, kv head) pairs
// the longest-first grid runs the batch in about one round of the 2048 wave
// slots, and a round ends when its fullest slot does: the partitions should
// be a little longer than the average load of a slot, so that full
// partitions and the tails that follow them pack the slots evenly.  A sweep
// of ten lognormal-length batches of 128 sequences x 8 kv heads (partitions
// of 768 .. 1536 tokens) found the fastest size at 1.2 times the average
// tokens per slot, rounded to 128, on eight of them and within 0.5% on the
// other two; on batches of 512 and 384 pairs it was never slower than the
// size-only default.  Other batches keep pa_decode_default_partition: with many
// pairs the grid runs several rounds of short partitions, with few the
// default already grows the partitions.
int32_t pa_decode_partition_for_lengths(const int32_t *context_lens, int32_t num_seqs,
                                        int32_t num_kv_heads, int32_t block_size,
                                        int32_t max_context_len) {
    const char *fn = "pa_decode_partition_for_lengths";
    if (num_seqs < 0 || num_kv_heads <= 0 || block_size <= 0 || max_context_len < 0 ||
        (num_seqs > 0 && !context_lens)) {
        pa::fail(PA_ERR_INVALID_ARG, "%s: num_seqs %d num_kv_heads %d block_size %d "
                 "max_context_len %d%s", fn, num_seqs, num_kv_heads, block_size,
                 max_context_len, num_seqs > 0 && !context_lens ? ", NULL lengths" : "");
        return 0;
    }
    const int32_t ps0 = pa::default_partition(num_seqs, num_kv_heads, block_size,
                                              max_context_len);
    pa::ok();
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    if (pairs <= 256 || pairs > 1024) return ps0;
    int64_t tokens = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t L = context_lens[s];
        if (L > 0 && L <= max_context_len) tokens += L;
    }
    const int64_t unit = block_size > 128 ? block_size : 128;  // a multiple of 32 and of BS
    const double target = 1.2 * (double)(tokens * num_kv_heads) / 2048.0;
    int64_t ps = (int64_t)(target / (double)unit + 0.5) * unit;
    if (ps < unit) ps = unit;
    if (ps > 4096) ps = 4096;
    return (int32_t)ps;
}

// Grouped calls (pa_decode_grouped): the grid holds one wave per (kv head,
// group chunk, shared partition) and per (kv head, sequence, own partition),
// and each wave pays a start-up (lengths, group arrays, table slice, first
// loads) before it streams, so longer partitions mean fewer start-ups.
// Starting from the plain decode's size, double it while that grid keeps at
// least 2048 waves (8 per compute unit), up to 4096 tokens.
int32_t pa_decode_grouped_partition(const int32_t *context_lens, const int32_t *group_offsets,
                                    const int32_t *seq_group, const int32_t *group_shared,
                                    int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                                    int32_t max_context_len) {
    const char *fn = "pa_decode_grouped_partition";
    if (num_seqs < 0 || num_groups < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 16 || block_size <= 0 ||
        max_context_len < 0 || (num_groups > 0 && max_group_size < 1)) {
        pa::fail(PA_ERR_INVALID_ARG,
                 "%s: num_seqs %d num_groups %d max_group_size %d heads %d/%d block_size %d "
                 "max_context_len %d", fn, num_seqs, num_groups, max_group_size, num_q_heads,
                 num_kv_heads, block_size, max_context_len);
        return 0;
    }
    if ((num_seqs > 0 && (!context_lens || !seq_group)) ||
        (num_groups > 0 && (!group_offsets || !group_shared))) {
        pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
        return 0;
    }
    int32_t ps = pa::default_partition(num_seqs, num_kv_heads, block_size, max_context_len);
    const int64_t mpw = 16 / (num_q_heads / num_kv_heads);  // members per group wave
    const int64_t cover = (max_group_size + mpw - 1) / mpw * mpw;
    // waves of the grouped grid at partition size q (the kernels' own
    // membership test, member_shares, on the host copies of the arrays)
    // whether group g has a member that shares its region
    auto group_shares = [&](int32_t g) {
        const int32_t lo = group_offsets[g], hi = group_offsets[g + 1];
        const int64_t T = (int64_t)group_shared[g] * block_size;
        if (lo < 0 || lo >= num_seqs || hi <= lo || T <= 0) return false;
        for (int32_t s = lo; s < hi && s < num_seqs && s - lo < cover; ++s)
            if (seq_group[s] == g && context_lens[s] > T && context_lens[s] <= max_context_len)
                return true;
        return false;
    };
    auto waves = [&](int64_t q) {
        int64_t n = 0;
        for (int32_t g = 0; g < num_groups; ++g) {
            if (!group_shares(g)) continue;
            const int32_t lo = group_offsets[g], hi = group_offsets[g + 1];
            const int64_t T = (int64_t)group_shared[g] * block_size;
            const int64_t members = (hi < num_seqs ? hi : num_seqs) - lo;
            n += ceil_div(members < cover ? members : cover, mpw) * ceil_div(T, q);
        }
        for (int32_t s = 0; s < num_seqs; ++s) {
            const int32_t L = context_lens[s], g = seq_group[s];
            int64_t own = L;
            if (g >= 0 && g < num_groups && L <= max_context_len) {
                const int32_t lo = group_offsets[g], hi = group_offsets[g + 1];
                const int64_t T = (int64_t)group_shared[g] * block_size;
                if (lo >= 0 && s >= lo && s < hi && s - lo < cover && T > 0 && T < L) own = L - T;
            }
            n += own > 0 ? ceil_div(own, q) : 1;
        }
        return n * num_kv_heads;
    };
    // nothing shared: the plain decode's size
    bool sharing = false;
    for (int32_t g = 0; g < num_groups && !sharing; ++g) sharing = group_shares(g);
    while (sharing && ps < 4096 && waves(2 * (int64_t)ps) >= 2048) ps *= 2;
    pa::ok();
    return ps;
}

}  // extern "C"
