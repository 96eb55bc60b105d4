// allocator.cpp — host block allocator with refcounted sharing and
// copy-on-write.
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — blocks taken on demand,
//        freed at once when a sequence ends, shared between sequences.
//   [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 code example 1 —
//        ceil(n / block_size) blocks per sequence; running out is an error.
//   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §2.1 — a
//        pre-allocated pool, per-block state, host-side block tables,
//        copy-on-write for shared prefixes, a free list popped at its end.
//
// State: refcount[b] per block (0 free, 1 owned, >1 shared), a free stack
// (top = back of the vector), and per sequence its table and length.  Every
// mutating call first works out everything it needs, checks it can be
// satisfied, and only then commits, so a failed call changes nothing.
#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace {

struct Sequence {
    std::vector<int32_t> table;
    int32_t length = 0;
};

// Blocks needed for n tokens: ceil(n / bs).
inline int64_t blocks_for(int64_t n, int64_t bs) { return (n + bs - 1) / bs; }

}  // namespace

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> refcount;
    std::vector<int32_t> free_stack;
    std::unordered_map<int64_t, Sequence> seqs;
    int64_t cow_copies = 0;
    int32_t num_shared = 0;

    int32_t take() {
        int32_t b = free_stack.back();
        free_stack.pop_back();
        refcount[b] = 1;
        return b;
    }
    void add_ref(int32_t b) {
        if (++refcount[b] == 2) ++num_shared;
    }
    // Drops one reference; returns true when the block became free.
    bool drop_ref(int32_t b) {
        if (refcount[b]-- == 2) --num_shared;
        return refcount[b] == 0;
    }

    // Blocks an append of n tokens needs, and whether it starts with a COW.
    void needs(const Sequence &s, int32_t n, int64_t *blocks, bool *cow) const {
        int64_t fresh = blocks_for((int64_t)s.length + n, block_size) -
                        blocks_for(s.length, block_size);
        *cow = n > 0 && s.length % block_size != 0 && refcount[s.table.back()] > 1;
        *blocks = fresh + (*cow ? 1 : 0);
    }

    // Commit an append whose block needs were checked by needs().  The COW
    // decision is taken again here: an earlier append in the same batch may
    // have copied away from a block this sequence shared, leaving it the sole
    // holder, so the check-time count is an upper bound.
    void commit_append(Sequence &s, int32_t n, int64_t *slots, int32_t *pairs,
                       int32_t *n_pairs) {
        int64_t unused;
        bool cow;
        needs(s, n, &unused, &cow);
        if (cow) {
            int32_t src = s.table.back();
            int32_t dst = take();
            drop_ref(src);  // src keeps >= 1 holder: it was shared
            s.table.back() = dst;
            pairs[0] = src;
            pairs[1] = dst;
            *n_pairs = 1;
            ++cow_copies;
        } else {
            *n_pairs = 0;
        }
        for (int32_t i = 0; i < n; ++i) {
            int64_t pos = (int64_t)s.length + i;
            if (pos % block_size == 0) s.table.push_back(take());
            slots[i] = (int64_t)s.table[pos / block_size] * block_size + pos % block_size;
        }
        s.length += n;
    }
};

extern "C" {

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t *free_order, pa_allocator **out) {
    if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_allocator_create: out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_allocator_create: num_blocks=%d block_size=%d",
                        num_blocks, block_size);
    pa_allocator *a = new (std::nothrow) pa_allocator;
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "pa_allocator_create: out of host memory");
    try {
        a->num_blocks = num_blocks;
        a->block_size = block_size;
        a->refcount.assign(num_blocks, 0);
        a->free_stack.resize(num_blocks);
        if (free_order) {
            std::vector<char> seen(num_blocks, 0);
            for (int32_t i = 0; i < num_blocks; ++i) {
                int32_t b = free_order[i];
                if (b < 0 || b >= num_blocks || seen[b]) {
                    delete a;
                    return pa::fail(PA_ERR_INVALID_ARG,
                                    "pa_allocator_create: free_order is not a permutation "
                                    "(entry %d = %d)", i, b);
                }
                seen[b] = 1;
                a->free_stack[num_blocks - 1 - i] = b;  // free_order[0] on top
            }
        } else {
            for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[num_blocks - 1 - i] = i;
        }
    } catch (...) {
        delete a;
        return pa::fail(PA_ERR_INVALID_ARG, "pa_allocator_create: out of host memory");
    }
    *out = a;
    return pa::ok();
}

void pa_allocator_destroy(pa_allocator *a) { delete a; }

pa_status pa_seq_create(pa_allocator *a, int64_t seq_id) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_create: NULL allocator");
    if (a->seqs.count(seq_id))
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_create: sequence %lld exists",
                        (long long)seq_id);
    try {
        a->seqs.emplace(seq_id, Sequence{});
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_create: out of host memory");
    }
    return pa::ok();
}

pa_status pa_seq_fork(pa_allocator *a, int64_t parent, int64_t child) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: NULL allocator");
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_fork: no sequence %lld", (long long)parent);
    if (a->seqs.count(child))
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: sequence %lld exists",
                        (long long)child);
    try {
        Sequence copy = it->second;
        for (int32_t b : copy.table) a->add_ref(b);
        a->seqs.emplace(child, std::move(copy));
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: out of host memory");
    }
    return pa::ok();
}

pa_status pa_seq_append(pa_allocator *a, int64_t seq_id, int32_t n_tokens,
                        int64_t *slots_out, int32_t *cow_pairs_out, int32_t cow_cap,
                        int32_t *n_cow) {
    return pa_batch_append(a, 1, &seq_id, &n_tokens, slots_out, cow_pairs_out, cow_cap, n_cow);
}

pa_status pa_batch_append(pa_allocator *a, int32_t num_seqs, const int64_t *seq_ids,
                          const int32_t *n_tokens, int64_t *slots_out, int32_t *cow_pairs_out,
                          int32_t cow_cap, int32_t *n_cow) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "append: NULL allocator");
    if (num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !n_tokens)) || !n_cow || cow_cap < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "append: bad arguments");
    std::vector<Sequence *> seqs(num_seqs);
    int64_t total_blocks = 0, total_tokens = 0, total_cow = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return pa::fail(PA_ERR_NOT_FOUND, "append: no sequence %lld", (long long)seq_ids[i]);
        if (n_tokens[i] < 0)
            return pa::fail(PA_ERR_INVALID_ARG, "append: n_tokens[%d] = %d", i, n_tokens[i]);
        if ((int64_t)it->second.length + n_tokens[i] > INT32_MAX)
            return pa::fail(PA_ERR_INVALID_ARG, "append: sequence length overflows int32");
        seqs[i] = &it->second;
        int64_t blocks;
        bool c;
        a->needs(*seqs[i], n_tokens[i], &blocks, &c);
        total_blocks += blocks;
        total_tokens += n_tokens[i];
        total_cow += c ? 1 : 0;
    }
    if (num_seqs > 1) {
        std::unordered_set<int64_t> ids(seq_ids, seq_ids + num_seqs);
        if ((int32_t)ids.size() != num_seqs)
            return pa::fail(PA_ERR_INVALID_ARG, "append: repeated sequence id in batch");
    }
    if (total_tokens > 0 && !slots_out)
        return pa::fail(PA_ERR_INVALID_ARG, "append: slots_out is NULL");
    if (total_cow > cow_cap || (total_cow > 0 && !cow_pairs_out))
        return pa::fail(PA_ERR_INVALID_ARG, "append: %lld copy-on-write pairs, cow_cap %d",
                        (long long)total_cow, cow_cap);
    if (total_blocks > (int64_t)a->free_stack.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "append: need %lld blocks, %zu free",
                        (long long)total_blocks, a->free_stack.size());
    // Reserve table capacity before committing anything: the commit loop
    // below then cannot fail part-way.
    try {
        for (int32_t i = 0; i < num_seqs; ++i)
            seqs[i]->table.reserve(blocks_for((int64_t)seqs[i]->length + n_tokens[i],
                                              a->block_size));
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "append: out of host memory");
    }
    int64_t slot_off = 0;
    int32_t pairs = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int32_t np = 0;
        a->commit_append(*seqs[i], n_tokens[i], slots_out + slot_off,
                         cow_pairs_out ? cow_pairs_out + 2 * pairs : nullptr, &np);
        slot_off += n_tokens[i];
        pairs += np;
    }
    *n_cow = pairs;
    return pa::ok();
}

pa_status pa_seq_free(pa_allocator *a, int64_t seq_id) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_free: NULL allocator");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_free: no sequence %lld", (long long)seq_id);
    const std::vector<int32_t> &t = it->second.table;
    for (auto r = t.rbegin(); r != t.rend(); ++r)
        if (a->drop_ref(*r)) a->free_stack.push_back(*r);  // capacity is num_blocks
    a->seqs.erase(it);
    return pa::ok();
}

pa_status pa_seq_length(const pa_allocator *a, int64_t seq_id, int32_t *len) {
    if (!a || !len) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_length: NULL argument");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_length: no sequence %lld", (long long)seq_id);
    *len = it->second.length;
    return pa::ok();
}

pa_status pa_seq_block_table(const pa_allocator *a, int64_t seq_id, int32_t *out, int32_t cap,
                             int32_t *n_out) {
    if (!a || !n_out) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_block_table: NULL argument");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_block_table: no sequence %lld",
                        (long long)seq_id);
    const std::vector<int32_t> &t = it->second.table;
    *n_out = (int32_t)t.size();
    if ((int32_t)t.size() > cap || (!t.empty() && !out))
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_block_table: table has %zu entries, cap %d",
                        t.size(), cap);
    std::copy(t.begin(), t.end(), out);
    return pa::ok();
}

pa_status pa_batch_tables(const pa_allocator *a, int32_t num_seqs, const int64_t *seq_ids,
                          int32_t *tables_out, int32_t stride, int32_t pad_value,
                          int32_t *context_lens_out) {
    if (!a || num_seqs < 0 || stride <= 0 ||
        (num_seqs > 0 && (!seq_ids || !tables_out || !context_lens_out)))
        return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_tables: bad arguments");
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return pa::fail(PA_ERR_NOT_FOUND, "pa_batch_tables: no sequence %lld",
                            (long long)seq_ids[i]);
        if ((int32_t)it->second.table.size() > stride)
            return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_tables: sequence %lld has %zu blocks > "
                            "stride %d", (long long)seq_ids[i], it->second.table.size(), stride);
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const Sequence &s = a->seqs.find(seq_ids[i])->second;
        int32_t *row = tables_out + (int64_t)i * stride;
        std::copy(s.table.begin(), s.table.end(), row);
        std::fill(row + s.table.size(), row + stride, pad_value);
        context_lens_out[i] = s.length;
    }
    return pa::ok();
}

pa_status pa_allocator_stats(const pa_allocator *a, pa_allocator_stats_t *out) {
    if (!a || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_allocator_stats: NULL argument");
    out->num_blocks = a->num_blocks;
    out->num_free = (int32_t)a->free_stack.size();
    out->num_used = a->num_blocks - out->num_free;
    out->num_shared = a->num_shared;
    out->cow_copies = a->cow_copies;
    return pa::ok();
}

pa_status pa_block_refcount(const pa_allocator *a, int32_t block, int32_t *refcount) {
    if (!a || !refcount) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_refcount: NULL argument");
    if (block < 0 || block >= a->num_blocks)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_block_refcount: block %d out of range", block);
    *refcount = a->refcount[block];
    return pa::ok();
}

}  // extern "C"
