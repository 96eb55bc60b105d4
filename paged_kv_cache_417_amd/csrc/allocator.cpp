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
//        copy-on-write for shared prefixes, a free list popped at its end;
//        allocation first reuses blocks shareable with the request's prefix,
//        and cold blocks leave under an LRU policy.
//   [NV] practical advice — the prefix-cache hit rate as a serving metric;
//        best practice 5 — preemption swaps a request's KV cache out to CPU
//        memory and back in when room returns.
//
// State: refcount[b] per block (0 free, 1 owned, >1 shared), a free stack
// (top = back of the vector), and per sequence its table and length.  Every
// mutating call first works out everything it needs, checks it can be
// satisfied, and only then commits, so a failed call changes nothing.
//
// Prefix cache.  A block all of whose positions were appended with token ids,
// along an unbroken chain from position 0, is registered under the key
// (parent, tokens): parent is the physical block of the previous logical
// block (-1 for the first), whose own key names everything before it, so a
// key names the whole prefix exactly.  Keys live in a hash map from a 64-bit
// hash to blocks, and every hit is checked against the stored parent and
// tokens.  Released registered blocks wait in an LRU queue instead of the
// free stack; taking a block pops the stack first, then the oldest queued
// block, whose key (and its registered descendants' keys) it drops.
//
// Swap space.  A host pool of blocks with its own free stack.  Swapping a
// sequence out gives every table entry a host block (pairs for the copy) and
// releases its device blocks as pa_seq_free does; swapping in takes fresh
// device blocks and returns the host ones.  A swapped sequence's table holds
// host block ids.
//
// Host tier of the prefix cache.  Registered entries are named by node ids:
// device block b is node b, host block h is node num_blocks + h, and a key's
// parent is a node id.  pa_prefix_cache_offload moves the oldest queued
// registered blocks to free host blocks (their device blocks become free);
// an entry keeps its key across the move, and its children's keys follow
// it.  Queued descendants are older than their ancestors, so a host entry's
// registered descendants are all on the host too.  pa_seq_create_prefix_ex
// brings host entries that a prompt hits back into fresh device blocks.
// Evicting a device entry drops its subtree, host entries included, whose
// host blocks go back to the host stack lowest id on top.
#include <algorithm>
#include <functional>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

struct Sequence {
    std::vector<int32_t> table;
    int32_t length = 0;
    bool chain = true;             // every position so far came with a token id
    std::vector<int32_t> pending;  // token ids of the partial last block
    int32_t parent = -1;           // block of the last registered full block
    bool swapped = false;          // table holds host block ids
    uint64_t stamp = 0;            // batch call that last named it (repeat check)
};

// 64-bit FNV-1a over the parent id and the block's token ids.
inline uint64_t key_hash(int32_t parent, const int32_t *tokens, int32_t n) {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&h](uint32_t v) {
        for (int i = 0; i < 4; ++i) {
            h ^= (v >> (8 * i)) & 0xffu;
            h *= 1099511628211ull;
        }
    };
    mix((uint32_t)parent);
    for (int32_t i = 0; i < n; ++i) mix((uint32_t)tokens[i]);
    return h;
}

// Blocks needed for n tokens: ceil(n / bs).
inline int64_t blocks_for(int64_t n, int64_t bs) { return (n + bs - 1) / bs; }

}  // namespace

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> refcount;
    std::vector<int32_t> free_stack;
    std::unordered_map<int64_t, Sequence> seqs;  // pending reserved to block_size
    int64_t cow_copies = 0;
    int32_t num_shared = 0;
    // batch calls: a counter that stamps the sequences a call names (so a
    // repeated id is found without a set), and the call's sequence list,
    // kept between calls so a warm call allocates nothing
    uint64_t batch_epoch = 0;
    mutable std::vector<const Sequence *> batch_seqs;

    // prefix cache
    std::vector<char> registered;        // per block
    std::vector<int32_t> key_parent;     // per registered block
    std::vector<int32_t> key_tokens;     // [num_blocks][block_size], registered blocks
    std::vector<uint64_t> key_hashes;    // per registered block
    std::vector<std::vector<int32_t>> children;  // registered children per block
    std::unordered_multimap<uint64_t, int32_t> key_map;
    // Released registered blocks, oldest first: an intrusive list over the
    // block ids (no allocation once the arrays exist).
    std::vector<int32_t> lru_prev, lru_next;
    std::vector<char> in_lru;
    int32_t lru_head = -1, lru_tail = -1;
    size_t lru_size = 0;
    int64_t queried_blocks = 0, hit_blocks = 0;
    int32_t num_registered = 0;

    // swap space
    int32_t num_host_blocks = 0;
    std::vector<int32_t> host_stack;  // top = back
    int32_t num_swapped = 0;
    int64_t swap_out_blocks = 0, swap_in_blocks = 0;
    // host tier of the prefix cache
    int32_t num_host_cached = 0;
    int64_t offloaded_blocks = 0, reloaded_blocks = 0;
    std::vector<int32_t> dropped_host;  // scratch of unregister_tree

    bool cache_ready() const { return !registered.empty(); }
    int32_t num_nodes() const { return num_blocks + num_host_blocks; }
    // Per-node prefix-cache arrays (device and host blocks) and per-block
    // queue arrays, sized on first use.
    void init_cache() {
        if (cache_ready()) return;
        const size_t nn = (size_t)num_nodes();
        registered.assign(nn, 0);
        key_parent.assign(nn, -1);
        key_tokens.assign(nn * block_size, 0);
        key_hashes.assign(nn, 0);
        children.resize(nn);
        key_map.reserve(nn);  // re-keying never rehashes
        dropped_host.reserve(num_host_blocks);
        lru_prev.assign(num_blocks, -1);
        lru_next.assign(num_blocks, -1);
        in_lru.assign(num_blocks, 0);
    }
    // The node arrays after the host pool changes size (no host entries).
    void resize_nodes() {
        if (!cache_ready()) return;
        const size_t nn = (size_t)num_nodes();
        registered.resize(nn, 0);
        key_parent.resize(nn, -1);
        key_tokens.resize(nn * block_size, 0);
        key_hashes.resize(nn, 0);
        children.resize(nn);
        key_map.reserve(nn);
        dropped_host.reserve(num_host_blocks);
    }
    bool on_host(int32_t node) const { return node >= num_blocks; }
    size_t num_free() const { return free_stack.size() + lru_size; }
    void lru_push_back(int32_t b) {
        lru_prev[b] = lru_tail;
        lru_next[b] = -1;
        if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
        lru_tail = b;
        in_lru[b] = 1;
        ++lru_size;
    }
    void lru_remove(int32_t b) {
        const int32_t pv = lru_prev[b], nx = lru_next[b];
        if (pv >= 0) lru_next[pv] = nx; else lru_head = nx;
        if (nx >= 0) lru_prev[nx] = pv; else lru_tail = pv;
        in_lru[b] = 0;
        --lru_size;
    }

    int32_t lookup(int32_t parent, const int32_t *tokens) const {
        if (!cache_ready()) return -1;
        auto range = key_map.equal_range(key_hash(parent, tokens, block_size));
        for (auto it = range.first; it != range.second; ++it) {
            const int32_t b = it->second;
            if (key_parent[b] == parent &&
                std::equal(tokens, tokens + block_size,
                           key_tokens.begin() + (size_t)b * block_size))
                return b;
        }
        return -1;
    }
    // Drops the key of b and of every registered descendant (all of them are
    // queued or on the host: whoever holds a block holds its parent).  Host
    // entries among them free their host blocks, lowest id on top.
    void unregister_tree(int32_t top) {
        const int32_t p = key_parent[top];
        if (p >= 0) {
            auto &sib = children[p];
            sib.erase(std::find(sib.begin(), sib.end(), top));
        }
        dropped_host.clear();
        std::vector<int32_t> todo{top};
        while (!todo.empty()) {
            const int32_t b = todo.back();
            todo.pop_back();
            for (int32_t c : children[b]) todo.push_back(c);
            children[b].clear();
            auto range = key_map.equal_range(key_hashes[b]);
            for (auto it = range.first; it != range.second; ++it)
                if (it->second == b) {
                    key_map.erase(it);
                    break;
                }
            registered[b] = 0;
            key_parent[b] = -1;
            --num_registered;
            if (on_host(b)) dropped_host.push_back(b - num_blocks);
        }
        std::sort(dropped_host.begin(), dropped_host.end(), std::greater<int32_t>());
        for (int32_t h : dropped_host) host_stack.push_back(h);  // capacity: the pool
        num_host_cached -= (int32_t)dropped_host.size();
    }
    // Moves entry `from` to node `to` (unregistered): its key, its place in
    // its parent's children and the map, and its children's keys (whose
    // parent is now `to`).  Allocates nothing: the map has room for every
    // node and map nodes are re-keyed in place.
    void move_node(int32_t from, int32_t to) {
        const int32_t p = key_parent[from];
        registered[to] = 1;
        key_parent[to] = p;
        key_hashes[to] = key_hashes[from];
        std::copy(key_tokens.begin() + (size_t)from * block_size,
                  key_tokens.begin() + (size_t)(from + 1) * block_size,
                  key_tokens.begin() + (size_t)to * block_size);
        auto range = key_map.equal_range(key_hashes[from]);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == from) {
                it->second = to;
                break;
            }
        if (p >= 0) *std::find(children[p].begin(), children[p].end(), from) = to;
        children[to].swap(children[from]);
        for (int32_t c : children[to]) {
            auto r = key_map.equal_range(key_hashes[c]);
            for (auto it = r.first; it != r.second; ++it)
                if (it->second == c) {
                    auto nh = key_map.extract(it);
                    key_parent[c] = to;
                    key_hashes[c] = key_hash(to, key_tokens.data() + (size_t)c * block_size,
                                             block_size);
                    nh.key() = key_hashes[c];
                    key_map.insert(std::move(nh));
                    break;
                }
        }
        registered[from] = 0;
        key_parent[from] = -1;
    }
    // Registers the just-filled block b of s under (s.parent, s.pending);
    // a key already present, or no memory, ends the sequence's chain.
    void register_block(Sequence &s, int32_t b) {
        const uint64_t h = key_hash(s.parent, s.pending.data(), block_size);
        bool ok = lookup(s.parent, s.pending.data()) < 0;
        if (ok) {
            try {
                if (s.parent >= 0) children[s.parent].push_back(b);
                try {
                    key_map.emplace(h, b);
                } catch (...) {
                    if (s.parent >= 0) children[s.parent].pop_back();
                    throw;
                }
            } catch (...) {
                ok = false;
            }
        }
        if (ok) {
            registered[b] = 1;
            key_parent[b] = s.parent;
            key_hashes[b] = h;
            std::copy(s.pending.begin(), s.pending.end(),
                      key_tokens.begin() + (size_t)b * block_size);
            ++num_registered;
            s.parent = b;
        } else {
            s.chain = false;
        }
        s.pending.clear();
    }

    int32_t take() {
        int32_t b;
        if (!free_stack.empty()) {
            b = free_stack.back();
            free_stack.pop_back();
        } else {
            b = lru_head;
            lru_remove(b);
            if (registered[b]) unregister_tree(b);
        }
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
    // A block whose last reference went: queued if registered, else stacked.
    void release(int32_t b) {
        if (cache_ready() && registered[b]) {
            lru_push_back(b);
        } else {
            free_stack.push_back(b);  // capacity is num_blocks
        }
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
    void commit_append(Sequence &s, int32_t n, const int32_t *tokens, int64_t *slots,
                       int32_t *pairs, int32_t *n_pairs) {
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
        if (!tokens && n > 0) {
            s.chain = false;
            s.pending.clear();
        }
        for (int32_t i = 0; i < n; ++i) {
            int64_t pos = (int64_t)s.length + i;
            if (pos % block_size == 0) s.table.push_back(take());
            slots[i] = (int64_t)s.table[pos / block_size] * block_size + pos % block_size;
            if (tokens && s.chain) {
                s.pending.push_back(tokens[i]);  // capacity reserved by the caller
                if (pos % block_size == block_size - 1)
                    register_block(s, s.table[pos / block_size]);
            }
        }
        s.length += n;
    }
};

int32_t pa::block_size(const pa_allocator *a) { return a->block_size; }

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
    if (it->second.swapped)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: sequence %lld is swapped out",
                        (long long)parent);
    try {
        Sequence copy = it->second;
        for (int32_t b : copy.table) a->add_ref(b);
        a->seqs.emplace(child, std::move(copy));
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: out of host memory");
    }
    return pa::ok();
}

}  // extern "C"

namespace {

// Shared body of the append calls; tokens (the concatenated token ids of the
// batch) may be NULL.
pa_status batch_append(pa_allocator *a, int32_t num_seqs, const int64_t *seq_ids,
                       const int32_t *n_tokens, const int32_t *tokens, int64_t *slots_out,
                       int32_t *cow_pairs_out, int32_t cow_cap, int32_t *n_cow) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "append: NULL allocator");
    if (num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !n_tokens)) || !n_cow || cow_cap < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "append: bad arguments");
    try {
        a->batch_seqs.resize(num_seqs);
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "append: out of host memory");
    }
    Sequence **seqs = const_cast<Sequence **>(a->batch_seqs.data());
    const uint64_t epoch = ++a->batch_epoch;
    int64_t total_blocks = 0, total_tokens = 0, total_cow = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return pa::fail(PA_ERR_NOT_FOUND, "append: no sequence %lld", (long long)seq_ids[i]);
        if (it->second.stamp == epoch)
            return pa::fail(PA_ERR_INVALID_ARG, "append: repeated sequence id in batch");
        it->second.stamp = epoch;
        if (n_tokens[i] < 0)
            return pa::fail(PA_ERR_INVALID_ARG, "append: n_tokens[%d] = %d", i, n_tokens[i]);
        if ((int64_t)it->second.length + n_tokens[i] > INT32_MAX)
            return pa::fail(PA_ERR_INVALID_ARG, "append: sequence length overflows int32");
        if (it->second.swapped)
            return pa::fail(PA_ERR_INVALID_ARG, "append: sequence %lld is swapped out",
                            (long long)seq_ids[i]);
        seqs[i] = &it->second;
        int64_t blocks;
        bool c;
        a->needs(*seqs[i], n_tokens[i], &blocks, &c);
        total_blocks += blocks;
        total_tokens += n_tokens[i];
        total_cow += c ? 1 : 0;
    }
    if (total_tokens > 0 && !slots_out)
        return pa::fail(PA_ERR_INVALID_ARG, "append: slots_out is NULL");
    if (total_cow > cow_cap || (total_cow > 0 && !cow_pairs_out))
        return pa::fail(PA_ERR_INVALID_ARG, "append: %lld copy-on-write pairs, cow_cap %d",
                        (long long)total_cow, cow_cap);
    if (total_blocks > (int64_t)a->num_free())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "append: need %lld blocks, %zu free",
                        (long long)total_blocks, a->num_free());
    // Reserve table (and pending-token) capacity before committing anything:
    // the commit loop below then cannot fail part-way.
    try {
        if (tokens) a->init_cache();
        for (int32_t i = 0; i < num_seqs; ++i) {
            seqs[i]->table.reserve(blocks_for((int64_t)seqs[i]->length + n_tokens[i],
                                              a->block_size));
            if (tokens) seqs[i]->pending.reserve(a->block_size);
        }
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "append: out of host memory");
    }
    int64_t slot_off = 0;
    int32_t pairs = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int32_t np = 0;
        a->commit_append(*seqs[i], n_tokens[i], tokens ? tokens + slot_off : nullptr,
                         slots_out + slot_off, cow_pairs_out ? cow_pairs_out + 2 * pairs : nullptr,
                         &np);
        slot_off += n_tokens[i];
        pairs += np;
    }
    *n_cow = pairs;
    return pa::ok();
}

}  // namespace

extern "C" {

pa_status pa_seq_append(pa_allocator *a, int64_t seq_id, int32_t n_tokens,
                        int64_t *slots_out, int32_t *cow_pairs_out, int32_t cow_cap,
                        int32_t *n_cow) {
    return batch_append(a, 1, &seq_id, &n_tokens, nullptr, slots_out, cow_pairs_out, cow_cap,
                        n_cow);
}

pa_status pa_batch_append(pa_allocator *a, int32_t num_seqs, const int64_t *seq_ids,
                          const int32_t *n_tokens, int64_t *slots_out, int32_t *cow_pairs_out,
                          int32_t cow_cap, int32_t *n_cow) {
    return batch_append(a, num_seqs, seq_ids, n_tokens, nullptr, slots_out, cow_pairs_out,
                        cow_cap, n_cow);
}

pa_status pa_seq_append_tokens(pa_allocator *a, int64_t seq_id, const int32_t *tokens,
                               int32_t n_tokens, int64_t *slots_out, int32_t *cow_pairs_out,
                               int32_t cow_cap, int32_t *n_cow) {
    if (n_tokens > 0 && !tokens)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_tokens: tokens is NULL");
    static const int32_t kNone = 0;
    return batch_append(a, 1, &seq_id, &n_tokens, tokens ? tokens : &kNone, slots_out,
                        cow_pairs_out, cow_cap, n_cow);
}

pa_status pa_batch_append_tokens(pa_allocator *a, int32_t num_seqs, const int64_t *seq_ids,
                                 const int32_t *n_tokens, const int32_t *tokens,
                                 int64_t *slots_out, int32_t *cow_pairs_out, int32_t cow_cap,
                                 int32_t *n_cow) {
    if (!tokens)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_append_tokens: tokens is NULL");
    return batch_append(a, num_seqs, seq_ids, n_tokens, tokens, slots_out, cow_pairs_out,
                        cow_cap, n_cow);
}

}  // extern "C"

namespace {

// Shared body of pa_seq_create_prefix (host == false: a host entry ends the
// chain) and pa_seq_create_prefix_ex (host entries are brought back into
// fresh device blocks, pairs (host block, device block) out).
pa_status create_prefix(pa_allocator *a, int64_t seq_id, const int32_t *tokens,
                        int32_t n_tokens, int32_t max_cached_tokens, int32_t *n_cached,
                        bool host, int32_t *pairs_out, int32_t cap, int32_t *n_pairs) {
    const char *fn = host ? "pa_seq_create_prefix_ex" : "pa_seq_create_prefix";
    if (!a || !n_cached || n_tokens < 0 || (n_tokens > 0 && !tokens) ||
        (host && (!n_pairs || cap < 0 || (cap > 0 && !pairs_out))))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (a->seqs.count(seq_id))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: sequence %lld exists", fn, (long long)seq_id);
    const int32_t bs = a->block_size;
    const int32_t full = n_tokens / bs;
    const int32_t limit = std::min(n_tokens, std::max(max_cached_tokens, 0)) / bs;
    std::vector<int32_t> hits;
    int32_t n_dev = 0, n_host = 0;
    try {
        a->init_cache();
        // The chain: device entries first; once an entry is on the host, so
        // are all the rest (a host entry's descendants are on the host).
        int32_t parent = -1;
        for (int32_t j = 0; j < limit; ++j) {
            const int32_t b = a->lookup(parent, tokens + (int64_t)j * bs);
            if (b < 0 || (a->on_host(b) && !host)) break;
            hits.push_back(b);
            parent = b;
        }
        // Device hits with no holder leave the free count once reused; each
        // host hit then needs a free device block (and a pair slot).
        int64_t avail = (int64_t)a->num_free();
        for (int32_t b : hits) {
            if (a->on_host(b)) break;
            ++n_dev;
            if (a->refcount[b] == 0) --avail;
        }
        n_host = (int32_t)std::min<int64_t>({(int64_t)hits.size() - n_dev, std::max<int64_t>(avail, 0),
                                             (int64_t)cap});
        if (!host) n_host = 0;
        hits.resize(n_dev + n_host);
        Sequence s;
        s.table = hits;
        s.length = (int32_t)hits.size() * bs;
        s.pending.reserve(bs);
        a->seqs.emplace(seq_id, std::move(s));
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    Sequence &s = a->seqs.find(seq_id)->second;
    for (int32_t j = 0; j < n_dev; ++j) {
        const int32_t b = hits[j];
        if (a->refcount[b] == 0) {
            a->lru_remove(b);
            a->refcount[b] = 1;
        } else {
            a->add_ref(b);
        }
    }
    // Every device hit is held now, so taking a block cannot evict one of
    // them or an ancestor of the host hits.
    for (int32_t j = n_dev; j < n_dev + n_host; ++j) {
        const int32_t node = hits[j];
        const int32_t d = a->take();
        a->move_node(node, d);
        a->host_stack.push_back(node - a->num_blocks);  // capacity: the pool
        pairs_out[2 * (j - n_dev)] = node - a->num_blocks;
        pairs_out[2 * (j - n_dev) + 1] = d;
        s.table[j] = d;
    }
    a->num_host_cached -= n_host;
    a->reloaded_blocks += n_host;
    s.parent = s.table.empty() ? -1 : s.table.back();
    a->queried_blocks += full;
    a->hit_blocks += (int64_t)s.table.size();
    *n_cached = (int32_t)s.table.size() * bs;
    if (host) *n_pairs = n_host;
    return pa::ok();
}

}  // namespace

extern "C" {

pa_status pa_seq_create_prefix(pa_allocator *a, int64_t seq_id, const int32_t *tokens,
                               int32_t n_tokens, int32_t max_cached_tokens, int32_t *n_cached) {
    return create_prefix(a, seq_id, tokens, n_tokens, max_cached_tokens, n_cached, false,
                         nullptr, 0, nullptr);
}

pa_status pa_seq_create_prefix_ex(pa_allocator *a, int64_t seq_id, const int32_t *tokens,
                                  int32_t n_tokens, int32_t max_cached_tokens, int32_t *n_cached,
                                  int32_t *pairs_out, int32_t cap, int32_t *n_pairs) {
    return create_prefix(a, seq_id, tokens, n_tokens, max_cached_tokens, n_cached, true,
                         pairs_out, cap, n_pairs);
}

pa_status pa_prefix_cache_offload(pa_allocator *a, int32_t max_blocks, int32_t *pairs_out,
                                  int32_t cap, int32_t *n_pairs) {
    const char *fn = "pa_prefix_cache_offload";
    if (!a || !n_pairs || max_blocks < 0 || cap < 0 || (cap > 0 && !pairs_out))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    int32_t n = 0;
    const int32_t limit = std::min(max_blocks, cap);
    if (a->cache_ready()) {
        for (int32_t b = a->lru_head; b >= 0 && n < limit && !a->host_stack.empty();) {
            const int32_t next = a->lru_next[b];
            if (a->registered[b]) {
                const int32_t h = a->host_stack.back();
                a->host_stack.pop_back();
                a->move_node(b, a->num_blocks + h);
                a->lru_remove(b);
                a->free_stack.push_back(b);  // capacity is num_blocks
                pairs_out[2 * n] = b;
                pairs_out[2 * n + 1] = h;
                ++n;
            }
            b = next;
        }
    }
    a->num_host_cached += n;
    a->offloaded_blocks += n;
    *n_pairs = n;
    return pa::ok();
}

pa_status pa_prefix_host_stats(const pa_allocator *a, pa_prefix_host_stats_t *out) {
    if (!a || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_prefix_host_stats: NULL argument");
    out->host_cached_blocks = a->num_host_cached;
    out->offloaded_blocks = a->offloaded_blocks;
    out->reloaded_blocks = a->reloaded_blocks;
    return pa::ok();
}

pa_status pa_prefix_cache_stats(const pa_allocator *a, pa_prefix_stats_t *out) {
    if (!a || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_prefix_cache_stats: NULL argument");
    out->queried_blocks = a->queried_blocks;
    out->hit_blocks = a->hit_blocks;
    out->cached_blocks = a->num_registered;
    int32_t queued = 0;
    for (int32_t b = a->lru_head; b >= 0; b = a->lru_next[b]) queued += a->registered[b] ? 1 : 0;
    out->cached_free_blocks = queued;
    return pa::ok();
}

pa_status pa_seq_free(pa_allocator *a, int64_t seq_id) {
    if (!a) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_free: NULL allocator");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_free: no sequence %lld", (long long)seq_id);
    const std::vector<int32_t> &t = it->second.table;
    if (it->second.swapped) {
        for (auto r = t.rbegin(); r != t.rend(); ++r) a->host_stack.push_back(*r);
        --a->num_swapped;
    } else {
        for (auto r = t.rbegin(); r != t.rend(); ++r)
            if (a->drop_ref(*r)) a->release(*r);
    }
    a->seqs.erase(it);
    return pa::ok();
}

pa_status pa_seq_blocks_needed(const pa_allocator *a, int64_t seq_id, int32_t n_tokens,
                               int32_t *blocks) {
    if (!a || !blocks || n_tokens < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_blocks_needed: bad arguments");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_blocks_needed: no sequence %lld",
                        (long long)seq_id);
    if (it->second.swapped)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_blocks_needed: sequence %lld is swapped out",
                        (long long)seq_id);
    int64_t b;
    bool cow;
    a->needs(it->second, n_tokens, &b, &cow);
    *blocks = (int32_t)b;
    return pa::ok();
}

pa_status pa_seq_num_blocks(const pa_allocator *a, int64_t seq_id, int32_t *n_blocks) {
    if (!a || !n_blocks) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_num_blocks: NULL argument");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_num_blocks: no sequence %lld",
                        (long long)seq_id);
    *n_blocks = (int32_t)it->second.table.size();
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
    try {
        a->batch_seqs.resize(num_seqs);
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_tables: out of host memory");
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return pa::fail(PA_ERR_NOT_FOUND, "pa_batch_tables: no sequence %lld",
                            (long long)seq_ids[i]);
        if (it->second.swapped)
            return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_tables: sequence %lld is swapped out",
                            (long long)seq_ids[i]);
        if ((int32_t)it->second.table.size() > stride)
            return pa::fail(PA_ERR_INVALID_ARG, "pa_batch_tables: sequence %lld has %zu blocks > "
                            "stride %d", (long long)seq_ids[i], it->second.table.size(), stride);
        a->batch_seqs[i] = &it->second;
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const Sequence &s = *a->batch_seqs[i];
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
    out->num_free = (int32_t)a->num_free();
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

pa_status pa_allocator_set_swap_space(pa_allocator *a, int32_t num_host_blocks) {
    const char *fn = "pa_allocator_set_swap_space";
    if (!a || num_host_blocks < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (a->num_swapped > 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %d sequences are swapped out", fn,
                        a->num_swapped);
    if (a->num_host_cached > 0)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %d prefix-cache blocks are on the host", fn,
                        a->num_host_cached);
    const int32_t old_n = a->num_host_blocks;
    try {
        std::vector<int32_t> st(num_host_blocks);
        for (int32_t i = 0; i < num_host_blocks; ++i) st[i] = num_host_blocks - 1 - i;
        a->num_host_blocks = num_host_blocks;
        a->resize_nodes();
        a->host_stack.swap(st);
    } catch (...) {
        a->num_host_blocks = old_n;
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    return pa::ok();
}

pa_status pa_seq_swap_out(pa_allocator *a, int64_t seq_id, int32_t *pairs_out, int32_t cap,
                          int32_t *n_pairs) {
    const char *fn = "pa_seq_swap_out";
    if (!a || !n_pairs || cap < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "%s: no sequence %lld", fn, (long long)seq_id);
    Sequence &s = it->second;
    if (s.swapped)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: sequence %lld is swapped out", fn,
                        (long long)seq_id);
    const size_t n = s.table.size();
    if ((int64_t)n > cap || (n > 0 && !pairs_out))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %zu pairs, cap %d", fn, n, cap);
    if (n > a->host_stack.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "%s: need %zu host blocks, %zu free", fn, n,
                        a->host_stack.size());
    for (size_t j = 0; j < n; ++j) {
        const int32_t h = a->host_stack.back();
        a->host_stack.pop_back();
        pairs_out[2 * j] = s.table[j];
        pairs_out[2 * j + 1] = h;
    }
    for (size_t j = n; j-- > 0;)  // device blocks released last entry first
        if (a->drop_ref(s.table[j])) a->release(s.table[j]);
    for (size_t j = 0; j < n; ++j) s.table[j] = pairs_out[2 * j + 1];
    s.swapped = true;
    ++a->num_swapped;
    a->swap_out_blocks += (int64_t)n;
    *n_pairs = (int32_t)n;
    return pa::ok();
}

pa_status pa_seq_swap_in(pa_allocator *a, int64_t seq_id, int32_t *pairs_out, int32_t cap,
                         int32_t *n_pairs) {
    const char *fn = "pa_seq_swap_in";
    if (!a || !n_pairs || cap < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "%s: no sequence %lld", fn, (long long)seq_id);
    Sequence &s = it->second;
    if (!s.swapped)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: sequence %lld is not swapped out", fn,
                        (long long)seq_id);
    const size_t n = s.table.size();
    if ((int64_t)n > cap || (n > 0 && !pairs_out))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %zu pairs, cap %d", fn, n, cap);
    if (n > a->num_free())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "%s: need %zu blocks, %zu free", fn, n,
                        a->num_free());
    for (size_t j = 0; j < n; ++j) {
        pairs_out[2 * j] = s.table[j];
        pairs_out[2 * j + 1] = a->take();
    }
    for (size_t j = n; j-- > 0;) a->host_stack.push_back(s.table[j]);  // capacity kept
    for (size_t j = 0; j < n; ++j) s.table[j] = pairs_out[2 * j + 1];
    s.swapped = false;
    s.chain = false;  // fresh private blocks: the registered chain is gone
    s.pending.clear();
    --a->num_swapped;
    a->swap_in_blocks += (int64_t)n;
    *n_pairs = (int32_t)n;
    return pa::ok();
}

pa_status pa_seq_is_swapped(const pa_allocator *a, int64_t seq_id, int32_t *swapped) {
    if (!a || !swapped) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_is_swapped: NULL argument");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_is_swapped: no sequence %lld",
                        (long long)seq_id);
    *swapped = it->second.swapped ? 1 : 0;
    return pa::ok();
}

pa_status pa_swap_stats(const pa_allocator *a, pa_swap_stats_t *out) {
    if (!a || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_swap_stats: NULL argument");
    out->num_host_blocks = a->num_host_blocks;
    out->num_host_free = (int32_t)a->host_stack.size();
    out->swapped_seqs = a->num_swapped;
    out->swap_out_blocks = a->swap_out_blocks;
    out->swap_in_blocks = a->swap_in_blocks;
    return pa::ok();
}

}  // extern "C"
