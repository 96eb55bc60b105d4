// scheduler.cpp — continuous-batching host scheduler over the block
// allocator: each step plans which requests decode, which prompt chunks are
// written, which requests are preempted (swap or recompute) or resumed, and
// every slot and block copy the caller must carry out on the GPU.
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.2 — continuous batching: requests
//        join the running batch at every iteration and leave as soon as they
//        finish.
//   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1 — prefill and
//        decode share an iteration; §2.2 — a pending queue, first blocks at
//        admission, resources released at once when a request finishes.
//   [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 best practice 5 —
//        first-come first-served; preemption moves a request's KV cache to CPU
//        memory and brings it back when room returns.
//
// Policy, step by step (the pages leave the details open):
//   1. Decode set = running requests whose prompt is written, in admission
//      order.  While the pool cannot hold one more position for each, the
//      most recently admitted running request is preempted: swapped out when
//      the host pool holds its blocks, else sent back to the head of the
//      waiting queue to start over.
//   2. Their positions are appended.
//   3. The token budget (max_batched_tokens minus the decode count) goes to
//      requests still in their prompt, in admission order, min(rest, budget,
//      max_prefill_chunk) positions each, while the pool holds them.
//   4. Swapped requests return in arrival order while fewer than
//      max_num_seqs run and the pool holds their blocks (no work that step).
//   5. Waiting requests are admitted in queue order while fewer than
//      max_num_seqs run, budget remains and the pool holds their first chunk;
//      a request with token ids first reuses its cached prompt blocks.
// The step that writes a prompt's last chunk yields its first token; each
// decode yields one more; at max_new tokens the request finishes and its
// blocks are freed (pa_sched_complete).
//
// Parallel sampling ([VE] §3.1: several outputs drawn from one prompt share
// its KV blocks, with copy-on-write on the block where they diverge): a
// request may ask for n samples.  It runs as one sequence until its prompt
// is written; pa_sched_complete of that step forks samples 2..n from it
// (pa_seq_fork), so all n hold the prompt's blocks and the first append of
// each into the shared partial block copies it.  From then on the request's
// n sequences decode side by side, adjacent in the decode order (the
// request's own id first), and are preempted, resumed and finished
// together.  max_num_seqs counts sequences: a request holds n of them from
// admission on.
#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

enum class St { Waiting, Running, Swapped, Finished };

struct Req {
    int64_t id = 0;
    int32_t n_prompt = 0, max_new = 0;
    std::vector<int32_t> tokens;  // empty: no token ids
    int64_t order = 0;
    int32_t done = 0, generated = 0;
    St state = St::Waiting;
    std::vector<int64_t> samples;  // ids of samples 2..n
    bool forked = false;           // the samples exist in the allocator

    int32_t seqs() const { return 1 + (int32_t)samples.size(); }
    // Calls f on each sequence that holds blocks now: the request's own id,
    // then its samples once forked; stops at the first nonzero status.
    template <class F>
    pa_status each_seq(F f) const {
        if (pa_status e = f(id)) return e;
        if (forked)
            for (int64_t x : samples)
                if (pa_status e = f(x)) return e;
        return PA_OK;
    }
};

}  // namespace

struct pa_sched {
    pa_allocator *a = nullptr;
    int32_t max_seqs = 0, max_tokens = 0, chunk = 0;
    std::unordered_map<int64_t, Req> reqs;
    std::unordered_map<int64_t, int64_t> sample_of;  // sample id -> its request
    std::deque<int64_t> waiting;
    std::vector<int64_t> running, swapped;  // request ids
    int32_t running_seqs = 0;               // seqs() summed over running
    int64_t arrivals = 0, swap_preempt = 0, recompute_preempt = 0, finished = 0, forks = 0;
    // the last plan, for pa_sched_complete
    std::vector<int64_t> last_decode;  // request ids
    std::vector<std::pair<int64_t, int32_t>> last_prefill_end;  // (id, start + len)
    bool plan_pending = false;
};

namespace {

int32_t free_blocks(const pa_allocator *a) {
    pa_allocator_stats_t st;
    pa_allocator_stats(a, &st);
    return st.num_free;
}

int32_t host_free(const pa_allocator *a) {
    pa_swap_stats_t st;
    pa_swap_stats(a, &st);
    return st.num_host_free;
}

int32_t need(const pa_allocator *a, int64_t id, int32_t n) {
    int32_t b = 0;
    pa_seq_blocks_needed(a, id, n, &b);
    return b;
}

int32_t nblocks(const pa_allocator *a, int64_t id) {
    int32_t n = 0;
    pa_seq_num_blocks(a, id, &n);
    return n;
}

// Appends n positions to sequence seq (prompt token ids toks, or NULL) and
// writes the slots and copy-on-write pairs into the plan.
pa_status append_into(pa_sched *s, int64_t seq, const int32_t *toks, int32_t n,
                      pa_sched_plan_t *p) {
    int32_t ncow = 0;
    pa_status st = toks ? pa_seq_append_tokens(s->a, seq, toks, n, p->slots + p->n_slots,
                                               p->cow_pairs + 2 * p->n_cow, p->cap_cow - p->n_cow,
                                               &ncow)
                        : pa_seq_append(s->a, seq, n, p->slots + p->n_slots,
                                        p->cow_pairs + 2 * p->n_cow, p->cap_cow - p->n_cow, &ncow);
    if (st) return st;
    p->n_slots += n;
    p->n_cow += ncow;
    return PA_OK;
}

// Blocks held by all of r's sequences, counted per sequence.
int32_t req_blocks(const pa_allocator *a, const Req &r) {
    int32_t n = 0;
    r.each_seq([&](int64_t x) {
        n += nblocks(a, x);
        return PA_OK;
    });
    return n;
}

bool id_taken(const pa_sched *s, int64_t id) {
    return s->reqs.count(id) || s->sample_of.count(id);
}

}  // namespace

extern "C" {

pa_status pa_sched_create(pa_allocator *a, int32_t max_num_seqs, int32_t max_batched_tokens,
                          int32_t max_prefill_chunk, pa_sched **out) {
    if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_create: out is NULL");
    *out = nullptr;
    if (!a || max_num_seqs <= 0 || max_batched_tokens <= 0 || max_prefill_chunk <= 0)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_create: bad arguments");
    if (max_batched_tokens < max_num_seqs)
        return pa::fail(PA_ERR_INVALID_ARG,
                        "pa_sched_create: max_batched_tokens %d < max_num_seqs %d (a step "
                        "decodes up to max_num_seqs positions)", max_batched_tokens,
                        max_num_seqs);
    pa_sched *s = new (std::nothrow) pa_sched;
    if (!s) return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_create: out of host memory");
    s->a = a;
    s->max_seqs = max_num_seqs;
    s->max_tokens = max_batched_tokens;
    s->chunk = max_prefill_chunk;
    *out = s;
    return pa::ok();
}

void pa_sched_destroy(pa_sched *s) { delete s; }

pa_status pa_sched_add_samples(pa_sched *s, int64_t id, int32_t n_prompt, int32_t max_new,
                               const int32_t *tokens, const int64_t *sample_ids,
                               int32_t num_samples) {
    const char *fn = "pa_sched_add";
    if (!s || n_prompt < 1 || max_new < 1 || num_samples < 1 ||
        (num_samples > 1 && !sample_ids))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (num_samples > s->max_seqs)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: %d samples > max_num_seqs %d", fn, num_samples,
                        s->max_seqs);
    if (id_taken(s, id))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: id %lld is taken", fn, (long long)id);
    {
        // Alone in the pool the request must be able to finish, else it
        // would be preempted and restarted for ever: each sequence ends at
        // n_prompt + max_new - 1 positions, samples may hold private copies
        // of every block (after a swap), and a fork's shared partial block
        // is counted once more by the decode-set check.
        pa_allocator_stats_t ast;
        pa_allocator_stats(s->a, &ast);
        const int64_t bs = pa::block_size(s->a);
        const int64_t per_seq = ((int64_t)n_prompt + max_new - 1 + bs - 1) / bs;
        const int64_t most = per_seq * num_samples + (num_samples > 1 ? 1 : 0);
        if (most > ast.num_blocks)
            return pa::fail(PA_ERR_INVALID_ARG,
                            "%s: the request may need %lld blocks, the pool has %d", fn,
                            (long long)most, ast.num_blocks);
    }
    for (int32_t i = 0; i + 1 < num_samples; ++i) {
        const int64_t x = sample_ids[i];
        bool dup = x == id || id_taken(s, x);
        for (int32_t j = 0; j < i && !dup; ++j) dup = sample_ids[j] == x;
        if (dup) return pa::fail(PA_ERR_INVALID_ARG, "%s: sample id %lld is taken", fn,
                                 (long long)x);
    }
    try {
        Req r;
        r.id = id;
        r.n_prompt = n_prompt;
        r.max_new = max_new;
        if (tokens) r.tokens.assign(tokens, tokens + n_prompt);
        if (num_samples > 1) r.samples.assign(sample_ids, sample_ids + num_samples - 1);
        r.order = s->arrivals;
        auto it = s->reqs.emplace(id, std::move(r)).first;  // throws: nothing changed
        try {
            for (int32_t i = 0; i + 1 < num_samples; ++i) s->sample_of.emplace(sample_ids[i], id);
            s->waiting.push_back(id);
        } catch (...) {
            for (int32_t i = 0; i + 1 < num_samples; ++i) s->sample_of.erase(sample_ids[i]);
            s->reqs.erase(it);
            throw;
        }
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    ++s->arrivals;
    return pa::ok();
}

pa_status pa_sched_add(pa_sched *s, int64_t id, int32_t n_prompt, int32_t max_new,
                       const int32_t *tokens) {
    return pa_sched_add_samples(s, id, n_prompt, max_new, tokens, nullptr, 1);
}

pa_status pa_sched_step(pa_sched *s, pa_sched_plan_t *p) {
    const char *fn = "pa_sched_step";
    if (!s || !p) return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL argument", fn);
    if (s->plan_pending)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: the previous plan was not completed", fn);
    pa_allocator_stats_t ast;
    pa_allocator_stats(s->a, &ast);
    pa_swap_stats_t sst;
    pa_swap_stats(s->a, &sst);
    // a step's swap-out pairs each take a host block, its swap-in pairs each
    // a device block
    const int32_t cap_swap = std::max(ast.num_blocks, sst.num_host_blocks);
    if (p->cap_seqs < s->max_seqs || p->cap_slots < s->max_tokens ||
        p->cap_cow < s->max_seqs || p->cap_swap_pairs < cap_swap ||
        !p->decode_ids || !p->decode_lens || !p->prefill_ids || !p->prefill_starts ||
        !p->prefill_lens || !p->slots || !p->swap_out_pairs || !p->swap_in_pairs ||
        !p->cow_pairs || !p->preempted_ids)
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: plan arrays missing or short (need %d sequences, %d slots, %d copy "
                        "pairs, %d swap pairs)", fn, s->max_seqs, s->max_tokens, s->max_seqs,
                        cap_swap);
    p->n_decode = p->n_prefill = p->n_slots = p->n_swap_out = p->n_swap_in = p->n_cow =
        p->n_preempted = 0;
    pa_allocator *a = s->a;
    std::vector<int64_t> dec;  // request ids
    pa_status st = PA_OK;
    try {
        // 1. decode set, preempting the newest running request while it does not fit
        for (;;) {
            dec.clear();
            int64_t want = 0;
            for (int64_t id : s->running) {
                const Req &r = s->reqs[id];
                if (r.done == r.n_prompt) {
                    dec.push_back(id);
                    r.each_seq([&](int64_t x) {
                        want += need(a, x, 1);
                        return PA_OK;
                    });
                }
            }
            if (want <= free_blocks(a) || s->running.empty()) break;
            const int64_t victim = s->running.back();
            s->running.pop_back();
            Req &v = s->reqs[victim];
            s->running_seqs -= v.seqs();
            if (req_blocks(a, v) <= host_free(a)) {
                if ((st = v.each_seq([&](int64_t x) {
                         int32_t n = 0;
                         pa_status e = pa_seq_swap_out(a, x, p->swap_out_pairs + 2 * p->n_swap_out,
                                                       p->cap_swap_pairs - p->n_swap_out, &n);
                         p->n_swap_out += n;
                         return e;
                     })))
                    return st;
                v.state = St::Swapped;
                s->swapped.push_back(victim);
                std::stable_sort(s->swapped.begin(), s->swapped.end(), [s](int64_t x, int64_t y) {
                    return s->reqs[x].order < s->reqs[y].order;
                });
                ++s->swap_preempt;
            } else {
                v.each_seq([&](int64_t x) { return pa_seq_free(a, x); });
                v.state = St::Waiting;
                v.done = v.generated = 0;
                v.forked = false;
                s->waiting.push_front(victim);
                p->preempted_ids[p->n_preempted++] = victim;
                ++s->recompute_preempt;
            }
        }
        // 2. decode positions: each request's sequences in a row
        for (int64_t id : dec) {
            if ((st = s->reqs[id].each_seq([&](int64_t x) {
                     if (pa_status e = append_into(s, x, nullptr, 1, p)) return e;
                     int32_t len = 0;
                     pa_seq_length(a, x, &len);
                     p->decode_ids[p->n_decode] = x;
                     p->decode_lens[p->n_decode++] = len;
                     return PA_OK;
                 })))
                return st;
        }
        int32_t budget = s->max_tokens - p->n_decode;
        auto prompt_chunk = [&](Req &r, int32_t c) -> pa_status {
            const int32_t *toks = r.tokens.empty() ? nullptr : r.tokens.data() + r.done;
            if (pa_status e = append_into(s, r.id, toks, c, p)) return e;
            p->prefill_ids[p->n_prefill] = r.id;
            p->prefill_starts[p->n_prefill] = r.done;
            p->prefill_lens[p->n_prefill++] = c;
            r.done += c;
            budget -= c;
            return PA_OK;
        };
        // 3. prompts in progress
        for (int64_t id : std::vector<int64_t>(s->running)) {
            Req &r = s->reqs[id];
            if (r.done == r.n_prompt) continue;
            const int32_t c = std::min({r.n_prompt - r.done, budget, s->chunk});
            if (c <= 0 || need(a, id, c) > free_blocks(a)) break;
            if ((st = prompt_chunk(r, c))) return st;
        }
        // 4. swapped requests come back
        while (!s->swapped.empty()) {
            const int64_t id = s->swapped.front();
            Req &r = s->reqs[id];
            if (s->running_seqs + r.seqs() > s->max_seqs || req_blocks(a, r) > free_blocks(a))
                break;
            if ((st = r.each_seq([&](int64_t x) {
                     int32_t n = 0;
                     pa_status e = pa_seq_swap_in(a, x, p->swap_in_pairs + 2 * p->n_swap_in,
                                                  p->cap_swap_pairs - p->n_swap_in, &n);
                     p->n_swap_in += n;
                     return e;
                 })))
                return st;
            s->swapped.erase(s->swapped.begin());
            r.state = St::Running;
            s->running.push_back(id);
            s->running_seqs += r.seqs();
        }
        // 5. admissions
        while (!s->waiting.empty() && budget > 0) {
            Req &r = s->reqs[s->waiting.front()];
            if (s->running_seqs + r.seqs() > s->max_seqs) break;
            int32_t cached = 0;
            if (!r.tokens.empty()) {
                if ((st = pa_seq_create_prefix(a, r.id, r.tokens.data(), r.n_prompt,
                                               r.n_prompt - 1, &cached)))
                    return st;
            } else if ((st = pa_seq_create(a, r.id))) {
                return st;
            }
            const int32_t c = std::min({r.n_prompt - cached, budget, s->chunk});
            if (need(a, r.id, c) > free_blocks(a)) {
                pa_seq_free(a, r.id);  // not admitted: reused blocks go back
                break;
            }
            s->waiting.pop_front();
            r.done = cached;
            r.state = St::Running;
            s->running.push_back(r.id);
            s->running_seqs += r.seqs();
            if ((st = prompt_chunk(r, c))) return st;
        }
        s->last_decode = dec;
        s->last_prefill_end.clear();
        for (int32_t i = 0; i < p->n_prefill; ++i)
            s->last_prefill_end.emplace_back(p->prefill_ids[i],
                                             p->prefill_starts[i] + p->prefill_lens[i]);
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    s->plan_pending = true;
    return pa::ok();
}

pa_status pa_sched_complete(pa_sched *s, int64_t *finished_ids, int32_t cap,
                            int32_t *n_finished) {
    const char *fn = "pa_sched_complete";
    if (!s || !n_finished || cap < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (!s->plan_pending) return pa::fail(PA_ERR_INVALID_ARG, "%s: no plan to complete", fn);
    if (cap < s->running_seqs || (s->running_seqs && !finished_ids))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: cap %d < %d running sequences", fn, cap,
                        s->running_seqs);
    std::vector<int64_t> keep, to_fork;
    try {
        keep.reserve(s->running.size());
        for (auto &e : s->last_prefill_end) {
            const Req &r = s->reqs[e.first];
            if (e.second == r.n_prompt && r.state == St::Running && !r.samples.empty())
                to_fork.push_back(r.id);
        }
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    // Fork first: a failure (an id the caller took in the allocator, host
    // memory) undoes the forks made so far and leaves the plan pending.
    for (size_t i = 0; i < to_fork.size(); ++i) {
        const Req &r = s->reqs[to_fork[i]];
        for (size_t j = 0; j < r.samples.size(); ++j) {
            if (pa_status st = pa_seq_fork(s->a, r.id, r.samples[j])) {
                for (size_t jj = 0; jj < j; ++jj) pa_seq_free(s->a, r.samples[jj]);
                for (size_t ii = 0; ii < i; ++ii)
                    for (int64_t x : s->reqs[to_fork[ii]].samples) pa_seq_free(s->a, x);
                return st;
            }
        }
    }
    for (int64_t id : to_fork) {
        Req &r = s->reqs[id];
        r.forked = true;
        s->forks += (int64_t)r.samples.size();
    }
    for (int64_t id : s->last_decode) ++s->reqs[id].generated;
    for (auto &e : s->last_prefill_end) {
        Req &r = s->reqs[e.first];
        if (e.second == r.n_prompt && r.state == St::Running) ++r.generated;
    }
    int32_t n = 0;
    for (int64_t id : s->running) {
        Req &r = s->reqs[id];
        if (r.generated >= r.max_new) {
            r.each_seq([&](int64_t x) {
                finished_ids[n++] = x;
                return pa_seq_free(s->a, x);
            });
            s->running_seqs -= r.seqs();
            r.state = St::Finished;
            ++s->finished;
        } else {
            keep.push_back(id);
        }
    }
    s->running.swap(keep);
    s->plan_pending = false;
    *n_finished = n;
    return pa::ok();
}

pa_status pa_sched_stats(const pa_sched *s, pa_sched_stats_t *out) {
    if (!s || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_stats: NULL argument");
    out->waiting = (int32_t)s->waiting.size();
    out->running = (int32_t)s->running.size();
    out->swapped = (int32_t)s->swapped.size();
    out->running_seqs = s->running_seqs;
    out->finished = s->finished;
    out->swap_preemptions = s->swap_preempt;
    out->recompute_preemptions = s->recompute_preempt;
    out->forked_samples = s->forks;
    return pa::ok();
}

}  // extern "C"
