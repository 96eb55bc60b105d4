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
};

}  // namespace

struct pa_sched {
    pa_allocator *a = nullptr;
    int32_t max_seqs = 0, max_tokens = 0, chunk = 0;
    std::unordered_map<int64_t, Req> reqs;
    std::deque<int64_t> waiting;
    std::vector<int64_t> running, swapped;
    int64_t arrivals = 0, swap_preempt = 0, recompute_preempt = 0, finished = 0;
    // the last plan, for pa_sched_complete
    std::vector<int64_t> last_decode;
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

// Writes appended slots and copy-on-write pairs into the plan.
pa_status append_into(pa_sched *s, Req &r, int32_t n, bool prompt, pa_sched_plan_t *p) {
    int32_t ncow = 0;
    const int32_t *toks = prompt && !r.tokens.empty() ? r.tokens.data() + r.done : nullptr;
    pa_status st = toks ? pa_seq_append_tokens(s->a, r.id, toks, n, p->slots + p->n_slots,
                                               p->cow_pairs + 2 * p->n_cow, p->cap_cow - p->n_cow,
                                               &ncow)
                        : pa_seq_append(s->a, r.id, n, p->slots + p->n_slots,
                                        p->cow_pairs + 2 * p->n_cow, p->cap_cow - p->n_cow, &ncow);
    if (st) return st;
    p->n_slots += n;
    p->n_cow += ncow;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_sched_create(pa_allocator *a, int32_t max_num_seqs, int32_t max_batched_tokens,
                          int32_t max_prefill_chunk, pa_sched **out) {
    if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_create: out is NULL");
    *out = nullptr;
    if (!a || max_num_seqs <= 0 || max_batched_tokens <= 0 || max_prefill_chunk <= 0)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_create: bad arguments");
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

pa_status pa_sched_add(pa_sched *s, int64_t id, int32_t n_prompt, int32_t max_new,
                       const int32_t *tokens) {
    if (!s || n_prompt < 1 || max_new < 1)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_add: bad arguments");
    if (s->reqs.count(id))
        return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_add: request %lld exists", (long long)id);
    try {
        Req r;
        r.id = id;
        r.n_prompt = n_prompt;
        r.max_new = max_new;
        if (tokens) r.tokens.assign(tokens, tokens + n_prompt);
        r.order = s->arrivals;
        s->waiting.push_back(id);
        try {
            s->reqs.emplace(id, std::move(r));
        } catch (...) {
            s->waiting.pop_back();
            throw;
        }
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "pa_sched_add: out of host memory");
    }
    ++s->arrivals;
    return pa::ok();
}

pa_status pa_sched_step(pa_sched *s, pa_sched_plan_t *p) {
    const char *fn = "pa_sched_step";
    if (!s || !p) return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL argument", fn);
    if (s->plan_pending)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: the previous plan was not completed", fn);
    pa_allocator_stats_t ast;
    pa_allocator_stats(s->a, &ast);
    if (p->cap_seqs < s->max_seqs || p->cap_slots < s->max_tokens ||
        p->cap_cow < s->max_seqs || p->cap_swap_pairs < ast.num_blocks ||
        !p->decode_ids || !p->decode_lens || !p->prefill_ids || !p->prefill_starts ||
        !p->prefill_lens || !p->slots || !p->swap_out_pairs || !p->swap_in_pairs ||
        !p->cow_pairs || !p->preempted_ids)
        return pa::fail(PA_ERR_INVALID_ARG,
                        "%s: plan arrays missing or short (need %d sequences, %d slots, %d copy "
                        "pairs, %d swap pairs)", fn, s->max_seqs, s->max_tokens, s->max_seqs,
                        ast.num_blocks);
    p->n_decode = p->n_prefill = p->n_slots = p->n_swap_out = p->n_swap_in = p->n_cow =
        p->n_preempted = 0;
    pa_allocator *a = s->a;
    std::vector<int64_t> dec;
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
                    want += need(a, id, 1);
                }
            }
            if (want <= free_blocks(a) || s->running.empty()) break;
            const int64_t victim = s->running.back();
            s->running.pop_back();
            Req &v = s->reqs[victim];
            if (nblocks(a, victim) <= host_free(a)) {
                int32_t n = 0;
                if ((st = pa_seq_swap_out(a, victim, p->swap_out_pairs + 2 * p->n_swap_out,
                                          p->cap_swap_pairs - p->n_swap_out, &n)))
                    return st;
                p->n_swap_out += n;
                v.state = St::Swapped;
                s->swapped.push_back(victim);
                std::stable_sort(s->swapped.begin(), s->swapped.end(), [s](int64_t x, int64_t y) {
                    return s->reqs[x].order < s->reqs[y].order;
                });
                ++s->swap_preempt;
            } else {
                pa_seq_free(a, victim);
                v.state = St::Waiting;
                v.done = v.generated = 0;
                s->waiting.push_front(victim);
                p->preempted_ids[p->n_preempted++] = victim;
                ++s->recompute_preempt;
            }
        }
        // 2. decode positions
        for (int64_t id : dec) {
            if ((st = append_into(s, s->reqs[id], 1, false, p))) return st;
            int32_t len = 0;
            pa_seq_length(a, id, &len);
            p->decode_ids[p->n_decode] = id;
            p->decode_lens[p->n_decode++] = len;
        }
        int32_t budget = s->max_tokens - (int32_t)dec.size();
        auto prompt_chunk = [&](Req &r, int32_t c) -> pa_status {
            if (pa_status e = append_into(s, r, c, true, p)) return e;
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
        while (!s->swapped.empty() && (int32_t)s->running.size() < s->max_seqs) {
            const int64_t id = s->swapped.front();
            if (nblocks(a, id) > free_blocks(a)) break;
            int32_t n = 0;
            if ((st = pa_seq_swap_in(a, id, p->swap_in_pairs + 2 * p->n_swap_in,
                                     p->cap_swap_pairs - p->n_swap_in, &n)))
                return st;
            p->n_swap_in += n;
            s->swapped.erase(s->swapped.begin());
            s->reqs[id].state = St::Running;
            s->running.push_back(id);
        }
        // 5. admissions
        while (!s->waiting.empty() && (int32_t)s->running.size() < s->max_seqs && budget > 0) {
            Req &r = s->reqs[s->waiting.front()];
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
            if ((st = prompt_chunk(r, c))) return st;
        }
        s->last_decode.assign(p->decode_ids, p->decode_ids + p->n_decode);
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
    if (cap < (int32_t)s->running.size() || (!s->running.empty() && !finished_ids))
        return pa::fail(PA_ERR_INVALID_ARG, "%s: cap %d < %zu running", fn, cap,
                        s->running.size());
    int32_t n = 0;
    std::vector<int64_t> keep;
    try {
        keep.reserve(s->running.size());
    } catch (...) {
        return pa::fail(PA_ERR_INVALID_ARG, "%s: out of host memory", fn);
    }
    for (int64_t id : s->last_decode) ++s->reqs[id].generated;
    for (auto &e : s->last_prefill_end) {
        Req &r = s->reqs[e.first];
        if (e.second == r.n_prompt && r.state == St::Running) ++r.generated;
    }
    for (int64_t id : s->running) {
        Req &r = s->reqs[id];
        if (r.generated >= r.max_new) {
            pa_seq_free(s->a, id);
            r.state = St::Finished;
            finished_ids[n++] = id;
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
    out->finished = s->finished;
    out->swap_preemptions = s->swap_preempt;
    out->recompute_preemptions = s->recompute_preempt;
    return pa::ok();
}

}  // extern "C"
