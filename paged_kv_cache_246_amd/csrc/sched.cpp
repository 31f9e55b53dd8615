// Continuous-batching step planner over a paged KV pool: block lifecycle and
// admission with KV-protection brakes. Host code; the plan it emits is the
// input of the prefill and decode kernels (context lengths, new-token counts,
// block-table rows).
//
// mini-infer README, "Project overview" / "Architecture": a scheduler with
// waiting and running queues; prefill runs as its own forward, then the
// request joins the batched decode steps; admission happens at every step;
// blocks come from the KV manager's free-block pool and each request owns a
// BlockTable. nxmr.cn inference-techniques article, section 2.1: n tokens
// hold ceil(n / page) pages popped from the free list. vLLM-based
// inference-framework report, "SLO-aware, KV-cache protecting scheduler":
// free KV space below a critical threshold (10 %) is a hard brake on new
// prefills; running decodes with free space below a safety threshold (30 %)
// are a soft brake; otherwise new requests proceed.
//
// One step: (1) retire requests that produced max_new_tokens, returning their
// blocks; (2) give each running request, in admission order, the block its
// decode write at position ctx needs; on an empty pool preempt the most
// recently admitted running request (blocks returned, re-queued at the head
// of the waiting queue to be prefilled again over prompt + generated tokens)
// and retry; (3) admit waiting requests in order while a running slot is
// free, no brake holds (free / pool is re-measured before each admission;
// "below" is strict) and the pool holds ceil(prompt / 16) blocks, stopping at
// the first that cannot be admitted; (4) emit prefills then decodes and
// advance (a prefill yields the first token, a decode one more).
//
// KV offload (course project, optional task "KV Cache Offloading": inactive
// KV blocks move to CPU memory and come back when needed, under an eviction
// policy). With a host swap space, a preemption victim whose blocks fit the
// free host slots is swapped out instead of recomputed (its (device block,
// host slot) pairs are emitted, it keeps its context). The victim, for
// swap-out and recompute alike, is picked by the eviction policy: LIFO (the
// default) the most recently admitted running request, FIFO the one that
// entered the running set first (admitted or swapped back in earliest); LRU
// picks the FIFO victim, since every running request's KV is read at every
// step and the longest-held one is the least recently used in a tie. The
// running list is kept in entry order. Swapped requests come back first, in
// swap order and regardless of the brakes, each with its blocks plus the
// block its decode needs ((host slot, device block) pairs emitted), and
// decode in the same step; while any request is swapped out nothing new is
// admitted. The caller runs the swap-outs, then the swap-ins, before the
// step's kernels (mi_kv_swap_out / mi_kv_swap_in).
#include <algorithm>
#include <cstddef>
#include <deque>
#include <new>
#include <vector>

#include "internal.h"

struct mi_sched_s {
    struct Req {
        int64_t id = 0;
        int32_t prompt = 0;
        int32_t max_new = 0;
        int32_t generated = 0;
        int32_t ctx = 0;
        std::vector<int32_t> blocks;
        std::vector<int32_t> host_slots;
    };
    mi_kv_pool_s* pool = nullptr;
    int32_t mbps = 0;
    int32_t max_running = 0;
    double hard = 0.0;
    double soft = 0.0;
    std::deque<Req> waiting;
    std::vector<Req> running;
    std::deque<Req> swapped;
    // host swap space: LIFO stack of free slots (first pop returns slot 0)
    int32_t host_slots = 0;
    std::vector<int32_t> host_free;
    int32_t evict = MI_EVICT_LIFO;
};

namespace {

int32_t ceil_div(int64_t a, int32_t b) { return static_cast<int32_t>((a + b - 1) / b); }

int brake_state(const mi_sched_s* s, bool decoding) {
    const double f = static_cast<double>(mi_kv_num_free_blocks(s->pool)) / s->pool->num_blocks;
    if (f < s->hard) return MI_BRAKE_HARD;
    if (decoding && f < s->soft) return MI_BRAKE_SOFT;
    return MI_BRAKE_PROCEED;
}

void release(mi_sched_s* s, mi_sched_s::Req& r) {
    if (!r.blocks.empty())
        (void)mi_kv_free_blocks(s->pool, static_cast<int32_t>(r.blocks.size()), r.blocks.data());
    r.blocks.clear();
}

}  // namespace

extern "C" int mi_sched_create(mi_sched_t* out, mi_kv_pool_t pool, int32_t max_blocks_per_seq,
                               int32_t max_running, double hard_free_frac, double soft_free_frac) {
    if (!out) return MI_ERR_INVALID_ARG;
    *out = nullptr;
    if (!pool || max_blocks_per_seq <= 0 || max_running <= 0) return MI_ERR_INVALID_ARG;
    if (!(hard_free_frac >= 0.0 && hard_free_frac <= 1.0) ||
        !(soft_free_frac >= 0.0 && soft_free_frac <= 1.0))
        return MI_ERR_INVALID_ARG;
    mi_sched_s* s = new (std::nothrow) mi_sched_s();
    if (!s) return MI_ERR_OUT_OF_MEMORY;
    s->pool = pool;
    s->mbps = max_blocks_per_seq;
    s->max_running = max_running;
    s->hard = hard_free_frac;
    s->soft = soft_free_frac;
    *out = s;
    return MI_OK;
}

extern "C" int mi_sched_destroy(mi_sched_t s) {
    if (!s) return MI_OK;
    for (auto& r : s->running) release(s, r);
    delete s;
    return MI_OK;
}

extern "C" int mi_sched_submit(mi_sched_t s, int64_t request_id, int32_t prompt_tokens,
                               int32_t max_new_tokens) {
    if (!s || prompt_tokens < 1 || max_new_tokens < 1) return MI_ERR_INVALID_ARG;
    const int64_t total = static_cast<int64_t>(prompt_tokens) + max_new_tokens;
    const int32_t need = ceil_div(total, mikv::kBlockSize);
    if (total > (int64_t{1} << 30) || need > s->mbps || need > s->pool->num_blocks)
        return MI_ERR_UNSUPPORTED;
    try {
        mi_sched_s::Req r;
        r.id = request_id;
        r.prompt = prompt_tokens;
        r.max_new = max_new_tokens;
        s->waiting.push_back(std::move(r));
    } catch (...) {
        return MI_ERR_OUT_OF_MEMORY;
    }
    return MI_OK;
}

extern "C" int mi_sched_set_swap_space(mi_sched_t s, int32_t host_slots) {
    if (!s || host_slots < 0) return MI_ERR_INVALID_ARG;
    if (!s->running.empty() || !s->swapped.empty()) return MI_ERR_INVALID_ARG;
    try {
        s->host_free.resize(static_cast<size_t>(host_slots));
    } catch (...) {
        return MI_ERR_OUT_OF_MEMORY;
    }
    for (int32_t i = 0; i < host_slots; ++i) s->host_free[i] = host_slots - 1 - i;
    s->host_slots = host_slots;
    return MI_OK;
}

extern "C" int mi_sched_set_eviction(mi_sched_t s, int32_t policy) {
    if (!s || (policy != MI_EVICT_LIFO && policy != MI_EVICT_FIFO && policy != MI_EVICT_LRU))
        return MI_ERR_INVALID_ARG;
    s->evict = policy;
    return MI_OK;
}

extern "C" int32_t mi_sched_num_swapped(mi_sched_t s) {
    return s ? static_cast<int32_t>(s->swapped.size()) : MI_ERR_INVALID_ARG;
}

extern "C" int32_t mi_sched_num_waiting(mi_sched_t s) {
    return s ? static_cast<int32_t>(s->waiting.size()) : MI_ERR_INVALID_ARG;
}

extern "C" int32_t mi_sched_num_running(mi_sched_t s) {
    return s ? static_cast<int32_t>(s->running.size()) : MI_ERR_INVALID_ARG;
}

extern "C" int mi_sched_step(mi_sched_t s, mi_sched_counts* counts, int64_t* seq_ids,
                             int32_t* context_lens, int32_t* new_tokens, int32_t* block_table,
                             int64_t* preempted_ids, int64_t* finished_ids, int64_t* swapped_ids,
                             int32_t* swap_out, int32_t* swap_in) {
    if (!s || !counts || !seq_ids || !context_lens || !new_tokens || !block_table ||
        !preempted_ids || !finished_ids || !swapped_ids || !swap_out || !swap_in)
        return MI_ERR_INVALID_ARG;
    try {
        int32_t n_fin = 0, n_pre = 0, n_swp = 0, n_so = 0, n_si = 0;
        // (1) retire
        std::vector<mi_sched_s::Req> keep;
        keep.reserve(s->running.size());
        for (auto& r : s->running) {
            if (r.generated >= r.max_new) {
                release(s, r);
                finished_ids[n_fin++] = r.id;
            } else {
                keep.push_back(std::move(r));
            }
        }
        s->running.swap(keep);
        // (2) decode growth, evicting a running request when the pool is empty
        size_t i = 0;
        while (i < s->running.size()) {
            auto& r = s->running[i];
            const int32_t need = ceil_div(static_cast<int64_t>(r.ctx) + 1, mikv::kBlockSize);
            if (static_cast<int32_t>(r.blocks.size()) >= need) {
                ++i;
                continue;
            }
            int32_t id = -1;
            if (mi_kv_alloc_blocks(s->pool, 1, &id) == MI_OK) {
                r.blocks.push_back(id);
                ++i;
                continue;
            }
            const size_t vi = s->evict == MI_EVICT_LIFO ? s->running.size() - 1 : 0;
            mi_sched_s::Req victim = std::move(s->running[vi]);
            s->running.erase(s->running.begin() + static_cast<std::ptrdiff_t>(vi));
            if (vi < i) --i;          // the request that needs a block moved down one place
            if (s->host_free.size() >= victim.blocks.size()) {
                for (int32_t dev : victim.blocks) {
                    const int32_t slot = s->host_free.back();
                    s->host_free.pop_back();
                    victim.host_slots.push_back(slot);
                    swap_out[2 * n_so] = dev;
                    swap_out[2 * n_so + 1] = slot;
                    ++n_so;
                }
                release(s, victim);
                swapped_ids[n_swp++] = victim.id;
                s->swapped.push_back(std::move(victim));
                continue;
            }
            release(s, victim);
            victim.prompt += victim.generated;
            victim.max_new -= victim.generated;
            victim.generated = 0;
            victim.ctx = 0;
            preempted_ids[n_pre++] = victim.id;
            s->waiting.push_front(std::move(victim));
        }
        // (3') swap-ins, oldest swapped first, regardless of the brakes
        while (!s->swapped.empty() && static_cast<int32_t>(s->running.size()) < s->max_running) {
            auto& r = s->swapped.front();
            const int32_t nb = static_cast<int32_t>(r.host_slots.size());
            const int32_t need = std::max(nb, ceil_div(static_cast<int64_t>(r.ctx) + 1, mikv::kBlockSize));
            std::vector<int32_t> ids(static_cast<size_t>(need));
            if (mi_kv_alloc_blocks(s->pool, need, ids.data()) != MI_OK) break;
            for (int32_t j = 0; j < nb; ++j) {
                swap_in[2 * n_si] = r.host_slots[j];
                swap_in[2 * n_si + 1] = ids[j];
                ++n_si;
            }
            for (int32_t slot : r.host_slots) s->host_free.push_back(slot);
            r.host_slots.clear();
            r.blocks = std::move(ids);
            s->running.push_back(std::move(r));
            s->swapped.pop_front();
        }
        // (3) admission
        const bool decoding = !s->running.empty();
        counts->brake = brake_state(s, decoding);
        std::vector<mi_sched_s::Req> admitted;
        while (!s->waiting.empty() && s->swapped.empty() &&
               static_cast<int32_t>(s->running.size() + admitted.size()) < s->max_running) {
            if (brake_state(s, decoding) != MI_BRAKE_PROCEED) break;
            auto& r = s->waiting.front();
            const int32_t need = ceil_div(r.prompt, mikv::kBlockSize);
            std::vector<int32_t> ids(static_cast<size_t>(need));
            if (mi_kv_alloc_blocks(s->pool, need, ids.data()) != MI_OK) break;
            r.blocks = std::move(ids);
            admitted.push_back(std::move(r));
            s->waiting.pop_front();
        }
        // (4) plan: prefills first, then decodes; then advance
        int32_t row = 0;
        auto emit = [&](const mi_sched_s::Req& r, int32_t ctx, int32_t n) {
            seq_ids[row] = r.id;
            context_lens[row] = ctx;
            new_tokens[row] = n;
            int32_t* t = block_table + static_cast<size_t>(row) * s->mbps;
            for (int32_t j = 0; j < s->mbps; ++j)
                t[j] = j < static_cast<int32_t>(r.blocks.size()) ? r.blocks[j] : -1;
            ++row;
        };
        for (const auto& r : admitted) emit(r, 0, r.prompt);
        for (const auto& r : s->running) emit(r, r.ctx, 1);
        counts->num_prefill = static_cast<int32_t>(admitted.size());
        counts->num_decode = static_cast<int32_t>(s->running.size());
        counts->num_preempted = n_pre;
        counts->num_finished = n_fin;
        counts->num_swapped_out = n_swp;
        counts->num_swap_out = n_so;
        counts->num_swap_in = n_si;
        for (auto& r : s->running) {
            r.ctx += 1;
            r.generated += 1;
        }
        for (auto& r : admitted) {
            r.ctx = r.prompt;
            r.generated = 1;
            s->running.push_back(std::move(r));
        }
        counts->free_blocks = mi_kv_num_free_blocks(s->pool);
    } catch (...) {
        return MI_ERR_OUT_OF_MEMORY;
    }
    return MI_OK;
}
