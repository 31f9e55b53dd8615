// Host-side checks of libmikv's pool, allocator and step planner, built with
// AddressSanitizer and UndefinedBehaviorSanitizer together with the host
// sources (pool.cpp, sched.cpp) by tests/test_host_sanitizers.py. Host-only
// pools touch no device. Exits non-zero on the first failed check; the
// sanitizers abort on any memory or UB error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "mikv.h"

// Device pools take the address of the library's scratch array (attention.hip,
// device code) at creation; host-only pools never do, so the host build links
// this stand-in, which a host-only pool never calls.
namespace mikv {
int setup_noalloc_scratch() { std::abort(); }
}

static int g_checks = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        ++g_checks;                                                              \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                                        \
        }                                                                        \
    } while (0)

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(uint32_t n) {   // splitmix64, then modulo n
    g_rng += 0x9e3779b97f4a7c15ull;
    uint64_t z = g_rng;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return static_cast<uint32_t>((z ^ (z >> 31)) % n);
}

static void pool_argument_checks() {
    mi_kv_pool_t p = nullptr;
    CHECK(mi_kv_pool_init(nullptr, 8, 16, 2, 64, nullptr, nullptr, MI_POOL_HOST_ONLY) == MI_ERR_INVALID_ARG);
    CHECK(mi_kv_pool_init(&p, 0, 16, 2, 64, nullptr, nullptr, MI_POOL_HOST_ONLY) != MI_OK);
    CHECK(mi_kv_pool_init(&p, 8, 8, 2, 64, nullptr, nullptr, MI_POOL_HOST_ONLY) != MI_OK);
    CHECK(mi_kv_pool_init(&p, 8, 16, 0, 64, nullptr, nullptr, MI_POOL_HOST_ONLY) != MI_OK);
    CHECK(mi_kv_pool_init(&p, 8, 16, 2, 96, nullptr, nullptr, MI_POOL_HOST_ONLY) != MI_OK);
    CHECK(mi_kv_pool_destroy(nullptr) == MI_OK);
    CHECK(mi_kv_num_free_blocks(nullptr) < 0);
    CHECK(mi_kv_alloc_blocks(nullptr, 1, nullptr) == MI_ERR_INVALID_ARG);
    CHECK(mi_kv_blocks_needed(0, 16) == 0 && mi_kv_blocks_needed(1, 16) == 1 &&
          mi_kv_blocks_needed(16, 16) == 1 && mi_kv_blocks_needed(17, 16) == 2);
    CHECK(mi_kv_blocks_needed(-1, 16) < 0 && mi_kv_blocks_needed(5, 0) < 0);
    CHECK(mi_kv_blocks_needed(2147483647, 16) == 134217728);
    CHECK(mi_kv_cache_bytes(1, 32, 2048, 32, 128) == 1073741824ull);
    CHECK(mi_kv_cache_bytes(-1, 1, 1, 1, 1) == 0);
    for (int st = 1; st >= -9; --st) CHECK(mi_status_string(st) != nullptr);
    uint32_t bits = 123;
    CHECK(mi_kv_pool_check_errors(nullptr, &bits) == MI_ERR_INVALID_ARG && bits == 0);
}

static void allocator_checks() {
    const int N = 257;
    mi_kv_pool_t p = nullptr;
    CHECK(mi_kv_pool_init(&p, N, 16, 4, 128, nullptr, nullptr, MI_POOL_HOST_ONLY) == MI_OK);
    void *k = &p, *v = &p;
    CHECK(mi_kv_pool_get(p, &k, &v) == MI_OK && k == nullptr && v == nullptr);
    int32_t nb = 0, bs = 0, hkv = 0, d = 0;
    CHECK(mi_kv_pool_shape(p, &nb, &bs, &hkv, &d) == MI_OK && nb == N && bs == 16 && hkv == 4 && d == 128);
    uint32_t bits = 7;
    CHECK(mi_kv_pool_check_errors(p, &bits) == MI_OK && bits == 0);
    // first pops are 0, 1, 2, ...
    std::vector<int32_t> ids(N);
    CHECK(mi_kv_alloc_blocks(p, 3, ids.data()) == MI_OK && ids[0] == 0 && ids[1] == 1 && ids[2] == 2);
    // exhaustion pops nothing
    CHECK(mi_kv_alloc_blocks(p, N, ids.data() + 3) == MI_ERR_NO_FREE_BLOCKS);
    CHECK(mi_kv_num_free_blocks(p) == N - 3);
    CHECK(mi_kv_alloc_blocks(p, N - 3, ids.data() + 3) == MI_OK && mi_kv_num_free_blocks(p) == 0);
    CHECK(mi_kv_alloc_blocks(p, 1, ids.data()) == MI_ERR_NO_FREE_BLOCKS);
    CHECK(mi_kv_alloc_blocks(p, 0, nullptr) == MI_OK);
    // bad frees free nothing
    const int32_t foreign[2] = {5, N};
    CHECK(mi_kv_free_blocks(p, 2, foreign) == MI_ERR_INVALID_ARG && mi_kv_num_free_blocks(p) == 0);
    const int32_t repeated[3] = {4, 9, 4};
    CHECK(mi_kv_free_blocks(p, 3, repeated) == MI_ERR_INVALID_ARG && mi_kv_num_free_blocks(p) == 0);
    const int32_t negative[1] = {-1};
    CHECK(mi_kv_free_blocks(p, 1, negative) == MI_ERR_INVALID_ARG);
    CHECK(mi_kv_free_blocks(p, -1, negative) == MI_ERR_INVALID_ARG);
    // LIFO: freed in order a, b, c -> handed out c, b, a
    const int32_t back[3] = {10, 200, 37};
    CHECK(mi_kv_free_blocks(p, 3, back) == MI_OK && mi_kv_num_free_blocks(p) == 3);
    CHECK(mi_kv_free_blocks(p, 1, back) == MI_ERR_INVALID_ARG);          // double free
    int32_t got[3];
    CHECK(mi_kv_alloc_blocks(p, 3, got) == MI_OK && got[0] == 37 && got[1] == 200 && got[2] == 10);
    // random churn against a model of the held set
    std::set<int32_t> held(ids.begin(), ids.end());
    std::vector<int32_t> freelist;
    for (int it = 0; it < 20000; ++it) {
        if (rnd(2) == 0 && !held.empty()) {
            const int n = 1 + static_cast<int>(rnd(std::min<size_t>(held.size(), 8)));
            std::vector<int32_t> out;
            auto itr = held.begin();
            std::advance(itr, rnd(static_cast<uint32_t>(held.size() - n + 1)));
            for (int i = 0; i < n; ++i) out.push_back(*itr++);
            CHECK(mi_kv_free_blocks(p, n, out.data()) == MI_OK);
            for (int32_t x : out) {
                held.erase(x);
                freelist.push_back(x);
            }
        } else {
            const int n = 1 + static_cast<int>(rnd(8));
            std::vector<int32_t> out(n);
            const int rc = mi_kv_alloc_blocks(p, n, out.data());
            if (static_cast<size_t>(n) > freelist.size()) {
                CHECK(rc == MI_ERR_NO_FREE_BLOCKS);
                continue;
            }
            CHECK(rc == MI_OK);
            for (int i = 0; i < n; ++i) {
                CHECK(out[i] == freelist.back());                        // LIFO order
                freelist.pop_back();
                CHECK(held.insert(out[i]).second);                       // never handed out twice
            }
        }
        CHECK(mi_kv_num_free_blocks(p) == static_cast<int32_t>(freelist.size()));
        CHECK(held.size() + freelist.size() == static_cast<size_t>(N));
    }
    CHECK(mi_kv_pool_destroy(p) == MI_OK);
}

static void planner_checks(bool swap) {
    const int N = 96, MB = 24, R = 6;
    mi_kv_pool_t p = nullptr;
    CHECK(mi_kv_pool_init(&p, N, 16, 2, 64, nullptr, nullptr, MI_POOL_HOST_ONLY) == MI_OK);
    mi_sched_t s = nullptr;
    CHECK(mi_sched_create(&s, p, MB, R, 0.10, 0.30) == MI_OK);
    if (swap) CHECK(mi_sched_set_swap_space(s, 64) == MI_OK);
    CHECK(mi_sched_submit(s, 1, 0, 4) == MI_ERR_INVALID_ARG);
    CHECK(mi_sched_submit(s, 1, MB * 16, 1) == MI_ERR_UNSUPPORTED);   // needs MB + 1 blocks
    std::vector<int64_t> seq(R), pre(R), fin(R), swp(R);
    std::vector<int32_t> ctx(R), nt(R), table(R * MB), sout(2 * R * MB), sin_(2 * R * MB);
    int64_t next_id = 100;
    int submitted = 0, finished = 0;
    for (int step = 0; step < 3000; ++step) {
        if (rnd(3) == 0 && submitted < 400) {
            const int prompt = 1 + static_cast<int>(rnd(200));
            const int max_new = 1 + static_cast<int>(rnd(120));
            const int rc = mi_sched_submit(s, next_id++, prompt, max_new);
            CHECK(rc == MI_OK || rc == MI_ERR_UNSUPPORTED);
            if (rc == MI_OK) ++submitted;
        }
        mi_sched_counts c{};
        CHECK(mi_sched_step(s, &c, seq.data(), ctx.data(), nt.data(), table.data(), pre.data(),
                            fin.data(), swp.data(), sout.data(), sin_.data()) == MI_OK);
        finished += c.num_finished;
        const int rows = c.num_prefill + c.num_decode;
        CHECK(rows >= 0 && rows <= R && c.num_preempted >= 0 && c.num_finished >= 0);
        CHECK(c.free_blocks == mi_kv_num_free_blocks(p));
        CHECK(c.brake >= MI_BRAKE_PROCEED && c.brake <= MI_BRAKE_HARD);
        // every row's blocks are distinct pool ids, never shared between rows,
        // and held blocks + free blocks = pool
        std::set<int32_t> used;
        for (int r = 0; r < rows; ++r) {
            const int need = mi_kv_blocks_needed(ctx[r] + nt[r], 16);
            CHECK(need >= 1 && need <= MB);
            for (int j = 0; j < MB; ++j) {
                const int32_t id = table[r * MB + j];
                if (j < need) {
                    CHECK(id >= 0 && id < N);
                    CHECK(used.insert(id).second);
                } else {
                    CHECK(id == -1);
                }
            }
        }
        CHECK(static_cast<int>(used.size()) <= N - c.free_blocks);
        if (!swap) CHECK(c.num_swap_out == 0 && c.num_swap_in == 0 && c.num_swapped_out == 0);
        for (int i = 0; i < c.num_swap_out; ++i)
            CHECK(sout[2 * i] >= 0 && sout[2 * i] < N && sout[2 * i + 1] >= 0 && sout[2 * i + 1] < 64);
        for (int i = 0; i < c.num_swap_in; ++i)
            CHECK(sin_[2 * i] >= 0 && sin_[2 * i] < 64 && sin_[2 * i + 1] >= 0 && sin_[2 * i + 1] < N);
    }
    CHECK(finished > 0);
    CHECK(mi_sched_destroy(s) == MI_OK);
    CHECK(mi_kv_num_free_blocks(p) == N);                              // every block returned
    CHECK(mi_kv_pool_destroy(p) == MI_OK);
}

int main() {
    pool_argument_checks();
    allocator_checks();
    planner_checks(false);
    planner_checks(true);
    std::printf("ok %d checks\n", g_checks);
    return 0;
}
