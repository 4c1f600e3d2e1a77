// Host test of the workspace registry (test infrastructure): hand-picked
// cases, then 200,000 random record / forget / find operations on a small
// address range compared with a plain list model, then several threads
// working on one registry at once.  Prints "ok" when every check passes.
#include <cstdint>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "../../direct_coulomb_potential_amd/csrc/workspace_registry.h"

using namespace cpmap;

static int failures = 0;
#define CHECK(c)                                                                     \
    do {                                                                             \
        if (!(c)) {                                                                  \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);     \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

static const void *P(uintptr_t a) { return reinterpret_cast<const void *>(a); }

static WorkspaceKey key(int64_t n, int32_t cap = 0, float rc = 12.0f)
{
    return WorkspaceKey::make(n, 200, 200, 200, 0.5f, 0.0f, 0.0f, 0.0f, 4.0f, rc, cap);
}

// The plain model: a list of records; a write drops every record it overlaps.
struct Model {
    struct R {
        uintptr_t a;
        size_t n;
        WorkspaceKind kind;
        WorkspaceKey key;
        uint64_t nonce;
    };
    std::vector<R> rs;
    uint64_t next = 1;
    void forget(uintptr_t a, size_t n)
    {
        if (a == 0 || n == 0)
            return;
        std::vector<R> keep;
        for (const R &r : rs)
            if (!(r.a < a + n && a < r.a + r.n))
                keep.push_back(r);
        rs.swap(keep);
    }
    uint64_t record(uintptr_t a, size_t n, WorkspaceKind k, const WorkspaceKey &key)
    {
        forget(a, n);
        rs.push_back(R{a, n, k, key, next});
        return next++;
    }
    uint64_t find(uintptr_t a, size_t n, WorkspaceKind k, const WorkspaceKey &key) const
    {
        for (const R &r : rs)
            if (r.a == a)
                return (r.n == n && r.kind == k && r.key == key) ? r.nonce : 0;
        return 0;
    }
};

int main()
{
    {
        WorkspaceRegistry reg;
        const uint64_t n1 = reg.record(P(1000), 500, kBinnedWorkspace, key(100));
        CHECK(n1 != 0);
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(100)) == n1);
        CHECK(reg.find(P(1000), 499, kBinnedWorkspace, key(100)) == 0);  // size
        CHECK(reg.find(P(1000), 500, kSlotWorkspace, key(100)) == 0);    // kind
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(101)) == 0);  // atom count
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(100, 0, 11.0f)) == 0);  // cutoff
        CHECK(reg.find(P(1001), 500, kBinnedWorkspace, key(100)) == 0);  // base
        reg.forget(P(900), 100);   // ends just before
        reg.forget(P(1500), 100);  // starts just after
        reg.forget(nullptr, 1u << 20);
        reg.forget(P(1200), 0);
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(100)) == n1);
        reg.forget(P(1499), 1);  // the last byte
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(100)) == 0);
        const uint64_t n2 = reg.record(P(1000), 500, kBinnedWorkspace, key(100));
        CHECK(n2 > n1);
        const uint64_t n3 = reg.record(P(2000), 300, kSlotWorkspace, key(100, 8));
        CHECK(n3 > n2 && reg.size() == 2);
        reg.forget(P(1400), 700);  // straddles both
        CHECK(reg.size() == 0);
        // a record over part of another replaces it
        reg.record(P(1000), 500, kBinnedWorkspace, key(100));
        const uint64_t n5 = reg.record(P(1200), 100, kBinnedWorkspace, key(7));
        CHECK(reg.find(P(1000), 500, kBinnedWorkspace, key(100)) == 0);
        CHECK(reg.find(P(1200), 100, kBinnedWorkspace, key(7)) == n5);
        // a range that wraps past the top of the address space
        reg.record(P(UINTPTR_MAX - 1000), 500, kBinnedWorkspace, key(1));
        reg.forget(P(UINTPTR_MAX - 600), SIZE_MAX);
        CHECK(reg.find(P(UINTPTR_MAX - 1000), 500, kBinnedWorkspace, key(1)) == 0);
        CHECK(reg.find(P(1200), 100, kBinnedWorkspace, key(7)) == n5);
    }
    {
        // random operations against the model
        WorkspaceRegistry reg;
        Model model;
        std::mt19937_64 rng(12345);
        auto pick = [&](uint64_t lo, uint64_t hi) {
            return std::uniform_int_distribution<uint64_t>(lo, hi)(rng);
        };
        for (int it = 0; it < 200000; ++it) {
            const uintptr_t a = 256 * pick(1, 64) + (pick(0, 3) == 0 ? pick(0, 255) : 0);
            const size_t n = (size_t)pick(1, 6) * 256 + pick(0, 1) * pick(0, 255);
            const WorkspaceKind k = pick(0, 1) ? kBinnedWorkspace : kSlotWorkspace;
            const WorkspaceKey kk = key((int64_t)pick(1, 3), k == kSlotWorkspace ? 8 : 0);
            switch (pick(0, 2)) {
            case 0:
                CHECK(reg.record(P(a), n, k, kk) == model.record(a, n, k, kk));
                break;
            case 1:
                reg.forget(P(a), n);
                model.forget(a, n);
                break;
            default:
                CHECK(reg.find(P(a), n, k, kk) == model.find(a, n, k, kk));
            }
            if (it % 1000 == 0) {
                CHECK(reg.size() == model.rs.size());
                for (const Model::R &r : model.rs)
                    CHECK(reg.find(P(r.a), r.n, r.kind, r.key) == r.nonce);
            }
        }
    }
    {
        // threads: each works on its own address range of one registry
        WorkspaceRegistry reg;
        std::vector<std::thread> ts;
        std::vector<int> bad(8, 0);
        for (int t = 0; t < 8; ++t)
            ts.emplace_back([&, t] {
                const uintptr_t base = (uintptr_t)(t + 1) << 32;
                for (int i = 0; i < 20000; ++i) {
                    const uintptr_t a = base + 4096 * (uintptr_t)(i % 17);
                    const uint64_t n = reg.record(P(a), 4096, kBinnedWorkspace, key(i));
                    if (reg.find(P(a), 4096, kBinnedWorkspace, key(i)) != n)
                        ++bad[t];
                    if (i % 3 == 0) {
                        reg.forget(P(a + 100), 1);
                        if (reg.find(P(a), 4096, kBinnedWorkspace, key(i)) != 0)
                            ++bad[t];
                    }
                }
            });
        for (auto &th : ts)
            th.join();
        for (int b : bad)
            CHECK(b == 0);
    }
    if (failures == 0)
        std::printf("ok\n");
    return failures != 0;
}
