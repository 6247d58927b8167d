// Host test of the paged cache's page bookkeeping (csrc/pager.h), with no GPU: a simulated
// address space stands in for the virtual-memory backend.  Each row of a page holds one tag; a
// model keeps, per open slot and plane, the tags a contiguous cache would hold, and after every
// operation each complete row read through the simulated page tables must equal the model.
//
// Built and run by tests/test_pager_host.py:  g++ -std=c++17 -O1 -I<csrc> pager_host_test.cpp
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <tuple>
#include <vector>

#include "pager.h"

using lca::Pager;
using lca::PagerPlane;

static int g_fail = 0;
#define CHECK(c)                                                           \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::printf("CHECK failed line %d: %s\n", __LINE__, #c);       \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

struct Sim : lca::PagerOps {
    std::vector<PagerPlane> pl;
    int max_seqs;
    std::vector<std::vector<uint32_t>> pool;               // pool page -> row tags
    std::map<std::tuple<int, int>, std::vector<uint32_t>> home;   // (plane, slot) -> page 0
    std::map<std::tuple<int, int>, std::vector<uint32_t>> state;  // (plane, slot) -> rows
    std::map<std::tuple<int, int, int64_t>, int32_t> va;  // (plane, slot, page) -> pool page
    int fail_after = -1;                                   // fail the n-th map from now (0 = next)
    int maps = 0, unmaps = 0, copies = 0;

    Sim(const std::vector<PagerPlane>& p, int ms, int64_t npool) : pl(p), max_seqs(ms) {
        for (size_t i = 0; i < pl.size(); ++i) {
            if (pl[i].state) {
                for (int s = 0; s < ms; ++s) state[{(int)i, s}].assign((size_t)pl[i].rows, 0u);
                continue;
            }
            for (int s = 0; s < ms; ++s) home[{(int)i, s}].assign((size_t)pl[i].rpp, 0u);
        }
        pool.assign((size_t)npool, {});
    }
    bool map(int p, int slot, int64_t page, int32_t phys) override {
        if (fail_after == 0) {
            fail_after = -1;
            return false;
        }
        if (fail_after > 0) --fail_after;
        if (page == 0 || va.count({p, slot, page})) {  // page 0 is home; no double mapping
            std::printf("bad map plane %d slot %d page %lld\n", p, slot, (long long)page);
            ++g_fail;
            return false;
        }
        // (a page keeps what its last holder wrote; sized for the plane with the most rows per page)
        if (pool[(size_t)phys].empty()) pool[(size_t)phys].assign(256, 0xdeadu);
        va[{p, slot, page}] = phys;
        ++maps;
        return true;
    }
    bool unmap(int p, int slot, int64_t page) override {
        auto it = va.find({p, slot, page});
        if (it == va.end()) {
            std::printf("unmap of an unmapped page\n");
            ++g_fail;
            return false;
        }
        va.erase(it);
        ++unmaps;
        return true;
    }
    std::vector<uint32_t>* page_mem(int p, int slot, int64_t page) {
        if (page == 0) return &home[{p, slot}];
        auto it = va.find({p, slot, page});
        return it == va.end() ? nullptr : &pool[(size_t)it->second];
    }
    bool copy_page(int p, int ds, int64_t dp, int ss, int64_t sp) override {
        auto* d = page_mem(p, ds, dp);
        auto* s = page_mem(p, ss, sp);
        if (!d || !s) {
            std::printf("copy through an unmapped page\n");
            ++g_fail;
            return false;
        }
        *d = *s;
        ++copies;
        return true;
    }
    bool copy_state(int p, int ds, int ss) override {
        state[{p, ds}] = state[{p, ss}];
        return true;
    }
    // row access through the page tables; false when unmapped
    bool write(int p, int slot, int64_t row, uint32_t tag) {
        if (pl[(size_t)p].state) {
            state[{p, slot}][(size_t)row] = tag;
            return true;
        }
        auto* m = page_mem(p, slot, row / pl[(size_t)p].rpp);
        if (!m) return false;
        (*m)[(size_t)(row % pl[(size_t)p].rpp)] = tag;
        return true;
    }
    bool read(int p, int slot, int64_t row, uint32_t* tag) {
        if (pl[(size_t)p].state) {
            *tag = state[{p, slot}][(size_t)row];
            return true;
        }
        auto* m = page_mem(p, slot, row / pl[(size_t)p].rpp);
        if (!m) return false;
        *tag = (*m)[(size_t)(row % pl[(size_t)p].rpp)];
        return true;
    }
};

static std::vector<PagerPlane> planes_small() {
    // CSA-like (m = 4) and HCA-like (m = 16) streams with different rows per page, and a state plane
    std::vector<PagerPlane> v;
    auto add = [&](int64_t rb, int64_t rows, int m, bool st, int64_t page) {
        PagerPlane p;
        p.row_bytes = rb;
        p.rows = rows;
        p.m = m;
        p.state = st;
        if (!st) {
            p.rpp = page / rb;
            p.pages = rows / p.rpp;
        }
        v.push_back(p);
    };
    add(512, 256, 4, false, 4096);   // 8 rows / page, 32 pages
    add(128, 256, 4, false, 4096);   // 32 rows / page, 8 pages
    add(1024, 32, 16, false, 4096);  // 4 rows / page, 8 pages
    add(64, 40, 1, true, 4096);      // state: 40 rows
    return v;
}

struct Model {
    // tags of the complete rows of each open slot (plane -> rows), tokens per slot
    std::map<int, std::vector<std::vector<uint32_t>>> rows;
    std::map<int, int64_t> tokens;
};

static uint32_t g_tag = 1;

// grow slot to n tokens: reserve, then write the newly complete rows and scribble on the next one
static int grow(Pager& pg, Sim& sim, Model& md, int slot, int64_t n) {
    const int rc = pg.reserve(slot, n, sim);
    if (rc != lca::kPgOk) return rc;
    const auto& pl = pg.planes();
    const int64_t n0 = md.tokens[slot];
    for (size_t p = 0; p < pl.size(); ++p) {
        auto& mr = md.rows[slot][p];
        if (pl[p].state) {  // state rows: the ring row of every new token
            for (int64_t t = n0; t < n; ++t) {
                const uint32_t tag = g_tag++;
                CHECK(sim.write((int)p, slot, t % pl[p].rows, tag));
                mr[(size_t)(t % pl[p].rows)] = tag;
            }
            continue;
        }
        const int64_t r0 = n0 / pl[p].m, r1 = std::min(n / pl[p].m, pl[p].rows);
        for (int64_t r = r0; r < r1; ++r) {
            const uint32_t tag = g_tag++;
            CHECK(sim.write((int)p, slot, r, tag));
            mr.resize((size_t)r + 1);
            mr[(size_t)r] = tag;
        }
        if (r1 < pl[p].rows) CHECK(sim.write((int)p, slot, r1, 0xbad0000u + (uint32_t)slot));  // in progress
    }
    md.tokens[slot] = n;
    return rc;
}

static void verify(Pager& pg, Sim& sim, Model& md) {
    const auto& pl = pg.planes();
    for (auto& [slot, n] : md.tokens) {
        CHECK(pg.tokens(slot) == n);
        for (size_t p = 0; p < pl.size(); ++p) {
            const auto& mr = md.rows[slot][p];
            const int64_t lim = pl[p].state ? pl[p].rows : std::min(n / pl[p].m, pl[p].rows);
            for (int64_t r = 0; r < lim; ++r) {
                uint32_t tag = 0;
                if (!sim.read((int)p, slot, r, &tag)) {
                    std::printf("slot %d plane %zu row %lld unmapped\n", slot, p, (long long)r);
                    ++g_fail;
                    return;
                }
                // (a state row tagged 0 has not been written since its slot was opened: stale)
                if (r < (int64_t)mr.size() && tag != mr[(size_t)r] && !(pl[p].state && mr[(size_t)r] == 0)) {
                    std::printf("slot %d plane %zu row %lld: %u, want %u\n", slot, p, (long long)r, tag, mr[(size_t)r]);
                    ++g_fail;
                    return;
                }
            }
            if (!pl[p].state && n / pl[p].m < pl[p].rows) {  // the row being built is backed too
                uint32_t tag;
                CHECK(sim.read((int)p, slot, n / pl[p].m, &tag));
            }
        }
    }
    // reference counts equal mappings; free pages are exactly the unmapped ones
    std::map<int32_t, int> cnt;
    for (auto& [k, ph] : sim.va) ++cnt[ph];
    const auto st = pg.stats();
    int64_t used = 0;
    for (int32_t ph = 0; ph < (int32_t)st.pool_pages; ++ph) {
        CHECK(pg.refs(ph) == (cnt.count(ph) ? cnt[ph] : 0));
        used += pg.refs(ph) > 0;
    }
    CHECK(st.free_pages + used == st.pool_pages);
    CHECK(st.mapped_pages == (int64_t)sim.va.size());
}

static int open_slot(Pager& pg, Model& md, const std::vector<PagerPlane>& pl) {
    int s = -1;
    if (pg.open(&s) != lca::kPgOk) return -1;
    md.tokens[s] = 0;
    md.rows[s].assign(pl.size(), {});
    for (size_t p = 0; p < pl.size(); ++p)
        if (pl[p].state) md.rows[s][p].assign((size_t)pl[p].rows, 0u);
    return s;
}

static void test_basic() {
    auto pl = planes_small();
    Pager pg;
    pg.init(pl, 4, 64);
    Sim sim(pl, 4, 64);
    Model md;
    const int a = open_slot(pg, md, pl);
    CHECK(a == 0);
    // a fresh sequence needs only its home pages
    CHECK(grow(pg, sim, md, a, 3) == lca::kPgOk);
    CHECK(sim.maps == 0);
    // 100 tokens: plane 0 rows [0, 26) -> pages 0..3 (3 pool pages); plane 1: rows 26 -> page 0 only;
    // plane 2: rows [0, 7) -> pages 0, 1 (1 pool page)
    CHECK(grow(pg, sim, md, a, 100) == lca::kPgOk);
    CHECK(sim.maps == 4);
    CHECK(pg.stats().free_pages == 60);
    verify(pg, sim, md);
    // a smaller reserve maps nothing
    CHECK(pg.reserve(a, 50, sim) == lca::kPgOk);
    CHECK(sim.maps == 4);
    // beyond a plane's rows
    CHECK(pg.reserve(a, 32 * 16 + 16, sim) == lca::kPgShape);
    CHECK(pg.reserve(7, 10, sim) == lca::kPgInval);
    CHECK(pg.reserve(1, 10, sim) == lca::kPgInval);  // slot 1 not open
    // fork at 100: plane 0 complete rows 25 -> pages 1, 2 shared, page 3 copied (row 24 complete);
    // plane 1: 25 rows -> page 0 only (copied); plane 2: 6 rows -> page 1 private copy (rows 4, 5)
    int b = -1;
    const int copies0 = sim.copies;
    CHECK(pg.fork(a, 100, &b, sim) == lca::kPgOk);
    CHECK(b == 1);
    md.tokens[b] = 100;
    md.rows[b] = md.rows[a];
    CHECK(pg.refs(pg.entry(0, a, 1)) == 2 && pg.refs(pg.entry(0, a, 2)) == 2);
    CHECK(pg.entry(0, b, 3) != pg.entry(0, a, 3));
    CHECK(pg.entry(2, b, 1) != pg.entry(2, a, 1));
    CHECK(sim.copies - copies0 == 3 /* page 0 of each plane */ + 2 /* plane 0 page 3, plane 2 page 1 */);
    CHECK(pg.stats().shared_pages == 2);
    verify(pg, sim, md);
    // both grow apart: the shared pages stay identical, the rest diverges
    CHECK(grow(pg, sim, md, a, 180) == lca::kPgOk);
    CHECK(grow(pg, sim, md, b, 140) == lca::kPgOk);
    verify(pg, sim, md);
    // closing the parent keeps the shared pages for the child
    CHECK(pg.close(a, sim) == lca::kPgOk);
    md.tokens.erase(a);
    md.rows.erase(a);
    verify(pg, sim, md);
    CHECK(pg.stats().shared_pages == 0);
    CHECK(pg.close(b, sim) == lca::kPgOk);
    md.tokens.erase(b);
    md.rows.erase(b);
    CHECK(pg.stats().free_pages == 64);
    CHECK(sim.va.empty());
    CHECK(pg.close(b, sim) == lca::kPgInval);
}

static void test_edges() {
    auto pl = planes_small();
    // fork on a page boundary and of a full sequence
    {
        Pager pg;
        pg.init(pl, 3, 200);
        Sim sim(pl, 3, 200);
        Model md;
        const int a = open_slot(pg, md, pl);
        CHECK(grow(pg, sim, md, a, 128) == lca::kPgOk);  // plane 0: 32 rows = 4 full pages
        const int c0 = sim.copies;
        int b = -1;
        CHECK(pg.fork(a, 128, &b, sim) == lca::kPgOk);
        md.tokens[b] = 128;
        md.rows[b] = md.rows[a];
        // plane 0: pages 1..3 shared, page 4 fresh, no copy (no complete row in it)
        CHECK(pg.refs(pg.entry(0, a, 3)) == 2);
        CHECK(pg.entry(0, b, 4) >= 0 && pg.entry(0, b, 4) != pg.entry(0, a, 4));
        // copies: page 0 of 3 planes; plane 1 (32 rows = page 0 full, boundary page 1 empty) none;
        // plane 2 (8 rows: pages 0, 1 full; boundary page 2 empty) none besides page 0
        CHECK(sim.copies - c0 == 3);
        verify(pg, sim, md);
        CHECK(grow(pg, sim, md, b, 200) == lca::kPgOk);
        verify(pg, sim, md);
        // the full sequence: 256 rows of plane 0 = 1024 tokens; plane 2 has 32 rows = 512 tokens
        Pager pf;
        Sim sf(pl, 2, 100);
        pf.init(pl, 2, 100);
        Model mf;
        const int x = open_slot(pf, mf, pl);
        CHECK(grow(pf, sf, mf, x, 512) == lca::kPgOk);
        int y = -1;
        CHECK(pf.fork(x, 512, &y, sf) == lca::kPgOk);  // plane 2 is full: every page but 0 shared
        mf.tokens[y] = 512;
        mf.rows[y] = mf.rows[x];
        CHECK(pf.refs(pf.entry(2, x, 7)) == 2);
        verify(pf, sf, mf);
        CHECK(pf.fork(x, 513, &y, sf) == lca::kPgInval);  // beyond the parent's tokens
    }
    // pool exhaustion and a failing backend leave everything as it was
    {
        Pager pg;
        pg.init(pl, 2, 10);
        Sim sim(pl, 2, 10);
        Model md;
        const int a = open_slot(pg, md, pl);
        CHECK(grow(pg, sim, md, a, 60) == lca::kPgOk);  // plane 0: 16 rows -> pages 1, 2; plane 2: page 0
        const auto s0 = pg.stats();
        const auto va0 = sim.va;
        CHECK(pg.reserve(a, 400, sim) == lca::kPgNoMem);
        CHECK(sim.va == va0 && pg.stats().free_pages == s0.free_pages && pg.tokens(a) == 60);
        sim.fail_after = 1;  // the second map fails
        CHECK(pg.reserve(a, 160, sim) == lca::kPgBackend);
        CHECK(sim.va == va0 && pg.stats().free_pages == s0.free_pages && pg.tokens(a) == 60);
        verify(pg, sim, md);
        sim.fail_after = 0;  // the fork's one fresh page (plane 0, page 1) fails to map
        int b = -1;
        CHECK(pg.fork(a, 60, &b, sim) == lca::kPgBackend);
        CHECK(sim.va == va0 && pg.stats().free_pages == s0.free_pages && pg.stats().open_slots == 1);
        verify(pg, sim, md);
        CHECK(pg.fork(a, 60, &b, sim) == lca::kPgOk);
        int c = -1;
        CHECK(pg.open(&c) == lca::kPgNoMem);  // both slots open
    }
}

static void test_random(unsigned seed) {
    auto pl = planes_small();
    const int ms = 6;
    const int64_t npool = 40;
    Pager pg;
    pg.init(pl, ms, npool);
    Sim sim(pl, ms, npool);
    Model md;
    std::mt19937 rng(seed);
    int nomem = 0, forks = 0;
    for (int it = 0; it < 3000; ++it) {
        const int op = (int)(rng() % 10);
        std::vector<int> open;
        for (auto& [s, n] : md.tokens) open.push_back(s);
        if (op == 0 || open.empty()) {
            open_slot(pg, md, pl);
        } else if (op <= 5) {  // grow
            const int s = open[rng() % open.size()];
            const int64_t n = std::min<int64_t>(md.tokens[s] + (int64_t)(rng() % 70), 512);
            const auto before = sim.va;
            const int rc = grow(pg, sim, md, s, n);
            if (rc == lca::kPgNoMem) {
                ++nomem;
                CHECK(sim.va == before);
            } else {
                CHECK(rc == lca::kPgOk);
            }
        } else if (op <= 7) {  // fork at a random point
            const int s = open[rng() % open.size()];
            const int64_t n = md.tokens[s] ? (int64_t)(rng() % (md.tokens[s] + 1)) : 0;
            int d = -1;
            const int rc = pg.fork(s, n, &d, sim);
            if (rc == lca::kPgOk) {
                ++forks;
                md.tokens[d] = n;
                md.rows[d] = md.rows[s];
                for (size_t p = 0; p < pl.size(); ++p)
                    if (!pl[p].state) md.rows[d][p].resize((size_t)std::min(n / pl[p].m, pl[p].rows));
                // the state rows: a fork earlier than the parent's length keeps the parent's ring
            } else {
                CHECK(rc == lca::kPgNoMem);
            }
        } else {  // close
            const int s = open[rng() % open.size()];
            CHECK(pg.close(s, sim) == lca::kPgOk);
            md.tokens.erase(s);
            md.rows.erase(s);
        }
        verify(pg, sim, md);
        if (g_fail) {
            std::printf("random test seed %u failed at step %d\n", seed, it);
            return;
        }
    }
    for (auto& [s, n] : md.tokens) CHECK(pg.close(s, sim) == lca::kPgOk);
    CHECK(pg.stats().free_pages == npool && sim.va.empty());
    std::printf("random seed %u: %d forks, %d pool-full refusals\n", seed, forks, nomem);
}

int main() {
    test_basic();
    test_edges();
    for (unsigned s = 1; s <= 4; ++s) test_random(s);
    if (g_fail) {
        std::printf("FAILED: %d checks\n", g_fail);
        return 1;
    }
    std::printf("pager host test: ok\n");
    return 0;
}
