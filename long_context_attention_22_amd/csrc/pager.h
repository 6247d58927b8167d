// pager.h -- page bookkeeping of the paged KV cache (host only, no HIP).
//
// The DeepSeek-V4 pages ("DeepSeek-V4 中文翻译" section 3.5.1, KV cache layout and cache
// management) split the cache in two: a classical cache of compressed CSA/HCA entries, paged in
// blocks whose raw-token count is a multiple of lcm(m, m'), and a fixed, preallocated state-cache
// pool (sliding-window rows and the not-yet-compressed tail) handed out per sequence.  Section
// 3.5.2 reuses the stored entries of a shared prefix instead of prefilling it again.
//
// Here a sequence occupies one slot of every plane (a plane is one storage array of the cache:
// the nope, rope or scale rows of one layer's stream).  Plane p reserves rows[p] rows per slot of
// virtual address space.  Classical planes are backed page by page from one pool of equal pages:
// page i of slot s covers rows [i * rpp, (i + 1) * rpp) with rpp = page_bytes / row_bytes, that is
// rpp * m raw tokens.  Page 0 of every (plane, slot) is a "home" page, mapped for the cache's whole
// life, so a read of row 0 (what a kernel does for padded lanes) never touches an unmapped address.
// State planes are fully backed at creation and are not tracked here.
//
// Prefix reuse (fork): the child maps the very pool pages of the parent whose rows are all
// complete entries of the prefix (entries are written once, when their last raw row arrives, so
// these pages never change again); the page holding the first entry the child will write is
// copied into a private page, and state planes are copied whole.
//
// The Pager decides; a PagerOps backend does (maps, unmaps and copies).  Every operation checks
// first that it can finish (slot state, capacity, free pages) and changes nothing when it cannot;
// a backend failure part way is rolled back.
#pragma once

#include <cstdint>
#include <vector>

namespace lca {

// status values (the library's LCA_* codes)
enum PagerStatus : int { kPgOk = 0, kPgInval = 1, kPgShape = 2, kPgBackend = 6, kPgNoMem = 7 };

struct PagerPlane {
    int64_t row_bytes = 0;
    int64_t rows = 0;      // rows per slot
    int32_t m = 1;         // raw tokens per row (classical planes)
    bool state = false;    // state-cache plane: fully backed, copied whole by fork
    int64_t rpp = 0;       // rows per page (classical planes)
    int64_t pages = 0;     // pages per slot (classical planes)
};

struct PagerOps {
    virtual ~PagerOps() = default;
    // map pool page `phys` at page `page` of the slot (home pages are the backend's own)
    virtual bool map(int plane, int slot, int64_t page, int32_t phys) = 0;
    virtual bool unmap(int plane, int slot, int64_t page) = 0;
    // contents of page `src_page` of src_slot into page `dst_page` of dst_slot (both mapped)
    virtual bool copy_page(int plane, int dst_slot, int64_t dst_page, int src_slot, int64_t src_page) = 0;
    // the whole slot of a state plane
    virtual bool copy_state(int plane, int dst_slot, int src_slot) = 0;
};

struct PagerStats {
    int64_t pool_pages = 0, free_pages = 0;
    int64_t mapped_pages = 0;     // pool pages mapped (a shared page counts once per mapping)
    int64_t shared_pages = 0;     // pool pages mapped by more than one slot
    int32_t open_slots = 0;
};

class Pager {
public:
    static constexpr int32_t kUnmapped = -1;
    static constexpr int32_t kHome = -2;

    // planes must already be validated (row_bytes divides page_bytes, whole pages per slot)
    int init(const std::vector<PagerPlane>& planes, int max_seqs, int64_t pool_pages) {
        planes_ = planes;
        max_seqs_ = max_seqs;
        refs_.assign((size_t)pool_pages, 0);
        free_.clear();
        for (int64_t i = pool_pages - 1; i >= 0; --i) free_.push_back((int32_t)i);
        table_.assign(planes_.size() * (size_t)max_seqs, {});
        for (size_t p = 0; p < planes_.size(); ++p) {
            if (planes_[p].state) continue;
            for (int s = 0; s < max_seqs; ++s) {
                auto& t = tab(p, s);
                t.assign((size_t)planes_[p].pages, kUnmapped);
                t[0] = kHome;
            }
        }
        tokens_.assign((size_t)max_seqs, -1);
        return kPgOk;
    }

    int max_seqs() const { return max_seqs_; }
    const std::vector<PagerPlane>& planes() const { return planes_; }
    int64_t tokens(int slot) const { return valid(slot) ? tokens_[(size_t)slot] : -1; }
    // page-table entry: pool page id, kHome or kUnmapped
    int32_t entry(int plane, int slot, int64_t page) const { return table_[(size_t)plane * max_seqs_ + slot][(size_t)page]; }
    int32_t refs(int32_t phys) const { return refs_[(size_t)phys]; }

    // the lowest closed slot, opened with no tokens
    int open(int* slot) {
        for (int s = 0; s < max_seqs_; ++s)
            if (tokens_[(size_t)s] < 0) {
                tokens_[(size_t)s] = 0;
                *slot = s;
                return kPgOk;
            }
        return kPgNoMem;
    }

    // back every row a sequence of n tokens can read or write: rows [0, min(rows, n / m + 1))
    int reserve(int slot, int64_t n, PagerOps& ops) {
        if (!is_open(slot) || n < 0) return kPgInval;
        for (const auto& pl : planes_)
            if (!pl.state && n / pl.m > pl.rows) return kPgShape;
        int64_t need = 0;
        for (size_t p = 0; p < planes_.size(); ++p) {
            if (planes_[p].state) continue;
            const auto& t = tab(p, slot);
            for (int64_t i = 1, e = pages_for(p, n); i < e; ++i) need += t[(size_t)i] == kUnmapped;
        }
        if (need > (int64_t)free_.size()) return kPgNoMem;
        std::vector<Undo> undo;
        for (size_t p = 0; p < planes_.size(); ++p) {
            if (planes_[p].state) continue;
            for (int64_t i = 1, e = pages_for(p, n); i < e; ++i) {
                if (tab(p, slot)[(size_t)i] != kUnmapped) continue;
                if (!map_fresh((int)p, slot, i, ops, undo)) return rollback(undo, ops);
            }
        }
        if (n > tokens_[(size_t)slot]) tokens_[(size_t)slot] = n;
        return kPgOk;
    }

    // a new slot holding the first n tokens of src (n <= tokens of src)
    int fork(int src, int64_t n, int* dst, PagerOps& ops) {
        if (!is_open(src) || n < 0 || n > tokens_[(size_t)src]) return kPgInval;
        int d = -1;
        for (int s = 0; s < max_seqs_; ++s)
            if (tokens_[(size_t)s] < 0) {
                d = s;
                break;
            }
        if (d < 0) return kPgNoMem;
        // fresh pages: the page holding the first row the child writes, when it is not page 0
        int64_t need = 0;
        for (size_t p = 0; p < planes_.size(); ++p)
            if (!planes_[p].state && boundary_page(p, n) >= 1) ++need;
        if (need > (int64_t)free_.size()) return kPgNoMem;
        std::vector<Undo> undo;
        for (size_t p = 0; p < planes_.size(); ++p) {
            const auto& pl = planes_[p];
            if (pl.state) {
                if (!ops.copy_state((int)p, d, src)) return rollback(undo, ops);
                continue;
            }
            const int64_t full = complete_rows(p, n) / pl.rpp;  // pages of complete entries only
            for (int64_t i = 1; i < full; ++i) {                 // shared (page 0 is always private)
                const int32_t ph = tab(p, src)[(size_t)i];
                if (!ops.map((int)p, d, i, ph)) return rollback(undo, ops);
                tab(p, d)[(size_t)i] = ph;
                ++refs_[(size_t)ph];
                undo.push_back({(int)p, d, i});
            }
            const int64_t bp = boundary_page(p, n);
            if (bp >= 1 && !map_fresh((int)p, d, bp, ops, undo)) return rollback(undo, ops);
            // page 0 and the complete rows of the boundary page are copied
            if (!ops.copy_page((int)p, d, 0, src, 0)) return rollback(undo, ops);
            if (bp >= 1 && complete_rows(p, n) % pl.rpp != 0 && !ops.copy_page((int)p, d, bp, src, bp))
                return rollback(undo, ops);
        }
        tokens_[(size_t)d] = n;
        *dst = d;
        return kPgOk;
    }

    // unmap every pool page of the slot (home pages stay) and free the slot
    int close(int slot, PagerOps& ops) {
        if (!is_open(slot)) return kPgInval;
        int rc = kPgOk;
        for (size_t p = 0; p < planes_.size(); ++p) {
            if (planes_[p].state) continue;
            auto& t = tab(p, slot);
            for (int64_t i = 1; i < (int64_t)t.size(); ++i) {
                const int32_t ph = t[(size_t)i];
                if (ph < 0) continue;
                if (!ops.unmap((int)p, slot, i)) {  // still mapped: the slot keeps it
                    rc = kPgBackend;
                    continue;
                }
                if (--refs_[(size_t)ph] == 0) free_.push_back(ph);
                t[(size_t)i] = kUnmapped;
            }
        }
        tokens_[(size_t)slot] = -1;
        return rc;
    }

    PagerStats stats() const {
        PagerStats s;
        s.pool_pages = (int64_t)refs_.size();
        s.free_pages = (int64_t)free_.size();
        for (int32_t r : refs_) {
            s.mapped_pages += r;
            s.shared_pages += r > 1;
        }
        for (int64_t t : tokens_) s.open_slots += t >= 0;
        return s;
    }

    bool is_open(int slot) const { return valid(slot) && tokens_[(size_t)slot] >= 0; }

private:
    struct Undo {
        int plane, slot;
        int64_t page;
    };

    bool valid(int slot) const { return slot >= 0 && slot < max_seqs_; }
    std::vector<int32_t>& tab(size_t p, int s) { return table_[p * (size_t)max_seqs_ + (size_t)s]; }
    const std::vector<int32_t>& tab(size_t p, int s) const { return table_[p * (size_t)max_seqs_ + (size_t)s]; }

    // pages that back rows [0, min(rows, n / m + 1))
    int64_t pages_for(size_t p, int64_t n) const {
        const auto& pl = planes_[p];
        int64_t r = n / pl.m + 1;
        if (r > pl.rows) r = pl.rows;
        return (r + pl.rpp - 1) / pl.rpp;
    }
    // entries a sequence of n tokens has completed (capped at the plane's rows)
    int64_t complete_rows(size_t p, int64_t n) const {
        const auto& pl = planes_[p];
        return n / pl.m < pl.rows ? n / pl.m : pl.rows;
    }
    // page of the first row a sequence of n tokens has not completed; -1 when every row is complete
    int64_t boundary_page(size_t p, int64_t n) const {
        const auto& pl = planes_[p];
        const int64_t r = complete_rows(p, n);
        return r < pl.rows ? r / pl.rpp : -1;
    }

    bool map_fresh(int p, int slot, int64_t page, PagerOps& ops, std::vector<Undo>& undo) {
        const int32_t ph = free_.back();
        if (!ops.map(p, slot, page, ph)) return false;
        free_.pop_back();
        refs_[(size_t)ph] = 1;
        tab((size_t)p, slot)[(size_t)page] = ph;
        undo.push_back({p, slot, page});
        return true;
    }

    int rollback(std::vector<Undo>& undo, PagerOps& ops) {
        for (auto it = undo.rbegin(); it != undo.rend(); ++it) {
            auto& t = tab((size_t)it->plane, it->slot);
            const int32_t ph = t[(size_t)it->page];
            ops.unmap(it->plane, it->slot, it->page);
            if (--refs_[(size_t)ph] == 0) free_.push_back(ph);
            t[(size_t)it->page] = kUnmapped;
        }
        undo.clear();
        return kPgBackend;
    }

    std::vector<PagerPlane> planes_;
    int max_seqs_ = 0;
    std::vector<std::vector<int32_t>> table_;  // [plane][slot] -> page -> pool page / kHome / kUnmapped
    std::vector<int32_t> refs_;                // mappings of each pool page
    std::vector<int32_t> free_;                // free pool pages (a stack: the lowest id on top)
    std::vector<int64_t> tokens_;              // tokens of each slot, -1 = closed
};

}  // namespace lca
