// cache.hip -- the paged heterogeneous KV cache (include/lca_cache.h) on HIP virtual memory.
//
// "DeepSeek-V4 中文翻译" section 3.5.1: compressed entries in a classical cache of blocks,
// sliding-window rows and the uncompressed tail in a fixed state-cache pool; section 3.5.2:
// entries of a shared prefix are reused.  Each plane is one reserved virtual range laid out as
// the [B][cap][row] planes the attention, indexer and compressor calls take, so the GPU's page
// tables act as the block table and the kernels read through them at no cost.  Page bookkeeping
// (which pool page backs which page of which slot, reference counts, rollback) is in pager.h;
// this file maps, unmaps and copies.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "../../include/lca.h"
#include "../../include/lca_cache.h"
#include "pager.h"
#include "status.h"

namespace {

using Handle = hipMemGenericAllocationHandle_t;

// n16 16-byte chunks from src to dst (grid-stride)
__global__ void __launch_bounds__(256) cache_copy(uint4* dst, const uint4* src, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) cache_zero(uint4* dst, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
        dst[i] = uint4{0u, 0u, 0u, 0u};
}

unsigned blocks_for(int64_t n16) {
    const int64_t b = (n16 + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

struct DeviceScope {
    int prev = -1;
    explicit DeviceScope(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceScope() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

}  // namespace

struct lca_cache : lca::PagerOps {
    int device = 0;
    int64_t page_bytes = 0;
    int max_seqs = 0;
    std::vector<lca_cache_plane> desc;
    std::vector<char*> base;           // reserved range of each plane
    std::vector<size_t> va_bytes;
    std::vector<Handle> pool;          // pool pages
    std::vector<Handle> home;          // [plane][slot] page 0 of classical planes
    std::vector<Handle> state;         // backing of each state plane (0 for classical planes)
    std::vector<size_t> state_bytes;
    int64_t device_bytes = 0;
    lca::Pager pager;
    hipStream_t op_stream = nullptr;   // stream of the copies of the running fork
    hipError_t last = hipSuccess;

    int64_t slot_bytes(int p) const { return desc[(size_t)p].rows * desc[(size_t)p].row_bytes; }
    char* page_va(int p, int slot, int64_t page) const {
        return base[(size_t)p] + (int64_t)slot * slot_bytes(p) + page * page_bytes;
    }

    bool map_handle(void* va, size_t bytes, Handle h) {
        if ((last = hipMemMap(va, bytes, 0, h, 0)) != hipSuccess) return false;
        hipMemAccessDesc acc = {};
        acc.location.type = hipMemLocationTypeDevice;
        acc.location.id = device;
        acc.flags = hipMemAccessFlagsProtReadWrite;
        if ((last = hipMemSetAccess(va, bytes, &acc, 1)) != hipSuccess) {
            (void)hipMemUnmap(va, bytes);
            return false;
        }
        return true;
    }

    // PagerOps
    bool map(int p, int slot, int64_t page, int32_t phys) override {
        return map_handle(page_va(p, slot, page), (size_t)page_bytes, pool[(size_t)phys]);
    }
    bool unmap(int p, int slot, int64_t page) override {
        return (last = hipMemUnmap(page_va(p, slot, page), (size_t)page_bytes)) == hipSuccess;
    }
    bool copy(void* dst, const void* src, int64_t bytes) {
        const int64_t n16 = bytes / 16;
        hipLaunchKernelGGL(cache_copy, dim3(blocks_for(n16)), dim3(256), 0, op_stream, (uint4*)dst,
                           (const uint4*)src, n16);
        return (last = hipGetLastError()) == hipSuccess;
    }
    bool copy_page(int p, int dslot, int64_t dpage, int sslot, int64_t spage) override {
        return copy(page_va(p, dslot, dpage), page_va(p, sslot, spage), page_bytes);
    }
    bool copy_state(int p, int dslot, int sslot) override {
        return copy(base[(size_t)p] + (int64_t)dslot * slot_bytes(p), base[(size_t)p] + (int64_t)sslot * slot_bytes(p),
                    slot_bytes(p));
    }

    // releases whatever create got so far (also the error path of create)
    void teardown() {
        (void)hipDeviceSynchronize();
        for (size_t p = 0; p < desc.size(); ++p) {
            if (!base[p]) continue;
            if (desc[p].m == 0) {
                if (state[p]) (void)hipMemUnmap(base[p], state_bytes[p]);
            } else {
                const auto& pl = pager.planes();
                for (int s = 0; s < max_seqs; ++s) {
                    if (home[p * (size_t)max_seqs + (size_t)s]) (void)hipMemUnmap(page_va((int)p, s, 0), (size_t)page_bytes);
                    if (p < pl.size())
                        for (int64_t i = 1; i < pl[p].pages; ++i)
                            if (pager.entry((int)p, s, i) >= 0) (void)hipMemUnmap(page_va((int)p, s, i), (size_t)page_bytes);
                }
            }
            (void)hipMemAddressFree(base[p], va_bytes[p]);
        }
        for (Handle h : pool) (void)hipMemRelease(h);
        for (Handle h : home)
            if (h) (void)hipMemRelease(h);
        for (Handle h : state)
            if (h) (void)hipMemRelease(h);
        pool.clear();
        home.clear();
        state.clear();
    }
};

namespace {

int hip_fail(const char* what, hipError_t e) {
    return lca::set_error(LCA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int pager_status(int rc, const lca_cache* c, const char* what) {
    switch (rc) {
    case lca::kPgOk: return LCA_OK;
    case lca::kPgNoMem: return lca::set_error(LCA_ENOMEM, "%s: no free slot or page in the pool", what);
    case lca::kPgShape: return lca::set_error(LCA_ESHAPE, "%s: the tokens exceed a plane's rows", what);
    case lca::kPgBackend: return hip_fail(what, c->last);
    default: return lca::set_error(LCA_EINVAL, "%s: slot not open or bad token count", what);
    }
}

}  // namespace

extern "C" {

int lca_cache_create(const lca_cache_plane* planes, int32_t n_planes, int32_t max_seqs, int64_t page_bytes,
                     int64_t pool_pages, lca_cache** out) {
    lca::clear_error();
    if (!planes || !out) return lca::set_error(LCA_EINVAL, "planes / cache is NULL");
    *out = nullptr;
    if (n_planes < 1 || n_planes > 1024) return lca::set_error(LCA_EINVAL, "n_planes %d outside [1, 1024]", n_planes);
    if (max_seqs < 1 || max_seqs > LCA_MAX_BATCH)
        return lca::set_error(LCA_EINVAL, "max_seqs %d outside [1, %d]", max_seqs, LCA_MAX_BATCH);
    if (pool_pages < 0 || pool_pages > INT32_MAX) return lca::set_error(LCA_EINVAL, "bad pool_pages");
    if (page_bytes <= 0) return lca::set_error(LCA_ESHAPE, "page_bytes must be positive");
    int64_t L = 1;  // lcm of the classical planes' m
    for (int p = 0; p < n_planes; ++p) {
        const lca_cache_plane& d = planes[p];
        if (d.m < 0 || d.reserved != 0 || d.row_bytes < 1 || d.rows < 1)
            return lca::set_error(LCA_EINVAL, "plane %d: bad row_bytes / rows / m / reserved", p);
        if (d.m == 0) {
            if ((d.rows * d.row_bytes) % 16 != 0)
                return lca::set_error(LCA_ESHAPE, "state plane %d: rows * row_bytes must be a multiple of 16", p);
            continue;
        }
        if (page_bytes % d.row_bytes != 0 || (d.rows * d.row_bytes) % page_bytes != 0)
            return lca::set_error(LCA_ESHAPE, "plane %d: row_bytes %lld must divide page_bytes and rows * row_bytes "
                                  "fill whole pages", p, (long long)d.row_bytes);
        L = L / gcd64(L, d.m) * d.m;
    }
    for (int p = 0; p < n_planes; ++p)
        if (planes[p].m > 0 && (page_bytes / planes[p].row_bytes) * planes[p].m % L != 0)
            return lca::set_error(LCA_ESHAPE, "plane %d: a page covers %lld raw tokens, not a multiple of lcm(m) = %lld",
                                  p, (long long)((page_bytes / planes[p].row_bytes) * planes[p].m), (long long)L);

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    int vmm = 0;
    e = hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, dev);
    if (e != hipSuccess || !vmm) return lca::set_error(LCA_EHIP, "device %d has no virtual memory management", dev);
    hipMemAllocationProp prop = {};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = dev;
    size_t gran = 0;
    if ((e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum)) != hipSuccess)
        return hip_fail("hipMemGetAllocationGranularity", e);
    if (page_bytes % (int64_t)gran != 0)
        return lca::set_error(LCA_ESHAPE, "page_bytes %lld is not a multiple of %zu", (long long)page_bytes, gran);

    lca_cache* c = new lca_cache();
    c->device = dev;
    c->page_bytes = page_bytes;
    c->max_seqs = max_seqs;
    c->desc.assign(planes, planes + n_planes);
    c->base.assign((size_t)n_planes, nullptr);
    c->va_bytes.assign((size_t)n_planes, 0);
    c->state.assign((size_t)n_planes, Handle{});
    c->state_bytes.assign((size_t)n_planes, 0);
    c->home.assign((size_t)n_planes * max_seqs, Handle{});
    std::vector<lca::PagerPlane> pp((size_t)n_planes);
    auto bail = [&](const char* what) {
        const int rc = hip_fail(what, e);
        c->teardown();
        delete c;
        return rc;
    };
    for (int p = 0; p < n_planes; ++p) {
        const lca_cache_plane& d = planes[p];
        const int64_t bytes = (int64_t)max_seqs * d.rows * d.row_bytes;
        const size_t va = (size_t)((bytes + (int64_t)gran - 1) / (int64_t)gran * (int64_t)gran);
        void* ptr = nullptr;
        if ((e = hipMemAddressReserve(&ptr, va, d.m ? (size_t)page_bytes : gran, nullptr, 0)) != hipSuccess)
            return bail("hipMemAddressReserve");
        c->base[(size_t)p] = (char*)ptr;
        c->va_bytes[(size_t)p] = va;
        pp[(size_t)p].row_bytes = d.row_bytes;
        pp[(size_t)p].rows = d.rows;
        pp[(size_t)p].m = d.m ? d.m : 1;
        pp[(size_t)p].state = d.m == 0;
        if (d.m == 0) {  // the state plane, backed whole
            if ((e = hipMemCreate(&c->state[(size_t)p], va, &prop, 0)) != hipSuccess) return bail("hipMemCreate (state)");
            c->state_bytes[(size_t)p] = va;
            c->device_bytes += (int64_t)va;
            if (!c->map_handle(ptr, va, c->state[(size_t)p])) {
                e = c->last;
                return bail("hipMemMap (state)");
            }
            const int64_t n16 = (int64_t)va / 16;
            hipLaunchKernelGGL(cache_zero, dim3(blocks_for(n16)), dim3(256), 0, nullptr, (uint4*)ptr, n16);
            continue;
        }
        pp[(size_t)p].rpp = page_bytes / d.row_bytes;
        pp[(size_t)p].pages = d.rows / pp[(size_t)p].rpp;
        for (int s = 0; s < max_seqs; ++s) {  // home pages
            Handle& h = c->home[(size_t)p * max_seqs + (size_t)s];
            if ((e = hipMemCreate(&h, (size_t)page_bytes, &prop, 0)) != hipSuccess) return bail("hipMemCreate (home)");
            c->device_bytes += page_bytes;
            if (!c->map_handle(c->page_va(p, s, 0), (size_t)page_bytes, h)) {
                e = c->last;
                return bail("hipMemMap (home)");
            }
            const int64_t n16 = page_bytes / 16;
            hipLaunchKernelGGL(cache_zero, dim3(blocks_for(n16)), dim3(256), 0, nullptr, (uint4*)c->page_va(p, s, 0), n16);
        }
    }
    c->pool.reserve((size_t)pool_pages);
    for (int64_t i = 0; i < pool_pages; ++i) {
        Handle h{};
        if ((e = hipMemCreate(&h, (size_t)page_bytes, &prop, 0)) != hipSuccess) return bail("hipMemCreate (pool)");
        c->pool.push_back(h);
        c->device_bytes += page_bytes;
    }
    c->pager.init(pp, max_seqs, pool_pages);
    if ((e = hipDeviceSynchronize()) != hipSuccess) return bail("zeroing the cache");
    *out = c;
    return LCA_OK;
}

int lca_cache_destroy(lca_cache* c) {
    lca::clear_error();
    if (!c) return LCA_OK;
    DeviceScope ds(c->device);
    c->teardown();
    delete c;
    return LCA_OK;
}

int lca_cache_plane_base(const lca_cache* c, int32_t plane, void** base) {
    lca::clear_error();
    if (!c || !base) return lca::set_error(LCA_EINVAL, "cache / base is NULL");
    if (plane < 0 || plane >= (int32_t)c->desc.size()) return lca::set_error(LCA_EINVAL, "no plane %d", plane);
    *base = c->base[(size_t)plane];
    return LCA_OK;
}

int lca_cache_open(lca_cache* c, int32_t* slot) {
    lca::clear_error();
    if (!c || !slot) return lca::set_error(LCA_EINVAL, "cache / slot is NULL");
    int s = -1;
    const int rc = c->pager.open(&s);
    if (rc != lca::kPgOk) return pager_status(rc, c, "lca_cache_open");
    *slot = s;
    return LCA_OK;
}

int lca_cache_reserve(lca_cache* c, int32_t slot, int64_t n_tokens) {
    lca::clear_error();
    if (!c) return lca::set_error(LCA_EINVAL, "cache is NULL");
    DeviceScope ds(c->device);
    return pager_status(c->pager.reserve(slot, n_tokens, *c), c, "lca_cache_reserve");
}

int lca_cache_fork(lca_cache* c, int32_t parent, int64_t n_tokens, void* stream, int32_t* child) {
    lca::clear_error();
    if (!c || !child) return lca::set_error(LCA_EINVAL, "cache / child is NULL");
    DeviceScope ds(c->device);
    c->op_stream = (hipStream_t)stream;
    int d = -1;
    const int rc = c->pager.fork(parent, n_tokens, &d, *c);
    c->op_stream = nullptr;
    if (rc != lca::kPgOk) return pager_status(rc, c, "lca_cache_fork");
    *child = d;
    return LCA_OK;
}

int lca_cache_close(lca_cache* c, int32_t slot) {
    lca::clear_error();
    if (!c) return lca::set_error(LCA_EINVAL, "cache is NULL");
    if (!c->pager.is_open(slot)) return lca::set_error(LCA_EINVAL, "lca_cache_close: slot %d is not open", slot);
    DeviceScope ds(c->device);
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail("lca_cache_close", e);
    return pager_status(c->pager.close(slot, *c), c, "lca_cache_close");
}

int lca_cache_tokens(const lca_cache* c, int32_t slot, int64_t* n_tokens) {
    lca::clear_error();
    if (!c || !n_tokens) return lca::set_error(LCA_EINVAL, "cache / n_tokens is NULL");
    if (slot < 0 || slot >= c->max_seqs) return lca::set_error(LCA_EINVAL, "no slot %d", slot);
    *n_tokens = c->pager.tokens(slot);
    return LCA_OK;
}

int lca_cache_get_stats(const lca_cache* c, lca_cache_stats* st) {
    lca::clear_error();
    if (!c || !st) return lca::set_error(LCA_EINVAL, "cache / stats is NULL");
    const lca::PagerStats s = c->pager.stats();
    st->pool_pages = s.pool_pages;
    st->free_pages = s.free_pages;
    st->mapped_pages = s.mapped_pages;
    st->shared_pages = s.shared_pages;
    st->device_bytes = c->device_bytes;
    st->page_bytes = c->page_bytes;
    st->open_slots = s.open_slots;
    st->max_seqs = c->max_seqs;
    return LCA_OK;
}

}  // extern "C"
