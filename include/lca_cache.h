/*
 * lca_cache.h -- the paged heterogeneous KV cache of the MI355X compressed-attention library.
 *
 * [R] "DeepSeek-V4 中文翻译", section 3.5.1 (KV cache layout and cache management): the
 * cache holds a classical part (the compressed CSA / HCA entries, kept in blocks whose number of
 * raw tokens may be any multiple of lcm(m, m')) and a state cache for the sliding-window rows and
 * the tail of raw tokens not yet compressed: a fixed pool, preallocated, whose pieces are handed
 * out to sequences as they come.  Section 3.5.2: the stored entries of a shared prefix are reused
 * instead of prefilling the prefix again.
 *
 * Design.  The GPU's own page tables are the block table.  Every plane (one storage array of the
 * cache, e.g. the nope rows of one layer's compressed stream) is a virtual address range of
 * max_seqs slots of `rows` rows each, laid out exactly as the lca.h calls expect a [B][cap][...]
 * plane: slot b of the cache is sequence b of a batch, and an lca_kv built from plane bases with
 * cap = rows is passed to those calls unchanged.  Nothing in the attention, indexer or compressor
 * kernels knows about pages.
 *   - Classical planes (m >= 1) are backed on demand by pages of `page_bytes` from one pool of
 *     pool_pages pages created with the cache.  A page of a plane with rows of r bytes and ratio m
 *     covers (page_bytes / r) * m raw tokens: the pages' block.  Page 0 of every (plane, slot) is
 *     backed for the cache's whole life (outside the pool), so the row-0 reads that kernels issue
 *     for padded lanes are always backed.
 *   - State planes are backed whole at creation (the fixed pool of the state cache); slot b's
 *     rows belong to whichever sequence holds slot b.
 *   - Prefix reuse: lca_cache_fork maps the parent's pages of complete entries into the child
 *     (shared, reference counted; complete entries are never written again) and copies the page
 *     holding the child's first incomplete entry, page 0, and the state planes.
 *
 * Memory: the cache owns all of it (unlike the lca.h calls, which never allocate).  create
 * allocates the pool, the home pages and the state planes; reserve and fork only map pages of
 * the pool; close and destroy wait for the device (hipDeviceSynchronize) before they unmap.
 *
 * Reads beyond the backed rows are not checked: a caller must reserve every sequence of a batch
 * for the tokens its calls touch (lca_cache_reserve with the sequence's length after the call)
 * and must pass only top-k indices below the reserved entries.  Slots that are not open may be
 * part of a batch with q_pos = 0 (their reads stay in page 0 and the state planes).
 *
 * Every function returns LCA_OK or an LCA_* status (lca.h), with lca_last_error() describing the
 * problem; on an error nothing is changed.  The cache belongs to the device that was current at
 * creation; its functions make that device current while they run and restore the caller's.
 * One cache must not be used from several host threads at once.
 */
#ifndef LCA_CACHE_H
#define LCA_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "lca.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lca_cache lca_cache;

typedef struct lca_cache_plane {
    int64_t row_bytes;  /* bytes of one row                                               */
    int64_t rows;       /* rows per slot: the cap of the lca_kv built on this plane        */
    int32_t m;          /* classical plane: raw tokens per row (1, or the compression
                           ratio m); 0 = state plane                                       */
    int32_t reserved;   /* must be 0                                                       */
} lca_cache_plane;

typedef struct lca_cache_stats {
    int64_t pool_pages;     /* pages in the pool                                           */
    int64_t free_pages;     /* pages of the pool not mapped anywhere                       */
    int64_t mapped_pages;   /* mappings of pool pages (a shared page counts per mapping)   */
    int64_t shared_pages;   /* pool pages mapped by more than one slot                     */
    int64_t device_bytes;   /* device memory the cache holds (pool, home pages, state)     */
    int64_t page_bytes;
    int32_t open_slots;
    int32_t max_seqs;
} lca_cache_stats;

/*
 * lca_cache_create -- n_planes planes (host array), max_seqs slots (1 .. LCA_MAX_BATCH), pages
 * of page_bytes (a multiple of the device's virtual-memory granularity, 4096 B on MI355X),
 * pool_pages pages in the pool.  Classical planes need page_bytes % row_bytes == 0 and
 * rows * row_bytes % page_bytes == 0, and every classical plane's page must cover a multiple of
 * lcm of the classical planes' m raw tokens ([R] 3.5.1's block rule); state planes need
 * rows * row_bytes % 16 == 0.  Errors: LCA_EINVAL (NULL, counts, m < 0, reserved != 0),
 * LCA_ESHAPE (the rules above), LCA_EHIP (no virtual memory management, or the runtime refused
 * an allocation).
 */
int lca_cache_create(const lca_cache_plane* planes, int32_t n_planes, int32_t max_seqs, int64_t page_bytes,
                     int64_t pool_pages, lca_cache** cache);

/* Waits for the device, then unmaps and frees everything.  NULL is accepted. */
int lca_cache_destroy(lca_cache* cache);

/* Device address of plane `plane`: [max_seqs][rows][row_bytes], page aligned. */
int lca_cache_plane_base(const lca_cache* cache, int32_t plane, void** base);

/* Opens the lowest free slot for a new sequence of 0 tokens.  LCA_ENOMEM when every slot is open. */
int lca_cache_open(lca_cache* cache, int32_t* slot);

/*
 * Backs every classical row that a sequence of n_tokens raw tokens can read or write: rows
 * [0, min(rows, n_tokens / m + 1)) of every classical plane.  Never unmaps (a smaller n_tokens
 * is a no-op).  Errors: LCA_EINVAL (slot not open, n_tokens < 0), LCA_ESHAPE (n_tokens / m
 * beyond a plane's rows), LCA_ENOMEM (too few free pages: nothing is mapped).
 */
int lca_cache_reserve(lca_cache* cache, int32_t slot, int64_t n_tokens);

/*
 * Opens a new slot *child holding the first n_tokens tokens of slot parent (n_tokens <= the
 * parent's reserved tokens): pages of the parent whose rows are all complete entries
 * (row < n_tokens / m) are mapped into the child, page 0 and the page holding row n_tokens / m
 * are copied into the child's own pages, and every state plane's slot is copied.  The copies are
 * enqueued on `stream` (hipStream_t as void*), after whatever the caller enqueued there before
 * (the writes of the parent's rows).  The state planes are copied as they are: a fork at the
 * parent's current length gets its exact window and tail; a fork at an earlier length must
 * rebuild them.  Errors: LCA_EINVAL, LCA_ENOMEM (no free slot or page), LCA_EHIP.
 */
int lca_cache_fork(lca_cache* cache, int32_t parent, int64_t n_tokens, void* stream, int32_t* child);

/* Waits for the device, unmaps the slot's pool pages (shared pages stay with their other
 * holders) and frees the slot.  Errors: LCA_EINVAL (slot not open), LCA_EHIP. */
int lca_cache_close(lca_cache* cache, int32_t slot);

/* Tokens reserved for a slot (-1 = not open). */
int lca_cache_tokens(const lca_cache* cache, int32_t slot, int64_t* n_tokens);

int lca_cache_get_stats(const lca_cache* cache, lca_cache_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* LCA_CACHE_H */
