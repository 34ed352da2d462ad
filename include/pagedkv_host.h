/*
 * pagedkv_host.h -- host control plane of the paged KV cache: the page
 * allocator, sequences that own (and share) pages, the builder of one step's
 * metadata (block_table, seq_lens, query_start_loc) and a page-trie prefix
 * index.  Pure host C++ in libpagedkv.so; nothing declared here makes a GPU
 * call, so all of it runs and is tested without an accelerator.
 *
 * What it implements, from the pages:
 *  - Memory is handed out in whole pages of page_size rows; a sequence's
 *    block_table row lists its pages in order and token position p lives at
 *    slot page * page_size + p % page_size (page "Add paged / block-table KV
 *    cache export (--features paged-cache)", onnxruntime/mobius #395, PR
 *    summary and "ONNX I/O contract").
 *  - The allocator of page "[Draft] kv paged kernels" (ROCm/maxtext #93),
 *    the commit adding the host page allocator (milestones M4, M4.5): it
 *    deals in pages rather than token indices; releasing a page that is not
 *    allocated is reported as an error rather than ignored; stale handles are
 *    caught by an epoch stored with each entry; and a released page counts as
 *    dirty (it still holds its previous owner's K/V) until the caller confirms
 *    it was overwritten, the metadata builder refusing to describe a dirty
 *    page.
 *  - The prefix index of the same page, the commit adding it (milestone M5):
 *    a trie whose nodes are single pages, keyed by a hash chained from the
 *    parent's key and started from a namespace digest (so two model
 *    configurations never share a root); recency is a monotonic counter, so
 *    eviction order is reproducible; a match stops one page short of a fully
 *    cached prompt, so the request keeps a query token to run; pages the
 *    index adopts stay alive while it holds them.
 *
 * Object model.  A pool manages page ids [0, num_pages).  A page handle is
 * (generation << 32 | page id) and a sequence handle (epoch << 32 | slot),
 * both counted modulo 2^31 so that handles are non-negative; the generation
 * of a page grows each time it returns to the free list and the epoch of a
 * sequence slot each time the sequence is released, so a handle kept past
 * that point no longer matches (until 2^31 more recyclings of the same page
 * or slot).  Each in-use page has a reference
 * count: one per sequence holding it and one while the prefix index holds it.
 * A page is in exactly one of: free, or in use with a positive count.
 *
 * Errors: every int function returns PKV_OK (0) or a negative status: the
 * argument statuses of pagedkv.h (PKV_ERR_NULL, PKV_ERR_SHAPE) and
 *   PKV_ERR_NO_PAGES   (-20)  too few free pages (nothing changed)
 *   PKV_ERR_BAD_HANDLE (-21)  a stale or unknown sequence or page handle, or
 *                             a page released more often than it is held
 *   PKV_ERR_DIRTY      (-22)  a page the builder would describe is dirty
 * A failing call changes nothing.  Output arrays are written only up to the
 * sizes the arguments state.  A pool is not thread-safe; one thread drives it.
 */
#ifndef PAGEDKV_HOST_H
#define PAGEDKV_HOST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ERR_NO_PAGES (-20)
#define PKV_ERR_BAD_HANDLE (-21)
#define PKV_ERR_DIRTY (-22)

typedef struct pkv_page_pool pkv_page_pool;

/* A pool over page ids [0, num_pages) of page_size rows each.  All pages start
 * free and clean.  Returns NULL for num_pages <= 0, page_size <= 0 or out of
 * host memory. */
pkv_page_pool* pkv_pool_create(int64_t num_pages, int32_t page_size);
void pkv_pool_destroy(pkv_page_pool* pool);
int64_t pkv_pool_free_pages(const pkv_page_pool* pool);
int64_t pkv_pool_used_pages(const pkv_page_pool* pool);

/* Page handles.  pkv_page_alloc takes n pages off the free list (all or none)
 * and writes their handles, reference count 1 each; the most recently freed
 * pages come back first.  pkv_page_release drops one reference per handle
 * listed (a handle may repeat up to its page's count); a page whose count
 * reaches 0 returns to the free list, dirty, with its generation bumped.
 * pkv_page_confirm marks in-use pages as overwritten (clean). */
int pkv_page_alloc(pkv_page_pool* pool, int64_t n, int64_t* handles_out);
int pkv_page_release(pkv_page_pool* pool, const int64_t* handles, int64_t n);
int pkv_page_confirm(pkv_page_pool* pool, const int64_t* page_ids, int64_t n);
/* Reference count of a page (0 = free, -1 = id out of range) and its dirty
 * flag (1 dirty, 0 clean, -1 out of range). */
int32_t pkv_page_refcount(const pkv_page_pool* pool, int64_t page_id);
int32_t pkv_page_dirty(const pkv_page_pool* pool, int64_t page_id);

/* Sequences.
 * pkv_seq_create: an empty sequence.
 * pkv_seq_append: grows the sequence by n tokens, taking new pages only as its
 *   last page fills, and writes the slot of each new token (page id *
 *   page_size + row) to slots_out[0 .. n).
 * pkv_seq_fork: a sequence holding the first n_tokens (<= the parent's
 *   length) of `parent`: the parent's whole pages among them are shared
 *   (reference counts grow).  If n_tokens ends inside a page, that page's
 *   first n_tokens % page_size rows must be copied into the child's own fresh
 *   page, so that the child can append without touching the parent: the
 *   slots of the first row to copy and of its destination, and the row
 *   count, are written to copy_out[0..2] (count 0 when nothing is to copy).
 *   The caller copies those rows of the KV pools before the child's first
 *   attention.
 * pkv_seq_release: drops the sequence and its page references.
 * pkv_seq_length: length in tokens (negative status for a bad handle).
 * pkv_seq_pages: writes min(count, capacity) page ids; returns the count. */
int pkv_seq_create(pkv_page_pool* pool, int64_t* seq_out);
int pkv_seq_append(pkv_page_pool* pool, int64_t seq, int64_t n, int64_t* slots_out);
int pkv_seq_fork(pkv_page_pool* pool, int64_t parent, int64_t n_tokens, int64_t* child_out, int64_t* copy_out);
/* pkv_seq_append for a batch: sequence seqs[b] grows by n[b] tokens, b in
 * [0, B), and the slots of all new tokens are written to slots_out in
 * sequence order (sum(n) entries).  All or nothing: with a bad handle, a
 * repeated sequence or too few free pages for the whole batch, nothing
 * changes.  One call per step instead of one per sequence. */
int pkv_seq_append_batch(pkv_page_pool* pool, const int64_t* seqs, int64_t B, const int64_t* n, int64_t* slots_out);
int pkv_seq_release(pkv_page_pool* pool, int64_t seq);
int64_t pkv_seq_length(const pkv_page_pool* pool, int64_t seq);
int64_t pkv_seq_pages(const pkv_page_pool* pool, int64_t seq, int64_t* page_ids_out, int64_t capacity);

/* One step's attention metadata for sequences seqs[0 .. B) whose last
 * n_new[b] tokens are this step's query rows (append them first):
 *   block_table [B, max_blocks]: row b = the page ids of seqs[b], padded with
 *                                pad_page (never read by the kernels);
 *   seq_lens [B]               : lengths;
 *   query_start_loc [B + 1]    : 0, then the running sum of n_new.
 * PKV_ERR_SHAPE if a sequence has more than max_blocks pages or n_new[b] is
 * negative or above its length; PKV_ERR_DIRTY if any listed page is dirty;
 * nothing is written then. */
int pkv_build_step(const pkv_page_pool* pool, const int64_t* seqs, int64_t B, const int64_t* n_new,
                   int64_t max_blocks, int64_t pad_page, int64_t* block_table, int64_t* seq_lens,
                   int64_t* query_start_loc);

/* Prefix index over token ids in page-sized blocks, within a namespace (a
 * digest of everything that changes the K/V of given token ids: weights,
 * tokenizer, KV dtype, ...).
 * pkv_prefix_insert: indexes the whole pages of `seq` under its tokens
 *   tokens[0 .. n_tokens) (n_tokens <= the sequence's length); blocks already
 *   indexed keep their page; each page the index adopts gains a reference.
 * pkv_prefix_match: the longest indexed run of leading whole blocks of
 *   tokens[0 .. n_tokens), but at most (n_tokens - 1) / page_size blocks, so at
 *   least one token is left to run; creates a sequence holding those pages
 *   (references grow) and writes its handle and the matched token count.
 * pkv_prefix_evict: drops index entries whose page nothing else holds,
 *   leaves first and least recently inserted or matched first, until `pages`
 *   pages are freed or no entry qualifies; writes how many were freed.
 * pkv_prefix_pages: pages the index holds. */
int pkv_prefix_insert(pkv_page_pool* pool, uint64_t namespace_digest, int64_t seq, const int32_t* tokens,
                      int64_t n_tokens);
int pkv_prefix_match(pkv_page_pool* pool, uint64_t namespace_digest, const int32_t* tokens, int64_t n_tokens,
                     int64_t* seq_out, int64_t* matched_out);
int pkv_prefix_evict(pkv_page_pool* pool, int64_t pages, int64_t* freed_out);
int64_t pkv_prefix_pages(const pkv_page_pool* pool);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_HOST_H */
