/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged KV write and paged attention on
 * one AMD Instinct MI355X (gfx950).
 *
 * The step these calls implement follows the I/O contract of the page "Add
 * paged / block-table KV cache export (--features paged-cache)"
 * (onnxruntime/mobius #395, table "ONNX I/O contract" and "How it works"):
 * new K/V rows are scattered into per-layer page pools through slot_mapping,
 * then causal attention runs over each sequence's pages, found through its
 * block_table row and cut to nonpad_kv_seqlen (here: seq_lens).  That page
 * fixes batch 1 and lists multi-sequence batches as future work; the batch
 * form here takes the row-padded 2-D block table, seq_lens and
 * query_start_loc of the vLLM-shaped metadata that the page "[Draft] kv paged
 * kernels" (ROCm/maxtext #93, gpu_paged commit) accepts.
 *
 * Conventions shared by every call:
 *  - Tensors are described by pkv_tensor: a device pointer to a dense,
 *    row-major (C-contiguous) buffer, its element type and its shape.  The
 *    library reads shapes only to validate them; it never copies a tensor.
 *  - Index tensors (slot_mapping, block_table, seq_lens, query_start_loc) are
 *    int64, as in the mobius I/O contract.
 *  - Ownership: the caller owns every buffer, including the workspace.  The
 *    library allocates no device memory and keeps no state beyond cached
 *    device properties.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).
 *  - Ordering: each call enqueues its kernels on `stream` and returns without
 *    waiting.  A write followed by an attention call on the same stream
 *    attends over exactly the rows the write stored (maxtext #93, gpu_paged
 *    commit: prefill and decode read the pages the append wrote).
 *  - Errors: argument problems the host can see are reported synchronously by
 *    a negative status before anything is enqueued.  Bad index *values* in
 *    device memory (slot or page ids out of range, duplicate slots, lengths
 *    that exceed the block table) are not checked by the fast path; call
 *    paged_validate_metadata to find them.
 *  - Supported geometry: page_size 16; head_dim 64 or 128; Hq a multiple of
 *    Hkv with Hq / Hkv <= 16; at most 4096 sequences per decode call, with
 *    B * ceil(max_blocks * 16 / 32) < 2^31; for
 *    calls with several query rows per sequence, block_table rows of at most
 *    2^31 - 1 positions and at most 65535 query tiles of 256 / (Hq / Hkv)
 *    rows (ceil(T / tile) <= 65535), and at most 2^22 (query tile, KV head)
 *    work items counting the key chunks of a split (in practice a bound on
 *    Hkv x query tiles).  Anything else is PKV_ERR_UNSUPPORTED; there is no
 *    fallback path.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3FN = 2, /* OCP 8-bit E4M3FN codes (bias 7, max 448, 0x7F/0xFF NaN) */
  PKV_I64 = 3
} pkv_dtype;

/* status codes */
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* rank or size mismatch between arguments */
  PKV_ERR_DTYPE = -3,       /* element type not allowed for this argument */
  PKV_ERR_UNSUPPORTED = -4, /* geometry outside the supported set */
  PKV_ERR_SCALE = -5,       /* non-finite scale, or fp8 pool without k/v scales */
  PKV_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = -7,         /* the HIP runtime reported an error */
  PKV_ERR_INDEX = -8,       /* (validator only) an index value is out of range */
  PKV_ERR_SCRATCH = -9      /* (paged_attention_noalloc only) the call needs more than its
                               fixed scratch of PKV_NOALLOC_SCRATCH_BYTES */
};

/* A dense row-major tensor in device memory. */
typedef struct {
  void* data;       /* device pointer (may be NULL only when the tensor has 0 elements) */
  int32_t dtype;    /* pkv_dtype */
  int32_t ndim;     /* 1..4 */
  int64_t shape[4]; /* shape[0..ndim-1]; row-major, no padding */
} pkv_tensor;

/* Options of paged_attention. */
typedef struct {
  const float* k_scale;   /* [Hkv] fp32 device pointer: per-KV-head dequantisation scale of
                             the key pool; required iff the pool dtype is PKV_FP8_E4M3FN,
                             otherwise must be NULL */
  const float* v_scale;   /* [Hkv] fp32 device pointer, same rule for the value pool */
  void* workspace;        /* device scratch owned by the caller; may be NULL when
                             paged_attention_workspace_size returns 0 */
  size_t workspace_bytes; /* size of `workspace` */
  int32_t max_query_len;  /* host-side upper bound of query_start_loc[b+1]-query_start_loc[b]
                             over b (1 for pure decode); sizes the grid without a
                             device->host copy.  A value below the true maximum is
                             undefined behaviour; 0 means "T" (always safe). */
  int32_t split_tokens;   /* decode only: approximate KV positions per split-K partition (a
                             multiple of the page size, at most 4096).  The decode work, the
                             list of (sequence, 32-position unit) pairs of all sequences, is
                             cut into equal contiguous ranges (stream-K; a range may cross
                             sequence boundaries, and each sequence's pieces are merged by
                             log-sum-exp).  split_tokens sets how many ranges: about
                             B * max_blocks * page_size / 2 / split_tokens (half the table's
                             capacity, the host's estimate of the positions without reading
                             seq_lens), rounded to a multiple of the CU count and capped at
                             2048 ranges.  0 = one range per CU (per parallel wave group
                             when Hkv < 8).  The result does not depend on it beyond
                             floating-point rounding. */
  void* timing_events[2]; /* optional pair of hipEvent_t (created by the caller), recorded on
                             `stream` immediately before and after the call's main attention
                             kernel: the split-K decode kernel, the prefill kernel or the fp32
                             kernel, without the plan and merge launches around it.  NULL =
                             none.  For measuring that kernel alone. */
  int32_t shared_prefix_pages; /* decode only (max_query_len 1): the caller states that the
                             first shared_prefix_pages entries of every block_table row are
                             the same pages and that every sequence with a query row holds
                             more than shared_prefix_pages * page_size positions.  The
                             prefix's attention then runs once for all sequences as MFMA
                             tiles (all query rows of a group of sequences against the
                             prefix keys) and is merged with the split-K decode of each
                             sequence's own positions; the result is the same attention.
                             The prefix tiles and the split-K decode of the private
                             positions run as one launch, on disjoint sets of CUs.
                             Must be even (32-position units) and <= max_blocks; 0 = off.
                             A statement that does not hold gives unspecified output. */
} pkv_attn_opts;

/*
 * paged_kv_write -- scatter new K/V rows into the page pools, in place.
 *
 * For every t with s = slot_mapping[t] >= 0, copies the Hkv*D elements of
 * k[t] to key_pool[s / page_size][s % page_size] and of v[t] to
 * value_pool[s / page_size][s % page_size], byte for byte (the pool keeps its
 * element type; no conversion, NaN payloads survive).  Negative slots are
 * skipped.  Everything else in the pools is left untouched.
 * (mobius #395, PR summary and "ONNX I/O contract": slot = page_id *
 * page_size + offset; the pools are written by ScatterND.)
 *
 *   k, v          [T_new, Hkv, D]                       pool dtype
 *   slot_mapping  [T_new]                               PKV_I64
 *   key_pool,     [num_pages, page_size, Hkv, D]        F32, BF16 or FP8_E4M3FN
 *   value_pool    (same shape and dtype as key_pool)
 *
 * Duplicate non-negative slots within one call are a caller error (the
 * surviving row is unspecified).  Returns PKV_OK or a negative status.
 */
int paged_kv_write(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                   pkv_tensor* key_pool, pkv_tensor* value_pool, void* stream);

/*
 * paged_kv_write_fp8 -- the write for fp8 pools, quantising on the way.
 *
 * For every t with s = slot_mapping[t] >= 0 and every KV head h, element x
 * of k[t][h] is stored in key_pool[s / page_size][s % page_size][h] as the
 * OCP E4M3FN code of y = x / k_scale[h] (one IEEE binary32 division), and
 * likewise for v with v_scale: round to nearest even, |y| beyond 448
 * (infinities included) saturated to +-448, a NaN x stored as the NaN code
 * with x's sign.  k_scale and v_scale are the per-head factors paged_attention
 * multiplies codes by, so a row written here reads back as code * scale.
 * Negative slots are skipped; everything else in the pools is untouched.
 * (The pages name an fp8 KV cache as a feature, mobius #395 "Features";
 * they do not say where quantisation happens.  The plain write above stores
 * codes the caller already holds; this form produces them from bf16 rows.)
 *
 *   k, v              [T_new, Hkv, D]                  PKV_BF16, D a multiple of 8
 *   slot_mapping      [T_new]                          PKV_I64
 *   key_pool,         [num_pages, page_size, Hkv, D]   PKV_FP8_E4M3FN
 *   value_pool        (same shape and dtype as key_pool)
 *   k_scale, v_scale  device pointers to [Hkv] fp32, positive and finite (not
 *                     checked: the host cannot read them without a sync)
 *
 * Duplicate non-negative slots are a caller error, as for paged_kv_write.
 * Returns PKV_OK, PKV_ERR_SCALE for a NULL scale pointer, or another
 * negative status for a bad argument; nothing is enqueued on error.
 */
int paged_kv_write_fp8(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                       pkv_tensor* key_pool, pkv_tensor* value_pool, const float* k_scale,
                       const float* v_scale, void* stream);

/*
 * paged_attention -- causal GQA attention over paged KV.
 *
 * Sequence b owns query rows query_start_loc[b] .. query_start_loc[b+1]-1
 * (n_b rows) and seq_lens[b] = L_b key positions (old context plus its n_b
 * new tokens, i.e. nonpad_kv_seqlen after the write).  Key position p of b is
 * row p % page_size of page block_table[b][p / page_size]; entries past
 * ceil(L_b / page_size) are never read.  Query row i of b sits at position
 * L_b - n_b + i and attends to positions 0 .. L_b - n_b + i.  Query head hq
 * reads KV head hq / (Hq / Hkv).  For every row and head:
 *     out = softmax_p(scale * <q, k_p>) . v_p
 * with k and v dequantised as code * k_scale[h] / code * v_scale[h] for fp8
 * pools.  `scale` is applied exactly as given; there is no implicit
 * 1/sqrt(D) (maxtext #93: the caller passes the scale, 1.0 for a query that
 * is already scaled).  Rows, tail slots and pages the sequence does not reach
 * may hold any bytes, NaN included, without affecting the result.
 * (mobius #395, "How it works" step 3: opset-24 Attention with is_causal=1
 * and nonpad_kv_seqlen; the batch form is described in the file header.)
 *
 *   q, out           [T, Hq, D]             F32 or BF16 (same dtype)
 *   key_pool,        [num_pages, page_size, Hkv, D]
 *   value_pool         F32 (requires F32 q), BF16 or FP8_E4M3FN (require BF16 q)
 *   block_table      [B, max_blocks]        PKV_I64
 *   seq_lens         [B]                    PKV_I64
 *   query_start_loc  [B+1]                  PKV_I64, non-decreasing, [0] = 0, [B] = T
 *   scale            finite float
 *   opts             see pkv_attn_opts; NULL is allowed when no fp8 scales and no
 *                    workspace are needed
 *
 * Accumulation is fp32; bf16 outputs are rounded to nearest even.  Results
 * are deterministic (no atomics): repeated calls give identical bits.
 * Returns PKV_OK or a negative status.
 */
int paged_attention(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                    const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                    const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                    const pkv_attn_opts* opts, void* stream);

/*
 * paged_kv_write_attention -- paged_kv_write followed by paged_attention, as
 * one call: the whole step of the pages' graph (mobius #395, "How it works":
 * the ScatterND of the new rows, then Attention over the pages they landed
 * in).  Arguments are those of the two calls (k, v, slot_mapping and the pools
 * as for paged_kv_write; q .. opts as for paged_attention, with the same
 * workspace size), and so are the results.
 *
 * A decode step (opts->max_query_len 1) whose T_new equals T runs as one
 * kernel pass that writes the new rows and attends (when the rows fit the
 * pass's registers: up to 16 KiB of K and V rows per workgroup, e.g. 2048
 * sequences of 8 KV heads x 128 bf16 dims on 256 CUs).  Such a call states that
 * the new rows are the query rows' own keys: row t of k and v is the key of
 * query row t, slot_mapping[t] is the slot of that row's position
 * (block_table[b][p / page_size] * page_size + p % page_size with p =
 * seq_lens[b] - 1), and no sequence reads a written slot at another position
 * (the pages' step builds slot_mapping exactly so: the new tokens are the last
 * ones of their sequences).  The kernel then takes each sequence's last key
 * from k and v directly and writes the pools alongside, so no read waits for
 * the write.  A statement that does not hold gives unspecified attention
 * output (the pools are still written as paged_kv_write writes them);
 * paged_validate_metadata with PKV_CHECK_NEW_ROWS_ARE_QUERY_ROWS checks it.
 * Any other call (prefill, fp32 pools, T_new != T) enqueues the write and then
 * the attention, exactly as the two calls do.
 */
int paged_kv_write_attention(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                             pkv_tensor* key_pool, pkv_tensor* value_pool, const pkv_tensor* q,
                             const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                             const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                             const pkv_attn_opts* opts, void* stream);

/*
 * paged_attention_noalloc -- paged_attention for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, computation and results as
 * paged_attention (the same kernels and launch shapes: bit-identical output),
 * except that opts->workspace must be NULL and opts->workspace_bytes 0: the
 * workspace is a fixed region of PKV_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory of its own, one per GPU, from the first call on that
 * GPU until the process ends.  The call allocates and frees nothing.
 *
 * The region is sized by this device's own decode grid (smaller than the
 * device-independent size paged_attention_workspace_size reports); a call
 * that needs more than PKV_NOALLOC_SCRATCH_BYTES returns PKV_ERR_SCRATCH
 * before anything is enqueued (128 MiB holds every workload of the design
 * notes, the largest being the key-split prefill of 8 sequences x 512 tokens
 * on 8704-position contexts with 1, 2 or 4 KV heads, about 40 MB).  Nothing in
 * the region needs to start at zero: every kernel writes what a later kernel
 * of the same call reads.  All calls on one GPU share its region, so calls
 * that may overlap on one GPU (different streams without ordering between
 * them) race and give unspecified output; order them on one stream.
 * Returns PKV_OK, PKV_ERR_SCRATCH, PKV_ERR_WORKSPACE for a non-NULL
 * opts->workspace, or any status paged_attention returns.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int paged_attention_noalloc(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                            const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                            const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                            const pkv_attn_opts* opts, void* stream);

/*
 * paged_attention_workspace_size -- bytes of workspace paged_attention needs
 * for these shapes and options (0 if none).  Depends only on the shapes and
 * dtypes of q, key_pool and block_table, on opts->max_query_len (decode or
 * prefill; for prefill the work list grows with the query rows, and with few
 * KV heads the key split's partials with max_blocks) and on
 * opts->shared_prefix_pages; opts->split_tokens does not change it.  The
 * workspace holds no state between calls.  Returns (size_t)-1 if the
 * arguments are invalid (the same ones paged_attention would reject).
 */
size_t paged_attention_workspace_size(const pkv_tensor* q, const pkv_tensor* key_pool,
                                      const pkv_tensor* block_table, const pkv_attn_opts* opts);

/*
 * paged_block_table_from_csr -- block_table and seq_lens from the packed
 * (CSR) page-list form of the same metadata.
 *
 * Sequence b's pages are kv_indices[kv_indptr[b] .. kv_indptr[b+1]) in order
 * (n_b of them) and its last page holds kv_last_page_len[b] rows, so
 *     block_table[b][j] = kv_indices[kv_indptr[b] + j]  for j < n_b, else pad_page
 *     seq_lens[b]       = (n_b - 1) * page_size + kv_last_page_len[b]  (0 if n_b = 0)
 * (page "Refactor KV Cache Manager with a new torch exportable KVCache
 * backend", NVIDIA/recsys-examples #400, the KVCacheMetadata fields kv_indices,
 * kv_indptr and kv_last_page_len; page "[Draft] kv paged kernels",
 * ROCm/maxtext #93, converts a row-padded table into this packed page list
 * for its kernels, the reverse of this call).  The result feeds
 * paged_attention directly.
 *
 *   kv_indptr         [B+1]               PKV_I64, non-decreasing from 0
 *   kv_indices        [nnz]               PKV_I64, nnz >= kv_indptr[B]
 *   kv_last_page_len  [B]                 PKV_I64, in 1..page_size for n_b > 0
 *   block_table       [B, max_blocks]     PKV_I64, written
 *   seq_lens          [B]                 PKV_I64, written
 *
 * Index values live in device memory and are not checked here (a sequence
 * with more than max_blocks pages, or a last-page length outside
 * 1..page_size, is a caller error); for memory safety its row is cut at
 * max_blocks pages and its length clamped to its row's pages, so what
 * paged_attention reads stays inside block_table, and page ids are read only
 * inside kv_indices.  Returns PKV_OK or a
 * negative status for bad arguments; one kernel is enqueued on `stream`.
 */
int paged_block_table_from_csr(const pkv_tensor* kv_indptr, const pkv_tensor* kv_indices,
                               const pkv_tensor* kv_last_page_len, int64_t page_size, int64_t pad_page,
                               pkv_tensor* block_table, pkv_tensor* seq_lens, void* stream);

/*
 * paged_validate_metadata -- debug check of index values in device memory.
 * Synchronises `stream`, copies the index tensors to the host and checks:
 * every slot in [-1 .. num_pages*page_size), no duplicate non-negative slot,
 * query_start_loc non-decreasing from 0 to T, n_b <= L_b, L_b <= max_blocks *
 * page_size, and every block_table entry a sequence reaches in [0, num_pages).
 * With shared_prefix_pages = N > 0 it also checks the statement a decode call
 * makes through pkv_attn_opts.shared_prefix_pages: N <= max_blocks, every
 * sequence with a query row holds more than N * page_size positions, and the
 * first N entries of all those sequences' rows are the same pages (0 = no
 * statement).  `checks` selects further statements to check (0 = none):
 * PKV_CHECK_NEW_ROWS_ARE_QUERY_ROWS, the statement of a fused decode step
 * (paged_kv_write_attention): one slot per query row, each the slot of its
 * row's position, and no sequence reading a written slot at an older
 * position.  slot_mapping may be NULL (attention-only check).  Returns
 * PKV_OK, PKV_ERR_INDEX on the first bad value (and, if `message` is
 * non-NULL, writes a NUL-terminated description of at most `message_len`
 * bytes), or another negative status for bad arguments.
 */
#define PKV_CHECK_NEW_ROWS_ARE_QUERY_ROWS 1u
int paged_validate_metadata(const pkv_tensor* slot_mapping, const pkv_tensor* block_table,
                            const pkv_tensor* seq_lens, const pkv_tensor* query_start_loc,
                            int64_t num_pages, int64_t page_size, int64_t num_query_rows,
                            int64_t shared_prefix_pages, uint32_t checks, void* stream, char* message,
                            size_t message_len);

/*
 * pkv_check_metadata_host -- the checks of paged_validate_metadata on index
 * arrays already in host memory (all int64, row-major: slots [n_slots] or NULL,
 * block_table [B, max_blocks], seq_lens [B], query_start_loc [B+1]).  Same
 * arguments, return values and message convention.
 */
int pkv_check_metadata_host(const int64_t* slots, int64_t n_slots, const int64_t* block_table,
                            int64_t B, int64_t max_blocks, const int64_t* seq_lens,
                            const int64_t* query_start_loc, int64_t num_pages, int64_t page_size,
                            int64_t num_query_rows, int64_t shared_prefix_pages, uint32_t checks,
                            char* message, size_t message_len);

/* Human-readable name of a status code (static string). */
const char* pkv_status_string(int status);

/* Version of this ABI; bumped on any incompatible change. */
int pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
