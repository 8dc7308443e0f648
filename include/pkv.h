/*
 * pkv.h -- C ABI of libpkv, a persistent-KV decode step for AMD Instinct
 * MI355X (gfx950).
 *
 * The library implements one per-token decode step over a KV cache that the
 * caller owns and keeps alive between steps:
 *
 *   1. an in-place cache update whose result is the input storage
 *      (contiguous or paged; optionally quantising new rows to INT4),
 *   2. attention of the new queries over the valid cache prefix
 *      (contiguous, paged bf16, paged INT4, pages of mixed formats; a
 *      causal chunk variant),
 *   3. greedy or seeded temperature sampling of final logits, and the
 *      bookkeeping of a generation loop (EOS, padding, stop).
 *
 * Sources: the onnx-light documentation pages "Mutable execution cache"
 * (in-place update contract, paged cache, runtime contract, memory planning),
 * "Persistent input/output feedback" (attention, paged KV, generation and
 * sampling semantics) and "Custom, quantized, and persistent values" (affine
 * INT4 encoding).  Each entry point below names the section it follows.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Ownership.  The caller allocates every buffer, host or device, and keeps
 *   it alive until the work enqueued on `stream` has finished.  The library
 *   never allocates device memory and keeps no pointer after returning,
 *   except inside pool and binding handles (host metadata only).
 * - Tensors.  `pkv_tensor` describes a dense row-major array: `data` plus
 *   dtype and shape, no strides.  Non-contiguous data is the caller's
 *   problem: it is rejected by the binding layer, never copied.  Unless a
 *   parameter says "host", `data` is device memory.
 * - Streams.  `stream` is a `hipStream_t` (NULL = the null stream).  All
 *   device work is enqueued on it; no call synchronises the device.
 * - Errors.  Every argument is validated on the host before any HIP call.
 *   On any error the function returns a non-zero `pkv_status`, enqueues no
 *   work and leaves every buffer untouched; `pkv_last_error()` gives the
 *   reason (thread-local).  `PKV_E_HIP` reports a failed launch.
 * - Concurrency.  Calls that write the same cache storage must not overlap
 *   on different streams; calls from several host threads are safe
 *   otherwise (the binding registry is locked; a pool handle is not and
 *   must be used by one thread at a time).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 10
#define PKV_MAX_DIMS 6

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_E_ARG = 1,       /* null pointer, bad size, bad enum, bad temperature   */
    PKV_E_CAPACITY = 2,  /* position < 0 or position + update_length > capacity */
    PKV_E_READONLY = 3,  /* cache storage is not inside a live writable binding */
    PKV_E_ALIAS = 4,     /* input storage overlaps the storage being written    */
    PKV_E_BUSY = 5,      /* writable binding overlaps an existing binding       */
    PKV_E_PAGE = 6,      /* page not reserved / page id or sequence out of range */
    PKV_E_NOMEM = 7,     /* page pool exhausted, or workspace too small         */
    PKV_E_DTYPE = 8,     /* unsupported or mismatched element type             */
    PKV_E_LAYOUT = 9,    /* rank or shape mismatch, unsupported head size       */
    PKV_E_HIP = 10       /* a HIP runtime call failed                           */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_BF16 = 1,
    PKV_F16 = 2,
    PKV_U8 = 3,
    PKV_I32 = 4,
    PKV_I64 = 5,
    PKV_F64 = 6   /* sampled logits only */
} pkv_dtype;

typedef struct pkv_tensor {
    void* data;                      /* first element                        */
    int32_t dtype;                   /* pkv_dtype                            */
    int32_t ndim;                    /* 1..PKV_MAX_DIMS                      */
    int64_t shape[PKV_MAX_DIMS];     /* dense row-major                      */
} pkv_tensor;

typedef struct pkv_binding pkv_binding;
typedef struct pkv_pool pkv_pool;

/* ------------------------------------------------------------------------ */
/* Library info                                                              */
/* ------------------------------------------------------------------------ */

/* Reason for the last non-OK status returned on this thread ("" if none).
 * The string stays valid until the next library call on this thread. */
const char* pkv_last_error(void);

/* PKV_ABI_VERSION of the built library. */
int32_t pkv_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Writable bindings                                                         */
/* "Mutable execution cache", sections "Required alias" and "Runtime
 * contract": the caller opts into mutation when binding the cache; one
 * writable binding cannot be used concurrently by several users; immutable or
 * shared storage is never accepted as a mutable cache.                      */
/* ------------------------------------------------------------------------ */

/* Register [base, base + bytes) as writable cache storage owned by the caller.
 * Fails with PKV_E_BUSY if the range overlaps a live binding, PKV_E_ARG if
 * base is NULL or bytes is 0.  The handle is freed by pkv_unbind. */
pkv_status pkv_bind_writable(void* base, size_t bytes, pkv_binding** out);

/* Release a binding (NULL is PKV_E_ARG).  Storage is not touched. */
pkv_status pkv_unbind(pkv_binding* binding);

/* ------------------------------------------------------------------------ */
/* Contiguous in-place cache update                                          */
/* "Mutable execution cache", sections "Value model", "ShapesContext",
 * "Required alias" and "Model example": updated_cache = CacheUpdate(cache,
 * values, position) writes only the range starting at position, the output
 * is the input storage, position + update_length <= capacity is checked and
 * overflow is an error (no growth, no copy fallback).                       */
/* ------------------------------------------------------------------------ */

/* cache  : [B, H, capacity, D], any dtype, inside a writable binding.
 * values : [B, H, update_length, D], same dtype; must not overlap `cache`.
 * position: host int32[B], the first row written for each batch row.
 * Writes cache[b, h, position[b] + t, :] = values[b, h, t, :] for t <
 * update_length and nothing else.  On success *out_cache = cache->data
 * (pointer identity).  Errors: PKV_E_CAPACITY when any position[b] < 0 or
 * position[b] + update_length > capacity; PKV_E_READONLY when the cache is
 * not inside a live writable binding; PKV_E_ALIAS when values overlap it. */
pkv_status pkv_cache_update(const pkv_tensor* cache, const pkv_tensor* values,
                            const int32_t* position, int32_t update_length,
                            void** out_cache, void* stream);

/* The same update for a K and a V cache in one launch (a decode step appends
 * both): the result equals pkv_cache_update of k_values into k_cache
 * followed by v_values into v_cache.  Every check of both runs before
 * anything is launched, so either both caches are written or neither.
 * k_cache and v_cache: same shape and dtype, disjoint, each inside a writable
 * binding; k_values and v_values: [B, H, update_length, D] of the caches,
 * neither overlapping either cache.  Errors as pkv_cache_update, plus
 * PKV_E_LAYOUT / PKV_E_DTYPE when K and V differ in shape or dtype and
 * PKV_E_ALIAS when the caches overlap. */
pkv_status pkv_cache_update_kv(const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                               const pkv_tensor* k_values, const pkv_tensor* v_values,
                               const int32_t* position, int32_t update_length, void* stream);

/* ------------------------------------------------------------------------ */
/* Fixed page pool (host metadata)                                           */
/* "Mutable execution cache", sections "Heterogeneous paged cache",
 * "Runtime contract" and "Existing implementations / ONNX Runtime GenAI":
 * a fixed pool of physical blocks and a per-request block table; only a
 * missing page may be allocated, existing pages are updated in place, the
 * pool never grows.                                                         */
/* ------------------------------------------------------------------------ */

/* Create the host bookkeeping of a pool of `num_blocks` physical pages of
 * `block_size` tokens, for sequences 0..max_seqs-1 of up to
 * max_blocks_per_seq pages each.  initial_free_order (host int32[num_blocks],
 * a permutation of 0..num_blocks-1, or NULL for ascending order) is the order
 * in which pages are handed out.  The physical K/V storage and the device
 * page table int32[max_seqs, max_blocks_per_seq] are caller-owned. */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                           int32_t max_blocks_per_seq, const int32_t* initial_free_order,
                           pkv_pool** out);

pkv_status pkv_pool_destroy(pkv_pool* pool);

/* For each i < n, make logical positions [0, new_len[i]) of sequence seqs[i]
 * (host arrays) backed by pages, taking only pages the sequence does not
 * hold yet.  All or nothing: PKV_E_NOMEM if the free pool is too small,
 * PKV_E_PAGE if a sequence id is out of range, listed twice, or needs more
 * than max_blocks_per_seq pages; nothing changes then.  When
 * page_table_dev is not NULL the new entries are written to that device
 * table on `stream` (ids travel as kernel arguments: nothing host-side must
 * outlive the call).  Shrinking is a no-op. */
pkv_status pkv_pool_reserve(pkv_pool* pool, int32_t n, const int32_t* seqs,
                            const int32_t* new_len, int32_t* page_table_dev, void* stream);

/* Return every page of `seq` to the back of the free list.  When
 * page_table_dev is not NULL its row is reset to -1 on `stream`. */
pkv_status pkv_pool_release(pkv_pool* pool, int32_t seq, int32_t* page_table_dev, void* stream);

/* Host mirror queries.  held_pages / reserved_len may be NULL. */
pkv_status pkv_pool_query(const pkv_pool* pool, int32_t seq, int32_t* held_pages,
                          int32_t* reserved_len);
pkv_status pkv_pool_free_count(const pkv_pool* pool, int32_t* free_pages);
/* Copy the host page table int32[max_seqs, max_blocks_per_seq] (-1 = none). */
pkv_status pkv_pool_table(const pkv_pool* pool, int32_t* out_host);

/* Page-id trust contract.  The device page table is caller-owned memory and
 * the library never copies it back to the host.  The calls that take host
 * positions or host lengths (pkv_paged_cache_update and its INT4 and mixed
 * forms, pkv_paged_gather, the paged decode calls, pkv_chunk_attention)
 * therefore check a row against the pool's host mirror by counting: with
 * `pool` given, each row must hold enough reserved pages for
 * the positions it writes or reads (else PKV_E_PAGE, nothing launched).  The
 * ids themselves are read from the device table inside the kernels and are
 * trusted there: a table that disagrees with what pkv_pool_reserve wrote
 * (edited by the caller, or a table of another pool) makes those kernels
 * read or write the pages it names, and with `pool == NULL` the counts are
 * not checked either.  Keep the table as pkv_pool_reserve / _release leave
 * it.  The device-driven calls (the *_dev entry points below) do range-check
 * every id they read against [0, num_blocks): an id outside it is never
 * dereferenced for a write, reads page 0 instead, and sets *status to
 * PKV_E_PAGE. */

/* ------------------------------------------------------------------------ */
/* Paged in-place cache update                                               */
/* "Mutable execution cache", sections "Heterogeneous paged cache" and
 * "Runtime contract": updated_cache = PagedCacheUpdate(cache, page_id,
 * values, position) aliases the cache, updates existing pages in place and
 * allocates nothing (pages come from pkv_pool_reserve).                     */
/* ------------------------------------------------------------------------ */

/* pool_kv   : [num_blocks, H, block_size, D] physical pages (one pool per K
 *             and per V), any dtype, inside a writable binding.
 * page_table_dev: int32[max_seqs, max_blocks_per_seq] kept by
 *             pkv_pool_reserve; row b of the batch is sequence b.
 * values    : [B, H, update_length, D], same dtype, no overlap with pool_kv.
 * position  : host int32[B]; logical position p of row b lives in slot
 *             p % block_size of page page_table[b][p / block_size].
 * Errors: PKV_E_PAGE when a written position lies on a page the pool has not
 * reserved for that row (no implicit allocation); PKV_E_CAPACITY when
 * position[b] < 0 or position[b] + update_length exceeds
 * max_blocks_per_seq * block_size.  On success *out_pool = pool_kv->data. */
pkv_status pkv_paged_cache_update(const pkv_pool* pool, const pkv_tensor* pool_kv,
                                  const int32_t* page_table_dev, const pkv_tensor* values,
                                  const int32_t* position, int32_t update_length,
                                  void** out_pool, void* stream);

/* The same update for the K and the V pool of one page table in one launch
 * (a decode step appends both): the result equals pkv_paged_cache_update of
 * k_values into k_pool followed by v_values into v_pool.  Every check of both
 * runs before anything is launched, so either both pools are written or
 * neither.  k_pool and v_pool: same shape and dtype, disjoint, each inside a
 * writable binding; k_values and v_values: same shape [B, H, update_length,
 * D], neither overlapping either pool.  Errors as pkv_paged_cache_update,
 * plus PKV_E_LAYOUT / PKV_E_DTYPE when K and V differ in shape or dtype and
 * PKV_E_ALIAS when the pools overlap.  The storage of each pool is its input
 * (no separate output pointers). */
pkv_status pkv_paged_cache_update_kv(const pkv_pool* pool, const pkv_tensor* k_pool,
                                     const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                     const pkv_tensor* k_values, const pkv_tensor* v_values,
                                     const int32_t* position, int32_t update_length, void* stream);

/* ------------------------------------------------------------------------ */
/* Device-driven step (positions and lengths in device memory)               */
/* "Mutable execution cache", section "Existing implementations": capturing a
 * decode step in a graph needs its buffers, positions included, to be shared
 * device state rather than values fixed at launch.  The *_dev entry points
 * take positions, valid lengths and the sampling step from device memory, so
 * a step enqueued once (for example captured in a HIP graph) can be replayed
 * as the sequences grow; pkv_advance moves that state on.  Host arguments
 * (shapes, dtypes, bindings, bounds) are checked on the host as everywhere
 * else.  Values read from device memory are checked by the kernels: a failed
 * check writes a non-zero pkv_status into the caller's device word
 * *status_dev and the check's rows are left alone (see each call).  The
 * library never clears *status_dev: zero it before the first step; a
 * non-zero value stays until the caller clears it.                           */
/* ------------------------------------------------------------------------ */

/* K and V appended in one launch at device positions ("Mutable execution
 * cache", "Required alias": the output is the input storage).
 * k_cache, v_cache: [B, H, capacity, D], one dtype, each inside a writable
 * binding; k_values, v_values: [B, H, update_length, D]; rows of D elements
 * a multiple of 16 bytes; every tensor 16-byte aligned.
 * position_dev: device int32[B].  update_length in [0, 64].
 * Device check: every row has 0 <= position <= capacity - update_length;
 * otherwise nothing is written and *status_dev = PKV_E_CAPACITY. */
pkv_status pkv_cache_update_kv_dev(const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                                   const pkv_tensor* k_values, const pkv_tensor* v_values,
                                   const int32_t* position_dev, int32_t update_length,
                                   int32_t* status_dev, void* stream);

/* Paged form ("Heterogeneous paged cache", "Runtime contract": existing
 * pages are updated in place, nothing is allocated): k_pool, v_pool
 * [num_blocks, H, block_size, D] matching `pool`; page_table_dev as for
 * pkv_paged_cache_update.  Device checks: every row has 0 <= position and
 * position + update_length <= max_blocks_per_seq * block_size (else
 * PKV_E_CAPACITY), and every page the call writes has an id in
 * [0, num_blocks) (a -1 entry is a page that was never reserved; else
 * PKV_E_PAGE); on a failure nothing is written. */
pkv_status pkv_paged_cache_update_kv_dev(const pkv_pool* pool, const pkv_tensor* k_pool,
                                         const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                         const pkv_tensor* k_values, const pkv_tensor* v_values,
                                         const int32_t* position_dev, int32_t update_length,
                                         int32_t* status_dev, void* stream);

/* values_dev[i] += delta for i < n (device int32), then *step_dev += 1 when
 * step_dev is not NULL (the counter pkv_sample_dev reads). */
pkv_status pkv_advance(int32_t* values_dev, int32_t n, int32_t delta, int64_t* step_dev, void* stream);

/* INT4 variant: quantise the new rows on append.
 * "Persistent input/output feedback", "Optional heterogeneous paged KV":
 * affine append uses scalar parameters, rounds ties to even and saturates;
 * "Custom, quantized, and persistent values", "Struct types and
 * byte-encodable layouts": two 4-bit codes per byte, least-significant first.
 * codes_pool : u8  [num_blocks, H, block_size, D/2]
 * params_pool: f16 [num_blocks, H, block_size, D/32, 2] (scale, zero_point)
 * values     : f32 or bf16 [B, H, update_length, D], D a multiple of 32.
 * scale_f16, zero_point_f16: IEEE binary16 bit patterns; scale > 0 finite,
 * zero_point an integer 0..15.  Code = clamp(rint(x / scale) + zp, 0, 15)
 * with a correctly rounded float32 divide; every block's param slot of a
 * written row receives (scale, zero_point).  Same checks as above. */
pkv_status pkv_paged_cache_update_int4(const pkv_pool* pool, const pkv_tensor* codes_pool,
                                       const pkv_tensor* params_pool,
                                       const int32_t* page_table_dev, const pkv_tensor* values,
                                       uint16_t scale_f16, uint16_t zero_point_f16,
                                       const int32_t* position, int32_t update_length,
                                       void** out_codes, void** out_params, void* stream);

/* Materialise the logical [H, length, D] rows of sequence `seq` from the
 * pages (a test/debug export; bit copy).  out must not overlap pool_kv. */
pkv_status pkv_paged_gather(const pkv_tensor* pool_kv, const int32_t* page_table_dev,
                            int32_t max_blocks_per_seq, int32_t seq, int32_t length,
                            pkv_tensor* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Decode attention                                                          */
/* "Persistent input/output feedback", "Optional heterogeneous paged KV",
 * sections "Versioned operator schema" and "Kernel implementation": query
 * heads are a multiple of the K/V heads; only valid tokens are read; online
 * softmax replaces K/V concatenation and any cache-length score matrix; the
 * current K/V take part.  A single query sits at the last valid position, so
 * the causal mask keeps the whole valid prefix.                             */
/* ------------------------------------------------------------------------ */

/* Workspace (bytes) the decode entry points need for B rows, Hq query heads,
 * value head size D and contexts of up to max_len tokens with `num_splits`
 * (0 = library choice, the same rule the call uses). */
size_t pkv_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_len, int32_t num_splits);

/* q       : [B, Hq, 1, Dk] or [B, Hq, Dk], f32, bf16 or f16.
 * k_cache : [B, Hkv, capacity, Dk]; v_cache [B, Hkv, capacity, Dv] (K and V
 *           head sizes may differ: "Persistent input/output feedback",
 *           "Contiguous CPU Attention feedback"), Dk, Dv <= 256, same dtype
 *           as q, Hq % Hkv == 0.  bf16 / f16 with Dk = Dv = 128 and
 *           Hq / Hkv in {1, 2, 4, 8} takes the fast kernel.
 * valid_len: host int32[B], 1 <= valid_len[b] <= capacity (includes the
 *           token appended by this step).
 * scale   : softmax scale; <= 0 means 1/sqrt(Dk).
 * left_window: -1 = unbounded; W >= 0 = the query (at position
 *           valid_len[b] - 1) sees only keys [max(0, valid_len[b] - 1 - W),
 *           valid_len[b] - 1] ("Persistent input/output feedback", "Optional
 *           heterogeneous paged KV", "Versioned operator schema":
 *           left_window_size).  Pages and rows wholly before the window are
 *           not read.  Values below -1: PKV_E_ARG.
 * out     : q's shape with Dv last; dtype of q or f32.  Query head h reads
 *           K/V head h / (Hq / Hkv).
 * workspace: device scratch of pkv_decode_workspace_size(...) bytes, 256-byte
 *           aligned; contents need no initialisation.
 * num_splits: 0 lets the library split long contexts; otherwise each row's
 *           context is cut into that many equal token ranges (at most). */
pkv_status pkv_decode_attention(const pkv_tensor* q, const pkv_tensor* k_cache,
                                const pkv_tensor* v_cache, const int32_t* valid_len,
                                float scale, int32_t left_window, pkv_tensor* out, void* workspace,
                                size_t workspace_bytes, int32_t num_splits, void* stream);

/* One decode step on contiguous caches in one launch: the same results, cache
 * bytes and output bits as pkv_cache_update_kv(k_cache, v_cache, k_values,
 * v_values, position, update_length) followed by pkv_decode_attention(q,
 * k_cache, v_cache, valid_len = position + update_length, ...) ("Mutable
 * execution cache", "Value model" and "Model example": the updated cache is
 * the input storage; "Persistent input/output feedback", "Kernel
 * implementation": the current K/V take part in the attention).  The
 * attention workgroup whose token range holds the new rows writes them
 * before it reads them, so no separate append launch is issued.
 * Arguments: those of the two calls; the caches must agree in batch, heads
 * and capacity (head sizes may differ), be bound writable, and not overlap
 * q, out, the new values or each other.  All checks of both calls run
 * before anything is written; on an error nothing is written.  update_length
 * 0 is a plain decode at valid_len = position. */
pkv_status pkv_decode_step(const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                           const pkv_tensor* k_values, const pkv_tensor* v_values,
                           const int32_t* position, int32_t update_length, const pkv_tensor* q,
                           float scale, int32_t left_window, pkv_tensor* out, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, void* stream);

/* pkv_decode_step with the positions in device memory ("Mutable execution
 * cache", "Existing implementations": a step captured in a graph reads its
 * positions from shared state): position_dev is device int32[B]; row b
 * appends at position_dev[b] and attends over position_dev[b] +
 * update_length tokens.  The positions are not moved (pkv_advance does that
 * after the step).  The split plan is made for max_len (1 <= max_len <=
 * capacity) as in pkv_decode_attention_dev, whose workspace size it takes.
 * Device check: a row with position < 0 or position + update_length outside
 * [1, max_len] writes nothing (cache or output) and sets *status_dev =
 * PKV_E_CAPACITY; the other rows proceed.  Host checks as for
 * pkv_decode_step, plus: position_dev and status_dev must not overlap a
 * cache. */
pkv_status pkv_decode_step_dev(const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                               const pkv_tensor* k_values, const pkv_tensor* v_values,
                               const int32_t* position_dev, int32_t update_length, const pkv_tensor* q,
                               int32_t max_len, float scale, int32_t left_window, pkv_tensor* out,
                               void* workspace, size_t workspace_bytes, int32_t num_splits,
                               int32_t* status_dev, void* stream);

/* Paged f32/bf16/f16: k_pool [num_blocks, Hkv, block_size, Dk], v_pool
 * [num_blocks, Hkv, block_size, Dv];
 * page_table_dev int32[>= B, max_blocks_per_seq]; block_size must equal
 * k_pool->shape[2].  When `pool` is not NULL every row must hold
 * ceil(valid_len[b] / block_size) reserved pages (else PKV_E_PAGE). */
pkv_status pkv_paged_decode_attention(const pkv_tensor* q, const pkv_tensor* k_pool,
                                      const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                      int32_t max_blocks_per_seq, int32_t block_size,
                                      const pkv_pool* pool, const int32_t* valid_len,
                                      float scale, int32_t left_window, pkv_tensor* out,
                                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                                      void* stream);

/* Variant of pkv_paged_decode_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc): same arguments and results without the workspace.  The
 * split partials live in a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * that the library keeps on every GPU it runs on until the process ends; the
 * call allocates nothing.  A call whose partials need more than that
 * (pkv_decode_workspace_size of the same arguments) fails with PKV_E_NOMEM
 * before any work is enqueued.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race; calls in order on one stream do not.  Its contents need no
 * initialisation. */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status pkv_paged_decode_attention_noalloc(const pkv_tensor* q, const pkv_tensor* k_pool,
                                              const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              const pkv_pool* pool, const int32_t* valid_len,
                                              float scale, int32_t left_window, pkv_tensor* out,
                                              int32_t num_splits, void* stream);

/* pkv_decode_attention / pkv_paged_decode_attention with the valid lengths
 * in device memory (valid_len_dev: device int32[B]).  max_len (host) bounds
 * every length and sizes the split plan and the workspace
 * (pkv_decode_workspace_size with max_len); with every row at max_len the
 * plan and the results are those of the host-length call.  The page table
 * is read as it stands when the kernels run.  Device checks: a row whose
 * length is outside [1, max_len] writes nothing and sets *status_dev =
 * PKV_E_CAPACITY; a page id outside [0, num_blocks) among a row's valid
 * pages sets PKV_E_PAGE (the read is redirected to page 0 and the row's
 * output is unspecified).  With a pool handle only its shape is checked. */
pkv_status pkv_decode_attention_dev(const pkv_tensor* q, const pkv_tensor* k_cache,
                                    const pkv_tensor* v_cache, const int32_t* valid_len_dev,
                                    int32_t max_len, float scale, int32_t left_window, pkv_tensor* out,
                                    void* workspace, size_t workspace_bytes, int32_t num_splits,
                                    int32_t* status_dev, void* stream);
pkv_status pkv_paged_decode_attention_dev(const pkv_tensor* q, const pkv_tensor* k_pool,
                                          const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                          int32_t max_blocks_per_seq, int32_t block_size,
                                          const pkv_pool* pool, const int32_t* valid_len_dev,
                                          int32_t max_len, float scale, int32_t left_window,
                                          pkv_tensor* out, void* workspace, size_t workspace_bytes,
                                          int32_t num_splits, int32_t* status_dev, void* stream);

/* Paged INT4: K/V rows decoded in registers as (code - zero_point) * scale
 * per 32-element block ("Custom, quantized, and persistent values",
 * "Quantization examples"); never materialised.  q and out are f32
 * [B, Hq, (1,) D]; D == 128; Hq / Hkv in {1, 2, 4, 8}; block_size a power of
 * two >= 16; codes/params pools as in pkv_paged_cache_update_int4, each
 * 16-byte aligned (else PKV_E_LAYOUT). */
pkv_status pkv_paged_decode_attention_int4(const pkv_tensor* q, const pkv_tensor* k_codes,
                                           const pkv_tensor* k_params, const pkv_tensor* v_codes,
                                           const pkv_tensor* v_params,
                                           const int32_t* page_table_dev,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           const pkv_pool* pool, const int32_t* valid_len,
                                           float scale, int32_t left_window, pkv_tensor* out,
                                           void* workspace, size_t workspace_bytes,
                                           int32_t num_splits, void* stream);

/* Causal chunk attention after a chunk of C tokens was appended at position
 * p0[b] (host int32[B]) with pkv_paged_cache_update: query t of row b sits at
 * p0[b] + t and attends keys [lo, p0[b] + t] with lo = 0 for left_window = -1
 * and max(0, p0[b] + t - left_window) for left_window >= 0 ("Persistent
 * input/output feedback", "Optional heterogeneous paged KV", "Versioned
 * operator schema": causal by default, left_window_size, equal new Q/K/V
 * lengths); key tiles wholly before every query's window are not read.
 * q, out: bf16 [B, Hq, C, D] with D == 128 and Hq / Hkv in {1, 2, 4, 8};
 * k_pool, v_pool: bf16 [num_blocks, Hkv, block_size, D], block_size a power
 * of two >= 4; q, out and both pools 16-byte aligned (else PKV_E_LAYOUT);
 * page_table_dev as
 * for pkv_paged_decode_attention.  Errors: PKV_E_CAPACITY when p0[b] < 0 or
 * p0[b] + C exceeds max_blocks_per_seq * block_size; PKV_E_PAGE when `pool` is
 * given and a row holds fewer than ceil((p0[b] + C) / block_size) pages.
 * Runs on the bf16 matrix cores with fp32 accumulation; no workspace. */
pkv_status pkv_chunk_attention(const pkv_tensor* q, const pkv_tensor* k_pool,
                               const pkv_tensor* v_pool, const int32_t* page_table_dev,
                               int32_t max_blocks_per_seq, int32_t block_size,
                               const pkv_pool* pool, const int32_t* p0, float scale,
                               int32_t left_window, pkv_tensor* out, void* stream);

/* Workspace (bytes) pkv_chunk_attention_split needs for B rows, Hq query
 * heads, Hkv K/V heads and C chunk tokens with `num_splits` parts (0 = the
 * most the library picks by itself on the current device); 0 when no
 * workspace is needed or the arguments are invalid. */
size_t pkv_chunk_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t C, int32_t num_splits);

/* pkv_chunk_attention with the key range of every workgroup (256 query rows
 * of one K/V head) cut into num_splits near-equal parts, each part its own
 * workgroup, and the parts' partial results combined by the log-sum-exp
 * merge of the decode calls: the online softmax of "Kernel implementation"
 * taken over a partition of the keys.  For small batches, whose launch
 * would leave compute units idle.  Arguments and results as for
 * pkv_chunk_attention, plus:
 * num_splits: 1 = no split (the pkv_chunk_attention launch, workspace
 *           unused); 2 .. 64 = that many parts (parts with no key tile write
 *           an empty partial); 0 = library choice from the launch size and
 *           the longest key range.  Other values: PKV_E_ARG.
 * workspace: device scratch of at least pkv_chunk_workspace_size(B, Hq,
 *           Hkv, C, num_splits) bytes, 256-byte aligned, disjoint from q,
 *           out and the pools (PKV_E_NOMEM when smaller, PKV_E_ARG when
 *           misaligned, PKV_E_ALIAS when overlapping); only read when more
 *           than one part is used.  Stream-ordered: the next call on the
 *           stream may reuse it. */
pkv_status pkv_chunk_attention_split(const pkv_tensor* q, const pkv_tensor* k_pool,
                                     const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                     int32_t max_blocks_per_seq, int32_t block_size,
                                     const pkv_pool* pool, const int32_t* p0, float scale,
                                     int32_t left_window, pkv_tensor* out, void* workspace,
                                     size_t workspace_bytes, int32_t num_splits, void* stream);

/* ------------------------------------------------------------------------ */
/* Mixed-format pages                                                        */
/* "Persistent input/output feedback", "Optional heterogeneous paged KV":
 * every append picks the storage of the pages it creates, dense or affine
 * INT8, UINT8, INT4, UINT4, INT2 or UINT2, K and V independently, with one
 * scalar scale and zero point; the choice is stored with each new page, so
 * successive appends may use different formats without converting earlier
 * pages.  Section "Selected-block quantization": chosen pages are re-encoded
 * from their dense or affine payload.  "Custom, quantized, and persistent
 * values", "Struct types and byte-encodable layouts" and "Quantization
 * examples": codes packed least-significant bits first, signed codes in two's
 * complement, value (code - zero_point) * scale.
 *
 * Storage: K and V slot pools, each bf16 or f16 [num_blocks, H, block_size, D]
 * (only the bytes matter: one slot of block_size * D * 2 bytes per (page,
 * head)).  A page's rows are packed from the start of its slot, row t at byte
 * t * D * bits / 8, so a pool of BF16 pages is a plain bf16 pool.  The format
 * of every physical page lives in a descriptor table `page_desc`: u8
 * [num_blocks, 16], one pkv_page_desc per page, owned by the caller.        */
/* ------------------------------------------------------------------------ */

typedef enum pkv_page_storage {
    PKV_PAGE_BF16 = 0,   /* dense bfloat16 */
    PKV_PAGE_F16 = 1,    /* dense IEEE binary16 */
    PKV_PAGE_INT8 = 2,   /* affine codes -128..127 */
    PKV_PAGE_UINT8 = 3,  /* affine codes 0..255 */
    PKV_PAGE_INT4 = 4,   /* affine codes -8..7, two per byte */
    PKV_PAGE_UINT4 = 5,  /* affine codes 0..15, two per byte */
    PKV_PAGE_INT2 = 6,   /* affine codes -2..1, four per byte */
    PKV_PAGE_UINT2 = 7   /* affine codes 0..3, four per byte */
} pkv_page_storage;

/* Format of the K or V rows of a page, as requested by a call.  Affine
 * storages need a positive finite scale and an integer zero point in the code
 * range; dense storages ignore both. */
typedef struct pkv_page_format {
    int32_t storage;     /* pkv_page_storage */
    float scale;
    int32_t zero_point;
} pkv_page_format;

/* Device descriptor of one physical page (16 bytes, written by the library). */
typedef struct pkv_page_desc {
    float k_scale, v_scale;
    int16_t k_zero, v_zero;
    uint8_t k_storage, v_storage;
    uint8_t reserved[2];
} pkv_page_desc;

/* Append update_length new tokens of every row at position[b] (host int32[B]).
 * k_values, v_values: bf16 [B, H, update_length, D], D a multiple of 16, no
 * overlap with the pools or the table.  A page whose first slot this call
 * writes gets k_format / v_format (and its descriptor); rows that continue a
 * partly filled page are encoded in that page's stored format.  Affine codes:
 * clamp(rint(x / scale) + zero_point) with a correctly rounded float32 divide
 * (ties to even); F16 pages round to nearest even.  Pools, page_desc and
 * values 16-byte aligned.  Errors as pkv_paged_cache_update, plus PKV_E_ARG
 * for a bad format.  The pools and page_desc must be in writable bindings. */
pkv_status pkv_mixed_cache_update(const pkv_pool* pool, const pkv_tensor* k_pool,
                                  const pkv_tensor* v_pool, const pkv_tensor* page_desc,
                                  const int32_t* page_table_dev, const pkv_tensor* k_values,
                                  const pkv_tensor* v_values, const int32_t* position,
                                  int32_t update_length, pkv_page_format k_format,
                                  pkv_page_format v_format, void* stream);

/* Re-encode pages: for i < n_pages, rows [0, valid_rows[i]) of physical page
 * pages[i] (both host int32 arrays) are decoded ((code - zero) * scale as
 * one float32 multiply, or the dense value) and encoded in the new format;
 * rows [valid_rows[i], block_size) become the new format's zero.  k_format /
 * v_format NULL keeps that tensor.  Bytes of a slot past the new rows are
 * left as they were.  Every page must have been written by an append.
 * Errors (nothing is written): PKV_E_ARG for duplicate pages, a valid row
 * count outside [0, block_size] or a bad format; PKV_E_PAGE for a page id
 * outside [0, num_blocks); PKV_E_LAYOUT when block_size * D * 2 > 65536. */
pkv_status pkv_mixed_convert_pages(const pkv_tensor* k_pool, const pkv_tensor* v_pool,
                                   const pkv_tensor* page_desc, const int32_t* pages,
                                   const int32_t* valid_rows, int32_t n_pages,
                                   const pkv_page_format* k_format,
                                   const pkv_page_format* v_format, void* stream);

/* Decode attention over mixed pages (as pkv_paged_decode_attention): q bf16
 * [B, Hq, (1,) 128], out bf16 or f32, Hq / Hkv in {1, 2, 4, 8}, block_size a
 * power of two >= 16.  Affine K/V are decoded in registers and never
 * materialised; the token appended by the step is read back as stored. */
pkv_status pkv_paged_decode_attention_mixed(const pkv_tensor* q, const pkv_tensor* k_pool,
                                            const pkv_tensor* v_pool, const pkv_tensor* page_desc,
                                            const int32_t* page_table_dev,
                                            int32_t max_blocks_per_seq, int32_t block_size,
                                            const pkv_pool* pool, const int32_t* valid_len,
                                            float scale, int32_t left_window, pkv_tensor* out,
                                            void* workspace, size_t workspace_bytes,
                                            int32_t num_splits, void* stream);

/* ------------------------------------------------------------------------ */
/* Sampling                                                                  */
/* "Persistent input/output feedback", section "Autoregressive generation":
 * temperature 0 is greedy, a positive temperature samples
 * softmax(logits / temperature), a seed makes the draw repeatable, the final
 * position of [B, S, V] logits predicts the next token.                     */
/* ------------------------------------------------------------------------ */

size_t pkv_sample_workspace_size(int32_t B, int64_t V);

/* logits : [B, V] or [B, S, V], f32, f64, bf16 or f16.
 * temperature == 0: argmax, lowest index on ties; f64 logits are compared as
 * f64 values.  temperature > 0: the Gumbel-max draw argmax_v (y_v -
 * log(-log u_v)) with y_v = fl32(x_v * fl32(1/T)) (f64 logits: y_v = x_v *
 * (1/T) in f64), u_v = ((h >> 40) | 1) * 2^-24 and h output number
 * b*V + v + 1 of SplitMix64 seeded with `seed`.  Non-finite scores follow
 * numpy's argmax: NaN ranks above every number (the first NaN wins) and an
 * all -inf row yields index 0, so every id lies in [0, V).  Negative, NaN or
 * infinite temperature: PKV_E_ARG.
 * out_ids: device int64[B]. */
pkv_status pkv_sample(const pkv_tensor* logits, float temperature, uint64_t seed,
                      int64_t* out_ids, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_sample whose seed is that of iteration *step_dev of one generation:
 * seed + step * B * V * 0x9E3779B97F4A7C15 (mod 2^64), i.e.
 * pkv_generate_step_seed(seed, *step_dev, B, V), with the step counter read
 * from device memory when the kernel runs (step_dev: device int64, advanced
 * by pkv_advance).  step_dev NULL is pkv_sample. */
pkv_status pkv_sample_dev(const pkv_tensor* logits, float temperature, uint64_t seed, const int64_t* step_dev,
                          int64_t* out_ids, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Generation loop                                                           */
/* "Persistent input/output feedback", section "Autoregressive generation":
 * the result holds the prompt and the generated tokens; temperature 0 is
 * greedy, a positive one samples softmax(logits / T) and a seed makes it
 * repeatable; generation stops at the token limit or once every row has
 * emitted EOS; finished rows are padded with pad_token_id (EOS by default);
 * each iteration consumes one new token.  A caller's loop runs its model,
 * pkv_sample with pkv_generate_step_seed(seed, t, B, V), then
 * pkv_generate_finish, and stops when *unfinished reaches 0.                */
/* ------------------------------------------------------------------------ */

/* Seed of iteration `step` of one generation: seed + step * B * V * gamma
 * (mod 2^64, gamma the SplitMix64 increment 0x9E3779B97F4A7C15), so the
 * draws of iteration t use SplitMix64 outputs t*B*V + b*V + v + 1 of `seed`:
 * one counter across the whole generation, no two draws alike. */
uint64_t pkv_generate_step_seed(uint64_t seed, int64_t step, int32_t B, int64_t V);

/* sampled   : device int64[B], this iteration's draws (pkv_sample).
 * finished  : device u8[B], 0 / 1, read and updated (zero it before the first
 *             iteration).
 * tokens    : device int64[B, row_stride]; column `column` receives, per
 *             row, the sampled id, or pad_token_id if the row had already
 *             finished.  A row finishes when the written token equals
 *             eos_token_id (eos_token_id < 0: no EOS, rows never finish).
 * next_ids  : device int64[B], the written tokens (the model's next input);
 *             it may be `sampled` itself.
 * unfinished: device int32[1], the number of rows not finished afterwards.
 * Errors: PKV_E_ARG for null pointers, B < 0, column outside
 * [0, row_stride); PKV_E_ALIAS when tokens overlaps another argument. */
pkv_status pkv_generate_finish(const int64_t* sampled, uint8_t* finished, int64_t* tokens,
                               int64_t row_stride, int32_t column, int32_t B,
                               int64_t eos_token_id, int64_t pad_token_id, int64_t* next_ids,
                               int32_t* unfinished, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
