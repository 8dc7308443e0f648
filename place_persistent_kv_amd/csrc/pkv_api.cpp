// Host layer of libpkv: the extern "C" entry points of include/pkv.h.
//
// Every entry point validates its arguments completely before the first HIP
// call, so an error never enqueues work or touches a buffer ("Mutable
// execution cache", "Runtime contract"; "Persistent input/output feedback",
// "Lifecycle and validation": a failed call publishes no partial update).
// The library never allocates device memory: caches, pools, page tables,
// outputs and workspaces all belong to the caller ("Mutable execution
// cache", "Memory planning": an in-place update costs zero extra cache bytes).

#include "pkv.h"
#include "pkv_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

using namespace pkv;

// ---------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------
namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

pkv_status ok() {
    g_err.clear();
    return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
    return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define PKV_TRY(expr)                        \
    do {                                     \
        pkv_status _s = (expr);              \
        if (_s != PKV_OK) return _s;         \
    } while (0)

#define PKV_HIP(expr, what)                  \
    do {                                     \
        hipError_t _e = (expr);              \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

// ---------------------------------------------------------------------------
// Tensor descriptors
// ---------------------------------------------------------------------------
int64_t dtype_size(int32_t dt) {
    switch (dt) {
        case PKV_F32: return 4;
        case PKV_BF16: return 2;
        case PKV_F16: return 2;
        case PKV_U8: return 1;
        case PKV_I32: return 4;
        case PKV_I64: return 8;
        case PKV_F64: return 8;
        default: return 0;
    }
}

int64_t numel(const pkv_tensor* t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

int64_t nbytes(const pkv_tensor* t) { return numel(t) * dtype_size(t->dtype); }

pkv_status check_tensor(const pkv_tensor* t, const char* name, int ndim_lo, int ndim_hi) {
    if (!t) return fail(PKV_E_ARG, "%s: null descriptor", name);
    if (t->ndim < ndim_lo || t->ndim > ndim_hi)
        return fail(PKV_E_LAYOUT, "%s: rank %d not in [%d, %d]", name, t->ndim, ndim_lo, ndim_hi);
    if (dtype_size(t->dtype) == 0) return fail(PKV_E_DTYPE, "%s: unknown dtype %d", name, t->dtype);
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] < 0 || t->shape[i] > (int64_t(1) << 40))
            return fail(PKV_E_LAYOUT, "%s: bad extent %lld on axis %d", name, (long long)t->shape[i], i);
    if (!t->data && numel(t) > 0) return fail(PKV_E_ARG, "%s: null data pointer", name);
    return PKV_OK;
}

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + static_cast<uintptr_t>(bytes)};
}
Span span(const pkv_tensor* t) { return span(t->data, nbytes(t)); }

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// ---------------------------------------------------------------------------
// Writable-binding registry ("Mutable execution cache", "Runtime contract")
// ---------------------------------------------------------------------------
std::mutex g_bind_mu;
std::vector<pkv_binding*> g_bindings;

}  // namespace

struct pkv_binding {
    Span range;
};

namespace {

bool inside_writable_binding(Span s) {
    std::lock_guard<std::mutex> lk(g_bind_mu);
    for (const pkv_binding* b : g_bindings)
        if (b->range.lo <= s.lo && s.hi <= b->range.hi) return true;
    return false;
}

pkv_status check_writable(const pkv_tensor* t, const char* name) {
    if (numel(t) == 0) return PKV_OK;
    if (!inside_writable_binding(span(t)))
        return fail(PKV_E_READONLY, "%s: storage is not inside a writable binding "
                                    "(bind it with pkv_bind_writable first)", name);
    return PKV_OK;
}

pkv_status check_disjoint(const pkv_tensor* a, const char* an, Span b, const char* bn) {
    if (overlap(span(a), b)) return fail(PKV_E_ALIAS, "%s overlaps %s", an, bn);
    return PKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Page pool
// ---------------------------------------------------------------------------
struct pkv_pool {
    int32_t num_blocks, block_size, max_seqs, maxb;
    std::deque<int32_t> free_list;   // front = next page handed out
    std::vector<int32_t> table;      // [max_seqs * maxb], -1 = none
    std::vector<int32_t> held;       // pages held per sequence
    std::vector<int32_t> length;     // reserved logical length per sequence
};

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pkv_status write_table(int32_t* table_dev, const std::vector<int32_t>& idx,
                       const std::vector<int32_t>& val, hipStream_t stream) {
    for (size_t i = 0; i < idx.size(); i += kMaxTableWrites) {
        TableWriteArgs a;
        a.table = table_dev;
        a.count = static_cast<int32_t>(std::min<size_t>(kMaxTableWrites, idx.size() - i));
        for (int j = 0; j < a.count; ++j) {
            a.index[j] = idx[i + j];
            a.value[j] = val[i + j];
        }
        PKV_HIP(launch_table_write(a, stream), "page-table write");
    }
    return PKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Decode split planning
// ---------------------------------------------------------------------------
namespace {

constexpr int kTargetWorkgroups = 1024;  // 4 per CU on 256 CUs: 2 resident x 2 rounds
// rows of unequal span on the bf16 / f16 fast kernel: smaller splits, so that
// the short last splits (launched last, longest first) even out the end
constexpr int kTargetWorkgroupsUneven = 2048;
constexpr int kMinAutoTps = 384;         // tokens per split, library choice: >= 6 steps per wave
constexpr int kTpsQuantum = 64;          // fast kernel: 4 waves x 16 tokens

struct Plan {
    int32_t tps = 0;
    int32_t S_max = 0;
    std::vector<int32_t> nsplit;  // per row
};

// Splits of one launch.  `units_per_token` weights tokens by the number of
// workgroups that stream them (Hkv for the fast kernels, Hq for the generic).
// Compute units of the current device (256 on a whole gfx950 part, fewer in
// a partitioned mode); 256 when no device answers.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

Plan plan_splits(const int32_t* len, int B, int units, int num_splits, int max_tps,
                 int target = kTargetWorkgroups) {
    Plan p;
    int64_t total = 0;
    int32_t lmax = 1;
    for (int b = 0; b < B; ++b) {
        total += len[b];
        lmax = std::max(lmax, len[b]);
    }
    int64_t tps;
    if (num_splits > 0) {
        tps = std::max<int64_t>(kTpsQuantum, ceil_div(ceil_div(lmax, num_splits), kTpsQuantum) * kTpsQuantum);
    } else {
        tps = ceil_div(total * units, target);
        tps = std::max<int64_t>(kMinAutoTps, ceil_div(tps, kTpsQuantum) * kTpsQuantum);
    }
    if (max_tps > 0) tps = std::min<int64_t>(tps, max_tps);
    p.tps = static_cast<int32_t>(tps);
    p.nsplit.resize(B);
    for (int b = 0; b < B; ++b) {
        p.nsplit[b] = static_cast<int32_t>(ceil_div(len[b], tps));
        p.S_max = std::max(p.S_max, p.nsplit[b]);
    }
    return p;
}

int64_t split_bound(int32_t max_len, int32_t num_splits) {
    int64_t s_auto = ceil_div(std::max(max_len, 1), kMinAutoTps);
    int64_t s_gen = ceil_div(std::max(max_len, 1), kGenericMaxTps);
    if (num_splits > 0) return std::max<int64_t>(num_splits, s_gen);
    return std::max(s_auto, s_gen);
}

// Work order of a launch over host lengths (the kernels' split_item): the
// splits of a whole tps tokens first, row by row, then each row's shorter
// last split, longest first.  span: the rows' split ranges (nsplit = ceil(span
// / tps) each); returns the number of work items, sum of nsplit.
int work_order(const int32_t* span, int rows, int32_t tps, int32_t* full_begin, uint16_t* tail_row) {
    int n_full = 0;
    for (int i = 0; i < rows; ++i) {
        full_begin[i] = n_full;
        n_full += span[i] / tps;
    }
    full_begin[rows] = n_full;
    int n_tail = 0;
    for (int i = 0; i < rows; ++i)
        if (span[i] % tps) tail_row[n_tail++] = static_cast<uint16_t>(i);
    std::stable_sort(tail_row, tail_row + n_tail,
                     [&](uint16_t x, uint16_t y) { return span[x] % tps > span[y] % tps; });
    return n_full + n_tail;
}

size_t ws_bytes_for(int64_t B, int64_t Hq, int64_t D, int64_t S) {
    // [B, Hq, S, D] partial outputs + [B, Hq, S, 2] (max, sum), each 256-aligned
    size_t o = static_cast<size_t>(B * Hq * S * D) * 4;
    size_t ml = static_cast<size_t>(B * Hq * S * 2) * 4;
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    return up(o) + up(ml);
}

}  // namespace

// ===========================================================================
// extern "C"
// ===========================================================================
extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

// ---------------------------------------------------------------------------
pkv_status pkv_bind_writable(void* base, size_t bytes, pkv_binding** out) {
    if (!base || bytes == 0 || !out) return fail(PKV_E_ARG, "bind_writable: null base, zero size or null out");
    Span s = span(base, static_cast<int64_t>(bytes));
    std::lock_guard<std::mutex> lk(g_bind_mu);
    for (const pkv_binding* b : g_bindings)
        if (overlap(b->range, s))
            return fail(PKV_E_BUSY, "bind_writable: range overlaps a live writable binding");
    pkv_binding* b = new pkv_binding{s};
    g_bindings.push_back(b);
    *out = b;
    return ok();
}

pkv_status pkv_unbind(pkv_binding* binding) {
    if (!binding) return fail(PKV_E_ARG, "unbind: null binding");
    std::lock_guard<std::mutex> lk(g_bind_mu);
    auto it = std::find(g_bindings.begin(), g_bindings.end(), binding);
    if (it == g_bindings.end()) return fail(PKV_E_ARG, "unbind: unknown binding");
    g_bindings.erase(it);
    delete binding;
    return ok();
}

// ---------------------------------------------------------------------------
namespace {

// Everything a contiguous append of `values` into `cache` checks before it
// launches (the launch itself is the caller's)
pkv_status cache_update_checks(const char* who, const pkv_tensor* cache, const pkv_tensor* values,
                               const int32_t* position, int32_t update_length) {
    PKV_TRY(check_tensor(cache, "cache", 4, 4));
    PKV_TRY(check_tensor(values, "values", 4, 4));
    if (update_length < 0) return fail(PKV_E_ARG, "%s: negative update_length", who);
    const int64_t B = cache->shape[0], H = cache->shape[1], cap = cache->shape[2], D = cache->shape[3];
    if (values->dtype != cache->dtype) return fail(PKV_E_DTYPE, "%s: values dtype != cache dtype", who);
    if (values->shape[0] != B || values->shape[1] != H || values->shape[2] != update_length ||
        values->shape[3] != D)
        return fail(PKV_E_LAYOUT, "%s: values must be [B, H, update_length, D] of the cache", who);
    if (B > 0 && !position) return fail(PKV_E_ARG, "%s: null position", who);
    for (int64_t b = 0; b < B; ++b)
        if (position[b] < 0 || int64_t(position[b]) + update_length > cap)
            return fail(PKV_E_CAPACITY, "%s: row %lld: position %d + update_length %d > capacity %lld", who,
                        (long long)b, position[b], update_length, (long long)cap);
    PKV_TRY(check_writable(cache, "cache"));
    PKV_TRY(check_disjoint(values, "values", span(cache), "cache"));
    return PKV_OK;
}

// One launch per kMaxRows rows; a second (values, cache) pair, when given,
// is written by the same launches
pkv_status cache_update_launch(const char* who, const pkv_tensor* cache, const pkv_tensor* cache2,
                               const pkv_tensor* values, const pkv_tensor* values2, const int32_t* position,
                               int32_t update_length, void* stream) {
    const int64_t B = cache->shape[0], H = cache->shape[1], cap = cache->shape[2], D = cache->shape[3];
    const int64_t row_bytes = D * dtype_size(cache->dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        CopyRowsArgs a;
        a.rows = static_cast<int32_t>(std::min<int64_t>(kMaxRows, B - b0));
        const int64_t src_off = b0 * H * update_length * row_bytes, dst_off = b0 * H * cap * row_bytes;
        a.src = static_cast<const uint8_t*>(values->data) + src_off;
        a.dst = static_cast<uint8_t*>(cache->data) + dst_off;
        if (cache2) {
            a.src2 = static_cast<const uint8_t*>(values2->data) + src_off;
            a.dst2 = static_cast<uint8_t*>(cache2->data) + dst_off;
        }
        a.row_bytes = row_bytes;
        a.H = static_cast<int32_t>(H);
        a.n = update_length;
        a.cap = static_cast<int32_t>(cap);
        for (int i = 0; i < a.rows; ++i) a.pos[i] = position[b0 + i];
        const hipError_t e = launch_copy_rows(a, s);
        if (e != hipSuccess) return fail(PKV_E_HIP, "%s launch: %s", who, hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

pkv_status pkv_cache_update(const pkv_tensor* cache, const pkv_tensor* values,
                            const int32_t* position, int32_t update_length,
                            void** out_cache, void* stream) {
    PKV_TRY(check_tensor(cache, "cache", 4, 4));
    PKV_TRY(check_tensor(values, "values", 4, 4));
    if (!out_cache) return fail(PKV_E_ARG, "cache_update: null out_cache");
    PKV_TRY(cache_update_checks("cache_update", cache, values, position, update_length));
    *out_cache = cache->data;
    if (numel(values) == 0) return ok();
    return cache_update_launch("cache_update", cache, nullptr, values, nullptr, position, update_length, stream);
}

pkv_status pkv_cache_update_kv(const pkv_tensor* k_cache, const pkv_tensor* v_cache, const pkv_tensor* k_values,
                               const pkv_tensor* v_values, const int32_t* position, int32_t update_length,
                               void* stream) {
    const char* who = "cache_update_kv";
    PKV_TRY(cache_update_checks(who, k_cache, k_values, position, update_length));
    PKV_TRY(cache_update_checks(who, v_cache, v_values, position, update_length));
    for (int i = 0; i < 4; ++i)
        if (k_cache->shape[i] != v_cache->shape[i])
            return fail(PKV_E_LAYOUT, "%s: K and V caches must have the same shape", who);
    if (k_cache->dtype != v_cache->dtype) return fail(PKV_E_DTYPE, "%s: K and V caches differ in dtype", who);
    if (overlap(span(k_cache), span(v_cache))) return fail(PKV_E_ALIAS, "%s: k_cache overlaps v_cache", who);
    PKV_TRY(check_disjoint(k_values, "k_values", span(v_cache), "v_cache"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(k_cache), "k_cache"));
    if (numel(k_values) == 0) return ok();
    return cache_update_launch(who, k_cache, v_cache, k_values, v_values, position, update_length, stream);
}

// ---------------------------------------------------------------------------
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                           int32_t max_blocks_per_seq, const int32_t* initial_free_order,
                           pkv_pool** out) {
    if (!out) return fail(PKV_E_ARG, "pool_create: null out");
    if (num_blocks <= 0 || block_size <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_E_ARG, "pool_create: dimensions must be positive");
    if (int64_t(max_seqs) * max_blocks_per_seq > (int64_t(1) << 31) - 1 ||
        int64_t(max_blocks_per_seq) * block_size > (int64_t(1) << 31) - 1)
        return fail(PKV_E_ARG, "pool_create: page table too large for int32 indexing");
    auto* p = new pkv_pool;
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->max_seqs = max_seqs;
    p->maxb = max_blocks_per_seq;
    if (initial_free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            int32_t id = initial_free_order[i];
            if (id < 0 || id >= num_blocks || seen[id]) {
                delete p;
                return fail(PKV_E_ARG, "pool_create: initial_free_order is not a permutation of 0..num_blocks-1");
            }
            seen[id] = 1;
            p->free_list.push_back(id);
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) p->free_list.push_back(i);
    }
    p->table.assign(size_t(max_seqs) * max_blocks_per_seq, -1);
    p->held.assign(max_seqs, 0);
    p->length.assign(max_seqs, 0);
    *out = p;
    return ok();
}

pkv_status pkv_pool_destroy(pkv_pool* pool) {
    if (!pool) return fail(PKV_E_ARG, "pool_destroy: null pool");
    delete pool;
    return ok();
}

pkv_status pkv_pool_reserve(pkv_pool* pool, int32_t n, const int32_t* seqs,
                            const int32_t* new_len, int32_t* page_table_dev, void* stream) {
    if (!pool) return fail(PKV_E_ARG, "pool_reserve: null pool");
    if (n < 0 || (n > 0 && (!seqs || !new_len))) return fail(PKV_E_ARG, "pool_reserve: bad arrays");
    std::vector<char> listed(pool->max_seqs, 0);
    int64_t missing_total = 0;
    std::vector<int32_t> missing(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        int32_t s = seqs[i];
        if (s < 0 || s >= pool->max_seqs) return fail(PKV_E_PAGE, "pool_reserve: sequence %d out of range", s);
        if (listed[s]) return fail(PKV_E_PAGE, "pool_reserve: sequence %d listed twice", s);
        listed[s] = 1;
        if (new_len[i] < 0) return fail(PKV_E_ARG, "pool_reserve: negative length");
        int64_t need = ceil_div(new_len[i], pool->block_size);
        if (need > pool->maxb)
            return fail(PKV_E_PAGE, "pool_reserve: sequence %d needs %lld pages > max_blocks_per_seq %d", s,
                        (long long)need, pool->maxb);
        missing[i] = static_cast<int32_t>(std::max<int64_t>(0, need - pool->held[s]));
        missing_total += missing[i];
    }
    if (missing_total > static_cast<int64_t>(pool->free_list.size()))
        return fail(PKV_E_NOMEM, "pool_reserve: need %lld pages, %zu free", (long long)missing_total,
                    pool->free_list.size());
    std::vector<int32_t> idx, val;
    for (int32_t i = 0; i < n; ++i) {
        int32_t s = seqs[i];
        for (int32_t k = 0; k < missing[i]; ++k) {
            int32_t phys = pool->free_list.front();
            pool->free_list.pop_front();
            int32_t slot = pool->held[s] + k;
            pool->table[size_t(s) * pool->maxb + slot] = phys;
            idx.push_back(s * pool->maxb + slot);
            val.push_back(phys);
        }
        pool->held[s] += missing[i];
        pool->length[s] = std::max(pool->length[s], new_len[i]);
    }
    if (page_table_dev && !idx.empty())
        PKV_TRY(write_table(page_table_dev, idx, val, static_cast<hipStream_t>(stream)));
    return ok();
}

pkv_status pkv_pool_release(pkv_pool* pool, int32_t seq, int32_t* page_table_dev, void* stream) {
    if (!pool) return fail(PKV_E_ARG, "pool_release: null pool");
    if (seq < 0 || seq >= pool->max_seqs) return fail(PKV_E_PAGE, "pool_release: sequence %d out of range", seq);
    std::vector<int32_t> idx, val;
    for (int32_t k = 0; k < pool->held[seq]; ++k) {
        int32_t& e = pool->table[size_t(seq) * pool->maxb + k];
        pool->free_list.push_back(e);
        e = -1;
        idx.push_back(seq * pool->maxb + k);
        val.push_back(-1);
    }
    pool->held[seq] = 0;
    pool->length[seq] = 0;
    if (page_table_dev && !idx.empty())
        PKV_TRY(write_table(page_table_dev, idx, val, static_cast<hipStream_t>(stream)));
    return ok();
}

pkv_status pkv_pool_query(const pkv_pool* pool, int32_t seq, int32_t* held_pages, int32_t* reserved_len) {
    if (!pool) return fail(PKV_E_ARG, "pool_query: null pool");
    if (seq < 0 || seq >= pool->max_seqs) return fail(PKV_E_PAGE, "pool_query: sequence %d out of range", seq);
    if (held_pages) *held_pages = pool->held[seq];
    if (reserved_len) *reserved_len = pool->length[seq];
    return ok();
}

pkv_status pkv_pool_free_count(const pkv_pool* pool, int32_t* free_pages) {
    if (!pool || !free_pages) return fail(PKV_E_ARG, "pool_free_count: null argument");
    *free_pages = static_cast<int32_t>(pool->free_list.size());
    return ok();
}

pkv_status pkv_pool_table(const pkv_pool* pool, int32_t* out_host) {
    if (!pool || !out_host) return fail(PKV_E_ARG, "pool_table: null argument");
    std::memcpy(out_host, pool->table.data(), pool->table.size() * sizeof(int32_t));
    return ok();
}

// ---------------------------------------------------------------------------
namespace {

// Checks shared by the paged updates: pages of every written position are
// reserved for the row, positions fit the page table.
pkv_status check_paged_positions(const pkv_pool* pool, int64_t B, const int32_t* position, int32_t n) {
    if (!pool) return fail(PKV_E_ARG, "paged update: a pool handle is required");
    if (B > pool->max_seqs) return fail(PKV_E_PAGE, "paged update: batch %lld > max_seqs %d", (long long)B, pool->max_seqs);
    if (B > 0 && !position) return fail(PKV_E_ARG, "paged update: null position");
    const int64_t cap = int64_t(pool->maxb) * pool->block_size;
    for (int64_t b = 0; b < B; ++b) {
        if (position[b] < 0 || int64_t(position[b]) + n > cap)
            return fail(PKV_E_CAPACITY, "paged update: row %lld: position %d + update_length %d > %lld",
                        (long long)b, position[b], n, (long long)cap);
        if (n > 0 && ceil_div(int64_t(position[b]) + n, pool->block_size) > pool->held[b])
            return fail(PKV_E_PAGE, "paged update: row %lld writes past its %d reserved pages "
                                    "(reserve with pkv_pool_reserve first)", (long long)b, pool->held[b]);
    }
    return PKV_OK;
}

// Everything a host-position paged append of `values` into `pool_kv` checks
// before it launches (the launch itself is the caller's)
pkv_status paged_update_checks(const char* who, const pkv_pool* pool, const pkv_tensor* pool_kv,
                               const int32_t* page_table_dev, const pkv_tensor* values,
                               const int32_t* position, int32_t update_length) {
    PKV_TRY(check_tensor(pool_kv, "pool_kv", 4, 4));
    PKV_TRY(check_tensor(values, "values", 4, 4));
    if (update_length < 0) return fail(PKV_E_ARG, "%s: negative update_length", who);
    if (!pool) return fail(PKV_E_ARG, "%s: a pool handle is required", who);
    const int64_t NB = pool_kv->shape[0], H = pool_kv->shape[1], bs = pool_kv->shape[2], D = pool_kv->shape[3];
    const int64_t B = values->shape[0];
    if (NB != pool->num_blocks || bs != pool->block_size)
        return fail(PKV_E_LAYOUT, "%s: pool_kv is [%lld, H, %lld, D] but the pool has %d blocks of %d", who,
                    (long long)NB, (long long)bs, pool->num_blocks, pool->block_size);
    if (values->dtype != pool_kv->dtype) return fail(PKV_E_DTYPE, "%s: values dtype != pool dtype", who);
    if (values->shape[1] != H || values->shape[2] != update_length || values->shape[3] != D)
        return fail(PKV_E_LAYOUT, "%s: values must be [B, H, update_length, D] of the pool", who);
    if (!page_table_dev && B > 0 && update_length > 0) return fail(PKV_E_ARG, "%s: null page table", who);
    PKV_TRY(check_paged_positions(pool, B, position, update_length));
    PKV_TRY(check_writable(pool_kv, "pool_kv"));
    PKV_TRY(check_disjoint(values, "values", span(pool_kv), "pool_kv"));
    return PKV_OK;
}

// One launch per kMaxRows rows; a second (values, pool) pair, when given,
// is written by the same launches
pkv_status paged_update_launch(const char* who, const pkv_pool* pool, const pkv_tensor* pool_kv,
                               const pkv_tensor* pool2, const int32_t* page_table_dev, const pkv_tensor* values,
                               const pkv_tensor* values2, const int32_t* position, int32_t update_length,
                               void* stream) {
    const int64_t H = pool_kv->shape[1], bs = pool_kv->shape[2], D = pool_kv->shape[3];
    const int64_t B = values->shape[0];
    const int64_t row_bytes = D * dtype_size(pool_kv->dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        PagedCopyArgs a;
        a.rows = static_cast<int32_t>(std::min<int64_t>(kMaxRows, B - b0));
        const int64_t src_off = b0 * H * update_length * row_bytes;
        a.src = static_cast<const uint8_t*>(values->data) + src_off;
        a.pool = static_cast<uint8_t*>(pool_kv->data);
        if (pool2) {
            a.src2 = static_cast<const uint8_t*>(values2->data) + src_off;
            a.pool2 = static_cast<uint8_t*>(pool2->data);
        }
        a.page_table = page_table_dev;
        a.row_bytes = row_bytes;
        a.H = static_cast<int32_t>(H);
        a.n = update_length;
        a.bs = static_cast<int32_t>(bs);
        a.maxb = pool->maxb;
        a.row0 = static_cast<int32_t>(b0);
        for (int i = 0; i < a.rows; ++i) a.pos[i] = position[b0 + i];
        const hipError_t e = launch_paged_copy(a, s);
        if (e != hipSuccess) return fail(PKV_E_HIP, "%s launch: %s", who, hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

pkv_status pkv_paged_cache_update(const pkv_pool* pool, const pkv_tensor* pool_kv,
                                  const int32_t* page_table_dev, const pkv_tensor* values,
                                  const int32_t* position, int32_t update_length,
                                  void** out_pool, void* stream) {
    PKV_TRY(check_tensor(pool_kv, "pool_kv", 4, 4));
    PKV_TRY(check_tensor(values, "values", 4, 4));
    if (!out_pool) return fail(PKV_E_ARG, "paged_cache_update: null out_pool");
    PKV_TRY(paged_update_checks("paged_cache_update", pool, pool_kv, page_table_dev, values, position, update_length));
    *out_pool = pool_kv->data;
    if (numel(values) == 0) return ok();
    return paged_update_launch("paged_cache_update", pool, pool_kv, nullptr, page_table_dev, values, nullptr,
                               position, update_length, stream);
}

pkv_status pkv_paged_cache_update_kv(const pkv_pool* pool, const pkv_tensor* k_pool, const pkv_tensor* v_pool,
                                     const int32_t* page_table_dev, const pkv_tensor* k_values,
                                     const pkv_tensor* v_values, const int32_t* position, int32_t update_length,
                                     void* stream) {
    const char* who = "paged_cache_update_kv";
    PKV_TRY(paged_update_checks(who, pool, k_pool, page_table_dev, k_values, position, update_length));
    PKV_TRY(paged_update_checks(who, pool, v_pool, page_table_dev, v_values, position, update_length));
    for (int i = 0; i < 4; ++i)
        if (k_pool->shape[i] != v_pool->shape[i] || k_values->shape[i] != v_values->shape[i])
            return fail(PKV_E_LAYOUT, "%s: K and V pools, and K and V values, must have the same shapes", who);
    if (k_pool->dtype != v_pool->dtype) return fail(PKV_E_DTYPE, "%s: K and V pools differ in dtype", who);
    if (overlap(span(k_pool), span(v_pool))) return fail(PKV_E_ALIAS, "%s: k_pool overlaps v_pool", who);
    PKV_TRY(check_disjoint(k_values, "k_values", span(v_pool), "v_pool"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(k_pool), "k_pool"));
    if (numel(k_values) == 0) return ok();
    return paged_update_launch(who, pool, k_pool, v_pool, page_table_dev, k_values, v_values, position,
                               update_length, stream);
}

namespace {

// K and V appended in one launch at positions held in device memory (the
// contiguous form when page_table is null).
pkv_status kv_append_dev(const char* who, const pkv_pool* pool, const pkv_tensor* k_dst,
                         const pkv_tensor* v_dst, const int32_t* page_table_dev, const pkv_tensor* k_values,
                         const pkv_tensor* v_values, const int32_t* position_dev, int32_t update_length,
                         int32_t* status_dev, void* stream, bool paged) {
    PKV_TRY(check_tensor(k_dst, "k", 4, 4));
    PKV_TRY(check_tensor(v_dst, "v", 4, 4));
    PKV_TRY(check_tensor(k_values, "k_values", 4, 4));
    PKV_TRY(check_tensor(v_values, "v_values", 4, 4));
    if (update_length < 0 || update_length > kMaxDevAppend)
        return fail(PKV_E_ARG, "%s: update_length must be in [0, %d]", who, kMaxDevAppend);
    if (!position_dev || !status_dev) return fail(PKV_E_ARG, "%s: null position or status", who);
    for (int i = 0; i < 4; ++i)
        if (k_dst->shape[i] != v_dst->shape[i]) return fail(PKV_E_LAYOUT, "%s: K and V storage shapes differ", who);
    if (k_dst->dtype != v_dst->dtype || k_values->dtype != k_dst->dtype || v_values->dtype != k_dst->dtype)
        return fail(PKV_E_DTYPE, "%s: values and storage must share one dtype", who);
    const int64_t H = k_dst->shape[1], D = k_dst->shape[3];
    const int64_t B = k_values->shape[0];
    for (const pkv_tensor* t : {k_values, v_values})
        if (t->shape[0] != B || t->shape[1] != H || t->shape[2] != update_length || t->shape[3] != D)
            return fail(PKV_E_LAYOUT, "%s: values must be [B, H, update_length, D] of the storage", who);
    const int64_t row_bytes = D * dtype_size(k_dst->dtype);
    if (row_bytes % 16) return fail(PKV_E_LAYOUT, "%s: a row must be a multiple of 16 bytes", who);
    for (const pkv_tensor* t : {k_dst, v_dst, k_values, v_values})
        if (reinterpret_cast<uintptr_t>(t->data) % 16) return fail(PKV_E_LAYOUT, "%s: tensors must be 16-byte aligned", who);
    int64_t cap;
    if (paged) {
        if (!pool) return fail(PKV_E_ARG, "%s: a pool handle is required", who);
        if (k_dst->shape[0] != pool->num_blocks || k_dst->shape[2] != pool->block_size)
            return fail(PKV_E_LAYOUT, "%s: pools do not match the pool handle", who);
        if (B > pool->max_seqs) return fail(PKV_E_PAGE, "%s: batch larger than the pool's max_seqs", who);
        if (!page_table_dev && B > 0) return fail(PKV_E_ARG, "%s: null page table", who);
        cap = int64_t(pool->maxb) * pool->block_size;
    } else {
        if (k_dst->shape[0] != B) return fail(PKV_E_LAYOUT, "%s: cache batch != values batch", who);
        cap = k_dst->shape[2];
    }
    if (cap > INT32_MAX) return fail(PKV_E_LAYOUT, "%s: capacity too large", who);
    PKV_TRY(check_writable(k_dst, "k"));
    PKV_TRY(check_writable(v_dst, "v"));
    if (overlap(span(k_dst), span(v_dst))) return fail(PKV_E_ALIAS, "%s: K and V storage overlap", who);
    for (const pkv_tensor* t : {k_values, v_values}) {
        PKV_TRY(check_disjoint(t, "values", span(k_dst), "k"));
        PKV_TRY(check_disjoint(t, "values", span(v_dst), "v"));
    }
    const Span st = span(status_dev, 4), ps = span(position_dev, B * 4);
    if (overlap(st, span(k_dst)) || overlap(st, span(v_dst)) || overlap(ps, span(k_dst)) || overlap(ps, span(v_dst)))
        return fail(PKV_E_ALIAS, "%s: position and status must not overlap the storage", who);
    if (B == 0 || update_length == 0 || H == 0) return ok();
    KvAppendDevArgs a;
    a.src[0] = static_cast<const uint8_t*>(k_values->data);
    a.src[1] = static_cast<const uint8_t*>(v_values->data);
    a.dst[0] = static_cast<uint8_t*>(k_dst->data);
    a.dst[1] = static_cast<uint8_t*>(v_dst->data);
    a.page_table = paged ? page_table_dev : nullptr;
    a.pos = position_dev;
    a.status = status_dev;
    a.row_bytes = row_bytes;
    a.B = static_cast<int32_t>(B);
    a.H = static_cast<int32_t>(H);
    a.n = update_length;
    a.cap = static_cast<int32_t>(cap);
    a.bs = paged ? pool->block_size : 0;
    a.maxb = paged ? pool->maxb : 0;
    a.nb = paged ? pool->num_blocks : 0;
    PKV_HIP(launch_kv_append_dev(a, static_cast<hipStream_t>(stream)), "kv append launch");
    return ok();
}

}  // namespace

pkv_status pkv_cache_update_kv_dev(const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                                   const pkv_tensor* k_values, const pkv_tensor* v_values,
                                   const int32_t* position_dev, int32_t update_length, int32_t* status_dev,
                                   void* stream) {
    return kv_append_dev("cache_update_kv_dev", nullptr, k_cache, v_cache, nullptr, k_values, v_values,
                         position_dev, update_length, status_dev, stream, false);
}

pkv_status pkv_paged_cache_update_kv_dev(const pkv_pool* pool, const pkv_tensor* k_pool,
                                         const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                         const pkv_tensor* k_values, const pkv_tensor* v_values,
                                         const int32_t* position_dev, int32_t update_length,
                                         int32_t* status_dev, void* stream) {
    return kv_append_dev("paged_cache_update_kv_dev", pool, k_pool, v_pool, page_table_dev, k_values, v_values,
                         position_dev, update_length, status_dev, stream, true);
}

pkv_status pkv_advance(int32_t* values_dev, int32_t n, int32_t delta, int64_t* step_dev, void* stream) {
    if (n < 0) return fail(PKV_E_ARG, "advance: negative count");
    if (n > 0 && !values_dev) return fail(PKV_E_ARG, "advance: null values");
    if (values_dev && step_dev && overlap(span(values_dev, int64_t(n) * 4), span(step_dev, 8)))
        return fail(PKV_E_ALIAS, "advance: values overlap the step counter");
    if (n == 0 && !step_dev) return ok();
    AdvanceArgs a;
    a.values = values_dev;
    a.step = step_dev;
    a.n = n;
    a.delta = delta;
    PKV_HIP(launch_advance(a, static_cast<hipStream_t>(stream)), "advance launch");
    return ok();
}

pkv_status pkv_paged_cache_update_int4(const pkv_pool* pool, const pkv_tensor* codes_pool,
                                       const pkv_tensor* params_pool,
                                       const int32_t* page_table_dev, const pkv_tensor* values,
                                       uint16_t scale_f16, uint16_t zero_point_f16,
                                       const int32_t* position, int32_t update_length,
                                       void** out_codes, void** out_params, void* stream) {
    PKV_TRY(check_tensor(codes_pool, "codes_pool", 4, 4));
    PKV_TRY(check_tensor(params_pool, "params_pool", 5, 5));
    PKV_TRY(check_tensor(values, "values", 4, 4));
    if (!out_codes || !out_params) return fail(PKV_E_ARG, "paged_cache_update_int4: null output pointer");
    if (update_length < 0) return fail(PKV_E_ARG, "paged_cache_update_int4: negative update_length");
    if (!pool) return fail(PKV_E_ARG, "paged_cache_update_int4: a pool handle is required");
    const int64_t NB = codes_pool->shape[0], H = codes_pool->shape[1], bs = codes_pool->shape[2];
    const int64_t D = codes_pool->shape[3] * 2;
    const int64_t B = values->shape[0];
    if (codes_pool->dtype != PKV_U8 || params_pool->dtype != PKV_F16)
        return fail(PKV_E_DTYPE, "paged_cache_update_int4: codes must be u8 and params f16");
    if (values->dtype != PKV_F32 && values->dtype != PKV_BF16)
        return fail(PKV_E_DTYPE, "paged_cache_update_int4: values must be f32 or bf16");
    if (NB != pool->num_blocks || bs != pool->block_size)
        return fail(PKV_E_LAYOUT, "paged_cache_update_int4: codes pool does not match the pool handle");
    if (D % 32 != 0 || D == 0) return fail(PKV_E_LAYOUT, "paged_cache_update_int4: D must be a positive multiple of 32");
    const int64_t ps[5] = {NB, H, bs, D / 32, 2};
    for (int i = 0; i < 5; ++i)
        if (params_pool->shape[i] != ps[i])
            return fail(PKV_E_LAYOUT, "paged_cache_update_int4: params must be [NB, H, bs, D/32, 2]");
    if (values->shape[1] != H || values->shape[2] != update_length || values->shape[3] != D)
        return fail(PKV_E_LAYOUT, "paged_cache_update_int4: values must be [B, H, update_length, D]");
    // scale: positive, finite binary16; zero point: integer 0..15 in binary16
    const uint16_t se = (scale_f16 >> 10) & 0x1F;
    if ((scale_f16 & 0x8000) || se == 0x1F || (scale_f16 & 0x7FFF) == 0)
        return fail(PKV_E_ARG, "paged_cache_update_int4: scale must be positive and finite");
    float zp = -1.0f;
    for (int c = 0; c <= 15; ++c) {
        // binary16 encoding of the integer c
        uint16_t bits = 0;
        if (c > 0) {
            int e = 0;
            while ((c >> (e + 1)) != 0) ++e;
            bits = static_cast<uint16_t>(((e + 15) << 10) | (((c << 10) >> e) & 0x3FF));
        }
        if (bits == zero_point_f16) zp = float(c);
    }
    if (zp < 0) return fail(PKV_E_ARG, "paged_cache_update_int4: zero point must be an integer 0..15");
    if (!page_table_dev && B > 0 && update_length > 0) return fail(PKV_E_ARG, "paged_cache_update_int4: null page table");
    PKV_TRY(check_paged_positions(pool, B, position, update_length));
    PKV_TRY(check_writable(codes_pool, "codes_pool"));
    PKV_TRY(check_writable(params_pool, "params_pool"));
    PKV_TRY(check_disjoint(values, "values", span(codes_pool), "codes_pool"));
    PKV_TRY(check_disjoint(values, "values", span(params_pool), "params_pool"));
    if (overlap(span(codes_pool), span(params_pool))) return fail(PKV_E_ALIAS, "codes_pool overlaps params_pool");
    *out_codes = codes_pool->data;
    *out_params = params_pool->data;
    if (numel(values) == 0) return ok();

    // widen the binary16 scale exactly
    const int sm = scale_f16 & 0x3FF;
    const float scale = se == 0 ? std::ldexp(float(sm), -24) : std::ldexp(float(sm | 0x400), se - 25);
    const int64_t esz = dtype_size(values->dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        PagedInt4Args a;
        a.rows = static_cast<int32_t>(std::min<int64_t>(kMaxRows, B - b0));
        a.src = static_cast<const uint8_t*>(values->data) + b0 * H * update_length * D * esz;
        a.codes = static_cast<uint8_t*>(codes_pool->data);
        a.params = static_cast<uint16_t*>(params_pool->data);
        a.page_table = page_table_dev;
        a.src_bf16 = values->dtype == PKV_BF16;
        a.H = static_cast<int32_t>(H);
        a.n = update_length;
        a.bs = static_cast<int32_t>(bs);
        a.maxb = pool->maxb;
        a.D = static_cast<int32_t>(D);
        a.row0 = static_cast<int32_t>(b0);
        a.scale = scale;
        a.zero_point = zp;
        a.scale_bits = scale_f16;
        a.zp_bits = zero_point_f16;
        for (int i = 0; i < a.rows; ++i) a.pos[i] = position[b0 + i];
        PKV_HIP(launch_paged_int4_append(a, s), "paged_cache_update_int4 launch");
    }
    return ok();
}

pkv_status pkv_paged_gather(const pkv_tensor* pool_kv, const int32_t* page_table_dev,
                            int32_t max_blocks_per_seq, int32_t seq, int32_t length,
                            pkv_tensor* out, void* stream) {
    PKV_TRY(check_tensor(pool_kv, "pool_kv", 4, 4));
    PKV_TRY(check_tensor(out, "out", 3, 3));
    if (!page_table_dev || max_blocks_per_seq <= 0 || seq < 0 || length < 0)
        return fail(PKV_E_ARG, "paged_gather: bad page table, sequence or length");
    const int64_t H = pool_kv->shape[1], bs = pool_kv->shape[2], D = pool_kv->shape[3];
    if (ceil_div(length, bs) > max_blocks_per_seq) return fail(PKV_E_PAGE, "paged_gather: length exceeds the page table row");
    if (out->dtype != pool_kv->dtype || out->shape[0] != H || out->shape[1] != length || out->shape[2] != D)
        return fail(PKV_E_LAYOUT, "paged_gather: out must be [H, length, D] of the pool's dtype");
    PKV_TRY(check_disjoint(out, "out", span(pool_kv), "pool_kv"));
    if (length == 0 || H == 0 || D == 0) return ok();
    GatherArgs a;
    a.pool = static_cast<const uint8_t*>(pool_kv->data);
    a.table_row = page_table_dev + int64_t(seq) * max_blocks_per_seq;
    a.out = static_cast<uint8_t*>(out->data);
    a.row_bytes = D * dtype_size(pool_kv->dtype);
    a.H = static_cast<int32_t>(H);
    a.bs = static_cast<int32_t>(bs);
    a.length = length;
    PKV_HIP(launch_gather(a, static_cast<hipStream_t>(stream)), "paged_gather launch");
    return ok();
}

// ---------------------------------------------------------------------------
size_t pkv_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_len,
                                 int32_t num_splits) {
    (void)Hkv;
    if (B <= 0 || Hq <= 0 || D <= 0 || max_len <= 0 || num_splits < 0) return 0;
    return ws_bytes_for(B, Hq, D, split_bound(max_len, num_splits));
}

namespace {

int kv_kind_of(int32_t dt) {
    switch (dt) {
        case PKV_F32: return kKvF32;
        case PKV_BF16: return kKvBF16;
        case PKV_F16: return kKvF16;
        default: return -1;
    }
}

struct QView {
    int64_t B, Hq, D;
};

// q [B, Hq, (1,) Dk]; out the same with the last dim dv (dv < 0: Dk)
pkv_status check_q_out(const pkv_tensor* q, const pkv_tensor* out, QView* v, int64_t dv = -1) {
    PKV_TRY(check_tensor(q, "q", 3, 4));
    PKV_TRY(check_tensor(out, "out", 3, 4));
    if (q->ndim == 4 && q->shape[2] != 1) return fail(PKV_E_LAYOUT, "q must be [B, Hq, 1, D] or [B, Hq, D]");
    v->B = q->shape[0];
    v->Hq = q->shape[1];
    v->D = q->shape[q->ndim - 1];
    if (dv < 0) dv = v->D;
    if (out->ndim != q->ndim) return fail(PKV_E_LAYOUT, "out must have the shape of q (value head size last)");
    for (int i = 0; i < q->ndim; ++i)
        if (out->shape[i] != (i == q->ndim - 1 ? dv : q->shape[i]))
            return fail(PKV_E_LAYOUT, "out must have the shape of q (value head size last)");
    return PKV_OK;
}

// New K/V rows that the attention launch writes into contiguous caches
// before it reads them (pkv_decode_step); checked by the caller.
struct FusedAppend {
    const pkv_tensor* k_values;
    const pkv_tensor* v_values;
    int32_t n;
};

// Shared body of the bf16/f32 decode entry points.
pkv_status decode_common(const pkv_tensor* q, const pkv_tensor* k, const pkv_tensor* v,
                         bool paged, const int32_t* page_table, int32_t maxb, int32_t bs,
                         const pkv_pool* pool, const int32_t* valid_len, float scale,
                         int32_t left_window, pkv_tensor* out, void* ws, size_t ws_bytes,
                         int32_t num_splits, void* stream, const pkv_tensor* page_desc = nullptr,
                         bool static_ws = false, const int32_t* len_dev = nullptr, int32_t max_len = 0,
                         int32_t* status = nullptr, const FusedAppend* app = nullptr) {
    const bool dev = len_dev != nullptr;   // valid lengths in device memory, bounded by max_len
    const bool mixed = page_desc != nullptr;
    QView qv;
    PKV_TRY(check_tensor(k, "k", 4, 4));
    PKV_TRY(check_tensor(v, "v", 4, 4));
    const int64_t Dv = v->shape[3];                  // value head size (may differ from the key's)
    PKV_TRY(check_q_out(q, out, &qv, Dv));
    const int64_t B = qv.B, Hq = qv.Hq, D = qv.D;
    const int64_t Hkv = k->shape[1];
    const int kind = kv_kind_of(q->dtype);
    if (kind < 0) return fail(PKV_E_DTYPE, "q must be f32, bf16 or f16");
    if (mixed) {
        if (q->dtype != PKV_BF16) return fail(PKV_E_DTYPE, "mixed pages: q must be bf16");
        if (dtype_size(k->dtype) != 2 || dtype_size(v->dtype) != 2)
            return fail(PKV_E_DTYPE, "mixed pages: the slot pools are described as bf16 or f16 tensors");
    } else if (k->dtype != q->dtype || v->dtype != q->dtype) {
        return fail(PKV_E_DTYPE, "q, k and v must share a dtype");
    }
    if (out->dtype != q->dtype && out->dtype != PKV_F32) return fail(PKV_E_DTYPE, "out must have q's dtype or f32");
    for (int i = 0; i < 3; ++i)
        if (v->shape[i] != k->shape[i]) return fail(PKV_E_LAYOUT, "k and v must agree in all but the head size");
    if (k->shape[3] != D) return fail(PKV_E_LAYOUT, "k head size %lld != q head size %lld", (long long)k->shape[3], (long long)D);
    if (Dv <= 0 || Dv > 256) return fail(PKV_E_LAYOUT, "value head size must be in [1, 256]");
    if (Hkv <= 0 || Hq % Hkv != 0) return fail(PKV_E_LAYOUT, "query heads %lld must be a multiple of K/V heads %lld", (long long)Hq, (long long)Hkv);
    if (D <= 0 || D > 256) return fail(PKV_E_LAYOUT, "head size must be in [1, 256]");
    if (num_splits < 0) return fail(PKV_E_ARG, "num_splits must be >= 0");
    int64_t cap;
    if (paged) {
        if (!page_table) return fail(PKV_E_ARG, "null page table");
        if (bs <= 0 || bs != k->shape[2]) return fail(PKV_E_LAYOUT, "block_size %d != pool slot count %lld", bs, (long long)k->shape[2]);
        if (maxb <= 0) return fail(PKV_E_ARG, "max_blocks_per_seq must be positive");
        cap = int64_t(maxb) * bs;
        if (pool) {
            if (pool->block_size != bs || pool->num_blocks != k->shape[0] || pool->maxb != maxb)
                return fail(PKV_E_LAYOUT, "pool handle does not match the K/V pools");
            if (B > pool->max_seqs) return fail(PKV_E_PAGE, "batch larger than the pool's max_seqs");
        }
    } else {
        if (k->shape[0] != B) return fail(PKV_E_LAYOUT, "cache batch %lld != q batch %lld", (long long)k->shape[0], (long long)B);
        cap = k->shape[2];
    }
    if (dev) {
        if (!status) return fail(PKV_E_ARG, "null status");
        if (max_len < 1 || max_len > cap)
            return fail(PKV_E_CAPACITY, "max_len %d not in [1, %lld]", max_len, (long long)cap);
        if (overlap(span(status, 4), span(out)) || overlap(span(len_dev, B * 4), span(out)))
            return fail(PKV_E_ALIAS, "status and valid_len must not overlap out");
    }
    if (B > 0 && !valid_len && !dev) return fail(PKV_E_ARG, "null valid_len");
    for (int64_t b = 0; b < B && !dev; ++b) {
        if (valid_len[b] < 1 || valid_len[b] > cap)
            return fail(PKV_E_CAPACITY, "row %lld: valid_len %d not in [1, %lld]", (long long)b, valid_len[b], (long long)cap);
        if (paged && pool && ceil_div(valid_len[b], bs) > pool->held[b])
            return fail(PKV_E_PAGE, "row %lld: valid_len %d needs %lld pages, %d reserved", (long long)b, valid_len[b],
                        (long long)ceil_div(valid_len[b], bs), pool->held[b]);
    }
    if (!(scale == scale) || std::isinf(scale)) return fail(PKV_E_ARG, "scale must be finite");
    if (left_window < -1) return fail(PKV_E_ARG, "left_window must be -1 (unbounded) or >= 0");
    if (mixed) {
        PKV_TRY(check_tensor(page_desc, "page_desc", 2, 2));
        if (page_desc->dtype != PKV_U8 || page_desc->shape[0] != k->shape[0] || page_desc->shape[1] != 16)
            return fail(PKV_E_LAYOUT, "page_desc must be u8 [num_blocks, 16]");
        if (!mixed_decode_supported(static_cast<int>(D), static_cast<int>(Hq / Hkv), bs) || Dv != D)
            return fail(PKV_E_LAYOUT, "mixed pages: D = 128, Hq / Hkv in {1, 2, 4, 8}, block_size a power of two >= 16");
        if (reinterpret_cast<uintptr_t>(k->data) % 16 || reinterpret_cast<uintptr_t>(v->data) % 16 ||
            reinterpret_cast<uintptr_t>(page_desc->data) % 16 || reinterpret_cast<uintptr_t>(q->data) % 16)
            return fail(PKV_E_LAYOUT, "mixed pages: pools, page_desc and q must be 16-byte aligned");
        PKV_TRY(check_disjoint(page_desc, "page_desc", span(out), "out"));
    }
    const Span os = span(out);
    PKV_TRY(check_disjoint(q, "q", os, "out"));
    PKV_TRY(check_disjoint(k, "k", os, "out"));
    PKV_TRY(check_disjoint(v, "v", os, "out"));
    if (B == 0 || Hq == 0) return ok();

    const int G = static_cast<int>(Hq / Hkv);
    const bool fast = mixed || (Dv == D && fast_decode_supported(kind, static_cast<int>(D), G, paged, bs));
    // size the workspace for the whole call (all row groups share it)
    // splits cover only each row's visible range (from its 64-token quantum on)
    // (device lengths: every row planned at the bound max_len)
    std::vector<int32_t> span_len(B);
    for (int64_t b = 0; b < B; ++b) {
        const int32_t L = dev ? max_len : valid_len[b];
        span_len[b] = L - split_base(L, left_window);
    }
    // Rows of one span on the memory-bound fast kernel, with every launch group
    // holding at least one workgroup per CU: one split per row.  All those
    // workgroups are resident together and share HBM evenly, so they end
    // together, and no merge launch is needed (splitting only helps when spans
    // differ, where the long rows would otherwise be left running alone).
    int32_t splits = num_splits;
    int target = kTargetWorkgroups;
    if (splits == 0 && fast && !mixed && !dev) {
        const int64_t last_group = B - (B - 1) / kMaxRows * kMaxRows;
        bool equal = true;
        for (int64_t b = 1; b < B && equal; ++b) equal = span_len[b] == span_len[0];
        if (equal && last_group * Hkv >= device_cus()) splits = 1;
        if (!equal) target = kTargetWorkgroupsUneven;
    }
    Plan full = plan_splits(span_len.data(), static_cast<int>(B), fast ? static_cast<int>(Hkv) : static_cast<int>(Hq),
                            splits, fast ? 0 : kGenericMaxTps, target);
    const size_t need = ws_bytes_for(B, Hq, Dv, full.S_max);
    if (static_ws && (full.S_max > 1 || !fast)) {
        // after every check: the scratch's device address is the first HIP call
        if (need > ws_bytes)
            return fail(PKV_E_NOMEM, "the split partials need %zu bytes, more than the %zu-byte static scratch "
                        "(fewer splits or fewer rows per call)", need, ws_bytes);
        const hipError_t e = noalloc_scratch(&ws);
        if (e != hipSuccess) return fail(PKV_E_HIP, "static scratch address: %s", hipGetErrorString(e));
    } else if (full.S_max > 1 || !fast) {
        if (!ws || ws_bytes < need)
            return fail(PKV_E_NOMEM, "workspace of %zu bytes needed, %zu given (pkv_decode_workspace_size)", need, ws_bytes);
        const Span wss = span(ws, static_cast<int64_t>(need));
        if (overlap(wss, os) || overlap(wss, span(q)) || overlap(wss, span(k)) || overlap(wss, span(v)) ||
            (app && (overlap(wss, span(app->k_values)) || overlap(wss, span(app->v_values)))))
            return fail(PKV_E_ALIAS, "workspace overlaps an input or the output");
        if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(PKV_E_ARG, "workspace must be 256-byte aligned");
    }
    const size_t o_bytes = (static_cast<size_t>(B * Hq * full.S_max * Dv) * 4 + 255) & ~size_t(255);
    float* ws_o = static_cast<float*>(ws);
    float* ws_ml = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes) : nullptr;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t esz = dtype_size(q->dtype);
    const int64_t out_esz = dtype_size(out->dtype);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        const int rows = static_cast<int>(std::min<int64_t>(kMaxRows, B - b0));
        DecodeArgs a;
        a.q = static_cast<const uint8_t*>(q->data) + b0 * Hq * D * esz;
        if (paged) {
            a.k = k->data;
            a.v = v->data;
            a.page_table = page_table + b0 * maxb;
        } else {
            a.k = static_cast<const uint8_t*>(k->data) + b0 * Hkv * cap * D * esz;
            a.v = static_cast<const uint8_t*>(v->data) + b0 * Hkv * cap * Dv * esz;
            a.page_table = nullptr;
        }
        a.out = static_cast<uint8_t*>(out->data) + b0 * Hq * Dv * out_esz;
        a.ws_o = ws_o ? ws_o + b0 * Hq * full.S_max * Dv : nullptr;
        a.ws_ml = ws_ml ? ws_ml + b0 * Hq * full.S_max * 2 : nullptr;
        a.kv_kind = kind;
        a.out_f32 = out->dtype == PKV_F32 && q->dtype != PKV_F32;
        a.Hq = static_cast<int32_t>(Hq);
        a.Hkv = static_cast<int32_t>(Hkv);
        a.D = static_cast<int32_t>(D);
        a.Dv = static_cast<int32_t>(Dv);
        a.cap = static_cast<int32_t>(paged ? 0 : cap);
        a.bs = paged ? bs : 0;
        a.maxb = paged ? maxb : 0;
        a.log2bs = 0;
        while (paged && (1 << a.log2bs) < bs) ++a.log2bs;
        a.S_max = full.S_max;
        a.tps = full.tps;
        a.row0 = static_cast<int32_t>(b0);
        a.rows = rows;
        const float sc = scale > 0 ? scale : 1.0f / std::sqrt(float(D));
        a.scale_log2 = sc * 1.4426950408889634f;
        a.window = left_window;
        a.page_desc = mixed ? page_desc->data : nullptr;
        if (app && app->n > 0) {
            a.app_k = static_cast<const uint8_t*>(app->k_values->data) + b0 * Hkv * app->n * D * esz;
            a.app_v = static_cast<const uint8_t*>(app->v_values->data) + b0 * Hkv * app->n * Dv * esz;
            a.app_n = app->n;
            const uintptr_t bases = reinterpret_cast<uintptr_t>(app->k_values->data) |
                                    reinterpret_cast<uintptr_t>(app->v_values->data) |
                                    reinterpret_cast<uintptr_t>(k->data) | reinterpret_cast<uintptr_t>(v->data);
            a.app_vec16 = (bases % 16 == 0 && (D * esz) % 16 == 0 && (Dv * esz) % 16 == 0) ? 1 : 0;
        }
        int total = 0;
        bool any_split = false;
        if (dev) {   // S_max split slots per row; the kernels read the lengths
            a.len_dev = len_dev;
            a.len_limit = max_len;
            a.nb = paged ? static_cast<int32_t>(k->shape[0]) : 0;
            a.status = status;
            total = rows * full.S_max;
            any_split = full.S_max > 1;
        } else {
            for (int i = 0; i < rows; ++i) {
                a.len[i] = valid_len[b0 + i];
                any_split |= full.nsplit[b0 + i] > 1;
            }
            total = work_order(span_len.data() + b0, rows, full.tps, a.full_begin, a.tail_row);
        }
        if (mixed) {
            PKV_HIP(launch_decode_mixed(a, G, total * static_cast<int>(Hkv), s), "mixed decode launch");
        } else if (fast) {
            PKV_HIP(launch_decode_fast(a, G, total * static_cast<int>(Hkv), s), "decode launch");
        } else {
            PKV_HIP(launch_decode_generic(a, total * static_cast<int>(Hq), s), "decode launch");
        }
        if (any_split) {
            MergeArgs m;
            m.ws_o = a.ws_o;
            m.ws_ml = a.ws_ml;
            m.out = a.out;
            m.out_kind = kv_kind_of(out->dtype);
            m.Hq = a.Hq;
            m.D = a.Dv;
            m.S_max = a.S_max;
            m.row0 = a.row0;
            m.rows = rows;
            m.min_splits = 2;  // every attention kernel finishes single-split rows itself
            if (dev) {
                m.len_dev = len_dev;
                m.len_limit = max_len;
                m.tps = full.tps;
                m.window = left_window;
                m.len_add = app ? app->n : 0;
            } else {
                for (int i = 0; i < rows; ++i) m.nsplit[i] = full.nsplit[b0 + i];
            }
            PKV_HIP(launch_merge(m, s), "merge launch");
        }
    }
    return ok();
}

}  // namespace

pkv_status pkv_decode_attention(const pkv_tensor* q, const pkv_tensor* k_cache,
                                const pkv_tensor* v_cache, const int32_t* valid_len,
                                float scale, int32_t left_window, pkv_tensor* out, void* workspace,
                                size_t workspace_bytes, int32_t num_splits, void* stream) {
    return decode_common(q, k_cache, v_cache, false, nullptr, 0, 0, nullptr, valid_len, scale, left_window,
                         out, workspace, workspace_bytes, num_splits, stream);
}

pkv_status pkv_decode_step(const pkv_tensor* k_cache, const pkv_tensor* v_cache, const pkv_tensor* k_values,
                           const pkv_tensor* v_values, const int32_t* position, int32_t update_length,
                           const pkv_tensor* q, float scale, int32_t left_window, pkv_tensor* out,
                           void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream) {
    const char* who = "decode_step";
    // the append's checks (pkv_cache_update_kv) ...
    PKV_TRY(cache_update_checks(who, k_cache, k_values, position, update_length));
    PKV_TRY(cache_update_checks(who, v_cache, v_values, position, update_length));
    for (int i = 0; i < 3; ++i)
        if (k_cache->shape[i] != v_cache->shape[i])
            return fail(PKV_E_LAYOUT, "%s: K and V caches must agree in batch, heads and capacity", who);
    if (k_cache->dtype != v_cache->dtype) return fail(PKV_E_DTYPE, "%s: K and V caches differ in dtype", who);
    if (overlap(span(k_cache), span(v_cache))) return fail(PKV_E_ALIAS, "%s: k_cache overlaps v_cache", who);
    PKV_TRY(check_disjoint(k_values, "k_values", span(v_cache), "v_cache"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(k_cache), "k_cache"));
    // ... and those of the step as a whole: the launch writes the caches
    // while it reads q and the new rows, and writes out
    PKV_TRY(check_tensor(q, "q", 3, 4));
    PKV_TRY(check_tensor(out, "out", 3, 4));
    for (const pkv_tensor* t : {k_cache, v_cache}) {
        PKV_TRY(check_disjoint(q, "q", span(t), "a cache"));
        PKV_TRY(check_disjoint(out, "out", span(t), "a cache"));
    }
    PKV_TRY(check_disjoint(k_values, "k_values", span(out), "out"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(out), "out"));
    const int64_t B = k_cache->shape[0];
    std::vector<int32_t> valid_len(static_cast<size_t>(B));
    for (int64_t b = 0; b < B; ++b) valid_len[b] = position[b] + update_length;
    const FusedAppend app{k_values, v_values, update_length};
    return decode_common(q, k_cache, v_cache, false, nullptr, 0, 0, nullptr, valid_len.data(), scale, left_window,
                         out, workspace, workspace_bytes, num_splits, stream, nullptr, false, nullptr, 0, nullptr,
                         &app);
}

pkv_status pkv_decode_step_dev(const pkv_tensor* k_cache, const pkv_tensor* v_cache, const pkv_tensor* k_values,
                               const pkv_tensor* v_values, const int32_t* position_dev, int32_t update_length,
                               const pkv_tensor* q, int32_t max_len, float scale, int32_t left_window,
                               pkv_tensor* out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                               int32_t* status_dev, void* stream) {
    const char* who = "decode_step_dev";
    PKV_TRY(check_tensor(k_cache, "k_cache", 4, 4));
    const int64_t B = k_cache->shape[0];
    if (!position_dev) return fail(PKV_E_ARG, "%s: null position", who);
    // the append's checks with every position 0 (the positions themselves are
    // checked on the device against max_len)
    const std::vector<int32_t> zeros(static_cast<size_t>(B), 0);
    PKV_TRY(cache_update_checks(who, k_cache, k_values, zeros.data(), update_length));
    PKV_TRY(cache_update_checks(who, v_cache, v_values, zeros.data(), update_length));
    for (int i = 0; i < 3; ++i)
        if (k_cache->shape[i] != v_cache->shape[i])
            return fail(PKV_E_LAYOUT, "%s: K and V caches must agree in batch, heads and capacity", who);
    if (k_cache->dtype != v_cache->dtype) return fail(PKV_E_DTYPE, "%s: K and V caches differ in dtype", who);
    if (overlap(span(k_cache), span(v_cache))) return fail(PKV_E_ALIAS, "%s: k_cache overlaps v_cache", who);
    PKV_TRY(check_disjoint(k_values, "k_values", span(v_cache), "v_cache"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(k_cache), "k_cache"));
    PKV_TRY(check_tensor(q, "q", 3, 4));
    PKV_TRY(check_tensor(out, "out", 3, 4));
    for (const pkv_tensor* t : {k_cache, v_cache}) {
        PKV_TRY(check_disjoint(q, "q", span(t), "a cache"));
        PKV_TRY(check_disjoint(out, "out", span(t), "a cache"));
        if (overlap(span(position_dev, B * 4), span(t)) || (status_dev && overlap(span(status_dev, 4), span(t))))
            return fail(PKV_E_ALIAS, "%s: position or status overlaps a cache", who);
    }
    PKV_TRY(check_disjoint(k_values, "k_values", span(out), "out"));
    PKV_TRY(check_disjoint(v_values, "v_values", span(out), "out"));
    const FusedAppend app{k_values, v_values, update_length};
    return decode_common(q, k_cache, v_cache, false, nullptr, 0, 0, nullptr, nullptr, scale, left_window, out,
                         workspace, workspace_bytes, num_splits, stream, nullptr, false, position_dev, max_len,
                         status_dev, &app);
}

pkv_status pkv_paged_decode_attention(const pkv_tensor* q, const pkv_tensor* k_pool,
                                      const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                      int32_t max_blocks_per_seq, int32_t block_size,
                                      const pkv_pool* pool, const int32_t* valid_len,
                                      float scale, int32_t left_window, pkv_tensor* out,
                                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                                      void* stream) {
    return decode_common(q, k_pool, v_pool, true, page_table_dev, max_blocks_per_seq, block_size, pool,
                         valid_len, scale, left_window, out, workspace, workspace_bytes, num_splits, stream);
}


static_assert(kNoallocScratchBytes == PKV_NOALLOC_SCRATCH_BYTES, "scratch size and its documented limit agree");

pkv_status pkv_paged_decode_attention_noalloc(const pkv_tensor* q, const pkv_tensor* k_pool,
                                              const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              const pkv_pool* pool, const int32_t* valid_len,
                                              float scale, int32_t left_window, pkv_tensor* out,
                                              int32_t num_splits, void* stream) {
    return decode_common(q, k_pool, v_pool, true, page_table_dev, max_blocks_per_seq, block_size, pool,
                         valid_len, scale, left_window, out, nullptr, kNoallocScratchBytes, num_splits, stream,
                         nullptr, true);
}

pkv_status pkv_decode_attention_dev(const pkv_tensor* q, const pkv_tensor* k_cache,
                                    const pkv_tensor* v_cache, const int32_t* valid_len_dev,
                                    int32_t max_len, float scale, int32_t left_window, pkv_tensor* out,
                                    void* workspace, size_t workspace_bytes, int32_t num_splits,
                                    int32_t* status_dev, void* stream) {
    if (!valid_len_dev) return fail(PKV_E_ARG, "decode_attention_dev: null valid_len");
    return decode_common(q, k_cache, v_cache, false, nullptr, 0, 0, nullptr, nullptr, scale, left_window, out,
                         workspace, workspace_bytes, num_splits, stream, nullptr, false, valid_len_dev, max_len,
                         status_dev);
}

pkv_status pkv_paged_decode_attention_dev(const pkv_tensor* q, const pkv_tensor* k_pool,
                                          const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                          int32_t max_blocks_per_seq, int32_t block_size,
                                          const pkv_pool* pool, const int32_t* valid_len_dev,
                                          int32_t max_len, float scale, int32_t left_window,
                                          pkv_tensor* out, void* workspace, size_t workspace_bytes,
                                          int32_t num_splits, int32_t* status_dev, void* stream) {
    if (!valid_len_dev) return fail(PKV_E_ARG, "paged_decode_attention_dev: null valid_len");
    return decode_common(q, k_pool, v_pool, true, page_table_dev, max_blocks_per_seq, block_size, pool, nullptr,
                         scale, left_window, out, workspace, workspace_bytes, num_splits, stream, nullptr, false,
                         valid_len_dev, max_len, status_dev);
}

pkv_status pkv_paged_decode_attention_mixed(const pkv_tensor* q, const pkv_tensor* k_pool,
                                            const pkv_tensor* v_pool, const pkv_tensor* page_desc,
                                            const int32_t* page_table_dev,
                                            int32_t max_blocks_per_seq, int32_t block_size,
                                            const pkv_pool* pool, const int32_t* valid_len,
                                            float scale, int32_t left_window, pkv_tensor* out,
                                            void* workspace, size_t workspace_bytes,
                                            int32_t num_splits, void* stream) {
    if (!page_desc) return fail(PKV_E_ARG, "decode_attention_mixed: null page_desc");
    return decode_common(q, k_pool, v_pool, true, page_table_dev, max_blocks_per_seq, block_size, pool,
                         valid_len, scale, left_window, out, workspace, workspace_bytes, num_splits, stream,
                         page_desc);
}

static_assert(sizeof(pkv_page_desc) == sizeof(PageDesc) && offsetof(pkv_page_desc, v_scale) == offsetof(PageDesc, v_scale) &&
                  offsetof(pkv_page_desc, k_zero) == offsetof(PageDesc, k_zero) &&
                  offsetof(pkv_page_desc, k_storage) == offsetof(PageDesc, k_st) &&
                  offsetof(pkv_page_desc, v_storage) == offsetof(PageDesc, v_st),
              "pkv_page_desc and the kernels' descriptor share one layout");

namespace {

// A requested page format: storage in range; affine: positive finite scale and
// an integer zero point inside the code range.  Dense formats are stored with
// scale 1 and zero point 0.
pkv_status check_page_format(const pkv_page_format& f, const char* name) {
    if (f.storage < PKV_PAGE_BF16 || f.storage > PKV_PAGE_UINT2)
        return fail(PKV_E_ARG, "%s: unknown page storage %d", name, f.storage);
    if (f.storage >= PKV_PAGE_INT8) {
        if (!(f.scale > 0.0f) || std::isinf(f.scale)) return fail(PKV_E_ARG, "%s: scale must be positive and finite", name);
        const int nb = storage_bits(f.storage);
        const int lo = storage_signed(f.storage) ? -(1 << (nb - 1)) : 0;
        const int hi = storage_signed(f.storage) ? (1 << (nb - 1)) - 1 : (1 << nb) - 1;
        if (f.zero_point < lo || f.zero_point > hi)
            return fail(PKV_E_ARG, "%s: zero point %d outside the code range [%d, %d]", name, f.zero_point, lo, hi);
    }
    return PKV_OK;
}

void set_desc(PageDesc& d, const pkv_page_format& f, bool v) {
    const bool aff = f.storage >= PKV_PAGE_INT8;
    const float sc = aff ? f.scale : 1.0f;
    const int16_t z = static_cast<int16_t>(aff ? f.zero_point : 0);
    if (v) {
        d.v_st = static_cast<uint8_t>(f.storage);
        d.v_scale = sc;
        d.v_zero = z;
    } else {
        d.k_st = static_cast<uint8_t>(f.storage);
        d.k_scale = sc;
        d.k_zero = z;
    }
}

// The two slot pools and the descriptor table of a mixed pool.
pkv_status check_mixed_pools(const pkv_tensor* k_pool, const pkv_tensor* v_pool, const pkv_tensor* page_desc,
                             const char* who) {
    PKV_TRY(check_tensor(k_pool, "k_pool", 4, 4));
    PKV_TRY(check_tensor(v_pool, "v_pool", 4, 4));
    PKV_TRY(check_tensor(page_desc, "page_desc", 2, 2));
    if (dtype_size(k_pool->dtype) != 2 || dtype_size(v_pool->dtype) != 2)
        return fail(PKV_E_DTYPE, "%s: the slot pools are described as bf16 or f16 tensors", who);
    for (int i = 0; i < 4; ++i)
        if (k_pool->shape[i] != v_pool->shape[i]) return fail(PKV_E_LAYOUT, "%s: k_pool and v_pool shapes differ", who);
    if (page_desc->dtype != PKV_U8 || page_desc->shape[0] != k_pool->shape[0] || page_desc->shape[1] != 16)
        return fail(PKV_E_LAYOUT, "%s: page_desc must be u8 [num_blocks, 16]", who);
    if (k_pool->shape[3] % 16 != 0) return fail(PKV_E_LAYOUT, "%s: D must be a multiple of 16", who);
    if (reinterpret_cast<uintptr_t>(k_pool->data) % 16 || reinterpret_cast<uintptr_t>(v_pool->data) % 16 ||
        reinterpret_cast<uintptr_t>(page_desc->data) % 16)
        return fail(PKV_E_LAYOUT, "%s: pools and page_desc must be 16-byte aligned", who);
    if (overlap(span(k_pool), span(v_pool))) return fail(PKV_E_ALIAS, "%s: k_pool overlaps v_pool", who);
    PKV_TRY(check_disjoint(page_desc, "page_desc", span(k_pool), "k_pool"));
    PKV_TRY(check_disjoint(page_desc, "page_desc", span(v_pool), "v_pool"));
    return PKV_OK;
}

}  // namespace

pkv_status pkv_mixed_cache_update(const pkv_pool* pool, const pkv_tensor* k_pool,
                                  const pkv_tensor* v_pool, const pkv_tensor* page_desc,
                                  const int32_t* page_table_dev, const pkv_tensor* k_values,
                                  const pkv_tensor* v_values, const int32_t* position,
                                  int32_t update_length, pkv_page_format k_format,
                                  pkv_page_format v_format, void* stream) {
    PKV_TRY(check_mixed_pools(k_pool, v_pool, page_desc, "mixed_cache_update"));
    PKV_TRY(check_tensor(k_values, "k_values", 4, 4));
    PKV_TRY(check_tensor(v_values, "v_values", 4, 4));
    if (update_length < 0) return fail(PKV_E_ARG, "mixed_cache_update: negative update_length");
    if (!pool) return fail(PKV_E_ARG, "mixed_cache_update: a pool handle is required");
    PKV_TRY(check_page_format(k_format, "mixed_cache_update k_format"));
    PKV_TRY(check_page_format(v_format, "mixed_cache_update v_format"));
    const int64_t NB = k_pool->shape[0], H = k_pool->shape[1], bs = k_pool->shape[2], D = k_pool->shape[3];
    const int64_t B = k_values->shape[0];
    if (NB != pool->num_blocks || bs != pool->block_size)
        return fail(PKV_E_LAYOUT, "mixed_cache_update: pools are [%lld, H, %lld, D] but the pool has %d blocks of %d",
                    (long long)NB, (long long)bs, pool->num_blocks, pool->block_size);
    if (k_values->dtype != PKV_BF16 || v_values->dtype != PKV_BF16)
        return fail(PKV_E_DTYPE, "mixed_cache_update: values must be bf16");
    for (const pkv_tensor* t : {k_values, v_values})
        if (t->shape[0] != B || t->shape[1] != H || t->shape[2] != update_length || t->shape[3] != D)
            return fail(PKV_E_LAYOUT, "mixed_cache_update: values must be [B, H, update_length, D] of the pools");
    if (reinterpret_cast<uintptr_t>(k_values->data) % 16 || reinterpret_cast<uintptr_t>(v_values->data) % 16)
        return fail(PKV_E_LAYOUT, "mixed_cache_update: values must be 16-byte aligned");
    if (!page_table_dev && B > 0 && update_length > 0) return fail(PKV_E_ARG, "mixed_cache_update: null page table");
    PKV_TRY(check_paged_positions(pool, B, position, update_length));
    PKV_TRY(check_writable(k_pool, "k_pool"));
    PKV_TRY(check_writable(v_pool, "v_pool"));
    PKV_TRY(check_writable(page_desc, "page_desc"));
    for (const pkv_tensor* t : {k_values, v_values}) {
        PKV_TRY(check_disjoint(t, "values", span(k_pool), "k_pool"));
        PKV_TRY(check_disjoint(t, "values", span(v_pool), "v_pool"));
        PKV_TRY(check_disjoint(t, "values", span(page_desc), "page_desc"));
    }
    if (B == 0 || update_length == 0 || H == 0) return ok();

    PageDesc fmt{};
    set_desc(fmt, k_format, false);
    set_desc(fmt, v_format, true);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        MixedAppendArgs a;
        a.rows = static_cast<int32_t>(std::min<int64_t>(kMaxRows, B - b0));
        a.k_src = static_cast<const uint16_t*>(k_values->data) + b0 * H * update_length * D;
        a.v_src = static_cast<const uint16_t*>(v_values->data) + b0 * H * update_length * D;
        a.k_pool = static_cast<uint8_t*>(k_pool->data);
        a.v_pool = static_cast<uint8_t*>(v_pool->data);
        a.desc = static_cast<PageDesc*>(page_desc->data);
        a.page_table = page_table_dev;
        a.fmt = fmt;
        a.H = static_cast<int32_t>(H);
        a.n = update_length;
        a.bs = static_cast<int32_t>(bs);
        a.maxb = pool->maxb;
        a.D = static_cast<int32_t>(D);
        a.row0 = static_cast<int32_t>(b0);
        for (int i = 0; i < a.rows; ++i) a.pos[i] = position[b0 + i];
        PKV_HIP(launch_mixed_append(a, s), "mixed_cache_update launch");
    }
    return ok();
}

pkv_status pkv_mixed_convert_pages(const pkv_tensor* k_pool, const pkv_tensor* v_pool,
                                   const pkv_tensor* page_desc, const int32_t* pages,
                                   const int32_t* valid_rows, int32_t n_pages,
                                   const pkv_page_format* k_format,
                                   const pkv_page_format* v_format, void* stream) {
    PKV_TRY(check_mixed_pools(k_pool, v_pool, page_desc, "mixed_convert_pages"));
    if (n_pages < 0) return fail(PKV_E_ARG, "mixed_convert_pages: negative page count");
    if (n_pages > 0 && (!pages || !valid_rows)) return fail(PKV_E_ARG, "mixed_convert_pages: null page list");
    if (k_format) PKV_TRY(check_page_format(*k_format, "mixed_convert_pages k_format"));
    if (v_format) PKV_TRY(check_page_format(*v_format, "mixed_convert_pages v_format"));
    const int64_t NB = k_pool->shape[0], H = k_pool->shape[1], bs = k_pool->shape[2], D = k_pool->shape[3];
    if (bs * D * 2 > 65536) return fail(PKV_E_LAYOUT, "mixed_convert_pages: block_size * D * 2 must be <= 65536");
    std::vector<int32_t> sorted(pages, pages + n_pages);
    for (int32_t i = 0; i < n_pages; ++i) {
        if (pages[i] < 0 || pages[i] >= NB)
            return fail(PKV_E_PAGE, "mixed_convert_pages: page %d outside [0, %lld)", pages[i], (long long)NB);
        if (valid_rows[i] < 0 || valid_rows[i] > bs)
            return fail(PKV_E_ARG, "mixed_convert_pages: valid rows %d outside [0, %lld]", valid_rows[i], (long long)bs);
    }
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
        return fail(PKV_E_ARG, "mixed_convert_pages: page ids must be unique");
    if (k_format) PKV_TRY(check_writable(k_pool, "k_pool"));
    if (v_format) PKV_TRY(check_writable(v_pool, "v_pool"));
    if (k_format || v_format) PKV_TRY(check_writable(page_desc, "page_desc"));
    if (n_pages == 0 || (!k_format && !v_format) || H == 0) return ok();

    PageDesc fmt{};
    if (k_format) set_desc(fmt, *k_format, false);
    if (v_format) set_desc(fmt, *v_format, true);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t i0 = 0; i0 < n_pages; i0 += kMaxConvert) {
        const int cnt = std::min<int32_t>(kMaxConvert, n_pages - i0);
        for (int which = 0; which < 2; ++which) {
            const pkv_page_format* f = which ? v_format : k_format;
            if (!f) continue;
            MixedConvertArgs a;
            a.pool = static_cast<uint8_t*>((which ? v_pool : k_pool)->data);
            a.desc = static_cast<const PageDesc*>(page_desc->data);
            a.which = which;
            a.st = f->storage;
            a.scale = which ? fmt.v_scale : fmt.k_scale;
            a.zero = which ? fmt.v_zero : fmt.k_zero;
            a.H = static_cast<int32_t>(H);
            a.bs = static_cast<int32_t>(bs);
            a.D = static_cast<int32_t>(D);
            a.count = cnt;
            for (int i = 0; i < cnt; ++i) {
                a.page[i] = pages[i0 + i];
                a.valid[i] = valid_rows[i0 + i];
            }
            PKV_HIP(launch_mixed_convert(a, s), "mixed_convert_pages launch");
        }
        MixedDescArgs d;
        d.desc = static_cast<PageDesc*>(page_desc->data);
        d.set_k = k_format != nullptr;
        d.set_v = v_format != nullptr;
        d.fmt = fmt;
        d.count = cnt;
        for (int i = 0; i < cnt; ++i) d.page[i] = pages[i0 + i];
        PKV_HIP(launch_mixed_desc(d, s), "mixed_convert_pages descriptor launch");
    }
    return ok();
}

pkv_status pkv_paged_decode_attention_int4(const pkv_tensor* q, const pkv_tensor* k_codes,
                                           const pkv_tensor* k_params, const pkv_tensor* v_codes,
                                           const pkv_tensor* v_params,
                                           const int32_t* page_table_dev,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           const pkv_pool* pool, const int32_t* valid_len,
                                           float scale, int32_t left_window, pkv_tensor* out,
                                           void* workspace,
                                           size_t workspace_bytes, int32_t num_splits,
                                           void* stream) {
    QView qv;
    PKV_TRY(check_q_out(q, out, &qv));
    PKV_TRY(check_tensor(k_codes, "k_codes", 4, 4));
    PKV_TRY(check_tensor(v_codes, "v_codes", 4, 4));
    PKV_TRY(check_tensor(k_params, "k_params", 5, 5));
    PKV_TRY(check_tensor(v_params, "v_params", 5, 5));
    const int64_t B = qv.B, Hq = qv.Hq, D = qv.D;
    if (q->dtype != PKV_F32 || out->dtype != PKV_F32) return fail(PKV_E_DTYPE, "int4 decode: q and out must be f32");
    if (k_codes->dtype != PKV_U8 || v_codes->dtype != PKV_U8 || k_params->dtype != PKV_F16 ||
        v_params->dtype != PKV_F16)
        return fail(PKV_E_DTYPE, "int4 decode: codes must be u8 and params f16");
    if (D != kFastD) return fail(PKV_E_LAYOUT, "int4 decode: head size must be %d", kFastD);
    const int64_t NB = k_codes->shape[0], Hkv = k_codes->shape[1], bs = k_codes->shape[2];
    for (int i = 0; i < 4; ++i)
        if (v_codes->shape[i] != k_codes->shape[i]) return fail(PKV_E_LAYOUT, "int4 decode: K and V code pools differ");
    if (k_codes->shape[3] != D / 2) return fail(PKV_E_LAYOUT, "int4 decode: codes must be [NB, Hkv, bs, D/2]");
    const int64_t ps[5] = {NB, Hkv, bs, D / 32, 2};
    for (int i = 0; i < 5; ++i)
        if (k_params->shape[i] != ps[i] || v_params->shape[i] != ps[i])
            return fail(PKV_E_LAYOUT, "int4 decode: params must be [NB, Hkv, bs, D/32, 2]");
    if (Hkv <= 0 || Hq % Hkv != 0) return fail(PKV_E_LAYOUT, "int4 decode: Hq must be a multiple of Hkv");
    const int G = static_cast<int>(Hq / Hkv);
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_E_LAYOUT, "int4 decode: Hq / Hkv must be 1, 2, 4 or 8");
    if (!page_table_dev) return fail(PKV_E_ARG, "int4 decode: null page table");
    if (block_size != bs || bs < kSlabTokens || (bs & (bs - 1)) != 0)
        return fail(PKV_E_LAYOUT, "int4 decode: block_size must equal the pool's and be a power of two >= %d", kSlabTokens);
    if (max_blocks_per_seq <= 0) return fail(PKV_E_ARG, "int4 decode: max_blocks_per_seq must be positive");
    for (const pkv_tensor* t : {k_codes, v_codes, k_params, v_params})
        if (reinterpret_cast<uintptr_t>(t->data) % 16)
            return fail(PKV_E_LAYOUT, "int4 decode: code and parameter pools must be 16-byte aligned");
    if (num_splits < 0) return fail(PKV_E_ARG, "num_splits must be >= 0");
    if (pool && (pool->block_size != bs || pool->num_blocks != NB || pool->maxb != max_blocks_per_seq))
        return fail(PKV_E_LAYOUT, "int4 decode: pool handle does not match the pools");
    if (pool && B > pool->max_seqs) return fail(PKV_E_PAGE, "int4 decode: batch larger than the pool's max_seqs");
    const int64_t cap = int64_t(max_blocks_per_seq) * bs;
    if (B > 0 && !valid_len) return fail(PKV_E_ARG, "null valid_len");
    for (int64_t b = 0; b < B; ++b) {
        if (valid_len[b] < 1 || valid_len[b] > cap)
            return fail(PKV_E_CAPACITY, "row %lld: valid_len %d not in [1, %lld]", (long long)b, valid_len[b], (long long)cap);
        if (pool && ceil_div(valid_len[b], bs) > pool->held[b])
            return fail(PKV_E_PAGE, "row %lld: valid_len %d needs more pages than reserved", (long long)b, valid_len[b]);
    }
    if (!(scale == scale) || std::isinf(scale)) return fail(PKV_E_ARG, "scale must be finite");
    const Span os = span(out);
    PKV_TRY(check_disjoint(q, "q", os, "out"));
    for (const pkv_tensor* t : {k_codes, v_codes, k_params, v_params}) PKV_TRY(check_disjoint(t, "K/V pool", os, "out"));
    if (B == 0) return ok();

    if (left_window < -1) return fail(PKV_E_ARG, "left_window must be -1 (unbounded) or >= 0");
    std::vector<int32_t> span_len(B);
    for (int64_t b = 0; b < B; ++b) span_len[b] = valid_len[b] - split_base(valid_len[b], left_window);
    Plan full = plan_splits(span_len.data(), static_cast<int>(B), static_cast<int>(Hkv), num_splits, 0);
    const size_t need = ws_bytes_for(B, Hq, D, full.S_max);
    if (full.S_max > 1) {
        if (!workspace || workspace_bytes < need)
            return fail(PKV_E_NOMEM, "workspace of %zu bytes needed, %zu given (pkv_decode_workspace_size)", need,
                        workspace_bytes);
        const Span wss = span(workspace, static_cast<int64_t>(need));
        if (overlap(wss, os) || overlap(wss, span(q))) return fail(PKV_E_ALIAS, "workspace overlaps q or out");
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(PKV_E_ARG, "workspace must be 256-byte aligned");
    }
    const size_t o_bytes = (static_cast<size_t>(B * Hq * full.S_max * D) * 4 + 255) & ~size_t(255);
    float* ws_o = static_cast<float*>(workspace);
    float* ws_ml = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes) : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        const int rows = static_cast<int>(std::min<int64_t>(kMaxRows, B - b0));
        Int4DecodeArgs a;
        a.q = static_cast<const float*>(q->data) + b0 * Hq * D;
        a.kc = static_cast<const uint8_t*>(k_codes->data);
        a.kp = static_cast<const uint16_t*>(k_params->data);
        a.vc = static_cast<const uint8_t*>(v_codes->data);
        a.vp = static_cast<const uint16_t*>(v_params->data);
        a.page_table = page_table_dev + b0 * max_blocks_per_seq;
        a.out = static_cast<float*>(out->data) + b0 * Hq * D;
        a.ws_o = ws_o ? ws_o + b0 * Hq * full.S_max * D : nullptr;
        a.ws_ml = ws_ml ? ws_ml + b0 * Hq * full.S_max * 2 : nullptr;
        a.Hq = static_cast<int32_t>(Hq);
        a.Hkv = static_cast<int32_t>(Hkv);
        a.bs = block_size;
        a.maxb = max_blocks_per_seq;
        a.log2bs = 0;
        while ((1 << a.log2bs) < block_size) ++a.log2bs;
        a.S_max = full.S_max;
        a.tps = full.tps;
        a.row0 = static_cast<int32_t>(b0);
        a.rows = rows;
        const float sc = scale > 0 ? scale : 1.0f / std::sqrt(float(D));
        a.scale_log2 = sc * 1.4426950408889634f;
        a.window = left_window;
        bool any_split = false;
        for (int i = 0; i < rows; ++i) {
            a.len[i] = valid_len[b0 + i];
            any_split |= full.nsplit[b0 + i] > 1;
        }
        const int total = work_order(span_len.data() + b0, rows, full.tps, a.full_begin, a.tail_row);
        PKV_HIP(launch_decode_int4(a, G, total * static_cast<int>(Hkv), s), "int4 decode launch");
        if (any_split) {
            MergeArgs m;
            m.ws_o = a.ws_o;
            m.ws_ml = a.ws_ml;
            m.out = a.out;
            m.out_kind = kKvF32;
            m.Hq = a.Hq;
            m.D = static_cast<int32_t>(D);
            m.S_max = a.S_max;
            m.row0 = a.row0;
            m.rows = rows;
            m.min_splits = 2;
            for (int i = 0; i < rows; ++i) m.nsplit[i] = full.nsplit[b0 + i];
            PKV_HIP(launch_merge(m, s), "merge launch");
        }
    }
    return ok();
}

// ---------------------------------------------------------------------------
namespace {


// Workgroups of one chunk launch of `rows` rows without a split.
int64_t chunk_workgroups(int64_t rows, int64_t Hkv, int G, int64_t C) {
    return rows * Hkv * ceil_div(C, kChunkQueryRows / G);
}

// Most parts the library picks by itself: at most four workgroups per CU in
// total (one workgroup fills a CU's LDS) and kChunkMaxAutoSplits.
constexpr int kChunkMaxAutoSplits = 16;
int chunk_auto_cap(int64_t base, int cus) {
    if (base >= cus) return 1;
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kChunkMaxAutoSplits, 4 * cus / base)));
}

// Parts per key range when the caller leaves the choice to the library.  A
// workgroup occupies a CU alone, so a launch of fewer workgroups than CUs
// leaves CUs idle; S parts multiply the workgroups by S and cost the partials
// (written by the attention, read by the merge) and a merge launch.  Modelled
// time of S parts: rounds of the grid over the CUs x (tiles / S + 2) tile
// times of about 1.9 us (256 query rows x 64 keys x 128 dims, both products,
// at the measured matrix rate per CU), plus 3 us and the partial bytes at
// 4 TB/s for the merge; the cheapest S up to the cap wins.
int chunk_auto_splits(int64_t base, int cus, int64_t max_tiles, int64_t query_rows) {
    const int cap = chunk_auto_cap(base, cus);
    int best = 1;
    double best_us = 0.0;
    for (int S = 1; S <= cap; ++S) {
        const double rounds = double(ceil_div(base * S, cus));
        double us = rounds * (double(ceil_div(max_tiles, S)) + 2.0) * 1.9;
        if (S > 1) us += 3.0 + 2.0 * double(S) * double(query_rows) * (kChunkD + 2) * 4.0 / 4.0e6;
        if (S == 1 || us < best_us) {
            best = S;
            best_us = us;
        }
    }
    return best;
}

pkv_status chunk_attention_impl(const pkv_tensor* q, const pkv_tensor* k_pool, const pkv_tensor* v_pool,
                                const int32_t* page_table_dev, int32_t max_blocks_per_seq, int32_t block_size,
                                const pkv_pool* pool, const int32_t* p0, float scale, int32_t left_window,
                                pkv_tensor* out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                void* stream) {
    PKV_TRY(check_tensor(q, "q", 4, 4));
    PKV_TRY(check_tensor(out, "out", 4, 4));
    PKV_TRY(check_tensor(k_pool, "k_pool", 4, 4));
    PKV_TRY(check_tensor(v_pool, "v_pool", 4, 4));
    const int64_t B = q->shape[0], Hq = q->shape[1], C = q->shape[2], D = q->shape[3];
    if (q->dtype != PKV_BF16 || out->dtype != PKV_BF16 || k_pool->dtype != PKV_BF16 || v_pool->dtype != PKV_BF16)
        return fail(PKV_E_DTYPE, "chunk attention: q, pools and out must be bf16");
    for (int i = 0; i < 4; ++i) {
        if (out->shape[i] != q->shape[i]) return fail(PKV_E_LAYOUT, "chunk attention: out must have q's shape");
        if (v_pool->shape[i] != k_pool->shape[i]) return fail(PKV_E_LAYOUT, "chunk attention: K and V pools differ");
    }
    const int64_t NB = k_pool->shape[0], Hkv = k_pool->shape[1], bs = k_pool->shape[2];
    if (k_pool->shape[3] != D) return fail(PKV_E_LAYOUT, "chunk attention: head size mismatch");
    if (Hkv <= 0 || Hq % Hkv != 0) return fail(PKV_E_LAYOUT, "chunk attention: Hq must be a multiple of Hkv");
    const int G = static_cast<int>(Hq / Hkv);
    if (!chunk_supported(static_cast<int>(D), G, static_cast<int>(bs), static_cast<int>(C)))
        return fail(PKV_E_LAYOUT, "chunk attention: needs D == 128, Hq / Hkv in {1, 2, 4, 8}, block_size >= 4 and C >= 1");
    if (!page_table_dev) return fail(PKV_E_ARG, "chunk attention: null page table");
    if (block_size != bs) return fail(PKV_E_LAYOUT, "chunk attention: block_size != pool slot count");
    if ((bs & (bs - 1)) != 0) return fail(PKV_E_LAYOUT, "chunk attention: block_size must be a power of two");
    if (reinterpret_cast<uintptr_t>(k_pool->data) % 16 || reinterpret_cast<uintptr_t>(v_pool->data) % 16 ||
        reinterpret_cast<uintptr_t>(q->data) % 16 || reinterpret_cast<uintptr_t>(out->data) % 16)
        return fail(PKV_E_LAYOUT, "chunk attention: q, out and the pools must be 16-byte aligned");
    if (max_blocks_per_seq <= 0) return fail(PKV_E_ARG, "chunk attention: max_blocks_per_seq must be positive");
    if (left_window < -1) return fail(PKV_E_ARG, "chunk attention: left_window must be -1 (unbounded) or >= 0");
    if (pool && (pool->block_size != bs || pool->num_blocks != NB || pool->maxb != max_blocks_per_seq))
        return fail(PKV_E_LAYOUT, "chunk attention: pool handle does not match the pools");
    if (pool && B > pool->max_seqs) return fail(PKV_E_PAGE, "chunk attention: batch larger than max_seqs");
    if (B > 0 && !p0) return fail(PKV_E_ARG, "chunk attention: null p0");
    const int64_t cap = int64_t(max_blocks_per_seq) * bs;
    for (int64_t b = 0; b < B; ++b) {
        if (p0[b] < 0 || p0[b] + C > cap)
            return fail(PKV_E_CAPACITY, "chunk attention: row %lld: p0 %d + C %lld > %lld", (long long)b, p0[b],
                        (long long)C, (long long)cap);
        if (pool && ceil_div(p0[b] + C, bs) > pool->held[b])
            return fail(PKV_E_PAGE, "chunk attention: row %lld holds fewer pages than p0 + C needs", (long long)b);
    }
    if (!(scale == scale) || std::isinf(scale)) return fail(PKV_E_ARG, "scale must be finite");
    const Span os = span(out);
    PKV_TRY(check_disjoint(q, "q", os, "out"));
    PKV_TRY(check_disjoint(k_pool, "k_pool", os, "out"));
    PKV_TRY(check_disjoint(v_pool, "v_pool", os, "out"));
    if (num_splits < 0 || num_splits > kChunkMaxSplits)
        return fail(PKV_E_ARG, "chunk attention: num_splits must be 0 (library choice) .. %d", kChunkMaxSplits);
    if (B == 0) return ok();
    const int64_t rows_max = std::min<int64_t>(B, kMaxRows);
    int S = num_splits;
    if (S == 0) {
        // longest key range of a workgroup: the last query tile of the longest row
        int64_t p0_max = 0;
        for (int64_t b = 0; b < B; ++b) p0_max = std::max<int64_t>(p0_max, p0[b]);
        const int64_t last = p0_max + C - 1;
        const int64_t first = left_window >= 0 ? std::max<int64_t>(0, last - (kChunkQueryRows / G) + 1 - left_window) : 0;
        S = chunk_auto_splits(chunk_workgroups(rows_max, Hkv, G, C), device_cus(),
                              last / kChunkKeys - first / kChunkKeys + 1, rows_max * Hq * C);
    }
    float* ws_o = nullptr;
    float* ws_ml = nullptr;
    if (S > 1) {
        const size_t need = ws_bytes_for(rows_max, Hq * C, kChunkD, S);
        if (!workspace || workspace_bytes < need)
            return fail(PKV_E_NOMEM, "chunk attention: workspace of %zu bytes needed, %zu given (pkv_chunk_workspace_size)",
                        need, workspace_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) % 256)
            return fail(PKV_E_ARG, "chunk attention: workspace must be 256-byte aligned");
        const Span wss = span(workspace, static_cast<int64_t>(need));
        if (overlap(wss, os) || overlap(wss, span(q)) || overlap(wss, span(k_pool)) || overlap(wss, span(v_pool)))
            return fail(PKV_E_ALIAS, "chunk attention: workspace overlaps q, out or a pool");
        const size_t o_bytes = (static_cast<size_t>(rows_max * Hq * C * S * kChunkD) * 4 + 255) & ~size_t(255);
        ws_o = static_cast<float*>(workspace);
        ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += kMaxRows) {
        ChunkArgs a;
        a.rows = static_cast<int32_t>(std::min<int64_t>(kMaxRows, B - b0));
        a.q = static_cast<const uint16_t*>(q->data) + b0 * Hq * C * D;
        a.k = static_cast<const uint16_t*>(k_pool->data);
        a.v = static_cast<const uint16_t*>(v_pool->data);
        a.page_table = page_table_dev + b0 * max_blocks_per_seq;
        a.out = static_cast<uint16_t*>(out->data) + b0 * Hq * C * D;
        a.Hq = static_cast<int32_t>(Hq);
        a.Hkv = static_cast<int32_t>(Hkv);
        a.C = static_cast<int32_t>(C);
        a.bs = block_size;
        a.maxb = max_blocks_per_seq;
        a.log2bs = 0;
        while ((1 << a.log2bs) < block_size) ++a.log2bs;
        a.row0 = static_cast<int32_t>(b0);
        const float sc = scale > 0 ? scale : 1.0f / std::sqrt(float(D));
        a.scale_log2 = sc * 1.4426950408889634f;
        a.window = left_window;
        for (int i = 0; i < a.rows; ++i) {
            a.p0[i] = p0[b0 + i];
            a.order[i] = static_cast<uint16_t>(i);
        }
        // longest rows first, so that the short ones fill the end of the launch
        std::stable_sort(a.order, a.order + a.rows, [&](uint16_t x, uint16_t y) { return a.p0[x] > a.p0[y]; });
        a.kv_splits = S;
        a.ws_o = ws_o;
        a.ws_ml = ws_ml;
        PKV_HIP(launch_chunk(a, G, s), "chunk attention launch");
        if (S > 1) {
            // the partials of query (row, head, token) sit where the merge
            // expects those of row `row` and "head" head * C + token
            MergeArgs m;
            m.ws_o = ws_o;
            m.ws_ml = ws_ml;
            m.out = a.out;
            m.out_kind = kKvBF16;
            m.Hq = static_cast<int32_t>(Hq * C);
            m.D = kChunkD;
            m.S_max = S;
            m.row0 = 0;
            m.rows = a.rows;
            m.min_splits = 1;
            for (int i = 0; i < a.rows; ++i) m.nsplit[i] = S;
            PKV_HIP(launch_merge(m, s), "chunk attention merge launch");
        }
    }
    return ok();
}

}  // namespace

size_t pkv_chunk_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t C, int32_t num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || C <= 0 || Hq % Hkv != 0 || num_splits < 0 || num_splits > kChunkMaxSplits)
        return 0;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return 0;
    const int64_t rows_max = std::min<int64_t>(B, kMaxRows);
    const int S = num_splits > 0 ? num_splits : chunk_auto_cap(chunk_workgroups(rows_max, Hkv, G, C), device_cus());
    return S > 1 ? ws_bytes_for(rows_max, int64_t(Hq) * C, kChunkD, S) : 0;
}

pkv_status pkv_chunk_attention(const pkv_tensor* q, const pkv_tensor* k_pool,
                               const pkv_tensor* v_pool, const int32_t* page_table_dev,
                               int32_t max_blocks_per_seq, int32_t block_size,
                               const pkv_pool* pool, const int32_t* p0, float scale,
                               int32_t left_window,
                               pkv_tensor* out, void* stream) {
    return chunk_attention_impl(q, k_pool, v_pool, page_table_dev, max_blocks_per_seq, block_size, pool, p0, scale,
                                left_window, out, nullptr, 0, 1, stream);
}

pkv_status pkv_chunk_attention_split(const pkv_tensor* q, const pkv_tensor* k_pool,
                                     const pkv_tensor* v_pool, const int32_t* page_table_dev,
                                     int32_t max_blocks_per_seq, int32_t block_size,
                                     const pkv_pool* pool, const int32_t* p0, float scale,
                                     int32_t left_window, pkv_tensor* out, void* workspace,
                                     size_t workspace_bytes, int32_t num_splits, void* stream) {
    return chunk_attention_impl(q, k_pool, v_pool, page_table_dev, max_blocks_per_seq, block_size, pool, p0, scale,
                                left_window, out, workspace, workspace_bytes, num_splits, stream);
}


// ---------------------------------------------------------------------------
namespace {

struct SamplePlan {
    int32_t chunks;
    int64_t chunk_len;
};

SamplePlan plan_sample(int64_t B, int64_t V) {
    // about 1024 workgroups in total, chunks of at least 4096 logits
    int64_t chunks = std::max<int64_t>(1, ceil_div(1024, std::max<int64_t>(B, 1)));
    chunks = std::min<int64_t>(chunks, std::max<int64_t>(1, ceil_div(V, 4096)));
    int64_t len = ceil_div(ceil_div(V, chunks), 1024) * 1024;
    return {static_cast<int32_t>(ceil_div(V, len)), len};
}

}  // namespace

size_t pkv_sample_workspace_size(int32_t B, int64_t V) {
    if (B <= 0 || V <= 0) return 0;
    const SamplePlan p = plan_sample(B, V);
    const size_t n = size_t(B) * p.chunks;
    return ((n * 8 + 255) & ~size_t(255)) + ((n * 4 + 255) & ~size_t(255));
}

pkv_status pkv_sample(const pkv_tensor* logits, float temperature, uint64_t seed,
                      int64_t* out_ids, void* workspace, size_t workspace_bytes, void* stream) {
    return pkv_sample_dev(logits, temperature, seed, nullptr, out_ids, workspace, workspace_bytes, stream);
}

pkv_status pkv_sample_dev(const pkv_tensor* logits, float temperature, uint64_t seed, const int64_t* step_dev,
                          int64_t* out_ids, void* workspace, size_t workspace_bytes, void* stream) {
    PKV_TRY(check_tensor(logits, "logits", 2, 3));
    const int kind = logits->dtype == PKV_F64 ? kKvF64 : kv_kind_of(logits->dtype);
    if (kind < 0) return fail(PKV_E_DTYPE, "sample: logits must be f32, f64, bf16 or f16");
    if (!(temperature >= 0.0f) || std::isinf(temperature))
        return fail(PKV_E_ARG, "sample: temperature must be finite and >= 0");
    if (!out_ids) return fail(PKV_E_ARG, "sample: null out_ids");
    const int64_t B = logits->shape[0];
    const int64_t S = logits->ndim == 3 ? logits->shape[1] : 1;
    const int64_t V = logits->shape[logits->ndim - 1];
    if (B <= 0 || S <= 0 || V <= 0) return fail(PKV_E_LAYOUT, "sample: empty logits");
    if (V > INT32_MAX) return fail(PKV_E_LAYOUT, "sample: vocabulary too large");
    const size_t need = pkv_sample_workspace_size(static_cast<int32_t>(B), V);
    if (!workspace || workspace_bytes < need)
        return fail(PKV_E_NOMEM, "sample: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    const Span wss = span(workspace, static_cast<int64_t>(need));
    if (overlap(wss, span(logits)) || overlap(wss, span(out_ids, B * 8)) || overlap(span(logits), span(out_ids, B * 8)))
        return fail(PKV_E_ALIAS, "sample: workspace, logits and out_ids must not overlap");
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(PKV_E_ARG, "sample: workspace must be 256-byte aligned");
    const SamplePlan p = plan_sample(B, V);
    SampleArgs a;
    a.row_stride = S * V;
    a.logits = static_cast<const uint8_t*>(logits->data) + (S - 1) * V * dtype_size(logits->dtype);
    a.V = V;
    a.kind = kind;
    a.B = static_cast<int32_t>(B);
    a.chunks = p.chunks;
    a.chunk_len = p.chunk_len;
    a.greedy = temperature == 0.0f;
    a.inv_t = a.greedy ? 0.0f : static_cast<float>(1.0 / static_cast<double>(temperature));
    a.inv_t64 = a.greedy ? 0.0 : 1.0 / static_cast<double>(temperature);
    a.seed = seed;
    const size_t n = size_t(B) * p.chunks;
    a.part_val = static_cast<double*>(workspace);
    a.part_idx = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + ((n * 8 + 255) & ~size_t(255)));
    a.out = out_ids;
    a.step = step_dev;
    if (step_dev && (overlap(span(step_dev, 8), wss) || overlap(span(step_dev, 8), span(out_ids, B * 8))))
        return fail(PKV_E_ALIAS, "sample: the step counter overlaps the workspace or out_ids");
    PKV_HIP(launch_sample(a, static_cast<hipStream_t>(stream)), "sample launch");
    return ok();
}


uint64_t pkv_generate_step_seed(uint64_t seed, int64_t step, int32_t B, int64_t V) {
    return seed + static_cast<uint64_t>(step) * static_cast<uint64_t>(B) * static_cast<uint64_t>(V) *
                      0x9E3779B97F4A7C15ull;
}

pkv_status pkv_generate_finish(const int64_t* sampled, uint8_t* finished, int64_t* tokens,
                               int64_t row_stride, int32_t column, int32_t B,
                               int64_t eos_token_id, int64_t pad_token_id, int64_t* next_ids,
                               int32_t* unfinished, void* stream) {
    if (B < 0) return fail(PKV_E_ARG, "generate_finish: negative batch");
    if (!sampled || !finished || !tokens || !next_ids || !unfinished)
        return fail(PKV_E_ARG, "generate_finish: null pointer");
    if (row_stride <= 0 || column < 0 || column >= row_stride)
        return fail(PKV_E_ARG, "generate_finish: column %d outside [0, %lld)", column, (long long)row_stride);
    const Span ts = span(tokens, int64_t(B) * row_stride * 8);
    if (overlap(ts, span(sampled, int64_t(B) * 8)) || overlap(ts, span(finished, B)) ||
        overlap(ts, span(next_ids, int64_t(B) * 8)) || overlap(ts, span(unfinished, 4)))
        return fail(PKV_E_ALIAS, "generate_finish: tokens overlaps another argument");
    GenerateArgs a;
    a.sampled = sampled;
    a.finished = finished;
    a.tokens = tokens;
    a.next_ids = next_ids;
    a.unfinished = unfinished;
    a.row_stride = row_stride;
    a.eos = eos_token_id;
    a.pad = pad_token_id;
    a.column = column;
    a.B = B;
    a.has_eos = eos_token_id >= 0;
    PKV_HIP(launch_generate_finish(a, static_cast<hipStream_t>(stream)), "generate_finish launch");
    return ok();
}
}  // extern "C"
