// In-place cache updates for gfx950: contiguous rows, paged rows, INT4
// quantise-on-append, page-table writes and the paged gather export.
//
// "Mutable execution cache", sections "Value model" and "Model example":
// CacheUpdate writes only the rows starting at `position`; the output is the
// input storage.  Section "Heterogeneous paged cache": PagedCacheUpdate
// writes existing pages in place.  All of these are byte copies (or a
// per-element quantisation) with integer address arithmetic: they are
// bound by HBM writes and use 16-byte vector accesses where the row size and
// alignment allow.

#include "pkv_internal.h"

#include <algorithm>

namespace pkv {
namespace {

constexpr int kThreads = 256;

// PAIR: indices [total / 2, total) copy the second (src2, dst2) pair
template <typename V, bool PAIR>
__global__ __launch_bounds__(kThreads) void copy_rows_kernel(CopyRowsArgs a, int64_t total) {
    // thread i copies vector c of row-slab (b, h): the n rows written for (b, h)
    // are contiguous both in `values` and at `position` in the cache.
    const int64_t vec_per_bh = a.n * a.row_bytes / int64_t(sizeof(V));
    const int64_t per_pair = PAIR ? total / 2 : total;
    for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < total;
         j += int64_t(gridDim.x) * kThreads) {
        const bool second = PAIR && j >= per_pair;
        const int64_t i = second ? j - per_pair : j;
        const int64_t bh = i / vec_per_bh;
        const int64_t c = i - bh * vec_per_bh;
        const int32_t b = static_cast<int32_t>(bh / a.H);
        const int32_t h = static_cast<int32_t>(bh - int64_t(b) * a.H);
        const V* src = reinterpret_cast<const V*>((second ? a.src2 : a.src) + bh * a.n * a.row_bytes);
        V* dst = reinterpret_cast<V*>((second ? a.dst2 : a.dst) +
                                      ((int64_t(b) * a.H + h) * a.cap + a.pos[b]) * a.row_bytes);
        dst[c] = src[c];
    }
}

// PAIR: indices [total / 2, total) copy the second (src2, pool2) pair
template <typename V, bool PAIR>
__global__ __launch_bounds__(kThreads) void paged_copy_kernel(PagedCopyArgs a, int64_t total) {
    const int64_t vec_per_row = a.row_bytes / int64_t(sizeof(V));
    const int64_t per_pair = PAIR ? total / 2 : total;
    for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < total;
         j += int64_t(gridDim.x) * kThreads) {
        const bool second = PAIR && j >= per_pair;
        const int64_t i = second ? j - per_pair : j;
        const int64_t r = i / vec_per_row;          // source row index (b, h, t)
        const int64_t c = i - r * vec_per_row;
        const int32_t t = static_cast<int32_t>(r % a.n);
        const int64_t bh = r / a.n;
        const int32_t h = static_cast<int32_t>(bh % a.H);
        const int32_t b = static_cast<int32_t>(bh / a.H);
        const int32_t p = a.pos[b] + t;
        const int32_t page = a.page_table[int64_t(a.row0 + b) * a.maxb + p / a.bs];
        const int32_t slot = p % a.bs;
        const V* src = reinterpret_cast<const V*>((second ? a.src2 : a.src) + r * a.row_bytes);
        V* dst = reinterpret_cast<V*>((second ? a.pool2 : a.pool) + ((int64_t(page) * a.H + h) * a.bs + slot) * a.row_bytes);
        dst[c] = src[c];
    }
}

// K and V rows at positions held in device memory.  Every workgroup first
// checks every row of the call (position in range; paged: the pages written
// hold ids inside the pool), so either all rows are written or none; a
// failing check sets *status.  Then thread i copies 16-byte vector c of row
// (tensor, b, h, t).
__global__ __launch_bounds__(kThreads) void kv_append_dev_kernel(KvAppendDevArgs a, int64_t total) {
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int b = threadIdx.x; b < a.B; b += kThreads) {
        const int32_t p = a.pos[b];
        if (p < 0 || p > a.cap - a.n) {
            bad = 2;                                  // PKV_E_CAPACITY
        } else if (a.page_table != nullptr && a.n > 0) {
            for (int32_t pg = p / a.bs; pg <= (p + a.n - 1) / a.bs; ++pg) {
                const int32_t id = a.page_table[int64_t(b) * a.maxb + pg];
                if (uint32_t(id) >= uint32_t(a.nb)) bad = 6;   // PKV_E_PAGE
            }
        }
    }
    if (bad) atomicMax(&s_bad, bad);
    __syncthreads();
    if (s_bad) {
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.status = s_bad;
        return;
    }
    const int64_t vec_per_row = a.row_bytes / 16;
    const int64_t rows_per_tensor = int64_t(a.B) * a.H * a.n;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kThreads) {
        const int64_t r = i / vec_per_row;            // (tensor, b, h, t)
        const int64_t c = i - r * vec_per_row;
        const int which = r >= rows_per_tensor;
        const int64_t rr = r - which * rows_per_tensor;
        const int32_t t = static_cast<int32_t>(rr % a.n);
        const int64_t bh = rr / a.n;
        const int32_t h = static_cast<int32_t>(bh % a.H);
        const int32_t b = static_cast<int32_t>(bh / a.H);
        const int32_t p = a.pos[b] + t;
        int64_t dst_row;
        if (a.page_table != nullptr) {
            const int32_t page = a.page_table[int64_t(b) * a.maxb + p / a.bs];
            dst_row = (int64_t(page) * a.H + h) * a.bs + p % a.bs;
        } else {
            dst_row = (int64_t(b) * a.H + h) * a.cap + p;
        }
        const uint4* src = reinterpret_cast<const uint4*>(a.src[which] + rr * a.row_bytes);
        uint4* dst = reinterpret_cast<uint4*>(a.dst[which] + dst_row * a.row_bytes);
        dst[c] = src[c];
    }
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// One thread per 8 elements (one code word) of one written row: 8 codes in
// one dword, element 2k in the low nibble of byte k; the thread of a block's
// first word also writes the block's (scale, zero point) slot.  Eight
// divisions per thread keep the latency of a short call low.
__global__ __launch_bounds__(kThreads) void paged_int4_kernel(PagedInt4Args a, int64_t total) {
    const int nword = a.D / 8;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kThreads) {
        const int32_t w = static_cast<int32_t>(i % nword);
        const int64_t r = i / nword;                // source row (b, h, t)
        const int32_t t = static_cast<int32_t>(r % a.n);
        const int64_t bh = r / a.n;
        const int32_t h = static_cast<int32_t>(bh % a.H);
        const int32_t b = static_cast<int32_t>(bh / a.H);
        const int32_t p = a.pos[b] + t;
        const int32_t page = a.page_table[int64_t(a.row0 + b) * a.maxb + p / a.bs];
        const int64_t row = (int64_t(page) * a.H + h) * a.bs + p % a.bs;

        uint32_t packed = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t src_idx = r * a.D + w * 8 + e;
            const float x = a.src_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.src)[src_idx])
                                       : static_cast<const float*>(a.src)[src_idx];
            // correctly rounded float32 divide, round half to even, saturate
            float c = rintf(x / a.scale) + a.zero_point;
            c = fminf(fmaxf(c, 0.0f), 15.0f);
            packed |= uint32_t(c) << (4 * e);
        }
        *reinterpret_cast<uint32_t*>(a.codes + row * (a.D / 2) + w * 4) = packed;
        if (w % 4 == 0)
            *reinterpret_cast<uint32_t*>(a.params + (row * (a.D / 32) + w / 4) * 2) =
                uint32_t(a.scale_bits) | (uint32_t(a.zp_bits) << 16);
    }
}

__global__ void table_write_kernel(TableWriteArgs a) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < a.count) a.table[a.index[i]] = a.value[i];
}

template <typename V>
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a, int64_t total) {
    const int64_t vec_per_row = a.row_bytes / int64_t(sizeof(V));
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kThreads) {
        const int64_t r = i / vec_per_row;          // output row (h, p)
        const int64_t c = i - r * vec_per_row;
        const int32_t p = static_cast<int32_t>(r % a.length);
        const int32_t h = static_cast<int32_t>(r / a.length);
        const int32_t page = a.table_row[p / a.bs];
        const V* src = reinterpret_cast<const V*>(a.pool + ((int64_t(page) * a.H + h) * a.bs + p % a.bs) * a.row_bytes);
        reinterpret_cast<V*>(a.out + r * a.row_bytes)[c] = src[c];
    }
}

int vec_bytes(int64_t row_bytes, const void* p0, const void* p1) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(p0) | reinterpret_cast<uintptr_t>(p1);
    if (row_bytes % 16 == 0 && al % 16 == 0) return 16;
    if (row_bytes % 4 == 0 && al % 4 == 0) return 4;
    return 1;
}

dim3 grid_for(int64_t total) {
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
    if (blocks < 1) blocks = 1;
    return dim3(static_cast<unsigned>(blocks));
}

}  // namespace

hipError_t launch_kv_append_dev(const KvAppendDevArgs& a, hipStream_t s) {
    const int64_t total = 2 * int64_t(a.B) * a.H * a.n * (a.row_bytes / 16);
    if (total <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(kv_append_dev_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a, total);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsArgs& a, hipStream_t s) {
    const bool pair = a.src2 != nullptr;
    int vb = vec_bytes(a.row_bytes, a.src, a.dst);
    if (pair) vb = std::min(vb, vec_bytes(a.row_bytes, a.src2, a.dst2));
    const int64_t total = (pair ? 2 : 1) * (int64_t(a.rows) * a.H * a.n * a.row_bytes / vb);
    if (total == 0) return hipSuccess;
#define PKV_COPY_ROWS(V)                                                                            \
    if (pair) hipLaunchKernelGGL((copy_rows_kernel<V, true>), grid_for(total), dim3(kThreads), 0, s, a, total); \
    else hipLaunchKernelGGL((copy_rows_kernel<V, false>), grid_for(total), dim3(kThreads), 0, s, a, total);
    if (vb == 16) { PKV_COPY_ROWS(uint4) }
    else if (vb == 4) { PKV_COPY_ROWS(uint32_t) }
    else { PKV_COPY_ROWS(uint8_t) }
#undef PKV_COPY_ROWS
    return hipGetLastError();
}

hipError_t launch_paged_copy(const PagedCopyArgs& a, hipStream_t s) {
    const bool pair = a.src2 != nullptr;
    int vb = vec_bytes(a.row_bytes, a.src, a.pool);
    if (pair) vb = std::min(vb, vec_bytes(a.row_bytes, a.src2, a.pool2));
    const int64_t total = (pair ? 2 : 1) * (int64_t(a.rows) * a.H * a.n * a.row_bytes / vb);
    if (total == 0) return hipSuccess;
#define PKV_PAGED_COPY(V)                                                                           \
    if (pair) hipLaunchKernelGGL((paged_copy_kernel<V, true>), grid_for(total), dim3(kThreads), 0, s, a, total); \
    else hipLaunchKernelGGL((paged_copy_kernel<V, false>), grid_for(total), dim3(kThreads), 0, s, a, total);
    if (vb == 16) { PKV_PAGED_COPY(uint4) }
    else if (vb == 4) { PKV_PAGED_COPY(uint32_t) }
    else { PKV_PAGED_COPY(uint8_t) }
#undef PKV_PAGED_COPY
    return hipGetLastError();
}

hipError_t launch_paged_int4_append(const PagedInt4Args& a, hipStream_t s) {
    const int64_t total = int64_t(a.rows) * a.H * a.n * (a.D / 8);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(paged_int4_kernel, grid_for(total), dim3(kThreads), 0, s, a, total);
    return hipGetLastError();
}

hipError_t launch_table_write(const TableWriteArgs& a, hipStream_t s) {
    if (a.count <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_write_kernel, dim3((a.count + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
    const int vb = vec_bytes(a.row_bytes, a.pool, a.out);
    const int64_t total = int64_t(a.H) * a.length * a.row_bytes / vb;
    if (total == 0) return hipSuccess;
    if (vb == 16) hipLaunchKernelGGL(gather_kernel<uint4>, grid_for(total), dim3(kThreads), 0, s, a, total);
    else if (vb == 4) hipLaunchKernelGGL(gather_kernel<uint32_t>, grid_for(total), dim3(kThreads), 0, s, a, total);
    else hipLaunchKernelGGL(gather_kernel<uint8_t>, grid_for(total), dim3(kThreads), 0, s, a, total);
    return hipGetLastError();
}

}  // namespace pkv
