// Device helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include "pkv_internal.h"

#include <float.h>

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a half-row; every lane of the group gets the total.
__device__ __forceinline__ float group8_sum(float x) {
    x += dpp<0x141>(x);  // row_half_mirror: lane i <- lane 7 - i
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    return x;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: K/V rows are streamed once per call, so
// they should not displace reusable lines in L2 / MALL.
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// largest b with split_begin[b] <= r (split_begin is non-decreasing, split_begin[rows] > r)
__device__ __forceinline__ int find_row(const int32_t* split_begin, int rows, int r) {
    int lo = 0, hi = rows;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (split_begin[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Row and split of work item r of a launch over host lengths.  The splits
// that hold a whole tps tokens come first, row by row (full_begin: prefix
// sums of their per-row counts, full_begin[rows] their total), then each
// row's shorter last split, longest first (tail_row), so that the largest
// workgroups are dispatched first and the short ones fill the end of the
// grid.  A row with r in its full range has full_begin[b] <= r <
// full_begin[b + 1]; its last split is split number full_begin[b + 1] -
// full_begin[b].
__device__ __forceinline__ void split_item(const int32_t* full_begin, const uint16_t* tail_row, int rows, int r,
                                           int& b, int& split) {
    const int n_full = full_begin[rows];
    if (r < n_full) {
        b = find_row(full_begin, rows, r);
        split = r - full_begin[b];
    } else {
        b = tail_row[r - n_full];
        split = full_begin[b + 1] - full_begin[b];
    }
}

}  // namespace
}  // namespace pkv
