// Greedy and seeded temperature sampling of final logits (gfx950).
//
// "Persistent input/output feedback", section "Autoregressive generation":
// temperature 0 decodes greedily; a positive temperature samples
// softmax(logits / temperature); a seed makes the draw repeatable.
//
// A temperature draw is the Gumbel-max choice
//     argmax_v  fl32(x_v * invT) - log(-log u_v)
// which has exactly the law softmax(x / T).  u_v comes from output number
// k = b * V + v + 1 of SplitMix64 seeded with `seed` (Steele, Lea and Flood,
// OOPSLA 2014): state = seed + k * 0x9E3779B97F4A7C15, then the SplitMix64
// finaliser; u = ((h >> 40) | 1) * 2^-24 is exact in float32.  Greedy ties go
// to the lowest index.  The pass is one read of the logits: each workgroup
// reduces a vocabulary chunk of one row to (best score, index); a second
// small kernel reduces the chunks of each row.

#include "pkv_internal.h"

#include <float.h>

namespace pkv {
namespace {

constexpr int kSampleThreads = 256;

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t k) {
    uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

template <int KIND>
__device__ __forceinline__ float logit_at(const void* p, int64_t i) {
    if constexpr (KIND == kKvF32) return static_cast<const float*>(p)[i];
    else if constexpr (KIND == kKvBF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
    else return static_cast<float>(static_cast<const _Float16*>(p)[i]);
}

// (score, index) order: larger score wins, equal scores -> lower index
__device__ __forceinline__ bool better(float s, int32_t i, float bs, int32_t bi) {
    return s > bs || (s == bs && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& s, int32_t& i) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float so = __shfl_xor(s, off);
        const int32_t io = __shfl_xor(i, off);
        if (better(so, io, s, i)) {
            s = so;
            i = io;
        }
    }
}

template <int KIND, bool GREEDY>
__global__ __launch_bounds__(kSampleThreads) void sample_chunk_kernel(SampleArgs a) {
#pragma clang fp contract(off)
    __shared__ float s_val[kSampleThreads / 64];
    __shared__ int32_t s_idx[kSampleThreads / 64];
    const int b = blockIdx.y;
    const int c = blockIdx.x;
    const int64_t beg = int64_t(c) * a.chunk_len;
    const int64_t end = min(a.V, beg + a.chunk_len);
    const void* row = KIND == kKvF32 ? static_cast<const void*>(static_cast<const float*>(a.logits) + b * a.row_stride)
                                     : static_cast<const void*>(static_cast<const uint16_t*>(a.logits) + b * a.row_stride);
    float best = -INFINITY;
    int32_t bidx = INT32_MAX;
    const uint64_t kbase = uint64_t(b) * uint64_t(a.V) + 1ull;
    for (int64_t v = beg + threadIdx.x; v < end; v += kSampleThreads) {
        const float x = logit_at<KIND>(row, v);
        float s;
        if constexpr (GREEDY) {
            s = x;
        } else {
            const uint64_t h = splitmix64(a.seed, kbase + uint64_t(v));
            const float u = static_cast<float>(static_cast<uint32_t>((h >> 40) | 1ull)) * 0x1p-24f;
            const float y = x * a.inv_t;               // rounded product (no contraction here)
            s = y - logf(-logf(u));
        }
        if (better(s, static_cast<int32_t>(v), best, bidx)) {
            best = s;
            bidx = static_cast<int32_t>(v);
        }
    }
    wave_argmax(best, bidx);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_val[w] = best;
        s_idx[w] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kSampleThreads / 64; ++k)
            if (better(s_val[k], s_idx[k], best, bidx)) {
                best = s_val[k];
                bidx = s_idx[k];
            }
        a.part_val[int64_t(b) * a.chunks + c] = best;
        a.part_idx[int64_t(b) * a.chunks + c] = bidx;
    }
}

__global__ __launch_bounds__(64) void sample_final_kernel(SampleArgs a) {
    const int b = blockIdx.x;
    float best = -INFINITY;
    int32_t bidx = INT32_MAX;
    for (int c = threadIdx.x; c < a.chunks; c += 64) {
        const float s = a.part_val[int64_t(b) * a.chunks + c];
        const int32_t i = a.part_idx[int64_t(b) * a.chunks + c];
        if (better(s, i, best, bidx)) {
            best = s;
            bidx = i;
        }
    }
    wave_argmax(best, bidx);
    if (threadIdx.x == 0) a.out[b] = bidx;
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    const dim3 grid(a.chunks, a.B), block(kSampleThreads);
#define PKV_SAMPLE(K)                                                                         \
    if (a.kind == K) {                                                                        \
        if (a.greedy) hipLaunchKernelGGL((sample_chunk_kernel<K, true>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((sample_chunk_kernel<K, false>), grid, block, 0, s, a);        \
    }
    PKV_SAMPLE(kKvF32)
    PKV_SAMPLE(kKvBF16)
    PKV_SAMPLE(kKvF16)
#undef PKV_SAMPLE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_final_kernel, dim3(a.B), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv
