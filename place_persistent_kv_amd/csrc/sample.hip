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
// to the lowest index.  Float64 logits are compared as float64 values (greedy)
// and scaled in float64 (y = x * (1 / T), T the float32 temperature widened).
//
// Non-finite scores follow numpy's argmax: NaN ranks above every number (the
// first NaN of a row wins), and a row whose scores are all -inf yields its
// first index, so every row gets an index inside the vocabulary.
//
// The pass is one read of the logits: each workgroup reduces a vocabulary
// chunk of one row to (best score, index); a second small kernel reduces the
// chunks of each row.  Partial scores are stored as float64 (exact for the
// float32 scores).

#include "pkv_internal.h"

#include <float.h>
#include <stdint.h>

#include <type_traits>

namespace pkv {
namespace {

constexpr int kSampleThreads = 256;

// Score type: float64 for float64 logits, float32 otherwise.
template <int KIND>
using score_t = typename std::conditional<KIND == kKvF64, double, float>::type;

template <int KIND>
__device__ __forceinline__ score_t<KIND> logit_at(const void* p, int64_t i) {
    if constexpr (KIND == kKvF32) return static_cast<const float*>(p)[i];
    else if constexpr (KIND == kKvF64) return static_cast<const double*>(p)[i];
    else if constexpr (KIND == kKvBF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
    else return static_cast<float>(static_cast<const _Float16*>(p)[i]);
}

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// element e (a constant) of a 16-byte vector of logits
template <int KIND>
__device__ __forceinline__ score_t<KIND> logit_of(u32x4v_t w, int e) {
    if constexpr (KIND == kKvF32) return __uint_as_float(w[e]);
    if constexpr (KIND == kKvF64)
        return __builtin_bit_cast(double, (uint64_t(w[2 * e + 1]) << 32) | w[2 * e]);
    const uint32_t h = (e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xFFFFu);
    if constexpr (KIND == kKvBF16) return __uint_as_float(h << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Score order: NaN above every number, otherwise numeric.  above(s, b): s
// ranks strictly above b.
// (bitwise, not short-circuit: two compares and one scalar AND, no branch)
template <typename T>
__device__ __forceinline__ bool above(T s, T b) {
    return !(s <= b) & (b == b);
}
template <typename T>
__device__ __forceinline__ bool same_rank(T s, T b) {
    return (s == b) | ((s != s) & (b != b));
}

// (score, index) order: higher-ranked score wins, equal ranks -> lower index
template <typename T>
__device__ __forceinline__ bool better(T s, int32_t i, T bs, int32_t bi) {
    return above(s, bs) || (same_rank(s, bs) && i < bi);
}

template <typename T>
__device__ __forceinline__ void wave_argmax(T& s, int32_t& i) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const T so = __shfl_xor(s, off);
        const int32_t io = __shfl_xor(i, off);
        if (better(so, io, s, i)) {
            s = so;
            i = io;
        }
    }
}

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr float kLn2 = 0.69314718055994531f;

// Gumbel term -ln(-ln u) of the SplitMix64 state (seed + k * gamma) `state`.
// Only the top 24 bits of the output are used.  The logarithms are the
// hardware base-2 ones (v_log_f32, about 1 ulp), scaled by ln 2.
__device__ __forceinline__ float gumbel_term(uint64_t state) {
#pragma clang fp contract(off)
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    const uint32_t top = static_cast<uint32_t>((z ^ (z >> 31)) >> 40);
    const float u = static_cast<float>(top | 1u) * 0x1p-24f;
    const float e = -__builtin_amdgcn_logf(u) * kLn2;        // -ln u, an Exp(1) draw
    return -__builtin_amdgcn_logf(e) * kLn2;
}

// Perturbed score y - ln(-ln u): y = fl32(x * invT) for float32 scores (a
// rounded product, no contraction), y = fl64(x * invT64) for float64 logits.
__device__ __forceinline__ float gumbel_score(float x, const SampleArgs& a, uint64_t state) {
#pragma clang fp contract(off)
    const float y = x * a.inv_t;
    return y + gumbel_term(state);
}
__device__ __forceinline__ double gumbel_score(double x, const SampleArgs& a, uint64_t state) {
#pragma clang fp contract(off)
    const double y = x * a.inv_t64;
    return y + static_cast<double>(gumbel_term(state));
}

// One workgroup reduces one vocabulary chunk of one row to (best score,
// index).  VEC: the row is 16-byte aligned and the chunk is read in 16-byte
// vectors, four per thread in flight; the ragged end of the row is read per
// element.
template <int KIND, bool GREEDY, bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sample_chunk_kernel(SampleArgs a) {
    using S = score_t<KIND>;
    __shared__ S s_val[kSampleThreads / 64];
    __shared__ int32_t s_idx[kSampleThreads / 64];
    constexpr int W = KIND == kKvF64 ? 2 : KIND == kKvF32 ? 4 : 8;   // logits per 16-byte vector
    const int b = blockIdx.y;
    const int c = blockIdx.x;
    const int64_t beg = int64_t(c) * a.chunk_len;
    const int64_t end = min(a.V, beg + a.chunk_len);
    const void* row = static_cast<const uint8_t*>(a.logits) + b * a.row_stride * (16 / W);
    const int64_t nvec = VEC ? (end - beg) / W : 0;          // whole vectors in the chunk
    const int64_t tail = beg + nvec * W;                      // first element read singly
    // A thread visits its logits in increasing index order.  It starts from
    // (-inf, its first index), so an all -inf run keeps that lowest index and
    // a later logit wins only by ranking strictly above the best so far.
    const int64_t first = threadIdx.x < nvec ? beg + int64_t(threadIdx.x) * W
                        : (tail + threadIdx.x < end ? tail + threadIdx.x : int64_t(INT32_MAX));
    S best = -INFINITY;
    int32_t bidx = static_cast<int32_t>(first);
    // state of logit v: seed + (b * V + v + 1) * gamma; with a device step
    // counter the seed is that of iteration *step (seed + step * B * V * gamma)
    uint64_t seed = a.seed;
    if (a.step != nullptr) seed += uint64_t(*a.step) * uint64_t(a.B) * uint64_t(a.V) * kGamma;
    const uint64_t state0 = seed + (uint64_t(b) * uint64_t(a.V) + 1ull) * kGamma;
    auto consider = [&](S x, int64_t v, uint64_t state) {
        const S s = GREEDY ? x : gumbel_score(x, a, state);
        const bool take = above(s, best);
        best = take ? s : best;
        bidx = take ? static_cast<int32_t>(v) : bidx;
    };
    if constexpr (VEC) {
        constexpr int U = 4;                                  // vectors in flight per thread
        const u32x4v_t* vp = reinterpret_cast<const u32x4v_t*>(static_cast<const uint8_t*>(row) + beg * (16 / W));
        int64_t i = threadIdx.x;
        for (; i + (U - 1) * kSampleThreads < nvec; i += U * kSampleThreads) {
            u32x4v_t w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = vp[i + u * kSampleThreads];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v0 = beg + (i + u * kSampleThreads) * W;
                const uint64_t st = state0 + uint64_t(v0) * kGamma;
#pragma unroll
                for (int e = 0; e < W; ++e) consider(logit_of<KIND>(w[u], e), v0 + e, st + uint64_t(e) * kGamma);
            }
        }
        for (; i < nvec; i += kSampleThreads) {
            const u32x4v_t w0 = vp[i];
            const int64_t v0 = beg + i * W;
            const uint64_t st = state0 + uint64_t(v0) * kGamma;
#pragma unroll
            for (int e = 0; e < W; ++e) consider(logit_of<KIND>(w0, e), v0 + e, st + uint64_t(e) * kGamma);
        }
    }
    for (int64_t v = tail + threadIdx.x; v < end; v += kSampleThreads)
        consider(logit_at<KIND>(row, v), v, state0 + uint64_t(v) * kGamma);

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
        a.part_val[int64_t(b) * a.chunks + c] = static_cast<double>(best);
        a.part_idx[int64_t(b) * a.chunks + c] = bidx;
    }
}

// Every chunk holds at least one logit, so the reduction of a row ends on an
// index inside the vocabulary.
__global__ __launch_bounds__(64) void sample_final_kernel(SampleArgs a) {
    const int b = blockIdx.x;
    double best = -INFINITY;
    int32_t bidx = INT32_MAX;
    for (int c = threadIdx.x; c < a.chunks; c += 64) {
        const double s = a.part_val[int64_t(b) * a.chunks + c];
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
    // 16-byte vectors when every row start is 16-byte aligned
    const int esize = a.kind == kKvF64 ? 8 : a.kind == kKvF32 ? 4 : 2;
    const bool vec = reinterpret_cast<uintptr_t>(a.logits) % 16 == 0 && (a.row_stride * esize) % 16 == 0 &&
                     (a.chunk_len * esize) % 16 == 0;
#define PKV_SAMPLE(K, V)                                                                           \
    if (a.kind == K && vec == V) {                                                                 \
        if (a.greedy) hipLaunchKernelGGL((sample_chunk_kernel<K, true, V>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((sample_chunk_kernel<K, false, V>), grid, block, 0, s, a);        \
    }
    PKV_SAMPLE(kKvF32, true)
    PKV_SAMPLE(kKvBF16, true)
    PKV_SAMPLE(kKvF16, true)
    PKV_SAMPLE(kKvF64, true)
    PKV_SAMPLE(kKvF32, false)
    PKV_SAMPLE(kKvBF16, false)
    PKV_SAMPLE(kKvF16, false)
    PKV_SAMPLE(kKvF64, false)
#undef PKV_SAMPLE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_final_kernel, dim3(a.B), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv
