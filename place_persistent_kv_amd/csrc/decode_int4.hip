// Paged decode attention over INT4 blockwise-affine K/V pages (gfx950).
//
// Format -- "Custom, quantized, and persistent values", sections "Struct
// types and byte-encodable layouts" and "Quantization examples": UINT4 codes,
// two per byte with the even element in the low nibble, decoded as
// (code - zero_point) * scale; here every 32-element block of a token row
// has its own fp16 (scale, zero_point).  "Persistent input/output feedback",
// "Optional heterogeneous paged KV": affine pages are decoded inside the
// attention loop, never materialised as a dense copy.
//
// Per (page, kv head) a token row is 64 bytes of codes + 16 bytes of
// parameters.  Eight lanes cover one token: lane j holds dims 16j..16j+15
// (8 code bytes, half of block j/2).  The dequantisation is folded into the
// dot products instead of being applied per element:
//   q . k = sum_blocks s_b * (sum_d q_d c_d - z_b * sum_d q_d)
//   o    += p * s_b * c - p * s_b * z_b   (the second term kept per block)
// so the codes are only converted to float (v_cvt_f32_ubyte) and fed to FMAs.
// The split / merge structure is that of the bf16 fast kernel.

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kWaves4 = 4;
constexpr int kD4 = 128;
constexpr float kLazy4 = 8.0f;

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// 8 code bytes -> 16 floats in element order (even element = low nibble)
__device__ __forceinline__ void unpack16(uint2 w, float c[16]) {
    const uint32_t lo0 = w.x & 0x0F0F0F0Fu, hi0 = (w.x >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo1 = w.y & 0x0F0F0F0Fu, hi1 = (w.y >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c[2 * k] = static_cast<float>((lo0 >> (8 * k)) & 0xFFu);
        c[2 * k + 1] = static_cast<float>((hi0 >> (8 * k)) & 0xFFu);
        c[8 + 2 * k] = static_cast<float>((lo1 >> (8 * k)) & 0xFFu);
        c[8 + 2 * k + 1] = static_cast<float>((hi1 >> (8 * k)) & 0xFFu);
    }
}

template <int G>
__global__ __launch_bounds__(256) void decode_int4_kernel(Int4DecodeArgs a) {
    __shared__ float s_o[kWaves4][G][kD4];
    __shared__ float s_ml[kWaves4][G][2];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 3;
    const int j = lane & 7;        // dims 16j .. 16j+15, block j/2

    const int work = blockIdx.x;
    const int kvh = work % a.Hkv;
    const int r = work / a.Hkv;
    const int b = find_row(a.split_begin, a.rows, r);
    const int split = r - a.split_begin[b];
    const int nsplit = a.split_begin[b + 1] - a.split_begin[b];
    const int L = a.len[b];
    const int t0 = split * a.tps;
    const int t1 = min(L, t0 + a.tps);
    const int quarter = a.tps / kWaves4;
    const int wbeg = t0 + wave * quarter;
    const int wend = min(t1, wbeg + quarter);
    const int32_t* __restrict__ pt = a.page_table + int64_t(b) * a.maxb;

    float q[G][16], qsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float* Q = a.q + (int64_t(b) * a.Hq + kvh * G + g) * kD4 + j * 16;
        qsum[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            const float4 x = *reinterpret_cast<const float4*>(Q + e);
            q[g][e] = x.x;
            q[g][e + 1] = x.y;
            q[g][e + 2] = x.z;
            q[g][e + 3] = x.w;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) qsum[g] += q[g][e];
    }

    float m[G], l[G], o[G][16], corr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -FLT_MAX;
        l[g] = 0.0f;
        corr[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[g][d] = 0.0f;
    }

    // row index (page, kvh, slot) of token t, clamped to [ts, t1)
    auto row_of = [&](int ts, int t) -> int64_t {
        const int tc = min(t, t1 - 1);
        const int page = pt[ts / a.bs];
        return (int64_t(page) * a.Hkv + kvh) * a.bs + (tc % a.bs);
    };

    struct Buf {
        uint2 kc0, kc1, vc0, vc1;
        uint32_t kp0, kp1, vp0, vp1;
    };
    auto load = [&](Buf& u, int ts) {
        const int64_t r0 = row_of(ts, ts + grp);
        const int64_t r1 = row_of(ts, ts + 8 + grp);
        u.kc0 = *reinterpret_cast<const uint2*>(a.kc + r0 * 64 + j * 8);
        u.kc1 = *reinterpret_cast<const uint2*>(a.kc + r1 * 64 + j * 8);
        u.vc0 = *reinterpret_cast<const uint2*>(a.vc + r0 * 64 + j * 8);
        u.vc1 = *reinterpret_cast<const uint2*>(a.vc + r1 * 64 + j * 8);
        u.kp0 = *reinterpret_cast<const uint32_t*>(a.kp + (r0 * 4 + (j >> 1)) * 2);
        u.kp1 = *reinterpret_cast<const uint32_t*>(a.kp + (r1 * 4 + (j >> 1)) * 2);
        u.vp0 = *reinterpret_cast<const uint32_t*>(a.vp + (r0 * 4 + (j >> 1)) * 2);
        u.vp1 = *reinterpret_cast<const uint32_t*>(a.vp + (r1 * 4 + (j >> 1)) * 2);
    };

    auto score = [&](uint2 codes, uint32_t par, float s[G]) {
        float c[16];
        unpack16(codes, c);
        const float sc = h2f(par & 0xFFFFu), zp = h2f(par >> 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc = fmaf(q[g][e], c[e], acc);
            s[g] = group8_sum(sc * fmaf(-zp, qsum[g], acc)) * a.scale_log2;
        }
    };

    auto compute = [&](const Buf& u, int ts) {
        const bool live0 = ts + grp < t1;
        const bool live1 = ts + 8 + grp < t1;
        float s0[G], s1[G];
        score(u.kc0, u.kp0, s0);
        score(u.kc1, u.kp1, s1);
        float c0[16], c1[16];
        unpack16(u.vc0, c0);
        unpack16(u.vc1, c1);
        const float vs0 = h2f(u.vp0 & 0xFFFFu), vz0 = h2f(u.vp0 >> 16);
        const float vs1 = h2f(u.vp1 & 0xFFFFu), vz1 = h2f(u.vp1 >> 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            s0[g] = live0 ? s0[g] : -INFINITY;
            s1[g] = live1 ? s1[g] : -INFINITY;
            const float mx = fmaxf(s0[g], s1[g]);
            if (mx > m[g] + kLazy4) {
                const float cf = exp2_fast(m[g] - mx);
                l[g] *= cf;
                corr[g] *= cf;
#pragma unroll
                for (int d = 0; d < 16; ++d) o[g][d] *= cf;
                m[g] = mx;
            }
            const float p0 = exp2_fast(s0[g] - m[g]);
            const float p1 = exp2_fast(s1[g] - m[g]);
            l[g] += p0 + p1;
            const float w0 = p0 * vs0, w1 = p1 * vs1;
            corr[g] = fmaf(w1, vz1, fmaf(w0, vz0, corr[g]));
#pragma unroll
            for (int d = 0; d < 16; ++d) o[g][d] = fmaf(w1, c1[d], fmaf(w0, c0[d], o[g][d]));
        }
    };

    if (wbeg < wend) {
        Buf A, Bf;
        load(A, wbeg);
        for (int ts = wbeg;; ts += 2 * kSlabTokens) {
            const bool has1 = ts + kSlabTokens < wend;
            if (has1) load(Bf, ts + kSlabTokens);
            compute(A, ts);
            if (!has1) break;
            const bool has2 = ts + 2 * kSlabTokens < wend;
            if (has2) load(A, ts + 2 * kSlabTokens);
            compute(Bf, ts + kSlabTokens);
            if (!has2) break;
        }
    }

    // subtract the zero-point term, then merge the eight token groups
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < 16; ++d) o[g][d] -= corr[g];
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], off);
            const float lo = __shfl_xor(l[g], off);
            const float mn = fmaxf(m[g], mo);
            const float cs = exp2_fast(m[g] - mn);
            const float co = exp2_fast(mo - mn);
            l[g] = l[g] * cs + lo * co;
#pragma unroll
            for (int d = 0; d < 16; ++d) o[g][d] = o[g][d] * cs + __shfl_xor(o[g][d], off) * co;
            m[g] = mn;
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int d = 0; d < 16; ++d) s_o[wave][g][j * 16 + d] = o[g][d];
            if (j == 0) {
                s_ml[wave][g][0] = m[g];
                s_ml[wave][g][1] = l[g];
            }
        }
    }
    __syncthreads();

    for (int e = threadIdx.x; e < G * kD4; e += 256) {
        const int g = e / kD4;
        const int d = e % kD4;
        float mn = -FLT_MAX;
#pragma unroll
        for (int w = 0; w < kWaves4; ++w) mn = fmaxf(mn, s_ml[w][g][0]);
        float ls = 0.0f, os = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves4; ++w) {
            const float c = exp2_fast(s_ml[w][g][0] - mn);
            ls += s_ml[w][g][1] * c;
            os += s_o[w][g][d] * c;
        }
        const int64_t bh = int64_t(b) * a.Hq + kvh * G + g;
        if (nsplit == 1) {
            a.out[bh * kD4 + d] = os / ls;
        } else {
            const int64_t slot = bh * a.S_max + split;
            a.ws_o[slot * kD4 + d] = os;
            if (d == 0) {
                a.ws_ml[slot * 2 + 0] = mn;
                a.ws_ml[slot * 2 + 1] = ls;
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_int4(const Int4DecodeArgs& a, int G, int total_work, hipStream_t s) {
    if (total_work <= 0) return hipSuccess;
    const dim3 grid(total_work), block(256);
    switch (G) {
        case 1: hipLaunchKernelGGL(decode_int4_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(decode_int4_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(decode_int4_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(decode_int4_kernel<8>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
