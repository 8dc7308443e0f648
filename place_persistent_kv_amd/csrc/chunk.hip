// Causal attention of a chunk of C new queries over a paged bf16 cache, on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// "Persistent input/output feedback", "Optional heterogeneous paged KV",
// section "Versioned operator schema": causal masking is the default, the
// left window is unbounded, and the new Q, K and V have the same length.
// After the chunk has been appended at position p0 (pkv_paged_cache_update),
// query t of a row sits at p0 + t and attends keys [0, p0 + t].
//
// Unlike the single-token step this is a dense contraction: per (row, kv
// head) the G * C query rows share every K/V tile, so Q.K^T and P.V run as
// bf16 MFMA tiles with fp32 accumulation (flash-attention style, online
// softmax, no score matrix in memory).
//
// Layout choice: the kernel computes S^T = K Q^T, so that one lane owns one
// query row (MFMA column) and 16 of its scores.  The row max / sum and the
// output rescale are then per-lane scalars, and the score registers are
// directly the B operand of O^T = V^T P^T once the 16 keys of each MFMA step
// are taken in the order the lanes hold them (the A operand reads V^T with
// the same key permutation).  Operand layouts (checked on the device):
//   A[i][k]: lane l holds i = l % 32, k = 8 (l / 32) + e, e = 0..7
//   B[k][j]: lane l holds k = 8 (l / 32) + e, j = l % 32
//   C[i][j]: lane l, register r holds i = 8 (r / 4) + 4 (l / 32) + r % 4, j = l % 32
//
// Workgroup: 4 waves, 128 query rows (128 / G positions x G heads of one kv
// head); key tiles of 64 tokens staged in LDS (K row-major, V transposed,
// rows padded against bank conflicts), next tile prefetched into registers
// while the current one is consumed.  Workgroups of the same (row, kv head)
// are placed on the same XCD so they share its L2.

#include "device_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kCD = 128;        // head size
constexpr int kRows = 128;      // query rows per workgroup
constexpr int kKeys = 64;       // keys per tile
constexpr int kKPad = kCD + 8;  // K row stride in LDS (bf16)
constexpr int kVPad = kKeys + 8;  // V^T row stride in LDS (bf16)
constexpr float kLazyC = 8.0f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16_rne(lo)) | (uint32_t(f32_to_bf16_rne(hi)) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int G>
__global__ __launch_bounds__(256) void chunk_attention_kernel(ChunkArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kKeys * kKPad];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[kCD * kVPad];

    constexpr int P = kRows / G;  // positions per workgroup
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane >> 5;     // which half of the wave
    const int col = lane & 31;    // MFMA column = query row within the wave

    // ---- work item: (row b, kv head, query tile), XCD-grouped when possible
    const int n_qt = (a.C + P - 1) / P;
    const int n_bkv = a.rows * a.Hkv;
    int bkv, qt;
    {
        const int id = blockIdx.x;
        if (n_bkv % 8 == 0) {
            const int xcd = id % 8, local = id / 8;
            qt = local % n_qt;
            bkv = (local / n_qt) * 8 + xcd;
        } else {
            qt = id % n_qt;
            bkv = id / n_qt;
        }
    }
    const int b = bkv / a.Hkv;
    const int kvh = bkv % a.Hkv;
    const int t0 = qt * P;
    const int p0 = a.p0[b];
    const int32_t* pt = a.page_table + int64_t(b) * a.maxb;

    // this lane's query row
    const int r = wave * 32 + col;           // 0..127
    const int t = t0 + r / G;                // position in the chunk
    const int g = r % G;
    const int h = kvh * G + g;
    const bool row_valid = t < a.C;
    const int limit = p0 + min(t, a.C - 1);  // last key this row attends
    const int wg_last_key = p0 + min(t0 + P, a.C) - 1;
    const int wg_first_limit = p0 + t0;      // smallest limit in the workgroup

    // Q^T operand (B of S^T = K Q^T): lane holds dims 8 hl + 16 s .. +7 of its row
    uint4 qB[8];
    {
        const uint16_t* Q = a.q + ((int64_t(b) * a.Hq + h) * a.C + min(t, a.C - 1)) * kCD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qB[s] = *reinterpret_cast<const uint4*>(Q + 16 * s + 8 * hl);
    }

    f32x16_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
    float m = -FLT_MAX, l = 0.0f;

    // ---- global -> register staging of one 64-key tile
    // K: thread handles 16-byte chunks c = tid + 256 i (key c / 16, dims 8 (c % 16) ..)
    // V: thread handles dims 2 (tid % 64), 2 (tid % 64) + 1 of keys 16 (tid / 64) .. +15
    struct Stage {
        uint4 k[4];
        uint32_t v[16];
    };
    auto key_row = [&](int key) -> int64_t {  // element offset of a key's row, key clamped to the valid range
        const int kc = min(key, wg_last_key);
        const int page = pt[kc / a.bs];
        return ((int64_t(page) * a.Hkv + kvh) * a.bs + kc % a.bs) * kCD;
    };
    auto stage_load = [&](Stage& st, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            st.k[i] = *reinterpret_cast<const uint4*>(a.k + key_row(k0 + c / 16) + 8 * (c % 16));
        }
        const int d2 = 2 * (tid % 64);
        const int kb = 16 * (tid / 64);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            st.v[i] = *reinterpret_cast<const uint32_t*>(a.v + key_row(k0 + kb + i) + d2);
    };
    auto stage_store = [&](const Stage& st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<uint4*>(sK + (c / 16) * kKPad + 8 * (c % 16)) = st.k[i];
        }
        const int d2 = 2 * (tid % 64);
        const int kb = 16 * (tid / 64);
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // keys kb + 2i, kb + 2i + 1: low halves -> dim d2, high halves -> dim d2 + 1
            lo[i] = __builtin_amdgcn_perm(st.v[2 * i + 1], st.v[2 * i], 0x05040100u);
            hi[i] = __builtin_amdgcn_perm(st.v[2 * i + 1], st.v[2 * i], 0x07060302u);
        }
        uint4* r0 = reinterpret_cast<uint4*>(sVt + d2 * kVPad + kb);
        uint4* r1 = reinterpret_cast<uint4*>(sVt + (d2 + 1) * kVPad + kb);
        r0[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        r0[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        r1[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        r1[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    };

    const int n_tiles = wg_last_key / kKeys + 1;
    Stage st;
    stage_load(st, 0);
    for (int it = 0; it < n_tiles; ++it) {
        const int k0 = it * kKeys;
        __syncthreads();               // the previous tile is consumed
        stage_store(st);
        __syncthreads();
        if (it + 1 < n_tiles) stage_load(st, k0 + kKeys);

        // S^T for keys k0 .. k0+31 (s[0]) and k0+32 .. k0+63 (s[1])
        f32x16_t s[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[half][e] = 0.0f;
            const uint16_t* krow = sK + (half * 32 + col) * kKPad + 8 * hl;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const uint4 kA = *reinterpret_cast<const uint4*>(krow + 16 * ks);
                s[half] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kA), as_bf16x8(qB[ks]), s[half], 0, 0, 0);
            }
        }
        // scale, causal mask, tile max of this query row
        const bool need_mask = k0 + kKeys - 1 > wg_first_limit;
        float mx = -INFINITY;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = s[half][e] * a.scale_log2;
                if (need_mask) {
                    const int key = k0 + half * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
                    x = key <= limit ? x : -INFINITY;
                }
                s[half][e] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m + kLazyC) {
            const float c = exp2_fast(m - mx);
            l *= c;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[d][e] *= c;
            m = mx;
        }
        // P^T as B operands: chunk q covers keys 16 q .. 16 q + 15 of the tile,
        // element e of this lane = register 8 (q % 2) + e of s[q / 2]
        uint4 pB[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = exp2_fast(s[q / 2][8 * (q % 2) + e] - m);
                l += p[e];
            }
            pB[q] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7]));
        }
        // O^T += V^T P^T: A[i = dim][k] with the keys of chunk q taken as
        // 16 q + 4 hl + 0..3 and 16 q + 8 + 4 hl + 0..3 (the order of pB)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint16_t* vrow = sVt + (32 * d + col) * kVPad + 4 * hl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 x0 = *reinterpret_cast<const uint2*>(vrow + 16 * q);
                const uint2 x1 = *reinterpret_cast<const uint2*>(vrow + 16 * q + 8);
                const uint4 vA = make_uint4(x0.x, x0.y, x1.x, x1.y);
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vA), as_bf16x8(pB[q]), o[d], 0, 0, 0);
            }
        }
    }

    // ---- normalise and store: lane holds dims 32 d + 8 (e / 4) + 4 hl + e % 4 of its row
    l += __shfl_xor(l, 32);
    if (row_valid) {
        const float inv = 1.0f / l;
        uint16_t* O = a.out + ((int64_t(b) * a.Hq + h) * a.C + t) * kCD;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int dim = 32 * d + 8 * e4 + 4 * hl;
                uint2 w;
                w.x = pack_bf16x2(o[d][4 * e4 + 0] * inv, o[d][4 * e4 + 1] * inv);
                w.y = pack_bf16x2(o[d][4 * e4 + 2] * inv, o[d][4 * e4 + 3] * inv);
                *reinterpret_cast<uint2*>(O + dim) = w;
            }
    }
}

}  // namespace

bool chunk_supported(int D, int G, int bs, int C) {
    (void)bs;
    return D == kCD && (G == 1 || G == 2 || G == 4 || G == 8) && C >= 1;
}

hipError_t launch_chunk(const ChunkArgs& a, int G, hipStream_t s) {
    const int P = kRows / G;
    const int blocks = a.rows * a.Hkv * ((a.C + P - 1) / P);
    if (blocks <= 0) return hipSuccess;
    switch (G) {
        case 1: hipLaunchKernelGGL(chunk_attention_kernel<1>, dim3(blocks), dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL(chunk_attention_kernel<2>, dim3(blocks), dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL(chunk_attention_kernel<4>, dim3(blocks), dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL(chunk_attention_kernel<8>, dim3(blocks), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
