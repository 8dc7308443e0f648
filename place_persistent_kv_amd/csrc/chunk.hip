// Causal attention of a chunk of C new queries over a paged bf16 cache, on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// "Persistent input/output feedback", "Optional heterogeneous paged KV",
// section "Versioned operator schema": causal masking is the default, the
// left window is unbounded, and the new Q, K and V have the same length.
// After the chunk has been appended at position p0 (pkv_paged_cache_update),
// query t of a row sits at p0 + t and attends keys [0, p0 + t], or with a left
// window W >= 0 keys [p0 + t - W, p0 + t] (left_window_size).
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
// Workgroup: 8 waves, 256 query rows (256 / G positions x G heads of one kv
// head), one 32-row MFMA column group per wave.  With about 210 VGPRs a wave,
// two waves share each SIMD, so one wave's softmax (vector ALU) overlaps the
// other's MFMAs.  Key tiles of 64 tokens are staged in LDS (K row-major, V
// transposed, both laid out so that neither the staging writes nor the
// operand reads conflict on banks) with the next two tiles' loads in flight
// in registers.  Workgroups of the same (row, kv head) are placed on the same
// XCD so they share its L2.  (PKV_CHUNK_WAVES=4 builds the variant with two
// column groups per wave, each K / V^T operand read feeding two MFMAs.)

#include "device_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;        // head size
#ifndef PKV_CHUNK_WAVES
#define PKV_CHUNK_WAVES 8
#endif
constexpr int kWavesC = PKV_CHUNK_WAVES;          // waves per workgroup
constexpr int kRowGroups = 8 / kWavesC;           // MFMA column groups of 32 query rows per wave
constexpr int kThreads = 64 * kWavesC;
constexpr int kRows = kWavesC * kRowGroups * 32;  // query rows per workgroup (256)
constexpr int kKL = 1024 / kThreads;              // K 16-byte chunks per thread and tile
constexpr int kVK = 1024 / kThreads;              // keys per thread in the V staging
constexpr int kKeys = 64;       // keys per tile
constexpr int kKPad = kCD + 8;  // K row stride in LDS (bf16)
constexpr int kVPad = kKeys + 4;  // V^T row stride in LDS (bf16): 34 dwords, see the staging notes
constexpr float kLazyC = 8.0f;

// two floats -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// the value of the lane 32 positions away, combined: lanes l and l ^ 32 hold
// the two halves of one query row's keys (v_permlane32_swap_b32)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int G, bool WIN>   // WIN: a left window is set (a.window >= 0)
__global__ __launch_bounds__(kThreads) void chunk_attention_kernel(ChunkArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kKeys * kKPad];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[kCD * kVPad];

    constexpr int P = kRows / G;  // positions per workgroup
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane >> 5;     // which half of the wave
    const int col = lane & 31;    // MFMA column = query row within a row group

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
    const int wg_last_key = p0 + min(t0 + P, a.C) - 1;
    const int wg_first_limit = p0 + t0;      // smallest limit in the workgroup
    // left window: a query at position p sees keys [p - window, p]; tiles below
    // the smallest lower limit are skipped, those below the largest are masked
    const int wg_lo_first = WIN ? max(0, wg_first_limit - a.window) : 0;
    const int wg_lo_last = WIN ? max(0, wg_last_key - a.window) : 0;

    // this lane's two query rows (row groups rg = 0, 1 of the wave)
    int t[kRowGroups], h[kRowGroups], limit[kRowGroups], lo_lim[kRowGroups];
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
        const int r = (wave * kRowGroups + rg) * 32 + col;
        t[rg] = t0 + r / G;
        h[rg] = kvh * G + r % G;
        limit[rg] = p0 + min(t[rg], a.C - 1);
        lo_lim[rg] = WIN ? max(0, limit[rg] - a.window) : 0;
    }

    // Q^T operand (B of S^T = K Q^T): lane holds dims 8 hl + 16 s .. +7 of its row
    u32x4_t qB[kRowGroups][8];
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
        const uint16_t* Q = a.q + ((int64_t(b) * a.Hq + h[rg]) * a.C + min(t[rg], a.C - 1)) * kCD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qB[rg][s] = *reinterpret_cast<const u32x4_t*>(Q + 16 * s + 8 * hl);
    }

    f32x16_t o[kRowGroups][4];
    float m[kRowGroups], l[kRowGroups];
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
        m[rg] = -FLT_MAX;
        l[rg] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[rg][d][e] = 0.0f;
    }

    // ---- global -> register staging of one 64-key tile
    // K: thread handles 16-byte chunks c = tid + kThreads i (key c / 16, dims 8 (c % 16) ..)
    // V: thread handles dims d8 .. d8 + 7 of the kVK keys kb .. kb + kVK - 1, which
    //    lie in one page (block_size is a power of two >= 4).  Transposed into
    //    V^T rows (one per dim) of 34 dwords: the 16 lanes of a write phase
    //    fill one row's 64 keys, and the 16 lanes of an operand read (dims
    //    r .. r + 15) start 34 dwords apart, i.e. on distinct bank pairs.
    // Keys past the workgroup's last key are clamped to it (valid rows, masked
    // later).  The page ids a tile needs are loaded one tile ahead of its K/V
    // rows, so no K/V load waits on a page-table load issued just before it.
    struct Pages {
        i32x4_t k;                    // first kKL entries used
        int v;
    };
    struct Stage {
        u32x4_t k[kKL];
        u32x4_t v[kVK];
    };
    const int kb = kVK * (tid % (64 / kVK));
    const int d8 = 8 * (tid / (64 / kVK));
    auto page_load = [&](int k0) -> Pages {
        Pages pg;
#pragma unroll
        for (int i = 0; i < kKL; ++i) pg.k[i] = pt[min(k0 + (tid + kThreads * i) / 16, wg_last_key) >> a.log2bs];
        pg.v = pt[min(k0 + kb, wg_last_key) >> a.log2bs];
        return pg;
    };
    // element offset of (page, kv head, slot of key): one 32x32->64 multiply-add
    const uint32_t page_stride = uint32_t(a.Hkv) * uint32_t(a.bs) * kCD;
    const uint32_t head_off = uint32_t(kvh) * uint32_t(a.bs) * kCD;
    auto row_of = [&](int page, int key) -> uint64_t {
        return uint64_t(uint32_t(page)) * page_stride + (head_off + uint32_t(min(key, wg_last_key) & (a.bs - 1)) * kCD);
    };
    auto stage_load = [&](int k0, const Pages& pg) -> Stage {
        Stage st;
#pragma unroll
        for (int i = 0; i < kKL; ++i) {
            const int c = tid + kThreads * i;
            st.k[i] = *reinterpret_cast<const u32x4_t*>(a.k + row_of(pg.k[i], k0 + c / 16) + 8 * (c % 16));
        }
#pragma unroll
        for (int i = 0; i < kVK; ++i)
            st.v[i] = *reinterpret_cast<const u32x4_t*>(a.v + row_of(pg.v, k0 + kb + i) + d8);
        return st;
    };
    auto stage_store = [&](Stage st) {
#pragma unroll
        for (int i = 0; i < kKL; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<u32x4_t*>(sK + (c / 16) * kKPad + 8 * (c % 16)) = st.k[i];
        }
        // transpose: dim d8 + 2m takes the low halves of the keys' word m, d8 + 2m + 1 the high halves
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            if constexpr (kVK == 4) {
                u32x2_t lo, hi;
                lo.x = __builtin_amdgcn_perm(st.v[1][mm], st.v[0][mm], 0x05040100u);
                lo.y = __builtin_amdgcn_perm(st.v[3][mm], st.v[2][mm], 0x05040100u);
                hi.x = __builtin_amdgcn_perm(st.v[1][mm], st.v[0][mm], 0x07060302u);
                hi.y = __builtin_amdgcn_perm(st.v[3][mm], st.v[2][mm], 0x07060302u);
                *reinterpret_cast<u32x2_t*>(sVt + (d8 + 2 * mm) * kVPad + kb) = lo;
                *reinterpret_cast<u32x2_t*>(sVt + (d8 + 2 * mm + 1) * kVPad + kb) = hi;
            } else {
                *reinterpret_cast<uint32_t*>(sVt + (d8 + 2 * mm) * kVPad + kb) =
                    __builtin_amdgcn_perm(st.v[1][mm], st.v[0][mm], 0x05040100u);
                *reinterpret_cast<uint32_t*>(sVt + (d8 + 2 * mm + 1) * kVPad + kb) =
                    __builtin_amdgcn_perm(st.v[1][mm], st.v[0][mm], 0x07060302u);
            }
        }
    };

    // ---- one 64-key tile from LDS, as two halves of 32 keys: S^T = K Q^T,
    // online softmax, O^T += V^T P^T
    auto compute = [&](int k0) {
        // only the diagonal tiles (reaching past the smallest causal limit of
        // the workgroup) test keys against the limits; a uniform branch
        const bool need_mask = k0 + kKeys - 1 > wg_first_limit || (WIN && k0 < wg_lo_last);

        // S^T for both 32-key halves, the two accumulation chains interleaved
        f32x16_t s[2][kRowGroups];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int rg = 0; rg < kRowGroups; ++rg)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[half][rg][e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const u32x4_t kA = *reinterpret_cast<const u32x4_t*>(sK + (half * 32 + col) * kKPad + 8 * hl + 16 * ks);
#pragma unroll
                for (int rg = 0; rg < kRowGroups; ++rg)
                    s[half][rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kA), as_bf16x8(qB[rg][ks]),
                                                                         s[half][rg], 0, 0, 0);
            }
        }

        // per half: online softmax (the matrix cores run the other half's
        // products meanwhile), then O^T += V^T P^T
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4_t pB[kRowGroups][2];
#pragma unroll
            for (int rg = 0; rg < kRowGroups; ++rg) {
                // causal mask and max of this query row over the 32 keys, in raw
                // score units (the scale is positive)
                if (need_mask) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + half * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
                        s[half][rg][e] = key <= limit[rg] && (!WIN || key >= lo_lim[rg]) ? s[half][rg][e] : -INFINITY;
                    }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[half][rg][e]);
                mx = max_halves(mx) * a.scale_log2;
                if (mx > m[rg] + kLazyC) {
                    const float c = exp2_fast(m[rg] - mx);
                    l[rg] *= c;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
#pragma unroll
                        for (int e = 0; e < 16; ++e) o[rg][d][e] *= c;
                    m[rg] = mx;
                }
                const float neg_m = -m[rg];
                // P^T as B operands: chunk qq covers keys 16 qq .. 16 qq + 15 of
                // the half, element e of this lane = register 8 qq + e of s
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = exp2_fast(fmaf(s[half][rg][8 * qq + e], a.scale_log2, neg_m));
                        l[rg] += p[e];
                    }
                    pB[rg][qq] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                         pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                }
            }
            // O^T += V^T P^T: A[i = dim][k] with the keys of chunk qq taken as
            // 16 qq + 4 hl + 0..3 and 16 qq + 8 + 4 hl + 0..3 (the order of pB)
            // (key chunk outer, dim block inner: consecutive products go to
            // different accumulators, none waits for the one before it)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint16_t* vrow = sVt + (32 * d + col) * kVPad + 32 * half + 4 * hl;
                    const u32x2_t x0 = *reinterpret_cast<const u32x2_t*>(vrow + 16 * qq);
                    const u32x2_t x1 = *reinterpret_cast<const u32x2_t*>(vrow + 16 * qq + 8);
                    const u32x4_t vA = u32x4_t{x0.x, x0.y, x1.x, x1.y};
#pragma unroll
                    for (int rg = 0; rg < kRowGroups; ++rg)
                        o[rg][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vA), as_bf16x8(pB[rg][qq]),
                                                                          o[rg][d], 0, 0, 0);
                }
            }
        }
    };

    // Tiles go in pairs with two register stages A and B (no copies between
    // them, so a wait is only ever for the stage about to be stored).  At a
    // step the stage is stored to LDS, refilled with the K/V rows two tiles
    // ahead, whose page ids were requested two steps earlier, and the ids four
    // tiles ahead are requested.  Loads past the last tile re-read the last one
    // (always valid); an odd tile count ends with one fully masked tile.
    const int n_tiles = wg_last_key / kKeys + 1;
    const int it0 = wg_lo_first / kKeys;     // first tile any query of the workgroup sees
    auto tile_key = [&](int it) { return min(it, n_tiles - 1) * kKeys; };
    // (the prologue keeps the loop's issue order, so that the waits at the
    // loop head are the same on entry as on every later pass)
    Pages pgA = page_load(tile_key(it0));
    Pages pgB = page_load(tile_key(it0 + 1));
    __builtin_amdgcn_sched_barrier(0);
    Stage A = stage_load(tile_key(it0), pgA);
    __builtin_amdgcn_sched_barrier(0);
    pgA = page_load(tile_key(it0 + 2));
    __builtin_amdgcn_sched_barrier(0);
    Stage B = stage_load(tile_key(it0 + 1), pgB);
    __builtin_amdgcn_sched_barrier(0);
    pgB = page_load(tile_key(it0 + 3));
    __builtin_amdgcn_sched_barrier(0);
    for (int it = it0; it < n_tiles; it += 2) {
        __syncthreads();               // the previous tile is consumed
        stage_store(A);
        __syncthreads();
        A = stage_load(tile_key(it + 2), pgA);
        pgA = page_load(tile_key(it + 4));
        compute(it * kKeys);

        __syncthreads();
        stage_store(B);
        __syncthreads();
        B = stage_load(tile_key(it + 3), pgB);
        pgB = page_load(tile_key(it + 5));
        compute((it + 1) * kKeys);
    }

    // ---- normalise and store: lane holds dims 32 d + 8 (e / 4) + 4 hl + e % 4 of its row
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
        const float lt = sum_halves(l[rg]);
        if (t[rg] < a.C) {
            const float inv = 1.0f / lt;
            uint16_t* O = a.out + ((int64_t(b) * a.Hq + h[rg]) * a.C + t[rg]) * kCD;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int dim = 32 * d + 8 * e4 + 4 * hl;
                    u32x2_t w;
                    w.x = pack_bf16x2(o[rg][d][4 * e4 + 0] * inv, o[rg][d][4 * e4 + 1] * inv);
                    w.y = pack_bf16x2(o[rg][d][4 * e4 + 2] * inv, o[rg][d][4 * e4 + 3] * inv);
                    *reinterpret_cast<u32x2_t*>(O + dim) = w;
                }
        }
    }
}

}  // namespace

bool chunk_supported(int D, int G, int bs, int C) {
    return D == kCD && (G == 1 || G == 2 || G == 4 || G == 8) && bs >= 4 && C >= 1;
}

hipError_t launch_chunk(const ChunkArgs& a, int G, hipStream_t s) {
    const int P = kRows / G;
    const int blocks = a.rows * a.Hkv * ((a.C + P - 1) / P);
    if (blocks <= 0) return hipSuccess;
    switch (G) {
#define PKV_CHUNK(GG)                                                                                  \
        case GG:                                                                                       \
            if (a.window >= 0) hipLaunchKernelGGL((chunk_attention_kernel<GG, true>), dim3(blocks), dim3(kThreads), 0, s, a); \
            else hipLaunchKernelGGL((chunk_attention_kernel<GG, false>), dim3(blocks), dim3(kThreads), 0, s, a); \
            break;
        PKV_CHUNK(1)
        PKV_CHUNK(2)
        PKV_CHUNK(4)
        PKV_CHUNK(8)
#undef PKV_CHUNK
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
