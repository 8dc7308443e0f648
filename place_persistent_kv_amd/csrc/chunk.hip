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
// head), one 32-row MFMA column group per wave; at about 200 VGPRs two waves
// share each SIMD, so one wave's softmax (vector ALU) overlaps the other's
// MFMAs.  Workgroups of the same (row, kv head) are placed on the same XCD so
// they share its L2.
//
// Key tiles of 64 tokens go from the pages straight into LDS with 16-byte
// global-to-LDS loads (global_load_lds_dwordx4: no staging registers, no LDS
// store instructions), two tile buffers, the next tile's loads in flight
// while the current one is computed, one barrier per tile.  K and V keep the
// pages' row-major [key][dim] layout in LDS, each 256-byte row's sixteen
// 16-byte chunks permuted by chunk ^ 2 (key % 8) (the loading lane fetches
// the chunk its slot holds).  The K operand of S^T is one 16-byte read per
// lane (8 consecutive rows of one read phase hit 8 distinct chunk columns);
// the V^T operand of O^T comes from the row-major V rows through the
// transposing LDS read ds_read_b64_tr_b16, which hands lane i of a 16-lane
// group element i % 4 of the 8-byte pieces read by lanes 4 k + i / 4
// (k = 0..3) -- so lanes that read 4 dims of 4 consecutive keys deliver each
// lane 4 keys of one dim (checked on the device).  Page ids are wave-uniform
// scalar loads, one tile ahead.

#include "device_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;        // head size
constexpr int kWavesC = 8;      // waves per workgroup
constexpr int kThreads = 64 * kWavesC;
constexpr int kRows = kWavesC * 32;  // query rows per workgroup (256)
constexpr int kKeys = 64;       // keys per tile
constexpr int kTileElems = kKeys * kCD;   // one K or V tile (bf16 elements, 16 KB)
constexpr float kLazyC = 8.0f;

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(1))) const uint8_t gbl_u8;

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

// element offset of (key, chunk) in a tile: row-major rows of 128 bf16, chunk
// c of row `key` stored at chunk column c ^ 2 (key % 8)
__device__ __forceinline__ int tile_off(int key, int chunk) { return key * kCD + 8 * (chunk ^ (2 * (key & 7))); }

// 8 bytes read through the transposing LDS path
__device__ __forceinline__ u32x2_t read_tr(const lds_u16* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// A wave-uniform 32-bit load through the scalar unit
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}

template <int G, bool WIN>   // WIN: a left window is set (a.window >= 0)
__global__ __launch_bounds__(kThreads) void chunk_attention_kernel(ChunkArgs a) {
    // two tile buffers, K and V each [64 keys][128 dims] (chunk-permuted rows)
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kTileElems], sV0[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kTileElems], sV1[kTileElems];

    constexpr int P = kRows / G;  // positions per workgroup
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hl = lane >> 5;     // which half of the wave
    const int col = lane & 31;    // MFMA column = query row within the wave's row group

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

    // this lane's query row
    const int r = wave * 32 + col;
    const int t = t0 + r / G;
    const int h = kvh * G + r % G;
    const int limit = p0 + min(t, a.C - 1);
    const int lo_lim = WIN ? max(0, limit - a.window) : 0;

    // Q^T operand (B of S^T = K Q^T): lane holds dims 8 hl + 16 s .. +7 of its row
    u32x4_t qB[8];
    {
        const uint16_t* Q = a.q + ((int64_t(b) * a.Hq + h) * a.C + min(t, a.C - 1)) * kCD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qB[s] = *reinterpret_cast<const u32x4_t*>(Q + 16 * s + 8 * hl);
    }

    f32x16_t o[4];
    float m = -FLT_MAX, l = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;

    // ---- global -> LDS loads of one tile.  Wave w fills rows 8 w .. 8 w + 7
    // of the K and V tiles with two 1 KB loads each (rows 8 w + 4 i .. + 3 for
    // i = 0, 1); lane L writes slot L of such a load, i.e. row 8 w + 4 i + L / 16,
    // chunk column L % 16, so it fetches chunk (L % 16) ^ 2 (row % 8) of its
    // row.  Keys past the workgroup's last key are clamped to it (valid rows,
    // masked later); an aligned 4-row group lies in one page (block_size >= 4).
    const uint32_t page_bytes = uint32_t(a.Hkv) * uint32_t(a.bs) * kCD * 2;
    const uint32_t head_bytes = uint32_t(kvh) * uint32_t(a.bs) * kCD * 2;
    const int lrow = lane >> 4;                              // row within a 1 KB load
    struct Pages {
        int32_t p[2];
    };
    auto page_load = [&](int k0) -> Pages {
        Pages pg;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            pg.p[i] = load_uniform(pt + (min(k0 + 8 * wave + 4 * i, wg_last_key) >> a.log2bs));
        return pg;
    };
    auto tile_load = [&](int k0, const Pages& pg, lds_u16* dK, lds_u16* dV) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 8 * wave + 4 * i + lrow;           // row of the tile
            const int key = min(k0 + row, wg_last_key);
            const int chunk = (lane & 15) ^ (2 * (row & 7));
            const uint32_t off = head_bytes + uint32_t(key & (a.bs - 1)) * (kCD * 2) + 16u * uint32_t(chunk);
            const uint64_t page_off = uint64_t(uint32_t(pg.p[i])) * page_bytes;
            gbl_u8* gk = (gbl_u8*)(reinterpret_cast<const uint8_t*>(a.k) + page_off) + off;
            gbl_u8* gv = (gbl_u8*)(reinterpret_cast<const uint8_t*>(a.v) + page_off) + off;
            __builtin_amdgcn_global_load_lds(gk, dK + (8 * wave + 4 * i) * kCD, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gv, dV + (8 * wave + 4 * i) * kCD, 16, 0, 0);
        }
    };

    // per-lane element offsets of the operand reads (without the key-tile base)
    //   K (A of S^T): row half * 32 + col, chunk hl + 2 ks
    //   V^T (A of O^T) through the transposing read: lane L of 16-lane group g
    //   reads dims 32 d + 16 (g % 2) + 4 (L % 4) .. + 3 of key
    //   half * 32 + 16 qq + 4 (g / 2) + (L % 16) / 4 (+ 8 for the second read)
    const int g16 = lane >> 4;
    const int vkey = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int vchunk = 2 * (g16 & 1) + ((lane & 3) >> 1);
    const int vsub = 4 * (lane & 1);

    // ---- one 64-key tile from LDS, as two halves of 32 keys: S^T = K Q^T,
    // online softmax, O^T += V^T P^T
    auto compute = [&](int k0, const lds_u16* tK, const lds_u16* tV) {
        // only the diagonal tiles (reaching past the smallest causal limit of
        // the workgroup) test keys against the limits; a uniform branch
        const bool need_mask = k0 + kKeys - 1 > wg_first_limit || (WIN && k0 < wg_lo_last);

        // S^T for both 32-key halves, the two accumulation chains interleaved
        f32x16_t s[2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int key = half * 32 + col;
                const u32x4_t kA = *(const __attribute__((address_space(3))) u32x4_t*)(tK + tile_off(key, hl + 2 * ks));
                const f32x16_t acc = ks == 0 ? f32x16_t{} : s[half];
                s[half] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kA), as_bf16x8(qB[ks]), acc, 0, 0, 0);
            }
        }

        // per half: online softmax (the matrix cores run the other half's
        // products meanwhile), then O^T += V^T P^T
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4_t pB[2];
            // causal mask and max of this query row over the 32 keys, in raw
            // score units (the scale is positive)
            if (need_mask) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + half * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
                    s[half][e] = key <= limit && (!WIN || key >= lo_lim) ? s[half][e] : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[half][e]);
            mx = max_halves(mx) * a.scale_log2;
            if (mx > m + kLazyC) {
                const float c = exp2_fast(m - mx);
                l *= c;
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[d][e] *= c;
                m = mx;
            }
            const float neg_m = -m;
            // P^T as B operands: chunk qq covers keys 16 qq .. 16 qq + 15 of
            // the half, element e of this lane = register 8 qq + e of s
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = exp2_fast(fmaf(s[half][8 * qq + e], a.scale_log2, neg_m));
                    l += p[e];
                }
                pB[qq] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            }
            // O^T += V^T P^T: A[i = dim][k] with the keys of chunk qq taken as
            // 16 qq + 4 hl + 0..3 and 16 qq + 8 + 4 hl + 0..3 (the order of pB)
            // (key chunk outer, dim block inner: consecutive products go to
            // different accumulators, none waits for the one before it)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int key = half * 32 + 16 * qq + vkey;
                    const u32x2_t x0 = read_tr(tV + tile_off(key, 4 * d + vchunk) + vsub);
                    const u32x2_t x1 = read_tr(tV + tile_off(key + 8, 4 * d + vchunk) + vsub);
                    const u32x4_t vA = u32x4_t{x0.x, x0.y, x1.x, x1.y};
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vA), as_bf16x8(pB[qq]), o[d], 0, 0, 0);
                }
            }
        }
    };

    // Tiles alternate between the two buffers (the loop is unrolled by two, so
    // each buffer is a fixed LDS array).  At a tile: wait for this wave's loads
    // of it, barrier (every wave's loads have landed, and every wave is done
    // with the other buffer), start the next tile's loads into the other
    // buffer, request the page ids of the tile after that, compute.  Loads
    // past the last tile re-read the last one (always valid); an odd tile
    // count ends with one fully masked tile.
    const int n_tiles = wg_last_key / kKeys + 1;
    const int it0 = wg_lo_first / kKeys;     // first tile any query of the workgroup sees
    auto tile_key = [&](int it) { return min(it, n_tiles - 1) * kKeys; };
    lds_u16* const K0 = (lds_u16*)(sK0);
    lds_u16* const V0 = (lds_u16*)(sV0);
    lds_u16* const K1 = (lds_u16*)(sK1);
    lds_u16* const V1 = (lds_u16*)(sV1);
    Pages pg = page_load(tile_key(it0));
    tile_load(tile_key(it0), pg, K0, V0);
    pg = page_load(tile_key(it0 + 1));
    for (int it = it0; it < n_tiles; it += 2) {
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's loads of the tile
        __syncthreads();
        tile_load(tile_key(it + 1), pg, K1, V1);
        pg = page_load(tile_key(it + 2));
        compute(it * kKeys, K0, V0);

        __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        tile_load(tile_key(it + 2), pg, K0, V0);
        pg = page_load(tile_key(it + 3));
        compute((it + 1) * kKeys, K1, V1);
    }

    // ---- normalise and store: lane holds dims 32 d + 8 (e / 4) + 4 hl + e % 4 of its row
    const float lt = sum_halves(l);
    if (t < a.C) {
        const float inv = 1.0f / lt;
        uint16_t* O = a.out + ((int64_t(b) * a.Hq + h) * a.C + t) * kCD;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int dim = 32 * d + 8 * e4 + 4 * hl;
                u32x2_t w;
                w.x = pack_bf16x2(o[d][4 * e4 + 0] * inv, o[d][4 * e4 + 1] * inv);
                w.y = pack_bf16x2(o[d][4 * e4 + 2] * inv, o[d][4 * e4 + 3] * inv);
                *reinterpret_cast<u32x2_t*>(O + dim) = w;
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
