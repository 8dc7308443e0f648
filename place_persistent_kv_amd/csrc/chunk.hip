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
// store instructions), three K and three V tile buffers, the loads of the
// next tiles in flight while the current one is computed, one barrier per
// tile.  K and V keep the
// pages' row-major [key][dim] layout in LDS, each 256-byte row's sixteen
// 16-byte chunks permuted by chunk ^ swz(key % 16) (the loading lane fetches
// the chunk its slot holds).  The LDS serves 256 bytes per cycle: 16 lanes of
// a 16-byte read or 32 lanes of an 8-byte read.  swz is a bijection of the 16
// rows (the 16 rows a K read phase touches use 16 distinct chunk columns), and
// within each aligned group of 4 rows it takes 4 distinct values of bits 2-3
// (a V read phase touches 4 chunks 4 d .. 4 d + 3 of 4 such rows, which then
// also land on 16 distinct columns); it also keeps both read kinds apart on
// 128-byte bank windows.  The K operand of S^T is one 16-byte read per
// lane; the V^T operand of O^T comes from the row-major V rows through the
// transposing LDS read ds_read_b64_tr_b16, which hands lane i of a 16-lane
// group element i % 4 of the 8-byte pieces read by lanes 4 k + i / 4
// (k = 0..3) -- so lanes that read 4 dims of 4 consecutive keys deliver each
// lane 4 keys of one dim (checked on the device).  Page ids are wave-uniform
// scalar loads, one tile ahead.

#include "device_common.h"

#include <type_traits>

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;        // head size
constexpr int kWavesC = 8;      // waves per workgroup
constexpr int kThreads = 64 * kWavesC;
constexpr int kRows = kWavesC * 32;  // query rows per workgroup (256)
constexpr int kKeys = 64;       // keys per tile
constexpr int kTileElems = kKeys * kCD;   // one K or V tile (bf16 elements, 16 KB)
static_assert(kRows == kChunkQueryRows && kKeys == kChunkKeys, "host and kernel tile shapes differ");
constexpr float kLazyC = 8.0f;
constexpr float kLazyP = 256.0f;   // 2^kLazyC

typedef __attribute__((address_space(3))) uint16_t lds_u16;

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

// chunk-column permutation of tile row `key`: for i = key % 4 the values
// 0, 6, 12, 10 (distinct in bits 2-3 and in bits 1-2), bit 1 flipped for rows
// 8..15 of 16, bit 0 set for rows 4..7 of 8
__device__ __forceinline__ int swz(int key) {
    const int i = key & 3;
    return ((i << 2) ^ (i << 1)) ^ (((key >> 3) & 1) << 1) ^ ((key >> 2) & 1);
}

// element offset of (key, chunk) in a tile: row-major rows of 128 bf16, chunk
// c of row `key` stored at chunk column c ^ swz(key)
__device__ __forceinline__ int tile_off(int key, int chunk) { return key * kCD + 8 * (chunk ^ swz(key)); }

// 16-byte global-to-LDS load (global_load_lds_dwordx4): lane L's 16 bytes at
// base + voff land at LDS byte address lds + 16 L (M0 holds lds; one wait
// state between the M0 write and the load).  Issued as inline assembly so
// that the compiler does not make the LDS operand reads of the other tile
// buffers wait for it: each wave waits for its own loads (vmcnt) before the
// barrier that hands the tile to the workgroup.
// M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
}

// Four such loads of consecutive 1 KB blocks: load i reads base + (voff0 ^
// 16 i) + 1024 i and writes LDS lds + 1024 i + 16 L (instruction offset 1024 i,
// which applies to both the global and the LDS address).
__device__ __forceinline__ void dma16x4(const void* base, uint32_t voff0, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "global_load_lds_dwordx4 %2, %6 offset:1024\n\t"
        "global_load_lds_dwordx4 %3, %6 offset:2048\n\t"
        "global_load_lds_dwordx4 %4, %6 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff0), "v"(voff0 ^ 16u), "v"(voff0 ^ 32u), "v"(voff0 ^ 48u), "s"(lds), "s"(base)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_u16* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Pin a value to this point of the program: the compiler must have computed it
// here and cannot sink its computation past the barrier that follows (which
// would move a phase's work into the next phase)
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// A value the compiler must treat as unknown (so that it adds constants to it
// as instruction offsets instead of folding them into new registers)
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// LDS reads at a byte address (16 bytes; 8 bytes through the transposing path)
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) u32x4_t*)(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ u32x2_t lds_read_tr(uint32_t addr) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(static_cast<uintptr_t>(addr)));
    return __builtin_bit_cast(u32x2_t, v);
}

// A wave-uniform 32-bit load through the scalar unit
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}

// WIN: a left window is set (a.window >= 0); FAST: block_size >= 16
template <int G, bool WIN, bool FAST>
__global__ __launch_bounds__(kThreads) void chunk_attention_kernel(ChunkArgs a) {
    // LDS (160 KB): three K and three V tile buffers (each [64 keys][128
    // dims], chunk-permuted rows), then the workgroup's 256 query rows, [row]
    // [128 dims], permuted like the tiles (wave w only touches rows 32 w ..
    // 32 w + 31)
    __shared__ __attribute__((aligned(16))) uint16_t smem[6 * kTileElems + kRows * kCD];

    constexpr int P = kRows / G;  // positions per workgroup
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hl = lane >> 5;     // which half of the wave
    const int col = lane & 31;    // MFMA column = query row within the wave's row group

    // ---- work item: (row b, kv head, query tile, key range), XCD-grouped
    // when possible (the query tiles of one (row, kv head, key range) share
    // its K/V tiles in that XCD's L2)
    const int n_qt = (a.C + P - 1) / P;
    const int n_bkv = a.rows * a.Hkv;
    const int S = a.kv_splits;
    int bkv, qt, ks;
    {
        const int id = blockIdx.x;
        if (n_bkv % 8 == 0) {
            const int xcd = id % 8, local = id / 8;
            qt = local % n_qt;
            const int rest = local / n_qt;
            ks = rest % S;
            bkv = (rest / S) * 8 + xcd;
        } else {
            qt = id % n_qt;
            const int rest = id / n_qt;
            ks = rest % S;
            bkv = rest / S;
        }
    }
    const int b = a.order[bkv / a.Hkv];
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


    f32x16_t o[4];
    float m = -FLT_MAX, l = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;

    // key tiles this workgroup visits: [it0, n_tiles), from the first tile
    // any of its queries sees to the tile of its last key, or (split over the
    // keys) part ks of S near-equal parts of that range
    int it0, n_tiles;
    {
        const int first = wg_lo_first / kKeys, end = wg_last_key / kKeys + 1;
        const int per = (end - first + S - 1) / S;
        it0 = first + ks * per;
        n_tiles = min(end, it0 + per);
    }
    const int n = n_tiles - it0;

    // split partial of this lane's query row: the unnormalised output (this
    // lane's dims), and from the lane of the first half the running max (log2
    // units) and the sum over both halves
    auto store_partial = [&](float lt) {
        if (t >= a.C) return;
        const int64_t row = ((int64_t(b) * a.Hq + h) * a.C + t) * S + ks;
        float* wo = a.ws_o + row * kCD;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<f32x4_t*>(wo + 32 * d + 8 * e4 + 4 * hl) =
                    f32x4_t{o[d][4 * e4], o[d][4 * e4 + 1], o[d][4 * e4 + 2], o[d][4 * e4 + 3]};
        if (hl == 0) *reinterpret_cast<f32x2_t*>(a.ws_ml + row * 2) = f32x2_t{m, lt};
    };
    if (n <= 0) {        // a part with no key tile (more parts than tiles): empty partial
        store_partial(0.0f);
        return;
    }

    // ---- global -> LDS loads of one tile, by the four waves of one group
    // (see below): wave w or w + 4 fills rows 16 w .. 16 w + 15 of a tile with
    // four 1 KB loads (rows 16 w + 4 i .. + 3); lane L writes slot L of such a
    // load, i.e. row 16 w + 4 i + L / 16, chunk column L % 16, so it fetches
    // chunk (L % 16) ^ swz(row) of its row.
    const uint32_t page_bytes = uint32_t(a.Hkv) * uint32_t(a.bs) * kCD * 2;
    const uint32_t head_bytes = uint32_t(kvh) * uint32_t(a.bs) * kCD * 2;
    const int lrow = lane >> 4;                              // row within a 1 KB load
    const int wr = 16 * (wave & 3);                          // first tile row of this wave's loads

    // block_size >= 16: the wave's 16 rows lie in one page, the page of key
    // min(k0 + wr, last key) (so no page past the row's last is touched); the
    // rows are not clamped: those past the last key hold whatever that page
    // holds there, K ones are masked out of the scores and V ones are zeroed
    // in LDS before they are read.  Row 16 w' + 4 i + L / 16 of load i sits
    // at in-page row (k0 % bs rounded down to 64) + (16 w' + 4 i + L / 16) %
    // bs, and swz(16 w' + 4 i + L / 16) = swz(L / 16) ^ i, so load i fetches
    // byte offset (voff0 ^ 16 i) + 1024 i and writes LDS at M0 + 1024 i +
    // 16 L, where the 1024 i is the instruction's offset (added to both).
    const uint32_t voff0 = head_bytes + uint32_t((wr + lrow) & (a.bs - 1)) * (kCD * 2) +
                           16u * uint32_t((lane & 15) ^ swz(lrow));
    auto page_fast = [&](int k0) -> int32_t { return load_uniform(pt + (min(k0 + wr, wg_last_key) >> a.log2bs)); };
    auto base_fast = [&](const uint16_t* src, int k0, int32_t page) -> const uint8_t* {
        return reinterpret_cast<const uint8_t*>(src) + uint64_t(uint32_t(page)) * page_bytes +
               uint32_t(k0 & (a.bs - 1) & ~(kKeys - 1)) * (kCD * 2);
    };
    // any block_size >= 4: rows past the last key clamped to it (valid rows,
    // masked later); an aligned 4-row group lies in one page
    auto load_general = [&](const uint16_t* src, int k0, lds_u16* dst) {
        const uint32_t lds = lds_addr(dst + wr * kCD);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int page = load_uniform(pt + (min(k0 + wr + 4 * i, wg_last_key) >> a.log2bs));
            const int row = wr + 4 * i + lrow;                   // row of the tile
            const int key = min(k0 + row, wg_last_key);
            const int chunk = (lane & 15) ^ swz(row);
            const uint32_t off = head_bytes + uint32_t(key & (a.bs - 1)) * (kCD * 2) + 16u * uint32_t(chunk);
            dma16(reinterpret_cast<const uint8_t*>(src) + uint64_t(uint32_t(page)) * page_bytes, off, lds + 1024u * i);
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
    // Per-lane LDS byte addresses of the operand reads, each the address of
    // the read in tile buffer 0 / at key block 0 (the rest are instruction
    // offsets: 16 KB per buffer, 8 KB per 32-key half, 4 KB per 16-key block):
    //   kaddr[ks]  K (A of S^T): key col, chunk hl + 2 ks (swz(key) = swz(col))
    //   vaddr[dv]  V^T (A of O^T), d = dv / 2, second read = dv % 2
    //   qaddr[ks]  Q^T (B of S^T): row r of this wave, chunk hl + 2 ks
    // Made opaque so that the three K and three V buffers share them.
    uint32_t kaddr[8], vaddr[8], qaddr[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        kaddr[ks] = opaque(lds_addr((lds_u16*)(smem) + tile_off(col, hl + 2 * ks)));
        qaddr[ks] = opaque(lds_addr((lds_u16*)(smem) + 6 * kTileElems + tile_off(r, hl + 2 * ks)));
    }
#pragma unroll
    for (int dv = 0; dv < 8; ++dv)
        vaddr[dv] = opaque(lds_addr((lds_u16*)(smem) + 3 * kTileElems + tile_off(vkey + 8 * (dv % 2), 4 * (dv / 2) + vchunk) + vsub));

    // Q rows of this wave into LDS (same 16-byte global-to-LDS loads: row
    // 32 wave + 4 i + L / 16, chunk column L % 16 for lane L of load i)
    lds_u16* const Qs = (lds_u16*)(smem) + 6 * kTileElems;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 32 * wave + 4 * i + lrow;
        const int qt_ = t0 + row / G;
        const int qh = kvh * G + row % G;
        const uint32_t qoff = uint32_t(((uint32_t(qh) * uint32_t(a.C) + uint32_t(min(qt_, a.C - 1))) * kCD) * 2u)
                              + 16u * uint32_t((lane & 15) ^ swz(row));
        dma16(a.q + int64_t(b) * a.Hq * a.C * kCD, qoff, lds_addr(Qs + (32 * wave + 4 * i) * kCD));
    }

    // O^T += V^T P^T of one tile; p[2 half + qq] covers keys 32 half + 16 qq ..
    // + 15, taken as 4 hl + 0..3 and 8 + 4 hl + 0..3 (the order the lanes hold
    // the scores in); the V^T operand reads use the same key order
    auto accumulate = [&](auto vbuf, const u32x4_t (&p)[4]) {
        constexpr uint32_t VB = decltype(vbuf)::value * kTileElems * 2;
#pragma unroll
        for (int hq = 0; hq < 4; ++hq) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x2_t x0 = lds_read_tr(vaddr[2 * d] + VB + hq * 4096);
                const u32x2_t x1 = lds_read_tr(vaddr[2 * d + 1] + VB + hq * 4096);
                const u32x4_t vA = u32x4_t{x0.x, x0.y, x1.x, x1.y};
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vA), as_bf16x8(p[hq]), o[d], 0, 0, 0);
            }
        }
    };

    // Online softmax of one tile's scores (raw units; the scale is positive):
    // causal / window mask on the diagonal tiles, lazy running max (moved only
    // when the tile's max exceeds it by kLazyC, in log2 units), P as bf16 B
    // operands, running sum.  Returns the factor the running output must be
    // multiplied by before this tile's P V is added (1 unless the max moved).
    auto softmax = [&](auto masked, int k0, f32x16_t (&s)[2], u32x4_t (&p)[4]) -> float {
        if constexpr (!decltype(masked)::value) {
            // First try the running max as it stands: if no P of the wave
            // exceeds 2^kLazyC (every lane's sum of its 32 P is at most that),
            // no row's max moves by the lazy rule below, and these are its P
            // bit for bit.  Otherwise (the first tile of a row, a max that
            // jumped, a NaN) the general path recomputes the tile.
            const float neg_m = -m;
            float psum = 0.0f;
            u32x4_t pt[4];
#pragma unroll
            for (int hq = 0; hq < 4; ++hq) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[e] = exp2_fast(fmaf(s[hq / 2][8 * (hq % 2) + e], a.scale_log2, neg_m));
                    psum += x[e];
                }
                pt[hq] = u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                 pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
            }
            if (__builtin_amdgcn_ballot_w64(!(psum <= kLazyP)) == 0) {
#pragma unroll
                for (int hq = 0; hq < 4; ++hq) p[hq] = pt[hq];
                l += psum;
                return 1.0f;
            }
        }
        if constexpr (decltype(masked)::value) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + half * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
                    s[half][e] = key <= limit && (!WIN || key >= lo_lim) ? s[half][e] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[half][e]);
        mx = max_halves(mx) * a.scale_log2;
        const float m_new = mx > m + kLazyC ? mx : m;
        const float c = exp2_fast(m - m_new);
        const float neg_m = -m_new;
        float psum = 0.0f;
#pragma unroll
        for (int hq = 0; hq < 4; ++hq) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = exp2_fast(fmaf(s[hq / 2][8 * (hq % 2) + e], a.scale_log2, neg_m));
                psum += x[e];
            }
            p[hq] = u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                            pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        }
        l = l * c + psum;
        m = m_new;
        return c;
    };

    // Two groups of waves in ping-pong.  Waves w and w + 4 share a SIMD;
    // each runs, per key tile j, a matrix phase M_j (O += V_{j-1} P_{j-1},
    // then S_j = K_j Q^T: 32 products) and a softmax phase V_j (vector ALU:
    // S_j -> P_j, running max / sum, output rescale); a final step adds the
    // last tile's P V.  Interval j ends with the one workgroup barrier of
    // tile j: in it group 0 (waves 0-3) runs M_j then V_j, group 1 (waves
    // 4-7) runs V_{j-1} then M_j, so that while one wave of a SIMD is in a
    // softmax phase the other feeds the matrix core.
    // Tiles: K_j in K buffer j % 3, V_j in V buffer j % 3.  In interval j
    // group 0 loads K_{j+2} and group 1 loads V_{j+1}, the loads interleaved
    // with the products of M_j so that the matrix core hides their issue;
    // each wave waits for its loads of interval j - 1 at the end of interval
    // j, so a tile loaded in interval j - 2 is in place after barrier j - 1,
    // before interval j reads it.  The buffers overwritten in interval j
    // held K_{j-1} and V_{j-2}, last read by M_{j-1} before barrier j - 1.
    // K_0, K_1 and V_0 are loaded before the loop.  Page ids for a wave's
    // next loads are requested where no LDS wait of a matrix phase follows
    // before their own wait (group 0: at the start of its V_j; group 1: at
    // the end of its M_j) and waited for at the end of the wave's next
    // softmax phase, since a wait on an LDS read would also wait for an
    // outstanding scalar load.  Loads past the last tile re-read it
    // (harmless).
    const int grp = wave >> 2;
    auto tile_key = [&](int j) { return min(it0 + j, n_tiles - 1) * kKeys; };
    auto need_mask = [&](int j) {
        const int k0 = (it0 + j) * kKeys;
        return k0 + kKeys - 1 > wg_first_limit || (WIN && k0 < wg_lo_last);
    };
    lds_u16* const Kb = (lds_u16*)(smem);                    // K buffers 0, 1, 2
    lds_u16* const Vb = Kb + 3 * kTileElems;                 // V buffers 0, 1, 2

    f32x16_t sc[2];             // S of the current tile
    u32x4_t pb[4];              // P of the current tile
#pragma unroll
    for (int q = 0; q < 4; ++q) pb[q] = u32x4_t{0u, 0u, 0u, 0u};
    {   // V buffer 2 is read by M_0 (times P = 0): zero it so that no stale
        // LDS bits (a NaN pattern) can reach the accumulators
        u32x4_t* z = (u32x4_t*)(Vb + 2 * kTileElems);
        for (int e = tid; e < kTileElems / 8; e += kThreads) z[e] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // the tile this wave loads during M_j is tile j + 2 of K (group 0) or
    // tile j + 1 of V (group 1); pgL: its page (fast path)
    const uint16_t* const lsrc = grp ? a.v : a.k;
    const int lahead = grp ? 1 : 2;
    int32_t pgL = 0;
    if constexpr (FAST) {
        if (grp == 1) {
            const int32_t p0g = page_fast(tile_key(0));
            dma16x4(base_fast(a.k, tile_key(0), p0g), voff0, lds_addr(Kb + wr * kCD));
            dma16x4(base_fast(a.k, tile_key(1), page_fast(tile_key(1))), voff0, lds_addr(Kb + (kTileElems + wr * kCD)));
            dma16x4(base_fast(a.v, tile_key(0), p0g), voff0, lds_addr(Vb + wr * kCD));
        }
        pgL = page_fast(tile_key(lahead));
    } else {
        if (grp == 1) {
            load_general(a.k, tile_key(0), Kb);
            load_general(a.k, tile_key(1), Kb + kTileElems);
            load_general(a.v, tile_key(0), Vb);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0) lgkmcnt(0): K_0, K_1, V_0, Q, page ids
    __syncthreads();

    // M_j: the 16 products of O += V_{j-1} P_{j-1} (A operand V^T through
    // the transposing read) alternate with the 16 of S_j = K_j Q^T, the
    // operand reads about two products ahead of their use (one wave per SIMD
    // is in this phase, so nothing else hides the LDS latency); with DMA,
    // this wave's four tile loads go out after the first eight products
    auto matrix_phase = [&](auto dma, auto vbuf, auto kbuf, const uint8_t* lbase, uint32_t llds) {
        constexpr uint32_t VB = decltype(vbuf)::value * kTileElems * 2;
        constexpr uint32_t KB = decltype(kbuf)::value * kTileElems * 2;
        u32x4_t va[16], ka[16], qa[8];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hq = i / 4, d = i % 4;
            const u32x2_t x0 = lds_read_tr(vaddr[2 * d] + VB + hq * 4096);
            const u32x2_t x1 = lds_read_tr(vaddr[2 * d + 1] + VB + hq * 4096);
            va[i] = u32x4_t{x0.x, x0.y, x1.x, x1.y};
            const int ks = i / 2, half = i % 2;
            if (half == 0) qa[ks] = lds_read16(qaddr[ks]);
            ka[i] = lds_read16(kaddr[ks] + KB + half * 8192);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hq = i / 4, d = i % 4;
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[i]), as_bf16x8(pb[hq]), o[d], 0, 0, 0);
            const int ks = i / 2, half = i % 2;
            const f32x16_t acc = ks == 0 ? f32x16_t{} : sc[half];
            sc[half] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[i]), as_bf16x8(qa[ks]), acc, 0, 0, 0);
            if constexpr (decltype(dma)::value) {
                if (i == 3) dma16x4(lbase, voff0, llds);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);          // operand reads of the first products
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // O product
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // S product
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // reads
        }
    };

    // softmax phase V_jt of this wave (its scores S_jt -> P_jt); group 0 also
    // requests the page ids of its next tile loads (waited for at the end)
    auto softmax_phase = [&](int jt) __attribute__((always_inline)) {
        if (FAST && grp == 0) pgL = page_fast(tile_key(jt + lahead + 1));
        const int k0 = (it0 + jt) * kKeys;
        const float c = need_mask(jt) ? softmax(std::true_type{}, k0, sc, pb)
                                      : softmax(std::false_type{}, k0, sc, pb);
        if (c < 1.0f) {
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[d][e] *= c;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) pin(pb[q]);
        __builtin_amdgcn_s_waitcnt(0xc07f);                       // lgkmcnt(0): the page ids
    };
    // interval j < n (PAR = j % 3): group 0 runs M_j then V_j, group 1 runs
    // V_{j-1} then M_j, then one barrier
    auto interval = [&](auto par, int j) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        using VBUF = std::integral_constant<int, (PAR + 2) % 3>;        // V_{j-1}
        using KBUF = std::integral_constant<int, PAR>;                  // K_j
        if (grp == 1 && j > 0) softmax_phase(j - 1);
        lds_u16* const ldst = grp ? Vb + ((PAR + 1) % 3) * kTileElems : Kb + ((PAR + 2) % 3) * kTileElems;
        const int lkey = tile_key(j + lahead);
        if constexpr (FAST) {
            matrix_phase(std::true_type{}, VBUF{}, KBUF{}, base_fast(lsrc, lkey, pgL), lds_addr(ldst + wr * kCD));
        } else {
            load_general(lsrc, lkey, ldst);
            matrix_phase(std::false_type{}, VBUF{}, KBUF{}, nullptr, 0u);
        }
        pin(sc[0]);
        pin(sc[1]);
        // group 1's page ids for M_{j+1}: requested now, after this phase's
        // LDS reads, waited for at the end of its V_j
        if (FAST && grp == 1) pgL = page_fast(tile_key(j + lahead + 1));
        if (grp == 0) softmax_phase(j);
        // this wave's loads of interval j - 1 (first read in interval j + 1);
        // those of interval j may stay in flight
        __builtin_amdgcn_s_waitcnt(0x0f74);                       // vmcnt(4)
        if (FAST && grp == 1 && j == n - 1) {
            // V_{n-1} (loaded by this wave's group in interval n - 2, or before
            // the loop): zero this wave's rows of it past the workgroup's last
            // key before M_n reads them
            const int first = wg_last_key - (it0 + j) * kKeys + 1;
            uint32_t* zb = (uint32_t*)(Vb + PAR * kTileElems);
            for (int rr = max(first, wr); rr < wr + 16; ++rr)
                for (int e = lane; e < kCD / 2; e += 64) zb[rr * (kCD / 2) + e] = 0u;
        }
        __syncthreads();
    };
    int j = 0;
    for (; j + 3 <= n; j += 3) {
        interval(std::integral_constant<int, 0>{}, j);
        interval(std::integral_constant<int, 1>{}, j + 1);
        interval(std::integral_constant<int, 2>{}, j + 2);
    }
    if (j < n) interval(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n) interval(std::integral_constant<int, 1>{}, j + 1);
    // interval n: group 1's V_{n-1}, then every wave's last P V (tile n - 1,
    // in V buffer (n - 1) % 3)
    if (grp == 1) softmax_phase(n - 1);
    {
        const int lb = (n - 1) % 3;
        if (lb == 0) accumulate(std::integral_constant<int, 0>{}, pb);
        else if (lb == 1) accumulate(std::integral_constant<int, 1>{}, pb);
        else accumulate(std::integral_constant<int, 2>{}, pb);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): no load may outlive the kernel

    // ---- normalise and store: lane holds dims 32 d + 8 (e / 4) + 4 hl + e % 4 of its row
    const float lt = sum_halves(l);
    if (S > 1) {
        store_partial(lt);
    } else if (t < a.C) {
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
    const int blocks = a.rows * a.Hkv * ((a.C + P - 1) / P) * a.kv_splits;
    if (blocks <= 0) return hipSuccess;
    switch (G) {
#define PKV_CHUNK(GG)                                                                                  \
        case GG:                                                                                       \
            if (a.bs >= 16) {                                                                          \
                if (a.window >= 0) hipLaunchKernelGGL((chunk_attention_kernel<GG, true, true>), dim3(blocks), dim3(kThreads), 0, s, a); \
                else hipLaunchKernelGGL((chunk_attention_kernel<GG, false, true>), dim3(blocks), dim3(kThreads), 0, s, a); \
            } else {                                                                                   \
                if (a.window >= 0) hipLaunchKernelGGL((chunk_attention_kernel<GG, true, false>), dim3(blocks), dim3(kThreads), 0, s, a); \
                else hipLaunchKernelGGL((chunk_attention_kernel<GG, false, false>), dim3(blocks), dim3(kThreads), 0, s, a); \
            }                                                                                          \
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
