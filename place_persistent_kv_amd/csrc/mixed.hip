// Mixed-format paged K/V for gfx950: per-page storage, append, conversion of
// selected pages and decode attention.
//
// "Persistent input/output feedback", "Optional heterogeneous paged KV": every
// append chooses the storage of the pages it creates (dense, or affine INT8,
// UINT8, INT4, UINT4, INT2, UINT2 with one scalar scale and zero point); the
// choice is stored with each new page, so successive appends may use
// different formats without converting earlier pages; quantisation rounds
// ties to even and saturates.  Section "Selected-block quantization": chosen
// pages are re-encoded from their dense or affine payload, K and V each to
// its own format, rows past the valid prefix becoming the new format's zero.
// "Custom, quantized, and persistent values", "Struct types and byte-encodable
// layouts": codes are packed least-significant bits first, signed codes in
// two's complement; a code is worth (code - zero_point) * scale.
//
// Layout: each (page, head) owns a slot of block_size * D * 2 bytes (a dense
// 16-bit page) and a page's rows are packed from the start of the slot, row t
// at byte t * D * bits / 8.  A pool of BF16 pages is byte for byte a bf16
// pool.  PageDesc[page] (16 bytes) holds the K and V storages, scales and
// zero points.
//
// Decode: 4 waves per (row, kv head, split); each wave streams its quarter of
// the split in sub-steps of 16 tokens of one page, eight lanes per row, lane j
// owning dims 8j..8j+7 and 64+8j..64+8j+7.  A lane loads 2 x 2 * bits bytes of
// each of its rows, so every load instruction reads whole row segments.  The
// wave walks its sub-steps in runs of one (K bits, V bits) class: each class
// has its own pipelined loop (V rows of a group in flight while its K rows are
// scored, K rows of the next group while its V rows are summed), and a group
// is two sub-steps when K and V have at most 8 bits, so narrow pages keep as
// many bytes in flight as dense ones in the same registers.  Page ids and
// descriptors of a group are read one group before its loads are issued.
// Dense BF16 pages use v_dot2_f32_bf16 with the bf16 query.  Every other
// storage is brought to fp16 pairs: F16 pages as stored, affine codes as the
// exact integers c - z (a code u enters as the fp16 number 1024 + u, bit
// pattern 0x6400 | u, built with v_perm_b32 / v_and_or_b32, and one packed
// fp16 add of -(1024 + z), bit pattern 0xE400 | z, removes the offset exactly;
// signed codes are offset to unsigned by flipping their top bit).  Q.K then
// uses v_dot2_f32_f16 against the query scaled by a power of two (exact in
// fp16; the largest |q| lands in [128, 256)), and the page's scale multiplies
// the score; P.V multiplies the fp16 values straight into the float32 sums
// (v_fma_mix_f32) with the value scale folded into p.  Both query copies live
// in LDS and are read at each use, which keeps the kernel at two waves per
// SIMD for four query heads per K/V head.

#include "device_common.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kThreadsM = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));   // nearest-even
}

// Stored bits of 16 consecutive elements x[0..15] in storage `st`, packed
// into 16 * bits / 32 dwords (least-significant bits first).
__device__ __forceinline__ void encode16(const float* x, int st, float scale, int zero, uint32_t* w) {
    const int nb = storage_bits(st);
    if (nb == 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = st == kStBF16 ? f32_to_bf16_rne(x[2 * i]) : f32_to_f16_bits(x[2 * i]);
            const uint32_t hi = st == kStBF16 ? f32_to_bf16_rne(x[2 * i + 1]) : f32_to_f16_bits(x[2 * i + 1]);
            w[i] = lo | (hi << 16);
        }
        return;
    }
    const bool sgn = storage_signed(st);
    const float lo = sgn ? -float(1 << (nb - 1)) : 0.0f;
    const float hi = sgn ? float((1 << (nb - 1)) - 1) : float((1 << nb) - 1);
    const uint32_t mask = (1u << nb) - 1u;
    const int per = 32 / nb;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        // correctly rounded float32 divide, ties to even, saturate
        float c = rintf(x[e] / scale) + float(zero);
        c = fminf(fmaxf(c, lo), hi);
        const uint32_t code = static_cast<uint32_t>(static_cast<int32_t>(c)) & mask;
        w[e / per] |= code << (nb * (e % per));
    }
}

// Values of 16 consecutive stored elements (dwords w, storage st) as float32;
// affine codes as one float32 multiply (code - zero) * scale.
__device__ __forceinline__ void decode16(const uint32_t* w, int st, float scale, int zero, float* x) {
    const int nb = storage_bits(st);
    if (nb == 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (st == kStBF16) {
                x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            } else {
                x[2 * i] = float(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i])));
                x[2 * i + 1] = float(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
            }
        }
        return;
    }
    const bool sgn = storage_signed(st);
    const uint32_t mask = (1u << nb) - 1u;
    const int per = 32 / nb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        int32_t c = static_cast<int32_t>((w[e / per] >> (nb * (e % per))) & mask);
        if (sgn && c >= (1 << (nb - 1))) c -= 1 << nb;
        x[e] = __fmul_rn(float(c - zero), scale);
    }
}

// ---------------------------------------------------------------------------
// Append: one thread per (tensor, row, head, token, 16-element chunk).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreadsM) void mixed_append_kernel(MixedAppendArgs a, int64_t total) {
    const int nch = a.D / 16;
    const int64_t per_tensor = total / 2;
    const int64_t slot_bytes = int64_t(a.bs) * a.D * 2;
    for (int64_t i = int64_t(blockIdx.x) * kThreadsM + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kThreadsM) {
        const int which = i >= per_tensor;                  // 0: K, 1: V
        const int64_t k = which ? i - per_tensor : i;
        const int c = static_cast<int>(k % nch);
        const int64_t r = k / nch;                          // source row (b, h, t)
        const int t = static_cast<int>(r % a.n);
        const int64_t bh = r / a.n;
        const int h = static_cast<int>(bh % a.H);
        const int b = static_cast<int>(bh / a.H);
        const int p = a.pos[b] + t;
        const int blk = p / a.bs;
        const int slot = p - blk * a.bs;
        const int page = a.page_table[int64_t(a.row0 + b) * a.maxb + blk];
        // a page whose first slot this append writes takes the call's format
        const bool fresh = blk * a.bs >= a.pos[b];
        int st;
        float scale;
        int zero;
        if (fresh) {
            st = which ? a.fmt.v_st : a.fmt.k_st;
            scale = which ? a.fmt.v_scale : a.fmt.k_scale;
            zero = which ? a.fmt.v_zero : a.fmt.k_zero;
        } else {
            const PageDesc d = a.desc[page];
            st = (which ? d.v_st : d.k_st) & 7;
            scale = which ? d.v_scale : d.k_scale;
            zero = which ? d.v_zero : d.k_zero;
        }
        const uint16_t* src = (which ? a.v_src : a.k_src) + r * a.D + c * 16;
        float x[16];
        const uint4 s0 = *reinterpret_cast<const uint4*>(src);
        const uint4 s1 = *reinterpret_cast<const uint4*>(src + 8);
        const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[2 * e] = bf16_bits_to_f32(sw[e] & 0xFFFFu);
            x[2 * e + 1] = bf16_bits_to_f32(sw[e] >> 16);
        }
        uint32_t w[8];
        encode16(x, st, scale, zero, w);
        const int nb = storage_bits(st);
        uint8_t* base = (which ? a.v_pool : a.k_pool) + (int64_t(page) * a.H + h) * slot_bytes;
        uint32_t* dst = reinterpret_cast<uint32_t*>(base + int64_t(slot) * a.D * nb / 8 + c * 2 * nb);
        const int ndw = nb / 2;
        for (int q = 0; q < ndw; ++q) dst[q] = w[q];
        if (fresh && slot == 0 && which == 0 && h == 0 && c == 0) a.desc[page] = a.fmt;
    }
}

// ---------------------------------------------------------------------------
// Conversion: one workgroup per (listed page, head).  The old rows are staged
// in LDS before any new byte is written (old and new rows overlap in the slot).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreadsM) void mixed_convert_kernel(MixedConvertArgs a) {
    extern __shared__ uint32_t s_old[];
    const int page = a.page[blockIdx.x];
    const int nv = a.valid[blockIdx.x];
    const int h = blockIdx.y;
    const PageDesc d = a.desc[page];
    const int ost = (a.which ? d.v_st : d.k_st) & 7;
    const float oscale = a.which ? d.v_scale : d.k_scale;
    const int ozero = a.which ? d.v_zero : d.k_zero;
    const int onb = storage_bits(ost);
    const int nnb = storage_bits(a.st);
    uint8_t* base = a.pool + (int64_t(page) * a.H + h) * (int64_t(a.bs) * a.D * 2);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(base);
    const int old_dw = nv * a.D * onb / 32;                 // dwords of the valid old rows
    for (int q = threadIdx.x; q < old_dw; q += kThreadsM) s_old[q] = src[q];
    __syncthreads();
    const int nch = a.D / 16;
    for (int q = threadIdx.x; q < a.bs * nch; q += kThreadsM) {
        const int row = q / nch;
        const int c = q - row * nch;
        float x[16];
        if (row < nv) {
            uint32_t w[8];
            const int odw = onb / 2;                        // dwords of 16 old elements
            const uint32_t* o = s_old + (row * a.D * onb / 8 + c * 2 * onb) / 4;
            for (int k = 0; k < 8; ++k) w[k] = k < odw ? o[k] : 0u;
            decode16(w, ost, oscale, ozero, x);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = 0.0f;
        }
        uint32_t w[8];
        encode16(x, a.st, a.scale, a.zero, w);
        uint32_t* dst = reinterpret_cast<uint32_t*>(base + int64_t(row) * a.D * nnb / 8 + c * 2 * nnb);
        const int ndw = nnb / 2;
        for (int k = 0; k < ndw; ++k) dst[k] = w[k];
    }
}

__global__ void mixed_desc_kernel(MixedDescArgs a) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.count) return;
    PageDesc d = a.desc[a.page[i]];
    if (a.set_k) {
        d.k_st = a.fmt.k_st;
        d.k_scale = a.fmt.k_scale;
        d.k_zero = a.fmt.k_zero;
    }
    if (a.set_v) {
        d.v_st = a.fmt.v_st;
        d.v_scale = a.fmt.v_scale;
        d.v_zero = a.fmt.v_zero;
    }
    a.desc[a.page[i]] = d;
}

// ---------------------------------------------------------------------------
// Decode attention over mixed pages
// ---------------------------------------------------------------------------
constexpr int kWavesM = 4;
constexpr int kDM = 128;
constexpr float kLazyM = 8.0f;   // rescale only when a score exceeds the running max by 2^8

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float group8_max(float x) {
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    return x;
}

// lane id recomputed at the point of use (volatile: not merged with other uses,
// so no copy of it stays live across the main loop)
__device__ __forceinline__ int lane_now() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t x, uint32_t y) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, x) + __builtin_bit_cast(f16x2_t, y));
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
    return float(__builtin_bit_cast(f16x2_t, w).x);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return float(__builtin_bit_cast(f16x2_t, w).y);
}

// A lane's 16 elements of one row (a: dims 8j..8j+7, b: dims 64+8j..64+8j+7,
// as loaded for storage class nb) as 8 fp16 pairs of natural dim order.
// Affine codes become c - z exactly: nz is the packed fp16 pair -(1024 + z'),
// z' the zero point in unsigned code units; flip offsets signed codes.
__device__ __forceinline__ void to_f16_pairs(u32x4_t a, u32x4_t b, int nb, uint32_t flip, uint32_t nz,
                                             uint32_t* out) {
    const uint32_t k6464 = 0x64646464u;
    if (nb == 16) {
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
        return;
    }
    if (nb == 8) {
        const uint32_t w[4] = {a.x ^ flip, a.y ^ flip, b.x ^ flip, b.y ^ flip};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = pk_add_f16(perm(w[i], k6464, 0x00050004u), nz);       // bytes 0, 1
            out[2 * i + 1] = pk_add_f16(perm(w[i], k6464, 0x00070006u), nz);   // bytes 2, 3
        }
        return;
    }
    if (nb == 4) {
        const uint32_t w[2] = {a.x ^ flip, b.x ^ flip};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w4 = w[i] >> 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // byte k: low nibble -> low half, high nibble -> high half
                const uint32_t x = perm(w[i], w4, 0x0C000C04u | (uint32_t(k) << 16) | uint32_t(k));
                out[4 * i + k] = pk_add_f16((x & 0x000F000Fu) | 0x64006400u, nz);
            }
        }
        return;
    }
    // 2-bit: one dword, dims 8j..8j+7 in the low half, 64+8j.. in the high half
    const uint32_t w = a.x ^ flip;
    const uint32_t w2 = w >> 2, w4 = w >> 4, w6 = w >> 6;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const uint32_t sel = 0x0C000C04u | (uint32_t(bb) << 16) | uint32_t(bb);
        const uint32_t x0 = perm(w, w2, sel);     // codes 4bb, 4bb + 1
        const uint32_t x1 = perm(w4, w6, sel);    // codes 4bb + 2, 4bb + 3
        out[2 * bb] = pk_add_f16((x0 & 0x00030003u) | 0x64006400u, nz);
        out[2 * bb + 1] = pk_add_f16((x1 & 0x00030003u) | 0x64006400u, nz);
    }
}

template <int G>
__global__ __launch_bounds__(256) void decode_mixed_kernel(DecodeArgs a) {
    __shared__ float s_o[kWavesM][G][kDM];
    __shared__ float s_ml[kWavesM][G][2];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int j = lane & 7;     // chunk of each half row

    const int work = blockIdx.x;
    const int kvh = work % a.Hkv;
    const int r = work / a.Hkv;
    int b, split;
    split_item(a.full_begin, a.tail_row, a.rows, r, b, split);
    const int L = a.len[b];
    const int nsplit = (L - split_base(L, a.window) + a.tps - 1) / a.tps;
    const int vis0 = visible_begin(L, a.window);
    const int t0 = split_base(L, a.window) + split * a.tps;
    const int t1 = min(L, t0 + a.tps);
    const int quarter = a.tps / kWavesM;
    const int wbeg = t0 + wave * quarter;
    const int wend = min(t1, wbeg + quarter);

    const uint8_t* __restrict__ K = static_cast<const uint8_t*>(a.k);
    const uint8_t* __restrict__ V = static_cast<const uint8_t*>(a.v);
    const PageDesc* __restrict__ desc = static_cast<const PageDesc*>(a.page_desc);
    const int32_t* __restrict__ pt = a.page_table + int64_t(b) * a.maxb;
    const int64_t slot_bytes = int64_t(a.bs) * kDM * 2;

    // query in LDS, read at every use: bf16 for dense BF16 pages, fp16 pairs of
    // q * 2^e for every other storage (2^-e, per head, in a register)
    __shared__ uint4 s_q[G][2][8];          // [head][half][lane chunk j]
    __shared__ uint4 s_qh[G][2][8];
    float qinv[G];
    {
        const uint16_t* Q = static_cast<const uint16_t*>(a.q) + (int64_t(b) * a.Hq + kvh * G) * kDM;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 qa = ld16(Q + g * kDM + j * 8);
            const uint4 qb = ld16(Q + g * kDM + 64 + j * 8);
            const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
            float mx = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fmaxf(fabsf(bf_lo(qw[k])), fabsf(bf_hi(qw[k]))));
            mx = group8_max(mx);
            const int E = __builtin_amdgcn_readfirstlane(mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0);
            const float up = __builtin_ldexpf(1.0f, 8 - E);   // largest |q| * up in [128, 256)
            qinv[g] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                    __builtin_bit_cast(int, __builtin_ldexpf(1.0f, E - 8))));
            uint32_t hw[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                hw[k] = f32_to_f16_bits(bf_lo(qw[k]) * up) | (f32_to_f16_bits(bf_hi(qw[k]) * up) << 16);
            if (threadIdx.x < 8) {
                s_q[g][0][j] = qa;
                s_q[g][1][j] = qb;
                s_qh[g][0][j] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                s_qh[g][1][j] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
            }
        }
    }
    __syncthreads();

    float m[G], l[G], o[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -FLT_MAX;
        l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[g][d] = 0.0f;
    }

    // Half-step pipeline over groups of sub-steps (16 tokens of one page
    // each): the V rows of a group are in flight while its K rows are scored,
    // and the K rows of the next group while its V rows are summed.  A group
    // is one sub-step, or two when both sub-steps hold K and V of at most 8
    // bits: their rows then share the 16 registers per lane that one dense
    // sub-step uses, so narrow pages keep as many bytes in flight.  The
    // prefetch after the last group re-reads the last sub-step.
    struct Fmt {
        int st, nb;              // storage and its bits (wave-uniform)
        float sc;                // scale (1 for dense pages)
        uint32_t flip, nz;       // signed-code offset, packed fp16 -(1024 + z')
    };
    struct Sub {
        int ts, page;            // first token, page
        Fmt kf, vf;
    };
    auto fmt_of = [&](const PageDesc& dd, bool v) {
        Fmt f;
        f.st = __builtin_amdgcn_readfirstlane((v ? dd.v_st : dd.k_st) & 7);
        f.nb = storage_bits(f.st);
        const bool aff = f.st >= kStI8;
        f.sc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                             __builtin_bit_cast(int, aff ? (v ? dd.v_scale : dd.k_scale) : 1.0f)));
        const bool sg = storage_signed(f.st);
        f.flip = sg ? (f.nb == 8 ? 0x80808080u : f.nb == 4 ? 0x88888888u : 0xAAAAAAAAu) : 0u;
        // -(1024 + z') in fp16 is 0xE400 | z' for 0 <= z' < 1024 (exponent 10, sign set)
        const uint32_t z = uint32_t((v ? dd.v_zero : dd.k_zero) + (sg ? (1 << (f.nb - 1)) : 0)) & 0x3FFu;
        f.nz = (0xE400u | z) * 0x00010001u;
        return f;
    };
    const int nsub = wbeg < wend ? (wend - wbeg + kSlabTokens - 1) / kSlabTokens : 0;
    // page ids and descriptors are wave-uniform: read through the scalar unit
    // (constant address space), so that waiting for them never waits for the
    // K/V rows in flight
    auto sub_of = [&](int i) {
        Sub u;
        u.ts = wbeg + i * kSlabTokens;
        u.page = *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
            reinterpret_cast<uintptr_t>(pt + (u.ts >> a.log2bs)));
        const PageDesc dd = __builtin_bit_cast(
            PageDesc, *reinterpret_cast<const __attribute__((address_space(4))) u32x4_t*>(
                          reinterpret_cast<uintptr_t>(desc + u.page)));
        u.kf = fmt_of(dd, false);
        u.vf = fmt_of(dd, true);
        return u;
    };
    const int64_t kvoff = int64_t(kvh) * slot_bytes;
    // Rows of a sub-step into a half buffer w[4]: dense rows take all four
    // vectors (row 0 halves, row 1 halves); narrow rows of slot s take w[2s]
    // (row 0) and w[2s + 1] (row 1), 8-bit as (lo.xy, hi.xy), 4-bit as (lo, -, hi, -),
    // 2-bit as one dword (lo | hi << 16).  Rows are clamped to the split's last token.
    auto load_sub = [&](u32x4_t* w, const uint8_t* base, const Sub& u, int nb, int slot) {
        // lane offsets are recomputed here (not hoisted: each storage would keep its own)
        const int lane_l = lane_now();
        const int gl = lane_l >> 3, jl = lane_l & 7;
        const int in_page = u.ts & (a.bs - 1);
        const int last = t1 - 1 - u.ts;
        const int r0 = in_page + min(gl, last), r1 = in_page + min(gl + 8, last);
        const uint8_t* head = base + int64_t(u.page) * a.Hkv * slot_bytes + kvoff;
        const uint8_t* p0 = head + (r0 * 16 + jl) * nb;
        const uint8_t* p1 = head + (r1 * 16 + jl) * nb;
        if (nb == 16) {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p0));
            w[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p0 + 128));
            w[2] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p1));
            w[3] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p1 + 128));
        } else if (nb == 8) {
            const u32x2_t a0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p0));
            const u32x2_t b0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p0 + 64));
            const u32x2_t a1 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p1));
            const u32x2_t b1 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p1 + 64));
            w[2 * slot] = u32x4_t{a0.x, a0.y, b0.x, b0.y};
            w[2 * slot + 1] = u32x4_t{a1.x, a1.y, b1.x, b1.y};
        } else if (nb == 4) {
            w[2 * slot].x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p0));
            w[2 * slot].z = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p0 + 32));
            w[2 * slot + 1].x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p1));
            w[2 * slot + 1].z = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p1 + 32));
        } else {
            const uint32_t a0 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p0));
            const uint32_t b0 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p0 + 16));
            const uint32_t a1 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p1));
            const uint32_t b1 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p1 + 16));
            w[2 * slot].x = a0 | (b0 << 16);
            w[2 * slot + 1].x = a1 | (b1 << 16);
        }
    };
    // fp16 pairs (natural dim order) of a narrow row held in one vector
    auto narrow_pairs = [](u32x4_t r, const Fmt& f, int nb, uint32_t* out) {
        to_f16_pairs(u32x4_t{r.x, r.y, 0u, 0u}, u32x4_t{r.z, r.w, 0u, 0u}, nb, f.flip, f.nz, out);
    };
    // scores (log2 units) of rows 0 and 1 of a sub-step of K bits nb held in slot `slot`
    auto scores = [&](const u32x4_t* w, const Fmt& f, int nb, int slot, float* x0, float* x1) {
        if (nb == 16 && f.st == kStBF16) {
            const int jj = lane_now() & 7;          // fresh: keeps the LDS query reads in the loop
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint4 qa = s_q[g][0][jj], qb = s_q[g][1][jj];
                float x = 0.0f, y = 0.0f;
                x = dot2_bf16(qa.x, w[0].x, x);
                y = dot2_bf16(qa.x, w[2].x, y);
                x = dot2_bf16(qa.y, w[0].y, x);
                y = dot2_bf16(qa.y, w[2].y, y);
                x = dot2_bf16(qa.z, w[0].z, x);
                y = dot2_bf16(qa.z, w[2].z, y);
                x = dot2_bf16(qa.w, w[0].w, x);
                y = dot2_bf16(qa.w, w[2].w, y);
                x = dot2_bf16(qb.x, w[1].x, x);
                y = dot2_bf16(qb.x, w[3].x, y);
                x = dot2_bf16(qb.y, w[1].y, x);
                y = dot2_bf16(qb.y, w[3].y, y);
                x = dot2_bf16(qb.z, w[1].z, x);
                y = dot2_bf16(qb.z, w[3].z, y);
                x = dot2_bf16(qb.w, w[1].w, x);
                y = dot2_bf16(qb.w, w[3].w, y);
                x0[g] = group8_sum(x) * a.scale_log2;
                x1[g] = group8_sum(y) * a.scale_log2;
            }
            return;
        }
        uint32_t k0[8], k1[8];
        if (nb == 16) {
            to_f16_pairs(w[0], w[1], 16, 0u, 0u, k0);
            to_f16_pairs(w[2], w[3], 16, 0u, 0u, k1);
        } else {
            narrow_pairs(w[2 * slot], f, nb, k0);
            narrow_pairs(w[2 * slot + 1], f, nb, k1);
        }
        const float ksc = f.sc * a.scale_log2;
        const int jj = lane_now() & 7;              // fresh: keeps the LDS query reads in the loop
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 ha = s_qh[g][0][jj], hb = s_qh[g][1][jj];
            const uint32_t qh[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
            float x = 0.0f, y = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                x = dot2_f16(qh[k], k0[k], x);
                y = dot2_f16(qh[k], k1[k], y);
            }
            const float sc = ksc * qinv[g];
            x0[g] = group8_sum(x) * sc;
            x1[g] = group8_sum(y) * sc;
        }
    };
    // o += p0 * v(row 0) + p1 * v(row 1) for a sub-step of V bits nb held in slot `slot`
    auto values = [&](const u32x4_t* w, const Fmt& f, int nb, int slot, const float* p0, const float* p1) {
        auto accumulate = [&](int d, float x0, float x1) {
#pragma unroll
            for (int g = 0; g < G; ++g) o[g][d] = fmaf(p1[g], x1, fmaf(p0[g], x0, o[g][d]));
        };
        if (nb == 16 && f.st == kStBF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                accumulate(2 * k, bf_lo(w[0][k]), bf_lo(w[2][k]));
                accumulate(2 * k + 1, bf_hi(w[0][k]), bf_hi(w[2][k]));
                accumulate(8 + 2 * k, bf_lo(w[1][k]), bf_lo(w[3][k]));
                accumulate(8 + 2 * k + 1, bf_hi(w[1][k]), bf_hi(w[3][k]));
            }
            return;
        }
        uint32_t w0[8], w1[8];
        if (nb == 16) {
            to_f16_pairs(w[0], w[1], 16, 0u, 0u, w0);
            to_f16_pairs(w[2], w[3], 16, 0u, 0u, w1);
        } else {
            narrow_pairs(w[2 * slot], f, nb, w0);
            narrow_pairs(w[2 * slot + 1], f, nb, w1);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            accumulate(2 * k, f16_lo(w0[k]), f16_lo(w1[k]));
            accumulate(2 * k + 1, f16_hi(w0[k]), f16_hi(w1[k]));
        }
    };
    // one softmax update for the (up to) four rows of a group; s[r][g] becomes
    // p times the V scale of the row's sub-step
    auto softmax = [&](float (*s)[G], int ts0, int np, float vs0, float vs1) {
        const int grp = lane_now() >> 3;
        const int ts1 = ts0 + kSlabTokens;
        const bool live[4] = {ts0 + grp < t1 && ts0 + grp >= vis0, ts0 + 8 + grp < t1 && ts0 + 8 + grp >= vis0,
                              np == 2 && ts1 + grp < t1 && ts1 + grp >= vis0,
                              np == 2 && ts1 + 8 + grp < t1 && ts1 + 8 + grp >= vis0};
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r][g] = live[r] ? s[r][g] : -INFINITY;
            const float mx = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
            if (mx > m[g] + kLazyM) {
                const float c = exp2_fast(m[g] - mx);
                l[g] *= c;
#pragma unroll
                for (int d = 0; d < 16; ++d) o[g][d] *= c;
                m[g] = mx;
            }
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[r][g] = exp2_fast(s[r][g] - m[g]);
                ps += s[r][g];
            }
            l[g] += ps;
            s[0][g] *= vs0;
            s[1][g] *= vs0;
            s[2][g] *= vs1;
            s[3][g] *= vs1;
        }
    };
    auto same_class = [](const Sub& u, int kb, int vb) { return u.kf.nb == kb && u.vf.nb == vb; };

    // A run of groups whose sub-steps all have K bits KB and V bits VB, two
    // sub-steps per group when both are at most 8 bits (the second may be
    // absent at the end of the run: its rows are then masked and its loads
    // repeat the first's), pipelined as above.  Returns the first sub-step it
    // did not process.
    auto run = [&](auto kbc, auto vbc, int i) -> int {
        constexpr int KB = decltype(kbc)::value, VB = decltype(vbc)::value;
        constexpr int P = KB <= 8 && VB <= 8 ? 2 : 1;
        u32x4_t kh[4], vh[4];    // components a storage does not use are never read
        // the second sub-step of the group at c0 (or c0 again when absent)
        auto second = [&](int at, const Sub& first, bool& has) {
            has = false;
            if (P == 1 || at + 1 >= nsub) return first;
            const Sub u = sub_of(at + 1);
            has = same_class(u, KB, VB);
            return has ? u : first;
        };
        // current group (c0, c1, h1) and the next one (n0, n1, nh1), resolved
        // one group ahead so that the page and format reads of a group are
        // issued a whole group before its loads need them
        Sub c0 = sub_of(i);
        bool h1;
        Sub c1 = second(i, c0, h1);
        int ni = i + (h1 ? 2 : 1);
        bool cont = ni < nsub;
        Sub n0 = c0, n1 = c1;
        bool nh1 = false;
        if (cont) {
            n0 = sub_of(ni);
            cont = same_class(n0, KB, VB);
            if (cont) n1 = second(ni, n0, nh1);
        }
        load_sub(kh, K, c0, KB, 0);
        if (P == 2) load_sub(kh, K, c1, KB, 1);
        for (;;) {
            load_sub(vh, V, c0, VB, 0);
            if (P == 2) load_sub(vh, V, c1, VB, 1);
            float sc[4][G];
            scores(kh, c0.kf, KB, 0, sc[0], sc[1]);
            if (P == 2) scores(kh, c1.kf, KB, 1, sc[2], sc[3]);
            softmax(sc, c0.ts, h1 ? 2 : 1, c0.vf.sc, c1.vf.sc);
            if (cont) {
                load_sub(kh, K, n0, KB, 0);
                if (P == 2) load_sub(kh, K, n1, KB, 1);
            }
            // the group after next
            const int nni = ni + (nh1 ? 2 : 1);
            bool mcont = cont && nni < nsub;
            Sub m0 = n0, m1 = n1;
            bool mh1 = false;
            if (mcont) {
                m0 = sub_of(nni);
                mcont = same_class(m0, KB, VB);
                if (mcont) m1 = second(nni, m0, mh1);
            }
            values(vh, c0.vf, VB, 0, sc[0], sc[1]);
            if (P == 2) values(vh, c1.vf, VB, 1, sc[2], sc[3]);
            if (!cont) return ni;
            i = ni;
            c0 = n0;
            c1 = n1;
            h1 = nh1;
            ni = nni;
            n0 = m0;
            n1 = m1;
            nh1 = mh1;
            cont = mcont;
        }
    };
    using I16 = std::integral_constant<int, 16>;
    using I8 = std::integral_constant<int, 8>;
    using I4 = std::integral_constant<int, 4>;
    using I2 = std::integral_constant<int, 2>;
    for (int i = 0; i < nsub;) {
        const Sub u = sub_of(i);
        const int kb = u.kf.nb, vb = u.vf.nb;
#define PKV_RUN(KBV, VBV, KT, VT) \
        if (kb == KBV && vb == VBV) { i = run(KT{}, VT{}, i); continue; }
        PKV_RUN(16, 16, I16, I16) PKV_RUN(16, 8, I16, I8) PKV_RUN(16, 4, I16, I4) PKV_RUN(16, 2, I16, I2)
        PKV_RUN(8, 16, I8, I16) PKV_RUN(4, 16, I4, I16) PKV_RUN(2, 16, I2, I16)
        PKV_RUN(8, 8, I8, I8) PKV_RUN(8, 4, I8, I4) PKV_RUN(8, 2, I8, I2)
        PKV_RUN(4, 8, I4, I8) PKV_RUN(4, 4, I4, I4) PKV_RUN(4, 2, I4, I2)
        PKV_RUN(2, 8, I2, I8) PKV_RUN(2, 4, I2, I4)
#undef PKV_RUN
        i = run(I2{}, I2{}, i);      // the remaining pair, (2, 2)
    }

    const int lane_e = lane_now();
    const int grp_e = lane_e >> 3, j_e = lane_e & 7;
    // merge the eight token groups of the wave (lanes with the same j)
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
    if (grp_e == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                s_o[wave][g][j_e * 8 + d] = o[g][d];
                s_o[wave][g][64 + j_e * 8 + d] = o[g][8 + d];
            }
            if (j_e == 0) {
                s_ml[wave][g][0] = m[g];
                s_ml[wave][g][1] = l[g];
            }
        }
    }
    __syncthreads();

    // merge the four waves; thread t handles (g, d) pairs t, t + 256, ...
    for (int e = wave * 64 + lane_e; e < G * kDM; e += 256) {
        const int g = e / kDM;
        const int d = e % kDM;
        float mn = -FLT_MAX;
#pragma unroll
        for (int w = 0; w < kWavesM; ++w) mn = fmaxf(mn, s_ml[w][g][0]);
        float ls = 0.0f, os = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesM; ++w) {
            const float c = exp2_fast(s_ml[w][g][0] - mn);
            ls += s_ml[w][g][1] * c;
            os += s_o[w][g][d] * c;
        }
        const int hh = kvh * G + g;
        const int64_t bh = int64_t(b) * a.Hq + hh;
        if (nsplit == 1) {
            const float y = os / ls;
            if (a.out_f32) static_cast<float*>(a.out)[bh * kDM + d] = y;
            else static_cast<uint16_t*>(a.out)[bh * kDM + d] = f32_to_bf16_rne(y);
        } else {
            const int64_t slot = bh * a.S_max + split;
            a.ws_o[slot * kDM + d] = os;
            if (d == 0) {
                a.ws_ml[slot * 2 + 0] = mn;
                a.ws_ml[slot * 2 + 1] = ls;
            }
        }
    }
}

dim3 grid_for_m(int64_t total) {
    int64_t blocks = (total + kThreadsM - 1) / kThreadsM;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return dim3(static_cast<unsigned>(blocks));
}

}  // namespace

hipError_t launch_mixed_append(const MixedAppendArgs& a, hipStream_t s) {
    const int64_t total = 2 * int64_t(a.rows) * a.H * a.n * (a.D / 16);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(mixed_append_kernel, grid_for_m(total), dim3(kThreadsM), 0, s, a, total);
    return hipGetLastError();
}

hipError_t launch_mixed_convert(const MixedConvertArgs& a, hipStream_t s) {
    if (a.count <= 0 || a.H <= 0) return hipSuccess;
    const size_t lds = size_t(a.bs) * a.D * 2;
    hipLaunchKernelGGL(mixed_convert_kernel, dim3(a.count, a.H), dim3(kThreadsM), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_mixed_desc(const MixedDescArgs& a, hipStream_t s) {
    if (a.count <= 0) return hipSuccess;
    hipLaunchKernelGGL(mixed_desc_kernel, dim3((a.count + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

bool mixed_decode_supported(int D, int G, int bs) {
    if (D != kDM) return false;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    return bs >= kSlabTokens && (bs & (bs - 1)) == 0;
}

hipError_t launch_decode_mixed(const DecodeArgs& a, int G, int total_work, hipStream_t s) {
    if (total_work <= 0) return hipSuccess;
    const dim3 grid(total_work), block(256);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_mixed_kernel<1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_mixed_kernel<2>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_mixed_kernel<4>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_mixed_kernel<8>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
