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
// parameters.  A wave takes its tokens in groups of 16 (one page holds a
// whole group: block_size is a power of two >= 16).
//
// Q.K on the matrix cores, in 4x4x4 blocks (v_mfma_f32_4x4x4bf16_1k): block
// (token group tg of 4, 32-dim block qb) multiplies the 4 query heads (rows;
// query split into bf16 high + low parts for float32-grade products) by the
// raw codes of 4 tokens, 4 dims per step, 8 steps per block.  A code c enters
// as the bf16 number 128 + c, whose bit pattern is 0x4300 | c, so two codes
// become one operand word with one v_and_or_b32.  With qs_b = sum of q over
// block b the dequantised product is
//     q . k = sum_b s_b * (S_b - (128 + z_b) * qs_b),   S_b = sum_{d in b} q_d (128 + c_d)
// Each lane loads its own token's 16 code bytes and (scale, zero) of one
// block, applies that block's dequantisation to its 4 head results, and a
// row rotation sums the four blocks; the lane then keeps one (token, head)
// score, so every lane of the softmax carries a distinct score (a 16-row MFMA
// would leave 12 of its 16 rows empty at 4 heads).
//
// P.V on the matrix cores as well, in the same 4x4x4 blocks: block
// (token quad tq, 32-dim block beta) multiplies the probabilities of 4 heads
// times the scale of block beta (rows; bf16 high + low parts) by the raw
// codes 128 + c of 4 tokens, each lane holding one code word (8 dims) of
// 4 consecutive rows, so that one instruction covers 64 dims and eight cover
// the lane's word.  With x = p * s per (head, token, block)
//     sum_t p s (c - z) = sum_t x (128 + c) - sum_t x 128 - sum_t x z
// the middle term is a ninth product (codes replaced by 128, so it matches
// the first one's operands exactly) and the zero-point term a vector FMA.
// The accumulators stay per token quad and are summed over the quads once,
// at the end.  The running max of every head is wave-uniform (a reduction
// over the head's lanes plus v_readlane), so the lazy rescale is a uniform
// branch, taken only when one ballot finds a head whose maximum rose.
//
// Loads: K codes as 16 bytes of one row per lane, K parameters as one dword,
// V codes and V parameters as contiguous 16 bytes / 4 bytes per lane (the
// whole group in one instruction each), passed through LDS to the lanes the
// P.V blocks need them in.  The query operands sit in LDS too, which keeps
// the kernel at four waves per SIMD; two groups are in flight per wave.
// The split / merge structure is that of the bf16 fast kernel.

#include "device_common.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kWaves4 = 4;
constexpr int kD4 = 128;
constexpr int kGroup = 16;       // tokens per Q.K step
constexpr float kLazy4 = 8.0f;
constexpr int kStages = 2;      // groups in flight per wave (register stages)

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_4x4x4bf16_1k: 16 independent 4x4x4 products; lane 4b + i holds
// A_b[i][0..3], lane 4b + j holds B_b[0..3][j] and D_b[0..3][j] (checked on the device)
__device__ __forceinline__ f32x4_t mfma4(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                  0, 0, 0);
}

// A constant in a VGPR, opaque to the optimiser, so that (x & m) | c with
// register operands becomes one v_and_or_b32 (literal constants cannot be
// VOP3 operands here, which would split it into an and plus an or).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "n"(c));
    return r;
}

// DPP move without an old value (every lane of the patterns used here reads
// a lane of its own row), so that it can fold into the instruction using it
template <int CTRL>
__device__ __forceinline__ float dppm(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// x (op) the value of lane l ^ 32 / l ^ 16, on the vector ALU (gfx950
// v_permlane{32,16}_swap: the two results hold, per lane, the values of the
// lane and of its partner)
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A wave-uniform 32-bit load through the scalar unit (constant address
// space: an s_load, counted apart from the vector loads in flight)
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}

template <int G>
__global__ __launch_bounds__(256, (G <= 4 ? 4 : 2)) void decode_int4_kernel(Int4DecodeArgs a) {
    constexpr int HP = G < 4 ? G : 4;           // heads per pass (rows of the 4x4 blocks)
    constexpr int NP = (G + 3) / 4;             // passes

    __shared__ float s_p[kWaves4][kStages][4 * NP][kGroup];   // probabilities [stage][head][token]; rows >= G stay 0
    // a group's V codes (row r at dword 16 (r + r / 4): the pad keeps the four
    // rows one P.V read spans in different banks) and V parameters
    __shared__ __align__(16) uint32_t s_vc[kWaves4][kStages][16 * 20];
    __shared__ uint32_t s_vpar[kWaves4][kStages][64];
    __shared__ float s_o[kWaves4][G][kD4];
    __shared__ float s_ml[kWaves4][G][2];

    // work-item and workgroup ids straight from the hardware registers: this
    // file is built without IEEE mode, and the device library's id functions
    // (built with it) would not be inlined, leaving the workgroup id in a VGPR
    const int tid = static_cast<int>(__builtin_amdgcn_workitem_id_x());
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // 16 blocks b = 4 tg + qb of 4 lanes.  Q.K: lane 16 tg + 4 qb + jj holds
    // token 4 tg + jj of the group, 32-dim block qb (B operand and result), and
    // head row jj of block qb (A operand).  P.V: the same lane holds code word
    // 4 qb + jj (dims 32 qb + 8 jj ..) of rows 4 tg .. 4 tg + 3 (B operand and
    // result) and head row jj for those rows and block qb (A operand).
    const int qtg = lane >> 4;
    const int qb = (lane >> 2) & 3;
    const int jj = lane & 3;
    const int tok = 4 * qtg + jj;

    const int work = static_cast<int>(__builtin_amdgcn_workgroup_id_x());
    const int kvh = work % a.Hkv;
    const int r = work / a.Hkv;
    int b, split;
    split_item(a.full_begin, a.tail_row, a.rows, r, b, split);
    const int L = a.len[b];
    const int nsplit = (L - split_base(L, a.window) + a.tps - 1) / a.tps;
    const int vis0 = visible_begin(L, a.window);   // first key the query sees
    const int t0 = split_base(L, a.window) + split * a.tps;
    const int t1 = min(L, t0 + a.tps);
    const int quarter = a.tps / kWaves4;
    const int wbeg = t0 + wave * quarter;
    const int wend = min(t1, wbeg + quarter);
    const int32_t* __restrict__ pt = a.page_table + int64_t(b) * a.maxb;

    if constexpr (G < 4) {
        for (int e = lane; e < kStages * (4 - G) * kGroup; e += 64)
            s_p[wave][e / ((4 - G) * kGroup)][G + (e / kGroup) % (4 - G)][e % kGroup] = 0.0f;
    }

    // ---- query operands: A rows = heads 4 p + jj (zero past G), 4 dims per
    // step in the order the code words unpack to, hi + lo bf16 parts
    // (step s: dims 8 (s / 2) + {0, 4, 1, 5} for even s, {2, 6, 3, 7} for odd s)
    // The query operands live in LDS (one copy per workgroup, read every
    // group) rather than in 32 VGPRs per pass: the registers they free allow
    // four waves per SIMD.
    __shared__ u32x4_t s_qa[NP][8][16];   // [pass][step][4 qb + jj]: hi.xy, lo.xy
    u32x2_t qa_hi[NP][8], qa_lo[NP][8];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int head = 4 * p + jj;
        const float* Q = a.q + (int64_t(b) * a.Hq + kvh * G + min(head, G - 1)) * kD4 + 32 * qb;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const int d0 = 8 * (st >> 1) + 2 * (st & 1);
            const int dims[4] = {d0, d0 + 4, d0 + 1, d0 + 5};
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const float x0 = head < G ? Q[dims[2 * e2]] : 0.0f;
                const float x1 = head < G ? Q[dims[2 * e2 + 1]] : 0.0f;
                const __bf16 h0 = static_cast<__bf16>(x0), h1 = static_cast<__bf16>(x1);
                const __bf16 l0 = static_cast<__bf16>(x0 - static_cast<float>(h0));
                const __bf16 l1 = static_cast<__bf16>(x1 - static_cast<float>(h1));
                hw[e2] = __builtin_bit_cast(uint32_t, bf16x2_t{h0, h1});
                lw[e2] = __builtin_bit_cast(uint32_t, bf16x2_t{l0, l1});
            }
            qa_hi[p][st] = u32x2_t{hw[0], hw[1]};
            qa_lo[p][st] = u32x2_t{lw[0], lw[1]};
        }
    }
    if (wave == 0 && qtg == 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int st = 0; st < 8; ++st)
                s_qa[p][st][4 * qb + jj] = u32x4_t{qa_hi[p][st].x, qa_hi[p][st].y, qa_lo[p][st].x, qa_lo[p][st].y};
    }
    // qs: sum of q over block qb for the heads 4 p + r of this lane's results
    // (the operands times ones, accumulated over the eight steps)
    f32x4_t qs[NP];
    {
        const u32x2_t ones = {0x3F803F80u, 0x3F803F80u};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            qs[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                qs[p] = mfma4(qa_hi[p][st], ones, qs[p]);
                qs[p] = mfma4(qa_lo[p][st], ones, qs[p]);
            }
        }
    }

    const uint32_t nib_mask = vconst(0x000F000Fu), nib_bias = vconst(0x43004300u);
    const u32x2_t b128 = {0x43004300u, 0x43004300u};   // bf16 128 in every row and column
    float m[G], lp[NP], offz[NP], mq[NP];   // mq[p]: m of head 4 p + qb (per lane)
    // acc[p][i][r]: head 4 p + r, dim 32 qb + 8 jj + i, summed over this lane's token quads
    f32x4_t acc[NP][8], off[NP];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -FLT_MAX;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        lp[p] = 0.0f;
        offz[p] = 0.0f;
        mq[p] = -FLT_MAX;
        off[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[p][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- one group's loads.  Rows past the valid length (inside the same
    // page) are read as they are: their scores become -inf, and their V
    // parameters are replaced by 0 before use.
    struct Stage {
        u32x4_t kc;                   // Q.K: the 32 codes of block qb of token tok
        uint32_t kp;                  // Q.K: (scale, zero) of that block
        u32x4_t vc;                   // V codes: row lane / 4, dims 32 (lane % 4) ..
        uint32_t vp;                  // V (scale, zero): row lane / 4, block lane % 4
    };
    // Per-lane byte offsets from a group's first row (the row base is
    // wave-uniform, so each load is a scalar base plus a 32-bit lane offset)
    const uint32_t o_kc = uint32_t(tok) * 64u + 16u * uint32_t(qb);
    const uint32_t o_kp = uint32_t(tok) * 16u + 4u * uint32_t(qb);
    const uint32_t o_vc = uint32_t(lane) * 16u;
    const uint32_t o_vp = uint32_t(lane) * 4u;
    auto stage_load = [&](int ts, int page) -> Stage {
        Stage st;
        const int64_t rb = (int64_t(page) * a.Hkv + kvh) * a.bs + (ts & (a.bs - 1));
        const uint8_t* kc = a.kc + rb * 64;
        const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.kp + rb * 8);
        const uint8_t* vc = a.vc + rb * 64;
        const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.vp + rb * 8);
        // lane offsets made opaque here, so that they are not folded into
        // loop-invariant 64-bit lane pointers (two VGPRs each) outside the loop
        uint32_t okc = o_kc, okp = o_kp, ovc = o_vc, ovp = o_vp;
        asm volatile("" : "+v"(okc), "+v"(okp), "+v"(ovc), "+v"(ovp));
        st.kc = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kc + okc));
        st.kp = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kp + okp));
        st.vc = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vc + ovc));
        st.vp = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vp + ovp));
        return st;
    };
    // LDS word offsets: this lane's V code store, and the P.V reads (code word
    // 4 qb + jj and block-qb parameters of rows 4 qtg + k)
    const int w_vc = 16 * ((lane >> 2) + (lane >> 4)) + 4 * (lane & 3);
    const int r_vc = 16 * (4 * qtg + qtg) + 4 * qb + jj;   // + 16 k for row 4 qtg + k
    const int r_vp = 16 * qtg + qb;                        // + 4 k

    auto compute = [&](const Stage& st, int ts, int buf) {
        // block-qb partial products of token tok for heads 4 p + r (hi and lo
        // chains accumulate separately), eight steps of four dims
        f32x4_t dh[NP], dl[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) dh[p] = dl[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        int qi = 4 * qb + jj;
        asm volatile("" : "+v"(qi));   // re-read every group, not hoisted into registers
#pragma unroll
        for (int stp = 0; stp < 8; ++stp) {
            const uint32_t w = st.kc[stp >> 1] >> (8 * (stp & 1));
            const u32x2_t kb = {(w & nib_mask) | nib_bias, ((w >> 4) & nib_mask) | nib_bias};
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const u32x4_t qv = s_qa[p][stp][qi];
                dh[p] = mfma4(u32x2_t{qv.x, qv.y}, kb, dh[p]);
                dl[p] = mfma4(u32x2_t{qv.z, qv.w}, kb, dl[p]);
            }
        }
        // the V tile to LDS, in the layout the P.V reads take it
        *reinterpret_cast<u32x4_t*>(&s_vc[wave][buf][w_vc]) = st.vc;
        s_vpar[wave][buf][lane] = st.vp;
        const float sc = h2f(st.kp & 0xFFFFu);
        const float zz = 128.0f + h2f(st.kp >> 16);
        const bool tok_live = ts + tok < wend && ts + tok >= vis0;
        float s[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // dequantised block contribution, summed over the four blocks (lanes
            // 4 apart in the row), then this lane keeps head 4 p + qb
            float tot[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = sc * fmaf(-zz, qs[p][r], dh[p][r] + dl[p][r]);
                x += dppm<0x124>(x);   // row_ror:4
                x += dppm<0x128>(x);   // row_ror:8
                tot[r] = x;
            }
            // all four totals exist before the lane picks one (a select, not a branch)
            asm volatile("" : "+v"(tot[0]), "+v"(tot[1]), "+v"(tot[2]), "+v"(tot[3]));
            const bool b0 = (lane & 4) != 0, b1 = (lane & 8) != 0;   // the bits of qb
            const float mine = b1 ? (b0 ? tot[3] : tot[2]) : (b0 ? tot[1] : tot[0]);
            s[p] = tok_live && 4 * p + qb < G ? mine * a.scale_log2 : -INFINITY;
        }
        // group maxima per head (lanes with the same qb), wave-uniform; lazy
        // rescale, checked for all heads at once
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float mx = fmaxf(s[p], dppm<0xB1>(s[p]));   // quad_perm [1,0,3,2]
            mx = fmaxf(mx, dppm<0x4E>(mx));              // quad_perm [2,3,0,1]
            mx = max_xor16(mx);
            mx = max_xor32(mx);
            if (__builtin_amdgcn_ballot_w64(mx > mq[p] + kLazy4) == 0) continue;
#pragma unroll
            for (int hh = 0; hh < HP; ++hh) {
                const int g = 4 * p + hh;
                const float mg = readlane_f(mx, 4 * hh);
                if (mg > m[g] + kLazy4) {
                    const float cf = exp2_fast(m[g] - mg);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[p][i][hh] *= cf;
                    off[p][hh] *= cf;
                    if (jj == hh) offz[p] *= cf;
                    if (qb == hh) {
                        lp[p] *= cf;
                        mq[p] = mg;
                    }
                    m[g] = mg;
                }
            }
        }
        // probabilities to LDS, [head][token]
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float pr = exp2_fast(s[p] - mq[p]);
            lp[p] += pr;
            if (4 * p + qb < G) s_p[wave][buf][4 * p + qb][tok] = pr;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // P.V.  B operands: for byte m of the word, the low nibbles (dim
        // 2 m) and the high nibbles (dim 2 m + 1) of rows (0, 1) and (2, 3),
        // each as bf16 128 + c
        uint32_t vw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) vw[k] = s_vc[wave][buf][r_vc + 16 * k];
        u32x2_t vb[8];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const uint32_t sel = uint32_t(mb) | 0x0C00u | (uint32_t(4 + mb) << 16) | 0x0C000000u;
            const uint32_t x01 = __builtin_amdgcn_perm(vw[1], vw[0], sel);
            const uint32_t x23 = __builtin_amdgcn_perm(vw[3], vw[2], sel);
            vb[2 * mb] = u32x2_t{(x01 & nib_mask) | nib_bias, (x23 & nib_mask) | nib_bias};
            vb[2 * mb + 1] = u32x2_t{((x01 >> 4) & nib_mask) | nib_bias, ((x23 >> 4) & nib_mask) | nib_bias};
        }
        // (scale, zero) of rows past the valid length read as 0, so that an
        // arbitrary unwritten value cannot turn a zero probability into NaN
        uint32_t vp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) vp[k] = s_vpar[wave][buf][r_vp + 4 * k];
        if (ts + kGroup > L) {
            const int last = L - 1 - ts - 4 * qtg;
#pragma unroll
            for (int k = 0; k < 4; ++k) vp[k] = k > last ? 0u : vp[k];
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // A operand: x = p * scale of block qb for head 4 p + jj and rows
            // 4 qtg + k, as a truncated bf16 high part plus a rounded low part
            const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(&s_p[wave][buf][4 * p + jj][4 * qtg]);
            float x[4], xl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[k] = pr[k] * h2f(vp[k] & 0xFFFFu);
                offz[p] = fmaf(x[k], h2f(vp[k] >> 16), offz[p]);
                xl[k] = x[k] - __uint_as_float(__float_as_uint(x[k]) & 0xFFFF0000u);
            }
            const u32x2_t ah = {__builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u),
                                __builtin_amdgcn_perm(__float_as_uint(x[3]), __float_as_uint(x[2]), 0x07060302u)};
            const u32x2_t al = {__builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(xl[0]),
                                                                     static_cast<__bf16>(xl[1])}),
                                __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(xl[2]),
                                                                     static_cast<__bf16>(xl[3])})};
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[p][i] = mfma4(ah, vb[i], acc[p][i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[p][i] = mfma4(al, vb[i], acc[p][i]);
            off[p] = mfma4(ah, b128, off[p]);
            off[p] = mfma4(al, b128, off[p]);
        }
        // no barrier here: the next group writes another buffer, and the
        // next writer of this one comes after that group's barrier
    };

    __syncthreads();   // the query operands in LDS

    // kStages register stages used in turn (no copies between them, so a
    // wait is only for the stage about to be used); page ids one round ahead.
    // Loads past the range re-read its last group; the last round ends with
    // up to kStages - 1 fully masked groups.
    if (wbeg < wend) {
        const int ng = (wend - wbeg + kGroup - 1) / kGroup;
        auto gts = [&](int i) { return wbeg + min(i, ng - 1) * kGroup; };
        auto page_of = [&](int i) { return load_uniform(pt + (gts(i) >> a.log2bs)); };
        Stage S[kStages];
        int pg[kStages];
#pragma unroll
        for (int u = 0; u < kStages; ++u) pg[u] = page_of(u);
#pragma unroll
        for (int u = 0; u < kStages; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            S[u] = stage_load(gts(u), pg[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kStages; ++u) pg[u] = page_of(kStages + u);
        __builtin_amdgcn_sched_barrier(0);
        for (int i = 0; i < ng; i += kStages) {
#pragma unroll
            for (int u = 0; u < kStages; ++u) {
                compute(S[u], wbeg + (i + u) * kGroup, u);
                __builtin_amdgcn_sched_barrier(0);
                S[u] = stage_load(gts(i + u + kStages), pg[u]);
                pg[u] = page_of(i + u + 2 * kStages);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- finish the wave: sums over the token quads (lanes 16 apart), the
    // 128 offset and the zero-point term, row sums of p
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[p][i][rr] = sum_xor32(sum_xor16(acc[p][i][rr]));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) off[p][rr] = sum_xor32(sum_xor16(off[p][rr]));
        offz[p] = sum_xor32(sum_xor16(offz[p]));
    }
    float l[G];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        float rs = lp[p] + dpp<0xB1>(lp[p]);
        rs += dpp<0x4E>(rs);
        rs = sum_xor32(sum_xor16(rs));
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) l[4 * p + hh] = readlane_f(rs, 4 * hh);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        // zero-point sums of heads 4 p + rr for block qb: lane jj of the quad holds head jj
        const float z0 = dpp<0x00>(offz[p]), z1 = dpp<0x55>(offz[p]);
        const float z2 = dpp<0xAA>(offz[p]), z3 = dpp<0xFF>(offz[p]);
        const float zr[4] = {z0, z1, z2, z3};
        if (qtg == 0) {
#pragma unroll
            for (int rr = 0; rr < HP; ++rr)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    s_o[wave][4 * p + rr][32 * qb + 8 * jj + i] = acc[p][i][rr] - off[p][rr] - zr[rr];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            s_ml[wave][g][0] = m[g];
            s_ml[wave][g][1] = l[g];
        }
    }
    __syncthreads();

    for (int e = tid; e < G * kD4; e += 256) {
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
