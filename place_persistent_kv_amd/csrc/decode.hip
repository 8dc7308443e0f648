// Decode attention for gfx950: one new query per (row, head) over the valid
// cache prefix, contiguous or paged, with a split over long contexts and a
// log-sum-exp merge.
//
// What is computed -- "Persistent input/output feedback", "Optional
// heterogeneous paged KV", sections "Versioned operator schema" and "Kernel
// implementation": grouped-query attention (query head h reads K/V head
// h / G), only valid and visible tokens are read (a left window W >= 0
// limits the query at L - 1 to keys [L - 1 - W, L - 1]; splits then cover
// only that range), online softmax instead of K/V concatenation or a
// cache-length score matrix.
//
// The single-token step is a bandwidth-bound GEMV (about 4 flops per K/V
// byte at G = 4), so it runs on the vector ALUs, not MFMA:
//
//  * fast kernel (bf16, D = 128, G <= 8): a workgroup of 4 waves owns one
//    (row, kv head, split); each wave streams its quarter of the split 16
//    tokens at a time.  Eight lanes cover one 256-byte K or V row with two
//    16-byte loads each (lane j reads dims 8j..8j+7 and 64+8j..64+8j+7), so
//    every load instruction moves eight full 128-byte lines.  The G query
//    heads of the group reuse each K/V row from registers.  Q.K uses
//    v_dot2_f32_bf16 on packed bf16 pairs; the 8-lane sum uses three DPP
//    adds (row_half_mirror, quad_perm [1,0,3,2], quad_perm [2,3,0,1]).
//    Each 8-lane group keeps its own running max / sum / output; the max is
//    refreshed lazily (only when a score exceeds it by 2^8), so the output
//    rescale is off the common path.  Groups and waves are merged at the end
//    through cross-lane shuffles and LDS.
//  * generic kernel (any D <= 256, f32/bf16/f16, any block size): one wave
//    per (row, query head, split) with scores staged in LDS.
//  * merge kernel: o = sum_i o_i 2^(m_i - m*) / sum_i l_i 2^(m_i - m*).

#include "device_common.h"

#include <type_traits>

namespace pkv {
namespace {

#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1
#endif


constexpr int kWaves = 4;
constexpr int kD = 128;
constexpr float kLazy = 8.0f;  // rescale only when a score exceeds the running max by 2^8
constexpr int32_t kStatusCapacity = 2;   // PKV_E_CAPACITY
constexpr int32_t kStatusPage = 6;       // PKV_E_PAGE

// A wave-uniform 32-bit load through the scalar unit (constant address
// space: an s_load, which never waits behind the vector loads in flight)
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}

// The (row, split) a workgroup works on.  With host lengths the split table
// of the launch gives it; with device lengths every row has S_max split slots
// and its split count follows from its length (a uniform load), and a length
// outside [1, len_limit] makes the row invalid.
struct SplitWork {
    int b, split, nsplit, L;
    bool ok;
};
__device__ __forceinline__ SplitWork split_work(const DecodeArgs& a, int r) {
    SplitWork w;
    if (a.len_dev == nullptr) {
        split_item(a.full_begin, a.tail_row, a.rows, r, w.b, w.split);
        w.L = a.len[w.b];
        w.nsplit = (w.L - split_base(w.L, a.window) + a.tps - 1) / a.tps;
        w.ok = true;
        return w;
    }
    w.b = r / a.S_max;
    w.split = r - w.b * a.S_max;
    // with a fused append the device value is the row's position and the
    // valid length is position + app_n
    const int pos = load_uniform(a.len_dev + a.row0 + w.b);
    w.ok = pos >= 0 && pos <= a.len_limit - a.app_n && pos + a.app_n >= 1;
    w.L = pos + a.app_n;
    w.nsplit = w.ok ? (w.L - split_base(w.L, a.window) + a.tps - 1) / a.tps : 0;
    return w;
}

// Fused append (contiguous caches): rows of the last a.app_n tokens of row
// b that fall in [t0, t1), plus those below t0 for split 0, copied from the
// new values into K/V head kvh of the caches by the nthreads threads of the
// workgroup; then every wave of the workgroup sees them (the rows it reads
// were written by this workgroup, or by another one with the same bytes).
__device__ __forceinline__ void append_rows(const DecodeArgs& a, int b, int kvh, int split, int t0, int t1, int L,
                                            int esz, int nthreads) {
    const int p0 = L - a.app_n;
    const int lo = split == 0 ? p0 : max(p0, t0);
    const int hi = t1;
    if (lo < hi) {
        const int64_t src_row = (int64_t(b) * a.Hkv + kvh) * a.app_n + (lo - p0);
        const int64_t dst_row = (int64_t(b) * a.Hkv + kvh) * a.cap + lo;
        const int64_t kb = int64_t(a.D) * esz, vb = int64_t(a.Dv) * esz;   // row bytes
        const uint8_t* sk = static_cast<const uint8_t*>(a.app_k) + src_row * kb;
        const uint8_t* sv = static_cast<const uint8_t*>(a.app_v) + src_row * vb;
        uint8_t* dk = static_cast<uint8_t*>(const_cast<void*>(a.k)) + dst_row * kb;
        uint8_t* dv = static_cast<uint8_t*>(const_cast<void*>(a.v)) + dst_row * vb;
        const int64_t nk = (hi - lo) * kb, nv = (hi - lo) * vb;
        if (a.app_vec16) {
            for (int64_t c = threadIdx.x; c < nk / 16; c += nthreads)
                reinterpret_cast<uint4*>(dk)[c] = reinterpret_cast<const uint4*>(sk)[c];
            for (int64_t c = threadIdx.x; c < nv / 16; c += nthreads)
                reinterpret_cast<uint4*>(dv)[c] = reinterpret_cast<const uint4*>(sv)[c];
        } else {
            for (int64_t c = threadIdx.x; c < nk / esz; c += nthreads) {
                if (esz == 4) reinterpret_cast<uint32_t*>(dk)[c] = reinterpret_cast<const uint32_t*>(sk)[c];
                else reinterpret_cast<uint16_t*>(dk)[c] = reinterpret_cast<const uint16_t*>(sk)[c];
            }
            for (int64_t c = threadIdx.x; c < nv / esz; c += nthreads) {
                if (esz == 4) reinterpret_cast<uint32_t*>(dv)[c] = reinterpret_cast<const uint32_t*>(sv)[c];
                else reinterpret_cast<uint16_t*>(dv)[c] = reinterpret_cast<const uint16_t*>(sv)[c];
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int G, bool PAGED, bool F16>   // F16: fp16 q/K/V (else bf16)
__global__ __launch_bounds__(256) void decode_fast_kernel(DecodeArgs a) {
    __shared__ float s_o[kWaves][G][kD];
    __shared__ float s_ml[kWaves][G][2];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 3;  // token within an 8-token slab
    const int j = lane & 7;     // 16-byte chunk within each half row
    auto dot2k = [](uint32_t x, uint32_t y, float c) { return F16 ? dot2_f16(x, y, c) : dot2_bf16(x, y, c); };
    auto cv_lo = [](uint32_t w) {
        return F16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w))) : bf_lo(w);
    };
    auto cv_hi = [](uint32_t w) {
        return F16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16))) : bf_hi(w);
    };

    const int work = blockIdx.x;
    const int kvh = work % a.Hkv;
    const SplitWork sw = split_work(a, work / a.Hkv);
    if (!sw.ok) {
        if (sw.split == 0 && kvh == 0 && threadIdx.x == 0) *a.status = kStatusCapacity;
        return;
    }
    if (sw.split >= sw.nsplit) return;
    const int b = sw.b, split = sw.split, nsplit = sw.nsplit, L = sw.L;
    const int vis0 = visible_begin(L, a.window);   // first key the query sees
    const int t0 = split_base(L, a.window) + split * a.tps;
    const int t1 = min(L, t0 + a.tps);
    const int quarter = a.tps / kWaves;
    const int wbeg = t0 + wave * quarter;
    const int wend = min(t1, wbeg + quarter);

    if constexpr (!PAGED) {
        if (a.app_n > 0) append_rows(a, b, kvh, split, t0, t1, L, 2, 256);
    }
    // (the appended rows were written before the reads below begin)
    const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
    const int32_t* __restrict__ pt = PAGED ? a.page_table + int64_t(b) * a.maxb : nullptr;

    // queries of the group, as packed bf16 pairs
    uint4 qa[G], qb[G];
    {
        const uint16_t* Q = static_cast<const uint16_t*>(a.q) + (int64_t(b) * a.Hq + kvh * G) * kD;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            qa[g] = ld16(Q + g * kD + j * 8);
            qb[g] = ld16(Q + g * kD + 64 + j * 8);
        }
    }

    float m[G], l[G], o[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -FLT_MAX;
        l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[g][d] = 0.0f;
    }

    // Element offset of the first row of the 16-token step at ts (wave-uniform):
    // ts is a multiple of 16 and block_size a power-of-two multiple of 16, so
    // the whole step lies in one page.
    // Page ids are wave-uniform scalar loads.  With device lengths a page id
    // outside the pool is replaced by page 0 (the reads stay inside the
    // pool) and reported through *status once the wave is done.
    bool bad_page = false;
    auto step_base = [&](int ts) -> int64_t {
        if constexpr (PAGED) {
            int page = load_uniform(pt + (ts >> a.log2bs));
            if (a.status != nullptr && uint32_t(page) >= uint32_t(a.nb)) {
                bad_page = true;
                page = 0;
            }
            return ((int64_t(page) * a.Hkv + kvh) * a.bs + (ts & (a.bs - 1))) * kD;
        } else {
            return ((int64_t(b) * a.Hkv + kvh) * a.cap + ts) * kD;
        }
    };

    struct Buf {
        uint4 ka0, kb0, ka1, kb1, va0, vb0, va1, vb1;
    };
    auto ldkv = [](const uint16_t* p) { return PKV_DECODE_NT ? ld16_nt(p) : ld16(p); };
    // Lane rows are clamped to the split's last token, so a partial last step
    // re-reads a valid row of the same page instead of leaving it.
    auto load = [&](Buf& u, int ts) {
        const int64_t base = step_base(ts);
        const int last = t1 - 1 - ts;
        const uint32_t o0 = uint32_t(min(grp, last)) * kD + j * 8;
        const uint32_t o1 = uint32_t(min(grp + 8, last)) * kD + j * 8;
        const uint16_t* kb = K + base;
        const uint16_t* vb = V + base;
        u.ka0 = ldkv(kb + o0);
        u.kb0 = ldkv(kb + o0 + 64);
        u.ka1 = ldkv(kb + o1);
        u.kb1 = ldkv(kb + o1 + 64);
        u.va0 = ldkv(vb + o0);
        u.vb0 = ldkv(vb + o0 + 64);
        u.va1 = ldkv(vb + o1);
        u.vb1 = ldkv(vb + o1 + 64);
    };

    auto compute = [&](const Buf& u, int ts) {
        const bool live0 = ts + grp < t1 && ts + grp >= vis0;
        const bool live1 = ts + 8 + grp < t1 && ts + 8 + grp >= vis0;
        float s0[G], s1[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float x = 0.0f, y = 0.0f;
            x = dot2k(qa[g].x, u.ka0.x, x);
            y = dot2k(qa[g].x, u.ka1.x, y);
            x = dot2k(qa[g].y, u.ka0.y, x);
            y = dot2k(qa[g].y, u.ka1.y, y);
            x = dot2k(qa[g].z, u.ka0.z, x);
            y = dot2k(qa[g].z, u.ka1.z, y);
            x = dot2k(qa[g].w, u.ka0.w, x);
            y = dot2k(qa[g].w, u.ka1.w, y);
            x = dot2k(qb[g].x, u.kb0.x, x);
            y = dot2k(qb[g].x, u.kb1.x, y);
            x = dot2k(qb[g].y, u.kb0.y, x);
            y = dot2k(qb[g].y, u.kb1.y, y);
            x = dot2k(qb[g].z, u.kb0.z, x);
            y = dot2k(qb[g].z, u.kb1.z, y);
            x = dot2k(qb[g].w, u.kb0.w, x);
            y = dot2k(qb[g].w, u.kb1.w, y);
            s0[g] = group8_sum(x) * a.scale_log2;
            s1[g] = group8_sum(y) * a.scale_log2;
            s0[g] = live0 ? s0[g] : -INFINITY;
            s1[g] = live1 ? s1[g] : -INFINITY;
        }
        const uint32_t w0[8] = {u.va0.x, u.va0.y, u.va0.z, u.va0.w, u.vb0.x, u.vb0.y, u.vb0.z, u.vb0.w};
        const uint32_t w1[8] = {u.va1.x, u.va1.y, u.va1.z, u.va1.w, u.vb1.x, u.vb1.y, u.vb1.z, u.vb1.w};
        float v0[16], v1[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v0[2 * k] = cv_lo(w0[k]);
            v0[2 * k + 1] = cv_hi(w0[k]);
            v1[2 * k] = cv_lo(w1[k]);
            v1[2 * k + 1] = cv_hi(w1[k]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mx = fmaxf(s0[g], s1[g]);
            if (mx > m[g] + kLazy) {
                const float c = exp2_fast(m[g] - mx);
                l[g] *= c;
#pragma unroll
                for (int d = 0; d < 16; ++d) o[g][d] *= c;
                m[g] = mx;
            }
            const float p0 = exp2_fast(s0[g] - m[g]);
            const float p1 = exp2_fast(s1[g] - m[g]);
            l[g] += p0 + p1;
#pragma unroll
            for (int d = 0; d < 16; ++d) o[g][d] = fmaf(p1, v1[d], fmaf(p0, v0[d], o[g][d]));
        }
    };

    // Stream the wave's range 16 tokens per step with the next step's loads in
    // flight.  The two-step main loop is straight-line code whose prefetch is
    // always valid, so the wait before each compute covers only that step's
    // own loads; the last one or two steps are finished after it.
    if (wbeg < wend) {
        const int nsteps = (wend - wbeg + kSlabTokens - 1) / kSlabTokens;
        Buf A, Bf;
        load(A, wbeg);
        int i = 0;
        for (; i + 2 < nsteps; i += 2) {
            const int ts = wbeg + i * kSlabTokens;
            load(Bf, ts + kSlabTokens);
            compute(A, ts);
            load(A, ts + 2 * kSlabTokens);
            compute(Bf, ts + kSlabTokens);
        }
        const int ts = wbeg + i * kSlabTokens;
        if (i + 1 < nsteps) {
            load(Bf, ts + kSlabTokens);
            compute(A, ts);
            compute(Bf, ts + kSlabTokens);
        } else {
            compute(A, ts);
        }
    }

    if (bad_page && lane == 0) *a.status = kStatusPage;

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
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                s_o[wave][g][j * 8 + d] = o[g][d];
                s_o[wave][g][64 + j * 8 + d] = o[g][8 + d];
            }
            if (j == 0) {
                s_ml[wave][g][0] = m[g];
                s_ml[wave][g][1] = l[g];
            }
        }
    }
    __syncthreads();

    // merge the four waves; thread t handles (g, d) pairs t, t + 256, ...
    for (int e = threadIdx.x; e < G * kD; e += 256) {
        const int g = e / kD;
        const int d = e % kD;
        float mn = -FLT_MAX;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mn = fmaxf(mn, s_ml[w][g][0]);
        float ls = 0.0f, os = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float c = exp2_fast(s_ml[w][g][0] - mn);
            ls += s_ml[w][g][1] * c;
            os += s_o[w][g][d] * c;
        }
        const int h = kvh * G + g;
        const int64_t bh = int64_t(b) * a.Hq + h;
        if (nsplit == 1) {
            const float y = os / ls;
            if (a.out_f32) static_cast<float*>(a.out)[bh * kD + d] = y;
            else if (F16) static_cast<_Float16*>(a.out)[bh * kD + d] = static_cast<_Float16>(y);
            else static_cast<uint16_t*>(a.out)[bh * kD + d] = f32_to_bf16_rne(y);
        } else {
            const int64_t slot = bh * a.S_max + split;
            a.ws_o[slot * kD + d] = os;
            if (d == 0) {
                a.ws_ml[slot * 2 + 0] = mn;
                a.ws_ml[slot * 2 + 1] = ls;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: one wave per (row, query head, split), any D <= 256.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
template <>
__device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return float(x); }

template <typename T>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
    __shared__ float s_p[kGenericMaxTps];
    const int lane = threadIdx.x;
    const int work = blockIdx.x;
    const int h = work % a.Hq;
    const SplitWork sw = split_work(a, work / a.Hq);
    if (!sw.ok) {
        if (sw.split == 0 && h == 0 && lane == 0) *a.status = kStatusCapacity;
        return;
    }
    if (sw.split >= sw.nsplit) return;
    const int b = sw.b, split = sw.split, L = sw.L;
    const int t0 = split_base(L, a.window) + split * a.tps;
    const int ta = max(t0, visible_begin(L, a.window));   // first visible token of the split
    const int t1 = min(L, t0 + a.tps);
    const int G = a.Hq / a.Hkv;
    const int kvh = h / G;
    const int D = a.D;
    if (a.app_n > 0) append_rows(a, b, kvh, split, t0, t1, L, int(sizeof(T)), 64);
    const T* Q = static_cast<const T*>(a.q) + (int64_t(b) * a.Hq + h) * D;
    const T* K = static_cast<const T*>(a.k);
    const T* V = static_cast<const T*>(a.v);

    // with device lengths a page id outside the pool reads page 0 and sets *status
    auto page_of = [&](int t) -> int {
        int page = a.page_table[int64_t(b) * a.maxb + t / a.bs];
        if (a.status != nullptr && uint32_t(page) >= uint32_t(a.nb)) {
            *a.status = kStatusPage;
            page = 0;
        }
        return page;
    };
    auto row = [&](int t) -> int64_t {  // element offset of token t's row
        if (a.page_table) return ((int64_t(page_of(t)) * a.Hkv + kvh) * a.bs + t % a.bs) * D;
        return ((int64_t(b) * a.Hkv + kvh) * a.cap + t) * D;
    };
    const int Dv = a.Dv;
    auto vrow = [&](int t) -> int64_t {  // element offset of token t's value row
        if (a.page_table) return ((int64_t(page_of(t)) * a.Hkv + kvh) * a.bs + t % a.bs) * Dv;
        return ((int64_t(b) * a.Hkv + kvh) * a.cap + t) * Dv;
    };

    // pass 1: scores (lanes over tokens)
    float mx = -FLT_MAX;
    for (int t = ta + lane; t < t1; t += 64) {
        const int64_t off = row(t);
        float s = 0.0f;
        for (int d = 0; d < D; ++d) s = fmaf(to_f32(Q[d]), to_f32(K[off + d]), s);
        s *= a.scale_log2;
        s_p[t - t0] = s;
        mx = fmaxf(mx, s);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float ls = 0.0f;
    for (int t = ta + lane; t < t1; t += 64) {
        const float p = exp2_fast(s_p[t - t0] - mx);
        s_p[t - t0] = p;
        ls += p;
    }
    for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
    __syncthreads();

    // pass 2: weighted values (lanes over dims).  A row with one split is
    // finished here (the merge would scale it by exactly 1 and then by 1 / ls,
    // which is what is done here); otherwise the partials go to the workspace.
    const int64_t bh = int64_t(b) * a.Hq + h;
    const int64_t slot = bh * a.S_max + split;
    const float inv = 1.0f / ls;
    for (int d = lane; d < Dv; d += 64) {
        float acc = 0.0f;
        for (int t = ta; t < t1; ++t) acc = fmaf(s_p[t - t0], to_f32(V[vrow(t) + d]), acc);
        if (sw.nsplit == 1) {
            const float y = acc * inv;
            if (a.out_f32 || std::is_same<T, float>::value) static_cast<float*>(a.out)[bh * Dv + d] = y;
            else if (std::is_same<T, _Float16>::value) static_cast<_Float16*>(a.out)[bh * Dv + d] = static_cast<_Float16>(y);
            else static_cast<uint16_t*>(a.out)[bh * Dv + d] = f32_to_bf16_rne(y);
        } else {
            a.ws_o[slot * Dv + d] = acc;
        }
    }
    if (sw.nsplit > 1 && lane == 0) {
        a.ws_ml[slot * 2 + 0] = mx;
        a.ws_ml[slot * 2 + 1] = ls;
    }
}

// ---------------------------------------------------------------------------
// Merge: one wave per (row, query head).  The partial outputs of the first
// kMergeU splits and the (max, sum) pairs of the first 64 splits are
// requested before anything else, so that one memory latency covers the
// weights and the first batch; weights are read across lanes (splits 64 and
// up: through LDS); lane l sums dims l, l + 64, ... over the splits.
// ---------------------------------------------------------------------------
constexpr int kMergeLdsSplits = 1024;
constexpr int kMergeU = 8;         // splits per batch of loads
constexpr int kMergeMaxDPL = 4;    // dims per lane (D <= 256)

__device__ __forceinline__ float wave_reduce(float x, bool is_max) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    return x;
}

__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
    __shared__ float s_w[kMergeLdsSplits];
    const int bh = blockIdx.x;
    const int b = bh / a.Hq;
    int n;
    if (a.len_dev != nullptr) {          // device lengths: the split count follows from the length
        const int pos = a.len_dev[a.row0 + b];     // length, or position before len_add new tokens
        if (pos < 0 || pos > a.len_limit - a.len_add || pos + a.len_add < 1) return;
        const int L = pos + a.len_add;
        n = (L - split_base(L, a.window) + a.tps - 1) / a.tps;
    } else {
        n = a.nsplit[b];
    }
    if (n < a.min_splits) return;
    const int lane = threadIdx.x;
    const int64_t gbh = int64_t(b) * a.Hq + (bh % a.Hq);
    const float* ml = a.ws_ml + gbh * a.S_max * 2;
    const float* po = a.ws_o + gbh * a.S_max * a.D;
    const int nd = (a.D + 63) >> 6;

    // first batch of partial outputs, in flight during the weight pass
    float x[kMergeMaxDPL][kMergeU];
    const int n0 = min(n, kMergeU);
#pragma unroll
    for (int j = 0; j < kMergeMaxDPL; ++j) {
        const int d = lane + 64 * j;
#pragma unroll
        for (int u = 0; u < kMergeU; ++u)
            x[j][u] = j < nd && d < a.D && u < n0 ? po[int64_t(u) * a.D + d] : 0.0f;
    }

    // (max, sum) of split `lane` in registers, requested with the outputs:
    // one memory round trip covers the common case of at most 64 splits;
    // splits 64 and up take further passes and keep their weights in LDS
    float m_l = -FLT_MAX, l_l = 0.0f;
    if (lane < n) {
        const float2 v = *reinterpret_cast<const float2*>(ml + 2 * lane);
        m_l = v.x;
        l_l = v.y;
    }
    float mx = m_l;
    for (int s = lane + 64; s < n; s += 64) mx = fmaxf(mx, ml[2 * s]);
    const float mn = wave_reduce(mx, true);
    const float w_l = lane < n ? exp2_fast(m_l - mn) : 0.0f;
    float ls = l_l * w_l;
    for (int s = lane + 64; s < n; s += 64) {
        const float w = exp2_fast(ml[2 * s] - mn);
        ls += ml[2 * s + 1] * w;
        if (s < kMergeLdsSplits) s_w[s] = w;
    }
    ls = wave_reduce(ls, false);
    if (n > 64) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    // weight of split su (uniform across the wave)
    auto weight = [&](int su) {
        if (su < 64) return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), su));
        return su < kMergeLdsSplits ? s_w[su] : exp2_fast(ml[2 * su] - mn);
    };
    const float inv = 1.0f / ls;

    float acc[kMergeMaxDPL][kMergeU];
#pragma unroll
    for (int j = 0; j < kMergeMaxDPL; ++j)
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) acc[j][u] = 0.0f;
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
        if (u < n0) {
            const float w = weight(u);
#pragma unroll
            for (int j = 0; j < kMergeMaxDPL; ++j) acc[j][u] = x[j][u] * w;
        }
    }
    for (int s = kMergeU; s < n; s += kMergeU) {
        const int nb = min(kMergeU, n - s);
#pragma unroll
        for (int j = 0; j < kMergeMaxDPL; ++j) {
            const int d = lane + 64 * j;
#pragma unroll
            for (int u = 0; u < kMergeU; ++u)
                x[j][u] = j < nd && d < a.D && u < nb ? po[int64_t(s + u) * a.D + d] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
            if (u < nb) {
                const float w = weight(s + u);
#pragma unroll
                for (int j = 0; j < kMergeMaxDPL; ++j) acc[j][u] = fmaf(x[j][u], w, acc[j][u]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMergeMaxDPL; ++j) {
        const int d = lane + 64 * j;
        if (j >= nd || d >= a.D) continue;
        const float os = ((acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3])) +
                         ((acc[j][4] + acc[j][5]) + (acc[j][6] + acc[j][7]));
        const float y = os * inv;
        const int64_t idx = gbh * a.D + d;
        if (a.out_kind == kKvF32) static_cast<float*>(a.out)[idx] = y;
        else if (a.out_kind == kKvBF16) static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(y);
        else static_cast<_Float16*>(a.out)[idx] = static_cast<_Float16>(y);
    }
}

}  // namespace

bool fast_decode_supported(int kv_kind, int D, int G, bool paged, int bs) {
    if ((kv_kind != kKvBF16 && kv_kind != kKvF16) || D != kD) return false;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    if (paged && (bs < kSlabTokens || (bs & (bs - 1)) != 0)) return false;
    return true;
}

hipError_t launch_decode_fast(const DecodeArgs& a, int G, int total_work, hipStream_t s) {
    if (total_work <= 0) return hipSuccess;
    const dim3 grid(total_work), block(256);
    const bool paged = a.page_table != nullptr;
    const bool f16 = a.kv_kind == kKvF16;
#define PKV_FAST(GG)                                                                              \
    if (G == GG) {                                                                                \
        if (f16) {                                                                                \
            if (paged) hipLaunchKernelGGL((decode_fast_kernel<GG, true, true>), grid, block, 0, s, a); \
            else hipLaunchKernelGGL((decode_fast_kernel<GG, false, true>), grid, block, 0, s, a);    \
        } else {                                                                                  \
            if (paged) hipLaunchKernelGGL((decode_fast_kernel<GG, true, false>), grid, block, 0, s, a); \
            else hipLaunchKernelGGL((decode_fast_kernel<GG, false, false>), grid, block, 0, s, a);   \
        }                                                                                         \
        return hipGetLastError();                                                                 \
    }
    PKV_FAST(1)
    PKV_FAST(2)
    PKV_FAST(4)
    PKV_FAST(8)
#undef PKV_FAST
    return hipErrorInvalidValue;
}

hipError_t launch_decode_generic(const DecodeArgs& a, int total_work, hipStream_t s) {
    if (total_work <= 0) return hipSuccess;
    const dim3 grid(total_work), block(64);
    switch (a.kv_kind) {
        case kKvF32: hipLaunchKernelGGL(decode_generic_kernel<float>, grid, block, 0, s, a); break;
        case kKvBF16: hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, block, 0, s, a); break;
        case kKvF16: hipLaunchKernelGGL(decode_generic_kernel<_Float16>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    const int blocks = a.rows * a.Hq;
    if (blocks <= 0) return hipSuccess;
    if (a.D > 64 * kMergeMaxDPL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv
