// Internal interface between the host layer (pkv_api.cpp) and the gfx950
// kernels (*.hip).  Per-row data (positions, lengths, split offsets) travels
// in kernel arguments, so a launch never depends on host memory that could
// change after the call returns; rows are processed in groups of kMaxRows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kMaxRows = 256;        // batch rows per launch
constexpr int kMaxTableWrites = 448; // page-table entries per launch
constexpr int kSlabTokens = 16;      // tokens a wave handles per step in the fast decode kernel
constexpr int kFastD = 128;          // head size of the fast bf16 / INT4 decode kernels

// ---------------------------------------------------------------------------
// Cache updates
// ---------------------------------------------------------------------------
struct CopyRowsArgs {            // contiguous: dst[b,h,pos_b+t,:] = src[b,h,t,:]
    const uint8_t* src;          // [rows, H, n, row_bytes]
    uint8_t* dst;                // [rows, H, cap, row_bytes]
    const uint8_t* src2 = nullptr;   // a second (values, cache) pair written by the same
    uint8_t* dst2 = nullptr;         // launch at the same positions (K and V), or nullptr
    int64_t row_bytes;
    int32_t H, n, cap, rows;
    int32_t pos[kMaxRows];
};

struct PagedCopyArgs {           // paged: pool[pt[b][p/bs], h, p%bs, :] = src[b,h,t,:]
    const uint8_t* src;          // [rows, H, n, row_bytes]
    uint8_t* pool;               // [NB, H, bs, row_bytes]
    const uint8_t* src2 = nullptr;   // a second (values, pool) pair written by the same
    uint8_t* pool2 = nullptr;        // launch at the same positions (K and V), or nullptr
    const int32_t* page_table;   // row (row0 + b) of [*, maxb]
    int64_t row_bytes;
    int32_t H, n, bs, maxb, row0, rows;
    int32_t pos[kMaxRows];
};

struct PagedInt4Args {           // paged INT4 quantise-on-append
    const void* src;             // [rows, H, n, D] f32 or bf16
    uint8_t* codes;              // [NB, H, bs, D/2]
    uint16_t* params;            // [NB, H, bs, D/32, 2]
    const int32_t* page_table;
    int32_t src_bf16;
    int32_t H, n, bs, maxb, D, row0, rows;
    float scale;                 // fp16 scale widened to f32
    float zero_point;            // integer 0..15
    uint16_t scale_bits, zp_bits;
    int32_t pos[kMaxRows];
};

struct TableWriteArgs {
    int32_t* table;
    int32_t count;
    int32_t index[kMaxTableWrites];
    int32_t value[kMaxTableWrites];
};

struct GatherArgs {              // out[h, p, :] = pool[pt[seq][p/bs], h, p%bs, :]
    const uint8_t* pool;
    const int32_t* table_row;
    uint8_t* out;
    int64_t row_bytes;
    int32_t H, bs, length;
};

// K and V appended by one launch at positions read from device memory (a
// captured step replays with the positions the device holds at replay time).
// Every workgroup first checks every row of the call; if any fails, nothing
// is written and *status receives the error.
struct KvAppendDevArgs {
    const uint8_t* src[2];       // K, V values [B, H, n, row_bytes]
    uint8_t* dst[2];             // contiguous caches [B, H, cap, row_bytes] or pools [NB, H, bs, row_bytes]
    const int32_t* page_table;   // [B, maxb] (nullptr: contiguous)
    const int32_t* pos;          // device int32[B]
    int32_t* status;             // device status word (sticky)
    int64_t row_bytes;
    int32_t B, H, n;
    int32_t cap;                 // contiguous capacity, or maxb * bs
    int32_t bs, maxb, nb;        // paged geometry (nb = pool blocks)
};
hipError_t launch_kv_append_dev(const KvAppendDevArgs& a, hipStream_t s);
constexpr int kMaxDevAppend = 64;   // tokens per device-position append (a decode step's few tokens)

hipError_t launch_copy_rows(const CopyRowsArgs& a, hipStream_t s);
hipError_t launch_paged_copy(const PagedCopyArgs& a, hipStream_t s);
hipError_t launch_paged_int4_append(const PagedInt4Args& a, hipStream_t s);
hipError_t launch_table_write(const TableWriteArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Decode attention
// ---------------------------------------------------------------------------
enum KvKind : int32_t { kKvF32 = 0, kKvBF16 = 1, kKvF16 = 2, kKvF64 = 3 };   // f64: sampled logits only

struct DecodeArgs {
    const void* q;               // [B, Hq, D]
    const void* k;               // contiguous [B, Hkv, cap, D] or pool [NB, Hkv, bs, D]
    const void* v;
    const int32_t* page_table;   // nullptr for the contiguous layout
    void* out;                   // [B, Hq, D]
    float* ws_o;                 // [B, Hq, S_max, D] unnormalised partial outputs
    float* ws_ml;                // [B, Hq, S_max, 2]  (running max (log2 units), sum)
    int32_t kv_kind;             // KvKind of q/k/v
    int32_t out_f32;             // 1: out is f32, 0: out has the KV element type
    int32_t Hq, Hkv, D;          // D: query / key head size
    int32_t Dv;                  // value (and output) head size
    int32_t cap;                 // contiguous capacity (tokens per row)
    int32_t bs, maxb;            // paged block size, page-table row length
    int32_t log2bs;              // log2(bs) (fast kernel: bs is a power of two >= 16)
    int32_t S_max;               // split slots per (b, h) in the workspace
    int32_t tps;                 // tokens per split
    int32_t row0, rows;          // batch rows handled by this launch
    int32_t window;              // left window (-1 = unbounded), see visible_begin
    float scale_log2;            // softmax scale * log2(e)
    const void* page_desc;       // mixed-format pages: PageDesc[NB] (else nullptr)
    // Device lengths (else nullptr): row row0 + i has length len_dev[row0 + i],
    // S_max split slots, splits past its own count exit at once; rows whose
    // length is outside [1, len_limit] and rows that meet a page id outside
    // [0, nb) set *status and write nothing.  len[], full_begin[] and
    // tail_row[] unused.
    const int32_t* len_dev = nullptr;
    int32_t len_limit = 0;
    int32_t nb = 0;
    int32_t* status = nullptr;
    // Append fused into the attention (contiguous caches; with device lengths
    // len_dev holds the positions, the lengths being app_n more): the
    // last app_n tokens of each row's valid length are first copied from
    // app_k / app_v ([rows, Hkv, app_n, D] and [.., Dv], the cache's element
    // type) into the caches k / v by the workgroups whose split holds them
    // (split 0 also takes any below its range); app_vec16: every base 16-byte
    // aligned, so rows are copied in 16-byte pieces.
    const void* app_k = nullptr;
    const void* app_v = nullptr;
    int32_t app_n = 0;
    int32_t app_vec16 = 0;
    int32_t len[kMaxRows];       // valid length per row
    // work order (split_item): prefix sums of the rows' whole-tps splits, and
    // the rows whose last split is shorter, by that split's size, longest first
    int32_t full_begin[kMaxRows + 1];
    uint16_t tail_row[kMaxRows];
};

struct Int4DecodeArgs {
    const float* q;              // [B, Hq, 128]
    const uint8_t* kc;           // [NB, Hkv, bs, 64]
    const uint16_t* kp;          // [NB, Hkv, bs, 4, 2]
    const uint8_t* vc;
    const uint16_t* vp;
    const int32_t* page_table;
    float* out;                  // [B, Hq, 128]
    float* ws_o;
    float* ws_ml;
    int32_t Hq, Hkv, bs, maxb, S_max, tps, row0, rows;
    int32_t log2bs;
    int32_t window;              // left window (-1 = unbounded)
    float scale_log2;
    int32_t len[kMaxRows];
    int32_t full_begin[kMaxRows + 1];   // work order as in DecodeArgs
    uint16_t tail_row[kMaxRows];
};

struct MergeArgs {
    const float* ws_o;
    const float* ws_ml;
    void* out;
    int32_t out_kind;            // KvKind of out
    int32_t Hq, D, S_max, row0, rows;
    int32_t min_splits;          // rows with fewer partials were finished by the attention kernel
    // device lengths (else nullptr): the split count of a row comes from its
    // length as in DecodeArgs; invalid rows are skipped
    const int32_t* len_dev = nullptr;
    int32_t len_limit = 0, tps = 0, window = -1;
    int32_t len_add = 0;         // device values are positions len_add tokens before the lengths
    int32_t nsplit[kMaxRows];
};

// Fast path: bf16 or f16, D == 128, G in {1, 2, 4, 8}, block_size a power of two >= 16 (or contiguous).
bool fast_decode_supported(int kv_kind, int D, int G, bool paged, int bs);
hipError_t launch_decode_fast(const DecodeArgs& a, int G, int total_work, hipStream_t s);

// Token range of a row with valid length L under left window W: the query at
// L - 1 sees [visible_begin, L); splits start at split_base (visible_begin
// rounded down to whole 64-token quanta, so the fast kernels' 16-token steps
// stay page-aligned) and tokens before visible_begin are masked.
__host__ __device__ inline int32_t visible_begin(int32_t L, int32_t W) {
    return W < 0 ? 0 : (L - 1 - W > 0 ? L - 1 - W : 0);
}
__host__ __device__ inline int32_t split_base(int32_t L, int32_t W) {
    return visible_begin(L, W) / 64 * 64;
}
// Any D <= 256, f32/bf16/f16, any block size; tps <= kGenericMaxTps.
constexpr int kGenericMaxTps = 1024;
hipError_t launch_decode_generic(const DecodeArgs& a, int total_work, hipStream_t s);
hipError_t launch_decode_int4(const Int4DecodeArgs& a, int G, int total_work, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Mixed-format pages
// ---------------------------------------------------------------------------
// Page storages (values of pkv_page_storage).
enum PageStorage : int32_t {
    kStBF16 = 0, kStF16 = 1, kStI8 = 2, kStU8 = 3, kStI4 = 4, kStU4 = 5, kStI2 = 6, kStU2 = 7
};
__host__ __device__ inline int storage_bits(int st) { return st <= kStF16 ? 16 : st <= kStU8 ? 8 : st <= kStU4 ? 4 : 2; }
__host__ __device__ inline bool storage_signed(int st) { return st == kStI8 || st == kStI4 || st == kStI2; }

// Format of one physical page (16 bytes; the layout of pkv_page_desc).
struct PageDesc {
    float k_scale, v_scale;      // affine scales (dense pages: unused)
    int16_t k_zero, v_zero;      // affine zero points, in code units
    uint8_t k_st, v_st;          // PageStorage
    uint8_t pad[2];
};
static_assert(sizeof(PageDesc) == 16, "page descriptor is 16 bytes");

struct MixedAppendArgs {
    const uint16_t* k_src;       // [rows, H, n, D] bf16
    const uint16_t* v_src;
    uint8_t* k_pool;             // [NB, H, bs * D * 2] bytes: one slot per (page, head)
    uint8_t* v_pool;
    PageDesc* desc;              // [NB]
    const int32_t* page_table;   // row (row0 + b) of [*, maxb]
    PageDesc fmt;                // formats of the pages this append creates
    int32_t H, n, bs, maxb, D, row0, rows;
    int32_t pos[kMaxRows];
};

constexpr int kMaxConvert = 256; // pages per conversion launch
struct MixedConvertArgs {
    uint8_t* pool;               // slots of K or of V
    const PageDesc* desc;
    int32_t which;               // 0: K, 1: V
    int32_t st;                  // target storage, scale and zero point
    float scale;
    int32_t zero;
    int32_t H, bs, D, count;
    int32_t page[kMaxConvert];
    int32_t valid[kMaxConvert];  // rows [0, valid) are converted, the rest become zeros
};

struct MixedDescArgs {           // desc[page[i]] fields of the converted tensors
    PageDesc* desc;
    int32_t set_k, set_v;
    PageDesc fmt;
    int32_t count;
    int32_t page[kMaxConvert];
};

hipError_t launch_mixed_append(const MixedAppendArgs& a, hipStream_t s);
hipError_t launch_mixed_convert(const MixedConvertArgs& a, hipStream_t s);
hipError_t launch_mixed_desc(const MixedDescArgs& a, hipStream_t s);
// Decode over mixed pages: bf16 q, D == 128, G in {1, 2, 4, 8}, block_size a
// power of two >= 16; a.k / a.v are the slot pools, a.page_desc the descriptors.
bool mixed_decode_supported(int D, int G, int bs);
hipError_t launch_decode_mixed(const DecodeArgs& a, int G, int total_work, hipStream_t s);

// ---------------------------------------------------------------------------
// Chunk attention (MFMA)
// ---------------------------------------------------------------------------
struct ChunkArgs {
    const uint16_t* q;           // [B, Hq, C, 128] bf16
    const uint16_t* k;           // pool [NB, Hkv, bs, 128]
    const uint16_t* v;
    const int32_t* page_table;
    uint16_t* out;               // [B, Hq, C, 128]
    int32_t Hq, Hkv, C, bs, maxb, row0, rows;
    int32_t log2bs;              // block_size is a power of two
    int32_t window;              // left window (-1 = unbounded)
    float scale_log2;
    int32_t p0[kMaxRows];
    uint16_t order[kMaxRows];    // rows by descending prefix: the longest go out first
    // Split over the keys (kv_splits > 1): workgroup (row, kv head, query
    // tile, part s) takes part s of kv_splits near-equal parts of its query
    // tile's key-tile range and writes, per query row, the unnormalised output
    // and (max in log2 units, sum) to the workspace for the merge; with
    // kv_splits == 1 the output is written directly.
    int32_t kv_splits = 1;
    float* ws_o = nullptr;       // [rows, Hq, C, kv_splits, 128]
    float* ws_ml = nullptr;      // [rows, Hq, C, kv_splits, 2]
};
constexpr int kChunkQueryRows = 256;   // query rows (token x head pairs of one K/V head) per workgroup
constexpr int kChunkKeys = 64;         // keys per tile
constexpr int kChunkD = 128;           // head size
constexpr int kChunkMaxSplits = 64;    // parts of a workgroup's key range
bool chunk_supported(int D, int G, int bs, int C);
hipError_t launch_chunk(const ChunkArgs& a, int G, hipStream_t s);

// ---------------------------------------------------------------------------
// Generation loop
// ---------------------------------------------------------------------------
struct GenerateArgs {
    const int64_t* sampled;      // [B] ids drawn this iteration
    uint8_t* finished;           // [B] 0 / 1, updated
    int64_t* tokens;             // [B, row_stride] output, column `column` written
    int64_t* next_ids;           // [B] the written tokens (may be `sampled`)
    int32_t* unfinished;         // [1] rows still running after this iteration
    int64_t row_stride;
    int64_t eos, pad;
    int32_t column, B, has_eos;
};
hipError_t launch_generate_finish(const GenerateArgs& a, hipStream_t s);

struct AdvanceArgs {             // values[i] += delta for i < n; ++*step
    int32_t* values;
    int64_t* step;
    int32_t n, delta;
};
hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Sampling
// ---------------------------------------------------------------------------
struct SampleArgs {
    const void* logits;          // row b at logits + (b * row_stride) elements
    int64_t row_stride;          // elements between rows
    int64_t V;
    int32_t kind;                // KvKind of the logits
    int32_t B;
    int32_t chunks;              // vocab chunks per row
    int64_t chunk_len;           // elements per chunk (multiple of 1024)
    int32_t greedy;
    float inv_t;                 // fl32(1 / T): float32, bf16 and f16 logits
    double inv_t64;              // 1 / T in float64: float64 logits
    uint64_t seed;
    const int64_t* step = nullptr;   // device step counter: seed + step * B * V * gamma
    double* part_val;            // [B, chunks] best score per chunk (float32 scores widened)
    int32_t* part_idx;           // [B, chunks]
    int64_t* out;                // [B]
};
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Static scratch (pkv_paged_decode_attention_noalloc)
// ---------------------------------------------------------------------------
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;   // == PKV_NOALLOC_SCRATCH_BYTES
// Device address of the current device's scratch array (taken once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace pkv
