// Internal interface between the host core (kvc_api.cpp) and the HIP kernels.
// Plain structs passed by value as kernel arguments (kept under 4 KB), and the
// launch functions each kernel file defines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cstddef>
#include <cstring>

#include <type_traits>

namespace kvc {

// Rows of the batch one launch covers; larger batches are split into several
// launches so that per-row tables fit in the kernel argument block.
constexpr int kMaxRowsPerLaunch = 256;
// Rotary pairs per head vector (d_head / 2 for d_head <= 128).
constexpr int kMaxRopePairs = 64;
// Query rows (query heads of one group x query positions) of one decode slab.
constexpr int kMaxDecodeRows = 32;
// Rows per workspace record of the split-K workspace as allocated (a launch
// with slabs of more rows uses fewer, wider records).
constexpr int kWsRecordRows = 8;
// Upper bound on decode work-groups per launch (sizes the split-K workspace).
constexpr int kMaxDecodeBlocks = 8192;

enum Dtype : int32_t { F32 = 0, F16 = 1, BF16 = 2 };

inline int itemsize(int dt) { return dt == F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Append: copy a [rows][H_kv][T][D] chunk into the cache with rounding.
// ---------------------------------------------------------------------------
struct AppendArgs {
    void* k_cache;           // storage base (element type = st_dtype)
    void* v_cache;
    const void* k_in;        // chunk base for row `row0` (element type = in_dtype)
    const void* v_in;
    int64_t layer_off;       // element offset of (layer, row0, head 0, slot 0)
    int64_t row_stride;      // elements between rows: H_kv * max_len * D
    int64_t head_stride;     // elements between heads: max_len * D
    int32_t rows, H, T, D;
    int32_t in_dtype, st_dtype;
    int32_t rope;                      // 1: rotate K at its positions (rotary embedding)
    int32_t n_tensors;                 // 2: K and V; 1: the first tensor only (k_in -> k_cache)
    // paged storage (btab non-null): position p of row b, head g sits in physical
    // block btab[b * btab_stride + (p >> bshift)] of the layer's pool, at
    // layer_off + ((block * H + g) << bshift + (p & mask)) * D
    const int32_t* btab;               // block table from row `row0` on
    int32_t btab_stride, bshift, pool_blocks;
    int32_t fill[kMaxRowsPerLaunch];   // first slot written, per row
    double inv_freq[kMaxRopePairs];    // rotary frequencies of pairs (i, i + D/2), i < D/2
};

// ---------------------------------------------------------------------------
// Rotary embedding of a [rows][H][T][D] tensor in place, row b's position t at
// pos0[b] + t (the queries of a chunk).
// ---------------------------------------------------------------------------
struct RopeArgs {
    void* x;                 // chunk base for row `row0` (element type = dtype)
    int32_t rows, H, T, D;
    int32_t dtype;
    int32_t pos0[kMaxRowsPerLaunch];
    double inv_freq[kMaxRopePairs];
};

// ---------------------------------------------------------------------------
// Split-K decode attention over a flattened key axis ("stream-K"):
// work unit u = (row b, KV head g) owns n_b keys; the units are laid end to
// end (b-major) and each work-group takes a slice of that axis.
// A slab is a set of query rows of one unit: query heads g*G + r0 .. + Gc and
// query positions i0 .. i0 + Tc of the chunk (Gc * Tc <= kMaxDecodeRows).
// ---------------------------------------------------------------------------
template <int PC>
struct DecodeArgsT {
    const void* k_cache;
    const void* v_cache;
    const void* q;           // [B][Hq][T][D], q_dtype, whole-batch base
    float* out;              // [B][Hq][T][D] float32, whole-batch base
    float* ws_o;             // [records][rec_rows][D] unnormalised partial outputs
    float* ws_ml;            // [records][rec_rows][2] running max (raw q.k units) and sum
    int64_t ws_rows_cap;     // rows the workspace holds (records x rec_rows <= this)
    int32_t rec_rows;        // rows per record in this launch (set by launch_decode)
    int64_t layer_off;       // element offset of (layer, row0, 0, 0, 0)
    int64_t row_stride;
    int64_t head_stride;
    int64_t total_keys;      // sum over rows of (n_b + unit_pad) * H_kv
    // slices of the key axis: work-group k < n_first takes keys_per_block
    // keys when k is even and keys_per_block_odd when k is odd; a later one
    // keys_per_block2 or keys_per_block2_odd by the same parity (work-group k
    // runs on XCD k mod 8, and the odd XCDs read HBM more slowly)
    int64_t keys_per_block;
    int64_t keys_per_block_odd;
    int64_t keys_per_block2;
    int64_t keys_per_block2_odd;
    // 1 / (keys_per_block + keys_per_block_odd) and the same for the later
    // pair, rounded to float: decode_slice_of's quotient estimates
    float pair_inv, pair2_inv;
    int32_t n_first;
    int32_t row0, rows;      // batch rows of this launch
    int32_t Hq, Hkv, G, T;   // T = query positions in the chunk
    int32_t D;
    int32_t r0, Gc, i0, Tc;  // the slab
    int32_t q_dtype, st_dtype;
    int32_t n_blocks;        // work-groups (set by launch_decode)
    int32_t merge_rows;      // the merge pass's rows of 256 outputs (its store row, if any, follows them)
    // The key axis may give every unit unit_pad virtual keys before its real
    // ones (the matrix-core kernel charges each unit one tile this way: a
    // slice that holds a unit boundary has a part tile on each side of it).
    // Positions and total_keys are on that padded axis; prefix counts real
    // keys, so row b starts at prefix[b] + b * Hkv * unit_pad.
    int32_t unit_pad;
    float scale_log2;        // log2(e) / sqrt(D)
    // paged storage (btab non-null): key j of unit (b, g) sits in physical block
    // btab[b * btab_stride + (j >> bshift)] of the layer's pool, at element
    // layer_off + ((block * Hkv + g) << bshift + (j & mask)) * D
    const int32_t* btab;     // block table from row `row0` on
    int32_t btab_stride, bshift, pool_blocks;
    // fused append (single slab on the vector kernel): the chunk's T new keys
    // and values, [B][Hkv][T][D] of the storage type (whole-batch base), are
    // read from here instead of the cache, and the merge pass stores them in the
    // cache afterwards; null: the cache already holds them
    const void* k_new;
    const void* v_new;
    // exact division by Hkv of a multiple of it (set by launch_decode):
    // x / Hkv = (x >> hkv_shift) * hkv_inv mod 2^64, hkv_inv the inverse of
    // Hkv's odd part modulo 2^64
    int32_t hkv_shift;
    uint64_t hkv_inv;
    int64_t prefix[PC];      // exclusive prefix of n_b * H_kv; INT64_MAX past the launch's rows
    static constexpr int kPrefix = PC;
};

// The arguments of a launch of up to kMaxRowsPerLaunch rows, and their first
// bytes (the prefix table cut to 33 entries) for a launch of at most 32 rows:
// the runtime copies a kernel's whole argument block at every launch, and the
// full table's 2 KB cost some 1.5 us more per launch on the host.
using DecodeArgs = DecodeArgsT<kMaxRowsPerLaunch + 1>;
constexpr int kSmallRows = 32;
using DecodeArgsSmall = DecodeArgsT<kSmallRows + 1>;
static_assert(offsetof(DecodeArgs, prefix) == offsetof(DecodeArgsSmall, prefix), "one layout up to the table");

// ---------------------------------------------------------------------------
// Prefill-chunk attention on matrix cores (fp16/bf16 caches): one work-group per
// (row, KV head, block of queries); columns are (query, head-in-group) pairs.
// ---------------------------------------------------------------------------
struct PrefillArgs {
    const void* k_cache;
    const void* v_cache;
    const void* q;           // [B][Hq][T][D], q_dtype, whole-batch base
    float* out;              // [B][Hq][T][D] float32, whole-batch base
    int64_t layer_off;       // element offset of (layer, row0, 0, 0, 0)
    int64_t row_stride;
    int64_t head_stride;
    int32_t row0, rows;
    int32_t Hq, Hkv, G, T, D;
    int32_t r0, Gc;          // query heads g*G + r0 .. + Gc of each group
    int32_t i0, Ti;          // queries i0 .. i0 + Ti of the chunk
    int32_t qpt;             // queries per 32-column tile (Gc * qpt <= 32)
    int32_t q_per_block;     // queries per work-group
    int32_t q_dtype, st_dtype;
    float scale_log2;
    int32_t p_split;         // 1: P as a 16-bit hi + lo pair (two products with V), 0: rounded once
    // paged storage (btab non-null), as in DecodeArgs
    const int32_t* btab;
    int32_t btab_stride, bshift, pool_blocks;
    int32_t offset[kMaxRowsPerLaunch];   // per row: s_b, the chunk's query offset
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Copy-out of positions [0, loc.T) of every row of one layer into dense
// [rows][H_kv][T][D] buffers of the storage type; position p of row b reads the
// stored value when p < loc.fill[b] and zero otherwise. loc gives the storage
// (contiguous or paged) exactly as for an append of the same rows.
// ---------------------------------------------------------------------------
struct GatherArgs {
    AppendArgs loc;
    void* k_out;             // output base for row `row0`
    void* v_out;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

// Entries of a device block table set in stream order (n <= kMaxTableSets).
constexpr int kMaxTableSets = 480;
struct TableSetArgs {
    int32_t* table;
    int32_t n;
    int32_t index[kMaxTableSets];
    int32_t value[kMaxTableSets];
};
hipError_t launch_table_set(const TableSetArgs& a, hipStream_t stream);
// floor(x / d) for x >= 0, d > 0 and a quotient below 2^31: a double-precision
// estimate (off by at most one: the operands convert with a relative error of
// 2^-53 each and the quotient is rounded once), then the exact remainder moves
// it by one where the estimate rounded across an integer. About 30
// instructions with no branch, against the long expansion of a 64-bit integer
// division.
__host__ __device__ inline int64_t decode_quot(int64_t x, int64_t d) {
    int64_t q = static_cast<int32_t>(static_cast<double>(x) / static_cast<double>(d));
    const int64_t r = x - q * d;
    q += r < 0 ? -1 : (r >= d ? 1 : 0);
    return q;
}
// floor(x / d) for x >= 0, d > 0 and a quotient below 2^20, from inv = 1 / d
// rounded to float: the estimate's relative error is at most about 2^-22 (d and
// x rounded to float, the reciprocal and the product rounded, 2^-24 each),
// under a quarter at such quotients, and the exact remainder corrects it by
// one where it fell across an integer.
__host__ __device__ inline int64_t decode_quot_rcp(int64_t x, int64_t d, float inv) {
    int64_t q = static_cast<int32_t>(static_cast<float>(x) * inv);
    const int64_t r = x - q * d;
    q += r < 0 ? -1 : (r >= d ? 1 : 0);
    return q;
}
// x / Hkv for x >= 0 a multiple of Hkv.
__host__ __device__ inline int64_t decode_div_exact(int64_t x, int shift, uint64_t inv) {
    return static_cast<int64_t>((static_cast<uint64_t>(x) >> shift) * inv);
}
template <class A>
__host__ __device__ inline int64_t decode_div_hkv(const A& a, int64_t x) {
    return decode_div_exact(x, a.hkv_shift, a.hkv_inv);
}
// hkv_shift and hkv_inv from Hkv (>= 1): Newton's iteration x <- x (2 - m x)
// doubles the number of correct low bits of m's inverse; m odd is its own
// inverse modulo 8, so five steps reach 96 bits.
inline void decode_set_hkv_div(DecodeArgs& a) {
    uint64_t m = static_cast<uint64_t>(a.Hkv);
    int s = 0;
    while ((m & 1) == 0) {
        m >>= 1;
        ++s;
    }
    uint64_t inv = m;
    for (int i = 0; i < 5; ++i) inv *= 2 - m * inv;
    a.hkv_shift = s;
    a.hkv_inv = inv;
}

// Decode work-group k's slice of the key axis starts at decode_slice_begin(a, k)
// and holds decode_slice_size(a, k) keys; key x lies in work-group
// decode_slice_of(a, x)'s slice. Slice sizes alternate by the parity of k (even
// first), and change once, at k = n_first.
__host__ __device__ inline int64_t decode_evens_below(int64_t k) { return (k + 1) >> 1; }
// (the same on the split's five values: n_first and the four slice sizes)
__host__ __device__ inline int64_t decode_slice_begin(int64_t k, int64_t n1, int64_t kpb, int64_t kpbo, int64_t kpb2,
                                                      int64_t kpb2o) {
    if (k <= n1) {
        const int64_t ne = decode_evens_below(k);
        return ne * kpb + (k - ne) * kpbo;
    }
    const int64_t ne1 = decode_evens_below(n1);
    const int64_t x1 = ne1 * kpb + (n1 - ne1) * kpbo;
    const int64_t ne = decode_evens_below(k) - ne1;
    return x1 + ne * kpb2 + (k - n1 - ne) * kpb2o;
}
__host__ __device__ inline int64_t decode_slice_size(int64_t k, int64_t n1, int64_t kpb, int64_t kpbo, int64_t kpb2,
                                                     int64_t kpb2o) {
    if (k < n1) return (k & 1) ? kpbo : kpb;
    return (k & 1) ? kpb2o : kpb2;
}
template <class A>
__host__ __device__ inline int64_t decode_slice_begin(const A& a, int64_t k) {
    return decode_slice_begin(k, a.n_first, a.keys_per_block, a.keys_per_block_odd, a.keys_per_block2,
                              a.keys_per_block2_odd);
}
template <class A>
__host__ __device__ inline int64_t decode_slice_size(const A& a, int64_t k) {
    return decode_slice_size(k, a.n_first, a.keys_per_block, a.keys_per_block_odd, a.keys_per_block2,
                             a.keys_per_block2_odd);
}
__host__ __device__ inline int64_t decode_slice_of(int64_t x, int64_t n1, int64_t kpb, int64_t kpbo, int64_t kpb2,
                                                   int64_t kpb2o, float pair_inv, float pair2_inv) {
    const int64_t x1 = decode_slice_begin(n1, n1, kpb, kpbo, kpb2, kpb2o);
    int64_t base = 0, first = kpb, second = kpbo;
    float inv = pair_inv;
    if (x >= x1) {
        // the later slices start at index n1; a pair is (even, odd) from an even n1
        base = n1;
        x -= x1;
        first = (n1 & 1) ? kpb2o : kpb2;
        second = (n1 & 1) ? kpb2 : kpb2o;
        inv = pair2_inv;
    }
    // (pairs on the axis: fewer than kMaxDecodeBlocks)
    const int64_t pair = first + second;
    const int64_t p = decode_quot_rcp(x, pair, inv);
    return base + 2 * p + (x - p * pair >= first ? 1 : 0);
}
template <class A>
__host__ __device__ inline int64_t decode_slice_of(const A& a, int64_t x) {
    return decode_slice_of(x, a.n_first, a.keys_per_block, a.keys_per_block_odd, a.keys_per_block2,
                           a.keys_per_block2_odd, a.pair_inv, a.pair2_inv);
}

// Cut the key axis into work-group slices: up to per_cu work-groups per CU, at
// least min_keys keys each, and no more records than the workspace holds.
// Work-groups beyond the first dispatch round (one per CU) share a CU with an
// older one, which the memory system serves first; they get a smaller slice,
// late_pct percent of a first-round one. Work-group k runs on XCD k mod 8, and
// the odd XCDs read HBM more slowly than the even ones: a work-group with odd
// k gets odd_pct percent of the slice of its round.
inline void decode_split_slices(DecodeArgs& a, int n_cu, int per_cu, int64_t min_keys, int late_pct, int odd_pct) {
    int64_t nb = static_cast<int64_t>(n_cu) * per_cu;
    if (nb > kMaxDecodeBlocks) nb = kMaxDecodeBlocks;
    const int64_t by_ws = a.ws_rows_cap / a.rec_rows - static_cast<int64_t>(a.rows) * a.Hkv;
    if (nb > by_ws) nb = by_ws;
    const int64_t by_size = (a.total_keys + min_keys - 1) / min_keys;
    if (nb > by_size) nb = by_size;
    if (nb < 1) nb = 1;
    const int64_t n1 = nb < n_cu ? nb : n_cu;
    const int64_t n1e = decode_evens_below(n1), n1o = n1 - n1e;
    const int64_t n2e = decode_evens_below(nb) - n1e, n2o = (nb - n1) - n2e;
    // slice weights in 1/10000 of a first-round even slice
    const int64_t w1e = 10000, w1o = 100 * odd_pct, w2e = 100 * late_pct, w2o = late_pct * odd_pct;
    const int64_t denom = n1e * w1e + n1o * w1o + n2e * w2e + n2o * w2o;
    const int64_t kpb = (a.total_keys * 10000 + denom - 1) / denom;
    // each size rounded up, so that the nb slices always cover the axis
    auto size = [&](int64_t w) { const int64_t v = (kpb * w + 9999) / 10000; return v < 1 ? int64_t(1) : v; };
    a.keys_per_block = kpb;
    a.keys_per_block_odd = size(w1o);
    a.keys_per_block2 = size(w2e);
    a.keys_per_block2_odd = size(w2o);
    a.pair_inv = 1.0f / static_cast<float>(a.keys_per_block + a.keys_per_block_odd);
    a.pair2_inv = 1.0f / static_cast<float>(a.keys_per_block2 + a.keys_per_block2_odd);
    a.n_first = static_cast<int32_t>(n1);
    // work-groups that hold keys (rounding up can leave the last ones empty)
    a.n_blocks = static_cast<int32_t>(decode_slice_of(a, a.total_keys - 1) + 1);
}

// Fills in the work split (n_blocks, slice sizes) from the device's resident capacity.
hipError_t launch_decode(DecodeArgs& a, hipStream_t stream);
// Scratch of the allocation-free attention call: a file-scope device array of
// kStaticScratchFloats floats (16 MiB) in the decode dispatcher's source, one
// copy per device. static_scratch gives its device address on `device`, taken
// once per device with hipGetSymbolAddress (the array's host-side name is not a
// device address and must never reach a kernel).
constexpr int64_t kStaticScratchFloats = int64_t(4) << 20;
hipError_t static_scratch(int device, float** ptr, int64_t* n_floats);

// The decode kernels of one (head dimension, storage type), and their key batch
// for a slab of `rows` query rows (one instantiation per translation unit).
template <int D, int ST>
hipError_t decode_run(DecodeArgs& a, hipStream_t stream);
template <int D, int ST>
int decode_batch_keys(int rows);
// Keys per work-group batch of the vector decode kernel for a slab of `rows`
// query rows (a paged cache's block must hold a whole number of batches).
int decode_vector_batch_keys(int D, int st_dtype, int rows);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Which kernel shapes exist (d_head x storage dtype).
bool decode_supported(int D, int st_dtype);
bool prefill_supported(int D, int st_dtype);
// Query-head columns of one prefill work-group (tiles of 32 columns).
int prefill_columns_per_block();

}  // namespace kvc
