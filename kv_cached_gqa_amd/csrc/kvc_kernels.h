// Internal interface between the host core (kvc_api.cpp) and the HIP kernels.
// Plain structs passed by value as kernel arguments (kept under 4 KB), and the
// launch functions each kernel file defines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
struct DecodeArgs {
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
    int64_t prefix[kMaxRowsPerLaunch + 1];  // exclusive prefix of n_b * H_kv
};

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
// Decode work-group k's slice of the key axis starts at decode_slice_begin(a, k);
// key x lies in work-group decode_slice_of(a, x)'s slice. Slice sizes alternate
// by the parity of k (even first).
__host__ __device__ inline int64_t decode_evens_below(int64_t k) { return (k + 1) >> 1; }
__host__ __device__ inline int64_t decode_slice_begin(const DecodeArgs& a, int64_t k) {
    const int64_t n1 = a.n_first;
    if (k <= n1) {
        const int64_t ne = decode_evens_below(k);
        return ne * a.keys_per_block + (k - ne) * a.keys_per_block_odd;
    }
    const int64_t ne1 = decode_evens_below(n1);
    const int64_t x1 = ne1 * a.keys_per_block + (n1 - ne1) * a.keys_per_block_odd;
    const int64_t ne = decode_evens_below(k) - ne1;
    return x1 + ne * a.keys_per_block2 + (k - n1 - ne) * a.keys_per_block2_odd;
}
__host__ __device__ inline int64_t decode_slice_of(const DecodeArgs& a, int64_t x) {
    const int64_t n1 = a.n_first;
    const int64_t x1 = decode_slice_begin(a, n1);
    int64_t base = 0, first = a.keys_per_block, second = a.keys_per_block_odd;
    if (x >= x1) {
        // the later slices start at index n1; a pair is (even, odd) from an even n1
        base = n1;
        x -= x1;
        first = (n1 & 1) ? a.keys_per_block2_odd : a.keys_per_block2;
        second = (n1 & 1) ? a.keys_per_block2 : a.keys_per_block2_odd;
    }
    const int64_t pair = first + second;
    const int64_t p = x / pair;
    return base + 2 * p + (x - p * pair >= first ? 1 : 0);
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
