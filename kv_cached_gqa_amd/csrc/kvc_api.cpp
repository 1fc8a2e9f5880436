// Host core and C ABI of libkvc (declared in include/kvc.h).
//
// The host side owns the bookkeeping the pages' KVCache contract defines
// ("KV cache, incremental decode, ...", sections 2.3-2.5 and 4): a fill count
// per (layer, batch row), the committed length as the minimum over layers,
// truncate as a metadata-only rollback of every layer, and the exact byte
// count. Every call validates all of its arguments before it touches state or
// enqueues device work, so an error leaves the cache unchanged.
//
// Device work is enqueued on the caller's stream; metadata advances when the
// enqueue succeeded, which keeps host state and stream order consistent
// without any synchronisation.
//
// A paged cache ("kv-cache-decoding", "Batching caches of different lengths")
// keeps the same bookkeeping and adds a pool of fixed-size blocks: a row takes
// a block from the free list when an append first grows into it and gives its
// blocks back when truncate cuts them off. The host holds the block table and
// the free list; each change to the table is enqueued on the caller's stream
// (a small kernel writes the device copy) ahead of the append that needs it.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kvc.h"
#include "kvc_kernels.h"

using kvc::kMaxDecodeBlocks;
using kvc::kMaxDecodeRows;
using kvc::kWsRecordRows;
using kvc::kMaxRowsPerLaunch;

struct kvc_cache {
    kvc_config cfg;
    void* k_store;
    void* v_store;
    std::vector<int64_t> fill;    // [n_layers][batch]
    // split-K workspace, allocated at create on the storage's device (null when
    // the storage is not device memory: such a handle launches nothing)
    int device;
    float* ws_o;
    float* ws_ml;
    int64_t ws_segments;
    // paged storage (block_size > 0): pools of [n_layers][n_blocks][n_kv_heads]
    // [block_size][d_head], one block table [batch][width] shared by all layers
    int32_t block_size;
    int32_t bshift;
    int32_t n_blocks;
    int32_t width;                 // table entries per row: ceil(max_len / block_size)
    int32_t* d_table;              // device copy of the table (library-owned)
    std::vector<int32_t> table;    // host table, -1 = no block
    std::vector<int32_t> held;     // blocks held per row (a prefix of its table row)
    std::vector<int32_t> free_ids; // free blocks, taken from the back
    int32_t prefill_precision = KVC_PREFILL_P_ROUNDED;   // kvc_set_prefill_precision
};

namespace {

bool dtype_ok(int32_t dt) { return dt == KVC_F32 || dt == KVC_F16 || dt == KVC_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t storage_bytes(const kvc_config& c) {
    return 2ull * static_cast<uint64_t>(c.n_layers) * c.batch * c.n_kv_heads * static_cast<uint64_t>(c.max_len) *
           c.d_head * kvc::itemsize(c.dtype);
}

// Elements of one layer's block pool.
int64_t pool_layer_elems(const kvc_cache* c) {
    return static_cast<int64_t>(c->n_blocks) * c->cfg.n_kv_heads * c->block_size * c->cfg.d_head;
}

uint64_t pool_bytes(const kvc_config& c, int32_t block_size, int32_t n_blocks) {
    return 2ull * static_cast<uint64_t>(c.n_layers) * static_cast<uint64_t>(n_blocks) * c.n_kv_heads *
           static_cast<uint64_t>(block_size) * c.d_head * kvc::itemsize(c.dtype);
}

int64_t committed(const kvc_cache* c, int b) {
    int64_t s = c->fill[b];
    for (int l = 1; l < c->cfg.n_layers; ++l) s = std::min(s, c->fill[static_cast<size_t>(l) * c->cfg.batch + b]);
    return s;
}

// Records of kWsRecordRows rows the decode workspace holds: one per work-group
// plus one per unit boundary inside a launch, with room for slabs of up to
// kMaxDecodeRows rows (whose records are kMaxDecodeRows rows wide).
int64_t workspace_segments(const kvc_config& c) {
    const int64_t units = static_cast<int64_t>(std::min(c.batch, kMaxRowsPerLaunch)) * c.n_kv_heads;
    return kMaxDecodeBlocks + (kMaxDecodeRows / kWsRecordRows) * units;
}

// The split-K workspace on the device that holds the storage, allocated when
// the handle is created. Storage that is not device memory (or no GPU runtime)
// leaves the handle without one: KVC_OK, and every call that would launch
// device work on it returns KVC_ERR_STORAGE. KVC_ERR_NOMEM if the allocation
// fails.
int alloc_workspace(kvc_cache* c) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, c->k_store) != hipSuccess || attr.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return KVC_OK;
    }
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return KVC_ERR_HIP;
    const int dev = attr.device;
    if (dev != prev && hipSetDevice(dev) != hipSuccess) return KVC_ERR_HIP;
    const int64_t segs = workspace_segments(c->cfg);
    const size_t o_bytes = static_cast<size_t>(segs) * kWsRecordRows * c->cfg.d_head * sizeof(float);
    const size_t ml_bytes = static_cast<size_t>(segs) * kWsRecordRows * 2 * sizeof(float);
    void* o = nullptr;
    void* ml = nullptr;
    int rc = KVC_OK;
    if (hipMalloc(&o, o_bytes) != hipSuccess || hipMalloc(&ml, ml_bytes) != hipSuccess) {
        rc = KVC_ERR_NOMEM;
        if (o) (void)hipFree(o);
        if (ml) (void)hipFree(ml);
        (void)hipGetLastError();
    }
    if (dev != prev) (void)hipSetDevice(prev);
    if (rc != KVC_OK) return rc;
    c->device = dev;
    c->ws_o = static_cast<float*>(o);
    c->ws_ml = static_cast<float*>(ml);
    c->ws_segments = segs;
    return KVC_OK;
}

// Whether the handle can launch device work (its storage is device memory).
bool on_device(const kvc_cache* c) { return c->ws_o != nullptr; }

}  // namespace

extern "C" {

const char* kvc_strerror(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_ARG: return "invalid argument";
        case KVC_ERR_CAPACITY: return "append would exceed max_len";
        case KVC_ERR_STATE: return "call not valid in the current cache state";
        case KVC_ERR_DTYPE: return "unknown dtype";
        case KVC_ERR_STORAGE: return "storage buffer null, too small or misaligned";
        case KVC_ERR_HIP: return "HIP runtime error";
        case KVC_ERR_NOMEM: return "out of memory";
        case KVC_ERR_UNSUPPORTED: return "shape not supported by the kernels";
        case KVC_ERR_SCRATCH: return "call needs more split-K scratch than the static array holds";
        default: return "unknown status";
    }
}

int kvc_create(const kvc_config* cfg, void* k_store, void* v_store, uint64_t store_bytes_each, kvc_cache** out) {
    if (!cfg || !out) return KVC_ERR_ARG;
    const kvc_config c = *cfg;
    if (c.n_layers < 1 || c.batch < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.d_head < 1 || c.max_len < 1)
        return KVC_ERR_ARG;
    if (c.n_q_heads % c.n_kv_heads) return KVC_ERR_ARG;
    if (c.max_len * static_cast<int64_t>(c.d_head) >= (int64_t(1) << 31)) return KVC_ERR_ARG;
    if (!dtype_ok(c.dtype)) return KVC_ERR_DTYPE;
    if (!kvc::decode_supported(c.d_head, c.dtype)) return KVC_ERR_UNSUPPORTED;
    if (!k_store || !v_store || !aligned16(k_store) || !aligned16(v_store)) return KVC_ERR_STORAGE;
    if (store_bytes_each < storage_bytes(c) / 2) return KVC_ERR_STORAGE;
    kvc_cache* h = new (std::nothrow) kvc_cache();
    if (!h) return KVC_ERR_NOMEM;
    try {
        h->fill.assign(static_cast<size_t>(c.n_layers) * c.batch, 0);
    } catch (...) {
        delete h;
        return KVC_ERR_NOMEM;
    }
    h->cfg = c;
    h->k_store = k_store;
    h->v_store = v_store;
    h->device = -1;
    h->ws_o = nullptr;
    h->ws_ml = nullptr;
    h->ws_segments = 0;
    h->block_size = 0;
    h->d_table = nullptr;
    const int rw = alloc_workspace(h);
    if (rw != KVC_OK) {
        delete h;
        return rw;
    }
    *out = h;
    return KVC_OK;
}

int kvc_create_paged(const kvc_config* cfg, int32_t block_size, int32_t n_blocks, void* k_pool, void* v_pool,
                     uint64_t pool_bytes_each, kvc_cache** out) {
    if (!cfg || !out) return KVC_ERR_ARG;
    const kvc_config c = *cfg;
    if (c.n_layers < 1 || c.batch < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.d_head < 1 || c.max_len < 1)
        return KVC_ERR_ARG;
    if (c.n_q_heads % c.n_kv_heads) return KVC_ERR_ARG;
    if (block_size < 64 || (block_size & (block_size - 1)) || block_size > 4096 || n_blocks < 1) return KVC_ERR_ARG;
    const int64_t width = (c.max_len + block_size - 1) / block_size;
    if (width * c.batch >= (int64_t(1) << 31) || c.max_len >= (int64_t(1) << 31)) return KVC_ERR_ARG;
    // as for a contiguous cache: a chunk's T * d_head elements index in 32 bits
    if (c.max_len * static_cast<int64_t>(c.d_head) >= (int64_t(1) << 31)) return KVC_ERR_ARG;
    if (!dtype_ok(c.dtype)) return KVC_ERR_DTYPE;
    if (!kvc::decode_supported(c.d_head, c.dtype)) return KVC_ERR_UNSUPPORTED;
    // a decode batch of keys spans at most two blocks
    if (block_size < std::max(kvc::decode_vector_batch_keys(c.d_head, c.dtype, 4),
                              kvc::decode_vector_batch_keys(c.d_head, c.dtype, 8)))
        return KVC_ERR_UNSUPPORTED;
    if (!k_pool || !v_pool || !aligned16(k_pool) || !aligned16(v_pool)) return KVC_ERR_STORAGE;
    if (pool_bytes_each < pool_bytes(c, block_size, n_blocks) / 2) return KVC_ERR_STORAGE;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, k_pool) != hipSuccess) {
        (void)hipGetLastError();
        return KVC_ERR_STORAGE;
    }
    kvc_cache* h = new (std::nothrow) kvc_cache();
    if (!h) return KVC_ERR_NOMEM;
    try {
        h->fill.assign(static_cast<size_t>(c.n_layers) * c.batch, 0);
        h->table.assign(static_cast<size_t>(width) * c.batch, -1);
        h->held.assign(c.batch, 0);
        h->free_ids.resize(n_blocks);
        for (int32_t i = 0; i < n_blocks; ++i) h->free_ids[i] = n_blocks - 1 - i;   // block 0 is taken first
    } catch (...) {
        delete h;
        return KVC_ERR_NOMEM;
    }
    h->cfg = c;
    h->k_store = k_pool;
    h->v_store = v_pool;
    h->device = -1;
    h->ws_o = nullptr;
    h->ws_ml = nullptr;
    h->ws_segments = 0;
    h->block_size = block_size;
    h->bshift = 0;
    while ((1 << h->bshift) < block_size) ++h->bshift;
    h->n_blocks = n_blocks;
    h->width = static_cast<int32_t>(width);
    h->d_table = nullptr;
    // the device table, on the pool's device; entries are written before use
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) {
        delete h;
        return KVC_ERR_HIP;
    }
    if (attr.device != prev && hipSetDevice(attr.device) != hipSuccess) {
        delete h;
        return KVC_ERR_HIP;
    }
    void* t = nullptr;
    const size_t tb = static_cast<size_t>(width) * c.batch * sizeof(int32_t);
    const bool ok = hipMalloc(&t, tb) == hipSuccess && hipMemset(t, 0, tb) == hipSuccess;
    if (attr.device != prev) (void)hipSetDevice(prev);
    if (!ok) {
        if (t) (void)hipFree(t);
        (void)hipGetLastError();
        delete h;
        return KVC_ERR_NOMEM;
    }
    h->d_table = static_cast<int32_t*>(t);
    const int rw = alloc_workspace(h);
    if (rw != KVC_OK) {
        kvc_destroy(h);
        return rw;
    }
    *out = h;
    return KVC_OK;
}

void kvc_destroy(kvc_cache* c) {
    if (!c) return;
    if (c->ws_o || c->d_table) {
        int prev = 0;
        (void)hipGetDevice(&prev);
        hipPointerAttribute_t attr;
        const int dev = c->ws_o ? c->device
                                : (hipPointerGetAttributes(&attr, c->d_table) == hipSuccess ? attr.device : prev);
        (void)hipSetDevice(dev);
        (void)hipDeviceSynchronize();
        if (c->ws_o) {
            (void)hipFree(c->ws_o);
            (void)hipFree(c->ws_ml);
        }
        if (c->d_table) (void)hipFree(c->d_table);
        (void)hipSetDevice(prev);
    }
    delete c;
}

}  // extern "C"

namespace {

bool rope_base_ok(double base) { return std::isfinite(base) && base > 0.0; }

// Frequencies of the rotary pairs (i, i + D/2): base^(-2i / D), i < D/2.
void rope_freqs(double base, int D, double* out) {
    for (int i = 0; i < D / 2; ++i) out[i] = std::pow(base, -2.0 * i / D);
}

// Blocks a row needs to hold n positions.
int32_t blocks_for(const kvc_cache* c, int64_t n) {
    return static_cast<int32_t>((n + c->block_size - 1) >> c->bshift);
}

void release_unused(kvc_cache* c);

// Paged cache: give every row the blocks that positions [0, f[b] + T) need,
// and enqueue the table entries that change. All or nothing: KVC_ERR_CAPACITY
// (pool exhausted) before anything changes.
int grow_blocks(kvc_cache* c, const int64_t* f, int32_t T, hipStream_t s) {
    const int B = c->cfg.batch;
    int64_t need = 0;
    for (int b = 0; b < B; ++b) need += std::max(0, blocks_for(c, f[b] + T) - c->held[b]);
    if (need == 0) return KVC_OK;
    if (need > static_cast<int64_t>(c->free_ids.size())) return KVC_ERR_CAPACITY;
    kvc::TableSetArgs a;
    a.table = c->d_table;
    a.n = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t want = blocks_for(c, f[b] + T);
        for (int32_t k = c->held[b]; k < want; ++k) {
            const int32_t id = c->free_ids.back();
            c->free_ids.pop_back();
            c->table[static_cast<size_t>(b) * c->width + k] = id;
            c->held[b] = k + 1;
            a.index[a.n] = b * c->width + k;
            a.value[a.n] = id;
            if (++a.n == kvc::kMaxTableSets) {
                if (kvc::launch_table_set(a, s) != hipSuccess) {
                    release_unused(c);
                    return KVC_ERR_HIP;
                }
                a.n = 0;
            }
        }
    }
    if (a.n > 0 && kvc::launch_table_set(a, s) != hipSuccess) {
        release_unused(c);
        return KVC_ERR_HIP;
    }
    return KVC_OK;
}

// Paged cache: give back the blocks past position n of row b.
void shrink_blocks(kvc_cache* c, int b, int64_t n) {
    const int32_t keep = blocks_for(c, n);
    for (int32_t k = c->held[b] - 1; k >= keep; --k) {
        int32_t& e = c->table[static_cast<size_t>(b) * c->width + k];
        c->free_ids.push_back(e);
        e = -1;
    }
    c->held[b] = std::min(c->held[b], keep);
}

// Paged cache: give back every block no layer's fill reaches (a row holds
// exactly the blocks of its longest layer). Used when a call that took blocks
// fails, so that the call leaves the block accounting as it found it.
void release_unused(kvc_cache* c) {
    if (!c->block_size) return;
    for (int b = 0; b < c->cfg.batch; ++b) {
        int64_t longest = 0;
        for (int l = 0; l < c->cfg.n_layers; ++l)
            longest = std::max(longest, c->fill[static_cast<size_t>(l) * c->cfg.batch + b]);
        shrink_blocks(c, b, longest);
    }
}

// Append with or without the rotary embedding of K (rope_base > 0).
int append_impl(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new, int32_t in_dtype, int32_t T,
                double rope_base, void* stream) {
    if (!c || !k_new || !v_new) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1) return KVC_ERR_ARG;
    if (!dtype_ok(in_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_ERR_ARG;
    int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] + T > cf.max_len) return KVC_ERR_CAPACITY;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->block_size) {
        const int rc = grow_blocks(c, f, T, s);
        if (rc != KVC_OK) return rc;
    }

    const int64_t head_stride = cf.max_len * cf.d_head;
    const int64_t row_stride = head_stride * cf.n_kv_heads;
    const int64_t in_row = static_cast<int64_t>(cf.n_kv_heads) * T * cf.d_head * kvc::itemsize(in_dtype);
    for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
        kvc::AppendArgs a;
        std::memset(&a, 0, sizeof(a));
        a.rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
        a.k_cache = c->k_store;
        a.v_cache = c->v_store;
        a.k_in = static_cast<const char*>(k_new) + row0 * in_row;
        a.v_in = static_cast<const char*>(v_new) + row0 * in_row;
        a.layer_off = (static_cast<int64_t>(layer) * cf.batch + row0) * row_stride;
        a.row_stride = row_stride;
        a.head_stride = head_stride;
        a.H = cf.n_kv_heads;
        a.T = T;
        a.D = cf.d_head;
        a.in_dtype = in_dtype;
        a.st_dtype = cf.dtype;
        a.rope = rope_base > 0.0 ? 1 : 0;
        a.n_tensors = 2;
        if (c->block_size) {
            a.layer_off = layer * pool_layer_elems(c);
            a.btab = c->d_table + static_cast<int64_t>(row0) * c->width;
            a.btab_stride = c->width;
            a.bshift = c->bshift;
            a.pool_blocks = c->n_blocks;
        }
        if (a.rope) rope_freqs(rope_base, cf.d_head, a.inv_freq);
        for (int b = 0; b < a.rows; ++b) a.fill[b] = static_cast<int32_t>(f[row0 + b]);
        if (kvc::launch_append(a, s) != hipSuccess) {
            // fills unchanged: launches that did run wrote only past the fills
            release_unused(c);
            return KVC_ERR_HIP;
        }
    }
    for (int b = 0; b < cf.batch; ++b) f[b] += T;
    return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_append(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new, int32_t in_dtype, int32_t T,
               void* stream) {
    return append_impl(c, layer, k_new, v_new, in_dtype, T, 0.0, stream);
}

int kvc_append_rope(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new, int32_t in_dtype,
                    int32_t T, double rope_base, void* stream) {
    if (!rope_base_ok(rope_base)) return KVC_ERR_ARG;
    return append_impl(c, layer, k_new, v_new, in_dtype, T, rope_base, stream);
}

int kvc_rope_q(const kvc_cache* c, int32_t layer, void* q, int32_t q_dtype, int32_t T, double rope_base,
               void* stream) {
    if (!c || !q) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1 || !rope_base_ok(rope_base)) return KVC_ERR_ARG;
    if (!dtype_ok(q_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(q)) return KVC_ERR_ARG;
    const int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] < T) return KVC_ERR_STATE;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    const int64_t row_bytes = static_cast<int64_t>(cf.n_q_heads) * T * cf.d_head * kvc::itemsize(q_dtype);
    for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
        kvc::RopeArgs a;
        std::memset(&a, 0, sizeof(a));
        a.x = static_cast<char*>(q) + row0 * row_bytes;
        a.rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
        a.H = cf.n_q_heads;
        a.T = T;
        a.D = cf.d_head;
        a.dtype = q_dtype;
        rope_freqs(rope_base, cf.d_head, a.inv_freq);
        for (int b = 0; b < a.rows; ++b) a.pos0[b] = static_cast<int32_t>(f[row0 + b] - T);
        if (kvc::launch_rope(a, static_cast<hipStream_t>(stream)) != hipSuccess) return KVC_ERR_HIP;
    }
    return KVC_OK;
}

}  // extern "C"

namespace {

// Attention of the last T positions of `layer` (arguments checked by the caller),
// each row's fill taken as fill + pending. k_new, v_new non-null: a fused
// append whose chunk (pending = T positions, not yet counted in the fills) the
// decode kernel reads from the input and its merge pass stores (one slab).
struct Workspace {
    float* o;
    float* ml;
    int64_t rows_cap;    // records x rows the two regions hold
};

Workspace handle_workspace(const kvc_cache* c) {
    return {c->ws_o, c->ws_ml, c->ws_segments * kWsRecordRows};
}

// Rows of split-K records a call's largest launch may need: one slab of up to
// kMaxDecodeRows rows per (row, KV head) unit of a launch, plus one record.
int64_t workspace_rows_needed(const kvc_config& cf) {
    return static_cast<int64_t>(kMaxDecodeRows) * (static_cast<int64_t>(std::min(cf.batch, kMaxRowsPerLaunch)) *
                                                   cf.n_kv_heads + 1);
}

int attend_impl(kvc_cache* c, int32_t layer, const void* q, int32_t q_dtype, int32_t T, float* out, void* stream,
                const void* k_new, const void* v_new, int64_t pending, const Workspace& ws) {
    const kvc_config& cf = c->cfg;
    const int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];

    const int G = cf.n_q_heads / cf.n_kv_heads;
    const int64_t head_stride = cf.max_len * cf.d_head;
    const int64_t row_stride = head_stride * cf.n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(cf.d_head)));

    // Dispatch: a 16-bit cache with more than 32 query rows per KV head (a prefill
    // chunk) runs on the matrix cores; everything else on the split-K decode kernel.
    const bool paged = c->block_size > 0;
    if (!k_new && cf.dtype != KVC_F32 && static_cast<int64_t>(T) * G > 32 &&
        kvc::prefill_supported(cf.d_head, cf.dtype)) {
        const int Gc = std::min(G, 32);
        for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
            const int rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
            for (int r0 = 0; r0 < G; r0 += Gc) {
                kvc::PrefillArgs a;
                std::memset(&a, 0, sizeof(a));
                a.k_cache = c->k_store;
                a.v_cache = c->v_store;
                a.q = q;
                a.out = out;
                a.layer_off = (static_cast<int64_t>(layer) * cf.batch + row0) * row_stride;
                a.row_stride = row_stride;
                a.head_stride = head_stride;
                a.row0 = row0;
                a.rows = rows;
                a.Hq = cf.n_q_heads;
                a.Hkv = cf.n_kv_heads;
                a.G = G;
                a.T = T;
                a.D = cf.d_head;
                a.r0 = r0;
                a.Gc = std::min(Gc, G - r0);
                a.i0 = 0;
                a.Ti = T;
                a.qpt = 32 / a.Gc;
                a.q_per_block = a.qpt * (kvc::prefill_columns_per_block() / 32);
                a.q_dtype = q_dtype;
                a.st_dtype = cf.dtype;
                a.scale_log2 = scale_log2;
                a.p_split = c->prefill_precision == KVC_PREFILL_P_SPLIT;
                if (paged) {
                    a.layer_off = layer * pool_layer_elems(c);
                    a.row_stride = 0;
                    a.head_stride = 0;
                    a.btab = c->d_table + static_cast<int64_t>(row0) * c->width;
                    a.btab_stride = c->width;
                    a.bshift = c->bshift;
                    a.pool_blocks = c->n_blocks;
                }
                for (int b = 0; b < rows; ++b) a.offset[b] = static_cast<int32_t>(f[row0 + b] + pending - T);
                if (kvc::launch_prefill(a, s) != hipSuccess) return KVC_ERR_HIP;
            }
        }
        return KVC_OK;
    }

    // Slabs of at most kMaxDecodeRows query rows per KV head: Gc query heads
    // of the group times Tc query positions.
    const int Gc = std::min(G, kMaxDecodeRows);
    const int Tc = std::max(1, kMaxDecodeRows / Gc);
    for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
        const int rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
        for (int r0 = 0; r0 < G; r0 += Gc) {
            for (int i0 = 0; i0 < T; i0 += Tc) {
                kvc::DecodeArgs a;
                std::memset(&a, 0, sizeof(a));
                a.k_cache = c->k_store;
                a.v_cache = c->v_store;
                a.q = q;
                a.out = out;
                a.ws_o = ws.o;
                a.ws_ml = ws.ml;
                a.ws_rows_cap = ws.rows_cap;
                a.layer_off = (static_cast<int64_t>(layer) * cf.batch + row0) * row_stride;
                a.row_stride = row_stride;
                a.head_stride = head_stride;
                a.row0 = row0;
                a.rows = rows;
                a.Hq = cf.n_q_heads;
                a.Hkv = cf.n_kv_heads;
                a.G = G;
                a.T = T;
                a.D = cf.d_head;
                a.r0 = r0;
                a.Gc = std::min(Gc, G - r0);
                a.i0 = i0;
                a.Tc = std::min(Tc, T - i0);
                a.q_dtype = q_dtype;
                a.st_dtype = cf.dtype;
                a.scale_log2 = scale_log2;
                if (paged) {
                    a.layer_off = layer * pool_layer_elems(c);
                    a.row_stride = 0;
                    a.head_stride = 0;
                    a.btab = c->d_table + static_cast<int64_t>(row0) * c->width;
                    a.btab_stride = c->width;
                    a.bshift = c->bshift;
                    a.pool_blocks = c->n_blocks;
                }
                int64_t acc = 0;
                for (int b = 0; b < rows; ++b) {
                    a.prefix[b] = acc;
                    const int64_t n_b = f[row0 + b] + pending - T + i0 + a.Tc;   // keys the slab's last query sees
                    acc += n_b * cf.n_kv_heads;
                }
                a.prefix[rows] = acc;
                // entries past the last row stay above every key position (the
                // kernels find a position's row by counting entries at or below it)
                for (int b = rows + 1; b <= kMaxRowsPerLaunch; ++b) a.prefix[b] = INT64_MAX;
                a.total_keys = acc;
                a.k_new = k_new;
                a.v_new = v_new;
                if (kvc::launch_decode(a, s) != hipSuccess) return KVC_ERR_HIP;
            }
        }
    }
    return KVC_OK;
}

// Whether append + attend of a chunk can run as one decode launch: the input
// already has the storage type and the chunk is one decode slab (at most 32
// query rows per KV head on a 16-bit cache, the matrix-core kernel; at most 8
// on an fp32 cache, the vector kernel).
bool fusable(const kvc_cache* c, int32_t in_dtype, int32_t T) {
    const kvc_config& cf = c->cfg;
    const int64_t rows = static_cast<int64_t>(T) * (cf.n_q_heads / cf.n_kv_heads);
    return in_dtype == cf.dtype && rows <= (cf.dtype == KVC_F32 ? 8 : kMaxDecodeRows);
}

}  // namespace

extern "C" {

int kvc_attend(kvc_cache* c, int32_t layer, const void* q, int32_t q_dtype, int32_t T, float* out, void* stream) {
    if (!c || !q || !out) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1) return KVC_ERR_ARG;
    if (!dtype_ok(q_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(q) || !aligned16(out)) return KVC_ERR_ARG;
    const int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] < T) return KVC_ERR_STATE;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    return attend_impl(c, layer, q, q_dtype, T, out, stream, nullptr, nullptr, 0, handle_workspace(c));
}

int kvc_attend_static(kvc_cache* c, int32_t layer, const void* q, int32_t q_dtype, int32_t T, float* out,
                      void* stream) {
    if (!c || !q || !out) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1) return KVC_ERR_ARG;
    if (!dtype_ok(q_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(q) || !aligned16(out)) return KVC_ERR_ARG;
    const int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] < T) return KVC_ERR_STATE;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    float* base = nullptr;
    int64_t n_floats = 0;
    if (kvc::static_scratch(c->device, &base, &n_floats) != hipSuccess) return KVC_ERR_HIP;
    // records of d_head outputs plus a (max, sum) pair per row
    const int64_t rows_cap = n_floats / (cf.d_head + 2);
    if (rows_cap < workspace_rows_needed(cf)) return KVC_ERR_SCRATCH;
    const Workspace ws{base, base + rows_cap * cf.d_head, rows_cap};
    return attend_impl(c, layer, q, q_dtype, T, out, stream, nullptr, nullptr, 0, ws);
}

int kvc_append_attend(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new, int32_t in_dtype,
                      const void* q, int32_t q_dtype, int32_t T, float* out, void* stream) {
    if (!c || !k_new || !v_new || !q || !out) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1) return KVC_ERR_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(q_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out)) return KVC_ERR_ARG;
    int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] + T > cf.max_len) return KVC_ERR_CAPACITY;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    if (!fusable(c, in_dtype, T)) {
        const int rc = append_impl(c, layer, k_new, v_new, in_dtype, T, 0.0, stream);
        if (rc != KVC_OK) return rc;
        const int ra = attend_impl(c, layer, q, q_dtype, T, out, stream, nullptr, nullptr, 0, handle_workspace(c));
        if (ra != KVC_OK) {
            // undo the append: fills back, blocks it took given back (its slots
            // now lie past the fills)
            for (int b = 0; b < cf.batch; ++b) f[b] -= T;
            release_unused(c);
        }
        return ra;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->block_size) {
        const int rg = grow_blocks(c, f, T, s);
        if (rg != KVC_OK) return rg;
    }
    const int ra = attend_impl(c, layer, q, q_dtype, T, out, stream, k_new, v_new, T, handle_workspace(c));
    if (ra != KVC_OK) {
        release_unused(c);
        return ra;
    }
    for (int b = 0; b < cf.batch; ++b) f[b] += T;
    return KVC_OK;
}

int kvc_gather(const kvc_cache* c, int32_t layer, int64_t n, void* k_out, void* v_out, void* stream) {
    if (!c || !k_out || !v_out) return KVC_ERR_ARG;
    const kvc_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || n < 1 || n > cf.max_len) return KVC_ERR_ARG;
    if (!aligned16(k_out) || !aligned16(v_out)) return KVC_ERR_ARG;
    if (!on_device(c)) return KVC_ERR_STORAGE;
    const int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    const int64_t head_stride = cf.max_len * cf.d_head;
    const int64_t row_stride = head_stride * cf.n_kv_heads;
    const int64_t out_row = static_cast<int64_t>(cf.n_kv_heads) * n * cf.d_head * kvc::itemsize(cf.dtype);
    for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
        kvc::GatherArgs a;
        std::memset(&a, 0, sizeof(a));
        kvc::AppendArgs& l = a.loc;
        l.rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
        l.k_cache = c->k_store;
        l.v_cache = c->v_store;
        l.layer_off = (static_cast<int64_t>(layer) * cf.batch + row0) * row_stride;
        l.row_stride = row_stride;
        l.head_stride = head_stride;
        l.H = cf.n_kv_heads;
        l.T = static_cast<int32_t>(n);
        l.D = cf.d_head;
        l.st_dtype = cf.dtype;
        if (c->block_size) {
            l.layer_off = layer * pool_layer_elems(c);
            l.btab = c->d_table + static_cast<int64_t>(row0) * c->width;
            l.btab_stride = c->width;
            l.bshift = c->bshift;
            l.pool_blocks = c->n_blocks;
        }
        for (int b = 0; b < l.rows; ++b) l.fill[b] = static_cast<int32_t>(f[row0 + b]);
        a.k_out = static_cast<char*>(k_out) + row0 * out_row;
        a.v_out = static_cast<char*>(v_out) + row0 * out_row;
        if (kvc::launch_gather(a, static_cast<hipStream_t>(stream)) != hipSuccess) return KVC_ERR_HIP;
    }
    return KVC_OK;
}

int kvc_seq_len(const kvc_cache* c, int32_t layer, int64_t* out_lens) {
    if (!c || !out_lens) return KVC_ERR_ARG;
    if (layer < -1 || layer >= c->cfg.n_layers) return KVC_ERR_ARG;
    for (int b = 0; b < c->cfg.batch; ++b)
        out_lens[b] = layer == -1 ? committed(c, b) : c->fill[static_cast<size_t>(layer) * c->cfg.batch + b];
    return KVC_OK;
}

int kvc_truncate(kvc_cache* c, const int64_t* n, int32_t count) {
    if (!c || !n) return KVC_ERR_ARG;
    const int B = c->cfg.batch;
    if (count != 1 && count != B) return KVC_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        const int64_t nb = n[count == 1 ? 0 : b];
        if (nb < 0 || nb > committed(c, b)) return KVC_ERR_STATE;
    }
    for (int b = 0; b < B; ++b) {
        const int64_t nb = n[count == 1 ? 0 : b];
        for (int l = 0; l < c->cfg.n_layers; ++l) c->fill[static_cast<size_t>(l) * B + b] = nb;
        if (c->block_size) shrink_blocks(c, b, nb);
    }
    return KVC_OK;
}

int kvc_set_prefill_precision(kvc_cache* c, int32_t mode) {
    if (!c || (mode != KVC_PREFILL_P_ROUNDED && mode != KVC_PREFILL_P_SPLIT)) return KVC_ERR_ARG;
    c->prefill_precision = mode;
    return KVC_OK;
}

int kvc_nbytes(const kvc_cache* c, uint64_t* out) {
    if (!c || !out) return KVC_ERR_ARG;
    *out = c->block_size ? pool_bytes(c->cfg, c->block_size, c->n_blocks) : storage_bytes(c->cfg);
    return KVC_OK;
}

int kvc_paged_blocks(const kvc_cache* c, int32_t* in_use, int32_t* total) {
    if (!c || !in_use || !total) return KVC_ERR_ARG;
    if (!c->block_size) return KVC_ERR_STATE;
    *total = c->n_blocks;
    *in_use = c->n_blocks - static_cast<int32_t>(c->free_ids.size());
    return KVC_OK;
}

int kvc_block_table(const kvc_cache* c, int32_t* out, int64_t n) {
    if (!c || !out) return KVC_ERR_ARG;
    if (!c->block_size) return KVC_ERR_STATE;
    if (n != static_cast<int64_t>(c->table.size())) return KVC_ERR_ARG;
    std::copy(c->table.begin(), c->table.end(), out);
    return KVC_OK;
}

}  // extern "C"
