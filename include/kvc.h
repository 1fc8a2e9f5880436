/*
 * kvc.h - C ABI of libkvc: a preallocated KV cache with grouped-query
 * attention over it, for AMD Instinct MI355X (gfx950).
 *
 * The contract follows the KVCache interface of "KV cache, incremental
 * decode, incremental UTF-8 detokenizer, generate" (section 4, The interface;
 * section 2.3 for the committed length, positions and mask; section 2.4 for
 * rollback; section 2.5 for the storage dtype and nbytes). Storage layout is
 * the (L, B, H, max_len, d_head) cache of "Generation and the KV Cache"
 * (the KVCache paragraph) with H = the number of KV heads; query heads share
 * KV heads in consecutive groups as in "Heads, GQA and K/V cache"
 * ("Four queries, two sets of K/V").
 *
 * Conventions for every call:
 *  - Return value: KVC_OK (0) or a negative kvc_status. On any error the
 *    cache state (fill counts and storage) is unchanged; arguments are
 *    validated before any device work is enqueued.
 *  - Device pointers are HIP device addresses on the device that holds the
 *    cache storage; they must stay valid until the work enqueued on
 *    `stream` has run. Host pointers are read during the call only.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). All calls
 *    on one handle must be issued in stream order by one thread: the host
 *    metadata advances when a call returns, the device work runs later in
 *    stream order. A handle is not thread-safe.
 *  - Tensors are dense, row-major (C order), with the shapes stated.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. fp32 = IEEE binary32, fp16 = IEEE binary16, bf16 = bfloat16. */
typedef enum kvc_dtype { KVC_F32 = 0, KVC_F16 = 1, KVC_BF16 = 2 } kvc_dtype;

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_ARG = -1,         /* a bad argument: null pointer, shape, layer index, T < 1 */
    KVC_ERR_CAPACITY = -2,    /* an append would write past max_len */
    KVC_ERR_STATE = -3,       /* attend before the chunk was appended; truncate past the committed length */
    KVC_ERR_DTYPE = -4,       /* unknown dtype code */
    KVC_ERR_STORAGE = -5,     /* storage null, too small or not 16-byte aligned */
    KVC_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    KVC_ERR_NOMEM = -7,       /* host or device allocation failed */
    KVC_ERR_UNSUPPORTED = -8, /* a shape outside what the kernels handle (d_head not 32, 64 or 128) */
    KVC_ERR_SCRATCH = -9      /* kvc_attend_static: the call needs more scratch than its static array */
} kvc_status;

/* Shape of a cache. n_q_heads must be a multiple of n_kv_heads (G = n_q_heads /
 * n_kv_heads query heads share each KV head; query head h reads KV head h / G).
 * d_head is 32, 64 or 128. max_len * d_head must be below 2^31. */
typedef struct kvc_config {
    int32_t n_layers;
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t d_head;
    int32_t dtype;      /* kvc_dtype of the stored keys and values */
    int64_t max_len;    /* preallocated positions per row, N_max */
} kvc_config;

typedef struct kvc_cache kvc_cache;

/* Create a handle over caller-owned storage.
 *  k_store, v_store: device buffers, each at least store_bytes_each bytes,
 *    holding [n_layers][batch][n_kv_heads][max_len][d_head] elements of
 *    cfg->dtype, 16-byte aligned, ZERO-FILLED by the caller (never-written
 *    slots read as zero, as in the shapes table of "kv-cache-decoding").
 *    store_bytes_each must be >= nbytes / 2. The caller keeps ownership and
 *    must keep both buffers alive for the life of the handle.
 *  out: receives the handle. Every fill count starts at 0.
 * The library also owns a device workspace for split-K partial results: when
 * the storage is device memory it is allocated here, on the storage's device
 * (so no later call allocates), and freed by kvc_destroy. Storage that is not
 * device memory gives a handle that keeps metadata (seq_len, truncate, nbytes)
 * but launches nothing: every call that would enqueue device work on it
 * returns KVC_ERR_STORAGE. No device work is done here.
 * Errors: KVC_ERR_ARG (null cfg/out, nonpositive dims, n_q_heads not a multiple
 * of n_kv_heads, max_len * d_head >= 2^31), KVC_ERR_DTYPE, KVC_ERR_UNSUPPORTED,
 * KVC_ERR_STORAGE, KVC_ERR_NOMEM. */
int kvc_create(const kvc_config* cfg, void* k_store, void* v_store,
               uint64_t store_bytes_each, kvc_cache** out);

/* Free the handle and its workspace (never the caller's storage). Waits for
 * the device to finish work that may use the workspace. NULL is a no-op. */
void kvc_destroy(kvc_cache* cache);

/* Append a chunk of T positions to one layer ("KV cache, ...", section 4,
 * update; "kv-cache-decoding", step 5).
 *  k_new, v_new: device [batch][n_kv_heads][T][d_head] of in_dtype.
 *  Row b's chunk is written at slots [fill[layer][b], fill[layer][b] + T),
 *  converted to the storage dtype with IEEE round-to-nearest-even (NaN becomes
 *  the canonical quiet NaN of its sign; overflow becomes infinity), and then
 *  fill[layer][b] += T. The inputs are copied: the caller may reuse them once
 *  the stream has passed this call. Earlier slots are never touched, so the
 *  stored values the cache hands back are exactly the rounded inputs.
 *  The committed length (kvc_seq_len with layer -1) moves only when every
 *  layer has appended ("KV cache, ...", section 2.3).
 * Errors: KVC_ERR_ARG (null handle or pointer, layer out of range, T < 1),
 * KVC_ERR_DTYPE, KVC_ERR_CAPACITY (fill + T > max_len for some row),
 * KVC_ERR_STORAGE (the handle's storage is not device memory), KVC_ERR_HIP.
 * On an error the fills and block accounting are unchanged; when a launch
 * fails (a batch above 256 rows takes several), slots past the fills may have
 * been written. */
int kvc_append(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
               int32_t in_dtype, int32_t T, void* stream);

/* Append with the rotary position embedding of the keys ("KV cache,
 * incremental decode, ...": keys are stored after RoPE, so a cached key never
 * changes; "kv-cache-decoding", "Position information with a cache"; the
 * rotary variant and base are left open there, this is the stated reading).
 *  As kvc_append, except that each key vector of row b at slot p = fill + t is
 *  rotated before it is stored: for each pair (i, i + d_head/2), i < d_head/2,
 *  with f_i = rope_base^(-2i / d_head) and angle a = p * f_i,
 *    k'[i]            = k[i] cos a - k[i + d_head/2] sin a
 *    k'[i + d_head/2] = k[i + d_head/2] cos a + k[i] sin a,
 *  computed in float64 (angles, sines and cosines; each product and the sum
 *  rounded, no fused multiply-add), rounded to float32, then to the storage
 *  dtype (round-to-nearest-even). Values are stored unrotated.
 * Errors: as kvc_append; KVC_ERR_ARG also for rope_base not finite or <= 0. */
int kvc_append_rope(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                    int32_t in_dtype, int32_t T, double rope_base, void* stream);

/* Rotate a chunk's queries in place with the same embedding, at the positions
 * the next kvc_attend of this layer gives them: row b's query t sits at
 * s_b + t, s_b = fill[layer][b] - T (so call it after the chunk's append).
 *  q: device [batch][n_q_heads][T][d_head] of q_dtype, 16-byte aligned; the
 *     result is rounded to q_dtype (float64 -> float32 -> q_dtype, nearest even).
 * Errors: KVC_ERR_ARG (null pointer, layer out of range, T < 1, bad rope_base),
 * KVC_ERR_DTYPE, KVC_ERR_STATE (fill[layer][b] < T for some row), KVC_ERR_HIP. */
int kvc_rope_q(const kvc_cache* cache, int32_t layer, void* q, int32_t q_dtype, int32_t T,
               double rope_base, void* stream);

/* Attention of a chunk's queries over everything a layer holds
 * ("KV cache, ...", section 2.3; "kv-cache-decoding", shapes table).
 *  q: device [batch][n_q_heads][T][d_head] of q_dtype. For an fp16/bf16 cache
 *     an fp32 q is first rounded to the storage dtype (round-to-nearest-even);
 *     a q already in a 16-bit type, or any q for an fp32 cache, is used exactly.
 *  out: device float32 [batch][n_q_heads][T][d_head].
 *  The chunk is the last T positions appended to the layer: row b's queries sit
 *  at absolute positions s_b + i, s_b = fill[layer][b] - T, i < T, and query i
 *  sees keys j <= s_b + i (causal_mask(T, s_b + T, q_offset = s_b)). Query head
 *  h reads KV head h / G. out = softmax(q K^T / sqrt(d_head)) V with float32
 *  accumulation. Read-only on the cache; fills are unchanged.
 * Errors: KVC_ERR_ARG (null pointer, layer out of range, T < 1), KVC_ERR_DTYPE,
 * KVC_ERR_STATE (fill[layer][b] < T for some row), KVC_ERR_STORAGE (storage
 * not device memory), KVC_ERR_HIP. Allocates nothing. */
int kvc_attend(kvc_cache* cache, int32_t layer, const void* q, int32_t q_dtype,
               int32_t T, float* out, void* stream);

/* kvc_attend without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it): the same arguments, semantics, kernels and results, except that
 * the split-K partial records live in a file-scope device array of the library
 * (16 MiB, kStaticScratchFloats floats, one per device, held until the process
 * ends) instead of the handle's workspace. The array's device address is looked
 * up once per device at the first call on it (hipGetSymbolAddress; no
 * allocation). Every call on one device shares that device's array: calls that
 * overlap on a device (several streams, threads or handles) race and must be
 * ordered by the caller. The call allocates nothing, host or device.
 * Errors: as kvc_attend; KVC_ERR_SCRATCH when min(batch, 256) * n_kv_heads
 * units of 32-row records (d_head + 2 floats a row), plus one, exceed the
 * array; nothing is enqueued then. */
int kvc_attend_static(kvc_cache* cache, int32_t layer, const void* q, int32_t q_dtype, int32_t T, float* out,
                      void* stream);

/* How a prefill chunk's probabilities enter the product with V on the matrix
 * cores (16-bit caches, chunks of more than 32 query rows per KV head): the
 * attention computed is the one of kvc_attend ("KV cache, incremental decode,
 * ...", section 2.3: softmax(q K^T / sqrt(d_head)) V), and this only sets how
 * closely. */
typedef enum kvc_prefill_precision {
    KVC_PREFILL_P_ROUNDED = 0,  /* P rounded once to the storage type (round to nearest even), the
                                   normaliser summing the rounded values: ~1e-3 relative error per
                                   call on bf16 caches, ~1.5e-4 on fp16 (the default) */
    KVC_PREFILL_P_SPLIT = 1     /* P as a hi + lo pair of the storage type (the residual of the first
                                   rounding rounded again, multiplied with V by a second product):
                                   ~1e-6, with half again as many matrix products (slower) */
} kvc_prefill_precision;

/* Select the prefill precision of one handle (every later kvc_attend and
 * kvc_attend_static on it). Decode calls (32 query rows per KV head or fewer)
 * and fp32 caches are unaffected: their probabilities are kept in float32, or
 * as a hi + lo pair on the matrix cores.
 *  mode: a kvc_prefill_precision value. Host state only; nothing is enqueued.
 * Errors: KVC_ERR_ARG (null handle, unknown mode); the setting is unchanged
 * then. */
int kvc_set_prefill_precision(kvc_cache* cache, int32_t mode);

/* Append a chunk, then attend to everything the layer holds, in one call: the
 * same state change and bit-identical results as kvc_append(k_new, v_new,
 * in_dtype, T) followed by kvc_attend(q, q_dtype, T, out) ("KV cache, ...",
 * section 2.3: a pass appends its chunk, then attends over all stored
 * positions; "kv-cache-decoding", steps 5-6).
 *  When in_dtype is the storage dtype and T * (n_q_heads / n_kv_heads) is at
 *  most 32 (8 for an fp32 cache), a decode step, the attention kernel reads the
 *  chunk's keys and values from k_new and v_new and the merge pass that
 *  follows it stores them in the cache, so no separate append launch runs.
 *  Otherwise the call runs kvc_append, then kvc_attend. Either way k_new, v_new
 *  and q must stay valid until the stream has passed the call, and the cache
 *  ends with the bits kvc_append stores (a 16-bit NaN input becomes the
 *  canonical quiet NaN of its sign on both paths).
 * Errors: those of kvc_append and kvc_attend. On any error the fills and the
 *  paged block accounting are as before the call: the fused path advances the
 *  fills only once its launches are enqueued, and the two-call path undoes its
 *  append when the attention launch fails (slots past the fills may then hold
 *  the chunk). */
int kvc_append_attend(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                      int32_t in_dtype, const void* q, int32_t q_dtype, int32_t T, float* out,
                      void* stream);

/* Copy out what one layer stores ("KV cache, ...", section 4: update returns
 * all stored keys and values, the new chunk included; for a paged cache they
 * are not one contiguous run, so this call assembles them).
 *  k_out, v_out: device [batch][n_kv_heads][n][d_head] of the storage dtype,
 *    16-byte aligned, written on `stream`: position p of row b is the stored
 *    value when p < fill[layer][b], zero otherwise. 1 <= n <= max_len.
 *  Read-only on the cache. Works on contiguous and paged handles.
 * Errors: KVC_ERR_ARG (null, layer out of range, n out of range, misaligned),
 * KVC_ERR_STORAGE (storage not device memory), KVC_ERR_HIP. */
int kvc_gather(const kvc_cache* cache, int32_t layer, int64_t n, void* k_out, void* v_out, void* stream);

/* Per-row lengths ("KV cache, ...", section 2.3, seq_len).
 *  layer = -1: the committed length s_b = min over layers of fill[layer][b];
 *  0 <= layer < n_layers: that layer's fill count.
 *  out_lens: host int64 [batch]. Host metadata only; no device work, no sync.
 * Errors: KVC_ERR_ARG. */
int kvc_seq_len(const kvc_cache* cache, int32_t layer, int64_t* out_lens);

/* Roll back ("KV cache, ...", section 2.4): set EVERY layer's fill of each row
 * to n. n: host int64, count = 1 (one length for all rows) or count = batch
 * (one per row). Each n_b must satisfy 0 <= n_b <= committed length s_b.
 * Storage is not cleared or copied; the next append overwrites from n_b.
 * Host metadata only. Errors: KVC_ERR_ARG (null, count), KVC_ERR_STATE (n out of
 * range). */
int kvc_truncate(kvc_cache* cache, const int64_t* n, int32_t count);

/* Storage bytes, 2 * L * B * H_kv * max_len * d_head * itemsize
 * ("KV cache, ...", section 2.5); for a paged handle the pools,
 * 2 * L * n_blocks * H_kv * block_size * d_head * itemsize. Workspace, block
 * table and metadata are not counted.
 * out: host uint64. Errors: KVC_ERR_ARG. */
int kvc_nbytes(const kvc_cache* cache, uint64_t* out);

/* ---- Paged cache ------------------------------------------------------------
 * The same cache in fixed-size blocks ("kv-cache-decoding", "Batching caches
 * of different lengths": a table maps each request to its blocks; a sequence
 * takes a block when it grows into it and frees its blocks when it ends;
 * "KV cache, incremental decode, ...", Key takeaways: a float16 paged cache
 * compares exactly with the contiguous one). A paged handle takes every call
 * above (append, append_rope, rope_q, attend, seq_len, truncate, nbytes) with
 * the same semantics and results; only the storage differs. */

/* Create a paged handle over caller-owned block pools.
 *  block_size: positions per block, a power of two from 64 to 4096 (at least
 *    the decode kernels' key batch for this d_head and dtype, else
 *    KVC_ERR_UNSUPPORTED; every supported shape's batch is at most 64 keys).
 *  cfg->max_len * d_head must be below 2^31, as for kvc_create.
 *  n_blocks: blocks in the pool, shared by all rows.
 *  k_pool, v_pool: device buffers, each at least pool_bytes_each bytes, holding
 *    [n_layers][n_blocks][n_kv_heads][block_size][d_head] elements of
 *    cfg->dtype, 16-byte aligned (zero-filling is not required: a position is
 *    read only after it was written). Caller-owned, alive for the handle's life.
 *  cfg->max_len bounds each row's length; the block table has
 *  ceil(max_len / block_size) entries per row, one table for all layers, so
 *  position p of row b, KV head g, layer l sits at element
 *    ((l * n_blocks + table[b][p / block_size]) * n_kv_heads + g) * block_size
 *    + p % block_size) * d_head
 *  of each pool. The library owns the device copy of the table (allocated and
 *  zeroed here, on the pools' device) and a free list of blocks.
 *  Blocks: an append (any layer) that takes row b past its held blocks takes
 *  the next ones from the free list, and enqueues the table update on its
 *  stream ahead of its own kernel; truncate to n gives back the row's blocks
 *  past ceil(n / block_size). If the free list cannot cover an append, the
 *  append fails with KVC_ERR_CAPACITY and nothing changes.
 *  Attention over a paged cache takes the same kernels, with the same work
 *  split, as over a contiguous one, so its results are bit-identical.
 * Errors: as kvc_create; KVC_ERR_ARG also for a bad block_size or n_blocks;
 * KVC_ERR_NOMEM if the device table cannot be allocated. */
int kvc_create_paged(const kvc_config* cfg, int32_t block_size, int32_t n_blocks, void* k_pool,
                     void* v_pool, uint64_t pool_bytes_each, kvc_cache** out);

/* Blocks in use and in the pool. Host metadata only.
 * Errors: KVC_ERR_ARG (null), KVC_ERR_STATE (not a paged handle). */
int kvc_paged_blocks(const kvc_cache* cache, int32_t* in_use, int32_t* total);

/* Copy the host block table, int32 [batch][ceil(max_len / block_size)], -1 for
 * an entry with no block, into out (n entries, which must equal that size).
 * Errors: KVC_ERR_ARG (null, n), KVC_ERR_STATE (not a paged handle). */
int kvc_block_table(const kvc_cache* cache, int32_t* out, int64_t n);

/* ---- Latent cache (multi-head latent attention) ---------------------------
 * One compressed latent c (rank r) and one shared rotary key k_R (d_R) per
 * position instead of per-head K and V, under the same rules as the K/V cache:
 * per-layer fill, committed length = min over layers, metadata-only rollback
 * ("KV cache, incremental decode, ...", section 2.6, LatentCache). */
typedef struct kvc_latent_config {
    int32_t n_layers;   /* L */
    int32_t batch;      /* B */
    int32_t rank;       /* r: latent width, a multiple of 8 */
    int32_t rope_dim;   /* d_R: shared rotary key width, a multiple of 8 */
    int32_t dtype;      /* kvc_dtype of the stored values */
    int64_t max_len;    /* preallocated positions per row, N_max */
} kvc_latent_config;

typedef struct kvc_latent kvc_latent;

/* Create a latent-cache handle over caller-owned storage.
 *  c_store: device [n_layers][batch][max_len][rank] of cfg->dtype, at least
 *    c_bytes >= that size; kr_store: [n_layers][batch][max_len][rope_dim],
 *    kr_bytes likewise. Both 16-byte aligned and zero-filled by the caller, who
 *    keeps ownership for the life of the handle. Every fill starts at 0.
 * Errors: KVC_ERR_ARG (null cfg/out, nonpositive dims, rank or rope_dim not a
 * multiple of 8 or below 8, max_len * width >= 2^31), KVC_ERR_DTYPE,
 * KVC_ERR_STORAGE, KVC_ERR_NOMEM. No device work. */
int kvc_latent_create(const kvc_latent_config* cfg, void* c_store, void* kr_store, uint64_t c_bytes,
                      uint64_t kr_bytes, kvc_latent** out);

/* Free the handle (never the caller's storage). NULL is a no-op. */
void kvc_latent_destroy(kvc_latent* cache);

/* Append T positions to one layer: c_new device [batch][T][rank], kr_new
 * [batch][T][rope_dim], both of in_dtype and 16-byte aligned; row b's chunk
 * goes to slots [fill[layer][b], + T), rounded to the storage dtype (nearest
 * even, as kvc_append), then fill[layer][b] += T. Inputs are copied.
 * Errors: KVC_ERR_ARG (null, layer out of range, T < 1, misaligned),
 * KVC_ERR_DTYPE, KVC_ERR_CAPACITY (fill + T > max_len), KVC_ERR_HIP. */
int kvc_latent_append(kvc_latent* cache, int32_t layer, const void* c_new, const void* kr_new,
                      int32_t in_dtype, int32_t T, void* stream);

/* Per-row lengths: layer -1 = committed (min over layers), else that layer's
 * fill. out_lens: host int64 [batch]. Errors: KVC_ERR_ARG. */
int kvc_latent_seq_len(const kvc_latent* cache, int32_t layer, int64_t* out_lens);

/* Set every layer's fill of each row to n (count 1: all rows; count = batch:
 * per row), 0 <= n_b <= committed length. Metadata only.
 * Errors: KVC_ERR_ARG (null, count), KVC_ERR_STATE (n out of range). */
int kvc_latent_truncate(kvc_latent* cache, const int64_t* n, int32_t count);

/* Storage bytes, L * B * N_max * (r + d_R) * itemsize ("KV cache, ...",
 * section 2.6). out: host uint64. Errors: KVC_ERR_ARG. */
int kvc_latent_nbytes(const kvc_latent* cache, uint64_t* out);

/* A static, human-readable text for a kvc_status code. */
const char* kvc_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
