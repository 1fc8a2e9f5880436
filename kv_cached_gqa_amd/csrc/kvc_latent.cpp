// Host core and C ABI of the latent cache (declared in include/kvc.h).
//
// Multi-head latent attention caches one compressed latent c (rank r) and one
// shared rotary key k_R (d_R) per position instead of per-head K and V; the
// cache follows the K/V cache's rules, per-layer fill, committed length as the
// minimum over layers, metadata-only rollback, on [B, T, r] and [B, T, d_R]
// chunks ("KV cache, incremental decode, ...", section 2.6). Storage is
// [n_layers][batch][max_len][r] for c and [n_layers][batch][max_len][d_R] for
// k_R, caller-owned; a chunk row is one contiguous run per tensor, so the
// append kernel of the K/V cache writes it (one head, width r or d_R).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kvc.h"
#include "kvc_kernels.h"

using kvc::kMaxRowsPerLaunch;

struct kvc_latent {
    kvc_latent_config cfg;
    void* c_store;
    void* kr_store;
    std::vector<int64_t> fill;    // [n_layers][batch]
};

namespace {

bool latent_dtype_ok(int32_t dt) { return dt == KVC_F32 || dt == KVC_F16 || dt == KVC_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t tensor_bytes(const kvc_latent_config& c, int32_t width) {
    return static_cast<uint64_t>(c.n_layers) * c.batch * static_cast<uint64_t>(c.max_len) * width *
           kvc::itemsize(c.dtype);
}

int64_t committed(const kvc_latent* c, int b) {
    int64_t s = c->fill[b];
    for (int l = 1; l < c->cfg.n_layers; ++l) s = std::min(s, c->fill[static_cast<size_t>(l) * c->cfg.batch + b]);
    return s;
}

// One tensor of the chunk (width D) into its storage for rows row0 .. row0 + rows.
hipError_t append_tensor(const kvc_latent* c, void* store, const void* in, int32_t D, int32_t layer, int32_t in_dtype,
                         int32_t T, const int64_t* f, hipStream_t s) {
    const kvc_latent_config& cf = c->cfg;
    const int64_t row_stride = cf.max_len * static_cast<int64_t>(D);
    const int64_t in_row = static_cast<int64_t>(T) * D * kvc::itemsize(in_dtype);
    for (int row0 = 0; row0 < cf.batch; row0 += kMaxRowsPerLaunch) {
        kvc::AppendArgs a;
        std::memset(&a, 0, sizeof(a));
        a.rows = std::min(kMaxRowsPerLaunch, cf.batch - row0);
        a.k_cache = store;
        a.v_cache = store;
        a.k_in = static_cast<const char*>(in) + row0 * in_row;
        a.v_in = a.k_in;
        a.layer_off = (static_cast<int64_t>(layer) * cf.batch + row0) * row_stride;
        a.row_stride = row_stride;
        a.head_stride = row_stride;
        a.H = 1;
        a.T = T;
        a.D = D;
        a.in_dtype = in_dtype;
        a.st_dtype = cf.dtype;
        a.n_tensors = 1;
        for (int b = 0; b < a.rows; ++b) a.fill[b] = static_cast<int32_t>(f[row0 + b]);
        const hipError_t e = kvc::launch_append(a, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

int kvc_latent_create(const kvc_latent_config* cfg, void* c_store, void* kr_store, uint64_t c_bytes,
                      uint64_t kr_bytes, kvc_latent** out) {
    if (!cfg || !out) return KVC_ERR_ARG;
    const kvc_latent_config c = *cfg;
    if (c.n_layers < 1 || c.batch < 1 || c.rank < 8 || c.rope_dim < 8 || c.max_len < 1) return KVC_ERR_ARG;
    if (c.rank % 8 || c.rope_dim % 8) return KVC_ERR_ARG;   // whole 8-element vectors per position
    if (c.max_len * static_cast<int64_t>(std::max(c.rank, c.rope_dim)) >= (int64_t(1) << 31)) return KVC_ERR_ARG;
    if (!latent_dtype_ok(c.dtype)) return KVC_ERR_DTYPE;
    if (!c_store || !kr_store || !aligned16(c_store) || !aligned16(kr_store)) return KVC_ERR_STORAGE;
    if (c_bytes < tensor_bytes(c, c.rank) || kr_bytes < tensor_bytes(c, c.rope_dim)) return KVC_ERR_STORAGE;
    kvc_latent* h = new (std::nothrow) kvc_latent();
    if (!h) return KVC_ERR_NOMEM;
    try {
        h->fill.assign(static_cast<size_t>(c.n_layers) * c.batch, 0);
    } catch (...) {
        delete h;
        return KVC_ERR_NOMEM;
    }
    h->cfg = c;
    h->c_store = c_store;
    h->kr_store = kr_store;
    *out = h;
    return KVC_OK;
}

void kvc_latent_destroy(kvc_latent* c) { delete c; }

int kvc_latent_append(kvc_latent* c, int32_t layer, const void* c_new, const void* kr_new, int32_t in_dtype,
                      int32_t T, void* stream) {
    if (!c || !c_new || !kr_new) return KVC_ERR_ARG;
    const kvc_latent_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || T < 1) return KVC_ERR_ARG;
    if (!latent_dtype_ok(in_dtype)) return KVC_ERR_DTYPE;
    if (!aligned16(c_new) || !aligned16(kr_new)) return KVC_ERR_ARG;
    int64_t* f = &c->fill[static_cast<size_t>(layer) * cf.batch];
    for (int b = 0; b < cf.batch; ++b)
        if (f[b] + T > cf.max_len) return KVC_ERR_CAPACITY;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (append_tensor(c, c->c_store, c_new, cf.rank, layer, in_dtype, T, f, s) != hipSuccess) return KVC_ERR_HIP;
    if (append_tensor(c, c->kr_store, kr_new, cf.rope_dim, layer, in_dtype, T, f, s) != hipSuccess)
        return KVC_ERR_HIP;
    for (int b = 0; b < cf.batch; ++b) f[b] += T;
    return KVC_OK;
}

int kvc_latent_seq_len(const kvc_latent* c, int32_t layer, int64_t* out_lens) {
    if (!c || !out_lens || layer < -1 || layer >= c->cfg.n_layers) return KVC_ERR_ARG;
    for (int b = 0; b < c->cfg.batch; ++b)
        out_lens[b] = layer < 0 ? committed(c, b) : c->fill[static_cast<size_t>(layer) * c->cfg.batch + b];
    return KVC_OK;
}

int kvc_latent_truncate(kvc_latent* c, const int64_t* n, int32_t count) {
    if (!c || !n || (count != 1 && count != c->cfg.batch)) return KVC_ERR_ARG;
    const int B = c->cfg.batch;
    for (int b = 0; b < B; ++b) {
        const int64_t nb = n[count == 1 ? 0 : b];
        if (nb < 0 || nb > committed(c, b)) return KVC_ERR_STATE;
    }
    for (int l = 0; l < c->cfg.n_layers; ++l)
        for (int b = 0; b < B; ++b) c->fill[static_cast<size_t>(l) * B + b] = n[count == 1 ? 0 : b];
    return KVC_OK;
}

int kvc_latent_nbytes(const kvc_latent* c, uint64_t* out) {
    if (!c || !out) return KVC_ERR_ARG;
    *out = tensor_bytes(c->cfg, c->cfg.rank) + tensor_bytes(c->cfg, c->cfg.rope_dim);
    return KVC_OK;
}

}  // extern "C"
