// Append kernel: write a chunk of T positions of K and V into the
// preallocated (L, B, H_kv, max_len, D) cache at each row's fill offset,
// rounding to the storage dtype on the way in ("KV cache, incremental decode,
// ...", sections 2.5 and 4; "kv-cache-decoding", step 5: slots t .. t+m-1).
//
// For one (row, KV head) the chunk is T*D contiguous elements in the input
// and T*D contiguous elements in the cache, so the copy is a set of
// rows*H_kv contiguous runs. Each thread moves 8 elements (16 or 32 bytes),
// consecutive threads move consecutive vectors: every wave reads and writes
// one contiguous stretch per run, fully coalesced. blockIdx.y selects K or V.
//
// With rope set, K is stored rotated at its absolute positions fill_b + t
// ("KV cache, incremental decode, ...": keys are kept after RoPE, so a cached
// key never changes; "kv-cache-decoding", "Position information with a
// cache"): each thread then takes 8 pairs (elements i and i + D/2) of one
// position. rope_kernel rotates a chunk's queries in place the same way.
#include "kvc_device.h"

namespace kvc {
namespace {

// Element offset of position p of row b, head g: contiguous (L, B, H, max_len,
// D) storage, or a paged pool (the block's id clamped into the pool, so a
// stale table entry can never address outside it).
__device__ __forceinline__ int64_t slot_offset(const AppendArgs& a, int b, int g, int64_t p) {
    if (a.btab == nullptr)
        return a.layer_off + b * a.row_stride + g * a.head_stride + p * a.D;
    int blk = a.btab[static_cast<int64_t>(b) * a.btab_stride + (p >> a.bshift)];
    blk = blk < 0 ? 0 : (blk >= a.pool_blocks ? a.pool_blocks - 1 : blk);
    const int64_t mask = (int64_t(1) << a.bshift) - 1;
    return a.layer_off + (((static_cast<int64_t>(blk) * a.H + g) << a.bshift) + (p & mask)) * a.D;
}

template <int IN, int ST>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const void* src = blockIdx.y == 0 ? a.k_in : a.v_in;
    void* dst = blockIdx.y == 0 ? a.k_cache : a.v_cache;
    if (blockIdx.y == 0 && a.rope) {
        const int half = a.D >> 1;
        const int blk_per_pos = half >> 3;                      // 8-pair blocks per position
        const int64_t n_blk = static_cast<int64_t>(a.rows) * a.H * a.T * blk_per_pos;
        for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < n_blk;
             v += static_cast<int64_t>(gridDim.x) * blockDim.x) {
            const int64_t run_t = v / blk_per_pos;              // (row, head, t)
            const int i0 = static_cast<int>(v - run_t * blk_per_pos) * 8;
            const int64_t run = run_t / a.T;
            const int t = static_cast<int>(run_t - run * a.T);
            const int b = static_cast<int>(run / a.H);
            const int g = static_cast<int>(run - static_cast<int64_t>(b) * a.H);
            float x1[8], x2[8], y1[8], y2[8];
            load8<IN>(src, run_t * a.D + i0, x1);
            load8<IN>(src, run_t * a.D + i0 + half, x2);
            rope8(x1, x2, static_cast<int64_t>(a.fill[b]) + t, a.inv_freq + i0, y1, y2);
            const int64_t d = slot_offset(a, b, g, static_cast<int64_t>(a.fill[b]) + t) + i0;
            store8<ST>(dst, d, y1);
            store8<ST>(dst, d + half, y2);
        }
        return;
    }
    const int vec_per_run = (a.T * a.D) >> 3;
    const int64_t n_vec = static_cast<int64_t>(a.rows) * a.H * vec_per_run;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < n_vec;
         v += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t run = v / vec_per_run;
        const int within = static_cast<int>(v - run * vec_per_run);
        const int b = static_cast<int>(run / a.H);
        const int g = static_cast<int>(run - static_cast<int64_t>(b) * a.H);
        float x[8];
        load8<IN>(src, v * 8, x);
        const int e = within * 8;
        const int64_t d = slot_offset(a, b, g, static_cast<int64_t>(a.fill[b]) + e / a.D) + e % a.D;
        store8<ST>(dst, d, x);
    }
}

template <int IN>
hipError_t dispatch_st(const AppendArgs& a, dim3 grid, hipStream_t s) {
    switch (a.st_dtype) {
        case F32: append_kernel<IN, F32><<<grid, 256, 0, s>>>(a); break;
        case F16: append_kernel<IN, F16><<<grid, 256, 0, s>>>(a); break;
        case BF16: append_kernel<IN, BF16><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DT>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
    const int half = a.D >> 1;
    const int blk_per_pos = half >> 3;
    const int64_t n_blk = static_cast<int64_t>(a.rows) * a.H * a.T * blk_per_pos;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < n_blk;
         v += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t run_t = v / blk_per_pos;
        const int i0 = static_cast<int>(v - run_t * blk_per_pos) * 8;
        const int64_t run = run_t / a.T;
        const int t = static_cast<int>(run_t - run * a.T);
        const int b = static_cast<int>(run / a.H);
        float x1[8], x2[8], y1[8], y2[8];
        load8<DT>(a.x, run_t * a.D + i0, x1);
        load8<DT>(a.x, run_t * a.D + i0 + half, x2);
        rope8(x1, x2, static_cast<int64_t>(a.pos0[b]) + t, a.inv_freq + i0, y1, y2);
        store8<DT>(a.x, run_t * a.D + i0, y1);
        store8<DT>(a.x, run_t * a.D + i0 + half, y2);
    }
}

// One 16-byte vector per thread and step; blockIdx.y selects K or V.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    const AppendArgs& l = a.loc;
    const int esz = l.st_dtype == F32 ? 4 : 2;
    const int vpp = l.D * esz / 16;                         // 16-byte vectors per position
    const int64_t n_vec = static_cast<int64_t>(l.rows) * l.H * l.T * vpp;
    const char* src = static_cast<const char*>(blockIdx.y == 0 ? l.k_cache : l.v_cache);
    char* dst = static_cast<char*>(blockIdx.y == 0 ? a.k_out : a.v_out);
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < n_vec;
         v += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t pos_run = v / vpp;                    // (row, head, position)
        const int within = static_cast<int>(v - pos_run * vpp);
        const int64_t run = pos_run / l.T;
        const int64_t p = pos_run - run * l.T;
        const int b = static_cast<int>(run / l.H);
        const int g = static_cast<int>(run - static_cast<int64_t>(b) * l.H);
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (p < l.fill[b]) x = *reinterpret_cast<const uint4*>(src + slot_offset(l, b, g, p) * esz + within * 16);
        *reinterpret_cast<uint4*>(dst + v * 16) = x;
    }
}

__global__ __launch_bounds__(256) void table_set_kernel(TableSetArgs a) {
    for (int i = threadIdx.x; i < a.n; i += 256) a.table[a.index[i]] = a.value[i];
}

}  // namespace

hipError_t launch_table_set(const TableSetArgs& a, hipStream_t s) {
    if (a.n < 1 || a.n > kMaxTableSets) return hipErrorInvalidValue;
    table_set_kernel<<<1, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
    const int64_t n_blk = static_cast<int64_t>(a.rows) * a.H * a.T * (a.D >> 4);
    int64_t blocks = (n_blk + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    switch (a.dtype) {
        case F32: rope_kernel<F32><<<static_cast<unsigned>(blocks), 256, 0, s>>>(a); break;
        case F16: rope_kernel<F16><<<static_cast<unsigned>(blocks), 256, 0, s>>>(a); break;
        case BF16: rope_kernel<BF16><<<static_cast<unsigned>(blocks), 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
    const int esz = a.loc.st_dtype == F32 ? 4 : 2;
    const int64_t n_vec = static_cast<int64_t>(a.loc.rows) * a.loc.H * a.loc.T * (a.loc.D * esz / 16);
    int64_t blocks = (n_vec + 255) / 256;
    if (blocks > 8192) blocks = 8192;   // grid-stride beyond this
    if (blocks < 1) blocks = 1;
    gather_kernel<<<dim3(static_cast<unsigned>(blocks), 2), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
    const int64_t n_vec = static_cast<int64_t>(a.rows) * a.H * ((a.T * a.D) >> 3);
    int64_t blocks = (n_vec + 255) / 256;
    if (blocks > 8192) blocks = 8192;   // grid-stride beyond this
    if (blocks < 1) blocks = 1;
    dim3 grid(static_cast<unsigned>(blocks), a.n_tensors == 1 ? 1 : 2);
    switch (a.in_dtype) {
        case F32: return dispatch_st<F32>(a, grid, s);
        case F16: return dispatch_st<F16>(a, grid, s);
        case BF16: return dispatch_st<BF16>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
