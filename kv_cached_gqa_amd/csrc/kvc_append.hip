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
#include "kvc_device.h"

namespace kvc {
namespace {

template <int IN, int ST>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int vec_per_run = (a.T * a.D) >> 3;
    const int64_t n_vec = static_cast<int64_t>(a.rows) * a.H * vec_per_run;
    const void* src = blockIdx.y == 0 ? a.k_in : a.v_in;
    void* dst = blockIdx.y == 0 ? a.k_cache : a.v_cache;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < n_vec;
         v += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t run = v / vec_per_run;
        const int within = static_cast<int>(v - run * vec_per_run);
        const int b = static_cast<int>(run / a.H);
        const int g = static_cast<int>(run - static_cast<int64_t>(b) * a.H);
        float x[8];
        load8<IN>(src, v * 8, x);
        const int64_t d = a.layer_off + b * a.row_stride + g * a.head_stride +
                          static_cast<int64_t>(a.fill[b]) * a.D + static_cast<int64_t>(within) * 8;
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

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
    const int64_t n_vec = static_cast<int64_t>(a.rows) * a.H * ((a.T * a.D) >> 3);
    int64_t blocks = (n_vec + 255) / 256;
    if (blocks > 8192) blocks = 8192;   // grid-stride beyond this
    if (blocks < 1) blocks = 1;
    dim3 grid(static_cast<unsigned>(blocks), 2);
    switch (a.in_dtype) {
        case F32: return dispatch_st<F32>(a, grid, s);
        case F16: return dispatch_st<F16>(a, grid, s);
        case BF16: return dispatch_st<BF16>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
