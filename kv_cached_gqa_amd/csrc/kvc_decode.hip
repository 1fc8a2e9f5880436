// Decode attention dispatch: picks the instantiation of the split-K decode
// kernels (kvc_decode_impl.h) for a cache's head dimension and storage type.
// The instantiations live in kvc_decode_d<D>_<type>.hip, one translation unit
// each, so that they compile in parallel.
#include <mutex>

#include "kvc_kernels.h"

namespace kvc {

namespace {

// The allocation-free attention call's split-K scratch: partial records and
// their (max, sum) pairs, carved by the caller. Every call on a device shares
// this device's copy (calls that overlap on one device race); it needs no
// clearing, since a launch writes every record it reads.
static __device__ __align__(256) float scratch[kStaticScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int device, float** ptr, int64_t* n_floats) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[device] == nullptr) {
        int prev = 0;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != device) (void)hipSetDevice(prev);
        if (e != hipSuccess) return e;
        scratch_ptr[device] = static_cast<float*>(p);
    }
    *ptr = scratch_ptr[device];
    *n_floats = kStaticScratchFloats;
    return hipSuccess;
}

int decode_vector_batch_keys(int D, int st_dtype, int rows) {
    auto pick = [&](auto d_c) -> int {
        constexpr int DD = decltype(d_c)::value;
        switch (st_dtype) {
            case F32: return decode_batch_keys<DD, F32>(rows);
            case F16: return decode_batch_keys<DD, F16>(rows);
            default: return decode_batch_keys<DD, BF16>(rows);
        }
    };
    switch (D) {
        case 32: return pick(std::integral_constant<int, 32>{});
        case 64: return pick(std::integral_constant<int, 64>{});
        default: return pick(std::integral_constant<int, 128>{});
    }
}

bool decode_supported(int D, int st_dtype) {
    return (D == 32 || D == 64 || D == 128) && (st_dtype == F32 || st_dtype == F16 || st_dtype == BF16);
}

namespace {

template <int D>
hipError_t run_d(DecodeArgs& a, hipStream_t s) {
    switch (a.st_dtype) {
        case F32: return decode_run<D, F32>(a, s);
        case F16: return decode_run<D, F16>(a, s);
        case BF16: return decode_run<D, BF16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(DecodeArgs& a, hipStream_t s) {
    if (a.Gc * a.Tc < 1 || a.Gc * a.Tc > kMaxDecodeRows) return hipErrorInvalidValue;
    if (a.ws_rows_cap < static_cast<int64_t>(kMaxDecodeRows) * (a.rows * a.Hkv + 1)) return hipErrorInvalidValue;
    if (a.total_keys < 1 || a.Hkv < 1) return hipErrorInvalidValue;
    decode_set_hkv_div(a);
    switch (a.D) {
        case 32: return run_d<32>(a, s);
        case 64: return run_d<64>(a, s);
        case 128: return run_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
