// Split-K decode kernels for head dimension 128, bf16 storage.
#include "kvc_decode_impl.h"

namespace kvc {
template hipError_t decode_run<128, BF16>(DecodeArgs& a, hipStream_t s);
template int decode_batch_keys<128, BF16>(int rows);
}  // namespace kvc

#if KVC_DECODE_TIMESTAMPS
// The timestamp probe's records of this unit's kernels (kv_cached_gqa_amd.probe):
// clear them, and copy out n_wg work-group records of 6 values and n_merge
// merge-block records of 4.
extern "C" int kvc_probe_clear() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(kvc::kvc_probe_wg)) != hipSuccess ||
        hipMemset(p, 0, sizeof(unsigned long long) * kvc::kMaxDecodeBlocks * 6) != hipSuccess)
        return -1;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(kvc::kvc_probe_merge)) != hipSuccess ||
        hipMemset(p, 0, sizeof(unsigned long long) * kvc::kProbeMergeBlocks * 4) != hipSuccess)
        return -1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
extern "C" int kvc_probe_read(unsigned long long* wg, int n_wg, unsigned long long* merge, int n_merge) {
    if (n_wg > kvc::kMaxDecodeBlocks || n_merge > kvc::kProbeMergeBlocks) return -1;
    if (hipDeviceSynchronize() != hipSuccess) return -1;
    if (hipMemcpyFromSymbol(wg, HIP_SYMBOL(kvc::kvc_probe_wg), sizeof(unsigned long long) * n_wg * 6) != hipSuccess)
        return -1;
    return hipMemcpyFromSymbol(merge, HIP_SYMBOL(kvc::kvc_probe_merge), sizeof(unsigned long long) * n_merge * 4) ==
                   hipSuccess ? 0 : -1;
}
#endif
