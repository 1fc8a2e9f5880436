// Split-K decode kernels for head dimension 128, bf16 storage.
#include "kvc_decode_impl.h"

namespace kvc {
template hipError_t decode_run<128, BF16>(DecodeArgs& a, hipStream_t s);
template int decode_batch_keys<128, BF16>(int rows);
}  // namespace kvc
