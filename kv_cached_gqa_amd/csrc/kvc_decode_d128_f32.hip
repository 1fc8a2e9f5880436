// Split-K decode kernels for head dimension 128, f32 storage.
#include "kvc_decode_impl.h"

namespace kvc {
template hipError_t decode_run<128, F32>(DecodeArgs& a, hipStream_t s);
template int decode_batch_keys<128, F32>(int rows);
}  // namespace kvc
