// Split-K decode kernels for head dimension 64, f32 storage.
#include "kvc_decode_impl.h"

namespace kvc {
template hipError_t decode_run<64, F32>(DecodeArgs& a, hipStream_t s);
template int decode_batch_keys<64, F32>(int rows);
}  // namespace kvc
