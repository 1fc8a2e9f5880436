// Split-K decode kernels for head dimension 32, f32 storage.
#include "kvc_decode_impl.h"

namespace kvc {
template hipError_t decode_run<32, F32>(DecodeArgs& a, hipStream_t s);
template int decode_batch_keys<32, F32>(int rows);
}  // namespace kvc
