// Decode kernels for bf16 caches (one translation unit per element type so
// the instances compile in parallel).
#include "pa_decode_impl.h"

namespace pa {

hipError_t launch_decode_bf16(const DecodeArgs& a) { return launch_decode_type<BF16>(a); }

}  // namespace pa
