// Decode kernels for f32 caches (one translation unit per element type so
// the instances compile in parallel).
#include "pa_decode_impl.h"

namespace pa {

hipError_t launch_decode_f32(const DecodeArgs& a) { return launch_decode_type<F32>(a); }

}  // namespace pa
