// Decode launch dispatch by element type.  The kernels live in
// pa_decode_impl.h and are instantiated by pa_decode_{f32,f16,bf16}.hip.
#include "pa_internal.h"

namespace pa {

hipError_t launch_decode(const DecodeArgs& a) {
    switch (a.dtype) {
        case 0: return launch_decode_f32(a);
        case 1: return launch_decode_f16(a);
        case 2: return launch_decode_bf16(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
