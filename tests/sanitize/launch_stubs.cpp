// Stand-ins for the kernel launchers, so that the validation layer links
// without device code.  Reaching one means a call passed validation, which
// none of the sanitizer checks does: they report an error instead.
#include "wkv_internal.h"

namespace finch {
hipError_t launch_serial(const Geometry &, const Tensors &, bool, Variant, hipStream_t, KernelTiming) {
    return hipErrorInvalidValue;
}
hipError_t launch_decode(const Geometry &, const Tensors &, bool, Variant, int, hipStream_t, KernelTiming) {
    return hipErrorInvalidValue;
}
hipError_t launch_chunked(const Geometry &, const Tensors &, const Workspace &, bool, Variant, hipStream_t,
                          KernelTiming) {
    return hipErrorInvalidValue;
}
hipError_t launch_layernorm_rows(const float *, const float *, const float *, float, void *, bool, int64_t, int,
                                 hipStream_t, KernelTiming) {
    return hipErrorInvalidValue;
}
hipError_t launch_gold_compress(const uint16_t *, const uint16_t *, void *, bool, int64_t, int, int, hipStream_t,
                                KernelTiming) {
    return hipErrorInvalidValue;
}
hipError_t launch_plan_varlen(const Geometry &, int32_t *, int32_t *, int32_t *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t split_launch_capacity(const Variant &, bool, int64_t *) { return hipErrorInvalidValue; }
}  // namespace finch
