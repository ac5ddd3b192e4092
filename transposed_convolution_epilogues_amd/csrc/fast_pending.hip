// fast_pending.hip - fast-path entry points not yet specialised: each reports
// "not supported" so the API takes the generic kernels.
#include "c3d_internal.h"

namespace c3d {
bool conv3x3x3_mfma_supported(const Geom&, const void*, const void*, const void*) { return false; }
hipError_t launch_conv3x3x3_mfma(const float*, const float*, const float*, float*, const Geom&, hipStream_t) {
    return hipErrorNotSupported;
}
bool convT_s2_sublattice_supported(const Geom&, const void*, const void*, const void*) { return false; }
hipError_t launch_convT_s2_sublattice(const float*, const float*, const float*, float*, const Geom&, hipStream_t) {
    return hipErrorNotSupported;
}
bool conv_k1last_supported(const Geom&, const void*, const void*, const void*) { return false; }
hipError_t launch_conv_k1last(const float*, const float*, const float*, float*, const Geom&, hipStream_t) {
    return hipErrorNotSupported;
}
bool convT_bn_pool_fast_supported(const PoolGeom&, const void*) { return false; }
hipError_t launch_convT_bn_pool_phase1_fast(const float*, const float*, float*, double*, const PoolGeom&,
                                            hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace c3d
