// Stand-ins for the device-side launchers of libhashgrid, so that the host
// C ABI (csrc/api.cpp) can be built on its own with AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.  The driver only takes
// paths that are rejected, or answered, on the host; a stand-in that is
// reached anyway reports it and fails the run.
#include <cstdio>
#include <cstdlib>

#include "hashgrid_internal.h"

namespace {
hipError_t reached(const char *what) {
    std::fprintf(stderr, "sanitizer driver reached the launcher %s\n", what);
    std::abort();
}
}  // namespace

namespace hg {
hipError_t launch_binned_backward_generic(BinParams, int, int, int, int, const float *, int64_t, const float *, int64_t,
                                          float *, void *, size_t, hipStream_t) {
    return reached("binned backward (generic)");
}
hipError_t launch_binned_backward(BinParams, int, int, const float *, int64_t, const float *, int64_t, float *, void *,
                                  size_t, hipStream_t) {
    return reached("binned backward");
}
hipError_t launch_forward(const LaunchParams &, const float *, int64_t, const void *, int, float *, int64_t,
                          const FwdTune &, float *, hipStream_t, float *, const uint32_t *) {
    return reached("forward");
}
size_t order_workspace_bytes(int64_t n) { return (size_t)n * 16 + (1 << 16); }
hipError_t launch_point_order(const float *, int64_t, void *, float **, uint32_t **, hipStream_t) {
    return reached("point order");
}
hipError_t launch_forward_dense(const LaunchParams &, const DenseLevels &, const float *, int64_t, const void *,
                                int, void *, bool, hipStream_t) {
    return reached("forward_dense");
}
hipError_t launch_backward(const LaunchParams &, const float *, int64_t, const float *, int64_t, float *, int,
                           hipStream_t) {
    return reached("backward");
}
hipError_t launch_forward_generic(const LaunchParams &, int, int, const float *, int64_t, const void *, int, float *,
                                  int64_t, int, float *, hipStream_t) {
    return reached("forward (generic)");
}
hipError_t launch_transpose(int, const float *, int64_t, int, float *, int64_t, hipStream_t) {
    return reached("transpose");
}
hipError_t launch_backward_generic(const LaunchParams &, int, int, const float *, int64_t, const float *, int64_t,
                                   float *, hipStream_t) {
    return reached("backward (generic)");
}
hipError_t launch_backward_dense(const LaunchParams &, const DenseLevels &, int, int, const float *, int64_t,
                                 const float *, int64_t, float *, hipStream_t) {
    return reached("backward (dense levels)");
}
hipError_t launch_debug_corners_generic(const LaunchParams &, int, const float *, int64_t, uint32_t *, float *,
                                        hipStream_t) {
    return reached("debug corners (generic)");
}
hipError_t launch_input_grad(const LaunchParams &, int, int, const float *, int64_t, const void *, int, const float *,
                             int64_t, float *, float *, float *, hipStream_t) {
    return reached("input grad");
}
hipError_t launch_encode_stage_f16(const LaunchParams &, const float *, int64_t, const void *, int, _Float16 *,
                                   hipStream_t) {
    return reached("encode stage");
}
// Host-side size of the MLP backward's partials (the kernels' file holds the
// real one); only workspace-size queries reach it here.
size_t mlp_partials_bytes(int64_t n) { return (size_t)(n + 15) / 16 * 4 + 4096; }
hipError_t launch_mlp_forward(const _Float16 *, const float *, int64_t, const MlpParams &, float *, hipStream_t) {
    return reached("mlp forward");
}
hipError_t launch_mlp_backward(const _Float16 *, const float *, int64_t, const MlpParams &, const float *, float *,
                               float *, const MlpGrads &, hipStream_t) {
    return reached("mlp backward");
}
hipError_t launch_adam(const AdamParams &, int64_t, float *, float *, float *, float *, void *, bool, hipStream_t) {
    return reached("adam");
}
hipError_t launch_debug_corners(const LaunchParams &, const float *, int64_t, uint32_t *, float *, hipStream_t) {
    return reached("debug corners");
}
hipError_t noalloc_scratch(void **) { return reached("no-alloc scratch"); }
}  // namespace hg
