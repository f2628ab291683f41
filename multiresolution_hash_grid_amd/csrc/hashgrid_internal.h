// Internal launch description shared by the host API and the HIP kernels of
// libhashgrid.  Not part of the public ABI (include/hashgrid.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hg {

constexpr int kMaxLevels = 64;
constexpr int kNumXcd = 8;       // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kBlock = 256;      // threads per workgroup of the encode kernels

// Multipliers of the spatial hash for y and z (x uses 1): ipipp.com
// HashGridEncoder.hash and the ijyty.com section 2.2 formula.
constexpr uint32_t kPrimeY = 2654435761u;
constexpr uint32_t kPrimeZ = 805459861u;

// Work decomposition: the launch covers `items` = L * chunks work items, item
// (pos, chunk) being the points [chunk * chunk_pts, (chunk+1) * chunk_pts) at
// level level_order[pos].  With xcd_map set, workgroup g runs on XCD g % 8
// (the dispatcher deals workgroups round-robin over the XCDs) and is given
// item (g % 8) * per_xcd + g / 8, so each XCD sweeps a contiguous run of
// items -- one or two whole levels for L = 16 -- and keeps that level's table
// hot in its own L2 instead of every XCD streaming all levels.
struct LaunchParams {
    int32_t n_levels;
    int32_t log2_table_size;
    uint32_t mask;          // T - 1
    int32_t chunk_pts;      // points per work item (power of two)
    int32_t chunks;         // work items per level
    int32_t items;          // n_levels * chunks
    int32_t per_xcd;        // ceil(items / 8)
    int32_t xcd_map;        // 0 or 1
    int32_t res[kMaxLevels];
    int8_t level_order[kMaxLevels];
};

// Kernel launchers (encode_kernels.hip).  They return the launch status.
hipError_t launch_forward(const LaunchParams &lp, const float *x, int64_t n, const void *table,
                          int table_dtype, float *out, int64_t out_stride, int lanes,
                          hipStream_t stream);
hipError_t launch_backward(const LaunchParams &lp, const float *x, int64_t n, const float *dout,
                           int64_t dout_stride, float *dtable, int lanes, hipStream_t stream);
hipError_t launch_debug_corners(const LaunchParams &lp, const float *x, int64_t n, uint32_t *idx,
                                float *w, hipStream_t stream);

}  // namespace hg
