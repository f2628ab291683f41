// Internal launch description shared by the host API and the HIP kernels of
// libhashgrid.  Not part of the public ABI (include/hashgrid.h is).
#pragma once

#include <hip/hip_fp16.h>
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

// Binned backward (binned_backward.hip): the table gradient routed to
// per-partition owners instead of global atomics.
// Points per bin tile of the D = 3, F = 2 grid (a 512-thread workgroup, two
// points per thread): a tile's run of one partition is ~32 records, so the
// accumulate kernel reads runs of ~3 lines instead of ~1.5 (measured on the
// binary16 T = 2^21 grid: 2.46 -> 2.31 ms; neutral at 2^18 points; 2048-point
// tiles were slower everywhere).
constexpr int kBinTile = 1024;
constexpr int kRecordBytes = 12;  // one binned corner-pair record
constexpr int kMaxParts = 4096;   // partitions per level
constexpr int kMaxSLog2 = 13;     // largest partition: 2^13 entries = 128 KB of 2 x int64 accumulators

struct BinParams {
    int32_t level0;          // first level of this launch group
    int32_t group;           // levels in this launch group
    int32_t tiles;           // ceil(n / tile_pts)
    int32_t parts;           // partitions per level = T >> s_log2
    int32_t s_log2;          // log2 entries per partition
    int32_t log2_table_size;
    uint32_t mask;           // T - 1
    int32_t tile_pts;        // points per bin tile
    int64_t n;
    int64_t level_records;   // record slots per level = tiles * rec_per_tile
    int32_t rec_per_tile;    // record slots of one tile (points x corner pairs)
    int32_t rec_bytes;       // bytes of one record
    int32_t grad_f16;        // the gradient holds binary16 values (else fp32)
    int32_t res[kMaxLevels];
};

// Binned backward of the other shapes (generic_binned.hip): records of
// 2 + F words (corner code, f_x, F upstream products), 2048 of them per tile
// (1024 for F = 8: 32, 48 or 40 KB), tiles of at most 1024 points, and
// partitions of S entries with S * F * 8 = 64 KB of fixed-point
// accumulators.  With many partitions (S = 8192 / F entries) a tile's runs
// are short, so F = 4 and 8 take larger tiles than 32 KB would allow: each
// accumulate workgroup then walks half as many tiles.
constexpr int generic_max_recs(int F) { return F <= 4 ? 2048 : 1024; }
constexpr int generic_tile(int D, int F) {
    return (generic_max_recs(F) >> (D - 1)) > 1024 ? 1024 : (generic_max_recs(F) >> (D - 1));
}
constexpr int generic_rec_per_tile(int D, int F) { return generic_tile(D, F) << (D - 1); }
constexpr int generic_rec_bytes(int F) { return (2 + F) * 4; }
constexpr int generic_s_log2(int F) { return F == 1 ? 13 : F == 2 ? 12 : F == 4 ? 11 : 10; }

// The allocation-free backward's device scratch (noalloc.hip): one fixed
// array per device; noalloc_scratch resolves the current device's address
// (once per device) and returns it.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void **out);

// Workspace bytes of one level (records, run starts, tile maxima).
inline size_t binned_level_bytes(const BinParams &bp) {
    const size_t recs = (size_t)bp.level_records * bp.rec_bytes;
    const size_t words = (size_t)bp.tiles * (bp.parts + 2);
    return recs + words * sizeof(uint32_t);
}
hipError_t launch_binned_backward_generic(BinParams bp, int D, int F, int n_levels, int max_group, const float *x,
                                          int64_t n, const float *dout, int64_t dout_stride, float *dtable,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream);
// Levels are binned and accumulated in equal groups of at most max_group
// levels (and no more than the workspace holds).
hipError_t launch_binned_backward(BinParams bp, int n_levels, int max_group, const float *x, int64_t n,
                                  const float *dout, int64_t dout_stride, float *dtable,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

// Forward launch shape: lanes per (point, level), points per lane pair in
// flight, non-temporal x reads / output writes.
struct FwdTune {
    int lanes;
    int unroll;
    int nt;
    int split_kib;  // staged gather: levels whose table exceeds this many KiB go one half per pass (0: never)
};

// Kernel launchers (encode_kernels.hip).  They return the launch status.
// stage == NULL: write rows directly; otherwise stage is an fp32 [L][n][2]
// scratch array and the rows are assembled by a transpose pass.
// stage2 (NULL, or a second [L][n][2] stage): where the gather takes a level
// one table half per pass (FwdTune::split_kib), the second half writes its
// partial blends there and the transpose adds them; without it the second
// half adds the first half's in place.
// perm (NULL, or with a stage): x is in a sorted order and perm[i] is the
// original index of point i; the transpose writes row i to out row perm[i].
hipError_t launch_forward(const LaunchParams &lp, const float *x, int64_t n, const void *table,
                          int table_dtype, float *out, int64_t out_stride, const FwdTune &ft,
                          float *stage, hipStream_t stream, float *stage2 = nullptr,
                          const uint32_t *perm = nullptr);
hipError_t launch_backward(const LaunchParams &lp, const float *x, int64_t n, const float *dout,
                           int64_t dout_stride, float *dtable, int lanes, hipStream_t stream);
// Shapes other than D = 3, F = 2 (generic_kernels.hip): D in 1..4,
// F in {1, 2, 4, 8}; hipErrorInvalidValue for an unbuilt shape.
hipError_t launch_forward_generic(const LaunchParams &lp, int D, int F, const float *x, int64_t n,
                                  const void *table, int table_dtype, float *out, int64_t out_stride, int lanes,
                                  float *stage, hipStream_t stream);
// [L][n][F] level-major stage -> rows out[p * ostride + l * F + j].
// Point order of the staged D = 3, F = 2 forward (point_order.hip): the
// points sorted by a coarse cell into xs [n][3], and perm[i] the original
// index of sorted point i.  The points are counted in at most
// kOrderMaxGroups groups of at least kOrderGroup points.  The workspace holds
// xs, perm and the count tables: order_workspace_bytes(n) bytes, 256-byte
// aligned.  n < 2^31.
constexpr int kOrderGroup = 1024;
constexpr int kOrderMaxGroups = 256;
size_t order_workspace_bytes(int64_t n);
hipError_t launch_point_order(const float *x, int64_t n, void *workspace, float **xs_out, uint32_t **perm_out,
                              hipStream_t stream);

hipError_t launch_transpose(int F, const float *stage, int64_t n, int L, float *out, int64_t ostride,
                            hipStream_t stream);
hipError_t launch_backward_generic(const LaunchParams &lp, int D, int F, const float *x, int64_t n,
                                   const float *dout, int64_t dout_stride, float *dtable, hipStream_t stream);

// Levels of the atomic backward that are accumulated in LDS first
// (generic_kernels.hip, bwd_dense_kernel): a level whose table holds at most
// kDenseVals values (T F), indexed by table entry, or whose vertex grid
// (N_l + 1)^D F does, indexed by vertex and hashed at the flush.
constexpr int kDenseVals = 16384;  // 128 KB of 64-bit accumulators
struct DenseLevels {
    int32_t count;
    int32_t max_vals;              // largest accumulator (or, forward, entry) count among them
    int8_t level[kMaxLevels];
    int8_t by_vertex[kMaxLevels];
};
// Forward of the D = 3, F = 2 grid (encode_kernels.hip, fwd_dense_kernel):
// the coarsest levels whose vertex grids (N_l + 1)^3, or tables, fit
// kFwdDenseBytes of LDS together as stored entries (max_vals: their entries
// in all) are blended from LDS into a level-major stage ([L][n][2], fp32 or,
// half_stage, binary16); the gather then takes the other levels
// (launch_forward, launch_encode_stage_f16 with those levels).
constexpr int kFwdDenseBytes = 128 << 10;
hipError_t launch_forward_dense(const LaunchParams &lp, const DenseLevels &dl, const float *x, int64_t n,
                                const void *table, int table_dtype, void *stage, bool half_stage,
                                hipStream_t stream);
hipError_t launch_backward_dense(const LaunchParams &lp, const DenseLevels &dl, int D, int F, const float *x,
                                 int64_t n, const float *dout, int64_t dout_stride, float *dtable,
                                 hipStream_t stream);
hipError_t launch_debug_corners_generic(const LaunchParams &lp, int D, const float *x, int64_t n, uint32_t *idx,
                                        float *w, hipStream_t stream);
// dL/dx of every shape; stage ([L][n][D] fp32) selects the level-major path,
// dlm ([L][n][2] fp32, D = 3 and F = 2 only, or NULL) a level-major copy of
// the upstream rows for it.
hipError_t launch_input_grad(const LaunchParams &lp, int D, int F, const float *x, int64_t n, const void *table,
                             int table_dtype, const float *dout, int64_t dout_stride, float *dx, float *stage,
                             float *dlm, hipStream_t stream);

// MLP head 32 -> 64 -> 64 -> 4 (mlp_kernels.hip).  Weights binary16 [out][in],
// biases and gradients fp32.
// Raw coordinates the TinyNeRF head puts before the encoding (u = [x, e]).
constexpr int kMlpCoords = 3;
struct MlpParams {
    const _Float16 *w1, *w2, *w3;
    const float *b1, *b2, *b3;
    int coords;  // 0 or kMlpCoords: W1 is [64][32 + coords]
};
struct MlpGrads {
    float *dw1, *db1, *dw2, *db2, *dw3, *db3;
};
// Encoding of the standard grid as a binary16 level-major stage [L][n][2].
hipError_t launch_encode_stage_f16(const LaunchParams &lp, const float *x, int64_t n, const void *table,
                                   int table_dtype, _Float16 *stage, hipStream_t stream);
size_t mlp_partials_bytes(int64_t n);
hipError_t launch_mlp_forward(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, float *y,
                              hipStream_t stream);
hipError_t launch_mlp_backward(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, const float *dy,
                               float *de, float *partials, const MlpGrads &g, hipStream_t stream);

struct AdamParams {
    float lr, beta1, beta2, eps;
    int32_t step;
};
hipError_t launch_adam(const AdamParams &a, int64_t count, float *param, float *m, float *v, float *grad,
                       void *param_f16, bool zero_grad, hipStream_t stream);

hipError_t launch_debug_corners(const LaunchParams &lp, const float *x, int64_t n, uint32_t *idx,
                                float *w, hipStream_t stream);

}  // namespace hg
