// Point order for the staged forward of the D = 3, F = 2 grid.
//
// The gather of one level makes a line request per corner pair
// (jsqmd.com HashEncoding section 3: the corners are hashed into the level's
// table), and neighbouring lanes share those lines only when their points
// share voxels.  Uniform batches put unrelated points side by side, so at the
// coarse and middle levels every lane fetches its own lines.  Ordering the
// points by a coarse cell first (4 bits per axis, 4096 cells in Morton order)
// gives each wave points of one or two cells, whose corners at those levels
// are few.  The forward then encodes the ordered points and writes every row
// back to its point's position: each row is computed from its own point
// alone, so the output is the same, bit for bit.
//
// A counting sort in three launches, with no memsets (it can be captured in
// a HIP graph):
//   order_count_kernel    one workgroup per group of points (at most
//                         kOrderMaxGroups groups of at least kOrderGroup
//                         points): the group's cell histogram in LDS,
//                         written whole to counts[g][cell];
//   order_prefix_kernel   one thread per cell: counts[g][c] becomes the number
//                         of points of cell c in the groups before g, and
//                         totals[c] the cell's points;
//   order_scatter_kernel  one workgroup per group: the cells' first positions
//                         (an exclusive scan of the totals, in LDS) plus its
//                         groups' offsets, then each point takes the next slot
//                         of its cell with an LDS atomic and writes its
//                         coordinates and index there.
// Within a cell and group the order of the points is not defined (the LDS
// atomics); the order of the cells and groups is.
#include <algorithm>

#include "hashgrid_internal.h"

namespace hg {
namespace {

constexpr int kOrderBits = 4;                           // per axis
constexpr int kOrderCells = 1 << (3 * kOrderBits);      // 4096
constexpr int kOrderThreads = 1024;                     // count and scatter workgroups
constexpr int kOrderUnroll = 4;                         // points per thread in flight
constexpr int kPrefixThreads = 256;

// The cell coordinate of one axis: floor(16 x) clamped to [0, 15]; a NaN
// coordinate goes to cell 0.
__device__ __forceinline__ uint32_t order_axis(float v) {
    const float s = v * (float)(1 << kOrderBits);
    if (!(s >= 0.f)) return 0u;
    return s >= (float)((1 << kOrderBits) - 1) ? (uint32_t)((1 << kOrderBits) - 1) : (uint32_t)s;
}

// Bits 0..3 of q moved to bits 0, 3, 6, 9.
__device__ __forceinline__ uint32_t order_spread(uint32_t q) {
    q = (q | (q << 4)) & 0x0C3u;
    return (q | (q << 2)) & 0x249u;
}

struct Point3 {
    float v[3];
};

__device__ __forceinline__ uint32_t order_key(const Point3 &q) {
    return (order_spread(order_axis(q.v[0])) << 2) | (order_spread(order_axis(q.v[1])) << 1) |
           order_spread(order_axis(q.v[2]));
}

// Group g: points [g gs, min(n, (g + 1) gs)).
__global__ __launch_bounds__(kOrderThreads) void order_count_kernel(const Point3 *__restrict__ x, int64_t n,
                                                                     int64_t gs, uint32_t *__restrict__ counts) {
    __shared__ uint32_t hist[kOrderCells];
    for (int c = threadIdx.x; c < kOrderCells; c += kOrderThreads) hist[c] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * gs;
    const int64_t p1 = min(n, p0 + gs);
    for (int64_t b = p0; b < p1; b += kOrderUnroll * kOrderThreads) {
        Point3 q[kOrderUnroll];
#pragma unroll
        for (int u = 0; u < kOrderUnroll; ++u) {
            const int64_t p = b + u * kOrderThreads + threadIdx.x;
            if (p < p1) q[u] = x[p];
        }
#pragma unroll
        for (int u = 0; u < kOrderUnroll; ++u)
            if (b + u * kOrderThreads + threadIdx.x < p1) atomicAdd(&hist[order_key(q[u])], 1u);
    }
    __syncthreads();
    uint32_t *row = counts + (int64_t)blockIdx.x * kOrderCells;
    for (int c = threadIdx.x; c < kOrderCells; c += kOrderThreads) row[c] = hist[c];
}

// Four threads per cell, each taking one segment of up to kPrefixSeg groups:
// a segment's counts are loaded at once, summed, the segment sums combined
// through LDS, and the counts replaced by their exclusive prefix over the
// groups (a cell's groups in order).
constexpr int kPrefixSeg = 64;
constexpr int kPrefixCells = kPrefixThreads / (kOrderMaxGroups / kPrefixSeg);  // cells per workgroup
__global__ __launch_bounds__(kPrefixThreads) void order_prefix_kernel(uint32_t *__restrict__ counts, int groups,
                                                                       uint32_t *__restrict__ totals) {
    constexpr int kSegs = kOrderMaxGroups / kPrefixSeg;
    __shared__ uint32_t segsum[kSegs][kPrefixCells];
    const int cl = threadIdx.x % kPrefixCells, seg = threadIdx.x / kPrefixCells;
    const int c = blockIdx.x * kPrefixCells + cl;  // the grid covers the cells exactly
    const int g0 = seg * kPrefixSeg;
    uint32_t v[kPrefixSeg], sum = 0;
#pragma unroll
    for (int i = 0; i < kPrefixSeg; ++i) {
        v[i] = g0 + i < groups ? counts[(int64_t)(g0 + i) * kOrderCells + c] : 0u;
        sum += v[i];
    }
    segsum[seg][cl] = sum;
    __syncthreads();
    uint32_t run = 0, total = 0;
#pragma unroll
    for (int t = 0; t < kSegs; ++t) {
        run += t < seg ? segsum[t][cl] : 0u;
        total += segsum[t][cl];
    }
#pragma unroll
    for (int i = 0; i < kPrefixSeg; ++i) {
        if (g0 + i < groups) counts[(int64_t)(g0 + i) * kOrderCells + c] = run;
        run += v[i];
    }
    if (seg == 0) totals[c] = total;
}

__global__ __launch_bounds__(kOrderThreads) void order_scatter_kernel(const Point3 *__restrict__ x, int64_t n,
                                                                       int64_t gs,
                                                                       const uint32_t *__restrict__ counts,
                                                                       const uint32_t *__restrict__ totals,
                                                                       Point3 *__restrict__ xs,
                                                                       uint32_t *__restrict__ perm) {
    constexpr int kPer = kOrderCells / kOrderThreads;  // cells per thread in the scan
    __shared__ uint32_t next[kOrderCells];
    __shared__ uint32_t wsum[kOrderThreads / 64];
    // Exclusive scan of the cell totals: thread t sums its kPer cells, the
    // waves scan their threads, the wave sums are added in order.
    const int c0 = threadIdx.x * kPer;
    uint32_t own[kPer], s = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        own[i] = totals[c0 + i];
        s += own[i];
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t run = incl - s;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    const uint32_t *row = counts + (int64_t)blockIdx.x * kOrderCells;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        next[c0 + i] = run + row[c0 + i];
        run += own[i];
    }
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * gs;
    const int64_t p1 = min(n, p0 + gs);
    for (int64_t b = p0; b < p1; b += kOrderUnroll * kOrderThreads) {
        Point3 q[kOrderUnroll];
#pragma unroll
        for (int u = 0; u < kOrderUnroll; ++u) {
            const int64_t p = b + u * kOrderThreads + threadIdx.x;
            if (p < p1) q[u] = x[p];
        }
#pragma unroll
        for (int u = 0; u < kOrderUnroll; ++u) {
            const int64_t p = b + u * kOrderThreads + threadIdx.x;
            if (p < p1) {
                const uint32_t pos = atomicAdd(&next[order_key(q[u])], 1u);
                xs[pos] = q[u];
                perm[pos] = (uint32_t)p;
            }
        }
    }
}

// Groups of at least kOrderGroup points, at most kOrderMaxGroups of them.
int64_t order_groups(int64_t n) { return std::min<int64_t>(kOrderMaxGroups, (n + kOrderGroup - 1) / kOrderGroup); }
int64_t order_group_size(int64_t n, int64_t groups) { return (n + groups - 1) / groups; }

}  // namespace

size_t order_workspace_bytes(int64_t n) {
    const int64_t groups = order_groups(n);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    return up((size_t)n * 3 * sizeof(float)) + up((size_t)n * sizeof(uint32_t)) +
           up((size_t)groups * kOrderCells * sizeof(uint32_t)) + up((size_t)kOrderCells * sizeof(uint32_t));
}

hipError_t launch_point_order(const float *x, int64_t n, void *workspace, float **xs_out, uint32_t **perm_out,
                              hipStream_t stream) {
    const int64_t groups = order_groups(n), gs = order_group_size(n, groups);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    char *p = reinterpret_cast<char *>(workspace);
    Point3 *xs = reinterpret_cast<Point3 *>(p);
    p += up((size_t)n * 3 * sizeof(float));
    uint32_t *perm = reinterpret_cast<uint32_t *>(p);
    p += up((size_t)n * sizeof(uint32_t));
    uint32_t *counts = reinterpret_cast<uint32_t *>(p);
    p += up((size_t)groups * kOrderCells * sizeof(uint32_t));
    uint32_t *totals = reinterpret_cast<uint32_t *>(p);
    const Point3 *xp = reinterpret_cast<const Point3 *>(x);
    order_count_kernel<<<(unsigned)groups, kOrderThreads, 0, stream>>>(xp, n, gs, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    order_prefix_kernel<<<kOrderCells / kPrefixCells, kPrefixThreads, 0, stream>>>(counts, (int)groups, totals);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    order_scatter_kernel<<<(unsigned)groups, kOrderThreads, 0, stream>>>(xp, n, gs, counts, totals, xs, perm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    *xs_out = reinterpret_cast<float *>(xs);
    *perm_out = perm;
    return hipSuccess;
}

}  // namespace hg
