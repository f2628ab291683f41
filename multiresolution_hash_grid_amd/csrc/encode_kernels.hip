// HIP kernels of the hash-grid encoder for gfx950 (CDNA4, wave64).
//
// Method: ipipp.com "Speeding up NeRFace with Instant-NGP hash encoding",
// section 2 and its HashGridEncoder listing; hash formula of the ijyty.com
// Instant-NGP overview, section 2.2.  Per (point, level):
//   pos_d = x_d * N_l (one fp32 multiply, round to nearest), v_d = floor(pos_d),
//   f_d = pos_d - v_d (exact), corner c = v + (dx, dy, dz),
//   h(c) = (c_x ^ c_y * 2654435761 ^ c_z * 805459861) mod 2^log2T in uint32,
//   out[l*F + j] = sum over the 8 corners of w_c * table[l][h(c)][j],
//   w_c = prod_d (d-th offset ? f_d : 1 - f_d).
// The backward here (used without a workspace; binned_backward.hip holds the
// default one) scatters dL/dout * w_c back into every table entry a corner
// hashed to (the adjoint of the gather) with fp32 atomic adds, after a wave
// has summed runs of consecutive points that share a voxel.
//
// Memory behaviour on MI355X.  The corner gathers are the traffic: 8 random
// F-vectors per point and level.  Because the x prime is 1, the corners
// (v_x, y, z) and (v_x + 1, y, z) differ only in the low bits of their index
// (they are 2^(t+1) - 1 apart at most, t = trailing ones of v_x), so they share
// a 128-byte line 15 times out of 16.  The "lane pair" layout below gives the
// two x-corners of one point to two adjacent lanes of the same load or atomic
// instruction, so the memory pipeline sees about 4 distinct lines per
// (point, level) instead of 8.
#include <algorithm>

#include "device_common.h"

namespace hg {
namespace {

// ---------------------------------------------------------------- helpers

// Table element pairs (F = 2).  fp16 entries are widened exactly (subnormals
// included) and all arithmetic is fp32.
template <int DT>
struct Table2;

// Raw is an entry as stored (both features), widen() its fp32 values.
template <>
struct Table2<0> {
    using Raw = float2;
    static __device__ __forceinline__ Raw raw(const void *base, uint64_t e) {
        return reinterpret_cast<const float2 *>(base)[e];
    }
    static __device__ __forceinline__ float2 widen(Raw r) { return r; }
    static __device__ __forceinline__ float2 load(const void *base, uint64_t e) { return raw(base, e); }
};

template <>
struct Table2<1> {
    using Raw = uint32_t;
    static __device__ __forceinline__ Raw raw(const void *base, uint64_t e) {
        return reinterpret_cast<const uint32_t *>(base)[e];
    }
    static __device__ __forceinline__ float2 widen(Raw r) {
        _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
        _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(r >> 16));
        return make_float2((float)lo, (float)hi);
    }
    static __device__ __forceinline__ float2 load(const void *base, uint64_t e) { return widen(raw(base, e)); }
};

// One x-half of a point's blend at a level: the four corners with x offset
// sub, e[c] = corner (v_x + sub, v_y + dy, v_z + dz), c = 2 dy + dz, both
// features.  The point's features are the sum of its two halves.  Explicit
// fused multiply-adds: the rounding does not depend on how the compiler
// contracts, so every kernel that blends through here gives the same bits.
__device__ __forceinline__ float2 half_blend(float a0, float a1, float a2, uint32_t sub, const float2 (&e)[4]) {
    const float wy0 = 1.f - a1, wz0 = 1.f - a2;
    const float wx = sub ? a0 : 1.f - a0;
    return make_float2(wx * fmaf(a1, fmaf(a2, e[3].x, wz0 * e[2].x), wy0 * fmaf(a2, e[1].x, wz0 * e[0].x)),
                       wx * fmaf(a1, fmaf(a2, e[3].y, wz0 * e[2].y), wy0 * fmaf(a2, e[1].y, wz0 * e[0].y)));
}

__device__ __forceinline__ void fadd(float *p, float v) { unsafeAtomicAdd(p, v); }

// ---------------------------------------------------------------- forward

// One lane per (point, level) takes all eight corners (the lane-pair kernel
// below is the default; this one is the HG_TUNE_FWD_LANES = 1 launch shape).
template <int DT>
__global__ __launch_bounds__(kBlock) void fwd_f2_kernel(const float *__restrict__ x, int64_t n,
                                                        const void *__restrict__ table,
                                                        float *__restrict__ out, int64_t ostride,
                                                        LaunchParams lp) {
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint32_t mask = lp.mask;
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p = it.p0 + threadIdx.x; p < end; p += kBlock) {
        int32_t v0, v1, v2;
        float a0, a1, a2;
        locate1(x[3 * p + 0], N, v0, a0);
        locate1(x[3 * p + 1], N, v1, a1);
        locate1(x[3 * p + 2], N, v2, a2);
        const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hy1 = hy0 + kPrimeY;
        const uint32_t hz0 = (uint32_t)v2 * kPrimeZ, hz1 = hz0 + kPrimeZ;
        const float wy0 = 1.f - a1, wz0 = 1.f - a2;
        float *orow = out + p * ostride + (int64_t)l * 2;
        const uint32_t c0 = (uint32_t)v0, c1 = c0 + 1u;
        float2 e[8];
        e[0] = Table2<DT>::load(table, lbase + ((c0 ^ hy0 ^ hz0) & mask));
        e[1] = Table2<DT>::load(table, lbase + ((c0 ^ hy0 ^ hz1) & mask));
        e[2] = Table2<DT>::load(table, lbase + ((c0 ^ hy1 ^ hz0) & mask));
        e[3] = Table2<DT>::load(table, lbase + ((c0 ^ hy1 ^ hz1) & mask));
        e[4] = Table2<DT>::load(table, lbase + ((c1 ^ hy0 ^ hz0) & mask));
        e[5] = Table2<DT>::load(table, lbase + ((c1 ^ hy0 ^ hz1) & mask));
        e[6] = Table2<DT>::load(table, lbase + ((c1 ^ hy1 ^ hz0) & mask));
        e[7] = Table2<DT>::load(table, lbase + ((c1 ^ hy1 ^ hz1) & mask));
        const float wx0 = 1.f - a0;
        float r[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float ej[8] = {j ? e[0].y : e[0].x, j ? e[1].y : e[1].x, j ? e[2].y : e[2].x,
                                 j ? e[3].y : e[3].x, j ? e[4].y : e[4].x, j ? e[5].y : e[5].x,
                                 j ? e[6].y : e[6].x, j ? e[7].y : e[7].x};
            const float lo = wy0 * (wz0 * ej[0] + a2 * ej[1]) + a1 * (wz0 * ej[2] + a2 * ej[3]);
            const float hi = wy0 * (wz0 * ej[4] + a2 * ej[5]) + a1 * (wz0 * ej[6] + a2 * ej[7]);
            r[j] = wx0 * lo + a0 * hi;
        }
        orow[0] = r[0];
        orow[1] = r[1];
    }
}

// Lane-pair forward with U points per pair in flight: all 4*U corner loads
// of a lane are issued before the first blend, so each wave keeps U times as
// many table requests outstanding.  NT marks the streamed x reads and output
// writes non-temporal so that they do not displace the level's table from L2.
// Output element (p, l, j) is out[p * ostride + l * lstride + j]: lstride = 2
// writes the [n][L*F] rows directly, ostride = 2 with lstride = 2 n writes a
// level-major [L][n][F] staging array whose stores are fully coalesced.
// SPLIT: one half of every level's table, the entries whose index has top bit
// `half` (T = 2^s entries, so the bit is idx >> (s - 1)); the other half's
// corners count as zero.  Two launches give the blend while each XCD's L2
// holds only half of a level's table at a time: half 0 writes its partial
// blend, and half 1 either writes its own to a second stage, which the
// transpose adds (add_prev = 0), or adds the first half's (add_prev = 1, when
// the workspace holds one stage).
template <int DT, int U, bool NT, typename OutT = float, bool SPLIT = false>
__global__ __launch_bounds__(kBlock) void fwd_f2_pair_kernel(const float *__restrict__ x, int64_t n,
                                                             const void *__restrict__ table,
                                                             OutT *__restrict__ out, int64_t ostride,
                                                             int64_t lstride, LaunchParams lp, int half,
                                                             int add_prev = 0) {
    Item it;
    if (!decode_item(lp, it)) return;
    constexpr int kPairs = kBlock / 2;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint32_t mask = lp.mask;
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const uint32_t sub = threadIdx.x & 1;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p0 = it.p0 + (threadIdx.x >> 1); p0 < end; p0 += (int64_t)kPairs * U) {
        float2 e[U][4];
        float a0[U], a1[U], a2[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = p0 + (int64_t)u * kPairs;
            ok[u] = p < end;
            const int64_t q = ok[u] ? p : p0;  // p0 < end: always a valid point
            const float x0 = NT ? __builtin_nontemporal_load(x + 3 * q + 0) : x[3 * q + 0];
            const float x1 = NT ? __builtin_nontemporal_load(x + 3 * q + 1) : x[3 * q + 1];
            const float x2 = NT ? __builtin_nontemporal_load(x + 3 * q + 2) : x[3 * q + 2];
            int32_t v0, v1, v2;
            locate1(x0, N, v0, a0[u]);
            locate1(x1, N, v1, a1[u]);
            locate1(x2, N, v2, a2[u]);
            const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hy1 = hy0 + kPrimeY;
            const uint32_t hz0 = (uint32_t)v2 * kPrimeZ, hz1 = hz0 + kPrimeZ;
            const uint32_t cx = (uint32_t)v0 + sub;
            auto corner = [&](uint32_t idx) -> float2 {
                if constexpr (SPLIT) {
                    if ((idx >> (lp.log2_table_size - 1)) != (uint32_t)half) return make_float2(0.f, 0.f);
                }
                return Table2<DT>::load(table, lbase + idx);
            };
            e[u][0] = corner((cx ^ hy0 ^ hz0) & mask);
            e[u][1] = corner((cx ^ hy0 ^ hz1) & mask);
            e[u][2] = corner((cx ^ hy1 ^ hz0) & mask);
            e[u][3] = corner((cx ^ hy1 ^ hz1) & mask);
        }
        // All U points' gathers are issued before the first blend waits for
        // its loads (left to itself the scheduler interleaves them, which
        // keeps only one point's four loads in flight per lane).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float2 r = half_blend(a0[u], a1[u], a2[u], sub, e[u]);
            const float rx = r.x, ry = r.y;
            // lane 0 keeps feature 0 and needs lane 1's x-half; lane 1 the reverse.
            float v = (sub ? ry : rx) + swap_pair(sub ? rx : ry);
            if (ok[u]) {
                OutT *dst = out + (p0 + (int64_t)u * kPairs) * ostride + (int64_t)l * lstride + sub;
                if constexpr (SPLIT) {
                    // (requesting this load with the gathers measured slower: 2.11 against 2.04 ms)
                    if (add_prev) v += NT ? __builtin_nontemporal_load(dst) : *dst;
                }
                if constexpr (NT) __builtin_nontemporal_store((OutT)v, dst);
                else *dst = (OutT)v;  // binary16 stage: round to nearest even
            }
        }
    }
}

// Coarse levels whose whole vertex grid (N_l + 1)^3 -- or whole table, if
// smaller -- fit in LDS together (kFwdDenseBytes): each workgroup copies them
// from the table once, then blends its chunk of points at every one of these
// levels from LDS (a point is read once for all of them), so the corners cost
// LDS reads instead of the L2 line requests that bound the gather.  A row of
// x-vertices maps to one or two table lines (the x prime is 1), so a copy
// costs a few hundred requests against four per point and level.  One thread
// per point adds the two x-halves that a lane pair of the gather adds, through
// the same half_blend, so the two kernels agree bit for bit.  Corners outside
// the grid (points at x = 1, or outside [0, 1)) are read from the table.
// Output: out[p * ostride + l * lstride + j] (a level-major stage).
constexpr int kDenseFwdThreads = 1024;

template <int DT, class OutT>
__global__ __launch_bounds__(kDenseFwdThreads) void fwd_dense_kernel(const float *__restrict__ x, int64_t n,
                                                                     const void *__restrict__ table,
                                                                     OutT *__restrict__ out, int64_t ostride,
                                                                     int64_t lstride, LaunchParams lp,
                                                                     DenseLevels dl, int64_t chunk_pts) {
    // The gather adds a point's two halves across a lane pair; here both are
    // in one thread, and a contracted (fused) final add would round differently.
#pragma clang fp contract(off)
    using T2 = Table2<DT>;
    using Raw = typename T2::Raw;
    extern __shared__ __align__(16) unsigned char dense_lds[];
    Raw *grids = reinterpret_cast<Raw *>(dense_lds);
    const uint32_t mask = lp.mask;
    // The levels' copies, one after the other.
    int base = 0;
    for (int li = 0; li < dl.count; ++li) {
        const int l = dl.level[li];
        const int R = lp.res[l] + 1;  // vertices per axis
        const bool by_vertex = dl.by_vertex[li] != 0;
        const int V = by_vertex ? R * R * R : (int)(mask + 1u);
        const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
        // v = cx + R (cy + R cz); q / R as the high word of q * ceil(2^32 / R),
        // exact for q < 2^20 (integer division is a long instruction sequence).
        const uint32_t M = 0xFFFFFFFFu / (uint32_t)R + 1u;
        // kCopyBatch loads in flight per thread before their LDS stores.
        constexpr int kCopyBatch = 8;
        for (int v0 = threadIdx.x; v0 < V; v0 += kCopyBatch * kDenseFwdThreads) {
            Raw r[kCopyBatch];
#pragma unroll
            for (int k = 0; k < kCopyBatch; ++k) {
                const int v = min(v0 + k * kDenseFwdThreads, V - 1);
                uint32_t e = (uint32_t)v;
                if (by_vertex) {
                    const uint32_t q = __umulhi((uint32_t)v, M), cz = __umulhi(q, M);
                    const uint32_t cx = (uint32_t)v - q * (uint32_t)R, cy = q - cz * (uint32_t)R;
                    e = (cx ^ cy * kPrimeY ^ cz * kPrimeZ) & mask;
                }
                r[k] = T2::raw(table, lbase + e);
            }
#pragma unroll
            for (int k = 0; k < kCopyBatch; ++k)
                if (v0 + k * kDenseFwdThreads < V) grids[base + v0 + k * kDenseFwdThreads] = r[k];
        }
        base += V;
    }
    __syncthreads();
    const int64_t p_begin = (int64_t)blockIdx.x * chunk_pts, p_end = min(p_begin + chunk_pts, n);
    // kDenseUnroll points per thread and pass: their coordinates are loaded
    // together, so that the loads overlap.
    constexpr int kDenseUnroll = 4;
    for (int64_t pq = p_begin + threadIdx.x; pq < p_end; pq += kDenseUnroll * kDenseFwdThreads) {
        float xs[kDenseUnroll][3];
#pragma unroll
        for (int u = 0; u < kDenseUnroll; ++u) {
            const int64_t q = min(pq + (int64_t)u * kDenseFwdThreads, p_end - 1);
            xs[u][0] = x[3 * q + 0];
            xs[u][1] = x[3 * q + 1];
            xs[u][2] = x[3 * q + 2];
        }
#pragma unroll
        for (int u = 0; u < kDenseUnroll; ++u) {
        const int64_t p = pq + (int64_t)u * kDenseFwdThreads;
        if (p >= p_end) break;
        const float x0 = xs[u][0], x1 = xs[u][1], x2 = xs[u][2];
        int gbase = 0;
        for (int li = 0; li < dl.count; ++li) {
            const int l = dl.level[li];
            const int R = lp.res[l] + 1;
            const bool by_vertex = dl.by_vertex[li] != 0;
            const Raw *grid = grids + gbase;
            gbase += by_vertex ? R * R * R : (int)(mask + 1u);
            const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
            const float N = (float)lp.res[l];
            int32_t v0, v1, v2;
            float a0, a1, a2;
            locate1(x0, N, v0, a0);
            locate1(x1, N, v1, a1);
            locate1(x2, N, v2, a2);
            // the voxel's 8 corners are vertices of the grid
            const bool inside = (uint32_t)v0 < (uint32_t)(R - 1) && (uint32_t)v1 < (uint32_t)(R - 1) &&
                                (uint32_t)v2 < (uint32_t)(R - 1);
            const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hz0 = (uint32_t)v2 * kPrimeZ;
            float2 h[2];
#pragma unroll
            for (uint32_t sub = 0; sub < 2; ++sub) {
                float2 e[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
                    if (by_vertex && inside) {
                        e[c] = T2::widen(grid[(v0 + (int)sub) + R * ((v1 + (int)dy) + R * (v2 + (int)dz))]);
                    } else {
                        const uint32_t idx =
                            (((uint32_t)v0 + sub) ^ (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ)) & mask;
                        e[c] = by_vertex ? T2::load(table, lbase + idx) : T2::widen(grid[idx]);
                    }
                }
                h[sub] = half_blend(a0, a1, a2, sub, e);
            }
            OutT *dst = out + p * ostride + (int64_t)l * lstride;
            dst[0] = (OutT)(h[0].x + h[1].x);
            dst[1] = (OutT)(h[1].y + h[0].y);
        }
        }
    }
}

// ---------------------------------------------------------------- backward

// Other launch shapes of the atomic backward (the default is
// bwd_f2_quad_kernel, four lanes (dx, feature) per point with the wave
// pre-reduction):  LANES = 2: lane dx adds both features of its four
// corners.  LANES = 1: one lane adds all sixteen values.
template <int LANES>
__global__ __launch_bounds__(kBlock) void bwd_f2_kernel(const float *__restrict__ x, int64_t n,
                                                        const float *__restrict__ dout,
                                                        int64_t dstride, float *__restrict__ grad,
                                                        LaunchParams lp) {
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint32_t mask = lp.mask;
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    float *__restrict__ g = grad + 2 * lbase;
    const int sub = threadIdx.x % LANES;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p = it.p0 + threadIdx.x / LANES; p < end; p += kBlock / LANES) {
        int32_t v0, v1, v2;
        float a0, a1, a2;
        locate1(x[3 * p + 0], N, v0, a0);
        locate1(x[3 * p + 1], N, v1, a1);
        locate1(x[3 * p + 2], N, v2, a2);
        const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hy1 = hy0 + kPrimeY;
        const uint32_t hz0 = (uint32_t)v2 * kPrimeZ, hz1 = hz0 + kPrimeZ;
        const float wy0 = 1.f - a1, wz0 = 1.f - a2;
        const float w00 = wy0 * wz0, w01 = wy0 * a2, w10 = a1 * wz0, w11 = a1 * a2;
        const float *drow = dout + p * dstride + (int64_t)l * 2;
        const float d0 = drow[0], d1 = drow[1];
#pragma unroll
        for (int dx = 0; dx < 2; ++dx) {
            if (LANES == 2 && dx != sub) continue;
            const uint32_t cx = (uint32_t)v0 + (uint32_t)dx;
            const float wx = dx ? a0 : 1.f - a0;
            const float g0 = d0 * wx, g1 = d1 * wx;
            const uint32_t i00 = (cx ^ hy0 ^ hz0) & mask, i01 = (cx ^ hy0 ^ hz1) & mask;
            const uint32_t i10 = (cx ^ hy1 ^ hz0) & mask, i11 = (cx ^ hy1 ^ hz1) & mask;
            fadd(g + 2 * i00, g0 * w00);
            fadd(g + 2 * i00 + 1, g1 * w00);
            fadd(g + 2 * i01, g0 * w01);
            fadd(g + 2 * i01 + 1, g1 * w01);
            fadd(g + 2 * i10, g0 * w10);
            fadd(g + 2 * i10 + 1, g1 * w10);
            fadd(g + 2 * i11, g0 * w11);
            fadd(g + 2 * i11 + 1, g1 * w11);
        }
    }
}

// Four lanes (dx, j) per point, 16 consecutive points per wave, with the
// wave pre-reduction of duplicate coarse-level corners: a run of consecutive
// points in one voxel (ray samples at coarse levels) shares all 8 corners.
// Each lane parks its 4 contributions (feature j of the corners (dx, dy, dz))
// in LDS; the lanes of the run's first point add the run's sums, in point
// order, and the other points of the run add nothing, so a run of m points
// costs 16 atomics instead of 16 m.  The four lanes of a point hit one or two
// lines, so each atomic instruction makes few requests.
__global__ __launch_bounds__(kBlock) void bwd_f2_quad_kernel(const float *__restrict__ x, int64_t n,
                                                             const float *__restrict__ dout, int64_t dstride,
                                                             float *__restrict__ grad, LaunchParams lp) {
    __shared__ float park[kBlock / 64][4 * 64];
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint32_t mask = lp.mask;
    float *__restrict__ g = grad + 2 * ((uint64_t)l << lp.log2_table_size);
    const int lane = threadIdx.x & 63, sub = lane & 3;
    const int dx = sub >> 1, j = sub & 1;
    float *wbuf = park[threadIdx.x >> 6];
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    // wave-uniform loop over the wave's 16 points: every lane runs the shuffles and the ballot
    for (int64_t pw = it.p0 + (threadIdx.x >> 2 & ~15); pw < end; pw += kBlock / 4) {
        const int64_t p = pw + (lane >> 2);
        const bool valid = p < end;
        const int64_t q = valid ? p : pw;
        int32_t v0, v1, v2;
        float a0, a1, a2;
        locate1(x[3 * q + 0], N, v0, a0);
        locate1(x[3 * q + 1], N, v1, a1);
        locate1(x[3 * q + 2], N, v2, a2);
        const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hy1 = hy0 + kPrimeY;
        const uint32_t hz0 = (uint32_t)v2 * kPrimeZ, hz1 = hz0 + kPrimeZ;
        const float gw = dout[q * dstride + 2 * l + j] * (dx ? a0 : 1.f - a0);
        const float wy0 = 1.f - a1, wz0 = 1.f - a2;
        float c[4] = {gw * (wy0 * wz0), gw * (wy0 * a2), gw * (a1 * wz0), gw * (a1 * a2)};
        const int32_t u0 = __shfl_up(v0, 4, 64), u1 = __shfl_up(v1, 4, 64), u2 = __shfl_up(v2, 4, 64);
        const bool same = valid && lane >= 4 && u0 == v0 && u1 == v1 && u2 == v2;
        const uint64_t dup = __ballot(same);  // the 4 lanes of a point agree
        bool emit = valid;
        if (dup != 0) {
            const uint64_t heads = ~dup, tails = (heads >> 4) | (0xFull << 60);
            const int first = (63 - __builtin_clzll(heads & ((2ull << lane) - 1ull))) >> 2;  // run's first point
            const int last = __builtin_ctzll(tails & (~0ull << lane)) >> 2;                  // run's last point
#pragma unroll
            for (int k = 0; k < 4; ++k) wbuf[k * 64 + lane] = c[k];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            emit = valid && first == (lane >> 2);
            if (emit && last > first) {
#pragma unroll
                for (int k = 0; k < 4; ++k) c[k] = 0.f;
                for (int i = first; i <= last; ++i)
#pragma unroll
                    for (int k = 0; k < 4; ++k) c[k] += wbuf[k * 64 + 4 * i + sub];
            }
            // the next pass overwrites this wave's parked values after these reads
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
        if (emit) {
            const uint32_t cx = (uint32_t)v0 + (uint32_t)dx;
            fadd(g + 2 * ((cx ^ hy0 ^ hz0) & mask) + j, c[0]);
            fadd(g + 2 * ((cx ^ hy0 ^ hz1) & mask) + j, c[1]);
            fadd(g + 2 * ((cx ^ hy1 ^ hz0) & mask) + j, c[2]);
            fadd(g + 2 * ((cx ^ hy1 ^ hz1) & mask) + j, c[3]);
        }
    }
}

// ---------------------------------------------------------------- debug export

__global__ __launch_bounds__(kBlock) void corners_kernel(const float *__restrict__ x, int64_t n,
                                                         uint32_t *__restrict__ idx,
                                                         float *__restrict__ w, LaunchParams lp) {
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int l = blockIdx.y;
    if (p >= n) return;
    const float N = (float)lp.res[l];
    int32_t v[3];
    float a[3];
    for (int d = 0; d < 3; ++d) locate1(x[3 * p + d], N, v[d], a[d]);
    const int64_t o = (p * lp.n_levels + l) * 8;
    for (int k = 0; k < 8; ++k) {
        const uint32_t dx = (k >> 2) & 1, dy = (k >> 1) & 1, dz = k & 1;
        const uint32_t h = ((uint32_t)v[0] + dx) ^ (((uint32_t)v[1] + dy) * kPrimeY) ^
                           (((uint32_t)v[2] + dz) * kPrimeZ);
        if (idx) idx[o + k] = h & lp.mask;
        if (w) w[o + k] = ((dx ? a[0] : 1.f - a[0]) * (dy ? a[1] : 1.f - a[1])) * (dz ? a[2] : 1.f - a[2]);
    }
}

int grid_blocks(const LaunchParams &lp) {
    return lp.xcd_map ? kNumXcd * lp.per_xcd : lp.items;
}

// Level-major staging [L][n][F] -> rows out[p * ostride + l * F + j], pts
// points per workgroup through LDS so that both sides move whole lines.
// VEC moves 16 bytes per access on both sides (F n and F L multiples of 4,
// rows and output 16-byte aligned); otherwise 4 bytes.
// stage2 (may be NULL): a second stage of partial blends, added element-wise
// while transposing at the levels whose bit is set in second.
template <int F, bool VEC>
__global__ __launch_bounds__(kBlock) void transpose_kernel(const float *__restrict__ stage,
                                                           const float *__restrict__ stage2, uint64_t second,
                                                           int64_t n, int L, int pts, float *__restrict__ out,
                                                           int64_t ostride, const uint32_t *__restrict__ perm) {
    extern __shared__ float tile[];  // [pts][F L + 4]: rows 16-byte aligned when F L is a multiple of 4
    const int row = F * L + 4;
    const int64_t p0 = (int64_t)blockIdx.x * pts;
    const int np = (int)min((int64_t)pts, n - p0);
    if constexpr (VEC) {
        // Level l of this block is F np contiguous floats, F np / 4 float4 (pts is a multiple of 4).
        const int q_per_level = F * pts / 4;
        for (int e = threadIdx.x; e < L * q_per_level; e += kBlock) {
            const int l = e / q_per_level, qd = e - l * q_per_level;
            if (4 * qd < F * np) {
                const int64_t off = ((int64_t)l * n + p0) * F + 4 * qd;
                float4 v = *reinterpret_cast<const float4 *>(stage + off);
                if (stage2 && ((second >> l) & 1u)) {
                    const float4 w = *reinterpret_cast<const float4 *>(stage2 + off);
                    v.x += w.x, v.y += w.y, v.z += w.z, v.w += w.w;
                }
                if constexpr (F == 1) {
                    tile[(4 * qd + 0) * row + l] = v.x;
                    tile[(4 * qd + 1) * row + l] = v.y;
                    tile[(4 * qd + 2) * row + l] = v.z;
                    tile[(4 * qd + 3) * row + l] = v.w;
                } else if constexpr (F == 2) {
                    // points 2 qd and 2 qd + 1, features 0 and 1 of level l
                    *reinterpret_cast<float2 *>(&tile[(2 * qd) * row + 2 * l]) = make_float2(v.x, v.y);
                    *reinterpret_cast<float2 *>(&tile[(2 * qd + 1) * row + 2 * l]) = make_float2(v.z, v.w);
                } else {
                    // features 4 qd mod F .. + 3 of point 4 qd / F
                    const int i = 4 * qd / F, f = 4 * qd - i * F;
                    *reinterpret_cast<float4 *>(&tile[i * row + F * l + f]) = v;
                }
            }
        }
        __syncthreads();
        const int q_per_row = F * L / 4;  // float4 per output row
        for (int e = threadIdx.x; e < pts * q_per_row; e += kBlock) {
            const int i = e / q_per_row, c = e - i * q_per_row;
            if (i < np) {
                const int64_t r = perm ? (int64_t)perm[p0 + i] : p0 + i;  // the row's point
                *reinterpret_cast<float4 *>(out + r * ostride + 4 * c) =
                    *reinterpret_cast<const float4 *>(&tile[i * row + 4 * c]);
            }
        }
    } else {
        const int total = pts * F * L;
        for (int e = threadIdx.x; e < total; e += kBlock) {
            const int l = e / (F * pts), r = e - l * F * pts;
            const int i = r / F, j = r - i * F;
            if (i < np) {
                const int64_t off = ((int64_t)l * n + p0 + i) * F + j;
                tile[i * row + F * l + j] = stage2 && ((second >> l) & 1u) ? stage[off] + stage2[off] : stage[off];
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < total; e += kBlock) {
            const int i = e / (F * L), c = e - i * F * L;
            if (i < np) out[(perm ? (int64_t)perm[p0 + i] : p0 + i) * ostride + c] = tile[i * row + c];
        }
    }
}

template <int F>
hipError_t launch_transpose_f(const float *stage, int64_t n, int L, float *out, int64_t ostride,
                              hipStream_t stream, const float *stage2 = nullptr, uint64_t second = ~0ull,
                              const uint32_t *perm = nullptr) {
    // Points per workgroup: 64, fewer for wide rows so that the tile stays near 32 KB.
    const int pts = std::max(4, std::min(64, 8192 / (F * L + 4)) / 4 * 4);
    const unsigned blocks = (unsigned)((n + pts - 1) / pts);
    const size_t lds = (size_t)pts * (F * L + 4) * sizeof(float);
    bool vec = (n * F) % 4 == 0 && (F * L) % 4 == 0 && ostride % 4 == 0 && ((uintptr_t)out & 15) == 0 &&
               ((uintptr_t)stage & 15) == 0;
    if (vec && stage2 && ((uintptr_t)stage2 & 15)) vec = false;
    if (vec)
        transpose_kernel<F, true><<<blocks, kBlock, lds, stream>>>(stage, stage2, second, n, L, pts, out, ostride,
                                                                   perm);
    else
        transpose_kernel<F, false><<<blocks, kBlock, lds, stream>>>(stage, stage2, second, n, L, pts, out, ostride,
                                                                    perm);
    return hipGetLastError();
}

// On the staged path a level's table above one XCD's L2 (4 MiB) is gathered
// in two launches, one per half (fwd_f2_pair_kernel SPLIT): measured on the
// 8 MiB levels of a binary16 T = 2^21 grid, 2.07 against 2.29 ms; quarters
// cost more in instructions than they gain (3.8 ms).  With room for a second
// stage the second half writes its own partial blends and the transpose adds
// the two (1.96 ms); adding into the first half's stage in place costs a
// dependent read of it (2.04 ms).  Splitting the standard grid's 4 MiB levels
// measured slower (110 against 98 us).  The direct path gathers
// in one pass: there the second half's read-modify-write of 8 bytes per row
// and level made the forward 1.6 times slower.  The other shapes' kernels
// gather in one pass: for F = 4 at 8 MiB a split gained 3 %, and F = 8 rows,
// written directly, cost 2.9 times as much.
//
// Only a level whose gathers can touch more table lines than that is split.
// The x prime is 1, so a row of N_l + 1 x-vertices (fixed y and z) lies in
// one aligned block of next_pow2(N_l + 1) entries, and a level has
// (N_l + 1)^2 such rows: the coarse levels of a large table touch a small
// part of it (the binary16 T = 2^21 grid's levels up to N_l = 79 touch at
// most 3.3 MB of its 8 MiB) and are gathered in one pass.
size_t level_footprint(const LaunchParams &lp, int l, size_t entry_bytes) {
    const uint64_t R = (uint64_t)lp.res[l] + 1;
    uint64_t block = 1;
    while (block < R) block <<= 1;
    const uint64_t per_line = 128 / entry_bytes;
    const uint64_t table_lines = std::max<uint64_t>(1, ((uint64_t)1 << lp.log2_table_size) / per_line);
    const uint64_t row_lines = (block + per_line - 1) / per_line;
    const uint64_t rows = R * R;
    // rows * row_lines, capped at the table (no overflow: R <= 2^20 + 1)
    const uint64_t lines = rows > table_lines / row_lines ? table_lines : std::min(table_lines, rows * row_lines);
    return (size_t)(lines * 128);
}

// The levels of lp (a staged gather) whose footprint exceeds ft.split_kib.
uint64_t split_levels(const LaunchParams &lp, size_t entry_bytes, const FwdTune &ft) {
    uint64_t split = 0;
    if (ft.split_kib <= 0) return 0;
    const int have = lp.chunks ? lp.items / lp.chunks : 0;
    for (int i = 0; i < have; ++i) {
        const int l = lp.level_order[i];
        if (level_footprint(lp, l, entry_bytes) > ((size_t)ft.split_kib << 10)) split |= 1ull << l;
    }
    return split;
}

// lp restricted to the levels of the bit mask (their order kept).
LaunchParams with_levels(const LaunchParams &lp, uint64_t levels) {
    LaunchParams r = lp;
    int pos = 0;
    const int have = lp.chunks ? lp.items / lp.chunks : 0;
    for (int i = 0; i < have; ++i) {
        const int l = lp.level_order[i];
        if ((levels >> l) & 1u) r.level_order[pos++] = (int8_t)l;
    }
    r.items = r.chunks * pos;
    r.per_xcd = (r.items + kNumXcd - 1) / kNumXcd;
    return r;
}

// split: the levels gathered one table half per pass (split_levels).
template <int DT>
hipError_t launch_gather_dt(const LaunchParams &lp, const float *x, int64_t n, const void *table, float *out,
                            int64_t ostride, int64_t lstride, const FwdTune &ft, hipStream_t stream,
                            float *out2 = nullptr, uint64_t split = 0) {
    dim3 grid(grid_blocks(lp)), block(kBlock);
    if (lstride == 2 && ft.lanes == 1) {
        fwd_f2_kernel<DT><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lp);
    } else if (split && lstride != 2) {  // staged output only
        // The levels of `split` one table half per pass, the others in one.
        const LaunchParams lw = with_levels(lp, ~split), ls = with_levels(lp, split);
        if (lw.items > 0) {
            hipError_t e = launch_gather_dt<DT>(lw, x, n, table, out, ostride, lstride, ft, stream, nullptr, 0);
            if (e != hipSuccess) return e;
        }
        const dim3 sgrid(grid_blocks(ls));
        for (int half = 0; half < 2 && ls.items > 0; ++half) {
            float *dst = half && out2 ? out2 : out;
            const int add = half && !out2;
            if (ft.nt) fwd_f2_pair_kernel<DT, 4, true, float, true><<<sgrid, block, 0, stream>>>(x, n, table, dst, ostride, lstride, ls, half, add);
            else fwd_f2_pair_kernel<DT, 4, false, float, true><<<sgrid, block, 0, stream>>>(x, n, table, dst, ostride, lstride, ls, half, add);
        }
    } else if (ft.nt) {
        if (ft.unroll == 1) fwd_f2_pair_kernel<DT, 1, true><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
        else if (ft.unroll == 2) fwd_f2_pair_kernel<DT, 2, true><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
        else fwd_f2_pair_kernel<DT, 4, true><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
    } else {
        if (ft.unroll == 1) fwd_f2_pair_kernel<DT, 1, false><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
        else if (ft.unroll == 2) fwd_f2_pair_kernel<DT, 2, false><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
        else fwd_f2_pair_kernel<DT, 4, false><<<grid, block, 0, stream>>>(x, n, table, out, ostride, lstride, lp, 0);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const LaunchParams &lp, const float *x, int64_t n, const void *table,
                          int table_dtype, float *out, int64_t out_stride, const FwdTune &ft,
                          float *stage, hipStream_t stream, float *stage2, const uint32_t *perm) {
    hipError_t e;
    if (!stage) {
        return table_dtype == 0 ? launch_gather_dt<0>(lp, x, n, table, out, out_stride, 2, ft, stream)
                                : launch_gather_dt<1>(lp, x, n, table, out, out_stride, 2, ft, stream);
    }
    // Levels of this gather (lp.level_order; the others came from launch_forward_dense)
    // that go one table half per pass; stage2, if any, holds their second halves.
    const uint64_t split = split_levels(lp, table_dtype == 0 ? sizeof(float2) : sizeof(uint32_t), ft);
    if (lp.items > 0) {
        e = table_dtype == 0 ? launch_gather_dt<0>(lp, x, n, table, stage, 2, 2 * n, ft, stream, stage2, split)
                             : launch_gather_dt<1>(lp, x, n, table, stage, 2, 2 * n, ft, stream, stage2, split);
        if (e != hipSuccess) return e;
    }
    return launch_transpose_f<2>(stage, n, lp.n_levels, out, out_stride, stream, stage2, split, perm);
}

template <int DT, class OutT>
hipError_t launch_dense_dt(const LaunchParams &lp, const DenseLevels &dl, const float *x, int64_t n,
                           const void *table, OutT *out, int64_t ostride, int64_t lstride, hipStream_t stream) {
    // dl.max_vals: the entries of all the levels' copies together.
    const size_t lds = (size_t)dl.max_vals * sizeof(typename Table2<DT>::Raw);
    hipError_t e = hipFuncSetAttribute((const void *)fwd_dense_kernel<DT, OutT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // About 256 workgroups (one per CU), of at least 1024 points.
    const int64_t chunk = std::max<int64_t>(1024, (n + 255) / 256 + 1023) / 1024 * 1024;
    const int64_t blocks = (n + chunk - 1) / chunk;
    fwd_dense_kernel<DT, OutT><<<(unsigned)blocks, kDenseFwdThreads, lds, stream>>>(x, n, table, out, ostride,
                                                                                   lstride, lp, dl, chunk);
    return hipGetLastError();
}

hipError_t launch_transpose(int F, const float *stage, int64_t n, int L, float *out, int64_t ostride,
                            hipStream_t stream) {
    switch (F) {
    case 1: return launch_transpose_f<1>(stage, n, L, out, ostride, stream);
    case 2: return launch_transpose_f<2>(stage, n, L, out, ostride, stream);
    case 4: return launch_transpose_f<4>(stage, n, L, out, ostride, stream);
    case 8: return launch_transpose_f<8>(stage, n, L, out, ostride, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_forward_dense(const LaunchParams &lp, const DenseLevels &dl, const float *x, int64_t n,
                                const void *table, int table_dtype, void *stage, bool half_stage,
                                hipStream_t stream) {
    if (!dl.count || n == 0) return hipSuccess;
    if (half_stage)
        return table_dtype == 0 ? launch_dense_dt<0>(lp, dl, x, n, table, (_Float16 *)stage, 2, 2 * n, stream)
                                : launch_dense_dt<1>(lp, dl, x, n, table, (_Float16 *)stage, 2, 2 * n, stream);
    return table_dtype == 0 ? launch_dense_dt<0>(lp, dl, x, n, table, (float *)stage, 2, 2 * n, stream)
                            : launch_dense_dt<1>(lp, dl, x, n, table, (float *)stage, 2, 2 * n, stream);
}

hipError_t launch_encode_stage_f16(const LaunchParams &lp, const float *x, int64_t n, const void *table,
                                   int table_dtype, _Float16 *stage, hipStream_t stream) {
    if (lp.items == 0) return hipSuccess;
    dim3 grid(grid_blocks(lp)), block(kBlock);
    if (table_dtype == 0)
        fwd_f2_pair_kernel<0, 4, false, _Float16><<<grid, block, 0, stream>>>(x, n, table, stage, 2, 2 * n, lp, 0);
    else
        fwd_f2_pair_kernel<1, 4, false, _Float16><<<grid, block, 0, stream>>>(x, n, table, stage, 2, 2 * n, lp, 0);
    return hipGetLastError();
}

hipError_t launch_backward(const LaunchParams &lp, const float *x, int64_t n, const float *dout,
                           int64_t dout_stride, float *dtable, int lanes, hipStream_t stream) {
    dim3 grid(grid_blocks(lp)), block(kBlock);
    if (lanes == 4) bwd_f2_quad_kernel<<<grid, block, 0, stream>>>(x, n, dout, dout_stride, dtable, lp);
    else if (lanes == 2) bwd_f2_kernel<2><<<grid, block, 0, stream>>>(x, n, dout, dout_stride, dtable, lp);
    else bwd_f2_kernel<1><<<grid, block, 0, stream>>>(x, n, dout, dout_stride, dtable, lp);
    return hipGetLastError();
}

hipError_t launch_debug_corners(const LaunchParams &lp, const float *x, int64_t n, uint32_t *idx,
                                float *w, hipStream_t stream) {
    dim3 grid((unsigned)((n + kBlock - 1) / kBlock), lp.n_levels), block(kBlock);
    corners_kernel<<<grid, block, 0, stream>>>(x, n, idx, w, lp);
    return hipGetLastError();
}

}  // namespace hg
