// Generic-shape kernels of the hash-grid encoder for gfx950: any input
// dimension D in 1..4 and F in {1, 2, 4, 8} features per entry, and the
// gradient with respect to the points for every shape.
//
// Shapes: the jsqmd.com HashEncoding hashes d-dimensional points with its
// list of seven primes (section 3; 2-D images, 4-D space-time) and its
// experiment table runs 2 to 4 features per entry (section 4).  The method is
// the same for every shape: per (point, level) the 2^D voxel corners
// c = v + b (b in {0,1}^D, corner k has b_d = bit D-1-d of k, so the first
// coordinate is the outermost loop), h(c) = XOR_d c_d * prime_d in uint32
// masked to T, weights w_k = prod_d (b_d ? f_d : 1 - f_d), and
// out[l*F + j] = sum_k w_k table[l][h(c_k)][j]; the backward adds
// w_k dL/dout[l*F + j] into every entry a corner hashed to.  The D = 3, F = 2
// grid has its own tuned kernels (encode_kernels.hip, binned_backward.hip);
// these cover the other shapes: a lane-pair forward (written level-major and
// transposed into the rows for F <= 4), a one-thread-per-(point, level)
// forward, the fp32-atomic backward used without a workspace (the binned one
// is generic_binned.hip) and the corner export.
//
// Gradient with respect to the points (implied by ipipp.com section 3, which
// puts a learned canonical-space transform before the encoder; never written
// on the pages): inside a voxel the blend is multilinear in f and f_d moves
// with x_d at rate N_l, so with s_k = sum_j dL/dout[l*F + j] table[l][h(c_k)][j]
//   dL/dx_d = sum_l N_l sum_k (b_d ? 1 : -1) prod_{e != d} (b_e ? f_e : 1 - f_e) s_k.
// Level-major work items write each level's D partial sums to a [L][n][D]
// stage, which a second kernel sums over levels in level order; without a
// stage one thread walks all levels of its point.  Both add the same fp32
// terms in the same order (contraction off), so they agree bit for bit.  The
// level-major pass uses the forward's lane pairs: a level's derivative is
// N_l (half(0) + half(1)), half(b) the corners with first-coordinate offset b.
#include <type_traits>

#include "binned_common.h"

namespace hg {
namespace {

// Voxel of a D-dimensional point at resolution N: per coordinate the hash
// terms of the lower and upper corner and the fraction.
template <int D>
struct Voxel {
    uint32_t h0[D], h1[D];
    float f[D];
};

template <int D>
__device__ __forceinline__ void locate_point(const float *__restrict__ xp, float N, Voxel<D> &vx) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        int32_t v;
        locate1(xp[d], N, v, vx.f[d]);
        vx.h0[d] = (uint32_t)v * kPrimeList[d];
        vx.h1[d] = vx.h0[d] + kPrimeList[d];
    }
}

template <int D>
__device__ __forceinline__ uint32_t corner_hash(const Voxel<D> &vx, int k, uint32_t mask) {
    uint32_t h = 0;
#pragma unroll
    for (int d = 0; d < D; ++d) h ^= ((k >> (D - 1 - d)) & 1) ? vx.h1[d] : vx.h0[d];
    return h & mask;
}

// Corner h of the half with first-coordinate offset b (corner k = b 2^(D-1) + h):
// only the first coordinate's choice depends on the runtime b, so the other
// terms stay compile-time register picks (a runtime k for every coordinate
// made the compiler index the Voxel arrays through scratch memory).
template <int D>
__device__ __forceinline__ uint32_t half_corner_hash(const Voxel<D> &vx, int b, int h, uint32_t mask) {
    uint32_t v = b ? vx.h1[0] : vx.h0[0];
#pragma unroll
    for (int d = 1; d < D; ++d) v ^= ((h >> (D - 1 - d)) & 1) ? vx.h1[d] : vx.h0[d];
    return v & mask;
}

template <int D>
__device__ __forceinline__ float half_corner_weight(const Voxel<D> &vx, int b, int h) {
    float w = b ? vx.f[0] : 1.f - vx.f[0];
#pragma unroll
    for (int d = 1; d < D; ++d) w *= ((h >> (D - 1 - d)) & 1) ? vx.f[d] : 1.f - vx.f[d];
    return w;
}

template <int D>
__device__ __forceinline__ float corner_weight(const Voxel<D> &vx, int k) {
    float w = 1.f;
#pragma unroll
    for (int d = 0; d < D; ++d) w *= ((k >> (D - 1 - d)) & 1) ? vx.f[d] : 1.f - vx.f[d];
    return w;
}

// ---------------------------------------------------------------- forward

// Output element (p, l, j) is out[p * ostride + l * lstride + j]: lstride = F
// writes [n][L*F] rows, ostride = F with lstride = F n a level-major [L][n][F]
// stage whose stores are whole lines.
template <int D, int F, int DT>
__global__ __launch_bounds__(kBlock) void fwd_generic_kernel(const float *__restrict__ x, int64_t n,
                                                             const void *__restrict__ table,
                                                             float *__restrict__ out, int64_t ostride,
                                                             int64_t lstride, LaunchParams lp) {
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p = it.p0 + threadIdx.x; p < end; p += kBlock) {
        Voxel<D> vx;
        locate_point<D>(x + p * D, N, vx);
        float acc[F];
#pragma unroll
        for (int j = 0; j < F; ++j) acc[j] = 0.f;
#pragma unroll
        for (int k = 0; k < (1 << D); ++k) {
            float e[F];
            load_features<F, DT>(table, lbase + corner_hash<D>(vx, k, lp.mask), e);
            const float w = corner_weight<D>(vx, k);
#pragma unroll
            for (int j = 0; j < F; ++j) acc[j] += w * e[j];
        }
        float *orow = out + p * ostride + (int64_t)l * lstride;
#pragma unroll
        for (int j = 0; j < F; ++j) orow[j] = acc[j];
    }
}

// Points per lane pair in flight: the 2^(D-1) corner loads of U points are
// issued before the first blend, within about 32 registers of features.
constexpr int pair_unroll(int D, int F) {
    const int per = (1 << (D - 1)) * F;
    return per <= 8 ? 4 : per <= 16 ? 2 : 1;
}

// Lane-pair forward of every shape: lane sub of a pair takes the corners whose
// first coordinate is v_0 + sub.  The first prime is 1, so the two corners of
// an x-pair differ in the low index bits and mostly share a 128-byte line: the
// pair's two loads are one line request where one thread per point makes two.
// The halves' partial sums are exchanged with a DPP swap and each lane writes
// half of the level's F features (F = 1: lane 0 writes); output layout as
// fwd_generic_kernel.
template <int D, int F, int DT>
__global__ __launch_bounds__(kBlock) void fwd_generic_pair_kernel(const float *__restrict__ x, int64_t n,
                                                                  const void *__restrict__ table,
                                                                  float *__restrict__ out, int64_t ostride,
                                                                  int64_t lstride, LaunchParams lp) {
    constexpr int U = pair_unroll(D, F), H = 1 << (D - 1), kPairs = kBlock / 2;
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const int sub = threadIdx.x & 1;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p0 = it.p0 + (threadIdx.x >> 1); p0 < end; p0 += (int64_t)kPairs * U) {
        float e[U][H][F];
        Voxel<D> vx[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = p0 + (int64_t)u * kPairs;
            ok[u] = p < end;
            locate_point<D>(x + (ok[u] ? p : p0) * D, N, vx[u]);  // p0 < end: always a valid point
#pragma unroll
            for (int h = 0; h < H; ++h)
                load_features<F, DT>(table, lbase + half_corner_hash<D>(vx[u], sub, h, lp.mask), e[u][h]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float part[F];
#pragma unroll
            for (int j = 0; j < F; ++j) part[j] = 0.f;
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const float w = half_corner_weight<D>(vx[u], sub, h);
#pragma unroll
                for (int j = 0; j < F; ++j) part[j] += w * e[u][h][j];
            }
            float *orow = out + (p0 + (int64_t)u * kPairs) * ostride + (int64_t)l * lstride;
            if constexpr (F == 1) {
                const float v = part[0] + swap_pair(part[0]);
                if (ok[u] && sub == 0) orow[0] = v;
            } else {
                constexpr int HF = F / 2;
                float v[HF];
#pragma unroll
                for (int i = 0; i < HF; ++i) {
                    // lane 0 writes features [0, F/2) and sends the upper half; lane 1 the reverse
                    const float mine = sub ? part[HF + i] : part[i];
                    v[i] = mine + swap_pair(sub ? part[i] : part[HF + i]);
                }
                if (ok[u]) {
#pragma unroll
                    for (int i = 0; i < HF; ++i) orow[sub * HF + i] = v[i];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- backward

template <int D, int F>
__global__ __launch_bounds__(kBlock) void bwd_generic_kernel(const float *__restrict__ x, int64_t n,
                                                             const float *__restrict__ dout, int64_t dstride,
                                                             float *__restrict__ grad, LaunchParams lp) {
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p = it.p0 + threadIdx.x; p < end; p += kBlock) {
        Voxel<D> vx;
        locate_point<D>(x + p * D, N, vx);
        float g[F];
#pragma unroll
        for (int j = 0; j < F; ++j) g[j] = dout[p * dstride + (int64_t)l * F + j];
#pragma unroll
        for (int k = 0; k < (1 << D); ++k) {
            float *e = grad + (lbase + corner_hash<D>(vx, k, lp.mask)) * F;
            const float w = corner_weight<D>(vx, k);
#pragma unroll
            for (int j = 0; j < F; ++j) unsafeAtomicAdd(e + j, w * g[j]);
        }
    }
}

// Atomic backward of the levels with few distinct accumulators (small
// tables, or coarse levels whose whole vertex grid fits): one workgroup per
// (chunk of kDensePts points, level) first sums its points' contributions in
// LDS, then adds each non-zero sum to the gradient with one fp32 atomic.  An
// entry that receives 10^4 or more additions (a 2-entry table under a few
// thousand points) would otherwise collect that many fp32 roundings in an
// arbitrary order; the LDS sums are 64-bit fixed point, exact and
// order-independent: contributions are rounded to 2^-k with k = 30 - e from
// the chunk's largest finite |dL/dout| < 2^e, so each fits 31 bits and a
// chunk's sum of at most 2^16 of them fits 47.  This is also the LDS
// pre-reduction of duplicate coarse-level corners: a vertex-indexed level
// makes one global atomic per touched vertex and chunk instead of one per
// point and corner.  Points with a non-finite upstream value, and points whose
// voxel leaves the vertex grid (outside [0,1)^D), add their contributions
// straight to the gradient with fp32 atomics.
constexpr int kDensePts = 4096;

template <int D, int F>
__global__ __launch_bounds__(kBlock) void bwd_dense_kernel(const float *__restrict__ x, int64_t n,
                                                           const float *__restrict__ dout, int64_t dstride,
                                                           float *__restrict__ grad, LaunchParams lp,
                                                           DenseLevels dl) {
    extern __shared__ unsigned long long acc[];  // [values]: entry- or vertex-indexed, F per index
    __shared__ float wmax[kBlock / 64];
    const int l = dl.level[blockIdx.y];
    const bool by_vertex = dl.by_vertex[blockIdx.y] != 0;
    const int res = lp.res[l];
    const float N = (float)res;
    const int V1 = res + 1;  // vertices per axis (by_vertex only)
    int size = 1 << lp.log2_table_size;
    if (by_vertex) {
        size = 1;
#pragma unroll
        for (int d = 0; d < D; ++d) size *= V1;
    }
    const int vals = size * F;
    float *__restrict__ g = grad + ((uint64_t)l << lp.log2_table_size) * F;
    const int64_t p0 = (int64_t)blockIdx.x * kDensePts;
    const int64_t end = min(p0 + (int64_t)kDensePts, n);
    for (int i = threadIdx.x; i < vals; i += kBlock) acc[i] = 0ull;
    // The chunk's largest finite |dL/dout| at this level sets the fixed-point step.
    float m = 0.f;
    for (int64_t p = p0 + threadIdx.x; p < end; p += kBlock) {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const float a = fabsf(dout[p * dstride + (int64_t)l * F + j]);
            if (a <= 3.40282347e38f) m = fmaxf(m, a);
        }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    for (int w = 0; w < kBlock / 64; ++w) m = fmaxf(m, wmax[w]);
    const int k = binned::fixed_exponent(__float_as_uint(m));
    for (int64_t p = p0 + threadIdx.x; p < end; p += kBlock) {
        int32_t v[D];
        float f[D];
        bool inside = true;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            locate1(x[p * D + d], N, v[d], f[d]);
            inside = inside && v[d] >= 0 && v[d] < res;
        }
        float gv[F];
        bool fin = true;
#pragma unroll
        for (int j = 0; j < F; ++j) {
            gv[j] = dout[p * dstride + (int64_t)l * F + j];
            fin = fin && isfinite(gv[j]);
        }
        const bool local = fin && (inside || !by_vertex);
#pragma unroll
        for (int c = 0; c < (1 << D); ++c) {
            uint32_t h = 0, vid = 0, stride = 1;
            float w = 1.f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const uint32_t b = (uint32_t)(c >> (D - 1 - d)) & 1u;
                h ^= ((uint32_t)v[d] + b) * kPrimeList[d];
                vid += ((uint32_t)v[d] + b) * stride;
                stride *= (uint32_t)V1;
                w *= b ? f[d] : 1.f - f[d];
            }
            h &= lp.mask;
            if (local) {
                const int base = (int)(by_vertex ? vid : h) * F;
#pragma unroll
                for (int j = 0; j < F; ++j) atomicAdd(acc + base + j, binned::to_fixed(w * gv[j], k));
            } else {
#pragma unroll
                for (int j = 0; j < F; ++j) unsafeAtomicAdd(g + (uint64_t)h * F + j, w * gv[j]);
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < vals; i += kBlock) {
        const long long s = (long long)acc[i];
        if (s == 0) continue;
        const int idx = i / F, j = i - idx * F;
        uint32_t e = (uint32_t)idx;
        if (by_vertex) {
            uint32_t h = 0;
            int r = idx;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                h ^= (uint32_t)(r % V1) * kPrimeList[d];
                r /= V1;
            }
            e = h & lp.mask;
        }
        unsafeAtomicAdd(g + (uint64_t)e * F + j, (float)ldexp((double)s, -k));
    }
}

// ---------------------------------------------------------------- corners

template <int D>
__global__ __launch_bounds__(kBlock) void corners_generic_kernel(const float *__restrict__ x, int64_t n,
                                                                 uint32_t *__restrict__ idx, float *__restrict__ w,
                                                                 LaunchParams lp) {
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int l = blockIdx.y;
    if (p >= n) return;
    Voxel<D> vx;
    locate_point<D>(x + p * D, (float)lp.res[l], vx);
    const int64_t o = (p * lp.n_levels + l) << D;
#pragma unroll
    for (int k = 0; k < (1 << D); ++k) {
        if (idx) idx[o + k] = corner_hash<D>(vx, k, lp.mask);
        if (w) w[o + k] = corner_weight<D>(vx, k);
    }
}

// ---------------------------------------------------------------- dL/dx

// Corner hh of the half with first-coordinate offset b (corner k = b 2^(D-1)
// + hh) adds its term to that half's sums h[0..D): with s = sum_j dl_j e_j,
// h[d] += (b_d ? 1 : -1) prod_{q != d} (b_q ? f_q : 1 - f_q) s.  A level's
// dL/dx is N_l (half(0) + half(1)), each half summed over hh in order: the
// lane-pair kernel and the point kernel both go through this function, so
// they agree bit for bit.
template <int D, int F>
__device__ __forceinline__ void corner_grad_term(const Voxel<D> &vx, const float (&e)[F], const float (&dl)[F],
                                                 int b, int hh, float (&h)[D]) {
#pragma clang fp contract(off)
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < F; ++j) s += dl[j] * e[j];
    // bit of coordinate d: b for d = 0, bit D-1-d of hh otherwise
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const bool bd = d == 0 ? b != 0 : ((hh >> (D - 1 - d)) & 1) != 0;
        float dw = bd ? 1.f : -1.f;
#pragma unroll
        for (int q = 0; q < D; ++q) {
            if (q == d) continue;
            const bool bq = q == 0 ? b != 0 : ((hh >> (D - 1 - q)) & 1) != 0;
            dw *= bq ? vx.f[q] : 1.f - vx.f[q];
        }
        h[d] += dw * s;
    }
}

// One half's sums from its corners' features e[hh].
template <int D, int F>
__device__ __forceinline__ void half_grad(const Voxel<D> &vx, const float (&e)[1 << (D - 1)][F],
                                          const float (&dl)[F], int b, float (&h)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) h[d] = 0.f;
#pragma unroll
    for (int hh = 0; hh < (1 << (D - 1)); ++hh) corner_grad_term<D, F>(vx, e[hh], dl, b, hh, h);
}

// Features of the corners with first-coordinate offset b.
template <int D, int F, int DT>
__device__ __forceinline__ void load_half(const void *__restrict__ table, uint64_t lbase, uint32_t mask,
                                          const Voxel<D> &vx, int b, float (&e)[1 << (D - 1)][F]) {
    constexpr int H = 1 << (D - 1);
#pragma unroll
    for (int hh = 0; hh < H; ++hh) load_features<F, DT>(table, lbase + half_corner_hash<D>(vx, b, hh, mask), e[hh]);
}

// N_l * d(sum_j dout_j out_j)/dx_d of one (point, level) into g[0..D).
template <int D, int F, int DT>
__device__ __forceinline__ void level_input_grad(const float *__restrict__ xp, const void *__restrict__ table,
                                                 const float *__restrict__ drow, int l, const LaunchParams &lp,
                                                 float (&g)[D]) {
#pragma clang fp contract(off)
    constexpr int H = 1 << (D - 1);
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    Voxel<D> vx;
    locate_point<D>(xp, N, vx);
    float dl[F];
#pragma unroll
    for (int j = 0; j < F; ++j) dl[j] = drow[(int64_t)l * F + j];
    // Corner by corner into the two half sums.
    float h0[D], h1[D];
#pragma unroll
    for (int d = 0; d < D; ++d) h0[d] = h1[d] = 0.f;
#pragma unroll
    for (int k = 0; k < 2 * H; ++k) {
        float e[F];
        load_features<F, DT>(table, lbase + half_corner_hash<D>(vx, k / H, k % H, lp.mask), e);
        if (k < H) corner_grad_term<D, F>(vx, e, dl, 0, k, h0);
        else corner_grad_term<D, F>(vx, e, dl, 1, k - H, h1);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) g[d] = N * (h0[d] + h1[d]);
}

// Level-major, as the forward: two adjacent lanes per point, lane sub takes
// the corners with first-coordinate offset sub (the first prime is 1, so the
// two corners of an x-pair mostly share a line and the pair's loads make one
// request), U points per pair in flight.  The pair swaps its halves; lane 0
// writes coordinates [0, ceil(D/2)) of stage[l][p][0..D), lane 1 the rest.
template <int D, int F, int DT>
__global__ __launch_bounds__(kBlock) void input_grad_generic_pair_kernel(const float *__restrict__ x, int64_t n,
                                                                         const void *__restrict__ table,
                                                                         const float *__restrict__ dout,
                                                                         int64_t dstride, float *__restrict__ stage,
                                                                         LaunchParams lp) {
#pragma clang fp contract(off)
    constexpr int U = pair_unroll(D, F), H = 1 << (D - 1), kPairs = kBlock / 2, DA = (D + 1) / 2;
    Item it;
    if (!decode_item(lp, it)) return;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const int sub = threadIdx.x & 1;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p0 = it.p0 + (threadIdx.x >> 1); p0 < end; p0 += (int64_t)kPairs * U) {
        float e[U][H][F], dl[U][F];
        Voxel<D> vx[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = p0 + (int64_t)u * kPairs;
            ok[u] = p < end;
            const int64_t q = ok[u] ? p : p0;  // p0 < end: always a valid point
            locate_point<D>(x + q * D, N, vx[u]);
#pragma unroll
            for (int j = 0; j < F; ++j) dl[u][j] = dout[q * dstride + (int64_t)l * F + j];
            load_half<D, F, DT>(table, lbase, lp.mask, vx[u], sub, e[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float h[D], g[D];
            half_grad<D, F>(vx[u], e[u], dl[u], sub, h);
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const float o = swap_pair(h[d]);
                g[d] = N * (sub ? o + h[d] : h[d] + o);  // half(0) + half(1) on both lanes
            }
            if (ok[u]) {
                float *dst = stage + ((int64_t)l * n + p0 + (int64_t)u * kPairs) * D;
#pragma unroll
                for (int d = 0; d < D; ++d)
                    if ((d < DA) == (sub == 0)) dst[d] = g[d];
            }
        }
    }
}

// dx[p][d] = sum over levels, in level order, of stage[l][p][d].
__global__ __launch_bounds__(kBlock) void input_grad_reduce_kernel(const float *__restrict__ stage, int64_t nd,
                                                                   int L, float *__restrict__ dx) {
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= nd) return;
    float acc = 0.f;
    for (int l = 0; l < L; ++l) acc += stage[(int64_t)l * nd + i];
    dx[i] = acc;
}

// One thread per point over all levels (no stage).
template <int D, int F, int DT>
__global__ __launch_bounds__(kBlock) void input_grad_point_kernel(const float *__restrict__ x, int64_t n,
                                                                  const void *__restrict__ table,
                                                                  const float *__restrict__ dout, int64_t dstride,
                                                                  float *__restrict__ dx, LaunchParams lp) {
#pragma clang fp contract(off)
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (p >= n) return;
    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    for (int l = 0; l < lp.n_levels; ++l) {
        float g[D];
        level_input_grad<D, F, DT>(x + p * D, table, dout + p * dstride, l, lp, g);
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] += g[d];
    }
#pragma unroll
    for (int d = 0; d < D; ++d) dx[p * D + d] = acc[d];
}

// ---------------------------------------------------------------- dL/dx, D = 3, F = 2

// The part of a level's dL/dx (before the factor N_l) that the four corners
// with x offset `sub` give, from their features e[(dy, dz)] (order 00, 01,
// 10, 11) and the level's upstream pair (d0, d1).  A level's derivative is
// half(0) + half(1), added in that order by both the lane-pair kernel and the
// point kernel so that the two agree bit for bit.
__device__ __forceinline__ void half_input_grad(float a0, float a1, float a2, const float2 (&e)[4], float d0,
                                                float d1, uint32_t sub, float (&h)[3]) {
#pragma clang fp contract(off)
    float s[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = d0 * e[c].x + d1 * e[c].y;
    const float wy0 = 1.f - a1, wz0 = 1.f - a2;
    const float wx = sub ? a0 : 1.f - a0;
    const float hx = wy0 * (wz0 * s[0] + a2 * s[1]) + a1 * (wz0 * s[2] + a2 * s[3]);
    h[0] = sub ? hx : -hx;
    h[1] = wx * (wz0 * (s[2] - s[0]) + a2 * (s[3] - s[1]));
    h[2] = wx * (wy0 * (s[1] - s[0]) + a1 * (s[3] - s[2]));
}

template <int DT>
__device__ __forceinline__ void corner_pairs(const void *__restrict__ table, uint64_t lbase, uint32_t mask,
                                             uint32_t cx, uint32_t hy0, uint32_t hz0, float2 (&e)[4]) {
    const uint32_t hy1 = hy0 + kPrimeList[1], hz1 = hz0 + kPrimeList[2];
    float v[2];
    load_features<2, DT>(table, lbase + ((cx ^ hy0 ^ hz0) & mask), v);
    e[0] = make_float2(v[0], v[1]);
    load_features<2, DT>(table, lbase + ((cx ^ hy0 ^ hz1) & mask), v);
    e[1] = make_float2(v[0], v[1]);
    load_features<2, DT>(table, lbase + ((cx ^ hy1 ^ hz0) & mask), v);
    e[2] = make_float2(v[0], v[1]);
    load_features<2, DT>(table, lbase + ((cx ^ hy1 ^ hz1) & mask), v);
    e[3] = make_float2(v[0], v[1]);
}

// Upstream rows [n][>= 2L] (row stride dstride) -> level-major [L][n][2], 64
// points per workgroup through LDS, so that the level-major pass reads its
// level's 8 bytes per point contiguously instead of every XCD fetching all of
// the 128-byte rows for the two levels it works on.
constexpr int kRowPts = 64;

template <bool VEC>
__global__ __launch_bounds__(kBlock) void rows_to_levels_kernel(const float *__restrict__ dout, int64_t dstride,
                                                                int64_t n, int L, float *__restrict__ dlm) {
    extern __shared__ float tile[];  // [kRowPts][2L + 4]
    const int row = 2 * L + 4;
    const int64_t p0 = (int64_t)blockIdx.x * kRowPts;
    const int np = (int)min((int64_t)kRowPts, n - p0);
    if constexpr (VEC) {  // rows and dlm 16-byte aligned, L even, n even
        const int q_per_row = L / 2;
        for (int e = threadIdx.x; e < kRowPts * q_per_row; e += kBlock) {
            const int i = e / q_per_row, c = e - i * q_per_row;
            if (i < np)
                *reinterpret_cast<float4 *>(&tile[i * row + 4 * c]) =
                    *reinterpret_cast<const float4 *>(dout + (p0 + i) * dstride + 4 * c);
        }
        __syncthreads();
        const int q_per_level = kRowPts / 2;
        for (int e = threadIdx.x; e < L * q_per_level; e += kBlock) {
            const int l = e / q_per_level, qd = e - l * q_per_level;
            if (2 * qd < np) {
                const float2 a = *reinterpret_cast<const float2 *>(&tile[(2 * qd) * row + 2 * l]);
                const float2 b = *reinterpret_cast<const float2 *>(&tile[(2 * qd + 1) * row + 2 * l]);
                *reinterpret_cast<float4 *>(dlm + ((int64_t)l * n + p0) * 2 + 4 * qd) = make_float4(a.x, a.y, b.x, b.y);
            }
        }
    } else {
        const int total = kRowPts * 2 * L;
        for (int e = threadIdx.x; e < total; e += kBlock) {
            const int i = e / (2 * L), c = e - i * 2 * L;
            if (i < np) tile[i * row + c] = dout[(p0 + i) * dstride + c];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < total; e += kBlock) {
            const int l = e / (2 * kRowPts), r = e - l * 2 * kRowPts;
            const int i = r >> 1, j = r & 1;
            if (i < np) dlm[((int64_t)l * n + p0 + i) * 2 + j] = tile[i * row + 2 * l + j];
        }
    }
}

// Level-major, as the forward: two adjacent lanes per point (lane `sub`
// gathers the corners with x offset sub, which share a cache line with the
// other lane's 15 times in 16), U points per pair in flight; the pair swaps
// its halves and lane 0 writes (dx, dy), lane 1 dz of stage[l][p][0..2].
// The level's upstream pair of point q is dl[q * pstride + l * lstride + 0..1]:
// (dstride, 2) for the rows, (2, 2 n) for a level-major copy.
template <int DT, int U>
__global__ __launch_bounds__(kBlock) void input_grad_pair_kernel(const float *__restrict__ x, int64_t n,
                                                                 const void *__restrict__ table,
                                                                 const float *__restrict__ dl, int64_t pstride,
                                                                 int64_t lstride, float *__restrict__ stage,
                                                                 LaunchParams lp) {
#pragma clang fp contract(off)
    Item it;
    if (!decode_item(lp, it)) return;
    constexpr int kPairs = kBlock / 2;
    const int l = it.level;
    const float N = (float)lp.res[l];
    const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
    const uint32_t sub = threadIdx.x & 1;
    const int64_t end = min(it.p0 + (int64_t)lp.chunk_pts, n);
    for (int64_t p0 = it.p0 + (threadIdx.x >> 1); p0 < end; p0 += (int64_t)kPairs * U) {
        float2 e[U][4];
        float a0[U], a1[U], a2[U], d0[U], d1[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = p0 + (int64_t)u * kPairs;
            ok[u] = p < end;
            const int64_t q = ok[u] ? p : p0;  // p0 < end: always a valid point
            int32_t v0, v1, v2;
            locate1(x[3 * q + 0], N, v0, a0[u]);
            locate1(x[3 * q + 1], N, v1, a1[u]);
            locate1(x[3 * q + 2], N, v2, a2[u]);
            d0[u] = dl[q * pstride + l * lstride];
            d1[u] = dl[q * pstride + l * lstride + 1];
            corner_pairs<DT>(table, lbase, lp.mask, (uint32_t)v0 + sub, (uint32_t)v1 * kPrimeList[1],
                             (uint32_t)v2 * kPrimeList[2], e[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float h[3];
            half_input_grad(a0[u], a1[u], a2[u], e[u], d0[u], d1[u], sub, h);
            float g[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const float o = swap_pair(h[d]);
                g[d] = N * (sub ? o + h[d] : h[d] + o);  // half(0) + half(1) on both lanes
            }
            if (ok[u]) {
                float *dst = stage + ((int64_t)l * n + p0 + (int64_t)u * kPairs) * 3;
                if (sub) {
                    dst[2] = g[2];
                } else {
                    dst[0] = g[0];
                    dst[1] = g[1];
                }
            }
        }
    }
}

// One thread per point over all levels, with the same arithmetic.
template <int DT>
__global__ __launch_bounds__(kBlock) void input_grad_point_pair_kernel(const float *__restrict__ x, int64_t n,
                                                                       const void *__restrict__ table,
                                                                       const float *__restrict__ dout, int64_t dstride,
                                                                       float *__restrict__ dx, LaunchParams lp) {
#pragma clang fp contract(off)
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (p >= n) return;
    float acc[3] = {0.f, 0.f, 0.f};
    for (int l = 0; l < lp.n_levels; ++l) {
        const float N = (float)lp.res[l];
        const uint64_t lbase = (uint64_t)l << lp.log2_table_size;
        int32_t v0, v1, v2;
        float a0, a1, a2;
        locate1(x[3 * p + 0], N, v0, a0);
        locate1(x[3 * p + 1], N, v1, a1);
        locate1(x[3 * p + 2], N, v2, a2);
        const float d0 = dout[p * dstride + 2 * l], d1 = dout[p * dstride + 2 * l + 1];
        float2 e0[4], e1[4];
        corner_pairs<DT>(table, lbase, lp.mask, (uint32_t)v0, (uint32_t)v1 * kPrimeList[1],
                         (uint32_t)v2 * kPrimeList[2], e0);
        corner_pairs<DT>(table, lbase, lp.mask, (uint32_t)v0 + 1u, (uint32_t)v1 * kPrimeList[1],
                         (uint32_t)v2 * kPrimeList[2], e1);
        float h0[3], h1[3];
        half_input_grad(a0, a1, a2, e0, d0, d1, 0, h0);
        half_input_grad(a0, a1, a2, e1, d0, d1, 1, h1);
#pragma unroll
        for (int d = 0; d < 3; ++d) acc[d] += N * (h0[d] + h1[d]);
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) dx[p * 3 + d] = acc[d];
}

int grid_blocks(const LaunchParams &lp) { return lp.xcd_map ? kNumXcd * lp.per_xcd : lp.items; }

// ---------------------------------------------------------------- dispatch

// Calls fn.template operator()<D, F>() for the runtime shape; false if unbuilt.
template <typename Fn>
bool dispatch_shape(int D, int F, Fn &&fn) {
    auto byF = [&](auto dc) {
        constexpr int DD = decltype(dc)::value;
        switch (F) {
        case 1: fn.template operator()<DD, 1>(); return true;
        case 2: fn.template operator()<DD, 2>(); return true;
        case 4: fn.template operator()<DD, 4>(); return true;
        case 8: fn.template operator()<DD, 8>(); return true;
        default: return false;
        }
    };
    switch (D) {
    case 1: return byF(std::integral_constant<int, 1>{});
    case 2: return byF(std::integral_constant<int, 2>{});
    case 3: return byF(std::integral_constant<int, 3>{});
    case 4: return byF(std::integral_constant<int, 4>{});
    default: return false;
    }
}

}  // namespace

hipError_t launch_forward_generic(const LaunchParams &lp, int D, int F, const float *x, int64_t n,
                                  const void *table, int table_dtype, float *out, int64_t out_stride, int lanes,
                                  float *stage, hipStream_t stream) {
    const dim3 grid(grid_blocks(lp)), block(kBlock);
    float *dst = stage ? stage : out;
    const int64_t os = stage ? F : out_stride, ls = stage ? (int64_t)F * n : F;
    const bool ok = dispatch_shape(D, F, [&]<int DD, int FF>() {
        if (lanes == 1) {  // one thread per (point, level)
            if (table_dtype == 0)
                fwd_generic_kernel<DD, FF, 0><<<grid, block, 0, stream>>>(x, n, table, dst, os, ls, lp);
            else
                fwd_generic_kernel<DD, FF, 1><<<grid, block, 0, stream>>>(x, n, table, dst, os, ls, lp);
        } else if (table_dtype == 0) {
            fwd_generic_pair_kernel<DD, FF, 0><<<grid, block, 0, stream>>>(x, n, table, dst, os, ls, lp);
        } else {
            fwd_generic_pair_kernel<DD, FF, 1><<<grid, block, 0, stream>>>(x, n, table, dst, os, ls, lp);
        }
    });
    if (!ok) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !stage) return e;
    return launch_transpose(F, stage, n, lp.n_levels, out, out_stride, stream);
}

hipError_t launch_backward_generic(const LaunchParams &lp, int D, int F, const float *x, int64_t n,
                                   const float *dout, int64_t dout_stride, float *dtable, hipStream_t stream) {
    const dim3 grid(grid_blocks(lp)), block(kBlock);
    const bool ok = dispatch_shape(D, F, [&]<int DD, int FF>() {
        bwd_generic_kernel<DD, FF><<<grid, block, 0, stream>>>(x, n, dout, dout_stride, dtable, lp);
    });
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_backward_dense(const LaunchParams &lp, const DenseLevels &dl, int D, int F, const float *x,
                                 int64_t n, const float *dout, int64_t dout_stride, float *dtable,
                                 hipStream_t stream) {
    if (dl.count == 0) return hipSuccess;
    if (dl.max_vals > kDenseVals) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + kDensePts - 1) / kDensePts), dl.count), block(kBlock);
    const size_t lds = (size_t)dl.max_vals * sizeof(unsigned long long);
    hipError_t e = hipSuccess;
    const bool ok = dispatch_shape(D, F, [&]<int DD, int FF>() {
        e = hipFuncSetAttribute((const void *)bwd_dense_kernel<DD, FF>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        if (e == hipSuccess)
            bwd_dense_kernel<DD, FF><<<grid, block, lds, stream>>>(x, n, dout, dout_stride, dtable, lp, dl);
    });
    if (!ok) return hipErrorInvalidValue;
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_debug_corners_generic(const LaunchParams &lp, int D, const float *x, int64_t n, uint32_t *idx,
                                        float *w, hipStream_t stream) {
    const dim3 grid((unsigned)((n + kBlock - 1) / kBlock), lp.n_levels), block(kBlock);
    const bool ok = dispatch_shape(D, 1, [&]<int DD, int FF>() {
        corners_generic_kernel<DD><<<grid, block, 0, stream>>>(x, n, idx, w, lp);
    });
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_input_grad(const LaunchParams &lp, int D, int F, const float *x, int64_t n, const void *table,
                             int table_dtype, const float *dout, int64_t dout_stride, float *dx, float *stage,
                             float *dlm, hipStream_t stream) {
    bool ok;
    if (D == 3 && F == 2) {  // lane pairs, as the forward
        if (stage) {
            const dim3 grid(grid_blocks(lp)), block(kBlock);
            const float *dl = dout;
            int64_t pstride = dout_stride, lstride = 2;
            if (dlm) {
                const unsigned blocks = (unsigned)((n + kRowPts - 1) / kRowPts);
                const size_t lds = (size_t)kRowPts * (2 * lp.n_levels + 4) * sizeof(float);
                const bool vec = n % 2 == 0 && lp.n_levels % 2 == 0 && dout_stride % 4 == 0 &&
                                 ((uintptr_t)dout & 15) == 0 && ((uintptr_t)dlm & 15) == 0;
                if (vec)
                    rows_to_levels_kernel<true><<<blocks, kBlock, lds, stream>>>(dout, dout_stride, n, lp.n_levels, dlm);
                else
                    rows_to_levels_kernel<false><<<blocks, kBlock, lds, stream>>>(dout, dout_stride, n, lp.n_levels, dlm);
                dl = dlm;
                pstride = 2;
                lstride = 2 * n;
            }
            if (table_dtype == 0)
                input_grad_pair_kernel<0, 4><<<grid, block, 0, stream>>>(x, n, table, dl, pstride, lstride, stage, lp);
            else
                input_grad_pair_kernel<1, 4><<<grid, block, 0, stream>>>(x, n, table, dl, pstride, lstride, stage, lp);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t nd = n * 3;
            input_grad_reduce_kernel<<<(unsigned)((nd + kBlock - 1) / kBlock), kBlock, 0, stream>>>(stage, nd,
                                                                                                 lp.n_levels, dx);
            return hipGetLastError();
        }
        const dim3 grid((unsigned)((n + kBlock - 1) / kBlock)), block(kBlock);
        if (table_dtype == 0)
            input_grad_point_pair_kernel<0><<<grid, block, 0, stream>>>(x, n, table, dout, dout_stride, dx, lp);
        else
            input_grad_point_pair_kernel<1><<<grid, block, 0, stream>>>(x, n, table, dout, dout_stride, dx, lp);
        return hipGetLastError();
    }
    // D <= 2: a level holds at most (N_l + 1)^2 corners, so the tables stay in
    // cache without level-major passes, and one thread walking its point's
    // levels beats staging (D1F2 23 vs 87 us, D2F2 72 vs 98 us at 2^18 points).
    if (stage && D >= 3) {
        const dim3 grid(grid_blocks(lp)), block(kBlock);
        ok = dispatch_shape(D, F, [&]<int DD, int FF>() {
            if (table_dtype == 0)
                input_grad_generic_pair_kernel<DD, FF, 0><<<grid, block, 0, stream>>>(x, n, table, dout,
                                                                                      dout_stride, stage, lp);
            else
                input_grad_generic_pair_kernel<DD, FF, 1><<<grid, block, 0, stream>>>(x, n, table, dout,
                                                                                      dout_stride, stage, lp);
        });
        if (!ok) return hipErrorInvalidValue;
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t nd = n * D;
        input_grad_reduce_kernel<<<(unsigned)((nd + kBlock - 1) / kBlock), kBlock, 0, stream>>>(stage, nd,
                                                                                             lp.n_levels, dx);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n + kBlock - 1) / kBlock)), block(kBlock);
    ok = dispatch_shape(D, F, [&]<int DD, int FF>() {
        if (table_dtype == 0)
            input_grad_point_kernel<DD, FF, 0><<<grid, block, 0, stream>>>(x, n, table, dout, dout_stride, dx, lp);
        else
            input_grad_point_kernel<DD, FF, 1><<<grid, block, 0, stream>>>(x, n, table, dout, dout_stride, dx, lp);
    });
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace hg
