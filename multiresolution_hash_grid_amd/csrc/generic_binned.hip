// Binned table backward of the other grid shapes (D in 1..4 inputs, F in
// {1, 2, 4, 8} features; jsqmd.com HashEncoding sections 3 and 4) for
// gfx950: the same method as the D = 3, F = 2 path of binned_backward.hip,
// with one record layout for every shape.
//
// Per (point, level) the 2^D corners form 2^(D-1) x-pairs: the two corners
// that differ only in the first coordinate, whose prime is 1, so their table
// indices differ in the low bits only (v_x XOR (v_x + 1) = 2^(t+1) - 1, t the
// trailing ones of v_x) and share a partition of 2^s entries unless that
// carry leaves the partition.  Each pair becomes a record
//   { x corner's index in the partition | t << 13,  f_x,  w_rest * g_0 ... w_rest * g_{F-1} }
// (2 + F words, fp32 values), w_rest being the product of the other
// coordinates' weights and g the level's upstream values.  bin counting-sorts
// a tile's records by partition in LDS and writes them contiguously with the
// run offsets; the shared accumulate kernel (binned_common.h) then adds each
// partition's runs into 64-bit fixed-point accumulators in LDS and the
// partition into the gradient.  A pair whose x+1 corner leaves the partition
// keeps its x corner (f_x = 0 in the record, weight folded in) and adds the
// x+1 corner with global atomics.
#include "binned_common.h"

namespace hg {
namespace {

using namespace binned;

constexpr int kGenThreads = 256;  // bin workgroup
// Accumulate workgroup width: 1024 threads (two per CU next to the 64 KB
// slices, 32 waves) where the kernel stays within 64 VGPRs (F <= 2); the
// F = 4 and F = 8 kernels need 70 and 92, so there 512 threads keep two
// workgroups per CU.  S * F / 4 = 2048 float4 either way.
constexpr int gen_acc_threads(int F) { return F <= 2 ? 1024 : 512; }

template <int F>
struct RecG {
    uint32_t head;  // x corner's index in the partition | t << 13
    float fx;
    float g[F];
};

template <int NF, int R>
struct GenPolicy {
    using Rec = RecG<NF>;
    static constexpr int F = NF;
    static constexpr int kRecPerTile = R;
    static __device__ __forceinline__ void apply(unsigned long long *slice, const Rec r, int k, uint32_t smask) {
        const uint32_t lo0 = r.head & 0x1FFFu, t = (r.head >> 13) & 0xFu;
        const uint32_t lo1 = lo0 ^ (((2u << t) - 1u) & smask);
        const float w0 = 1.f - r.fx;
#pragma unroll
        for (int j = 0; j < F; ++j) atomicAdd(slice + lo0 * F + j, to_fixed(w0 * r.g[j], k));
        if (r.fx != 0.f) {
#pragma unroll
            for (int j = 0; j < F; ++j) atomicAdd(slice + lo1 * F + j, to_fixed(r.fx * r.g[j], k));
        }
    }
};

// Workgroup (tile, level of the group).  Item i of the tile is corner pair
// i % 2^(D-1) of point i / 2^(D-1).
template <int D, int F>
__global__ __launch_bounds__(kGenThreads) void bin_generic_kernel(const float *__restrict__ x, int64_t n,
                                                                  const float *__restrict__ dout, int64_t dstride,
                                                                  BinParams bp, Space<RecG<F>> sp,
                                                                  float *__restrict__ grad) {
    constexpr int TILE = generic_tile(D, F), P = 1 << (D - 1), R = TILE * P;
    constexpr int kItems = (R + kGenThreads - 1) / kGenThreads;
    __shared__ RecG<F> stage[R];
    __shared__ uint32_t wmax[kGenThreads / 64];
    __shared__ uint32_t wsum[kGenThreads / 64];
    extern __shared__ uint32_t dyn[];  // cnt[parts], base[parts + 1]
    uint32_t *cnt = dyn;
    uint32_t *base = dyn + bp.parts;
    const int tile = blockIdx.x;
    const int g = blockIdx.y;
    const int l = bp.level0 + g;
    const float N = (float)bp.res[l];
    const uint32_t smask = (1u << bp.s_log2) - 1u;
    for (int i = threadIdx.x; i < bp.parts; i += kGenThreads) cnt[i] = 0;
    __syncthreads();
    RecG<F> rec[kItems];
    uint32_t part[kItems], rank[kItems];
    bool valid[kItems];
    float dm = 0.f;
    // A thread locates a point once and makes kPer of its P pairs: all of
    // them, for kPts points kGenThreads apart (kItems >= P), else kItems
    // consecutive pairs of one point.
    constexpr int kPts = kItems >= P ? kItems / P : 1, kPer = kItems >= P ? P : kItems;
    static_assert(kPts * kPer == kItems && R == kItems * kGenThreads, "items per thread");
#pragma unroll
    for (int ps = 0; ps < kPts; ++ps) {
        const int pi = kItems >= P ? ps * kGenThreads + (int)threadIdx.x : (int)threadIdx.x * kItems / P;
        const int c0 = kItems >= P ? 0 : (int)threadIdx.x * kItems % P;
        const int64_t p = (int64_t)tile * TILE + pi;
        const bool vp = p < n;
        const int64_t q = vp ? p : n - 1;  // in bounds; emits nothing
        int32_t vv[D];
        float ff[D];
#pragma unroll
        for (int d = 0; d < D; ++d) locate1(x[q * D + d], N, vv[d], ff[d]);
        float gv[F];
        bool fin = true;
#pragma unroll
        for (int j = 0; j < F; ++j) {
            gv[j] = dout[q * dstride + (int64_t)l * F + j];
            fin = fin && isfinite(gv[j]);
        }
        // A pair whose upstream values are not all finite (NaN, +-Inf) is not
        // binned: both corners go to the gradient with fp32 atomics, so NaN and
        // Inf reach the entries they touch, and the level's fixed-point scale
        // comes from the finite values only.
        if (vp && fin) {
#pragma unroll
            for (int j = 0; j < F; ++j) dm = fmaxf(dm, fabsf(gv[j]));
        }
        const int32_t v0 = vv[0];
        const float f0 = ff[0];
        const uint32_t cx0 = (uint32_t)v0;
#pragma unroll
        for (int cc = 0; cc < kPer; ++cc) {
            const int it = ps * kPer + cc, c = c0 + cc;
            float w_rest = 1.f;
            uint32_t K = 0;
#pragma unroll
            for (int d = 1; d < D; ++d) {
                const uint32_t up = (c >> (D - 1 - d)) & 1;
                K ^= ((uint32_t)vv[d] + up) * kPrimeList[d];
                w_rest *= up ? ff[d] : 1.f - ff[d];
            }
            const uint32_t i0 = (cx0 ^ K) & bp.mask, i1 = ((cx0 + 1u) ^ K) & bp.mask;
            part[it] = i0 >> bp.s_log2;
            valid[it] = vp;
            const uint64_t lbase = (uint64_t)l << bp.log2_table_size;  // level l's first entry
            if (vp && !fin) {
                grad_atomic_entry<F>(grad, bp.grad_f16, (lbase + i0) * F,
                                     [&](int j) { return (1.f - f0) * (w_rest * gv[j]); });
                grad_atomic_entry<F>(grad, bp.grad_f16, (lbase + i1) * F,
                                     [&](int j) { return f0 * (w_rest * gv[j]); });
                valid[it] = false;  // no record
            } else if ((i1 >> bp.s_log2) == part[it]) {
                const uint32_t t = min((uint32_t)__builtin_ctz(~cx0 | 0x80000000u), 15u);
                rec[it].head = (i0 & smask) | (t << 13);
                rec[it].fx = f0;
#pragma unroll
                for (int j = 0; j < F; ++j) rec[it].g[j] = w_rest * gv[j];
            } else {
                rec[it].head = i0 & smask;
                rec[it].fx = 0.f;
#pragma unroll
                for (int j = 0; j < F; ++j) rec[it].g[j] = (1.f - f0) * (w_rest * gv[j]);
                if (vp)
                    grad_atomic_entry<F>(grad, bp.grad_f16, (lbase + i1) * F,
                                         [&](int j) { return f0 * (w_rest * gv[j]); });
            }
            rank[it] = valid[it] ? atomicAdd(&cnt[part[it]], 1u) : 0u;
        }
    }
    for (int off = 32; off > 0; off >>= 1) dm = fmaxf(dm, __shfl_xor(dm, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = __float_as_uint(dm);
    __syncthreads();
    block_exclusive_scan<kGenThreads>(cnt, bp.parts, base, wsum);
    if (threadIdx.x == 0) {
        uint32_t m = wmax[0];
        for (int w = 1; w < kGenThreads / 64; ++w) m = max(m, wmax[w]);
        sp.dmax[(int64_t)g * bp.tiles + tile] = m;
    }
    __syncthreads();
    uint32_t *runs = sp.runs + ((int64_t)g * bp.tiles + tile) * (bp.parts + 1);
    for (int i = threadIdx.x; i <= bp.parts; i += kGenThreads) runs[i] = base[i];
#pragma unroll
    for (int it = 0; it < kItems; ++it)
        if (valid[it]) stage[base[part[it]] + rank[it]] = rec[it];
    __syncthreads();
    const uint32_t total = base[bp.parts];
    RecG<F> *trec = sp.records + (int64_t)g * bp.level_records + (int64_t)tile * R;
    for (uint32_t i = threadIdx.x; i < total; i += kGenThreads) trec[i] = stage[i];
}

template <int D, int F>
hipError_t launch_shape(BinParams bp, int n_levels, int max_group, const float *x, int64_t n, const float *dout,
                        int64_t dout_stride, float *dtable, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    constexpr int R = generic_rec_per_tile(D, F);
    if (bp.rec_per_tile != R || bp.rec_bytes != (int)sizeof(RecG<F>) || bp.tile_pts != generic_tile(D, F))
        return hipErrorInvalidValue;
    const size_t per_level = binned_level_bytes(bp);
    int group = (int)std::min<size_t>(workspace_bytes / per_level, (size_t)std::min(max_group, n_levels));
    if (group < 1) return hipErrorInvalidValue;
    const int ngroups = (n_levels + group - 1) / group;
    group = (n_levels + ngroups - 1) / ngroups;
    // The run counters of up to 4096 partitions (32 KB) next to a record stage
    // of up to 48 KB can pass the default 64 KB of LDS per workgroup.  One level per workgroup, in
    // tile order: the XCD-paired order of the standard bin kernel (bin_slot)
    // measured mixed here (D2F2, D3F4 faster; D4F2 17 % slower).
    const size_t dyn = (2 * (size_t)bp.parts + 1) * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute((const void *)bin_generic_kernel<D, F>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    for (int l0 = 0; l0 < n_levels; l0 += group) {
        bp.level0 = l0;
        bp.group = min(group, n_levels - l0);
        const Space<RecG<F>> sp = carve<RecG<F>>(workspace, bp);
        bin_generic_kernel<D, F><<<dim3(bp.tiles, bp.group), kGenThreads, dyn, stream>>>(x, n, dout, dout_stride, bp,
                                                                                   sp, dtable);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_accumulate<gen_acc_threads(F), GenPolicy<F, R>>(bp, sp, dtable, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
hipError_t launch_d(BinParams bp, int F, int n_levels, int max_group, const float *x, int64_t n, const float *dout,
                    int64_t ds, float *dt, void *ws, size_t wb, hipStream_t st) {
    switch (F) {
    case 1: return launch_shape<D, 1>(bp, n_levels, max_group, x, n, dout, ds, dt, ws, wb, st);
    case 2: return launch_shape<D, 2>(bp, n_levels, max_group, x, n, dout, ds, dt, ws, wb, st);
    case 4: return launch_shape<D, 4>(bp, n_levels, max_group, x, n, dout, ds, dt, ws, wb, st);
    case 8: return launch_shape<D, 8>(bp, n_levels, max_group, x, n, dout, ds, dt, ws, wb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_binned_backward_generic(BinParams bp, int D, int F, int n_levels, int max_group, const float *x,
                                          int64_t n, const float *dout, int64_t dout_stride, float *dtable,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    switch (D) {
    case 1: return launch_d<1>(bp, F, n_levels, max_group, x, n, dout, dout_stride, dtable, workspace, workspace_bytes, stream);
    case 2: return launch_d<2>(bp, F, n_levels, max_group, x, n, dout, dout_stride, dtable, workspace, workspace_bytes, stream);
    case 3: return launch_d<3>(bp, F, n_levels, max_group, x, n, dout, dout_stride, dtable, workspace, workspace_bytes, stream);
    case 4: return launch_d<4>(bp, F, n_levels, max_group, x, n, dout, dout_stride, dtable, workspace, workspace_bytes, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hg
