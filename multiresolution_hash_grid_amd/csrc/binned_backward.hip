// Binned backward of the hash-grid encoder for gfx950: the table gradient
// without global atomics on the hot path.
//
// The backward is the adjoint of the forward gather (ipipp.com section 2:
// only the corners a point sampled receive gradient): every point, level and
// corner adds w_corner * dL/dout into one table entry.  On MI355X a global
// atomic of any type is serviced at about one 64-byte request per clock per
// XCD (~20 G requests/s for the chip), and the random corners of a point give
// ~4 requests per (point, level), which bounds an atomic scatter near 1 ms for
// 2^18 points at L = 16.  Instead the work is routed to owners:
//
//   bin        : per (level, tile of 512 points), each corner pair (the two
//                x-corners of one (dy, dz), which share a table partition of
//                2^s entries unless x+1 carries above bit s) becomes a 16-byte
//                record {local index of both corners, f_x, w_y w_z g_0,
//                w_y w_z g_1}; the tile's 2048 records are counting-sorted by
//                partition in LDS and written contiguously to the tile's own
//                region together with the run offsets of every partition;
//   accumulate : one workgroup per (level, partition) gathers its run from
//                every tile, adds the records into the partition's gradient
//                held in LDS, then adds the partition into dtable with plain
//                coalesced loads and stores -- it is the only writer of those
//                entries.
//
// LDS accumulation is 64-bit fixed point: each contribution c is rounded to
// the integer nearest c * 2^k and added with ds_add_u64.  On this chip the
// LDS fp32 atomic add runs an order of magnitude slower than integer LDS
// atomics, and a compare-and-swap loop serialises on the many same-entry
// updates of coarse levels and ray-ordered points; integer adds are resolved
// by the LDS itself and are associative, so the binned gradient does not
// depend on the order of the additions.  k is chosen per level from
// max|dL/dout| < 2^e as k = 30 - e: every contribution (a weight <= 1 times an
// upstream value) then fits a signed 32-bit integer, the sum of n points'
// contributions to one entry stays below n * 2^30 < 2^63, and the rounding
// step is 2^-k < 2^-29 * max|dL/dout|.
//
// A corner pair whose x+1 corner lands in another partition (only when the
// low s bits of the x coordinate are all ones, e.g. x = -1) keeps the x
// corner in its record and adds the x+1 corner with a global fp32 atomic.
#include "hashgrid_internal.h"

namespace hg {
namespace {

constexpr int kBinThreads = 256;
constexpr int kPtsPerThread = kBinTile / kBinThreads;  // 2
constexpr int kRecPerTile = kBinTile * 4;              // 4 corner pairs per point
constexpr int kLevelsPerBlock = 4;                     // levels per bin workgroup
constexpr int kAccThreads = 1024;

// Workspace of one launch group.
struct Space {
    uint4 *records;     // [group][tiles][kRecPerTile], each tile sorted by partition
    uint32_t *runs;     // [group][tiles][parts + 1], start of every partition's run in the tile
    uint32_t *dmax;     // [group], bits of max |dL/dout| (non-negative floats order as uints)
};

Space carve(void *ws, const BinParams &bp) {
    Space s;
    char *p = reinterpret_cast<char *>(ws);
    s.records = reinterpret_cast<uint4 *>(p);
    p += (size_t)bp.group * bp.tiles * kRecPerTile * sizeof(uint4);
    s.runs = reinterpret_cast<uint32_t *>(p);
    p += (size_t)bp.group * bp.tiles * (bp.parts + 1) * sizeof(uint32_t);
    s.dmax = reinterpret_cast<uint32_t *>(p);
    return s;
}

__device__ __forceinline__ void locate1b(float xd, float N, int32_t &v, float &f) {
#pragma clang fp contract(off)
    float s = xd * N;
    float fl = floorf(s);
    v = (int32_t)fl;
    f = s - fl;
}

// The four corner pairs (dy, dz) of one point at one level.
struct Pairs {
    uint32_t part[4];
    uint4 rec[4];
    uint32_t split_idx[4];  // table entry of an x+1 corner outside the pair's partition, or ~0u
    float2 split_val[4];
    float dabs;             // max(|g_0|, |g_1|)
};

__device__ __forceinline__ void make_pairs(const float *__restrict__ x, const float *__restrict__ dout,
                                           int64_t dstride, int64_t p, int l, const BinParams &bp,
                                           Pairs &out) {
    const float N = (float)bp.res[l];
    int32_t v0, v1, v2;
    float a0, a1, a2;
    locate1b(x[3 * p + 0], N, v0, a0);
    locate1b(x[3 * p + 1], N, v1, a1);
    locate1b(x[3 * p + 2], N, v2, a2);
    const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hz0 = (uint32_t)v2 * kPrimeZ;
    const uint32_t cx0 = (uint32_t)v0, cx1 = cx0 + 1u;
    const uint32_t smask = (1u << bp.s_log2) - 1u;
    const float d0 = dout[p * dstride + 2 * l];
    const float d1 = dout[p * dstride + 2 * l + 1];
    out.dabs = fmaxf(fabsf(d0), fabsf(d1));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
        const uint32_t K = (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ);
        const uint32_t i0 = (cx0 ^ K) & bp.mask, i1 = (cx1 ^ K) & bp.mask;
        const uint32_t p0 = i0 >> bp.s_log2;
        const float wyz = (dy ? a1 : 1.f - a1) * (dz ? a2 : 1.f - a2);
        const float A = wyz * d0, B = wyz * d1;
        out.part[c] = p0;
        if ((i1 >> bp.s_log2) == p0) {
            out.rec[c] = make_uint4((i0 & smask) | ((i1 & smask) << 16), __float_as_uint(a0),
                                    __float_as_uint(A), __float_as_uint(B));
            out.split_idx[c] = ~0u;
            out.split_val[c] = make_float2(0.f, 0.f);
        } else {
            const float w0 = 1.f - a0;
            out.rec[c] = make_uint4((i0 & smask) | ((i0 & smask) << 16), 0u, __float_as_uint(w0 * A),
                                    __float_as_uint(w0 * B));
            out.split_idx[c] = i1;
            out.split_val[c] = make_float2(a0 * A, a0 * B);
        }
    }
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    return v;
}

// ---------------------------------------------------------------- init

__global__ void init_kernel(uint32_t *dmax, int group) {
    if ((int)threadIdx.x < group) dmax[threadIdx.x] = 0u;
}

// ---------------------------------------------------------------- bin

__global__ __launch_bounds__(kBinThreads) void bin_kernel(const float *__restrict__ x, int64_t n,
                                                          const float *__restrict__ dout, int64_t dstride,
                                                          BinParams bp, Space sp, float *__restrict__ grad) {
    __shared__ uint4 stage[kRecPerTile];
    __shared__ uint32_t wmax[kBinThreads / 64];
    extern __shared__ uint32_t dyn[];  // cnt[parts], base[parts + 1]
    uint32_t *cnt = dyn;
    uint32_t *base = dyn + bp.parts;
    const int tile = blockIdx.x;
    const int g_end = min(bp.group, (int)(blockIdx.y + 1) * kLevelsPerBlock);
    for (int g = blockIdx.y * kLevelsPerBlock; g < g_end; ++g) {
        const int l = bp.level0 + g;
        for (int i = threadIdx.x; i < bp.parts; i += kBinThreads) cnt[i] = 0;
        __syncthreads();
        Pairs pr[kPtsPerThread];
        uint32_t rank[kPtsPerThread][4];
        bool valid[kPtsPerThread];
        float dm = 0.f;
#pragma unroll
        for (int k = 0; k < kPtsPerThread; ++k) {
            const int64_t p = (int64_t)tile * kBinTile + k * kBinThreads + threadIdx.x;
            valid[k] = p < n;
            // Points past n recompute the last point (always initialised) and emit nothing.
            make_pairs(x, dout, dstride, valid[k] ? p : n - 1, l, bp, pr[k]);
            dm = fmaxf(dm, pr[k].dabs);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rank[k][c] = valid[k] ? atomicAdd(&cnt[pr[k].part[c]], 1u) : 0u;
                if (valid[k] && pr[k].split_idx[c] != ~0u) {
                    float *e = grad + (((uint64_t)l << bp.log2_table_size) + pr[k].split_idx[c]) * 2;
                    unsafeAtomicAdd(e, pr[k].split_val[c].x);
                    unsafeAtomicAdd(e + 1, pr[k].split_val[c].y);
                }
            }
        }
        for (int off = 32; off > 0; off >>= 1) dm = fmaxf(dm, __shfl_xor(dm, off, 64));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = __float_as_uint(dm);
        __syncthreads();
        // Run starts of the tile's partitions (wave 0), published for the owners.
        uint32_t *runs = sp.runs + ((int64_t)g * bp.tiles + tile) * (bp.parts + 1);
        if (threadIdx.x < 64) {
            const int per = (bp.parts + 63) / 64;
            const int b = per * threadIdx.x, e = min(bp.parts, b + per);
            uint32_t s = 0;
            for (int i = b; i < e; ++i) s += cnt[i];
            const uint32_t incl = wave_inclusive_scan(s);
            uint32_t run = incl - s;
            for (int i = b; i < e; ++i) {
                base[i] = run;
                runs[i] = run;
                run += cnt[i];
            }
            if (threadIdx.x == 63) {
                base[bp.parts] = incl;
                runs[bp.parts] = incl;
            }
            if (threadIdx.x == 0) {
                uint32_t m = wmax[0];
                for (int w = 1; w < kBinThreads / 64; ++w) m = max(m, wmax[w]);
                atomicMax(sp.dmax + g, m);
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPtsPerThread; ++k) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (valid[k]) stage[base[pr[k].part[c]] + rank[k][c]] = pr[k].rec[c];
            }
        }
        __syncthreads();
        const uint32_t total = base[bp.parts];
        uint4 *trec = sp.records + ((int64_t)g * bp.tiles + tile) * kRecPerTile;
        for (uint32_t i = threadIdx.x; i < total; i += kBinThreads) trec[i] = stage[i];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- accumulate

// c * 2^k rounded to nearest; |c * 2^k| < 2^31 by the choice of k.
__device__ __forceinline__ unsigned long long to_fixed(float c, int k) {
    return (unsigned long long)(long long)(int32_t)rintf(ldexpf(c, k));
}

__device__ __forceinline__ void apply_record(unsigned long long *slice, const uint4 r, int k) {
    const uint32_t lo0 = r.x & 0xFFFFu, lo1 = r.x >> 16;
    const float fx = __uint_as_float(r.y), A = __uint_as_float(r.z), B = __uint_as_float(r.w);
    const float w0 = 1.f - fx;
    atomicAdd(slice + 2 * lo0, to_fixed(w0 * A, k));
    atomicAdd(slice + 2 * lo0 + 1, to_fixed(w0 * B, k));
    if (fx != 0.f) {
        atomicAdd(slice + 2 * lo1, to_fixed(fx * A, k));
        atomicAdd(slice + 2 * lo1 + 1, to_fixed(fx * B, k));
    }
}

// Fixed-point exponent of a level: max|dL/dout| < 2^e  ->  k = 30 - e.
__device__ __forceinline__ int fixed_exponent(uint32_t dmax_bits) {
    const float m = __uint_as_float(dmax_bits);
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int e;
    frexpf(m, &e);  // m < 2^e
    return 30 - e;
}

// Workgroup (level, partition).  The tiles are walked in chunks of 1024:
// wave w takes tiles chunk + w + 16 i (lane i), scans its lanes' run lengths
// and then works through the concatenation of those runs, 64 records per
// step and kAccBatch steps in flight, finding each record's tile by a binary
// search over the wave's 64 run offsets.
constexpr int kAccBatch = 4;
constexpr int kAccWaves = kAccThreads / 64;

__global__ __launch_bounds__(kAccThreads) void accumulate_kernel(BinParams bp, Space sp,
                                                                 float *__restrict__ grad) {
    extern __shared__ unsigned long long slice[];    // [2^s][2] fixed-point accumulators
    __shared__ uint32_t pre[kAccWaves][65];         // per wave: run offsets in the concatenation
    __shared__ uint32_t start[kAccWaves][64];       // per wave: run start inside each tile
    __shared__ uint32_t touched;
    const int g = blockIdx.x / bp.parts;
    const int part = blockIdx.x - g * bp.parts;
    const int l = bp.level0 + g;
    const int S = 1 << bp.s_log2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 2 * S; i += kAccThreads) slice[i] = 0ull;
    if (threadIdx.x == 0) touched = 0;
    const int k = fixed_exponent(sp.dmax[g]);
    const uint4 *grec = sp.records + (int64_t)g * bp.tiles * kRecPerTile;
    for (int chunk = 0; chunk < bp.tiles; chunk += kAccThreads) {
        const int t = chunk + wave + kAccWaves * lane;
        uint32_t s = 0, len = 0;
        if (t < bp.tiles) {
            const uint32_t *r = sp.runs + ((int64_t)g * bp.tiles + t) * (bp.parts + 1) + part;
            s = r[0];
            len = r[1] - s;
        }
        const uint32_t incl = wave_inclusive_scan(len);
        pre[wave][lane] = incl - len;
        start[wave][lane] = s;
        if (lane == 63) pre[wave][64] = incl;
        __syncthreads();
        const uint32_t total = pre[wave][64];
        if (total && lane == 0) touched = 1;
        const uint32_t *wp = pre[wave];
        for (uint32_t base = 0; base < total; base += 64 * kAccBatch) {
            uint4 q[kAccBatch];
            bool ok[kAccBatch];
#pragma unroll
            for (int u = 0; u < kAccBatch; ++u) {
                const uint32_t i = base + u * 64 + lane;
                ok[u] = i < total;
                int lo = 0;
                if (ok[u]) {
                    // last run j with pre[j] <= i
#pragma unroll
                    for (int step = 32; step > 0; step >>= 1)
                        if (wp[lo + step] <= i) lo += step;
                    const int64_t tile = chunk + wave + kAccWaves * lo;
                    q[u] = grec[tile * kRecPerTile + start[wave][lo] + (i - wp[lo])];
                }
            }
#pragma unroll
            for (int u = 0; u < kAccBatch; ++u)
                if (ok[u]) apply_record(slice, q[u], k);
        }
        __syncthreads();
    }
    if (!touched) return;  // no corner of this batch fell in the partition: nothing to add
    // The partition's entries are [part * S, (part + 1) * S) of level l.
    float4 *gl = reinterpret_cast<float4 *>(grad + ((((uint64_t)l << bp.log2_table_size) + (uint64_t)part * S) * 2));
    const long long *sl = reinterpret_cast<const long long *>(slice);
    for (int j = threadIdx.x; j < S / 2; j += kAccThreads) {
        float4 a = gl[j];
        a.x += (float)ldexp((double)sl[4 * j + 0], -k);
        a.y += (float)ldexp((double)sl[4 * j + 1], -k);
        a.z += (float)ldexp((double)sl[4 * j + 2], -k);
        a.w += (float)ldexp((double)sl[4 * j + 3], -k);
        gl[j] = a;
    }
}

}  // namespace

size_t binned_level_bytes(const BinParams &bp) {
    const size_t recs = (size_t)bp.tiles * kRecPerTile * sizeof(uint4);
    const size_t words = (size_t)bp.tiles * (bp.parts + 1) + 1;
    return recs + words * sizeof(uint32_t);
}

hipError_t launch_binned_backward(BinParams bp, int n_levels, const float *x, int64_t n,
                                  const float *dout, int64_t dout_stride, float *dtable,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const size_t per_level = binned_level_bytes(bp);
    int group = (int)(workspace_bytes / per_level);
    if (group > n_levels) group = n_levels;
    if (group < 1) return hipErrorInvalidValue;
    const size_t acc_lds = ((size_t)2 << bp.s_log2) * sizeof(unsigned long long);
    // The partition slice can exceed the default 64 KB of dynamic LDS.
    hipError_t e = hipFuncSetAttribute((const void *)accumulate_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)acc_lds);
    if (e != hipSuccess) return e;
    for (int l0 = 0; l0 < n_levels; l0 += group) {
        bp.level0 = l0;
        bp.group = min(group, n_levels - l0);
        const Space sp = carve(workspace, bp);
        init_kernel<<<1, 64, 0, stream>>>(sp.dmax, bp.group);
        const dim3 tgrid(bp.tiles, (bp.group + kLevelsPerBlock - 1) / kLevelsPerBlock);
        bin_kernel<<<tgrid, kBinThreads, (2 * bp.parts + 1) * sizeof(uint32_t), stream>>>(x, n, dout, dout_stride,
                                                                                         bp, sp, dtable);
        accumulate_kernel<<<bp.group * bp.parts, kAccThreads, acc_lds, stream>>>(bp, sp, dtable);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hg
