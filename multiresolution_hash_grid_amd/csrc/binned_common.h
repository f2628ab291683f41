// Shared pieces of the binned table backward (binned_backward.hip for the
// D = 3, F = 2 grid, generic_binned.hip for the other shapes): the workspace
// layout of a level group, block scans, the fixed-point helpers, and the
// accumulate kernel that walks one partition's runs in every tile.  The
// accumulate kernel is generic over a record policy P:
//   P::Rec                 the record type (4-byte aligned);
//   P::F                   features per table entry;
//   P::kRecPerTile         record slots of one tile;
//   P::apply(slice, r, k, smask)  adds one record into the LDS slice [S][F]
//                          of 64-bit fixed-point accumulators.
#pragma once

#include <algorithm>

#include "device_common.h"

namespace hg {
namespace binned {

// The gradient holds fp32 values, or binary16 values when bp.grad_f16 is set
// (the same element indices: element e of [L][T][F]).  The binned path adds to
// it directly only for the few contributions it does not bin (non-finite
// upstream values, x+1 corners outside their pair's partition, run sums past
// fp32); these helpers add them with atomics of the gradient's own type.  A
// binary16 atomic is a packed add of an aligned pair of halves: where only one
// half takes a value the other adds -0, which leaves every value as it is
// (-0 + -0 = -0, +0 + -0 = +0).
using Half2 = _Float16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void grad_atomic_half2(float *grad, uint64_t e_even, Half2 v) {
    __builtin_amdgcn_flat_atomic_fadd_v2f16(reinterpret_cast<Half2 *>(reinterpret_cast<_Float16 *>(grad) + e_even), v);
}
__device__ __forceinline__ void grad_atomic_add(float *grad, bool f16, uint64_t e, float v) {
    if (!f16) {
        unsafeAtomicAdd(grad + e, v);
        return;
    }
    const _Float16 h = (_Float16)v, z = (_Float16)-0.0f;
    grad_atomic_half2(grad, e & ~1ull, (e & 1) ? Half2{z, h} : Half2{h, z});
}
// Elements e and e + 1, e even.
__device__ __forceinline__ void grad_atomic_add2(float *grad, bool f16, uint64_t e, float a, float b) {
    if (!f16) {
        unsafeAtomicAdd(grad + e, a);
        unsafeAtomicAdd(grad + e + 1, b);
        return;
    }
    grad_atomic_half2(grad, e, Half2{(_Float16)a, (_Float16)b});
}
// The F values value(j) of the entry whose first element is e (e a multiple of F).
template <int F, class Fn>
__device__ __forceinline__ void grad_atomic_entry(float *grad, bool f16, uint64_t e, Fn value) {
    if constexpr (F == 1) {
        grad_atomic_add(grad, f16, e, value(0));
    } else {
#pragma unroll
        for (int j = 0; j < F; j += 2) grad_atomic_add2(grad, f16, e + j, value(j), value(j + 1));
    }
}

// Workspace of one launch group.
template <class Rec>
struct Space {
    Rec *records;       // [group][tiles][records per tile], each tile's records sorted by partition
    uint32_t *runs;     // [group][tiles][parts + 1], start of every partition's run in the tile
    uint32_t *dmax;     // [group][tiles], bits of each tile's max |dL/dout| (non-negative floats order as uints)
};

template <class Rec>
Space<Rec> carve(void *ws, const BinParams &bp) {
    Space<Rec> s;
    char *p = reinterpret_cast<char *>(ws);
    s.records = reinterpret_cast<Rec *>(p);
    p += (size_t)bp.group * bp.level_records * sizeof(Rec);
    s.runs = reinterpret_cast<uint32_t *>(p);
    p += (size_t)bp.group * bp.tiles * (bp.parts + 1) * sizeof(uint32_t);
    s.dmax = reinterpret_cast<uint32_t *>(p);
    return s;
}

// Bin workgroup -> (tile, block of levels).  The nb blocks of one tile read
// the same points and the same dout rows (each a slice of every row).
// Workgroups are dispatched to the XCDs round-robin, so workgroup ids w,
// w + 8, w + 16 ... run back to back on one XCD: giving a tile's blocks those
// ids lets the later blocks find the rows in that XCD's L2.
struct BinSlot {
    int tile, block;
};
__device__ __forceinline__ BinSlot bin_slot(int nb) {
    const int k = (int)(blockIdx.x / kNumXcd);
    return {(k / nb) * kNumXcd + (int)(blockIdx.x % kNumXcd), k % nb};
}
// Grid for bin_slot: tiles rounded up to a multiple of kNumXcd, nb blocks each
// (workgroups past the last tile return at once).  The standard grid's bin
// kernel uses it; the generic bin kernels keep a (tile, level) grid in tile
// order, where this order measured slower for some shapes.
inline unsigned bin_grid(int tiles, int nb) {
    return (unsigned)(((int64_t)tiles + kNumXcd - 1) / kNumXcd * kNumXcd * nb);
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

// Exclusive prefix of cnt[0..count) into base[0..count] (base[count] = total)
// by all THREADS threads: each thread sums a contiguous slice, the wave
// sums are combined through wsum, and every thread writes its slice.
template <int THREADS>
__device__ __forceinline__ void block_exclusive_scan(const uint32_t *cnt, int count, uint32_t *base,
                                                     uint32_t *wsum) {
    const int per = (count + THREADS - 1) / THREADS;
    const int b = per * threadIdx.x, e = min(count, b + per);
    uint32_t s = 0;
    for (int i = b; i < e; ++i) s += cnt[i];
    const uint32_t incl = wave_inclusive_scan(s);
    if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
    __syncthreads();
    uint32_t run = incl - s;
    for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) run += wsum[w];
    for (int i = b; i < e; ++i) {
        base[i] = run;
        run += cnt[i];
    }
    if (threadIdx.x == THREADS - 1) base[count] = run;
}

// c * 2^k rounded to nearest; |c * 2^k| < 2^31 by the choice of k.
__device__ __forceinline__ unsigned long long to_fixed(float c, int k) {
    return (unsigned long long)(long long)(int32_t)rintf(ldexpf(c, k));
}

// The same for |c * 2^k| < 2^39 (sums of up to 2^8 contributions): past 2^31
// the rounded value is an fp32 integer whose ulp is at least 2^8, so it is
// 2^8 times an integer below 2^31.
__device__ __forceinline__ unsigned long long to_fixed_wide(float c, int k) {
    const float v = rintf(ldexpf(c, k));
    if (fabsf(v) < 2147483648.f) return (unsigned long long)(long long)(int32_t)v;
    return (unsigned long long)((long long)(int32_t)(v * 0x1p-8f) * 256);
}

// Fixed-point exponent of a level: max|dL/dout| < 2^e  ->  k = 30 - e.
__device__ __forceinline__ int fixed_exponent(uint32_t dmax_bits) {
    const float m = __uint_as_float(dmax_bits);
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int e;
    frexpf(m, &e);  // m < 2^e
    return 30 - e;
}

// Workgroup (level, partition) of THREADS threads.  The tiles are walked in
// chunks of THREADS: lane i of wave w takes tile chunk + i * waves + w (the
// waves share out a short chunk evenly) and the wave works through the
// concatenation of its tiles' runs, 64 records per step.  The
// run that holds concatenation position i comes from a byte map built per
// window of kMapWindow positions: every run that starts inside the window
// marks its start with its lane index + 1, and a max-scan along the window
// spreads each mark to the positions up to the next start (0 stays where the
// run in progress when the window opened continues).  A record address is
// then two LDS reads away (map entry, run offset) instead of a search.  Two
// batches of kAccBatch steps are in flight: the next batch is requested
// before the current one is added.
constexpr int kAccBatch = 2;
// Consecutive (level, partition) slots an XCD takes at a time (accumulate_kernel).
constexpr uint32_t kAccXcdRun = 4;
// float4 gradient values per thread of a partition: S * F / 4 <= kFlushPer *
// THREADS for the partition size each workgroup width serves (launch_accumulate
// checks).
constexpr int kFlushPer = 4;
// A wave's run map holds PPL positions per lane: 16 (one uint4, windows of
// 1024 positions) or 8 (one uint2, windows of 512), a multiple of 64 *
// kAccBatch either way.
template <int PPL>
struct MapVec;
template <>
struct MapVec<16> {
    using T = uint4;
    static __device__ __forceinline__ void split(const T v, uint32_t (&w)[4]) { w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w; }
    static __device__ __forceinline__ T join(const uint32_t (&w)[4]) { return make_uint4(w[0], w[1], w[2], w[3]); }
};
template <>
struct MapVec<8> {
    using T = uint2;
    static __device__ __forceinline__ void split(const T v, uint32_t (&w)[2]) { w[0] = v.x, w[1] = v.y; }
    static __device__ __forceinline__ T join(const uint32_t (&w)[2]) { return make_uint2(w[0], w[1]); }
};

// LDS order between lanes of one wave (the wave's LDS operations complete in
// issue order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Byte map of window [w0, w0 + 64 PPL) of a wave's run concatenation; lane l
// owns bytes [l PPL, (l + 1) PPL).  pre / len: this lane's run offset and length.
template <int PPL>
__device__ __forceinline__ void build_run_map(typename MapVec<PPL>::T *map, uint32_t w0, uint32_t pre, uint32_t len) {
    using M = MapVec<PPL>;
    constexpr int W = PPL / 4;
    constexpr uint32_t kWindow = 64 * PPL;
    const int lane = threadIdx.x & 63;
    uint32_t w[W];
#pragma unroll
    for (int m = 0; m < W; ++m) w[m] = 0;
    map[lane] = M::join(w);
    wave_lds_fence();
    if (len > 0 && pre > w0 && pre < w0 + kWindow) reinterpret_cast<uint8_t *>(map)[pre - w0] = (uint8_t)(lane + 1);
    wave_lds_fence();
    M::split(map[lane], w);
    uint32_t run = 0;
    uint32_t loc[PPL];
#pragma unroll
    for (int b = 0; b < PPL; ++b) {
        run = max(run, (w[b >> 2] >> (8 * (b & 3))) & 0xFFu);
        loc[b] = run;
    }
    // Largest mark in the lanes below (the window positions before this lane's PPL).
    uint32_t incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off, 64);
        if (lane >= off) incl = max(incl, t);
    }
    uint32_t below = __shfl_up(incl, 1, 64);
    if (lane == 0) below = 0;
#pragma unroll
    for (int m = 0; m < W; ++m)
        w[m] = max(loc[4 * m], below) | (max(loc[4 * m + 1], below) << 8) | (max(loc[4 * m + 2], below) << 16) |
               (max(loc[4 * m + 3], below) << 24);
    map[lane] = M::join(w);
    wave_lds_fence();
}

// An empty use of a value's registers: the compiler waits here for the load
// that writes them.
template <class T>
__device__ __forceinline__ void hold_registers(const T &v) {
    static_assert(sizeof(T) % 4 == 0, "whole dwords");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"v"(w[i]));
}

template <int THREADS, class P>
__global__ __launch_bounds__(THREADS) void accumulate_kernel(BinParams bp, Space<typename P::Rec> sp,
                                                            float *__restrict__ grad) {
    using Rec = typename P::Rec;
    constexpr int F = P::F;
    constexpr int kRecPerTile = P::kRecPerTile;
    constexpr int kWaves = THREADS / 64;
    // 1024-thread workgroups keep their 16 maps at 512 B so that two fit a CU
    // next to 64 KB slices (32 waves per CU).
    constexpr int PPL = THREADS >= 1024 ? 8 : 16;
    constexpr uint32_t kMapWindow = 64 * PPL;
    static_assert(kMapWindow % (64 * kAccBatch) == 0, "map windows must hold whole batches");
    using MapT = typename MapVec<PPL>::T;
    extern __shared__ unsigned long long slice[];       // [2^s][F] fixed-point accumulators
    __shared__ int32_t offs[kWaves][64];                // per run: record index minus concatenation position
    __shared__ MapT maps[kWaves][64];                    // per wave: byte map of the current window
    __shared__ uint32_t touched;
    __shared__ uint32_t wmax[kWaves];
    // Workgroups reach the XCDs round-robin.  A tile's runs of neighbouring
    // partitions lie next to each other in the records and in the run table,
    // sharing cache lines, so each XCD takes kAccXcdRun consecutive
    // (level, partition) slots at a time: most shared lines are then fetched
    // into one L2, not two.  Longer stretches (a contiguous range per XCD)
    // leave the XCDs unevenly loaded, coarse levels having fewer records.
    const uint32_t nblocks = gridDim.x;
    const uint32_t kk = blockIdx.x / kNumXcd;
    const uint32_t slot = nblocks % (kNumXcd * kAccXcdRun)
                              ? blockIdx.x
                              : (kk / kAccXcdRun) * (kNumXcd * kAccXcdRun) + (blockIdx.x % kNumXcd) * kAccXcdRun +
                                    kk % kAccXcdRun;
    const int g = (int)(slot / (uint32_t)bp.parts);
    const int part = (int)slot - g * bp.parts;
    const int l = bp.level0 + g;
    const int S = 1 << bp.s_log2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t *truns = sp.runs + (int64_t)g * bp.tiles * (bp.parts + 1) + part;
    const int tl = lane * kWaves + wave;  // this lane's tile within a chunk
    // Run start and length of tile chunk + tl (0, 0 past the last tile).
    auto load_run = [&](int chunk, uint32_t &s, uint32_t &len) {
        s = len = 0;
        if (chunk + tl < bp.tiles) {
            const uint32_t *r = truns + (int64_t)(chunk + tl) * (bp.parts + 1);
            s = r[0];
            len = r[1] - s;
        }
    };
    uint32_t s_next, len_next;
    load_run(0, s_next, len_next);
    // The partition's entries [part * S, (part + 1) * S) of level l: only this
    // workgroup writes them.  They are read at the flush: holding them in
    // registers through the record loop (87 instead of 63 VGPRs) cost more
    // than the exposed read latency (standard backward 162 -> 158 us without).
    const uint64_t e0 = (((uint64_t)l << bp.log2_table_size) + (uint64_t)part * S) * F;  // first element
    for (int i = threadIdx.x; i < S * F; i += THREADS) slice[i] = 0ull;
    if (threadIdx.x == 0) touched = 0;
    // The level's max |dL/dout| over the tiles' maxima.
    uint32_t dm = 0;
    for (int t = threadIdx.x; t < bp.tiles; t += THREADS) dm = max(dm, sp.dmax[(int64_t)g * bp.tiles + t]);
    for (int off = 32; off > 0; off >>= 1) dm = max(dm, __shfl_xor(dm, off, 64));
    if (lane == 0) wmax[wave] = dm;
    const Rec *grec = sp.records + (int64_t)g * bp.level_records;
    const uint32_t smask = (uint32_t)S - 1u;
    MapT *map = maps[wave];
    const uint8_t *mapb = reinterpret_cast<const uint8_t *>(map);
    __syncthreads();
    dm = wmax[0];
    for (int w = 1; w < kWaves; ++w) dm = max(dm, wmax[w]);
    const int k = fixed_exponent(dm);
    for (int chunk = 0; chunk < bp.tiles; chunk += THREADS) {
        const uint32_t s = s_next, len = len_next;
        if (chunk + THREADS < bp.tiles) load_run(chunk + THREADS, s_next, len_next);
        const uint32_t incl = wave_inclusive_scan(len);
        const uint32_t pre = incl - len;
        // wave-uniform, and known to be: the record loop below is then scalar
        const uint32_t total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
        // Records of the chunk's tiles, relative to the first of them.
        const Rec *trec = grec + (int64_t)chunk * kRecPerTile;
        offs[wave][lane] = tl * kRecPerTile + (int32_t)s - (int32_t)pre;
        if (total && lane == 0) touched = 1;
        // Run holding position i (the window that holds i is in the map).
        uint32_t carry = 0;
        auto fetch = [&](uint32_t i) -> Rec {
            const uint32_t m = mapb[i % kMapWindow];
            const int j = m ? (int)m - 1 : (int)carry;
            return trec[offs[wave][j] + (int32_t)i];
        };
        auto open_window = [&](uint32_t w0) {
            // The run in progress at w0: the last run starting at or before it.
            carry = (uint32_t)__popcll(__ballot(pre <= w0)) - 1u;
            build_run_map<PPL>(map, w0, pre, len);
        };
        // Batches alternate between two register sets, so a batch's loads
        // stay in flight while the previous batch is added (copying the
        // next batch into the current one would wait for its loads).
        constexpr uint32_t kStep = 64 * kAccBatch;
        Rec ra[kAccBatch], rb[kAccBatch];
        auto request = [&](Rec(&r)[kAccBatch], uint32_t b) {
            // The batches in flight already have their addresses: the map may move on.
            if (b > 0 && b < total && b % kMapWindow == 0) open_window(b);
            // Every lane loads, also past the end (the last record again, to be
            // ignored), so the number of loads in flight is fixed and the adds
            // wait only for their own batch.
#pragma unroll
            for (int u = 0; u < kAccBatch; ++u) r[u] = fetch(min(b + u * 64 + lane, total - 1));
        };
        // Each record is marked as used before the lanes past the end are
        // masked off: a wait for its load inside a block the wave may skip
        // would leave the compiler unsure what is in flight, and it would
        // then wait for every load.
        auto add = [&](const Rec(&r)[kAccBatch], uint32_t b) {
#pragma unroll
            for (int u = 0; u < kAccBatch; ++u) {
                hold_registers(r[u]);
                if (b + u * 64 + lane < total) P::apply(slice, r[u], k, smask);
            }
        };
        if (total) {
            open_window(0);
            request(ra, 0);
            request(rb, kStep);
            for (uint32_t b0 = 0;; b0 += 2 * kStep) {
                add(ra, b0);
                if (b0 + kStep >= total) break;
                request(ra, b0 + 2 * kStep);
                add(rb, b0 + kStep);
                if (b0 + 2 * kStep >= total) break;
                request(rb, b0 + 3 * kStep);
            }
        }
        // The last batch requested is never added: wait for it here, so that
        // the next chunk's loop does not inherit loads in flight.
        __builtin_amdgcn_s_waitcnt(0);
        wave_lds_fence();
    }
    __syncthreads();
    if (!touched) return;  // no corner of this batch fell in the partition: nothing to add
    const long long *sl = reinterpret_cast<const long long *>(slice);
    auto sum = [&](int i) { return (float)ldexp((double)sl[i], -k); };
    if (bp.grad_f16) {
        // binary16: each value rounded once, from the fp32 sum of the old value
        // and the partition's sum.
        _Float16 *hbase = reinterpret_cast<_Float16 *>(grad) + e0;
        if (S * F < 4) {
            if (threadIdx.x < S * F) hbase[threadIdx.x] = (_Float16)((float)hbase[threadIdx.x] + sum(threadIdx.x));
            return;
        }
        using Half4 = _Float16 __attribute__((ext_vector_type(4)));
        Half4 *hl = reinterpret_cast<Half4 *>(hbase);
#pragma unroll
        for (int u = 0; u < kFlushPer; ++u) {
            const int j = threadIdx.x + u * THREADS;
            if (j >= S * F / 4) break;
            Half4 a = hl[j];
            a.x = (_Float16)((float)a.x + sum(4 * j + 0));
            a.y = (_Float16)((float)a.y + sum(4 * j + 1));
            a.z = (_Float16)((float)a.z + sum(4 * j + 2));
            a.w = (_Float16)((float)a.w + sum(4 * j + 3));
            hl[j] = a;
        }
        return;
    }
    float *gbase = grad + e0;
    if (S * F < 4) {  // a 2-entry table with one feature: two floats, less than a float4
        if (threadIdx.x < S * F) gbase[threadIdx.x] += sum(threadIdx.x);
        return;
    }
    float4 *gl = reinterpret_cast<float4 *>(gbase);
#pragma unroll
    for (int u = 0; u < kFlushPer; ++u) {
        const int j = threadIdx.x + u * THREADS;
        if (j >= S * F / 4) break;
        float4 a = gl[j];
        a.x += sum(4 * j + 0);
        a.y += sum(4 * j + 1);
        a.z += sum(4 * j + 2);
        a.w += sum(4 * j + 3);
        gl[j] = a;
    }
}

template <int THREADS, class P>
hipError_t launch_accumulate(const BinParams &bp, const Space<typename P::Rec> &sp, float *dtable,
                             hipStream_t stream) {
    const size_t lds = ((size_t)P::F << bp.s_log2) * sizeof(unsigned long long);
    if (((size_t)P::F << bp.s_log2) / 4 > (size_t)kFlushPer * THREADS) return hipErrorInvalidValue;
    // The partition slice can exceed the default 64 KB of dynamic LDS.
    hipError_t e = hipFuncSetAttribute((const void *)accumulate_kernel<THREADS, P>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    accumulate_kernel<THREADS, P><<<bp.group * bp.parts, THREADS, lds, stream>>>(bp, sp, dtable);
    return hipGetLastError();
}

}  // namespace binned
}  // namespace hg
