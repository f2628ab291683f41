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
//   bin        : per (level, tile of 1024 points), each corner pair (the two
//                x-corners of one (dy, dz), which share a table partition of
//                2^s entries unless x+1 carries above bit s) becomes a 12-byte
//                record {local index of the x corner, the x+1 corner's offset
//                code, f_x, w_y w_z g_0, w_y w_z g_1}; the tile's 4096 records
//                are counting-sorted by partition in LDS and written
//                contiguously to the tile's own region together with the run
//                offsets of every partition;
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
//
// Record packing (three 32-bit words; the records are three quarters of the
// backward's memory traffic, written once and read once):
//   words 0, 1   w_y w_z g_0 and w_y w_z g_1, each an fp32 value rounded to
//                nearest on its 4 lowest mantissa bits (relative error
//                <= 2^-21, far inside the gradient's 1e-5 bound); the freed
//                low 4 bits hold bits 0..3 (word 0) and 4..7 (word 1) of f_x;
//   word 2       bits 0..14 bits 8..22 of f_x * 2^23, bits 15..27 lo0, bits
//                28..31 t, where
//     f_x * 2^23 is exact, as f_x is a multiple of the ulp of the fp32
//                position, >= 2^-23 once the position is >= 1 (below 1, i.e.
//                in the first voxel, it is rounded to 2^-24);
//     lo0        is the x corner's index inside the partition (s <= 13);
//     t          = min(trailing ones of v_x, 14): the x+1 corner's index is
//                lo0 XOR (2^(t+1) - 1) within the partition, because
//                v_x XOR (v_x + 1) = 2^(t+1) - 1 and the x prime is 1 (the
//                cap is exact as partitions have at most 2^13 entries).
// t = 15 marks a single-corner record instead: words 0 and 1 are its two
// fp32 sums, unrounded, and word 2 holds only lo0 and t.  Each field is one
// or two instructions to pack and to unpack.
//
// Wave pre-reduction: the 64 lanes of a wave hold 64 consecutive points.
// Where consecutive points fall in the same voxel of a level (coarse levels
// of ray-ordered batches, where a ray crosses one voxel in many samples), the
// run of lanes shares all 8 corners: a segmented scan across the wave adds
// the run's 16 corner contributions (8 corners x 2 features, in lane order),
// and the run's first and last lanes emit 4 single-corner records each in
// place of the run's 4 pair records per lane.  This cuts the records, and the
// same-entry LDS atomics in the owners, by the run length; a run of 2 breaks
// even.
#include <algorithm>

#include "binned_common.h"

namespace hg {
namespace {

using namespace binned;

constexpr int kBinThreads = kBinTile / 2;  // 512
constexpr int kPtsPerThread = kBinTile / kBinThreads;  // 2
constexpr int kRecPerTile = kBinTile * 4;              // 4 corner pairs per point
constexpr int kLevelsPerBlock = 4;                     // levels per bin workgroup (even)

// One corner-pair or single-corner record (see the packing above); 4-byte aligned, 12 bytes.
struct Rec12 {
    uint32_t a, b, c;
};
static_assert(sizeof(Rec12) == kRecordBytes, "records are 12 bytes");
using Rec = Rec12;
using StdSpace = binned::Space<Rec>;

// fp32 bits rounded to nearest on the 4 lowest mantissa bits, which then hold n.
__device__ __forceinline__ uint32_t round28(float v, uint32_t n) { return ((__float_as_uint(v) + 8u) & ~0xFu) | n; }

// A pair record; head = t << 28 | (f_x 2^23) >> 8, n0 / n1 = bits 0..3 / 4..7 of f_x 2^23.
__device__ __forceinline__ Rec pack_record(uint32_t lo0, uint32_t head, uint32_t n0, uint32_t n1, float A, float B) {
    return Rec{round28(A, n0), round28(B, n1), (lo0 << 15) | head};
}

constexpr uint32_t kSingle = 15u;  // t of a single-corner record

__device__ __forceinline__ Rec single_record(uint32_t lo, float A, float B) {
    return Rec{__float_as_uint(A), __float_as_uint(B), (kSingle << 28) | (lo << 15)};
}

// The records of one point at one level: the four corner pairs (dy, dz), or
// none or four single corners after the wave pre-reduction.
struct Pairs {
    uint32_t part[4];
    Rec rec[4];
    uint32_t nrec;          // 4 or 0 (0: not binned, or inside a pre-reduced run of lanes)
    float dabs;             // max(|g_0|, |g_1|)
};

// wbuf: this wave's 16 x 64 floats of LDS, free while the records are made.
// grad: the gradient [L][T][2] (fp32 or binary16, bp.grad_f16), which takes
// the contributions that are not binned (non-finite upstream values, x+1
// corners outside their pair's partition, non-finite run sums).
__device__ __forceinline__ void make_pairs(const float xp[3], float d0, float d1, int l, const BinParams &bp,
                                           bool valid, float *wbuf, float *__restrict__ grad, Pairs &out) {
    const uint64_t lbase = (uint64_t)l << bp.log2_table_size;  // level l's first entry
    const bool f16 = bp.grad_f16 != 0;
    const float N = (float)bp.res[l];
    int32_t v0, v1, v2;
    float a0, a1, a2;
    locate1(xp[0], N, v0, a0);
    locate1(xp[1], N, v1, a1);
    locate1(xp[2], N, v2, a2);
    const uint32_t hy0 = (uint32_t)v1 * kPrimeY, hz0 = (uint32_t)v2 * kPrimeZ;
    const uint32_t cx0 = (uint32_t)v0, cx1 = cx0 + 1u;
    const uint32_t smask = (1u << bp.s_log2) - 1u;
    // A point whose upstream values are not both finite (NaN, +-Inf) is not
    // binned: its 16 contributions go to the gradient with fp32 atomics, so
    // NaN and Inf reach the entries they touch as IEEE arithmetic has them,
    // and the level's fixed-point scale comes from the finite values only.
    const bool fin = isfinite(d0) && isfinite(d1);
    out.dabs = fin ? fmaxf(fabsf(d0), fabsf(d1)) : 0.f;
    out.nrec = valid && fin ? 4u : 0u;
    // trailing ones of v_x (bit 31 set keeps ctz defined for v_x = -1)
    const uint32_t t = min((uint32_t)__builtin_ctz(~cx0 | 0x80000000u), 14u);
    // f_x * 2^23 (exact for positions >= 1; the first voxel's fraction rounds)
    const uint32_t fx23 = min(__float2uint_rn(a0 * 8388608.f), 8388607u);
    const uint32_t head = (t << 28) | (fx23 >> 8), n0 = fx23 & 0xFu, n1 = (fx23 >> 4) & 0xFu;
    const float wx0 = 1.f - a0;
    uint32_t splits = 0;  // bit c: pair c's x+1 corner lies outside its partition
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
        const uint32_t K = (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ);
        const uint32_t i0 = (cx0 ^ K) & bp.mask, i1 = (cx1 ^ K) & bp.mask;
        const uint32_t p0 = i0 >> bp.s_log2;
        const float wyz = (dy ? a1 : 1.f - a1) * (dz ? a2 : 1.f - a2);
        const float A = wyz * d0, B = wyz * d1;
        out.part[c] = p0;
        // Branch-free: a pair whose x+1 corner lies in another partition keeps
        // only its x corner, with f_x = 0 and the weight 1 - f_x folded in
        // (times 1 is exact, so the pair values are A and B themselves).
        const bool split = (i1 >> bp.s_log2) != p0;
        const float s = split ? wx0 : 1.f;
        out.rec[c] = pack_record(i0 & smask, split ? 0u : head, split ? 0u : n0, split ? 0u : n1, s * A, s * B);
        splits |= split ? 1u << c : 0u;
    }
    if (!(valid && fin)) splits = 0;
    if (valid && !fin) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
            const uint32_t K = (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ);
            const uint32_t i0 = (cx0 ^ K) & bp.mask, i1 = (cx1 ^ K) & bp.mask;
            const float wyz = (dy ? a1 : 1.f - a1) * (dz ? a2 : 1.f - a2);
            const float A = wyz * d0, B = wyz * d1;
            grad_atomic_add2(grad, f16, (lbase + i0) * 2, wx0 * A, wx0 * B);
            grad_atomic_add2(grad, f16, (lbase + i1) * 2, a0 * A, a0 * B);
        }
    }
    // The x+1 corners outside their pair's partition, added with atomics by a
    // lane that keeps its pair records (recomputed here rather than held in
    // registers across the wave pre-reduction).
    auto add_splits = [&]() {
        if (!splits) return;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (!((splits >> c) & 1u)) continue;
            const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
            const uint32_t K = (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ);
            const uint32_t i1 = (cx1 ^ K) & bp.mask;
            const float wyz = (dy ? a1 : 1.f - a1) * (dz ? a2 : 1.f - a2);
            const float A = wyz * d0, B = wyz * d1;
            grad_atomic_add2(grad, f16, (lbase + i1) * 2, a0 * A, a0 * B);
        }
    };
    // Wave pre-reduction of runs of consecutive lanes in one voxel.
    const int lane = threadIdx.x & 63;
    // Every lane takes part in the shifts (a short-circuited shift would read
    // inactive lanes).  DPP wave_shr:1: lane i reads lane i - 1's value, lane 0
    // keeps its own (it never continues a run).
    auto up1 = [](int32_t v) { return __builtin_amdgcn_update_dpp(v, v, 0x138, 0xF, 0xF, false); };
    const int32_t u0 = up1(v0), u1 = up1(v1), u2 = up1(v2);
    const int prev_fin = up1((int)fin);
    // Points with non-finite upstream values stay runs of one (they are not binned).
    const bool same = valid && fin && prev_fin && lane > 0 && u0 == v0 && u1 == v1 && u2 == v2;
    const uint64_t dup = __ballot(same);
    if (dup == 0) {  // wave-uniform: no two neighbouring points share a voxel
        add_splits();
        return;
    }
    const uint64_t heads = ~dup, tails = (heads >> 1) | (1ull << 63);
    const int start = 63 - __builtin_clzll(heads & ((2ull << lane) - 1ull));  // first lane of this lane's run
    const int end = __builtin_ctzll(tails & (~0ull << lane));                // last lane of this lane's run
    // Each lane parks its 16 corner contributions (corner (dx, c), c = 2 dy + dz,
    // feature j at wbuf[(8 dx + 2 c + j) * 64 + lane]); the run's first lane
    // sums the x corners over the run and its last lane the x+1 corners, in
    // lane order.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float wyz = ((c >> 1) ? a1 : 1.f - a1) * ((c & 1) ? a2 : 1.f - a2);
        const float w0 = (1.f - a0) * wyz, w1 = a0 * wyz;
        wbuf[(2 * c + 0) * 64 + lane] = w0 * d0;
        wbuf[(2 * c + 1) * 64 + lane] = w0 * d1;
        wbuf[(8 + 2 * c + 0) * 64 + lane] = w1 * d0;
        wbuf[(8 + 2 * c + 1) * 64 + lane] = w1 * d1;
    }
    wave_lds_fence();
    if (start == end) {  // a run of one lane keeps its pair records
        add_splits();
        return;
    }
    // A run of m >= 2 lanes emits 8 single-corner records in place of 4 m pair
    // records: 4 from its first lane, 4 from its last (the run sums hold the
    // x+1 corners, so no lane of the run adds them separately).
    const bool first = lane == start;
    out.nrec = first || lane == end ? 4u : 0u;
    if (!out.nrec) return;
    const float *src = wbuf + (first ? 0 : 8 * 64);
    float sum[4][2] = {};
    for (int i = start; i <= end; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sum[c][0] += src[(2 * c + 0) * 64 + i];
            sum[c][1] += src[(2 * c + 1) * 64 + i];
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t dy = (uint32_t)(c >> 1), dz = (uint32_t)(c & 1);
        const uint32_t K = (hy0 + dy * kPrimeY) ^ (hz0 + dz * kPrimeZ);
        const uint32_t i = ((first ? cx0 : cx1) ^ K) & bp.mask;
        out.part[c] = i >> bp.s_log2;
        if (isfinite(sum[c][0]) && isfinite(sum[c][1])) {
            out.rec[c] = single_record(i & smask, sum[c][0], sum[c][1]);
        } else {  // finite values whose sum overflows fp32: added as it is, the record adds zero
            grad_atomic_add2(grad, f16, (lbase + i) * 2, sum[c][0], sum[c][1]);
            out.rec[c] = single_record(i & smask, 0.f, 0.f);
        }
    }
}

// ---------------------------------------------------------------- loads

// The coordinates and the block's dL/dout of one thread's points, loaded once
// per workgroup (one 32-byte row segment per point when aligned).
struct TilePoints {
    float xs[kPtsPerThread][3];
    float dv[kPtsPerThread][kLevelsPerBlock][2];
    bool valid[kPtsPerThread];
};

template <bool kDout>
__device__ __forceinline__ void load_points(const float *__restrict__ x, int64_t n, const float *__restrict__ dout,
                                            int64_t dstride, int tile, int lfirst, int nlev, TilePoints &tp) {
    const bool vec = nlev == kLevelsPerBlock && (dstride & 3) == 0 &&
                     (((uintptr_t)(dout + 2 * lfirst)) & 15) == 0;
#pragma unroll
    for (int k = 0; k < kPtsPerThread; ++k) {
        const int64_t p = (int64_t)tile * kBinTile + k * kBinThreads + threadIdx.x;
        tp.valid[k] = p < n;
        // Points past n recompute the last point (always initialised) and emit nothing.
        const int64_t q = tp.valid[k] ? p : n - 1;
        tp.xs[k][0] = x[3 * q + 0];
        tp.xs[k][1] = x[3 * q + 1];
        tp.xs[k][2] = x[3 * q + 2];
        if (!kDout) continue;
        const float *drow = dout + q * dstride + 2 * lfirst;
        if (vec) {
#pragma unroll
            for (int h = 0; h < kLevelsPerBlock / 2; ++h) {
                const float4 a = *reinterpret_cast<const float4 *>(drow + 4 * h);
                tp.dv[k][2 * h][0] = a.x;
                tp.dv[k][2 * h][1] = a.y;
                tp.dv[k][2 * h + 1][0] = a.z;
                tp.dv[k][2 * h + 1][1] = a.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kLevelsPerBlock; ++j) {
                tp.dv[k][j][0] = j < nlev ? drow[2 * j] : 0.f;
                tp.dv[k][j][1] = j < nlev ? drow[2 * j + 1] : 0.f;
            }
        }
    }
}

// ---------------------------------------------------------------- bin

// Workgroup (tile, block of kLevelsPerBlock consecutive levels).
__global__ __launch_bounds__(kBinThreads) void bin_kernel(const float *__restrict__ x, int64_t n,
                                                          const float *__restrict__ dout, int64_t dstride,
                                                          BinParams bp, StdSpace sp, float *__restrict__ grad) {
    __shared__ uint32_t wmax[kBinThreads / 64];
    __shared__ uint32_t wsum[kBinThreads / 64];
    extern __shared__ uint32_t dyn[];  // stage[kRecPerTile] records, cnt[parts], base[parts + 1]
    Rec *stage = reinterpret_cast<Rec *>(dyn);
    uint32_t *cnt = dyn + kRecPerTile * (sizeof(Rec) / sizeof(uint32_t));
    uint32_t *base = cnt + bp.parts;
    const BinSlot slot = bin_slot((bp.group + kLevelsPerBlock - 1) / kLevelsPerBlock);
    if (slot.tile >= bp.tiles) return;
    const int tile = slot.tile;
    const int gb = slot.block * kLevelsPerBlock;
    const int nlev = min(bp.group - gb, kLevelsPerBlock);
    // Each wave copies its own slice of the sorted stage out to the records,
    // and its wave pre-reduction parks its values in that same slice: a wave
    // starts the next level while the others still copy theirs, with no
    // barrier between the levels (the next level's sorted writes into the
    // stage come after the barrier that follows every wave's counting).
    constexpr int kWaveRecs = kRecPerTile / (kBinThreads / 64);
    static_assert(16 * 64 * sizeof(float) <= kWaveRecs * sizeof(Rec), "wave slice too small");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float *wbuf = reinterpret_cast<float *>(stage + wave * kWaveRecs);
    TilePoints tp;
    load_points<true>(x, n, dout, dstride, tile, bp.level0 + gb, nlev, tp);
    for (int i = threadIdx.x; i < bp.parts; i += kBinThreads) cnt[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kLevelsPerBlock; ++j) {
        if (j >= nlev) break;
        const int g = gb + j;
        const int l = bp.level0 + g;
        Pairs pr[kPtsPerThread];
        uint32_t rank[kPtsPerThread][4];
        float dm = 0.f;
#pragma unroll
        for (int k = 0; k < kPtsPerThread; ++k) {
            make_pairs(tp.xs[k], tp.dv[k][j][0], tp.dv[k][j][1], l, bp, tp.valid[k], wbuf,
                       grad, pr[k]);
            if (tp.valid[k]) dm = fmaxf(dm, pr[k].dabs);
#pragma unroll
            for (int c = 0; c < 4; ++c) rank[k][c] = 0u;
            if (pr[k].nrec) {
#pragma unroll
                for (int c = 0; c < 4; ++c) rank[k][c] = atomicAdd(&cnt[pr[k].part[c]], 1u);
            }
        }
        for (int off = 32; off > 0; off >>= 1) dm = fmaxf(dm, __shfl_xor(dm, off, 64));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = __float_as_uint(dm);
        __syncthreads();
        // Run starts of the tile's partitions, published for the owners.
        block_exclusive_scan<kBinThreads>(cnt, bp.parts, base, wsum);
        if (threadIdx.x == 0) {
            uint32_t m = wmax[0];
            for (int w = 1; w < kBinThreads / 64; ++w) m = max(m, wmax[w]);
            sp.dmax[(int64_t)g * bp.tiles + tile] = m;
        }
        __syncthreads();
        uint32_t *runs = sp.runs + ((int64_t)g * bp.tiles + tile) * (bp.parts + 1);
        for (int i = threadIdx.x; i <= bp.parts; i += kBinThreads) runs[i] = base[i];
#pragma unroll
        for (int k = 0; k < kPtsPerThread; ++k) {
            if (pr[k].nrec) {
#pragma unroll
                for (int c = 0; c < 4; ++c) stage[base[pr[k].part[c]] + rank[k][c]] = pr[k].rec[c];
            }
        }
        // The scan has consumed the counts: clear them for the next level.
        for (int i = threadIdx.x; i < bp.parts; i += kBinThreads) cnt[i] = 0;
        __syncthreads();
        const uint32_t total = base[bp.parts];
        Rec *trec = sp.records + (int64_t)g * bp.level_records + (int64_t)tile * kRecPerTile;
        const uint32_t w0 = (uint32_t)(wave * kWaveRecs), w1 = min(total, w0 + (uint32_t)kWaveRecs);
        if (w1 > w0) {
            // The slice as 16-byte words (slices start at multiples of 16 bytes;
            // a record region is 16-byte aligned when the workspace is).
            const uint32_t words = (w1 - w0) * 3;  // dwords
            const uint32_t *src = reinterpret_cast<const uint32_t *>(stage + w0);
            uint32_t *dst = reinterpret_cast<uint32_t *>(trec + w0);
            uint32_t i = 0;
            if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                for (uint32_t q = lane; q < words / 4; q += 64)
                    reinterpret_cast<uint4 *>(dst)[q] = reinterpret_cast<const uint4 *>(src)[q];
                i = words & ~3u;
            }
            for (uint32_t q = i + lane; q < words; q += 64) dst[q] = src[q];
        }
    }
}

// ---------------------------------------------------------------- accumulate

// The records of this grid for the shared accumulate kernel.
struct StdPolicy {
    using Rec = Rec12;
    static constexpr int F = 2;
    static constexpr int kRecPerTile = kBinTile * 4;
    static __device__ __forceinline__ void apply(unsigned long long *slice, const Rec r, int k, uint32_t smask) {
        const uint32_t t = r.c >> 28, lo0 = (r.c >> 15) & 0x1FFFu;
        if (t == kSingle) {  // a pre-reduced run's corner: its sums may exceed max|dL/dout|
            atomicAdd(slice + 2 * lo0, to_fixed_wide(__uint_as_float(r.a), k));
            atomicAdd(slice + 2 * lo0 + 1, to_fixed_wide(__uint_as_float(r.b), k));
            return;
        }
        const uint32_t lo1 = lo0 ^ (((2u << t) - 1u) & smask);
        const uint32_t fx23 = ((r.c & 0x7FFFu) << 8) | ((r.b & 0xFu) << 4) | (r.a & 0xFu);
        const float fx = (float)fx23 * 0x1p-23f;  // exact: fx23 < 2^23
        const float A = __uint_as_float(r.a & ~0xFu), B = __uint_as_float(r.b & ~0xFu);
        const float w0 = 1.f - fx;
        atomicAdd(slice + 2 * lo0, to_fixed(w0 * A, k));
        atomicAdd(slice + 2 * lo0 + 1, to_fixed(w0 * B, k));
        if (fx != 0.f) {
            atomicAdd(slice + 2 * lo1, to_fixed(fx * A, k));
            atomicAdd(slice + 2 * lo1 + 1, to_fixed(fx * B, k));
        }
    }
};

}  // namespace

hipError_t launch_binned_backward(BinParams bp, int n_levels, int max_group, const float *x, int64_t n,
                                  const float *dout, int64_t dout_stride, float *dtable,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const size_t per_level = binned_level_bytes(bp);
    int group = (int)std::min<size_t>(workspace_bytes / per_level, (size_t)std::min(max_group, n_levels));
    if (group < 1) return hipErrorInvalidValue;
    // Equal groups: 16 levels in groups of at most 6 run as 6 + 5 + 5.
    const int ngroups = (n_levels + group - 1) / group;
    group = (n_levels + ngroups - 1) / ngroups;
    // the tile's record stage and the run counters (32 KB at 4096 partitions)
    const size_t dyn = (size_t)kRecPerTile * sizeof(Rec) + (2 * (size_t)bp.parts + 1) * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute((const void *)bin_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    for (int l0 = 0; l0 < n_levels; l0 += group) {
        bp.level0 = l0;
        bp.group = min(group, n_levels - l0);
        const StdSpace sp = carve<Rec>(workspace, bp);
        const dim3 tgrid(bin_grid(bp.tiles, (bp.group + kLevelsPerBlock - 1) / kLevelsPerBlock));
        bin_kernel<<<tgrid, kBinThreads, dyn, stream>>>(x, n, dout, dout_stride, bp, sp, dtable);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        // 2^12- and 2^13-entry partitions: 1024 threads (16 waves) on one slice;
        // with 64 KB slices two workgroups share a CU, 32 waves to hide the
        // record loads.  Smaller partitions (short runs per tile): 256.
        if (bp.s_log2 >= 12) e = launch_accumulate<1024, StdPolicy>(bp, sp, dtable, stream);
        else e = launch_accumulate<256, StdPolicy>(bp, sp, dtable, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hg
