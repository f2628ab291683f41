// MLP head after the encoder, on the gfx950 matrix cores.
//
// The network is the NeRFace head of ipipp.com (section 3 listing):
// Linear(32, 64), ReLU, Linear(64, 64), ReLU, Linear(64, 4), biases on,
//   y = W3 relu(W2 relu(W1 e + b1) + b2) + b3,
// e being the 32 encoded features (L = 16 levels x F = 2) of a point.  It is
// a dense contraction, so it runs on the matrix cores: binary16 operands,
// fp32 accumulation.  The contractions over features and units (K = 32 and
// 64) use gfx950's v_mfma_f32_16x16x32_f16, and so do the weight gradients,
// which contract over 32 points at a time; dz2 = W3^T dL/dy (K = 4 outputs)
// takes one v_mfma_f32_16x16x16f16 per 16 units.
//
// Layout.  For D[i][j] = sum_k A[i][k] B[k][j] (16 x 16 x 16), lane l of the
// wave holds A[l%16][4(l/16) + r], B[4(l/16) + r][l%16] and
// D[4(l/16) + r][l%16], r = 0..3.  The kernels put the weights in A (rows =
// output units) and 16 points in the columns of B and D; then the D of one
// layer, rounded to binary16, is already the B operand of the next layer (the
// four rows a lane holds are the four k a lane supplies), so activations go
// from layer to layer in registers.  The 16 x 16 x 32 shape takes eight k
// per lane in A and B alike and the same D layout, and a contraction does not
// depend on which k sits in which slot as long as A and B agree: a lane
// supplies the k of two 16 x 16 x 16 operands, k-block 2h in slots 0..3 and
// 2h + 1 in slots 4..7, and the weights are loaded in that order.
//
// Forward: the encoder's gather writes the encoding level-major as binary16
// ([L][n][2], one 64-byte read per point here instead of a 128-byte fp32
// row), and each wave runs the three layers on 16 points at a time.  The
// stage is kept for the backward.
//
// Backward: each wave recomputes z1, h1, z2, h2 from the stage, takes
// dL/dy to dz2 = (W3^T g) * [z2 > 0], dz1 = (W2^T dz2) * [z1 > 0] and
// dL/de = W1^T dz1 with the transposed weights in A, and writes dL/de as
// the fp32 upstream rows of the encoder's table backward.  dL/dy enters the
// matrix cores scaled by one power of two s per call, chosen so that the
// largest finite |dL/dy| lands in [1, 2): a loss averaged over millions of
// points gives dL/dy ~ 1e-7, which unscaled would sit at binary16's
// subnormal floor.  dz2 and dz1 carry the scale; dL/de and the weight and
// bias gradients are multiplied by 1/s in fp32, which is exact.  The weight
// gradients contract over points (dW2 = dz2 h1^T etc.), so the activations of
// a workgroup's 64 points go through LDS, transposed, to put the points on
// the k axis, and the four waves split the weight gradients between them:
// each keeps a quarter of the running dW and db in registers (two waves then
// fit a SIMD) and writes it once per workgroup, and two reduction kernels
// add the workgroups' partials, in a fixed order, into the caller's fp32
// gradients.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "device_common.h"

namespace hg {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kIn = 32, kHid = 64, kOut = 4;  // kIn: the encoding's features
constexpr int kMlpWaves = 4;  // waves per workgroup
// Per-workgroup partial sums: dW1's encoding columns [64][32], db1 [64], dW2
// [64][64], db2 [64], dW3 [4][64], db3 [4], then (with coordinate inputs)
// dW1's coordinate columns [64][3].
constexpr int kOffW1 = 0, kOffB1 = kOffW1 + kHid * kIn, kOffW2 = kOffB1 + kHid, kOffB2 = kOffW2 + kHid * kHid,
              kOffW3 = kOffB2 + kHid, kOffB3 = kOffW3 + kOut * kHid, kOffW1x = kOffB3 + kOut,
              kPartial = kOffW1x + kHid * kMlpCoords;
// Partial entries a head writes: the coordinate columns only with coordinate inputs.
constexpr int partial_count(int coords) { return coords ? kPartial : kOffW1x; }

__device__ __forceinline__ float4_t mfma(half4_t a, half4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma32(half8_t a, half8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two 16 x 16 x 16 operands as one 16 x 16 x 32 operand: lo in slots 0..3, hi in 4..7.
__device__ __forceinline__ half8_t join8(half4_t lo, half4_t hi) {
    return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half4_t to_half4(float4_t v) {
    const half2_t lo = __builtin_convertvector(float2_t{v[0], v[1]}, half2_t);
    const half2_t hi = __builtin_convertvector(float2_t{v[2], v[3]}, half2_t);
    return half4_t{lo[0], lo[1], hi[0], hi[1]};
}

// ReLU of fp32 pre-activations, rounded to binary16 (to nearest even).  A
// unit whose input is not > 0 (NaN included) gets -0 rather than +0: the
// same value in every product, while the sign bit keeps the ReLU's decision
// for the backward (an input in (0, 2^-25) rounds to +0 and still passes the
// gradient, as [z > 0] has it).
__device__ __forceinline__ half4_t relu_half(float4_t v) {
    float4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i] > 0.f ? v[i] : -0.f;
    return to_half4(r);
}

// dL/dz of four units: the fp32 sums v rounded to binary16 where the unit's
// activation h has a clear sign bit (the ReLU passed), +0 elsewhere.
__device__ __forceinline__ half4_t relu_grad(float4_t v, half4_t h) {
    typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));
    const uint2_t g = __builtin_bit_cast(uint2_t, to_half4(v));
    const uint2_t hb = __builtin_bit_cast(uint2_t, h);
    // 0xFFFF in each half whose sign bit is set (the vector elements are
    // copied to scalars first: clang bit-casts an element operand of
    // __builtin_bit_cast from the wrong element)
    const uint32_t h0 = hb[0], h1 = hb[1];
    const uint32_t blo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2_t, h0) >> (short)15);
    const uint32_t bhi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2_t, h1) >> (short)15);
    return __builtin_bit_cast(half4_t, uint2_t{g[0] & ~blo, g[1] & ~bhi});
}

// The forward weights as 16 x 16 x 32 A operands: row = output unit, slot
// s of lane group q = input k-block 2h + s / 4, k = 16 (2h + s / 4) + 4 q + s % 4.
// With XIN coordinate inputs, W1's coordinate columns form one more A
// operand per 16 units, non-zero only in lane group q = 0's first XIN slots
// (k = 0 .. XIN - 1).
struct FwdWeights {
    half8_t a1[4], a2[4][2], a3[2];
    half4_t a1x[4];
    float4_t b1[4], b2[4], b3;
};

template <int XIN>
__device__ __forceinline__ void load_fwd_weights(const MlpParams &mp, int q, int c, FwdWeights &w) {
    constexpr int ld = kIn + XIN;  // W1's row: XIN coordinates, then the encoding
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w.a1x[mb][r] = XIN && 4 * q + r < XIN ? mp.w1[(16 * mb + c) * ld + 4 * q + r] : (_Float16)0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int kk = 16 * (s >> 2) + 4 * q + (s & 3);  // k within a 32-wide block
            w.a1[mb][s] = mp.w1[(16 * mb + c) * ld + XIN + kk];
#pragma unroll
            for (int h = 0; h < 2; ++h) w.a2[mb][h][s] = mp.w2[(16 * mb + c) * kHid + 32 * h + kk];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w.b1[mb][r] = mp.b1[16 * mb + 4 * q + r];
            w.b2[mb][r] = mp.b2[16 * mb + 4 * q + r];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s = 0; s < 8; ++s)
            w.a3[h][s] = c < kOut ? mp.w3[c * kHid + 32 * h + 16 * (s >> 2) + 4 * q + (s & 3)] : (_Float16)0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) w.b3[r] = q == 0 ? mp.b3[r] : 0.f;
}

// The encoding of point p as the two B operands of layer 1: k = 16 kb + 4 q + r
// is feature r % 2 of level 8 kb + 2 q + r / 2.
__device__ __forceinline__ void load_encoding(const _Float16 *__restrict__ stage, int64_t n, int64_t p, int q,
                                              half4_t (&eb)[2]) {
    const uint32_t *s = reinterpret_cast<const uint32_t *>(stage);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int l0 = 8 * kb + 2 * q;
        const uint32_t a = s[(int64_t)l0 * n + p], b = s[(int64_t)(l0 + 1) * n + p];
        eb[kb][0] = __builtin_bit_cast(_Float16, (uint16_t)(a & 0xFFFFu));
        eb[kb][1] = __builtin_bit_cast(_Float16, (uint16_t)(a >> 16));
        eb[kb][2] = __builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
        eb[kb][3] = __builtin_bit_cast(_Float16, (uint16_t)(b >> 16));
    }
}

// The point's coordinates as the B operand of W1's coordinate columns:
// lane (q, c) holds x[p][4 q + r] for 4 q + r < XIN, zero elsewhere (binary16).
template <int XIN>
__device__ __forceinline__ half4_t coord_operand(const float (&xc)[kMlpCoords], int q) {
    half4_t b = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < XIN; ++r) b[r] = q == 0 ? (_Float16)xc[r] : (_Float16)0.f;
    return b;
}

// The coordinates of point p (XIN of them; lanes of group q = 0 only).
template <int XIN>
__device__ __forceinline__ void load_coords(const float *__restrict__ x, int64_t p, int q, float (&xc)[kMlpCoords]) {
#pragma unroll
    for (int r = 0; r < kMlpCoords; ++r) xc[r] = 0.f;
    if (XIN && q == 0) {
#pragma unroll
        for (int r = 0; r < XIN; ++r) xc[r] = x[3 * p + r];
    }
}

// Layers 1 and 2 of 16 points: binary16 activations, -0 where the ReLU blocked.
template <int XIN>
__device__ __forceinline__ void hidden_layers(const FwdWeights &w, const half4_t (&eb)[2], half4_t xb,
                                              half4_t (&h1)[4], half4_t (&h2)[4]) {
    const half8_t e8 = join8(eb[0], eb[1]);
    // The coordinate term accumulates onto the encoding's with the same
    // 16 x 16 x 32 shape: only lane group 0's first XIN k-slots are non-zero,
    // and they are k = 0 .. XIN - 1 in either shape's layout.  (Chained onto a
    // 16 x 16 x 32 result as a 16 x 16 x 16 MFMA, it read that result before
    // it was complete where the compiler issued the two seven instructions
    // apart.)
    const half4_t zh = {0, 0, 0, 0};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        float4_t z = mfma32(w.a1[mb], e8, w.b1[mb]);
        if constexpr (XIN) z = mfma32(join8(w.a1x[mb], zh), join8(xb, zh), z);
        h1[mb] = relu_half(z);
    }
    const half8_t h1lo = join8(h1[0], h1[1]), h1hi = join8(h1[2], h1[3]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) h2[mb] = relu_half(mfma32(w.a2[mb][1], h1hi, mfma32(w.a2[mb][0], h1lo, w.b2[mb])));
}

// Slices of dL/dy whose largest finite magnitude mlp_dy_max_kernel writes.
constexpr int kDyMaxParts = 1024;

__device__ __forceinline__ float finite_abs_max(float m, float v) {
    const float a = fabsf(v);
    return a <= 3.40282347e38f ? fmaxf(m, a) : m;  // NaN and Inf fail the comparison
}

// parts[b]: bits of the largest finite |dy| over the float4 rows b, b + grid, ...
__global__ __launch_bounds__(256) void mlp_dy_max_kernel(const float4 *__restrict__ dy, int64_t n,
                                                         uint32_t *__restrict__ parts) {
    __shared__ float wmax[4];
    float m = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)kDyMaxParts * 256) {
        const float4 v = dy[i];
        m = finite_abs_max(finite_abs_max(finite_abs_max(finite_abs_max(m, v.x), v.y), v.z), v.w);
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) parts[blockIdx.x] = __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
}

// Persistent grids: as many workgroups as the chip holds at once (the
// kernel's occupancy times the CU count, found once per device and kernel),
// so that no round of workgroups runs alone at the end; never more than the
// 16-point tiles need.  1024 workgroups when the occupancy query fails.
int resident_workgroups(const void *kernel, size_t lds_bytes) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1024;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end()) return it->second;
    int per_cu = 0, cus = 0;
    int r = 1024;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kMlpWaves, lds_bytes) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0 &&
        cus > 0)
        r = per_cu * cus;
    cache[{dev, kernel}] = r;
    return r;
}

constexpr int kMaxMlpGrid = 1024;  // the partials workspace is sized for this many workgroups

int mlp_grid(int64_t tiles, const void *kernel, size_t lds_bytes = 0) {
    const int64_t want = (tiles + kMlpWaves - 1) / kMlpWaves;
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, (int64_t)resident_workgroups(kernel, lds_bytes), kMaxMlpGrid}));
}

// ---------------------------------------------------------------- forward

// Tiles whose encodings a forward wave has requested ahead of the one it
// works on.  With one tile ahead a wave had 1 KB of loads in flight and the
// kernel streamed the stage at about 3 TB/s, bound by load latency; the ring
// is walked in an unrolled loop, so each slot stays a register set of its own
// (copying a slot with a load in flight into another would wait for that load).
constexpr int kFwdAhead = 3;

template <int XIN>
__global__ __launch_bounds__(64 * kMlpWaves) void mlp_fwd_kernel(const _Float16 *__restrict__ stage,
                                                                 const float *__restrict__ x, int64_t n,
                                                                 MlpParams mp, float *__restrict__ y,
                                                                 int64_t tiles) {
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
    FwdWeights w;
    load_fwd_weights<XIN>(mp, q, c, w);
    const int64_t nwaves = (int64_t)gridDim.x * kMlpWaves;
    const int64_t t0 = (int64_t)blockIdx.x * kMlpWaves + (threadIdx.x >> 6);
    // Past the last tile a slot loads the last point again (its result is not used).
    half4_t ring[kFwdAhead][2];
    float ring_x[kFwdAhead][kMlpCoords];
    auto request = [&](int64_t t, int s) {
        const int64_t p = min(t * 16 + c, n - 1);
        load_encoding(stage, n, p, q, ring[s]);
        load_coords<XIN>(x, p, q, ring_x[s]);
    };
#pragma unroll
    for (int s = 0; s < kFwdAhead; ++s) request(t0 + s * nwaves, s);
    for (int64_t t = t0; t < tiles; t += kFwdAhead * nwaves) {
#pragma unroll
        for (int s = 0; s < kFwdAhead; ++s) {
            const int64_t ts = t + s * nwaves;
            if (ts >= tiles) break;  // wave-uniform
            const int64_t p = ts * 16 + c;
            half4_t h1[4], h2[4];
            hidden_layers<XIN>(w, ring[s], coord_operand<XIN>(ring_x[s], q), h1, h2);
            const float4_t o = mfma32(w.a3[1], join8(h2[2], h2[3]), mfma32(w.a3[0], join8(h2[0], h2[1]), w.b3));
            request(ts + kFwdAhead * nwaves, s);
            if (q == 0 && p < n) *reinterpret_cast<float4 *>(y + p * kOut) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
}

// ---------------------------------------------------------------- backward

// One workgroup's block of kBlockPts points for the weight gradients: the
// activations transposed, units as rows and the block's points as columns
// (binary16), so that an operand with the points on the k axis is two
// 8-byte LDS reads per lane.  Rows are padded to 136 bytes: the 16 rows a
// read or write touches then start 34 banks apart, and a half-wave's 8-byte
// accesses meet 64 distinct banks.
constexpr int kBlockPts = 16 * kMlpWaves;  // 64
constexpr int kRowH = kBlockPts + 4;       // halves per row
template <int XIN>
struct BlockLds {
    _Float16 e[kIn][kRowH];
    _Float16 h1[kHid][kRowH];
    _Float16 h2[kHid][kRowH];
    _Float16 dz1[kHid][kRowH];
    _Float16 dz2[kHid][kRowH];
    _Float16 g3[kOut][kRowH];               // dL/dy, scaled
    _Float16 x[XIN ? XIN : 1][kRowH];       // the coordinate inputs (XIN > 0)
};
// Two blocks: one barrier per block.
template <int XIN>
constexpr size_t bwd_lds() { return 2 * sizeof(BlockLds<XIN>); }

// A 16 x 16 block X that a wave holds in the D layout (lane (q, c) holds
// X[4 q + r][c], r = 0..3), transposed on the matrix cores: with X's
// registers as the A operand (A[i][k] = X[k][i]) and the identity as B, the
// product is X^T, so lane (q, c) then holds X[c][4 q + r].  Each sum has one
// non-zero term, so the binary16 values come back exactly.
__device__ __forceinline__ half4_t transpose16(half4_t x, half4_t ident) {
    return to_half4(mfma(x, ident, float4_t{0.f, 0.f, 0.f, 0.f}));
}

// X (units u0 .. u0 + 15 of this wave's 16 points, D layout) into rows
// u0 + c, columns col0 + 4 q .. + 3 of a block array.
__device__ __forceinline__ void put_cols(_Float16 (*dst)[kRowH], int u0, int q, int c, int col0, half4_t x,
                                         half4_t ident) {
    *reinterpret_cast<half4_t *>(&dst[u0 + c][col0 + 4 * q]) = transpose16(x, ident);
}

// A 16 x 16 x 32 operand with the points of half h of the block on the k
// axis (slots 0..3: points 32 h + 4 q + 0..3, slots 4..7: 16 further), row
// `row` of src on this lane.
__device__ __forceinline__ half8_t get_k(const _Float16 (*src)[kRowH], int row, int q, int h) {
    const half4_t lo = *reinterpret_cast<const half4_t *>(&src[row][32 * h + 4 * q]);
    const half4_t hi = *reinterpret_cast<const half4_t *>(&src[row][32 * h + 16 + 4 * q]);
    return join8(lo, hi);
}

// Each workgroup walks blocks of 64 points.  Wave w takes points 16 w + c of
// the block through the layers (recomputed forward, dz2, dz1, dL/de) and
// stores its tile's activations, transposed, in the block's LDS; after one
// barrier, wave w contracts the whole block over its points for its quarter
// of the weight gradients: rows 16 w .. 16 w + 15 of dW1 and dW2 (and of db1,
// db2), columns 16 w .. 16 w + 15 of dW3 (and db3 on wave 0).  The bias
// gradients are the same contractions against a ones operand.  The running
// sums of a wave are 40 registers instead of the whole head's 148, which
// lets two waves share a SIMD.  Each workgroup writes one set of partials.
// With XIN coordinate inputs the coordinates go through the first layer as
// one more operand, through the block's LDS like the encoding, and into
// dW1's coordinate columns (wave w's rows, XIN more sums); dL/de skips them.
// (The coordinate operands and sums do not fit two waves per SIMD: the
// TinyNeRF instantiation takes the whole register file of one.)
template <int XIN>
__global__ __launch_bounds__(64 * kMlpWaves, XIN ? 1 : 2) void mlp_bwd_kernel(const _Float16 *__restrict__ stage,
                                                                    const float *__restrict__ x, int64_t n,
                                                                    MlpParams mp, const float *__restrict__ dy,
                                                                    const uint32_t *__restrict__ dmax,
                                                                    float *__restrict__ de,
                                                                    float *__restrict__ partials) {
    extern __shared__ __align__(16) unsigned char mlp_lds[];
    BlockLds<XIN> *blk = reinterpret_cast<BlockLds<XIN> *>(mlp_lds);
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15, wave = threadIdx.x >> 6;
    // The call's scale s = 2^(1-e), max|dL/dy| in [2^(e-1), 2^e) (1 if dL/dy has no finite non-zero value).
    uint32_t mbits = 0;
    for (int i = lane; i < kDyMaxParts; i += 64) mbits = max(mbits, dmax[i]);
    for (int off = 32; off > 0; off >>= 1) mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, off, 64));
    float gscale = 1.f, ginv = 1.f;
    if (__uint_as_float(mbits) > 0.f) {
        int e;
        frexpf(__uint_as_float(mbits), &e);
        gscale = ldexpf(1.f, 1 - e);
        ginv = ldexpf(1.f, e - 1);
    }
    FwdWeights w;
    load_fwd_weights<XIN>(mp, q, c, w);
    // Transposed weights as A operands: row = input unit of the layer, k = its
    // output unit (t2, t1: 16 x 16 x 32 slots as the forward's; t3: K = 4
    // outputs padded to one 16 x 16 x 16 operand).
    half4_t t3[4];
    half8_t t2[4][2], t1[2][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t3[mb][r] = q == 0 ? mp.w3[r * kHid + 16 * mb + c] : (_Float16)0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int k = 32 * h + 16 * (s >> 2) + 4 * q + (s & 3);
                t2[mb][h][s] = mp.w2[k * kHid + 16 * mb + c];
                if (mb < 2) t1[mb][h][s] = mp.w1[k * (kIn + XIN) + XIN + 16 * mb + c];
            }
    }
    // B operands: the identity (k = 4 q + r against column c) and all ones.
    half4_t ident;
#pragma unroll
    for (int r = 0; r < 4; ++r) ident[r] = 4 * q + r == c ? (_Float16)1.f : (_Float16)0.f;
    const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t gw1[2], gw2[4], gw3, gb1 = zero4, gb2 = zero4, gb3 = zero4, gw1x = zero4;
    gw1[0] = gw1[1] = gw3 = zero4;
#pragma unroll
    for (int j = 0; j < 4; ++j) gw2[j] = zero4;
    const int64_t nblocks = (n + kBlockPts - 1) / kBlockPts;
    // The next block's encoding is requested before the current block is
    // worked on; dL/dy, needed after the two hidden layers, at its start.
    auto load_tile = [&](int64_t b, half4_t (&eb)[2], float (&xc)[kMlpCoords]) {
        const int64_t p = b * kBlockPts + 16 * wave + c;
        load_encoding(stage, n, p < n ? p : n - 1, q, eb);
        load_coords<XIN>(x, p < n ? p : n - 1, q, xc);
    };
    half4_t eb_next[2];
    float xc_next[kMlpCoords];
    int64_t b = blockIdx.x;
    if (b < nblocks) load_tile(b, eb_next, xc_next);
    for (int buf = 0; b < nblocks; b += gridDim.x, buf ^= 1) {
        BlockLds<XIN> &bl = blk[buf];
        const int64_t p = b * kBlockPts + 16 * wave + c;
        const bool ok = p < n;
        half4_t eb[2] = {eb_next[0], eb_next[1]}, h1[4], h2[4], dz1[4], dz2[4], g3;
        // binary16 before the next block's coordinates are requested into the same registers
        const half4_t xb = coord_operand<XIN>(xc_next, q);
        // dL/dy of the point as the B operand (k = output 0..3 on lanes q = 0); points past n give 0.
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q == 0 && ok) g = *reinterpret_cast<const float4 *>(dy + p * kOut);
        if (b + gridDim.x < nblocks) load_tile(b + gridDim.x, eb_next, xc_next);
        hidden_layers<XIN>(w, eb, xb, h1, h2);
        // The tile's activations into the block, transposed (each as soon as
        // it is made, so that few of them are live at once).
        const int col0 = 16 * wave;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) put_cols(bl.e, 16 * kb, q, c, col0, eb[kb], ident);
        if constexpr (XIN) {
            if (q == 0) {
#pragma unroll
                for (int r = 0; r < XIN; ++r) bl.x[r][col0 + c] = xb[r];
            }
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            put_cols(bl.h1, 16 * mb, q, c, col0, h1[mb], ident);
            put_cols(bl.h2, 16 * mb, q, c, col0, h2[mb], ident);
        }
        g3 = to_half4(float4_t{g.x * gscale, g.y * gscale, g.z * gscale, g.w * gscale});
        {
            const half4_t g3t = transpose16(g3, ident);  // rows c >= 4 are zero
            if (c < kOut) *reinterpret_cast<half4_t *>(&bl.g3[c][col0 + 4 * q]) = g3t;
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            dz2[mb] = relu_grad(mfma(t3[mb], g3, zero4), h2[mb]);
            put_cols(bl.dz2, 16 * mb, q, c, col0, dz2[mb], ident);
        }
        const half8_t dz2lo = join8(dz2[0], dz2[1]), dz2hi = join8(dz2[2], dz2[3]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            dz1[mb] = relu_grad(mfma32(t2[mb][1], dz2hi, mfma32(t2[mb][0], dz2lo, zero4)), h1[mb]);
            put_cols(bl.dz1, 16 * mb, q, c, col0, dz1[mb], ident);
        }
        const half8_t dz1lo = join8(dz1[0], dz1[1]), dz1hi = join8(dz1[2], dz1[3]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const float4_t acc = mfma32(t1[mb][1], dz1hi, mfma32(t1[mb][0], dz1lo, zero4));
            if (ok)
                *reinterpret_cast<float4 *>(de + p * kIn + 16 * mb + 4 * q) =
                    make_float4(acc[0] * ginv, acc[1] * ginv, acc[2] * ginv, acc[3] * ginv);
        }
        __syncthreads();
        // This wave's quarter of the weight gradients over the block's 64 points.
        const int u = 16 * wave + c;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const half8_t a2 = get_k(bl.dz2, u, q, h), a1 = get_k(bl.dz1, u, q, h);
            const half8_t a3 = c < kOut ? get_k(bl.g3, c, q, h) : half8_t{};
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) gw2[nb] = mfma32(a2, get_k(bl.h1, 16 * nb + c, q, h), gw2[nb]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) gw1[nb] = mfma32(a1, get_k(bl.e, 16 * nb + c, q, h), gw1[nb]);
            gw3 = mfma32(a3, get_k(bl.h2, u, q, h), gw3);
            if constexpr (XIN) gw1x = mfma32(a1, c < XIN ? get_k(bl.x, c, q, h) : half8_t{}, gw1x);
            gb2 = mfma32(a2, ones, gb2);
            gb1 = mfma32(a1, ones, gb1);
            if (wave == 0) gb3 = mfma32(a3, ones, gb3);
        }
    }
    // Lane (q, c) holds D[4 q + r][c]: rows 16 w + 4 q + r of dW1, dW2, db1,
    // db2 (the bias sums are equal in every column c), outputs 4 q + r of dW3.
    float *part = partials + (int64_t)blockIdx.x * kPartial;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * wave + 4 * q + r;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) part[kOffW1 + row * kIn + 16 * nb + c] = gw1[nb][r] * ginv;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) part[kOffW2 + row * kHid + 16 * nb + c] = gw2[nb][r] * ginv;
        if (q == 0) part[kOffW3 + r * kHid + 16 * wave + c] = gw3[r] * ginv;
        if (XIN && c < XIN) part[kOffW1x + row * kMlpCoords + c] = gw1x[r] * ginv;
        if (c == 0) {
            part[kOffB1 + row] = gb1[r] * ginv;
            part[kOffB2 + row] = gb2[r] * ginv;
            if (wave == 0 && q == 0) part[kOffB3 + r] = gb3[r] * ginv;
        }
    }
}

// Two-pass sum of the per-wave partials, in a fixed order: pass 1 sums
// waves s, s + kSplit, ... into row s of a [kSplit][kPartial] block (stored
// after the partials); pass 2 adds rows 0..kSplit-1 into the gradients.
constexpr int kSplit = 64;

// np: the partial entries the head wrote (partial_count).
__global__ __launch_bounds__(256) void mlp_reduce1_kernel(const float *__restrict__ partials, int nparts, int np,
                                                          float *__restrict__ rows) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int sidx = blockIdx.y;
    if (j >= np) return;
    float acc = 0.f;
    for (int w = sidx; w < nparts; w += kSplit) acc += partials[(int64_t)w * kPartial + j];
    rows[(int64_t)sidx * kPartial + j] = acc;
}

// dW1 is [64][coords + 32]: its coordinate columns first, then the encoding's.
__global__ __launch_bounds__(256) void mlp_reduce2_kernel(const float *__restrict__ rows, int coords, MlpGrads g) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= partial_count(coords)) return;
    float acc = 0.f;
    for (int sidx = 0; sidx < kSplit; ++sidx) acc += rows[(int64_t)sidx * kPartial + j];
    const int ld1 = kIn + coords;
    float *dst;
    if (j < kOffB1) dst = g.dw1 + (j - kOffW1) / kIn * ld1 + coords + (j - kOffW1) % kIn;
    else if (j < kOffW2) dst = g.db1 + (j - kOffB1);
    else if (j < kOffB2) dst = g.dw2 + (j - kOffW2);
    else if (j < kOffW3) dst = g.db2 + (j - kOffB2);
    else if (j < kOffB3) dst = g.dw3 + (j - kOffW3);
    else if (j < kOffW1x) dst = g.db3 + (j - kOffB3);
    else dst = g.dw1 + (j - kOffW1x) / kMlpCoords * ld1 + (j - kOffW1x) % kMlpCoords;
    *dst += acc;
}

template <int XIN>
hipError_t mlp_forward_xin(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, float *y,
                           hipStream_t stream) {
    const int64_t tiles = (n + 15) / 16;
    mlp_fwd_kernel<XIN><<<mlp_grid(tiles, (const void *)mlp_fwd_kernel<XIN>), 64 * kMlpWaves, 0, stream>>>(
        stage, x, n, mp, y, tiles);
    return hipGetLastError();
}

template <int XIN>
hipError_t mlp_backward_xin(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, const float *dy,
                            float *de, float *partials, const MlpGrads &g, hipStream_t stream) {
    const int64_t tiles = (n + 15) / 16;
    constexpr size_t lds = bwd_lds<XIN>();
    hipError_t e = hipFuncSetAttribute((const void *)mlp_bwd_kernel<XIN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    // One set of partials per workgroup (its four waves own a quarter each).
    const int grid = mlp_grid(tiles, (const void *)mlp_bwd_kernel<XIN>, lds);
    const int nparts = grid;
    float *rows = partials + (int64_t)nparts * kPartial;
    uint32_t *dmax = reinterpret_cast<uint32_t *>(rows + (int64_t)kSplit * kPartial);
    mlp_dy_max_kernel<<<kDyMaxParts, 256, 0, stream>>>(reinterpret_cast<const float4 *>(dy), n, dmax);
    mlp_bwd_kernel<XIN><<<grid, 64 * kMlpWaves, lds, stream>>>(stage, x, n, mp, dy, dmax, de, partials);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int np = partial_count(XIN);
    mlp_reduce1_kernel<<<dim3((np + 255) / 256, kSplit), 256, 0, stream>>>(partials, nparts, np, rows);
    mlp_reduce2_kernel<<<(np + 255) / 256, 256, 0, stream>>>(rows, XIN, g);
    return hipGetLastError();
}

}  // namespace

size_t mlp_partials_bytes(int64_t n) {
    const int64_t tiles = (n + 15) / 16;
    const size_t grid = (size_t)std::max<int64_t>(1, std::min<int64_t>((tiles + kMlpWaves - 1) / kMlpWaves, kMaxMlpGrid));
    return (grid + kSplit) * kPartial * sizeof(float) + kDyMaxParts * sizeof(uint32_t);
}

hipError_t launch_mlp_forward(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, float *y,
                              hipStream_t stream) {
    return mp.coords ? mlp_forward_xin<kMlpCoords>(stage, x, n, mp, y, stream)
                     : mlp_forward_xin<0>(stage, x, n, mp, y, stream);
}

hipError_t launch_mlp_backward(const _Float16 *stage, const float *x, int64_t n, const MlpParams &mp, const float *dy,
                               float *de, float *partials, const MlpGrads &g, hipStream_t stream) {
    return mp.coords ? mlp_backward_xin<kMlpCoords>(stage, x, n, mp, dy, de, partials, g, stream)
                     : mlp_backward_xin<0>(stage, x, n, mp, dy, de, partials, g, stream);
}

}  // namespace hg
