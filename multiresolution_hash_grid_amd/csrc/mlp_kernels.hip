// MLP head after the encoder, on the gfx950 matrix cores.
//
// The network is the NeRFace head of ipipp.com (section 3 listing):
// Linear(32, 64), ReLU, Linear(64, 64), ReLU, Linear(64, 4), biases on,
//   y = W3 relu(W2 relu(W1 e + b1) + b2) + b3,
// e being the 32 encoded features (L = 16 levels x F = 2) of a point.  It is
// a dense contraction, so it runs on v_mfma_f32_16x16x16f16: binary16
// operands, fp32 accumulation.
//
// Layout.  For D[i][j] = sum_k A[i][k] B[k][j] (16 x 16 x 16), lane l of the
// wave holds A[l%16][4(l/16) + r], B[4(l/16) + r][l%16] and
// D[4(l/16) + r][l%16], r = 0..3.  The kernels put the weights in A (rows =
// output units) and 16 points in the columns of B and D; then the D of one
// layer, rounded to binary16, is already the B operand of the next layer (the
// four rows a lane holds are the four k a lane supplies), so activations go
// from layer to layer in registers.
//
// Forward: the encoder's gather writes the encoding level-major as binary16
// ([L][n][2], one 64-byte read per point here instead of a 128-byte fp32
// row), and each wave runs the three layers on 16 points at a time.  The
// stage is kept for the backward.
//
// Backward: each wave recomputes z1, h1, z2, h2 from the stage, takes
// dL/dy to dz2 = (W3^T g) * [z2 > 0], dz1 = (W2^T dz2) * [z1 > 0] and
// dL/de = W1^T dz1 with the transposed weights in A, and writes dL/de as
// the fp32 upstream rows of the encoder's table backward.  The weight
// gradients contract over points, so a tile's activations go through LDS
// to put the 16 points on the k axis (dW2 = dz2 h1^T etc.); every wave keeps
// its running dW and db in registers and writes them once, and two reduction
// kernels add the per-wave partials, in a fixed order, into the caller's fp32
// gradients.
#include <algorithm>

#include "device_common.h"

namespace hg {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kIn = 32, kHid = 64, kOut = 4;
constexpr int kMlpWaves = 4;  // waves per workgroup
// Per-wave partial sums: dW1 [64][32], db1 [64], dW2 [64][64], db2 [64], dW3 [4][64], db3 [4].
constexpr int kOffW1 = 0, kOffB1 = kOffW1 + kHid * kIn, kOffW2 = kOffB1 + kHid, kOffB2 = kOffW2 + kHid * kHid,
              kOffW3 = kOffB2 + kHid, kOffB3 = kOffW3 + kOut * kHid, kPartial = kOffB3 + kOut;

__device__ __forceinline__ float4_t mfma(half4_t a, half4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half4_t relu_half(float4_t v, uint32_t &mask, int shift) {
    half4_t h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool pos = v[r] > 0.f;
        mask |= (uint32_t)pos << (shift + r);
        h[r] = (_Float16)(pos ? v[r] : 0.f);
    }
    return h;
}

// The forward weights as A operands: row = output unit, k = input.
struct FwdWeights {
    half4_t a1[4][2], a2[4][4], a3[4];
    float4_t b1[4], b2[4], b3;
};

__device__ __forceinline__ void load_fwd_weights(const MlpParams &mp, int q, int c, FwdWeights &w) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) w.a1[mb][kb][r] = mp.w1[(16 * mb + c) * kIn + 16 * kb + 4 * q + r];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) w.a2[mb][kb][r] = mp.w2[(16 * mb + c) * kHid + 16 * kb + 4 * q + r];
            w.b1[mb][r] = mp.b1[16 * mb + 4 * q + r];
            w.b2[mb][r] = mp.b2[16 * mb + 4 * q + r];
        }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w.a3[kb][r] = c < kOut ? mp.w3[c * kHid + 16 * kb + 4 * q + r] : (_Float16)0.f;
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

// Layers 1 and 2 of 16 points: binary16 activations and their ReLU masks
// (bit 4 mb + r: unit 16 mb + 4 q + r had a positive input).
__device__ __forceinline__ void hidden_layers(const FwdWeights &w, const half4_t (&eb)[2], half4_t (&h1)[4],
                                              half4_t (&h2)[4], uint32_t &m1, uint32_t &m2) {
    m1 = m2 = 0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        float4_t acc = w.b1[mb];
        acc = mfma(w.a1[mb][0], eb[0], acc);
        acc = mfma(w.a1[mb][1], eb[1], acc);
        h1[mb] = relu_half(acc, m1, 4 * mb);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        float4_t acc = w.b2[mb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mfma(w.a2[mb][kb], h1[kb], acc);
        h2[mb] = relu_half(acc, m2, 4 * mb);
    }
}

int mlp_grid(int64_t tiles) {
    const int64_t want = (tiles + kMlpWaves - 1) / kMlpWaves;
    return (int)std::min<int64_t>(want, 1024);  // persistent: 4 waves per CU-slot, 4096 waves at most
}

// ---------------------------------------------------------------- forward

__global__ __launch_bounds__(64 * kMlpWaves) void mlp_fwd_kernel(const _Float16 *__restrict__ stage, int64_t n,
                                                                 MlpParams mp, float *__restrict__ y,
                                                                 int64_t tiles) {
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
    FwdWeights w;
    load_fwd_weights(mp, q, c, w);
    const int64_t nwaves = (int64_t)gridDim.x * kMlpWaves;
    half4_t eb_next[2];
    int64_t t = (int64_t)blockIdx.x * kMlpWaves + (threadIdx.x >> 6);
    if (t < tiles) load_encoding(stage, n, min(t * 16 + c, n - 1), q, eb_next);
    for (; t < tiles; t += nwaves) {
        const int64_t p = t * 16 + c;
        const bool ok = p < n;
        half4_t eb[2] = {eb_next[0], eb_next[1]}, h1[4], h2[4];
        if (t + nwaves < tiles) load_encoding(stage, n, min((t + nwaves) * 16 + c, n - 1), q, eb_next);
        uint32_t m1, m2;
        hidden_layers(w, eb, h1, h2, m1, m2);
        float4_t o = w.b3;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) o = mfma(w.a3[kb], h2[kb], o);
        if (q == 0 && ok) *reinterpret_cast<float4 *>(y + p * kOut) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// ---------------------------------------------------------------- backward

// LDS rows of one wave's tile, points as rows, binary16, padded against bank conflicts.
struct TileLds {
    _Float16 e[16][kIn + 8];
    _Float16 h1[16][kHid + 8];
    _Float16 h2[16][kHid + 8];
    _Float16 dz1[16][kHid + 8];
    _Float16 dz2[16][kHid + 8];
    _Float16 g3[16][8];
};

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Lane (q, c) holds rows 16 m + 4 q + r of point c (the D / B layout): store them as row c.
template <int W>
__device__ __forceinline__ void put_rows(_Float16 (*dst)[W], int m, int q, int c, half4_t v) {
    *reinterpret_cast<half4_t *>(&dst[c][16 * m + 4 * q]) = v;
}

// Operand with the points on the k axis: points 4 q + r, column 16 m + c.
template <int W>
__device__ __forceinline__ half4_t get_cols(_Float16 (*src)[W], int m, int q, int c) {
    half4_t v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = src[4 * q + r][16 * m + c];
    return v;
}

__global__ __launch_bounds__(64 * kMlpWaves) void mlp_bwd_kernel(const _Float16 *__restrict__ stage, int64_t n,
                                                                 MlpParams mp, const float *__restrict__ dy,
                                                                 float *__restrict__ de,
                                                                 float *__restrict__ partials, int64_t tiles) {
    __shared__ TileLds lds[kMlpWaves];
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15, wave = threadIdx.x >> 6;
    TileLds &tl = lds[wave];
    FwdWeights w;
    load_fwd_weights(mp, q, c, w);
    // Transposed weights as A operands: row = input unit of the layer, k = its output unit.
    half4_t t3[4], t2[4][4], t1[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            t3[mb][r] = q == 0 ? mp.w3[r * kHid + 16 * mb + c] : (_Float16)0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) t2[mb][kb][r] = mp.w2[(16 * kb + 4 * q + r) * kHid + 16 * mb + c];
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) t1[mb][kb][r] = mp.w1[(16 * kb + 4 * q + r) * kIn + 16 * mb + c];
    }
    float4_t gw1[4][2], gw2[4][4], gw3[4];
    float4_t gb1[4], gb2[4], gb3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gw3[i] = gb1[i] = gb2[i] = float4_t{0.f, 0.f, 0.f, 0.f};
        gw1[i][0] = gw1[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) gw2[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    gb3 = float4_t{0.f, 0.f, 0.f, 0.f};
    const int64_t nwaves = (int64_t)gridDim.x * kMlpWaves;
    // The next tile's encoding and dL/dy are requested before the current tile
    // is worked on (one wave per SIMD at this register count: the loads must
    // not stall it).
    auto load_tile = [&](int64_t t, half4_t (&eb)[2], float4 &g) {
        const int64_t p = t * 16 + c;
        const bool ok = p < n;
        load_encoding(stage, n, ok ? p : n - 1, q, eb);
        // dL/dy of the point as the B operand (k = output 0..3 on lanes q = 0); points past n give 0.
        g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q == 0 && ok) g = *reinterpret_cast<const float4 *>(dy + p * kOut);
    };
    half4_t eb_next[2];
    float4 g_next;
    int64_t t = (int64_t)blockIdx.x * kMlpWaves + wave;
    if (t < tiles) load_tile(t, eb_next, g_next);
    for (; t < tiles; t += nwaves) {
        const int64_t p = t * 16 + c;
        const bool ok = p < n;
        half4_t eb[2] = {eb_next[0], eb_next[1]}, h1[4], h2[4], dz1[4], dz2[4], g3;
        const float4 g = g_next;
        if (t + nwaves < tiles) load_tile(t + nwaves, eb_next, g_next);
        uint32_t m1, m2;
        hidden_layers(w, eb, h1, h2, m1, m2);
        g3 = half4_t{(_Float16)g.x, (_Float16)g.y, (_Float16)g.z, (_Float16)g.w};
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const float4_t acc = mfma(t3[mb], g3, float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) dz2[mb][r] = (_Float16)(((m2 >> (4 * mb + r)) & 1) ? acc[r] : 0.f);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc = mfma(t2[mb][kb], dz2[kb], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) dz1[mb][r] = (_Float16)(((m1 >> (4 * mb + r)) & 1) ? acc[r] : 0.f);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc = mfma(t1[mb][kb], dz1[kb], acc);
            if (ok) *reinterpret_cast<float4 *>(de + p * kIn + 16 * mb + 4 * q) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        // Bias gradients: this lane's units, summed over the points it sees.
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gb1[mb][r] += (float)dz1[mb][r];
                gb2[mb][r] += (float)dz2[mb][r];
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) gb3[r] += (float)g3[r];
        // Weight gradients: the tile through LDS with the points on the k axis.
        wave_lds_fence();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) put_rows(tl.e, kb, q, c, eb[kb]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            put_rows(tl.h1, mb, q, c, h1[mb]);
            put_rows(tl.h2, mb, q, c, h2[mb]);
            put_rows(tl.dz1, mb, q, c, dz1[mb]);
            put_rows(tl.dz2, mb, q, c, dz2[mb]);
        }
        if (q < 2) *reinterpret_cast<half4_t *>(&tl.g3[c][4 * q]) = g3;  // q = 1 writes the zero padding
        wave_lds_fence();
        half4_t ga;  // A of dW3: row = output c (< 4), k = point
#pragma unroll
        for (int r = 0; r < 4; ++r) ga[r] = c < kOut ? tl.g3[4 * q + r][c] : (_Float16)0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const half4_t bh2 = get_cols(tl.h2, nb, q, c), bh1 = get_cols(tl.h1, nb, q, c);
            gw3[nb] = mfma(ga, bh2, gw3[nb]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) gw2[mb][nb] = mfma(get_cols(tl.dz2, mb, q, c), bh1, gw2[mb][nb]);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const half4_t be = get_cols(tl.e, nb, q, c);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) gw1[mb][nb] = mfma(get_cols(tl.dz1, mb, q, c), be, gw1[mb][nb]);
        }
    }
    // Bias sums over the 16 point columns (lanes of equal q).
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gb1[mb][r] += __shfl_xor(gb1[mb][r], off, 64);
                gb2[mb][r] += __shfl_xor(gb2[mb][r], off, 64);
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) gb3[r] += __shfl_xor(gb3[r], off, 64);
    }
    float *part = partials + ((int64_t)blockIdx.x * kMlpWaves + wave) * kPartial;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int row = 16 * mb + 4 * q + r;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) part[kOffW1 + row * kIn + 16 * nb + c] = gw1[mb][nb][r];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) part[kOffW2 + row * kHid + 16 * nb + c] = gw2[mb][nb][r];
            if (c == 0) {
                part[kOffB1 + row] = gb1[mb][r];
                part[kOffB2 + row] = gb2[mb][r];
            }
        }
        if (q == 0) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) part[kOffW3 + r * kHid + 16 * nb + c] = gw3[nb][r];
            if (c == 0) part[kOffB3 + r] = gb3[r];
        }
    }
}

// Two-pass sum of the per-wave partials, in a fixed order: pass 1 sums
// waves s, s + kSplit, ... into row s of a [kSplit][kPartial] block (stored
// after the partials); pass 2 adds rows 0..kSplit-1 into the gradients.
constexpr int kSplit = 64;

__global__ __launch_bounds__(256) void mlp_reduce1_kernel(const float *__restrict__ partials, int nparts,
                                                          float *__restrict__ rows) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int sidx = blockIdx.y;
    if (j >= kPartial) return;
    float acc = 0.f;
    for (int w = sidx; w < nparts; w += kSplit) acc += partials[(int64_t)w * kPartial + j];
    rows[(int64_t)sidx * kPartial + j] = acc;
}

__global__ __launch_bounds__(256) void mlp_reduce2_kernel(const float *__restrict__ rows, MlpGrads g) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= kPartial) return;
    float acc = 0.f;
    for (int sidx = 0; sidx < kSplit; ++sidx) acc += rows[(int64_t)sidx * kPartial + j];
    float *dst;
    if (j < kOffB1) dst = g.dw1 + (j - kOffW1);
    else if (j < kOffW2) dst = g.db1 + (j - kOffB1);
    else if (j < kOffB2) dst = g.dw2 + (j - kOffW2);
    else if (j < kOffW3) dst = g.db2 + (j - kOffB2);
    else if (j < kOffB3) dst = g.dw3 + (j - kOffW3);
    else dst = g.db3 + (j - kOffB3);
    *dst += acc;
}

}  // namespace

size_t mlp_partials_bytes(int64_t n) {
    const int64_t tiles = (n + 15) / 16;
    return ((size_t)mlp_grid(tiles) * kMlpWaves + kSplit) * kPartial * sizeof(float);
}

hipError_t launch_mlp_forward(const _Float16 *stage, int64_t n, const MlpParams &mp, float *y, hipStream_t stream) {
    const int64_t tiles = (n + 15) / 16;
    mlp_fwd_kernel<<<mlp_grid(tiles), 64 * kMlpWaves, 0, stream>>>(stage, n, mp, y, tiles);
    return hipGetLastError();
}

hipError_t launch_mlp_backward(const _Float16 *stage, int64_t n, const MlpParams &mp, const float *dy, float *de,
                               float *partials, const MlpGrads &g, hipStream_t stream) {
    const int64_t tiles = (n + 15) / 16;
    const int grid = mlp_grid(tiles);
    mlp_bwd_kernel<<<grid, 64 * kMlpWaves, 0, stream>>>(stage, n, mp, dy, de, partials, tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nparts = grid * kMlpWaves;
    float *rows = partials + (int64_t)nparts * kPartial;
    mlp_reduce1_kernel<<<dim3((kPartial + 255) / 256, kSplit), 256, 0, stream>>>(partials, nparts, rows);
    mlp_reduce2_kernel<<<(kPartial + 255) / 256, 256, 0, stream>>>(rows, g);
    return hipGetLastError();
}

}  // namespace hg
