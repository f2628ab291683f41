// Device helpers shared by the HIP kernels of libhashgrid (gfx950).
#pragma once

#include "hashgrid_internal.h"

namespace hg {

// Multipliers of the spatial hash, one per input coordinate: the jsqmd.com
// HashEncoding prime list (section 3); the first three are the x, y, z primes
// of ipipp.com HashGridEncoder.hash and the ijyty.com section 2.2 formula.
constexpr int kMaxDims = 4;
__constant__ constexpr uint32_t kPrimeList[7] = {1u,          2654435761u, 805459861u, 3674653429u,
                                                 2097192037u, 1434869437u, 2165219737u};

struct Item {
    int level;
    int64_t p0;
};

// Work item of this workgroup (see LaunchParams); false past the last item.
__device__ __forceinline__ bool decode_item(const LaunchParams &lp, Item &it) {
    int g = blockIdx.x;
    int item = lp.xcd_map ? (g % kNumXcd) * lp.per_xcd + g / kNumXcd : g;
    if (item >= lp.items) return false;
    int pos = item / lp.chunks;
    it.level = lp.level_order[pos];
    it.p0 = (int64_t)(item - pos * lp.chunks) * lp.chunk_pts;
    return true;
}

// Voxel of one coordinate: scaled position rounded to fp32, its floor as a
// signed integer and the fraction s - floor(s), which is exact.  Contraction
// is off here: fusing the multiply into the subtraction would compute the
// fraction of the unrounded product and move the weights off the voxel that
// floor(s) picked.
__device__ __forceinline__ void locate1(float xd, float N, int32_t &v, float &f) {
#pragma clang fp contract(off)
    float s = xd * N;
    float fl = floorf(s);
    v = (int32_t)fl;
    f = s - fl;
}

// Exchange a value with the other lane of an aligned lane pair (DPP
// quad_perm [1,0,3,2]); the pair never leaves its quad.
__device__ __forceinline__ float swap_pair(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// F features of table entry e as fp32: DT 0 reads fp32, DT 1 binary16
// (widened exactly, subnormals included), with one vector load per entry.
template <int F, int DT>
__device__ __forceinline__ void load_features(const void *__restrict__ t, uint64_t e, float (&v)[F]) {
    if constexpr (DT == 0) {
        const float *p = reinterpret_cast<const float *>(t) + e * F;
        if constexpr (F == 1) {
            v[0] = p[0];
        } else if constexpr (F == 2) {
            const float2 a = *reinterpret_cast<const float2 *>(p);
            v[0] = a.x, v[1] = a.y;
        } else {
#pragma unroll
            for (int q = 0; q < F / 4; ++q) {
                const float4 a = reinterpret_cast<const float4 *>(p)[q];
                v[4 * q] = a.x, v[4 * q + 1] = a.y, v[4 * q + 2] = a.z, v[4 * q + 3] = a.w;
            }
        }
    } else {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(t) + e * F;
        uint32_t w[(F + 1) / 2];
        if constexpr (F == 1) {
            w[0] = p[0];
        } else if constexpr (F == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else if constexpr (F == 4) {
            const uint2 a = *reinterpret_cast<const uint2 *>(p);
            w[0] = a.x, w[1] = a.y;
        } else {
            const uint4 a = *reinterpret_cast<const uint4 *>(p);
            w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w;
        }
#pragma unroll
        for (int j = 0; j < F; ++j)
            v[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)((w[j / 2] >> (16 * (j & 1))) & 0xFFFFu));
    }
}

}  // namespace hg
