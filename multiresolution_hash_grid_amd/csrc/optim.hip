// Adam update of the hash tables for gfx950.
//
// The pages train the tables with Adam, no weight decay on them (ipipp.com
// section 4) and torch.optim.Adam in the training loop (ijyty.com overview,
// section 4).  Every entry is updated, as torch.optim.Adam does: the moments
// of entries no point touched this step still decay and move the entry.
//
// One pass over L*T*F entries, bound by HBM: it reads param, m, v and grad
// (16 B per entry) and writes param, m, v (12 B), plus 4 B when it clears the
// gradient for the next backward and 2 B when it refreshes an fp16 copy of
// the tables.  Each thread takes four consecutive entries with 16-byte loads
// and stores; a scalar kernel covers unaligned buffers.
#include "hashgrid_internal.h"

namespace hg {
namespace {

struct AdamCoef {
    float beta1, beta2;
    float omb1, omb2;   // 1 - beta, formed in double from the fp32 betas
    float step_size;    // lr / (1 - beta1^t)
    float inv_bc2_sqrt; // 1 / sqrt(1 - beta2^t)
    float eps;
};

__device__ __forceinline__ void adam1(float &p, float &m, float &v, float g, const AdamCoef &c) {
    m = c.beta1 * m + c.omb1 * g;
    v = c.beta2 * v + c.omb2 * (g * g);
    const float denom = sqrtf(v) * c.inv_bc2_sqrt + c.eps;
    p -= c.step_size * m / denom;
}

template <bool kZero, bool kHalf>
__global__ __launch_bounds__(256) void adam_vec_kernel(float4 *__restrict__ param, float4 *__restrict__ m,
                                                       float4 *__restrict__ v, float4 *__restrict__ grad,
                                                       uint2 *__restrict__ half4, int64_t n4, AdamCoef c) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 p = param[i], mm = m[i], vv = v[i];
    const float4 g = grad[i];
    adam1(p.x, mm.x, vv.x, g.x, c);
    adam1(p.y, mm.y, vv.y, g.y, c);
    adam1(p.z, mm.z, vv.z, g.z, c);
    adam1(p.w, mm.w, vv.w, g.w, c);
    param[i] = p;
    m[i] = mm;
    v[i] = vv;
    if (kZero) grad[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (kHalf) {
        const __half2 a = __floats2half2_rn(p.x, p.y), b = __floats2half2_rn(p.z, p.w);
        half4[i] = make_uint2(*reinterpret_cast<const uint32_t *>(&a), *reinterpret_cast<const uint32_t *>(&b));
    }
}

__global__ __launch_bounds__(256) void adam_scalar_kernel(float *__restrict__ param, float *__restrict__ m,
                                                          float *__restrict__ v, float *__restrict__ grad,
                                                          __half *__restrict__ half1, int64_t n, int zero,
                                                          AdamCoef c) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float p = param[i], mm = m[i], vv = v[i];
    adam1(p, mm, vv, grad[i], c);
    param[i] = p;
    m[i] = mm;
    v[i] = vv;
    if (zero) grad[i] = 0.f;
    if (half1) half1[i] = __float2half_rn(p);
}

template <bool kZero, bool kHalf>
void launch_vec(float *param, float *m, float *v, float *grad, void *half, int64_t n4, const AdamCoef &c,
                hipStream_t stream) {
    const int64_t blocks = (n4 + 255) / 256;
    adam_vec_kernel<kZero, kHalf><<<dim3((unsigned)blocks), 256, 0, stream>>>(
        reinterpret_cast<float4 *>(param), reinterpret_cast<float4 *>(m), reinterpret_cast<float4 *>(v),
        reinterpret_cast<float4 *>(grad), reinterpret_cast<uint2 *>(half), n4, c);
}

}  // namespace

hipError_t launch_adam(const AdamParams &a, int64_t count, float *param, float *m, float *v, float *grad,
                       void *param_f16, bool zero_grad, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const double bc1 = 1.0 - pow((double)a.beta1, (double)a.step);
    const double bc2 = 1.0 - pow((double)a.beta2, (double)a.step);
    const AdamCoef c{a.beta1,
                     a.beta2,
                     (float)(1.0 - (double)a.beta1),
                     (float)(1.0 - (double)a.beta2),
                     (float)((double)a.lr / bc1),
                     (float)(1.0 / sqrt(bc2)),
                     a.eps};
    auto al = [](const void *p, uintptr_t k) { return ((uintptr_t)p % k) == 0; };
    const bool vec = count % 4 == 0 && al(param, 16) && al(m, 16) && al(v, 16) && al(grad, 16) &&
                     (!param_f16 || al(param_f16, 8));
    if (vec) {
        const int64_t n4 = count / 4;
        if (zero_grad) {
            if (param_f16) launch_vec<true, true>(param, m, v, grad, param_f16, n4, c, stream);
            else launch_vec<true, false>(param, m, v, grad, param_f16, n4, c, stream);
        } else {
            if (param_f16) launch_vec<false, true>(param, m, v, grad, param_f16, n4, c, stream);
            else launch_vec<false, false>(param, m, v, grad, param_f16, n4, c, stream);
        }
    } else {
        const int64_t blocks = (count + 255) / 256;
        adam_scalar_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(
            param, m, v, grad, reinterpret_cast<__half *>(param_f16), count, zero_grad ? 1 : 0, c);
    }
    return hipGetLastError();
}

}  // namespace hg
