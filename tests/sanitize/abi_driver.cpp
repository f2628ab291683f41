// Drives the host side of the C ABI (include/hashgrid.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer: every query and every
// argument check that is answered on the host, over many configurations.  No
// call here reaches a kernel launcher (the stand-ins abort if one does).
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hashgrid.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static hg_config make(int D, int L, int F, int log2T, int nmin, int nmax, int dt = HG_F32) {
    return hg_config{D, L, F, log2T, nmin, nmax, dt, HG_F32};
}

int main() {
    EXPECT(hashgrid_abi_version() == HASHGRID_ABI_VERSION);
    EXPECT(std::strlen(hashgrid_last_error()) == 0 || hashgrid_last_error()[0] != '\0');
    int32_t res[64];
    // resolutions over many grids, including L = 1 and the widest ranges
    for (int L : {1, 2, 3, 16, 32, 64})
        for (int nmin : {1, 3, 16})
            for (int nmax : {nmin, 2 * nmin + 1, 512, (1 << 24) - 1}) {
                hg_config c = make(3, L, 2, 19, nmin, nmax);
                EXPECT(hashgrid_resolutions(&c, res) == HG_OK);
                EXPECT(res[0] == nmin);
                for (int l = 1; l < L; ++l) EXPECT(res[l] >= res[l - 1]);
            }
    EXPECT(hashgrid_resolutions(nullptr, res) == HG_EINVAL);
    // workspace queries
    size_t a = 0, b = 0, c2 = 0;
    for (int D = 1; D <= 4; ++D)
        for (int F : {1, 2, 4, 8})
            for (int log2T : {1, 10, 19, 25, 28})
                for (int64_t n : {(int64_t)0, (int64_t)1, (int64_t)4097, (int64_t)1 << 18, (int64_t)1 << 28}) {
                    hg_config c = make(D, 16, F, log2T, 16, 512);
                    EXPECT(hashgrid_forward_workspace_size(&c, n, &a) == HG_OK);
                    EXPECT(hashgrid_backward_workspace_size(&c, n, &a, &b) == HG_OK);
                    EXPECT(a >= b);
                    EXPECT(hashgrid_input_grad_workspace_size(&c, n, &a) == HG_OK);
                    const int mrc = hashgrid_mlp_workspace_size(&c, n, &a, &c2);
                    EXPECT(mrc == (D == 3 && F == 2 ? HG_OK : HG_EUNSUPPORTED));
                }
    hg_config std_cfg = make(3, 16, 2, 19, 16, 512);
    EXPECT(hashgrid_forward_workspace_size(&std_cfg, -1, &a) == HG_EINVAL);
    EXPECT(hashgrid_backward_workspace_size(&std_cfg, 1 << 18, nullptr, nullptr) == HG_EINVAL);
    // invalid configurations, on every entry point
    const hg_config bad[] = {make(0, 16, 2, 19, 16, 512), make(5, 16, 2, 19, 16, 512), make(3, 0, 2, 19, 16, 512),
                             make(3, 65, 2, 19, 16, 512), make(3, 16, 3, 19, 16, 512), make(3, 16, 2, 0, 16, 512),
                             make(3, 16, 2, 29, 16, 512), make(3, 16, 2, 19, 0, 512), make(3, 16, 2, 19, 64, 32),
                             make(3, 16, 2, 19, 16, 1 << 24), make(3, 16, 2, 19, 16, 512, 7)};
    float *x = reinterpret_cast<float *>(0x1000), *d = reinterpret_cast<float *>(0x2000);
    float *t = reinterpret_cast<float *>(0x3000), *o = reinterpret_cast<float *>(0x4000);
    for (const hg_config &c : bad) {
        EXPECT(hashgrid_forward(&c, x, 16, t, o, 32, nullptr, 0, nullptr) < 0);
        EXPECT(hashgrid_backward(&c, x, 16, d, 32, t, nullptr, 0, nullptr) < 0);
        EXPECT(hashgrid_backward_noalloc(&c, x, 16, d, 32, t, nullptr) < 0);
        EXPECT(hashgrid_input_grad(&c, x, 16, t, d, 32, o, nullptr, 0, nullptr) < 0);
        EXPECT(hashgrid_debug_corners(&c, x, 16, nullptr, nullptr, nullptr) < 0);
        EXPECT(std::strlen(hashgrid_last_error()) > 0);
    }
    hg_config g16 = std_cfg;
    g16.grad_dtype = HG_F16;
    EXPECT(hashgrid_backward(&g16, x, 16, d, 32, t, nullptr, 0, nullptr) == HG_EUNSUPPORTED);
    // bad pointers, sizes, strides and alignments
    EXPECT(hashgrid_forward(&std_cfg, nullptr, 16, t, o, 32, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_forward(&std_cfg, x, -3, t, o, 32, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_forward(&std_cfg, x, 16, reinterpret_cast<float *>(0x3004), o, 32, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_forward(&std_cfg, x, 16, t, o, 31, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_forward(&std_cfg, x, 16, t, o, 32, reinterpret_cast<void *>(0x5008), 1 << 20, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_backward(&std_cfg, x, 16, nullptr, 32, t, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_backward(&std_cfg, x, 16, d, 30, t, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_backward(&std_cfg, reinterpret_cast<float *>(0x1002), 16, d, 32, t, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_backward_noalloc(&std_cfg, x, (int64_t)1 << 21, d, 32, t, nullptr) == HG_EINVAL);
    EXPECT(std::strstr(hashgrid_last_error(), "at most") != nullptr);
    EXPECT(hashgrid_input_grad(&std_cfg, x, 16, t, d, 32, nullptr, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_debug_corners(&std_cfg, x, (int64_t)1 << 31, nullptr, nullptr, nullptr) == HG_EINVAL);
    // n == 0 is a no-op on every entry point (pointers are not inspected)
    EXPECT(hashgrid_forward(&std_cfg, nullptr, 0, nullptr, nullptr, 32, nullptr, 0, nullptr) == HG_OK);
    EXPECT(hashgrid_backward(&std_cfg, nullptr, 0, nullptr, 32, nullptr, nullptr, 0, nullptr) == HG_OK);
    EXPECT(hashgrid_backward_noalloc(&std_cfg, nullptr, 0, nullptr, 32, nullptr, nullptr) == HG_OK);
    EXPECT(hashgrid_input_grad(&std_cfg, nullptr, 0, nullptr, nullptr, 32, nullptr, nullptr, 0, nullptr) == HG_OK);
    EXPECT(hashgrid_debug_corners(&std_cfg, nullptr, 0, nullptr, nullptr, nullptr) == HG_OK);
    // the MLP head: other grids, missing parameters and buffers
    hg_config f4 = make(3, 16, 4, 19, 16, 512);
    hg_mlp_params mp{};
    EXPECT(hashgrid_mlp_forward(&f4, x, 16, t, &mp, o, o, 1 << 20, nullptr) == HG_EUNSUPPORTED);
    EXPECT(hashgrid_mlp_forward(&std_cfg, x, 16, t, &mp, o, o, 1 << 20, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_mlp_forward(&std_cfg, x, 16, t, nullptr, o, o, 1 << 20, nullptr) == HG_EINVAL);
    hg_mlp_grads mg{};
    EXPECT(hashgrid_mlp_backward(&std_cfg, x, 16, o, &mp, d, &mg, t, o, 1 << 20, nullptr) == HG_EINVAL);
    const void *w = reinterpret_cast<const void *>(0x7000);
    const float *bias = reinterpret_cast<const float *>(0x7100);
    hg_mlp_params tiny{w, bias, w, bias, w, bias, 7};  // coord_inputs is 0 or 3
    EXPECT(hashgrid_mlp_forward(&std_cfg, x, 16, t, &tiny, o, o, 1 << 20, nullptr) == HG_EINVAL);
    EXPECT(std::strstr(hashgrid_last_error(), "coord_inputs") != nullptr);
    // Adam: every hyperparameter check
    float *p = reinterpret_cast<float *>(0x6000);
    hg_adam ok_opt{1e-2f, 0.9f, 0.999f, 1e-8f, 1};
    const hg_adam bad_opts[] = {{1e-2f, 0.9f, 0.999f, 1e-8f, 0}, {1e-2f, 1.0f, 0.999f, 1e-8f, 1},
                                {1e-2f, 0.9f, -0.1f, 1e-8f, 1},  {1e-2f, 0.9f, 0.999f, -1.f, 1},
                                {__builtin_inff(), 0.9f, 0.999f, 1e-8f, 1}};
    for (const hg_adam &op : bad_opts) EXPECT(hashgrid_adam_step(&op, 16, p, p, p, p, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_adam_step(&ok_opt, 16, p, p, p, p, nullptr, 2, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_adam_step(&ok_opt, -1, p, p, p, p, nullptr, 0, nullptr) == HG_EINVAL);
    EXPECT(hashgrid_adam_step(&ok_opt, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == HG_OK);
    EXPECT(hashgrid_adam_step(nullptr, 16, p, p, p, p, nullptr, 0, nullptr) == HG_EINVAL);
    // tuning keys: each valid value and the neighbours of the range
    for (int key = -1; key <= 12; ++key) {
        const int before = hashgrid_tune_get(key);
        for (int v : {-1, 0, 1, 2, 3, 4, 11, 13, 64, 1024, 65536, 1 << 20, (1 << 20) + 1}) hashgrid_tune(key, v);
        if (before >= 0) EXPECT(hashgrid_tune(key, before) == HG_OK && hashgrid_tune_get(key) == before);
        else EXPECT(hashgrid_tune(key, 0) == HG_EINVAL);
    }
    if (failures) {
        std::fprintf(stderr, "%d failed expectations\n", failures);
        return 1;
    }
    std::printf("abi driver: all host-side checks passed\n");
    return 0;
}
