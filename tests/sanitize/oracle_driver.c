/* Drives the C oracle (oracle/hashgrid_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: corners, forward, backward and dL/dx for every
 * input dimension and feature count it serves, fp32 and binary16 tables,
 * points inside and outside the unit cube, with two of its invariants checked
 * on the way (the weights of a point sum to one; the backward is the adjoint
 * of the forward). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int32_t n_dims, n_levels, n_features, log2_table_size, base_resolution, finest_resolution, table_is_half;
} oracle_grid;

int oracle_resolutions(int32_t, int32_t, int32_t, int32_t *);
int oracle_corners(const oracle_grid *, const float *, int64_t, uint32_t *, double *);
int oracle_forward(const oracle_grid *, const float *, int64_t, const void *, double *);
int oracle_backward(const oracle_grid *, const float *, int64_t, const float *, int64_t, double *);
int oracle_input_grad(const oracle_grid *, const float *, int64_t, const void *, const float *, int64_t, double *);
void oracle_set_threads(int);

static uint64_t state = 12345;
static double uni(void) {
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(state >> 11) * 0x1p-53;
}

int main(void) {
    int fails = 0;
    int32_t res[64];
    for (int L = 1; L <= 64; L += 9)
        if (oracle_resolutions(L, 3, 4000, res)) ++fails;
    oracle_set_threads(2);
    for (int D = 1; D <= 4; ++D) {
        for (int F = 1; F <= 8; F *= 2) {
            for (int half = 0; half <= 1; ++half) {
                const oracle_grid g = {D, 5, F, 9, 2, 40, half};
                const int64_t n = 97, T = 512, K = (int64_t)1 << D, L = 5, C = L * F;
                float *x = malloc(sizeof(float) * n * D);
                float *dout = malloc(sizeof(float) * n * C);
                void *table = malloc((half ? 2 : 4) * L * T * F);
                double *out = malloc(sizeof(double) * n * C);
                double *grad = calloc((size_t)(L * T * F), sizeof(double));
                double *dx = malloc(sizeof(double) * n * D);
                uint32_t *idx = malloc(sizeof(uint32_t) * n * L * K);
                double *w = malloc(sizeof(double) * n * L * K);
                for (int64_t i = 0; i < n * D; ++i) x[i] = (float)(uni() * 1.5 - 0.25);
                for (int64_t i = 0; i < n * C; ++i) dout[i] = (float)(uni() * 2 - 1);
                for (int64_t i = 0; i < L * T * F; ++i) {
                    if (half) ((uint16_t *)table)[i] = (uint16_t)(uni() * 65536.0) & 0x7BFF;  /* finite halves */
                    else ((float *)table)[i] = (float)(uni() * 2e-4 - 1e-4);
                }
                if (oracle_corners(&g, x, n, idx, w) || oracle_forward(&g, x, n, table, out) ||
                    oracle_backward(&g, x, n, dout, C, grad) || oracle_input_grad(&g, x, n, table, dout, C, dx)) {
                    ++fails;
                } else {
                    for (int64_t p = 0; p < n * L; ++p) {
                        double s = 0;
                        for (int64_t k = 0; k < K; ++k) s += w[p * K + k];
                        if (fabs(s - 1.0) > 1e-12) ++fails;
                    }
                    if (!half) {  /* <dout, forward(table)> == <backward(dout), table> */
                        double lhs = 0, rhs = 0, mag = 0;
                        for (int64_t i = 0; i < n * C; ++i) lhs += dout[i] * out[i], mag += fabs(dout[i] * out[i]);
                        for (int64_t i = 0; i < L * T * F; ++i) rhs += grad[i] * ((float *)table)[i];
                        if (fabs(lhs - rhs) > 1e-12 * (mag + 1e-30)) ++fails;
                    }
                    for (int64_t i = 0; i < n * D; ++i)
                        if (!isfinite(dx[i])) ++fails;
                }
                free(x), free(dout), free(table), free(out), free(grad), free(dx), free(idx), free(w);
            }
        }
    }
    if (fails) {
        fprintf(stderr, "oracle driver: %d failed checks\n", fails);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
