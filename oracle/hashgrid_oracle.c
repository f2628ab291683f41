/*
 * CPU oracle of the multiresolution hash-grid encoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant generator with the HIP library: everything below is written out
 * again from the pages' description of the method.
 *
 * Deliberately plain: one loop per level, per point, per corner, float64
 * accumulation, no blocking and no reordering beyond running independent
 * levels on separate OpenMP threads (each level owns disjoint output columns
 * and a disjoint gradient slice, and every sum is still taken in point order).
 *
 * Sources (web pages on Instant-NGP hash encoding):
 *  - "Speeding up NeRFace with Instant-NGP hash encoding" (ipipp.com), section 2,
 *    HashGridEncoder: resolution progression, per-level tables, spatial hash,
 *    voxel location, 8 corners, trilinear blend, level-major concatenation.
 *  - "Reproduce Instant-NGP hash encoding in PyTorch" (jsqmd.com), section 2.2
 *    hash_function (generic d-dimensional XOR hash) and section 3 HashEncoding
 *    (prime list for up to seven dimensions).
 *  - "Instant-NGP ... hash encoding" overview (ijyty.com), section 2.2, hash
 *    formula h(x) = (XOR_i x_i pi_i) mod T.
 * Readings where the pages disagree or are silent (scale x*N_l, not x*(N_l-1);
 * true trilinear weights; fp32 position; power-of-two T; accumulate into the
 * gradient buffer) are listed with the tests that pin them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_DIMS 7
#define ORACLE_MAX_LEVELS 64

typedef struct {
    int32_t n_dims;            /* D, number of input coordinates                     */
    int32_t n_levels;          /* L                                                  */
    int32_t n_features;        /* F, features per table entry                        */
    int32_t log2_table_size;   /* T = 2^log2_table_size entries per level            */
    int32_t base_resolution;   /* N_min                                              */
    int32_t finest_resolution; /* N_max                                              */
    int32_t table_is_half;     /* 0: float32 table, 1: IEEE binary16 bits (uint16)   */
} oracle_grid;

/* Primes of the spatial hash, one per input dimension, in the order the
 * jsqmd.com HashEncoding lists them; the first three are also the ones the
 * ipipp.com HashGridEncoder.hash uses for x, y and z. */
static const int64_t kPrimes[ORACLE_MAX_DIMS] = {
    1LL, 2654435761LL, 805459861LL, 3674653429LL, 2097192037LL, 1434869437LL, 2165219737LL};

static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_get_threads(void) { return g_threads; }

/* Level resolutions, ipipp.com HashGridEncoder.__init__:
 *   b = exp((ln N_max - ln N_min) / (L - 1)),  N_l = floor(N_min * b^l),
 * evaluated in IEEE float64 exactly as written (Python float semantics:
 * math.exp, math.log and float ** int, which is C pow).  With L == 1 the
 * formula divides by zero; the single level then takes N_min. */
int oracle_resolutions(int32_t n_levels, int32_t n_min, int32_t n_max, int32_t *res) {
    if (n_levels < 1 || n_levels > ORACLE_MAX_LEVELS || n_min < 1 || n_max < n_min) return -1;
    if (n_levels == 1) {
        res[0] = n_min;
        return 0;
    }
    double b = exp((log((double)n_max) - log((double)n_min)) / (double)(n_levels - 1));
    for (int l = 0; l < n_levels; ++l) res[l] = (int32_t)floor((double)n_min * pow(b, (double)l));
    return 0;
}

/* Spatial hash of one integer vertex (ipipp.com HashGridEncoder.hash,
 * jsqmd.com hash_function): XOR of coordinate times prime, taken in signed
 * 64-bit integers without wraparound as the PyTorch code does, then reduced
 * modulo T with Python's non-negative remainder. */
static int64_t spatial_hash(const int64_t *c, int dims, int64_t T) {
    int64_t h = 0;
    for (int d = 0; d < dims; ++d) h ^= c[d] * kPrimes[d];
    int64_t r = h % T;
    return r < 0 ? r + T : r;
}

/* IEEE 754 binary16 -> value, from the format's definition: sign bit,
 * 5-bit exponent with bias 15, 10-bit fraction; exponent 0 is subnormal
 * (fraction * 2^-24), exponent 31 is infinity or NaN. */
double oracle_half_to_double(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -v : v;
}

static double table_value(const oracle_grid *g, const void *table, int64_t l, int64_t e, int j) {
    int64_t T = (int64_t)1 << g->log2_table_size;
    int64_t at = (l * T + e) * g->n_features + j;
    if (g->table_is_half) return oracle_half_to_double(((const uint16_t *)table)[at]);
    return (double)((const float *)table)[at];
}

static int check_grid(const oracle_grid *g) {
    if (g->n_dims < 1 || g->n_dims > ORACLE_MAX_DIMS) return -1;
    if (g->n_levels < 1 || g->n_levels > ORACLE_MAX_LEVELS) return -1;
    if (g->n_features < 1 || g->log2_table_size < 1 || g->log2_table_size > 30) return -1;
    if (g->base_resolution < 1 || g->finest_resolution < g->base_resolution) return -1;
    return 0;
}

/* Voxel of point p at resolution N (ipipp.com HashGridEncoder.forward):
 * scaled = x * N as one float32 multiply, v = floor(scaled), frac = scaled - v. */
static void locate(const float *xp, int dims, int32_t N, int64_t *v, double *frac) {
    for (int d = 0; d < dims; ++d) {
        float scaled = xp[d] * (float)N;
        float fl = floorf(scaled);
        v[d] = (int64_t)fl;
        frac[d] = (double)scaled - (double)fl;
    }
}

/* Corner k of the voxel: offset bit of dimension d is bit (D-1-d) of k, so for
 * D = 3 the corners come in the pages' loop order dx outer, dz inner
 * (k = 4 dx + 2 dy + dz).  Its trilinear weight is the product over d of
 * frac_d where the corner sits on the upper side and 1 - frac_d otherwise. */
static double corner(const int64_t *v, const double *frac, int dims, int k, int64_t *c) {
    double w = 1.0;
    for (int d = 0; d < dims; ++d) {
        int up = (k >> (dims - 1 - d)) & 1;
        c[d] = v[d] + up;
        w *= up ? frac[d] : 1.0 - frac[d];
    }
    return w;
}

/* Per point, per level, per corner: hashed table index and interpolation
 * weight.  idx and w are [n][L][2^D]. */
int oracle_corners(const oracle_grid *g, const float *x, int64_t n, uint32_t *idx, double *w) {
    if (check_grid(g)) return -1;
    int32_t res[ORACLE_MAX_LEVELS];
    if (oracle_resolutions(g->n_levels, g->base_resolution, g->finest_resolution, res)) return -1;
    const int D = g->n_dims, K = 1 << D, L = g->n_levels;
    const int64_t T = (int64_t)1 << g->log2_table_size;
    for (int64_t p = 0; p < n; ++p) {
        for (int l = 0; l < L; ++l) {
            int64_t v[ORACLE_MAX_DIMS], c[ORACLE_MAX_DIMS];
            double frac[ORACLE_MAX_DIMS];
            locate(x + p * D, D, res[l], v, frac);
            for (int k = 0; k < K; ++k) {
                double wk = corner(v, frac, D, k, c);
                int64_t at = (p * L + l) * K + k;
                idx[at] = (uint32_t)spatial_hash(c, D, T);
                w[at] = wk;
            }
        }
    }
    return 0;
}

/* Forward encoding: out[p][l*F + j] = sum_k w_k * table[l][h(corner_k)][j],
 * the per-level blends concatenated level-major (ipipp.com torch.cat of the
 * per-level features).  out is [n][L*F] float64. */
int oracle_forward(const oracle_grid *g, const float *x, int64_t n, const void *table, double *out) {
    if (check_grid(g)) return -1;
    int32_t res[ORACLE_MAX_LEVELS];
    if (oracle_resolutions(g->n_levels, g->base_resolution, g->finest_resolution, res)) return -1;
    const int D = g->n_dims, K = 1 << D, L = g->n_levels, F = g->n_features;
    const int64_t T = (int64_t)1 << g->log2_table_size;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int l = 0; l < L; ++l) {
        for (int64_t p = 0; p < n; ++p) {
            int64_t v[ORACLE_MAX_DIMS], c[ORACLE_MAX_DIMS];
            double frac[ORACLE_MAX_DIMS];
            double acc[64];
            for (int j = 0; j < F; ++j) acc[j] = 0.0;
            locate(x + p * D, D, res[l], v, frac);
            for (int k = 0; k < K; ++k) {
                double wk = corner(v, frac, D, k, c);
                int64_t e = spatial_hash(c, D, T);
                for (int j = 0; j < F; ++j) acc[j] += wk * table_value(g, table, l, e, j);
            }
            for (int j = 0; j < F; ++j) out[p * (int64_t)L * F + (int64_t)l * F + j] = acc[j];
        }
    }
    return 0;
}

/* Backward: the gather above is linear in the table, so its adjoint scatters
 * dL/dout * w_k into every entry a corner hashed to (ipipp.com section 2: only
 * the sampled corners receive gradient).  grad is [L][T][F] float64 and is
 * ADDED to; dout is [n] rows of at least L*F floats, row stride dout_stride. */
int oracle_backward(const oracle_grid *g, const float *x, int64_t n, const float *dout,
                    int64_t dout_stride, double *grad) {
    if (check_grid(g)) return -1;
    int32_t res[ORACLE_MAX_LEVELS];
    if (oracle_resolutions(g->n_levels, g->base_resolution, g->finest_resolution, res)) return -1;
    const int D = g->n_dims, K = 1 << D, L = g->n_levels, F = g->n_features;
    const int64_t T = (int64_t)1 << g->log2_table_size;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int l = 0; l < L; ++l) {
        for (int64_t p = 0; p < n; ++p) {
            int64_t v[ORACLE_MAX_DIMS], c[ORACLE_MAX_DIMS];
            double frac[ORACLE_MAX_DIMS];
            locate(x + p * D, D, res[l], v, frac);
            for (int k = 0; k < K; ++k) {
                double wk = corner(v, frac, D, k, c);
                int64_t e = spatial_hash(c, D, T);
                for (int j = 0; j < F; ++j)
                    grad[((int64_t)l * T + e) * F + j] +=
                        wk * (double)dout[p * dout_stride + (int64_t)l * F + j];
            }
        }
    }
    return 0;
}

/* Gradient with respect to the points, dL/dx.  The pages imply it (ipipp.com
 * section 3 places a learned canonical-space transform in front of the
 * encoder, which needs it) but never write it down; it is the derivative of
 * the blend of oracle_forward.  Inside a voxel the blend is multilinear in
 * frac, and frac_d grows with x_d at the rate N_l (scaled = x * N_l), so
 *   d out[l*F + j] / d x_d = N_l * sum_k (d w_k / d frac_d) * table[l][h(c_k)][j]
 * where d w_k / d frac_d is +-1 (corner k on the upper / lower side in d) times
 * the weight factors of the other dimensions.  On a voxel face (frac_d = 0)
 * this is the derivative inside the voxel floor() chose, i.e. from above.
 * dx[p][d] = sum_l sum_j dout[p][l*F + j] * d out[l*F + j] / d x_d, summed in
 * level order; dx is [n][D] float64 and is WRITTEN. */
int oracle_input_grad(const oracle_grid *g, const float *x, int64_t n, const void *table,
                      const float *dout, int64_t dout_stride, double *dx) {
    if (check_grid(g)) return -1;
    int32_t res[ORACLE_MAX_LEVELS];
    if (oracle_resolutions(g->n_levels, g->base_resolution, g->finest_resolution, res)) return -1;
    const int D = g->n_dims, K = 1 << D, L = g->n_levels, F = g->n_features;
    const int64_t T = (int64_t)1 << g->log2_table_size;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t p = 0; p < n; ++p) {
        double acc[ORACLE_MAX_DIMS];
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int l = 0; l < L; ++l) {
            int64_t v[ORACLE_MAX_DIMS], c[ORACLE_MAX_DIMS];
            double frac[ORACLE_MAX_DIMS];
            locate(x + p * D, D, res[l], v, frac);
            for (int k = 0; k < K; ++k) {
                corner(v, frac, D, k, c);
                int64_t e = spatial_hash(c, D, T);
                /* s = dL/dout of this level dotted with the corner's features */
                double s = 0.0;
                for (int j = 0; j < F; ++j)
                    s += (double)dout[p * dout_stride + (int64_t)l * F + j] * table_value(g, table, l, e, j);
                for (int d = 0; d < D; ++d) {
                    double dw = 1.0;
                    for (int q = 0; q < D; ++q) {
                        int up = (k >> (D - 1 - q)) & 1;
                        if (q == d) dw *= up ? 1.0 : -1.0;
                        else dw *= up ? frac[q] : 1.0 - frac[q];
                    }
                    acc[d] += (double)res[l] * dw * s;
                }
            }
        }
        for (int d = 0; d < D; ++d) dx[p * D + d] = acc[d];
    }
    return 0;
}
