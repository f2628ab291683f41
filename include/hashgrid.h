/*
 * hashgrid.h -- C ABI of the MI355X (gfx950) multiresolution hash-grid encoder.
 *
 * The method (Instant-NGP style multiresolution hash encoding) is described on
 * the page "Speeding up NeRFace with Instant-NGP hash encoding" (ipipp.com),
 * section 2 and its HashGridEncoder listing, and on the Instant-NGP overview
 * (ijyty.com) section 2.2:
 *   - L levels with resolutions N_l = floor(N_min * b^l),
 *     b = exp((ln N_max - ln N_min) / (L - 1)), evaluated in IEEE float64;
 *   - one table of T = 2^log2_table_size entries of F features per level;
 *   - a point x is scaled by N_l, the 2^D corners of its voxel are hashed with
 *     h(c) = (c_0 * 1) XOR (c_1 * 2654435761) XOR (c_2 * 805459861) mod T,
 *     the corner features are gathered and blended with multilinear weights;
 *   - the per-level F-vectors are concatenated level-major into L*F outputs.
 * Other input dimensions (jsqmd.com HashEncoding, section 3: 2-D images,
 * 4-D space-time) hash c_3 with 3674653429, the fourth of that page's primes;
 * its section 4 runs F from 2 to 4.  D = 3, F = 2 (the pages' standard
 * encoder) has tuned kernels; the other shapes run generic ones.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers (memory of the current HIP device)
 *     unless the comment says "host".  The caller owns every buffer; the library
 *     allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work on it; they never synchronise.  Results are ready when
 *     the stream's work has completed.
 *   - Return value: HG_OK (0) on success, a negative HG_E* code otherwise; the
 *     thread-local text of the last failure is returned by hashgrid_last_error().
 *     Argument checks happen on the host before anything is enqueued, so a
 *     rejected call has no effect.
 *   - n == 0 is valid and does nothing (pointers are then not inspected).
 *   - Points outside [0,1)^D are processed by the same formula (the voxel index
 *     is floor(x * N_l) as a signed 32-bit integer and the hash wraps in uint32),
 *     and every table access is masked into [0, T): no input can make the
 *     library read or write out of bounds.  Inputs with |x * N_l| >= 2^31, NaN
 *     or Inf give unspecified (but in-bounds) results.
 */
#ifndef HASHGRID_H
#define HASHGRID_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HASHGRID_ABI_VERSION 2

/* Return codes. */
#define HG_OK 0
#define HG_EINVAL (-1)       /* bad config, pointer, alignment, size or stride */
#define HG_EUNSUPPORTED (-2) /* valid but not built: F, D or dtype combination */
#define HG_EHIP (-3)         /* the HIP runtime reported an error on launch     */

/* Element types. */
#define HG_F32 0 /* IEEE binary32                                        */
#define HG_F16 1 /* IEEE binary16 (storage only; all arithmetic is fp32) */

/* Grid description.  Field names follow the pages' constructor arguments
 * (n_levels, n_features_per_level, log2_hashmap_size, base_resolution,
 * finest_resolution). */
typedef struct hg_config {
    int32_t n_dims;            /* D, coordinates per point: 1..4                                */
    int32_t n_levels;          /* L, 1..64                                                      */
    int32_t n_features;        /* F, features per table entry: 1, 2, 4 or 8                     */
    int32_t log2_table_size;   /* T = 2^log2_table_size entries per level, 1..28                */
    int32_t base_resolution;   /* N_min >= 1                                                    */
    int32_t finest_resolution; /* N_max, N_min <= N_max < 2^24                                  */
    int32_t table_dtype;       /* HG_F32 or HG_F16                                              */
    int32_t grad_dtype;        /* HG_F32, or HG_F16 (binned backward only, see hashgrid_backward) */
} hg_config;

/* Version of this ABI (HASHGRID_ABI_VERSION of the built library). */
int hashgrid_abi_version(void);

/* Text of the last failure on the calling thread ("" if none).  Valid until
 * the next call on the same thread. */
const char *hashgrid_last_error(void);

/* Level resolutions N_0..N_{L-1} (ipipp.com HashGridEncoder.__init__: the
 * float64 expression floor(N_min * b^l); with L == 1 the only level is N_min).
 * res_out: HOST int32[L].  Errors: HG_EINVAL on a bad config or NULL. */
int hashgrid_resolutions(const hg_config *cfg, int32_t *res_out);

/* Bytes of device workspace with which hashgrid_forward stages the encoding
 * level-major before writing the rows: L * n * F * 4 rounded up to 256
 * (32 MiB for L = 16, F = 2, n = 2^18), twice that for a D = 3, F = 2 grid
 * whose levels are gathered one table half per pass (below), whose second
 * half then writes its own stage.  *bytes_out is a HOST size_t.
 * Errors: HG_EINVAL, HG_EUNSUPPORTED. */
int hashgrid_forward_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out);

/* Forward encoding (ipipp.com section 2 and HashGridEncoder.forward).
 *   x     : float32 [n][D], row-major (AoS), 4-byte aligned.
 *   table : [L][T][F] of cfg->table_dtype, contiguous, level-major; aligned to
 *           F * sizeof(element) (8 bytes for fp32 F=2, 4 bytes for fp16 F=2).
 *   out   : float32, row p holds the L*F encoded features of point p at
 *           out[p * out_row_stride + l * F + j]; columns beyond L*F are not
 *           touched, so the encoding can be written into a wider buffer.
 *           4-byte aligned; out_row_stride >= L*F (elements).
 *   workspace, workspace_bytes : caller-owned device scratch, 256-byte
 *           aligned, contents clobbered; may be NULL.  With at least
 *           hashgrid_forward_workspace_size bytes each level's encodings are
 *           first written level-major (whole cache lines, so the level's table
 *           stays in L2) and then transposed into the rows; without it every
 *           level writes its F values straight into the rows.  F = 8 grids
 *           always write the rows directly (32 bytes per level and row).
 *           Results are identical either way, except on the levels the
 *           blend above gathers in two halves.  Concurrent calls must not share
 *           a workspace.
 *   The blend of level l is sum_k w_k * table[l][h(corner_k)][j] computed in
 *   fp32, with w_k the trilinear weight of corner k.  For the D = 3, F = 2
 *   grid with a workspace, a level whose table exceeds 4 MiB (fp32
 *   T >= 2^20, binary16 T >= 2^21) is gathered one table half per pass, so
 *   that the half fits one XCD's L2, and the two partial blends are added
 *   (while transposing when the workspace holds two stages, in place when it
 *   holds one; the sums are the same either way): such levels round
 *   differently from the one-pass direct path, by a few fp32 roundings of the
 *   blend (measured: 1.5e-7 of the largest table value).  With a workspace
 *   and from 2^21 points (HG_TUNE_FWD_DENSE), the coarsest levels whose
 *   vertex grids fit 128 KiB of LDS together are blended from LDS copies of
 *   them, with the same arithmetic as the one-pass gather (same bits).
 * Errors: HG_EINVAL (config, NULL, alignment, n < 0, stride), HG_EUNSUPPORTED,
 *         HG_EHIP. */
int hashgrid_forward(const hg_config *cfg, const float *x, int64_t n, const void *table,
                     float *out, int64_t out_row_stride, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Bytes of device workspace that let hashgrid_backward route the whole
 * gradient of n points through its binned (atomic-free) path at full speed:
 * per level, 48 * ceil(n / 1024) * 1024 bytes of records plus small counters
 * (about 12.9 MB for n = 2^18) for the D = 3, F = 2 grid; for other shapes
 * (2 + F) * 4 bytes per corner pair, 2^(D-1) pairs per point -- times the
 * number of levels binned together.
 * That group is sized so its records fit the MI355X last-level cache (the
 * HG_TUNE_BWD_GROUP_MIB budget, 160 MiB by default: 8 levels for n = 2^18,
 * about 103 MB) when such groups still give the accumulate kernel at least
 * 1024 workgroups; otherwise (larger batches: 2^20 points and up at T = 2^19)
 * it holds all levels, e.g. about 3.1 GiB for n = 2^22 and L = 16.
 * *bytes_out is a HOST size_t.  A workspace of at least
 * *min_bytes_out (one level's share; may be NULL) also works -- the levels
 * are then processed in smaller groups.  Returns 0 bytes when the
 * configuration has no binned path (more than 4096 partitions: T > 2^25 for
 * the D = 3, F = 2 grid, partitions of 8192 / F entries for other shapes; or
 * n >= 2^29).
 * Errors: HG_EINVAL, HG_EUNSUPPORTED. */
int hashgrid_backward_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out,
                                     size_t *min_bytes_out);

/* Backward: gradient of the encoding with respect to the tables (ipipp.com
 * section 2 -- only the corners a point sampled receive gradient -- i.e. the
 * adjoint of the forward gather).
 *   x      : float32 [n][D], the points of the forward call.
 *   dout   : float32, dL/dout with row stride dout_row_stride >= L*F elements;
 *            element (p, l*F + j) is read, other columns are ignored.
 *   dtable : float32 [L][T][F] (binary16 with grad_dtype HG_F16, below),
 *            4-byte aligned.  ACCUMULATED INTO:
 *            dtable[l][h(corner_k)][j] += w_k * dout[p][l*F + j] for every point,
 *            level and corner.  The caller zeroes the buffer when it wants the
 *            gradient of one batch alone.  On the binned path the D = 3, F = 2
 *            grid stores each corner pair's products w_y w_z dout with 20
 *            significant bits (relative error <= 2^-21), each contribution is
 *            rounded to 64-bit fixed point (a step below 2^-29 max|dout| of the
 *            level, taken over its finite values) and the integer sums do not
 *            depend on the order of the additions: for points in [0,1)^D the
 *            result is reproducible bit for bit.  The atomic path (no
 *            workspace) first sums, per workgroup of 4096 points, the levels
 *            of at most 16384 values (T F, or the vertex grid (N_l + 1)^D F)
 *            in the same 64-bit fixed point in LDS and adds each sum with one
 *            fp32 atomic; other levels it scatters with fp32 atomics in an
 *            unspecified order, so its results can differ from run to run in
 *            the last bits.  Non-finite dout values (NaN, +-Inf) are never
 *            summed in fixed point: their contributions are added with fp32
 *            atomics, so they reach the entries they touch as IEEE arithmetic
 *            has them (NaN stays NaN, Inf + finite = Inf, Inf - Inf = NaN) and
 *            the other entries keep the precision of the finite values.  Both
 *            paths
 *            first sum, inside each wavefront, runs of consecutive points that
 *            share a voxel (ray samples at coarse levels) for the D = 3, F = 2
 *            grid.
 *   workspace, workspace_bytes : caller-owned device scratch (contents need
 *            not be initialised and are clobbered).  With at least the minimum
 *            of hashgrid_backward_workspace_size and a 16-byte aligned dtable
 *            the gradient is binned by table partition and accumulated in
 *            on-chip memory with no global atomics; with NULL or too little
 *            workspace it is scattered with fp32 global atomics (correct, but
 *            an order of magnitude slower on MI355X).  Concurrent calls must
 *            not share a workspace.
 * grad_dtype HG_F16 (a binary16 gradient buffer beside binary16 tables,
 * jsqmd.com section 5's half-precision tip): the binned path sums each
 * partition in fixed point as above and rounds every entry once, from the fp32
 * sum of its old value and the partition's sum to binary16 (relative error
 * <= 2^-11 of the entry; magnitudes past 65504 become +-Inf).  The few
 * contributions it adds directly (non-finite dout values, corners whose pair
 * straddles two partitions, run sums past fp32) use packed binary16 atomics,
 * each addition rounded.  For points in [0,1)^D such pairs are rare (v_x + 1
 * a multiple of the partition size, which needs N_l >= 8192 / F, 4096 for the
 * D = 3, F = 2 grid up to T = 2^20), so the bound above holds.  Outside the
 * cube every point with v_x = -1 (x_0 in [-1/N_l, 0)) straddles, so at coarse
 * levels many points can reach one entry, each addition rounded to binary16.  Summing with atomics alone would round at every
 * addition, an error that grows with the additions an entry takes, so HG_F16 needs
 * the binned path: without a workspace of at least the minimum, with a dtable
 * that is not 16-byte aligned, or on a grid without a binned path the call
 * returns HG_EUNSUPPORTED and changes nothing.
 * Errors: as hashgrid_forward. */
int hashgrid_backward(const hg_config *cfg, const float *x, int64_t n, const float *dout,
                      int64_t dout_row_stride, float *dtable, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Allocation-free variant of hashgrid_backward, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same table gradient, accumulated into
 * dtable (arguments as hashgrid_backward), with the binned path's workspace
 * taken from a fixed scratch array of HASHGRID_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on each device it runs on until the process ends.
 * Nothing is allocated or freed per call.  Levels are binned in groups that
 * fit the scratch (4 levels at a time for n = 2^18 on the D = 3, F = 2 grid),
 * so the result equals hashgrid_backward's binned result; grids without a
 * binned path take the atomic scatter, as hashgrid_backward does without a
 * workspace.  Every call on one device shares that device's scratch: calls
 * that overlap on a device (other streams, other host threads) race, and the
 * caller must order them.  Errors: as hashgrid_backward, and HG_EINVAL when
 * one level's records of n points exceed the scratch (the message gives the
 * largest n of the grid: about 1.37 * 10^6 points for D = 3, F = 2 at
 * T = 2^19); HG_EHIP when the scratch's device address cannot be resolved. */
#define HASHGRID_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int hashgrid_backward_noalloc(const hg_config *cfg, const float *x, int64_t n, const float *dout,
                              int64_t dout_row_stride, float *dtable, void *stream);

/* Debug export of the corner table indices and interpolation weights.
 *   idx : uint32 [n][L][2^D]  -- hashed index in [0, T) of corner k of level l,
 *   w   : float32 [n][L][2^D] -- its fp32 weight,
 * with corners ordered k = 4*dx + 2*dy + dz (the pages' loop nesting, x outer).
 * Either pointer may be NULL to skip that output.  Errors: as hashgrid_forward. */
int hashgrid_debug_corners(const hg_config *cfg, const float *x, int64_t n, uint32_t *idx,
                           float *w, void *stream);

/* MLP head after the encoder: the NeRFace head of ipipp.com (section 3
 * listing), Linear(32, 64), ReLU, Linear(64, 64), ReLU, Linear(64, 4) with
 * biases,  y = W3 relu(W2 relu(W1 u + b1) + b2) + b3,  where u = e is the
 * 32-wide encoding of a point (grids with D = 3, F = 2, L = 16).  With
 * coord_inputs = 3 it is instead the TinyNeRF head of the jsqmd.com page
 * (section 4: the network concatenates the raw point before its hash
 * features, then Linear(35, 64) and the same two layers): u = [x, e], the
 * point's 3 coordinates first, and W1 is [64][35].  It runs on the matrix
 * cores: binary16 operands (u -- coordinates included --, the hidden
 * activations and, in the backward, dL/dy and the pre-activation gradients
 * are rounded to binary16 where they enter a product), fp32 accumulation.
 * The encoding is computed once, in the forward, into a binary16 stage the
 * backward reuses.  Weights are binary16 [out][in] (nn.Linear layout),
 * biases fp32. */
typedef struct {
    const void *w1;       /* binary16 [64][32], or [64][35] with coord_inputs = 3; 8-byte aligned */
    const float *b1;      /* [64]                                                                 */
    const void *w2;       /* binary16 [64][64]                                                     */
    const float *b2;      /* [64]                                                                 */
    const void *w3;       /* binary16 [4][64]                                                      */
    const float *b3;      /* [4]                                                                  */
    int32_t coord_inputs; /* 0: u = e (NeRFace head); 3: u = [x, e] (TinyNeRF head); else HG_EINVAL */
} hg_mlp_params;

/* fp32 gradients of the weights and biases, same shapes (dw1 [64][32] or
 * [64][35]); ACCUMULATED.  The points are inputs: the head gives no gradient
 * to x (the table backward's rule; dL/dx is hashgrid_input_grad's). */
typedef struct {
    float *dw1, *db1, *dw2, *db2, *dw3, *db3;
} hg_mlp_grads;

/* Workspace sizes of the MLP head over n points (HOST size_t outputs):
 *   *stage_bytes_out : the binary16 encoding stage, n * 64 bytes (rounded);
 *                      written by hashgrid_mlp_forward, read by the backward;
 *   *bwd_bytes_out   : the backward's workspace: dL/de (n * 128 bytes), the
 *                      per-wave weight-gradient partials, and the binned table
 *                      backward's workspace.
 * Errors: HG_EINVAL, HG_EUNSUPPORTED (a grid other than D = 3, L * F = 32). */
int hashgrid_mlp_workspace_size(const hg_config *cfg, int64_t n, size_t *stage_bytes_out, size_t *bwd_bytes_out);

/* Forward of encoder + MLP head: y [n][4] fp32 (16-byte aligned), WRITTEN.
 *   x, table : as hashgrid_forward.
 *   stage    : device buffer of stage_bytes >= n * 64 (256-byte aligned) that
 *              receives the binary16 encoding [L][n][2]; keep it for the
 *              backward.
 * Errors: as hashgrid_forward, plus HG_EINVAL for parameter pointers. */
int hashgrid_mlp_forward(const hg_config *cfg, const float *x, int64_t n, const void *table,
                         const hg_mlp_params *params, float *y, void *stage, size_t stage_bytes, void *stream);

/* Backward of encoder + MLP head for upstream dy = dL/dy [n][4] fp32
 * (16-byte aligned): adds the weight and bias gradients into *grads and the
 * table gradient into dtable ([L][T][F] fp32, or binary16 with grad_dtype
 * HG_F16, as hashgrid_backward).
 *   stage     : the stage the forward of the same x, table and params wrote.
 *   workspace : hashgrid_mlp_workspace_size's bwd bytes (256-byte aligned);
 *               at least the dL/de rows and partials are required, and with
 *               less than the full size the table gradient takes the smaller
 *               binned groups or the atomic scatter, as in hashgrid_backward.
 *               A binary16 dtable (grad_dtype HG_F16) needs the binned
 *               backward's minimum beyond the head's part; without it the
 *               call returns HG_EUNSUPPORTED before anything is enqueued.
 * The weight gradients are summed per wave in registers and the wave
 * partials added in a fixed order: results do not depend on scheduling.
 * Errors: as hashgrid_backward. */
int hashgrid_mlp_backward(const hg_config *cfg, const float *x, int64_t n, const void *stage,
                          const hg_mlp_params *params, const float *dy, const hg_mlp_grads *grads, float *dtable,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace that let hashgrid_input_grad stage per-level
 * partial sums level-major: L * n * D * 4, rounded up to 256, plus for the
 * D = 3, F = 2 grid L * n * 2 * 4 for a level-major copy of the upstream rows
 * (a workspace holding only the stage also works).  0 for D <= 2: a level
 * there holds at most (N_l + 1)^2 corners, the tables stay in cache, and the
 * point-major path is faster with or without a workspace.  *bytes_out is a
 * HOST size_t.  Errors: HG_EINVAL, HG_EUNSUPPORTED. */
int hashgrid_input_grad_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out);

/* Gradient of the loss with respect to the points, dL/dx.  The pages imply
 * it (ipipp.com section 3 places a learned canonical-space transform in front
 * of the encoder) but do not write it; it is the derivative of the forward's
 * blend: inside a voxel the blend is multilinear in the fractions f and f_d
 * moves with x_d at rate N_l, so
 *   dx[p][d] = sum_l N_l sum_k (b_d ? 1 : -1) prod_{e != d} (b_e ? f_e : 1 - f_e)
 *              * sum_j dout[p][l*F + j] * table[l][h(c_k)][j]
 * over the corners c_k = v + b of the voxel floor() picked (on a voxel face,
 * the derivative from that voxel), summed over levels in level order in fp32.
 *   x, table : as hashgrid_forward;  dout : as hashgrid_backward.
 *   dx       : float32 [n][D], 4-byte aligned; WRITTEN (not accumulated).
 *   workspace: NULL, or hashgrid_input_grad_workspace_size bytes (256-byte
 *              aligned) to run level-major (each level's table stays in L2)
 *              and then sum the levels; without it (and for D <= 2) one thread
 *              walks all levels of a point.  The two give identical results.
 *              Concurrent calls must not share a workspace.
 * Errors: as hashgrid_forward. */
int hashgrid_input_grad(const hg_config *cfg, const float *x, int64_t n, const void *table, const float *dout,
                        int64_t dout_row_stride, float *dx, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Adam update of the tables (ipipp.com section 4: Adam, no weight decay on
 * the hash tables, whose learning rate is 5-10x the MLP's per section 3;
 * ijyty.com overview section 4: torch.optim.Adam).  The algorithm is Adam as
 * published (Kingma and Ba 2015): m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2,
 * param -= lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps), in fp32, for
 * every one of the count entries (entries with a zero gradient still move,
 * as in torch.optim.Adam).
 *   opt       : host struct; step is the 1-based index t of this update.  The
 *               hyperparameters are the fp32 values given (1 - beta and the
 *               bias corrections are formed from them in double).
 *   param, m, v, grad : fp32 device arrays of count elements (the [L][T][F]
 *               tables, their two moments -- zero before step 1 -- and the
 *               gradient hashgrid_backward accumulated), 4-byte aligned;
 *               16-byte alignment and count % 4 == 0 take the vector path.
 *   param_f16 : optional device array of count binary16 values that receives
 *               the updated tables rounded to nearest-even (the fp16 tables a
 *               fp16-table forward reads), or NULL.
 *   flags     : HG_ADAM_ZERO_GRAD writes 0 into grad after reading it, ready
 *               for the next backward, which accumulates.
 * Errors: HG_EINVAL (NULL pointer, count < 0, step < 1, lr/eps not finite,
 * betas outside [0, 1)), HG_EHIP. */
typedef struct {
    float lr;      /* step size (alpha)                                      */
    float beta1;   /* decay of the first moment, in [0, 1)                   */
    float beta2;   /* decay of the second moment, in [0, 1)                  */
    float eps;     /* added to the root of the corrected second moment, >= 0 */
    int32_t step;  /* t >= 1                                                 */
} hg_adam;
#define HG_ADAM_ZERO_GRAD 1
int hashgrid_adam_step(const hg_adam *opt, int64_t count, float *param, float *m, float *v,
                       float *grad, void *param_f16, int32_t flags, void *stream);

/* Performance knobs (launch shapes).  Two change results within rounding:
 * HG_TUNE_FWD_LANES (the order in which the blend's eight terms are added) and
 * HG_TUNE_BWD_BINNED (fixed-point binned accumulation or fp32 atomics, whose
 * order is unspecified), as do the atomic path's HG_TUNE_BWD_LANES shapes,
 * and HG_TUNE_FWD_STAGED on levels above 4 MiB (the staged forward gathers
 * those in two halves).  The others give identical results.  Process-wide;
 * not thread-safe against
 * concurrent launches.  Returns HG_EINVAL for an unknown key or an
 * out-of-range value. */
#define HG_TUNE_FWD_LANES 0    /* lanes per (point, level) in the forward: 1 or 2        */
#define HG_TUNE_BWD_LANES 1    /* lanes per (point, level) in the backward: 1, 2 or 4    */
#define HG_TUNE_CHUNK_POINTS 2 /* points per workgroup work item: 64..65536, power of 2  */
#define HG_TUNE_XCD_MAP 3      /* 1: give each XCD its own levels, 0: plain linear order */
#define HG_TUNE_BWD_BINNED 4   /* 1: binned backward when the workspace allows, 0: atomics */
#define HG_TUNE_FWD_UNROLL 5   /* points per lane pair in flight in the forward: 1, 2 or 4 */
#define HG_TUNE_FWD_NT 6       /* 1: non-temporal point reads and output writes         */
#define HG_TUNE_FWD_STAGED 7   /* 1: stage the forward level-major when given workspace */
#define HG_TUNE_BWD_PART_LOG2 8 /* log2 entries per binned-backward partition: 11..13, 0 = by T */
#define HG_TUNE_BWD_GROUP_MIB 9 /* record MiB per binned level group (levels binned and
                                   accumulated together), 0 = all levels in one group   */
#define HG_TUNE_BWD_DENSE 10    /* atomic backward: 1 sums levels of at most 16384 values
                                   (T * F, or the vertex grid (N_l + 1)^D * F) in LDS per
                                   workgroup first, 0 scatters every level directly     */
#define HG_TUNE_FWD_SPLIT_KIB 11 /* staged D = 3, F = 2 forward: levels whose table exceeds
                                   this many KiB are gathered one table half per pass
                                   (64..2^20; 0 = never); 4096 by default              */
#define HG_TUNE_FWD_DENSE 12    /* staged D = 3, F = 2 forward and the MLP head's stage:
                                   blend the coarsest levels whose vertex grids or tables
                                   fit 128 KiB of LDS together from LDS (same bits as the
                                   gather): 1 (default) from 2^21 points, 2 always,
                                   0 never                                             */
#define HG_TUNE_FWD_ORDER 13    /* staged D = 3, F = 2 forward: encode the points in the
                                   order of a coarse cell (16^3 cells, Morton order) and
                                   write each row back to its point's position (same
                                   bits; the forward workspace grows by about 16 bytes
                                   per point): 0 (default) never, 1 from 2^18 points,
                                   2 always.  Pays on uniform batches (7 % at 2^18
                                   points, 17 % at 2^22); costs on batches already in a
                                   coherent order, such as ray samples (7 % at 2^20) */
int hashgrid_tune(int key, int value);
int hashgrid_tune_get(int key);

#ifdef __cplusplus
}
#endif

#endif /* HASHGRID_H */
