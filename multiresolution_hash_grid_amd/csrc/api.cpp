// Host side of libhashgrid: the C ABI declared in include/hashgrid.h --
// argument checks, level resolutions, work decomposition and kernel launch.
// No device memory is allocated here and nothing synchronises the stream.
#include "hashgrid.h"

#include <math.h>
#include <cmath>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "hashgrid_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return HG_OK;
}

struct Tuning {
    int fwd_lanes = 2;
    int bwd_lanes = 4;
    int chunk_points = 1024;
    int xcd_map = 1;
    int bwd_binned = 1;
    int fwd_unroll = 4;
    int fwd_nt = 0;
    int fwd_staged = 1;
    int bwd_part_log2 = 0;  // 0: by table size
    int bwd_group_mib = 160;  // record bytes per binned level group, 0: all levels at once
    int bwd_dense = 1;        // atomic backward: sum small levels in LDS first
    int fwd_split_kib = 4096; // staged gather of levels above this table size: one half per pass
    int fwd_dense = 1;        // staged forward: blend levels that fit LDS from LDS (1: from kFwdDenseMinPoints)
    int fwd_order = 0;        // staged forward: order the points by a coarse cell (1: from kFwdOrderMinPoints)
};
Tuning g_tune;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Level resolutions: ipipp.com HashGridEncoder.__init__, the float64
// expression floor(N_min * b^l) with b = exp((ln N_max - ln N_min) / (L - 1)).
void resolutions(const hg_config &c, int32_t *res) {
    if (c.n_levels == 1) {
        res[0] = c.base_resolution;
        return;
    }
    const double b = exp((log((double)c.finest_resolution) - log((double)c.base_resolution)) /
                         (double)(c.n_levels - 1));
    for (int l = 0; l < c.n_levels; ++l) res[l] = (int32_t)floor((double)c.base_resolution * pow(b, (double)l));
}

int check_config(const hg_config *c) {
    if (!c) return fail(HG_EINVAL, "config is NULL");
    if (c->n_levels < 1 || c->n_levels > hg::kMaxLevels)
        return fail(HG_EINVAL, "n_levels %d outside 1..%d", c->n_levels, hg::kMaxLevels);
    if (c->log2_table_size < 1 || c->log2_table_size > 28)
        return fail(HG_EINVAL, "log2_table_size %d outside 1..28", c->log2_table_size);
    if (c->base_resolution < 1) return fail(HG_EINVAL, "base_resolution %d < 1", c->base_resolution);
    if (c->finest_resolution < c->base_resolution || c->finest_resolution >= (1 << 24))
        return fail(HG_EINVAL, "finest_resolution %d outside [base_resolution, 2^24)", c->finest_resolution);
    if (c->n_dims < 1 || c->n_features < 1) return fail(HG_EINVAL, "n_dims and n_features must be >= 1");
    if (c->table_dtype != HG_F32 && c->table_dtype != HG_F16)
        return fail(HG_EINVAL, "table_dtype %d is neither HG_F32 nor HG_F16", c->table_dtype);
    if (c->grad_dtype != HG_F32 && c->grad_dtype != HG_F16)
        return fail(HG_EINVAL, "grad_dtype %d is neither HG_F32 nor HG_F16", c->grad_dtype);
    if (c->n_dims > 4) return fail(HG_EUNSUPPORTED, "n_dims %d: 1..4 are built", c->n_dims);
    if (c->n_features != 1 && c->n_features != 2 && c->n_features != 4 && c->n_features != 8)
        return fail(HG_EUNSUPPORTED, "n_features %d: 1, 2, 4 and 8 are built", c->n_features);
    return HG_OK;
}

int plan(const hg_config &c, int64_t n, hg::LaunchParams &lp) {
    lp.n_levels = c.n_levels;
    lp.log2_table_size = c.log2_table_size;
    lp.mask = (uint32_t)((1ull << c.log2_table_size) - 1);
    lp.chunk_pts = g_tune.chunk_points;
    const int64_t chunks = (n + lp.chunk_pts - 1) / lp.chunk_pts;
    if (chunks * c.n_levels > ((int64_t)1 << 30))
        return fail(HG_EINVAL, "n = %lld: too many points for one call", (long long)n);
    lp.chunks = (int32_t)chunks;
    lp.items = lp.chunks * c.n_levels;
    lp.per_xcd = (lp.items + hg::kNumXcd - 1) / hg::kNumXcd;
    lp.xcd_map = g_tune.xcd_map;
    resolutions(c, lp.res);
    // Levels ordered by (l mod 8, l): the contiguous run of work items an XCD
    // receives then mixes coarse and fine levels (L = 16: levels x and x + 8).
    int pos = 0;
    for (int r = 0; r < hg::kNumXcd; ++r)
        for (int l = r; l < c.n_levels; l += hg::kNumXcd) lp.level_order[pos++] = (int8_t)l;
    return HG_OK;
}

// Keeps the work items of the levels flagged in keep[] (their order
// unchanged); returns how many levels remain.
int restrict_levels(hg::LaunchParams &lp, const bool *keep) {
    int pos = 0;
    for (int i = 0; i < lp.n_levels; ++i) {
        const int l = lp.level_order[i];
        if (keep[l]) lp.level_order[pos++] = (int8_t)l;
    }
    lp.items = lp.chunks * pos;
    lp.per_xcd = (lp.items + hg::kNumXcd - 1) / hg::kNumXcd;
    return pos;
}

// Levels of the atomic backward summed in LDS first: the table, or else the
// level's whole vertex grid (N_l + 1)^D, holds at most kDenseVals values.
void dense_levels(const hg_config &c, const hg::LaunchParams &lp, hg::DenseLevels &dl, bool *sparse) {
    dl.count = 0;
    dl.max_vals = 0;
    for (int l = 0; l < c.n_levels; ++l) {
        sparse[l] = true;
        if (!g_tune.bwd_dense) continue;
        const int64_t table_vals = ((int64_t)1 << c.log2_table_size) * c.n_features;
        int64_t vertex_vals = c.n_features;
        for (int d = 0; d < c.n_dims && vertex_vals <= hg::kDenseVals; ++d) vertex_vals *= (int64_t)lp.res[l] + 1;
        int64_t vals;
        if (table_vals <= hg::kDenseVals) {
            dl.by_vertex[dl.count] = 0;
            vals = table_vals;
        } else if (vertex_vals <= hg::kDenseVals) {
            dl.by_vertex[dl.count] = 1;
            vals = vertex_vals;
        } else {
            continue;
        }
        sparse[l] = false;
        dl.level[dl.count++] = (int8_t)l;
        dl.max_vals = std::max<int32_t>(dl.max_vals, (int32_t)vals);
    }
}

// Levels of the staged D = 3, F = 2 forward blended from LDS: from the
// coarsest up, each level's vertex grid (N_l + 1)^3, or else its table, as
// long as their entries fit kFwdDenseBytes together.  keep[l] is left true
// for the levels the gather takes.  The copies cost a fixed ~8 us a call,
// recovered from about 2^20 uniform points (measured at 2^18: +3 %, 2^20:
// -3 %, 2^22: -4 % fp32 and -11 % with the binary16 stage of the MLP head);
// ray-ordered points, whose coarse gathers already share lines, lose 2 % at
// 2^20.  So the default takes them from kFwdDenseMinPoints points.
constexpr int64_t kFwdDenseMinPoints = (int64_t)1 << 21;
void fwd_dense_levels(const hg_config &c, int64_t n, const hg::LaunchParams &lp, hg::DenseLevels &dl, bool *keep) {
    dl.count = 0;
    dl.max_vals = 0;
    const int64_t esize = c.table_dtype == HG_F32 ? 8 : 4;
    const bool on = g_tune.fwd_dense == 2 || (g_tune.fwd_dense == 1 && n >= kFwdDenseMinPoints);
    int64_t room = on ? hg::kFwdDenseBytes / esize : 0;
    for (int l = 0; l < c.n_levels; ++l) {
        keep[l] = true;
        const int64_t table_entries = (int64_t)1 << c.log2_table_size;
        const int64_t r = (int64_t)lp.res[l] + 1;
        const int64_t vertex_entries = r <= 4096 ? r * r * r : INT64_MAX;
        const int64_t entries = std::min(table_entries, vertex_entries);
        if (entries > room) continue;
        room -= entries;
        keep[l] = false;
        dl.by_vertex[dl.count] = vertex_entries < table_entries ? 1 : 0;
        dl.level[dl.count++] = (int8_t)l;
        dl.max_vals += (int32_t)entries;
    }
}

// Binned backward layout; returns false when the configuration has no binned
// path (partition count or record count beyond the kernels' index widths).
bool plan_binned(const hg_config &c, int64_t n, hg::BinParams &bp) {
    const bool std_shape = c.n_dims == 3 && c.n_features == 2;
    int want, tile_pts, rec_per_tile, rec_bytes;
    if (std_shape) {
        // Partitions of 2^12 entries (64 KB of 64-bit accumulators, 1024-thread
        // owners, two per CU) for tables up to 2^20 entries; 2^13 (128 KB, one
        // per CU) for larger tables, whose runs per tile would otherwise get short.
        want = g_tune.bwd_part_log2 ? g_tune.bwd_part_log2 : (c.log2_table_size <= 20 ? 12 : 13);
        tile_pts = hg::kBinTile;
        rec_per_tile = hg::kBinTile * 4;
        rec_bytes = hg::kRecordBytes;
    } else {
        want = hg::generic_s_log2(c.n_features);
        tile_pts = hg::generic_tile(c.n_dims, c.n_features);
        rec_per_tile = hg::generic_rec_per_tile(c.n_dims, c.n_features);
        rec_bytes = hg::generic_rec_bytes(c.n_features);
    }
    const int s_log2 = c.log2_table_size < want ? c.log2_table_size : want;
    const int64_t parts = (int64_t)1 << (c.log2_table_size - s_log2);
    const int64_t tiles = (n + tile_pts - 1) / tile_pts;
    if (parts > hg::kMaxParts || n >= ((int64_t)1 << 29)) return false;
    bp.level0 = 0;
    bp.group = c.n_levels;
    bp.tiles = (int32_t)tiles;
    bp.parts = (int32_t)parts;
    bp.s_log2 = s_log2;
    bp.log2_table_size = c.log2_table_size;
    bp.mask = (uint32_t)((1ull << c.log2_table_size) - 1);
    bp.tile_pts = tile_pts;
    bp.n = n;
    bp.level_records = tiles * rec_per_tile;
    bp.rec_per_tile = rec_per_tile;
    bp.rec_bytes = rec_bytes;
    bp.grad_f16 = c.grad_dtype == HG_F16;
    resolutions(c, bp.res);
    return true;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The D = 3, F = 2 grid of the pages' standard encoder has tuned kernels
// (lane pairs, staged forward, binned backward); other shapes take the
// generic ones.
bool standard_shape(const hg_config &c) { return c.n_dims == 3 && c.n_features == 2; }

// The staged forward of the D = 3, F = 2 grid gathers levels whose table
// exceeds the split threshold one half per pass.
bool split_forward(const hg_config &c) {
    const size_t level_bytes = (size_t)(c.table_dtype == HG_F32 ? 8 : 4) << c.log2_table_size;
    return standard_shape(c) && g_tune.fwd_split_kib > 0 && level_bytes > ((size_t)g_tune.fwd_split_kib << 10);
}

// The staged D = 3, F = 2 forward can order its points by a coarse cell first
// (point_order.hip: three short launches and 16 bytes per point), so that
// neighbouring lanes share the coarse and middle levels' table lines; the
// rows go back to the points' own positions.  Uniform batches gain from
// 2^18 points (98 -> 91 us there, 1394 -> 1161 us at 2^22); batches whose
// order is already coherent, as ray-ordered samples are, only pay for the
// sort (2^20 ray samples: 256 -> 273 us), and so do binary16 tables and
// levels gathered one half per pass.  The caller knows its batches, so the
// order is off unless asked for (HG_TUNE_FWD_ORDER: 1 from
// kFwdOrderMinPoints, 2 always).
constexpr int64_t kFwdOrderMinPoints = (int64_t)1 << 18;
bool fwd_order(const hg_config &c, int64_t n) {
    if (!standard_shape(c) || n <= 0 || n >= ((int64_t)1 << 31)) return false;
    return g_tune.fwd_order == 2 || (g_tune.fwd_order == 1 && n >= kFwdOrderMinPoints);
}

// Levels per binned group.  Where the budget (sized for the 256 MB last-level
// cache of the MI355X) holds enough levels for at least 1024 accumulate
// workgroups (two rounds of two per CU), groups take as many levels as keep
// their records (written by the bin kernel, read back by the accumulate
// kernel right after) within it, made equal.  Otherwise, for large batches
// whose records cannot stay in the cache in groups that fill the chip, all
// levels form one group: the accumulate grid of every level at once balances
// the uneven partitions of coarse levels and of structured batches.
int binned_group(const hg::BinParams &bp, int n_levels) {
    if (g_tune.bwd_group_mib <= 0) return n_levels;
    const size_t rec_bytes = (size_t)bp.level_records * bp.rec_bytes;
    const size_t budget = (size_t)g_tune.bwd_group_mib << 20;
    const int cap = (int)std::min<size_t>(n_levels, std::max<size_t>(1, budget / std::max<size_t>(rec_bytes, 1)));
    if ((int64_t)cap * bp.parts < 1024) return n_levels;
    const int ngroups = (n_levels + cap - 1) / cap;
    return (n_levels + ngroups - 1) / ngroups;
}

int check_points(int64_t n, const float *x) {
    if (n < 0) return fail(HG_EINVAL, "n = %lld < 0", (long long)n);
    if (!x) return fail(HG_EINVAL, "x is NULL");
    if (!aligned(x, 4)) return fail(HG_EINVAL, "x is not 4-byte aligned");
    return HG_OK;
}

int launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(HG_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// A binary16 gradient is summed exactly in fixed point and rounded once per
// entry on the binned path; the atomic scatter would round at every addition.
// So HG_F16 needs the binned path with this workspace and dtable: refused
// before anything is enqueued otherwise.
int check_half_grad(const hg_config *cfg, int64_t n, const void *dtable, const void *workspace,
                    size_t workspace_bytes) {
    if (cfg->grad_dtype != HG_F16) return HG_OK;
    hg::BinParams bp;
    if (!plan_binned(*cfg, n, bp))
        return fail(HG_EUNSUPPORTED, "grad_dtype HG_F16 needs the binned backward, which this grid and n lack");
    const size_t per_level = round_up(hg::binned_level_bytes(bp), 256);
    if (!g_tune.bwd_binned || !workspace || !aligned(dtable, 16) || workspace_bytes < per_level)
        return fail(HG_EUNSUPPORTED,
                    "grad_dtype HG_F16 needs the binned backward: a workspace of at least %zu bytes and a "
                    "16-byte aligned dtable",
                    per_level);
    return HG_OK;
}

// The table gradient of upstream rows dout (validated by the caller).
int table_backward(const hg_config *cfg, const float *x, int64_t n, const float *dout, int64_t dout_row_stride,
                   float *dtable, void *workspace, size_t workspace_bytes, void *stream) {
    int rc;
    hg::BinParams bp;
    if ((rc = check_half_grad(cfg, n, dtable, workspace, workspace_bytes))) return rc;
    if (g_tune.bwd_binned && workspace && aligned(dtable, 16) && plan_binned(*cfg, n, bp)) {
        const size_t per_level = round_up(hg::binned_level_bytes(bp), 256);
        if (workspace_bytes >= per_level) {
            // Whole levels per group; the launcher splits the workspace itself.
            const size_t usable = workspace_bytes / per_level * hg::binned_level_bytes(bp);
            const int group = binned_group(bp, cfg->n_levels);
            if (!standard_shape(*cfg))
                return launch_status(hg::launch_binned_backward_generic(bp, cfg->n_dims, cfg->n_features, cfg->n_levels,
                                                                        group, x, n, dout, dout_row_stride, dtable,
                                                                        workspace, usable, (hipStream_t)stream),
                                     "binned backward");
            return launch_status(hg::launch_binned_backward(bp, cfg->n_levels, group, x, n, dout, dout_row_stride,
                                                            dtable, workspace, usable, (hipStream_t)stream),
                                 "binned backward");
        }
    }
    hg::LaunchParams lp;
    if ((rc = plan(*cfg, n, lp))) return rc;
    // Small tables and coarse vertex grids are summed per workgroup in LDS
    // first; the other levels are scattered with fp32 atomics directly.
    hg::DenseLevels dl;
    bool sparse[hg::kMaxLevels];
    dense_levels(*cfg, lp, dl, sparse);
    if (dl.count) {
        rc = launch_status(hg::launch_backward_dense(lp, dl, cfg->n_dims, cfg->n_features, x, n, dout,
                                                     dout_row_stride, dtable, (hipStream_t)stream),
                           "backward (LDS-summed levels)");
        if (rc) return rc;
    }
    if (restrict_levels(lp, sparse) == 0) return ok();
    if (!standard_shape(*cfg))
        return launch_status(hg::launch_backward_generic(lp, cfg->n_dims, cfg->n_features, x, n, dout,
                                                         dout_row_stride, dtable, (hipStream_t)stream),
                             "backward");
    return launch_status(hg::launch_backward(lp, x, n, dout, dout_row_stride, dtable, g_tune.bwd_lanes,
                                             (hipStream_t)stream),
                         "backward");
}

// Binned-backward workspace of n points: (bytes for the default level groups, one level's bytes).
void table_backward_workspace(const hg_config &c, int64_t n, size_t &full, size_t &least) {
    hg::BinParams bp;
    full = least = 0;
    if (n > 0 && plan_binned(c, n, bp)) {
        least = round_up(hg::binned_level_bytes(bp), 256);
        full = least * (size_t)binned_group(bp, c.n_levels);
    }
}

bool mlp_shape(const hg_config &c) { return standard_shape(c) && c.n_levels * c.n_features == 32; }

int check_mlp_params(const hg_mlp_params *mp) {
    if (!mp) return fail(HG_EINVAL, "params is NULL");
    if (!mp->w1 || !mp->w2 || !mp->w3 || !mp->b1 || !mp->b2 || !mp->b3)
        return fail(HG_EINVAL, "every weight and bias must be a device pointer");
    if (!aligned(mp->w1, 8) || !aligned(mp->w2, 8) || !aligned(mp->w3, 8) || !aligned(mp->b1, 4) ||
        !aligned(mp->b2, 4) || !aligned(mp->b3, 4))
        return fail(HG_EINVAL, "weights must be 8-byte and biases 4-byte aligned");
    if (mp->coord_inputs != 0 && mp->coord_inputs != hg::kMlpCoords)
        return fail(HG_EINVAL, "coord_inputs %d: 0 (u = e) or 3 (u = [x, e])", (int)mp->coord_inputs);
    return HG_OK;
}

hg::MlpParams mlp_params(const hg_mlp_params *mp) {
    return hg::MlpParams{(const _Float16 *)mp->w1, (const _Float16 *)mp->w2, (const _Float16 *)mp->w3,
                         mp->b1, mp->b2, mp->b3, (int)mp->coord_inputs};
}

}  // namespace

extern "C" {

int hashgrid_abi_version(void) { return HASHGRID_ABI_VERSION; }

const char *hashgrid_last_error(void) { return g_last_error.c_str(); }

int hashgrid_resolutions(const hg_config *cfg, int32_t *res_out) {
    int rc = check_config(cfg);
    if (rc == HG_EINVAL) return rc;
    if (!res_out) return fail(HG_EINVAL, "res_out is NULL");
    resolutions(*cfg, res_out);
    return ok();
}

int hashgrid_forward_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n < 0) return fail(HG_EINVAL, "n = %lld < 0", (long long)n);
    if (!bytes_out) return fail(HG_EINVAL, "bytes_out is NULL");
    // One stage, or two where the gather splits levels (the second half's
    // blends), then the ordered points.
    const size_t stage = round_up((size_t)n * cfg->n_levels * cfg->n_features * sizeof(float), 256);
    *bytes_out = (split_forward(*cfg) ? 2 * stage : stage) + (fwd_order(*cfg, n) ? hg::order_workspace_bytes(n) : 0);
    return ok();
}

int hashgrid_forward(const hg_config *cfg, const float *x, int64_t n, const void *table, float *out,
                     int64_t out_row_stride, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    const size_t esize = cfg->table_dtype == HG_F32 ? 4 : 2;
    if (!table || !aligned(table, esize * cfg->n_features))
        return fail(HG_EINVAL, "table is NULL or not %zu-byte aligned", esize * cfg->n_features);
    if (!out || !aligned(out, 4)) return fail(HG_EINVAL, "out is NULL or not 4-byte aligned");
    if (out_row_stride < (int64_t)cfg->n_levels * cfg->n_features)
        return fail(HG_EINVAL, "out_row_stride %lld < L*F", (long long)out_row_stride);
    if (workspace && !aligned(workspace, 256)) return fail(HG_EINVAL, "workspace is not 256-byte aligned");
    hg::LaunchParams lp;
    if ((rc = plan(*cfg, n, lp))) return rc;
    const size_t stage_bytes = (size_t)n * cfg->n_levels * cfg->n_features * sizeof(float);
    float *stage = (g_tune.fwd_staged && workspace && workspace_bytes >= stage_bytes) ? (float *)workspace : nullptr;
    // F = 8 rows take 32 bytes per level, whole enough that staging costs more than it saves.
    if (!standard_shape(*cfg))
        return launch_status(hg::launch_forward_generic(lp, cfg->n_dims, cfg->n_features, x, n, table,
                                                        cfg->table_dtype, out, out_row_stride, g_tune.fwd_lanes,
                                                        cfg->n_features <= 4 ? stage : nullptr, (hipStream_t)stream),
                             "forward");
    const hg::FwdTune ft{g_tune.fwd_lanes, g_tune.fwd_unroll, g_tune.fwd_nt, g_tune.fwd_split_kib};
    float *stage2 = nullptr;
    const size_t stage_round = round_up(stage_bytes, 256);
    if (stage && split_forward(*cfg) && workspace_bytes >= stage_round + stage_bytes)
        stage2 = (float *)((char *)workspace + stage_round);
    const float *xg = x;            // the points in the order the kernels encode them
    const uint32_t *perm = nullptr;  // their original indices (NULL: the caller's order)
    if (stage && fwd_order(*cfg, n)) {
        const size_t off = (split_forward(*cfg) ? 2 : 1) * stage_round;
        if (workspace_bytes >= off + hg::order_workspace_bytes(n)) {
            float *xs;
            uint32_t *pm;
            rc = launch_status(hg::launch_point_order(x, n, (char *)workspace + off, &xs, &pm, (hipStream_t)stream),
                               "forward (point order)");
            if (rc) return rc;
            xg = xs;
            perm = pm;
        }
    }
    if (stage) {  // coarse levels from LDS, the others gathered
        hg::DenseLevels dl;
        bool keep[hg::kMaxLevels];
        fwd_dense_levels(*cfg, n, lp, dl, keep);
        if (dl.count) {
            rc = launch_status(hg::launch_forward_dense(lp, dl, xg, n, table, cfg->table_dtype, stage, false,
                                                        (hipStream_t)stream),
                               "forward (LDS levels)");
            if (rc) return rc;
            restrict_levels(lp, keep);
        }
    }
    return launch_status(hg::launch_forward(lp, xg, n, table, cfg->table_dtype, out, out_row_stride, ft, stage,
                                            (hipStream_t)stream, stage2, perm),
                         "forward");
}

int hashgrid_backward_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out,
                                     size_t *min_bytes_out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n < 0) return fail(HG_EINVAL, "n = %lld < 0", (long long)n);
    if (!bytes_out) return fail(HG_EINVAL, "bytes_out is NULL");
    size_t full, least;
    table_backward_workspace(*cfg, n, full, least);
    *bytes_out = full;
    if (min_bytes_out) *min_bytes_out = least;
    return ok();
}

int hashgrid_backward(const hg_config *cfg, const float *x, int64_t n, const float *dout,
                      int64_t dout_row_stride, float *dtable, void *workspace, size_t workspace_bytes,
                      void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    if (!dout || !aligned(dout, 4)) return fail(HG_EINVAL, "dout is NULL or not 4-byte aligned");
    if (!dtable || !aligned(dtable, 4)) return fail(HG_EINVAL, "dtable is NULL or not 4-byte aligned");
    if (dout_row_stride < (int64_t)cfg->n_levels * cfg->n_features)
        return fail(HG_EINVAL, "dout_row_stride %lld < L*F", (long long)dout_row_stride);
    if (workspace && !aligned(workspace, 256)) return fail(HG_EINVAL, "workspace is not 256-byte aligned");
    return table_backward(cfg, x, n, dout, dout_row_stride, dtable, workspace, workspace_bytes, stream);
}

int hashgrid_backward_noalloc(const hg_config *cfg, const float *x, int64_t n, const float *dout,
                              int64_t dout_row_stride, float *dtable, void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    if (!dout || !aligned(dout, 4)) return fail(HG_EINVAL, "dout is NULL or not 4-byte aligned");
    if (!dtable || !aligned(dtable, 4)) return fail(HG_EINVAL, "dtable is NULL or not 4-byte aligned");
    if (dout_row_stride < (int64_t)cfg->n_levels * cfg->n_features)
        return fail(HG_EINVAL, "dout_row_stride %lld < L*F", (long long)dout_row_stride);
    // The scratch must hold one level's records (levels are binned in groups
    // that fit it); a grid without a binned path uses no scratch.
    hg::BinParams bp;
    if (plan_binned(*cfg, n, bp)) {
        const size_t per_level = round_up(hg::binned_level_bytes(bp), 256);
        if (per_level > hg::kNoallocScratchBytes) {
            const size_t per_tile = (size_t)bp.rec_per_tile * bp.rec_bytes + ((size_t)bp.parts + 2) * sizeof(uint32_t);
            const long long max_n = (long long)((hg::kNoallocScratchBytes - 256) / per_tile) * bp.tile_pts;
            return fail(HG_EINVAL,
                        "n = %lld: one level's binned records take %zu bytes, more than the %zu-byte scratch of "
                        "the allocation-free backward; it takes at most %lld points of this grid per call",
                        (long long)n, per_level, hg::kNoallocScratchBytes, max_n);
        }
    }
    void *scratch = nullptr;
    const hipError_t e = hg::noalloc_scratch(&scratch);
    if (e != hipSuccess)
        return fail(HG_EHIP, "device scratch of the allocation-free backward: %s", hipGetErrorString(e));
    return table_backward(cfg, x, n, dout, dout_row_stride, dtable, scratch, hg::kNoallocScratchBytes, stream);
}

int hashgrid_mlp_workspace_size(const hg_config *cfg, int64_t n, size_t *stage_bytes_out, size_t *bwd_bytes_out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!mlp_shape(*cfg)) return fail(HG_EUNSUPPORTED, "the MLP head takes the 32 features of D = 3, L*F = 32 grids");
    if (n < 0) return fail(HG_EINVAL, "n = %lld < 0", (long long)n);
    if (!stage_bytes_out || !bwd_bytes_out) return fail(HG_EINVAL, "output pointers must be non-NULL");
    *stage_bytes_out = round_up((size_t)n * 32 * 2, 256);
    size_t full, least;
    table_backward_workspace(*cfg, n, full, least);
    *bwd_bytes_out = n ? round_up((size_t)n * 32 * 4, 256) + round_up(hg::mlp_partials_bytes(n), 256) + full : 0;
    return ok();
}

int hashgrid_mlp_forward(const hg_config *cfg, const float *x, int64_t n, const void *table,
                         const hg_mlp_params *params, float *y, void *stage, size_t stage_bytes, void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!mlp_shape(*cfg)) return fail(HG_EUNSUPPORTED, "the MLP head takes the 32 features of D = 3, L*F = 32 grids");
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    if ((rc = check_mlp_params(params))) return rc;
    const size_t esize = cfg->table_dtype == HG_F32 ? 4 : 2;
    if (!table || !aligned(table, esize * 2)) return fail(HG_EINVAL, "table is NULL or misaligned");
    if (!y || !aligned(y, 16)) return fail(HG_EINVAL, "y is NULL or not 16-byte aligned");
    if (!stage || !aligned(stage, 256) || stage_bytes < (size_t)n * 64)
        return fail(HG_EINVAL, "stage must be 256-byte aligned and hold n * 64 bytes");
    hg::LaunchParams lp;
    if ((rc = plan(*cfg, n, lp))) return rc;
    hg::DenseLevels dl;
    bool keep[hg::kMaxLevels];
    fwd_dense_levels(*cfg, n, lp, dl, keep);
    if (dl.count) {
        rc = launch_status(hg::launch_forward_dense(lp, dl, x, n, table, cfg->table_dtype, stage, true,
                                                    (hipStream_t)stream),
                           "encode stage (LDS levels)");
        if (rc) return rc;
        restrict_levels(lp, keep);
    }
    hipError_t e = hg::launch_encode_stage_f16(lp, x, n, table, cfg->table_dtype, (_Float16 *)stage,
                                               (hipStream_t)stream);
    if (e != hipSuccess) return launch_status(e, "encode stage");
    return launch_status(hg::launch_mlp_forward((const _Float16 *)stage, x, n, mlp_params(params), y,
                                                (hipStream_t)stream),
                         "mlp forward");
}

int hashgrid_mlp_backward(const hg_config *cfg, const float *x, int64_t n, const void *stage,
                          const hg_mlp_params *params, const float *dy, const hg_mlp_grads *grads, float *dtable,
                          void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!mlp_shape(*cfg)) return fail(HG_EUNSUPPORTED, "the MLP head takes the 32 features of D = 3, L*F = 32 grids");
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    if ((rc = check_mlp_params(params))) return rc;
    if (!stage || !aligned(stage, 256)) return fail(HG_EINVAL, "stage is NULL or not 256-byte aligned");
    if (!dy || !aligned(dy, 16)) return fail(HG_EINVAL, "dy is NULL or not 16-byte aligned");
    if (!grads || !grads->dw1 || !grads->db1 || !grads->dw2 || !grads->db2 || !grads->dw3 || !grads->db3)
        return fail(HG_EINVAL, "every gradient must be a device pointer");
    if (!dtable || !aligned(dtable, 4)) return fail(HG_EINVAL, "dtable is NULL or not 4-byte aligned");
    const size_t de_bytes = round_up((size_t)n * 32 * 4, 256);
    const size_t part_bytes = round_up(hg::mlp_partials_bytes(n), 256);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < de_bytes + part_bytes)
        return fail(HG_EINVAL, "workspace must be 256-byte aligned and hold at least n * 128 bytes plus the "
                               "weight-gradient partials (hashgrid_mlp_workspace_size)");
    // The encoder's table gradient takes dL/de as its upstream rows and the
    // rest of the workspace for the binned backward.
    const size_t used = de_bytes + part_bytes;
    void *rest = workspace_bytes > used ? (char *)workspace + used : nullptr;
    if ((rc = check_half_grad(cfg, n, dtable, rest, workspace_bytes - used))) return rc;
    float *de = (float *)workspace;
    float *partials = (float *)((char *)workspace + de_bytes);
    const hg::MlpGrads g{grads->dw1, grads->db1, grads->dw2, grads->db2, grads->dw3, grads->db3};
    hipError_t e = hg::launch_mlp_backward((const _Float16 *)stage, x, n, mlp_params(params), dy, de, partials, g,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return launch_status(e, "mlp backward");
    return table_backward(cfg, x, n, de, 32, dtable, rest, workspace_bytes - used, stream);
}

int hashgrid_input_grad_workspace_size(const hg_config *cfg, int64_t n, size_t *bytes_out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n < 0) return fail(HG_EINVAL, "n = %lld < 0", (long long)n);
    if (!bytes_out) return fail(HG_EINVAL, "bytes_out is NULL");
    // The [L][n][D] stage, and for the D = 3, F = 2 grid a level-major copy of
    // the upstream rows.  D <= 2 runs point-major whatever the workspace.
    if (cfg->n_dims <= 2) {
        *bytes_out = 0;
        return ok();
    }
    const size_t stage = round_up((size_t)n * cfg->n_levels * cfg->n_dims * sizeof(float), 256);
    const size_t copy = standard_shape(*cfg) ? round_up((size_t)n * cfg->n_levels * 2 * sizeof(float), 256) : 0;
    *bytes_out = stage + copy;
    return ok();
}

int hashgrid_input_grad(const hg_config *cfg, const float *x, int64_t n, const void *table, const float *dout,
                        int64_t dout_row_stride, float *dx, void *workspace, size_t workspace_bytes,
                        void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    const size_t esize = cfg->table_dtype == HG_F32 ? 4 : 2;
    if (!table || !aligned(table, esize * cfg->n_features))
        return fail(HG_EINVAL, "table is NULL or not %zu-byte aligned", esize * cfg->n_features);
    if (!dout || !aligned(dout, 4)) return fail(HG_EINVAL, "dout is NULL or not 4-byte aligned");
    if (dout_row_stride < (int64_t)cfg->n_levels * cfg->n_features)
        return fail(HG_EINVAL, "dout_row_stride %lld < L*F", (long long)dout_row_stride);
    if (!dx || !aligned(dx, 4)) return fail(HG_EINVAL, "dx is NULL or not 4-byte aligned");
    if (workspace && !aligned(workspace, 256)) return fail(HG_EINVAL, "workspace is not 256-byte aligned");
    hg::LaunchParams lp;
    if ((rc = plan(*cfg, n, lp))) return rc;
    const size_t stage_bytes = round_up((size_t)n * cfg->n_levels * cfg->n_dims * sizeof(float), 256);
    const size_t copy_bytes = (size_t)n * cfg->n_levels * 2 * sizeof(float);
    float *stage = (workspace && workspace_bytes >= stage_bytes) ? (float *)workspace : nullptr;
    float *dlm = (stage && standard_shape(*cfg) && workspace_bytes >= stage_bytes + copy_bytes)
                     ? (float *)((char *)workspace + stage_bytes)
                     : nullptr;
    return launch_status(hg::launch_input_grad(lp, cfg->n_dims, cfg->n_features, x, n, table, cfg->table_dtype,
                                               dout, dout_row_stride, dx, stage, dlm, (hipStream_t)stream),
                         "input_grad");
}

int hashgrid_adam_step(const hg_adam *opt, int64_t count, float *param, float *m, float *v, float *grad,
                       void *param_f16, int32_t flags, void *stream) {
    if (!opt) return fail(HG_EINVAL, "opt is NULL");
    if (count < 0) return fail(HG_EINVAL, "count = %lld < 0", (long long)count);
    if (opt->step < 1) return fail(HG_EINVAL, "step %d < 1", opt->step);
    if (!std::isfinite(opt->lr) || !std::isfinite(opt->eps) || opt->eps < 0.f)
        return fail(HG_EINVAL, "lr and eps must be finite, eps >= 0");
    if (!(opt->beta1 >= 0.f && opt->beta1 < 1.f) || !(opt->beta2 >= 0.f && opt->beta2 < 1.f))
        return fail(HG_EINVAL, "betas must lie in [0, 1)");
    if (flags & ~HG_ADAM_ZERO_GRAD) return fail(HG_EINVAL, "unknown flags 0x%x", flags);
    if (count == 0) return ok();
    if (!param || !m || !v || !grad) return fail(HG_EINVAL, "param, m, v and grad must be device pointers");
    if (!aligned(param, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(grad, 4) ||
        (param_f16 && !aligned(param_f16, 2)))
        return fail(HG_EINVAL, "misaligned buffer");
    const hg::AdamParams a{opt->lr, opt->beta1, opt->beta2, opt->eps, opt->step};
    return launch_status(hg::launch_adam(a, count, param, m, v, grad, param_f16, (flags & HG_ADAM_ZERO_GRAD) != 0,
                                         (hipStream_t)stream),
                         "adam");
}

int hashgrid_debug_corners(const hg_config *cfg, const float *x, int64_t n, uint32_t *idx, float *w,
                           void *stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n == 0) return ok();
    if ((rc = check_points(n, x))) return rc;
    if (idx && !aligned(idx, 4)) return fail(HG_EINVAL, "idx is not 4-byte aligned");
    if (w && !aligned(w, 4)) return fail(HG_EINVAL, "w is not 4-byte aligned");
    if (n > ((int64_t)1 << 31) - 256) return fail(HG_EINVAL, "n too large for the debug export");
    hg::LaunchParams lp;
    if ((rc = plan(*cfg, n, lp))) return rc;
    if (cfg->n_dims != 3)
        return launch_status(hg::launch_debug_corners_generic(lp, cfg->n_dims, x, n, idx, w, (hipStream_t)stream),
                             "debug_corners");
    return launch_status(hg::launch_debug_corners(lp, x, n, idx, w, (hipStream_t)stream), "debug_corners");
}

int hashgrid_tune(int key, int value) {
    switch (key) {
    case HG_TUNE_FWD_LANES:
        if (value != 1 && value != 2) break;
        g_tune.fwd_lanes = value;
        return ok();
    case HG_TUNE_BWD_LANES:
        if (value != 1 && value != 2 && value != 4) break;
        g_tune.bwd_lanes = value;
        return ok();
    case HG_TUNE_CHUNK_POINTS:
        if (value < 64 || value > 65536 || (value & (value - 1))) break;
        g_tune.chunk_points = value;
        return ok();
    case HG_TUNE_XCD_MAP:
        if (value != 0 && value != 1) break;
        g_tune.xcd_map = value;
        return ok();
    case HG_TUNE_BWD_BINNED:
        if (value != 0 && value != 1) break;
        g_tune.bwd_binned = value;
        return ok();
    case HG_TUNE_FWD_UNROLL:
        if (value != 1 && value != 2 && value != 4) break;
        g_tune.fwd_unroll = value;
        return ok();
    case HG_TUNE_FWD_NT:
        if (value != 0 && value != 1) break;
        g_tune.fwd_nt = value;
        return ok();
    case HG_TUNE_FWD_STAGED:
        if (value != 0 && value != 1) break;
        g_tune.fwd_staged = value;
        return ok();
    case HG_TUNE_BWD_GROUP_MIB:
        if (value < 0 || value > (1 << 20)) return fail(HG_EINVAL, "BWD_GROUP_MIB %d outside 0..2^20", value);
        g_tune.bwd_group_mib = value;
        return ok();
    case HG_TUNE_BWD_PART_LOG2:
        if (value != 0 && (value < 11 || value > hg::kMaxSLog2)) break;
        g_tune.bwd_part_log2 = value;
        return ok();
    case HG_TUNE_BWD_DENSE:
        if (value != 0 && value != 1) break;
        g_tune.bwd_dense = value;
        return ok();
    case HG_TUNE_FWD_SPLIT_KIB:
        if (value != 0 && (value < 64 || value > (1 << 20))) break;
        g_tune.fwd_split_kib = value;
        return ok();
    case HG_TUNE_FWD_DENSE:
        if (value < 0 || value > 2) break;
        g_tune.fwd_dense = value;
        return ok();
    case HG_TUNE_FWD_ORDER:
        if (value < 0 || value > 2) break;
        g_tune.fwd_order = value;
        return ok();
    default:
        return fail(HG_EINVAL, "unknown tuning key %d", key);
    }
    return fail(HG_EINVAL, "value %d out of range for tuning key %d", value, key);
}

int hashgrid_tune_get(int key) {
    switch (key) {
    case HG_TUNE_FWD_LANES: return g_tune.fwd_lanes;
    case HG_TUNE_BWD_LANES: return g_tune.bwd_lanes;
    case HG_TUNE_CHUNK_POINTS: return g_tune.chunk_points;
    case HG_TUNE_XCD_MAP: return g_tune.xcd_map;
    case HG_TUNE_BWD_BINNED: return g_tune.bwd_binned;
    case HG_TUNE_FWD_UNROLL: return g_tune.fwd_unroll;
    case HG_TUNE_FWD_NT: return g_tune.fwd_nt;
    case HG_TUNE_FWD_STAGED: return g_tune.fwd_staged;
    case HG_TUNE_BWD_PART_LOG2: return g_tune.bwd_part_log2;
    case HG_TUNE_BWD_GROUP_MIB: return g_tune.bwd_group_mib;
    case HG_TUNE_BWD_DENSE: return g_tune.bwd_dense;
    case HG_TUNE_FWD_SPLIT_KIB: return g_tune.fwd_split_kib;
    case HG_TUNE_FWD_DENSE: return g_tune.fwd_dense;
    case HG_TUNE_FWD_ORDER: return g_tune.fwd_order;
    default: return fail(HG_EINVAL, "unknown tuning key %d", key);
    }
}

}  // extern "C"
