/*
 * Sequential CPU oracle for PointPillars-style pillar / voxel binning.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition the GPU library is checked against. Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the library itself
 * never does, and the two share no code, headers or tables.
 *
 * Source: "Voxelize" (ethan-howes.github.io/projects/voxelize).
 *   - Output tensors: the introduction (a [V,32,4] per-pillar point stack,
 *     [V,3] grid coordinates, [V] per-pillar counts).
 *   - Binning: section "Binning a point" (NaN/Inf check, z-slab, floorf cell
 *     index, strict < on the upper grid bound, flattened id cy*grid_x+cx).
 *   - Coordinates (z, y, x) with z = 0 for pillars, and "keep the first K"
 *     (points past max_points are dropped): section "Claiming a pillar and
 *     packing points".
 *   - Pillar assignment by a dictionary in insertion order, as the page's
 *     NumPy reference does: section "Results".
 *
 * Readings taken where the page is silent (each one fixes a single output):
 *   - pillars are numbered in order of first occurrence in the input;
 *   - the first max_voxels pillars are kept; points of later pillars are
 *     dropped and create no pillar, later points of kept pillars still count;
 *   - inside a pillar the max_points lowest input indices are kept, in order;
 *   - counts = min(total points of the pillar, max_points);
 *   - rows past the count are +0.0f;
 *   - the NaN/Inf check applies to x, y, z only (intensity is copied as bits);
 *   - the z-slab is z_min <= z < z_max; in 3D mode (gz > 1) the z cell index
 *     floorf((z - z_min) / vz) must also lie in [0, gz);
 *   - x_max and y_max do not enter binning: the grid size bounds the cell;
 *   - range tests are made on the float floor value before any conversion,
 *     every operation in IEEE fp32 round-to-nearest, no FMA contraction.
 *
 * oracle_downsample adds voxel-grid downsampling, one mean point per kept
 * voxel, from a second page; oracle_spherical (end of file) adds the
 * spherical binning and voxel-contiguous reorder that the RadiusFPS page
 * runs before its sampler (see each function's comment).
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float x_min, y_min, z_min;
    float vx, vy, vz;
    int64_t gx, gy, gz;
} oracle_grid;

static oracle_grid make_grid(const float range[6], const float cell[3], const int32_t grid[3])
{
    oracle_grid g;
    g.x_min = range[0];
    g.y_min = range[1];
    g.z_min = range[2];
    g.vx = cell[0];
    g.vy = cell[1];
    g.vz = cell[2];
    g.gx = grid[0];
    g.gy = grid[1];
    g.gz = grid[2];
    return g;
}

/*
 * Bin one point, following "Binning a point": returns 1 and writes the cell
 * (cx, cy, cz) when the point is kept, 0 when it is rejected.
 */
static int bin_point(const float *p, const oracle_grid *g, float z_max,
                     int64_t *cx, int64_t *cy, int64_t *cz)
{
    float x = p[0], y = p[1], z = p[2];

    /* NaN/Inf check on the coordinates. */
    if (isnan(x) || isinf(x) || isnan(y) || isinf(y) || isnan(z) || isinf(z))
        return 0;

    /* Drop points outside the z-slab. */
    if (!(z >= g->z_min && z < z_max))
        return 0;

    /* Cell index with floorf of ((coordinate - min) / cell size). */
    float fx = floorf((x - g->x_min) / g->vx);
    float fy = floorf((y - g->y_min) / g->vy);

    /* Reject anything outside the grid, strict < on the upper bound. */
    if (!(fx >= 0.0f && fx < (float)g->gx))
        return 0;
    if (!(fy >= 0.0f && fy < (float)g->gy))
        return 0;

    float fz = 0.0f;
    if (g->gz > 1) {
        fz = floorf((z - g->z_min) / g->vz);
        if (!(fz >= 0.0f && fz < (float)g->gz))
            return 0;
    }

    *cx = (int64_t)fx;
    *cy = (int64_t)fy;
    *cz = (int64_t)fz;
    return 1;
}

/* Flattened cell id: cy*grid_x + cx for pillars, (cz*gy + cy)*gx + cx in 3D. */
static int64_t flat_key(const oracle_grid *g, int64_t cx, int64_t cy, int64_t cz)
{
    return (cz * g->gy + cy) * g->gx + cx;
}

/*
 * Per-point binning, exported so the tests can compare it with an independent
 * float32 evaluation: valid[i] = 1/0 and key[i] = flattened id or -1.
 */
int oracle_bin(const float *points, int64_t n, const float range[6], const float cell[3],
               const int32_t grid[3], int8_t *valid, int64_t *key)
{
    oracle_grid g = make_grid(range, cell, grid);
    for (int64_t i = 0; i < n; i++) {
        int64_t cx, cy, cz;
        if (bin_point(points + 4 * i, &g, range[5], &cx, &cy, &cz)) {
            valid[i] = 1;
            key[i] = flat_key(&g, cx, cy, cz);
        } else {
            valid[i] = 0;
            key[i] = -1;
        }
    }
    return 0;
}

/*
 * The dictionary: flattened key -> pillar id, holding only the kept pillars.
 * A plain open-addressing map; nothing about it is visible in the output.
 */
typedef struct {
    int64_t cap;      /* power of two */
    int64_t *keys;    /* -1 = empty */
    int32_t *vals;
} key_map;

static int map_init(key_map *m, int64_t max_entries)
{
    m->cap = 16;
    while (m->cap < 2 * max_entries + 2)
        m->cap *= 2;
    m->keys = (int64_t *)malloc((size_t)m->cap * sizeof(int64_t));
    m->vals = (int32_t *)malloc((size_t)m->cap * sizeof(int32_t));
    if (!m->keys || !m->vals)
        return -1;
    for (int64_t s = 0; s < m->cap; s++)
        m->keys[s] = -1;
    return 0;
}

static void map_free(key_map *m)
{
    free(m->keys);
    free(m->vals);
}

/* Returns the slot holding `key`, or the empty slot where it would go. */
static int64_t map_slot(const key_map *m, int64_t key)
{
    uint64_t h = (uint64_t)key * 0x9E3779B97F4A7C15ull;
    int64_t s = (int64_t)(h >> 20) & (m->cap - 1);
    while (m->keys[s] != -1 && m->keys[s] != key)
        s = (s + 1) & (m->cap - 1);
    return s;
}

/*
 * The whole operation, one point at a time in input order.
 *
 * voxels is [max_voxels, max_points, 4] float, coords [max_voxels, 3] int32
 * (z, y, x), num_points [max_voxels] int32; rows [0, V) are written, V goes to
 * *num_voxels. Returns 0, or -1 if memory for the dictionary is unavailable.
 */
int oracle_voxelize_map(const float *points, int64_t n, const float range[6],
                        const float cell[3], const int32_t grid[3], int32_t max_points,
                        int32_t max_voxels, float *voxels, int32_t *coords,
                        int32_t *num_points, int32_t *num_voxels, int32_t *point_pillar);

int oracle_voxelize(const float *points, int64_t n, const float range[6], const float cell[3],
                    const int32_t grid[3], int32_t max_points, int32_t max_voxels,
                    float *voxels, int32_t *coords, int32_t *num_points, int32_t *num_voxels)
{
    return oracle_voxelize_map(points, n, range, cell, grid, max_points, max_voxels, voxels,
                               coords, num_points, num_voxels, NULL);
}

/*
 * The same operation, also writing the inverse map when point_pillar is not
 * NULL: point_pillar[i] = the pillar id of point i's cell when that pillar is
 * kept (whether or not the point is among the pillar's first max_points), -1
 * for a rejected point or a point whose pillar is past the cap. The map is
 * what a consumer needs to scatter per-point results back through the pillars.
 */
int oracle_voxelize_map(const float *points, int64_t n, const float range[6],
                        const float cell[3], const int32_t grid[3], int32_t max_points,
                        int32_t max_voxels, float *voxels, int32_t *coords,
                        int32_t *num_points, int32_t *num_voxels, int32_t *point_pillar)
{
    oracle_grid g = make_grid(range, cell, grid);
    const int64_t K = max_points;
    key_map dict;
    if (map_init(&dict, max_voxels) != 0) {
        map_free(&dict);
        return -1;
    }
    int64_t *total = (int64_t *)calloc((size_t)max_voxels + 1, sizeof(int64_t));
    if (!total) {
        map_free(&dict);
        return -1;
    }
    int64_t V = 0;

    for (int64_t i = 0; i < n; i++) {
        const float *p = points + 4 * i;
        int64_t cx, cy, cz;
        if (point_pillar)
            point_pillar[i] = -1;
        if (!bin_point(p, &g, range[5], &cx, &cy, &cz))
            continue;
        int64_t key = flat_key(&g, cx, cy, cz);

        int64_t s = map_slot(&dict, key);
        int64_t pid;
        if (dict.keys[s] == key) {
            pid = dict.vals[s];
        } else if (V < max_voxels) {
            /* A new pillar, numbered in order of first occurrence. */
            pid = V++;
            dict.keys[s] = key;
            dict.vals[s] = (int32_t)pid;
            coords[3 * pid + 0] = (int32_t)cz;  /* z (0 for pillars) */
            coords[3 * pid + 1] = (int32_t)cy;  /* y */
            coords[3 * pid + 2] = (int32_t)cx;  /* x */
        } else {
            continue;  /* its pillar is past the max_voxels cap: dropped */
        }

        if (point_pillar)
            point_pillar[i] = (int32_t)pid;
        total[pid] += 1;
        if (total[pid] <= K) {
            /* keep the first K points of the pillar, copied bit for bit */
            memcpy(voxels + (pid * K + (total[pid] - 1)) * 4, p, 4 * sizeof(float));
        }
    }

    for (int64_t pid = 0; pid < V; pid++) {
        int64_t c = total[pid] < K ? total[pid] : K;
        num_points[pid] = (int32_t)c;
        for (int64_t j = c; j < K; j++)
            memset(voxels + (pid * K + j) * 4, 0, 4 * sizeof(float));
    }
    *num_voxels = (int32_t)V;

    free(total);
    map_free(&dict);
    return 0;
}

/*
 * Voxel-grid downsampling: one output point per kept voxel, the mean of the
 * points in it. Source: the GPU K-D tree ICP page ("operation 1" of its
 * section 4.4, a voxel_downsample kernel), whose kernel truncates the cell
 * index and accumulates with float atomics, so its result depends on thread
 * order. Readings taken:
 *   - binning, numbering in first-occurrence order and the max_voxels cap are
 *     those of oracle_voxelize_map above (floorf cell index, not truncation);
 *   - each of x, y, z and intensity is summed over the voxel's points in
 *     input order in double precision, the sum divided by the count in double
 *     precision, and the quotient rounded once to float (round to nearest);
 *   - counts[p] = every point of the voxel (there is no max_points here).
 * centroids is [max_voxels, 4] float, coords [max_voxels, 3] int32 (z, y, x),
 * counts [max_voxels] int32; rows [0, V) are written and V goes to
 * *num_voxels. Returns 0, or -1 if memory is unavailable.
 */
int oracle_downsample(const float *points, int64_t n, const float range[6], const float cell[3],
                      const int32_t grid[3], int32_t max_voxels, float *centroids,
                      int32_t *coords, int32_t *counts, int32_t *num_voxels)
{
    oracle_grid g = make_grid(range, cell, grid);
    key_map dict;
    if (map_init(&dict, max_voxels) != 0) {
        map_free(&dict);
        return -1;
    }
    double *sum = (double *)calloc((size_t)max_voxels * 4 + 4, sizeof(double));
    int64_t *total = (int64_t *)calloc((size_t)max_voxels + 1, sizeof(int64_t));
    if (!sum || !total) {
        free(sum);
        free(total);
        map_free(&dict);
        return -1;
    }
    int64_t V = 0;
    for (int64_t i = 0; i < n; i++) {
        const float *p = points + 4 * i;
        int64_t cx, cy, cz;
        if (!bin_point(p, &g, range[5], &cx, &cy, &cz))
            continue;
        int64_t key = flat_key(&g, cx, cy, cz);
        int64_t s = map_slot(&dict, key);
        int64_t pid;
        if (dict.keys[s] == key) {
            pid = dict.vals[s];
        } else if (V < max_voxels) {
            pid = V++;
            dict.keys[s] = key;
            dict.vals[s] = (int32_t)pid;
            coords[3 * pid + 0] = (int32_t)cz;
            coords[3 * pid + 1] = (int32_t)cy;
            coords[3 * pid + 2] = (int32_t)cx;
        } else {
            continue;  /* its voxel is past the cap */
        }
        for (int c = 0; c < 4; c++)
            sum[4 * pid + c] += (double)p[c];  /* input order, double precision */
        total[pid] += 1;
    }
    for (int64_t pid = 0; pid < V; pid++) {
        for (int c = 0; c < 4; c++)
            centroids[4 * pid + c] = (float)(sum[4 * pid + c] / (double)total[pid]);
        counts[pid] = (int32_t)total[pid];
    }
    *num_voxels = (int32_t)V;
    free(sum);
    free(total);
    map_free(&dict);
    return 0;
}

/*
 * Spherical-coordinate binning and voxel-contiguous reorder: the
 * preprocessing of the RadiusFPS page ("Spherical voxel partition" and the
 * preprocessing step of RadiusFPS-G): each point gets spherical coordinates
 * r = sqrt(x^2 + y^2 + z^2), elevation theta = atan2(z, sqrt(x^2 + y^2)) and
 * azimuth phi = atan2(y, x), each axis is split uniformly, and the points are
 * sorted by voxel id so that a voxel's points are contiguous. Readings taken:
 *   - r in float: sqrtf((x*x + y*y) + z*z), correctly rounded; r bin =
 *     floorf((r - r_min) / dr), kept when in [0, nr) (the same rule as the
 *     Cartesian axes of "Binning a point");
 *   - angles are not rounded: a point is in angular bin k when its direction
 *     is at or above boundary k and below boundary k + 1. Boundary angle
 *     a_k = a_min + k * da is taken in double from the float parameters.
 *     A boundary at or below the axis's lowest angle (-pi/2 for elevation,
 *     -pi for azimuth) has every direction above it; one above the axis's
 *     highest angle (pi/2, pi) has none. Any other boundary is the direction
 *     (cos a_k, sin a_k) rounded to float. Elevation uses the direction
 *     (sqrtf(x*x + y*y), z); azimuth uses (x, y) with angles in (-pi, pi]
 *     (a zero y of either sign counts as 0, so the negative x axis has angle
 *     pi). Every comparison of two directions is the sign of a cross product
 *     of float operands evaluated in double, which is exact. The bin is the
 *     largest k at or below which the direction lies;
 *   - a point with x = y = 0 has azimuth 0; a point at the origin has no
 *     elevation and is not kept; NaN/Inf coordinates are not kept;
 *   - voxel id = (ir * ntheta + itheta) * nphi + iphi;
 *   - the sort is by voxel id; inside a voxel the points are in input order
 *     here (the page does not fix that order).
 * sph_min = (r_min, theta_min, phi_min), sph_cell = (dr, dtheta, dphi),
 * bins = (nr, ntheta, nphi). Outputs: voxel_of[N] (id or -1), offsets[nvox + 1]
 * (start of each voxel in the sorted order), order[N] (indices of kept points
 * by voxel), *n_kept. Returns 0, or -1 if memory is unavailable.
 */

/* half-plane index of a direction for angles in (-pi, pi]:
 * 0 = angle in (-pi, 0), 1 = [0, pi), 2 = pi */
static int angle_half(double x, double y)
{
    if (y < 0.0)
        return 0;
    if (y > 0.0 || x > 0.0)
        return 1;
    return 2;
}

/* angle of direction p >= angle of direction d, both in (-pi, pi], exact */
static int angle_ge(double px, double py, double dx, double dy)
{
    int hp = angle_half(px, py), hd = angle_half(dx, dy);
    if (hp != hd)
        return hp > hd;
    return dx * py - dy * px >= 0.0; /* float operands: exact products */
}

/* pi and pi/2 rounded to double; both roundings fall below the true value */
#define SPH_PI 3.141592653589793
#define SPH_HALF_PI 1.5707963267948966

/* One boundary: cls -1 = below the axis (every direction passes),
 * +1 = above it (none passes), 0 = compare with the direction (c, s).
 * lim is the axis's half-width (pi/2 or pi) as the nearest double below it,
 * so a < -lim exactly when a <= -half-width, and a > lim when a > half-width. */
typedef struct {
    int cls;
    float c, s;
} sph_bound;

static void sph_bounds(sph_bound *b, int nb, float a_min, float da, double lim)
{
    for (int k = 0; k <= nb; k++) {
        double a = (double)a_min + (double)k * (double)da;
        b[k].cls = a < -lim ? -1 : (a > lim ? 1 : 0);
        b[k].c = (float)cos(a);
        b[k].s = (float)sin(a);
    }
}

/* largest k whose boundary the direction is at or above, -1 if none */
static int sph_bin_elev(const sph_bound *b, int nb, double rxy, double z)
{
    int bin = -1;
    for (int k = 0; k <= nb; k++) {
        int ge = b[k].cls < 0 ||
                 (b[k].cls == 0 && (double)b[k].c * z - (double)b[k].s * rxy >= 0.0);
        if (ge)
            bin = k;
    }
    return bin;
}

static int sph_bin_azim(const sph_bound *b, int nb, double x, double y)
{
    int bin = -1;
    for (int k = 0; k <= nb; k++) {
        int ge = b[k].cls < 0 ||
                 (b[k].cls == 0 && angle_ge(x, y, (double)b[k].c, (double)b[k].s));
        if (ge)
            bin = k;
    }
    return bin;
}

int oracle_spherical(const float *points, int64_t n, const float sph_min[3],
                     const float sph_cell[3], const int32_t bins[3], int32_t *voxel_of,
                     int32_t *offsets, int32_t *order, int32_t *n_kept)
{
    const int nr = bins[0], nt = bins[1], np_ = bins[2];
    const int64_t nvox = (int64_t)nr * nt * np_;
    sph_bound *tb = (sph_bound *)malloc(sizeof(sph_bound) * (size_t)(nt + 1));
    sph_bound *pb = (sph_bound *)malloc(sizeof(sph_bound) * (size_t)(np_ + 1));
    int64_t *cnt = (int64_t *)calloc((size_t)nvox + 1, sizeof(int64_t));
    if (!tb || !pb || !cnt) {
        free(tb);
        free(pb);
        free(cnt);
        return -1;
    }
    sph_bounds(tb, nt, sph_min[1], sph_cell[1], SPH_HALF_PI);
    sph_bounds(pb, np_, sph_min[2], sph_cell[2], SPH_PI);
    for (int64_t i = 0; i < n; i++) {
        const float *p = points + 4 * i;
        float x = p[0], y = p[1], z = p[2];
        voxel_of[i] = -1;
        if (!isfinite(x) || !isfinite(y) || !isfinite(z))
            continue;
        float xx = x * x, yy = y * y, zz = z * z;
        float sxy = xx + yy;
        float r = sqrtf(sxy + zz);
        float rxy = sqrtf(sxy);
        if (r == 0.0f)
            continue; /* no direction */
        float fr = floorf((r - sph_min[0]) / sph_cell[0]);
        if (!(fr >= 0.0f && fr < (float)nr))
            continue;
        int it = sph_bin_elev(tb, nt, (double)rxy, (double)z);
        if (it < 0 || it >= nt)
            continue;
        int ip = (x == 0.0f && y == 0.0f) ? sph_bin_azim(pb, np_, 1.0, 0.0)
                                          : sph_bin_azim(pb, np_, (double)x, (double)y);
        if (ip < 0 || ip >= np_)
            continue;
        int64_t v = ((int64_t)fr * nt + it) * np_ + ip;
        voxel_of[i] = (int32_t)v;
        cnt[v] += 1;
    }
    int64_t run = 0;
    for (int64_t v = 0; v < nvox; v++) {
        offsets[v] = (int32_t)run;
        run += cnt[v];
        cnt[v] = offsets[v]; /* cursor */
    }
    offsets[nvox] = (int32_t)run;
    for (int64_t i = 0; i < n; i++) /* counting sort, input order inside a voxel */
        if (voxel_of[i] >= 0)
            order[cnt[voxel_of[i]]++] = (int32_t)i;
    *n_kept = (int32_t)run;
    free(tb);
    free(pb);
    free(cnt);
    return 0;
}
