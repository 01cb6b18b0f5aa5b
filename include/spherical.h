/*
 * spherical.h -- C ABI of the spherical binning and voxel-contiguous reorder
 * (MI355X, gfx950), part of the same library as voxelize.h and sharing its
 * return codes and conventions (see voxelize.h: host-side argument checks,
 * caller-owned device memory on the current device, work enqueued on
 * `stream` without synchronising, nothing allocated on the device).
 *
 * The operation is the preprocessing of the RadiusFPS page (hankli.space,
 * "RadiusFPS"): each point of an [N, 4] float32 cloud gets spherical
 * coordinates r = sqrt(x^2 + y^2 + z^2), elevation atan2(z, sqrt(x^2 + y^2))
 * and azimuth atan2(y, x) (section "Spherical voxel partition"); each axis is
 * split uniformly into bins, giving spherical-shell-slice voxels; and the
 * points are sorted once by voxel id so that every voxel's points are
 * contiguous, each voxel then being described by its [start, end) range
 * (the one-off sort and the voxel record of RadiusFPS-G).
 *
 * Binning, exactly (no atan2 rounding enters a result):
 *   - voxel id = (i_r * n_elev + i_elev) * n_azim + i_azim;
 *   - i_r = floorf((r - r_min) / dr) in IEEE fp32 with
 *     r = sqrtf((x*x + y*y) + z*z) (every step correctly rounded, no FMA),
 *     kept when 0 <= i_r < n_r. A point with r == 0 or a NaN/Inf x, y or z
 *     is not kept;
 *   - angle bins compare directions, not rounded angles: boundary k of an
 *     axis is a_k = a_min + k * da (in double, from the float parameters); a
 *     boundary at or below the axis's lowest angle (-pi/2 for elevation, -pi
 *     for azimuth) has every direction above it, one above the highest
 *     (pi/2, pi) has none, and any other is the direction
 *     (float(cos a_k), float(sin a_k)). The bin is the largest k whose
 *     boundary the point's direction is at or above, kept when in [0, n).
 *     Elevation uses the direction (sqrtf(x*x + y*y), z); azimuth uses (x, y)
 *     with angles in (-pi, pi], a -0 y read as +0, and (1, 0) when x = y = 0.
 *     Direction comparisons are exact (cross products of float operands in
 *     double);
 *   - the order lists kept points by voxel id and, inside a voxel, by input
 *     index (a stable counting sort).
 *
 * The angle boundaries need cos and sin, which the device does not evaluate:
 * they are computed once per parameter set on the host into a table
 * (sph_make_table) that the caller copies to device memory and passes to
 * every call with those parameters.
 */
#ifndef SPHERICAL_H
#define SPHERICAL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "voxelize.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits: n_points <= 2^24; every bin count >= 1; n_elev, n_azim <= 65535;
 * n_r * n_elev * n_azim <= 2^22 voxels. dr, d_elev, d_azim finite and > 0;
 * the minima finite. */
#define SPH_MAX_POINTS (1ll << 24)
#define SPH_MAX_VOXELS (1ll << 22)
#define SPH_MAX_ANGLE_BINS 65535

/* Written to n_kept[0] instead of the count when the table does not belong
 * to the call's parameters; nothing else is written. */
#define SPH_STATUS_BAD_TABLE (-18)

/* ---- options (tests and tuning; NULL = defaults) ------------------------- */
/* Two routes give the same results.
 *   Two kernels: when nvox <= 65536 (kept keys of at most 16 bits) and
 *   digit_bits is 0. The binning kernel also groups each tile's kept points
 *   by the key's low digit; the second kernel reads each group of low digits
 *   across all tiles, in input order, and places the points by the high
 *   digit (at most 8 bits) after a look-back over the preceding groups.
 *   Radix passes otherwise: a least-significant-digit radix sort over the
 *   keys [0, nvox] (nvox marks a point that is not kept), ceil(key bits /
 *   digit bits) stable passes, then a kernel for the offsets and rows. */
typedef struct sph_options {
    int32_t points_per_thread; /* binning kernel: 0 = automatic; else 1, 2, 4 or 8
                                  (256-thread blocks, tile = 256 x this) */
    int32_t digit_bits;        /* bits sorted per radix pass: 0 = 8 (the most), or the
                                  two-kernel route when it applies; 1..8 = radix passes */
    int32_t sort_tile;         /* entries per block in a radix pass (1024 threads):
                                  0 = automatic; else 1024, 2048 or 4096 */
} sph_options;

/*
 * Size in bytes of the boundary table for bins (n_r, n_elev, n_azim), or
 * VOX_EINVAL.
 */
int64_t sph_table_bytes(const int32_t bins[3]);

/*
 * Fill the HOST buffer `table` (at least sph_table_bytes(bins) bytes) with
 * the boundary table of these parameters: sph_min = (r_min, elev_min,
 * azim_min), sph_cell = (dr, d_elev, d_azim), bins = (n_r, n_elev, n_azim).
 * The caller copies the bytes to device memory (4-byte aligned) and passes
 * that copy to sph_reorder. Synchronous, host only. Returns VOX_OK or
 * VOX_EINVAL.
 */
int sph_make_table(const float sph_min[3], const float sph_cell[3], const int32_t bins[3],
                   void* table, int64_t table_bytes);

/*
 * Workspace size in bytes for a call with n_points points and these bins
 * (and options, NULL for defaults), or VOX_EINVAL. The workspace is device
 * memory the caller owns, 256-byte aligned. Its first Z bytes,
 * Z = sph_workspace_zero_bytes(same arguments), must be zero before a call
 * (hipMemset or torch.zeros once); a completed call leaves them zero again.
 * The rest needs no initial contents.
 */
int64_t sph_workspace_bytes(int64_t n_points, const int32_t bins[3], const sph_options* options);

/* Z above (16 copies of the global digit histograms, an error word that each
 * call clears itself and, on the two-kernel route, a block counter), or
 * VOX_EINVAL. */
int64_t sph_workspace_zero_bytes(int64_t n_points, const int32_t bins[3],
                                 const sph_options* options);

/* Kernels one call launches, or VOX_EINVAL: 2 on the two-kernel route, else
 * the binning kernel, one per radix pass and the final kernel (at least 3).
 * The length of sph_profile_stages' stage_ms. */
int32_t sph_num_kernels(int64_t n_points, const int32_t bins[3], const sph_options* options);

/*
 * Bin n_points points (device, [n_points, 4] float32, 16-byte aligned) and
 * sort them by voxel. `table` is the device copy of sph_make_table's output
 * for the same sph_min, sph_cell and bins. Outputs, all device memory:
 *   voxel_of [n_points] int32   voxel id of each point, -1 when not kept
 *   offsets  [nvox + 1] int32   first sorted position of each voxel; the
 *                               voxel's points are order[offsets[v] ..
 *                               offsets[v + 1]); offsets[nvox] = kept count
 *   order    [n_points] int32   the first n_kept entries: input indices of the
 *                               kept points in sorted order; the entries past
 *                               n_kept are unspecified
 *   sorted   [n_points, 4] f32  optional (NULL = skipped): the kept rows in
 *                               sorted order, bit copies of the input rows
 *   n_kept   [1] int32          kept count, or SPH_STATUS_BAD_TABLE, or
 *                               VOX_STATUS_DEVICE_ERROR (a bounded wait ran
 *                               out; not reachable with valid inputs)
 * Returns VOX_OK, VOX_EINVAL, VOX_EWORKSPACE or VOX_EHIP.
 */
int sph_reorder(const float* points, int64_t n_points, const float sph_min[3],
                const float sph_cell[3], const int32_t bins[3], const void* table,
                int32_t* voxel_of, int32_t* offsets, int32_t* order, float* sorted,
                int32_t* n_kept, void* workspace, int64_t workspace_bytes,
                const sph_options* options, hipStream_t stream);

/*
 * Run sph_reorder `iters` times (same arguments) and report the mean
 * duration of each kernel in milliseconds, from events recorded with the
 * kernel launches, in launch order (sph_num_kernels() entries): on the
 * two-kernel route the binning kernel and the placing kernel; else the
 * binning kernel, the radix passes and the final kernel. *total_ms is the
 * mean time from the first kernel's start to the last one's end.
 * Synchronises the stream.
 */
int sph_profile_stages(const float* points, int64_t n_points, const float sph_min[3],
                       const float sph_cell[3], const int32_t bins[3], const void* table,
                       int32_t* voxel_of, int32_t* offsets, int32_t* order, float* sorted,
                       int32_t* n_kept, void* workspace, int64_t workspace_bytes,
                       const sph_options* options, hipStream_t stream, int32_t iters,
                       float* stage_ms, float* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SPHERICAL_H */
