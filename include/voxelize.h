/*
 * voxelize.h -- C ABI of the MI355X (gfx950) pillar / voxel binning library.
 *
 * The operation is the one described on the "Voxelize" page
 * (ethan-howes.github.io/projects/voxelize): an unordered [N, 4] float32
 * cloud (x, y, z, intensity) is turned into the three tensors PointPillars
 * consumes (introduction): a [V, K, 4] stack of per-pillar points, [V, 3]
 * int32 grid coordinates (z, y, x) and [V] int32 per-pillar counts. Points are
 * grouped through an open-addressing hash table ("A hash table instead of a
 * sort") sized from the pillar budget, as the page's is ("A fixed table, sized
 * 8x the voxel budget"); here 16 slots per pillar, see vox_options.
 *
 * Output order and content are deterministic (the page's kernel writes pillars
 * in hash-slot order and points in arrival order; this library does not):
 *   - pillars are numbered in order of first occurrence in the input, and the
 *     first max_voxels of them are kept; points whose pillar is past the cap
 *     are dropped;
 *   - each pillar keeps its max_points lowest input indices, in index order
 *     ("keep the first K", section "Claiming a pillar and packing points");
 *   - num_points[p] = min(points in pillar p, max_points); rows past it are
 *     +0.0f; rows are bit copies of the input rows;
 *   - coords[p] = (z, y, x) cell indices, z = 0 in pillar mode (grid[2] == 1).
 * Binning follows section "Binning a point": NaN/Inf in x, y or z rejects a
 * point; the z-slab is z_min <= z < z_max; cell = floorf((v - v_min) / cell)
 * in IEEE fp32 (correctly rounded divide, no FMA, denormals kept); a cell is
 * kept when 0 <= cell < grid (strict upper bound). In 3D mode (grid[2] > 1)
 * the z cell must also lie in [0, grid[2]). x_max and y_max are validated but
 * do not enter binning: the grid size bounds the cell.
 *
 * Conventions for every entry point:
 *   - Returns VOX_OK (0) or a negative VOX_E* code. Argument checks happen on
 *     the host before any HIP call; on an argument error nothing is launched.
 *   - Device pointers belong to the caller and must live on the current HIP
 *     device. Host pointers are read during the call only.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising, unless the entry point says otherwise. Nothing
 *     is allocated on the device.
 *   - The library keeps no mutable global state. Calls on different streams
 *     with different workspaces may run concurrently; two calls that share a
 *     workspace must be ordered (same stream, or synchronised).
 */
#ifndef VOXELIZE_H
#define VOXELIZE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes -------------------------------------------------------- */
#define VOX_OK 0
#define VOX_EINVAL -1      /* bad argument (null pointer, bad size, range, cell or grid) */
#define VOX_EWORKSPACE -2  /* workspace smaller than vox_workspace_bytes() or misaligned */
#define VOX_EHIP -4        /* a HIP call failed; vox_last_hip_error() returns its code */
#define VOX_ESCRATCH -5    /* voxelize_static: the call needs more than its 64 MiB array */

/* ---- device status written to num_voxels[0] instead of V ----------------- */
/* The single-pass path inserts the first P points into
 * the table and decides the max_voxels cap among them. When N > P and those P
 * points hold fewer than max_voxels distinct cells, the cap cannot be decided
 * in one pass: num_voxels[0] is set to VOX_STATUS_NEEDS_CHUNKED, the outputs
 * are not written, the workspace is left clean, and the caller repeats the
 * call with voxelize_chunked(). */
#define VOX_STATUS_NEEDS_CHUNKED (-16)
/* An internal bound was exceeded (a probe sequence longer than the table or a
 * look-back wait past its spin limit). Not reachable with valid inputs; the
 * outputs are not written and the workspace must be re-zeroed. */
#define VOX_STATUS_DEVICE_ERROR (-17)

/* ---- options (tests and tuning; NULL = defaults) ------------------------- */
typedef struct vox_options {
    int64_t table_slots;    /* hash table slots S; 0 = 16 * max_voxels (at least 64);
                               otherwise 2 * max_voxels <= S <= 2^31 - 16; rounded up to
                               a multiple of 16 (one 128-byte line) */
    int64_t prefix_points;  /* points inserted before the cap is decided; 0 = min(N,
                               2 max_voxels, S/4);
                               at most S/2 (and N) */
    int32_t hash;           /* home slot: 0 = key folded to 32 bits times 0x9E3779B1, then a
                               multiply-high reduction to [0, S); 1 = key mod S; 2 = a
                               64-bit mixer, then the same reduction */
    int32_t bucket_cap;     /* per-pillar arrival slots before the overflow row; 0 = 16 * K
                               rounded up to a multiple of 64 (K <= 64); at most 2^20 */
    int32_t compact_table;  /* 1 = lookups past the prefix probe a small table of the
                               kept cells (4 slots per pillar) built by rank; 0 = they
                               probe the main table (default) */
    int32_t select_path;    /* route from lookups to rows (the output is the same):
                               1 = per-pillar buckets filled by one device atomic per
                               point; 2 = partitioned by pillar-id bins in LDS after a
                               rank kernel, rows gathered from the cloud; 3 = as 2, rows
                               carried through the workspace's scratch; 4 = partitioned
                               by first-index bins with no rank kernel (pillar ids from
                               per-tile counts), rows gathered; 0 = automatic: 4 when
                               K <= 64 and the prefix is at most 524,288 points
                               (2048 bins of 256 pillar slots), else 2 when
                               K <= 64 and max_voxels <= 262144, else 1. 2, 3 and 4
                               outside their limits: VOX_EINVAL. The chunked path
                               always takes route 2 (or 1). */
    int32_t kept_map;       /* partitioned routes: 0 = rank also writes a map from grid
                               cell to kept pillar (2 bytes per cell when max_voxels
                               <= 65534, else 4; in the workspace's zero part,
                               2 x table_slots cells at most)
                               and lookups past the prefix read it when the grid has
                               at most that many cells; 1 = lookups probe the table.
                               The map is not used with compact_table = 1. */
    int32_t first_map;      /* route 4: 0 = the claim step writes a map from grid cell to
                               the cell's lowest prefix index (4 bytes per cell, in the
                               kept-cell map's region) when the grid has at most
                               2 x table_slots cells, else it fills the table; 1 = always
                               the table */
    int32_t lane_merge;     /* 1 = lanes of a wavefront that fall in the same cell are
                               merged before the claim atomics (one atomic per distinct
                               cell per wavefront); 0 = one atomic per point (default) */
    int32_t bin_ids;        /* route 4: pillar slots per bin (a power of two, 16 to 256;
                               0 = 128, or 256 when 128 would need more than 512 bins):
                               bins = prefix_points / bin_ids rounded up to a power of
                               two, at most 2048 */
} vox_options;

/*
 * Workspace size in bytes for a call with n_points points, max_voxels and
 * max_points (and options, NULL for defaults). The workspace is device memory
 * the caller owns, 256-byte aligned. It has two parts:
 *   [0, Z)      Z = vox_workspace_zero_bytes(same arguments): must be all zero
 *               before a call (hipMemset or torch.zeros). A completed call
 *               whose num_voxels is not VOX_STATUS_DEVICE_ERROR leaves it
 *               ready again: every byte of [256, Z) is zero, and the first 256
 *               hold only two result words that the next call overwrites.
 *   [Z, bytes)  scratch (the partitioned select route's staging): written
 *               before it is read in every call, left as it is afterwards.
 * A workspace can serve calls of other shapes as long as the new call's
 * [0, Z') is zero: bytes a previous call used as scratch must be zeroed
 * first when Z' reaches into them. After a device error the workspace must
 * be zeroed again. Returns >= 0, or VOX_EINVAL.
 */
int64_t vox_workspace_bytes(int64_t n_points, int32_t max_voxels, int32_t max_points,
                            const vox_options* options);

/* Z above: the size of the workspace's zero part (<= vox_workspace_bytes). */

int64_t vox_workspace_zero_bytes(int64_t n_points, int32_t max_voxels, int32_t max_points,
                                 const vox_options* options);

/*
 * Pillar / voxel binning of one cloud (the whole operation described above).
 *
 *   points      device, [n_points, 4] float32, row-major, 16-byte aligned
 *   n_points    N >= 0, N <= 2^30 - 1; N = 0 gives V = 0
 *   range       host, 6 floats: x_min, y_min, z_min, x_max, y_max, z_max
 *               (finite, min < max)
 *   cell        host, 3 floats: vx, vy, vz (finite, > 0)
 *   grid        host, 3 int32: gx, gy, gz (1 <= g <= 2^24, gx * gy * gz <= 2^33 - 2;
 *               gz == 1 is pillar mode)
 *   max_points  K >= 1 (rows per pillar)
 *   max_voxels  M >= 1 (pillar cap)
 *   voxels      device, [M, K, 4] float32, 16-byte aligned; rows [0, V) written
 *   coords      device, [M, 3] int32 (z, y, x); rows [0, V) written
 *   num_points  device, [M] int32; entries [0, V) written
 *   num_voxels  device, int32[1]: V, or a VOX_STATUS_* code (< 0)
 *   workspace   device, vox_workspace_bytes(N, M, K, options) bytes, zero on entry
 *   stream      HIP stream
 *
 * Rows >= V of the outputs are not touched. Asynchronous: read num_voxels
 * after the stream has completed.
 */
int voxelize(const float* points, int64_t n_points, const float range[6], const float cell[3],
             const int32_t grid[3], int32_t max_points, int32_t max_voxels, float* voxels,
             int32_t* coords, int32_t* num_points, int32_t* num_voxels, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/* voxelize() with options (table size, prefix length, hash); same contract. */
int voxelize_ex(const float* points, int64_t n_points, const float range[6],
                const float cell[3], const int32_t grid[3], int32_t max_points,
                int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                int32_t* num_voxels, void* workspace, size_t workspace_bytes,
                hipStream_t stream, const vox_options* options);

/*
 * The same operation for any input, including the case voxelize() reports as
 * VOX_STATUS_NEEDS_CHUNKED: the table is filled chunk by chunk (each chunk at
 * most table_slots/2 - (cells already in the table) points, so the load never
 * exceeds one half) until max_voxels cells are in it or every point is in.
 * SYNCHRONISES `stream` once per chunk to read the number of cells so far.
 * Same arguments, workspace size and outputs as voxelize_ex().
 */
int voxelize_chunked(const float* points, int64_t n_points, const float range[6],
                     const float cell[3], const int32_t grid[3], int32_t max_points,
                     int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                     int32_t* num_voxels, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const vox_options* options);

/*
 * voxelize_ex() that also returns the inverse map, and can run the chunked
 * path itself:
 *   point_pillar  device int32[n_points] (4-byte aligned), or NULL: for each
 *                 input point, the pillar id of its cell when that pillar is
 *                 kept (whether or not the point is among the pillar's first
 *                 max_points), else -1 (rejected point, or pillar past the cap).
 *                 Written unless num_voxels reports a VOX_STATUS_* code.
 *   chunked       0: single pass, asynchronous (as voxelize_ex());
 *                 1: the chunked path (as voxelize_chunked(), synchronising);
 *                 2: automatic: the single pass, then SYNCHRONISES `stream` once
 *                    to read num_voxels, and only when it reports
 *                    VOX_STATUS_NEEDS_CHUNKED runs the chunked path (which leaves
 *                    the final V or status in num_voxels). The single pass leaves
 *                    the workspace clean, so nothing else is needed between them.
 *                 Other values: VOX_EINVAL.
 * This is what a consumer needs to send per-pillar results back to points.
 */
int voxelize_map(const float* points, int64_t n_points, const float range[6],
                 const float cell[3], const int32_t grid[3], int32_t max_points,
                 int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                 int32_t* num_voxels, int32_t* point_pillar, void* workspace,
                 size_t workspace_bytes, hipStream_t stream, const vox_options* options,
                 int32_t chunked);

/*
 * voxelize() for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same operation, arguments and outputs, with
 * the workspace taken from an array of 64 MiB (VOX_STATIC_SCRATCH_BYTES)
 * that the library holds on each GPU it runs on, from the first call there
 * until the process ends. Calls no hipMalloc, hipFree or other allocating
 * routine.
 *   - Size limit: a call whose vox_workspace_bytes(n_points, max_voxels,
 *     max_points, NULL) exceeds the array returns VOX_ESCRATCH before any HIP
 *     call (with the defaults: 2,097,152 points at 60,000 pillars need about
 *     43 MiB).
 *   - Set-up: the first call on a device takes the array's device address and
 *     enqueues a kernel that clears it on `stream`; keep that first call out
 *     of graph capture. Later calls enqueue only the voxelization kernels (and,
 *     when a larger layout reaches into scratch an earlier call left, or after
 *     a call that returned VOX_EHIP, one clearing kernel first).
 *   - Sharing: every call on a GPU uses that GPU's one array, which keeps the
 *     last call's contents. Calls that overlap on one GPU (two streams or
 *     two host threads without ordering) race on it and give wrong results:
 *     order them. Host-side bookkeeping is guarded by a mutex.
 *   - Status: as voxelize(); an undecided cap (VOX_STATUS_NEEDS_CHUNKED)
 *     needs voxelize_chunked() with a workspace. After a device error the
 *     call's last kernel clears the array's zero part itself.
 * Asynchronous on `stream`; read num_voxels after the stream has completed.
 */
#define VOX_STATIC_SCRATCH_BYTES (64ll << 20)
int voxelize_static(const float* points, int64_t n_points, const float range[6],
                    const float cell[3], const int32_t grid[3], int32_t max_points,
                    int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                    int32_t* num_voxels, hipStream_t stream);

/* The select route a single pass would take (1 to 4, as select_path above), or
 * VOX_EINVAL. */
int32_t vox_select_route(int64_t n_points, int32_t max_voxels, int32_t max_points,
                         const vox_options* options);

/*
 * The sizes a call would use (for reports and tests): table slots S, prefix
 * length P and bucket slots per pillar (0 when max_points > 64 or when the
 * partitioned select path is taken, which has no buckets). Any output
 * pointer may be NULL. Returns VOX_OK or VOX_EINVAL.
 */
int vox_plan(int64_t n_points, int32_t max_voxels, int32_t max_points,
             const vox_options* options, int64_t* table_slots, int64_t* prefix_points,
             int32_t* bucket_cap);

/*
 * Voxel-grid downsampling (the voxel_downsample operation, section 4.4
 * "operation 1", of the GPU K-D tree ICP page, which truncates the cell
 * index and averages with float atomics). One mean point per kept voxel:
 *   - binning, voxel numbering in first-occurrence order and the max_voxels
 *     cap are voxelize()'s (floorf cell index, same reject rules);
 *   - centroids[p] (x, y, z, intensity) = for each channel, the sum over the
 *     voxel's points in input order in double precision, divided by the count
 *     in double precision, rounded once to float (round to nearest); NaN and
 *     Inf propagate through the sums;
 *   - coords[p] = (z, y, x) of the voxel, counts[p] = all of its points.
 * points: device [N,4] f32, 16-byte aligned. centroids: device [max_voxels,4]
 * f32, 16-byte aligned; coords [max_voxels,3] i32; counts [max_voxels] i32;
 * num_voxels [1] i32 receives V or a VOX_STATUS_* code, as for voxelize().
 * Rows [0, V) are written, rows past V untouched. options: table_slots,
 * prefix_points, hash, compact_table, kept_map, first_map, lane_merge and
 * bin_ids apply; select_path 0 (automatic: route 4 with rows carried where
 * it applies, as for voxelize(), else 3), 3 (rows carried through route 2's
 * partition) or 4 (VOX_EINVAL where it does not apply); others VOX_EINVAL;
 * max_voxels <= 262144. Route 4's workspace also holds route 3's layout,
 * which the chunked path takes.
 * chunked = 1 inserts chunk by chunk with a host sync between chunks (needed
 * when the status is VOX_STATUS_NEEDS_CHUNKED). The workspace follows the
 * rules of vox_workspace_bytes() with the two sizes below. Asynchronous on
 * `stream` unless chunked; allocates nothing. Returns VOX_OK or a negative
 * code (VOX_EINVAL, VOX_EWORKSPACE, VOX_EHIP).
 */
int vox_downsample(const float* points, int64_t n_points, const float range[6],
                   const float cell[3], const int32_t grid[3], int32_t max_voxels,
                   float* centroids, int32_t* coords, int32_t* counts, int32_t* num_voxels,
                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                   const vox_options* options, int32_t chunked);
int64_t vox_downsample_workspace_bytes(int64_t n_points, int32_t max_voxels,
                                       const vox_options* options);
int64_t vox_downsample_workspace_zero_bytes(int64_t n_points, int32_t max_voxels,
                                            const vox_options* options);

/*
 * The per-point binning step alone ("Binning a point"), for parity tests:
 * valid[i] = 1 if point i is kept, else 0; key[i] = (cz * gy + cy) * gx + cx
 * as int64 (cz = 0 in pillar mode), or -1. valid and key are device arrays of
 * n_points entries. Asynchronous.
 */
int vox_bin_points(const float* points, int64_t n_points, const float range[6],
                   const float cell[3], const int32_t grid[3], int8_t* valid, int64_t* key,
                   hipStream_t stream);

/*
 * Stage timing for the benchmark: runs voxelize_ex() `iters` times on
 * `stream`, each kernel launched with a start and a stop event that the HIP
 * runtime stamps at the kernel's own start and end (hipExtLaunchKernel), and
 * writes the mean milliseconds of each stage's kernel to
 * stage_ms[0..VOX_NUM_STAGES) (insert, rank, select, pack) and from the first
 * kernel's start to the last one's end to *total_ms. Synchronises `stream`.
 */
#define VOX_NUM_STAGES 4
int vox_profile_stages(const float* points, int64_t n_points, const float range[6],
                       const float cell[3], const int32_t grid[3], int32_t max_points,
                       int32_t max_voxels, float* voxels, int32_t* coords,
                       int32_t* num_points, int32_t* num_voxels, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, const vox_options* options,
                       int32_t iters, float* stage_ms, float* total_ms);

/* Name of each stage, for reports ("insert", "rank", "select", "pack"). */
const char* vox_stage_name(int32_t stage);

/* Human-readable text for a return code or a device status. */
const char* vox_strerror(int32_t code);

/* The hipError_t of the last HIP failure seen by this thread (0 if none). */
int32_t vox_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VOXELIZE_H */
