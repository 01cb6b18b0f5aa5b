// Spherical binning and voxel-contiguous reorder for MI355X (gfx950).
//
// The preprocessing of the RadiusFPS page (hankli.space, "RadiusFPS"):
// spherical coordinates per point and uniform bins per axis (section
// "Spherical voxel partition"), then one sort of the cloud by voxel id so a
// voxel's points are contiguous and the voxel is a [start, end) range (the
// preprocessing step and voxel record of RadiusFPS-G). The exact binning
// rules are stated in spherical.h.
//
// Grids of up to 65,536 voxels (kept keys of at most 16 bits) take two
// kernels, k_sph_lowpart and k_sph_place (described where they are defined):
// the binning kernel groups each tile's kept points by the key's low digit,
// and the placing kernel reads one group of low digits across every tile in
// input order and places the points by the high digit, so no pass over all
// points is needed between binning and the final write.
//
// Larger grids, or a digit width given in the options, take a
// least-significant-digit radix sort of (voxel id, point index) pairs, so
// every kernel does the same work per tile whatever the spread of points
// over voxels (a LiDAR scan puts most of its points in a few near shells):
//   k_sph_key    bins each point, writes its voxel id (a dropped point gets
//                the key nvox, which sorts after every voxel) and adds the
//                block's digit counts of every pass to global histograms.
//   k_sph_pass   one per digit (at most 8 bits): each tile of 256 x PER
//                entries ranks its entries by digit stably in LDS, finds
//                where each digit's run goes from the global histogram and a
//                decoupled look-back over the preceding tiles' counts, and
//                writes the tile out in digit order (coalesced runs). Stable
//                passes from the lowest digit up leave the pairs sorted by
//                voxel id and, inside a voxel, by input index.
//   k_sph_final  voxel offsets from the boundaries between sorted keys, the
//                kept count, the rows gathered in sorted order, and the
//                histograms reset to zero for the next call.
//
// Angle bins: an estimate of the bin (a polynomial atan2) is refined by
// exact direction tests against the table's boundary directions (cross
// products of float operands in double), so the estimate never decides a bin.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <math.h>
#include <string.h>

#include "spherical.h"
#include "wave_ops.h"

int ssh_hip_fail(hipError_t e);  // records the error for vox_last_hip_error()

namespace {

constexpr int kSBlock = 256;                 // 4 wavefronts (binning and final kernels)
constexpr int kSPassBlock = 1024;            // 16 wavefronts (sort passes)
constexpr int kSPassWaves = kSPassBlock / kWave;
constexpr int kSMaxDigitBits = 8;
constexpr int kSMaxDigits = 1 << kSMaxDigitBits;
constexpr int kSMaxPasses = 23;              // 1-bit digits over a 23-bit key
constexpr int kSHistWords = 768;             // digits summed over the passes, at most
constexpr long long kSMaxTiles = 65536;
constexpr int kSHistCopies = 16;             // global histograms, block b adds to copy b % 16
constexpr int kSTableLds = 2048;             // boundary directions staged in LDS, at most
constexpr int kSLookBack = 32;               // predecessor tiles read per look-back round trip
constexpr int kSLookBackLane = 24;           // predecessors per lane in look_back_wide
constexpr int kSWavesPart = kSBlock / kWave; // wavefronts of a binning block
constexpr int kSMaxRuns = 4096;              // runs one k_sph_place block reads, at most
constexpr int kSPlacePer = 6;                // entries per thread in a k_sph_place chunk
constexpr int kSPlacePerSmall = 3;           // the same up to 2,048 points per placing block
constexpr int kSPairsMax = 4096;             // (low digit, high digit) counters per block, at most
constexpr int kSMaxLowBits = 11;             // low digit of the two-kernel route, at most
constexpr unsigned kSMagic = 0x31485053u;    // "SPH1"
constexpr unsigned kSSpinLimit = 1u << 22;   // look-back poll bound (never reached in practice)
constexpr unsigned kSAgg = 1u << 30;         // look-back word: flag bits 31..30, count below
constexpr unsigned kSIncl = 2u << 30;
constexpr unsigned kSValue = (1u << 30) - 1u;
constexpr double kSPi = 3.141592653589793;       // both roundings lie below the true value
constexpr double kSHalfPi = 1.5707963267948966;

// Head of the boundary table; elevation then azimuth directions follow as
// float2 (cos, sin), n + 1 per axis.
struct SphHeader {
    unsigned magic;
    int nr, nt, np;
    float mn[3];
    float cell[3];
    int t_lo, t_hi;   // elevation boundaries k < t_lo: every direction is at or above;
    int p_lo, p_hi;   // k > t_hi: none is. Same for azimuth.
    unsigned bytes, pad;
};
static_assert(sizeof(SphHeader) == 64, "table header is 64 bytes");

struct SphArgs {
    float mn[3];
    float cell[3];
    float inv_cell[3];   // 1 / cell, for the angle estimates only
    int nr, nt, np;
    int nvox;         // also the key of a dropped point
    int ntiles;       // binning kernel: tiles of 256 x PER points
    int tile;
    int sort_tiles;   // sort passes: tiles of 1024 x PER entries
    int sort_tile;
};

// Digit layout of the passes: pass p sorts by (key >> shift[p]) & (2^bits[p] - 1);
// its counts sit at hoff[p] in the histogram words.
struct SphDigits {
    int passes;
    int shift[kSMaxPasses];
    int bits[kSMaxPasses];
    int hoff[kSMaxPasses];
    int hist_words;
};

__device__ __forceinline__ unsigned load_relaxed32(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed32(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool table_ok(const SphHeader* __restrict__ h, const SphArgs& a) {
    bool ok = h->magic == kSMagic && h->nr == a.nr && h->nt == a.nt && h->np == a.np;
#pragma unroll
    for (int d = 0; d < 3; ++d)
        ok = ok && __float_as_uint(h->mn[d]) == __float_as_uint(a.mn[d]) &&
             __float_as_uint(h->cell[d]) == __float_as_uint(a.cell[d]);
    return ok;
}

// ---------------------------------------------------------------- binning --

// Half-turn of a direction for angles in (-pi, pi]: 0 below the x axis,
// 1 for [0, pi), 2 for the negative x axis (angle pi).
__device__ __forceinline__ int half_turn(float x, float y) {
    return y < 0.0f ? 0 : ((y > 0.0f || x > 0.0f) ? 1 : 2);
}

// Largest k in [-1, n] whose boundary the direction is at or above, starting
// from the estimate k0; ge(k) is monotone (true up to some k, then false).
template <typename Ge>
__device__ __forceinline__ int refine(int k0, int n, Ge ge) {
    int k = k0;
    while (k >= 0 && !ge(k)) --k;
    while (k < n && ge(k + 1)) ++k;
    return k;
}

__device__ __forceinline__ int clamp_estimate(float f, int n) {
    return (int)fminf(fmaxf(f, -1.0f), (float)n);   // NaN -> -1
}

// Angle of the direction (x, y) in [-pi, pi], as an estimate only: the bin
// it suggests is refined by exact tests, so its error decides nothing but
// the number of refinement steps. Octant reduction to t = min/max in [0, 1],
// then atan(t) ~ t P(t^2) with P of degree 6 fitted to atan(t)/t by least
// squares on [0, 1] (at most 7e-7 rad off in float arithmetic). x = y = 0
// gives NaN, which the caller's clamp turns into a start at -1.
__device__ __forceinline__ float atan2_estimate(float y, float x) {
    const float ax = fabsf(x), ay = fabsf(y);
    const float t = fminf(ax, ay) * __builtin_amdgcn_rcpf(fmaxf(ax, ay));
    const float u = t * t;
    float q = 0.008096857f;
    q = q * u - 0.03775049f;
    q = q * u + 0.0847584382f;
    q = q * u - 0.13537614f;
    q = q * u + 0.198950127f;
    q = q * u - 0.333279759f;
    q = q * u + 0.999999702f;
    float r = t * q;
    if (ay > ax) r = 1.57079633f - r;
    if (x < 0.0f) r = 3.14159265f - r;
    return y < 0.0f ? -r : r;
}

// Voxel id of one point, -1 when not kept.
__device__ __forceinline__ int sph_voxel(float4 p, const SphArgs& a, const SphHeader* __restrict__ h,
                                         const float2* __restrict__ tb,
                                         const float2* __restrict__ pb) {
    const float x = p.x, y = p.y, z = p.z;
    if (!(isfinite(x) && isfinite(y) && isfinite(z))) return -1;
    const float sxy = x * x + y * y;          // no contraction: two products, one sum
    const float r = sqrtf(sxy + z * z);       // correctly rounded
    if (r == 0.0f) return -1;
    const float fr = floorf((r - a.mn[0]) / a.cell[0]);
    if (!(fr >= 0.0f && fr < (float)a.nr)) return -1;
    const float rxy = sqrtf(sxy);

    const int t_lo = h->t_lo, t_hi = h->t_hi;
    const int it = refine(
        clamp_estimate(floorf((atan2_estimate(z, rxy) - a.mn[1]) * a.inv_cell[1]), a.nt), a.nt,
        [&](int k) {
            if (k < t_lo) return true;
            if (k > t_hi) return false;
            const float2 d = tb[k];
            return (double)d.x * (double)z - (double)d.y * (double)rxy >= 0.0;
        });
    if (it < 0 || it >= a.nt) return -1;

    float ax = x, ay = y + 0.0f;              // -0 + 0 = +0
    if (x == 0.0f && y == 0.0f) {
        ax = 1.0f;
        ay = 0.0f;
    }
    const int hp = half_turn(ax, ay);
    const int p_lo = h->p_lo, p_hi = h->p_hi;
    const int ip = refine(
        clamp_estimate(floorf((atan2_estimate(ay, ax) - a.mn[2]) * a.inv_cell[2]), a.np), a.np,
        [&](int k) {
            if (k < p_lo) return true;
            if (k > p_hi) return false;
            const float2 d = pb[k];
            const int hd = half_turn(d.x, d.y);
            if (hp != hd) return hp > hd;
            return (double)d.x * (double)ay - (double)d.y * (double)ax >= 0.0;
        });
    if (ip < 0 || ip >= a.np) return -1;
    return (int)(((long long)fr * a.nt + it) * a.np + ip);
}

// ------------------------------------------------------------------- keys --

// Tile t = blockIdx.x holds points [t T, t T + T), T = 256 PER; wavefront w
// takes [t T + 64 PER w, t T + 64 PER (w + 1)), 64 at a time (the layout of
// every kernel here). Also clears the look-back words of every pass and the
// error word the passes may set. The digit counts go to one of 16 copies of
// the histograms (by block), so no counter takes an add from every block.
template <int PER, bool LDS_TABLE>
__global__ __launch_bounds__(kSBlock) void k_sph_key(const float4* __restrict__ pts, long long N,
                                                     SphArgs a, const SphHeader* __restrict__ tab,
                                                     SphDigits dg, int* __restrict__ voxel_of,
                                                     unsigned* __restrict__ ghist,
                                                     unsigned* __restrict__ state,
                                                     long long state_words,
                                                     unsigned* __restrict__ err) {
    __shared__ unsigned h[kSHistWords];
    __shared__ float2 stab[LDS_TABLE ? kSTableLds : 1];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid / kWave;
    const long long stride = (long long)gridDim.x * kSBlock;
    for (long long j = (long long)blockIdx.x * kSBlock + tid; j < state_words; j += stride)
        state[j] = 0u;
    if (blockIdx.x == 0 && tid == 0) *err = 0u;
    if (!table_ok(tab, a)) return;   // same for every block
    const float2* gtb = reinterpret_cast<const float2*>(tab + 1);
    const int ndirs = a.nt + 1 + a.np + 1;
    if (LDS_TABLE)
        for (int j = tid; j < ndirs; j += kSBlock) stab[j] = gtb[j];
    const float2* tb = LDS_TABLE ? stab : gtb;
    const float2* pb = tb + (a.nt + 1);
    for (int j = tid; j < dg.hist_words; j += kSBlock) h[j] = 0u;
    const long long wbase = (long long)blockIdx.x * a.tile + (long long)w * kWave * PER;
    float4 p[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const long long i = wbase + k * kWave + lane;
        p[k] = i < N ? pts[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();   // h cleared, directions staged
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const long long i = wbase + k * kWave + lane;
        if (i >= N) continue;
        const int v = sph_voxel(p[k], a, tab, tb, pb);
        voxel_of[i] = v;
        const unsigned key = v < 0 ? (unsigned)a.nvox : (unsigned)v;
        for (int q = 0; q < dg.passes; ++q)
            atomicAdd(&h[dg.hoff[q] + ((key >> dg.shift[q]) & ((1u << dg.bits[q]) - 1u))], 1u);
    }
    __syncthreads();
    unsigned* gcopy = ghist + (blockIdx.x % kSHistCopies) * dg.hist_words;
    for (int j = tid; j < dg.hist_words; j += kSBlock)
        if (h[j]) atomicAdd(&gcopy[j], h[j]);
}

// ------------------------------------------------------------------ passes --

// One stable pass by the digit (key >> shift) & (2^dbits - 1). keys_in is
// the voxel_of array on the first pass (a negative id reads as nvox) and
// vals_in is then null (the value is the point index). ghist holds this
// pass's global digit counts (16 copies, hist_words apart), state its look-back words (ntiles x 2^dbits,
// zero at launch). Every tile publishes its digit counts before it looks
// back, so the wait only covers tiles that have not counted yet.
template <int PER>
__global__ __launch_bounds__(kSPassBlock) void k_sph_pass(
    const int* __restrict__ keys_in, const unsigned* __restrict__ vals_in,
    unsigned* __restrict__ keys_out, unsigned* __restrict__ vals_out, long long N, SphArgs a,
    const SphHeader* __restrict__ tab, int shift, int dbits, const unsigned* __restrict__ ghist,
    int hist_words, unsigned* __restrict__ state, unsigned* __restrict__ err) {
    constexpr int T = kSPassBlock * PER;
    constexpr int NW = kSPassWaves;
    __shared__ unsigned hist[NW * kSMaxDigits];
    __shared__ unsigned sk[T], sv[T];
    __shared__ unsigned lstart[kSMaxDigits], gbase[kSMaxDigits];
    __shared__ unsigned wsum[kWsumWords];
    if (!table_ok(tab, a)) return;
    const int tid = threadIdx.x, lane = __lane_id(), w = tid / kWave;
    // Tiles follow block indices. A tile waits only on lower-numbered
    // blocks; the dispatcher starts workgroups in increasing order, so
    // those are resident or finished, and they never wait on a higher one:
    // every wait ends. The poll bound turns a stall that this argument
    // rules out into an error status instead of a hang.
    const int tile = blockIdx.x;
    const int nb = 1 << dbits;
    const unsigned dmask = (unsigned)nb - 1u;
    for (int j = tid; j < NW * nb; j += kSPassBlock) hist[j] = 0u;
    // this digit's global count (thread tid owns digit tid), loaded early
    unsigned gd = 0;
    if (tid < nb)
#pragma unroll
        for (int c = 0; c < kSHistCopies; ++c) gd += ghist[c * hist_words + tid];
    const long long base = (long long)tile * T;
    const long long wbase = base + (long long)w * kWave * PER;
    unsigned key[PER], val[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const long long i = wbase + k * kWave + lane;
        key[k] = 0u;
        val[k] = (unsigned)i;
        if (i < N) {
            const int kin = keys_in[i];
            key[k] = kin < 0 ? (unsigned)a.nvox : (unsigned)kin;
            if (vals_in) val[k] = vals_in[i];
        }
    }
    __syncthreads();   // hist cleared

    // stable rank inside (wavefront, digit): earlier k first, then lower lanes
    unsigned* hw = hist + w * nb;
    unsigned rk[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const bool ok = wbase + k * kWave + lane < N;
        const unsigned d = (key[k] >> shift) & dmask;
        const unsigned long long peers = match_mask(d, ok, dbits);
        rk[k] = ok ? hw[d] + (unsigned)__popcll(peers & lanes_below(lane)) : 0u;
        if (ok && (peers & lanes_above(lane)) == 0ull) hw[d] += (unsigned)__popcll(peers);
    }
    __syncthreads();

    // thread d owns digit d: tile count, per-wavefront prefix, publication
    const int d = tid;
    unsigned c = 0;
    if (d < nb) {
        for (int ww = 0; ww < NW; ++ww) {
            const unsigned x = hist[ww * nb + d];
            hist[ww * nb + d] = c;
            c += x;
        }
        store_relaxed32(&state[(long long)tile * nb + d], (tile == 0 ? kSIncl : kSAgg) | c);
    }
    // the first look-back window is in flight while the block scans run
    int hi = tile - 1;
    unsigned sw[kSLookBack];
#pragma unroll
    for (int j = 0; j < kSLookBack; ++j)
        sw[j] = (d < nb && hi - j >= 0) ? load_relaxed32(&state[(long long)(hi - j) * nb + d])
                                        : kSIncl;
    unsigned tile_total, all;
    const unsigned ls = block_excl_scan<NW>(d < nb ? c : 0u, wsum, &tile_total);
    const unsigned g0 = block_excl_scan<NW>(gd, wsum, &all);
    if (d < nb) {
        // kSLookBack predecessors per round trip, nearest first: add their
        // counts up to the nearest inclusive prefix; a tile that has not
        // published yet is polled again (the counts before it are final)
        unsigned excl = 0;
        unsigned polls = 0;
        bool failed = false;
        while (true) {
            bool done = false, wait = false;
            int used = 0;
#pragma unroll
            for (int j = 0; j < kSLookBack; ++j) {
                if (done || wait) continue;
                const unsigned flag = sw[j] & ~kSValue;
                if (flag == 0u) {
                    wait = true;
                } else {
                    excl += sw[j] & kSValue;
                    used = j + 1;
                    done = flag == kSIncl;
                }
            }
            if (done) break;
            hi -= used;
            if (wait) {
                if (++polls > kSSpinLimit) {
                    atomicOr(err, 1u);
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int j = 0; j < kSLookBack; ++j)
                sw[j] = hi - j >= 0 ? load_relaxed32(&state[(long long)(hi - j) * nb + d]) : kSIncl;
        }
        // an inclusive word built on a partial prefix is never published:
        // after a failed wait the tile's successors keep waiting on it and
        // fail in turn, and the call reports the error
        if (tile > 0 && !failed)
            store_relaxed32(&state[(long long)tile * nb + d], kSIncl | (excl + c));
        lstart[d] = ls;
        gbase[d] = g0 + excl;
    }
    __syncthreads();

    // the tile in digit order in LDS, then written out run by run
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (wbase + k * kWave + lane >= N) continue;
        const unsigned dd = (key[k] >> shift) & dmask;
        const unsigned lp = lstart[dd] + hist[w * nb + dd] + rk[k];
        sk[lp] = key[k];
        sv[lp] = val[k];
    }
    __syncthreads();
    const int n_here = (int)(N - base < T ? N - base : T);
    for (int q = tid; q < n_here; q += kSPassBlock) {
        const unsigned kq = sk[q];
        const unsigned dd = (kq >> shift) & dmask;
        const unsigned out = gbase[dd] + ((unsigned)q - lstart[dd]);
        keys_out[out] = kq;
        vals_out[out] = sv[q];
    }
}

// ------------------------------------------------------------------- final --

// offsets[v] = q for v in [lo, hi] (empty when lo > hi). Ranges longer than
// a few entries are written by the whole wavefront together; every lane of
// the wavefront must call this.
__device__ __forceinline__ void fill_offsets(int* __restrict__ offsets, long long lo, long long hi,
                                             int value, int lane) {
    const bool longr = hi - lo >= 16;
    if (!longr)
        for (long long v = lo; v <= hi; ++v) offsets[v] = value;
    unsigned long long m = __ballot(longr);
    while (m) {
        const int src = __builtin_ctzll(m);
        m &= m - 1ull;
        const long long l0 = __shfl(lo, src), h0 = __shfl(hi, src);
        const int val = __shfl(value, src);
        for (long long v = l0 + lane; v <= h0; v += kWave) offsets[v] = val;
    }
}

// Sorted keys -> voxel offsets: position q starts every voxel in
// (key[q - 1], key[q]]; after the last kept key, the voxels up to nvox start
// at the kept count. Rows are gathered in sorted order. Block 0 resets the
// digit histograms (every pass has read them) and writes the status when
// there is one; with a status, no block reads the sorted arrays.
__global__ __launch_bounds__(kSBlock) void k_sph_final(
    const unsigned* __restrict__ skeys, const int* __restrict__ order,
    const float4* __restrict__ pts, float4* __restrict__ sorted, int* __restrict__ offsets,
    int* __restrict__ n_kept, long long N, SphArgs a, const SphHeader* __restrict__ tab,
    unsigned* __restrict__ ghist, int hist_words, const unsigned* __restrict__ err) {
    const int tid = threadIdx.x, lane = __lane_id(), w = tid / kWave;
    const bool ok = table_ok(tab, a);
    const bool failed = *err != 0u;   // set by a pass, cleared only by the next call's first kernel
    if (blockIdx.x == 0) {
        for (int j = tid; j < kSHistCopies * hist_words; j += kSBlock) ghist[j] = 0u;
        if (tid == 0) {
            if (!ok) *n_kept = SPH_STATUS_BAD_TABLE;
            else if (failed) *n_kept = VOX_STATUS_DEVICE_ERROR;
        }
    }
    if (!ok || failed) return;
    const long long nvox = a.nvox;
    if (N == 0) {
        for (long long v = (long long)blockIdx.x * kSBlock + tid; v <= nvox;
             v += (long long)gridDim.x * kSBlock)
            offsets[v] = 0;
        if (blockIdx.x == 0 && tid == 0) *n_kept = 0;
        return;
    }
    const long long stride = (long long)gridDim.x * kSBlock;
    for (long long q0 = (long long)blockIdx.x * kSBlock + w * kWave; q0 < N; q0 += stride) {
        const long long q = q0 + lane;
        const bool valid = q < N;
        const long long key = valid ? (long long)skeys[q] : 0;
        const long long prev = (valid && q > 0) ? (long long)skeys[q - 1] : -1;
        const bool starts = valid && key != prev;
        fill_offsets(offsets, starts ? prev + 1 : 1, starts ? key : 0, (int)q, lane);
        if (starts && key == nvox) *n_kept = (int)q;
        const bool last_kept = valid && q == N - 1 && key < nvox;
        fill_offsets(offsets, last_kept ? key + 1 : 1, last_kept ? nvox : 0, (int)N, lane);
        if (last_kept) *n_kept = (int)N;
        if (valid && key < nvox && sorted) sorted[q] = pts[order[q]];
    }
}

// ------------------------------------------------------ two-kernel route --
//
// For keys of at most 16 bits (grids of up to 65,536 voxels) the sort takes
// two kernels. The key is split into a low digit (b0 bits) and a high digit
// (b1 <= 8 bits); only kept points are sorted. A point's voxel is
// (high digit << b0) | low digit, so sorted order is high digit first.
//   k_sph_lowpart  bins the points (as k_sph_key) and partitions each tile of
//                  256 x PER points stably by the low digit in LDS: the tile's
//                  kept entries (and rows) go out to its staging slice grouped
//                  by low digit, one (start, length) word per (low digit,
//                  tile) goes to cm, and the high digits are counted into 16
//                  copies of a global histogram.
//   k_sph_place    one 1,024-thread block per (group of per_block low digits,
//                  range of tiles); a group split over several ranges has one
//                  low digit. Reading the block's runs digit by digit, tile by
//                  tile, visits its entries in the order a stable pass by the
//                  low digit would leave them. The block counts them per (low
//                  digit, high digit), takes each high digit's start from the
//                  global histogram and a look-back over the preceding blocks
//                  (blocks ordered group-major, range-minor, which is that
//                  same order), writes the offsets of its voxels, ranks its
//                  entries stably by high digit (per-wavefront counts in
//                  LDS) and stores each at its sorted position: the block's
//                  entries of one high digit fill one contiguous range.
// The last block to finish (a counter in the zero part) writes the kept
// count and returns the histograms and the counter to zero.

// Tile layout of k_sph_key; the tile index is spread so that each XCD takes
// neighbouring tiles. LDS (dynamic): hist[4 x 2^b0], the boundary directions
// when staged, then the tile's partitioned words [T] and rows [T] (rows only
// when srows is set).
template <int PER, bool LDS_TABLE>
__global__ __launch_bounds__(kSBlock) void k_sph_lowpart(
    const float4* __restrict__ pts, long long N, SphArgs a, const SphHeader* __restrict__ tab,
    int b0, int b1, int* __restrict__ voxel_of, unsigned* __restrict__ cm,
    unsigned* __restrict__ swords, float4* __restrict__ srows, unsigned* __restrict__ ghist,
    unsigned* __restrict__ state, long long state_words, unsigned* __restrict__ err,
    int nt_stores) {
    constexpr int T = kSBlock * PER;
    extern __shared__ __align__(16) unsigned lds[];
    __shared__ unsigned h1[kSMaxDigits];
    __shared__ unsigned wsum[kWsumWords];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid / kWave;
    const long long stride = (long long)gridDim.x * kSBlock;
    for (long long j = (long long)blockIdx.x * kSBlock + tid; j < state_words; j += stride)
        state[j] = 0u;
    if (blockIdx.x == 0 && tid == 0) *err = 0u;
    if (!table_ok(tab, a)) return;   // same for every block
    const int nb0 = 1 << b0, nb1 = 1 << b1;
    const unsigned m0 = (unsigned)nb0 - 1u;
    const int ndirs = a.nt + 1 + a.np + 1;
    unsigned* hist = lds;
    float2* stab = reinterpret_cast<float2*>(lds + kSWavesPart * nb0);   // 16-byte aligned
    const int ndl = LDS_TABLE ? ((ndirs + 1) & ~1) : 0;                  // keeps 16-byte alignment
    unsigned* tw = reinterpret_cast<unsigned*>(stab + ndl);
    float4* tr = reinterpret_cast<float4*>(tw + T);
    const float2* gtb = reinterpret_cast<const float2*>(tab + 1);
    if (LDS_TABLE)
        for (int j = tid; j < ndirs; j += kSBlock) stab[j] = gtb[j];
    const float2* tb = LDS_TABLE ? stab : gtb;
    const float2* pb = tb + (a.nt + 1);
    for (int j = tid; j < kSWavesPart * nb0; j += kSBlock) hist[j] = 0u;
    for (int j = tid; j < nb1; j += kSBlock) h1[j] = 0u;
    const long long ntiles = a.ntiles;
    const long long tile = xcd_tile(blockIdx.x, ntiles);
    const long long base = tile * T;
    const long long wbase = base + (long long)w * kWave * PER;
    float4 p[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const long long i = wbase + k * kWave + lane;
        p[k] = i < N ? pts[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();   // hist, h1 cleared; directions staged
    int vox[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const long long i = wbase + k * kWave + lane;
        int v = -1;
        if (i < N) {
            v = sph_voxel(p[k], a, tab, tb, pb);
            voxel_of[i] = v;
            if (v >= 0) atomicAdd(&h1[(unsigned)v >> b0], 1u);
        }
        vox[k] = v;
    }
    // stable rank inside (wavefront, low digit): earlier k first, then lower lanes
    unsigned* hw = hist + w * nb0;
    unsigned rk[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const bool ok = vox[k] >= 0;
        const unsigned d0 = ok ? ((unsigned)vox[k] & m0) : 0u;
        const unsigned long long peers = match_mask(d0, ok, b0);
        rk[k] = ok ? hw[d0] + (unsigned)__popcll(peers & lanes_below(lane)) : 0u;
        if (ok && (peers & lanes_above(lane)) == 0ull) hw[d0] += (unsigned)__popcll(peers);
    }
    __syncthreads();
    // digit-major offsets: each thread owns bpt consecutive low digits
    const int bpt = (nb0 + kSBlock - 1) / kSBlock;
    const int d0s = tid * bpt;
    unsigned mine = 0;
    for (int j = 0; j < bpt; ++j) {
        const int d = d0s + j;
        if (d < nb0)
            for (int ww = 0; ww < kSWavesPart; ++ww) mine += hist[ww * nb0 + d];
    }
    unsigned kept;
    unsigned run = block_excl_scan<kSWavesPart>(mine, wsum, &kept);
    for (int j = 0; j < bpt; ++j) {
        const int d = d0s + j;
        if (d >= nb0) break;
        const unsigned start = run;
        for (int ww = 0; ww < kSWavesPart; ++ww) {
            const unsigned c = hist[ww * nb0 + d];
            hist[ww * nb0 + d] = run;
            run += c;
        }
        cm[(long long)d * ntiles + tile] = start | ((run - start) << 16);
    }
    __syncthreads();
    // the tile in low-digit order in LDS, then written out contiguously
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (vox[k] < 0) continue;
        const unsigned v = (unsigned)vox[k];
        const unsigned pos = hw[v & m0] + rk[k];
        tw[pos] = ((v >> b0) << 16) | (unsigned)(w * kWave * PER + k * kWave + lane);
        if (srows) tr[pos] = p[k];
    }
    __syncthreads();
    if (nt_stores) {   // block-uniform
        // streaming stores: on large scans they measured faster than
        // ordinary ones, the staging slices being read only once, by the
        // placing kernel
        typedef float v4f __attribute__((ext_vector_type(4)));
        for (int q = tid; q < (int)kept; q += kSBlock) {
            __builtin_nontemporal_store(tw[q], &swords[base + q]);
            if (srows) {
                const float4 r = tr[q];
                v4f x;
                x.x = r.x;
                x.y = r.y;
                x.z = r.z;
                x.w = r.w;
                __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(&srows[base + q]));
            }
        }
    } else {
        for (int q = tid; q < (int)kept; q += kSBlock) {
            swords[base + q] = tw[q];
            if (srows) srows[base + q] = tr[q];
        }
    }
    unsigned* gcopy = ghist + (blockIdx.x % kSHistCopies) * nb1;
    for (int j = tid; j < nb1; j += kSBlock)
        if (h1[j]) atomicAdd(&gcopy[j], h1[j]);
}

// Stable rank of a chunk's entries by high digit (word >> 16): entry (w, k,
// lane) comes after the chunk's earlier entries in wavefront w (lower k, then
// lower lanes); hist[w * nb1 + d] gets wavefront w's count of digit d.
template <int E>
__device__ __forceinline__ void rank_high(const unsigned (&word)[E], const bool (&ok)[E],
                                          unsigned (&rk)[E], unsigned* hist, int w, int lane,
                                          int b1) {
    unsigned* hw = hist + w * (1 << b1);
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const unsigned d = word[k] >> 16;
        const unsigned long long peers = match_mask(d, ok[k], b1);
        rk[k] = ok[k] ? hw[d] + (unsigned)__popcll(peers & lanes_below(lane)) : 0u;
        if (ok[k] && (peers & lanes_above(lane)) == 0ull) hw[d] += (unsigned)__popcll(peers);
    }
}

// Entries e0 + 64 k (k < E) of the block's run list. The run of entry e is
// the largest r < R with runpref[r] <= e, found by binary searches of fixed
// depth (top = the largest power of two <= R), the E searches side by side;
// rpos[r] is the run's first staging position. word[k] = (high digit << 16)
// | low digit within the block, idx[k] = point index, pos[k] = staging
// position, ok[k] = e < total. An entry past the total reads entry 0 (the
// caller ensures total > 0), so every load is unconditional.
template <int E>
__device__ __forceinline__ void load_chunk(const unsigned* __restrict__ swords,
                                           const unsigned* runpref, const unsigned* rpos, int R,
                                           int top, int nt, int lgT, unsigned total, unsigned e0,
                                           unsigned (&word)[E], unsigned (&idx)[E],
                                           unsigned (&pos)[E], bool (&ok)[E]) {
    unsigned e[E];
    int r[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        e[k] = e0 + k * kWave;
        ok[k] = e[k] < total;
        if (!ok[k]) e[k] = 0u;
        r[k] = 0;
    }
    for (int step = top; step > 0; step >>= 1)
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int c = r[k] + step;
            const unsigned pv = runpref[c < R ? c : R];
            r[k] = (c < R && pv <= e[k]) ? c : r[k];
        }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        pos[k] = rpos[r[k]] + (e[k] - runpref[r[k]]);
        word[k] = swords[pos[k]];
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        idx[k] = ((pos[k] >> lgT) << lgT) | (word[k] & 0xffffu);
        word[k] = (word[k] & 0xffff0000u) | (unsigned)(r[k] / nt);
    }
}

// Global count of high digit d: the sum of the 16 histogram copies.
__device__ __forceinline__ unsigned gd_of(const unsigned* __restrict__ ghist, int nb1, int d) {
    unsigned g = 0;
#pragma unroll
    for (int c = 0; c < kSHistCopies; ++c) g += ghist[c * nb1 + d];
    return g;
}

// Decoupled look-back over the preceding blocks' words of one digit,
// state[b' * nb1 + d] = flag | count, by the S lanes (a power of two, at most
// a wavefront, aligned) that serve the digit: lane s of the group reads
// predecessors hi - s W - j (j < W), so one round trip covers S W blocks,
// nearest first. The counts are added up to the nearest inclusive prefix; at
// a block that has not published, the words before it are kept and it is
// polled again. Returns the sum of the counts of blocks before b (the same
// in every lane of the group). Every lane of the wavefront calls this;
// `idle` lanes (their group has nothing to do) return 0. A poll limit that
// runs out sets *err.
__device__ __forceinline__ unsigned look_back_wide(const unsigned* state, int nb1, int b, int d,
                                                   int S, bool idle, int lane, unsigned* err) {
    constexpr int W = kSLookBackLane;
    const int gbase = lane & ~(S - 1);
    const int s = lane - gbase;
    const unsigned long long gmask = S == kWave ? ~0ull : ((1ull << S) - 1ull) << gbase;
    int hi = b - 1;
    unsigned excl = 0, polls = 0;
    bool fin = idle;
    while (__ballot(!fin) != 0ull) {
        unsigned v[W];
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int pb = hi - s * W - j;
            v[j] = (!fin && pb >= 0) ? load_relaxed32(&state[(long long)pb * nb1 + d]) : kSIncl;
        }
        // this lane's part: counts before its first unpublished or inclusive
        // word, plus that inclusive word's count
        int stop = W;
        bool incl = false;
        unsigned part = 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            if (stop != W) continue;
            const unsigned flag = v[j] & ~kSValue;
            if (flag == 0u) {
                stop = j;
            } else {
                part += v[j] & kSValue;
                if (flag == kSIncl) {
                    stop = j;
                    incl = true;
                }
            }
        }
        const unsigned long long sm = __ballot(stop != W) & gmask;
        const int first = sm ? __builtin_ctzll(sm) - gbase : S;
        const int src = gbase + (first < S ? first : 0);
        const int stop_j = __shfl(stop, src);
        const bool stop_incl = __shfl((int)incl, src) != 0;
        unsigned tot = s <= first ? part : 0u;
        for (int off = S >> 1; off > 0; off >>= 1) tot += (unsigned)__shfl_xor((int)tot, off);
        if (!fin) {
            excl += tot;
            if (first == S) {
                hi -= S * W;
            } else if (stop_incl) {
                fin = true;
            } else {
                hi -= first * W + stop_j;
                if (++polls > kSSpinLimit) {
                    *err = 1u;
                    fin = true;
                } else {
                    __builtin_amdgcn_s_sleep(1);
                }
            }
        }
    }
    return idle ? 0u : excl;
}

// Block b = (group g = b / nsplit of per_block low digits, tile range
// s = b % nsplit of tps tiles); nsplit > 1 only with per_block = 1.
// LDS (dynamic): runpref[R + 1], rpos[R] (R = per_block x the range's tiles),
// cnt2[per_block x nb1], hist[16 x nb1], running[nb1], base[nb1].
// Entries are taken in chunks of CH = 1,024 x E; entry e of a chunk
// is held by wavefront e / (64 E), register (e / 64) % E, lane e % 64. The
// first chunk (nearly always the only one) is loaded before the look-back.
// With rows_early its rows are in flight during the look-back; otherwise they
// are loaded after it: vector loads complete in order, so a look-back poll
// also waits for every row load issued before it, which on large scans (many
// rows in flight across the chip) costs more than the overlap gains.
template <int E>
__global__ __launch_bounds__(kSPassBlock) void k_sph_place(
    long long N, SphArgs a, const SphHeader* __restrict__ tab, int b0, int b1, int per_block,
    int nsplit, int tps, int rows_early, const unsigned* __restrict__ cm,
    const unsigned* __restrict__ swords,
    const float4* __restrict__ srows, unsigned* __restrict__ ghist, unsigned* __restrict__ state,
    unsigned* __restrict__ done, int* __restrict__ offsets, int* __restrict__ order,
    float4* __restrict__ sorted, int* __restrict__ n_kept) {
    constexpr int NW = kSPassWaves;
    constexpr int CH = kSPassBlock * E;
    constexpr int RPT = kSMaxRuns / kSPassBlock;
    extern __shared__ __align__(16) unsigned lds[];
    __shared__ unsigned wsum[kWsumWords];
    __shared__ unsigned gsum_sh, blk_err;
    __shared__ bool last_sh, failed_sh;
    const int tid = threadIdx.x, lane = __lane_id(), w = tid / kWave;
    const int b = blockIdx.x;  // waits only on lower blocks: see k_sph_pass
    if (tid == 0) blk_err = 0u;
    const int ntiles = a.ntiles, T = a.tile;
    const int lgT = __builtin_ctz((unsigned)T);
    const int nb1 = 1 << b1;
    const int g = b / nsplit, sp = b - g * nsplit;
    const int t0 = sp * tps;
    const int t1 = t0 + tps < ntiles ? t0 + tps : ntiles;
    const int nt = t1 > t0 ? t1 - t0 : 0;
    const int R = per_block * nt;
    unsigned* runpref = lds;
    unsigned* rpos = runpref + (R + 1);
    unsigned* cnt2 = rpos + R;
    unsigned* hist = cnt2 + per_block * nb1;
    unsigned* running = hist + NW * nb1;
    unsigned* basev = running + nb1;
    for (int j = tid; j < (per_block + NW + 1) * nb1; j += kSPassBlock) cnt2[j] = 0u;
    // lanes [S d1, S d1 + S) serve high digit d1 in the look-back (S = 1,024 /
    // nb1, at most a wavefront); the group's first lane loads the digit's
    // global count now
    const int S = nb1 >= 16 ? kSPassBlock / nb1 : kWave;
    const int d1 = tid / S;
    const bool lead = d1 < nb1 && (tid & (S - 1)) == 0;
    const unsigned gd = lead ? gd_of(ghist, nb1, d1) : 0u;

    // the block's runs, low digit by low digit, tile by tile (cm is
    // digit-major); thread t holds runs [t rpt, t rpt + rpt)
    const int rpt = (R + kSPassBlock - 1) / kSPassBlock;
    unsigned cw[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid * rpt + q;
        const int rr = r < R ? r : (R > 0 ? R - 1 : 0);
        const int j = nt > 0 ? rr / nt : 0;
        cw[q] = R > 0 ? cm[(long long)(g * per_block + j) * ntiles + t0 + (rr - j * nt)] : 0u;
    }
    // The table header is checked once the run words are on their way (their
    // addresses come from the plan alone); nothing read through them is used,
    // and nothing is written, before the check. Uniform: every thread returns.
    if (!table_ok(tab, a)) {
        if (b == 0 && tid == 0) *n_kept = SPH_STATUS_BAD_TABLE;
        return;
    }
    unsigned mine = 0;
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid * rpt + q;
        if (q < rpt && r < R) {
            const int j = r / nt;
            rpos[r] = (unsigned)((t0 + (r - j * nt)) * T) + (cw[q] & 0xffffu);
            mine += cw[q] >> 16;
        }
    }
    unsigned total;
    unsigned run = block_excl_scan<NW>(mine, wsum, &total);
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid * rpt + q;
        if (q < rpt && r < R) {
            runpref[r] = run;
            run += cw[q] >> 16;
        }
    }
    if (tid == 0) runpref[R] = total;
    __syncthreads();

    // first chunk: words and rows in registers; counts of every chunk
    int top = 1;
    while (top * 2 <= R) top *= 2;
    const unsigned ebase = (unsigned)(w * kWave * E + lane);
    unsigned word[E], rk[E], idx[E], spos[E];
    bool ok[E];
    float4 row[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        word[k] = idx[k] = spos[k] = rk[k] = 0u;
        ok[k] = false;
        row[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (total > 0) {   // uniform
        load_chunk<E>(swords, runpref, rpos, R, top, nt, lgT, total, ebase, word, idx, spos, ok);
#pragma unroll
        for (int k = 0; k < E; ++k)
            if (ok[k]) atomicAdd(&cnt2[(word[k] & 0xffffu) * nb1 + (word[k] >> 16)], 1u);
    }
    for (unsigned c0 = CH; c0 < total; c0 += CH) {   // later chunks: counts only
        unsigned wd[E], ix[E], ps[E];
        bool okk[E];
        load_chunk<E>(swords, runpref, rpos, R, top, nt, lgT, total, c0 + ebase, wd, ix, ps, okk);
#pragma unroll
        for (int k = 0; k < E; ++k)
            if (okk[k]) atomicAdd(&cnt2[(wd[k] & 0xffffu) * nb1 + (wd[k] >> 16)], 1u);
    }
    rank_high<E>(word, ok, rk, hist, w, lane, b1);
    // rows last, so no wait for a word or a count waits for them
    if (rows_early && total > 0 && sorted)   // block-uniform
#pragma unroll
        for (int k = 0; k < E; ++k) row[k] = srows[spos[k]];
    __syncthreads();

    // the digit's count in this block, publication, look-back, global start
    unsigned c = 0;
    if (d1 < nb1) {
        for (int j = 0; j < per_block; ++j) c += cnt2[j * nb1 + d1];
        if (lead) store_relaxed32(&state[(long long)b * nb1 + d1], (b == 0 ? kSIncl : kSAgg) | c);
    }
    unsigned gall;
    const unsigned g0 = block_excl_scan<NW>(gd, wsum, &gall);
    unsigned excl = 0;
    if (b > 0)   // block-uniform: the first block has no predecessor
        excl = look_back_wide(state, nb1, b, d1 < nb1 ? d1 : 0, S, d1 >= nb1, lane, &blk_err);
    if (lead) {
        // (after a failed wait the word stays an aggregate: no inclusive
        // word rests on a partial prefix; the error is reported)
        if (b > 0 && !blk_err) store_relaxed32(&state[(long long)b * nb1 + d1], kSIncl | (excl + c));
        basev[d1] = g0 + excl;
    }
    if (tid == 0) gsum_sh = gall;

    // offsets of the group's voxels, by the block holding the first tiles:
    // (high digit, low digit) -> the start of the high digit's run plus this
    // block's earlier low digits of it
    const long long nvox = a.nvox;
    __syncthreads();
    if (sp == 0 && tid < nb1) {
        unsigned at = basev[tid];
        for (int j = 0; j < per_block; ++j) {
            const long long v = ((long long)tid << b0) | ((long long)g * per_block + j);
            if (v < nvox) offsets[v] = (int)at;
            at += cnt2[j * nb1 + tid];
        }
    }

    if (!rows_early && total > 0 && sorted)
#pragma unroll
        for (int k = 0; k < E; ++k) row[k] = srows[spos[k]];
    // chunks: per-wavefront starts of each digit, then every entry stored
    // after the block's earlier entries of its digit
    for (unsigned c0 = 0; c0 < total; c0 += CH) {   // uniform: total is the block's
        if (c0 > 0) {
            __syncthreads();   // the previous chunk's hist reads and resets are done
            load_chunk<E>(swords, runpref, rpos, R, top, nt, lgT, total, c0 + ebase, word, idx, spos,
                          ok);
            rank_high<E>(word, ok, rk, hist, w, lane, b1);
            if (sorted)
#pragma unroll
                for (int k = 0; k < E; ++k) row[k] = srows[spos[k]];
            __syncthreads();
        }
        unsigned chunk_n = 0;
        if (tid < nb1)
            for (int ww = 0; ww < NW; ++ww) {
                const unsigned x = hist[ww * nb1 + tid];
                hist[ww * nb1 + tid] = chunk_n;
                chunk_n += x;
            }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (!ok[k]) continue;
            const unsigned d = word[k] >> 16;
            const unsigned pos = basev[d] + running[d] + hist[w * nb1 + d] + rk[k];
            if (pos < gsum_sh && idx[k] < N) {   // always, unless the workspace was disturbed
                order[pos] = (int)idx[k];
                if (sorted) sorted[pos] = row[k];
            } else {
                blk_err = 1u;
            }
        }
        __syncthreads();
        if (tid < nb1) {
            running[tid] += chunk_n;
            for (int ww = 0; ww < NW; ++ww) hist[ww * nb1 + tid] = 0u;
        }
    }

    // the last block: kept count, status, and the zero part back to zero.
    // The counter's low 16 bits count finished blocks, the bits above count
    // blocks that met an error, so it carries everything the last block
    // needs; every block has read the histograms before it counts itself.
    __syncthreads();
    if (tid == 0) {
        const unsigned mine_done = 1u + (blk_err ? 0x10000u : 0u);
        const unsigned prev =
            __hip_atomic_fetch_add(done, mine_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_sh = (prev & 0xffffu) + 1u == gridDim.x;
        failed_sh = (prev >> 16) != 0u || blk_err != 0u;
    }
    __syncthreads();
    if (!last_sh) return;
    for (int j = tid; j < kSHistCopies * nb1; j += kSPassBlock) ghist[j] = 0u;
    if (tid == 0) {
        const int kept = (int)gsum_sh;
        offsets[nvox] = kept;
        *n_kept = failed_sh ? VOX_STATUS_DEVICE_ERROR : kept;
        *done = 0u;
    }
}

// ------------------------------------------------------------------- host --

inline long long s_cdiv(long long a, long long b) { return (a + b - 1) / b; }
inline size_t s_align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SPlan {
    int per, tile, ntiles, sort_per, sort_tile, sort_tiles;
    long long nvox;
    SphDigits dg;
    size_t off_hist, zero_bytes, off_state, off_k0, off_v0, off_k1, off_v1, bytes;
    long long state_words;
    int final_blocks;
    // two-kernel route (fused = true): low digit b0 bits, high digit b1 bits,
    // pblocks k_sph_place blocks of pk low digits each
    bool fused;
    int b0, b1, pk, nsplit, tps, pblocks, rows_early, place_per, nt_stores;
    size_t off_cm, off_stage, off_rows, place_lds;
};

bool bins_ok(const int32_t bins[3]) {
    if (!bins) return false;
    for (int d = 0; d < 3; ++d)
        if (bins[d] < 1) return false;
    if (bins[1] > SPH_MAX_ANGLE_BINS || bins[2] > SPH_MAX_ANGLE_BINS) return false;
    return (long long)bins[0] * bins[1] * bins[2] <= SPH_MAX_VOXELS;
}

bool params_ok(const float mn[3], const float cell[3]) {
    if (!mn || !cell) return false;
    for (int d = 0; d < 3; ++d)
        if (!isfinite(mn[d]) || !isfinite(cell[d]) || !(cell[d] > 0.0f)) return false;
    return true;
}

// The two-kernel route, when the kept keys [0, nvox) fit 16 bits; false
// leaves the radix passes to make_splan. At least 2,048 entries per
// k_sph_place block, at most 256 blocks up to 2^20 points; the high digit
// takes up to 8 bits, fewer
// when two look-back round trips (1,024 x kSLookBackLane block words each)
// would not reach back over every block; a group of low digits is split over
// tile ranges when there are fewer groups than blocks.
bool plan_fused(long long N, SPlan* p) {
    int kb = 0;
    while ((1ll << kb) < p->nvox) ++kb;
    if (kb > 16) return false;
    // every block resident at once (one 1,024-thread block a CU): N / 256 a
    // block, at least 2,048
    const long long per_block_target = N / 256 > 2048 ? (N + 255) / 256 : 2048;
    int lgb = 0;
    while ((per_block_target << lgb) < N) ++lgb;
    int b1 = kb < kSMaxDigitBits ? kb : kSMaxDigitBits;
    while (b1 > 0 && ((1ll << lgb) << b1) > 2ll * kSPassBlock * kSLookBackLane &&
           kb - (b1 - 1) <= kSMaxLowBits)
        --b1;
    const int b0 = kb - b1;
    if (b0 > kSMaxLowBits) return false;
    const long long nb0 = 1ll << b0;
    long long pk = 1, nsplit = 1;
    if ((1ll << lgb) <= nb0)
        pk = nb0 >> lgb;
    else
        nsplit = (1ll << lgb) / nb0;
    if (nsplit > p->ntiles) nsplit = p->ntiles;
    while ((pk << b1) > kSPairsMax) pk >>= 1;
    long long tps = (p->ntiles + nsplit - 1) / nsplit;
    while (pk * tps > kSMaxRuns) {
        if (pk > 1) {
            pk >>= 1;
        } else {
            nsplit *= 2;
            tps = (p->ntiles + nsplit - 1) / nsplit;
        }
    }
    nsplit = (p->ntiles + tps - 1) / tps;   // no empty range
    if ((nb0 / pk) * nsplit > 0xffff) return false;   // the block counter's width
    p->fused = true;
    p->b0 = b0;
    p->b1 = b1;
    p->pk = (int)pk;
    p->nsplit = (int)nsplit;
    p->tps = (int)tps;
    p->pblocks = (int)((nb0 / pk) * nsplit);
    // rows in flight during the look-back up to 2^18 points: one MI355X
    // measured 0.7 us faster that way at 2^16 points and 3.7 us slower at 2^20
    p->rows_early = N <= (1ll << 18) ? 1 : 0;
    // streaming staging stores past 2^18 points: one MI355X measured 1.7 us
    // faster that way at 2^20 points and 1.3 us slower at 2^16
    p->nt_stores = N > (1ll << 18) ? 1 : 0;
    // entries per thread in a placing chunk: 3 up to 2,048 points per block
    // (one chunk of 3,072 holds nearly every block), 6 beyond. Measured on
    // one MI355X: 26.6 us at 2^16 points with 3 against 30.9 with 6, and at
    // 2^20 points 59.9 us with 6 against 62.9 to 67.6 with 3, 4 or 5.
    p->place_per = N <= (long long)p->pblocks * 2048 ? kSPlacePerSmall : kSPlacePer;
    const long long R = pk * tps;
    const long long nb1 = 1ll << b1;
    p->place_lds = (size_t)(4 * ((2 * R + 1) + (pk + kSPassWaves + 2) * nb1));
    p->state_words = (long long)p->pblocks * nb1;
    p->off_hist = 0;
    p->zero_bytes =   // the high-digit histogram copies, the error word, the block counter
        s_align256(sizeof(unsigned) * ((size_t)kSHistCopies * nb1 + 2));
    p->off_state = p->zero_bytes;
    p->off_cm = s_align256(p->off_state + sizeof(unsigned) * (size_t)p->state_words);
    p->off_stage = s_align256(p->off_cm + sizeof(unsigned) * ((size_t)p->ntiles << b0));
    p->off_rows = s_align256(p->off_stage + sizeof(unsigned) * (size_t)p->ntiles * p->tile);
    p->bytes = s_align256(p->off_rows + sizeof(float4) * (size_t)p->ntiles * p->tile);
    p->dg.passes = 0;
    p->dg.hist_words = (int)nb1;
    p->final_blocks = 0;
    return true;
}

int make_splan(long long N, const int32_t bins[3], const sph_options* opt, SPlan* p) {
    if (N < 0 || N > SPH_MAX_POINTS || !bins_ok(bins)) return VOX_EINVAL;
    p->nvox = (long long)bins[0] * bins[1] * bins[2];
    const int per_opt = opt ? opt->points_per_thread : 0;
    if (per_opt != 0 && per_opt != 1 && per_opt != 2 && per_opt != 4 && per_opt != 8)
        return VOX_EINVAL;
    // measured on the 64-beam scan recipe: 1 per thread at 2^16 points (25.8 us
    // against 26.4 with 2 and 29.9 with 4), 4 at 2^20 (57.7 us against 59.4
    // with 2 and 62.8 with 8)
    p->per = per_opt ? per_opt
                     : (N <= (1ll << 16) ? 1 : N <= (1ll << 17) ? 2 : N <= (1ll << 21) ? 4 : 8);
    p->tile = kSBlock * p->per;
    p->ntiles = (int)(N > 0 ? s_cdiv(N, p->tile) : 1);
    if (p->ntiles > kSMaxTiles) return VOX_EINVAL;
    const int st_opt = opt ? opt->sort_tile : 0;
    if (st_opt != 0 && st_opt != 1024 && st_opt != 2048 && st_opt != 4096) return VOX_EINVAL;
    // large tiles keep the look-back short (each round trip to another tile's
    // word costs about a microsecond)
    p->sort_tile = st_opt ? st_opt : (N <= (1ll << 17) ? 2048 : 4096);
    p->sort_per = p->sort_tile / kSPassBlock;
    p->sort_tiles = (int)(N > 0 ? s_cdiv(N, p->sort_tile) : 1);
    const int db_opt = opt ? opt->digit_bits : 0;
    if (db_opt < 0 || db_opt > kSMaxDigitBits) return VOX_EINVAL;
    p->fused = false;
    if (db_opt == 0 && plan_fused(N, p)) return VOX_OK;
    // keys run over [0, nvox] (nvox = a dropped point)
    int key_bits = 1;
    while ((1ll << key_bits) <= p->nvox) ++key_bits;
    const int db = db_opt ? db_opt : kSMaxDigitBits;
    SphDigits& dg = p->dg;
    dg.passes = (key_bits + db - 1) / db;
    const int each = (key_bits + dg.passes - 1) / dg.passes;   // spread the bits evenly
    int shift = 0, hoff = 0;
    for (int q = 0; q < dg.passes; ++q) {
        const int bits = key_bits - shift < each ? key_bits - shift : each;
        dg.shift[q] = shift;
        dg.bits[q] = bits;
        dg.hoff[q] = hoff;
        shift += bits;
        hoff += 1 << bits;
    }
    dg.hist_words = hoff;
    if (dg.passes > kSMaxPasses || hoff > kSHistWords) return VOX_EINVAL;
    for (int q = dg.passes; q < kSMaxPasses; ++q) dg.shift[q] = dg.bits[q] = dg.hoff[q] = 0;
    p->state_words = 0;
    for (int q = 0; q < dg.passes; ++q) p->state_words += (long long)p->sort_tiles << dg.bits[q];
    const size_t n4 = sizeof(unsigned) * (size_t)(N > 0 ? N : 1);
    p->off_hist = 0;
    p->zero_bytes =   // the histogram copies and the error word
        s_align256(sizeof(unsigned) * ((size_t)kSHistCopies * dg.hist_words + 1));
    p->off_state = p->zero_bytes;
    p->off_k0 = s_align256(p->off_state + sizeof(unsigned) * (size_t)p->state_words);
    p->off_v0 = s_align256(p->off_k0 + n4);
    p->off_k1 = s_align256(p->off_v0 + n4);
    p->off_v1 = s_align256(p->off_k1 + n4);
    p->bytes = dg.passes >= 3 ? s_align256(p->off_v1 + n4) : p->off_v1;
    const long long fb = s_cdiv(N > p->nvox + 1 ? N : p->nvox + 1, kSBlock);
    p->final_blocks = (int)(fb < 4096 ? fb : 4096);
    return VOX_OK;
}

SphArgs make_args(const float mn[3], const float cell[3], const int32_t bins[3], const SPlan& p) {
    SphArgs a;
    for (int d = 0; d < 3; ++d) {
        a.mn[d] = mn[d];
        a.cell[d] = cell[d];
        a.inv_cell[d] = 1.0f / cell[d];
    }
    a.nr = bins[0];
    a.nt = bins[1];
    a.np = bins[2];
    a.nvox = (int)p.nvox;
    a.ntiles = p.ntiles;
    a.tile = p.tile;
    a.sort_tiles = p.sort_tiles;
    a.sort_tile = p.sort_tile;
    return a;
}

// Boundaries [0, lo) lie at or below the axis's lowest angle, (hi, n] above
// its highest (a_k never decreases in k); lim is that half-width rounded to
// double, which is below the true one, so a < -lim exactly when a is at or
// below -half-width, and a > lim exactly when a is above half-width.
void axis_bounds(float a_min, float da, int n, double lim, float2* dirs, int* lo, int* hi) {
    *lo = 0;
    *hi = n;
    bool above = false;
    for (int k = 0; k <= n; ++k) {
        const double ak = (double)a_min + (double)k * (double)da;
        dirs[k].x = (float)cos(ak);
        dirs[k].y = (float)sin(ak);
        if (ak < -lim) *lo = k + 1;
        if (!above && ak > lim) {
            *hi = k - 1;
            above = true;
        }
    }
}

int check_call(const float* points, long long N, const float mn[3], const float cell[3],
               const int32_t bins[3], const void* table, int32_t* voxel_of, int32_t* offsets,
               int32_t* order, float* sorted, int32_t* n_kept, void* ws, long long ws_bytes,
               const sph_options* opt, SPlan* p) {
    if (!params_ok(mn, cell)) return VOX_EINVAL;
    const int rc = make_splan(N, bins, opt, p);
    if (rc != VOX_OK) return rc;
    if (!table || !offsets || !n_kept) return VOX_EINVAL;
    if (N > 0 && (!points || !voxel_of || !order)) return VOX_EINVAL;
    if (points && (reinterpret_cast<uintptr_t>(points) & 15u)) return VOX_EINVAL;
    if (sorted && (reinterpret_cast<uintptr_t>(sorted) & 15u)) return VOX_EINVAL;
    if (reinterpret_cast<uintptr_t>(table) & 3u) return VOX_EINVAL;
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) || ws_bytes < (long long)p->bytes)
        return VOX_EWORKSPACE;
    return VOX_OK;
}

int s_last_launch() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? VOX_OK : ssh_hip_fail(e);
}

template <int PER>
void launch_pass(const int* kin, const unsigned* vin, unsigned* kout, unsigned* vout, long long N,
                 const SphArgs& a, const SphHeader* tab, int shift, int bits, const unsigned* gh,
                 int hist_words, unsigned* state, unsigned* err, hipStream_t st, hipEvent_t e0,
                 hipEvent_t e1) {
    hipExtLaunchKernelGGL(k_sph_pass<PER>, dim3((unsigned)a.sort_tiles), dim3(kSPassBlock), 0, st, e0, e1,
                          0, kin, vin, kout, vout, N, a, tab, shift, bits, gh, hist_words, state,
                          err);
}

template <int PER>
void launch_key(const float4* pts, long long N, const SphArgs& a, const SphHeader* tab,
                const SphDigits& dg, int* voxel_of, unsigned* gh, unsigned* state,
                long long state_words, unsigned* err, hipStream_t st, hipEvent_t e0,
                hipEvent_t e1) {
    if (a.nt + 1 + a.np + 1 <= kSTableLds)
        hipExtLaunchKernelGGL(k_sph_key<PER, true>, dim3((unsigned)a.ntiles), dim3(kSBlock), 0, st,
                              e0, e1, 0, pts, N, a, tab, dg, voxel_of, gh, state, state_words, err);
    else
        hipExtLaunchKernelGGL(k_sph_key<PER, false>, dim3((unsigned)a.ntiles), dim3(kSBlock), 0, st,
                              e0, e1, 0, pts, N, a, tab, dg, voxel_of, gh, state, state_words, err);
}

template <int PER>
void launch_lowpart(const float4* pts, long long N, const SphArgs& a, const SphHeader* tab,
                    const SPlan& p, int* voxel_of, unsigned* cm, unsigned* swords, float4* srows,
                    unsigned* gh, unsigned* state, unsigned* err, hipStream_t st, hipEvent_t e0,
                    hipEvent_t e1) {
    const int ndirs = a.nt + 1 + a.np + 1;
    const bool lt = ndirs <= kSTableLds;
    const unsigned lds = (unsigned)(sizeof(unsigned) * kSWavesPart << p.b0) +
                         (lt ? (unsigned)sizeof(float2) * ((ndirs + 1) & ~1) : 0u) +
                         (unsigned)(sizeof(unsigned) + (srows ? sizeof(float4) : 0)) * p.tile;
    if (lt)
        hipExtLaunchKernelGGL(k_sph_lowpart<PER, true>, dim3((unsigned)a.ntiles), dim3(kSBlock), lds,
                              st, e0, e1, 0, pts, N, a, tab, p.b0, p.b1, voxel_of, cm, swords, srows,
                              gh, state, p.state_words, err, p.nt_stores);
    else
        hipExtLaunchKernelGGL(k_sph_lowpart<PER, false>, dim3((unsigned)a.ntiles), dim3(kSBlock),
                              lds, st, e0, e1, 0, pts, N, a, tab, p.b0, p.b1, voxel_of, cm, swords,
                              srows, gh, state, p.state_words, err, p.nt_stores);
}

int run_fused(const float* points, long long N, const SphArgs& a, const SPlan& p,
              const void* table, int32_t* voxel_of, int32_t* offsets, int32_t* order,
              float* sorted, int32_t* n_kept, void* ws, hipStream_t st, hipEvent_t* ev) {
    char* w = static_cast<char*>(ws);
    unsigned* gh = reinterpret_cast<unsigned*>(w + p.off_hist);
    unsigned* err = gh + kSHistCopies * (1 << p.b1);
    unsigned* done = err + 1;
    unsigned* state = reinterpret_cast<unsigned*>(w + p.off_state);
    unsigned* cm = reinterpret_cast<unsigned*>(w + p.off_cm);
    unsigned* swords = reinterpret_cast<unsigned*>(w + p.off_stage);
    float4* srows = sorted ? reinterpret_cast<float4*>(w + p.off_rows) : nullptr;
    const float4* pts = reinterpret_cast<const float4*>(points);
    const SphHeader* tab = static_cast<const SphHeader*>(table);
    hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};
    if (ev)
        for (int k = 0; k < 4; ++k) e[k] = ev[k];
    switch (p.per) {
        case 1: launch_lowpart<1>(pts, N, a, tab, p, voxel_of, cm, swords, srows, gh, state, err, st, e[0], e[1]); break;
        case 2: launch_lowpart<2>(pts, N, a, tab, p, voxel_of, cm, swords, srows, gh, state, err, st, e[0], e[1]); break;
        case 4: launch_lowpart<4>(pts, N, a, tab, p, voxel_of, cm, swords, srows, gh, state, err, st, e[0], e[1]); break;
        default: launch_lowpart<8>(pts, N, a, tab, p, voxel_of, cm, swords, srows, gh, state, err, st, e[0], e[1]); break;
    }
    int rc = s_last_launch();
    if (rc != VOX_OK) return rc;
    hipExtLaunchKernelGGL(p.place_per == kSPlacePerSmall ? k_sph_place<kSPlacePerSmall>
                                                         : k_sph_place<kSPlacePer>,
                          dim3((unsigned)p.pblocks), dim3(kSPassBlock),
                          (unsigned)p.place_lds, st, e[2], e[3], 0, N, a, tab, p.b0, p.b1, p.pk,
                          p.nsplit, p.tps, p.rows_early, cm, swords, srows, gh, state, done,
                          offsets, order,
                          reinterpret_cast<float4*>(sorted), n_kept);
    return s_last_launch();
}

int num_kernels(const SPlan& p) { return p.fused ? 2 : p.dg.passes + 2; }

// ev (optional): a start and a stop event per kernel, passes + 2 kernels.
int run_sph(const float* points, long long N, const SphArgs& a, const SPlan& p, const void* table,
            int32_t* voxel_of, int32_t* offsets, int32_t* order, float* sorted, int32_t* n_kept,
            void* ws, hipStream_t st, hipEvent_t* ev) {
    if (p.fused)
        return run_fused(points, N, a, p, table, voxel_of, offsets, order, sorted, n_kept, ws, st,
                         ev);
    char* w = static_cast<char*>(ws);
    unsigned* gh = reinterpret_cast<unsigned*>(w + p.off_hist);
    unsigned* err = gh + kSHistCopies * p.dg.hist_words;
    unsigned* state = reinterpret_cast<unsigned*>(w + p.off_state);
    unsigned* kbuf[2] = {reinterpret_cast<unsigned*>(w + p.off_k0),
                         reinterpret_cast<unsigned*>(w + p.off_k1)};
    unsigned* vbuf[2] = {reinterpret_cast<unsigned*>(w + p.off_v0),
                         reinterpret_cast<unsigned*>(w + p.off_v1)};
    const float4* pts = reinterpret_cast<const float4*>(points);
    const SphHeader* tab = static_cast<const SphHeader*>(table);
    auto evs = [&](int k) { return ev ? ev[2 * k] : nullptr; };
    auto eve = [&](int k) { return ev ? ev[2 * k + 1] : nullptr; };
    switch (p.per) {
        case 1: launch_key<1>(pts, N, a, tab, p.dg, voxel_of, gh, state, p.state_words, err, st, evs(0), eve(0)); break;
        case 2: launch_key<2>(pts, N, a, tab, p.dg, voxel_of, gh, state, p.state_words, err, st, evs(0), eve(0)); break;
        case 4: launch_key<4>(pts, N, a, tab, p.dg, voxel_of, gh, state, p.state_words, err, st, evs(0), eve(0)); break;
        default: launch_key<8>(pts, N, a, tab, p.dg, voxel_of, gh, state, p.state_words, err, st, evs(0), eve(0)); break;
    }
    int rc = s_last_launch();
    long long soff = 0;
    for (int q = 0; rc == VOX_OK && q < p.dg.passes; ++q) {
        const int* kin = q == 0 ? voxel_of : reinterpret_cast<const int*>(kbuf[(q - 1) & 1]);
        const unsigned* vin = q == 0 ? nullptr : vbuf[(q - 1) & 1];
        unsigned* kout = kbuf[q & 1];
        unsigned* vout = q == p.dg.passes - 1 ? reinterpret_cast<unsigned*>(order) : vbuf[q & 1];
        const unsigned* ghq = gh + p.dg.hoff[q];
        unsigned* sq = state + soff;
        soff += (long long)p.sort_tiles << p.dg.bits[q];
        switch (p.sort_per) {
            case 1: launch_pass<1>(kin, vin, kout, vout, N, a, tab, p.dg.shift[q], p.dg.bits[q], ghq, p.dg.hist_words, sq, err, st, evs(1 + q), eve(1 + q)); break;
            case 2: launch_pass<2>(kin, vin, kout, vout, N, a, tab, p.dg.shift[q], p.dg.bits[q], ghq, p.dg.hist_words, sq, err, st, evs(1 + q), eve(1 + q)); break;
            default: launch_pass<4>(kin, vin, kout, vout, N, a, tab, p.dg.shift[q], p.dg.bits[q], ghq, p.dg.hist_words, sq, err, st, evs(1 + q), eve(1 + q)); break;
        }
        rc = s_last_launch();
    }
    if (rc != VOX_OK) return rc;
    const int last = 1 + p.dg.passes;
    hipExtLaunchKernelGGL(k_sph_final, dim3((unsigned)p.final_blocks), dim3(kSBlock), 0, st,
                          evs(last), eve(last), 0, kbuf[(p.dg.passes - 1) & 1], order, pts,
                          reinterpret_cast<float4*>(sorted), offsets, n_kept, N, a, tab, gh,
                          p.dg.hist_words, err);
    return s_last_launch();
}

}  // namespace

extern "C" {

int64_t sph_table_bytes(const int32_t bins[3]) {
    if (!bins_ok(bins)) return VOX_EINVAL;
    return (int64_t)sizeof(SphHeader) + (int64_t)sizeof(float2) * ((int64_t)bins[1] + 1 + bins[2] + 1);
}

int sph_make_table(const float sph_min[3], const float sph_cell[3], const int32_t bins[3],
                   void* table, int64_t table_bytes) {
    if (!params_ok(sph_min, sph_cell) || !bins_ok(bins) || !table) return VOX_EINVAL;
    const int64_t need = sph_table_bytes(bins);
    if (table_bytes < need) return VOX_EINVAL;
    SphHeader h;
    memset(&h, 0, sizeof h);
    h.magic = kSMagic;
    h.nr = bins[0];
    h.nt = bins[1];
    h.np = bins[2];
    for (int d = 0; d < 3; ++d) {
        h.mn[d] = sph_min[d];
        h.cell[d] = sph_cell[d];
    }
    h.bytes = (unsigned)need;
    float2* tb = reinterpret_cast<float2*>(static_cast<char*>(table) + sizeof(SphHeader));
    float2* pb = tb + (bins[1] + 1);
    axis_bounds(sph_min[1], sph_cell[1], bins[1], kSHalfPi, tb, &h.t_lo, &h.t_hi);
    axis_bounds(sph_min[2], sph_cell[2], bins[2], kSPi, pb, &h.p_lo, &h.p_hi);
    memcpy(table, &h, sizeof h);
    return VOX_OK;
}

int64_t sph_workspace_bytes(int64_t n_points, const int32_t bins[3], const sph_options* options) {
    SPlan p;
    const int rc = make_splan(n_points, bins, options, &p);
    return rc == VOX_OK ? (int64_t)p.bytes : rc;
}

int64_t sph_workspace_zero_bytes(int64_t n_points, const int32_t bins[3],
                                 const sph_options* options) {
    SPlan p;
    const int rc = make_splan(n_points, bins, options, &p);
    return rc == VOX_OK ? (int64_t)p.zero_bytes : rc;
}

int32_t sph_num_kernels(int64_t n_points, const int32_t bins[3], const sph_options* options) {
    SPlan p;
    const int rc = make_splan(n_points, bins, options, &p);
    return rc == VOX_OK ? num_kernels(p) : rc;
}

int sph_reorder(const float* points, int64_t n_points, const float sph_min[3],
                const float sph_cell[3], const int32_t bins[3], const void* table,
                int32_t* voxel_of, int32_t* offsets, int32_t* order, float* sorted,
                int32_t* n_kept, void* workspace, int64_t workspace_bytes,
                const sph_options* options, hipStream_t stream) {
    SPlan p;
    const int rc = check_call(points, n_points, sph_min, sph_cell, bins, table, voxel_of, offsets,
                              order, sorted, n_kept, workspace, workspace_bytes, options, &p);
    if (rc != VOX_OK) return rc;
    const SphArgs a = make_args(sph_min, sph_cell, bins, p);
    return run_sph(points, n_points, a, p, table, voxel_of, offsets, order, sorted, n_kept,
                   workspace, stream, nullptr);
}

int sph_profile_stages(const float* points, int64_t n_points, const float sph_min[3],
                       const float sph_cell[3], const int32_t bins[3], const void* table,
                       int32_t* voxel_of, int32_t* offsets, int32_t* order, float* sorted,
                       int32_t* n_kept, void* workspace, int64_t workspace_bytes,
                       const sph_options* options, hipStream_t stream, int32_t iters,
                       float* stage_ms, float* total_ms) {
    if (iters < 1 || !stage_ms || !total_ms) return VOX_EINVAL;
    SPlan p;
    int rc = check_call(points, n_points, sph_min, sph_cell, bins, table, voxel_of, offsets,
                        order, sorted, n_kept, workspace, workspace_bytes, options, &p);
    if (rc != VOX_OK) return rc;
    const SphArgs a = make_args(sph_min, sph_cell, bins, p);
    const int nk = num_kernels(p);
    const int nev = 2 * nk;
    hipEvent_t* ev = new hipEvent_t[(size_t)iters * nev];
    int created = 0;
    for (; created < iters * nev; ++created) {
        const hipError_t e = hipEventCreate(&ev[created]);
        if (e != hipSuccess) {
            rc = ssh_hip_fail(e);
            break;
        }
    }
    for (int it = 0; rc == VOX_OK && it < iters; ++it)
        rc = run_sph(points, n_points, a, p, table, voxel_of, offsets, order, sorted, n_kept,
                     workspace, stream, ev + (size_t)it * nev);
    if (rc == VOX_OK) {
        const hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess) rc = ssh_hip_fail(e);
    }
    if (rc == VOX_OK) {
        double acc[kSMaxPasses + 2] = {0};
        double tot = 0;
        for (int it = 0; it < iters && rc == VOX_OK; ++it) {
            hipEvent_t* e = ev + (size_t)it * nev;
            for (int k = 0; k < nk; ++k) {
                float ms = 0;
                const hipError_t he = hipEventElapsedTime(&ms, e[2 * k], e[2 * k + 1]);
                if (he != hipSuccess) {
                    rc = ssh_hip_fail(he);
                    break;
                }
                acc[k] += ms;
            }
            float ms = 0;
            if (hipEventElapsedTime(&ms, e[0], e[nev - 1]) == hipSuccess) tot += ms;
        }
        for (int k = 0; k < nk; ++k) stage_ms[k] = (float)(acc[k] / iters);
        *total_ms = (float)(tot / iters);
    }
    for (int k = 0; k < created; ++k) (void)hipEventDestroy(ev[k]);
    delete[] ev;
    return rc;
}

}  // extern "C"
