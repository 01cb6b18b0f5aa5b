// Pillar / voxel binning for MI355X (gfx950): HIP kernels and the C ABI.
//
// The operation is the one of the "Voxelize" page
// (ethan-howes.github.io/projects/voxelize); the contract (deterministic
// order, cap, truncation) is stated in include/voxelize.h. The page's own
// kernel ("Claiming a pillar and packing points", "Compaction") writes each
// pillar at its hash slot in arrival order and compacts the table with a
// copy_if; this design makes the result a pure function of the input. The
// default route (4, first-index bins) runs three kernels:
//
//   claim   points [0, P), P = min(N, 2 max_voxels, S/4): bin each point and
//           lower its cell's entry to the lowest index seen, with one
//           non-returning atomicMax in a map indexed by cell (grids of at
//           most 2 S cells) or, for larger grids, a CAS claim plus an
//           atomicMax in a linear-probe table of 64-bit words (key and
//           lowest index), with a plain byte store into a filter indexed by
//           a hash of the cell. The first max_voxels cells in first-occurrence
//           order are all among these P points, or the call says it cannot
//           decide (VOX_STATUS_NEEDS_CHUNKED).
//   part    every point: bin, look up its cell's lowest prefix index i0 (no
//           entry: its pillar is past the cap; on the table, a zero filter
//           byte settles that without a probe), and partition the tile's
//           points by bin i0 mod nbins, keeping index order inside each bin's
//           run; prefix tiles also count their first occurrences (i == i0)
//           and rank them inside the tile.
//   bins    one block per bin: every block sums the prefix tiles' counts
//           itself, so pillar id(i0) = (first occurrences before i0's tile) +
//           (i0's rank in it); ids below max_voxels are kept. It walks the
//           bin's runs tile after tile, so each pillar's points arrive in
//           index order: a point's rank is the number of earlier arrivals of
//           its pillar, and ranks below max_points become rows (bit copies,
//           16-byte loads) with zero padding, coordinates and counts. Then
//           every workspace word the call dirtied is returned to zero.
//
// Routes 2 and 3 (the chunked path, and on request) put a rank kernel with
// a decoupled look-back between the claim and the partition and bin by
// pillar id; route 1 (max_points > 64) fills per-pillar buckets with one
// atomic per point and orders them in a pack kernel.
//
// gfx950 notes that shape the code. Blocks are dealt round-robin to the 8
// XCDs, each with its own L2. Device-scope read-modify-write atomics are
// executed beyond the L2 at a fixed rate whatever the footprint, so each
// stage issues at most one returning atomic per point, and no counter is hit
// by every block. An agent-scope acquire or release (and __threadfence) costs
// an L2 invalidate or write-back on this part, so no kernel uses one: the
// look-back publishes its value inside the atomic word with relaxed loads
// and stores, and everything else crosses kernel boundaries.
//
// No fast-math: binning must be IEEE fp32 (correctly rounded divide, no FMA
// contraction, denormals kept) to agree bit for bit with any other fp32
// implementation of "Binning a point".

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "wave_ops.h"
#include "spherical.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "voxelize.h"

namespace {

constexpr int kBlock = 256;                 // 4 wavefronts of 64 lanes
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kRankTileMin = kBlock;         // points per look-back tile: 256, 512 or 1024
constexpr int kRankTilesAim = 128;           // the smallest tile leaving at most this many
constexpr unsigned kSpinLimit = 1u << 22;   // look-back poll bound (never reached in practice)
constexpr int kPackMaxBlocks = 4096;
constexpr int kSortLanes = 64;              // pillars with K <= 64 use the bucket + bitonic path

// One table slot is a single 64-bit word, 0 = empty:
//   bits 63..31  cell key + 1 (so grids hold at most 2^33 - 2 cells)
//   bit  30      kept flag, set by rank once the cell is among the kept pillars
//   bits 29..0   ~(lowest point index) while inserting, the pillar id once kept
// A cell is claimed with one CAS; later points of the cell lower its index
// with one 64-bit atomicMax (the key bits are equal and the flag is clear, so
// the maximum is taken on ~index). Point indices are < 2^30.
constexpr int kKeyShift = 31;
constexpr unsigned long long kKeptFlag = 1ull << 30;
constexpr unsigned long long kIdxMask = (1ull << 30) - 1ull;
constexpr unsigned long long kMaxCells = (1ull << 33) - 2ull;
constexpr long long kMaxPoints = (1ll << 30) - 1;

__host__ __device__ __forceinline__ unsigned long long slot_key1(unsigned long long w) {
    return w >> kKeyShift;
}
__host__ __device__ __forceinline__ unsigned long long slot_word(unsigned long long key1,
                                                                 unsigned i) {
    return (key1 << kKeyShift) | ((unsigned long long)(~i) & kIdxMask);
}

// First 256 bytes of the workspace. status and distinct are result words
// assigned by every call; the other words are zero between calls.
struct alignas(256) Header {
    unsigned int claims;       // cells inserted (chunked path only); cleared by rank
    unsigned int rank_ticket;  // look-back tile tickets; cleared by select
    int status;                // V, or a VOX_STATUS_* code; written by the last rank tile
    int distinct;              // cells in the table (first occurrences in [0, P))
    unsigned int error;        // nonzero: an internal bound was exceeded (sticky)
    unsigned int heal;         // blocks of the last kernel that cleared their share after an error
    unsigned int pad[58];
};
static_assert(sizeof(Header) == 256, "header is 256 bytes");

struct Grid {
    float x_min, y_min, z_min, z_max;
    float vx, vy, vz;
    int gx, gy, gz;
};

// The kept-cell map: pillar id + 1 per grid cell, 0 = not kept. Entries are
// 16-bit when every id + 1 fits (max_voxels <= 65,534), halving the footprint
// that random lookups cover; p is null when there is no map.
struct KMap {
    void* p;
    int narrow;
    __device__ __forceinline__ unsigned get(long long key) const {
        return narrow ? (unsigned)static_cast<const unsigned short*>(p)[key]
                      : static_cast<const unsigned*>(p)[key];
    }
    __device__ __forceinline__ void put(long long key, unsigned v) const {
        if (narrow) static_cast<unsigned short*>(p)[key] = (unsigned short)v;
        else static_cast<unsigned*>(p)[key] = v;
    }
};

// ---------------------------------------------------------------- binning --

// "Binning a point": NaN/Inf check on x, y, z; z-slab z_min <= z < z_max;
// cell = floorf((v - v_min) / cell) tested in float against [0, g) before any
// conversion. Returns the flattened key (cz * gy + cy) * gx + cx, or -1.
__device__ __forceinline__ long long bin_key(float4 p, const Grid& g) {
    // bitwise & on ints: every test is evaluated, no branches
    int ok = (int)isfinite(p.x) & (int)isfinite(p.y) & (int)isfinite(p.z);
    ok &= (int)(p.z >= g.z_min) & (int)(p.z < g.z_max);
    const float fx = floorf((p.x - g.x_min) / g.vx);
    const float fy = floorf((p.y - g.y_min) / g.vy);
    ok &= (int)(fx >= 0.0f) & (int)(fx < (float)g.gx) & (int)(fy >= 0.0f) & (int)(fy < (float)g.gy);
    float fz = 0.0f;
    if (g.gz > 1) {
        fz = floorf((p.z - g.z_min) / g.vz);
        ok &= (int)(fz >= 0.0f) & (int)(fz < (float)g.gz);
    }
    if (!ok) return -1;
    // each index is a whole number below 2^24 here, so 32-bit conversions are
    // exact, and the key is below 2^33 (the host bounds gx gy gz)
    const unsigned ix = (unsigned)(int)fx, iy = (unsigned)(int)fy, iz = (unsigned)(int)fz;
    const unsigned long long row = (unsigned long long)iz * (unsigned)g.gy + iy;
    return (long long)(row * (unsigned)g.gx + ix);
}

// ------------------------------------------------------------------ table --

__device__ __forceinline__ unsigned long long mix64(unsigned long long k) {
    // 64-bit finaliser (xor-shift / multiply), spreads neighbouring cells
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdull;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ull;
    k ^= k >> 33;
    return k;
}

// hash 0: multiplicative (Fibonacci) hashing of the key folded to 32 bits,
//         then a multiply-high range reduction (a few instructions; grid keys
//         of neighbouring cells land far apart);
// hash 1: key mod S;
// hash 2: a 64-bit mixer, then the same reduction.
__device__ __forceinline__ unsigned home_slot(long long key, unsigned S, int hash) {
    if (hash == 1) return (unsigned)((unsigned long long)key % S);
    if (hash == 2)
        return (unsigned)__umul64hi(mix64((unsigned long long)key), (unsigned long long)S);
    const unsigned h = ((unsigned)key ^ (unsigned)((unsigned long long)key >> 32)) * 0x9E3779B1u;
    return __umulhi(h, S);
}

// First-index route on the table: a byte filter of 2^(32 - shift) entries,
// one byte per hash of a prefix cell, set (to 1) by the claim. A lookup past
// the prefix whose byte is 0 has no prefix point in its cell and skips the
// table; the others probe it. Plain byte stores of the same value need no
// atomics, and the bins kernel clears each first occurrence's byte.
__device__ __forceinline__ unsigned filt_index(long long key, int shift) {
    const unsigned h = ((unsigned)key ^ (unsigned)((unsigned long long)key >> 32)) * 0x85EBCA77u;
    return h >> shift;
}

// Lookups read the aligned slot pair holding the home slot first (16 bytes);
// when that does not settle it, they probe a cache line at a time: the 16
// slots (128 bytes) of the line come in with eight independent 16-byte loads,
// so a probe sequence costs one memory round trip per line, not per slot. (Inserts probe slot by slot with CAS: a line snapshot sends
// every lane that hashes into the line to the same empty slot.) S is a
// multiple of 16.
constexpr unsigned kLineSlots = 16;

__device__ __forceinline__ void load_line(const unsigned long long* __restrict__ table,
                                          unsigned line_base, unsigned long long w[kLineSlots]) {
    const uint4* q = reinterpret_cast<const uint4*>(table + line_base);
#pragma unroll
    for (int k = 0; k < (int)kLineSlots / 2; ++k) {
        const uint4 v = q[k];
        w[2 * k] = ((unsigned long long)v.y << 32) | v.x;
        w[2 * k + 1] = ((unsigned long long)v.w << 32) | v.z;
    }
}

// The aligned pair holding the home slot h, as one 16-byte load. At the
// insert load (at most 1/4) it nearly always settles a lookup.
__device__ __forceinline__ uint4 load_pair(const unsigned long long* __restrict__ table,
                                           unsigned h) {
    return *reinterpret_cast<const uint4*>(table + (h & ~1u));
}

// True when the pair settles the lookup of k1 (= key + 1): *out is then the
// word holding the key, or 0 when an empty slot ends the probe first.
__device__ __forceinline__ bool pair_settles(uint4 q, unsigned h, unsigned long long k1,
                                             unsigned long long* out) {
    const unsigned long long w0 = ((unsigned long long)q.y << 32) | q.x;
    const unsigned long long w1 = ((unsigned long long)q.w << 32) | q.z;
    if (!(h & 1u)) {
        if (slot_key1(w0) == k1) { *out = w0; return true; }
        if (w0 == 0ull) { *out = 0ull; return true; }
    }
    if (slot_key1(w1) == k1) { *out = w1; return true; }
    if (w1 == 0ull) { *out = 0ull; return true; }
    return false;
}

// Lookup only, probing line by line from the home slot h. The table is not
// modified while lookups run, so plain loads see final words.
__device__ __forceinline__ unsigned long long find_word_lines(
    const unsigned long long* __restrict__ table, unsigned S, unsigned h, unsigned long long k1,
    unsigned* err) {
    unsigned base = h & ~(kLineSlots - 1u);
    unsigned off = h - base;
    // The first line examines slots [off, 16); after wrapping all the way
    // round, the home line is read again whole, so its [0, off) part is seen.
    for (unsigned seen = 0; seen < S;) {
        unsigned long long w[kLineSlots];
        load_line(table, base, w);
#pragma unroll
        for (unsigned k = 0; k < kLineSlots; ++k) {
            if (k < off) continue;
            if (slot_key1(w[k]) == k1) return w[k];
            if (w[k] == 0ull) return 0ull;
        }
        seen += kLineSlots - off;
        off = 0;
        base = (base + kLineSlots == S) ? 0u : base + kLineSlots;
    }
    atomicOr(err, 1u);
    return 0ull;
}

// Lookup only: the word of the slot holding the key, or 0.
__device__ __forceinline__ unsigned long long find_word(const unsigned long long* __restrict__ table,
                                                        unsigned S, int hash, long long key,
                                                        unsigned* err) {
    const unsigned long long k1 = (unsigned long long)key + 1ull;
    const unsigned h = home_slot(key, S, hash);
    unsigned long long wd;
    if (pair_settles(load_pair(table, h), h, k1, &wd)) return wd;
    return find_word_lines(table, S, h, k1, err);
}

__device__ __forceinline__ void report_error(Header* hdr, int* num_voxels, unsigned bit) {
    atomicOr(&hdr->error, bit);
    num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
}

// The error word as this block sees it when it starts: read by one thread
// and shared through LDS, so that every thread of the block takes the same
// branch (another block may set the word meanwhile). Contains a barrier.
// A plain load: earlier kernels' writes are visible at this kernel's start,
// and a block that misses a word set meanwhile by another block of this
// kernel is a case the heal already allows for; a relaxed agent-scope load
// would go past the L2 on every block, and the whole block waits for it.
__device__ __forceinline__ unsigned block_error(const Header* hdr) {
    __shared__ unsigned err_sh;
    if (threadIdx.x == 0) err_sh = hdr->error;
    __syncthreads();
    return err_sh;
}

// A call whose last kernel starts with the error word set returns the whole
// zero part of its workspace to zero (each block clears a share, so the
// call's outputs are void, which its status already says), and the last
// block to get here resets the error word: after a device error the next
// call finds the workspace ready, with no help from the caller. The final
// kernels write only zeros into the zero part, so nothing undoes the clear.
// A block that saw a clear word (set later by another block of this kernel)
// does not count, so the word then stays set and the next call heals.
__device__ __forceinline__ void heal_workspace(Header* hdr, long long zero_words, unsigned err) {
    if (!err) return;
    unsigned* w = reinterpret_cast<unsigned*>(hdr);
    const long long nthreads = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)(sizeof(Header) / 4) + (long long)blockIdx.x * blockDim.x +
                       threadIdx.x;
         i < zero_words; i += nthreads)
        w[i] = 0u;
    if (threadIdx.x == 0 && atomicAdd(&hdr->heal, 1u) == gridDim.x - 1u) {
        hdr->claims = 0u;
        hdr->rank_ticket = 0u;
        hdr->heal = 0u;
        hdr->error = 0u;
    }
}

// ----------------------------------------------------------------- insert --

// Lanes of the wavefront whose 64-bit value equals this lane's (among lanes
// with `valid`), over the low nbits bits: match_mask on each half.
__device__ __forceinline__ unsigned long long match_mask64(unsigned long long v, bool valid,
                                                           int nbits) {
    const unsigned long long lo = match_mask((unsigned)v, valid, nbits < 32 ? nbits : 32);
    if (nbits <= 32) return lo;
    return lo & match_mask((unsigned)(v >> 32), valid, nbits - 32);
}

// merge = 1: lanes of a wavefront that fall in the same cell are merged
// before the atomics ("one atomic per distinct cell per wavefront"): the
// lowest such lane (the lowest index, lanes follow the input order) claims
// or lowers the slot for all of them and the others take its slot. kbits
// is the number of significant key bits (the match costs one ballot each).
__global__ __launch_bounds__(kBlock) void k_insert(const float4* __restrict__ pts,
                                                   long long begin, long long end, Grid g,
                                                   unsigned long long* __restrict__ table,
                                                   unsigned S, int hash,
                                                   int* __restrict__ slot_of,
                                                   Header* __restrict__ hdr, int count_claims,
                                                   int merge, int kbits,
                                                   unsigned char* __restrict__ filt, int fshift) {
    const long long i = begin + (long long)blockIdx.x * kBlock + threadIdx.x;
    const int lane = __lane_id();
    bool claimed = false;
    const long long key = i < end ? bin_key(pts[i], g) : -1;
    bool lead = key >= 0;
    int leader = lane;
    if (merge) {  // uniform branch: every lane of the wavefront takes part
        const unsigned long long m = match_mask64((unsigned long long)key, key >= 0, kbits);
        if (key >= 0) leader = __builtin_ctzll(m);
        lead = key >= 0 && leader == lane;
    }
    int out = -1;
    if (i < end) {
        if (lead) {
            const unsigned long long k1 = (unsigned long long)key + 1ull;
            const unsigned long long mine = slot_word(k1, (unsigned)i);
            unsigned s = home_slot(key, S, hash);
            unsigned probe = 0;
            // CAS first: the returned word says whether the slot was empty
            // (now ours), holds this cell, or holds another cell (probe on).
            // Every step reads fresh state, so lanes that collide spread out.
            for (;;) {
                const unsigned long long cur = atomicCAS(&table[s], 0ull, mine);
                if (cur == 0ull) {
                    claimed = true;
                    out = (int)s;
                    break;
                }
                if (slot_key1(cur) == k1) {
                    if (cur < mine) atomicMax(&table[s], mine);  // lower index wins
                    out = (int)s;
                    break;
                }
                s = (s + 1u == S) ? 0u : s + 1u;
                if (++probe >= S) {
                    atomicOr(&hdr->error, 1u);
                    break;
                }
            }
        }
    }
    if (merge) {
        // the merged lanes take their leader's slot (every lane shuffles)
        const int ls = __shfl(out, leader);
        if (key >= 0) out = ls;
    }
    if (filt && key >= 0) filt[filt_index(key, fshift)] = 1u;
    if (i < end) slot_of[i] = out;
    if (count_claims) {
        // only the chunked path reads the number of cells; one atomic per wave
        const unsigned long long b = __ballot(claimed);
        if (__lane_id() == 0 && b != 0ull) atomicAdd(&hdr->claims, (unsigned)__popcll(b));
    }
}

// Direct cell map (grids small enough to index by cell): first[key] holds
// ~(the lowest prefix index in the cell), 0 while no prefix point fell in it.
// One non-returning 32-bit atomicMax per valid prefix point, no probing:
// the larger ~i is the lower index, so the last value is the lowest index.
// merge as for k_insert (kbits <= 32 here).
__global__ __launch_bounds__(kBlock) void k_claim(const float4* __restrict__ pts, long long P,
                                                  Grid g, unsigned* __restrict__ first, int merge,
                                                  int kbits) {
    const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
    const long long key = i < P ? bin_key(pts[i], g) : -1;
    bool issue = key >= 0;
    if (merge) {  // uniform branch
        const unsigned long long m = match_mask((unsigned)key, key >= 0, kbits);
        issue = issue && (m & lanes_below(__lane_id())) == 0ull;
    }
    if (issue) atomicMax(&first[key], ~(unsigned)i);
}

// ------------------------------------------------------------------- rank --

constexpr unsigned long long kFlagAgg = 1ull << 62;
constexpr unsigned long long kFlagIncl = 2ull << 62;
constexpr unsigned long long kValueMask = (1ull << 62) - 1ull;

// Exclusive prefix of this tile from its predecessors' published words, read
// 64 tiles per poll by the whole wavefront (lane l looks at tile - 1 - l).
// Every published word carries its own value, so relaxed accesses suffice.
// All 64 lanes must call this together.
__device__ unsigned long long look_back(unsigned long long* tile_state, long long tile,
                                        unsigned* err, bool* failed) {
    const int lane = __lane_id();
    unsigned long long excl = 0;
    long long hi = tile - 1;
    unsigned polls = 0;
    while (true) {
        const long long j = hi - lane;
        const unsigned long long v = j >= 0 ? load_relaxed(&tile_state[j]) : kFlagIncl;
        const unsigned long long flag = v & ~kValueMask;
        const unsigned long long incl = __ballot(flag == kFlagIncl);
        const unsigned long long waiting = __ballot(flag == 0ull);
        const int stop = incl ? __builtin_ctzll(incl) : kWave - 1;   // nearest inclusive
        const unsigned long long need = (stop == kWave - 1) ? ~0ull : ((2ull << stop) - 1ull);
        if (waiting & need) {
            if (++polls > kSpinLimit) {
                if (lane == 0) atomicOr(err, 2u);
                *failed = true;
                return 0;
            }
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += wave_sum64(lane <= stop ? (v & kValueMask) : 0ull);
        if (incl) return excl;
        hi -= kWave;
    }
}

template <int ITERS>
__global__ __launch_bounds__(kBlock) void k_rank(long long P, long long N, int M,
                                                 unsigned long long* __restrict__ table,
                                                 unsigned long long* __restrict__ compact,
                                                 unsigned C, int hash,
                                                 int* __restrict__ kept_cslot,
                                                 const int* __restrict__ slot_of,
                                                 unsigned long long* __restrict__ tile_state,
                                                 long long ntiles, int* __restrict__ occ_slot,
                                                 long long* __restrict__ kept_key,
                                                 KMap kmap,
                                                 Header* __restrict__ hdr,
                                                 int* __restrict__ num_voxels) {
    __shared__ unsigned tile_sh;
    __shared__ unsigned wave_cnt[ITERS][kWavesPerBlock];
    __shared__ unsigned long long excl_sh;
    __shared__ int failed_sh;

    const int t = threadIdx.x;
    const int w = t / kWave;
    const int lane = __lane_id();
    if (t == 0) {
        tile_sh = atomicAdd(&hdr->rank_ticket, 1u);  // tiles in dispatch order
        failed_sh = 0;
        if (blockIdx.x == 0) hdr->claims = 0u;       // read by the host between inserts only
    }
    __syncthreads();
    const long long tile = tile_sh;
    const long long base = tile * (kBlock * ITERS);

    bool is_first[ITERS];
    int slot[ITERS];
    unsigned long long key1[ITERS];
    unsigned before[ITERS];  // first occurrences before this lane in its wave
    // every slot load, then every word load, unconditionally (clamped
    // indices): two round trips for the ITERS points, not two per point
    int sl[ITERS];
    unsigned long long wd[ITERS];
#pragma unroll
    for (int k = 0; k < ITERS; ++k) {
        const long long i = base + (long long)k * kBlock + t;
        sl[k] = slot_of[i < P ? i : (P > 0 ? P - 1 : 0)];
    }
#pragma unroll
    for (int k = 0; k < ITERS; ++k) wd[k] = table[sl[k] >= 0 ? sl[k] : 0];
#pragma unroll
    for (int k = 0; k < ITERS; ++k) {
        const long long i = base + (long long)k * kBlock + t;
        is_first[k] = false;
        slot[k] = -1;
        key1[k] = 0;
        if (i < P && sl[k] >= 0) {
            slot[k] = sl[k];
            key1[k] = slot_key1(wd[k]);
            // a kept word was tagged by the tile of its own first point,
            // so a flagged word never marks a first occurrence here
            is_first[k] = (wd[k] & (kKeptFlag | kIdxMask)) ==
                          ((unsigned long long)(~(unsigned)i) & kIdxMask);
        }
        const unsigned long long b = __ballot(is_first[k]);
        before[k] = (unsigned)__popcll(b & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[k][w] = (unsigned)__popcll(b);
    }
    __syncthreads();

    // Tile-local exclusive offset of this lane's points (index order is
    // k-major, then wave, then lane).
    unsigned local[ITERS];
    unsigned run = 0;
#pragma unroll
    for (int k = 0; k < ITERS; ++k) {
        unsigned off = run;
        for (int ww = 0; ww < kWavesPerBlock; ++ww) {
            if (ww < w) off += wave_cnt[k][ww];
            run += wave_cnt[k][ww];
        }
        local[k] = off + before[k];
    }
    const unsigned aggregate = run;

    if (w == 0) {
        unsigned long long excl = 0;
        bool failed = false;
        if (tile == 0) {
            if (lane == 0) store_relaxed(&tile_state[0], kFlagIncl | (unsigned long long)aggregate);
        } else {
            if (lane == 0) store_relaxed(&tile_state[tile], kFlagAgg | (unsigned long long)aggregate);
            excl = look_back(tile_state, tile, &hdr->error, &failed);
            if (lane == 0 && !failed)
                store_relaxed(&tile_state[tile], kFlagIncl | (excl + aggregate));
        }
        if (lane == 0) {
            excl_sh = excl;
            failed_sh = failed ? 1 : 0;
            if (tile == ntiles - 1) {
                // the last tile knows the number of distinct cells in [0, P)
                const long long distinct = (long long)excl + aggregate;
                int status = (int)(distinct < M ? distinct : M);
                if (N > P && distinct < M) status = VOX_STATUS_NEEDS_CHUNKED;
                if (failed || __hip_atomic_load(&hdr->error, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) != 0u)
                    status = VOX_STATUS_DEVICE_ERROR;
                hdr->distinct = (int)distinct;
                hdr->status = status;
                num_voxels[0] = status;
            }
        }
    }
    __syncthreads();
    if (failed_sh) {
        if (t == 0) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
        return;
    }
    const unsigned long long excl = excl_sh;

#pragma unroll
    for (int k = 0; k < ITERS; ++k) {
        if (!is_first[k]) continue;
        const long long r = (long long)excl + local[k];
        if (r >= P) {  // cannot happen: there are at most P first occurrences
            report_error(hdr, num_voxels, 2u);
            continue;
        }
        occ_slot[r] = slot[k];
        if (r < M) {
            table[slot[k]] = (key1[k] << kKeyShift) | kKeptFlag | (unsigned long long)r;
            kept_key[r] = (long long)(key1[k] - 1ull);
            if (kmap.p) kmap.put((long long)(key1[k] - 1ull), (unsigned)r + 1u);  // the kept-cell map
            if (C > 0) {
                // the kept cells also go into a small table that lookups past
                // the prefix probe instead of the big one (it stays in L2)
                const unsigned long long wd = (key1[k] << kKeyShift) | (unsigned long long)r;
                unsigned cs = home_slot((long long)(key1[k] - 1ull), C, hash);
                unsigned probe = 0;
                while (atomicCAS(&compact[cs], 0ull, wd) != 0ull) {
                    cs = (cs + 1u == C) ? 0u : cs + 1u;
                    if (++probe >= C) {
                        report_error(hdr, num_voxels, 32u);
                        cs = 0xffffffffu;
                        break;
                    }
                }
                kept_cslot[r] = (int)cs;
            }
        }
    }
}

// ----------------------------------------------------------------- select --

// Insert encoded index v (= ~i, larger = lower index) into row[0..K) which
// holds the K largest encoded values seen, in descending order (0 = empty).
// Values at a position only grow, so a stale read is never larger than the
// current value: skipping positions whose read value exceeds v, and dropping
// v when the last position already exceeds it, are both exact.
__device__ __forceinline__ void cascade(unsigned* __restrict__ row, int K, unsigned v) {
    if (row[K - 1] > v) return;
    int j = 0;
    while (j < K && row[j] > v) ++j;
    for (; j < K; ++j) {
        const unsigned old = atomicMax(&row[j], v);
        if (old == 0u) return;   // took an empty position
        if (old < v) v = old;    // displaced a higher index: carry it on
    }
}

__global__ __launch_bounds__(kBlock) void k_select(const float4* __restrict__ pts, long long N,
                                                   long long P, Grid g,
                                                   const unsigned long long* __restrict__ table,
                                                   unsigned S,
                                                   const unsigned long long* __restrict__ compact,
                                                   unsigned C, int hash,
                                                   int* __restrict__ slot_of,
                                                   unsigned* __restrict__ cnt,
                                                   unsigned* __restrict__ bucket, int cap,
                                                   unsigned* __restrict__ ovf, int K,
                                                   Header* __restrict__ hdr,
                                                   int* __restrict__ num_voxels,
                                                   int* __restrict__ point_pillar) {
    const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr->rank_ticket = 0u;  // rank is done with it
        if (hdr->error != 0u) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
    }
    if (i >= N) return;
    const int status = hdr->status;
    int s = -1;
    if (i < P) {
        s = slot_of[i];
        slot_of[i] = 0;  // last reader: return the word to zero for the next call
    }
    if (status <= 0) {  // nothing kept, cap undecided, or an error
        if (status == 0 && point_pillar) point_pillar[i] = -1;
        return;
    }
    unsigned long long wd = 0ull;
    if (i < P) {
        if (s >= 0) wd = table[s];
    } else {
        const long long key = bin_key(pts[i], g);
        if (key >= 0) {
            if (C > 0) {
                // the compact table holds only kept cells: found means kept
                wd = find_word(compact, C, hash, key, &hdr->error);
                if (wd != 0ull) wd |= kKeptFlag;
            } else {
                wd = find_word(table, S, hash, key, &hdr->error);
            }
        }
    }
    if (!(wd & kKeptFlag)) {  // no cell, or not among the kept pillars
        if (point_pillar) point_pillar[i] = -1;
        return;
    }
    const unsigned pid = (unsigned)(wd & kIdxMask);
    if (pid >= (unsigned)status) {  // cannot happen on a clean workspace
        report_error(hdr, num_voxels, 4u);
        return;
    }
    if (point_pillar) point_pillar[i] = (int)pid;  // the inverse map, when asked for
    if (cap > 0) {
        const unsigned a = atomicAdd(&cnt[pid], 1u);  // one returning atomic per point
        if (a < (unsigned)cap) {
            bucket[(size_t)pid * cap + a] = (unsigned)i + 1u;  // 0 = empty slot
            return;
        }
    }
    cascade(ovf + (size_t)pid * K, K, ~(unsigned)i);
}

// ------------------------------------------------------------------- pack --

// Ascending bitonic sort of one value per lane across the 64-lane wavefront.
__device__ __forceinline__ unsigned sort64(unsigned v, int lane) {
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const unsigned o = (unsigned)__shfl_xor((int)v, j);
            const bool keep_min = ((lane & j) == 0) == ((lane & k) == 0);
            v = keep_min ? (v < o ? v : o) : (v > o ? v : o);
        }
    }
    return v;
}

// a and b ascending across the wavefront: returns the 64 smallest of both,
// ascending (elementwise min against the reversed b is bitonic; then merge).
__device__ __forceinline__ unsigned merge64(unsigned a, unsigned b, int lane) {
    const unsigned rb = (unsigned)__shfl((int)b, kWave - 1 - lane);
    unsigned v = a < rb ? a : rb;
#pragma unroll
    for (int j = kWave >> 1; j > 0; j >>= 1) {
        const unsigned o = (unsigned)__shfl_xor((int)v, j);
        v = ((lane & j) == 0) ? (v < o ? v : o) : (v > o ? v : o);
    }
    return v;
}

__device__ __forceinline__ void write_coords(int* __restrict__ coords, long long p, long long key,
                                             int gx, int gy) {
    const long long plane = (long long)gx * gy;
    coords[3 * p + 0] = (int)(key / plane);
    coords[3 * p + 1] = (int)((key % plane) / gx);
    coords[3 * p + 2] = (int)(key % gx);
}

// One kept pillar with the whole wavefront (K <= 64): bucket of any size,
// overflow row, bitonic ordering. Used when a pillar has more candidates than
// its lane segment holds.
__device__ void pack_pillar_wave(long long p, const float4* __restrict__ pts, long long N,
                                 unsigned* __restrict__ cnt, unsigned* __restrict__ bucket,
                                 int cap, unsigned* __restrict__ ovf, int K,
                                 float4* __restrict__ voxels, int* __restrict__ num_points,
                                 int* __restrict__ num_voxels, Header* __restrict__ hdr,
                                 int lane) {
    unsigned* bk = bucket + (size_t)p * cap;
    const unsigned total = cnt[p];
    const unsigned b = total < (unsigned)cap ? total : (unsigned)cap;
    const unsigned count = total < (unsigned)K ? total : (unsigned)K;
    unsigned best = 0xffffffffu;  // lane j: j-th lowest index so far
    for (unsigned c0 = 0; c0 < b; c0 += kWave) {
        const unsigned c = c0 + lane;
        unsigned v = 0xffffffffu;
        if (c < b) {
            v = bk[c] - 1u;  // entries hold index + 1
            bk[c] = 0u;
        }
        v = sort64(v, lane);
        best = c0 == 0 ? v : merge64(best, v, lane);
    }
    if (total > (unsigned)cap) {
        // arrivals past the bucket: their K lowest, already ascending
        unsigned o = 0xffffffffu;
        if (lane < K) {
            const unsigned e = ovf[(size_t)p * K + lane];
            if (e != 0u) {
                o = ~e;
                ovf[(size_t)p * K + lane] = 0u;
            }
        }
        best = merge64(best, o, lane);
    }
    if (lane < K) {
        float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
        if ((unsigned)lane < count) {
            if (best < N) row = pts[best];
            else report_error(hdr, num_voxels, 8u);
        }
        voxels[p * K + lane] = row;
    }
    if (lane == 0) {
        num_points[p] = (int)count;
        cnt[p] = 0u;
    }
}

// Return kept pillar r's compact-table slot and its record to zero.
__device__ __forceinline__ void clear_compact(unsigned long long* __restrict__ compact, unsigned C,
                                              int* __restrict__ kept_cslot, long long r,
                                              Header* __restrict__ hdr, int* __restrict__ num_voxels) {
    const int cs = kept_cslot[r];
    kept_cslot[r] = 0;
    if (cs >= 0 && (unsigned)cs < C) compact[cs] = 0ull;
    else report_error(hdr, num_voxels, 16u);
}

// Clears every table slot the call claimed (through the list rank wrote),
// the list itself, the kept keys of ids past V that no pillar pass consumed,
// and the look-back tiles: grid-stride over the calling kernel's threads.
__device__ __forceinline__ void release_workspace(long long gtid, long long nthreads,
                                                  long long distinct, long long V, int M,
                                                  int* __restrict__ occ_slot,
                                                  unsigned long long* __restrict__ table,
                                                  unsigned S, long long* __restrict__ kept_key,
                                                  unsigned long long* __restrict__ compact,
                                                  unsigned C, int* __restrict__ kept_cslot,
                                                  unsigned long long* __restrict__ tile_state,
                                                  long long ntiles, KMap kmap,
                                                  Header* __restrict__ hdr,
                                                  int* __restrict__ num_voxels) {
    const long long kept_written = distinct < M ? distinct : M;
    for (long long r = gtid; r < distinct; r += nthreads) {
        const int s = occ_slot[r];
        occ_slot[r] = 0;
        if (s >= 0 && (unsigned)s < S) {
            table[s] = 0ull;
        } else {
            report_error(hdr, num_voxels, 16u);
        }
        if (r >= V && r < kept_written) {
            if (kmap.p) kmap.put(kept_key[r], 0u);
            kept_key[r] = 0;
            if (C > 0) clear_compact(compact, C, kept_cslot, r, hdr, num_voxels);
        }
    }
    for (long long r = gtid; r < ntiles; r += nthreads) tile_state[r] = 0ull;
}

__global__ __launch_bounds__(kBlock) void k_pack(const float4* __restrict__ pts, long long N,
                                                 unsigned* __restrict__ cnt,
                                                 unsigned* __restrict__ bucket, int cap,
                                                 unsigned* __restrict__ ovf, int K, int M,
                                                 int seg, long long* __restrict__ kept_key,
                                                 unsigned long long* __restrict__ compact,
                                                 unsigned C, int* __restrict__ kept_cslot,
                                                 int gx, int gy, float4* __restrict__ voxels,
                                                 int* __restrict__ coords,
                                                 int* __restrict__ num_points,
                                                 int* __restrict__ num_voxels,
                                                 int* __restrict__ occ_slot,
                                                 unsigned long long* __restrict__ table, unsigned S,
                                                 unsigned long long* __restrict__ tile_state,
                                                 long long ntiles, Header* __restrict__ hdr,
                                                 long long zero_words) {
    const unsigned err = block_error(hdr);
    heal_workspace(hdr, zero_words, err);
    const int status = hdr->status;
    const long long distinct = hdr->distinct;
    const long long V = status > 0 ? status : 0;
    const int lane = __lane_id();
    const long long nthreads = (long long)gridDim.x * kBlock;
    const long long gtid = (long long)blockIdx.x * kBlock + threadIdx.x;
    const long long nwaves = nthreads / kWave;
    const long long gwave = gtid / kWave;
    if (gtid == 0 && err != 0u) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;

    // 1) pillars. Nothing else touches a pillar's counter, bucket or overflow
    //    row, so they are read and cleared here.
    if (cap > 0) {
        // K <= 64: a wavefront serves W = 64 / seg pillars at once, seg lanes
        // each (seg = next power of two >= max(K, 8)). Bucket entries hold
        // index + 1 (0 = empty), so a segment reads its first seg entries
        // together with the counter instead of after it.
        const int W = kWave / seg;
        const int sidx = lane / seg;          // this lane's pillar within the pass
        const int l = lane - sidx * seg;      // lane within the segment
        const unsigned fit = (unsigned)(cap < seg ? cap : seg);
        for (long long g0 = gwave * W; g0 < V; g0 += nwaves * W) {
            const long long p = g0 + sidx;
            const bool live = p < V;
            unsigned raw = 0u, total = 0u;
            if (live) {
                if ((unsigned)l < fit) raw = bucket[(size_t)p * cap + l];
                total = cnt[p];
            }
            if (__ballot(live && total > fit) == 0ull) {
                // every pillar of the pass has at most `fit` candidates and
                // no overflow: a lane's rank is the number of smaller
                // candidates in its segment (indices are distinct)
                const unsigned b = total;
                unsigned bmax = 0;
                for (int q = 0; q < W; ++q) {
                    const unsigned bq = (unsigned)__builtin_amdgcn_readlane((int)b, q * seg);
                    bmax = bq > bmax ? bq : bmax;
                }
                const unsigned v = raw - 1u;  // empty lanes become 0xffffffff
                if (raw != 0u) bucket[(size_t)p * cap + l] = 0u;
                unsigned rank = 0;
                for (unsigned t = 0; t < bmax; ++t) {
                    unsigned u = 0xffffffffu;
                    for (int q = 0; q < W; ++q) {
                        const unsigned x =
                            (unsigned)__builtin_amdgcn_readlane((int)v, q * seg + (int)t);
                        if (q == sidx) u = x;
                    }
                    rank += (t < b && u < v) ? 1u : 0u;
                }
                if (live) {
                    const unsigned count = total < (unsigned)K ? total : (unsigned)K;
                    if ((unsigned)l < b && rank < (unsigned)K) {
                        float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
                        if (v < N) row = pts[v];
                        else report_error(hdr, num_voxels, 8u);
                        voxels[p * K + rank] = row;
                    }
                    if ((unsigned)l >= count && l < K)
                        voxels[p * K + l] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (l == 0) {
                        num_points[p] = (int)count;
                        cnt[p] = 0u;
                    }
                }
            } else {
                // a pillar of this pass is heavy: take them one at a time
                for (int q = 0; q < W; ++q) {
                    const long long pq = g0 + q;
                    if (pq < V)
                        pack_pillar_wave(pq, pts, N, cnt, bucket, cap, ovf, K, voxels,
                                         num_points, num_voxels, hdr, lane);
                }
            }
            if (live && l == 0) {
                write_coords(coords, p, kept_key[p], gx, gy);
                kept_key[p] = 0;
                if (C > 0) clear_compact(compact, C, kept_cslot, p, hdr, num_voxels);
            }
        }
    } else {
        // K > 64: the overflow row is the whole selection, in order
        for (long long p = gwave; p < V; p += nwaves) {
            int count = 0;
            for (int j0 = 0; j0 < K; j0 += kWave) {
                const int j = j0 + lane;
                unsigned v = 0u;
                if (j < K) v = ovf[(size_t)p * K + j];
                count += __popcll(__ballot(v != 0u));
                if (j < K) {
                    float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (v != 0u) {
                        const unsigned src = ~v;
                        if (src < N) row = pts[src];
                        else report_error(hdr, num_voxels, 8u);
                        ovf[(size_t)p * K + j] = 0u;
                    }
                    voxels[p * K + j] = row;
                }
            }
            if (lane == 0) {
                num_points[p] = count;
                write_coords(coords, p, kept_key[p], gx, gy);
                kept_key[p] = 0;
                if (C > 0) clear_compact(compact, C, kept_cslot, p, hdr, num_voxels);
            }
        }
    }

    // 2) return the rest of the workspace to zero
    release_workspace(gtid, nthreads, distinct, V, M, occ_slot, table, S, kept_key, compact, C,
                      kept_cslot, tile_state, ntiles, KMap{nullptr, 0}, hdr, num_voxels);
}

// ------------------------------------------------- partitioned select/pack --
//
// For K <= 64 and up to kMaxBins * 128 pillars (kMaxBins * 64 when K > 32),
// select and pack avoid the per-point counter atomic (device atomics run at
// a fixed rate beyond the L2) and any sorting. Pillar ids are dealt to nbins bins round-robin (bin =
// id mod nbins), at most G = 2^gshift per bin: ids follow first occurrence,
// so the dense cells that come first spread over all bins.
//   k_part  one block per tile of 256-4096 points finds each point's pillar
//           (as select does) and writes the tile's kept points to its stretch
//           of a staging array, bin after bin, as one 32-bit word each (id
//           within the bin << 16 | index within the tile). Inside a bin's run
//           the words are in index order: each wavefront owns a contiguous
//           stretch of the tile, ranks its lanes among equal bins with
//           ballots and its own LDS histogram, and the per-bin scan places
//           the wavefronts' stretches one after another.
//           The start and length of every bin's run in the tile go to a
//           [bins x tiles] count table.
//   k_bins  one block per bin reads the bin's runs tile after tile, so each
//           pillar's points arrive in index order: a point's rank in its
//           pillar is the number of earlier arrivals with the same id
//           (ballots within the wavefront, a per-wavefront prefix in LDS and
//           a running count per pillar); a rank below K is a row, copied from
//           the row k_part staged next to the word (no gather from the cloud).
// Staging and the count table are scratch: every call writes each entry it
// reads, so they are left as they are (the rest of the workspace is zeroed).
// The rows are those of the bucket path bit for bit; only the route differs.

constexpr int kPartMaxPer = 16;                // points per k_part thread, at most
constexpr int kPartBatch = 4;                  // lookups in flight per thread
constexpr int kWideBlock = 2 * kBlock;         // k_part threads from 4 points per thread
constexpr long long kWideTilesMin = 192;       // 512-thread tiles below 4 points per thread from here
constexpr long long kWideTilesMax = 640;       // partition tiles of 512 threads, at most (about 512)
constexpr int kMaxBins = 2048;                 // bins per call (k_part: one LDS histogram per wavefront)
constexpr int kBinBlock = 1024;                // k_bins threads (16 wavefronts)
constexpr int kBinWaves = kBinBlock / kWave;
constexpr unsigned kNoPid = 0xffffffffu;

// CARRY: also copy each kept point's row into a scratch array next to its
// staging word, so that k_bins copies rows from there instead of gathering
// them from the cloud (pays off for large clouds).
// BLK threads and PER points per thread: wavefront w of the block takes the
// contiguous points [base + 64 PER w, base + 64 PER (w + 1)), 64 at a time.
// The hist LDS holds one 2048-bin histogram per wavefront. Lookups go
// PER_B at a time: within a batch every load is issued before any result is
// used, and only block-uniform branches guard them.
template <int PER, bool CARRY, int BLK>
__global__ __launch_bounds__(BLK) void k_part(const float4* __restrict__ pts, long long N,
                                                 long long P, Grid g,
                                                 const unsigned long long* __restrict__ table,
                                                 unsigned S,
                                                 const unsigned long long* __restrict__ compact,
                                                 unsigned C, int hash, int* __restrict__ slot_of,
                                                 KMap kmap,
                                                 int nbits, long long ptiles,
                                                 unsigned* __restrict__ cm,
                                                 unsigned* __restrict__ staging,
                                                 float4* __restrict__ stage_pt,
                                                 Header* __restrict__ hdr,
                                                 int* __restrict__ num_voxels,
                                                 int* __restrict__ point_pillar) {
    constexpr int TILE = BLK * PER;
    constexpr int WPB = BLK / kWave;      // wavefronts per block
    constexpr int BPT = kMaxBins / BLK;   // bins per thread in the tile's scan
    constexpr int PER_B = PER < kPartBatch ? PER : kPartBatch;
    __shared__ unsigned hist[WPB][kMaxBins];  // one histogram per wavefront
    __shared__ unsigned wsum[kWsumWords];
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    // Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
    // range of tiles, so that neighbouring count-table words (one row per
    // bin, one word per tile) are written through the same L2.
    const long long tile = xcd_tile(blockIdx.x, ptiles);
    const long long base = tile * TILE;
    const long long wbase = base + (long long)w * (kWave * PER);
    const bool any_prefix = base < P;                              // block-uniform
    // The first batch's point rows and slot entries do not depend on the
    // header: they are loaded before the barrier that waits for its status.
    const bool rest_range = base + TILE > P && base < N;          // block-uniform
    float4 row0[PER_B];
    int sl0[PER_B];
#pragma unroll
    for (int k = 0; k < PER_B; ++k) {
        const long long i0 = wbase + (long long)k * kWave + lane;
        row0[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (base < N && (CARRY || rest_range)) row0[k] = pts[i0 < N ? i0 : N - 1];
        sl0[k] = -1;
        if (any_prefix) sl0[k] = slot_of[i0 < P ? i0 : P - 1];
    }
    if (blockIdx.x == 0 && t == 0) {
        hdr->rank_ticket = 0u;  // rank is done with it
        if (hdr->error != 0u) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
    }
    const int status = hdr->status;
    const int nbins = 1 << nbits;
    const unsigned bmask = (unsigned)nbins - 1u;
    const int nb = status > 0 ? nbins : 0;
    // each wavefront clears its own histogram (only it writes it before the
    // barrier that follows the ranking), so no barrier is needed here
    for (int b = lane; b < nb; b += kWave) hist[w][b] = 0u;

    // lookups go to the kept-cell table when there is one (found = kept)
    const unsigned long long* __restrict__ look = C > 0 ? compact : table;
    const unsigned LS = C > 0 ? C : S;
    const bool any_rest = status > 0 && rest_range;
    unsigned pid[PER];
    float4 row[PER];  // each point's row (kept to the end when CARRY)
#pragma unroll
    for (int k0 = 0; k0 < PER; k0 += PER_B) {
        unsigned long long wd[PER_B];
        long long ii[PER_B];
#pragma unroll
        for (int k = 0; k < PER_B; ++k) {
            ii[k] = wbase + (long long)(k0 + k) * kWave + lane;
            wd[k] = 0ull;
            if (k0 == 0) {
                row[k] = row0[k];
            } else {
                row[k0 + k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (base < N && (CARRY || any_rest)) row[k0 + k] = pts[ii[k] < N ? ii[k] : N - 1];
            }
        }
        if (kmap.p && any_rest) {
            // the kept-cell map answers every point of a tile that reaches
            // past the prefix with one 2- or 4-byte load; its prefix points only
            // return their slot_of entries to zero (tiles inside the prefix
            // take the slot_of path below)
            if (any_prefix) {
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    if (ii[k] < P) slot_of[ii[k]] = 0;
            }
            if (status > 0 && base < N) {
                unsigned mv[PER_B];
#pragma unroll
                for (int k = 0; k < PER_B; ++k) {
                    const long long key = ii[k] < N ? bin_key(row[k0 + k], g) : -1;
                    mv[k] = key >= 0 ? kmap.get(key) : 0u;
                }
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    wd[k] = mv[k] ? (kKeptFlag | (unsigned long long)(mv[k] - 1u)) : 0ull;
            }
        } else if (any_prefix) {
            // prefix points: the slot insert recorded, then its word
            int sl[PER_B];
#pragma unroll
            for (int k = 0; k < PER_B; ++k)
                sl[k] = k0 == 0 ? sl0[k] : slot_of[ii[k] < P ? ii[k] : P - 1];
#pragma unroll
            for (int k = 0; k < PER_B; ++k)
                if (ii[k] < P) slot_of[ii[k]] = 0;  // last reader: back to zero
            if (status > 0) {
                unsigned long long w[PER_B];
#pragma unroll
                for (int k = 0; k < PER_B; ++k) {
                    const bool ok = ii[k] < P && sl[k] >= 0 && (unsigned)sl[k] < S;
                    w[k] = table[ok ? sl[k] : 0];
                    if (!ok) w[k] = 0ull;
                }
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    if (ii[k] < P) wd[k] = w[k];
            }
        }
        if (any_rest && !kmap.p) {
            // later points: bin, then probe the home pair, then (rarely) lines
            long long key[PER_B];
            unsigned h[PER_B];
            uint4 q[PER_B];
#pragma unroll
            for (int k = 0; k < PER_B; ++k) {
                key[k] = (ii[k] >= P && ii[k] < N) ? bin_key(row[k0 + k], g) : -1;
                h[k] = home_slot(key[k] >= 0 ? key[k] : 0, LS, hash);
                q[k] = load_pair(look, h[k]);
            }
            // Lookups the home pair does not settle go on pair by pair; all
            // of the batch's pending probes are issued together each round.
            bool pend[PER_B];
            unsigned cur[PER_B], seen[PER_B];
            unsigned long long w[PER_B];
            bool any = false;
#pragma unroll
            for (int k = 0; k < PER_B; ++k) {
                w[k] = 0ull;
                pend[k] = false;
                cur[k] = 0u;
                seen[k] = 0u;
                if (key[k] >= 0) {
                    const unsigned long long k1 = (unsigned long long)key[k] + 1ull;
                    if (!pair_settles(q[k], h[k], k1, &w[k])) {
                        pend[k] = true;
                        any = true;
                        const unsigned nx = (h[k] | 1u) + 1u;  // next aligned pair
                        cur[k] = nx == LS ? 0u : nx;
                        seen[k] = 2u - (h[k] & 1u);
                    }
                }
            }
            while (__ballot(any) != 0ull) {
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    if (pend[k]) q[k] = load_pair(look, cur[k]);
                any = false;
#pragma unroll
                for (int k = 0; k < PER_B; ++k) {
                    if (!pend[k]) continue;
                    const unsigned long long k1 = (unsigned long long)key[k] + 1ull;
                    // cur is even: the pair's slots are checked in probe order
                    if (pair_settles(q[k], cur[k], k1, &w[k])) {
                        pend[k] = false;
                        continue;
                    }
                    seen[k] += 2u;
                    if (seen[k] >= LS) {  // every slot seen: cannot happen
                        atomicOr(&hdr->error, 1u);
                        w[k] = 0ull;
                        pend[k] = false;
                        continue;
                    }
                    cur[k] = cur[k] + 2u == LS ? 0u : cur[k] + 2u;
                    any = true;
                }
            }
#pragma unroll
            for (int k = 0; k < PER_B; ++k) {
                if (key[k] >= 0) {
                    if (C > 0 && w[k] != 0ull) w[k] |= kKeptFlag;
                    wd[k] = w[k];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < PER_B; ++k) {
            const long long i = ii[k];
            unsigned p = kNoPid;
            if (wd[k] & kKeptFlag) {
                const unsigned v = (unsigned)(wd[k] & kIdxMask);
                if (v < (unsigned)status) p = v;
                else report_error(hdr, num_voxels, 4u);  // not on a clean workspace
            }
            if (point_pillar && i < N && status >= 0) point_pillar[i] = p == kNoPid ? -1 : (int)p;
            pid[k0 + k] = p;
        }
    }

    // Rank among equal bins inside this wavefront's stretch, in index order
    // (k, then lane): ballots within the step, the wavefront's own LDS
    // histogram across steps.
    unsigned pos[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const bool valid = pid[k] != kNoPid;
        const unsigned bin = valid ? pid[k] & bmask : 0u;
        const unsigned long long m = match_mask(bin, valid, nbits);
        pos[k] = 0u;
        if (valid) {
            const unsigned before = hist[w][bin];  // the whole group reads first,
            pos[k] = before + (unsigned)__popcll(m & lanes_below(lane));
            if ((m & lanes_above(lane)) == 0ull)    // then its last lane adds
                hist[w][bin] = before + (unsigned)__popcll(m);
        }
    }
    __syncthreads();

    // bin starts within the tile, then each wavefront's start within its bin;
    // each thread owns bpt consecutive bins
    // (bpt = nbins / BLK, at least 1: with fewer bins than threads each
    // thread takes one bin, so the bins spread over every wavefront)
    const int bpt = nb > BLK ? nb / BLK : 1;
    unsigned c[BPT];
    unsigned mine = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * bpt + q;
        c[q] = 0u;
        if (q < bpt && b < nb) {
#pragma unroll
            for (int ww = 0; ww < WPB; ++ww) c[q] += hist[ww][b];
        }
        mine += c[q];
    }
    unsigned total;
    unsigned run = block_excl_scan<WPB>(mine, wsum, &total);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * bpt + q;
        if (q < bpt && b < nb) {
            cm[(size_t)b * ptiles + tile] = run | (c[q] << 16);
            unsigned at = run;
#pragma unroll
            for (int ww = 0; ww < WPB; ++ww) {
                const unsigned cw = hist[ww][b];
                hist[ww][b] = at;
                at += cw;
            }
        }
        run += c[q];
    }
    __syncthreads();
    // With CARRY and a tile's rows fitting the histogram's LDS (PER <= 8),
    // the rows are placed there in staging order and written out in one
    // contiguous run; otherwise each row goes straight to its position.
    constexpr bool kRowsViaLds = CARRY && BLK * PER * sizeof(float4) <= sizeof(hist);
    // The staging words go through the histograms' LDS too: placed in
    // staging order once every position is read, then written as one
    // contiguous run per tile instead of one scattered 4-byte store each.
    static_assert(BLK * PER * sizeof(unsigned) <= sizeof(hist), "a tile's words fit the histograms");
    unsigned lat[PER];  // position within the tile's staging slice
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        lat[k] = 0u;
        if (pid[k] == kNoPid) continue;
        lat[k] = hist[w][pid[k] & bmask] + pos[k];
        if (CARRY && !kRowsViaLds) stage_pt[base + lat[k]] = row[k];  // the row, bit for bit
    }
    unsigned* tword = &hist[0][0];
    __syncthreads();   // every position is read from hist
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (pid[k] == kNoPid) continue;
        const unsigned local = (unsigned)(w * (kWave * PER) + k * kWave + lane);  // in the tile
        tword[lat[k]] = ((pid[k] >> nbits) << 16) | local;  // id within the bin, index in tile
    }
    __syncthreads();
    for (unsigned q = t; q < total; q += BLK) staging[base + q] = tword[q];
    if (kRowsViaLds) {
        float4* trow = reinterpret_cast<float4*>(&hist[0][0]);
        __syncthreads();   // every word is read from LDS
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (pid[k] != kNoPid) trow[lat[k]] = row[k];
        __syncthreads();
        for (unsigned q = t; q < total; q += BLK) stage_pt[base + q] = trow[q];
    }
}

// ------------------------------------------------ first-index route (4) --
//
// The same partition without a rank kernel. A pillar is named by i0, the
// lowest prefix index of its cell, which the claim step leaves in the cell's
// map entry (direct) or table word (hashed) and which is final once the
// claim kernel has ended. k_part_fb bins every point of a prefix cell by
// i0 mod nbins (id within the bin i0 / nbins), as k_part bins by pillar id;
// points whose cell holds no prefix point belong to no kept pillar (the cap
// is decided within the prefix) and are dropped. Its prefix tiles also count
// their first occurrences (points with i0 == i): the tile's count, and each
// first occurrence's rank inside the tile, with the cell key. A pillar's id,
// its rank in first-occurrence order, is then the count of the tiles before
// i0's tile plus i0's rank inside it: k_bins_fb scans the few tile counts
// itself (every block), keeps the ids below max_voxels and gathers rows as
// k_bins does. No kernel waits on another block.

// Lookups of a batch of keys in the table (home pair first, then pair by
// pair with every pending probe of the batch issued together each round).
// w[k] gets the cell's word, or 0 when the key is absent (or key[k] < 0).
template <int NB>
__device__ __forceinline__ void probe_batch(const unsigned long long* __restrict__ look,
                                            unsigned LS, int hash, const long long key[NB],
                                            unsigned long long w[NB], Header* __restrict__ hdr) {
    unsigned h[NB];
    uint4 q[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        h[k] = home_slot(key[k] >= 0 ? key[k] : 0, LS, hash);
        q[k] = load_pair(look, h[k]);
    }
    bool pend[NB];
    unsigned cur[NB], seen[NB];
    bool any = false;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        w[k] = 0ull;
        pend[k] = false;
        cur[k] = 0u;
        seen[k] = 0u;
        if (key[k] >= 0) {
            const unsigned long long k1 = (unsigned long long)key[k] + 1ull;
            if (!pair_settles(q[k], h[k], k1, &w[k])) {
                pend[k] = true;
                any = true;
                const unsigned nx = (h[k] | 1u) + 1u;  // next aligned pair
                cur[k] = nx == LS ? 0u : nx;
                seen[k] = 2u - (h[k] & 1u);
            }
        }
    }
    while (__ballot(any) != 0ull) {
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (pend[k]) q[k] = load_pair(look, cur[k]);
        any = false;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (!pend[k]) continue;
            const unsigned long long k1 = (unsigned long long)key[k] + 1ull;
            if (pair_settles(q[k], cur[k], k1, &w[k])) {  // cur is even
                pend[k] = false;
                continue;
            }
            seen[k] += 2u;
            if (seen[k] >= LS) {  // every slot seen: cannot happen
                atomicOr(&hdr->error, 1u);
                w[k] = 0ull;
                pend[k] = false;
                continue;
            }
            cur[k] = cur[k] + 2u == LS ? 0u : cur[k] + 2u;
            any = true;
        }
    }
}

// DIRECT: the cell's entry in the direct map `first` (grids of at most
// 2 S cells); otherwise prefix points read their word through slot_of and
// later points probe the table. Block layout, ranking by bin, the count
// table and the staging words are k_part's. CARRY (downsampling): each
// staged point's row is also copied to stage_pt next to its staging word.
template <int PER, int BLK, bool DIRECT, bool CARRY = false>
__global__ __launch_bounds__(BLK) void k_part_fb(
    const float4* __restrict__ pts, long long N, long long P, Grid g,
    const unsigned long long* __restrict__ table, unsigned S, int hash,
    const unsigned* __restrict__ first, int* __restrict__ slot_of, int nbits, long long ptiles,
    unsigned* __restrict__ cm, unsigned* __restrict__ staging,
    unsigned long long* __restrict__ fkey, unsigned* __restrict__ frank,
    unsigned* __restrict__ tile_firsts, Header* __restrict__ hdr,
    int* __restrict__ point_pillar, const unsigned char* __restrict__ filt, int fltshift,
    float4* __restrict__ stage_pt) {
    constexpr int TILE = BLK * PER;
    constexpr int WPB = BLK / kWave;
    constexpr int BPT = kMaxBins / BLK;
    constexpr int PER_B = PER < kPartBatch ? PER : kPartBatch;
    __shared__ unsigned hist[WPB][kMaxBins];
    __shared__ unsigned wsum[kWsumWords];
    __shared__ unsigned wfirst[WPB];
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    const long long tile = xcd_tile(blockIdx.x, ptiles);
    const long long base = tile * TILE;
    const long long wbase = base + (long long)w * (kWave * PER);
    const bool any_prefix = base < P;                      // block-uniform
    const bool any_rest = base + TILE > P && base < N;     // block-uniform
    const int nbins = 1 << nbits;
    const unsigned bmask = (unsigned)nbins - 1u;
    // each wavefront clears its own histogram (only it writes it before the
    // barrier that follows the ranking)
    for (int b = lane; b < nbins; b += kWave) hist[w][b] = 0u;

    unsigned i0v[PER];             // the point's pillar as its first index, or kNoPid
    bool isf[PER];                 // a first occurrence (i0 == i)
    unsigned long long k1v[PER];   // cell key + 1 (first occurrences)
    float4 rowk[CARRY ? PER : 1];  // CARRY: each point's row, kept to the staging stores
#pragma unroll
    for (int k0 = 0; k0 < PER; k0 += PER_B) {
        long long ii[PER_B];
        long long key[PER_B];
        unsigned long long wd[PER_B];  // direct: ~i0 or 0; hashed: the cell's word or 0
#pragma unroll
        for (int k = 0; k < PER_B; ++k) {
            ii[k] = wbase + (long long)(k0 + k) * kWave + lane;
            key[k] = -1;
            wd[k] = 0ull;
        }
        if (DIRECT) {
            float4 row[PER_B];
#pragma unroll
            for (int k = 0; k < PER_B; ++k) {
                row[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (base < N) row[k] = pts[ii[k] < N ? ii[k] : N - 1];
            }
            unsigned f[PER_B];
#pragma unroll
            for (int k = 0; k < PER_B; ++k) {
                key[k] = ii[k] < N ? bin_key(row[k], g) : -1;
                f[k] = key[k] >= 0 ? first[key[k]] : 0u;
            }
#pragma unroll
            for (int k = 0; k < PER_B; ++k) wd[k] = f[k];
            if (CARRY) {
#pragma unroll
                for (int k = 0; k < PER_B; ++k) rowk[k0 + k] = row[k];
            }
        } else {
            if (CARRY) {  // prefix points' rows too (the lookups below load only the rest)
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    rowk[k0 + k] = base < N ? pts[ii[k] < N ? ii[k] : N - 1]
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if (any_prefix) {
                int sl[PER_B];
                unsigned long long tw[PER_B];
#pragma unroll
                for (int k = 0; k < PER_B; ++k) sl[k] = slot_of[ii[k] < P ? ii[k] : P - 1];
#pragma unroll
                for (int k = 0; k < PER_B; ++k) {
                    const bool ok = ii[k] < P && sl[k] >= 0 && (unsigned)sl[k] < S;
                    tw[k] = table[ok ? sl[k] : 0];
                    if (!ok) tw[k] = 0ull;
                }
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    if (ii[k] < P) wd[k] = tw[k];
            }
            if (any_rest) {
                float4 row[PER_B];
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    row[k] = pts[ii[k] < N ? ii[k] : N - 1];
                long long rk[PER_B];
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    rk[k] = (ii[k] >= P && ii[k] < N) ? bin_key(row[k], g) : -1;
                if (filt) {  // uniform: cells whose filter byte is 0 skip the table
                    unsigned char fv[PER_B];
#pragma unroll
                    for (int k = 0; k < PER_B; ++k)
                        fv[k] = filt[rk[k] >= 0 ? filt_index(rk[k], fltshift) : 0u];
#pragma unroll
                    for (int k = 0; k < PER_B; ++k)
                        if (fv[k] == 0u) rk[k] = -1;
                }
                unsigned long long rw[PER_B];
                probe_batch<PER_B>(table, S, hash, rk, rw, hdr);
#pragma unroll
                for (int k = 0; k < PER_B; ++k)
                    if (ii[k] >= P) wd[k] = rw[k];
            }
        }
#pragma unroll
        for (int k = 0; k < PER_B; ++k) {
            const long long i = ii[k];
            unsigned i0 = kNoPid;
            bool f = false;
            unsigned long long k1 = 0ull;
            if (i < N && wd[k] != 0ull) {
                if (DIRECT) {
                    i0 = ~(unsigned)wd[k];
                    k1 = (unsigned long long)key[k] + 1ull;
                } else {
                    i0 = (unsigned)(~wd[k] & kIdxMask);
                    k1 = slot_key1(wd[k]);
                }
                if ((long long)i0 >= P) {  // not on a clean workspace
                    atomicOr(&hdr->error, 4u);
                    i0 = kNoPid;
                }
                f = i < P && (long long)i0 == i;
            }
            i0v[k0 + k] = i0;
            isf[k0 + k] = f;
            k1v[k0 + k] = k1;
            // last reader of a prefix point's slot; first occurrences keep
            // theirs until k_bins_fb has cleared their table slot
            if (!DIRECT && i < P && !f) slot_of[i] = 0;
            if (point_pillar && i < N && i0 == kNoPid) point_pillar[i] = -1;
        }
    }

    // first occurrences in index order within the wavefront's stretch
    unsigned fb[PER];
    unsigned wf = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const unsigned long long bb = __ballot(isf[k]);
        fb[k] = wf + (unsigned)__popcll(bb & lanes_below(lane));
        wf += (unsigned)__popcll(bb);
    }
    if (lane == 0) wfirst[w] = wf;  // read after the ranking's barrier

    // rank among equal bins inside this wavefront's stretch (as k_part)
    unsigned pos[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const bool valid = i0v[k] != kNoPid;
        const unsigned bin = valid ? i0v[k] & bmask : 0u;
        const unsigned long long m = match_mask(bin, valid, nbits);
        pos[k] = 0u;
        if (valid) {
            const unsigned before = hist[w][bin];
            pos[k] = before + (unsigned)__popcll(m & lanes_below(lane));
            if ((m & lanes_above(lane)) == 0ull) hist[w][bin] = before + (unsigned)__popcll(m);
        }
    }
    __syncthreads();

    // (bpt = nbins / BLK, at least 1: with fewer bins than threads each
    // thread takes one bin, so the bins spread over every wavefront)
    const int bpt = nbins > BLK ? nbins / BLK : 1;
    unsigned c[BPT];
    unsigned mine = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * bpt + q;
        c[q] = 0u;
        if (q < bpt && b < nbins) {
#pragma unroll
            for (int ww = 0; ww < WPB; ++ww) c[q] += hist[ww][b];
        }
        mine += c[q];
    }
    unsigned total;
    unsigned run = block_excl_scan<WPB>(mine, wsum, &total);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * bpt + q;
        if (q < bpt && b < nbins) {
            cm[(size_t)b * ptiles + tile] = run | (c[q] << 16);
            unsigned at = run;
#pragma unroll
            for (int ww = 0; ww < WPB; ++ww) {
                const unsigned cw = hist[ww][b];
                hist[ww][b] = at;
                at += cw;
            }
        }
        run += c[q];
    }
    __syncthreads();
    unsigned woff = 0, tfirst = 0;
#pragma unroll
    for (int ww = 0; ww < WPB; ++ww) {
        const unsigned x = wfirst[ww];
        if (ww < w) woff += x;
        tfirst += x;
    }
    // CARRY with a tile's rows fitting the histograms' LDS (PER <= 8 at 512
    // threads): the rows are placed there in staging order after the
    // positions are read, and written out as one contiguous run
    constexpr bool kRowsViaLds = CARRY && BLK * PER * sizeof(float4) <= sizeof(hist);
    // The staging words go through the same LDS: placed in staging order once
    // every position has been read, then written out as one contiguous run
    // (the tile's slice of at most BLK PER words fits the histograms).
    static_assert(BLK * PER * sizeof(unsigned) <= sizeof(hist), "a tile's words fit the histograms");
    unsigned lat[PER];  // each staged point's position in the tile's slice
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        lat[k] = 0u;
        if (i0v[k] == kNoPid) continue;
        const unsigned local = (unsigned)(w * (kWave * PER) + k * kWave + lane);
        const unsigned bin = i0v[k] & bmask;
        lat[k] = hist[w][bin] + pos[k];
        if (CARRY && !kRowsViaLds) stage_pt[base + lat[k]] = rowk[k];  // the row, bit for bit
        if (isf[k]) {
            const long long i = base + local;
            frank[i] = woff + fb[k];
            fkey[i] = k1v[k];
        }
    }
    if (t == 0 && any_prefix) tile_firsts[tile] = tfirst;
    unsigned* tword = &hist[0][0];
    __syncthreads();  // every position has been read from hist
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (i0v[k] == kNoPid) continue;
        const unsigned local = (unsigned)(w * (kWave * PER) + k * kWave + lane);
        tword[lat[k]] = ((i0v[k] >> nbits) << 16) | local;
    }
    __syncthreads();
    for (unsigned q = t; q < total; q += BLK) staging[base + q] = tword[q];
    if (kRowsViaLds) {
        float4* trow = reinterpret_cast<float4*>(&hist[0][0]);
        __syncthreads();  // every word has been read from LDS
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (i0v[k] != kNoPid) trow[lat[k]] = rowk[k];
        __syncthreads();
        for (unsigned q = t; q < total; q += BLK) stage_pt[base + q] = trow[q];
    }
}

// At most 64 VGPRs: two 1024-thread blocks per CU. CARRY: rows come from
// the copies k_part staged; otherwise the K lowest indices are kept in LDS
// and the rows gathered from the cloud at the end.
template <bool CARRY>
__global__ __launch_bounds__(kBinBlock) __attribute__((amdgpu_waves_per_eu(8)))
void k_bins(
    const float4* __restrict__ pts, long long N, const unsigned* __restrict__ cm,
    const unsigned* __restrict__ staging, const float4* __restrict__ stage_pt, long long ptiles,
    int ptile, int gshift, int nbits, int K,
    int M, long long* __restrict__ kept_key, unsigned long long* __restrict__ compact, unsigned C,
    int* __restrict__ kept_cslot, int gx, int gy, float4* __restrict__ voxels,
    int* __restrict__ coords, int* __restrict__ num_points, int* __restrict__ num_voxels,
    int* __restrict__ occ_slot, unsigned long long* __restrict__ table, unsigned S,
    unsigned long long* __restrict__ tile_state, long long ntiles, KMap kmap,
    Header* __restrict__ hdr, int nt_out, long long zero_words) {
    extern __shared__ unsigned lds[];
    const int G = 1 << gshift;
    unsigned* running = lds;                     // [G] arrivals so far per pillar
    unsigned* wbuf = running + G;                // [3][kBinWaves * G] per-wavefront counts
    unsigned* roff = wbuf + 3 * kBinWaves * G;   // [kBinBlock + 1] run offsets in the group
    unsigned* rsrc = roff + kBinBlock + 1;       // [kBinBlock] run start within its tile
    unsigned* wsum = rsrc + kBinBlock;           // [kWsumWords]
    unsigned* best = wsum + kWsumWords;          // [G * K] without CARRY: the K lowest, in order

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    // Blocks are dealt to the 8 XCDs round-robin; each XCD takes a contiguous
    // range of bins, whose runs lie side by side in every k_part tile, so the
    // staging lines they share come through one L2.
    const long long b = xcd_tile(blockIdx.x, gridDim.x);
    // the first group's count entries do not depend on the header: load them
    // together with it
    unsigned e = 0u;
    if ((long long)t < ptiles) e = cm[(size_t)b * ptiles + t];
    const int status = hdr->status;
    const long long V = status > 0 ? status : 0;
    const long long distinct = hdr->distinct;
    const unsigned err = block_error(hdr);
    heal_workspace(hdr, zero_words, err);
    if (b == 0 && t == 0 && err != 0u) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
    // the release touches nothing below; its memory traffic overlaps the bins.
    // It goes by block index, not by bin: clearing in bin order measured
    // slower in the next call's inserts.
    release_workspace((long long)blockIdx.x * kBinBlock + t, (long long)gridDim.x * kBinBlock,
                      distinct, V, M, occ_slot, table, S, kept_key, compact, C, kept_cslot,
                      tile_state, ntiles, kmap, hdr, num_voxels);
    if (status <= 0) return;  // nothing was staged

    // bin b holds the ids b, b + nbins, b + 2 nbins, ... below V
    const long long nbins = 1ll << nbits;
    const int Gb = b < V ? (int)((V - b + nbins - 1) >> nbits) : 0;
    // the coordinates' keys, needed only at the end, are loaded now
    const long long key_t = t < Gb ? kept_key[b + ((long long)t << nbits)] : 0;
    for (int x = t; x < G; x += kBinBlock) running[x] = 0u;
    for (int x = t; x < 3 * kBinWaves * G; x += kBinBlock) wbuf[x] = 0u;
    unsigned round = 0;
    bool has_row = false;
    float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
    long long row_at = 0;
    for (long long tg = 0; tg < ptiles; tg += kBinBlock) {
        // this group's runs: tile tg + t holds one of length e >> 16
        const long long tt = tg + t;
        if (tg > 0) {
            e = 0u;
            if (tt < ptiles) e = cm[(size_t)b * ptiles + tt];
        }
        unsigned ng;
        const unsigned ro = block_excl_scan<kBinWaves>(e >> 16, wsum, &ng);
        roff[t] = ro;
        rsrc[t] = e & 0xffffu;
        const int nruns = (int)(ptiles - tg < kBinBlock ? ptiles - tg : kBinBlock);
        __syncthreads();
        // arrivals in order, kBinBlock per round and up to four rounds read
        // ahead: arrival x of the group lies in the last run whose offset is
        // <= x
        for (unsigned x0 = 0; x0 < ng; x0 += 4u * kBinBlock) {
            unsigned v[4], src4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const unsigned x = x0 + (unsigned)(u * kBinBlock + t);
                v[u] = 0u;
                src4[u] = 0u;
                if (x < ng) {
                    int lo = 0, hi = nruns;
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (roff[mid] <= x) lo = mid;
                        else hi = mid;
                    }
                    const size_t src = (size_t)(tg + lo) * ptile + rsrc[lo] + (x - roff[lo]);
                    v[u] = staging[src];
                    // CARRY: where the row is; otherwise the tile's first index
                    src4[u] = CARRY ? (unsigned)src : (unsigned)((tg + lo) * ptile);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const unsigned xr = x0 + (unsigned)(u * kBinBlock);
                if (xr >= ng) break;  // block-uniform
                bool valid = xr + (unsigned)t < ng;
                unsigned pl = v[u] >> 16;
                if (valid && pl >= (unsigned)Gb) {  // not on a clean workspace
                    report_error(hdr, num_voxels, 4u);
                    valid = false;
                }
                if (!valid) pl = 0u;
                // counts of three rounds rotate: round r writes buffer r % 3
                // and clears (r + 1) % 3, last read two rounds ago
                unsigned* cur = wbuf + (round % 3u) * (kBinWaves * G);
                unsigned* nxt = wbuf + ((round + 1u) % 3u) * (kBinWaves * G);
                for (int y = t; y < kBinWaves * G; y += kBinBlock) nxt[y] = 0u;
                const unsigned long long m = match_mask(pl, valid, gshift);
                const unsigned rank = (unsigned)__popcll(m & lanes_below(lane));
                if (valid && (m & lanes_above(lane)) == 0ull) cur[w * G + pl] = (unsigned)__popcll(m);
                __syncthreads();
                if (t < G) {
                    // exclusive prefix over the wavefronts, on top of the
                    // arrivals of earlier rounds
                    unsigned acc = running[t];
#pragma unroll
                    for (int h0 = 0; h0 < kBinWaves; h0 += 8) {
                        unsigned cw[8];  // eight reads in flight, then eight writes
#pragma unroll
                        for (int ww = 0; ww < 8; ++ww) cw[ww] = cur[(h0 + ww) * G + t];
#pragma unroll
                        for (int ww = 0; ww < 8; ++ww) {
                            cur[(h0 + ww) * G + t] = acc;
                            acc += cw[ww];
                        }
                    }
                    running[t] = acc;
                }
                __syncthreads();
                // a rank below K is a row: load it now, store it one round
                // later (the load stays in flight across the barriers)
                if (CARRY && has_row) voxels[row_at] = row;
                has_row = false;
                if (valid) {
                    const unsigned r = cur[w * G + pl] + rank;
                    if (r < (unsigned)K) {
                        if (CARRY) {
                            row = stage_pt[src4[u]];
                            row_at = (b + ((long long)pl << nbits)) * K + r;
                            has_row = true;
                        } else {
                            best[pl * K + r] = src4[u] + (v[u] & 0xffffu);  // point index
                        }
                    }
                }
                ++round;
            }
        }
    }
    if (CARRY && has_row) voxels[row_at] = row;  // the last round's rows
    __syncthreads();
    const int rows = Gb * K;
    if (CARRY) {
        // zero padding: rows at or past each pillar's count
        for (int x = t; x < rows; x += kBinBlock) {
            const int p = x / K;
            const int r = x - p * K;
            if ((unsigned)r >= running[p])
                voxels[(b + ((long long)p << nbits)) * K + r] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        // rows gathered by index (four in flight per thread), then zero padding
        for (int x0 = 0; x0 < rows; x0 += 4 * kBinBlock) {
            float4 rw[4];
            int xx[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xx[u] = x0 + u * kBinBlock + t;
                rw[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (xx[u] < rows) {
                    const int p = xx[u] / K;
                    const int r = xx[u] - p * K;
                    if ((unsigned)r < running[p]) {
                        const unsigned vv = best[p * K + r];
                        if (vv < N) rw[u] = pts[vv];
                        else report_error(hdr, num_voxels, 8u);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (xx[u] >= rows) continue;
                const int p = xx[u] / K;
                float4* dst = &voxels[(b + ((long long)p << nbits)) * K + (xx[u] - p * K)];
                if (nt_out) {   // uniform
                    typedef float v4f __attribute__((ext_vector_type(4)));
                    v4f x;
                    x.x = rw[u].x;
                    x.y = rw[u].y;
                    x.z = rw[u].z;
                    x.w = rw[u].w;
                    __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(dst));
                } else {
                    *dst = rw[u];
                }
            }
        }
    }
    for (int p = t; p < Gb; p += kBinBlock) {
        const long long pp = b + ((long long)p << nbits);
        num_points[pp] = (int)(running[p] < (unsigned)K ? running[p] : (unsigned)K);
        const long long key = p == t ? key_t : kept_key[pp];
        write_coords(coords, pp, key, gx, gy);
        if (kmap.p) kmap.put(key, 0u);
        kept_key[pp] = 0;
        if (C > 0) clear_compact(compact, C, kept_cslot, pp, hdr, num_voxels);
    }
}

// One block per bin of the first-index route. Pillar slot j of bin b is the
// cell whose first index is i0 = b + j nbins (when i0 is a first occurrence):
// its id = (first occurrences in the tiles before i0's) + (i0's rank in its
// tile), kept when below max_voxels. The walk over the bin's runs and the
// ranking of arrivals within their pillar are k_bins' (arrivals of pillars
// that are not kept are skipped). Every block clears the claim state of its
// bin's cells; block 0 writes the status.
//
// Ordered for latency: the first loads (run words, tile counts, the block's
// slots) go out together; one scan serves both the run offsets and the tile
// prefix; the first batch of staging words is in flight while the pillar
// ids are worked out. A bin whose arrivals fit one round (the clouds of a
// frame or so) loads a row as soon as its rank is known to be below K and
// stores it after the round; a bin with more rounds keeps the K lowest
// indices in LDS and gathers the rows after the walk, all at once (a row
// per round would put a load's round trip into every round). The padding
// rows follow.
constexpr int kScanTiles = 4096;                 // prefix tiles a k_bins_fb block scans, at most
constexpr int kScanPer = kScanTiles / kBinBlock;
constexpr int kAhead = 4;                        // rounds of arrivals loaded ahead

// The first-index bins' arrivals, found without a search. The runs of a
// group that hold arrivals are listed in order (croff: offset of the run's
// first arrival in the group; csrc: tile within the group << 16 | start of
// the run in its tile's staging slice). For a window of kWin arrivals
// [x0, x0 + kWin), bit i of `bits` is set when a listed run starts at x0 + i,
// and wpre holds the exclusive prefix of the words' bit counts (wpre[kWinWords]
// the window's total). Arrival x then belongs to listed run
// base + (starts in [x0, x]) - 1, where base counts the listed runs that
// start before x0: a rank query of a few LDS reads instead of a binary
// search over the runs.
constexpr int kWin = kAhead * kBinBlock;         // arrivals per window
constexpr int kWinWords = kWin / 32;             // words of the window's start bits

// Every run listed at or after `from` that starts in the window sets its bit
// (bits must be zero). One listed run per thread.
__device__ __forceinline__ void mark_window(const unsigned* croff, int nlist, unsigned x0,
                                            unsigned* bits) {
    const int k = threadIdx.x;
    if (k < nlist) {
        const unsigned r = croff[k];
        if (r >= x0 && r - x0 < (unsigned)kWin)
            atomicOr(&bits[(r - x0) >> 5], 1u << ((r - x0) & 31u));
    }
}

// Wavefront 0: the exclusive prefix of the window's per-word start counts.
__device__ __forceinline__ void prefix_window(const unsigned* bits, unsigned* wpre) {
    static_assert(kWinWords == 2 * kWave, "two words per lane");
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const unsigned c0 = (unsigned)__popc(bits[2 * lane]);
        const unsigned c1 = (unsigned)__popc(bits[2 * lane + 1]);
        const unsigned incl = wave_incl_scan(c0 + c1, lane);
        wpre[2 * lane] = incl - c0 - c1;
        wpre[2 * lane + 1] = incl - c1;
        if (lane == kWave - 1) wpre[kWinWords] = incl;
    }
}

// Arrivals x0 + u kBinBlock + t (u < kAhead) of the current window: the
// staging word and the index of its tile's first point. The loads are
// unconditional (word 0 for lanes past the group's arrivals, whose values
// the caller ignores): a load under a branch makes the compiler wait for it
// where the branch joins, which would serialise the round trips this is meant
// to overlap.
__device__ __forceinline__ void load_arrivals_ranked(const unsigned* __restrict__ staging,
                                                     const unsigned* croff, const unsigned* csrc,
                                                     const unsigned* bits, const unsigned* wpre,
                                                     unsigned base, long long tg, int ptile,
                                                     unsigned x0, unsigned ng,
                                                     unsigned v[kAhead], unsigned idx[kAhead]) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        const unsigned i = (unsigned)(u * kBinBlock) + threadIdx.x;  // within the window
        const unsigned x = x0 + i;
        const bool ok = x < ng;
        const unsigned wd = i >> 5;
        const unsigned below = bits[wd] & (0xffffffffu >> (31u - (i & 31u)));  // bits <= i
        int k = (int)(base + wpre[wd] + (unsigned)__popc(below)) - 1;
        k = ok && k >= 0 ? k : 0;
        const unsigned cs = csrc[k];
        const long long tile = tg + (cs >> 16);
        const size_t at = ok ? (size_t)tile * ptile + (cs & 0xffffu) + (x - croff[k]) : 0;
        idx[u] = ok ? (unsigned)(tile * ptile) : 0u;
        v[u] = staging[at];
    }
}

__device__ __forceinline__ void store_row(float4* d, float4 r, int nt) {
    if (nt) {  // uniform
        typedef float v4f __attribute__((ext_vector_type(4)));
        v4f x;
        x.x = r.x;
        x.y = r.y;
        x.z = r.z;
        x.w = r.w;
        __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(d));
    } else {
        *d = r;
    }
}

// Return slot i0's claim state to zero: the direct map entry or table slot
// of its cell (fk = key + 1, 0 when i0 is not a first occurrence), its
// slot_of entry (hashed route) and its key.
__device__ __forceinline__ void release_slot(unsigned* __restrict__ first,
                                             unsigned long long cells,
                                             unsigned long long* __restrict__ fkey,
                                             unsigned long long* __restrict__ table, unsigned S,
                                             int* __restrict__ slot_of, unsigned i0,
                                             unsigned long long fk, int fs, Header* hdr,
                                             int* num_voxels, unsigned char* __restrict__ filt,
                                             int fltshift) {
    if (fk == 0ull) return;
    if (first) {
        if (fk - 1ull < cells) first[fk - 1ull] = 0u;
        else report_error(hdr, num_voxels, 16u);  // not on a clean workspace
    } else {
        if (fs >= 0 && (unsigned)fs < S) table[fs] = 0ull;
        else report_error(hdr, num_voxels, 16u);
        slot_of[i0] = 0;
        if (filt) filt[filt_index((long long)(fk - 1ull), fltshift)] = 0u;
    }
    fkey[i0] = 0ull;
}

// WPE: wavefronts per SIMD the kernel is compiled for. 8 (at most 64 VGPRs)
// lets two blocks share a CU, which plans of more bins than CUs need; with 4
// a block has the CU to itself, and the extra SGPRs keep the kernel's
// arguments out of VGPR lanes (at 8 the compiler spills several dozen and
// reloads them with v_readlane inside the walk).
template <int WPE>
__global__ __launch_bounds__(kBinBlock) __attribute__((amdgpu_waves_per_eu(WPE)))
void k_bins_fb(const float4* __restrict__ pts, long long N, long long P, int M, int K,
               const unsigned* __restrict__ cm, const unsigned* __restrict__ staging,
               long long ptiles, int ptile, int tshift, int gshift, int nbits,
               const unsigned* __restrict__ tile_firsts, int ptp,
               unsigned long long* __restrict__ fkey, const unsigned* __restrict__ frank,
               unsigned* __restrict__ first, unsigned long long cells,
               unsigned long long* __restrict__ table, unsigned S,
               int* __restrict__ slot_of, int gx, int gy, float4* __restrict__ voxels,
               int* __restrict__ coords, int* __restrict__ num_points,
               int* __restrict__ num_voxels, int* __restrict__ point_pillar,
               Header* __restrict__ hdr, int nt_out, long long zero_words,
               unsigned char* __restrict__ filt, int fltshift) {
    extern __shared__ unsigned lds[];
    const int G = 1 << gshift;
    // per-wavefront counts are 16-bit (a wavefront adds at most 64 arrivals
    // to a slot per round, and the prefixes saturate at 65535: only ranks
    // below K <= 64 matter); the region first holds the tile prefix
    const int wwords = 3 * kBinWaves * G / 2 > kScanTiles ? 3 * kBinWaves * G / 2 : kScanTiles;
    unsigned* running = lds;                     // [G] arrivals so far per pillar slot
    unsigned* wbuf = running + G;                // [wwords] the tile prefix, then the counts
    unsigned short* wcnt = reinterpret_cast<unsigned short*>(wbuf);  // [3][kBinWaves * G]
    unsigned* croff = wbuf + wwords;             // [kBinBlock] listed runs: first arrival
    unsigned* csrc = croff + kBinBlock;          // [kBinBlock] listed runs: tile << 16 | start
    unsigned* bits = csrc + kBinBlock;           // [kWinWords] run starts in the window
    unsigned* wpre = bits + kWinWords;           // [kWinWords + 2] their prefix, and total
    unsigned* wsum = wpre + kWinWords + 2;       // [kWsumWords]
    unsigned* pid_of = wsum + kWsumWords;        // [G] pillar id of each slot, kNoPid if none kept
    // [G] cell key + 1 of each slot (8-byte aligned: every count above is even)
    unsigned long long* key_of = reinterpret_cast<unsigned long long*>(pid_of + G);
    int* slot_at = reinterpret_cast<int*>(key_of + G);         // [G] table slot (hashed route)
    unsigned* first_at = reinterpret_cast<unsigned*>(slot_at + G);  // [G] the slot's first index
    unsigned* best = first_at + G;               // [G K] the K lowest, in order

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    const long long b = xcd_tile(blockIdx.x, gridDim.x);  // contiguous bins per XCD, as k_bins
    const long long nbins = 1ll << nbits;
    const int Gb = b < P ? (int)((P - b + nbins - 1) >> nbits) : 0;  // slots with i0 < P
    // independent loads first: the first group's run words, the tile
    // counts, and the slot this thread owns (t < Gb)
    unsigned e = 0u;
    if ((long long)t < ptiles) e = cm[(size_t)b * ptiles + t];
    unsigned tc[kScanPer];
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
        const int q = t * kScanPer + u;
        tc[u] = q < ptp ? tile_firsts[q] : 0u;
    }
    // slot indices are below P <= 2^30: 32-bit arithmetic
    const unsigned i0 = (unsigned)b + ((unsigned)t << nbits);
    unsigned long long fk = 0ull;
    unsigned fr = 0u;
    int fs = -1;
    if (t < Gb) {
        fk = fkey[i0];
        fr = frank[i0];
        if (!first) fs = slot_of[i0];
    }
    if (t < kWinWords) bits[t] = 0u;
    // the error word, one value for the whole block (the status below must
    // be block-uniform)
    const unsigned err = block_error(hdr);
    heal_workspace(hdr, zero_words, err);
    // the slot's key, rank, table slot and first index wait in LDS (pid_of
    // holds the rank until the id is known), so that no register carries
    // them past the scan
    if (t < G) {
        pid_of[t] = fr;
        key_of[t] = fk;
        slot_at[t] = fs;
        first_at[t] = i0;
    }

    // one scan for three prefixes: the first group's run offsets, its
    // listed runs, and the tile counts of first occurrences
    unsigned s = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) s += tc[u];
    const unsigned sv[3] = {e >> 16, (e >> 16) != 0u ? 1u : 0u, s};
    unsigned sx[3], st[3];
    block_excl_scan_n<kBinWaves, 3>(sv, wsum, sx, st);
    unsigned ng = st[0];
    int nlist = (int)st[1];
    const unsigned distinct_u = st[2];
    unsigned ex = sx[2];
    if ((e >> 16) != 0u) {
        croff[sx[1]] = sx[0];
        csrc[sx[1]] = ((unsigned)t << 16) | (e & 0xffffu);
        if (sx[0] < (unsigned)kWin) atomicOr(&bits[sx[0] >> 5], 1u << (sx[0] & 31u));
    }
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
        const int q = t * kScanPer + u;
        if (q < ptp) wbuf[q] = ex;
        ex += tc[u];
    }
    // This bin's cells are done with their claim state: back to zero. The
    // stores go out after the last use of a loaded value and before the
    // staging loads: nothing waits on memory until the walk, whose first
    // wait they long precede, and the compiler's wait counts for the
    // staging loads are not blurred by stores issued after them.
    if (t < Gb)
        release_slot(first, cells, fkey, table, S, slot_of, i0, fk, fs, hdr, num_voxels, filt,
                     fltshift);
    __syncthreads();
    const long long distinct = distinct_u;
    const long long V = distinct < M ? distinct : M;
    int status = (int)V;
    if (N > P && distinct < M) status = VOX_STATUS_NEEDS_CHUNKED;
    if (err != 0u) status = VOX_STATUS_DEVICE_ERROR;
    prefix_window(bits, wpre);
    if (blockIdx.x == 0 && t == 0) {
        hdr->status = status;
        hdr->distinct = (int)distinct;
        num_voxels[0] = status;
    }
    if (t < G) {
        unsigned mypid = kNoPid;
        if (key_of[t] != 0ull) {
            const unsigned pid = wbuf[first_at[t] >> tshift] + pid_of[t];
            if ((long long)pid >= distinct) report_error(hdr, num_voxels, 4u);  // not on a clean workspace
            else if (status > 0 && (long long)pid < V) mypid = pid;
        }
        pid_of[t] = mypid;
    }
    __syncthreads();  // the window prefix, pid_of written; the tile prefix in wbuf read
    // the first batch of staging words goes out now (unused when status <= 0)
    unsigned v[kAhead], idx[kAhead];
    unsigned base = 0u;  // listed runs that start before the window
    load_arrivals_ranked(staging, croff, csrc, bits, wpre, base, 0, ptile, 0u,
                         status > 0 ? ng : 0u, v, idx);
    if (status <= 0) return;  // block-uniform: nothing kept, or no decision
    const bool one_round = ptiles <= kBinBlock && ng <= (unsigned)kBinBlock;  // block-uniform

    // each wavefront clears its own counts in the three rotating buffers (in
    // a round only wavefront w writes entries w G to w G + G - 1), so no
    // barrier is needed before the first round writes them
    for (int x = t; x < G; x += kBinBlock) running[x] = 0u;
    for (int x = lane; x < G; x += kWave) {
#pragma unroll
        for (int r3 = 0; r3 < 3; ++r3) wcnt[r3 * (kBinWaves * G) + w * G + x] = 0u;
    }
    unsigned round = 0;
    bool has_row = false;     // one-round bins: this thread's row is kept
    float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
    long long row_at = 0;
    for (long long tg = 0; tg < ptiles; tg += kBinBlock) {
        if (tg > 0) {
            // the next group of runs (the previous group's rounds have passed
            // their barriers, so nobody reads the listed runs any more)
            const long long tt = tg + t;
            e = 0u;
            if (tt < ptiles) e = cm[(size_t)b * ptiles + tt];
            const unsigned gv[2] = {e >> 16, (e >> 16) != 0u ? 1u : 0u};
            unsigned gx2[2], gt[2];
            block_excl_scan_n<kBinWaves, 2>(gv, wsum, gx2, gt);
            ng = gt[0];
            nlist = (int)gt[1];
            if ((e >> 16) != 0u) {
                croff[gx2[1]] = gx2[0];
                csrc[gx2[1]] = ((unsigned)t << 16) | (e & 0xffffu);
            }
            base = 0u;
            __syncthreads();
        }
        for (unsigned x0 = 0; x0 < ng; x0 += (unsigned)kWin) {
            if (tg > 0 || x0 > 0) {
                // the window's start bits (the previous window's readers have
                // passed the rounds' barriers)
                if (x0 > 0) base += wpre[kWinWords];
                __syncthreads();  // everyone has the old total
                if (t < kWinWords) bits[t] = 0u;
                __syncthreads();
                mark_window(croff, nlist, x0, bits);
                __syncthreads();
                prefix_window(bits, wpre);
                __syncthreads();
                load_arrivals_ranked(staging, croff, csrc, bits, wpre, base, tg, ptile, x0, ng, v,
                                     idx);
            }
#pragma unroll
            for (int u = 0; u < kAhead; ++u) {
                const unsigned xr = x0 + (unsigned)(u * kBinBlock);
                if (xr >= ng) break;  // block-uniform
                bool valid = xr + (unsigned)t < ng;
                unsigned pl = v[u] >> 16;
                const unsigned src = idx[u] + (v[u] & 0xffffu);  // the point's index
                unsigned pid = kNoPid;
                if (valid && pl >= (unsigned)Gb) {  // not on a clean workspace
                    report_error(hdr, num_voxels, 4u);
                    valid = false;
                }
                if (valid) {
                    pid = pid_of[pl];
                    if (point_pillar) point_pillar[src] = pid == kNoPid ? -1 : (int)pid;
                    valid = pid != kNoPid;  // points of pillars past the cap are dropped
                }
                if (!valid) pl = 0u;
                // a one-round bin loads every kept arrival's row now, before
                // its rank is known, so that the load overlaps the ranking;
                // rows ranked past max_points are not stored
                if (one_round) row = pts[valid && src < N ? src : 0u];
                // counts of three rounds rotate: round r writes buffer r % 3
                // and clears (r + 1) % 3, last read two rounds ago
                unsigned short* cur = wcnt + (round % 3u) * (kBinWaves * G);
                unsigned* nxt = wbuf + ((round + 1u) % 3u) * (kBinWaves * G / 2);
                for (int y = t; y < kBinWaves * G / 2; y += kBinBlock) nxt[y] = 0u;
                const unsigned long long m = match_mask(pl, valid, gshift);
                const unsigned rank = (unsigned)__popcll(m & lanes_below(lane));
                if (valid && (m & lanes_above(lane)) == 0ull)
                    cur[w * G + pl] = (unsigned short)__popcll(m);
                __syncthreads();
                if (t < G) {
                    unsigned acc = running[t];
#pragma unroll
                    for (int h0 = 0; h0 < kBinWaves; h0 += 8) {
                        unsigned cw[8];
#pragma unroll
                        for (int ww = 0; ww < 8; ++ww) cw[ww] = cur[(h0 + ww) * G + t];
#pragma unroll
                        for (int ww = 0; ww < 8; ++ww) {
                            cur[(h0 + ww) * G + t] = (unsigned short)(acc < 0xffffu ? acc : 0xffffu);
                            acc += cw[ww];
                        }
                    }
                    running[t] = acc;
                }
                __syncthreads();
                if (valid) {
                    const unsigned r = (unsigned)cur[w * G + pl] + rank;
                    if (r < (unsigned)K) {
                        if (!one_round) {
                            best[pl * K + r] = src;
                        } else if (src < N) {
                            row_at = (long long)pid * K + r;  // the row is stored after the round
                            has_row = true;
                        } else {
                            report_error(hdr, num_voxels, 8u);
                        }
                    }
                }
                ++round;
            }
        }
    }
    if (has_row) store_row(&voxels[row_at], row, nt_out);  // the one round's row
    __syncthreads();  // the final counts (and the selection)
    const int rows = Gb * K;
    if (one_round) {
        // zero padding: rows at or past each kept pillar's count
        for (int x = t; x < rows; x += kBinBlock) {
            const int p = x / K;
            const int r = x - p * K;
            const unsigned pid = pid_of[p];
            if (pid != kNoPid && (unsigned)r >= running[p])
                store_row(&voxels[(long long)pid * K + r], make_float4(0.f, 0.f, 0.f, 0.f),
                          nt_out);
        }
    } else {
        // rows gathered by index (four in flight per thread), then padding
        for (int x0 = 0; x0 < rows; x0 += 4 * kBinBlock) {
            float4 rw[4];
            long long dst[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int x = x0 + u * kBinBlock + t;
                rw[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                dst[u] = -1;
                if (x < rows) {
                    const int p = x / K;
                    const int r = x - p * K;
                    const unsigned pid = pid_of[p];
                    if (pid != kNoPid) {
                        dst[u] = (long long)pid * K + r;
                        if ((unsigned)r < running[p]) {
                            const unsigned vv = best[p * K + r];
                            if (vv < N) rw[u] = pts[vv];
                            else report_error(hdr, num_voxels, 8u);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (dst[u] >= 0) store_row(&voxels[dst[u]], rw[u], nt_out);
        }
    }
    if (t < G && pid_of[t] != kNoPid) {  // this thread's own slot
        const unsigned pid = pid_of[t];
        num_points[pid] = (int)(running[t] < (unsigned)K ? running[t] : (unsigned)K);
        write_coords(coords, pid, (long long)(key_of[t] - 1ull), gx, gy);
    }
}

// ------------------------------------------------- voxel-grid downsampling --
//
// One mean point per kept voxel (the voxel_downsample operation of the GPU
// K-D tree ICP page, "operation 1" of its section 4.4): the pipeline up to
// k_part (with rows carried) is the one above; k_centroid takes one block
// per bin like k_bins and ranks each arrival in its voxel the same way. Each
// round's arrivals are placed in LDS grouped by voxel in arrival order, which
// is input order, and one thread per voxel adds its group into four double
// sums in that order; the means are the sums over the counts, rounded once to
// float. The sums are sequential in input order, so the result is the same
// on every run and matches any other double-precision implementation of the
// same order.

__global__ __launch_bounds__(kBinBlock) __attribute__((amdgpu_waves_per_eu(8))) void k_centroid(
    const unsigned* __restrict__ cm, const unsigned* __restrict__ staging,
    const float4* __restrict__ stage_pt, long long ptiles, int ptile, int gshift, int nbits,
    int M, long long* __restrict__ kept_key, unsigned long long* __restrict__ compact, unsigned C,
    int* __restrict__ kept_cslot, int gx, int gy, float4* __restrict__ centroids,
    int* __restrict__ coords, int* __restrict__ counts, int* __restrict__ num_voxels,
    int* __restrict__ occ_slot, unsigned long long* __restrict__ table, unsigned S,
    unsigned long long* __restrict__ tile_state, long long ntiles, KMap kmap,
    Header* __restrict__ hdr, long long zero_words) {
    extern __shared__ float4 lds_rows[];
    const int G = 1 << gshift;
    float4* rowbuf = lds_rows;                   // [kBinBlock] this round's rows, by voxel
    unsigned* running = reinterpret_cast<unsigned*>(rowbuf + kBinBlock);  // [G] arrivals so far
    unsigned* wbuf = running + G;                // [3][kBinWaves * G] per-wavefront counts
    unsigned* roff = wbuf + 3 * kBinWaves * G;   // [kBinBlock + 1]
    unsigned* rsrc = roff + kBinBlock + 1;       // [kBinBlock]
    unsigned* wsum = rsrc + kBinBlock;           // [kWsumWords]
    unsigned* before = wsum + kWsumWords;        // [G] arrivals before this round
    unsigned* cnt_round = before + G;            // [G] arrivals in this round
    unsigned* seg = cnt_round + G;               // [G] start of the voxel's group in rowbuf

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    const long long b = xcd_tile(blockIdx.x, gridDim.x);  // contiguous bins per XCD, as k_bins
    unsigned e = 0u;
    if ((long long)t < ptiles) e = cm[(size_t)b * ptiles + t];
    const int status = hdr->status;
    const long long V = status > 0 ? status : 0;
    const long long distinct = hdr->distinct;
    const unsigned err = block_error(hdr);
    heal_workspace(hdr, zero_words, err);
    if (b == 0 && t == 0 && err != 0u) num_voxels[0] = VOX_STATUS_DEVICE_ERROR;
    release_workspace((long long)blockIdx.x * kBinBlock + t, (long long)gridDim.x * kBinBlock,
                      distinct, V, M, occ_slot, table, S, kept_key, compact, C, kept_cslot,
                      tile_state, ntiles, kmap, hdr, num_voxels);
    if (status <= 0) return;

    const long long nbins = 1ll << nbits;
    const int Gb = b < V ? (int)((V - b + nbins - 1) >> nbits) : 0;
    for (int x = t; x < G; x += kBinBlock) running[x] = 0u;
    for (int x = t; x < 3 * kBinWaves * G; x += kBinBlock) wbuf[x] = 0u;
    // thread t < 4 Gb: component t % 4 (x, y, z, intensity) of voxel t / 4
    double sum = 0.0;
    unsigned round = 0;
    for (long long tg = 0; tg < ptiles; tg += kBinBlock) {
        const long long tt = tg + t;
        if (tg > 0) {
            e = 0u;
            if (tt < ptiles) e = cm[(size_t)b * ptiles + tt];
        }
        unsigned ng;
        const unsigned ro = block_excl_scan<kBinWaves>(e >> 16, wsum, &ng);
        roff[t] = ro;
        rsrc[t] = e & 0xffffu;
        const int nruns = (int)(ptiles - tg < kBinBlock ? ptiles - tg : kBinBlock);
        __syncthreads();
        for (unsigned x0 = 0; x0 < ng; x0 += kBinBlock) {
            const unsigned x = x0 + (unsigned)t;
            bool valid = x < ng;
            unsigned pl = 0u;
            float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) {
                int lo = 0, hi = nruns;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (roff[mid] <= x) lo = mid;
                    else hi = mid;
                }
                const size_t src = (size_t)(tg + lo) * ptile + rsrc[lo] + (x - roff[lo]);
                pl = staging[src] >> 16;
                row = stage_pt[src];
                if (pl >= (unsigned)Gb) {  // not on a clean workspace
                    report_error(hdr, num_voxels, 4u);
                    valid = false;
                    pl = 0u;
                }
            }
            unsigned* cur = wbuf + (round % 3u) * (kBinWaves * G);
            unsigned* nxt = wbuf + ((round + 1u) % 3u) * (kBinWaves * G);
            for (int y = t; y < kBinWaves * G; y += kBinBlock) nxt[y] = 0u;
            const unsigned long long m = match_mask(pl, valid, gshift);
            const unsigned rank = (unsigned)__popcll(m & lanes_below(lane));
            if (valid && (m & lanes_above(lane)) == 0ull) cur[w * G + pl] = (unsigned)__popcll(m);
            __syncthreads();
            // thread p < G, voxel p: prefix over the wavefronts on top of the
            // earlier arrivals (eight reads in flight, then eight writes) and
            // this round's count; then the groups' starts in rowbuf
            unsigned cnt = 0u;
            if (t < G) {
                const unsigned b0 = running[t];
                unsigned acc = b0;
#pragma unroll
                for (int h0 = 0; h0 < kBinWaves; h0 += 8) {
                    unsigned cw[8];
#pragma unroll
                    for (int ww = 0; ww < 8; ++ww) cw[ww] = cur[(h0 + ww) * G + t];
#pragma unroll
                    for (int ww = 0; ww < 8; ++ww) {
                        cur[(h0 + ww) * G + t] = acc;
                        acc += cw[ww];
                    }
                }
                before[t] = b0;
                cnt = acc - b0;
                cnt_round[t] = cnt;
                running[t] = acc;
            }
            unsigned round_total;
            const unsigned sg = block_excl_scan<kBinWaves>(cnt, wsum, &round_total);
            if (t < G) seg[t] = sg;
            __syncthreads();
            if (valid) {
                const unsigned r = cur[w * G + pl] + rank;  // arrival rank in the voxel
                rowbuf[seg[pl] + (r - before[pl])] = row;
            }
            __syncthreads();
            if (t < 4 * Gb) {
                // one component of this voxel's rows of the round, added in
                // input order; the LDS reads go four at a time ahead of the
                // additions
                const unsigned s0 = seg[t >> 2], n = cnt_round[t >> 2];
                const float* col = reinterpret_cast<const float*>(rowbuf + s0) + (t & 3);
                unsigned k = 0;
                for (; k + 4u <= n; k += 4u) {
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) f[j] = col[4 * (k + j)];
#pragma unroll
                    for (int j = 0; j < 4; ++j) sum += (double)f[j];
                }
                for (; k < n; ++k) sum += (double)col[4 * k];
            }
            __syncthreads();  // rowbuf and the per-voxel words are reused
            ++round;
        }
    }
    // the four sums of voxel p meet in LDS (rowbuf is free now)
    double* dsum = reinterpret_cast<double*>(rowbuf);
    if (t < 4 * Gb) dsum[t] = sum;
    __syncthreads();
    if (t < Gb) {
        const long long pp = b + ((long long)t << nbits);
        const unsigned n = running[t];
        const double dn = (double)n;
        centroids[pp] = make_float4((float)(dsum[4 * t] / dn), (float)(dsum[4 * t + 1] / dn),
                                    (float)(dsum[4 * t + 2] / dn), (float)(dsum[4 * t + 3] / dn));
        counts[pp] = (int)n;
        const long long key = kept_key[pp];
        write_coords(coords, pp, key, gx, gy);
        if (kmap.p) kmap.put(key, 0u);
        kept_key[pp] = 0;
        if (C > 0) clear_compact(compact, C, kept_cslot, pp, hdr, num_voxels);
    }
}

// Downsampling on the first-index route: the bins of k_bins_fb (slot j of
// bin b is the cell whose lowest prefix index is i0 = b + j nbins; its id
// comes from the prefix tiles' counts, ids below max_voxels are kept) with
// k_centroid's sums. The rows arrive carried (stage_pt), bin after bin in
// index order; each round's arrivals are grouped by slot in LDS in arrival
// order and four threads per slot add its group's x, y, z and intensity into
// double sums in that order. The set-up returns the bin's claim state to
// zero, as k_bins_fb does. WPE as for k_bins_fb.
template <int WPE>
__global__ __launch_bounds__(kBinBlock) __attribute__((amdgpu_waves_per_eu(WPE))) void k_centroid_fb(
    const unsigned* __restrict__ cm, const unsigned* __restrict__ staging,
    const float4* __restrict__ stage_pt, long long N, long long P, int M, long long ptiles,
    int ptile, int tshift, int gshift, int nbits, const unsigned* __restrict__ tile_firsts,
    int ptp, unsigned long long* __restrict__ fkey, const unsigned* __restrict__ frank,
    unsigned* __restrict__ first, unsigned long long cells,
    unsigned long long* __restrict__ table, unsigned S, int* __restrict__ slot_of,
    unsigned char* __restrict__ filt, int fltshift, int gx, int gy,
    float4* __restrict__ centroids, int* __restrict__ coords, int* __restrict__ counts,
    int* __restrict__ num_voxels, Header* __restrict__ hdr, long long zero_words) {
    extern __shared__ float4 lds_rows[];
    const int G = 1 << gshift;
    // per-wavefront counts are 16-bit offsets within the round (at most
    // kBinBlock); the region first holds the tile prefix
    const int wwords = 3 * kBinWaves * G / 2 > kScanTiles ? 3 * kBinWaves * G / 2 : kScanTiles;
    float4* rowbuf = lds_rows;                   // [kBinBlock] this round's rows, by slot
    unsigned* running = reinterpret_cast<unsigned*>(rowbuf + kBinBlock);  // [G] arrivals so far
    unsigned* wbuf = running + G;                // [wwords] the tile prefix, then the counts
    unsigned short* wcnt = reinterpret_cast<unsigned short*>(wbuf);  // [3][kBinWaves * G]
    unsigned* roff = wbuf + wwords;              // [kBinBlock + 2] run offsets in the group
    unsigned* rsrc = roff + kBinBlock + 2;       // [kBinBlock] run start within its tile
    unsigned* wsum = rsrc + kBinBlock;           // [kWsumWords]
    unsigned* cnt_round = wsum + kWsumWords;     // [G] arrivals of the slot in this round
    unsigned* seg = cnt_round + G;               // [G] start of the slot's group in rowbuf
    unsigned* pid_of = seg + G;                  // [G] voxel id of each slot, kNoPid if none kept
    // [G] cell key + 1 of each slot (8-byte aligned: every count above is even)
    unsigned long long* key_of = reinterpret_cast<unsigned long long*>(pid_of + G);

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int w = t / kWave;
    const long long b = xcd_tile(blockIdx.x, gridDim.x);  // contiguous bins per XCD
    const long long nbins = 1ll << nbits;
    const int Gb = b < P ? (int)((P - b + nbins - 1) >> nbits) : 0;  // slots with i0 < P
    unsigned e = 0u;
    if ((long long)t < ptiles) e = cm[(size_t)b * ptiles + t];
    unsigned tc[kScanPer];
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
        const int q = t * kScanPer + u;
        tc[u] = q < ptp ? tile_firsts[q] : 0u;
    }
    const unsigned i0 = (unsigned)b + ((unsigned)t << nbits);  // this thread's slot
    unsigned long long fk = 0ull;
    unsigned fr = 0u;
    int fs = -1;
    if (t < Gb) {
        fk = fkey[i0];
        fr = frank[i0];
        if (!first) fs = slot_of[i0];
    }
    const unsigned err = block_error(hdr);
    heal_workspace(hdr, zero_words, err);
    if (t < G) {
        pid_of[t] = fr;  // the rank until the id is known
        key_of[t] = fk;
    }
    // one scan: the first group's run offsets and the tile counts
    unsigned s = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) s += tc[u];
    const unsigned sv[2] = {e >> 16, s};
    unsigned sx[2], st[2];
    block_excl_scan_n<kBinWaves, 2>(sv, wsum, sx, st);
    unsigned ng = st[0];
    const unsigned distinct_u = st[1];
    roff[t] = sx[0];
    rsrc[t] = e & 0xffffu;
    unsigned ex = sx[1];
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
        const int q = t * kScanPer + u;
        if (q < ptp) wbuf[q] = ex;
        ex += tc[u];
    }
    if (t < Gb)
        release_slot(first, cells, fkey, table, S, slot_of, i0, fk, fs, hdr, num_voxels, filt,
                     fltshift);
    __syncthreads();
    const long long distinct = distinct_u;
    const long long V = distinct < M ? distinct : M;
    int status = (int)V;
    if (N > P && distinct < M) status = VOX_STATUS_NEEDS_CHUNKED;
    if (err != 0u) status = VOX_STATUS_DEVICE_ERROR;
    if (blockIdx.x == 0 && t == 0) {
        hdr->status = status;
        hdr->distinct = (int)distinct;
        num_voxels[0] = status;
    }
    if (t < G) {
        unsigned mypid = kNoPid;
        if (key_of[t] != 0ull) {
            const unsigned pid = wbuf[i0 >> tshift] + pid_of[t];
            if ((long long)pid >= distinct) report_error(hdr, num_voxels, 4u);  // not on a clean workspace
            else if (status > 0 && (long long)pid < V) mypid = pid;
        }
        pid_of[t] = mypid;
    }
    __syncthreads();  // pid_of written, the tile prefix read
    if (status <= 0) return;  // block-uniform
    for (int x = t; x < G; x += kBinBlock) running[x] = 0u;
    for (int x = t; x < 3 * kBinWaves * G / 2; x += kBinBlock) wbuf[x] = 0u;
    __syncthreads();

    // thread t < 4 Gb: component t % 4 (x, y, z, intensity) of slot t / 4
    double sum = 0.0;
    unsigned round = 0;
    for (long long tg = 0; tg < ptiles; tg += kBinBlock) {
        if (tg > 0) {
            const long long tt = tg + t;
            e = 0u;
            if (tt < ptiles) e = cm[(size_t)b * ptiles + tt];
            const unsigned ro = block_excl_scan<kBinWaves>(e >> 16, wsum, &ng);
            roff[t] = ro;
            rsrc[t] = e & 0xffffu;
            __syncthreads();
        }
        const int nruns = (int)(ptiles - tg < kBinBlock ? ptiles - tg : kBinBlock);
        for (unsigned x0 = 0; x0 < ng; x0 += kBinBlock) {
            const unsigned x = x0 + (unsigned)t;
            bool valid = x < ng;
            unsigned pl = 0u;
            float4 row = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) {
                int lo = 0, hi = nruns;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (roff[mid] <= x) lo = mid;
                    else hi = mid;
                }
                const size_t src = (size_t)(tg + lo) * ptile + rsrc[lo] + (x - roff[lo]);
                pl = staging[src] >> 16;
                row = stage_pt[src];
                if (pl >= (unsigned)Gb) {  // not on a clean workspace
                    report_error(hdr, num_voxels, 4u);
                    valid = false;
                } else {
                    valid = pid_of[pl] != kNoPid;  // points of voxels past the cap are dropped
                }
                if (!valid) pl = 0u;
            }
            // counts of three rounds rotate: round r writes buffer r % 3 and
            // clears (r + 1) % 3, last read two rounds ago
            unsigned short* cur = wcnt + (round % 3u) * (kBinWaves * G);
            unsigned* nxt = wbuf + ((round + 1u) % 3u) * (kBinWaves * G / 2);
            for (int y = t; y < kBinWaves * G / 2; y += kBinBlock) nxt[y] = 0u;
            const unsigned long long m = match_mask(pl, valid, gshift);
            const unsigned rank = (unsigned)__popcll(m & lanes_below(lane));
            if (valid && (m & lanes_above(lane)) == 0ull)
                cur[w * G + pl] = (unsigned short)__popcll(m);
            __syncthreads();
            // thread p < G, slot p: the wavefronts' offsets within the round
            // (eight reads in flight, then eight writes) and the round's count
            unsigned cnt = 0u;
            if (t < G) {
                unsigned acc = 0u;
#pragma unroll
                for (int h0 = 0; h0 < kBinWaves; h0 += 8) {
                    unsigned cw[8];
#pragma unroll
                    for (int ww = 0; ww < 8; ++ww) cw[ww] = cur[(h0 + ww) * G + t];
#pragma unroll
                    for (int ww = 0; ww < 8; ++ww) {
                        cur[(h0 + ww) * G + t] = (unsigned short)acc;
                        acc += cw[ww];
                    }
                }
                cnt = acc;
                cnt_round[t] = cnt;
                running[t] += cnt;
            }
            unsigned round_total;
            const unsigned sg = block_excl_scan<kBinWaves>(cnt, wsum, &round_total);
            if (t < G) seg[t] = sg;
            __syncthreads();
            if (valid) rowbuf[seg[pl] + (unsigned)cur[w * G + pl] + rank] = row;
            __syncthreads();
            if (t < 4 * Gb) {
                // one component of this slot's rows of the round, added in
                // input order; the LDS reads go four at a time ahead of the
                // additions
                const unsigned s0 = seg[t >> 2], n = cnt_round[t >> 2];
                const float* col = reinterpret_cast<const float*>(rowbuf + s0) + (t & 3);
                unsigned k = 0;
                for (; k + 4u <= n; k += 4u) {
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) f[j] = col[4 * (k + j)];
#pragma unroll
                    for (int j = 0; j < 4; ++j) sum += (double)f[j];
                }
                for (; k < n; ++k) sum += (double)col[4 * k];
            }
            __syncthreads();  // rowbuf and the per-slot words are reused
            ++round;
        }
    }
    // the four sums of slot p meet in LDS (rowbuf is free now)
    double* dsum = reinterpret_cast<double*>(rowbuf);
    if (t < 4 * Gb) dsum[t] = sum;
    __syncthreads();
    if (t < Gb && pid_of[t] != kNoPid) {
        const unsigned pid = pid_of[t];
        const unsigned n = running[t];
        const double dn = (double)n;
        centroids[pid] = make_float4((float)(dsum[4 * t] / dn), (float)(dsum[4 * t + 1] / dn),
                                     (float)(dsum[4 * t + 2] / dn), (float)(dsum[4 * t + 3] / dn));
        counts[pid] = (int)n;
        write_coords(coords, pid, (long long)(key_of[t] - 1ull), gx, gy);
    }
}

// -------------------------------------------------------------- bin only --

__global__ __launch_bounds__(kBlock) void k_bin(const float4* __restrict__ pts, long long N,
                                                Grid g, int8_t* __restrict__ valid,
                                                long long* __restrict__ key) {
    const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
    if (i >= N) return;
    const long long k = bin_key(pts[i], g);
    valid[i] = k >= 0 ? 1 : 0;
    key[i] = k;
}

// =================================================================== host ==

thread_local int32_t g_last_hip_error = 0;

inline int hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return VOX_EHIP;
}

inline long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// k_rank's tile for a prefix of P points: the smallest of 256, 512 and 1,024
// points that leaves at most kRankTilesAim tiles (many small tiles spread the
// two dependent loads of a small prefix over more CUs; past that, the
// look-back over many tiles costs more than it saves).
inline int rank_tile(long long P) {
    int tile = kRankTileMin;
    while (tile < 4 * kRankTileMin && cdiv(P, tile) > kRankTilesAim) tile *= 2;
    return tile;
}
inline long long rank_tiles(long long P) { return P > 0 ? cdiv(P, rank_tile(P)) : 1; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    long long N, P, S, C;  // C: compact kept-cell table slots (0 = not used)
    long long mapn;        // kept-cell map entries (0 = no map region)
    int K, M, hash, cap;
    long long ntiles;
    // partitioned select/pack (part = 1): bins of 2^gshift pillar ids, ptiles
    // k_part tiles of pblock x pper points, nbits = bits of a bin number, lds
    // bytes of a k_bins block
    int part, carry, gshift, nbins, nbits, pper, pblock;
    long long ptiles;
    size_t lds;
    // first-index route (fb = 1, single pass only): bins of 2^fshift slots,
    // 2^fbits bins, ptp prefix tiles, fblds bytes of a k_bins_fb block;
    // merge = lane merge before the claim atomics; first_map = 1 forbids the
    // direct cell map
    int fb, fbits, fshift, merge, first_map, kmap_ok;
    int fltshift;  // first-index route on the table: 32 - log2(filter bytes)
    long long ptp;
    size_t fblds;
    // byte offsets into the workspace; [0, zero_bytes) is zero between calls,
    // [zero_bytes, bytes) is scratch every call writes before reading
    size_t off_table, off_slot, off_tiles, off_occ, off_kept, off_cnt, off_bucket, off_ovf,
        off_compact, off_kcs, off_map, off_fkey, off_filt, off_cm, off_stage, off_stage_pt, off_frank,
        off_tfirst, zero_bytes, bytes;
};

// LDS of one k_bins block for bins of G pillars (plus the selection when rows
// are gathered rather than carried)
inline size_t bins_lds_bytes(int G, int K, bool carry) {
    return 4u * (size_t)(G + 3 * kBinWaves * G + kBinBlock + 1 + kBinBlock + kWsumWords +
                         (carry ? 0 : G * K));
}
// LDS of one k_centroid block for bins of G voxels
inline size_t centroid_lds_bytes(int G) {
    return 16u * (size_t)kBinBlock +
           4u * (size_t)(G + 3 * kBinWaves * G + kBinBlock + 1 + kBinBlock + kWsumWords + 3 * G);
}
// LDS of one k_centroid_fb block for bins of G slots (16-bit counts; the
// words before key_of are an even count: it is 8-byte aligned)
inline size_t centroid_fb_lds_bytes(int G) {
    const size_t ww = (size_t)3 * kBinWaves * G / 2 > (size_t)kScanTiles
                          ? (size_t)3 * kBinWaves * G / 2 : (size_t)kScanTiles;
    return 16u * (size_t)kBinBlock +
           4u * ((size_t)G + ww + kBinBlock + 2 + kBinBlock + kWsumWords + 3 * (size_t)G) +
           8u * (size_t)G;
}
// LDS of one k_bins_fb block for bins of G pillar slots
inline size_t bins_fb_lds_bytes(int G, int K) {
    const size_t ww = (size_t)3 * kBinWaves * G / 2 > (size_t)kScanTiles
                          ? (size_t)3 * kBinWaves * G / 2 : (size_t)kScanTiles;
    // (the words before key_of are an even count: it is 8-byte aligned)
    return 4u * ((size_t)G + ww + kBinBlock + kBinBlock + kWinWords + kWinWords + 2 +
                 kWsumWords + (size_t)G) +
           8u * (size_t)G + 8u * (size_t)G + 4u * (size_t)G * K;
}
constexpr int kFbMaxIds = 256;     // pillar slots per k_bins_fb bin, at most
constexpr int kFbOneRound = 512;   // k_bins_fb blocks that fit the chip at once (2 per CU)
constexpr int kFbOneBlockPerCu = 256;  // bins that get one k_bins_fb block per CU (256 CUs)

inline bool finite_f(float v) { return isfinite(v); }

// Default bucket capacity: 16 K rounded up to a whole number of wavefronts.
inline int default_cap(int K) {
    if (K > kSortLanes) return 0;
    return (int)cdiv(16ll * K, kWave) * kWave;
}

// fb_carry (downsampling): the first-index route with rows carried, beside
// route 3's layout (which the chunked path then takes).
int make_plan(long long N, int M, int K, const vox_options* opt, Plan* pl,
              bool fb_carry = false) {
    if (N < 0 || N > kMaxPoints) return VOX_EINVAL;
    if (M < 1 || K < 1) return VOX_EINVAL;
    if ((long long)M > (1ll << 27)) return VOX_EINVAL;
    if ((long long)M * (long long)K > (1ll << 40)) return VOX_EINVAL;
    // 16 slots per kept pillar and a prefix of S/4 points: inserts see a load
    // of at most 1/4, which keeps probe chains (one atomic round trip per
    // step) short. Only occupied slots are ever cleared, so the size is free.
    long long S = 16ll * M;
    if (S < 64) S = 64;
    int hash = 0;
    long long P = 0;
    int cap = default_cap(K);
    if (opt) {
        if (opt->table_slots < 0 || opt->prefix_points < 0 || opt->bucket_cap < 0)
            return VOX_EINVAL;
        if (opt->table_slots > 0) S = opt->table_slots;
        if (opt->hash < 0 || opt->hash > 2) return VOX_EINVAL;
        if (opt->compact_table < 0 || opt->compact_table > 1) return VOX_EINVAL;
        if (opt->select_path < 0 || opt->select_path > 4) return VOX_EINVAL;
        if (opt->kept_map < 0 || opt->kept_map > 1) return VOX_EINVAL;
        if (opt->select_path == 4 && opt->compact_table) return VOX_EINVAL;
        if (opt->first_map < 0 || opt->first_map > 1) return VOX_EINVAL;
        if (opt->lane_merge < 0 || opt->lane_merge > 1) return VOX_EINVAL;
        if (opt->bin_ids != 0 && (opt->bin_ids < 16 || opt->bin_ids > kFbMaxIds ||
                                  (opt->bin_ids & (opt->bin_ids - 1))))
            return VOX_EINVAL;
        hash = opt->hash;
        P = opt->prefix_points;
        if (opt->bucket_cap > 0 && K <= kSortLanes) {
            if (opt->bucket_cap > (1 << 20)) return VOX_EINVAL;
            cap = opt->bucket_cap;
        }
    }
    // S >= 2M: while fewer than M cells are in the table, a chunk of
    // S/2 - cells >= 1 points always fits at load <= 1/2. Probing works a
    // cache line (16 slots) at a time, so S is rounded up to a multiple of 16.
    if (S < 2ll * M || S > 2147483647ll - 15) return VOX_EINVAL;
    S = (S + (long long)kLineSlots - 1) / (long long)kLineSlots * (long long)kLineSlots;
    // Default prefix: 2 max_voxels points (at most S/4). The cap is decided by
    // the first max_voxels distinct cells, which on the measured clouds occur
    // within 1.0-1.75 max_voxels points; a cloud that needs more reports
    // VOX_STATUS_NEEDS_CHUNKED and takes the chunked entry point. Inserting
    // fewer points makes both the insert and the rank shorter.
    if (P == 0) P = S / 4 < 2ll * M ? S / 4 : 2ll * M;
    if (P > S / 2) P = S / 2;
    if (P > N) P = N;
    pl->N = N;
    pl->P = P;
    pl->S = S;
    pl->K = K;
    pl->M = M;
    pl->hash = hash;
    // On request, rank also copies the kept cells into a table of 4 slots per
    // pillar that lookups past the prefix probe instead of the big one (it
    // stays in L2). Off by default: on the measured workloads the extra CAS
    // chain in rank costs more than the lookups save.
    pl->C = (opt && opt->compact_table == 1)
                ? (4ll * M + kLineSlots - 1) / kLineSlots * kLineSlots : 0;
    // arrays indexed by point go to N: the chunked path can insert every point
    const long long Nw = N > 0 ? N : 1;
    pl->ntiles = cdiv(Nw, kRankTileMin);   // look-back words for the smallest tile
    // Select/pack route: per-bin partition (no per-point device atomic) when
    // K <= 64 and the ids fit kMaxBins bins of at most 128; buckets otherwise.
    const int path = opt ? opt->select_path : 0;
    // bins of at most 128 ids (k_bins' LDS holds at most 128 x 64 selected indices)
    const int max_per_bin = 128;
    const bool part_ok = K <= kSortLanes && cdiv(M, max_per_bin) <= kMaxBins;
    if (path >= 2 && !part_ok) return VOX_EINVAL;
    pl->part = (path >= 2 || (path == 0 && part_ok)) ? 1 : 0;
    // rows are carried only on request: gathering the selected rows in k_bins
    // measured faster than carrying every kept point's row through k_part
    pl->carry = pl->part && path == 3 ? 1 : 0;
    pl->gshift = 0;
    pl->nbins = 0;
    pl->nbits = 0;
    pl->pper = 0;
    pl->pblock = kBlock;
    pl->ptiles = 0;
    pl->lds = 0;
    if (pl->part) {
        // a power-of-two number of bins, about M / 64 (M / 128 past 32768
        // pillars), and G = 2^gshift >= the ids one bin can hold
        const long long want = cdiv(M, M > 32768 ? max_per_bin : 64);
        while ((1ll << pl->nbits) < want) ++pl->nbits;
        pl->nbins = 1 << pl->nbits;
        const long long per_bin = cdiv(M, pl->nbins);
        while ((1ll << pl->gshift) < per_bin) ++pl->gshift;
        pl->lds = bins_lds_bytes(1 << pl->gshift, K, pl->carry);  // <= 66 KB
        // points per k_part thread: the smallest power of two up to 16 that
        // leaves at most kWideTilesMax 512-thread tiles. About 512 tiles
        // keeps both kernels busy: every bins block walks one run per tile,
        // so more tiles cost the bins kernel, and fewer leave CUs idle in
        // the partition.
        int per = 1;
        while (per < kPartMaxPer && cdiv(Nw, (long long)kWideBlock * per) > kWideTilesMax) per *= 2;
        pl->pper = per;
        // from 4 points per thread the tiles take 512 threads: as many threads
        // per CU (two blocks instead of four), half the tiles, so every bin's
        // run in a tile, which k_bins reads, is twice as long; with fewer
        // points per thread too, as long as that leaves kWideTilesMin tiles
        // (a frame of 122,880 points: 240 tiles, and bins kernels that walk
        // half as many runs; smaller clouds keep 256-thread tiles, which
        // spread them over more CUs)
        pl->pblock = (per >= 4 || cdiv(Nw, (long long)kWideBlock * per) >= kWideTilesMin)
                         ? kWideBlock : kBlock;
        pl->ptiles = cdiv(Nw, (long long)pl->pblock * per);
        cap = 0;  // no buckets
    }
    pl->cap = cap;
    // First-index route: bins of pillar slots i0 = b + j * bins for i0 < P,
    // about bin_ids slots per bin; each k_bins_fb block scans the counts of
    // the ptp prefix tiles itself.
    pl->fb = 0;
    pl->fbits = 0;
    pl->fshift = 0;
    pl->ptp = 0;
    pl->fblds = 0;
    pl->merge = opt ? opt->lane_merge : 0;
    pl->first_map = opt ? opt->first_map : 0;
    if (pl->part && (fb_carry || (!pl->carry && (path == 0 || path == 4))) && !pl->C) {
        // default: 128 slots per bin, or 256 when 128 would need more bins
        // than the chip runs at once
        const long long Pw = P > 0 ? P : 1;
        long long ids = 128;
        if (opt && opt->bin_ids) ids = opt->bin_ids;
        else if (cdiv(Pw, 128) > kFbOneRound) ids = 256;
        int fbits = 0;
        while ((1ll << fbits) < cdiv(Pw, ids) && (1 << fbits) < kMaxBins) ++fbits;
        int fshift = 0;
        while ((1ll << fshift) < cdiv(Pw, 1ll << fbits)) ++fshift;
        const long long tile = (long long)pl->pblock * pl->pper;
        const long long ptp = P > 0 ? cdiv(P, tile) : 0;  // tiles that write a count
        const bool ok = (1 << fshift) <= kFbMaxIds && ptp <= kScanTiles;
        if (ok) {
            pl->fb = 1;
            pl->fbits = fbits;
            pl->fshift = fshift;
            pl->ptp = ptp;
            pl->fblds = bins_fb_lds_bytes(1 << fshift, K);
        }
    }
    if (path == 4 && !pl->fb) return VOX_EINVAL;
    size_t off = sizeof(Header);
    pl->off_table = off;
    off = align256(off + (size_t)S * sizeof(unsigned long long));
    pl->off_slot = off;
    off = align256(off + (size_t)Nw * sizeof(int));
    pl->off_tiles = off;
    off = align256(off + (size_t)pl->ntiles * sizeof(unsigned long long));
    pl->off_occ = off;
    off = align256(off + (size_t)Nw * sizeof(int));
    pl->off_kept = off;
    off = align256(off + (size_t)M * sizeof(long long));
    pl->off_cnt = off;
    off = align256(off + (pl->part ? 0 : (size_t)M * sizeof(unsigned)));
    pl->off_bucket = off;
    off = align256(off + (size_t)M * (size_t)cap * sizeof(unsigned));
    pl->off_ovf = off;
    off = align256(off + (pl->part ? 0 : (size_t)M * (size_t)K * sizeof(unsigned)));
    pl->off_compact = off;
    off = align256(off + (size_t)pl->C * sizeof(unsigned long long));
    pl->off_kcs = off;
    off = align256(off + (pl->C > 0 ? (size_t)M * sizeof(int) : 0));
    // the kept-cell map: 2 S cells of 4 bytes (the table's own size), used
    // when the grid has at most that many cells
    // (the first-index route's direct cell map, 4 bytes per cell, shares it:
    // each route leaves the region zero)
    const bool kmap_ok = pl->part && pl->C == 0 && !(opt && opt->kept_map == 1);
    const bool dmap_ok = pl->fb && !pl->first_map;
    pl->kmap_ok = kmap_ok ? 1 : 0;
    pl->mapn = (kmap_ok || dmap_ok) ? 2 * S : 0;
    pl->off_map = off;
    off = align256(off + (size_t)pl->mapn * sizeof(unsigned));
    // first-index route: the cell key + 1 of each first occurrence in [0, P)
    pl->off_fkey = off;
    off = align256(off + (pl->fb ? (size_t)(P > 0 ? P : 1) * sizeof(unsigned long long) : 0));
    // first-index route: the claim's byte filter (used when the claim fills
    // the table), about 8 bytes per prefix point, a power of two from 64 KiB
    // to 4 MiB
    pl->fltshift = 0;
    pl->off_filt = off;
    if (pl->fb) {
        int lb = 16;
        while (lb < 22 && (1ll << lb) < 8 * (P > 0 ? P : 1)) ++lb;
        pl->fltshift = 32 - lb;
        off = align256(off + ((size_t)1 << lb));
    }
    pl->zero_bytes = off;  // the scratch tail starts here
    pl->off_cm = off;
    const long long cm_bins = pl->fb && (1ll << pl->fbits) > pl->nbins ? (1ll << pl->fbits)
                                                                        : pl->nbins;
    off = align256(off + (size_t)cm_bins * (size_t)pl->ptiles * sizeof(unsigned));
    pl->off_stage = off;
    off = align256(off + (size_t)pl->ptiles * (size_t)(pl->pblock * pl->pper) * sizeof(unsigned));
    pl->off_stage_pt = off;
    off = align256(off + (pl->carry ? (size_t)pl->ptiles * (size_t)(pl->pblock * pl->pper) *
                                          sizeof(float4)
                                    : 0));
    // first-index route: each first occurrence's rank in its tile, and each
    // prefix tile's count of first occurrences
    pl->off_frank = off;
    off = align256(off + (pl->fb ? (size_t)(P > 0 ? P : 1) * sizeof(unsigned) : 0));
    pl->off_tfirst = off;
    off = align256(off + (pl->fb ? (size_t)pl->ptp * sizeof(unsigned) : 0));
    pl->bytes = off;
    return VOX_OK;
}

int check_grid(const float range[6], const float cell[3], const int32_t grid[3], Grid* g) {
    if (!range || !cell || !grid) return VOX_EINVAL;
    for (int a = 0; a < 3; ++a) {
        if (!finite_f(range[a]) || !finite_f(range[a + 3]) || !(range[a] < range[a + 3]))
            return VOX_EINVAL;
        if (!finite_f(cell[a]) || !(cell[a] > 0.0f)) return VOX_EINVAL;
        if (grid[a] < 1 || grid[a] > (1 << 24)) return VOX_EINVAL;
    }
    if ((unsigned long long)grid[0] * (unsigned long long)grid[1] * (unsigned long long)grid[2] >
        kMaxCells)
        return VOX_EINVAL;
    g->x_min = range[0];
    g->y_min = range[1];
    g->z_min = range[2];
    g->z_max = range[5];
    g->vx = cell[0];
    g->vy = cell[1];
    g->vz = cell[2];
    g->gx = grid[0];
    g->gy = grid[1];
    g->gz = grid[2];
    return VOX_OK;
}

int check_args(const float* points, long long N, const float range[6], const float cell[3],
               const int32_t grid[3], float* voxels, int32_t* coords, int32_t* num_points,
               int32_t* num_voxels, void* ws, Grid* g) {
    if (!voxels || !coords || !num_points || !num_voxels || !ws) return VOX_EINVAL;
    if (N > 0 && !points) return VOX_EINVAL;
    if (points && ((uintptr_t)points & 15u)) return VOX_EINVAL;
    if (((uintptr_t)voxels & 15u) || ((uintptr_t)coords & 3u) || ((uintptr_t)num_points & 3u) ||
        ((uintptr_t)num_voxels & 3u))
        return VOX_EINVAL;
    return check_grid(range, cell, grid, g);
}

struct Buffers {
    Header* hdr;
    unsigned long long* table;
    int* slot_of;
    unsigned long long* tiles;
    int* occ;
    long long* kept;
    unsigned* cnt;
    unsigned* bucket;
    unsigned* ovf;
    unsigned long long* compact;
    int* kcs;
    unsigned* cm;
    unsigned* stage;
    float4* stage_pt;
    KMap kmap;  // the kept-cell map (p null when the grid does not fit it)
    // first-index route: the direct cell map (null: the table is used),
    // first occurrences' keys and ranks, prefix tiles' counts
    unsigned* first;
    unsigned long long* fkey;
    unsigned* frank;
    unsigned* tfirst;
    unsigned char* filt;  // the claim's byte filter (first-index route on the table), or null
};

Buffers carve(void* ws, const Plan& pl, const Grid& g) {
    char* b = static_cast<char*>(ws);
    Buffers x;
    x.hdr = reinterpret_cast<Header*>(b);
    x.table = reinterpret_cast<unsigned long long*>(b + pl.off_table);
    x.slot_of = reinterpret_cast<int*>(b + pl.off_slot);
    x.tiles = reinterpret_cast<unsigned long long*>(b + pl.off_tiles);
    x.occ = reinterpret_cast<int*>(b + pl.off_occ);
    x.kept = reinterpret_cast<long long*>(b + pl.off_kept);
    x.cnt = reinterpret_cast<unsigned*>(b + pl.off_cnt);
    x.bucket = reinterpret_cast<unsigned*>(b + pl.off_bucket);
    x.ovf = reinterpret_cast<unsigned*>(b + pl.off_ovf);
    x.compact = reinterpret_cast<unsigned long long*>(b + pl.off_compact);
    x.kcs = reinterpret_cast<int*>(b + pl.off_kcs);
    x.cm = reinterpret_cast<unsigned*>(b + pl.off_cm);
    x.stage = reinterpret_cast<unsigned*>(b + pl.off_stage);
    x.stage_pt = reinterpret_cast<float4*>(b + pl.off_stage_pt);
    const long long cells = (long long)g.gx * g.gy * g.gz;
    // no map when the prefix holds every point: nothing would look it up
    x.kmap.p = (pl.kmap_ok && pl.mapn > 0 && cells <= pl.mapn && pl.P < pl.N) ? b + pl.off_map
                                                                               : nullptr;
    x.kmap.narrow = pl.M <= 65534 ? 1 : 0;
    x.first = (pl.fb && !pl.first_map && pl.mapn > 0 && cells <= pl.mapn)
                  ? reinterpret_cast<unsigned*>(b + pl.off_map) : nullptr;
    x.fkey = reinterpret_cast<unsigned long long*>(b + pl.off_fkey);
    x.filt = (pl.fb && !x.first) ? reinterpret_cast<unsigned char*>(b + pl.off_filt) : nullptr;
    x.frank = reinterpret_cast<unsigned*>(b + pl.off_frank);
    x.tfirst = reinterpret_cast<unsigned*>(b + pl.off_tfirst);
    return x;
}

// Significant bits of a grid's cell keys (the lane merge matches on them).
inline int key_bits(const Grid& g) {
    const unsigned long long cells =
        (unsigned long long)g.gx * (unsigned long long)g.gy * (unsigned long long)g.gz;
    int b = 1;
    while (b < 64 && (1ull << b) < cells) ++b;
    return b;
}

int last_launch() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? VOX_OK : hip_fail(e);
}

// Every launch goes through hipExtLaunchKernelGGL: with a pair of events the
// runtime stamps them at the kernel's own start and end (stage profiling);
// without, it is a plain launch.
inline hipEvent_t ev_start(hipEvent_t* ev) { return ev ? ev[0] : nullptr; }
inline hipEvent_t ev_stop(hipEvent_t* ev) { return ev ? ev[1] : nullptr; }

int launch_insert(const float* points, long long begin, long long end, const Grid& g,
                  const Plan& pl, const Buffers& bf, hipStream_t st, int count_claims,
                  hipEvent_t* ev) {
    const long long n = end - begin;
    const unsigned blocks = (unsigned)(n > 0 ? cdiv(n, kBlock) : 1);
    hipExtLaunchKernelGGL(k_insert, dim3(blocks), dim3(kBlock), 0, st, ev_start(ev), ev_stop(ev), 0,
                       reinterpret_cast<const float4*>(points), begin, end, g, bf.table,
                       (unsigned)pl.S, pl.hash, bf.slot_of, bf.hdr, count_claims, pl.merge,
                       key_bits(g), bf.filt, pl.fltshift);
    return last_launch();
}

// First-index route, steps 1-3: the claim (direct map or table), the
// partition, the bins.
int launch_claim_fb(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                    hipStream_t st, hipEvent_t* ev) {
    if (!bf.first) return launch_insert(points, 0, pl.P, g, pl, bf, st, 0, ev);
    const unsigned blocks = (unsigned)(pl.P > 0 ? cdiv(pl.P, kBlock) : 1);
    hipExtLaunchKernelGGL(k_claim, dim3(blocks), dim3(kBlock), 0, st, ev_start(ev), ev_stop(ev), 0,
                          reinterpret_cast<const float4*>(points), pl.P, g, bf.first, pl.merge,
                          key_bits(g));
    return last_launch();
}

template <int PER, int BLK>
int launch_part_fb_t(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                     int32_t* point_pillar, hipStream_t st, hipEvent_t* ev, bool carry) {
    if (carry) {  // downsampling: rows carried, no inverse map
        if (bf.first)
            hipExtLaunchKernelGGL(k_part_fb<PER, BLK, true, true>, dim3((unsigned)pl.ptiles),
                                  dim3(BLK), 0, st, ev_start(ev), ev_stop(ev), 0,
                                  reinterpret_cast<const float4*>(points), pl.N, pl.P, g, bf.table,
                                  (unsigned)pl.S, pl.hash, bf.first, bf.slot_of, pl.fbits,
                                  pl.ptiles, bf.cm, bf.stage, bf.fkey, bf.frank, bf.tfirst, bf.hdr,
                                  nullptr, bf.filt, pl.fltshift, bf.stage_pt);
        else
            hipExtLaunchKernelGGL(k_part_fb<PER, BLK, false, true>, dim3((unsigned)pl.ptiles),
                                  dim3(BLK), 0, st, ev_start(ev), ev_stop(ev), 0,
                                  reinterpret_cast<const float4*>(points), pl.N, pl.P, g, bf.table,
                                  (unsigned)pl.S, pl.hash, bf.first, bf.slot_of, pl.fbits,
                                  pl.ptiles, bf.cm, bf.stage, bf.fkey, bf.frank, bf.tfirst, bf.hdr,
                                  nullptr, bf.filt, pl.fltshift, bf.stage_pt);
        return last_launch();
    }
    if (bf.first)
        hipExtLaunchKernelGGL(k_part_fb<PER, BLK, true>, dim3((unsigned)pl.ptiles), dim3(BLK), 0, st,
                              ev_start(ev), ev_stop(ev), 0, reinterpret_cast<const float4*>(points),
                              pl.N, pl.P, g, bf.table, (unsigned)pl.S, pl.hash, bf.first,
                              bf.slot_of, pl.fbits, pl.ptiles, bf.cm, bf.stage, bf.fkey, bf.frank,
                              bf.tfirst, bf.hdr, point_pillar, bf.filt, pl.fltshift,
                              static_cast<float4*>(nullptr));
    else
        hipExtLaunchKernelGGL(k_part_fb<PER, BLK, false>, dim3((unsigned)pl.ptiles), dim3(BLK), 0,
                              st, ev_start(ev), ev_stop(ev), 0,
                              reinterpret_cast<const float4*>(points), pl.N, pl.P, g, bf.table,
                              (unsigned)pl.S, pl.hash, bf.first, bf.slot_of, pl.fbits, pl.ptiles,
                              bf.cm, bf.stage, bf.fkey, bf.frank, bf.tfirst, bf.hdr, point_pillar,
                              bf.filt, pl.fltshift, static_cast<float4*>(nullptr));
    return last_launch();
}

int launch_part_fb(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                   int32_t* point_pillar, hipStream_t st, hipEvent_t* ev, bool carry = false) {
    const bool wide = pl.pblock == kWideBlock;
    switch (pl.pper) {
        case 2:
            return wide ? launch_part_fb_t<2, kWideBlock>(points, g, pl, bf, point_pillar, st, ev,
                                                          carry)
                        : launch_part_fb_t<2, kBlock>(points, g, pl, bf, point_pillar, st, ev, carry);
        case 4:
            return launch_part_fb_t<4, kWideBlock>(points, g, pl, bf, point_pillar, st, ev, carry);
        case 8:
            return launch_part_fb_t<8, kWideBlock>(points, g, pl, bf, point_pillar, st, ev, carry);
        case 16:
            return launch_part_fb_t<16, kWideBlock>(points, g, pl, bf, point_pillar, st, ev, carry);
        default:
            return wide ? launch_part_fb_t<1, kWideBlock>(points, g, pl, bf, point_pillar, st, ev,
                                                          carry)
                        : launch_part_fb_t<1, kBlock>(points, g, pl, bf, point_pillar, st, ev, carry);
    }
}

int launch_bins_fb(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                   float* voxels, int32_t* coords, int32_t* num_points, int32_t* num_voxels,
                   int32_t* point_pillar, hipStream_t st, hipEvent_t* ev) {
    const int nt_out = (double)pl.M * pl.K * sizeof(float4) >= 16.0 * 1024 * 1024 ? 1 : 0;
    const long long tile = (long long)pl.pblock * pl.pper;
    int tshift = 0;
    while ((1ll << tshift) < tile) ++tshift;
    // up to one bin per CU: the kernel built for one block per CU
    hipExtLaunchKernelGGL((1 << pl.fbits) <= kFbOneBlockPerCu ? &k_bins_fb<4> : &k_bins_fb<8>,
                          dim3(1u << pl.fbits), dim3(kBinBlock), (unsigned)pl.fblds, st,
                          ev_start(ev), ev_stop(ev), 0, reinterpret_cast<const float4*>(points),
                          pl.N, pl.P, pl.M, pl.K, bf.cm, bf.stage, pl.ptiles, (int)tile, tshift,
                          pl.fshift, pl.fbits, bf.tfirst, (int)pl.ptp, bf.fkey, bf.frank, bf.first,
                          (unsigned long long)g.gx * g.gy * g.gz, bf.table, (unsigned)pl.S,
                          bf.slot_of, g.gx, g.gy,
                          reinterpret_cast<float4*>(voxels), coords, num_points, num_voxels,
                          point_pillar, bf.hdr, nt_out, (long long)(pl.zero_bytes / 4), bf.filt,
                          pl.fltshift);
    return last_launch();
}

int launch_rank(long long P, const Plan& pl, const Buffers& bf, int32_t* num_voxels,
                hipStream_t st, hipEvent_t* ev) {
    const long long ntiles = rank_tiles(P);
    const int tile = P > 0 ? rank_tile(P) : kRankTileMin;
    decltype(&k_rank<1>) kern = tile == 1024 ? &k_rank<4> : tile == 512 ? &k_rank<2> : &k_rank<1>;
    hipExtLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(kBlock), 0, st, ev_start(ev),
                          ev_stop(ev), 0, P, pl.N, pl.M,
                       bf.table, bf.compact, (unsigned)pl.C, pl.hash, bf.kcs, bf.slot_of,
                       bf.tiles, ntiles, bf.occ, bf.kept, bf.kmap, bf.hdr, num_voxels);
    return last_launch();
}

int launch_select(const float* points, long long P, const Grid& g, const Plan& pl,
                  const Buffers& bf, int32_t* num_voxels, int32_t* point_pillar,
                  hipStream_t st, hipEvent_t* ev) {
    if (pl.part) {
        // the plan's tile: 256 or 512 threads below 4 points per thread,
        // 512 from 4
        const bool wide = pl.pblock == kWideBlock;
        decltype(&k_part<1, false, kBlock>) kern =
            wide ? (pl.carry ? &k_part<1, true, kWideBlock> : &k_part<1, false, kWideBlock>)
                 : (pl.carry ? &k_part<1, true, kBlock> : &k_part<1, false, kBlock>);
        switch (pl.pper) {
            case 2:
                kern = wide ? (pl.carry ? &k_part<2, true, kWideBlock> : &k_part<2, false, kWideBlock>)
                            : (pl.carry ? &k_part<2, true, kBlock> : &k_part<2, false, kBlock>);
                break;
            case 4:
                kern = pl.carry ? &k_part<4, true, kWideBlock> : &k_part<4, false, kWideBlock>;
                break;
            case 8:
                kern = pl.carry ? &k_part<8, true, kWideBlock> : &k_part<8, false, kWideBlock>;
                break;
            case 16:
                kern = pl.carry ? &k_part<16, true, kWideBlock> : &k_part<16, false, kWideBlock>;
                break;
            default: break;
        }
        hipExtLaunchKernelGGL(kern, dim3((unsigned)pl.ptiles), dim3(pl.pblock), 0, st, ev_start(ev),
                              ev_stop(ev), 0,
                           reinterpret_cast<const float4*>(points), pl.N, P, g, bf.table,
                           (unsigned)pl.S, bf.compact, (unsigned)pl.C, pl.hash, bf.slot_of,
                           bf.kmap, pl.nbits, pl.ptiles, bf.cm, bf.stage, bf.stage_pt, bf.hdr,
                           num_voxels, point_pillar);
        return last_launch();
    }
    const unsigned blocks = (unsigned)(pl.N > 0 ? cdiv(pl.N, kBlock) : 1);
    hipExtLaunchKernelGGL(k_select, dim3(blocks), dim3(kBlock), 0, st, ev_start(ev), ev_stop(ev), 0,
                       reinterpret_cast<const float4*>(points), pl.N, P, g, bf.table,
                       (unsigned)pl.S, bf.compact, (unsigned)pl.C, pl.hash, bf.slot_of, bf.cnt,
                       bf.bucket, pl.cap, bf.ovf, pl.K, bf.hdr, num_voxels, point_pillar);
    return last_launch();
}

int launch_pack(const float* points, long long P, const Grid& g, const Plan& pl,
                const Buffers& bf, float* voxels, int32_t* coords, int32_t* num_points,
                int32_t* num_voxels, hipStream_t st, hipEvent_t* ev) {
    const long long ntiles = rank_tiles(P);
    if (pl.part) {
        // Outputs of 16 MiB and more are written with streaming stores (one
        // MI355X measured 0.7 us faster that way on a 30.7 MB stack; on
        // stacks of a few MB it was level or slower).
        const int nt_out = (double)pl.M * pl.K * sizeof(float4) >= 16.0 * 1024 * 1024 ? 1 : 0;
        // one block per bin; all blocks share the workspace release
        hipExtLaunchKernelGGL(pl.carry ? k_bins<true> : k_bins<false>, dim3((unsigned)pl.nbins),
                              dim3(kBinBlock), (unsigned)pl.lds, st,
                              ev_start(ev), ev_stop(ev), 0,
                           reinterpret_cast<const float4*>(points), pl.N, bf.cm, bf.stage,
                           bf.stage_pt, pl.ptiles, pl.pblock * pl.pper, pl.gshift, pl.nbits, pl.K,
                           pl.M,
                           bf.kept, bf.compact,
                           (unsigned)pl.C, bf.kcs, g.gx, g.gy,
                           reinterpret_cast<float4*>(voxels), coords, num_points, num_voxels,
                           bf.occ, bf.table, (unsigned)pl.S, bf.tiles, ntiles, bf.kmap, bf.hdr,
                           nt_out, (long long)(pl.zero_bytes / 4));
        return last_launch();
    }
    // lanes per pillar: next power of two >= max(K, 8) (a whole wave if K > 64)
    int seg = 8;
    while (seg < pl.K && seg < kWave) seg *= 2;
    const long long per_wave = kWave / seg;
    // enough wavefronts for at most M pillars, and threads for the cleanup of
    // at most P table slots
    long long blocks = cdiv(cdiv((long long)pl.M, per_wave), kWavesPerBlock);
    const long long clean_blocks = cdiv(P > 0 ? P : 1, kBlock);
    if (clean_blocks > blocks) blocks = clean_blocks;
    if (blocks < 1) blocks = 1;
    if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
    hipExtLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(kBlock), 0, st, ev_start(ev),
                          ev_stop(ev), 0,
                       reinterpret_cast<const float4*>(points), pl.N, bf.cnt, bf.bucket, pl.cap,
                       bf.ovf, pl.K, pl.M, seg, bf.kept, bf.compact, (unsigned)pl.C, bf.kcs,
                       g.gx, g.gy,
                       reinterpret_cast<float4*>(voxels), coords, num_points, num_voxels,
                       bf.occ, bf.table, (unsigned)pl.S, bf.tiles, ntiles, bf.hdr,
                       (long long)(pl.zero_bytes / 4));
    return last_launch();
}

int prepare(const float* points, int64_t n_points, const float range[6], const float cell[3],
            const int32_t grid[3], int32_t max_points, int32_t max_voxels, float* voxels,
            int32_t* coords, int32_t* num_points, int32_t* num_voxels, void* workspace,
            size_t workspace_bytes, const vox_options* options, Grid* g, Plan* pl) {
    int rc = check_args(points, n_points, range, cell, grid, voxels, coords, num_points,
                        num_voxels, workspace, g);
    if (rc != VOX_OK) return rc;
    rc = make_plan(n_points, max_voxels, max_points, options, pl);
    if (rc != VOX_OK) return rc;
    if (((uintptr_t)workspace & 255u) || workspace_bytes < pl->bytes) return VOX_EWORKSPACE;
    return VOX_OK;
}

// The four stages of one call; with ev (2 events per stage), each kernel's
// own start and end are stamped.
int run_pipeline(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                 float* voxels, int32_t* coords, int32_t* num_points, int32_t* num_voxels,
                 int32_t* point_pillar, hipStream_t st, hipEvent_t* ev) {
    int rc;
    if (pl.fb) {  // three kernels: no rank stage (its events are left unrecorded)
        if ((rc = launch_claim_fb(points, g, pl, bf, st, ev)) != VOX_OK) return rc;
        if ((rc = launch_part_fb(points, g, pl, bf, point_pillar, st, ev ? ev + 4 : nullptr)) !=
            VOX_OK)
            return rc;
        return launch_bins_fb(points, g, pl, bf, voxels, coords, num_points, num_voxels,
                              point_pillar, st, ev ? ev + 6 : nullptr);
    }
    if ((rc = launch_insert(points, 0, pl.P, g, pl, bf, st, 0, ev ? ev : nullptr)) != VOX_OK)
        return rc;
    if ((rc = launch_rank(pl.P, pl, bf, num_voxels, st, ev ? ev + 2 : nullptr)) != VOX_OK)
        return rc;
    if ((rc = launch_select(points, pl.P, g, pl, bf, num_voxels, point_pillar, st,
                            ev ? ev + 4 : nullptr)) != VOX_OK)
        return rc;
    return launch_pack(points, pl.P, g, pl, bf, voxels, coords, num_points, num_voxels, st,
                       ev ? ev + 6 : nullptr);
}

// Fill the table chunk by chunk while fewer than M cells are in it, reading
// the claim count on the host between chunks. Before each chunk `have` < M
// cells are present, so a chunk of S/2 - have points keeps the load at or
// below one half. *done = the points inserted (the prefix rank then scans).
int insert_chunked(const float* points, const Grid& g, const Plan& pl, const Buffers& bf,
                   hipStream_t stream, long long* done_out) {
    long long done = 0;
    long long have = 0;
    const long long half = pl.S / 2;
    int rc;
    // the rank, select and pack kernels that follow never clear the
    // first-index route's key filter, so the chunks leave it untouched
    Buffers nb = bf;
    nb.filt = nullptr;
    while (done < pl.N && have < pl.M) {
        long long chunk = half - have;
        if (chunk > pl.N - done) chunk = pl.N - done;
        if ((rc = launch_insert(points, done, done + chunk, g, pl, nb, stream, 1, nullptr)) !=
            VOX_OK)
            return rc;
        done += chunk;
        unsigned claims = 0;
        hipError_t e = hipMemcpyAsync(&claims, &bf.hdr->claims, sizeof(claims),
                                      hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e);
        have = claims;
    }
    *done_out = done;
    return VOX_OK;
}

// Downsampling carries the rows through the partition and has no
// max_points (the plan takes K = 1). select_path 0: the first-index route
// where it applies (route 3's layout beside it, for the chunked path), else
// route 3; 3: route 3; 4: the first-index route or VOX_EINVAL.
int downsample_plan(long long N, int M, const vox_options* options, Plan* pl) {
    vox_options o;
    if (options) {
        o = *options;
        if (o.select_path != 0 && o.select_path != 3 && o.select_path != 4) return VOX_EINVAL;
    } else {
        memset(&o, 0, sizeof(o));
    }
    const int want = o.select_path;
    o.select_path = 3;
    const int rc = make_plan(N, M, 1, &o, pl, want != 3);
    if (rc != VOX_OK) return rc;
    if (want == 4 && !pl->fb) return VOX_EINVAL;
    pl->lds = centroid_lds_bytes(1 << pl->gshift);
    if (pl->fb) pl->fblds = centroid_fb_lds_bytes(1 << pl->fshift);
    return VOX_OK;
}

int launch_centroid_fb(const Plan& pl, const Buffers& bf, const Grid& g, float* centroids,
                       int32_t* coords, int32_t* counts, int32_t* num_voxels, hipStream_t st) {
    const long long tile = (long long)pl.pblock * pl.pper;
    int tshift = 0;
    while ((1ll << tshift) < tile) ++tshift;
    hipExtLaunchKernelGGL((1 << pl.fbits) <= kFbOneBlockPerCu ? &k_centroid_fb<4> : &k_centroid_fb<8>,
                          dim3(1u << pl.fbits), dim3(kBinBlock),
                          (unsigned)pl.fblds, st, nullptr, nullptr, 0, bf.cm, bf.stage,
                          bf.stage_pt, pl.N, pl.P, pl.M, pl.ptiles, (int)tile, tshift, pl.fshift,
                          pl.fbits, bf.tfirst, (int)pl.ptp, bf.fkey, bf.frank, bf.first,
                          (unsigned long long)g.gx * g.gy * g.gz, bf.table, (unsigned)pl.S,
                          bf.slot_of, bf.filt, pl.fltshift, g.gx, g.gy,
                          reinterpret_cast<float4*>(centroids), coords, counts, num_voxels,
                          bf.hdr, (long long)(pl.zero_bytes / 4));
    return last_launch();
}

int launch_centroid(const Plan& pl, long long P, const Buffers& bf, const Grid& g,
                    float* centroids, int32_t* coords, int32_t* counts, int32_t* num_voxels,
                    hipStream_t st) {
    const long long ntiles = rank_tiles(P);
    hipExtLaunchKernelGGL(k_centroid, dim3((unsigned)pl.nbins), dim3(kBinBlock),
                          (unsigned)pl.lds, st, nullptr, nullptr, 0, bf.cm, bf.stage,
                          bf.stage_pt, pl.ptiles, pl.pblock * pl.pper, pl.gshift, pl.nbits, pl.M,
                          bf.kept, bf.compact, (unsigned)pl.C, bf.kcs, g.gx, g.gy,
                          reinterpret_cast<float4*>(centroids), coords, counts, num_voxels,
                          bf.occ, bf.table, (unsigned)pl.S, bf.tiles, ntiles, bf.kmap, bf.hdr,
                          (long long)(pl.zero_bytes / 4));
    return last_launch();
}

// Zeroes words [0, n) of p (grid-stride).
__global__ __launch_bounds__(kBlock) void k_zero(unsigned* __restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (long long)gridDim.x * kBlock)
        p[i] = 0u;
}

int launch_zero(void* p, size_t lo, size_t hi, hipStream_t st) {
    if (hi <= lo) return VOX_OK;
    const long long n = (long long)((hi - lo) / 4);
    const long long blocks = cdiv(n, kBlock) < 2048 ? cdiv(n, kBlock) : 2048;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                       reinterpret_cast<unsigned*>(static_cast<char*>(p) + lo), n);
    return last_launch();
}

}  // namespace

// ------------------------------------------------- allocation-free entry --
//
// voxelize_static's scratch: one array of kStaticScratchBytes per GPU, in
// the library's own code object, which each device that loads the library
// keeps until the process ends. In host code `scratch` only names the
// symbol: its device address is taken once per device, with that device
// current, by hipGetSymbolAddress, and only that address is ever passed on.
constexpr size_t kStaticScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Per device: the array's address, and which bytes may be nonzero. A call
// leaves [0, its zero part) zero and may leave scratch up to its layout's
// end, so after calls of several shapes [dlo, dhi) may be dirty; a call
// whose zero part reaches into it clears that stretch first, as the Python
// binding does for its cached workspaces. all_dirty: a call stopped
// between launches (a HIP error), so the whole array is cleared next time.
struct StaticScratch {
    void* p;
    size_t dlo, dhi;
    bool all_dirty;
};
std::mutex g_static_mu;
StaticScratch g_static[kMaxDevices];

}  // namespace

// Records a HIP error for vox_last_hip_error(); used by the library's other
// translation units.
__attribute__((visibility("hidden"))) int ssh_hip_fail(hipError_t e) { return hip_fail(e); }

// =================================================================== C ABI ==

extern "C" {

int64_t vox_workspace_bytes(int64_t n_points, int32_t max_voxels, int32_t max_points,
                            const vox_options* options) {
    Plan pl;
    const int rc = make_plan(n_points, max_voxels, max_points, options, &pl);
    if (rc != VOX_OK) return rc;
    return (int64_t)pl.bytes;
}

int64_t vox_workspace_zero_bytes(int64_t n_points, int32_t max_voxels, int32_t max_points,
                                 const vox_options* options) {
    Plan pl;
    const int rc = make_plan(n_points, max_voxels, max_points, options, &pl);
    if (rc != VOX_OK) return rc;
    return (int64_t)pl.zero_bytes;
}

int32_t vox_select_route(int64_t n_points, int32_t max_voxels, int32_t max_points,
                         const vox_options* options) {
    Plan pl;
    const int rc = make_plan(n_points, max_voxels, max_points, options, &pl);
    if (rc != VOX_OK) return rc;
    return pl.fb ? 4 : pl.part ? (pl.carry ? 3 : 2) : 1;
}

int vox_plan(int64_t n_points, int32_t max_voxels, int32_t max_points,
             const vox_options* options, int64_t* table_slots, int64_t* prefix_points,
             int32_t* bucket_cap) {
    Plan pl;
    const int rc = make_plan(n_points, max_voxels, max_points, options, &pl);
    if (rc != VOX_OK) return rc;
    if (table_slots) *table_slots = pl.S;
    if (prefix_points) *prefix_points = pl.P;
    if (bucket_cap) *bucket_cap = pl.cap;
    return VOX_OK;
}

int voxelize_ex(const float* points, int64_t n_points, const float range[6],
                const float cell[3], const int32_t grid[3], int32_t max_points,
                int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                int32_t* num_voxels, void* workspace, size_t workspace_bytes,
                hipStream_t stream, const vox_options* options) {
    Grid g;
    Plan pl;
    const int rc = prepare(points, n_points, range, cell, grid, max_points, max_voxels, voxels,
                           coords, num_points, num_voxels, workspace, workspace_bytes, options,
                           &g, &pl);
    if (rc != VOX_OK) return rc;
    const Buffers bf = carve(workspace, pl, g);
    return run_pipeline(points, g, pl, bf, voxels, coords, num_points, num_voxels, nullptr,
                        stream, nullptr);
}

int voxelize(const float* points, int64_t n_points, const float range[6], const float cell[3],
             const int32_t grid[3], int32_t max_points, int32_t max_voxels, float* voxels,
             int32_t* coords, int32_t* num_points, int32_t* num_voxels, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
    return voxelize_ex(points, n_points, range, cell, grid, max_points, max_voxels, voxels,
                       coords, num_points, num_voxels, workspace, workspace_bytes, stream,
                       nullptr);
}

int voxelize_chunked(const float* points, int64_t n_points, const float range[6],
                     const float cell[3], const int32_t grid[3], int32_t max_points,
                     int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                     int32_t* num_voxels, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const vox_options* options) {
    return voxelize_map(points, n_points, range, cell, grid, max_points, max_voxels, voxels,
                        coords, num_points, num_voxels, nullptr, workspace, workspace_bytes,
                        stream, options, 1);
}

int voxelize_map(const float* points, int64_t n_points, const float range[6],
                 const float cell[3], const int32_t grid[3], int32_t max_points,
                 int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                 int32_t* num_voxels, int32_t* point_pillar, void* workspace,
                 size_t workspace_bytes, hipStream_t stream, const vox_options* options,
                 int32_t chunked) {
    Grid g;
    Plan pl;
    int rc = prepare(points, n_points, range, cell, grid, max_points, max_voxels, voxels,
                     coords, num_points, num_voxels, workspace, workspace_bytes, options, &g,
                     &pl);
    if (rc != VOX_OK) return rc;
    if (n_points > 0 && point_pillar && ((uintptr_t)point_pillar & 3u)) return VOX_EINVAL;
    if (chunked < 0 || chunked > 2) return VOX_EINVAL;
    const Buffers bf = carve(workspace, pl, g);
    if (chunked != 1) {
        rc = run_pipeline(points, g, pl, bf, voxels, coords, num_points, num_voxels,
                          point_pillar, stream, nullptr);
        if (rc != VOX_OK || chunked == 0) return rc;
        // automatic: read the status; only an undecided cap takes the chunked path
        int32_t status = 0;
        hipError_t e = hipMemcpyAsync(&status, num_voxels, sizeof(status), hipMemcpyDeviceToHost,
                                      stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e);
        if (status != VOX_STATUS_NEEDS_CHUNKED) return VOX_OK;
    }
    long long done = 0;
    if ((rc = insert_chunked(points, g, pl, bf, stream, &done)) != VOX_OK) return rc;
    Plan p2 = pl;
    p2.P = done;
    if ((rc = launch_rank(done, p2, bf, num_voxels, stream, nullptr)) != VOX_OK) return rc;
    if ((rc = launch_select(points, done, g, p2, bf, num_voxels, point_pillar, stream,
                            nullptr)) != VOX_OK)
        return rc;
    return launch_pack(points, done, g, p2, bf, voxels, coords, num_points, num_voxels, stream,
                       nullptr);
}

int vox_bin_points(const float* points, int64_t n_points, const float range[6],
                   const float cell[3], const int32_t grid[3], int8_t* valid, int64_t* key,
                   hipStream_t stream) {
    if (!range || !cell || !grid || n_points < 0 || n_points > 2147483647ll) return VOX_EINVAL;
    if (n_points > 0 && (!points || !valid || !key)) return VOX_EINVAL;
    if (points && ((uintptr_t)points & 15u)) return VOX_EINVAL;
    if (key && ((uintptr_t)key & 7u)) return VOX_EINVAL;
    Grid g;
    const int rc = check_grid(range, cell, grid, &g);
    if (rc != VOX_OK) return rc;
    if (n_points == 0) return VOX_OK;
    hipLaunchKernelGGL(k_bin, dim3((unsigned)cdiv(n_points, kBlock)), dim3(kBlock), 0, stream,
                       reinterpret_cast<const float4*>(points), (long long)n_points, g, valid,
                       reinterpret_cast<long long*>(key));
    return last_launch();
}

int64_t vox_downsample_workspace_bytes(int64_t n_points, int32_t max_voxels,
                                       const vox_options* options) {
    Plan pl;
    const int rc = downsample_plan(n_points, max_voxels, options, &pl);
    return rc != VOX_OK ? rc : (int64_t)pl.bytes;
}

int64_t vox_downsample_workspace_zero_bytes(int64_t n_points, int32_t max_voxels,
                                            const vox_options* options) {
    Plan pl;
    const int rc = downsample_plan(n_points, max_voxels, options, &pl);
    return rc != VOX_OK ? rc : (int64_t)pl.zero_bytes;
}

int vox_downsample(const float* points, int64_t n_points, const float range[6],
                   const float cell[3], const int32_t grid[3], int32_t max_voxels,
                   float* centroids, int32_t* coords, int32_t* counts, int32_t* num_voxels,
                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                   const vox_options* options, int32_t chunked) {
    if (!centroids || !coords || !counts || !num_voxels || !workspace) return VOX_EINVAL;
    if (n_points > 0 && !points) return VOX_EINVAL;
    if ((points && ((uintptr_t)points & 15u)) || ((uintptr_t)centroids & 15u) ||
        ((uintptr_t)coords & 3u) || ((uintptr_t)counts & 3u) || ((uintptr_t)num_voxels & 3u))
        return VOX_EINVAL;
    Grid g;
    int rc = check_grid(range, cell, grid, &g);
    if (rc != VOX_OK) return rc;
    Plan pl;
    if ((rc = downsample_plan(n_points, max_voxels, options, &pl)) != VOX_OK) return rc;
    if (((uintptr_t)workspace & 255u) || workspace_bytes < pl.bytes) return VOX_EWORKSPACE;
    const Buffers bf = carve(workspace, pl, g);
    if (!chunked && pl.fb) {
        // first-index route: claim, partition with rows carried, centroids
        if ((rc = launch_claim_fb(points, g, pl, bf, stream, nullptr)) != VOX_OK) return rc;
        if ((rc = launch_part_fb(points, g, pl, bf, nullptr, stream, nullptr, true)) != VOX_OK)
            return rc;
        return launch_centroid_fb(pl, bf, g, centroids, coords, counts, num_voxels, stream);
    }
    long long P = pl.P;
    if (chunked) {
        if ((rc = insert_chunked(points, g, pl, bf, stream, &P)) != VOX_OK) return rc;
    } else if ((rc = launch_insert(points, 0, P, g, pl, bf, stream, 0, nullptr)) != VOX_OK) {
        return rc;
    }
    Plan p2 = pl;
    p2.P = P;
    if ((rc = launch_rank(P, p2, bf, num_voxels, stream, nullptr)) != VOX_OK) return rc;
    if ((rc = launch_select(points, P, g, p2, bf, num_voxels, nullptr, stream, nullptr)) !=
        VOX_OK)
        return rc;
    return launch_centroid(p2, P, bf, g, centroids, coords, counts, num_voxels, stream);
}

int vox_profile_stages(const float* points, int64_t n_points, const float range[6],
                       const float cell[3], const int32_t grid[3], int32_t max_points,
                       int32_t max_voxels, float* voxels, int32_t* coords,
                       int32_t* num_points, int32_t* num_voxels, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, const vox_options* options,
                       int32_t iters, float* stage_ms, float* total_ms) {
    if (iters < 1 || !stage_ms || !total_ms) return VOX_EINVAL;
    Grid g;
    Plan pl;
    int rc = prepare(points, n_points, range, cell, grid, max_points, max_voxels, voxels,
                     coords, num_points, num_voxels, workspace, workspace_bytes, options, &g,
                     &pl);
    if (rc != VOX_OK) return rc;
    const Buffers bf = carve(workspace, pl, g);
    const int nev = 2 * VOX_NUM_STAGES;  // a start and a stop per kernel
    hipEvent_t* ev = new hipEvent_t[(size_t)iters * nev];
    int created = 0;
    for (; created < iters * nev; ++created) {
        const hipError_t e = hipEventCreate(&ev[created]);
        if (e != hipSuccess) {
            rc = hip_fail(e);
            break;
        }
    }
    for (int it = 0; rc == VOX_OK && it < iters; ++it)
        rc = run_pipeline(points, g, pl, bf, voxels, coords, num_points, num_voxels, nullptr,
                          stream, ev + (size_t)it * nev);
    if (rc == VOX_OK) {
        const hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess) rc = hip_fail(e);
    }
    if (rc == VOX_OK) {
        double acc[VOX_NUM_STAGES] = {0};
        double tot = 0;
        for (int it = 0; it < iters && rc == VOX_OK; ++it) {
            hipEvent_t* e = ev + (size_t)it * nev;
            for (int s = 0; s < VOX_NUM_STAGES; ++s) {
                float ms = 0;
                if (pl.fb && s == 1) continue;  // the first-index route has no rank kernel
                const hipError_t he = hipEventElapsedTime(&ms, e[2 * s], e[2 * s + 1]);
                if (he != hipSuccess) {
                    rc = hip_fail(he);
                    break;
                }
                acc[s] += ms;
            }
            float ms = 0;
            if (hipEventElapsedTime(&ms, e[0], e[nev - 1]) == hipSuccess) tot += ms;
        }
        for (int s = 0; s < VOX_NUM_STAGES; ++s) stage_ms[s] = (float)(acc[s] / iters);
        *total_ms = (float)(tot / iters);
    }
    for (int k = 0; k < created; ++k) (void)hipEventDestroy(ev[k]);
    delete[] ev;
    return rc;
}

const char* vox_stage_name(int32_t stage) {
    static const char* names[VOX_NUM_STAGES] = {"insert", "rank", "select", "pack"};
    if (stage < 0 || stage >= VOX_NUM_STAGES) return "unknown";
    return names[stage];
}

const char* vox_strerror(int32_t code) {
    switch (code) {
        case VOX_OK: return "ok";
        case VOX_EINVAL: return "invalid argument";
        case VOX_EWORKSPACE: return "workspace too small or not 256-byte aligned";
        case VOX_EHIP: return "HIP runtime error (see vox_last_hip_error)";
        case VOX_ESCRATCH:
            return "the call needs more scratch than voxelize_static's array holds";
        case VOX_STATUS_NEEDS_CHUNKED:
            return "cap not decidable in one pass: repeat with voxelize_chunked";
        case VOX_STATUS_DEVICE_ERROR: return "internal device bound exceeded";
        case SPH_STATUS_BAD_TABLE: return "boundary table does not match the call's parameters";
        default: return "unknown error";
    }
}

int32_t vox_last_hip_error(void) { return g_last_hip_error; }

int voxelize_static(const float* points, int64_t n_points, const float range[6],
                    const float cell[3], const int32_t grid[3], int32_t max_points,
                    int32_t max_voxels, float* voxels, int32_t* coords, int32_t* num_points,
                    int32_t* num_voxels, hipStream_t stream) {
    Grid g;
    Plan pl;
    // argument checks first: nothing touches the GPU on an argument error
    // (the array's address stands in for the workspace pointer)
    int rc = check_args(points, n_points, range, cell, grid, voxels, coords, num_points,
                        num_voxels, static_cast<void*>(&g), &g);
    if (rc != VOX_OK) return rc;
    if ((rc = make_plan(n_points, max_voxels, max_points, nullptr, &pl)) != VOX_OK) return rc;
    if (pl.bytes > kStaticScratchBytes) return VOX_ESCRATCH;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return VOX_EINVAL;
    std::lock_guard<std::mutex> lk(g_static_mu);
    StaticScratch& st = g_static[dev];
    if (!st.p) {
        // set-up, once per device: the array's device address, and the
        // whole array cleared (a kernel on the call's stream, no memset)
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        st.p = p;
        st.all_dirty = true;
    }
    if (st.all_dirty) {
        if ((rc = launch_zero(st.p, 0, kStaticScratchBytes, stream)) != VOX_OK) return rc;
        st.all_dirty = false;
        st.dlo = st.dhi = 0;
    } else if (pl.zero_bytes > st.dlo && st.dhi > st.dlo) {
        const size_t hi = pl.zero_bytes < st.dhi ? pl.zero_bytes : st.dhi;
        if ((rc = launch_zero(st.p, st.dlo, hi, stream)) != VOX_OK) {
            st.all_dirty = true;
            return rc;
        }
    }
    const Buffers bf = carve(st.p, pl, g);
    rc = run_pipeline(points, g, pl, bf, voxels, coords, num_points, num_voxels, nullptr, stream,
                      nullptr);
    if (rc != VOX_OK) {
        st.all_dirty = true;  // some kernels may have run without the last one
        return rc;
    }
    if (st.dhi < pl.bytes) st.dhi = pl.bytes;
    st.dlo = pl.zero_bytes;
    return VOX_OK;
}

}  // extern "C"
