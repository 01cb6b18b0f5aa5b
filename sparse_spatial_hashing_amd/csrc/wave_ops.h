// Wavefront and block primitives shared by the library's kernels (gfx950,
// 64-lane wavefronts). Device code only.
#ifndef SSH_WAVE_OPS_H
#define SSH_WAVE_OPS_H

#include <hip/hip_runtime.h>

constexpr int kWave = 64;

__device__ __forceinline__ unsigned long long load_relaxed(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long wave_sum64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Inclusive prefix sum over the wavefront with DPP moves (no LDS path):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in
// from outside the row add 0), then the last lane of row 0 into row 1 and
// of row 2 into row 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31). GFX9 DPP; every lane of the wavefront must be active
// (the block scans below are called by every thread).
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v, int /*lane*/) {
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Inclusive prefix sum within each row of 16 lanes (the first four steps
// of wave_incl_scan). Every lane of the wavefront must be active.
__device__ __forceinline__ unsigned row16_incl_scan(unsigned v) {
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    return v;
}

// LDS words the block scans below need (wsum): the wavefronts' totals of up
// to four sums (row i of 16 words each) in [0, 64), their exclusive prefixes
// in [64, 128), the block totals in [128, 132).
constexpr int kWsumWords = 132;

// NV exclusive prefix sums over the block at once (NW <= 16 wavefronts,
// NV <= 4): ex[i] gets value i's prefix, tot[i] its block total. Wavefront 0
// scans the wavefront totals, sum i in its row i of 16 lanes, and every
// wavefront reads its own prefixes. Contains two barriers; wsum may be
// reused by the next scan right away.
template <int NW, int NV>
__device__ __forceinline__ void block_excl_scan_n(const unsigned (&v)[NV], unsigned* wsum,
                                                  unsigned (&ex)[NV], unsigned (&tot)[NV]) {
    static_assert(NW >= 1 && NW <= 16, "one row of 16 lanes scans the wavefront totals");
    static_assert(NV >= 1 && NV <= 4, "one row of wavefront 0 per sum");
    int lane = __lane_id();
    // an empty asm that "changes" the lane id: the LDS addresses derived
    // from it are then computed here, not hoisted out of a caller's loop to
    // be held (or spilled) across it
    asm volatile("" : "+v"(lane));
    const int w = threadIdx.x / kWave;
    unsigned incl[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) incl[i] = wave_incl_scan(v[i], lane);
    if (lane == kWave - 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i) wsum[16 * i + w] = incl[i];
    }
    __syncthreads();
    if (w == 0) {
        const bool in = lane < 16 * NV && (lane & 15) < NW;
        const unsigned x = in ? wsum[lane] : 0u;
        const unsigned xi = row16_incl_scan(x);
        if (in) wsum[64 + lane] = xi - x;
        if ((lane & 15) == 15 && lane < 16 * NV) wsum[128 + (lane >> 4)] = xi;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        tot[i] = wsum[128 + i];
        ex[i] = wsum[64 + 16 * i + w] + incl[i] - v[i];
    }
}

// Exclusive prefix sum over the block; *total gets the sum. Two barriers.
template <int NW>
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* wsum, unsigned* total) {
    const unsigned vv[1] = {v};
    unsigned ex[1], tot[1];
    block_excl_scan_n<NW, 1>(vv, wsum, ex, tot);
    *total = tot[0];
    return ex[0];
}

// Two exclusive prefix sums over the block at once (a and b); totals in *ta
// and *tb, b's prefix in *eb, a's returned. Two barriers.
template <int NW>
__device__ __forceinline__ unsigned block_excl_scan2(unsigned a, unsigned b, unsigned* wsum,
                                                     unsigned* ta, unsigned* eb, unsigned* tb) {
    const unsigned vv[2] = {a, b};
    unsigned ex[2], tot[2];
    block_excl_scan_n<NW, 2>(vv, wsum, ex, tot);
    *ta = tot[0];
    *tb = tot[1];
    *eb = ex[1];
    return ex[0];
}

// Block bid of a grid of n blocks -> tile: XCD x = bid % 8 takes the
// contiguous tiles [x q + min(x, r), ...) with q = n / 8, r = n % 8 (a
// bijection onto [0, n)).
__device__ __forceinline__ long long xcd_tile(long long bid, long long n) {
    const long long q = n / 8, r = n % 8;
    const long long x = bid % 8, y = bid / 8;
    return x * q + (x < r ? x : r) + y;
}

// Lanes of the wavefront whose value v (nbits low bits) equals this lane's,
// among the lanes with `valid` set: one ballot per bit. Every lane calls it.
__device__ __forceinline__ unsigned long long match_mask(unsigned v, bool valid, int nbits) {
    const unsigned long long m0 = __ballot(valid);
    unsigned lo = (unsigned)m0, hi = (unsigned)(m0 >> 32);
    for (int b = 0; b < nbits; ++b) {
        const unsigned s = (unsigned)__builtin_amdgcn_sbfe((int)v, b, 1);  // bit b, as 0 or all ones
        const unsigned long long bb = __ballot(s != 0u);  // m already excludes invalid lanes
        // keep the lanes whose bit b equals this lane's: m & ~(bb ^ s), one
        // three-input bit operation per half (truth table 0x90 over m, bb, s)
        lo = __builtin_amdgcn_bitop3_b32(lo, (unsigned)bb, s, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (unsigned)(bb >> 32), s, 0x90);
    }
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
    return (1ull << lane) - 1ull;
}
__device__ __forceinline__ unsigned long long lanes_above(int lane) {
    return ~((2ull << lane) - 1ull);  // lane 63: 2 << 63 wraps to 0, mask 0
}

#endif  // SSH_WAVE_OPS_H
