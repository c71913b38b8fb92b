// The grouped FFN's tile plan: from the per-expert row offsets, the m-tile
// prefix of every group and one 16-byte descriptor per output tile of each
// projection (the persistent GEMM's work list). Shared by the FFN stage and
// the dispatch permute, which runs it in a whole-layer forward so that the
// plan costs no launch of its own.
#pragma once

#include "moe_device.h"

namespace moe {

// Where a plan goes when the dispatch permute writes it (plan == nullptr: it
// does not): its first nblk work-groups do the plan's work, beside the
// permute's, so that the plan costs no launch of its own.
struct FfnPlanArgs {
    int32_t* plan;      // m-tile prefix [E+S+1]
    int4* tiles;        // tile descriptors of both projections
    int32_t* counters;  // tile counters and m-tile counts
    int bm, n_up, ntn_up, ntn_down, nblk, S;
};

// plan[g] = number of m-tiles of groups before g (g = 0..E+S); routed group g
// has ceil(n_g / bm) m-tiles and each shared group ceil(T / bm).
//
// With `tiles` set (the persistent kernels) it also writes one descriptor per
// tile (m-tile x n-tile) for each projection and clears their tile counters:
//   tiles[0 .. n_up)            up-projection: the S shared groups' tiles,
//                               then the routed full m-tiles' group by group,
//                               then the routed half m-tiles';
//   tiles[n_up .. n_up+n_down)  down-projection: the shared tiles (one group
//                               over the S concatenated hidden blocks, if
//                               S > 0), then the routed ones, in the same
//                               order;
// sized for the bound on routed m-tiles. Within a group the tiles go in
// supertiles (swz_tile). Every block computes the prefix sums; block 0
// writes plan[] and the counters, and the blocks share out the tiles.
// Words after the 16 tile counters: routed half and full m-tile counts.
constexpr int kTileMetaHalf = 16, kTileMetaFull = 17;

// Tiles go in supertiles of kSwzM x kSwzN within a group: n-blocks of kSwzN
// n-tiles, within those m-blocks of kSwzM m-tiles, within a supertile
// n-major. Tiles that follow each other in the list then share operand
// panels (an m-tile's token rows, an n-tile's weight rows), so work-groups
// that take them at about the same time find the panels in L2.
constexpr int kSwzM = 4, kSwzN = 4;
// tile j of an M x N grid in that order -> (m, nt)
__device__ __forceinline__ void swz_tile(int M, int N, int j, int& m, int& nt) {
    const int nb = j / (kSwzN * M);
    const int w = min(kSwzN, N - nb * kSwzN);
    const int r = j - nb * kSwzN * M;
    const int mb = r / (kSwzM * w);
    const int hgt = min(kSwzM, M - mb * kSwzM);
    const int rr = r - mb * kSwzM * w;
    nt = nb * kSwzN + rr / hgt;
    m = mb * kSwzM + rr % hgt;
}

// out[0..n] = exclusive prefix sums of in[0..n) (out[n] = the total), by
// one wave: each lane sums a run of consecutive entries, the runs' sums are
// scanned across lanes. in and out may be the same LDS array.
__device__ __forceinline__ void wave_exclusive_scan(const int* in, int* out, int n) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) / 64, b = min(n, lane * per), e = min(n, b + per);
    int run = 0;
    for (int i = b; i < e; ++i) run += in[i];
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    int acc = incl - run;
    for (int i = b; i < e; ++i) {
        const int v = in[i];
        out[i] = acc;
        acc += v;
    }
    if (lane == 63) out[n] = incl;
}

// the last g in [0, n) with key[g] <= v (key non-decreasing, key[0] <= v)
__device__ __forceinline__ int last_le(const int* key, int n, int v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (key[mid] <= v) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The plan of one launch, computed by work-group `blk` of `nblk` (any
// block size of at least three waves): every work-group redoes the prefix
// sums, work-group 0 writes plan[] and the counters, and the work-groups
// share out the tile descriptors. Run by the FFN's plan kernel, or by the
// first work-groups of the dispatch permute in a whole-layer forward.
__device__ __forceinline__ void ffn_plan_block(const int32_t* __restrict__ offsets, int E, int S,
                                               int64_t T, int bm, int32_t* __restrict__ plan,
                                               int4* __restrict__ tiles, int n_up, int ntn_up,
                                               int ntn_down, int32_t* __restrict__ counters,
                                               int blk, int nblk) {
    __shared__ int off_s[kMaxE + 1];
    __shared__ int mt[kMaxE + kMaxS];
    __shared__ int pre[kMaxE + kMaxS + 1];
    __shared__ int fpre[kMaxE + 1], hpre[kMaxE + 1];
    const int G = E + S;
    for (int g = threadIdx.x; g <= E; g += blockDim.x) off_s[g] = offsets[g];
    __syncthreads();
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const int64_t n = g < E ? static_cast<int64_t>(off_s[g + 1] - off_s[g]) : T;
        mt[g] = static_cast<int>((n + bm - 1) / bm);
    }
    // a routed group's last m-tile holding at most bm/2 rows is a half
    // tile; the persistent kernels schedule those after all full tiles
    for (int g = threadIdx.x; g < E; g += blockDim.x) {
        const int n = off_s[g + 1] - off_s[g];
        hpre[g] = mt[g] > 0 && n - (mt[g] - 1) * bm <= bm / 2 ? 1 : 0;
        fpre[g] = mt[g] - hpre[g];
    }
    __syncthreads();
    // exclusive prefix sums, one wave each
    const int wave = threadIdx.x >> 6;
    if (wave == 0) wave_exclusive_scan(mt, pre, G);
    if (wave == 1) wave_exclusive_scan(fpre, fpre, E);
    if (wave == 2) wave_exclusive_scan(hpre, hpre, E);
    __syncthreads();
    if (blk == 0) {
        for (int g = threadIdx.x; g <= G; g += blockDim.x) plan[g] = pre[g];
        if (tiles != nullptr) {
            if (threadIdx.x == 0) {
                counters[kTileMetaHalf] = hpre[E];
                counters[kTileMetaFull] = fpre[E];
            }
            if (threadIdx.x < 16) counters[threadIdx.x] = 0;
        }
    }
    if (tiles == nullptr) return;
    const int mtT = static_cast<int>((T + bm - 1) / bm);
    const int nT = static_cast<int>(T);
    const int nfull = fpre[E], nhalf = hpre[E];
    // one projection's list: the shared groups, the routed full m-tiles
    // group by group, then the routed half m-tiles; every thread takes
    // tiles in turn and finds its group by binary search
    auto write_list = [&](int4* list, int ntn, bool down) {
        const int nsg = down ? (S > 0 ? 1 : 0) : S;  // shared groups in this list
        const int nsh = nsg * mtT * ntn;
        const int i0 = blk * blockDim.x + threadIdx.x, stride = nblk * blockDim.x;
        for (int i = i0; i < nsh; i += stride) {
            const int q = i / (mtT * ntn);
            int m, nt;
            swz_tile(mtT, ntn, i - q * mtT * ntn, m, nt);
            list[i] = make_int4((E + q) | (nt << 16), m * bm, 0, nT);
        }
        int4* routed = list + nsh;
        for (int i = i0; i < nfull * ntn; i += stride) {
            const int g = last_le(fpre, E, i / ntn);
            const int j = i - fpre[g] * ntn;
            int m, nt;
            swz_tile(fpre[g + 1] - fpre[g], ntn, j, m, nt);
            routed[i] = make_int4(g | (nt << 16), m * bm, off_s[g], off_s[g + 1] - off_s[g]);
        }
        for (int i = i0; i < nhalf * ntn; i += stride) {
            const int g = last_le(hpre, E, i / ntn);
            const int nt = i - hpre[g] * ntn;
            routed[nfull * ntn + i] =
                make_int4(g | (nt << 16), (mt[g] - 1) * bm, off_s[g], off_s[g + 1] - off_s[g]);
        }
    };
    write_list(tiles, ntn_up, false);
    write_list(tiles + n_up, ntn_down, true);
}

}  // namespace moe
