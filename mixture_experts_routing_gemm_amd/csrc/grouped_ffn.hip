// Grouped SwiGLU expert FFN on the matrix cores (bf16) and a float32 variant.
//
// The expert stage of the DeepEP notes (zzszmyf.github.io), section 7: after
// dispatch every row of an expert's contiguous block goes through that expert's
// FFN, with no communication. Routed experts are the E groups of x_perm rows
// given by offsets; the shared experts ("DeepSeek 中 MoE 的同步税", wmrh.cn,
// section 2.1) are extra groups over all T tokens of x. Each expert is a
// SwiGLU FFN, y = W2 (silu(W1 v) * (W3 v)).
//
// Two launches: the up-projection computes a = W1 v and b = W3 v for the same
// output columns in one tile and writes H = bf16(silu(a) * b); the
// down-projection writes Y = bf16(H W2^T). The shared experts' down
// projections are ONE GEMM whose K runs over the S hidden blocks in turn, so
// their outputs are summed in float32 before the single rounding.
//
// Tiles are scheduled on the device from offsets (no host round trip): a plan
// kernel turns the per-expert row counts into an m-tile prefix, and every
// work-group maps its index to (group, m-tile, n-tile); the grid is sized for
// the worst case and surplus work-groups exit at once. Work-group indices are
// remapped so that each of the 8 XCDs walks a contiguous range of tiles, which
// keeps an expert's weights and rows within one XCD's L2 as far as possible.
#include <algorithm>
#include <type_traits>

#include "ffn_plan.h"
#include "lds_ring.h"
#include "moe_device.h"

namespace moe {

// kModeUp / kModeDown: bf16 operands; kModeUpFp8: fp8 token rows converted to
// bf16 in LDS; kModeUpF8W / kModeDownF8W: fp8 token (or hidden) rows and fp8
// weights on the fp8 matrix cores, the scales applied in the epilogue.
// For the backward (persistent kernel only): kModeUpSave / kModeUpFp8Save are
// kModeUp / kModeUpFp8 that also store the pre-activations a and b;
// kModeDh computes dhid = dy W2 (K = d, from the transposed W2, one weight
// row per output column) with the SwiGLU backward in its epilogue.
enum {
    kModeUp = 0, kModeUpFp8 = 1, kModeDown = 2, kModeUpF8W = 3, kModeDownF8W = 4,
    kModeUpSave = 5, kModeUpFp8Save = 6, kModeDh = 7
};
constexpr bool is_down(int m) { return m == kModeDown || m == kModeDownF8W; }
constexpr bool is_fp8rows(int m) { return m == kModeUpFp8 || m == kModeUpFp8Save; }
constexpr bool is_save(int m) { return m == kModeUpSave || m == kModeUpFp8Save; }
constexpr bool is_f8w(int m) { return m == kModeUpF8W || m == kModeDownF8W; }
// bf16 operands in both roles: the upper row of waves (0-3) issues every
// buffer -> LDS request of a slice, its own and those of its SIMD's partner
// in the lower row (wave + 4), so that one wave of each SIMD never stalls
// on a request while HBM misses fill the CU's queue (C4 down-projection
// 1384 -> 1295 us, up-projection -1 %). The fp8 modes keep one request set
// per wave (fp8 rows: each wave converts the codes it requested).
constexpr bool pairs_issue(int m) { return !is_fp8rows(m) && !is_f8w(m); }

constexpr int kBM = 128, kBN = 128, kBK = 64;  // bf16 tile: rows x B rows x K
constexpr int kFfnThreads = 256;
constexpr int kLdsStage = (kBM + kBN) * kBK * 2;  // bytes per pipeline stage
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

__global__ __launch_bounds__(256) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                       int E, int S, int64_t T, int bm,
                                                       int32_t* __restrict__ plan,
                                                       int4* __restrict__ tiles, int n_up,
                                                       int ntn_up, int ntn_down,
                                                       int32_t* __restrict__ counters) {
    ffn_plan_block(offsets, E, S, T, bm, plan, tiles, n_up, ntn_up, ntn_down, counters,
                   blockIdx.x, gridDim.x);
}

struct GemmArgs {
    const uint8_t* a_routed;  // routed A rows: x_perm (bf16 or fp8 codes) or H_r
    // bf16 up-projection of the persistent kernel: when set, routed row r is
    // token a_gather[r] of a_shared (x) and a_routed is not read, so the
    // permuted rows never have to be written out
    const int32_t* a_gather;
    const float* qparams;     // fp8 rows: [rows, 2] = (scale, centre)
    const uint8_t* a_shared;  // shared A rows: x [T, d] (up) or H_s [T, S*h] (down)
    const int32_t* offsets;   // [E+1]
    const int32_t* plan;      // [E+S+1]
    const int4* tiles;        // m-tile descriptors of this projection (persistent kernel)
    int32_t* counters;        // tile counters of the persistent kernel ([0]: the pool's), zeroed by the plan
    const int32_t* tile_meta; // [routed half m-tiles, routed full m-tiles] (persistent kernel)
    const uint8_t* wa;        // up: W1 [G, h, d]; down: W2 [G, d, h]
    const uint8_t* wb;        // up: W3 [G, h, d]
    uint8_t* out_routed;      // up: H_r [T*k, h]; down: Y_perm [T*k, d]
    uint8_t* out_shared;      // up: H_s [T, S*h]; down: y_sh [T, d]
    // up-projection that also keeps its pre-activations (the backward's
    // recomputation): a = W1 v and b = W3 v in bf16, laid out as H
    uint8_t* pre_a_routed;
    uint8_t* pre_b_routed;
    uint8_t* pre_a_shared;
    uint8_t* pre_b_shared;
    // fp8-weight modes: (scale, centre) of the shared experts' token rows
    // [T, 2]; the weight scales s1 | qsum1 | s3 | qsum3 [G, h] | s2 [G, d];
    // the hidden rows' scales, routed [rows] and shared [T]
    const float* q_shared;
    const float* wscale;
    const float* hsc_r;
    const float* hsc_s;
    int64_t T;
    int E, S, d, h;
    int hs;   // row stride of one group's hidden block in H_r / H_s (h rounded up to 8)
    int ntn;  // n-tiles per group
    // operand sizes in bytes (the persistent kernel reads through buffer
    // resources of these sizes; each is below 4 GiB there)
    uint32_t a_routed_bytes, a_shared_bytes, w_bytes;
};

// Finds the group and m-tile of m-tile index mtg. Down-projection: the S
// shared experts form ONE group (index E). Returns false past the last tile.
template <int MODE>
__device__ __forceinline__ bool locate_tile(const GemmArgs& a, int mtg, int bm, int& g, int& mloc,
                                            int64_t& row_base, int& nrows) {
    const int routed_tiles = a.plan[a.E];
    const int mtT = static_cast<int>((a.T + bm - 1) / bm);
    if (mtg >= routed_tiles) {
        const int q = mtg - routed_tiles;
        const int nshared = MODE == kModeDown ? (a.S > 0 ? 1 : 0) : a.S;
        if (q >= nshared * mtT) return false;
        g = a.E + q / mtT;
        mloc = q % mtT;
        row_base = 0;
        nrows = static_cast<int>(a.T);
        return true;
    }
    int lo = 0, hi = a.E - 1;  // largest g with plan[g] <= mtg
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.plan[mid] <= mtg)
            lo = mid;
        else
            hi = mid - 1;
    }
    g = lo;
    mloc = mtg - a.plan[g];
    row_base = a.offsets[g];
    nrows = a.offsets[g + 1] - a.offsets[g];
    return true;
}

// byte offset of 16-byte chunk c of row r in a [rows][64] bf16 LDS tile. The
// XOR swizzle spreads the 16-byte reads of 8 (or 16) consecutive rows over
// distinct banks for a 32-bank (or 64-bank) LDS.
__device__ __forceinline__ int lds_off(int r, int c) {
    return (r << 7) + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// silu(v) = v / (1 + e^-v), with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// 8 e4m3 codes -> 8 bf16 values of code*scale + centre (one 16-byte chunk)
__device__ __forceinline__ uint32_t dequant2(float lo, float hi, float scale, float centre) {
    return pack_bf16x2(__builtin_fmaf(lo, scale, centre), __builtin_fmaf(hi, scale, centre));
}
__device__ __forceinline__ u32x4 dequant8(uint2 codes, float scale, float centre) {
    u32x4 out;
    // v_cvt_pk_f32_fp8: codes 0,1 (false) or 2,3 (true) of a word
    const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), false);
    const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), true);
    const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), false);
    const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), true);
    out[0] = dequant2(p0[0], p0[1], scale, centre);
    out[1] = dequant2(p1[0], p1[1], scale, centre);
    out[2] = dequant2(p2[0], p2[1], scale, centre);
    out[3] = dequant2(p3[0], p3[1], scale, centre);
    return out;
}

// Register-staged 128 x 128 tile kernel for the shapes the persistent kernel
// does not take: any d % 8 == 0 and any h. Operands move as 16-byte chunks of
// 8 values. The hidden rows H are stored with their blocks padded to hs = h
// rounded up to 8 (the padding columns hold zeros, written by the
// up-projection from zero weight rows), so in the down-projection K runs
// over whole chunks of hs; a chunk is either wholly inside K or wholly past
// it. Chunks past K, and weight rows past N, are read as zeros, and outputs
// past N are not stored. W2 rows have h values each: when h is not a
// multiple of 8 their chunks are not 16-byte aligned and are read value by
// value, up to h. In the shared down-projection K runs over the S hidden
// blocks in turn, so each chunk finds its own block.
template <int MODE, bool SAVE = false>
__global__ __launch_bounds__(kFfnThreads, 2) void ffn_gemm_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int L = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int mtg = L / a.ntn;
    const int nt = L - mtg * a.ntn;
    int g, mloc, nrows;
    int64_t row_base;
    if (!locate_tile<MODE>(a, mtg, kBM, g, mloc, row_base, nrows)) return;
    const int m0 = mloc * kBM;
    const bool shared = g >= a.E;

    // operand geometry
    const int K = MODE == kModeDown ? (shared ? a.S * a.hs : a.hs) : a.d;
    const int N = MODE == kModeDown ? a.d : a.h;  // output features of the group
    const int lda = K;  // elements (codes for fp8) per A row
    const int tid = threadIdx.x;
    const int c = tid & 7;     // 16-byte chunk within a 64-wide K slice
    const int rr = tid >> 3;   // first of this thread's 4 rows (rr + 32*i)

    const uint8_t* arow[4];
    float qs[4], qc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + rr + 32 * i;
        arow[i] = nullptr;
        qs[i] = 0.0f;
        qc[i] = 0.0f;
        if (r < nrows) {
            const int64_t row = row_base + r;
            if (MODE == kModeUpFp8 && !shared) {
                arow[i] = a.a_routed + row * lda;
                qs[i] = a.qparams[2 * row];
                qc[i] = a.qparams[2 * row + 1];
            } else {
                const uint8_t* base = shared ? a.a_shared : a.a_routed;
                arow[i] = base + row * lda * 2;
            }
        }
    }
    // B rows of this thread (weight rows = output features); NULL past N
    const uint8_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int br = rr + 32 * i;  // 0..127 within the B tile
        if (MODE == kModeDown) {
            const int n = nt * kBN + br;
            // shared: the hidden block of each chunk is added in load_tile
            brow[i] = n < N ? a.wa + (static_cast<int64_t>(shared ? a.E : g) * a.d + n) * a.h * 2
                            : nullptr;
        } else {
            const int q = br >> 6, within = br & 63;
            const int n = nt * (kBN / 2) + q * 32 + (within & 31);
            const uint8_t* w = (within < 32) ? a.wa : a.wb;
            brow[i] = n < N ? w + (static_cast<int64_t>(g) * a.h + n) * a.d * 2 : nullptr;
        }
    }

    const bool fp8_rows = MODE == kModeUpFp8 && !shared;
    u32x4 ra[4], rb[4];
    auto load_tile = [&](int k0) {
        const int kk = k0 + c * 8;  // this thread's chunk
        const bool kin = kk < K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (arow[i] == nullptr || !kin) {
                ra[i] = u32x4{0u, 0u, 0u, 0u};
            } else if (fp8_rows) {
                const uint2 codes = *reinterpret_cast<const uint2*>(arow[i] + kk);
                ra[i] = dequant8(codes, qs[i], qc[i]);
            } else {
                ra[i] = load16(arow[i] + static_cast<int64_t>(kk) * 2);
            }
        }
        if (MODE == kModeDown) {
            // the shared expert whose hidden block holds the chunk (0: routed)
            const int seg = kk / a.hs;
            const int local = kk - seg * a.hs;  // position within that block
            const int64_t boff = static_cast<int64_t>(seg) * a.d * a.h * 2 + static_cast<int64_t>(local) * 2;
            const int nval = a.h - local;  // values of the W2 row left from `local`
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (brow[i] == nullptr || !kin || nval <= 0) {
                    rb[i] = u32x4{0u, 0u, 0u, 0u};
                } else if ((a.h & 7) == 0) {
                    rb[i] = load16(brow[i] + boff);
                } else {
                    const uint16_t* p = reinterpret_cast<const uint16_t*>(brow[i] + boff);
                    uint32_t w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = 2 * q < nval ? p[2 * q] : 0u;
                        const uint32_t hi = 2 * q + 1 < nval ? p[2 * q + 1] : 0u;
                        w[q] = lo | (hi << 16);
                    }
                    rb[i] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rb[i] = (brow[i] == nullptr || !kin) ? u32x4{0u, 0u, 0u, 0u}
                                                     : load16(brow[i] + static_cast<int64_t>(kk) * 2);
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t* As = lds + buf * kLdsStage;
        uint8_t* Bs = As + kBM * kBK * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rr + 32 * i;
            *reinterpret_cast<u32x4*>(As + lds_off(r, c)) = ra[i];
            *reinterpret_cast<u32x4*>(Bs + lds_off(r, c)) = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lg = lane >> 5;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int KT = (K + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load_tile((kt + 1) * kBK);
        const uint8_t* As = lds + (kt & 1) * kLdsStage;
        const uint8_t* Bs = As + kBM * kBK * 2;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int ch = ks * 2 + lg;
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int r = wm * 64 + mb * 32 + lr;
                af[mb] = *reinterpret_cast<const bf16x8*>(As + lds_off(r, ch));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int r = wn * 64 + nb * 32 + lr;
                bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(r, ch));
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < KT) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane holds column lr of each 32x32 block and rows
    // 8*(v/4) + 4*lg + v%4
    if (MODE == kModeDown) {
        bf16_t* out = reinterpret_cast<bf16_t*>(shared ? a.out_shared : a.out_routed);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (r < nrows) {
                    const int64_t row = row_base + r;
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const int col = nt * kBN + wn * 64 + nb * 32 + lr;
                        if (col < N) out[row * a.d + col] = f32_to_bf16(acc[mb][nb][v]);
                    }
                }
            }
    } else {
        bf16_t* out = reinterpret_cast<bf16_t*>(shared ? a.out_shared : a.out_routed);
        bf16_t* pa = reinterpret_cast<bf16_t*>(shared ? a.pre_a_shared : a.pre_a_routed);
        bf16_t* pb = reinterpret_cast<bf16_t*>(shared ? a.pre_b_shared : a.pre_b_routed);
        const int ldo = shared ? a.S * a.hs : a.hs;
        const int cloc = nt * (kBN / 2) + wn * 32 + lr;  // hidden feature within the group
        const int col = (shared ? (g - a.E) * a.hs : 0) + cloc;
        // columns h..hs-1 are padding: zero weight rows give silu(0) * 0 = 0
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (r < nrows && cloc < a.hs) {
                    const int64_t row = row_base + r;
                    const float hv = silu(acc[mb][0][v]) * acc[mb][1][v];
                    out[row * ldo + col] = f32_to_bf16(hv);
                    if constexpr (SAVE) {
                        pa[row * ldo + col] = f32_to_bf16(acc[mb][0][v]);
                        pb[row * ldo + col] = f32_to_bf16(acc[mb][1][v]);
                    }
                }
            }
    }
}

// ------------------------------------------------------ large-tile bf16 --
// Persistent grouped GEMM: one 512-thread work-group per CU walks a list of
// 256 x 256 output tiles (tokens x weight rows), K sliced by 32. Eight waves
// (two per SIMD, so one's memory requests overlap the other's MFMAs) each own
// a 128 x 64 block, a 4 x 2 grid of 32x32x16 bf16 MFMAs.
//  - Both operand slices go global -> LDS with the direct-to-LDS 16-byte loads
//    into a 4-slot ring; each slice is requested three steps before it is
//    read, and the waits count outstanding loads instead of draining them.
//  - LDS fragments of the next 16-wide half-slice are read while the current
//    one's MFMAs run.
//  - The ring runs across tiles: the next tile's first slices are in flight
//    while the current tile's epilogue runs, and no work-group is launched
//    per tile.
//  - Each XCD works through one contiguous range of tiles (tile order: m-tile
//    major, n-tile minor), so concurrent work-groups on an XCD share an
//    expert's weights and rows in that XCD's L2.
// The weights are the MFMA's first operand: each lane's accumulator holds
// four consecutive output features of one token, stored as one 8-byte word.
// fp8 token rows stay as codes in LDS and are dequantised as fragments are
// read.
// (A 128 x 256 tile with three slots and two work-groups per CU measured
// slower on both projections.)
constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 32, kBigSlots = 4;
constexpr int kBigWM = 128, kBigWN = 64;  // eight waves: 2 (M) x 4 (N)
constexpr int kBigMB = kBigWM / 32, kBigNB = kBigWN / 32;
constexpr int kBigABytes = 2 * kBigBM * kBigBK;  // bf16 token rows (fp8 rows use half)
constexpr int kBigBBytes = 2 * kBigBN * kBigBK;
constexpr int kBigSlot = kBigABytes + kBigBBytes;
// vector-memory instructions per wave per slice (fp8 slices are padded to it)
constexpr int kBigLoads = 4;  // per wave per slice: 2 token-row and 2 weight-row requests

// A ring slot holds the token rows (A) and weight rows (B) of one K slice in
// blocks of 64 rows: block q of A at byte 8192*q, block q of B at 8192*q +
// 4096. Wave w fills half of block w/2 of both: two 1 KB requests each.
//
// byte offset of 16-byte chunk c (0..3) of bf16 row r (32 values); the XOR
// swizzle makes 16-byte reads of aligned runs of 8 rows (32 banks) or 16 rows
// (64 banks) conflict-free
__device__ __forceinline__ int lds_off32(int r, int c) {
    return ((r >> 6) << 13) + ((r & 63) << 6) + ((c ^ (((r >> 1) & 3) ^ ((r >> 3) & 1))) << 4);
}
// fp8 token rows: wave w's request lands the codes of rows 32w..32w+31 (32 B
// each, plain order) in the upper half of the 2 KB those rows take as bf16,
// so that the wave can convert them in place.
__device__ __forceinline__ int fp8_codes_off(int wave) {
    return (wave >> 1) * 8192 + (wave & 1) * 2048 + 1024;
}

// Converts the 16 codes `w` this lane's request brought into `slot` (row
// 32*wave + lane/2, K offsets 16*(lane&1)..+15, read from fp8_codes_off) to
// bf16 code*scale + centre and writes them where the bf16 fragment reads
// expect that row. The wave has read all its codes before it writes (a
// wave's LDS accesses complete in order), so the in-place overwrite is safe;
// no other wave touches these bytes until the next barrier.
__device__ __forceinline__ void convert_codes(uint8_t* slot, int wave, int lane, u32x4 w,
                                              float scale, float centre) {
    const u32x4 lo = dequant8(uint2{w[0], w[1]}, scale, centre);
    const u32x4 hi = dequant8(uint2{w[2], w[3]}, scale, centre);
    const int r = wave * 32 + (lane >> 1), ch = 2 * (lane & 1);
    *reinterpret_cast<bf16x8*>(slot + lds_off32(r, ch)) = __builtin_bit_cast(bf16x8, lo);
    *reinterpret_cast<bf16x8*>(slot + lds_off32(r, ch + 1)) = __builtin_bit_cast(bf16x8, hi);
}

// a 16-byte store to global memory (the operands of the kernels are global:
// a generic pointer would make it a flat store, which also counts in lgkmcnt)
__device__ __forceinline__ void store16g(void* p, u32x4 v) {
    *(__attribute__((address_space(1))) u32x4*)(p) = v;
}

// (The flags are ints: a struct with bool members was copied through
// scratch memory at every tile, and the wait for that scratch load drained
// the prefetched slices.)
struct TileInfo {
    int g, nt, m0, row_base, nrows, KT;
    int shared;
    int half;  // at most kBigBM/2 valid rows: the lower row of waves idles
};

// What one lane needs to fetch slices of one tile: 32-bit byte offsets of
// its token rows within the A operand and of its weight rows within the
// tile's weight group (the launcher keeps every operand under 4 GiB for this
// kernel), and the wave-uniform byte offset of that group within W1/W2 (and
// W3). In the up-projection the weight rows of a wave's DMA requests come
// from W1 for even waves and from W3 for odd ones.
struct TileSrc {
    const uint8_t* abuf;  // token operand of the tile (wave-uniform)
    uint32_t abytes;      // its size in bytes
    uint32_t gofs;
    int shared;
    uint32_t aoff[2];   // token rows of this lane's DMA chunks
    uint32_t boff[2];   // weight rows of this lane's DMA chunks
    uint32_t paoff[2];  // the same for the partner wave (pairs_issue modes)
    uint32_t pboff[2];
    float cs, cc;      // fp8 rows: (scale, centre) of the row this lane converts
};

// a 16-byte load from a wave-uniform address, through the scalar unit
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 load_uniform(const int4* p) {
    return *(const __attribute__((address_space(4))) i32x4*)(p);
}

// Tile L of a projection's list (a descriptor written by the plan kernel;
// the first nsh * ntn tiles are the shared experts').
template <int MODE>
__device__ __forceinline__ TileInfo decode_tile(const GemmArgs& a, int L, int nsh) {
    TileInfo ti;
    const i32x4 t = load_uniform(a.tiles + L);
    ti.g = t[0] & 0xffff;
    ti.nt = t[0] >> 16;
    ti.m0 = t[1];
    ti.row_base = t[2];
    ti.nrows = t[3];
    ti.shared = L < nsh * a.ntn;
    ti.half = ti.nrows - ti.m0 <= kBigBM / 2;
    const int K = is_down(MODE) ? (ti.shared ? a.S * a.h : a.h) : a.d;
    ti.KT = K / (is_f8w(MODE) ? 2 * kBigBK : kBigBK);  // fp8: 64 values per 64-byte slice
    return ti;
}

// the bf16 up-projection may read its routed rows straight from x
template <int MODE>
constexpr bool can_gather() { return MODE == kModeUp; }

// Tokens of the rows that this lane's requests (q = 0, 1) and its partner's
// (q = 2, 3) fetch for a routed tile, numbered as tile_sources numbers them,
// when the rows are gathered from x.
template <int MODE>
__device__ __forceinline__ void gather_tokens(const GemmArgs& a, const TileInfo& ti, int wave,
                                              int lane, int (&tok)[4]) {
    const int last = ti.nrows - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int wv = q < 2 ? wave : (wave & 3) + 4;
        const int r = wv * 32 + (q & 1) * 16 + (lane >> 2);
        tok[q] = a.a_gather[ti.row_base + min(ti.m0 + r, last)];
    }
}

template <int MODE>
__device__ __forceinline__ void tile_sources(const GemmArgs& a, const TileInfo& ti, int wave,
                                             int lane, const uint8_t* op_ar, const uint8_t* op_as,
                                             uint32_t by_ar, uint32_t by_as, bool gather,
                                             const int (&tok)[4], TileSrc& src) {
    // routed rows gathered from x by token
    const bool gat = can_gather<MODE>() && gather && !ti.shared;
    // chosen here, by value, once per tile: a choice between two captured
    // locals inside the request code became a load through a chosen
    // address from a private copy
    src.abuf = uniform_ptr(ti.shared || gat ? op_as : op_ar);
    src.abytes = __builtin_amdgcn_readfirstlane(ti.shared || gat ? by_as : by_ar);
    const bool fp8 = is_fp8rows(MODE) && !ti.shared;
    const int K = is_down(MODE) ? (ti.shared ? a.S * a.h : a.h) : a.d;
    const uint32_t eb = is_f8w(MODE) ? 1 : 2;  // bytes per operand value
    const int last = ti.nrows - 1;
    src.shared = ti.shared;
    // token DMA: a wave instruction fills 1 KB of LDS, lane i at byte 16*i:
    // 16 bf16 rows of 64 B (row = wave*32 + i*16 + lane/4), each lane
    // fetching the chunk the swizzle places at its position, or the codes of
    // 32 fp8 rows of 32 B in plain order (row = wave*32 + lane/2, half
    // lane&1), which the same lane converts to bf16 later. Rows past the
    // group's end re-read its last row; their outputs are never stored.
    auto token_rows = [&](int wv, uint32_t* out, int q0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (gat) {
                const int r = wv * 32 + i * 16 + (lane >> 2);
                const int c = (lane & 3) ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
                out[i] = static_cast<uint32_t>(tok[q0 + i]) * static_cast<uint32_t>(K) * eb + c * 16;
            } else if (fp8) {
                const int r = wv * 32 + (lane >> 1);
                const int64_t row = ti.row_base + min(ti.m0 + r, last);
                out[i] = static_cast<uint32_t>(row * K + (lane & 1) * 16);
            } else {
                const int r = wv * 32 + i * 16 + (lane >> 2);
                const int c = (lane & 3) ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
                const int64_t row = ti.row_base + min(ti.m0 + r, last);
                out[i] = static_cast<uint32_t>(row * K * eb + c * 16);
            }
        }
    };
    token_rows(wave, src.aoff, 0);
    // (written in every mode: fields left unwritten made the copy of the
    // sources at a tile boundary go through scratch memory, and its wait
    // drained the prefetched slices)
    src.paoff[0] = src.paoff[1] = src.pboff[0] = src.pboff[1] = 0u;
    if constexpr (pairs_issue(MODE)) token_rows((wave & 3) + 4, src.paoff, 2);
    src.cs = 0.0f;
    src.cc = 0.0f;
    if (fp8) {
        const int64_t row = ti.row_base + min(ti.m0 + wave * 32 + (lane >> 1), last);
        const float2 q = *reinterpret_cast<const float2*>(a.qparams + 2 * row);
        src.cs = q.x;
        src.cc = q.y;
    }
    src.gofs = static_cast<uint32_t>(is_down(MODE) && ti.shared ? a.E : ti.g) * a.d * a.h * eb;
    auto weight_rows = [&](int wv, uint32_t* out) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int br = wv * 32 + i * 16 + (lane >> 2);
            const int c = (lane & 3) ^ (((br >> 1) & 3) ^ ((br >> 3) & 1));
            if (is_down(MODE)) {
                const int n = ti.nt * kBigBN + br;
                out[i] = static_cast<uint32_t>(n) * a.h * eb + c * 16;
            } else if (MODE == kModeDh) {
                // the transposed W2 [G, h, d]: weight row n is hidden feature n
                // (rows past h, in a last partial n-tile, are read and unused)
                const int n = ti.nt * kBigBN + br;
                out[i] = static_cast<uint32_t>(n) * a.d * eb + c * 16;
            } else {
                // weight row br of the tile: 32-row blocks alternate W1 / W3
                const int n = ti.nt * (kBigBN / 2) + ((br >> 5) >> 1) * 32 + (br & 31);
                out[i] = static_cast<uint32_t>(n) * a.d * eb + c * 16;
            }
        }
    };
    weight_rows(wave, src.boff);
    if constexpr (pairs_issue(MODE)) weight_rows((wave & 3) + 4, src.pboff);
}

template <int MODE>
__device__ __forceinline__ void persistent_gemm(const GemmArgs& a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int* lds_next = reinterpret_cast<int*>(lds + kBigSlots * kBigSlot);
    constexpr int MB = kBigMB, NB = kBigNB;
    constexpr bool kFp8 = is_fp8rows(MODE);
    constexpr bool kF8W = is_f8w(MODE);
    constexpr bool kDown = is_down(MODE);
    // Tile claims. A work-group takes its XCD's claims round-robin (claim c
    // goes to work-group c mod per_xcd) for all but the last tenth of the
    // XCD's list; those tiles form the XCD's pool segment. A work-group whose
    // own claims are done draws from its XCD's segment first (one atomic
    // counter per segment), then from the other XCDs' in turn (the
    // fp8-weight modes have no pool).
    //  - Round-robin: the n-tiles that share a token panel start together on
    //    neighbouring work-groups and, with equal work, stay in step, so the
    //    panel's slices are still in L2 when the siblings ask for them. With
    //    claims from a per-XCD counter the siblings drifted about a tenth of
    //    a tile apart, more than the few steps of traffic that L2 holds: the
    //    up-projection's L2 misses were 12 % higher.
    //  - Pool: the XCDs run at different speeds, and the up-projection's
    //    long tiles split 16 or 17 per work-group; with round-robin claims
    //    alone the work-groups sat idle 5 % of the kernel at its end. The
    //    pool cut the up-projection by 2.8 % and the down-projection by 3 %
    //    on the 65536-token workload, the fp8-row up-projection by 4 %.
    //    Drawing from any segment in one order cost 18 % more L2 misses in
    //    the up-projection (4.25 against 5.0 GB on that workload) for the
    //    same time: the stolen tiles' panels are in another XCD's L2.
    constexpr int KS = kF8W ? 2 * kBigBK : kBigBK;  // operand values per slice
    constexpr uint32_t EB = kF8W ? 1 : 2;          // bytes per operand value
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wn = wave & 3, wm = wave >> 2;
    const int lr = lane & 31, lg = lane >> 5;
    // operand bases and sizes as wave-uniform values, chosen by value below
    // (a choice between two fields of the argument struct can otherwise
    // become a load through a chosen address, from a private copy)
    const uint8_t* const op_ar = uniform_ptr(a.a_routed);
    const uint8_t* const op_as = uniform_ptr(a.a_shared);
    const uint32_t by_ar = __builtin_amdgcn_readfirstlane(a.a_routed_bytes);
    const uint32_t by_as = __builtin_amdgcn_readfirstlane(a.a_shared_bytes);
    const uint32_t by_w = __builtin_amdgcn_readfirstlane(a.w_bytes);
    // up-projection: a wave's weight rows lie in one 32-row block, W1 for
    // even waves and W3 for odd ones
    const uint8_t* const op_w = uniform_ptr(!kDown && (wave & 1) ? a.wb : a.wa);
    bf16_t* const out_r = reinterpret_cast<bf16_t*>(const_cast<uint8_t*>(uniform_ptr(a.out_routed)));
    bf16_t* const out_s = reinterpret_cast<bf16_t*>(const_cast<uint8_t*>(uniform_ptr(a.out_shared)));

    // The tile list: the shared m-tiles first (in the down-projection each
    // runs over S hidden blocks, S times the work of a routed tile), then the
    // routed full m-tiles, then the routed half m-tiles; n-tile minor. XCD x
    // (work-groups b with b % 8 == x) owns the full tiles whose work starts
    // in the x-th eighth of the full part, then the x-th eighth of the half
    // tiles, so the XCDs get equal work, each keeps its experts' weights in
    // its own L2, and the short tiles come last. Claims: see above.
    const int routed = a.plan[a.E];
    const int n_half = a.tile_meta[0];
    const int mtT = static_cast<int>((a.T + kBigBM - 1) / kBigBM);
    const int nsh = kDown ? (a.S > 0 ? mtT : 0) : a.S * mtT;
    const int64_t wsh = kDown ? max(a.S, 1) : 1;
    const int n_sh = nsh * a.ntn;
    const int n_full = n_sh + (routed - n_half) * a.ntn;  // tiles before the half ones
    const int n_halft = n_half * a.ntn;
    const int64_t sh_work = n_sh * wsh;
    const int64_t work = sh_work + (n_full - n_sh);
    auto tile_at = [&](int64_t w) -> int {  // first tile whose work starts at or after w
        return w <= sh_work ? static_cast<int>((w + wsh - 1) / wsh)
                            : n_sh + static_cast<int>(w - sh_work);
    };
    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int flo = tile_at(work * xcd / 8), fhi = tile_at(work * (xcd + 1) / 8);
    const int hlo = n_full + n_halft * xcd / 8, hhi = n_full + n_halft * (xcd + 1) / 8;
    const int nclaim = (fhi - flo) + (hhi - hlo);  // tiles of this XCD
    auto tile_of_x = [&](int c) -> int { return c < fhi - flo ? flo + c : hlo + (c - (fhi - flo)); };
    // Claim codes: [0, nstatic) this XCD's round-robin claims, then
    // nstatic + y q + j for claim j of XCD y's segment (its last q claims).
    int nstatic = nclaim, npool = 0;
    auto ranges = [&](int y, int& f0, int& f1, int& h0, int& h1) {
        f0 = tile_at(work * y / 8);
        f1 = tile_at(work * (y + 1) / 8);
        h0 = n_full + n_halft * y / 8;
        h1 = n_full + n_halft * (y + 1) / 8;
    };
    {
        int nmin = nclaim;
        for (int y = 0; y < 8; ++y) {
            int f0, f1, h0, h1;
            ranges(y, f0, f1, h0, h1);
            nmin = min(nmin, (f1 - f0) + (h1 - h0));
        }
        // (none for the fp8-weight modes: at their register limit, the pool's
        // bookkeeping spilled registers that every tile then reloaded)
        const int q = is_f8w(MODE) ? 0 : (nmin / 10) & ~3;
        nstatic = nclaim - q;
        npool = 8 * q;
    }
    const int kNone = nstatic + npool;
    auto tile_of = [&](int code) -> int {
        if (code < nstatic) return tile_of_x(code);
        const int pidx = code - nstatic, q = npool / 8;
        const int y = pidx / q, j = pidx - y * q;  // segment y: XCD y's last q claims
        int f0, f1, h0, h1;
        ranges(y, f0, f1, h0, h1);
        const int c = (f1 - f0) + (h1 - h0) - q + j;
        return c < f1 - f0 ? f0 + c : h0 + (c - (f1 - f0));
    };
    // this work-group's next claim (thread 0): its own claims C,
    // C + per_xcd, ... below nstatic, then pool indices (the count of its
    // claims is kept in LDS, not in a register the whole kernel long)
    auto claim_next = [&]() -> int {
        const int jc = lds_next[2];
        lds_next[2] = jc + 1;
        const int c = static_cast<int>(blockIdx.x >> 3) + jc * per_xcd;
        if (c < nstatic) return c;
        // the pool: this XCD's segment first (its panels are in this L2),
        // then the other XCDs' in turn; lds_next[3] skips segments found empty
        const int q = npool / 8;
        if (q == 0) return kNone;
        for (int t = lds_next[3]; t < 8; ++t) {
            const int y = (xcd + t) & 7;
            const int j = atomicAdd(a.counters + y, 1);
            if (j < q) return nstatic + y * q + j;
            lds_next[3] = t + 1;
        }
        return kNone;
    };
    int C, Cn;  // claim codes of the current and the next tile
    if (tid == 0) {
        lds_next[2] = 0;
        lds_next[3] = 0;
        lds_next[0] = claim_next();
        lds_next[1] = claim_next();
    }
    __syncthreads();
    C = __builtin_amdgcn_readfirstlane(lds_next[0]);
    Cn = __builtin_amdgcn_readfirstlane(lds_next[1]);
    if (C >= kNone) return;

    TileInfo cur = decode_tile<MODE>(a, tile_of(C), nsh);
    // the next tile's descriptor: a scalar load, issued a tile ahead (for
    // later tiles during the previous epilogue), so that its latency -- the
    // descriptors were written by another kernel, often on another XCD --
    // is not exposed by the wait at the top of the tile
    TileInfo pre = cur;
    if (Cn < kNone) pre = decode_tile<MODE>(a, tile_of(Cn), nsh);
    // Rows gathered from x: the tokens of this tile's rows and of the next
    // one's. Later tiles' tokens are loaded at the end of the epilogue two
    // tiles ahead, so the drain there covers them and no wait on them falls
    // inside the K loop or at the top of a tile.
    const bool gather = can_gather<MODE>() && a.a_gather != nullptr;
    int tok[4] = {0, 0, 0, 0}, ptok[4] = {0, 0, 0, 0};
    if (gather && !cur.shared) gather_tokens<MODE>(a, cur, wave, lane, tok);
    if (gather && Cn < kNone && !pre.shared) gather_tokens<MODE>(a, pre, wave, lane, ptok);
    TileSrc src;
    tile_sources<MODE>(a, cur, wave, lane, op_ar, op_as, by_ar, by_as, gather, tok, src);
    if (gather) wait_vmcnt<0>();
    TileInfo nxt = cur;
    TileSrc nsrc = src;
    // the claim on the tile after next; later ones are issued at the end of
    // each epilogue, whose drain of the stores also waits for the claim
    int claim = 0;
    if (Cn < kNone && tid == 0) claim = claim_next();

    // Requests of slice k of a tile into ring slot `slot`: kBigLoads
    // buffer-to-LDS instructions per wave, issued one at a time (i). Wave w
    // fills block w of A (LDS base `abase`) and of B (`bbase`); request i
    // lands at its base + 1024*(i % 4).
    struct SliceReq {
        uint32_t ka;     // byte offset of the slice within a token row
        uint32_t kb;     // byte offset of the slice's weight columns, group included
        uint8_t* abase;
        uint8_t* bbase;
    };
    auto slice_req = [&](const TileSrc& ts, bool shared, int k, int slot) {
        SliceReq q;
        const int k0 = k * KS;
        q.abase = lds + slot * kBigSlot +
                  (kFp8 && !shared ? fp8_codes_off(wave) : (wave >> 1) * 8192 + (wave & 1) * 2048);
        q.bbase = lds + slot * kBigSlot + (wave >> 1) * 8192 + 4096 + (wave & 1) * 2048;
        q.ka = static_cast<uint32_t>(kFp8 && !shared ? k0 : k0 * EB);
        uint32_t kb = static_cast<uint32_t>(k0) * EB;
        if (kDown) {
            // the shared group's K runs over the S hidden blocks in turn:
            // slice k0 lies in block seg (always 0 for a routed group)
            int seg = 0;
#pragma unroll
            for (int s = 1; s < kMaxS; ++s) seg += k0 >= s * a.h ? 1 : 0;
            kb = static_cast<uint32_t>(k0 - seg * a.h) * EB + static_cast<uint32_t>(seg) * a.d * a.h * EB;
        }
        q.kb = __builtin_amdgcn_readfirstlane(ts.gofs + kb);
        q.ka = __builtin_amdgcn_readfirstlane(q.ka);
        return q;
    };
    // request i of a slice: rows at a0/a1 (token) and b0/b1 (weight), LDS
    // blocks at abase/bbase (the offsets passed by value: a choice between
    // two fields of the tile's sources would go through a private copy)
    auto issue_one = [&](const TileSrc& ts, bool shared, const SliceReq& q, auto I, uint32_t a0, uint32_t a1,
                         uint32_t b0, uint32_t b1, uint8_t* abase, uint8_t* bbase) {
        constexpr int i = decltype(I)::value;
        // every operand of a buffer resource must be wave-uniform (the
        // compiler cannot prove it for a tile read back from LDS, and would
        // otherwise loop over lanes and drain the outstanding requests)
        const uint8_t* abuf = ts.abuf;
        const uint32_t abytes = ts.abytes;
        const uint8_t* wbuf = op_w;
        if constexpr (i < 2) {
            if (kFp8 && !shared) {
                // fp8 rows take one request; the other rewrites weight rows
                if constexpr (i == 0)
                    buffer_to_lds16<0>(abuf, abytes, a0, q.ka, abase);
                else
                    buffer_to_lds16<0>(wbuf, by_w, b0, q.kb, bbase);
            } else {
                buffer_to_lds16<1024 * i>(abuf, abytes, i == 0 ? a0 : a1, q.ka, abase);
            }
        } else {
            buffer_to_lds16<1024 * (i - 2)>(wbuf, by_w, i == 2 ? b0 : b1, q.kb, bbase);
        }
    };
    // request i of a slice: on the pairs_issue modes the upper row of waves
    // issues its own and its partner's (whose blocks lie 16 KB further in
    // the slot), the lower row nothing
    auto issue_req = [&](const TileSrc& ts, bool shared, const SliceReq& q, auto I) {
        if constexpr (pairs_issue(MODE)) {
            if (wave < 4) {
                issue_one(ts, shared, q, I, ts.aoff[0], ts.aoff[1], ts.boff[0], ts.boff[1], q.abase, q.bbase);
                issue_one(ts, shared, q, I, ts.paoff[0], ts.paoff[1], ts.pboff[0], ts.pboff[1],
                          q.abase + 16384, q.bbase + 16384);
            }
        } else {
            issue_one(ts, shared, q, I, ts.aoff[0], ts.aoff[1], ts.boff[0], ts.boff[1], q.abase, q.bbase);
        }
    };
    // requests outstanding per slice on an issuing wave
    constexpr int kReqs = (pairs_issue(MODE) ? 2 : 1) * kBigLoads;
    auto issue = [&](const TileSrc& ts, bool shared, int k, int slot) {
        const SliceReq q = slice_req(ts, shared, k, slot);
        issue_req(ts, shared, q, ic<0>());
        issue_req(ts, shared, q, ic<1>());
        issue_req(ts, shared, q, ic<2>());
        issue_req(ts, shared, q, ic<3>());
    };
    // LDS -> register fragment i (B fragments 0..NB-1, then A fragments) of
    // 16-wide half-slice ks of a slot
    auto read_frag = [&](int slot, int ks, bf16x8* fa, bf16x8* fb, const TileSrc& ts, bool shared, int i) {
        const uint8_t* As = lds + slot * kBigSlot;
        const uint8_t* Bs = As + 4096;
        const int ch = ks * 2 + lg;
        if (i < NB) {
            fb[i] = *reinterpret_cast<const bf16x8*>(Bs + lds_off32(wn * kBigWN + i * 32 + lr, ch));
        } else {
            const int mb = i - NB;
            const int r = wm * kBigWM + mb * 32 + lr;
            fa[mb] = *reinterpret_cast<const bf16x8*>(As + lds_off32(r, ch));
        }
    };
    auto load_frags = [&](int slot, int ks, bf16x8* fa, bf16x8* fb, const TileSrc& ts, bool shared) {
#pragma unroll
        for (int i = 0; i < MB + NB; ++i) read_frag(slot, ks, fa, fb, ts, shared, i);
    };

    f32x16 acc[MB][NB];
    auto mma_one = [&](const bf16x8* fa, const bf16x8* fb, int i) {
        const int mb = i / NB, nb = i % NB;
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb], acc[mb][nb], 0, 0, 0);
    };
    // fp8-weight modes: one 32x32x64 e4m3 MFMA per (mb, nb) and slice. A
    // lane's 32-byte fragment of row r holds the slice's K values 16*lg ..
    // 16*lg+15 and 32+16*lg .. 32+16*lg+15 (chunks lg and 2+lg), the same
    // positions for the weight and the token operand, so every K value of
    // the slice meets its partner once.
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    i32x8 fa8[MB], fb8[NB];
    auto read_frag8 = [&](int slot, bool isb, int r, i32x8& out) {
        const uint8_t* base = lds + slot * kBigSlot + (isb ? 4096 : 0);
        const u32x4 lo = __builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(base + lds_off32(r, lg)));
        const u32x4 hi = __builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(base + lds_off32(r, 2 + lg)));
        out = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                    static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                    static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    };
    auto rfa8 = [&](int slot, int mb) { read_frag8(slot, false, wm * kBigWM + mb * 32 + lr, fa8[mb]); };
    auto rfb8 = [&](int slot, int nb) { read_frag8(slot, true, wn * kBigWN + nb * 32 + lr, fb8[nb]); };
    auto mma8 = [&](int mb, int nb) {
        // operand formats 0 / 0: e4m3 for both; scales 127: 2^0
        acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[nb], fa8[mb], acc[mb][nb], 0, 0,
                                                                       0, 127, 0, 127);
    };

    // prologue: the first tile's slices 0..2; fp8 rows of slice 0 are
    // converted once this wave's request for them has landed (the barrier at
    // the top of the tile loop publishes them)
    issue(src, cur.shared, 0, 0);
    issue(src, cur.shared, 1, 1);
    issue(src, cur.shared, 2, 2);
    if (kFp8 && !cur.shared) {
        wait_vmcnt<2 * kBigLoads>();
        const u32x4 c0 = __builtin_bit_cast(
            u32x4, *reinterpret_cast<const bf16x8*>(lds + fp8_codes_off(wave) + 16 * lane));
        convert_codes(lds, wave, lane, c0, src.cs, src.cc);
    }

    bf16x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
    while (true) {
        const bool has_next = Cn < kNone;
        // the claim on the tile after the next one is already in `claim` and
        // goes out to the other waves before the last four slices. After the
        // last tile the "next" tile is this one again: its first slices are
        // re-read into free slots and never used, which keeps the last steps
        // the same for every tile.
        if (has_next) nxt = pre;

        wait_vmcnt<2 * kReqs>();  // slice 0 of this tile has landed
        ring_barrier();
        if (has_next) {
            tile_sources<MODE>(a, nxt, wave, lane, op_ar, op_as, by_ar, by_as, gather, ptok, nsrc);
        } else {
            nxt = cur;
            nsrc = src;
        }
        if constexpr (kF8W) {
            // slice 0: both weight fragments and the first two token ones
            rfb8(0, 0);
            rfb8(0, 1);
            rfa8(0, 0);
            rfa8(0, 1);
        } else {
            load_frags(0, 0, fa0, fb0, src, cur.shared);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        const int KT = cur.KT;
        // One step computes slice k from ring slot J = k % 4 and requests
        // slice k+3 into slot (J+3) % 4: from this tile (ISS 1) or, in the
        // last three steps, from the next tile (ISS 2). Before its second
        // half it waits until at most WN requested slices are still in
        // flight (WN < 0: the tile's last step, nothing left to wait for).
        // An IDLE wave (the lower row of waves on a half tile) keeps the
        // requests, waits and barriers but does no MFMAs or fragment reads.
        auto step = [&](auto J, auto ISS, auto WN, auto IDLE, int k) {
            constexpr int j = decltype(J)::value, iss = decltype(ISS)::value;
            constexpr int wn_ = decltype(WN)::value;
            constexpr bool idle = decltype(IDLE)::value;
            // first half: MFMAs on half-slice 0 (fa0, fb0), each followed by
            // one request of slice k+3 and one fragment read of half-slice 1
            const TileSrc& ts = iss == 2 ? nsrc : src;
            const bool tsh = iss == 2 ? nxt.shared : cur.shared;
            const SliceReq q = slice_req(ts, tsh, iss == 2 ? k + 3 - KT : k + 3, (j + 3) & 3);
            if constexpr (kF8W) {
                // first half: MFMAs of token blocks 0, 1 on slice k, each
                // with one request of slice k+3; the fragments of token
                // blocks 2, 3 of slice k are read meanwhile
                static_for<0, 4>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    if constexpr (!idle) mma8(i & 1, i >> 1);
                    if constexpr (iss != 0) issue_req(ts, tsh, q, I);
                    if constexpr (!idle && i < 2) rfa8(j, 2 + i);
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (wn_ >= 0) {
                    // second half: slice k+1 must have landed; token blocks
                    // 2, 3 on slice k, each MFMA followed by a read of the
                    // next slice's fragment its predecessors no longer need
                    wait_vmcnt<wn_ * kBigLoads>();
                    ring_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (!idle) {
                        constexpr int nj = (j + 1) & 3;
                        mma8(2, 0);
                        rfa8(nj, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        mma8(3, 0);
                        rfa8(nj, 1);
                        __builtin_amdgcn_sched_barrier(0);
                        mma8(2, 1);
                        rfb8(nj, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        mma8(3, 1);
                        rfb8(nj, 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else if constexpr (!idle) {
                    mma8(2, 0);
                    mma8(3, 0);
                    mma8(2, 1);
                    mma8(3, 1);
                }
                return;
            }
            // fp8 rows: this wave converts its rows of slice k+1 (the next
            // tile's slice 0 in a tile's last step), every wave alike, idle
            // or not. Its codes request was the first of the eight issued
            // in the last two steps, so at most seven may still be in flight.
            const bool conv = kFp8 && !(wn_ < 0 ? nxt.shared : cur.shared);
            const TileSrc& cts = wn_ < 0 ? nsrc : src;
            uint8_t* const cslot = lds + ((j + 1) & 3) * kBigSlot;
            u32x4 codes;
            static_for<0, MB * NB>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (kFp8 && i == 0) {
                    if (conv) {
                        wait_vmcnt<2 * kBigLoads - 1>();
                        codes = __builtin_bit_cast(
                            u32x4, *reinterpret_cast<const bf16x8*>(cslot + fp8_codes_off(wave) + 16 * lane));
                    }
                }
                if constexpr (!idle) mma_one(fa0, fb0, i);
                if constexpr (iss != 0 && i < kBigLoads) issue_req(ts, tsh, q, I);
                if constexpr (!idle && i < MB + NB) read_frag(j, 1, fa1, fb1, src, cur.shared, i);
                if constexpr (kFp8 && i == 2) {
                    if (conv) convert_codes(cslot, wave, lane, codes, cts.cs, cts.cc);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (wn_ >= 0) {
                // second half: the next slice must have landed (at most WN
                // requested slices still in flight) and be visible to all
                // waves; its first fragments are read between the MFMAs on
                // half-slice 1
                wait_vmcnt<wn_ * kReqs>();
                ring_barrier();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!idle) {
#pragma unroll
                    for (int i = 0; i < MB * NB; ++i) {
                        mma_one(fa1, fb1, i);
                        if (i < MB + NB) read_frag((j + 1) & 3, 0, fa0, fb0, src, cur.shared, i);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else if constexpr (!idle) {
#pragma unroll
                for (int i = 0; i < MB * NB; ++i) mma_one(fa1, fb1, i);
            }
        };
        auto k_loop = [&](auto IDLE) {
            int k = 0;
            for (; k < KT - 4; k += 4) {
                step(ic<0>(), ic<1>(), ic<2>(), IDLE, k);
                step(ic<1>(), ic<1>(), ic<2>(), IDLE, k + 1);
                step(ic<2>(), ic<1>(), ic<2>(), IDLE, k + 2);
                step(ic<3>(), ic<1>(), ic<2>(), IDLE, k + 3);
            }
            // the last four slices; the claimed tile index goes out through
            // LDS with the first of these steps' barrier
            if (tid == 0) lds_next[0] = has_next ? claim : kNone;
            step(ic<0>(), ic<1>(), ic<2>(), IDLE, k);
            step(ic<1>(), ic<2>(), ic<2>(), IDLE, k + 1);
            step(ic<2>(), ic<2>(), ic<2>(), IDLE, k + 2);
            step(ic<3>(), ic<2>(), ic<-1>(), IDLE, k + 3);
        };
        if (cur.half && wm == 1)
            k_loop(std::true_type{});
        else
            k_loop(std::false_type{});
        const int Cn2 = __builtin_amdgcn_readfirstlane(lds_next[0]);
        if (has_next && Cn2 < kNone) pre = decode_tile<MODE>(a, tile_of(Cn2), nsh);

        // epilogue: acc[mb][nb][v] is token (m0 + wm*128 + mb*32 + lr) and
        // weight row (wn*64 + nb*32 + 8*(v/4) + 4*lg + v%4) of the tile. A
        // lane packs four bf16 per group q of 8 columns; lanes lr and lr+32
        // hold the two halves of each group (lg). One half-wave swap per
        // pair of groups gives lane lg=0 the 8 columns of group 2p and lane
        // lg=1 those of group 2p+1, so each lane stores 16 contiguous bytes.
        bf16_t* out = cur.shared ? out_s : out_r;
        auto store_groups = [&](bf16_t* rowp, const uint32_t (&w)[4][2], bool ok) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * p][0], w[2 * p + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * p][1], w[2 * p + 1][1], false, false);
                if (ok) store16g(rowp + 16 * p + 8 * lg, u32x4{s0[0], s1[0], s0[1], s1[1]});
            }
        };
        // fp8-weight modes: the weight rows' scales of this lane's 16 output
        // features per 32-row block (4*lg + 8*q + u, u < 4): up-projection
        // s1, qsum1, s3, qsum3 of hidden features fb + ...; down-projection
        // s2 of output features (per block nb)
        f32x4 wsc[4][4];
        if constexpr (kF8W) {
            const int64_t G = a.E + a.S, H = a.h;
            if constexpr (kDown) {
                const float* s2 = a.wscale + 4 * G * H + static_cast<int64_t>(cur.shared ? a.E : cur.g) * a.d +
                                  cur.nt * kBigBN + wn * kBigWN + 4 * lg;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        wsc[nb][q] = *reinterpret_cast<const f32x4*>(s2 + nb * 32 + 8 * q);
            } else {
                const float* sc = a.wscale + static_cast<int64_t>(cur.g) * H + cur.nt * (kBigBN / 2) +
                                  wn * (kBigWN / 2) + 4 * lg;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        wsc[t][q] = *reinterpret_cast<const f32x4*>(sc + t * G * H + 8 * q);
            }
        }
        // Down-projections stage their output through the ring slot of the
        // tile's last slice (slot 3: the next tile's first slices go to slots
        // 0..2), so that each store writes 8 rows x 128 contiguous bytes
        // rather than 32 rows x 32 bytes: rows of d values lie d*2 bytes apart,
        // and the narrow pattern measured 2.9 TB/s against 5.4 for the wide
        // one in a store-only kernel. Every wave must be done reading that
        // slot first; each then uses its own 4 KB of it, a 32-row block at a
        // time (128 bytes a row, 16-byte chunks at position c ^ ((row / 2) % 8)).
        // (The fp8-weight down-projection stores directly: its epilogue holds
        // the weight scales as well and has no registers to spare.)
        constexpr bool kStage = MODE == kModeDown;
        uint8_t* stage = nullptr;
        // staged stores go through a buffer resource over the group's rows,
        // so rows past the group fall outside it and are dropped by the
        // range check (no branch per store); lane L stores 16 bytes of row
        // L / 8 of each 8-row group, chunk L % 8 of the wave's 128 bytes.
        // The rows are written once and read once, by combine: the stores
        // are non-temporal (aux 2), so they do not evict operand panels.
        const uint32_t orow = static_cast<uint32_t>(a.d) * 2;
        // (wave-uniform by construction; said so, or the compiler loops over
        // lanes around every store)
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(uniform_ptr(reinterpret_cast<const uint8_t*>(out + static_cast<int64_t>(cur.row_base) * a.d))), 0,
            static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(cur.nrows) * orow)), kBufferFlags);
        const uint32_t obase = static_cast<uint32_t>(cur.m0 + wm * kBigWM + (lane >> 3)) * orow +
                               static_cast<uint32_t>(cur.nt * kBigBN + wn * kBigWN + (lane & 7) * 8) * 2;
        // dh: the recomputed a and b of the lane's 4 x 8 values of each
        // 32-row block, loaded as a batch (one round trip per block)
        uint2 dh_ab[1][NB][4][2];
        auto dh_load = [&](int mbi, int buf) {
            const int rr = cur.m0 + wm * kBigWM + mbi * 32 + lr;
            const int sg = cur.shared ? cur.g - a.E : 0;
            const int lpre = cur.shared ? a.S * a.h : a.h;
            const int64_t prow = static_cast<int64_t>(cur.row_base) + min(rr, cur.nrows - 1);
            const bf16_t* pa = reinterpret_cast<const bf16_t*>(cur.shared ? a.pre_a_shared : a.pre_a_routed) +
                               prow * lpre + sg * a.h;
            const bf16_t* pb = reinterpret_cast<const bf16_t*>(cur.shared ? a.pre_b_shared : a.pre_b_routed) +
                               prow * lpre + sg * a.h;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int col = cur.nt * kBigBN + wn * kBigWN + nb * 32;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int f = col + 8 * q + 4 * lg;
                    dh_ab[buf][nb][q][0] = col < a.h ? *reinterpret_cast<const uint2*>(pa + f) : uint2{0u, 0u};
                    dh_ab[buf][nb][q][1] = col < a.h ? *reinterpret_cast<const uint2*>(pb + f) : uint2{0u, 0u};
                }
            }
        };
        if constexpr (MODE == kModeDh) dh_load(0, 0);
        if constexpr (kStage) {
            ring_barrier();
            stage = lds + 3 * kBigSlot + wave * 4096;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int r = cur.m0 + wm * kBigWM + mb * 32 + lr;
            const bool ok = r < cur.nrows;  // the same for lanes lr and lr+32
            const int64_t row = static_cast<int64_t>(cur.row_base) + r;
            // fp8-weight modes: this token row's scale (and centre)
            float ts = 1.0f, tc = 0.0f;
            if constexpr (kF8W) {
                const int rc = min(r, cur.nrows - 1);
                if constexpr (kDown) {
                    ts = cur.shared ? a.hsc_s[rc] : a.hsc_r[cur.row_base + rc];
                } else {
                    const float2 q2 = cur.shared
                                          ? *reinterpret_cast<const float2*>(a.q_shared + 2 * static_cast<int64_t>(rc))
                                          : *reinterpret_cast<const float2*>(a.qparams + 2 * (static_cast<int64_t>(cur.row_base) + rc));
                    ts = q2.x;
                    tc = q2.y;
                }
            }
            if constexpr (kDown) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    uint32_t w[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            v[u] = kF8W ? ts * (wsc[nb][q][u] * acc[mb][nb][4 * q + u]) : acc[mb][nb][4 * q + u];
                        w[q][0] = pack_bf16x2(v[0], v[1]);
                        w[q][1] = pack_bf16x2(v[2], v[3]);
                    }
                    if constexpr (!kStage) {
                        store_groups(out + row * a.d + cur.nt * kBigBN + wn * kBigWN + nb * 32, w, ok);
                        continue;
                    }
                    // the half-wave swap of store_groups, then the 16 bytes
                    // of columns nb*32 + 16 p + 8 lg (chunk nb*4 + 2p + lg of
                    // the wave's 128-byte row) go to the staging area
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * p][0], w[2 * p + 1][0], false, false);
                        const auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * p][1], w[2 * p + 1][1], false, false);
                        const int c = nb * 4 + 2 * p + lg;
                        *reinterpret_cast<u32x4*>(stage + lr * 128 + ((c ^ ((lr >> 1) & 7)) << 4)) =
                            u32x4{s0[0], s1[0], s0[1], s1[1]};
                    }
                }
                // four stores of 8 rows x 128 bytes: lane L takes row 8 i + L/8,
                // chunk L % 8
                if constexpr (kStage) {
                    u32x4 v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 8 * i + (lane >> 3), cc = lane & 7;
                        v[i] = *reinterpret_cast<const u32x4*>(stage + rr * 128 + ((cc ^ ((rr >> 1) & 7)) << 4));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v[i], orsrc, obase + static_cast<uint32_t>(mb * 32 + 8 * i) * orow, 0, 2);
                }
            } else if constexpr (MODE == kModeDh) {
                // dhid -> da = dhid b s (1 + a (1 - s)), db = dhid silu(a)
                // (s = sigmoid(a)) from the recomputed a, b; da and db of a
                // group's row side by side: [da | db], 2h values per group
                const int sg = cur.shared ? cur.g - a.E : 0;
                const int lpre = cur.shared ? a.S * a.h : a.h;
                const int lout = 2 * lpre;
                const int cb = 0;
                if (mb > 0) dh_load(mb, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int col = cur.nt * kBigBN + wn * kBigWN + nb * 32;
                    if (col >= a.h) continue;  // a last partial n-tile (h % 256 == 128)
                    uint32_t wa_[4][2], wb_[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint2 av4 = dh_ab[cb][nb][q][0];
                        const uint2 bv4 = dh_ab[cb][nb][q][1];
                        const float av[4] = {bf16_lo(av4.x), bf16_hi(av4.x), bf16_lo(av4.y), bf16_hi(av4.y)};
                        const float bv[4] = {bf16_lo(bv4.x), bf16_hi(bv4.x), bf16_lo(bv4.y), bf16_hi(bv4.y)};
                        float da[4], db[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float dh = acc[mb][nb][4 * q + u];
                            const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-av[u]));
                            da[u] = dh * bv[u] * (sgm * (1.0f + av[u] * (1.0f - sgm)));
                            db[u] = dh * (av[u] * sgm);
                        }
                        wa_[q][0] = pack_bf16x2(da[0], da[1]);
                        wa_[q][1] = pack_bf16x2(da[2], da[3]);
                        wb_[q][0] = pack_bf16x2(db[0], db[1]);
                        wb_[q][1] = pack_bf16x2(db[2], db[3]);
                    }
                    bf16_t* orow = out + row * lout + sg * 2 * a.h + col;
                    store_groups(orow, wa_, ok);
                    store_groups(orow + a.h, wb_, ok);
                }
            } else {
                const int ldo = cur.shared ? a.S * a.h : a.h;
                const int cbase = (cur.shared ? (cur.g - a.E) * a.h : 0) + cur.nt * (kBigBN / 2) +
                                  wn * (kBigWN / 2);
#pragma unroll
                for (int pq = 0; pq < NB / 2; ++pq) {
                    uint32_t w[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float hv[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            float av = acc[mb][2 * pq][4 * q + u], bv = acc[mb][2 * pq + 1][4 * q + u];
                            if constexpr (kF8W) {
                                // sum_i (qx s + c) (qw sw) = sw (s sum qx qw + c sum qw)
                                av = wsc[0][q][u] * __builtin_fmaf(ts, av, tc * wsc[1][q][u]);
                                bv = wsc[2][q][u] * __builtin_fmaf(ts, bv, tc * wsc[3][q][u]);
                            }
                            hv[u] = silu(av) * bv;
                        }
                        w[q][0] = pack_bf16x2(hv[0], hv[1]);
                        w[q][1] = pack_bf16x2(hv[2], hv[3]);
                    }
                    store_groups(out + row * ldo + cbase + pq * 32, w, ok);
                    if constexpr (is_save(MODE)) {
                        // the pre-activations a, b (bf16), laid out as H
                        uint32_t wa_[4][2], wb_[4][2];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            wa_[q][0] = pack_bf16x2(acc[mb][2 * pq][4 * q], acc[mb][2 * pq][4 * q + 1]);
                            wa_[q][1] = pack_bf16x2(acc[mb][2 * pq][4 * q + 2], acc[mb][2 * pq][4 * q + 3]);
                            wb_[q][0] = pack_bf16x2(acc[mb][2 * pq + 1][4 * q], acc[mb][2 * pq + 1][4 * q + 1]);
                            wb_[q][1] = pack_bf16x2(acc[mb][2 * pq + 1][4 * q + 2], acc[mb][2 * pq + 1][4 * q + 3]);
                        }
                        const int64_t at = row * ldo + cbase + pq * 32;
                        store_groups(reinterpret_cast<bf16_t*>(cur.shared ? a.pre_a_shared : a.pre_a_routed) + at, wa_, ok);
                        store_groups(reinterpret_cast<bf16_t*>(cur.shared ? a.pre_b_shared : a.pre_b_routed) + at, wb_, ok);
                    }
                }
            }
        }
        // the tokens of the tile after next (used at the top of the next tile)
        if (gather && has_next && Cn2 < kNone && !pre.shared) gather_tokens<MODE>(a, pre, wave, lane, ptok);
        // the next tile's claim on the one after it
        if (has_next && Cn2 < kNone && tid == 0) claim = claim_next();
        // the epilogue's stores also count in vmcnt: drain before the next
        // tile's counted waits (and, after the last tile, let the re-read
        // slices land before the work-group's LDS is released)
        wait_vmcnt<0>();
        if (!has_next) break;
        Cn = Cn2;
        cur = nxt;
        src = nsrc;
    }
}

// one work-group of eight waves per CU, 256 registers per lane
template <int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ffn_gemm_persistent_kernel(GemmArgs a) {
    persistent_gemm<MODE>(a);
}

// ---------------------------------------------------------------- float32 --
// Plain float32 FFN for act = MOE_F32 (vector FMA; the bf16 matrix cores
// cannot reach float32 accuracy). 64x64 output tiles, 4x4 per thread.
template <bool UP>
__global__ __launch_bounds__(256) void ffn_gemm_f32_kernel(GemmArgs a, int mt_max) {
    __shared__ float As[kF32BK][kF32BM + 4];
    __shared__ float Bs[2][kF32BK][kF32BN + 4];
    const int L = blockIdx.x;
    const int mtg = L / a.ntn;
    const int nt = L - mtg * a.ntn;
    int g, mloc, nrows;
    int64_t row_base;
    if (!locate_tile<UP ? kModeUp : kModeDown>(a, mtg, kF32BM, g, mloc, row_base, nrows)) return;
    const bool shared = g >= a.E;
    const int m0 = mloc * kF32BM;
    const int K = UP ? a.d : (shared ? a.S * a.h : a.h);
    const int N = UP ? a.h : a.d;
    const int n0 = nt * kF32BN;
    const float* A = reinterpret_cast<const float*>(shared ? a.a_shared : a.a_routed);
    const float* W1 = reinterpret_cast<const float*>(a.wa);
    const float* W3 = reinterpret_cast<const float*>(a.wb);
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    float acc[2][4][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[q][i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kF32BK) {
        for (int q = tid; q < kF32BM * kF32BK; q += 256) {
            const int r = q / kF32BK, kk = q % kF32BK;
            const int kg = k0 + kk;
            float v = 0.0f;
            if (m0 + r < nrows && kg < K) v = A[(row_base + m0 + r) * static_cast<int64_t>(K) + kg];
            As[kk][r] = v;
        }
        for (int q = tid; q < kF32BN * kF32BK; q += 256) {
            const int n = q / kF32BK, kk = q % kF32BK;
            const int kg = k0 + kk, ng = n0 + n;
            float v1 = 0.0f, v3 = 0.0f;
            if (ng < N && kg < K) {
                if (UP) {
                    const int64_t off = (static_cast<int64_t>(g) * a.h + ng) * a.d + kg;
                    v1 = W1[off];
                    v3 = W3[off];
                } else {
                    const int gg = shared ? a.E + kg / a.h : g;
                    const int kl = shared ? kg % a.h : kg;
                    v1 = W1[(static_cast<int64_t>(gg) * a.d + ng) * a.h + kl];
                }
            }
            Bs[0][kk][n] = v1;
            Bs[1][kk][n] = v3;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kF32BK; ++kk) {
            float av[4], b1[4], b3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = As[kk][ty * 4 + i];
                b1[i] = Bs[0][kk][tx * 4 + i];
                b3[i] = Bs[1][kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[0][i][j] = __builtin_fmaf(av[i], b1[j], acc[0][i][j]);
                    if (UP) acc[1][i][j] = __builtin_fmaf(av[i], b3[j], acc[1][i][j]);
                }
        }
        __syncthreads();
    }
    float* out = reinterpret_cast<float*>(shared ? a.out_shared : a.out_routed);
    const int ldo = UP ? (shared ? a.S * a.h : a.h) : a.d;
    const int cbase = (UP && shared) ? (g - a.E) * a.h : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + ty * 4 + i;
        if (r >= nrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            const float v = UP ? silu(acc[0][i][j]) * acc[1][i][j] : acc[0][i][j];
            out[(row_base + r) * ldo + cbase + n] = v;
        }
    }
}

// Plan area of the workspace: plan [E+S+1] ints, 16 tile counters (8 per
// projection), then the up- and down-projection tile descriptors of the
// persistent kernels (16 bytes each).
struct PlanLayout {
    size_t counters, tiles, bytes;
    int n_up, n_down;      // tile descriptors of each projection
    int ntn_up, ntn_down;  // n-tiles per group
};

// (ntn_up, ntn_down: n-tiles per group of the two tile lists; the forward's
// are 2h/256 and d/256)
PlanLayout plan_layout(const moe_shape& s, int ntn_up, int ntn_down) {
    PlanLayout p;
    const int64_t mtT = (s.T + kBigBM - 1) / kBigBM;
    const int64_t rmax = s.T * s.k / kBigBM + s.E;  // routed m-tiles, at most
    p.ntn_up = ntn_up;
    p.ntn_down = ntn_down;
    p.n_up = static_cast<int>((s.S * mtT + rmax) * p.ntn_up);
    p.n_down = static_cast<int>((mtT + rmax) * p.ntn_down);
    p.counters = ((static_cast<size_t>(s.E + s.S + 1) * 4 + 63) / 64) * 64;
    p.tiles = p.counters + 128;  // 16 counters, then the m-tile counts
    p.bytes = p.tiles + static_cast<size_t>(p.n_up + p.n_down) * sizeof(int4);
    return p;
}
PlanLayout plan_layout(const moe_shape& s) { return plan_layout(s, 2 * s.h / kBigBN, s.d / kBigBN); }

size_t ffn_plan_bytes(const moe_shape& s) { return plan_layout(s).bytes; }

// values per group block of a hidden row: h, rounded up to 8 for bf16 so that
// every hidden row and block starts on 16 bytes (float32 rows keep h)
int ffn_hidden_stride(const moe_shape& s) { return s.act == MOE_F32 ? s.h : (s.h + 7) & ~7; }

namespace {

// upper bound on the m-tiles of one launch
int64_t max_mtiles(const moe_shape& s, int bm, bool down) {
    const int64_t mtT = (s.T + bm - 1) / bm;
    const int64_t routed = (s.T * s.k) / bm + s.E;
    const int64_t shared = down ? (s.S > 0 ? mtT : 0) : s.S * mtT;
    return routed + shared;
}

}  // namespace

// the persistent kernels need 128 KB of LDS (the 4-slot ring) and a word for
// handing a claimed tile index to the work-group
constexpr int kBigLds = kBigSlots * kBigSlot + 16;
template <int MODE>
hipError_t allow_big_lds() {
    static hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ffn_gemm_persistent_kernel<MODE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kBigLds);
    return err;
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// one work-group per CU (at most one per tile), a multiple of 8 (XCDs)
template <int MODE>
hipError_t launch_persistent(const GemmArgs& a, int64_t mtiles, hipStream_t st) {
    const hipError_t e = allow_big_lds<MODE>();
    if (e != hipSuccess) return e;
    int64_t blocks = std::min<int64_t>(device_cus(), mtiles * a.ntn);
    blocks = (blocks + 7) & ~int64_t(7);
    ffn_gemm_persistent_kernel<MODE><<<static_cast<unsigned>(blocks), 512, kBigLds, st>>>(a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_gemm(const GemmArgs& a, int64_t mtiles, bool big, hipStream_t st) {
    if (big) {
        return launch_persistent<MODE>(a, mtiles, st);
    } else {
        int64_t blocks = mtiles * a.ntn;
        blocks = (blocks + 7) & ~int64_t(7);
        ffn_gemm_kernel<MODE><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
    }
    return hipGetLastError();
}

namespace {
// work-groups of a plan of the persistent kernels: every one redoes the
// prefix sums, the tile lists are shared out
int plan_blocks(const PlanLayout& pl) {
    return static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>(64, (std::max(pl.n_up, pl.n_down) + 255) / 256)));
}

}  // namespace

// large tiles when both projections divide evenly into them (and K into
// whole groups of four slices)
bool use_big_tiles(const moe_shape& s) {
    const uint64_t rows = static_cast<uint64_t>(s.T) * (s.k + s.S);
    const uint64_t wbytes = static_cast<uint64_t>(s.E + s.S) * s.d * s.h * 2;
    const bool fits32 = rows * s.d * 2 < (uint64_t(1) << 32) && rows * s.h * 2 < (uint64_t(1) << 32) &&
                        wbytes < (uint64_t(1) << 32);
    return s.act != MOE_F32 && fits32 && s.h % (kBigBN / 2) == 0 && s.d % kBigBN == 0 &&
           s.d % (4 * kBigBK) == 0 && s.h % (4 * kBigBK) == 0;
}

bool ffn_gathers_rows(const moe_shape& s) {
    return use_big_tiles(s) && s.act == MOE_BF16 && s.dispatch == MOE_BF16;
}

bool ffn_fused_plan(const moe_shape& s, int32_t* plan, FfnPlanArgs* fp) {
    fp->plan = nullptr;
    if (!use_big_tiles(s)) return false;
    const PlanLayout pl = plan_layout(s);
    fp->plan = plan;
    fp->counters = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan) + pl.counters);
    fp->tiles = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + pl.tiles);
    fp->bm = kBigBM;
    fp->n_up = pl.n_up;
    fp->ntn_up = pl.ntn_up;
    fp->ntn_down = pl.ntn_down;
    fp->nblk = plan_blocks(pl);
    fp->S = s.S;
    return true;
}

hipError_t launch_grouped_ffn(const moe_shape& s, const void* x_perm, const float* qparams,
                              const int32_t* offsets, const void* x, const void* w1,
                              const void* w3, const void* w2, void* y_perm, void* y_shared,
                              int32_t* plan, void* h_routed, void* h_shared, bool plan_done,
                              hipStream_t st, const Marks* mk, const int32_t* gather, void* pre_a_r,
                              void* pre_b_r, void* pre_a_s, void* pre_b_s) {
    const bool f32 = s.act == MOE_F32;
    if (gather != nullptr && !ffn_gathers_rows(s)) return hipErrorInvalidValue;
    // with pre_a_r: the up-projection also stores a = W1 v and b = W3 v
    // (the persistent tiles only)
    const bool save = pre_a_r != nullptr;
    if (save && !use_big_tiles(s)) return hipErrorInvalidValue;
    const bool big = use_big_tiles(s);
    const int bm = f32 ? kF32BM : (big ? kBigBM : kBM);
    const PlanLayout pl = plan_layout(s);
    int32_t* counters = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan) + pl.counters);
    int4* tiles = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + pl.tiles);
    // (plan_done: the dispatch permute of a whole-layer forward wrote it)
    if (!plan_done)
        ffn_plan_kernel<<<big ? plan_blocks(pl) : 1, 256, 0, st>>>(
            offsets, s.E, s.S, s.T, bm, plan, big ? tiles : nullptr, pl.n_up, pl.ntn_up,
            pl.ntn_down, counters);
    mark(mk);

    GemmArgs a{};
    a.qparams = qparams;
    a.offsets = offsets;
    a.plan = plan;
    a.tiles = tiles;
    a.counters = counters;
    a.tile_meta = counters + kTileMetaHalf;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    a.hs = ffn_hidden_stride(s);

    const uint64_t esd = s.dispatch == MOE_FP8_E4M3 ? 1 : 2;
    const uint64_t Tk = static_cast<uint64_t>(s.T) * s.k, TS = static_cast<uint64_t>(s.T) * s.S;
    const uint64_t wgroup = static_cast<uint64_t>(s.d) * s.h * 2;

    // up-projection + SwiGLU
    a.a_routed = static_cast<const uint8_t*>(x_perm);
    a.a_gather = gather;
    a.a_shared = static_cast<const uint8_t*>(x);
    a.a_routed_bytes = static_cast<uint32_t>(Tk * s.d * esd);
    a.a_shared_bytes =
        static_cast<uint32_t>(s.S > 0 || gather != nullptr ? static_cast<uint64_t>(s.T) * s.d * 2 : 0);
    a.w_bytes = static_cast<uint32_t>((s.E + s.S) * wgroup);
    a.wa = static_cast<const uint8_t*>(w1);
    a.wb = static_cast<const uint8_t*>(w3);
    a.out_routed = static_cast<uint8_t*>(h_routed);
    a.out_shared = static_cast<uint8_t*>(h_shared);
    a.pre_a_routed = static_cast<uint8_t*>(pre_a_r);
    a.pre_b_routed = static_cast<uint8_t*>(pre_b_r);
    a.pre_a_shared = static_cast<uint8_t*>(pre_a_s);
    a.pre_b_shared = static_cast<uint8_t*>(pre_b_s);
    hipError_t err;
    if (save) {
        a.ntn = 2 * s.h / kBigBN;
        const int64_t mt = max_mtiles(s, bm, false);
        err = s.dispatch == MOE_FP8_E4M3 ? launch_persistent<kModeUpFp8Save>(a, mt, st)
                                         : launch_persistent<kModeUpSave>(a, mt, st);
    } else if (f32) {
        a.ntn = (s.h + kF32BN - 1) / kF32BN;
        const int64_t mt = max_mtiles(s, kF32BM, false);
        ffn_gemm_f32_kernel<true><<<static_cast<unsigned>(mt * a.ntn), 256, 0, st>>>(a, 0);
        err = hipGetLastError();
    } else {
        a.ntn = big ? 2 * s.h / kBigBN : (s.h + kBN / 2 - 1) / (kBN / 2);
        const int64_t mt = max_mtiles(s, bm, false);
        err = s.dispatch == MOE_FP8_E4M3 ? launch_gemm<kModeUpFp8>(a, mt, big, st)
                                         : launch_gemm<kModeUp>(a, mt, big, st);
    }
    mark(mk);
    if (err != hipSuccess) return err;

    // down-projection
    a.a_gather = nullptr;
    a.a_routed = static_cast<const uint8_t*>(h_routed);
    a.a_shared = static_cast<const uint8_t*>(h_shared);
    a.a_routed_bytes = static_cast<uint32_t>(Tk * a.hs * 2);
    a.a_shared_bytes = static_cast<uint32_t>(TS * a.hs * 2);
    a.wa = static_cast<const uint8_t*>(w2);
    a.wb = nullptr;
    a.out_routed = static_cast<uint8_t*>(y_perm);
    a.out_shared = static_cast<uint8_t*>(y_shared);
    a.tiles = tiles + pl.n_up;
    a.counters = counters + 8;
    if (f32) {
        a.ntn = (s.d + kF32BN - 1) / kF32BN;
        const int64_t mt = max_mtiles(s, kF32BM, true);
        ffn_gemm_f32_kernel<false><<<static_cast<unsigned>(mt * a.ntn), 256, 0, st>>>(a, 0);
        err = hipGetLastError();
    } else {
        a.ntn = big ? s.d / kBigBN : (s.d + kBN - 1) / kBN;
        err = launch_gemm<kModeDown>(a, max_mtiles(s, bm, true), big, st);
    }
    mark(mk);
    return err;
}

// The backward's recomputation of the up-projection (128 x 128 tile kernel):
// a = W1 v, b = W3 v and H = silu(a) * b of every routed row and every
// shared-expert block, in bf16, laid out as the forward's H (row stride hs,
// shared blocks side by side). `plan` must hold the m-tile prefix for 128-row
// tiles (ffn_plan_kernel with bm = 128).
hipError_t launch_ffn_recompute(const moe_shape& s, const void* x_perm, const float* qparams,
                                const int32_t* offsets, const void* x, const void* w1,
                                const void* w3, const int32_t* plan, void* h_r, void* h_s,
                                void* a_r, void* b_r, void* a_s, void* b_s, hipStream_t st) {
    GemmArgs a{};
    a.qparams = qparams;
    a.offsets = offsets;
    a.plan = plan;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    a.hs = ffn_hidden_stride(s);
    a.a_routed = static_cast<const uint8_t*>(x_perm);
    a.a_shared = static_cast<const uint8_t*>(x);
    a.wa = static_cast<const uint8_t*>(w1);
    a.wb = static_cast<const uint8_t*>(w3);
    a.out_routed = static_cast<uint8_t*>(h_r);
    a.out_shared = static_cast<uint8_t*>(h_s);
    a.pre_a_routed = static_cast<uint8_t*>(a_r);
    a.pre_b_routed = static_cast<uint8_t*>(b_r);
    a.pre_a_shared = static_cast<uint8_t*>(a_s);
    a.pre_b_shared = static_cast<uint8_t*>(b_s);
    a.ntn = (s.h + kBN / 2 - 1) / (kBN / 2);
    int64_t blocks = max_mtiles(s, kBM, false) * a.ntn;
    blocks = (blocks + 7) & ~int64_t(7);
    if (s.dispatch == MOE_FP8_E4M3)
        ffn_gemm_kernel<kModeUpFp8, true><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
    else
        ffn_gemm_kernel<kModeUp, true><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_ffn_plan128(const moe_shape& s, const int32_t* offsets, int32_t* plan,
                              hipStream_t st) {
    ffn_plan_kernel<<<1, 256, 0, st>>>(offsets, s.E, s.S, s.T, kBM, plan, nullptr, 0, 0, 0,
                                       nullptr);
    return hipGetLastError();
}

hipError_t launch_hidden_quant(const moe_shape& s, int hs, const void* h_r, const void* h_s,
                               const int32_t* offsets, uint8_t* h8_r, uint8_t* h8_s,
                               float* hsc_r, float* hsc_s, hipStream_t st);

// The fp8-weight path of the expert stage takes the persistent kernels only:
// d and h multiples of 256 (whole groups of four 64-value slices) and every
// operand below 4 GiB.
bool f8w_supported(const moe_shape& s) {
    return use_big_tiles(s) && s.d % 256 == 0 && s.h % 256 == 0;
}

// The expert stage with fp8 weights: up-projection on the fp8 matrix cores
// (routed rows x_perm and the shared experts' rows x8, both per-token fp8
// codes), the hidden rows quantised per row, then the down-projection on the
// fp8 matrix cores. Weight codes w1q, w3q [G, h, d], w2q [G, d, h] with the
// scales of launch_quantize_weights.
hipError_t launch_grouped_ffn_f8w(const moe_shape& s, const void* x_perm, const float* qparams,
                                  const int32_t* offsets, const void* x8, const float* q8,
                                  const uint8_t* w1q, const uint8_t* w3q, const uint8_t* w2q,
                                  const float* wscale, void* y_perm, void* y_shared,
                                  int32_t* plan, void* h_r, void* h_s, uint8_t* h8_r,
                                  uint8_t* h8_s, float* hsc_r, float* hsc_s, bool plan_done,
                                  hipStream_t st, const Marks* mk) {
    const PlanLayout pl = plan_layout(s);
    int32_t* counters = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan) + pl.counters);
    int4* tiles = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + pl.tiles);
    if (!plan_done)
        ffn_plan_kernel<<<plan_blocks(pl), 256, 0, st>>>(offsets, s.E, s.S, s.T, kBigBM, plan, tiles,
                                                         pl.n_up, pl.ntn_up, pl.ntn_down, counters);
    mark(mk);
    const uint64_t Tk = static_cast<uint64_t>(s.T) * s.k, T = static_cast<uint64_t>(s.T);
    const uint64_t G = static_cast<uint64_t>(s.E + s.S);
    GemmArgs a{};
    a.qparams = qparams;
    a.offsets = offsets;
    a.plan = plan;
    a.tiles = tiles;
    a.counters = counters;
    a.tile_meta = counters + kTileMetaHalf;
    a.q_shared = q8;
    a.wscale = wscale;
    a.hsc_r = hsc_r;
    a.hsc_s = hsc_s;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    a.hs = s.h;
    // up-projection + SwiGLU
    a.a_routed = static_cast<const uint8_t*>(x_perm);
    a.a_shared = static_cast<const uint8_t*>(x8);
    a.a_routed_bytes = static_cast<uint32_t>(Tk * s.d);
    a.a_shared_bytes = static_cast<uint32_t>(s.S > 0 ? T * s.d : 0);
    a.w_bytes = static_cast<uint32_t>(G * s.h * s.d);
    a.wa = w1q;
    a.wb = w3q;
    a.out_routed = static_cast<uint8_t*>(h_r);
    a.out_shared = static_cast<uint8_t*>(h_s);
    a.ntn = 2 * s.h / kBigBN;
    hipError_t err = launch_gemm<kModeUpF8W>(a, max_mtiles(s, kBigBM, false), true, st);
    mark(mk);
    if (err != hipSuccess) return err;
    // hidden rows -> per-row fp8 codes
    err = launch_hidden_quant(s, s.h, h_r, h_s, offsets, h8_r, h8_s, hsc_r, hsc_s, st);
    mark(mk);
    if (err != hipSuccess) return err;
    // down-projection
    a.a_routed = h8_r;
    a.a_shared = h8_s;
    a.a_routed_bytes = static_cast<uint32_t>(Tk * s.h);
    a.a_shared_bytes = static_cast<uint32_t>(T * s.S * s.h);
    a.wa = w2q;
    a.wb = nullptr;
    a.out_routed = static_cast<uint8_t*>(y_perm);
    a.out_shared = static_cast<uint8_t*>(y_shared);
    a.tiles = tiles + pl.n_up;
    a.counters = counters + 8;
    a.ntn = s.d / kBigBN;
    err = launch_gemm<kModeDownF8W>(a, max_mtiles(s, kBigBM, true), true, st);
    mark(mk);
    return err;
}

// ------------------------------------------------- backward on big tiles --
// The expert FFN backward's GEMMs on the persistent kernel, for the shapes it
// takes (use_big_tiles) with [da | db] rows (2h values) within 32-bit offsets:
//   recompute  a = W1 v, b = W3 v and H of every row (kModeUpSave);
//   dh         dhid = dy W2 with the SwiGLU backward (kModeDh), from W2T
//              [G, h, d] = W2 transposed per group, writing [da | db] rows;
//   dx         dv = [da | db] W13T^T (kModeDown with K = 2h), W13T [G, d, 2h]
//              = [W1 | W3] transposed per group (the shared experts' K
//              blocks concatenated, so their dx is summed in the accumulator).
// Two tile plans: the forward's (up list: recompute, down list: dx) and one
// with h/256 n-tiles per group for dh.
bool ffn_backward_big(const moe_shape& s) {
    const uint64_t rows = static_cast<uint64_t>(s.T) * (s.k + s.S);
    const uint64_t wbytes = static_cast<uint64_t>(s.E + s.S) * s.d * s.h * 2;
    return use_big_tiles(s) && rows * 2 * s.h * 2 < (uint64_t(1) << 32) &&
           2 * wbytes < (uint64_t(1) << 32);
}

size_t ffn_plan_bytes_dh(const moe_shape& s) {
    return plan_layout(s, (s.h + kBigBN - 1) / kBigBN, s.d / kBigBN).bytes;
}

hipError_t launch_ffn_bwd_gemms(const moe_shape& s, const void* x_perm, const float* qparams,
                                const int32_t* offsets, const void* x, const void* w1,
                                const void* w3, const void* w2t, const void* w13t,
                                const void* dy_perm, const void* dy_sh, void* dx_perm, void* dx_sh,
                                int32_t* plan_f, int32_t* plan_dh, void* h_r, void* h_s, void* a_r,
                                void* b_r, void* a_s, void* b_s, void* dd_r, void* dd_s,
                                hipStream_t st, const Marks* mk, bool recompute) {
    const PlanLayout pf = plan_layout(s);
    const PlanLayout pd = plan_layout(s, (s.h + kBigBN - 1) / kBigBN, s.d / kBigBN);
    int32_t* cf = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan_f) + pf.counters);
    int4* tf = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan_f) + pf.tiles);
    int32_t* cd = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan_dh) + pd.counters);
    int4* td = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan_dh) + pd.tiles);
    ffn_plan_kernel<<<plan_blocks(pf), 256, 0, st>>>(offsets, s.E, s.S, s.T, kBigBM, plan_f, tf, pf.n_up,
                                                     pf.ntn_up, pf.ntn_down, cf);
    ffn_plan_kernel<<<plan_blocks(pd), 256, 0, st>>>(offsets, s.E, s.S, s.T, kBigBM, plan_dh, td, pd.n_up,
                                                     pd.ntn_up, pd.ntn_down, cd);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const uint64_t R = static_cast<uint64_t>(s.T) * s.k, T = static_cast<uint64_t>(s.T);
    const uint64_t G = static_cast<uint64_t>(s.E + s.S);
    const uint64_t esd = s.dispatch == MOE_FP8_E4M3 ? 1 : 2;
    GemmArgs a{};
    a.qparams = qparams;
    a.offsets = offsets;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    a.hs = s.h;
    // recompute: a, b and H
    a.plan = plan_f;
    a.tiles = tf;
    a.counters = cf;
    a.tile_meta = cf + kTileMetaHalf;
    a.a_routed = static_cast<const uint8_t*>(x_perm);
    a.a_shared = static_cast<const uint8_t*>(x);
    a.a_routed_bytes = static_cast<uint32_t>(R * s.d * esd);
    a.a_shared_bytes = static_cast<uint32_t>(s.S > 0 ? T * s.d * 2 : 0);
    a.w_bytes = static_cast<uint32_t>(G * s.d * s.h * 2);
    a.wa = static_cast<const uint8_t*>(w1);
    a.wb = static_cast<const uint8_t*>(w3);
    a.out_routed = static_cast<uint8_t*>(h_r);
    a.out_shared = static_cast<uint8_t*>(h_s);
    a.pre_a_routed = static_cast<uint8_t*>(a_r);
    a.pre_b_routed = static_cast<uint8_t*>(b_r);
    a.pre_a_shared = static_cast<uint8_t*>(a_s);
    a.pre_b_shared = static_cast<uint8_t*>(b_s);
    a.ntn = pf.ntn_up;
    // (not when the forward saved a, b and H)
    if (recompute) {
        err = s.dispatch == MOE_FP8_E4M3 ? launch_persistent<kModeUpFp8Save>(a, max_mtiles(s, kBigBM, false), st)
                                         : launch_persistent<kModeUpSave>(a, max_mtiles(s, kBigBM, false), st);
        if (err != hipSuccess) return err;
    }
    mark(mk);
    // dh: [da | db] rows
    a.plan = plan_dh;
    a.tiles = td;
    a.counters = cd;
    a.tile_meta = cd + kTileMetaHalf;
    a.a_routed = static_cast<const uint8_t*>(dy_perm);
    a.a_shared = static_cast<const uint8_t*>(dy_sh);
    a.a_routed_bytes = static_cast<uint32_t>(R * s.d * 2);
    a.a_shared_bytes = static_cast<uint32_t>(s.S > 0 ? T * s.d * 2 : 0);
    a.wa = static_cast<const uint8_t*>(w2t);
    a.wb = static_cast<const uint8_t*>(w2t);
    a.out_routed = static_cast<uint8_t*>(dd_r);
    a.out_shared = static_cast<uint8_t*>(dd_s);
    a.ntn = pd.ntn_up;
    err = launch_persistent<kModeDh>(a, max_mtiles(s, kBigBM, false), st);
    mark(mk);
    if (err != hipSuccess) return err;
    // dx = [da | db] W13T^T: the down-projection with 2h hidden values
    a.plan = plan_f;
    a.tiles = tf + pf.n_up;
    a.counters = cf + 8;
    a.tile_meta = cf + kTileMetaHalf;
    a.h = 2 * s.h;
    a.hs = 2 * s.h;
    a.a_routed = static_cast<const uint8_t*>(dd_r);
    a.a_shared = static_cast<const uint8_t*>(dd_s);
    a.a_routed_bytes = static_cast<uint32_t>(R * 2 * s.h * 2);
    a.a_shared_bytes = static_cast<uint32_t>(T * s.S * 2 * s.h * 2);
    a.w_bytes = static_cast<uint32_t>(G * s.d * 2 * s.h * 2);
    a.wa = static_cast<const uint8_t*>(w13t);
    a.wb = nullptr;
    a.pre_a_routed = a.pre_b_routed = a.pre_a_shared = a.pre_b_shared = nullptr;
    a.out_routed = static_cast<uint8_t*>(dx_perm);
    a.out_shared = static_cast<uint8_t*>(dx_sh);
    a.ntn = pf.ntn_down;
    err = launch_persistent<kModeDown>(a, max_mtiles(s, kBigBM, true), st);
    mark(mk);
    return err;
}

}  // namespace moe
