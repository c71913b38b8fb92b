// Backward of the grouped SwiGLU expert FFN on the matrix cores (bf16
// operands, float32 accumulation).
//
// "Deepseek-MoE同步税本质与四层实战优化指南" (gsyq.cn), section 2.4: in the
// backward pass the gradients go back along the same routing -- through
// combine, the experts' own computation, then dispatch. This file is the
// middle part: for every expert group g with input rows v (the dispatched
// rows; fp8 rows dequantised, the quantiser passing the gradient straight
// through) and output gradients dy,
//     a = W1 v, b = W3 v, u = silu(a), hid = u * b           (recomputed)
//     dhid = W2^T dy
//     da = dhid * b * silu'(a),  silu'(a) = s (1 + a (1 - s)), s = sigmoid(a)
//     db = dhid * u
//     dv  = W1^T da + W3^T db
//     dW2 = sum_rows dy hid^T,  dW1 = sum_rows da v^T,  dW3 = sum_rows db v^T
// with the shared experts ("DeepSeek 中 MoE 的同步税", wmrh.cn, section 2.1)
// as extra groups over every token, whose dv are summed per token.
//
// Four launches after the 128-row tile plan:
//   recompute  a, b and hid of every row (the forward's 128 x 128 tile kernel
//              keeping its pre-activations; grouped_ffn.hip);
//   dh         dhid = dy W2 per group, with the SwiGLU backward in the
//              epilogue, writing da and db;
//   dx         dv = [da | db] [W1; W3] per group (the shared experts' blocks
//              concatenated along K, so their sum happens in the accumulator);
//   wgrad      dW2, dW1, dW3: one work-group per 128 x 128 output tile of one
//              group's gradient, summing over that group's rows in order
//              (each element has one owner: no atomics, same bits every call).
// All four use 128 x 128 tiles, K in steps of 64, four waves each holding a
// 64 x 64 block of 32x32x16 bf16 MFMAs, operands staged global -> registers
// -> LDS with the next step's loads in flight during the current step's
// MFMAs. An operand whose rows are contiguous along K is stored to LDS as
// 16-byte chunks; one whose rows are contiguous along M (or N) -- the weights
// read transposed in dh and dx, both operands of wgrad -- is read as 16-byte
// chunks of 8 rows at two consecutive K and written to LDS transposed, as
// 4-byte pairs.
#include "ffn_plan.h"
#include "moe_device.h"

namespace moe {

constexpr int kTB = 128;        // rows of A (M) and of B (N) per tile
constexpr int kTK = 64;         // K per step
constexpr int kBwdThreads = 256;
constexpr int kBwdOp = kTB * kTK * 2;     // bytes of one operand per step
constexpr int kBwdStage = 2 * kBwdOp;     // A and B
constexpr int kBwdLds = 2 * kBwdStage;    // double buffered

struct BwdArgs {
    const int32_t* offsets;  // [E+1] routed row offsets
    const int32_t* plan;     // [E+S+1] m-tile prefix for 128-row tiles
    int64_t T;
    int E, S, d, h, hs;      // hs: row stride of a hidden block (h rounded up to 8)
    int fp8;                 // routed rows are fp8 codes with qparams
    const uint8_t* x_perm;   // [R, d] routed input rows (bf16 or fp8 codes)
    const float* qparams;    // [R, 2] (scale, centre) of fp8 rows
    const uint8_t* x;        // [T, d] shared experts' input (bf16)
    const uint8_t* w1;       // [G, h, d]
    const uint8_t* w3;       // [G, h, d]
    const uint8_t* w2;       // [G, d, h]
    const uint8_t* dy_perm;  // [R, d] gradient of the routed output rows
    const uint8_t* dy_sh;    // [T, d] gradient of the shared experts' sum
    const uint8_t* a_r;      // recomputed pre-activations and hidden rows:
    const uint8_t* b_r;      //   routed [R, hs], shared [T, S*hs]
    const uint8_t* h_r;
    const uint8_t* a_s;
    const uint8_t* b_s;
    const uint8_t* h_s;
    uint8_t* da_r;           // SwiGLU backward outputs, laid out like a and b
    uint8_t* db_r;
    uint8_t* da_s;
    uint8_t* db_s;
    uint8_t* dx_perm;        // [R, d]
    uint8_t* dx_sh;          // [T, d]
    float* dw1;              // [G, h, d]
    float* dw3;              // [G, h, d]
    float* dw2;              // [G, d, h]
    int ntn;                 // n-tiles per group (dh, dx)
    int tpg;                 // output tiles per group and gradient (wgrad)
    // layout of the da / db rows the weight gradients read: row stride of a
    // routed row and of a shared row, and the step between shared groups
    int dd_ld, dd_lds, dd_gs;
};

// byte offset of 16-byte chunk c (0..7) of row r of a [128][64] bf16 tile
// (XOR swizzle: 16-byte reads of 8 consecutive rows hit distinct banks)
__device__ __forceinline__ int bl(int r, int c) { return (r << 7) + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

__device__ __forceinline__ float sigmoid_fast(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// 8 e4m3 codes -> 8 bf16 values of code * scale + centre
__device__ __forceinline__ u32x4 dequant8_bwd(uint2 codes, float scale, float centre) {
    u32x4 out;
    const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), false);
    const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), true);
    const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), false);
    const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), true);
    out[0] = pack_bf16x2(__builtin_fmaf(p0[0], scale, centre), __builtin_fmaf(p0[1], scale, centre));
    out[1] = pack_bf16x2(__builtin_fmaf(p1[0], scale, centre), __builtin_fmaf(p1[1], scale, centre));
    out[2] = pack_bf16x2(__builtin_fmaf(p2[0], scale, centre), __builtin_fmaf(p2[1], scale, centre));
    out[3] = pack_bf16x2(__builtin_fmaf(p3[0], scale, centre), __builtin_fmaf(p3[1], scale, centre));
    return out;
}

// Eight bf16 values n0..n0+7 of a row that holds `count` values from p (a
// 16-byte load when the row pointer is 16-byte aligned, value by value
// otherwise); values at or past `count` read as zero.
__device__ __forceinline__ u32x4 load8_bf16(const uint8_t* p, int count, bool aligned) {
    if (count <= 0) return u32x4{0u, 0u, 0u, 0u};
    if (aligned && count >= 8) return load16(p);
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = 2 * i < count ? q[2 * i] : 0u;
        const uint32_t hi = 2 * i + 1 < count ? q[2 * i + 1] : 0u;
        w[i] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// K-contiguous operand: thread (c = tid & 7, rr = tid >> 3) holds the 16-byte
// chunk c of rows rr + 32 i, i = 0..3.
__device__ __forceinline__ void store_krows(uint8_t* op, const u32x4 (&v)[4], int tid) {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(op + bl(rr + 32 * i, c)) = v[i];
}

// Row-contiguous operand: unit u = tid + 256 j (j = 0, 1) covers rows
// 8 (u & 15) .. +7 at K = 2 (u >> 4) and the next K; v[2j] holds the first
// K's 8 values, v[2j+1] the second's. Written transposed as 4-byte pairs.
__device__ __forceinline__ void store_mrows(uint8_t* op, const u32x4 (&v)[4], int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int u = tid + 256 * j;
        const int r0 = 8 * (u & 15), k = 2 * (u >> 4);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t e0 = (v[2 * j][q >> 1] >> (16 * (q & 1))) & 0xffffu;
            const uint32_t e1 = (v[2 * j + 1][q >> 1] >> (16 * (q & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t*>(op + bl(r0 + q, k >> 3) + (k & 7) * 2) = e0 | (e1 << 16);
        }
    }
}

// one K step of the tile: acc[mb][nb] += A rows (wm*64 + mb*32 ..) x B rows
// (wn*64 + nb*32 ..) over the 64 K values in LDS
__device__ __forceinline__ void mma_step(const uint8_t* As, const uint8_t* Bs, f32x16 (&acc)[2][2],
                                         int wm, int wn, int lr, int lg) {
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
        const int ch = ks * 2 + lg;
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            af[mb] = *reinterpret_cast<const bf16x8*>(As + bl(wm * 64 + mb * 32 + lr, ch));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            bf[nb] = *reinterpret_cast<const bf16x8*>(Bs + bl(wn * 64 + nb * 32 + lr, ch));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
}

// The K loop shared by the four kernels: load(k0, ra, rb) fills the staging
// registers of step k0; KA / KB tell whether A / B are K-contiguous.
template <bool KA, bool KB, class Load>
__device__ __forceinline__ void k_loop(int K, Load&& load, f32x16 (&acc)[2][2]) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const int KT = (K + kTK - 1) / kTK;
    if (KT == 0) return;
    u32x4 ra[4], rb[4];
    auto put = [&](int buf) {
        uint8_t* As = lds + buf * kBwdStage;
        uint8_t* Bs = As + kBwdOp;
        if constexpr (KA) store_krows(As, ra, tid); else store_mrows(As, ra, tid);
        if constexpr (KB) store_krows(Bs, rb, tid); else store_mrows(Bs, rb, tid);
    };
    load(0, ra, rb);
    put(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load((kt + 1) * kTK, ra, rb);
        const uint8_t* As = lds + (kt & 1) * kBwdStage;
        mma_step(As, As + kBwdOp, acc, wm, wn, lr, lg);
        if (kt + 1 < KT) put((kt + 1) & 1);
        __syncthreads();
    }
}

// tile L of a dgrad launch -> (group, first row of the group, rows, m-tile,
// n-tile); routed groups from the plan, then S shared groups over T tokens
// (nshared = S) or one shared group over the S concatenated blocks
// (nshared = 1). False past the last tile.
__device__ __forceinline__ bool bwd_locate(const BwdArgs& a, int nshared, int& g, int64_t& row_base,
                                           int& nrows, int& m0, int& nt) {
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int L = (bid & 7) * (nwg >> 3) + (bid >> 3);  // contiguous tile range per XCD
    const int mtg = L / a.ntn;
    nt = L - mtg * a.ntn;
    const int routed = a.plan[a.E];
    const int mtT = static_cast<int>((a.T + kTB - 1) / kTB);
    if (mtg >= routed) {
        const int q = mtg - routed;
        if (q >= nshared * mtT) return false;
        g = a.E + q / mtT;
        m0 = (q % mtT) * kTB;
        row_base = 0;
        nrows = static_cast<int>(a.T);
        return true;
    }
    int lo = 0, hi = a.E - 1;  // largest g with plan[g] <= mtg
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.plan[mid] <= mtg) lo = mid;
        else hi = mid - 1;
    }
    g = lo;
    m0 = (mtg - a.plan[g]) * kTB;
    row_base = a.offsets[g];
    nrows = a.offsets[g + 1] - a.offsets[g];
    return true;
}

// dhid = dy W2 (K = d, N = h) with the SwiGLU backward in the epilogue.
__global__ __launch_bounds__(kBwdThreads, 2) void ffn_bwd_dh_kernel(BwdArgs a) {
    int g, nrows, m0, nt;
    int64_t row_base;
    if (!bwd_locate(a, a.S, g, row_base, nrows, m0, nt)) return;
    const bool shared = g >= a.E;
    const int tid = threadIdx.x;
    const int c = tid & 7, rr = tid >> 3;
    const uint8_t* arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + rr + 32 * i;
        arow[i] = r < nrows ? (shared ? a.dy_sh + static_cast<int64_t>(r) * a.d * 2
                                      : a.dy_perm + (row_base + r) * a.d * 2)
                            : nullptr;
    }
    const uint8_t* w2g = a.w2 + static_cast<int64_t>(g) * a.d * a.h * 2;
    const bool aligned = (a.h & 7) == 0;
    auto load = [&](int k0, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
        const int kk = k0 + c * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ra[i] = (arow[i] != nullptr && kk < a.d) ? load16(arow[i] + static_cast<int64_t>(kk) * 2)
                                                     : u32x4{0u, 0u, 0u, 0u};
        // B (n = j, k = i) = W2[g][i][j]: rows of W2 are contiguous along j
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int u = tid + 256 * j;
            const int n0 = nt * kTB + 8 * (u & 15), k = k0 + 2 * (u >> 4);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int kq = k + q;
                rb[2 * j + q] = kq < a.d ? load8_bf16(w2g + (static_cast<int64_t>(kq) * a.h + n0) * 2,
                                                      a.h - n0, aligned)
                                         : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    f32x16 acc[2][2];
    k_loop<true, false>(a.d, load, acc);

    // epilogue: (row, j) -> da, db from dhid and the recomputed a, b
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
    const int s = shared ? g - a.E : 0;
    const int ld = shared ? a.S * a.hs : a.hs;
    const bf16_t* pa = reinterpret_cast<const bf16_t*>(shared ? a.a_s : a.a_r);
    const bf16_t* pb = reinterpret_cast<const bf16_t*>(shared ? a.b_s : a.b_r);
    bf16_t* oa = reinterpret_cast<bf16_t*>(shared ? a.da_s : a.da_r);
    bf16_t* ob = reinterpret_cast<bf16_t*>(shared ? a.db_s : a.db_r);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
            if (r >= nrows) continue;
            const int64_t row = shared ? r : row_base + r;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int j = nt * kTB + wn * 64 + nb * 32 + lr;
                if (j >= a.hs) continue;
                const int64_t at = row * ld + s * a.hs + j;
                float da = 0.0f, db = 0.0f;
                if (j < a.h) {
                    const float dh = acc[mb][nb][v];
                    const float av = bf16_to_f32(pa[at]), bv = bf16_to_f32(pb[at]);
                    const float sg = sigmoid_fast(av);
                    da = dh * bv * (sg * (1.0f + av * (1.0f - sg)));
                    db = dh * (av * sg);
                }
                oa[at] = f32_to_bf16(da);
                ob[at] = f32_to_bf16(db);
            }
        }
}

// dv = [da | db] [W1; W3] (K = 2 hs per group, S * 2 hs for the shared
// experts as one group; N = d).
__global__ __launch_bounds__(kBwdThreads, 2) void ffn_bwd_dx_kernel(BwdArgs a) {
    int g, nrows, m0, nt;
    int64_t row_base;
    if (!bwd_locate(a, a.S > 0 ? 1 : 0, g, row_base, nrows, m0, nt)) return;
    const bool shared = g >= a.E;
    const int tid = threadIdx.x;
    const int c = tid & 7, rr = tid >> 3;
    const int K = (shared ? a.S : 1) * 2 * a.hs;
    const int ld = shared ? a.S * a.hs : a.hs;
    const uint8_t* dA = shared ? a.da_s : a.da_r;
    const uint8_t* dB = shared ? a.db_s : a.db_r;
    int64_t arow[4];  // element offset of each of this thread's rows, -1 past the group
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + rr + 32 * i;
        arow[i] = r < nrows ? (shared ? static_cast<int64_t>(r) : row_base + r) * ld : -1;
    }
    auto load = [&](int k0, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
        {
            const int kk = k0 + c * 8;
            const int seg = kk / a.hs, local = kk - seg * a.hs;
            const uint8_t* base = (seg & 1) ? dB : dA;
            const int col = (seg >> 1) * a.hs + local;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ra[i] = (arow[i] >= 0 && kk < K) ? load16(base + (arow[i] + col) * 2)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
        // B (n = i, k) = W1 or W3 [group][j][i]: rows contiguous along i
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int u = tid + 256 * j;
            const int n0 = nt * kTB + 8 * (u & 15);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int kq = k0 + 2 * (u >> 4) + q;
                const int seg = kq / a.hs, local = kq - seg * a.hs;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (kq < K && local < a.h && n0 < a.d) {
                    const int gg = shared ? a.E + (seg >> 1) : g;
                    const uint8_t* w = (seg & 1) ? a.w3 : a.w1;
                    v = load16(w + ((static_cast<int64_t>(gg) * a.h + local) * a.d + n0) * 2);
                }
                rb[2 * j + q] = v;
            }
        }
    };
    f32x16 acc[2][2];
    k_loop<true, false>(K, load, acc);

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
    bf16_t* out = reinterpret_cast<bf16_t*>(shared ? a.dx_sh : a.dx_perm);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
            if (r >= nrows) continue;
            const int64_t row = shared ? r : row_base + r;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int i = nt * kTB + wn * 64 + nb * 32 + lr;
                if (i < a.d) out[row * a.d + i] = f32_to_bf16(acc[mb][nb][v]);
            }
        }
}

// The weight gradients: block (q, g, tile) with q = 0 dW2 [d, h], 1 dW1
// [h, d], 2 dW3 [h, d]; K runs over the group's rows.
__global__ __launch_bounds__(kBwdThreads, 2) void ffn_bwd_wgrad_kernel(BwdArgs a) {
    const int G = a.E + a.S;
    const int64_t b = blockIdx.x;
    const int q = static_cast<int>(b / (static_cast<int64_t>(G) * a.tpg));
    const int64_t rem = b - static_cast<int64_t>(q) * G * a.tpg;
    const int g = static_cast<int>(rem / a.tpg);
    const int tile = static_cast<int>(rem - static_cast<int64_t>(g) * a.tpg);
    const int M = q == 0 ? a.d : a.h, N = q == 0 ? a.h : a.d;
    const int ntm = (M + kTB - 1) / kTB;
    const int mt = tile % ntm, nt = tile / ntm;
    const bool shared = g >= a.E;
    const int s = shared ? g - a.E : 0;
    const int64_t r0 = shared ? 0 : a.offsets[g];
    const int nr = shared ? static_cast<int>(a.T) : a.offsets[g + 1] - a.offsets[g];
    const int m0 = mt * kTB, n0 = nt * kTB;
    const int tid = threadIdx.x;
    const int ldh = shared ? a.S * a.hs : a.hs;  // row stride of hidden-side rows
    const int hoff = s * a.hs;                   // this group's block within them
    // A (m, k = row): q = 0: dy[row][m]; else da / db [row][m]
    const uint8_t* A = q == 0 ? (shared ? a.dy_sh : a.dy_perm) : (q == 1 ? (shared ? a.da_s : a.da_r)
                                                                         : (shared ? a.db_s : a.db_r));
    const int lda = q == 0 ? a.d : (shared ? a.dd_lds : a.dd_ld);
    const int aoff = q == 0 ? 0 : s * a.dd_gs, acount = q == 0 ? a.d : a.hs;
    // B (n, k = row): q = 0: hid[row][n]; else the input row v[row][n]
    const uint8_t* B = q == 0 ? (shared ? a.h_s : a.h_r) : (shared ? a.x : a.x_perm);
    const int ldb = q == 0 ? ldh : a.d, boff = q == 0 ? hoff : 0, bcount = q == 0 ? a.hs : a.d;
    const bool bfp8 = q != 0 && !shared && a.fp8;
    auto load = [&](int k0, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int u = tid + 256 * j;
            const int e8 = 8 * (u & 15);
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int k = k0 + 2 * (u >> 4) + qq;  // row within the group
                const bool kin = k < nr;
                const int64_t row = r0 + k;
                const int am = m0 + e8, bn = n0 + e8;
                ra[2 * j + qq] = (kin && am < acount)
                                     ? load16(A + (row * lda + aoff + am) * 2)
                                     : u32x4{0u, 0u, 0u, 0u};
                u32x4 vb = u32x4{0u, 0u, 0u, 0u};
                if (kin && bn < bcount) {
                    if (bfp8) {
                        const uint2 codes = *reinterpret_cast<const uint2*>(B + row * a.d + bn);
                        const float2 qp = *reinterpret_cast<const float2*>(a.qparams + 2 * row);
                        vb = dequant8_bwd(codes, qp.x, qp.y);
                    } else {
                        vb = load16(B + (row * ldb + boff + bn) * 2);
                    }
                }
                rb[2 * j + qq] = vb;
            }
        }
    };
    f32x16 acc[2][2];
    k_loop<false, false>(nr, load, acc);

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
    float* out = (q == 0 ? a.dw2 : (q == 1 ? a.dw1 : a.dw3)) + static_cast<int64_t>(g) * M * N;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
            if (m >= M) continue;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int n = n0 + wn * 64 + nb * 32 + lr;
                if (n < N) out[static_cast<int64_t>(m) * N + n] = acc[mb][nb][v];
            }
        }
}

// dst[b][c][dcol0 + r] = src[b][r][c] for a batch of [rows, cols] bf16
// matrices (rows and cols multiples of 64; dst rows hold ldd values). One
// work-group per 64 x 64 block through LDS: 16-byte reads along the source
// rows, 16-byte writes along the destination rows. Routed groups b < E with
// no rows (offsets[b + 1] == offsets[b]) are skipped: no tile of the
// backward's GEMMs reads their transposed weights.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ src, int rows,
                                                             int cols, int64_t sstride,
                                                             bf16_t* __restrict__ dst, int ldd,
                                                             int dcol0, int64_t dstride,
                                                             const int32_t* __restrict__ offsets, int E) {
    __shared__ uint16_t t[64][66];
    if (static_cast<int>(blockIdx.z) < E && offsets[blockIdx.z + 1] == offsets[blockIdx.z]) return;
    const int tid = threadIdx.x, c8 = tid & 7, rr = tid >> 3;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const bf16_t* sb = src + blockIdx.z * sstride;
    bf16_t* db = dst + blockIdx.z * dstride;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = rr + 32 * i;
        const u32x4 v = load16(reinterpret_cast<const uint8_t*>(sb + static_cast<int64_t>(r0 + r) * cols + c0 + 8 * c8));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            t[r][8 * c8 + 2 * u] = static_cast<uint16_t>(v[u] & 0xffffu);
            t[r][8 * c8 + 2 * u + 1] = static_cast<uint16_t>(v[u] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = rr + 32 * i;  // a destination row
        u32x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = static_cast<uint32_t>(t[8 * c8 + 2 * u][c]) | (static_cast<uint32_t>(t[8 * c8 + 2 * u + 1][c]) << 16);
        *reinterpret_cast<u32x4*>(db + static_cast<int64_t>(c0 + c) * ldd + dcol0 + r0 + 8 * c8) = v;
    }
}

int ffn_hidden_stride(const moe_shape& s);
bool ffn_backward_big(const moe_shape& s);
size_t ffn_plan_bytes(const moe_shape& s);
size_t ffn_plan_bytes_dh(const moe_shape& s);
hipError_t launch_ffn_bwd_gemms(const moe_shape& s, const void* x_perm, const float* qparams,
                                const int32_t* offsets, const void* x, const void* w1,
                                const void* w3, const void* w2t, const void* w13t,
                                const void* dy_perm, const void* dy_sh, void* dx_perm, void* dx_sh,
                                int32_t* plan_f, int32_t* plan_dh, void* h_r, void* h_s, void* a_r,
                                void* b_r, void* a_s, void* b_s, void* dd_r, void* dd_s,
                                hipStream_t st, const Marks* mk, bool recompute);
bool wgrad_supported(const moe_shape& s);
size_t wgrad_ws_bytes(const moe_shape& s);
hipError_t launch_ffn_wgrad(const moe_shape& s, const int32_t* offsets, const void* dd_r,
                            const void* dd_s, const void* v_r, const void* v_s, const void* dy_r,
                            const void* dy_s, const void* hid_r, const void* hid_s, float* dw1,
                            float* dw3, float* dw2, void* ws, hipStream_t st);
hipError_t launch_ffn_plan128(const moe_shape& s, const int32_t* offsets, int32_t* plan,
                              hipStream_t st);
hipError_t launch_ffn_recompute(const moe_shape& s, const void* x_perm, const float* qparams,
                                const int32_t* offsets, const void* x, const void* w1,
                                const void* w3, const int32_t* plan, void* h_r, void* h_s,
                                void* a_r, void* b_r, void* a_s, void* b_s, hipStream_t st);

// Workspace of the backward: the 128-row plan, then a, b, hid, da, db of the
// routed rows ([R, hs] bf16 each) and of the shared experts ([T, S*hs]).
struct BwdLayout {
    bool big;  // the persistent-kernel path
    bool wg;   // the weight gradients on the persistent kernel too
    size_t plan, plan_dh, a_r, b_r, h_r, da_r, db_r, a_s, b_s, h_s, da_s, db_s, w2t, w13t, wgq, bytes;
};
// Workspace: the 128-row plan (or the two persistent plans), the recomputed
// a, b, H and the gradients da, db of every row; on the persistent path da
// and db share rows ([da | db], 2h values per group) and the transposed
// weights W2T [G, h, d] and W13T [G, d, 2h] follow.
BwdLayout bwd_layout(const moe_shape& s) {
    BwdLayout L{};
    L.big = ffn_backward_big(s);
    const size_t hs = static_cast<size_t>(ffn_hidden_stride(s));
    const size_t R = static_cast<size_t>(s.T) * s.k, TS = static_cast<size_t>(s.T) * s.S;
    const size_t G = static_cast<size_t>(s.E + s.S), dh = static_cast<size_t>(s.d) * s.h;
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t at = off;
        off = (off + n + 255) & ~static_cast<size_t>(255);
        return at;
    };
    if (L.big) {
        L.plan = take(ffn_plan_bytes(s));
        L.plan_dh = take(ffn_plan_bytes_dh(s));
    } else {
        L.plan = take(static_cast<size_t>(s.E + s.S + 1) * 4);
    }
    L.a_r = take(R * hs * 2);
    L.b_r = take(R * hs * 2);
    L.h_r = take(R * hs * 2);
    L.a_s = take(TS * hs * 2);
    L.b_s = take(TS * hs * 2);
    L.h_s = take(TS * hs * 2);
    if (L.big) {
        L.da_r = take(R * 2 * hs * 2);
        L.db_r = L.da_r + hs * 2;
        L.da_s = take(TS * 2 * hs * 2);
        L.db_s = L.da_s + hs * 2;
        L.w2t = take(G * dh * 2);
        L.w13t = take(G * dh * 2 * 2);
        L.wg = wgrad_supported(s);
        if (L.wg) L.wgq = take(wgrad_ws_bytes(s));
    } else {
        L.da_r = take(R * hs * 2);
        L.db_r = take(R * hs * 2);
        L.da_s = take(TS * hs * 2);
        L.db_s = take(TS * hs * 2);
    }
    L.bytes = off;
    return L;
}

size_t ffn_backward_ws_bytes(const moe_shape& s) { return bwd_layout(s).bytes; }

// The activations a forward may save for the backward: a = W1 v, b = W3 v
// and hid = silu(a) b, bf16, routed rows [T*k, hs] then the shared experts'
// token rows [T, S*hs] (hs = h rounded up to 8), 256-byte aligned sections.
SavedLayout saved_layout(const moe_shape& s) {
    SavedLayout L;
    const size_t hs = static_cast<size_t>(ffn_hidden_stride(s));
    const size_t R = static_cast<size_t>(s.T) * s.k, TS = static_cast<size_t>(s.T) * s.S;
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t at = off;
        off = (off + n + 255) & ~static_cast<size_t>(255);
        return at;
    };
    L.a_r = take(R * hs * 2);
    L.b_r = take(R * hs * 2);
    L.h_r = take(R * hs * 2);
    L.a_s = take(TS * hs * 2);
    L.b_s = take(TS * hs * 2);
    L.h_s = take(TS * hs * 2);
    L.bytes = off;
    return L;
}

hipError_t launch_ffn_backward(const moe_shape& s, const void* x_perm, const float* qparams,
                               const int32_t* offsets, const void* x, const void* w1,
                               const void* w3, const void* w2, const void* dy_perm,
                               const void* dy_sh, void* dx_perm, void* dx_sh, float* dw1,
                               float* dw3, float* dw2, void* ws, hipStream_t st,
                               const Marks* mk, const void* saved) {
    const BwdLayout L = bwd_layout(s);
    uint8_t* w = static_cast<uint8_t*>(ws);
    // a, b and hid: saved by the forward, or recomputed into the workspace
    const SavedLayout SL = saved_layout(s);
    uint8_t* sv = static_cast<uint8_t*>(const_cast<void*>(saved));
    uint8_t* const p_a_r = sv != nullptr ? sv + SL.a_r : w + L.a_r;
    uint8_t* const p_b_r = sv != nullptr ? sv + SL.b_r : w + L.b_r;
    uint8_t* const p_h_r = sv != nullptr ? sv + SL.h_r : w + L.h_r;
    uint8_t* const p_a_s = sv != nullptr ? sv + SL.a_s : w + L.a_s;
    uint8_t* const p_b_s = sv != nullptr ? sv + SL.b_s : w + L.b_s;
    uint8_t* const p_h_s = sv != nullptr ? sv + SL.h_s : w + L.h_s;
    BwdArgs a{};
    a.offsets = offsets;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    a.hs = ffn_hidden_stride(s);
    a.fp8 = s.dispatch == MOE_FP8_E4M3 ? 1 : 0;
    a.x_perm = static_cast<const uint8_t*>(x_perm);
    a.qparams = qparams;
    a.x = static_cast<const uint8_t*>(x);
    a.w1 = static_cast<const uint8_t*>(w1);
    a.w3 = static_cast<const uint8_t*>(w3);
    a.w2 = static_cast<const uint8_t*>(w2);
    a.dy_perm = static_cast<const uint8_t*>(dy_perm);
    a.dy_sh = static_cast<const uint8_t*>(dy_sh);
    a.a_r = p_a_r;
    a.b_r = p_b_r;
    a.h_r = p_h_r;
    a.a_s = p_a_s;
    a.b_s = p_b_s;
    a.h_s = p_h_s;
    a.da_r = w + L.da_r;
    a.db_r = w + L.db_r;
    a.da_s = w + L.da_s;
    a.db_s = w + L.db_s;
    a.dx_perm = static_cast<uint8_t*>(dx_perm);
    a.dx_sh = static_cast<uint8_t*>(dx_sh);
    a.dw1 = dw1;
    a.dw3 = dw3;
    a.dw2 = dw2;
    hipError_t e;
    mark(mk);
    if (L.big) {
        // W2T [G, h, d] and W13T [G, d, 2h] = [W1 | W3] transposed per group
        const int G = s.E + s.S;
        const int64_t dh = static_cast<int64_t>(s.d) * s.h;
        bf16_t* w2t = reinterpret_cast<bf16_t*>(w + L.w2t);
        bf16_t* w13t = reinterpret_cast<bf16_t*>(w + L.w13t);
        transpose_bf16_kernel<<<dim3(s.h / 64, s.d / 64, G), 256, 0, st>>>(
            static_cast<const bf16_t*>(w2), s.d, s.h, dh, w2t, s.d, 0, dh, offsets, s.E);
        transpose_bf16_kernel<<<dim3(s.d / 64, s.h / 64, G), 256, 0, st>>>(
            static_cast<const bf16_t*>(w1), s.h, s.d, dh, w13t, 2 * s.h, 0, 2 * dh, offsets, s.E);
        transpose_bf16_kernel<<<dim3(s.d / 64, s.h / 64, G), 256, 0, st>>>(
            static_cast<const bf16_t*>(w3), s.h, s.d, dh, w13t, 2 * s.h, s.h, 2 * dh, offsets, s.E);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = launch_ffn_bwd_gemms(s, x_perm, qparams, offsets, x, w1, w3, w2t, w13t, dy_perm, dy_sh,
                                 dx_perm, dx_sh, reinterpret_cast<int32_t*>(w + L.plan),
                                 reinterpret_cast<int32_t*>(w + L.plan_dh), p_h_r, p_h_s,
                                 p_a_r, p_b_r, p_a_s, p_b_s, w + L.da_r, w + L.da_s,
                                 st, mk, sv == nullptr);
        if (e != hipSuccess) return e;
        // the weight gradients read [da | db] rows and the routed m-tile
        // prefix of 128-row tiles is not needed by them
        a.dd_ld = 2 * s.h;
        a.dd_lds = 2 * s.S * s.h;
        a.dd_gs = 2 * s.h;
    } else {
        a.plan = reinterpret_cast<const int32_t*>(w + L.plan);
        a.dd_ld = a.hs;
        a.dd_lds = s.S * a.hs;
        a.dd_gs = a.hs;
        e = launch_ffn_plan128(s, offsets, reinterpret_cast<int32_t*>(w + L.plan), st);
        if (e != hipSuccess) return e;
        if (sv == nullptr) {
            e = launch_ffn_recompute(s, x_perm, qparams, offsets, x, w1, w3,
                                     reinterpret_cast<const int32_t*>(w + L.plan), w + L.h_r, w + L.h_s,
                                     w + L.a_r, w + L.b_r, w + L.a_s, w + L.b_s, st);
            if (e != hipSuccess) return e;
        }
        mark(mk);
        const int64_t mtT = (s.T + kTB - 1) / kTB;
        const int64_t routed = static_cast<int64_t>(s.T) * s.k / kTB + s.E;  // routed m-tiles, at most
        auto grid = [](int64_t n) { return static_cast<unsigned>((n + 7) & ~int64_t(7)); };
        a.ntn = (a.hs + kTB - 1) / kTB;
        ffn_bwd_dh_kernel<<<grid((routed + s.S * mtT) * a.ntn), kBwdThreads, kBwdLds, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        mark(mk);
        a.ntn = (s.d + kTB - 1) / kTB;
        ffn_bwd_dx_kernel<<<grid((routed + (s.S > 0 ? mtT : 0)) * a.ntn), kBwdThreads, kBwdLds, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        mark(mk);
    }
    if (L.big && L.wg) {
        e = launch_ffn_wgrad(s, offsets, w + L.da_r, w + L.da_s, x_perm, x, dy_perm, dy_sh, p_h_r,
                             p_h_s, dw1, dw3, dw2, w + L.wgq, st);
        if (e != hipSuccess) return e;
        mark(mk);
        return hipSuccess;
    }
    a.tpg = ((s.d + kTB - 1) / kTB) * ((s.h + kTB - 1) / kTB);
    const int64_t nblk = 3 * static_cast<int64_t>(s.E + s.S) * a.tpg;
    ffn_bwd_wgrad_kernel<<<static_cast<unsigned>(nblk), kBwdThreads, kBwdLds, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    mark(mk);
    return hipSuccess;
}

}  // namespace moe
