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
#include "moe_device.h"

namespace moe {

enum { kModeUp = 0, kModeUpFp8 = 1, kModeDown = 2 };

constexpr int kBM = 128, kBN = 128, kBK = 64;  // bf16 tile: rows x B rows x K
constexpr int kFfnThreads = 256;
constexpr int kLdsStage = (kBM + kBN) * kBK * 2;  // bytes per pipeline stage
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

// plan[g] = number of m-tiles of groups before g (g = 0..E+S); routed group g
// has ceil(n_g / bm) m-tiles and each shared group ceil(T / bm).
__global__ __launch_bounds__(256) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                       int E, int S, int64_t T, int bm,
                                                       int32_t* __restrict__ plan) {
    __shared__ int mt[kMaxE + kMaxS];
    const int G = E + S;
    for (int g = threadIdx.x; g < G; g += 256) {
        const int64_t n = g < E ? static_cast<int64_t>(offsets[g + 1] - offsets[g]) : T;
        mt[g] = static_cast<int>((n + bm - 1) / bm);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0;
        for (int g = 0; g < G; ++g) {
            plan[g] = s;
            s += mt[g];
        }
        plan[G] = s;
    }
}

struct GemmArgs {
    const uint8_t* a_routed;  // routed A rows: x_perm (bf16 or fp8 codes) or H_r
    const float* qparams;     // fp8 rows: [rows, 2] = (scale, centre)
    const uint8_t* a_shared;  // shared A rows: x [T, d] (up) or H_s [T, S*h] (down)
    const int32_t* offsets;   // [E+1]
    const int32_t* plan;      // [E+S+1]
    const uint8_t* wa;        // up: W1 [G, h, d]; down: W2 [G, d, h]
    const uint8_t* wb;        // up: W3 [G, h, d]
    uint8_t* out_routed;      // up: H_r [T*k, h]; down: Y_perm [T*k, d]
    uint8_t* out_shared;      // up: H_s [T, S*h]; down: y_sh [T, d]
    int64_t T;
    int E, S, d, h;
    int ntn;  // n-tiles per group
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

// byte offset of 16-byte chunk c of row r in a [rows][64] bf16 LDS tile,
// XOR-swizzled so a wave's fragment reads spread over the banks
__device__ __forceinline__ int lds_off(int r, int c) { return (r << 7) + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// 8 e4m3 codes -> 8 bf16 values of code*scale + centre (one 16-byte chunk)
__device__ __forceinline__ uint32_t dequant2(float lo, float hi, float scale, float centre) {
    return pack_bf16x2(__builtin_fmaf(lo, scale, centre), __builtin_fmaf(hi, scale, centre));
}
__device__ __forceinline__ u32x4 dequant8(uint2 codes, float scale, float centre) {
    u32x4 out;
    out[0] = dequant2(__builtin_amdgcn_cvt_f32_fp8(codes.x, 0), __builtin_amdgcn_cvt_f32_fp8(codes.x, 1),
                      scale, centre);
    out[1] = dequant2(__builtin_amdgcn_cvt_f32_fp8(codes.x, 2), __builtin_amdgcn_cvt_f32_fp8(codes.x, 3),
                      scale, centre);
    out[2] = dequant2(__builtin_amdgcn_cvt_f32_fp8(codes.y, 0), __builtin_amdgcn_cvt_f32_fp8(codes.y, 1),
                      scale, centre);
    out[3] = dequant2(__builtin_amdgcn_cvt_f32_fp8(codes.y, 2), __builtin_amdgcn_cvt_f32_fp8(codes.y, 3),
                      scale, centre);
    return out;
}

template <int MODE>
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
    const int K = MODE == kModeDown ? (shared ? a.S * a.h : a.h) : a.d;
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
    // B rows of this thread (weight rows = output features)
    const uint8_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int br = rr + 32 * i;  // 0..127 within the B tile
        if (MODE == kModeDown) {
            const int n = nt * kBN + br;
            // shared: segment base chosen per K tile below
            brow[i] = a.wa + (static_cast<int64_t>(shared ? a.E : g) * a.d + n) * a.h * 2;
        } else {
            const int q = br >> 6, within = br & 63;
            const int n = nt * (kBN / 2) + q * 32 + (within & 31);
            const uint8_t* w = (within < 32) ? a.wa : a.wb;
            brow[i] = w + (static_cast<int64_t>(g) * a.h + n) * a.d * 2;
        }
    }

    const bool fp8_rows = MODE == kModeUpFp8 && !shared;
    u32x4 ra[4], rb[4];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (arow[i] == nullptr) {
                ra[i] = u32x4{0u, 0u, 0u, 0u};
            } else if (fp8_rows) {
                const uint2 codes = *reinterpret_cast<const uint2*>(arow[i] + k0 + c * 8);
                ra[i] = dequant8(codes, qs[i], qc[i]);
            } else {
                ra[i] = load16(arow[i] + (static_cast<int64_t>(k0) + c * 8) * 2);
            }
        }
        int64_t boff = (static_cast<int64_t>(k0) + c * 8) * 2;
        if (MODE == kModeDown && shared) {
            const int seg = k0 / a.h;  // shared expert whose hidden block holds k0
            boff = static_cast<int64_t>(seg) * a.d * a.h * 2 +
                   (static_cast<int64_t>(k0 - seg * a.h) + c * 8) * 2;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = load16(brow[i] + boff);
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

    const int KT = K / kBK;
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
                        out[row * a.d + col] = f32_to_bf16(acc[mb][nb][v]);
                    }
                }
            }
    } else {
        bf16_t* out = reinterpret_cast<bf16_t*>(shared ? a.out_shared : a.out_routed);
        const int ldo = shared ? a.S * a.h : a.h;
        const int col = (shared ? (g - a.E) * a.h : 0) + nt * (kBN / 2) + wn * 32 + lr;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (r < nrows) {
                    const int64_t row = row_base + r;
                    const float hv = silu(acc[mb][0][v]) * acc[mb][1][v];
                    out[row * ldo + col] = f32_to_bf16(hv);
                }
            }
    }
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

namespace {

// upper bound on the m-tiles of one launch
int64_t max_mtiles(const moe_shape& s, int bm, bool down) {
    const int64_t mtT = (s.T + bm - 1) / bm;
    const int64_t routed = (s.T * s.k) / bm + s.E;
    const int64_t shared = down ? (s.S > 0 ? mtT : 0) : s.S * mtT;
    return routed + shared;
}

}  // namespace

size_t ffn_lds_bytes() { return 2 * kLdsStage; }

hipError_t launch_grouped_ffn(const moe_shape& s, const void* x_perm, const float* qparams,
                              const int32_t* offsets, const void* x, const void* w1,
                              const void* w3, const void* w2, void* y_perm, void* y_shared,
                              int32_t* plan, void* h_routed, void* h_shared, hipStream_t st,
                              const Marks* mk) {
    const bool f32 = s.act == MOE_F32;
    const int bm = f32 ? kF32BM : kBM;
    ffn_plan_kernel<<<1, 256, 0, st>>>(offsets, s.E, s.S, s.T, bm, plan);
    mark(mk);

    GemmArgs a;
    a.qparams = qparams;
    a.offsets = offsets;
    a.plan = plan;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;

    // up-projection + SwiGLU
    a.a_routed = static_cast<const uint8_t*>(x_perm);
    a.a_shared = static_cast<const uint8_t*>(x);
    a.wa = static_cast<const uint8_t*>(w1);
    a.wb = static_cast<const uint8_t*>(w3);
    a.out_routed = static_cast<uint8_t*>(h_routed);
    a.out_shared = static_cast<uint8_t*>(h_shared);
    if (f32) {
        a.ntn = (s.h + kF32BN - 1) / kF32BN;
        const int64_t mt = max_mtiles(s, kF32BM, false);
        ffn_gemm_f32_kernel<true><<<static_cast<unsigned>(mt * a.ntn), 256, 0, st>>>(a, 0);
    } else {
        a.ntn = s.h / (kBN / 2);
        int64_t blocks = max_mtiles(s, kBM, false) * a.ntn;
        blocks = (blocks + 7) & ~int64_t(7);
        if (s.dispatch == MOE_FP8_E4M3)
            ffn_gemm_kernel<kModeUpFp8><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
        else
            ffn_gemm_kernel<kModeUp><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
    }
    mark(mk);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    // down-projection
    a.a_routed = static_cast<const uint8_t*>(h_routed);
    a.a_shared = static_cast<const uint8_t*>(h_shared);
    a.wa = static_cast<const uint8_t*>(w2);
    a.wb = nullptr;
    a.out_routed = static_cast<uint8_t*>(y_perm);
    a.out_shared = static_cast<uint8_t*>(y_shared);
    if (f32) {
        a.ntn = (s.d + kF32BN - 1) / kF32BN;
        const int64_t mt = max_mtiles(s, kF32BM, true);
        ffn_gemm_f32_kernel<false><<<static_cast<unsigned>(mt * a.ntn), 256, 0, st>>>(a, 0);
    } else {
        a.ntn = s.d / kBN;
        int64_t blocks = max_mtiles(s, kBM, true) * a.ntn;
        blocks = (blocks + 7) & ~int64_t(7);
        ffn_gemm_kernel<kModeDown><<<static_cast<unsigned>(blocks), kFfnThreads, 2 * kLdsStage, st>>>(a);
    }
    mark(mk);
    return hipGetLastError();
}

}  // namespace moe
