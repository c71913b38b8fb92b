// Device code shared by the gate kernels: bf16/float32 staging helpers, the
// top-k over logits held in LDS, and the row-broadcast gate kernel with its
// host-side shape choice (instantiated per input type in gate_rows_*.hip).
//
// What it computes: "DeepSeek 中 MoE 的同步税" (wmrh.cn), section 4.1 (gate ->
// softmax -> top-k -> divide by the selected sum), fused as in section 4.3,
// router in float32 (section 5.1); each logit is one float32 fused
// multiply-add chain over i = 0..d-1 from +0.0, then + bias.
#pragma once

#include "moe_device.h"

namespace moe {

template <typename TIn>
__device__ __forceinline__ void chunk_to_f32(u32x4 raw, float* v);

template <>
__device__ __forceinline__ void chunk_to_f32<float>(u32x4 raw, float* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(raw[u]);
}

template <>
__device__ __forceinline__ void chunk_to_f32<bf16_t>(u32x4 raw, float* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v[2 * u] = bf16_lo(raw[u]);
        v[2 * u + 1] = bf16_hi(raw[u]);
    }
}

// Is (za, ia) ranked before (zb, ib)? Larger logit first, then lower id; a
// NaN logit ranks after every number, NaNs among themselves by id.
__device__ __forceinline__ bool ranks_before(float za, int ia, float zb, int ib) {
    const bool na = za != za, nb = zb != zb;
    if (na || nb) return na == nb ? ia < ib : nb;
    return za > zb || (za == zb && ia < ib);
}

// a selected logit as the softmax sees it: NaN counts as -inf (weight 0)
__device__ __forceinline__ float softmax_logit(float z) { return z != z ? -__builtin_inff() : z; }

// Top-k and weights of TT tokens whose logits sit in LDS (zs[r*zld + e]),
// under the order "larger logit first, then lower id, NaN last"
// (ranks_before), which is total, so the k experts that rank first, listed
// in that order, are unique. Two ways to find them, by cost:
//  - rank counting (small E): expert e of token r is selected iff fewer
//    than k experts rank before it, and that count is its slot; every
//    (token, expert) pair is one independent count, E*E*TT comparisons;
//  - k argmax rounds (large E: E*E > 2560*k, where the counting's E*E
//    reads outgrow about 40 dependent shuffle steps per round): one wave
//    per token row, each lane keeps the best of its not yet taken experts
//    (e = lane + 64*q), a butterfly of shuffles gives every lane the row's
//    best, and its owner marks it taken; round p's winner is slot p.
// The weights are the softmax over the k selected logits (slot 0 holds the
// largest), every slot summing the same k terms in slot order. `sel` is LDS
// for TT*kMaxK logits and TT*kMaxK ids. Called by all threads of the block.
__device__ __forceinline__ void topk_rows(const float* zs, int zld, int TT, int E, int k,
                                          int64_t t0, int64_t T, float* sel,
                                          int32_t* __restrict__ topk_idx,
                                          float* __restrict__ topk_w) {
    float* sz = sel;                                        // [TT][kMaxK] selected logits
    int* si = reinterpret_cast<int*>(sz + TT * kMaxK);      // [TT][kMaxK] selected ids
    if (E * E <= 2560 * k) {
        for (int q = threadIdx.x; q < TT * E; q += blockDim.x) {
            const int r = q / E, e = q - r * E;
            const float z = zs[r * zld + e];
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) rank += ranks_before(zs[r * zld + e2], e2, z, e) ? 1 : 0;
            if (rank < k) {
                sz[r * kMaxK + rank] = z;
                si[r * kMaxK + rank] = e;
            }
        }
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
    constexpr int kPerLane = (kMaxE + 63) / 64;
    for (int r = wave; r < TT && E * E > 2560 * k; r += nwaves) {
        float z[kPerLane];
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            const int e = lane + 64 * q;
            z[q] = e < E ? zs[r * zld + e] : 0.0f;
        }
        unsigned taken = 0u;
        for (int p = 0; p < k; ++p) {
            float bz = __builtin_nanf("");
            int be = E;  // ranks after every real expert, NaN ones included
#pragma unroll
            for (int q = 0; q < kPerLane; ++q) {
                const int e = lane + 64 * q;
                if (e < E && !((taken >> q) & 1u) && ranks_before(z[q], e, bz, be)) {
                    bz = z[q];
                    be = e;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float oz = __shfl_xor(bz, o, 64);
                const int oe = __shfl_xor(be, o, 64);
                if (ranks_before(oz, oe, bz, be)) {
                    bz = oz;
                    be = oe;
                }
            }
            if ((be & 63) == lane && be < E) taken |= 1u << (be >> 6);
            if (lane == 0) {
                sz[r * kMaxK + p] = bz;
                si[r * kMaxK + p] = be;
            }
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < TT * k; q += blockDim.x) {
        const int r = q / k, p = q - r * k;
        const int64_t t = t0 + r;
        if (t >= T) continue;
        const float zmax = softmax_logit(sz[r * kMaxK]);
        float sum = 0.0f;
        for (int p2 = 0; p2 < k; ++p2) sum += expf(softmax_logit(sz[r * kMaxK + p2]) - zmax);
        topk_idx[t * k + p] = si[r * kMaxK + p];
        topk_w[t * k + p] = expf(softmax_logit(sz[r * kMaxK + p]) - zmax) / sum;
    }
}

// ------------------------------------------------------ row-broadcast gate --
// The gate as used by the layer: one kernel, lanes = tokens x expert groups.
//
// A block of four waves takes TW tokens and all E experts. In a wave, lane l
// holds token l % TW and expert group l / TW (64 / TW groups per wave, 16
// lanes or more each), and runs ME chains, one per expert of its group. The
// block stages its tokens' K chunk and its experts' weight rows in LDS as
// float32 rows. Each lane reads its token's row in full; of the weights it
// reads only 4 of every 64 (lane q of a 16-lane row: K offsets 4q..4q+3),
// and the FMA takes its weight operand from lane n of its own row (DPP row
// broadcast). Each chain is one fma per K step, in K order, from +0.0, so
// the logits are those of the plain definition; top-k and the weights then
// run on the block's logits in LDS.

constexpr int kRbKB = 64;  // K per weight block (16 lanes x 4)

// acc = fma(w from lane N of this lane's 16-lane row, x, acc), one rounding
// (the operation fmaf performs). The compiler does not see the DPP inside
// the asm: w must not have been written by a VALU instruction in the two
// preceding wait states. Here w always comes straight from an LDS read, and
// a CPU test scans the built code for that hazard.
template <int N>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float w, float x) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc)
                 : "v"(w), "v"(x), "n"(N));
}

template <typename TIn>
__device__ __forceinline__ float elem_f32(const TIn* p) {
    if constexpr (sizeof(TIn) == 2) return bf16_to_f32(*p);
    else return *p;
}

// K per LDS stage: about 2048 FMA cycles per stage (ME * KC * 4), at least
// one weight block, at most 256, and at most 8192 staged token elements
__host__ __device__ constexpr int rb_kc(int me, int tw) {
    int kc = 512 / me;
    if (kc > 256) kc = 256;
    if (kc < kRbKB) kc = kRbKB;
    while (tw * kc > 8192) kc /= 2;
    return kc;
}

template <typename TIn, int ME, int TW>
__global__ __launch_bounds__(256) void gate_rows_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg) {
    constexpr int KC = rb_kc(ME, TW);
    constexpr int LD = KC + 4;                     // padded float32 row
    constexpr int NB = KC / kRbKB;                 // weight blocks per stage
    constexpr int EB = 4 * (64 / TW) * ME;         // experts per block
    constexpr int ROWS = TW + EB;                  // staged rows: tokens, then experts
    constexpr int VEC = 16 / sizeof(TIn);          // elements per 16-byte piece
    constexpr int PPR = KC / VEC;                  // pieces per staged row
    constexpr int PIECES = ROWS * PPR;
    constexpr int NP = (PIECES + 255) / 256;       // pieces per thread
    constexpr int STAGE = ROWS * LD;               // floats per LDS stage
    constexpr int EPI = TW * (EB + 1) + 2 * TW * kMaxK;
    constexpr int LDS = 2 * STAGE > EPI ? 2 * STAGE : EPI;
    __shared__ __attribute__((aligned(16))) float smem[LDS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int p = lane % TW;                       // token within the block
    const int grp = wave * (64 / TW) + lane / TW;  // expert group (uniform per 16 lanes)
    const int e0 = grp * ME;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TW;
    const int wq = 4 * (lane & 15);                // this lane's weights in a block

    // Staging loads are unconditional, from clamped addresses: rows past T
    // or E and K offsets past d load some valid element, whose products are
    // never computed (K tail) or never stored (rows past T or E).
    u32x4 reg[NP];
    auto fetch = [&](int i0) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int q = min(tid + u * 256, PIECES - 1), r = q / PPR, c = q % PPR;
            const int col = min(i0 + c * VEC, d - VEC);
            const TIn* src = r < TW ? x + min(t0 + r, T - 1) * d
                                    : wg + static_cast<int64_t>(min(r - TW, E - 1)) * d;
            reg[u] = load16(src + col);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int q = tid + u * 256;
            if (PIECES % 256 != 0 && q >= PIECES) continue;
            const int r = q / PPR, c = q % PPR;
            float v[VEC];
            chunk_to_f32<TIn>(reg[u], v);
            f32x4* dst = reinterpret_cast<f32x4*>(smem + buf * STAGE + r * LD + c * VEC);
#pragma unroll
            for (int w = 0; w < VEC / 4; ++w)
                dst[w] = f32x4{v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3]};
        }
    };

    float acc[ME];
#pragma unroll
    for (int m = 0; m < ME; ++m) acc[m] = 0.0f;

    fetch(0);
    stash(0);
    __syncthreads();
    int buf = 0;
    for (int i0 = 0; i0 < d; i0 += KC) {
        const int kc = min(KC, d - i0);
        const bool more = i0 + KC < d;
        if (more) fetch(i0 + KC);  // the next stage's loads are in flight during the FMAs
        const float* xrow = smem + buf * STAGE + p * LD;
        const float* wrow = smem + buf * STAGE + (TW + e0) * LD + wq;
        // x values of block h (all 64) and this lane's weights of block h
        auto read = [&](int h, f32x4* xv, f32x4* wv) __attribute__((always_inline)) {
#pragma unroll
            for (int n = 0; n < 16; ++n) xv[n] = *reinterpret_cast<const f32x4*>(xrow + h * kRbKB + 4 * n);
#pragma unroll
            for (int m = 0; m < ME; ++m) wv[m] = *reinterpret_cast<const f32x4*>(wrow + m * LD + h * kRbKB);
        };
        // 64 K steps of every chain
        auto block = [&](const f32x4* xv, const f32x4* wv) __attribute__((always_inline)) {
            static_for<0, 16 * 4 * ME>([&](auto I) __attribute__((always_inline)) {
                constexpr int n = decltype(I)::value / (4 * ME);
                constexpr int j = decltype(I)::value / ME % 4, m = decltype(I)::value % ME;
                fmac_row_bcast<n>(acc[m], wv[m][j], xv[n][j]);
            });
        };
        if (kc == KC) {
            // a whole stage: block h+1's operands are read during block h
            f32x4 xa[16], xb[16], wa[ME], wb[ME];
            read(0, xa, wa);
            static_for<0, NB>([&](auto H) __attribute__((always_inline)) {
                constexpr int h = decltype(H)::value;
                if constexpr (h % 2 == 0) {
                    if constexpr (h + 1 < NB) read(h + 1, xb, wb);
                    block(xa, wa);
                } else {
                    if constexpr (h + 1 < NB) read(h + 1, xa, wa);
                    block(xb, wb);
                }
            });
        } else {
            // the last, partial stage: whole blocks, then plain fmaf
            const int nfull = kc / kRbKB;
            static_for<0, NB>([&](auto H) __attribute__((always_inline)) {
                constexpr int h = decltype(H)::value;
                if (h < nfull) {
                    f32x4 xa[16], wa[ME];
                    read(h, xa, wa);
                    block(xa, wa);
                }
            });
            const float* wfull = smem + buf * STAGE + (TW + e0) * LD;
            for (int kk = nfull * kRbKB; kk < kc; ++kk) {
                const float xk = xrow[kk];
#pragma unroll
                for (int m = 0; m < ME; ++m) acc[m] = __builtin_fmaf(xk, wfull[m * LD + kk], acc[m]);
            }
        }
        if (more) stash(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    // logits (+ bias) to LDS, over the staging space, and optionally out
    float* zs = smem;
    constexpr int zld = EB + 1;
#pragma unroll
    for (int m = 0; m < ME; ++m) {
        const int e = e0 + m;
        if (e >= E) continue;
        float z = acc[m];
        if (bias != nullptr) z = z + bias[e];
        zs[p * zld + e] = z;
        const int64_t t = t0 + p;
        if (logits_dbg != nullptr && t < T) logits_dbg[t * E + e] = z;
    }
    __syncthreads();
    const int TT = static_cast<int>(min<int64_t>(TW, T - t0));
    topk_rows(zs, zld, TT, E, k, t0, T, zs + TW * zld, topk_idx, topk_w);
}

// Shape of the row-broadcast gate: TW tokens per block and ME experts per
// lane, 4 * (64 / TW) * ME >= E experts per block. The cost model counts FMA
// issue cycles per K step of a lane over the rounds of blocks on the CUs,
// with the measured cycles per dependent-chain FMA at ME chains (fewer
// chains leave latency exposed). ME = 0: no shape covers E.
struct RbShape {
    int me, tw;
};
constexpr RbShape kRbShapes[] = {{1, 16}, {2, 16}, {4, 16}, {8, 16}, {8, 32}, {4, 64}};
inline double rb_cycles_per_fma(int me) {
    return me >= 8 ? 4.9 : me >= 4 ? 5.3 : me >= 2 ? 6.5 : 9.75;
}
inline RbShape rb_shape(int E, int64_t T, int cus) {
    RbShape best{0, 0};
    double best_cost = 0.0;
    int best_eb = 0;
    for (const RbShape& c : kRbShapes) {
        const int eb = 4 * (64 / c.tw) * c.me;
        if (eb < E) continue;
        const int64_t blocks = (T + c.tw - 1) / c.tw;
        const double cost = static_cast<double>((blocks + cus - 1) / cus) * c.me * rb_cycles_per_fma(c.me);
        if (best.me == 0 || cost < best_cost || (cost == best_cost && eb < best_eb)) {
            best = c;
            best_cost = cost;
            best_eb = eb;
        }
    }
    return best;
}

template <typename TIn, int ME, int TW>
void launch_rb(const moe_shape& s, const TIn* x, const TIn* wg, const float* bias, int32_t* idx,
               float* w, float* dbg, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>((s.T + TW - 1) / TW);
    gate_rows_kernel<TIn, ME, TW><<<blocks, 256, 0, st>>>(x, wg, bias, s.T, s.d, s.E, s.k, idx, w,
                                                          dbg);
}

// false when no row-broadcast shape covers E
template <typename TIn>
bool launch_rb_t(const moe_shape& s, const void* x, const void* wg, const float* bias,
                 int32_t* idx, float* w, float* dbg, hipStream_t st) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const RbShape sh = rb_shape(s.E, s.T, cus);
    const TIn* xp = static_cast<const TIn*>(x);
    const TIn* gp = static_cast<const TIn*>(wg);
    const int key = sh.me * 100 + sh.tw;
    switch (key) {
        case 116: launch_rb<TIn, 1, 16>(s, xp, gp, bias, idx, w, dbg, st); break;
        case 216: launch_rb<TIn, 2, 16>(s, xp, gp, bias, idx, w, dbg, st); break;
        case 416: launch_rb<TIn, 4, 16>(s, xp, gp, bias, idx, w, dbg, st); break;
        case 816: launch_rb<TIn, 8, 16>(s, xp, gp, bias, idx, w, dbg, st); break;
        case 832: launch_rb<TIn, 8, 32>(s, xp, gp, bias, idx, w, dbg, st); break;
        case 464: launch_rb<TIn, 4, 64>(s, xp, gp, bias, idx, w, dbg, st); break;
        default: return false;
    }
    return true;
}
}  // namespace moe
