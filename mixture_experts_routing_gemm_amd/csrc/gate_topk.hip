// Gate GEMM + softmax + top-k + renormalised weights in one kernel.
//
// What it computes: "DeepSeek 中 MoE 的同步税" (wmrh.cn), section 4.1 (gate ->
// softmax -> top-k -> divide by the selected sum) fused into one pass as in
// section 4.3, with the router kept in float32 (section 5.1). The per-token
// top-k over an [N, E] score matrix is the job of the top-k gating kernel in
// the lpnh.cn routing deep dive, section 2.2; here each token's E logits are
// produced and consumed on chip, so no score matrix is written.
//
// Bit-exact routing: each logit is ONE float32 fused-multiply-add chain over
// i = 0..d-1 starting from +0.0 (then + bias). Neither kernel splits or
// reorders that chain, so the float32 logits, and the selection they decide,
// are reproducible. This keeps the gate on the vector ALUs rather than the
// matrix cores.
//
// The layer uses the row-broadcast kernel of gate_common.h (up to 128
// experts). This file holds the register-blocked kernel used above that, and
// the choice between the two.
#include "gate_common.h"

namespace moe {

constexpr int kGateThreads = 256;
constexpr int kGateSub = 32;   // K steps unrolled at a time
constexpr int kGateNReg = 6;   // staging registers (16 B each) per thread, bf16 input
// float32 rows hold half as many elements per register; give them twice as many
template <typename TIn>
constexpr int gate_nreg() { return sizeof(TIn) == 4 ? 2 * kGateNReg : kGateNReg; }
constexpr size_t kGateMaxLds = 160 * 1024;

// Thread layout: EGP = 2^egp_log2 groups of ME experts across the threads'
// low bits, TG = 256/EGP token groups of MT tokens each. A block handles
// TT = TG*MT tokens and all E experts (padded to EP = ME*EGP). K advances in
// chunks of KC staged in LDS as K-contiguous float rows (double-buffered
// through registers). One 16-byte LDS read gives an operand for 4 K steps;
// the reads for 32 steps are issued before their FMAs, and each thread runs
// MT*ME independent chains, each strictly in K order.
template <typename TIn, int MT, int ME>
__global__ __launch_bounds__(kGateThreads) void gate_topk_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, int egp_log2, int KC, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg) {
    constexpr int VEC = 16 / sizeof(TIn);  // elements per 16-byte chunk
    const int CPR = KC / VEC;              // chunks per staged row (KC: multiple of 32)
    const int LD = KC + 4;                 // padded LDS row (floats)
    const int EGP = 1 << egp_log2;
    const int EP = EGP * ME;
    const int TT = (kGateThreads >> egp_log2) * MT;
    const int stage = LD * (TT + EP);  // floats per LDS buffer

    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int eg = tid & (EGP - 1);
    const int tg = tid >> egp_log2;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TT;

    // staging: this thread's share of the (TT + EP) x CPR chunks of a K chunk
    const int nchunks = (TT + EP) * CPR;
    const int per_thread = (nchunks + kGateThreads - 1) / kGateThreads;  // <= NREG (launcher)
    constexpr int NREG = gate_nreg<TIn>();
    u32x4 reg[NREG];
    auto fetch = [&](int i0) {
        const int kc = min(KC, d - i0);
#pragma unroll
        for (int u = 0; u < NREG; ++u) {
            const int q = tid + u * kGateThreads;
            reg[u] = u32x4{0u, 0u, 0u, 0u};
            if (u < per_thread && q < nchunks) {
                const int r = q / CPR, c = q % CPR;
                if (c * VEC < kc) {
                    if (r < TT) {
                        const int64_t t = t0 + r;
                        if (t < T) reg[u] = load16(x + t * d + i0 + c * VEC);
                    } else if (r - TT < E) {
                        reg[u] = load16(wg + static_cast<int64_t>(r - TT) * d + i0 + c * VEC);
                    }
                }
            }
        }
    };
    // rows 0..TT-1 are tokens, TT..TT+EP-1 experts; row r, K offset j at r*LD + j
    auto stash = [&](int buf) {
        float* rows = smem + buf * stage;
#pragma unroll
        for (int u = 0; u < NREG; ++u) {
            const int q = tid + u * kGateThreads;
            if (u < per_thread && q < nchunks) {
                const int r = q / CPR, c = q % CPR;
                float v[VEC];
                chunk_to_f32<TIn>(reg[u], v);
                f32x4* dst = reinterpret_cast<f32x4*>(rows + r * LD + c * VEC);
#pragma unroll
                for (int w = 0; w < VEC / 4; ++w)
                    dst[w] = f32x4{v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3]};
            }
        }
    };

    float acc[MT][ME];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < ME; ++c) acc[m][c] = 0.0f;

    // 32 K steps from kk: operands for all of them first, then the FMAs
    auto fma32 = [&](const float* rows, int kk) {
        f32x4 xq[8][MT], wq[8][ME];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                xq[j][m] = *reinterpret_cast<const f32x4*>(rows + (tg * MT + m) * LD + kk + 4 * j);
#pragma unroll
            for (int c = 0; c < ME; ++c)
                wq[j][c] = *reinterpret_cast<const f32x4*>(rows + (TT + eg * ME + c) * LD + kk + 4 * j);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int c = 0; c < ME; ++c)
                        acc[m][c] = __builtin_fmaf(xq[j][m][q], wq[j][c][q], acc[m][c]);
    };
    auto fma1 = [&](const float* rows, int kk) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int c = 0; c < ME; ++c)
                acc[m][c] = __builtin_fmaf(rows[(tg * MT + m) * LD + kk], rows[(TT + eg * ME + c) * LD + kk],
                                           acc[m][c]);
    };

    fetch(0);
    stash(0);
    __syncthreads();
    int buf = 0;
    for (int i0 = 0; i0 < d; i0 += KC) {
        const int kc = min(KC, d - i0);
        const bool more = i0 + KC < d;
        if (more) fetch(i0 + KC);  // global loads in flight during the FMAs
        const float* rows = smem + buf * stage;
        int kk = 0;
        for (; kk + kGateSub <= kc; kk += kGateSub) fma32(rows, kk);
        for (; kk < kc; ++kk) fma1(rows, kk);
        if (more) stash(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    // logits to LDS (reusing the staging space) and optionally to memory
    float* zs = smem;  // [TT][EP + 1]
    const int zld = EP + 1;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = tg * MT + m;
        const int64_t t = t0 + r;
#pragma unroll
        for (int c = 0; c < ME; ++c) {
            const int e = eg * ME + c;
            float z = acc[m][c];
            if (bias != nullptr && e < E) z = z + bias[e];
            zs[r * zld + e] = z;
            if (logits_dbg != nullptr && e < E && t < T) logits_dbg[t * E + e] = z;
        }
    }
    __syncthreads();

    topk_rows(zs, zld, TT, E, k, t0, T, zs + TT * zld, topk_idx, topk_w);
}

namespace {

struct GateLaunch {
    int egp_log2, mt, me, tt, kc;
    size_t smem;
};

// Tile shape for E experts and T tokens: the most independent chains per
// thread (MT tokens x ME experts) that still gives at least 512 work-groups
// (two per CU), falling back to the most work-groups when T is small; the
// staging and logit buffers must fit the registers and the LDS. Every E in
// 1..256 has a candidate (ME = 2, MT = 1 always fits). Each work-group walks
// K in chunks of kc (longest that fits) so the next chunk's loads overlap
// enough FMAs.
GateLaunch gate_launch_shape(int E, int64_t T, int vec) {
    GateLaunch best{};
    int64_t best_blocks = -1;
    int best_chains = -1;
    for (int me : {4, 2}) {
        int egp_log2 = 0;
        while ((me << egp_log2) < E) ++egp_log2;
        if (egp_log2 > 7) continue;
        const int tg = kGateThreads >> egp_log2;
        if (tg == 0) continue;
        const int ep = me << egp_log2;
        for (int mt : {8, 4, 2, 1}) {
            const int tt = tg * mt;
            if (tt > kGateThreads) continue;
            // the longest K chunk (multiple of 32, at most 256) whose staging
            // fits the registers and whose double buffer fits 128 KB of LDS
            int kc = 0;
            for (int c = 256; c >= kGateSub; c /= 2) {
                const size_t stage = 2 * static_cast<size_t>(c + 4) * (tt + ep) * sizeof(float);
                const int nreg = vec == 4 ? 2 * kGateNReg : kGateNReg;
                if ((tt + ep) * (c / vec) <= nreg * kGateThreads && stage <= 128 * 1024) {
                    kc = c;
                    break;
                }
            }
            if (kc == 0) continue;
            const size_t stage = 2 * static_cast<size_t>(kc + 4) * (tt + ep);
            const size_t zbuf = static_cast<size_t>(tt) * (ep + 1 + 2 * kMaxK);
            const size_t smem = sizeof(float) * (stage > zbuf ? stage : zbuf);
            if (smem > kGateMaxLds) continue;
            const int64_t blocks = (T + tt - 1) / tt;
            const int chains = mt * me;
            const bool ok = blocks >= 512;
            const bool best_ok = best_blocks >= 512;
            bool take;
            if (best_blocks < 0) take = true;
            else if (ok != best_ok) take = ok;
            else if (ok) take = chains > best_chains;
            else take = blocks > best_blocks || (blocks == best_blocks && chains > best_chains);
            if (take) {
                best.egp_log2 = egp_log2;
                best.mt = mt;
                best.me = me;
                best.tt = tt;
                best.kc = kc;
                best.smem = smem;
                best_blocks = blocks;
                best_chains = chains;
            }
        }
    }
    return best;
}

template <typename TIn, int MT, int ME>
void launch_shape(const GateLaunch& g, unsigned blocks, const moe_shape& s, const TIn* xp,
                  const TIn* gp, const float* bias, int32_t* idx, float* w, float* dbg,
                  hipStream_t st) {
    if (g.smem > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_topk_kernel<TIn, MT, ME>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(g.smem)) != hipSuccess)
        return;  // the launch error is reported by hipGetLastError
    gate_topk_kernel<TIn, MT, ME><<<blocks, kGateThreads, g.smem, st>>>(
        xp, gp, bias, s.T, s.d, s.E, s.k, g.egp_log2, g.kc, idx, w, dbg);
}

template <typename TIn>
hipError_t launch_gate_t(const moe_shape& s, const void* x, const void* wg, const float* bias,
                         int32_t* idx, float* w, float* dbg, hipStream_t st) {
    const GateLaunch g = gate_launch_shape(s.E, s.T, 16 / static_cast<int>(sizeof(TIn)));
    if (g.tt <= 0) return hipErrorInvalidConfiguration;
    const unsigned blocks = static_cast<unsigned>((s.T + g.tt - 1) / g.tt);
    const TIn* xp = static_cast<const TIn*>(x);
    const TIn* gp = static_cast<const TIn*>(wg);
    if (g.me == 4) {
        switch (g.mt) {
            case 1: launch_shape<TIn, 1, 4>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            case 2: launch_shape<TIn, 2, 4>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            case 4: launch_shape<TIn, 4, 4>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            default: launch_shape<TIn, 8, 4>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
        }
    } else {
        switch (g.mt) {
            case 1: launch_shape<TIn, 1, 2>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            case 2: launch_shape<TIn, 2, 2>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            case 4: launch_shape<TIn, 4, 2>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
            default: launch_shape<TIn, 8, 2>(g, blocks, s, xp, gp, bias, idx, w, dbg, st); break;
        }
    }
    return hipGetLastError();
}


}  // namespace

// row-broadcast gate, per input type (gate_rows_*.hip); false when no
// row-broadcast shape covers E
bool launch_gate_rows_f32(const moe_shape& s, const void* x, const void* wg, const float* bias,
                          int32_t* idx, float* w, float* dbg, hipStream_t st);
bool launch_gate_rows_bf16(const moe_shape& s, const void* x, const void* wg, const float* bias,
                           int32_t* idx, float* w, float* dbg, hipStream_t st);

bool launch_gate_two_phase(const moe_shape& s, const void* x, const void* wg, const float* bias,
                           int32_t* idx, float* w, hipStream_t st, hipError_t* err);

hipError_t launch_gate_topk(const moe_shape& s, const void* x, const void* wg, const float* bias,
                            int32_t* idx, float* w, float* dbg, hipStream_t st, const Marks* mk) {
    (void)mk;
    if (s.T == 0) return hipSuccess;
    // bf16 without the logits dump: approximate logits on the matrix cores,
    // exact chains only for the experts that can still be selected
    hipError_t err = hipSuccess;
    if (dbg == nullptr && launch_gate_two_phase(s, x, wg, bias, idx, w, st, &err)) return err;
    const bool f32 = s.act == MOE_F32;
    if (f32 ? launch_gate_rows_f32(s, x, wg, bias, idx, w, dbg, st)
            : launch_gate_rows_bf16(s, x, wg, bias, idx, w, dbg, st))
        return hipGetLastError();
    // more experts than a row-broadcast block covers: register-blocked kernel
    if (f32) return launch_gate_t<float>(s, x, wg, bias, idx, w, dbg, st);
    return launch_gate_t<bf16_t>(s, x, wg, bias, idx, w, dbg, st);
}

}  // namespace moe
