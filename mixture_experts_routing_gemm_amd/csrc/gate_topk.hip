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
// i = 0..d-1 starting from +0.0 (then + bias). The GEMM below is register
// blocked across tokens and experts but never splits or reorders that chain,
// so the float32 logits, and the selection they decide, are reproducible.
// This keeps the gate on the vector ALUs rather than the matrix cores.
#include "moe_device.h"

namespace moe {

constexpr int kGateThreads = 256;
constexpr int kGateKC = 32;  // K elements staged in LDS per step

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

// Is (za, ia) ranked before (zb, ib)? Larger logit first, then lower id.
__device__ __forceinline__ bool ranks_before(float za, int ia, float zb, int ib) {
    return za > zb || (za == zb && ia < ib);
}

// Thread layout: EGP = 2^egp_log2 groups of 4 experts across the threads'
// low bits, TG = 256/EGP token groups of MT tokens each. A block handles
// TT = TG*MT tokens and all E experts (padded to EP = 4*EGP).
template <typename TIn, int MT>
__global__ __launch_bounds__(kGateThreads) void gate_topk_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, int egp_log2, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg) {
    constexpr int VEC = 16 / sizeof(TIn);  // elements per 16-byte chunk
    constexpr int CPR = kGateKC / VEC;     // chunks per staged row
    const int EGP = 1 << egp_log2;
    const int EP = EGP * 4;
    const int TT = (kGateThreads >> egp_log2) * MT;

    extern __shared__ float smem[];
    float* xs = smem;                 // [KC][TT]
    float* ws = smem + kGateKC * TT;  // [KC][EP]

    const int tid = threadIdx.x;
    const int eg = tid & (EGP - 1);
    const int tg = tid >> egp_log2;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TT;

    float acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = 0.0f;

    for (int i0 = 0; i0 < d; i0 += kGateKC) {
        const int kc = min(kGateKC, d - i0);
        const int cpr = kc / VEC;
        for (int q = tid; q < TT * CPR; q += kGateThreads) {
            const int r = q / CPR, c = q % CPR;
            if (c < cpr) {
                float v[VEC];
                const int64_t t = t0 + r;
                if (t < T) {
                    chunk_to_f32<TIn>(load16(x + t * d + i0 + c * VEC), v);
                } else {
#pragma unroll
                    for (int u = 0; u < VEC; ++u) v[u] = 0.0f;
                }
#pragma unroll
                for (int u = 0; u < VEC; ++u) xs[(c * VEC + u) * TT + r] = v[u];
            }
        }
        for (int q = tid; q < EP * CPR; q += kGateThreads) {
            const int e = q / CPR, c = q % CPR;
            if (c < cpr) {
                float v[VEC];
                if (e < E) {
                    chunk_to_f32<TIn>(load16(wg + static_cast<int64_t>(e) * d + i0 + c * VEC), v);
                } else {
#pragma unroll
                    for (int u = 0; u < VEC; ++u) v[u] = 0.0f;
                }
#pragma unroll
                for (int u = 0; u < VEC; ++u) ws[(c * VEC + u) * EP + e] = v[u];
            }
        }
        __syncthreads();
        for (int kk = 0; kk < kc; ++kk) {
            float xv[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) xv[m] = xs[kk * TT + tg * MT + m];
            const f32x4 wv = *reinterpret_cast<const f32x4*>(ws + kk * EP + eg * 4);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[m][c] = __builtin_fmaf(xv[m], wv[c], acc[m][c]);
        }
        __syncthreads();
    }

    // logits to LDS (reusing the staging space) and optionally to memory
    float* zs = smem;  // [TT][EP + 1]
    const int zld = EP + 1;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = tg * MT + m;
        const int64_t t = t0 + r;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = eg * 4 + c;
            float z = acc[m][c];
            if (bias != nullptr && e < E) z = z + bias[e];
            zs[r * zld + e] = z;
            if (logits_dbg != nullptr && e < E && t < T) logits_dbg[t * E + e] = z;
        }
    }
    __syncthreads();

    // top-k: one thread per token keeps a sorted list of the best k so far
    for (int r = tid; r < TT; r += kGateThreads) {
        const int64_t t = t0 + r;
        if (t >= T) continue;
        float bv[kMaxK];
        int bi[kMaxK];
#pragma unroll
        for (int p = 0; p < kMaxK; ++p) {
            bv[p] = -__builtin_inff();
            bi[p] = 0x7fffffff;
        }
        for (int e = 0; e < E; ++e) {
            float cv = zs[r * zld + e];
            int ci = e;
#pragma unroll
            for (int p = 0; p < kMaxK; ++p) {
                if (p < k && ranks_before(cv, ci, bv[p], bi[p])) {
                    const float tv = bv[p];
                    const int ti = bi[p];
                    bv[p] = cv;
                    bi[p] = ci;
                    cv = tv;
                    ci = ti;
                }
            }
        }
        float ex[kMaxK];
        float sum = 0.0f;
#pragma unroll
        for (int p = 0; p < kMaxK; ++p) {
            if (p < k) {
                ex[p] = expf(bv[p] - bv[0]);
                sum += ex[p];
            }
        }
#pragma unroll
        for (int p = 0; p < kMaxK; ++p) {
            if (p < k) {
                topk_idx[t * k + p] = bi[p];
                topk_w[t * k + p] = ex[p] / sum;
            }
        }
    }
}

namespace {

struct GateLaunch {
    int egp_log2, mt, tt;
    size_t smem;
};

GateLaunch gate_launch_shape(int E) {
    int egp_log2 = 0;
    while ((4 << egp_log2) < E) ++egp_log2;  // 4*EGP >= E, EGP <= 64
    const int tg = kGateThreads >> egp_log2;
    int mt = 1;
    while (tg * mt < 32) mt *= 2;  // at least 32 tokens per block
    GateLaunch g;
    g.egp_log2 = egp_log2;
    g.mt = mt;
    g.tt = tg * mt;
    const int ep = 4 << egp_log2;
    const size_t stage = static_cast<size_t>(kGateKC) * (g.tt + ep);
    const size_t zbuf = static_cast<size_t>(g.tt) * (ep + 1);
    g.smem = sizeof(float) * (stage > zbuf ? stage : zbuf);
    return g;
}

template <typename TIn>
hipError_t launch_gate_t(const moe_shape& s, const void* x, const void* wg, const float* bias,
                         int32_t* idx, float* w, float* dbg, hipStream_t st) {
    const GateLaunch g = gate_launch_shape(s.E);
    const unsigned blocks = static_cast<unsigned>((s.T + g.tt - 1) / g.tt);
    const TIn* xp = static_cast<const TIn*>(x);
    const TIn* gp = static_cast<const TIn*>(wg);
    switch (g.mt) {
        case 1:
            gate_topk_kernel<TIn, 1><<<blocks, kGateThreads, g.smem, st>>>(
                xp, gp, bias, s.T, s.d, s.E, s.k, g.egp_log2, idx, w, dbg);
            break;
        case 2:
            gate_topk_kernel<TIn, 2><<<blocks, kGateThreads, g.smem, st>>>(
                xp, gp, bias, s.T, s.d, s.E, s.k, g.egp_log2, idx, w, dbg);
            break;
        case 4:
            gate_topk_kernel<TIn, 4><<<blocks, kGateThreads, g.smem, st>>>(
                xp, gp, bias, s.T, s.d, s.E, s.k, g.egp_log2, idx, w, dbg);
            break;
        default:
            gate_topk_kernel<TIn, 8><<<blocks, kGateThreads, g.smem, st>>>(
                xp, gp, bias, s.T, s.d, s.E, s.k, g.egp_log2, idx, w, dbg);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_topk(const moe_shape& s, const void* x, const void* wg, const float* bias,
                            int32_t* idx, float* w, float* dbg, hipStream_t st) {
    if (s.act == MOE_F32) return launch_gate_t<float>(s, x, wg, bias, idx, w, dbg, st);
    return launch_gate_t<bf16_t>(s, x, wg, bias, idx, w, dbg, st);
}

}  // namespace moe
