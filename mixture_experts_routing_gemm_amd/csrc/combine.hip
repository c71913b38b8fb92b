// Combine: un-permute and gate-weighted sum back to token order.
//
// Each token's output is the gate-weighted sum of its k experts' outputs
// ("Deepseek-MoE同步税本质与四层实战优化指南", gsyq.cn, section 2.3), placed
// back in the original token order from the metadata saved at dispatch (the
// DeepEP notes, zzszmyf.github.io, section 7 "Combine" and 7.5(2)). The shared
// experts' output, which every token receives with weight one ("DeepSeek 中
// MoE 的同步税", wmrh.cn, section 2.1), is added in the same pass.
//
// One wave per token: the k source rows are gathered with 16-byte loads
// (rows are contiguous), summed in float32 and rounded once. Every row is
// read once and every output written once, so the loads and stores are
// non-temporal: they are not kept in L2 or the Infinity Cache, which
// measured about 9 % faster on the largest workload. With no weights
// (topk_w == NULL) every slot has weight one: that is the backward of
// dispatch, dx[t] = dx_sh[t] + sum_j dx_perm[dest_row[t,j]].
//
// The backward of combine (the gradients going back along the routing path,
// gsyq.cn section 2.4) is its own kernel below.
#include "moe_device.h"

namespace moe {

template <typename TAct>
__global__ __launch_bounds__(256) void combine_kernel(
    const TAct* __restrict__ y_perm, const TAct* __restrict__ y_sh,
    const int32_t* __restrict__ dest_row, const float* __restrict__ topk_w, int64_t T, int d,
    int k, int64_t rows, TAct* __restrict__ y) {
    using V = ActVec<TAct>;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    int p = -1;
    float wt = 0.0f;
    if (lane < k) {
        p = dest_row[t * k + lane];
        wt = topk_w != nullptr ? topk_w[t * k + lane] : 1.0f;
        if (p < 0 || p >= rows) p = -1;
    }
    int pj[kMaxK];
    float wj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        pj[j] = __shfl(p, j, kWave);
        wj[j] = __shfl(wt, j, kWave);
    }
    // four chunks per lane per iteration: all of their loads are in flight
    // before the first sum (the sums themselves are unchanged: per element,
    // y_sh then w_j * row_j in slot order, rounded once); with two, the
    // 65536-token workload's combine took 483 us instead of 452
    const int nchunk = d / V::N;
    for (int c0 = lane; c0 < nchunk; c0 += 4 * kWave) {
        u32x4 src[4][kMaxK], sh[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int c = c0 + h * kWave;
            if (c >= nchunk) continue;
            const int64_t col = static_cast<int64_t>(c) * V::N;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j)
                if (j < k && pj[j] >= 0)
                    src[h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y_perm + static_cast<int64_t>(pj[j]) * d + col));
            if (y_sh != nullptr) sh[h] = load16(y_sh + t * d + col);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int c = c0 + h * kWave;
            if (c >= nchunk) continue;
            const int64_t col = static_cast<int64_t>(c) * V::N;
            float acc[V::N];
            if (y_sh != nullptr) {
                V::unpack(sh[h], acc);
            } else {
#pragma unroll
                for (int u = 0; u < V::N; ++u) acc[u] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k && pj[j] >= 0) {
                    float v[V::N];
                    V::unpack(src[h][j], v);
#pragma unroll
                    for (int u = 0; u < V::N; ++u) acc[u] = __builtin_fmaf(wj[j], v[u], acc[u]);
                }
            }
            __builtin_nontemporal_store(V::pack(acc), reinterpret_cast<u32x4*>(y + t * d + col));
        }
    }
}

// Backward of combine, one wave per token: dy_perm[dest_row[t,j]] =
// bf16/f32(w_j * dy[t]) and dtopk_w[t,j] = <dy[t], y_perm[dest_row[t,j]]>,
// accumulated in float32 per lane over its chunks and then across the wave;
// a dropped slot (dest_row < 0) gets 0 and writes no row.
template <typename TAct>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const TAct* __restrict__ dy, const TAct* __restrict__ y_perm,
    const int32_t* __restrict__ dest_row, const float* __restrict__ topk_w, int64_t T, int d,
    int k, int64_t rows, TAct* __restrict__ dy_perm, float* __restrict__ dtopk_w) {
    using V = ActVec<TAct>;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    int p = -1;
    float wt = 0.0f;
    if (lane < k) {
        p = dest_row[t * k + lane];
        wt = topk_w[t * k + lane];
        if (p < 0 || p >= rows) p = -1;
    }
    int pj[kMaxK];
    float wj[kMaxK], dot[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        pj[j] = __shfl(p, j, kWave);
        wj[j] = __shfl(wt, j, kWave);
        dot[j] = 0.0f;
    }
    const int nchunk = d / V::N;
    for (int c = lane; c < nchunk; c += kWave) {
        const int64_t col = static_cast<int64_t>(c) * V::N;
        float g[V::N];
        V::unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dy + t * d + col)), g);
        u32x4 src[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k && pj[j] >= 0)
                src[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y_perm + static_cast<int64_t>(pj[j]) * d + col));
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && pj[j] >= 0) {
                float v[V::N], o[V::N];
                V::unpack(src[j], v);
#pragma unroll
                for (int u = 0; u < V::N; ++u) {
                    dot[j] = __builtin_fmaf(g[u], v[u], dot[j]);
                    o[u] = wj[j] * g[u];
                }
                __builtin_nontemporal_store(V::pack(o), reinterpret_cast<u32x4*>(dy_perm + static_cast<int64_t>(pj[j]) * d + col));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
            float sum = dot[j];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
            if (lane == 0) dtopk_w[t * k + j] = pj[j] >= 0 ? sum : 0.0f;
        }
    }
}

hipError_t launch_combine_backward(const moe_shape& s, const void* dy, const void* y_perm,
                                   const int32_t* dest_row, const float* topk_w, void* dy_perm,
                                   float* dtopk_w, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>((s.T + 3) / 4);
    const int64_t rows = s.T * s.k;
    if (s.act == MOE_F32) {
        combine_backward_kernel<float><<<blocks, 256, 0, st>>>(
            static_cast<const float*>(dy), static_cast<const float*>(y_perm), dest_row, topk_w, s.T,
            s.d, s.k, rows, static_cast<float*>(dy_perm), dtopk_w);
    } else {
        combine_backward_kernel<bf16_t><<<blocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(y_perm), dest_row, topk_w,
            s.T, s.d, s.k, rows, static_cast<bf16_t*>(dy_perm), dtopk_w);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_sh,
                          const int32_t* dest_row, const float* topk_w, void* y, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>((s.T + 3) / 4);
    const int64_t rows = s.T * s.k;
    if (s.act == MOE_F32) {
        combine_kernel<float><<<blocks, 256, 0, st>>>(
            static_cast<const float*>(y_perm), static_cast<const float*>(y_sh), dest_row, topk_w,
            s.T, s.d, s.k, rows, static_cast<float*>(y));
    } else {
        combine_kernel<bf16_t><<<blocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(y_perm), static_cast<const bf16_t*>(y_sh), dest_row, topk_w,
            s.T, s.d, s.k, rows, static_cast<bf16_t*>(y));
    }
    return hipGetLastError();
}

}  // namespace moe
