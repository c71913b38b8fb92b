// Per-row symmetric absmax e4m3 quantisation of bf16 rows: the expert weights
// of the fp8-weight path and its hidden rows.
//
// The pages define FP8 only for the dispatched activations: a per-token
// min/max affine map onto e4m3 ("Deepseek-MoE同步税本质与四层实战优化指南",
// gsyq.cn, section 3.1). Weight quantisation is left open; the reading taken
// here applies the same map to each weight row (one output feature) over the
// symmetric range [-max|w|, max|w|], so its centre is 0 and its scale
// max|w| / 448, and quantises the bf16 hidden rows of the fp8 expert GEMMs the
// same way. A row may be split into segments stored apart (the shared
// experts' W2 rows, one segment per shared expert, are quantised together so
// that the concatenated down-projection has one scale per output feature).
#include "moe_device.h"

namespace moe {

// 8 bf16 values -> 8 e4m3 codes of clamp(v * inv, +-448) (round to nearest
// even, in float32 -- the activation quantiser's arithmetic with centre 0)
__device__ __forceinline__ uint2 quant8_sym(u32x4 a, float inv, bool flat) {
    uint2 out;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float v[4] = {bf16_lo(a[2 * u]), bf16_hi(a[2 * u]), bf16_lo(a[2 * u + 1]),
                      bf16_hi(a[2 * u + 1])};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float s = (v[q] - 0.0f) * inv;
            s = fminf(fmaxf(s, -448.0f), 448.0f);
            v[q] = flat ? 0.0f : s;
        }
        uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
        (u == 0 ? out.x : out.y) = word;
    }
    return out;
}

// the sum of the values of 4 codes packed in a word
__device__ __forceinline__ float code_sum4(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    return (lo[0] + lo[1]) + (hi[0] + hi[1]);
}

// One wave per row r < nrows (nrows_dev, if given, bounds it further): the
// row's nseg segments of K values at src + r * row_stride + s * seg_stride
// (elements); codes go to the same element offsets of `codes`; scale[r +
// c * copy_stride] = max|row| / 448 for c < copies; qsum[r] (if given) = the
// sum of the row's code values (float32, a fixed order).
__global__ __launch_bounds__(256) void quant_rows_absmax_kernel(
    const bf16_t* __restrict__ src, int64_t nrows, const int32_t* __restrict__ nrows_dev, int K,
    int64_t row_stride, int nseg, int64_t seg_stride, uint8_t* __restrict__ codes,
    float* __restrict__ scale, int copies, int64_t copy_stride, float* __restrict__ qsum) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    int64_t n = nrows;
    if (nrows_dev != nullptr) n = min(n, static_cast<int64_t>(*nrows_dev));
    if (r >= n) return;
    const int per = K >> 3;  // 8-value chunks per segment
    const int nch = per * nseg;
    auto at = [&](int ch) {
        const int s = ch / per;
        return r * row_stride + s * seg_stride + static_cast<int64_t>(ch - s * per) * 8;
    };
    float amax = 0.0f;
    for (int ch = lane; ch < nch; ch += kWave) {
        const u32x4 a = load16(src + at(ch));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(a[u])), fabsf(bf16_hi(a[u]))));
    }
    amax = wave_max(amax);
    // the affine map of [mn, mx] = [-amax, amax]: centre 0, half range amax
    const float mx = amax, mn = -amax;
    const float half = 0.5f * (mx - mn);
    const bool flat = half == 0.0f;
    const float inv = flat ? 0.0f : 448.0f / half;
    if (lane < copies) scale[r + lane * copy_stride] = flat ? 0.0f : half / 448.0f;
    float sum = 0.0f;
    for (int ch = lane; ch < nch; ch += kWave) {
        const int64_t o = at(ch);
        const uint2 q = quant8_sym(load16(src + o), inv, flat);
        *reinterpret_cast<uint2*>(codes + o) = q;
        sum += code_sum4(q.x) + code_sum4(q.y);
    }
    if (qsum != nullptr) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
        if (lane == 0) qsum[r] = sum;
    }
}

namespace {
hipError_t launch_rows(const bf16_t* src, int64_t nrows, const int32_t* nrows_dev, int K,
                       int64_t row_stride, int nseg, int64_t seg_stride, uint8_t* codes,
                       float* scale, int copies, int64_t copy_stride, float* qsum,
                       hipStream_t st) {
    if (nrows <= 0) return hipSuccess;
    quant_rows_absmax_kernel<<<static_cast<unsigned>((nrows + 3) / 4), 256, 0, st>>>(
        src, nrows, nrows_dev, K, row_stride, nseg, seg_stride, codes, scale, copies, copy_stride,
        qsum);
    return hipGetLastError();
}
}  // namespace

// Float32 scales of the fp8 weights, in one array:
//   s1 [G, h] | qsum1 [G, h] | s3 [G, h] | qsum3 [G, h] | s2 [G, d]
// (qsum: the sum of a W1 / W3 row's code values, for the activations' centre
// term; s2 of the shared experts is one value per output feature, repeated
// for each of them).
size_t fp8w_scale_floats(const moe_shape& s) {
    const size_t G = static_cast<size_t>(s.E + s.S);
    return 4 * G * s.h + G * s.d;
}

hipError_t launch_quantize_weights(const moe_shape& s, const void* w1, const void* w3,
                                   const void* w2, uint8_t* w1q, uint8_t* w3q, uint8_t* w2q,
                                   float* wscale, hipStream_t st) {
    const int64_t G = s.E + s.S, h = s.h, d = s.d;
    float* s1 = wscale;
    float* q1 = s1 + G * h;
    float* s3 = q1 + G * h;
    float* q3 = s3 + G * h;
    float* s2 = q3 + G * h;
    hipError_t e;
    // W1, W3: G*h rows of d values
    if ((e = launch_rows(static_cast<const bf16_t*>(w1), G * h, nullptr, s.d, d, 1, 0, w1q, s1, 1,
                         0, q1, st)) != hipSuccess)
        return e;
    if ((e = launch_rows(static_cast<const bf16_t*>(w3), G * h, nullptr, s.d, d, 1, 0, w3q, s3, 1,
                         0, q3, st)) != hipSuccess)
        return e;
    // W2 of the routed experts: E*d rows of h values
    if ((e = launch_rows(static_cast<const bf16_t*>(w2), s.E * d, nullptr, s.h, h, 1, 0, w2q, s2,
                         1, 0, nullptr, st)) != hipSuccess)
        return e;
    // W2 of the shared experts: d rows of S segments of h values, one scale
    if (s.S > 0) {
        const int64_t base = s.E * d * h;
        e = launch_rows(static_cast<const bf16_t*>(w2) + base, d, nullptr, s.h, h, s.S, d * h,
                        w2q + base, s2 + s.E * d, s.S, d, nullptr, st);
    }
    return e;
}

// The hidden rows of the fp8 down-projection: routed rows [R, hs] (the first
// offsets[E] of them) and the shared rows [T, S*hs], one scale per row.
hipError_t launch_hidden_quant(const moe_shape& s, int hs, const void* h_r, const void* h_s,
                               const int32_t* offsets, uint8_t* h8_r, uint8_t* h8_s,
                               float* hsc_r, float* hsc_s, hipStream_t st) {
    const int64_t R = s.T * s.k;
    hipError_t e = launch_rows(static_cast<const bf16_t*>(h_r), R, offsets + s.E, hs, hs, 1, 0,
                               h8_r, hsc_r, 1, 0, nullptr, st);
    if (e != hipSuccess || s.S == 0) return e;
    return launch_rows(static_cast<const bf16_t*>(h_s), s.T, nullptr, s.S * hs,
                       static_cast<int64_t>(s.S) * hs, 1, 0, h8_s, hsc_s, 1, 0, nullptr, st);
}

}  // namespace moe
