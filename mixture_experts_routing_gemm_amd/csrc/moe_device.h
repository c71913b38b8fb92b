// Device-side helpers shared by the HIP kernels of the MoE layer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage: the upper 16 bits of a float32

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxK = 8;
constexpr int kMaxE = 256;
constexpr int kMaxS = 8;

// tokens per dispatch ranking block (4 waves x 64 tokens)
constexpr int kRankBlockTokens = 256;

// workspace header words (the header is the first 256 bytes of a workspace)
constexpr int kHdrErrorFlag = 0;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// (one v_cvt_pk_bf16_f32 for the pair, the same rounding as f32_to_bf16)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// wave-wide reductions over the 64 lanes
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Eight bf16 or four float32 values per 16-byte chunk, widened to float32
template <typename TAct>
struct ActVec;

template <>
struct ActVec<float> {
    static constexpr int N = 4;
    __device__ static void unpack(u32x4 r, float* v) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(r[u]);
    }
    __device__ static u32x4 pack(const float* v) {
        u32x4 r;
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = __float_as_uint(v[u]);
        return r;
    }
};

template <>
struct ActVec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void unpack(u32x4 r, float* v) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[2 * u] = bf16_lo(r[u]);
            v[2 * u + 1] = bf16_hi(r[u]);
        }
    }
    __device__ static u32x4 pack(const float* v) {
        u32x4 r;
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = pack_bf16x2(v[2 * u], v[2 * u + 1]);
        return r;
    }
};

template <int N>
using ic = std::integral_constant<int, N>;

// f(ic<B>()), f(ic<B+1>()), ..., f(ic<E-1>()): a loop whose index is a
// constant in every body
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>());
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ void set_error(uint32_t* hdr, uint32_t bit) {
    if (hdr) atomicOr(hdr + kHdrErrorFlag, bit);
}

// Grid of the gate-backward weight-gradient kernel (host and workspace
// sizing): tiles of W columns times token ranges of per_block tokens. Up to
// E = 128 the E x W float32 accumulator takes at most 32 KiB of LDS (four
// blocks per compute unit); above, 128 KiB (one). Short ranges keep each
// wave's walk over the tokens short, but every range stores an [E, d]
// float32 partial: the partials may take as many bytes as x (at least
// 32 MiB), and aim at about 2048 blocks, 256 tokens or fewer a range.
struct GateWgradGrid {
    int W, nslice;
    bool big;
    int64_t nchunk, per_block;
};
inline GateWgradGrid gate_wgrad_grid(int64_t T, int d, int E, int act_bytes) {
    GateWgradGrid g;
    g.big = E > 128;
    g.W = g.big ? 128 : (E <= 32 ? 256 : (E <= 64 ? 128 : 64));
    g.nslice = (d + g.W - 1) / g.W;
    const int64_t x_bytes = T * d * act_bytes;
    const int64_t budget = x_bytes > (int64_t(32) << 20) ? x_bytes : (int64_t(32) << 20);
    const int64_t by_budget = budget / (int64_t(E) * d * 4);
    const int64_t by_blocks = (2048 + g.nslice - 1) / g.nslice;
    const int64_t by_length = (T + 255) / 256;
    int64_t n = by_blocks > by_length ? by_blocks : by_length;
    if (n > by_budget) n = by_budget;
    const int64_t most = (T + 15) / 16;  // at least 16 tokens a range
    if (n > most) n = most;
    if (n > 65535) n = 65535;  // the grid's y extent
    if (n < 1) n = 1;
    g.per_block = (T + n - 1) / n;
    g.nchunk = g.per_block > 0 ? (T + g.per_block - 1) / g.per_block : 0;
    return g;
}

// The gate backward's weight gradient on the matrix cores, for bf16 x with d
// a multiple of 256. dz is split exactly into three bf16 planes (hi = bf16(dz),
// mid = bf16(dz - hi), lo = dz - hi - mid: 8 + 8 + 8 significant bits), laid
// out as [T, F] rows [hi | mid | lo | zeros] (plane p of expert e at feature
// p E + e; F = 3E rounded up to 256), and Zp^T x is summed per chunk of
// tokens by the expert FFN's weight-gradient kernel: every product of a
// plane value and an x value is exact in float32, so only the order of the
// float32 sums differs from a per-token sum. About two 256 x 256 tiles per
// CU, chunks of at least 256 tokens.
// byte offsets of a, b and hid (routed, then shared) in the buffer of
// activations a forward saves for the backward (ffn_backward.hip)
struct SavedLayout {
    size_t a_r = 0, b_r = 0, h_r = 0, a_s = 0, b_s = 0, h_s = 0, bytes = 0;
};
SavedLayout saved_layout(const moe_shape& s);

struct GateMfmaPlan {
    bool use;
    int F, C;       // plane features; token chunks
    int64_t chunk;  // tokens per chunk (the last one may be shorter)
};
inline GateMfmaPlan gate_mfma_plan(int64_t T, int d, int E, bool bf16) {
    GateMfmaPlan p{};
    p.F = ((3 * E + 255) / 256) * 256;
    const int64_t lim = int64_t(1) << 32;
    p.use = bf16 && T > 0 && d % 256 == 0 && T * d * 2 < lim && T * p.F * 2 < lim;
    if (!p.use) return p;
    const int64_t tiles = static_cast<int64_t>(p.F / 256) * (d / 256);  // per chunk
    int64_t C = (512 + tiles - 1) / tiles;
    const int64_t most = (T + 255) / 256;
    if (C > most) C = most;
    if (C > 256) C = 256;
    if (C < 1) C = 1;
    p.chunk = (T + C - 1) / C;
    p.C = static_cast<int>((T + p.chunk - 1) / p.chunk);
    return p;
}

// Host side: optional events recorded on the stream after each kernel, for
// per-kernel timing of the whole-layer call (a NULL entry is skipped).
struct Marks {
    hipEvent_t const* events;
    int n;
    mutable int next;
    hipStream_t st;
};
inline void mark(const Marks* mk) {
    if (mk != nullptr && mk->events != nullptr && mk->next < mk->n) {
        hipEvent_t e = mk->events[mk->next++];
        if (e != nullptr) (void)hipEventRecord(e, mk->st);
    }
}

}  // namespace moe
