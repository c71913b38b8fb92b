// Dispatch: expert histogram, exclusive scan and stable permutation.
//
// The single-GPU form of the dispatch step of the DeepEP notes
// (zzszmyf.github.io), section 7 "Dispatch": tokens are reordered by target
// expert and packed into one contiguous block per expert ([Local_Batch,
// Hidden] -> [Num_Experts * Tokens_Per_Expert, Hidden]); the target positions
// (dest_row) and source positions (src_token) are kept for combine (section
// 7.5(2)); only real rows are packed, no padding (section 7.5(4)); and every
// count is known on the device before any row moves (section 8.3), so the host
// never waits. With fp8 dispatch each row is quantised on the way, per token,
// by its min/max affine map ("Deepseek-MoE同步税本质与四层实战优化指南",
// gsyq.cn, section 3.1).
//
// Three kernels:
//   rank     per block of 256 tokens: the block's per-expert counts and each
//            (token, slot)'s rank among the block's earlier tokens with the
//            same expert. A 64-bit LDS mask per (wave, expert) marks which
//            lanes chose that expert, so a rank is a popcount -- stable and
//            deterministic with no ordering of atomics.
//   scan     one block: totals per expert, exclusive scan -> offsets, and
//            each rank block's base row per expert. With a per-expert
//            capacity C (the notes' DeepSeek-V3 load balancing, part A: a
//            strict token cap per expert) the counts are clamped to C first.
//   permute  one wave per token: 16-byte row loads once, k row stores. A
//            slot whose rank among its expert's assignments (token order)
//            reaches C is dropped: dest_row = -1, no row.
#include "moe_device.h"

namespace moe {

constexpr int kRankThreads = kRankBlockTokens;  // one token per thread
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kRankThreads) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int E, int k, int32_t* __restrict__ rank,
    int32_t* __restrict__ blk, uint32_t* __restrict__ hdr) {
    __shared__ unsigned long long mask[4][kMaxE];
    __shared__ int pre[4][kMaxE];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 4 * kMaxE; i += kRankThreads) (&mask[0][0])[i] = 0ull;
    __syncthreads();

    const int64_t t = static_cast<int64_t>(blockIdx.x) * kRankThreads + tid;
    int ev[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) ev[j] = -1;
    if (t < T) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k) {
                const int e = topk_idx[t * k + j];
                bool ok = static_cast<unsigned>(e) < static_cast<unsigned>(E);
#pragma unroll
                for (int jj = 0; jj < kMaxK; ++jj)
                    if (jj < j) ok = ok && (ev[jj] != e);
                if (ok) {
                    ev[j] = e;
                    atomicOr(&mask[w][e], 1ull << lane);
                } else {
                    set_error(hdr, 1u);
                }
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRankThreads) {
        const int c0 = __popcll(mask[0][e]);
        const int c1 = __popcll(mask[1][e]);
        const int c2 = __popcll(mask[2][e]);
        const int c3 = __popcll(mask[3][e]);
        pre[0][e] = 0;
        pre[1][e] = c0;
        pre[2][e] = c0 + c1;
        pre[3][e] = c0 + c1 + c2;
        blk[static_cast<int64_t>(blockIdx.x) * E + e] = c0 + c1 + c2 + c3;
    }
    __syncthreads();
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k) {
                const int e = ev[j];
                rank[t * k + j] = e < 0 ? -1 : pre[w][e] + __popcll(mask[w][e] & below);
            }
        }
    }
}

// blk[nblk][E] holds each rank block's per-expert counts on entry and, on
// exit, the block's first destination row per expert.
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    int32_t* __restrict__ blk, int nblk, int E, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets) {
    __shared__ int part[kScanThreads];  // [P][E] partial sums
    __shared__ int tot[kMaxE];
    __shared__ int off[kMaxE + 1];
    const int tid = threadIdx.x;
    const int P = kScanThreads / E;  // parts of the block range per expert
    const int e = tid % E, p = tid / E;
    const bool active = p < P;
    const int per = (nblk + P - 1) / P;
    const int b0 = active ? min(nblk, p * per) : 0, b1 = active ? min(nblk, b0 + per) : 0;
    int run = 0;
    for (int b = b0; b < b1; ++b) {
        const int64_t i = static_cast<int64_t>(b) * E + e;
        const int c = blk[i];
        blk[i] = run;
        run += c;
    }
    if (active) part[p * E + e] = run;
    __syncthreads();
    if (tid < E) {
        int s = 0;
        for (int q = 0; q < P; ++q) {
            const int c = part[q * E + tid];
            part[q * E + tid] = s;
            s += c;
        }
        tot[tid] = cap > 0 ? min(s, cap) : s;  // rows the expert keeps
    }
    __syncthreads();
    if (tid == 0) {
        int s = 0;
        for (int q = 0; q < E; ++q) {
            off[q] = s;
            s += tot[q];
        }
        off[E] = s;
    }
    __syncthreads();
    if (tid < E) {
        counts[tid] = tot[tid];
        offsets[tid] = off[tid];
    }
    if (tid == 0) offsets[E] = off[E];
    if (active) {
        const int base = off[e] + part[p * E + e];
        for (int b = b0; b < b1; ++b) blk[static_cast<int64_t>(b) * E + e] += base;
    }
}

// Destination rows of token t's k slots, computed by lanes 0..k-1 and
// broadcast to the wave. Lanes 0..k-1 also write dest_row and src_token.
// With cap > 0, a slot whose rank among all of its expert's assignments
// (blk - offsets + r: earlier blocks' count plus the rank within the block)
// is cap or more is dropped.
__device__ __forceinline__ int token_dest(const int32_t* __restrict__ topk_idx,
                                          const int32_t* __restrict__ rank,
                                          const int32_t* __restrict__ blk,
                                          const int32_t* __restrict__ offsets, int cap,
                                          int64_t t, int E, int k, int lane,
                                          int32_t* __restrict__ dest_row,
                                          int32_t* __restrict__ src_token) {
    int dst = -1;
    if (lane < k) {
        const int r = rank[t * k + lane];
        if (r >= 0) {
            const int e = topk_idx[t * k + lane];
            dst = blk[(t / kRankBlockTokens) * E + e] + r;
            if (cap > 0 && dst - offsets[e] >= cap) dst = -1;
            if (dst >= 0) src_token[dst] = static_cast<int32_t>(t);
        }
        dest_row[t * k + lane] = dst;
    }
    return dst;
}

__global__ __launch_bounds__(256) void dispatch_permute_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ offsets, int cap, int64_t T, int E, int k, int row_bytes,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    uint8_t* __restrict__ x_perm) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    const int dst =
        token_dest(topk_idx, rank, blk, offsets, cap, t, E, k, lane, dest_row, src_token);
    int dj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) dj[j] = __shfl(dst, j, kWave);
    const int nchunk = row_bytes >> 4;
    const uint8_t* src = x + t * row_bytes;
    for (int c0 = 0; c0 < nchunk; c0 += 4 * kWave) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c < nchunk) v[u] = load16(src + (static_cast<int64_t>(c) << 4));
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && dj[j] >= 0) {
                uint8_t* out = x_perm + static_cast<int64_t>(dj[j]) * row_bytes;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = c0 + u * kWave + lane;
                    if (c < nchunk) store16(out + (static_cast<int64_t>(c) << 4), v[u]);
                }
            }
        }
    }
}

// 16 bf16 values (two 16-byte chunks) -> 16 e4m3 codes (one 16-byte chunk)
__device__ __forceinline__ u32x4 quant16(u32x4 a, u32x4 b, float c, float inv, bool flat) {
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const u32x4 src = h == 0 ? a : b;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float v[4] = {bf16_lo(src[2 * u]), bf16_hi(src[2 * u]), bf16_lo(src[2 * u + 1]),
                          bf16_hi(src[2 * u + 1])};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = (v[q] - c) * inv;
                s = fminf(fmaxf(s, -448.0f), 448.0f);
                v[q] = flat ? 0.0f : s;
            }
            uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
            out[2 * h + u] = word;
        }
    }
    return out;
}

__global__ __launch_bounds__(256) void dispatch_permute_fp8_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ offsets, int cap, int64_t T, int E, int k, int d,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    uint8_t* __restrict__ x_perm, float* __restrict__ qparams) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    const int dst =
        token_dest(topk_idx, rank, blk, offsets, cap, t, E, k, lane, dest_row, src_token);
    int dj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) dj[j] = __shfl(dst, j, kWave);

    const uint8_t* src = reinterpret_cast<const uint8_t*>(x + t * d);
    const int ngroups = d >> 4;  // groups of 16 values (32 bytes in, 16 bytes out)
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int g = lane; g < ngroups; g += kWave) {
        const u32x4 a = load16(src + (static_cast<int64_t>(g) << 5));
        const u32x4 b = load16(src + (static_cast<int64_t>(g) << 5) + 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            mn = fminf(mn, fminf(bf16_lo(a[u]), bf16_hi(a[u])));
            mx = fmaxf(mx, fmaxf(bf16_lo(a[u]), bf16_hi(a[u])));
            mn = fminf(mn, fminf(bf16_lo(b[u]), bf16_hi(b[u])));
            mx = fmaxf(mx, fmaxf(bf16_lo(b[u]), bf16_hi(b[u])));
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    const float centre = 0.5f * (mx + mn);
    const float half = 0.5f * (mx - mn);
    const bool flat = half == 0.0f;
    const float scale = flat ? 0.0f : half / 448.0f;
    const float inv = flat ? 0.0f : 448.0f / half;
    if (lane < k && dst >= 0) {
        qparams[2 * static_cast<int64_t>(dst)] = scale;
        qparams[2 * static_cast<int64_t>(dst) + 1] = centre;
    }
    for (int g = lane; g < ngroups; g += kWave) {
        const u32x4 a = load16(src + (static_cast<int64_t>(g) << 5));
        const u32x4 b = load16(src + (static_cast<int64_t>(g) << 5) + 16);
        const u32x4 q = quant16(a, b, centre, inv, flat);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && dj[j] >= 0)
                store16(x_perm + static_cast<int64_t>(dj[j]) * d + (static_cast<int64_t>(g) << 4), q);
        }
    }
}

hipError_t launch_dispatch(const moe_shape& s, const void* x, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* dest_row,
                           int32_t* src_token, void* x_perm, float* qparams, int32_t* rank,
                           int32_t* blk, uint32_t* hdr, hipStream_t st, const Marks* mk) {
    const int nblk = static_cast<int>((s.T + kRankBlockTokens - 1) / kRankBlockTokens);
    dispatch_rank_kernel<<<nblk, kRankThreads, 0, st>>>(topk_idx, s.T, s.E, s.k, rank, blk, hdr);
    mark(mk);
    dispatch_scan_kernel<<<1, kScanThreads, 0, st>>>(blk, nblk, s.E, s.capacity, counts, offsets);
    mark(mk);
    const unsigned pblocks = static_cast<unsigned>((s.T + 3) / 4);
    if (s.dispatch == MOE_FP8_E4M3) {
        dispatch_permute_fp8_kernel<<<pblocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(x), topk_idx, rank, blk, offsets, s.capacity, s.T, s.E,
            s.k, s.d, dest_row, src_token, static_cast<uint8_t*>(x_perm), qparams);
    } else {
        const int row_bytes = s.d * (s.act == MOE_F32 ? 4 : 2);
        dispatch_permute_kernel<<<pblocks, 256, 0, st>>>(
            static_cast<const uint8_t*>(x), topk_idx, rank, blk, offsets, s.capacity, s.T, s.E,
            s.k, row_bytes, dest_row, src_token, static_cast<uint8_t*>(x_perm));
    }
    mark(mk);
    return hipGetLastError();
}

}  // namespace moe
