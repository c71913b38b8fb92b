// Backward of the gate, with each token's top-k choice held fixed.
//
// The gradients return along the routing path ("Deepseek-MoE同步税本质与四层
// 实战优化指南", gsyq.cn, section 2.4); the gate's part is the derivative of
// the renormalised top-k weights (gate, softmax, top-k, renormalise by the
// selected sum: "DeepSeek 中 MoE 的同步税", wmrh.cn, section 4.1; the top-k
// gating step of gsyq.cn, section 2.1). Restricted to the
// chosen experts the full softmax's normaliser cancels, so the weights are a
// softmax over the k chosen logits and, for slot j of token t,
//   dz[t,j] = w[t,j] (dw[t,j] - sum_l w[t,l] dw[t,l])
// is the gradient of logit topk_idx[t,j]; every other logit's gradient is
// zero. Through z = x Wg^T that sparse dz gives
//   dx[t]  += sum_j dz[t,j] Wg[topk_idx[t,j]]   (k rows of Wg, L2-resident)
//   dWg[e]  = sum over slots with topk_idx = e of dz[t,j] x[t].
// dx is HBM-bound (x and dx are each streamed once). dWg, for bf16 x with d
// a multiple of 256, is dense on the matrix cores: dz spread over [T, E] and
// split exactly into three bf16 planes (GateMfmaPlan), so that dWg = Zp^T x
// has exact products; the token kernel writes the plane rows, the expert
// FFN's weight-gradient kernel sums them against x per chunk of tokens, and
// the chunks and planes are added in a fixed order. Otherwise dWg is summed
// per range of tokens in LDS (each sum by one thread, in token order),
// stored as one float32 partial per range, and the partials are then added
// in range order. No atomics either way: the result is the same on every
// call.
#include "moe_device.h"

namespace moe {

// weight-gradient accumulators: E x W float32 in LDS, E * W at most 8192
// (E <= 128) or 32768 (E <= 256)
constexpr int kWgradSmall = 8192;
constexpr int kWgradBig = 32768;
// tokens whose (expert, dz) pairs are staged in LDS at a time
constexpr int kWgradStage = 64;

// the most plane features of a token row (E <= 256)
constexpr int kMaxPlaneF = 768;

// One wave per token: dz, then dx[t] = act(dx[t] + sum_j dz_j Wg[e_j]) in
// float32 (slot order, rounded once). With zp, also the token's plane row
// (GateMfmaPlan; F features): slots with the same expert are summed first
// (in slot order, into the first of them), and the row is built in LDS and
// stored whole.
template <typename TAct>
__global__ __launch_bounds__(256) void gate_backward_token_kernel(
    const TAct* __restrict__ wg, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ dtopk_w, int64_t T, int d, int E,
    int k, float* __restrict__ dz, TAct* __restrict__ dx, bf16_t* __restrict__ zp, int F) {
    using V = ActVec<TAct>;
    __shared__ __attribute__((aligned(16))) uint16_t zrow[4][kMaxPlaneF];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    int e = -1;
    float wt = 0.0f, gw = 0.0f;
    if (lane < k) {
        e = topk_idx[t * k + lane];
        wt = topk_w[t * k + lane];
        gw = dtopk_w[t * k + lane];
    }
    float mean = wt * gw;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mean += __shfl_xor(mean, o, kWave);
    const float g = wt * (gw - mean);
    if (lane < k) dz[t * k + lane] = g;
    if (e < 0 || e >= E) e = -1;
    int ej[kMaxK];
    float gj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        ej[j] = __shfl(e, j, kWave);
        gj[j] = __shfl(g, j, kWave);
    }
    if (zp != nullptr) {
        uint16_t* row = zrow[w];
        for (int c = lane; c < F / 8; c += kWave) *reinterpret_cast<u32x4*>(row + 8 * c) = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros are written
        __builtin_amdgcn_wave_barrier();
        if (lane < k && e >= 0) {
            float gs = 0.0f;
            bool first = true;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k && ej[j] == e) {
                    gs += gj[j];
                    if (j < lane) first = false;
                }
            }
            if (first) {
                const bf16_t hi = f32_to_bf16(gs);
                const float r1 = gs - bf16_to_f32(hi);
                const bf16_t mid = f32_to_bf16(r1);
                const bf16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
                row[e] = hi;
                row[E + e] = mid;
                row[2 * E + e] = lo;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        for (int c = lane; c < F / 8; c += kWave)
            store16(zp + t * F + 8 * c, *reinterpret_cast<const u32x4*>(row + 8 * c));
    }
    if (dx == nullptr) return;
    const int nchunk = d / V::N;
    for (int c = lane; c < nchunk; c += kWave) {
        const int64_t col = static_cast<int64_t>(c) * V::N;
        u32x4 src[kMaxK];
        const u32x4 cur = load16(dx + t * d + col);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k && ej[j] >= 0) src[j] = load16(wg + static_cast<int64_t>(ej[j]) * d + col);
        float acc[V::N];
        V::unpack(cur, acc);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && ej[j] >= 0) {
                float v[V::N];
                V::unpack(src[j], v);
#pragma unroll
                for (int u = 0; u < V::N; ++u) acc[u] = __builtin_fmaf(gj[j], v[u], acc[u]);
            }
        }
        store16(dx + t * d + col, V::pack(acc));
    }
}

// CPL consecutive columns of row p widened to float32 (2 to 16 bytes)
template <typename TAct, int CPL>
__device__ __forceinline__ void load_cols(const TAct* p, float* v) {
    if constexpr (CPL == 1) {
        if constexpr (sizeof(TAct) == 4)
            v[0] = *p;
        else
            v[0] = bf16_to_f32(*p);
    } else if constexpr (sizeof(TAct) == 4) {
        if constexpr (CPL == 4) {
            const f32x4 r = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = r[u];
        } else {
            const float2 r = *reinterpret_cast<const float2*>(p);
            v[0] = r.x;
            v[1] = r.y;
        }
    } else {
        if constexpr (CPL == 4) {
            const uint2 r = *reinterpret_cast<const uint2*>(p);
            v[0] = bf16_lo(r.x);
            v[1] = bf16_hi(r.x);
            v[2] = bf16_lo(r.y);
            v[3] = bf16_hi(r.y);
        } else {
            const uint32_t r = *reinterpret_cast<const uint32_t*>(p);
            v[0] = bf16_lo(r);
            v[1] = bf16_hi(r);
        }
    }
}

// dWg over a tile of W = 64 * CPL columns and a range of tokens. Lane l of
// every wave owns columns l*CPL .. l*CPL+CPL-1 of the tile; wave q owns the
// experts e with e % 4 == q. Each wave walks every token of the range (the
// rows come from HBM once, the other three waves hit the cache), and the
// E x W float32 sums in LDS (at e * W + column) each have exactly one owner
// thread, which adds its slots in token order: plain read-modify-writes, no
// atomics, the same result on every call. A token's k (expert, dz) pairs
// are staged at a stride of kMaxK and read with 16-byte LDS loads, KS
// slots (4 when k <= 4, else 8) a token. The tile then goes to this block's
// partial, part[blockIdx.y][e][column].
template <typename TAct, int CPL, int ACC, int KS>
__global__ __launch_bounds__(256) void gate_backward_wgrad_kernel(
    const TAct* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dz, int64_t T, int d, int E, int k, int64_t per_block,
    float* __restrict__ part) {
    constexpr int W = 64 * CPL;
    constexpr int kAhead = 8;  // rows loaded before they are used
    __shared__ float acc[ACC];
    __shared__ __align__(16) int32_t s_e[kWgradStage * kMaxK];
    __shared__ __align__(16) float s_g[kWgradStage * kMaxK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c0 = blockIdx.x * W;
    const int col = c0 + lane * CPL;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * per_block;
    const int64_t t1 = t0 + per_block < T ? t0 + per_block : T;
    for (int i = tid; i < E * W; i += 256) acc[i] = 0.0f;
    for (int64_t s0 = t0; s0 < t1; s0 += kWgradStage) {
        const int ns = static_cast<int>(t1 - s0 < kWgradStage ? t1 - s0 : kWgradStage);
        __syncthreads();  // the accumulator is cleared / the last batch is consumed
        for (int i = tid; i < ns * kMaxK; i += 256) {
            const int tt = i / kMaxK, j = i % kMaxK;
            int32_t e = -1;
            float g = 0.0f;
            if (j < k) {
                e = topk_idx[(s0 + tt) * k + j];
                g = dz[(s0 + tt) * k + j];
            }
            s_e[i] = (e >= 0 && e < E) ? e : -1;
            s_g[i] = g;
        }
        __syncthreads();
        if (col < d) {
            for (int tb = 0; tb < ns; tb += kAhead) {
                // every load is issued before the first is used: a row past
                // the batch reloads its last row (in bounds, never used), so
                // no load sits behind a branch of its own
                float xv[kAhead][CPL];
#pragma unroll
                for (int b = 0; b < kAhead; ++b) {
                    const int r = tb + b < ns ? tb + b : ns - 1;
                    load_cols<TAct, CPL>(x + (s0 + r) * d + col, xv[b]);
                }
#pragma unroll
                for (int b = 0; b < kAhead; ++b) {
                    if (tb + b >= ns) break;
                    const int4* pe = reinterpret_cast<const int4*>(s_e + (tb + b) * kMaxK);
                    const f32x4* pg = reinterpret_cast<const f32x4*>(s_g + (tb + b) * kMaxK);
                    int ev[KS];
                    float gv[KS];
#pragma unroll
                    for (int q = 0; q < KS / 4; ++q) {
                        const int4 eq = pe[q];
                        const f32x4 gq = pg[q];
                        ev[4 * q] = eq.x;
                        ev[4 * q + 1] = eq.y;
                        ev[4 * q + 2] = eq.z;
                        ev[4 * q + 3] = eq.w;
#pragma unroll
                        for (int u = 0; u < 4; ++u) gv[4 * q + u] = gq[u];
                    }
#pragma unroll
                    for (int j = 0; j < KS; ++j) {
                        const int e = ev[j];
                        if (e < 0 || (e & 3) != wave) continue;
                        float* a = acc + e * W + lane * CPL;
#pragma unroll
                        for (int u = 0; u < CPL; ++u) a[u] = __builtin_fmaf(gv[j], xv[b][u], a[u]);
                    }
                }
            }
        }
    }
    __syncthreads();
    float* out = part + static_cast<int64_t>(blockIdx.y) * E * d + c0;
    for (int i = tid; i < E * W; i += 256) {
        const int e = i / W, c = i % W;
        if (c0 + c < d) out[static_cast<int64_t>(e) * d + c] = acc[i];
    }
}

// The chunk boundaries of the matrix-core weight gradient: offsets[c] =
// min(T, c * chunk), c = 0..C.
__global__ __launch_bounds__(256) void gate_chunk_offsets_kernel(int64_t T, int64_t chunk, int C,
                                                                 int32_t* __restrict__ offsets) {
    for (int c = threadIdx.x; c <= C; c += 256) {
        const int64_t o = static_cast<int64_t>(c) * chunk;
        offsets[c] = static_cast<int32_t>(o < T ? o : T);
    }
}

// dWg[e] = sum over the chunks, in order, of (hi + (mid + lo)) of the plane
// partials: plane p of expert e is feature f = p E + e, in p1 [C, F/2, d]
// when f < F/2, else in p3 (four columns a thread).
__global__ __launch_bounds__(256) void gate_plane_reduce_kernel(const float* __restrict__ p1,
                                                                const float* __restrict__ p3, int C,
                                                                int E, int d, int F,
                                                                f32x4* __restrict__ dwg) {
    const int64_t n4 = static_cast<int64_t>(E) * d / 4;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    const int e = static_cast<int>(i / (d / 4));
    const int col = static_cast<int>(i - static_cast<int64_t>(e) * (d / 4)) * 4;
    const int hh = F / 2;
    auto plane = [&](int c, int f) {
        const float* src = f < hh ? p1 + (static_cast<int64_t>(c) * hh + f) * d
                                  : p3 + (static_cast<int64_t>(c) * hh + (f - hh)) * d;
        return *reinterpret_cast<const f32x4*>(src + col);
    };
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < C; ++c) {
        const f32x4 hi = plane(c, e), mid = plane(c, E + e), lo = plane(c, 2 * E + e);
        s += hi + (mid + lo);
    }
    dwg[i] = s;
}

// dWg = sum of the nchunk partials, in block order (four columns a thread).
__global__ __launch_bounds__(256) void gate_backward_reduce_kernel(
    const f32x4* __restrict__ part, int64_t nchunk, int64_t n4, f32x4* __restrict__ dwg) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t c = 0;
    for (; c + 8 <= nchunk; c += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(c + u) * n4 + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < nchunk; ++c) s += part[c * n4 + i];
    dwg[i] = s;
}

template <typename TAct, int KS>
void launch_wgrad_k(const GateWgradGrid& g, const TAct* x, const int32_t* topk_idx,
                    const float* dz, const moe_shape& s, float* part, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(g.nslice), static_cast<unsigned>(g.nchunk));
    if (g.big)
        gate_backward_wgrad_kernel<TAct, 2, kWgradBig, KS><<<grid, 256, 0, st>>>(
            x, topk_idx, dz, s.T, s.d, s.E, s.k, g.per_block, part);
    else if (g.W == 256)
        gate_backward_wgrad_kernel<TAct, 4, kWgradSmall, KS><<<grid, 256, 0, st>>>(
            x, topk_idx, dz, s.T, s.d, s.E, s.k, g.per_block, part);
    else if (g.W == 128)
        gate_backward_wgrad_kernel<TAct, 2, kWgradSmall, KS><<<grid, 256, 0, st>>>(
            x, topk_idx, dz, s.T, s.d, s.E, s.k, g.per_block, part);
    else
        gate_backward_wgrad_kernel<TAct, 1, kWgradSmall, KS><<<grid, 256, 0, st>>>(
            x, topk_idx, dz, s.T, s.d, s.E, s.k, g.per_block, part);
}

template <typename TAct>
void launch_wgrad(const GateWgradGrid& g, const TAct* x, const int32_t* topk_idx, const float* dz,
                  const moe_shape& s, float* part, hipStream_t st) {
    if (s.k <= 4)
        launch_wgrad_k<TAct, 4>(g, x, topk_idx, dz, s, part, st);
    else
        launch_wgrad_k<TAct, kMaxK>(g, x, topk_idx, dz, s, part, st);
}

hipError_t launch_wgrad_planes(const int32_t* offsets, int C, int64_t T, int d, int F,
                               const void* zp, const void* x, float* p1, float* p3, void* ws,
                               hipStream_t st);

namespace {
// the parts of the matrix-core path's workspace: plane partials [C, F, d]
// float32 (p1 then p3), plane rows [T, F] bf16, chunk offsets and the
// weight-gradient kernel's order and queues
struct GateMfmaWs {
    size_t p1, p3, zp, offsets, meta, total;
};
GateMfmaWs gate_mfma_ws(const GateMfmaPlan& p, int64_t T, int d) {
    GateMfmaWs w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (off + bytes + 255) / 256 * 256;
        return at;
    };
    const size_t half = static_cast<size_t>(p.C) * (p.F / 2) * d * 4;
    w.p1 = take(half);
    w.p3 = take(half);
    w.zp = take(static_cast<size_t>(T) * p.F * 2);
    w.offsets = take(static_cast<size_t>(p.C + 1) * 4);
    w.meta = take(static_cast<size_t>(p.C + 32) * 4);
    w.total = off;
    return w;
}
}  // namespace

size_t gate_backward_ws_bytes(const moe_shape& s) {
    const GateMfmaPlan p = gate_mfma_plan(s.T, s.d, s.E, s.act == MOE_BF16);
    if (p.use) return gate_mfma_ws(p, s.T, s.d).total;
    const GateWgradGrid g = gate_wgrad_grid(s.T, s.d, s.E, s.act == MOE_F32 ? 4 : 2);
    return static_cast<size_t>(g.nchunk > 0 ? g.nchunk : 1) * s.E * s.d * 4;
}

hipError_t launch_gate_backward(const moe_shape& s, const void* x, const void* wg,
                                const int32_t* topk_idx, const float* topk_w,
                                const float* dtopk_w, float* dz, void* dx, float* dwg,
                                float* part, hipStream_t st) {
    const int64_t T = s.T;
    const GateWgradGrid g = gate_wgrad_grid(T, s.d, s.E, s.act == MOE_F32 ? 4 : 2);
    const GateMfmaPlan mp = gate_mfma_plan(T, s.d, s.E, s.act == MOE_BF16);
    const int64_t n4 = static_cast<int64_t>(s.E) * s.d / 4;
    const unsigned tblocks = static_cast<unsigned>((T + 3) / 4);
    if (mp.use) {
        uint8_t* base = reinterpret_cast<uint8_t*>(part);
        const GateMfmaWs w = gate_mfma_ws(mp, T, s.d);
        float* p1 = reinterpret_cast<float*>(base + w.p1);
        float* p3 = reinterpret_cast<float*>(base + w.p3);
        bf16_t* zp = reinterpret_cast<bf16_t*>(base + w.zp);
        int32_t* offsets = reinterpret_cast<int32_t*>(base + w.offsets);
        gate_backward_token_kernel<bf16_t><<<tblocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(wg), topk_idx, topk_w, dtopk_w, T, s.d, s.E, s.k, dz,
            static_cast<bf16_t*>(dx), zp, mp.F);
        gate_chunk_offsets_kernel<<<1, 256, 0, st>>>(T, mp.chunk, mp.C, offsets);
        const hipError_t err =
            launch_wgrad_planes(offsets, mp.C, T, s.d, mp.F, zp, x, p1, p3, base + w.meta, st);
        if (err != hipSuccess) return err;
        gate_plane_reduce_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, st>>>(
            p1, p3, mp.C, s.E, s.d, mp.F, reinterpret_cast<f32x4*>(dwg));
        return hipGetLastError();
    }
    if (T > 0) {
        if (s.act == MOE_F32) {
            gate_backward_token_kernel<float><<<tblocks, 256, 0, st>>>(
                static_cast<const float*>(wg), topk_idx, topk_w, dtopk_w, T, s.d, s.E, s.k, dz,
                static_cast<float*>(dx), nullptr, 0);
            launch_wgrad<float>(g, static_cast<const float*>(x), topk_idx, dz, s, part, st);
        } else {
            gate_backward_token_kernel<bf16_t><<<tblocks, 256, 0, st>>>(
                static_cast<const bf16_t*>(wg), topk_idx, topk_w, dtopk_w, T, s.d, s.E, s.k, dz,
                static_cast<bf16_t*>(dx), nullptr, 0);
            launch_wgrad<bf16_t>(g, static_cast<const bf16_t*>(x), topk_idx, dz, s, part, st);
        }
    }
    gate_backward_reduce_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, st>>>(
        reinterpret_cast<const f32x4*>(part), T > 0 ? g.nchunk : 0, n4,
        reinterpret_cast<f32x4*>(dwg));
    return hipGetLastError();
}

}  // namespace moe
