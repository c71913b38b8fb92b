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
//   overflow (capacity with reassignment only) one block per rank block:
//            the assignments that overflow their expert, in token order, go
//            one at a time to the least-loaded expert (same notes, part A);
//            see dispatch_overflow_kernel.
//   permute  one wave per token: 16-byte row loads once, k row stores. A
//            slot whose rank among its expert's assignments (token order)
//            reaches C is dropped (dest_row = -1, no row) or takes the row
//            the overflow kernel gave it.
#include "ffn_plan.h"
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

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// exclusive prefix sum of v over the lanes of a wave
__device__ __forceinline__ int wave_excl_scan(int v) {
    const int lane = threadIdx.x & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    return incl - v;
}

// Final per-expert loads when the overflow is reassigned, by one wave.
// load[e] holds the first-pass loads L_e = min(n_e, cap) on entry and the
// final loads on exit; n[e] are the assignments per expert. The O
// overflowing assignments go one at a time to the least-loaded expert (ties
// to the lower id) while one is below cap, which fills level by level:
// raising every expert to level v takes N(v) = sum_e max(0, v - L_e) of them.
// With V the highest level N(V) <= O reaches (V < cap), every expert ends at
// max(L_e, V), plus one for the first O - N(V) experts in id order with
// L_e <= V; if N(cap) <= O every expert ends full.
__device__ void water_fill_loads(const int* n, int* load, int E, int cap) {
    const int lane = threadIdx.x & 63;
    int L[4];
    int64_t over = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        L[q] = e < E ? load[e] : 0;
        over += e < E ? n[e] - load[e] : 0;
    }
    const int64_t O = wave_sum64(over);
    auto N = [&](int v) {
        int64_t acc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane * 4 + q < E) acc += max(0, v - L[q]);
        return wave_sum64(acc);
    };
    if (N(cap) <= O) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane * 4 + q < E) load[lane * 4 + q] = cap;
        return;
    }
    int lo = 0, hi = cap - 1;  // N(0) = 0 <= O < N(cap)
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (N(mid) <= O) lo = mid;
        else hi = mid - 1;
    }
    const int V = lo;
    const int64_t r = O - N(V);
    int below = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) below += (lane * 4 + q < E && L[q] <= V) ? 1 : 0;
    int rk = wave_excl_scan(below);  // id-order position among the experts at or below V
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        if (e >= E) continue;
        int f = max(L[q], V);
        if (L[q] <= V) {
            if (rk < r) f += 1;
            ++rk;
        }
        load[e] = f;
    }
}

// blk[nblk][E] holds each rank block's per-expert counts; pre[nblk][E]
// receives the number of the expert's assignments in earlier rank blocks.
// (Two arrays, so that the loads of a thread's run of blocks are not held
// behind its stores.) With cap > 0, first_loads[e] receives min(n_e, cap);
// with reassign the counts are the loads after reassignment.
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ blk, int32_t* __restrict__ pre, int nblk, int E, int cap,
    int reassign, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ first_loads, uint32_t* __restrict__ qstats) {
    __shared__ int part[kScanThreads];  // [P][E] partial sums
    __shared__ int raw[kMaxE];
    __shared__ int tot[kMaxE];
    __shared__ int off[kMaxE + 1];
    const int tid = threadIdx.x;
    if (qstats != nullptr && tid <= E) {  // empty (min, max) ranges for the fp8 group modes
        qstats[2 * tid] = 0xffffffffu;
        qstats[2 * tid + 1] = 0u;
    }
    const int P = kScanThreads / E;  // parts of the block range per expert
    const int e = tid % E, p = tid / E;
    const bool active = p < P;
    const int per = (nblk + P - 1) / P;
    const int b0 = active ? min(nblk, p * per) : 0, b1 = active ? min(nblk, b0 + per) : 0;
    int run = 0;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) run += blk[static_cast<int64_t>(b) * E + e];
    if (active) part[p * E + e] = run;
    __syncthreads();
    if (tid < E) {
        int s = 0;
        for (int q = 0; q < P; ++q) {
            const int c = part[q * E + tid];
            part[q * E + tid] = s;
            s += c;
        }
        raw[tid] = s;
        tot[tid] = cap > 0 ? min(s, cap) : s;  // rows the expert keeps in the first pass
        if (cap > 0) first_loads[tid] = tot[tid];
    }
    __syncthreads();
    if (cap > 0 && reassign) {
        if (tid < kWave) water_fill_loads(raw, tot, E, cap);
        __syncthreads();
    }
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
        int acc = part[p * E + e];
#pragma unroll 8
        for (int b = b0; b < b1; ++b) {
            const int64_t i = static_cast<int64_t>(b) * E + e;
            pre[i] = acc;
            acc += blk[i];
        }
    }
}

// In a whole-layer forward the permute kernels' first fp.nblk work-groups
// write the FFN's tile plan; returns the work-group's index among the
// permute's own, or -1 for a plan work-group.
__device__ __forceinline__ int permute_or_plan(const FfnPlanArgs& fp,
                                               const int32_t* __restrict__ offsets, int E,
                                               int64_t T) {
    if (fp.plan == nullptr) return blockIdx.x;
    if (static_cast<int>(blockIdx.x) < fp.nblk) {
        ffn_plan_block(offsets, E, fp.S, T, fp.bm, fp.plan, fp.tiles, fp.n_up, fp.ntn_up,
                       fp.ntn_down, fp.counters, blockIdx.x, fp.nblk);
        return -1;
    }
    return blockIdx.x - fp.nblk;
}

// Capacity with reassignment: one block per rank block of 256 tokens, one
// thread per token. An assignment overflows iff its rank g among its
// expert's assignments (token order) is cap or more. Its overflow index o
// in token order is the block's base -- sum_e max(0, (expert e's assignments
// in earlier blocks) - cap) -- plus the overflows of earlier tokens of the
// block and of its own earlier slots. The o-th overflow lands, by the same
// level filling as water_fill_loads, at level v with N(v) <= o < N(v+1) on
// the (o - N(v))-th expert in id order among those with L_e <= v, as that
// expert's row v; with o >= N(cap) it is dropped. With the first-pass loads
// sorted ascending (s_i) and P_i their prefix sums, N(s_i) = i*s_i - P_i and
// each level in [s_i, s_{i+1}) holds i+1 overflows, those of the experts at
// sorted positions 0..i; a 256-bit mask of their ids per i turns "the p-th
// in id order" into a select of the p-th set bit.
__global__ __launch_bounds__(kRankThreads) void dispatch_overflow_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ pre, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ first_loads, int64_t T, int E, int k, int cap,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token) {
    __shared__ int Ls[kMaxE];
    __shared__ int sl[kMaxE];
    __shared__ int sid[kMaxE];                 // expert id at each sorted position
    __shared__ unsigned long long msk[kMaxE][kMaxE / 64];  // ids at sorted positions 0..i
    __shared__ long long Bk[kMaxE + 1];  // N at each sorted load; Bk[E] = N(cap)
    __shared__ long long wred[4];
    __shared__ int wtot[4];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x;
    for (int e = tid; e < E; e += kRankThreads) Ls[e] = first_loads[e];
    __syncthreads();
    // sorted first-pass loads (ties by id) and this block's overflow base
    long long ob = 0;
    for (int e = tid; e < E; e += kRankThreads) {
        int pos = 0;
        for (int q = 0; q < E; ++q) pos += (Ls[q] < Ls[e] || (Ls[q] == Ls[e] && q < e)) ? 1 : 0;
        sl[pos] = Ls[e];
        sid[pos] = e;
        ob += max(0, pre[static_cast<int64_t>(b) * E + e] - cap);
    }
    ob = wave_sum64(ob);
    if (lane == 0) wred[w] = ob;
    __syncthreads();
    ob = wred[0] + wred[1] + wred[2] + wred[3];
    if (w == 1 && lane < kMaxE / 64) {  // prefix ORs of the sorted ids, one word per lane
        unsigned long long acc = 0ull;
        for (int i = 0; i < E; ++i) {
            if ((sid[i] >> 6) == lane) acc |= 1ull << (sid[i] & 63);
            msk[i][lane] = acc;
        }
    }
    if (w == 0) {
        // prefix sums of the sorted loads, four entries per lane
        int v4[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = lane * 4 + q;
            v4[q] = i < E ? sl[i] : 0;
            sum += v4[q];
        }
        long long P = wave_excl_scan(sum);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = lane * 4 + q;
            if (i < E) Bk[i] = static_cast<long long>(i) * v4[q] - P;
            P += v4[q];
        }
        if (lane == 63) Bk[E] = static_cast<long long>(E) * cap - P;
    }
    // this token's overflowing slots
    const int64_t t = static_cast<int64_t>(b) * kRankThreads + tid;
    int mine = 0;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int r = rank[t * k + j];
            if (r < 0) continue;
            const int e = topk_idx[t * k + j];
            mine += pre[static_cast<int64_t>(b) * E + e] + r >= cap ? 1 : 0;
        }
    }
    const int wex = wave_excl_scan(mine);
    if (lane == 63) wtot[w] = wex + mine;
    __syncthreads();
    int before = wex;
    for (int q = 0; q < w; ++q) before += wtot[q];
    if (t >= T || mine == 0) return;
    long long o = ob + before;
    for (int j = 0; j < k; ++j) {
        const int r = rank[t * k + j];
        if (r < 0) continue;
        const int e = topk_idx[t * k + j];
        if (pre[static_cast<int64_t>(b) * E + e] + r < cap) continue;
        int dst = -1;
        if (o < Bk[E]) {
            int lo = 0, hi = E - 1;  // the last i with Bk[i] <= o
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (Bk[mid] <= o) lo = mid;
                else hi = mid - 1;
            }
            const long long within = o - Bk[lo];
            const int v = sl[lo] + static_cast<int>(within / (lo + 1));
            int pth = static_cast<int>(within % (lo + 1));
            // the pth set bit of the ids at sorted positions 0..lo
            int ee = E;
            for (int q = 0; q < kMaxE / 64; ++q) {
                unsigned long long m = msk[lo][q];
                const int c = __popcll(m);
                if (pth >= c) {
                    pth -= c;
                    continue;
                }
                int base = 0;
                for (int half = 32; half > 0; half >>= 1) {
                    const unsigned long long low = m & ((1ull << half) - 1ull);
                    const int cl = __popcll(low);
                    if (pth >= cl) {
                        pth -= cl;
                        m >>= half;
                        base += half;
                    } else {
                        m = low;
                    }
                }
                ee = q * 64 + base;
                break;
            }
            // the loads the scan kernel derived give expert ee more than v
            // rows; checked so that no row outside its range is written
            if (ee < E && v < offsets[ee + 1] - offsets[ee]) {
                dst = offsets[ee] + v;
                src_token[dst] = static_cast<int32_t>(t);
            }
        }
        dest_row[t * k + j] = dst;
        ++o;
    }
}

// Destination rows of token t's k slots, computed by lanes 0..k-1 and
// broadcast to the wave. Lanes 0..k-1 also write dest_row and src_token.
// A slot's rank g among all of its expert's assignments is the expert's
// count in earlier rank blocks plus its rank within the block; its row is
// offsets[e] + g. With cap > 0 a slot with g >= cap is dropped or, with
// reassign, takes the row the overflow kernel wrote to dest_row.
__device__ __forceinline__ int token_dest(const int32_t* __restrict__ topk_idx,
                                          const int32_t* __restrict__ rank,
                                          const int32_t* __restrict__ pre,
                                          const int32_t* __restrict__ offsets, int cap,
                                          int reassign, int64_t t, int E, int k, int lane,
                                          int32_t* __restrict__ dest_row,
                                          int32_t* __restrict__ src_token) {
    int dst = -1;
    if (lane < k) {
        const int r = rank[t * k + lane];
        if (r >= 0) {
            const int e = topk_idx[t * k + lane];
            const int g = pre[(t / kRankBlockTokens) * E + e] + r;
            if (cap > 0 && g >= cap) {
                dst = reassign ? dest_row[t * k + lane] : -1;
            } else {
                dst = offsets[e] + g;
                src_token[dst] = static_cast<int32_t>(t);
            }
        }
        dest_row[t * k + lane] = dst;
    }
    return dst;
}

__global__ __launch_bounds__(256) void dispatch_permute_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ pre,
    const int32_t* __restrict__ offsets, int cap, int reassign, int64_t T, int E, int k,
    int row_bytes,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    uint8_t* __restrict__ x_perm, FfnPlanArgs fp) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pb = permute_or_plan(fp, offsets, E, T);
    if (pb < 0) return;
    const int64_t t = static_cast<int64_t>(pb) * 4 + w;
    if (t >= T) return;
    const int dst =
        token_dest(topk_idx, rank, pre, offsets, cap, reassign, t, E, k, lane, dest_row,
                   src_token);
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

// The maps only (dest_row, src_token), one thread per (token, slot): for a
// whole-layer forward whose up-projection gathers the rows from x itself.
// Its first fp.nblk work-groups write the FFN's tile plan, as the permute's do.
__global__ __launch_bounds__(256) void dispatch_map_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ pre, const int32_t* __restrict__ offsets, int cap, int reassign,
    int64_t T, int E, int k, int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    FfnPlanArgs fp) {
    const int pb = permute_or_plan(fp, offsets, E, T);
    if (pb < 0) return;
    const int64_t i = static_cast<int64_t>(pb) * 256 + threadIdx.x;  // slot t * k + j
    if (i >= T * k) return;
    const int64_t t = i / k;
    token_dest(topk_idx, rank, pre, offsets, cap, reassign, t, E, k, static_cast<int>(i - t * k),
               dest_row, src_token);
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
    const int32_t* __restrict__ rank, const int32_t* __restrict__ pre,
    const int32_t* __restrict__ offsets, int cap, int reassign, int64_t T, int E, int k, int d,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    uint8_t* __restrict__ x_perm, float* __restrict__ qparams, FfnPlanArgs fp, int sym,
    uint8_t* __restrict__ x_self, float* __restrict__ q_self) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pb = permute_or_plan(fp, offsets, E, T);
    if (pb < 0) return;
    const int64_t t = static_cast<int64_t>(pb) * 4 + w;
    if (t >= T) return;
    const int dst =
        token_dest(topk_idx, rank, pre, offsets, cap, reassign, t, E, k, lane, dest_row,
                   src_token);
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
    if (sym) {
        // symmetric absmax: the same map over the range [-max|x|, max|x|]
        mx = fmaxf(-mn, mx);
        mn = -mx;
    }
    const float centre = 0.5f * (mx + mn);
    const float half = 0.5f * (mx - mn);
    const bool flat = half == 0.0f;
    const float scale = flat ? 0.0f : half / 448.0f;
    const float inv = flat ? 0.0f : 448.0f / half;
    if (lane < k && dst >= 0) {
        qparams[2 * static_cast<int64_t>(dst)] = scale;
        qparams[2 * static_cast<int64_t>(dst) + 1] = centre;
    }
    if (x_self != nullptr && lane == 0) {
        q_self[2 * t] = scale;
        q_self[2 * t + 1] = centre;
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
        // the token's own codes, for the shared experts of the fp8-weight path
        if (x_self != nullptr) store16(x_self + t * d + (static_cast<int64_t>(g) << 4), q);
    }
}

// ------------------------------------------- fp8 per-expert / global ranges --
// The quantiser's per-expert and global modes ("Deepseek-MoE同步税本质与四层实战
// 优化指南", gsyq.cn, section 5.2, beside the per-token mode of section 3.1):
// the same affine min/max map, with the range taken over all rows dispatched
// to an expert (its final rows, after any capacity limit) or over the whole
// batch. A float's order is kept by an unsigned key, so ranges merge with
// integer atomics.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// expert whose row range holds `row` (offsets non-decreasing, row < offsets[E]);
// `offsets` is the block's LDS copy
__device__ __forceinline__ int expert_of_row(const int* offsets, int E, int row) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= row) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

constexpr int kStatsTokensPerWave = 4;

// Places every slot (dest_row, src_token, as the permute does) and merges
// each token's row min/max into its experts' ranges (qstats[2e], [2e+1]) or
// into the batch's (qstats[2E], [2E+1]); a block reduces in LDS first and
// then makes one pair of atomics per range it touched.
__global__ __launch_bounds__(256) void dispatch_fp8_stats_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ pre,
    const int32_t* __restrict__ offsets, int cap, int reassign, int global, int64_t T, int E,
    int k, int d, int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    uint32_t* __restrict__ qstats) {
    __shared__ uint32_t smin[kMaxE + 1], smax[kMaxE + 1];
    __shared__ int off_s[kMaxE + 1];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    for (int g = tid; g <= E; g += 256) {
        smin[g] = 0xffffffffu;
        smax[g] = 0u;
        off_s[g] = offsets[g];
    }
    __syncthreads();
    const int64_t tbase = (static_cast<int64_t>(blockIdx.x) * 4 + w) * kStatsTokensPerWave;
    for (int i = 0; i < kStatsTokensPerWave; ++i) {
        const int64_t t = tbase + i;
        if (t >= T) break;
        const int dst = token_dest(topk_idx, rank, pre, offsets, cap, reassign, t, E, k, lane,
                                   dest_row, src_token);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(x + t * d);
        float mn = __builtin_inff(), mx = -__builtin_inff();
        for (int c = lane; c < (d >> 3); c += kWave) {
            const u32x4 a = load16(src + (static_cast<int64_t>(c) << 4));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                mn = fminf(mn, fminf(bf16_lo(a[u]), bf16_hi(a[u])));
                mx = fmaxf(mx, fmaxf(bf16_lo(a[u]), bf16_hi(a[u])));
            }
        }
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (global) {
            if (lane == 0) {
                atomicMin(&smin[E], order_key(mn));
                atomicMax(&smax[E], order_key(mx));
            }
        } else if (lane < k && dst >= 0) {
            const int g = expert_of_row(off_s, E, dst);
            atomicMin(&smin[g], order_key(mn));
            atomicMax(&smax[g], order_key(mx));
        }
    }
    __syncthreads();
    for (int g = tid; g <= E; g += 256) {
        if (smin[g] != 0xffffffffu) {
            atomicMin(&qstats[2 * g], smin[g]);
            atomicMax(&qstats[2 * g + 1], smax[g]);
        }
    }
}

// Writes each dispatched copy of a row as e4m3 codes of its range's affine
// map (the per-token kernel's arithmetic with the group's min/max), with
// (scale, centre) per row. dest_row comes from the stats kernel.
__global__ __launch_bounds__(256) void dispatch_permute_fp8_group_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ dest_row,
    const int32_t* __restrict__ offsets, const uint32_t* __restrict__ qstats, int global,
    int64_t T, int E, int k, int d, uint8_t* __restrict__ x_perm, float* __restrict__ qparams,
    FfnPlanArgs fp) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pb = permute_or_plan(fp, offsets, E, T);
    if (pb < 0) return;
    __shared__ int off_s[kMaxE + 1];
    if (!global) {
        for (int g = threadIdx.x; g <= E; g += blockDim.x) off_s[g] = offsets[g];
        __syncthreads();
    }
    const int64_t t = static_cast<int64_t>(pb) * 4 + w;
    if (t >= T) return;
    int dst = -1;
    float centre = 0.0f, inv = 0.0f;
    bool flat = true;
    if (lane < k) {
        dst = dest_row[t * k + lane];
        if (dst >= 0) {
            const int g = global ? E : expert_of_row(off_s, E, dst);
            const float mn = key_value(qstats[2 * g]), mx = key_value(qstats[2 * g + 1]);
            centre = 0.5f * (mx + mn);
            const float half = 0.5f * (mx - mn);
            flat = half == 0.0f;
            inv = flat ? 0.0f : 448.0f / half;
            qparams[2 * static_cast<int64_t>(dst)] = flat ? 0.0f : half / 448.0f;
            qparams[2 * static_cast<int64_t>(dst) + 1] = centre;
        }
    }
    int dj[kMaxK];
    float cj[kMaxK], ij[kMaxK];
    bool fj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        dj[j] = __shfl(dst, j, kWave);
        cj[j] = __shfl(centre, j, kWave);
        ij[j] = __shfl(inv, j, kWave);
        fj[j] = __shfl(flat ? 1 : 0, j, kWave) != 0;
    }
    const uint8_t* src = reinterpret_cast<const uint8_t*>(x + t * d);
    const int ngroups = d >> 4;
    for (int g = lane; g < ngroups; g += kWave) {
        const u32x4 a = load16(src + (static_cast<int64_t>(g) << 5));
        const u32x4 b = load16(src + (static_cast<int64_t>(g) << 5) + 16);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && dj[j] >= 0)
                store16(x_perm + static_cast<int64_t>(dj[j]) * d + (static_cast<int64_t>(g) << 4),
                        quant16(a, b, cj[j], ij[j], fj[j]));
        }
    }
}

hipError_t launch_dispatch(const moe_shape& s, const void* x, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* dest_row,
                           int32_t* src_token, void* x_perm, float* qparams, int32_t* rank,
                           int32_t* blk, int32_t* pre, int32_t* first_loads, uint32_t* qstats,
                           uint32_t* hdr, const FfnPlanArgs& fp, hipStream_t st,
                           const Marks* mk, uint8_t* x_self, float* q_self) {
    const int nblk = static_cast<int>((s.T + kRankBlockTokens - 1) / kRankBlockTokens);
    const int reassign = s.capacity > 0 && s.overflow == MOE_OVERFLOW_REASSIGN ? 1 : 0;
    dispatch_rank_kernel<<<nblk, kRankThreads, 0, st>>>(topk_idx, s.T, s.E, s.k, rank, blk, hdr);
    mark(mk);
    const bool fp8 = s.dispatch == MOE_FP8_E4M3;
    const bool group = fp8 && (s.quant == MOE_QUANT_EXPERT || s.quant == MOE_QUANT_GLOBAL);
    dispatch_scan_kernel<<<1, kScanThreads, 0, st>>>(blk, pre, nblk, s.E, s.capacity, reassign,
                                                     counts, offsets, first_loads,
                                                     group ? qstats : nullptr);
    mark(mk);
    // (its time is counted with the permute's in a traced forward)
    if (reassign)
        dispatch_overflow_kernel<<<nblk, kRankThreads, 0, st>>>(topk_idx, rank, pre, offsets,
                                                                first_loads, s.T, s.E, s.k,
                                                                s.capacity, dest_row, src_token);
    // with a plan to write (whole-layer forward), its work-groups come first
    const unsigned pblocks =
        static_cast<unsigned>((s.T + 3) / 4) + (fp.plan != nullptr ? static_cast<unsigned>(fp.nblk) : 0u);
    if (group) {
        // (the stats kernel's time is counted with the permute's in a traced forward)
        const int global = s.quant == MOE_QUANT_GLOBAL ? 1 : 0;
        const unsigned sblocks =
            static_cast<unsigned>((s.T + 4 * kStatsTokensPerWave - 1) / (4 * kStatsTokensPerWave));
        dispatch_fp8_stats_kernel<<<sblocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(x), topk_idx, rank, pre, offsets, s.capacity, reassign,
            global, s.T, s.E, s.k, s.d, dest_row, src_token, qstats);
        dispatch_permute_fp8_group_kernel<<<pblocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(x), dest_row, offsets, qstats, global, s.T, s.E, s.k, s.d,
            static_cast<uint8_t*>(x_perm), qparams, fp);
    } else if (fp8) {
        dispatch_permute_fp8_kernel<<<pblocks, 256, 0, st>>>(
            static_cast<const bf16_t*>(x), topk_idx, rank, pre, offsets, s.capacity, reassign, s.T,
            s.E, s.k, s.d, dest_row, src_token, static_cast<uint8_t*>(x_perm), qparams, fp,
            s.quant == MOE_QUANT_TOKEN_ABSMAX ? 1 : 0, x_self, q_self);
    } else {
        const int row_bytes = s.d * (s.act == MOE_F32 ? 4 : 2);
        if (x_perm == nullptr) {
            // no x_perm: the maps only (the rows are gathered where they are used)
            const unsigned mblocks = static_cast<unsigned>((s.T * s.k + 255) / 256) +
                                     (fp.plan != nullptr ? static_cast<unsigned>(fp.nblk) : 0u);
            dispatch_map_kernel<<<mblocks, 256, 0, st>>>(topk_idx, rank, pre, offsets, s.capacity,
                                                         reassign, s.T, s.E, s.k, dest_row,
                                                         src_token, fp);
        } else {
            dispatch_permute_kernel<<<pblocks, 256, 0, st>>>(
                static_cast<const uint8_t*>(x), topk_idx, rank, pre, offsets, s.capacity, reassign,
                s.T, s.E, s.k, row_bytes, dest_row, src_token, static_cast<uint8_t*>(x_perm), fp);
        }
    }
    mark(mk);
    return hipGetLastError();
}

}  // namespace moe
