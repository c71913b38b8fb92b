// Gate + top-k in two phases, with results identical to the one-chain-per-
// logit gate.
//
// What is computed is unchanged: "DeepSeek 中 MoE 的同步税" (wmrh.cn), section
// 4.1 (gate -> softmax -> top-k -> divide by the selected sum), fused as in
// section 4.3, the router in float32 (section 5.1), each logit one float32
// fused multiply-add chain over i = 0..d-1 from +0.0, then + bias, and the k
// experts that rank first under "larger logit, then lower id". Only the k
// selected logits (and which experts they are) leave the gate, so the
// chains of experts that cannot be selected need not be run:
//
// Phase 1 (matrix cores). An approximate logit zt[t,e] = x[t] . wg[e] on the
// bf16 MFMAs (float32 accumulation in the hardware's own order), plus the
// bias, for every (t, e). Both zt and the exact chain z are float32 sums of
// the same exact bf16 products (a bf16 x bf16 product fits in float32), so
// each is within about d * 2^-24 * sum_i |x_i w_i| of the exact sum; with
// Cauchy-Schwarz, sum_i |x_i w_i| <= |x| |w|. The bound used,
//     eps = 8 d 2^-24 |x| |w| + 8 * 2^-24 |zt| + 2^-126,
// allows four times the chain's error on each side (rounding other than to
// nearest, the float32 norms' own error, the bias addition).
// Phase 2 (candidates). With L = zt - eps and U = zt + eps, tau = the k-th
// largest L of the token: k experts have z >= tau, so the k-th largest z is
// at least tau, and an expert with U < tau has z < that and cannot be
// selected. The candidates are the experts with U >= tau (at least k).
// Phase 3 (exact). The canonical chain for every candidate, then the top-k
// among the candidates by (z, id) and the softmax over the selected logits,
// exactly as the one-phase kernel computes them.
//
// One work-group of four waves takes 128 tokens: phase 1 stages 64-wide K
// slices of x and of the gate weight through LDS (as 16-byte chunks, the
// next slice's loads in flight during the current MFMAs); each wave holds
// 32 tokens x all experts (EB blocks of 32) in accumulators, one 32x32x16
// MFMA per block and 16 K values. A lane then holds half of one token's
// approximate logits, its partner lane (lane ^ 32) the other half; they
// find tau and the candidate mask together. Phase 3 streams x and the
// weights through LDS once more and runs the chains of the wave's candidate
// (token, expert) pairs, up to eight per lane; each token's lane then picks
// its top-k.
#include <cstdlib>
#include <cstring>

#include "gate_common.h"

namespace moe {

constexpr int kTpTok = 128;         // tokens per work-group
constexpr int kTpK = 64;            // K values per step
constexpr int kTpPairCap = 512;     // candidate pairs per wave per pass (LDS)

__device__ __forceinline__ int tp_off(int r, int c) { return (r << 7) + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// NC chains of one lane over a 64-value K slice in LDS, in the canonical
// order (i ascending within each chain); pc[j] = (token row << 16) | expert.
// No branches, so the chains' loads and FMAs interleave.
template <int NC>
__device__ __forceinline__ void run_chains(const uint8_t* X, const uint8_t* W, const int* pc,
                                           float* z) {
#pragma unroll 2
    for (int g = 0; g < kTpK / 8; ++g) {
        u32x4 xv[NC], wv[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int xrow = pc[j] >> 16, e = pc[j] & 0xffff;
            xv[j] = *reinterpret_cast<const u32x4*>(X + tp_off(xrow, g));
            wv[j] = *reinterpret_cast<const u32x4*>(W + (e >> 7) * (128 * 128) + tp_off(e & 127, g));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int j = 0; j < NC; ++j) z[j] = __builtin_fmaf(bf16_lo(xv[j][u]), bf16_lo(wv[j][u]), z[j]);
#pragma unroll
            for (int j = 0; j < NC; ++j) z[j] = __builtin_fmaf(bf16_hi(xv[j][u]), bf16_hi(wv[j][u]), z[j]);
        }
    }
}

// Rank key of (logit z, expert e): a larger key ranks first, in the order
// "larger logit, then lower id, NaN after every number" -- the logit's
// order-preserving bits (-0 taken as +0; every NaN as 0) above ~e.
__device__ __forceinline__ uint64_t rank_key(float z, int e) {
    const uint32_t b = __float_as_uint(z + 0.0f);
    uint32_t o = (b & 0x80000000u) != 0u ? ~b : (b | 0x80000000u);
    if (z != z) o = 0u;
    return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}
__device__ __forceinline__ int key_id(uint64_t key) {
    return static_cast<int>(~static_cast<uint32_t>(key));
}
// the logit of a key as the softmax takes it (NaN as -inf)
__device__ __forceinline__ float key_softmax_logit(uint64_t key) {
    const uint32_t o = static_cast<uint32_t>(key >> 32);
    if (o == 0u) return -__builtin_inff();
    return __uint_as_float((o & 0x80000000u) != 0u ? (o & 0x7fffffffu) : ~o);
}

template <int EB>
__global__ __launch_bounds__(256, EB >= 8 ? 1 : 2) void gate_two_phase_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    constexpr int XB = kTpTok * kTpK * 2;        // bytes of an x slice
    constexpr int WB = EB * 32 * kTpK * 2;       // bytes of a weight slice
    constexpr int STAGE = XB + WB;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float* nx = reinterpret_cast<float*>(lds + 2 * STAGE);      // [128] |x|^2
    float* nw = nx + kTpTok;                                    // [EB*32] |w|^2
    uint32_t* masks = reinterpret_cast<uint32_t*>(nw + EB * 32);  // [128][EB] candidates

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTpTok;
    const int c = tid & 7, rr = tid >> 3;  // staging: chunk c of rows rr + 32 i

    // ---- phase 1: approximate logits on the matrix cores, and the norms
    const bf16_t* xr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + rr + 32 * i;
        xr[i] = t < T ? x + t * d : nullptr;
    }
    const bf16_t* wr[EB];
#pragma unroll
    for (int i = 0; i < EB; ++i) {
        const int e = rr + 32 * i;
        wr[i] = e < E ? wg + static_cast<int64_t>(e) * d : nullptr;
    }
    float sx[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sw[EB];
#pragma unroll
    for (int i = 0; i < EB; ++i) sw[i] = 0.0f;
    u32x4 rx[4], rw[EB];
    auto sumsq = [](u32x4 v) {
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float a = bf16_lo(v[u]), b = bf16_hi(v[u]);
            s = __builtin_fmaf(a, a, s);
            s = __builtin_fmaf(b, b, s);
        }
        return s;
    };
    // the staging loads of one K step (with the norms' sums in phase 1)
    auto load = [&](int k0, bool sums) {
        const int kk = k0 + c * 8;
        const bool kin = kk < d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rx[i] = (xr[i] != nullptr && kin) ? load16(xr[i] + kk) : u32x4{0u, 0u, 0u, 0u};
            if (sums) sx[i] += sumsq(rx[i]);
        }
#pragma unroll
        for (int i = 0; i < EB; ++i) {
            rw[i] = (wr[i] != nullptr && kin) ? load16(wr[i] + kk) : u32x4{0u, 0u, 0u, 0u};
            if (sums) sw[i] += sumsq(rw[i]);
        }
    };
    auto put = [&](int buf) {
        uint8_t* X = lds + buf * STAGE;
        uint8_t* W = X + XB;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(X + tp_off(rr + 32 * i, c)) = rx[i];
#pragma unroll
        for (int i = 0; i < EB; ++i) {
            const int e = rr + 32 * i;  // weight block e / 128 at its own 16 KB
            *reinterpret_cast<u32x4*>(W + (e >> 7) * (128 * 128) + tp_off(e & 127, c)) = rw[i];
        }
    };
    f32x16 acc[EB];
#pragma unroll
    for (int i = 0; i < EB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    const int KT = (d + kTpK - 1) / kTpK;
    load(0, true);
    put(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load((kt + 1) * kTpK, true);
        const uint8_t* X = lds + (kt & 1) * STAGE;
        const uint8_t* W = X + XB;
#pragma unroll
        for (int ks = 0; ks < kTpK / 16; ++ks) {
            const int ch = ks * 2 + lg;
            const bf16x8 xf = *reinterpret_cast<const bf16x8*>(X + tp_off(wave * 32 + lr, ch));
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) {
                const int e = eb * 32 + lr;
                const bf16x8 wf = *reinterpret_cast<const bf16x8*>(W + (e >> 7) * (128 * 128) + tp_off(e & 127, ch));
                acc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc[eb], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) put((kt + 1) & 1);
        __syncthreads();
    }
    // norms: the 8 lanes of a row group (c = 0..7) hold one row's partial sums
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = sx[i];
        v += __shfl_xor(v, 1, kWave);
        v += __shfl_xor(v, 2, kWave);
        v += __shfl_xor(v, 4, kWave);
        if (c == 0) nx[rr + 32 * i] = v;
    }
#pragma unroll
    for (int i = 0; i < EB; ++i) {
        float v = sw[i];
        v += __shfl_xor(v, 1, kWave);
        v += __shfl_xor(v, 2, kWave);
        v += __shfl_xor(v, 4, kWave);
        if (c == 0) nw[rr + 32 * i] = v;
    }
    __syncthreads();

    // ---- phase 2: candidates. acc[eb][v] is token wave*32 + lr and expert
    // eb*32 + 8*(v/4) + 4*lg + v%4.
    {
        const int tl = wave * 32 + lr;
        const float sxn = __builtin_sqrtf(nx[tl]);
        const float du = static_cast<float>(d) * 0x1p-24f;
        float top[kMaxK];
#pragma unroll
        for (int p = 0; p < kMaxK; ++p) top[p] = -__builtin_inff();
        // a NaN or infinity in any approximate logit or bound (NaN or
        // infinite inputs, a NaN bias, sums near the float32 range): every
        // expert of the token is a candidate, and the exact chains decide
        bool bad = false;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int e = eb * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (e >= E) continue;
                const float zt = acc[eb][v] + (bias != nullptr ? bias[e] : 0.0f);
                const float eps = 8.0f * du * sxn * __builtin_sqrtf(nw[e]) +
                                  8.0f * 0x1p-24f * __builtin_fabsf(zt) + 0x1p-126f;
                const float L = zt - eps;
                acc[eb][v] = zt;  // keep zt for the upper bounds
                bad = bad || !(__builtin_fabsf(zt) < __builtin_inff()) || !(eps < __builtin_inff());
                // insert L into the descending top-k list
                float cur = L;
#pragma unroll
                for (int p = 0; p < kMaxK; ++p) {
                    if (p < k && cur > top[p]) {
                        const float t = top[p];
                        top[p] = cur;
                        cur = t;
                    }
                }
            }
        // merge with the partner's list: tau = k-th largest of both
        float ot[kMaxK];
#pragma unroll
        for (int p = 0; p < kMaxK; ++p) ot[p] = __shfl_xor(top[p], 32, kWave);
        float tau = -__builtin_inff();
        {
            int i = 0, j = 0;
#pragma unroll
            for (int p = 0; p < 2 * kMaxK; ++p) {
                if (p < k) {
                    const float a = i < kMaxK ? top[i] : -__builtin_inff();
                    const float b = j < kMaxK ? ot[j] : -__builtin_inff();
                    if (a >= b) {
                        tau = a;
                        ++i;
                    } else {
                        tau = b;
                        ++j;
                    }
                }
            }
        }
        bad = bad || __shfl_xor(bad ? 1 : 0, 32, kWave) != 0 || !(tau == tau);
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            uint32_t word = 0u;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int b = 8 * (v >> 2) + 4 * lg + (v & 3);
                const int e = eb * 32 + b;
                if (e >= E) continue;
                const float zt = acc[eb][v];
                const float eps = 8.0f * du * sxn * __builtin_sqrtf(nw[e]) +
                                  8.0f * 0x1p-24f * __builtin_fabsf(zt) + 0x1p-126f;
                if (bad || zt + eps >= tau) word |= 1u << b;
            }
            word |= __shfl_xor(word, 32, kWave);
            if (lg == 0) masks[tl * EB + eb] = word;
        }
    }
    __syncthreads();

    // ---- phase 3: the exact chains of the candidates, then the top-k.
    // Each wave lists its tokens' candidate (token, expert) pairs, as many
    // tokens as fit (kTpPairCap pairs; one token always does) per pass; all
    // waves run as many passes as the wave that needs most. A pass streams
    // x and the gate weight through LDS again, 64 K values at a time, and
    // lane l advances the chains of pairs l + 64 j, j < nc (nc = the list's
    // length over 64, rounded up to 1, 2, 4 or 8; lanes past the end repeat
    // pair 0 and discard it) in the canonical order. The pair list and the
    // logits live in the wave's part of the staging area while it is idle.
    int* pair = reinterpret_cast<int*>(lds) + wave * 2 * kTpPairCap;
    float* pz = reinterpret_cast<float*>(pair + kTpPairCap);
    int* npass = reinterpret_cast<int*>(masks + kTpTok * EB);  // [4] passes per wave
    const int tw = wave * 32;  // the wave's first token within the block
    int cnt = 0;  // candidates of lane lr's token (lanes < 32; none past T)
    if (lane < 32 && t0 + tw + lane < T) {
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) cnt += __popc(masks[(tw + lane) * EB + eb]);
    }
    // the greedy split of the wave's tokens into passes: [next, returned) in a pass
    auto take_range = [&](int next, int& pre, bool& take, int& total) {
        const int mine = (lane >= next && lane < 32) ? cnt : 0;
        int incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += u;
        }
        pre = incl - mine;
        take = lane >= next && lane < 32 && incl <= kTpPairCap;
        const unsigned long long tk = __ballot(take);
        const int last = 63 - __clzll(static_cast<long long>(tk));
        total = __shfl(incl, last, kWave);
        return last + 1;
    };
    {
        int np = 0;
        for (int next = 0; next < 32; ++np) {
            int pre, total;
            bool take;
            next = take_range(next, pre, take, total);
        }
        if (lane == 0) npass[wave] = np;
    }
    __syncthreads();
    const int passes = max(max(npass[0], npass[1]), max(npass[2], npass[3]));
    int next = 0;
    for (int pass = 0; pass < passes; ++pass) {
        int pre = 0, total = 0;
        bool take = false;
        int nnext = next;
        if (next < 32) {
            nnext = take_range(next, pre, take, total);
            if (take && cnt > 0) {
                int q = pre;
#pragma unroll
                for (int eb = 0; eb < EB; ++eb) {
                    uint32_t m = masks[(tw + lane) * EB + eb];
                    while (m != 0u) {
                        const int b = __ffs(m) - 1;
                        m &= m - 1u;
                        pair[q++] = ((tw + lane) << 16) | (eb * 32 + b);
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the list is written
        __builtin_amdgcn_wave_barrier();
        constexpr int kCh = kTpPairCap / kWave;
        const int nc = total <= kWave ? 1 : (total <= 2 * kWave ? 2 : (total <= 4 * kWave ? 4 : 8));
        int pc[kCh];
        float z[kCh];
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int r = j * kWave + lane;
            pc[j] = (total > 0 && r < total) ? pair[r] : (total > 0 ? pair[0] : 0);
            z[j] = 0.0f;
        }
        __syncthreads();  // every list is read before the staging area refills
        load(0, false);
        put(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            if (kt + 1 < KT) load((kt + 1) * kTpK, false);
            const uint8_t* X = lds + (kt & 1) * STAGE;
            const uint8_t* W = X + XB;
            if (total > 0) {
                if (nc == 1) run_chains<1>(X, W, pc, z);
                else if (nc == 2) run_chains<2>(X, W, pc, z);
                else if (nc == 4) run_chains<4>(X, W, pc, z);
                else run_chains<8>(X, W, pc, z);
            }
            if (kt + 1 < KT) put((kt + 1) & 1);
            __syncthreads();
        }
        // the exact logits of the listed pairs, in the wave's own part
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int r = j * kWave + lane;
            if (r < total) {
                const int e = pc[j] & 0xffff;
                pz[r] = bias != nullptr ? z[j] + bias[e] : z[j];
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // each taken token's lane: its k best candidates (its mask's experts
        // in the list's order), then the weights
        if (take) {
            const int64_t t = t0 + tw + lane;
            // the k largest rank keys, kept sorted by one max / min pass
            // per candidate (0 is below every key)
            uint64_t sk[kMaxK];
#pragma unroll
            for (int p = 0; p < kMaxK; ++p) sk[p] = 0u;
            int q = pre;
            for (int eb = 0; eb < EB && cnt > 0; ++eb) {
                uint32_t m = masks[(tw + lane) * EB + eb];
                while (m != 0u) {
                    const int b = __ffs(m) - 1;
                    m &= m - 1u;
                    uint64_t ck = rank_key(pz[q++], eb * 32 + b);
#pragma unroll
                    for (int p = 0; p < kMaxK; ++p) {
                        if (p < k) {
                            const uint64_t hi = ck > sk[p] ? ck : sk[p];
                            ck = ck > sk[p] ? sk[p] : ck;
                            sk[p] = hi;
                        }
                    }
                }
            }
            if (t < T) {
                float sz[kMaxK];
#pragma unroll
                for (int p = 0; p < kMaxK; ++p) sz[p] = key_softmax_logit(sk[p]);
                const float zmax = sz[0];
                float sum = 0.0f;
#pragma unroll
                for (int p = 0; p < kMaxK; ++p)
                    if (p < k) sum += expf(sz[p] - zmax);
#pragma unroll
                for (int p = 0; p < kMaxK; ++p) {
                    if (p < k) {
                        topk_idx[t * k + p] = key_id(sk[p]);
                        topk_w[t * k + p] = expf(sz[p] - zmax) / sum;
                    }
                }
            }
        }
        next = nnext;
        __syncthreads();  // every wave is done with its list before the next pass writes
    }
}

namespace {
template <int EB>
hipError_t launch_tp(const moe_shape& s, const void* x, const void* wg, const float* bias,
                     int32_t* idx, float* w, hipStream_t st) {
    constexpr int lds = 2 * (kTpTok * kTpK * 2 + EB * 32 * kTpK * 2) + (kTpTok + EB * 32) * 4 +
                        kTpTok * EB * 4 + 16;
    static_assert(2 * (kTpTok * kTpK * 2) >= 4 * 2 * kTpPairCap * 4, "pair lists fit in the staging area");
    static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_two_phase_kernel<EB>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    const unsigned blocks = static_cast<unsigned>((s.T + kTpTok - 1) / kTpTok);
    gate_two_phase_kernel<EB><<<blocks, 256, lds, st>>>(static_cast<const bf16_t*>(x),
                                                         static_cast<const bf16_t*>(wg), bias, s.T,
                                                         s.d, s.E, s.k, idx, w);
    return hipGetLastError();
}
}  // namespace

// The two-phase gate for bf16 inputs where it is the faster one: its cost
// follows the reads of x (twice) and the candidates' chains, the one-phase
// kernel's the T*E chains, so it wins with many experts -- measured: E = 128,
// T = 65536, d = 4096 in 0.51 ms against 1.37 ms; E = 64, T = 32768 in 0.47
// against 0.36 -- and needs enough 128-token work-groups to fill the chip.
// Returns false (nothing launched) otherwise.
// The environment variable MOE_GATE_PATH = "two_phase" or "one_phase"
// overrides the choice (both give the same results; tests use it to run
// each path at any size).
bool gate_two_phase_chosen(const moe_shape& s) {
    if (s.act != MOE_BF16 || s.E > 256) return false;
    const char* force = std::getenv("MOE_GATE_PATH");
    if (force != nullptr && std::strcmp(force, "one_phase") == 0) return false;
    const bool forced = force != nullptr && std::strcmp(force, "two_phase") == 0;
    return forced || (s.E >= 96 && s.T >= 256 * kTpTok);
}

bool launch_gate_two_phase(const moe_shape& s, const void* x, const void* wg, const float* bias,
                           int32_t* idx, float* w, hipStream_t st, hipError_t* err) {
    if (!gate_two_phase_chosen(s)) return false;
    const int nb = (s.E + 31) / 32;
    if (nb <= 1) *err = launch_tp<1>(s, x, wg, bias, idx, w, st);
    else if (nb <= 2) *err = launch_tp<2>(s, x, wg, bias, idx, w, st);
    else if (nb <= 4) *err = launch_tp<4>(s, x, wg, bias, idx, w, st);
    else *err = launch_tp<8>(s, x, wg, bias, idx, w, st);
    return true;
}

}  // namespace moe
