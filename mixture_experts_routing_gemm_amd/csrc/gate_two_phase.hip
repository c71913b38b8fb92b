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
// A work-group takes 256 tokens (eight waves) with 65 to 128 experts, else
// 128 (four waves: with more than 128 experts the accumulators need the
// registers of two waves; with 64 or fewer, two work-groups fit on a CU). Both phases that read x stream 32-wide K slices of x and of the
// gate weight through a ring of six LDS slots filled by direct buffer-to-LDS
// loads, five slices in flight: the reads of x bound the gate, and with about
// 4 us of loaded HBM latency it takes some 80 KB of x in flight per CU to
// approach the bandwidth (one slice in flight per work-group of 128 tokens,
// as staged through registers before, read x at about 2 TB/s). In phase 1 each
// wave holds 32 tokens x all experts (EB blocks of 32) in accumulators, one
// 32x32x16 MFMA per block and 16 K values, and sums the squares of the
// fragments it reads for the norms. A lane then holds half of one token's
// approximate logits, its partner lane (lane ^ 32) the other half; they
// find tau and the candidate mask together. Phase 3 streams x and the
// weights once more and runs the chains of the wave's candidate (token,
// expert) pairs, up to eight per lane; each token's lane then picks its
// top-k.
#include <cstdlib>
#include <cstring>

#include "gate_common.h"
#include "lds_ring.h"

namespace moe {

constexpr int kTpK = 32;            // K values per ring slot (64 bytes of a row)
constexpr int kTpPairCap = 512;     // candidate pairs per wave per pass (LDS)

// byte offset of 16-byte chunk c (0..3) of row r in a slot's area of 64-byte
// rows; the XOR swizzle keeps 16-byte reads of aligned runs of 8 rows (32
// banks) or 16 rows (64 banks) conflict-free
__device__ __forceinline__ int tp_off(int r, int c) {
    return (r << 6) + ((c ^ (((r >> 1) & 3) ^ ((r >> 3) & 1))) << 4);
}

// Work-group and ring geometry for EB blocks of 32 experts. A slot holds
// the work-group's x rows and the weight rows of one K slice; the weight
// rows are padded to 16 per wave so that every wave issues the same number
// of 1 KB requests per slot.
template <int EB>
struct TpRing {
    static constexpr int kTok = EB == 4 ? 256 : 128;  // tokens per work-group
    static constexpr int kWaves = kTok / 32;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kWRows = EB * 32 > 16 * kWaves ? EB * 32 : 16 * kWaves;
    static constexpr int kXBytes = kTok * 64;
    static constexpr int kSlot = kXBytes + kWRows * 64;
    static constexpr int kSlots = 6;
    static constexpr int kReq = 2 + kWRows / (16 * kWaves);  // per wave per slot: 2 of x, the rest weights
    static constexpr int kLds = kSlots * kSlot + (kTok + 2 * EB * 32) * 4 + kTok * EB * 4 + 4 * kWaves;
};

// waits until at most `ahead` slots' requests (R per slot) are in flight
template <int R, int A>
__device__ __forceinline__ void tp_wait_slots(int ahead) {
    if constexpr (A == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A)
            wait_vmcnt<A * R>();
        else
            tp_wait_slots<R, A - 1>(ahead);
    }
}

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
            wv[j] = *reinterpret_cast<const u32x4*>(W + tp_off(e, g));
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
__global__ __launch_bounds__(TpRing<EB>::kThreads, 1) void gate_two_phase_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    using RG = TpRing<EB>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float* nx = reinterpret_cast<float*>(lds + RG::kSlots * RG::kSlot);  // [kTok] |x|
    float* nw = nx + RG::kTok;                                            // [EB*32] |w|
    uint32_t* masks = reinterpret_cast<uint32_t*>(nw + EB * 32);           // [kTok][EB] candidates
    float* nb = reinterpret_cast<float*>(masks + RG::kTok * EB);           // [EB*32] the bias

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RG::kTok;
    // the bias, read once (phases 2 and 3 take every expert's from LDS; the
    // barrier after phase 1 publishes it)
    if (bias != nullptr)
        for (int e = tid; e < EB * 32; e += RG::kThreads) nb[e] = e < E ? bias[e] : 0.0f;

    // The ring. Request i (< kReq) of a slot, issued by every wave, is block
    // j = wave + kWaves i of 16 rows: x rows 16 j.. for i < 2, weight rows
    // 16 (j - 2 kWaves).. after. Lane l brings the logical chunk (l % 4) ^ swizzle
    // of row l / 4 of its block, which the direct load writes at byte 16 l:
    // where tp_off puts it. Rows past the token count or the experts, and
    // chunks past d, read as zeros (offsets beyond the buffer's size).
    const int64_t nrows = T - t0 < RG::kTok ? T - t0 : RG::kTok;
    const uint8_t* xbuf = uniform_ptr(reinterpret_cast<const uint8_t*>(x + t0 * d));
    const uint32_t xbytes = static_cast<uint32_t>(nrows * d * 2);
    const uint8_t* wbuf = uniform_ptr(reinterpret_cast<const uint8_t*>(wg));
    const uint32_t wbytes = static_cast<uint32_t>(static_cast<int64_t>(E) * d * 2);
    uint32_t voff[RG::kReq];
    int kch[RG::kReq];  // K offset of the lane's chunk within a slice
#pragma unroll
    for (int i = 0; i < RG::kReq; ++i) {
        const int j = wave + RG::kWaves * i;
        const int row = (i < 2 ? j : j - 2 * RG::kWaves) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ (((row >> 1) & 3) ^ ((row >> 3) & 1));
        voff[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(d) * 2u + static_cast<uint32_t>(c) * 16u;
        kch[i] = c * 8;
    }
    const int KT = (d + kTpK - 1) / kTpK;
    // slice kt of a walk that starts at slice rot (and wraps) goes to slot kt % kSlots
    auto issue = [&](int kt, int rot, auto AX) {
        uint8_t* S = lds + (kt % RG::kSlots) * RG::kSlot;
        const int kr = kt + rot < KT ? kt + rot : kt + rot - KT;
        const int k0 = kr * kTpK;
        const uint32_t soff = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(k0 * 2));
#pragma unroll
        for (int i = 0; i < RG::kReq; ++i) {
            const int j = wave + RG::kWaves * i;
            const uint32_t v = k0 + kch[i] < d ? voff[i] : 0x80000000u;
            if (i < 2)
                buffer_to_lds16<0, decltype(AX)::value>(xbuf, xbytes, v, soff, S + j * 1024);
            else
                buffer_to_lds16<0>(wbuf, wbytes, v, soff, S + RG::kXBytes + (j - 2 * RG::kWaves) * 1024);
        }
    };
    // Runs body(slot) on the KT slices, starting at slice rot and wrapping
    // around, each once it has landed and every wave may read it. The slice
    // kSlots - 1 ahead is requested right after the barrier into the slot
    // read one step earlier, which every wave has finished by then. Ends
    // with nothing in flight; the caller synchronises before the ring's
    // bytes are used otherwise.
    auto stream = [&](int rot, auto body, auto AX) {
        for (int s = 0; s < RG::kSlots - 1 && s < KT; ++s) issue(s, rot, AX);
        for (int kt = 0; kt < KT; ++kt) {
            const int ahead = min(RG::kSlots - 2, KT - 1 - kt);
            tp_wait_slots<RG::kReq, RG::kSlots - 2>(ahead);
            ring_barrier();
            if (kt + RG::kSlots - 1 < KT) issue(kt + RG::kSlots - 1, rot, AX);
            body(lds + (kt % RG::kSlots) * RG::kSlot);
        }
    };

    // ---- phase 1: approximate logits on the matrix cores, and the norms
    // from the fragments read for them: a lane sums the squares of its
    // token's chunks; wave w those of weight blocks w, w + kWaves. Neither
    // depends on the order of the slices (the bound covers any order of
    // the sums), so each work-group starts at its own slice: when every
    // work-group reads the same columns of rows d*2 bytes apart at once,
    // the reads share their low address bits and go at about 3 TB/s; the
    // staggered walk measured 3.7.
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
    constexpr int kNwq = (EB + RG::kWaves - 1) / RG::kWaves;
    float sx = 0.0f, sw[kNwq];
#pragma unroll
    for (int q = 0; q < kNwq; ++q) sw[q] = 0.0f;
    f32x16 acc[EB];
#pragma unroll
    for (int i = 0; i < EB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    stream(static_cast<int>(blockIdx.x % static_cast<unsigned>(KT)), [&](const uint8_t* S) {
        const uint8_t* X = S;
        const uint8_t* W = S + RG::kXBytes;
        // every fragment of the slice first, then the MFMAs, then the
        // squares (a branch among the reads would expose each one's latency)
        bf16x8 xf[kTpK / 16], wf[kTpK / 16][EB];
#pragma unroll
        for (int ks = 0; ks < kTpK / 16; ++ks) {
            const int ch = ks * 2 + lg;
            xf[ks] = *reinterpret_cast<const bf16x8*>(X + tp_off(wave * 32 + lr, ch));
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
                wf[ks][eb] = *reinterpret_cast<const bf16x8*>(W + tp_off(eb * 32 + lr, ch));
        }
#pragma unroll
        for (int ks = 0; ks < kTpK / 16; ++ks)
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
                acc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][eb], xf[ks], acc[eb], 0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < kTpK / 16; ++ks) sx += sumsq(__builtin_bit_cast(u32x4, xf[ks]));
#pragma unroll
        for (int q = 0; q < kNwq; ++q) {
            const int eb = wave + RG::kWaves * q;
            if (eb < EB) {
#pragma unroll
                for (int ks = 0; ks < kTpK / 16; ++ks)
                    sw[q] += sumsq(*reinterpret_cast<const u32x4*>(W + tp_off(eb * 32 + lr, ks * 2 + lg)));
            }
        }
    }, std::integral_constant<int, 2>{});  // x requests non-temporal (aux 2): with x about the
                                             // Infinity Cache's size, the chains' pass then hits it
                                             // more often (-8 % on 32768 x 4096 tokens)
    // norms: lanes lr and lr + 32 hold the two halves of a row's sum
    {
        const float v = sx + __shfl_xor(sx, 32, kWave);
        if (lg == 0) nx[wave * 32 + lr] = __builtin_sqrtf(v);
#pragma unroll
        for (int q = 0; q < kNwq; ++q) {
            const int eb = wave + RG::kWaves * q;
            if (eb < EB) {
                const float u = sw[q] + __shfl_xor(sw[q], 32, kWave);
                if (lg == 0) nw[eb * 32 + lr] = __builtin_sqrtf(u);
            }
        }
    }
    __syncthreads();

    // ---- phase 2: candidates. acc[eb][v] is token wave*32 + lr and expert
    // eb*32 + 8*(v/4) + 4*lg + v%4.
    {
        const int tl = wave * 32 + lr;
        const float du = static_cast<float>(d) * 0x1p-24f;
        const float c1 = 8.0f * du * nx[tl];  // eps = c1 |w| + 8 * 2^-24 |zt| + 2^-126
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
                const float zt = acc[eb][v] + (bias != nullptr ? nb[e] : 0.0f);
                const float eps = c1 * nw[e] + 8.0f * 0x1p-24f * __builtin_fabsf(zt) + 0x1p-126f;
                const float L = zt - eps;
                acc[eb][v] = zt + eps;  // keep the upper bound U for the mask
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
                if (bad || acc[eb][v] >= tau) word |= 1u << b;
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
    // x and the gate weight through the ring again, and lane l advances the
    // chains of pairs l + 64 j, j < nc (nc = the list's length over 64,
    // rounded up; lanes past the end repeat pair 0 and discard it) in the
    // canonical order. The pair list and the logits live in the wave's part
    // of the ring while it is idle.
    int* pair = reinterpret_cast<int*>(lds) + wave * 2 * kTpPairCap;
    float* pz = reinterpret_cast<float*>(pair + kTpPairCap);
    int* npass = reinterpret_cast<int*>(nb + EB * 32);  // [kWaves] passes per wave
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
    int passes = 0;
#pragma unroll
    for (int w = 0; w < RG::kWaves; ++w) passes = max(passes, npass[w]);
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
        const int nc = total <= kWave ? 1 : (total + kWave - 1) / kWave;
        int pc[kCh];
        float z[kCh];
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int r = j * kWave + lane;
            pc[j] = (total > 0 && r < total) ? pair[r] : (total > 0 ? pair[0] : 0);
            z[j] = 0.0f;
        }
        __syncthreads();  // every list is read before the ring refills
        stream(0, [&](const uint8_t* S) {  // the chains' order: from slice 0
            const uint8_t* X = S;
            const uint8_t* W = S + RG::kXBytes;
            if (total > 0) {
                switch (nc) {
                    case 1: run_chains<1>(X, W, pc, z); break;
                    case 2: run_chains<2>(X, W, pc, z); break;
                    case 3: run_chains<3>(X, W, pc, z); break;
                    case 4: run_chains<4>(X, W, pc, z); break;
                    case 5: run_chains<5>(X, W, pc, z); break;
                    case 6: run_chains<6>(X, W, pc, z); break;
                    case 7: run_chains<7>(X, W, pc, z); break;
                    default: run_chains<8>(X, W, pc, z); break;
                }
            }
        }, std::integral_constant<int, 0>{});
        __syncthreads();  // every wave is done with the last slice before the lists' bytes are rewritten
        // the exact logits of the listed pairs, in the wave's own part
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int r = j * kWave + lane;
            if (r < total) {
                const int e = pc[j] & 0xffff;
                pz[r] = bias != nullptr ? z[j] + nb[e] : z[j];
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
    using RG = TpRing<EB>;
    constexpr int lds = RG::kLds;
    static_assert(RG::kSlots * RG::kSlot >= RG::kWaves * 2 * kTpPairCap * 4, "pair lists fit in the ring");
    static_assert(lds <= 160 * 1024, "LDS of one work-group");
    static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_two_phase_kernel<EB>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    const unsigned blocks = static_cast<unsigned>((s.T + RG::kTok - 1) / RG::kTok);
    gate_two_phase_kernel<EB><<<blocks, RG::kThreads, lds, st>>>(static_cast<const bf16_t*>(x),
                                                         static_cast<const bf16_t*>(wg), bias, s.T,
                                                         s.d, s.E, s.k, idx, w);
    return hipGetLastError();
}
}  // namespace

// The two-phase gate for bf16 inputs where it is the faster one: its cost
// follows the reads of x (twice) and the candidates' chains, the one-phase
// kernel's the T*E chains, so it wins with many experts -- measured at
// d = 4096: E = 128, T = 65536, k = 4 in 0.36-0.41 ms against 1.37 ms;
// E = 64, T = 32768, k = 6 in 0.35 against 0.39; E = 32, T = 4096 in 0.14
// against 0.03 -- and needs enough work-groups to fill the chip.
// Returns false (nothing launched) otherwise.
// The environment variable MOE_GATE_PATH = "two_phase" or "one_phase"
// overrides the choice (both give the same results; tests use it to run
// each path at any size).
bool gate_two_phase_chosen(const moe_shape& s) {
    // (d below 2^21: the ring's offsets, and the out-of-range offset it
    // uses for chunks past d, stay within 32 bits)
    if (s.act != MOE_BF16 || s.E > 256 || s.d >= (1 << 21)) return false;
    const char* force = std::getenv("MOE_GATE_PATH");
    if (force != nullptr && std::strcmp(force, "one_phase") == 0) return false;
    const bool forced = force != nullptr && std::strcmp(force, "two_phase") == 0;
    return forced || (s.E >= 64 && s.T >= 32768);
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
