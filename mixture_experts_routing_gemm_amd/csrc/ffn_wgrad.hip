// Weight gradients of the grouped SwiGLU expert FFN on the matrix cores.
//
// "Deepseek-MoE同步税本质与四层实战优化指南" (gsyq.cn), section 2.4: the
// backward returns along the forward's routing through the experts' own
// computation. For every expert group g with rows r (routed: its dispatched
// rows; shared experts, "DeepSeek 中 MoE 的同步税" (wmrh.cn) section 2.1:
// every token), input rows v, hidden rows hid, output gradients dy and the
// SwiGLU gradients [da | db] (2h values per row):
//     [dW1; dW3]_g = sum_r [da | db]_r^T v_r      (a [2h, d] product)
//     dW2_g        = sum_r dy_r^T hid_r           (a [d, h] product)
// Both are sums over token rows, and every operand is stored row by row
// (token-major), so the contraction index runs across rows: one 16-byte chunk
// of a row holds 8 consecutive output features. Slices of 32 rows stream
// global -> LDS as they are stored (direct buffer-to-LDS loads, a ring of four
// slots, three slices ahead), and the matrix-core fragments, which need 8
// consecutive rows of one feature per lane, come out of LDS through the
// transposing read (ds_read_b64_tr_b16: within each 16 lanes, lane i gets
// element r of the 4 values that lane (i >> 2) + 4 r points at, value i & 3),
// interleaved one fragment per MFMA.
//
// One work-group of eight waves per CU takes 256 x 256 output tiles from a
// list ordered by the group's rows, longest first; each output element has
// one owner, which sums its group's rows in order, so every call gives the
// same bits.
#include <algorithm>

#include "lds_ring.h"
#include "moe_device.h"

namespace moe {

constexpr int kWgT = 256;         // output tile: M x N
constexpr int kWgK = 32;          // token rows per slice
constexpr int kWgOp = kWgK * kWgT * 2;  // bytes of one operand's slice (16 KB)
constexpr int kWgSlot = 2 * kWgOp;
constexpr int kWgSlots = 4;
constexpr int kWgLds = kWgSlots * kWgSlot;

struct WgradArgs {
    const int32_t* offsets;  // [E+1] routed row offsets
    const int32_t* order;    // [E+S] groups by rows, descending (written by the plan)
    int32_t* counters;       // [8] tile queues, one per XCD
    int64_t T;
    int E, S, d, h;
    // [da | db] rows: routed [R, 2h], shared [T, S*2h]
    const uint8_t* dd_r;
    const uint8_t* dd_s;
    // input rows: routed x_perm [R, d], shared x [T, d]
    const uint8_t* v_r;
    const uint8_t* v_s;
    // output gradient rows: routed [R, d], shared [T, d]
    const uint8_t* dy_r;
    const uint8_t* dy_s;
    // hidden rows: routed [R, h], shared [T, S*h]
    const uint8_t* hid_r;
    const uint8_t* hid_s;
    float* dw1;  // [G, h, d]
    float* dw3;  // [G, h, d]
    float* dw2;  // [G, d, h]
    uint32_t bytes_dd_r, bytes_dd_s, bytes_v_r, bytes_v_s, bytes_dy_r, bytes_dy_s, bytes_hid_r,
        bytes_hid_s;
    int ntiles;  // tiles per group: t13 [dW1; dW3] tiles, then the dW2 ones
    int t13;
};

// Plan: the groups ordered by rows, descending (ties by index), and the
// queues cleared. One work-group.
__global__ __launch_bounds__(256) void wgrad_plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int S, int64_t T, int32_t* __restrict__ order,
                                                         int32_t* __restrict__ counters) {
    __shared__ int rows[kMaxE + kMaxS];
    const int G = E + S;
    for (int g = threadIdx.x; g < G; g += blockDim.x)
        rows[g] = g < E ? offsets[g + 1] - offsets[g] : static_cast<int>(T);
    __syncthreads();
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        int rank = 0;
        for (int q = 0; q < G; ++q) rank += (rows[q] > rows[g] || (rows[q] == rows[g] && q < g)) ? 1 : 0;
        order[rank] = g;
    }
    if (threadIdx.x < 8) counters[threadIdx.x] = 0;
}

// The tile list (groups longest first, then their tiles) is dealt to the 8
// XCDs in chunks of kWgChunk consecutive tiles, chunk j to XCD j % 8: every
// XCD gets about an eighth of every group's work (balance), and the tiles of
// a chunk, which share one row panel, run under one L2. Position c of XCD
// x's list is tile (c / kWgChunk * 8 + x) * kWgChunk + c % kWgChunk.
constexpr int kWgChunk = 4;
__device__ __forceinline__ int wg_tile_of(int x, int c) {
    return ((c / kWgChunk) * 8 + x) * kWgChunk + c % kWgChunk;
}

// swizzle of the 16-byte chunks of slice row k: chunk c is stored at c ^ sw(k),
// so that the transposing reads (4 rows x 32 or 64 bytes per 16 or 32 lanes)
// hit distinct banks
__device__ __forceinline__ int wg_sw(int k) { return (0xEA40 >> (4 * (k & 3))) & 15; }  // 0, 4, 10, 14
__device__ __forceinline__ int wg_off(int k, int m) {
    return k * (kWgT * 2) + ((((m >> 3) ^ wg_sw(k))) << 4) + (m & 7) * 2;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
// This lane's byte offset, within an operand slice, of the 8 bytes it points
// the transposing read at for the fragment of features f0 .. f0+31 and rows
// 0 .. 15: row k = 8 (lane / 32) + (lane % 16) / 4, features f = f0 + 16
// ((lane / 16) % 2) + 4 (lane % 4) .. +3. Rows 4 and 16 further are a
// constant offset (k % 4 and so the swizzle stay the same).
__device__ __forceinline__ uint32_t wg_frag_off(int f0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int k = 8 * (g >> 1) + (s >> 2);
    const int f = f0 + 16 * (g & 1) + 4 * (s & 3);
    return static_cast<uint32_t>(wg_off(k, f));
}
// the LDS byte address of a pointer into the work-group's LDS
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// The slices' buffer -> LDS requests are inline asm, with the LDS address
// bound to M0 as an input so that the compiler sets M0 itself (the asm has no
// register results: the request writes LDS only, and the kernel's counted
// waits and barriers order it). Issued through the builtin instead, each
// request counts as an LDS write to the compiler, which then waits for every
// outstanding request before each transposing read it cannot tell apart from
// them, draining the prefetched slices at every step. The reads themselves
// are builtins, so the compiler schedules them among the MFMAs with partial
// waits. (s_nop 0: one wait state between an M0 write and an LDS DMA.)
typedef int i32x4w __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void wg_dma16(i32x4w rsrc, uint32_t voff, uint32_t ldsaddr) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(ldsaddr));
}
// a raw buffer resource over [base, base + bytes), wave-uniform
__device__ __forceinline__ i32x4w wg_rsrc(const uint8_t* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4w r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r[3] = kBufferFlags;
    return r;
}
// One fragment: the transposing reads of rows +0 and +4 (2048 bytes apart) at
// byte offset a of the work-group's LDS (lds_base).
__device__ __forceinline__ bf16x8 wg_frag(const uint8_t* lds_base, uint32_t a) {
    typedef __attribute__((address_space(3))) v4i16 lv4;
    const __attribute__((address_space(3))) uint8_t* p = (const __attribute__((address_space(3))) uint8_t*)lds_base;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4*)(p + a));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4*)(p + a + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

struct WgTile {
    int g, type, mt, nt;  // type 0: [dW1; dW3] (M = 2h, N = d), 1: dW2 (M = d, N = h)
    int nrows;
    int64_t row0;         // first row of the group in its operands
    int shared, sidx;     // shared expert s = sidx
};

__device__ __forceinline__ WgTile wg_decode(const WgradArgs& a, int L) {
    WgTile t;
    const int p = L / a.ntiles, j = L - p * a.ntiles;
    t.g = a.order[p];
    t.shared = t.g >= a.E ? 1 : 0;
    t.sidx = t.shared ? t.g - a.E : 0;
    t.row0 = t.shared ? 0 : a.offsets[t.g];
    t.nrows = t.shared ? static_cast<int>(a.T) : a.offsets[t.g + 1] - a.offsets[t.g];
    if (j < a.t13) {
        const int ntm = 2 * a.h / kWgT;  // consecutive tiles share an input-row panel
        t.type = 0;
        t.nt = j / ntm;
        t.mt = j - t.nt * ntm;
    } else {
        const int j2 = j - a.t13, ntm = a.d / kWgT;
        t.type = 1;
        t.nt = j2 / ntm;
        t.mt = j2 - t.nt * ntm;
    }
    return t;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ffn_wgrad_kernel(WgradArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int* lds_next = reinterpret_cast<int*>(lds + kWgLds);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wn = wave & 3, wm = wave >> 2;
    const int lr = lane & 31, lg = lane >> 5;
    // this lane's offsets of the six fragments of a half-slice: the two B
    // blocks (features wn*64 + 32 i), then the four A blocks (wm*128 + 32 i)
    uint32_t fo[6];
#pragma unroll
    for (int i = 0; i < 6; ++i)
        fo[i] = wg_frag_off(i < 2 ? wn * 64 + i * 32 : wm * 128 + (i - 2) * 32, lane);
    // XCD x (work-groups b with b % 8 == x) takes the tiles of its list: the
    // first one static, later ones from its queue
    const int xcd = blockIdx.x & 7, per_xcd = static_cast<int>(gridDim.x >> 3);
    const int total = (a.E + a.S) * a.ntiles;
    int c = static_cast<int>(blockIdx.x >> 3);
    for (int it = 0; wg_tile_of(xcd, c) < total; ++it) {
        const WgTile t = wg_decode(a, wg_tile_of(xcd, c));
        // the claim on the next tile, published through LDS at the end (two
        // words by tile parity: a word is rewritten only after every wave
        // has passed the barrier that follows its read)
        if (tid == 0) lds_next[it & 1] = per_xcd + atomicAdd(a.counters + xcd, 1);

        if (t.nrows == 0) {
            // a group without rows (common under skewed routing): its
            // gradient tile is zero, stored a row of 16-byte chunks per
            // 64 lanes instead of through the accumulator layout
            const int M0 = t.mt * kWgT, N0 = t.nt * kWgT;
            const int ncols = t.type == 0 ? kWgT : min(kWgT, a.h - N0);
            const int q = ncols / 4;  // 16-byte chunks a row
            for (int i = tid; i < kWgT * q; i += 512) {
                const int m = M0 + i / q, col = N0 + 4 * (i % q);
                float* out;
                if (t.type == 0)
                    out = m < a.h ? a.dw1 + (static_cast<int64_t>(t.g) * a.h + m) * a.d + col
                                  : a.dw3 + (static_cast<int64_t>(t.g) * a.h + (m - a.h)) * a.d + col;
                else
                    out = a.dw2 + (static_cast<int64_t>(t.g) * a.d + m) * a.h + col;
                *reinterpret_cast<f32x4*>(out) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            wait_vmcnt<0>();
            __syncthreads();
            c = lds_next[it & 1];
            continue;
        }
        // operands of this tile: A rows hold its M features, B rows its N
        const uint8_t* abuf;
        const uint8_t* bbuf;
        uint32_t abytes, bbytes, lda, ldb, acol, bcol;  // row strides and column offsets in bytes
        if (t.type == 0) {
            abuf = t.shared ? a.dd_s : a.dd_r;
            abytes = t.shared ? a.bytes_dd_s : a.bytes_dd_r;
            lda = static_cast<uint32_t>((t.shared ? a.S : 1) * 2 * a.h) * 2;
            acol = static_cast<uint32_t>(t.sidx * 2 * a.h + t.mt * kWgT) * 2;
            bbuf = t.shared ? a.v_s : a.v_r;
            bbytes = t.shared ? a.bytes_v_s : a.bytes_v_r;
            ldb = static_cast<uint32_t>(a.d) * 2;
            bcol = static_cast<uint32_t>(t.nt * kWgT) * 2;
        } else {
            abuf = t.shared ? a.dy_s : a.dy_r;
            abytes = t.shared ? a.bytes_dy_s : a.bytes_dy_r;
            lda = static_cast<uint32_t>(a.d) * 2;
            acol = static_cast<uint32_t>(t.mt * kWgT) * 2;
            bbuf = t.shared ? a.hid_s : a.hid_r;
            bbytes = t.shared ? a.bytes_hid_s : a.bytes_hid_r;
            ldb = static_cast<uint32_t>((t.shared ? a.S : 1) * a.h) * 2;
            bcol = static_cast<uint32_t>(t.sidx * a.h + t.nt * kWgT) * 2;
        }
        abuf = uniform_ptr(abuf);
        bbuf = uniform_ptr(bbuf);
        abytes = __builtin_amdgcn_readfirstlane(abytes);
        bbytes = __builtin_amdgcn_readfirstlane(bbytes);
        const i32x4w ars = wg_rsrc(abuf, abytes), brs = wg_rsrc(bbuf, bbytes);
        // this lane's two chunks per operand and slice: request q (0, 1) of
        // the wave fills LDS bytes 1024 (2 wave + q) + 16 lane of the
        // operand's slice, i.e. slice row k = 4 wave + 2 q + lane / 32 and
        // stored chunk lane % 32, which holds source chunk (lane % 32) ^ sw(k)
        uint32_t arow[2], brow[2];  // byte offsets of the chunk in row 0 of the group
        int krow[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = 4 * wave + 2 * q + (lane >> 5);
            const int c = (lane & 31) ^ wg_sw(k);
            krow[q] = k;
            arow[q] = static_cast<uint32_t>(t.row0) * lda + acol + 16 * c;
            brow[q] = static_cast<uint32_t>(t.row0) * ldb + bcol + 16 * c;
        }
        const int KT = (t.nrows + kWgK - 1) / kWgK;
        auto issue = [&](int s) {
            uint8_t* slot = lds + (s & 3) * kWgSlot;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int k = s * kWgK + krow[q];
                // rows past the group read as zero (an offset past the buffer)
                const bool in = k < t.nrows;
                const uint32_t ao = in ? arow[q] + static_cast<uint32_t>(k) * lda : 0xfffffff0u;
                const uint32_t bo = in ? brow[q] + static_cast<uint32_t>(k) * ldb : 0xfffffff0u;
                wg_dma16(ars, ao, __builtin_amdgcn_readfirstlane(lds_addr(slot + 1024 * (2 * wave + q))));
                wg_dma16(brs, bo, __builtin_amdgcn_readfirstlane(lds_addr(slot + kWgOp + 1024 * (2 * wave + q))));
            }
        };

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // One step per slice k. First half: slice k+3 is requested (into the
        // slot of slice k-1), and the MFMAs of slice k's first 16 rows (fa0,
        // fb0, read before) are issued, each followed by the read of one
        // fragment of its last 16 rows; then, once slice k+1 has landed and
        // every wave has passed the barrier, the MFMAs of the last 16 rows,
        // each followed by the read of one of slice k+1's first fragments.
        // (After the last slice those reads take a settled slot and are not
        // used: one MFMA chain per half, with no branch around it.)
        bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
        // fragment i of half-slice KS of slot R: the two B blocks, then the
        // four A blocks
        auto frag_of = [&](const uint8_t* R, auto KS, int i) {
            constexpr int ks = decltype(KS)::value;
            const uint32_t base = static_cast<uint32_t>(R - lds) + ks * 8192;
            return wg_frag(lds, base + (i < 2 ? kWgOp : 0) + fo[i]);
        };
        auto read_half = [&](const uint8_t* R, auto KS, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
            fb[0] = frag_of(R, KS, 0);
            fb[1] = frag_of(R, KS, 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = frag_of(R, KS, 2 + i);
        };
        if (KT > 0) {
            issue(0);
            if (KT > 1) issue(1);
            if (KT > 2) issue(2);
            // slice 0 has landed once at most the later slices' requests
            // (four per slice) are outstanding
            if (KT > 2) wait_vmcnt<8>();
            else if (KT > 1) wait_vmcnt<4>();
            else wait_vmcnt<0>();
            ring_barrier();
            read_half(lds, ic<0>(), fa0, fb0);
        }
        // the MFMAs of one half-slice (fa, fb), each followed by the read of
        // one fragment of half-slice KS of slot R (into na, nb)
        auto mma_read = [&](const bf16x8* fa, const bf16x8* fb, const uint8_t* R, auto KS, bf16x8 (&na)[4],
                            bf16x8 (&nb)[2]) {
            static_for<0, 8>([&](auto I) {
                constexpr int i = decltype(I)::value;
                acc[i / 2][i % 2] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i / 2], fb[i % 2], acc[i / 2][i % 2], 0, 0, 0);
                if constexpr (i < 2)
                    nb[i] = frag_of(R, KS, i);
                else if constexpr (i < 6)
                    na[i - 2] = frag_of(R, KS, i);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int k = 0; k < KT; ++k) {
            const uint8_t* A = lds + (k & 3) * kWgSlot;
            if (k + 3 < KT) issue(k + 3);
            mma_read(fa0, fb0, A, ic<1>(), fa1, fb1);
            const bool next = k + 1 < KT;
            if (next) {
                // slices issued after k+1: k+2 and k+3, as far as they exist
                if (k + 3 < KT) wait_vmcnt<8>();
                else if (k + 2 < KT) wait_vmcnt<4>();
                else wait_vmcnt<0>();
                ring_barrier();
            }
            mma_read(fa1, fb1, lds + ((k + 1) & 3) * kWgSlot, ic<0>(), fa0, fb0);
        }

        // epilogue: acc[mb][nb][v] is output row m = wm*128 + mb*32 + 8 (v/4)
        // + 4 lg + v%4 and column n = wn*64 + nb*32 + lr of the tile
        const int M0 = t.mt * kWgT, N0 = t.nt * kWgT;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int mblk = M0 + wm * 128 + mb * 32;  // 32 rows, all in dW1, dW3 or dW2
            float* out;
            int ldo;
            if (t.type == 0) {
                out = mblk < a.h ? a.dw1 + (static_cast<int64_t>(t.g) * a.h + mblk) * a.d
                                 : a.dw3 + (static_cast<int64_t>(t.g) * a.h + (mblk - a.h)) * a.d;
                ldo = a.d;
            } else {
                out = a.dw2 + (static_cast<int64_t>(t.g) * a.d + mblk) * a.h;
                ldo = a.h;
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int n = N0 + wn * 64 + nb * 32;
                if (t.type == 1 && n >= a.h) continue;  // a last partial tile of dW2 (h % 256 == 128)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 8 * (v >> 2) + 4 * lg + (v & 3);
                    out[static_cast<int64_t>(m) * ldo + n + lr] = acc[mb][nb][v];
                }
            }
        }
        // the stores complete before the next tile's counted waits; the claim
        // is visible, and every wave is done with the ring
        wait_vmcnt<0>();
        __syncthreads();
        c = lds_next[it & 1];
    }
}

// Shapes it takes: bf16 input rows, d % 256 == 0, h % 128 == 0, every operand
// under 4 GiB (32-bit offsets).
bool wgrad_supported(const moe_shape& s) {
    const uint64_t R = static_cast<uint64_t>(s.T) * s.k, T = static_cast<uint64_t>(s.T);
    const uint64_t lim = uint64_t(1) << 32;
    return s.act == MOE_BF16 && s.dispatch == MOE_BF16 && s.d % kWgT == 0 && s.h % (kWgT / 2) == 0 &&
           R * s.d * 2 < lim && T * s.d * 2 < lim && R * 2 * s.h * 2 < lim && T * s.S * 2 * s.h * 2 < lim;
}

size_t wgrad_ws_bytes(const moe_shape& s) { return static_cast<size_t>(s.E + s.S + 32) * 4; }

int device_cus();

// ws: wgrad_ws_bytes(s) (the group order and the queue). [da | db] rows as the
// backward's persistent path writes them.
hipError_t launch_ffn_wgrad(const moe_shape& s, const int32_t* offsets, const void* dd_r,
                            const void* dd_s, const void* v_r, const void* v_s, const void* dy_r,
                            const void* dy_s, const void* hid_r, const void* hid_s, float* dw1,
                            float* dw3, float* dw2, void* ws, hipStream_t st) {
    static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_wgrad_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kWgLds + 16);
    static_assert(kWgLds + 16 <= 160 * 1024, "LDS");
    if (attr != hipSuccess) return attr;
    const int G = s.E + s.S;
    int32_t* order = static_cast<int32_t*>(ws);
    int32_t* counters = order + G + 16;
    const int t13 = (2 * s.h / kWgT) * (s.d / kWgT);
    const int ntiles = t13 + (s.d / kWgT) * ((s.h + kWgT - 1) / kWgT);
    wgrad_plan_kernel<<<1, 256, 0, st>>>(offsets, s.E, s.S, s.T, order, counters);
    WgradArgs a{};
    a.offsets = offsets;
    a.order = order;
    a.counters = counters;
    a.T = s.T;
    a.E = s.E;
    a.S = s.S;
    a.d = s.d;
    a.h = s.h;
    const uint64_t R = static_cast<uint64_t>(s.T) * s.k, T = static_cast<uint64_t>(s.T);
    a.dd_r = static_cast<const uint8_t*>(dd_r);
    a.dd_s = static_cast<const uint8_t*>(dd_s);
    a.v_r = static_cast<const uint8_t*>(v_r);
    a.v_s = static_cast<const uint8_t*>(v_s);
    a.dy_r = static_cast<const uint8_t*>(dy_r);
    a.dy_s = static_cast<const uint8_t*>(dy_s);
    a.hid_r = static_cast<const uint8_t*>(hid_r);
    a.hid_s = static_cast<const uint8_t*>(hid_s);
    a.bytes_dd_r = static_cast<uint32_t>(R * 2 * s.h * 2);
    a.bytes_dd_s = static_cast<uint32_t>(T * s.S * 2 * s.h * 2);
    a.bytes_v_r = static_cast<uint32_t>(R * s.d * 2);
    a.bytes_v_s = static_cast<uint32_t>(s.S > 0 ? T * s.d * 2 : 0);
    a.bytes_dy_r = static_cast<uint32_t>(R * s.d * 2);
    a.bytes_dy_s = static_cast<uint32_t>(s.S > 0 ? T * s.d * 2 : 0);
    a.bytes_hid_r = static_cast<uint32_t>(R * s.h * 2);
    a.bytes_hid_s = static_cast<uint32_t>(T * s.S * s.h * 2);
    a.dw1 = dw1;
    a.dw3 = dw3;
    a.dw2 = dw2;
    a.t13 = t13;
    a.ntiles = ntiles;
    // a multiple of 8 work-groups (one per CU): the same count on every XCD
    const unsigned blocks = static_cast<unsigned>(std::max(8, device_cus() & ~7));
    ffn_wgrad_kernel<<<blocks, 512, kWgLds + 16, st>>>(a);
    return hipGetLastError();
}

// The gate backward's weight gradient (see GateMfmaPlan): for the C chunks
// of token rows at `offsets` (C + 1 entries, in the workspace), the [dW1;
// dW3] tiles of the kernel with the chunks as groups, Zp [T, F] as the
// [da | db] rows (h = F / 2) and x [T, d] as the input rows: chunk c's
// features f < F / 2 go to p1 [C, F / 2, d], the others to p3. No dW2 tiles.
// ws: C + 32 ints (the chunk order and the queues).
hipError_t launch_wgrad_planes(const int32_t* offsets, int C, int64_t T, int d, int F,
                               const void* zp, const void* x, float* p1, float* p3, void* ws,
                               hipStream_t st) {
    static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_wgrad_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kWgLds + 16);
    if (attr != hipSuccess) return attr;
    if (C < 1 || C > kMaxE || F % kWgT != 0 || d % kWgT != 0) return hipErrorInvalidValue;
    int32_t* order = static_cast<int32_t*>(ws);
    int32_t* counters = order + C + 16;
    wgrad_plan_kernel<<<1, 256, 0, st>>>(offsets, C, 0, T, order, counters);
    WgradArgs a{};
    a.offsets = offsets;
    a.order = order;
    a.counters = counters;
    a.T = T;
    a.E = C;
    a.S = 0;
    a.d = d;
    a.h = F / 2;
    a.dd_r = static_cast<const uint8_t*>(zp);
    a.v_r = static_cast<const uint8_t*>(x);
    a.bytes_dd_r = static_cast<uint32_t>(static_cast<uint64_t>(T) * F * 2);
    a.bytes_v_r = static_cast<uint32_t>(static_cast<uint64_t>(T) * d * 2);
    a.dw1 = p1;
    a.dw3 = p3;
    a.t13 = (F / kWgT) * (d / kWgT);
    a.ntiles = a.t13;
    const unsigned blocks = static_cast<unsigned>(std::max(8, device_cus() & ~7));
    ffn_wgrad_kernel<<<blocks, 512, kWgLds + 16, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
