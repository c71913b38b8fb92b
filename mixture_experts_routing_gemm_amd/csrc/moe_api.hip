// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and the launch sequence. No call here allocates device
// memory or synchronises, except moe_get_device_error (documented).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "ffn_plan.h"
#include "moe.h"
#include "moe_device.h"

namespace moe {
bool gate_two_phase_chosen(const moe_shape& s);
hipError_t launch_gate_topk(const moe_shape& s, const void* x, const void* wg, const float* bias,
                            int32_t* idx, float* w, float* dbg, hipStream_t st, const Marks* mk);
hipError_t launch_dispatch(const moe_shape& s, const void* x, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* dest_row,
                           int32_t* src_token, void* x_perm, float* qparams, int32_t* rank,
                           int32_t* blk, int32_t* pre, int32_t* first_loads, uint32_t* qstats,
                           uint32_t* hdr, const FfnPlanArgs& fp, hipStream_t st,
                           const Marks* mk, uint8_t* x_self = nullptr, float* q_self = nullptr);
hipError_t launch_grouped_ffn(const moe_shape& s, const void* x_perm, const float* qparams,
                              const int32_t* offsets, const void* x, const void* w1,
                              const void* w3, const void* w2, void* y_perm, void* y_shared,
                              int32_t* plan, void* h_routed, void* h_shared, bool plan_done,
                              hipStream_t st, const Marks* mk, const int32_t* gather = nullptr,
                              void* pre_a_r = nullptr, void* pre_b_r = nullptr, void* pre_a_s = nullptr,
                              void* pre_b_s = nullptr);
bool use_big_tiles(const moe_shape& s);
// whether the whole-layer forward's up-projection reads its routed rows from
// x through src_token (bf16 rows, persistent tiles) instead of from x_perm
bool ffn_gathers_rows(const moe_shape& s);
size_t ffn_plan_bytes(const moe_shape& s);
int ffn_hidden_stride(const moe_shape& s);
bool ffn_fused_plan(const moe_shape& s, int32_t* plan, FfnPlanArgs* fp);
hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_sh,
                          const int32_t* dest_row, const float* topk_w, void* y, hipStream_t st);
size_t gate_backward_ws_bytes(const moe_shape& s);
hipError_t launch_gate_backward(const moe_shape& s, const void* x, const void* wg,
                                const int32_t* topk_idx, const float* topk_w,
                                const float* dtopk_w, float* dz, void* dx, float* dwg,
                                float* part, hipStream_t st);
hipError_t launch_combine_backward(const moe_shape& s, const void* dy, const void* y_perm,
                                   const int32_t* dest_row, const float* topk_w, void* dy_perm,
                                   float* dtopk_w, hipStream_t st);

size_t ffn_backward_ws_bytes(const moe_shape& s);
size_t fp8w_scale_floats(const moe_shape& s);
bool f8w_supported(const moe_shape& s);
hipError_t launch_quantize_weights(const moe_shape& s, const void* w1, const void* w3,
                                   const void* w2, uint8_t* w1q, uint8_t* w3q, uint8_t* w2q,
                                   float* wscale, hipStream_t st);
hipError_t launch_grouped_ffn_f8w(const moe_shape& s, const void* x_perm, const float* qparams,
                                  const int32_t* offsets, const void* x8, const float* q8,
                                  const uint8_t* w1q, const uint8_t* w3q, const uint8_t* w2q,
                                  const float* wscale, void* y_perm, void* y_shared,
                                  int32_t* plan, void* h_r, void* h_s, uint8_t* h8_r,
                                  uint8_t* h8_s, float* hsc_r, float* hsc_s, bool plan_done,
                                  hipStream_t st, const Marks* mk);
hipError_t launch_ffn_backward(const moe_shape& s, const void* x_perm, const float* qparams,
                               const int32_t* offsets, const void* x, const void* w1,
                               const void* w3, const void* w2, const void* dy_perm,
                               const void* dy_sh, void* dx_perm, void* dx_sh, float* dw1,
                               float* dw3, float* dw2, void* ws, hipStream_t st,
                               const Marks* mk, const void* saved = nullptr);

__global__ void clear_header_kernel(uint32_t* hdr) { hdr[threadIdx.x] = 0u; }

__global__ void zero_f32_kernel(float* p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0.0f;
}
}  // namespace moe

using namespace moe;

// ------------------------------------------------ allocation-free dispatch --
// Device memory for moe_dispatch_noalloc's working arrays (the header with
// the error flag, the per-slot ranks, the per-block counts and prefixes, the
// first-pass loads and the fp8 ranges): one copy per GPU, held by the loaded
// code object until the process ends. Host code never passes `scratch`
// itself to a kernel -- in host code that name is only a stand-in -- but the
// device address of the current GPU's copy, looked up once per device.
static constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr size_t kHeaderBytes = 256;
// kernels of moe_forward_fp8w, in order: gate_topk, dispatch_rank,
// dispatch_scan, dispatch_permute_fp8, ffn_plan, ffn_up, ffn_hidden_quant,
// ffn_down, combine
constexpr int kFp8wKernels = 9;

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

size_t act_bytes(int32_t dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
    size_t x8 = 0, q8 = 0, h8_r = 0, h8_s = 0, hsc_r = 0, hsc_s = 0;  // fp8-weight forward
    size_t fbwd = 0, part = 0, rank = 0, blk = 0, pre = 0, loads = 0, qstats = 0, plan = 0, x_perm = 0, qparams = 0, h_r = 0, h_s = 0, y_perm = 0,
           y_sh = 0, total = 0;
};

Layout layout(const moe_shape& s, int stage) {
    Layout L;
    const size_t T = static_cast<size_t>(s.T), k = s.k, d = s.d, S = s.S, E = s.E;
    const size_t es = act_bytes(s.act), esd = act_bytes(s.dispatch);
    const size_t nblk = (T + kRankBlockTokens - 1) / kRankBlockTokens;
    size_t off = kHeaderBytes;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const bool fwd = stage == MOE_STAGE_FORWARD || stage == MOE_STAGE_FORWARD_FP8W;
    const bool disp = stage == MOE_STAGE_DISPATCH || fwd;
    const bool ffn = stage == MOE_STAGE_FFN || fwd;
    if (disp) {
        L.rank = take(T * k * 4);
        L.blk = take(nblk * E * 4);
        L.pre = take(nblk * E * 4);
        L.loads = take(E * 4);  // first-pass loads under a capacity limit
        L.qstats = take((E + 1) * 8);  // fp8 (min, max) ranges of the group modes
    }
    if (ffn) {
        // m-tile prefix, tile counters and tile descriptors
        L.plan = take(ffn_plan_bytes(s));
        const size_t hs = static_cast<size_t>(ffn_hidden_stride(s));
        L.h_r = take(T * k * hs * es);
        L.h_s = take(T * S * hs * es);
    }
    if (fwd) {
        // (no permuted rows when the up-projection gathers them from x)
        const bool gather = stage == MOE_STAGE_FORWARD && ffn_gathers_rows(s);
        L.x_perm = take(gather ? 0 : T * k * d * esd);
        L.qparams = take(s.dispatch == MOE_FP8_E4M3 ? T * k * 8 : 0);
        L.y_perm = take(T * k * d * es);
        L.y_sh = take(S > 0 ? T * d * es : 0);
    }
    if (stage == MOE_STAGE_FORWARD_FP8W) {
        // the shared experts' fp8 token rows, the hidden rows' codes and scales
        L.x8 = take(S > 0 ? T * d : 0);
        L.q8 = take(S > 0 ? T * 8 : 0);
        L.h8_r = take(T * k * static_cast<size_t>(s.h));
        L.h8_s = take(T * S * static_cast<size_t>(s.h));
        L.hsc_r = take(T * k * 4);
        L.hsc_s = take(S > 0 ? T * 4 : 0);
    }
    if (stage == MOE_STAGE_GATE_BACKWARD) {
        // the weight gradient's partials (and, on the matrix-core path, the
        // plane rows and the chunk queue)
        L.part = take(gate_backward_ws_bytes(s));
    }
    if (stage == MOE_STAGE_FFN_BACKWARD) {
        // plan, recomputed a / b / hidden rows and their gradients
        L.fbwd = take(ffn_backward_ws_bytes(s));
    }
    L.total = (disp || ffn || stage == MOE_STAGE_GATE_BACKWARD || stage == MOE_STAGE_FFN_BACKWARD)
                  ? off
                  : 0;
    return L;
}

// shape checks common to every entry point (`ffn`: the call runs the expert
// GEMMs; they take any shape the other stages take)
int32_t check_shape(const moe_shape* s, bool ffn) {
    (void)ffn;
    if (s == nullptr) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->S < 0 || s->h <= 0 || s->k > s->E ||
        s->capacity < 0 || (s->overflow != MOE_OVERFLOW_DROP && s->overflow != MOE_OVERFLOW_REASSIGN) ||
        s->quant < MOE_QUANT_TOKEN || s->quant > MOE_QUANT_TOKEN_ABSMAX ||
        (s->quant != MOE_QUANT_TOKEN && s->dispatch != MOE_FP8_E4M3))
        return MOE_ERR_INVALID_ARG;
    if (s->E > kMaxE || s->k > kMaxK || s->S > kMaxS) return MOE_ERR_UNSUPPORTED;
    if (s->act != MOE_F32 && s->act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const bool fp8 = s->dispatch == MOE_FP8_E4M3;
    if (s->dispatch != s->act && !(fp8 && s->act == MOE_BF16)) return MOE_ERR_UNSUPPORTED;
    if (s->act == MOE_F32 && s->d % 4 != 0) return MOE_ERR_UNSUPPORTED;
    if (s->act == MOE_BF16 && s->d % (fp8 ? 16 : 8) != 0) return MOE_ERR_UNSUPPORTED;
    if (s->T * s->k >= (int64_t(1) << 31) || s->T * (s->S + 1) >= (int64_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;
    if (s->d > (1 << 20) || s->h > (1 << 20)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// the fp8-weight path: bf16 activations with fp8 rows quantised per token
// (affine or symmetric), on the persistent expert GEMMs
bool f8w_shape_ok(const moe_shape& s) {
    return s.act == MOE_BF16 && s.dispatch == MOE_FP8_E4M3 &&
           (s.quant == MOE_QUANT_TOKEN || s.quant == MOE_QUANT_TOKEN_ABSMAX) && f8w_supported(s);
}

int32_t check_ptrs(std::initializer_list<const void*> required) {
    for (const void* p : required)
        if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int32_t check_opt(std::initializer_list<const void*> optional) {
    for (const void* p : optional)
        if (p != nullptr && !aligned16(p)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int32_t check_ws(const moe_shape& s, int stage, const void* ws, size_t ws_bytes) {
    const size_t need = layout(s, stage).total;
    if (need == 0) return MOE_OK;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_WORKSPACE;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

#define MOE_TRY(expr)                       \
    do {                                    \
        const int32_t _rc = (expr);         \
        if (_rc != MOE_OK) return _rc;      \
    } while (0)

int32_t forward_impl(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                     const void* w1, const void* w3, const void* w2, void* y, int32_t* topk_idx,
                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                     int32_t* src_token, void* ws, size_t ws_bytes, void* stream,
                     const Marks* mk) {
    MOE_TRY(check_shape(s, true));
    if (s->T == 0) return MOE_OK;  // nothing to do; empty arrays may be null
    MOE_TRY(check_ptrs({x, w_gate, w1, w3, w2, y, topk_idx, topk_w, counts, offsets, dest_row,
                        src_token}));
    MOE_TRY(check_opt({bias}));
    MOE_TRY(check_ws(*s, MOE_STAGE_FORWARD, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FORWARD);
    hipStream_t st = static_cast<hipStream_t>(stream);
    mark(mk);
    MOE_TRY(hip_status(launch_gate_topk(*s, x, w_gate, bias, topk_idx, topk_w, nullptr, st, mk)));
    mark(mk);
    const bool fp8 = s->dispatch == MOE_FP8_E4M3;
    // With bf16 rows on the persistent tiles the permutation is applied where
    // the rows are consumed: dispatch writes only dest_row and src_token, and
    // the up-projection fetches routed row r from x[src_token[r]].
    const bool gather = ffn_gathers_rows(*s);
    void* x_perm = gather ? nullptr : at<void>(ws, L.x_perm);
    float* qp = fp8 ? at<float>(ws, L.qparams) : nullptr;
    // the FFN's tile plan is written by the dispatch permute's first work-groups
    FfnPlanArgs fplan;
    const bool plan_done = ffn_fused_plan(*s, at<int32_t>(ws, L.plan), &fplan);
    MOE_TRY(hip_status(launch_dispatch(*s, x, topk_idx, counts, offsets, dest_row, src_token,
                                       x_perm, qp, at<int32_t>(ws, L.rank),
                                       at<int32_t>(ws, L.blk), at<int32_t>(ws, L.pre),
                                       at<int32_t>(ws, L.loads), at<uint32_t>(ws, L.qstats),
                                       at<uint32_t>(ws, 0), fplan, st, mk)));
    void* y_perm = at<void>(ws, L.y_perm);
    void* y_sh = s->S > 0 ? at<void>(ws, L.y_sh) : nullptr;
    MOE_TRY(hip_status(launch_grouped_ffn(*s, x_perm, qp, offsets, x, w1, w3, w2, y_perm, y_sh,
                                          at<int32_t>(ws, L.plan), at<void>(ws, L.h_r),
                                          at<void>(ws, L.h_s), plan_done, st, mk,
                                          gather ? src_token : nullptr)));
    MOE_TRY(hip_status(launch_combine(*s, y_perm, y_sh, dest_row, topk_w, y, st)));
    mark(mk);
    return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (found with hipGetSymbolAddress on
// the first call on that device, with the device current).
int32_t scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

int32_t forward_fp8w_impl(const moe_shape* s, const void* x, const void* w_gate,
                          const float* bias, const uint8_t* w1q, const uint8_t* w3q,
                          const uint8_t* w2q, const float* wscale, void* y, int32_t* topk_idx,
                          float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                          int32_t* src_token, void* ws, size_t ws_bytes, void* stream,
                          const Marks* mk) {
    MOE_TRY(check_shape(s, true));
    if (!f8w_shape_ok(*s)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, w_gate, w1q, w3q, w2q, wscale, y, topk_idx, topk_w, counts, offsets,
                        dest_row, src_token}));
    MOE_TRY(check_opt({bias}));
    MOE_TRY(check_ws(*s, MOE_STAGE_FORWARD_FP8W, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FORWARD_FP8W);
    hipStream_t st = static_cast<hipStream_t>(stream);
    mark(mk);
    MOE_TRY(hip_status(launch_gate_topk(*s, x, w_gate, bias, topk_idx, topk_w, nullptr, st, mk)));
    mark(mk);
    void* x_perm = at<void>(ws, L.x_perm);
    float* qp = at<float>(ws, L.qparams);
    uint8_t* x8 = s->S > 0 ? at<uint8_t>(ws, L.x8) : nullptr;
    float* q8 = s->S > 0 ? at<float>(ws, L.q8) : nullptr;
    FfnPlanArgs fplan;
    const bool plan_done = ffn_fused_plan(*s, at<int32_t>(ws, L.plan), &fplan);
    MOE_TRY(hip_status(launch_dispatch(*s, x, topk_idx, counts, offsets, dest_row, src_token,
                                       x_perm, qp, at<int32_t>(ws, L.rank), at<int32_t>(ws, L.blk),
                                       at<int32_t>(ws, L.pre), at<int32_t>(ws, L.loads),
                                       at<uint32_t>(ws, L.qstats), at<uint32_t>(ws, 0), fplan, st,
                                       mk, x8, q8)));
    void* y_perm = at<void>(ws, L.y_perm);
    void* y_sh = s->S > 0 ? at<void>(ws, L.y_sh) : nullptr;
    MOE_TRY(hip_status(launch_grouped_ffn_f8w(
        *s, x_perm, qp, offsets, x8, q8, w1q, w3q, w2q, wscale, y_perm, y_sh,
        at<int32_t>(ws, L.plan), at<void>(ws, L.h_r), at<void>(ws, L.h_s),
        at<uint8_t>(ws, L.h8_r), at<uint8_t>(ws, L.h8_s), at<float>(ws, L.hsc_r),
        s->S > 0 ? at<float>(ws, L.hsc_s) : nullptr, plan_done, st, mk)));
    MOE_TRY(hip_status(launch_combine(*s, y_perm, y_sh, dest_row, topk_w, y, st)));
    mark(mk);
    return MOE_OK;
}

const char* const kKernelNames[] = {"gate_topk",  "dispatch_rank", "dispatch_scan",
                                    "dispatch_permute", "ffn_plan", "ffn_up",
                                    "ffn_down",   "combine"};

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s, int32_t stage) {
    if (stage < MOE_STAGE_GATE || stage > MOE_STAGE_FORWARD_FP8W) return 0;
    if (stage == MOE_STAGE_FORWARD_FP8W && (check_shape(s, true) != MOE_OK || !f8w_shape_ok(*s)))
        return 0;
    const bool ffn = stage == MOE_STAGE_FFN || stage == MOE_STAGE_FORWARD;
    if (check_shape(s, ffn) != MOE_OK) return 0;
    return layout(*s, stage).total;
}

int32_t moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (ws == nullptr || ws_bytes < kHeaderBytes || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return MOE_ERR_WORKSPACE;
    clear_header_kernel<<<1, kHeaderBytes / 4, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<uint32_t*>(ws));
    return hip_status(hipGetLastError());
}

const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null, misaligned or inconsistent)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_BAD_INDEX: return "bad or repeated expert id in topk_idx";
        default: return "unknown status";
    }
}

int32_t moe_gate_topk(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                      int32_t* topk_idx, float* topk_w, float* logits_dbg, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, w_gate, topk_idx, topk_w}));
    MOE_TRY(check_opt({bias, logits_dbg}));
    return hip_status(launch_gate_topk(*s, x, w_gate, bias, topk_idx, topk_w, logits_dbg,
                                       static_cast<hipStream_t>(stream), nullptr));
}

int32_t moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* dest_row, int32_t* src_token, void* x_perm,
                     float* qparams, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, topk_idx, counts, offsets, dest_row, src_token, x_perm}));
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({qparams}));
    MOE_TRY(check_ws(*s, MOE_STAGE_DISPATCH, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_DISPATCH);
    return hip_status(launch_dispatch(*s, x, topk_idx, counts, offsets, dest_row, src_token,
                                      x_perm, qparams, at<int32_t>(ws, L.rank),
                                      at<int32_t>(ws, L.blk), at<int32_t>(ws, L.pre),
                                      at<int32_t>(ws, L.loads), at<uint32_t>(ws, L.qstats),
                                      at<uint32_t>(ws, 0), FfnPlanArgs{nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0},
                                      static_cast<hipStream_t>(stream),
                                      nullptr));
}

int32_t moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* topk_idx,
                             int32_t* counts, int32_t* offsets, int32_t* dest_row,
                             int32_t* src_token, void* x_perm, float* qparams, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, topk_idx, counts, offsets, dest_row, src_token, x_perm}));
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({qparams}));
    if (layout(*s, MOE_STAGE_DISPATCH).total > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
    void* ws = nullptr;
    MOE_TRY(scratch_address(&ws));
    const Layout L = layout(*s, MOE_STAGE_DISPATCH);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the error flag left by an earlier call starts at zero again (a kernel,
    // not a memset, so that the call can be captured in a graph)
    clear_header_kernel<<<1, kHeaderBytes / 4, 0, st>>>(static_cast<uint32_t*>(ws));
    MOE_TRY(hip_status(hipGetLastError()));
    return hip_status(launch_dispatch(*s, x, topk_idx, counts, offsets, dest_row, src_token,
                                      x_perm, qparams, at<int32_t>(ws, L.rank),
                                      at<int32_t>(ws, L.blk), at<int32_t>(ws, L.pre),
                                      at<int32_t>(ws, L.loads), at<uint32_t>(ws, L.qstats),
                                      at<uint32_t>(ws, 0),
                                      FfnPlanArgs{nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0}, st,
                                      nullptr));
}

int32_t moe_grouped_ffn(const moe_shape* s, const void* x_perm, const float* qparams,
                        const int32_t* offsets, const void* x, const void* w1, const void* w3,
                        const void* w2, void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                        void* stream) {
    MOE_TRY(check_shape(s, true));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x_perm, offsets, w1, w3, w2, y_perm}));
    if (s->S > 0) MOE_TRY(check_ptrs({x, y_shared}));
    else if (y_shared != nullptr) return MOE_ERR_INVALID_ARG;
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({x, qparams}));
    MOE_TRY(check_ws(*s, MOE_STAGE_FFN, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FFN);
    return hip_status(launch_grouped_ffn(*s, x_perm, qparams, offsets, x, w1, w3, w2, y_perm,
                                         y_shared, at<int32_t>(ws, L.plan), at<void>(ws, L.h_r),
                                         at<void>(ws, L.h_s), false, static_cast<hipStream_t>(stream),
                                         nullptr));
}

int32_t moe_combine(const moe_shape* s, const void* y_perm, const void* y_shared,
                    const int32_t* dest_row, const float* topk_w, void* y, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({y_perm, dest_row, topk_w, y}));
    MOE_TRY(check_opt({y_shared}));
    return hip_status(launch_combine(*s, y_perm, y_shared, dest_row, topk_w, y,
                                     static_cast<hipStream_t>(stream)));
}

int32_t moe_combine_backward(const moe_shape* s, const void* dy, const void* y_perm,
                             const int32_t* dest_row, const float* topk_w, void* dy_perm,
                             float* dtopk_w, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({dy, y_perm, dest_row, topk_w, dy_perm, dtopk_w}));
    return hip_status(launch_combine_backward(*s, dy, y_perm, dest_row, topk_w, dy_perm, dtopk_w,
                                              static_cast<hipStream_t>(stream)));
}

int32_t moe_dispatch_backward(const moe_shape* s, const void* dx_perm, const void* dx_shared,
                              const int32_t* dest_row, void* dx, void* stream) {
    MOE_TRY(check_shape(s, false));
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({dx_perm, dest_row, dx}));
    MOE_TRY(check_opt({dx_shared}));
    // the transpose of copying each row to its k places: combine with unit weights
    return hip_status(launch_combine(*s, dx_perm, dx_shared, dest_row, nullptr, dx,
                                     static_cast<hipStream_t>(stream)));
}

int32_t moe_gate_backward(const moe_shape* s, const void* x, const void* w_gate,
                          const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                          float* dlogits_topk, void* dx, float* dw_gate, void* ws,
                          size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s, false));
    MOE_TRY(check_ptrs({dw_gate}));
    MOE_TRY(check_ws(*s, MOE_STAGE_GATE_BACKWARD, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_GATE_BACKWARD);
    if (s->T > 0) {
        MOE_TRY(check_ptrs({x, w_gate, topk_idx, topk_w, dtopk_w, dlogits_topk}));
        MOE_TRY(check_opt({dx}));
    }
    return hip_status(launch_gate_backward(*s, x, w_gate, topk_idx, topk_w, dtopk_w, dlogits_topk,
                                           s->T > 0 ? dx : nullptr, dw_gate, at<float>(ws, L.part),
                                           static_cast<hipStream_t>(stream)));
}

int32_t moe_grouped_ffn_backward(const moe_shape* s, const void* x_perm, const float* qparams,
                                 const int32_t* offsets, const void* x, const void* w1,
                                 const void* w3, const void* w2, const void* dy_perm,
                                 const void* dy_shared, void* dx_perm, void* dx_shared, float* dw1,
                                 float* dw3, float* dw2, void* ws, size_t ws_bytes,
                                 void* stream) {
    MOE_TRY(check_shape(s, true));
    if (s->act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_ptrs({w1, w3, w2, dw1, dw3, dw2}));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s->T == 0) {
        // no rows: every weight gradient is zero
        const int64_t n13 = static_cast<int64_t>(s->E + s->S) * s->h * s->d;
        for (float* p : {dw1, dw3, dw2}) zero_f32_kernel<<<1024, 256, 0, st>>>(p, n13);
        return hip_status(hipGetLastError());
    }
    MOE_TRY(check_ptrs({x_perm, offsets, dy_perm, dx_perm}));
    if (s->S > 0) MOE_TRY(check_ptrs({x, dy_shared, dx_shared}));
    else if (dx_shared != nullptr || dy_shared != nullptr) return MOE_ERR_INVALID_ARG;
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({x, qparams}));
    MOE_TRY(check_ws(*s, MOE_STAGE_FFN_BACKWARD, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FFN_BACKWARD);
    return hip_status(launch_ffn_backward(*s, x_perm, qparams, offsets, x, w1, w3, w2, dy_perm,
                                          dy_shared, dx_perm, dx_shared, dw1, dw3, dw2,
                                          at<void>(ws, L.fbwd), st, nullptr));
}

size_t moe_ffn_saved_bytes(const moe_shape* s) {
    if (check_shape(s, true) != MOE_OK || s->act != MOE_BF16 || !use_big_tiles(*s)) return 0;
    return saved_layout(*s).bytes;
}

int32_t moe_grouped_ffn_save(const moe_shape* s, const void* x_perm, const float* qparams,
                             const int32_t* offsets, const void* x, const void* w1, const void* w3,
                             const void* w2, void* y_perm, void* y_shared, void* saved,
                             size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s, true));
    if (s->act != MOE_BF16 || !use_big_tiles(*s)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x_perm, offsets, w1, w3, w2, y_perm, saved}));
    if (s->S > 0) MOE_TRY(check_ptrs({x, y_shared}));
    else if (y_shared != nullptr) return MOE_ERR_INVALID_ARG;
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({x, qparams}));
    const SavedLayout SL = saved_layout(*s);
    if ((reinterpret_cast<uintptr_t>(saved) & 255u) != 0 || saved_bytes < SL.bytes)
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_ws(*s, MOE_STAGE_FFN, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FFN);
    uint8_t* sv = static_cast<uint8_t*>(saved);
    return hip_status(launch_grouped_ffn(*s, x_perm, qparams, offsets, x, w1, w3, w2, y_perm,
                                         y_shared, at<int32_t>(ws, L.plan), sv + SL.h_r,
                                         s->S > 0 ? sv + SL.h_s : nullptr, false,
                                         static_cast<hipStream_t>(stream), nullptr, nullptr,
                                         sv + SL.a_r, sv + SL.b_r, s->S > 0 ? sv + SL.a_s : nullptr,
                                         s->S > 0 ? sv + SL.b_s : nullptr));
}

int32_t moe_grouped_ffn_backward_saved(const moe_shape* s, const void* x_perm,
                                       const float* qparams, const int32_t* offsets,
                                       const void* x, const void* w1, const void* w3,
                                       const void* w2, const void* saved, size_t saved_bytes,
                                       const void* dy_perm, const void* dy_shared, void* dx_perm,
                                       void* dx_shared, float* dw1, float* dw3, float* dw2,
                                       void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s, true));
    if (s->act != MOE_BF16 || !use_big_tiles(*s)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0)
        return moe_grouped_ffn_backward(s, x_perm, qparams, offsets, x, w1, w3, w2, dy_perm,
                                        dy_shared, dx_perm, dx_shared, dw1, dw3, dw2, ws, ws_bytes,
                                        stream);
    MOE_TRY(check_ptrs({saved}));
    if ((reinterpret_cast<uintptr_t>(saved) & 255u) != 0 || saved_bytes < saved_layout(*s).bytes)
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_ptrs({w1, w3, w2, dw1, dw3, dw2, x_perm, offsets, dy_perm, dx_perm}));
    if (s->S > 0) MOE_TRY(check_ptrs({x, dy_shared, dx_shared}));
    else if (dx_shared != nullptr || dy_shared != nullptr) return MOE_ERR_INVALID_ARG;
    if (s->dispatch == MOE_FP8_E4M3) MOE_TRY(check_ptrs({qparams}));
    MOE_TRY(check_opt({x, qparams}));
    MOE_TRY(check_ws(*s, MOE_STAGE_FFN_BACKWARD, ws, ws_bytes));
    const Layout L = layout(*s, MOE_STAGE_FFN_BACKWARD);
    return hip_status(launch_ffn_backward(*s, x_perm, qparams, offsets, x, w1, w3, w2, dy_perm,
                                          dy_shared, dx_perm, dx_shared, dw1, dw3, dw2,
                                          at<void>(ws, L.fbwd), static_cast<hipStream_t>(stream),
                                          nullptr, saved));
}

size_t moe_fp8_weight_scale_floats(const moe_shape* s) {
    if (check_shape(s, true) != MOE_OK) return 0;
    return fp8w_scale_floats(*s);
}

int32_t moe_quantize_weights(const moe_shape* s, const void* w1, const void* w3, const void* w2,
                             uint8_t* w1q, uint8_t* w3q, uint8_t* w2q, float* wscale,
                             void* stream) {
    MOE_TRY(check_shape(s, true));
    if (s->act != MOE_BF16 || s->d % 8 != 0 || s->h % 8 != 0) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_ptrs({w1, w3, w2, w1q, w3q, w2q, wscale}));
    return hip_status(launch_quantize_weights(*s, w1, w3, w2, w1q, w3q, w2q, wscale,
                                              static_cast<hipStream_t>(stream)));
}

int32_t moe_forward_fp8w(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                         const uint8_t* w1q, const uint8_t* w3q, const uint8_t* w2q,
                         const float* wscale, void* y, int32_t* topk_idx, float* topk_w,
                         int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token,
                         void* ws, size_t ws_bytes, void* stream, void* const* events,
                         int32_t n_events) {
    if (events != nullptr && n_events < kFp8wKernels + 1) return MOE_ERR_INVALID_ARG;
    Marks mk{reinterpret_cast<hipEvent_t const*>(events), n_events, 0,
             static_cast<hipStream_t>(stream)};
    return forward_fp8w_impl(s, x, w_gate, bias, w1q, w3q, w2q, wscale, y, topk_idx, topk_w,
                             counts, offsets, dest_row, src_token, ws, ws_bytes, stream,
                             events != nullptr ? &mk : nullptr);
}

int32_t moe_forward(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                    const void* w1, const void* w3, const void* w2, void* y, int32_t* topk_idx,
                    float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                    int32_t* src_token, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(s, x, w_gate, bias, w1, w3, w2, y, topk_idx, topk_w, counts, offsets,
                        dest_row, src_token, ws, ws_bytes, stream, nullptr);
}

int32_t moe_forward_traced(const moe_shape* s, const void* x, const void* w_gate,
                           const float* bias, const void* w1, const void* w3, const void* w2,
                           void* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* dest_row, int32_t* src_token, void* ws,
                           size_t ws_bytes, void* stream, void* const* events, int32_t n_events) {
    if (events == nullptr || n_events < moe_forward_kernel_count(s) + 1) return MOE_ERR_INVALID_ARG;
    Marks mk{reinterpret_cast<hipEvent_t const*>(events), n_events, 0,
             static_cast<hipStream_t>(stream)};
    return forward_impl(s, x, w_gate, bias, w1, w3, w2, y, topk_idx, topk_w, counts, offsets,
                        dest_row, src_token, ws, ws_bytes, stream, &mk);
}

int32_t moe_forward_kernel_count(const moe_shape* s) {
    (void)s;
    return static_cast<int32_t>(sizeof(kKernelNames) / sizeof(kKernelNames[0]));
}

const char* moe_forward_kernel_name(const moe_shape* s, int32_t i) {
    if (i < 0 || i >= moe_forward_kernel_count(s)) return nullptr;
    if (i == 0 && s != nullptr && s->T > 0 && gate_two_phase_chosen(*s)) return "gate_two_phase";
    if (i == 3 && s != nullptr && s->dispatch == MOE_FP8_E4M3) return "dispatch_permute_fp8";
    if (i == 3 && s != nullptr && s->T > 0 && ffn_gathers_rows(*s)) return "dispatch_map";
    return kKernelNames[i];
}

int32_t moe_get_device_error(void* ws, size_t ws_bytes, void* stream) {
    if (ws == nullptr || ws_bytes < kHeaderBytes || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return MOE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t flag = 0;
    if (hipMemcpyAsync(&flag, ws, sizeof flag, hipMemcpyDeviceToHost, st) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
    clear_header_kernel<<<1, 1, 0, st>>>(static_cast<uint32_t*>(ws));
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    return flag != 0 ? MOE_ERR_BAD_INDEX : MOE_OK;
}

}  // extern "C"
