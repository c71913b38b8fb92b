// Row-broadcast gate kernels for bf16 inputs (the kernel and its shapes are
// in gate_common.h; one translation unit per input type keeps builds short).
#include "gate_common.h"

namespace moe {

bool launch_gate_rows_bf16(const moe_shape& s, const void* x, const void* wg, const float* bias,
                          int32_t* idx, float* w, float* dbg, hipStream_t st) {
    return launch_rb_t<bf16_t>(s, x, wg, bias, idx, w, dbg, st);
}

}  // namespace moe
