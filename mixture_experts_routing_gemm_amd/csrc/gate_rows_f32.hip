// Row-broadcast gate kernels for float32 inputs (the kernel and its shapes are
// in gate_common.h; one translation unit per input type keeps builds short).
#include "gate_common.h"

namespace moe {

bool launch_gate_rows_f32(const moe_shape& s, const void* x, const void* wg, const float* bias,
                          int32_t* idx, float* w, float* dbg, hipStream_t st) {
    return launch_rb_t<float>(s, x, wg, bias, idx, w, dbg, st);
}

}  // namespace moe
