// Helpers of the kernels that stream operands global -> LDS through a ring of
// slots with direct buffer-to-LDS loads (the persistent expert GEMMs and the
// expert weight gradients).
#pragma once

#include "moe_device.h"

namespace moe {

// fourth word of a raw buffer resource on gfx950 (untyped, no swizzle)
constexpr int kBufferFlags = 0x00020000;

// Work-group barrier without the release/acquire fences of __syncthreads():
// those would drain every outstanding load, including the prefetched slices.
// The counted vmcnt wait before it orders the slice about to be read; the
// empty asm keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding): at most n vector-memory
// instructions of this wave outstanding, and its LDS reads complete -- the
// latter so that no ring slot can be refilled while a read of it is in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// a wave-uniform pointer (lets the compiler keep it in SGPRs)
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One 16-byte-per-lane request through a raw buffer resource over
// [base, base + bytes): lane i reads base + voff_i + soff (zero when past the
// end) and writes it to LDS at lds + OFF + 16*i. (The instruction's immediate
// offset would move the source address as well, so the LDS offset goes into
// the LDS base instead.) AUX is the cache policy: 0, or 2 for non-temporal.
template <int OFF, int AUX = 0>
__device__ __forceinline__ void buffer_to_lds16(const uint8_t* base, uint32_t bytes, uint32_t voff,
                                                uint32_t soff, uint8_t* lds) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, static_cast<int>(bytes), kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + OFF), 16, voff,
                                             soff, 0, AUX);
}

}  // namespace moe
