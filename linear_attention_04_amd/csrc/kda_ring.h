// kda_ring.h -- device helpers shared by the recurrent kernels (forward and reverse):
// the state-decay broadcast of gamma, counter waits, buffer descriptors and the
// workgroup barrier that publishes a ring slot.
#pragma once

#include "kda_device.h"

namespace kda {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int M, int I>
__device__ __forceinline__ float gamma_of(const float2 gam) {
    // element e = 4M + I of this lane group's permuted gamma sits in lane e >> 1, slot e & 1
    return row_bcast<((4 * M + I) >> 1)>((I & 1) ? gam.y : gam.x);
}

template <int M>
__device__ __forceinline__ void decay_tile(f32x4 &s, const float2 gam) {
    s[0] *= gamma_of<M, 0>(gam);
    s[1] *= gamma_of<M, 1>(gam);
    s[2] *= gamma_of<M, 2>(gam);
    s[3] *= gamma_of<M, 3>(gam);
}

// s_waitcnt vmcnt(N) without waiting on the LDS / export counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this (producer) wave's loads for one chunk have landed: at most
// `later` chunks' loads, issued after that chunk's, may stay outstanding. Vector
// memory loads complete in issue order and producers issue nothing else, so the
// count is exact. `later` is wave-uniform and in [0, DEPTH - 2].
template <int PER_WAVE, int DEPTH>
__device__ __forceinline__ void wait_for_chunk(int later) {
    static_assert(DEPTH >= 2 && DEPTH <= 8, "extend the switch");
    switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<(DEPTH > 2 ? 1 : 0) * PER_WAVE>(); break;
    case 2: wait_vmcnt<(DEPTH > 3 ? 2 : 0) * PER_WAVE>(); break;
    case 3: wait_vmcnt<(DEPTH > 4 ? 3 : 0) * PER_WAVE>(); break;
    case 4: wait_vmcnt<(DEPTH > 5 ? 4 : 0) * PER_WAVE>(); break;
    case 5: wait_vmcnt<(DEPTH > 6 ? 5 : 0) * PER_WAVE>(); break;
    default: wait_vmcnt<(DEPTH > 7 ? 6 : 0) * PER_WAVE>(); break;
    }
}

// Buffer descriptor over `bytes` bytes at `base` (wave-uniform). Buffer accesses
// are range-checked by the hardware: loads past the end return zero and stores
// past the end are dropped, which is how rows past a short chunk are handled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14)); }

__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");  // no LDS or global access moves across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace kda
