// moe_device.h -- device helpers shared by libmoe's kernels: vector types,
// lane reductions, wave-uniform values, explicit waits and barriers, and the
// device-coherent accesses that hand data between blocks of one launch.
// gfx950 (CDNA4) only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum over each aligned group of 8 lanes; every lane of the group ends with
// the group sum.  quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror.
__device__ __forceinline__ float sum8_lanes(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A pointer every lane of the wave holds, made explicitly uniform (SGPRs).
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Non-temporal load of a T from global memory, emitted as a global (not a
// flat) instruction even where the compiler cannot trace p back to a kernel
// argument (e.g. a pointer made uniform through inline asm).  A flat load
// also counts against the LDS wait counter, so every wait for an LDS read
// would then wait for all the weight loads in flight as well.
template <class T>
__device__ __forceinline__ T load_nt_global(const void *p)
{
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) T *)p);
}

// Ordinary (cached) load of a T from global memory, emitted as a global
// instruction for the same reason.
template <class T>
__device__ __forceinline__ T load_global(const void *p)
{
    return *(const __attribute__((address_space(1))) T *)p;
}

// Wait until at most N of this wave's vector memory loads are in flight
// (vmcnt(N); expcnt and lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm0() { wait_vm<0>(); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt 0) but not for its global loads, which __syncthreads would drain.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0); vmcnt and expcnt not waited
    asm volatile("s_barrier" ::: "memory");
}

// Device-coherent relaxed accesses (device-scope atomics): a store writes
// through to memory and a load reads past this XCD's L2, so data handed
// between blocks of one launch needs no whole-cache write-back or
// invalidation.  The writer waits for its stores (wait_vm0) before it
// publishes; the reader loads only after it has seen the publication.
__device__ __forceinline__ void store_dev(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
