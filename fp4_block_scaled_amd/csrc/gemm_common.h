// gemm_common.h -- pieces shared by the grouped-GEMM tiers (FP8 activations
// with E4M3 banks, bf16 activations with NVFP4 banks): the XCD-aware mapping
// of blocks to (row tile, column block) work items, the LDS swizzle, and the
// global-to-LDS DMA with its explicit waits.  Both tiers take their row tiles
// from gemm_tiles_kernel (128 expert-sorted rows each).
#pragma once

#include "moe_internal.h"

namespace {

// Block -> (tile, column block).  The hardware hands blocks to the 8 XCDs
// round-robin (block b to XCD b % 8), each XCD with its own L2: give every
// XCD one contiguous run of the W = tiles x column-blocks work items, so the
// blocks running together on an XCD share A rows in its L2.  Within an
// expert the items go column-block-major: its tiles read each weight block
// at about the same time.  False for blocks past W.
template <class Args>
__device__ __forceinline__ bool gemm_item(const Args &a, int4 &tile, int &nb)
{
    const int W = moe::uniform(*a.ntiles) * a.ntn;
    const int b = blockIdx.x;
    if (b >= W) return false;
    const int q = W >> 3, r = W & 7, x = b & 7;
    const int L = x * q + min(x, r) + (b >> 3);
    const int4 head = a.tiles[L / a.ntn];
    const int f = moe::uniform(head.z), n = moe::uniform(head.w);
    const int local = L - f * a.ntn;
    nb = local / n;
    const int4 tl = a.tiles[f + local % n];
    tile = make_int4(moe::uniform(tl.x), moe::uniform(tl.y), f, n);
    return true;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lane_f(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Physical 16-byte chunk of logical chunk `chunk` in tile row `row`.  An
// operand read has 16 consecutive rows read the same logical chunk; with
// f(row) = (row & 7) ^ ((row >> 3) & 1) any 8 consecutive rows land on 8
// distinct chunks of a 128-byte bank line, and the 8 rows of one parity among
// 16 consecutive rows on 8 distinct chunks, so those reads are conflict-free
// whether the LDS serves 128 or 256 bytes per clock.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }

// LDS DMA: lane i of the wave reads `size` bytes at base + off_i (base
// wave-uniform, off_i a 32-bit byte offset) and the hardware writes them to
// LDS at M0 + i * size (M0 = the wave-uniform LDS byte address of the run).  Written as inline asm so the compiler does
// not track these loads: it would otherwise place a full vmcnt(0) before the
// first LDS read of each loop trip.  The waits for them are the explicit
// vmcnt waits below; the compiler's own waits for its own loads only get more
// conservative, since vector memory loads retire in order.  One wait state
// separates the M0 write from the DMA.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(size_t)(const lds_void *)p;
}

__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void dma4(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" :: "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// s_waitcnt with only vmcnt = N (expcnt and lgkmcnt left alone), and lgkmcnt(0)
#define MOE_WAIT_VM(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | (7 << 4) | (15 << 8) | ((((N) >> 4) & 3) << 14)))
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)
#define MOE_BARRIER() asm volatile("s_barrier" ::: "memory")

// vmcnt wait that leaves min(n, N) stages of PER DMA instructions in flight
template <int PER, int N>
__device__ __forceinline__ void wait_stages(int n)
{
    if constexpr (N == 0) {
        MOE_WAIT_VM(0);
    } else {
        if (n >= N) MOE_WAIT_VM(N * PER);
        else wait_stages<PER, N - 1>(n);
    }
}

// Ring of NST LDS stages: K step kb lives in stage kb % NST.  The DMA for
// step kb + NST - 1 goes out once every wave has passed the barrier of step
// kb, i.e. is done reading stage (kb - 1) % NST; before that barrier each
// wave waits until its own share of stage kb has landed, leaving the later
// stages in flight.
template <int NST, int PER, class Issue, class Compute>
__device__ __forceinline__ void k_loop(int KB, uint8_t *sm, int stage_bytes, const Issue &issue,
                                       const Compute &compute)
{
    MOE_WAIT_VM(0);    // retire the set-up loads before the DMA starts
#pragma unroll
    for (int j = 0; j < NST - 1; ++j)
        if (j < KB) issue(j, sm + j * stage_bytes);
    int cs = 0, is = NST - 1;
    for (int kb = 0; kb < KB; ++kb) {
        wait_stages<PER, NST - 2>(KB - 1 - kb);
        MOE_WAIT_LGKM0();
        MOE_BARRIER();
        if (kb + NST - 1 < KB) issue(kb + NST - 1, sm + is * stage_bytes);
        compute(sm + cs * stage_bytes, kb);
        cs = cs + 1 == NST ? 0 : cs + 1;
        is = is + 1 == NST ? 0 : is + 1;
    }
    MOE_WAIT_VM(0);
}

}  // namespace
