// Device helpers of the bf16 MFMA Newton–Schulz kernels (gfx950): LDS
// transposing reads, direct-to-LDS buffer loads, buffer resources, the
// compile-time block masks of diagonal and edge tiles, and a compile-time
// loop.
#pragma once

#include <type_traits>

#include "kernel_common.hpp"

namespace muon {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ bf16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(LDS_AS char*)p);
}

// 16 bytes per lane, global -> LDS: lane i lands at lds + 16 i (lds is
// wave-uniform, passed in M0). Issued as inline assembly so that the compiler
// does not track these LDS writes: it would otherwise wait for every load in
// flight (vmcnt(0)) before LDS reads it cannot prove disjoint, which undoes
// the ring; the kernel orders the ring itself with explicit vmcnt waits and
// barriers, and every such load has completed before any compiler-managed
// vector memory wait (the epilogue) is reached.
// M0: the asm sets it itself, in the same block, right before the load. The
// compiler reserves M0 and does not honour a clobber of it, so what makes
// this safe is that the kernels built on this helper hold no M0 value of the
// compiler's own: their gfx950 assembly has no instruction that reads or
// writes M0 besides these pairs (a host test compiles them and checks that).
__device__ __forceinline__ void dma16(u32x4 r, char* lds, int voff, int soff) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)lds);
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "s"(m0v));
}

// Buffer resource of `bytes` bytes at `base` (stride 0, raw buffer): word 0
// and the low half of word 1 hold the address, word 2 the byte range that
// the hardware bounds-checks, word 3 the format word. Built from wave-uniform
// words (readfirstlane) so that it stays in scalar registers.
__device__ __forceinline__ u32x4 rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// The 32 x 32 blocks a wave computes on a diagonal tile (on or above the
// diagonal), as a bit mask over f = fi * 2 + fj: the wave (wi, wj) of a
// 2 x WN grid owns row blocks wi FRI + fi and column blocks wj, 2 WN - 1 - wj.
constexpr unsigned diag_mask(int wi, int wj, int WN, int FRI) {
    unsigned m = 0;
    for (int fi = 0; fi < FRI; ++fi)
        for (int fj = 0; fj < 2; ++fj) {
            const int c = fj == 0 ? wj : 2 * WN - 1 - wj;
            if (c >= wi * FRI + fi) m |= 1u << (fi * 2 + fj);
        }
    return m;
}
// The blocks of a wave on an edge tile: row blocks fi < RV, column block
// fj = 0 if CM >= 1 and fj = 1 if CM == 2 (same bit order as diag_mask).
constexpr unsigned edge_mask(int RV, int CM, int FRI) {
    unsigned m = 0;
    for (int fi = 0; fi < RV && fi < FRI; ++fi)
        for (int fj = 0; fj < 2; ++fj)
            if (CM > fj) m |= 1u << (fi * 2 + fj);
    return m;
}
constexpr int bit_count(unsigned m) { return m ? (int)(m & 1u) + bit_count(m >> 1) : 0; }
// the position of the k-th set bit of m
constexpr int nth_bit(unsigned m, int k) {
    for (int b = 0; b < 32; ++b)
        if ((m >> b) & 1u) {
            if (k == 0) return b;
            --k;
        }
    return -1;
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// s_waitcnt vmcnt(0), leaving the LDS / scalar counters alone
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace muon
