// Building blocks shared by the 16-bit forward kernels (gfx950): matrix-core
// fragment shapes, tile geometry, LDS swizzles, HBM->LDS tile copies and the
// transposed V read.  Internal header.
#pragma once

#include <utility>

#include "fa_common.h"

namespace fa {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// 16-bit element types of the kernels: bf16 (the default) and fp16, with
// their 8- and 4-wide vectors and the 32x32x16 matrix-core product
// (fp32 accumulation) on them.
template <class T>
struct Elem;
template <>
struct Elem<__bf16> {
    using x8 = bf16x8_t;
    using x4 = bf16x4_t;
    __device__ static f32x16_t mfma(x8 a, x8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elem<_Float16> {
    using x8 = f16x8_t;
    using x4 = f16x4_t;
    __device__ static f32x16_t mfma(x8 a, x8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// ----------------------------------------------------------------------------
// Matrix-core fragment shapes.

template <int MF>
struct Frag;

// 32x32 output tile, K = 16 per instruction.  Accumulator register i of
// lane l holds row 8*(i/4) + 4*(l/32) + i%4, column l%32.
template <>
struct Frag<32> {
    using acc_t = f32x16_t;
    static constexpr int ACC = 16;
    static constexpr int KQK = 16;  // head-dim depth per QK instruction
    __device__ static acc_t qk(bf16x8_t a, bf16x8_t b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) {
        return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    }
};

// 16x16 output tile, K = 32 per QK instruction and K = 16 per PV
// instruction.  Accumulator register i of lane l holds row 4*(l/16) + i,
// column l%16.
template <>
struct Frag<16> {
    using acc_t = f32x4_t;
    static constexpr int ACC = 4;
    static constexpr int KQK = 32;
    __device__ static acc_t qk(bf16x8_t a, bf16x8_t b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 4 * (lane >> 4) + i; }
};

template <int D, int BC, int MF, int NW>
struct Cfg {
    static constexpr int NT = NW * 64;
    static constexpr int BR = MF * NW;
    static constexpr int NKB = BC / MF;            // score blocks per tile
    static constexpr int ND = D / MF;              // output blocks
    static constexpr int NQK = D / Frag<MF>::KQK;  // Q fragments
    static constexpr int SLOTS = D / 8;            // 16-byte slots per row
    static constexpr int RPL = 128 / D;            // rows per 256-byte LDS bank line
    static constexpr int TILE = BC * D;            // bf16 per K (or V) tile
    static constexpr int NCOPY = TILE / 512;       // 1 KiB copy instructions per tile
    static_assert(BC % MF == 0 && D % MF == 0, "tile must be a multiple of MF");
    static_assert(BC % 16 == 0 && 128 % BC == 0, "BC must divide the 128 mask block");
    static_assert(128 % BR == 0 || BR % 128 == 0, "BR and the mask block must nest");
    static_assert(TILE % 512 == 0, "tile must be a whole number of 1 KiB copies");

    // Slot swizzle of K rows: the 16 rows read by one 16-lane group of a
    // 16-byte read land in 16 distinct bank groups.
    __device__ static int zk(int r) { return (r / RPL) % SLOTS; }
    // Slot swizzle of V rows: the rows touched by one transposed read of a
    // half-wave (4 rows x 4 slots for MF=32, 8 rows x 2 slots for MF=16)
    // land in distinct bank groups.
    __device__ static int zv(int r) {
        if constexpr (MF == 32)
            return 4 * ((r / RPL) % (D / 32));
        else
            return 2 * ((r / RPL) % (D / 16));
    }
};

// Issue the copies of key tile rows [kbase, kbase+BC) of K and V into LDS.
// Copy instruction q moves LDS chunks [64q, 64q+64) of the tile; chunk ci is
// row ci/SLOTS, physical slot ci%SLOTS, which holds logical slot
// (phys ^ swizzle(row)).  Rows past the last valid key are clamped to it:
// those keys are masked, and the clamp keeps the data finite.
template <class C, int D>
__device__ __forceinline__ void copy_tile(const __bf16 *K, const __bf16 *V, __bf16 *Ks,
                                          __bf16 *Vs, int kbase, int klast, int wave,
                                          int lane) {
    constexpr int ROUNDS = (C::NCOPY + C::NT / 64 - 1) / (C::NT / 64);
#pragma unroll ROUNDS <= 8 ? ROUNDS : 2
    for (int q0 = 0; q0 < C::NCOPY; q0 += C::NT / 64) {
        const int q = q0 + wave;
        if (C::NCOPY % (C::NT / 64) != 0 && q >= C::NCOPY) break;
        const int ci = q * 64 + lane;
        const int r = ci / C::SLOTS, p = ci % C::SLOTS;
        const int64_t key = min(kbase + r, klast);
        const __bf16 *gk = K + key * D + ((p ^ C::zk(r)) << 3);
        const __bf16 *gv = V + key * D + ((p ^ C::zv(r)) << 3);
        __builtin_amdgcn_global_load_lds(gk, (__attribute__((address_space(3))) void *)(Ks + q * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(gv, (__attribute__((address_space(3))) void *)(Vs + q * 512), 16, 0, 0);
    }
}

__device__ __forceinline__ void wait_copies() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One HBM->LDS copy of 16 bytes per lane (global_load_lds_dwordx4 with a
// wave-uniform 64-bit base and a 32-bit per-lane byte offset); lane i's bytes
// land at lds_dst + 16*i.  Issued from inline asm so that the compiler's LDS
// DMA bookkeeping does not insert waits for it before unrelated LDS reads (it
// cannot tell the pipeline's stages apart); the pipeline waits for its copies
// explicitly (s_waitcnt vmcnt) before the barrier that publishes a stage.
// M0 (the LDS destination base) is saved and restored around the copy.
__device__ __forceinline__ void lds_copy16(const void *base, uint32_t voff, const void *lds_dst) {
    const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)lds_dst;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(m), "s"(base)
        : "memory");
}

// Workgroup barrier for the copy pipeline.  Unlike __syncthreads() it carries
// no memory fence (which would also wait for the HBM->LDS copies still in
// flight for later stages); the copies a stage needs are waited for
// explicitly, and this wave's LDS reads are drained so that no wave can
// overwrite a stage while another still reads it.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// V^T fragment via ds_read_b64_tr_b16: within each 16-lane group, lane i
// points at row (i/4), columns 4*(i%4)..+3 of a 4-row x 16-column block and
// receives column i of that block (4 consecutive rows).
template <class C, int D>
__device__ __forceinline__ s16x4_t read_vt(const __bf16 *Vs, int row, int col) {
    const int off = row * D + (((col >> 3) ^ C::zv(row)) << 3) + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(Vs + off));
}

// Compile-time integer carried through a generic lambda argument.
template <int V>
struct IntTag {
    static constexpr int value = V;
};

// f(IntTag<0>{}), f(IntTag<1>{}), ..., f(IntTag<N-1>{}): a loop whose index
// is a constant expression in the body (guaranteed unrolling, `if constexpr`
// on the index).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(IntTag<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace
}  // namespace fa
