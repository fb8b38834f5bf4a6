// Device helpers shared by the bf16 and fp32 forward kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// Hardware base-2 exponential (v_exp_f32): exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// Reductions over the lanes that hold the same query row.  With 32x32 matrix
// tiles a query's scores sit in lanes l and l^32; with 16x16 tiles in lanes
// l, l^16, l^32, l^48.  v_permlane32_swap / v_permlane16_swap exchange the
// halves without going through LDS; the two results of each swap hold the
// value from both partner lanes, so combining them is order-independent.
template <int MF>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (MF == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
        x = fmaxf(u2f(r[0]), u2f(r[1]));
    }
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
}

template <int MF>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (MF == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
        x = u2f(r[0]) + u2f(r[1]);
    }
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}

// Multiplier c of the base-2 logits, c = |scale| * log2(e) (a negative scale
// is folded into Q as an exact sign flip).  It is kept >= 1e-30 so that a
// masked logit (-inf) always gives c*s - m = -inf and exp2 = 0 without a
// select; for scale = 0 every |c*(s - max s)| stays far below half an ulp of
// 1, so each allowed key still gets weight exactly 1.
__device__ __forceinline__ float scale_factor(float scale_log2) {
    return fmaxf(fabsf(scale_log2), 1e-30f);
}

// True in every lane when any lane of the wave has `pred` set.
__device__ __forceinline__ bool wave_any(bool pred) {
    return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// Issue priority of the calling wave (s_setprio takes an immediate).  The
// SIMD picks the highest-priority ready wave, the oldest among equals.
__device__ __forceinline__ void set_wave_priority(int level) {
    if (level >= 3) __builtin_amdgcn_s_setprio(3);
    else if (level == 2) __builtin_amdgcn_s_setprio(2);
    else if (level == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// Key/value head read by query head bh = b*H + h: consecutive groups of
// H/Hkv query heads share one key/value head (grouped-query attention;
// Hkv = H is plain multi-head attention, Hkv = 1 multi-query attention).
template <class Args>
__device__ __forceinline__ int kv_head_of(int bh, const Args &a) {
    const int b = bh / a.H;
    return b * a.Hkv + (bh - b * a.H) / a.group;
}

// Work item of this workgroup.  The grid's items come in runs of per_head
// (one head's tiles, heaviest first when the mask is causal).  Workgroups
// are handed to the 8 XCDs round-robin (blockIdx % 8), and each XCD has its
// own L2, so each XCD gets a contiguous share of the items: whole heads
// when a head fits in one share, so that a head's K/V (or Q/dO) stays in one
// L2.  When a head's run spans X XCDs, those X XCDs take its items
// round-robin instead of X contiguous pieces, so that each gets heavy and
// light tiles alike; contiguous pieces would hand one XCD all the long
// causal rows.
__device__ __forceinline__ int xcd_item(int per_head) {
    const int G = gridDim.x;
    const int id = blockIdx.x;
    if ((G & 7) != 0) return id;
    const int per = G >> 3, x = id & 7, local = id >> 3;
    if (per_head > per && per_head % per == 0) {
        const int X = per_head / per;  // XCDs per head; G = (8 / X) heads * per_head
        const int head = x / X, j = x - head * X;
        return head * per_head + j + X * local;
    }
    return x * per + local;
}

// Work item of this workgroup on a grid whose items differ by batch entry
// (per-batch key lengths) but not within a head.  The contiguous shares of
// xcd_item would give each XCD a few whole batch entries, and the XCD with
// the longest ones would set the time.  Here units of `unit` consecutive
// items (the query heads that share one key/value head, all their tiles)
// go to the XCDs round-robin: XCD x takes units x, x + 8, x + 16, ..., so
// every XCD gets the same slice of every batch entry, and the CUs of an XCD
// (which take its workgroups l, l + 32, ...; see xcd_item_causal) get units
// of different entries.  A unit stays on one XCD, so its K/V re-reads stay
// in one L2.  Falls back to xcd_item when the shares do not hold whole
// units.
__device__ __forceinline__ int xcd_item_units(int unit, int per_head) {
    const int G = gridDim.x;
    const int id = blockIdx.x;
    if ((G & 7) != 0) return id;
    const int per = G >> 3;
    if (unit < 1 || per % unit != 0) return xcd_item(per_head);
    const int x = id & 7, local = id >> 3;
    const int k = local / unit;
    return (x + 8 * k) * unit + (local - k * unit);
}

// Work item of this workgroup on a causal grid, where the items of a head
// differ in cost (query tile qt sees the keys of query tiles 0..qt).  The
// XCD shares are those of xcd_item; within a share the order changes so
// that the workgroups that share a CU carry balanced work.  Within an XCD
// the dispatcher deals consecutive workgroups to its CUs in turn (observed
// with the hardware ID registers: the XCD's workgroups l, l + 32, l + 64, ...
// land on one CU), so the rounds that are resident together, the first
// `resident` rounds of kCusPerXcd workgroups (resident = workgroups of the
// kernel that fit on a CU at once), are dealt in a snake: forward for even
// rounds, backward for odd ones, so a CU that gets one of the heaviest
// items in one round gets one of the lighter ones in the next.  Later
// rounds are handed out as CUs free up and keep the heaviest-first order
// (snaking them hands out light items first: the GQA-4 16K backward, one
// dK/dV workgroup per CU, ran 17 % slower).  Where whole heads fit in a share they are first taken
// rank-major (the heaviest item of every head, then the next heaviest,
// ...); where a head spans X XCDs, its items stay round-robin over them as
// in xcd_item and each XCD's part is snaked.  For B8 H12 N1024 (one round
// of 768 workgroups, three per CU) the work per CU goes from 6..48 key
// tiles to 24..30; for B1 H4 N16384 (512 workgroups, two per CU, each head
// over two XCDs) from 68..192 to 130 tile units.  On long grids the
// rank-major order is longest-first across all heads of the XCD, which
// shortens the tail; it also keeps several heads' K/V streams in the XCD's
// L2 at once, which raised the HBM fetches of B1 H16 N16384 d128 from 365
// to 699 MB per launch (0.7 TB/s) while the time went down (head-major
// within the snake measured 1 % slower there and 6 % slower at d = 64).
// The order is a permutation of the items for every grid; a final partial
// round keeps its order.
constexpr int kCusPerXcd = 32;

__device__ __forceinline__ int snake_local(int local, int per, int resident) {
    const int j = local / kCusPerXcd, c = local - j * kCusPerXcd;
    const bool reverse = (j & 1) && j < resident && (j + 1) * kCusPerXcd <= per;
    return reverse ? j * kCusPerXcd + kCusPerXcd - 1 - c : local;
}

__device__ __forceinline__ int xcd_item_causal(int per_head, int resident) {
    const int G = gridDim.x;
    const int id = blockIdx.x;
    if ((G & 7) != 0) return id;
    const int per = G >> 3, x = id & 7, local = id >> 3;
    const int p = snake_local(local, per, resident);
    if (per_head > per && per_head % per == 0) {
        // a head spans X XCDs, which take its items round-robin (xcd_item)
        const int X = per_head / per;
        const int head = x / X, j = x - head * X;
        return head * per_head + j + X * p;
    }
    if (per % per_head == 0) {
        const int heads = per / per_head;
        const int rank = p / heads, head = p - rank * heads;
        return x * per + head * per_head + rank;
    }
    return x * per + p;
}

// Workgroup -> (head, query tile).  Causal grids take the longest query
// tiles first, in the CU-balanced order of xcd_item_causal; other grids
// take each head's tiles in order, whole heads per XCD where possible
// (keeping a head's K/V re-reads inside one XCD's L2), and with
// unit > 0 (per-batch key lengths) units of that many items dealt to the
// XCDs round-robin (xcd_item_units).
__device__ __forceinline__ void tile_of_block(int nqt, bool longest_first, int resident,
                                              int *bh, int *qt, int unit = 0) {
    const int id = longest_first ? xcd_item_causal(nqt, resident)
                                 : (unit > 0 ? xcd_item_units(unit, nqt) : xcd_item(nqt));
    *bh = id / nqt;
    const int r = id - *bh * nqt;
    *qt = longest_first ? nqt - 1 - r : r;
}

}  // namespace fa
