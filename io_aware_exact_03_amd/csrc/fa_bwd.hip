// Exact-attention backward pass for gfx950: the gradients dQ, dK, dV of the
// loss sum(dO * O), bf16 or fp16 inputs and outputs (every kernel is a
// template on the element type T), fp32 accumulation.
//
// The pages give the forward definition (page "Ch.04 Attention
// optimisation: FlashAttention and sparse attention", mdooai.com, "Core
// formula") and say the method's speed-ups are training speed-ups (page
// "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", ai-paper-library, Summary); the backward is the chain rule
// applied to that definition, computed with the same IO-aware structure as
// the forward: the probabilities are recomputed tile by tile from Q, K and
// the forward's per-row log-sum-exp, never stored in HBM.  With
// P = exp(S - LSE), dP = dO V^T, Delta_i = dO_i . O_i, dS = P * (dP - Delta):
//     dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K.
//
// Kernels:
//  * bwd_delta: Delta_i = dO_i . O_i per query row (fp32, caller workspace).
//  * bwd_dkdv: one workgroup per block of 32*NW keys of one key/value head;
//    each wave keeps its 32 keys' K fragments (and, unless VL, V fragments)
//    and the dK^T, dV^T accumulators in registers and walks the query tiles
//    (32*QT rows of Q and dO, with their LSE and Delta, staged in LDS per
//    step) of every query head that reads this key/value head.  Per step:
//    S = Q K^T and dP = dO V^T (lane = key), then dV^T += dO^T P^T and
//    dK^T += Q^T dS^T.  Used for d = 64 without the causal mask (V in
//    registers, 64 rows per step) and for d = 128 grids of two or more
//    rounds (VL: V read from the key block's LDS tile, 32 rows per step;
//    two workgroups per CU).
//  * bwd_dkdv_pair (causal d = 64, and d = 128 grids that fill the CUs
//    only once): the same product chain with 8 waves per 128 keys, two
//    waves per 32 keys splitting each 64-row query tile, so that a wave's
//    registers fit two waves per SIMD at d = 128; the pair's partial dK, dV
//    are added through LDS at the end.
//  * bwd_dq: one workgroup per 32*NW query rows; each wave keeps its rows'
//    Q and dO fragments and the dQ^T accumulator in registers and walks the
//    key tiles (64 keys of K and V staged in LDS per step, taken as two
//    32-key chunks).  Per chunk: S^T = K Q^T, dP^T = V dO^T (lane = query),
//    then dQ^T += K^T dS^T.
//  * bwd_reduce: with a query-head split of grouped heads (fa_bwd_ex with a
//    workspace), the dK/dV kernels write fp32 partials per split and this
//    kernel adds them in split order and rounds once.
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomics
// and no fp32 scratch for dQ, and keeps the results deterministic.
//
// Layouts of the 32x32x16 bf16 / fp16 matrix-core products (fp32 accumulate) are
// those of the forward kernels: a product's 16 accumulator values per lane
// are one column (lane % 32) and 16 rows; fed back as the B operand of the
// next product, 8 of them give the 16-row reduction block with the row
// permutation r(half, j) = 8*(j/4) + 4*half + j%4, which the transposed LDS
// reads of the A operand reproduce.
#include "fa_bf16_tiles.h"

namespace fa {
namespace {

// Swizzle of the 16-byte slots of a tile row for tiles that are read both
// as rows (ds_read_b128, 16 consecutive rows per 16-lane group) and
// transposed (ds_read_b64_tr_b16, 4 rows x 4 slots per half-wave): for D =
// 128, z(r) = 4*(r%4) + (r/4)%4 gives 16 distinct slots over any 16 aligned
// rows and 16 distinct (row, slot) banks for a transposed read; for D = 64
// (two rows per 256-byte bank line) the same on r/2.  z depends on r % 16
// only.
template <int D>
__device__ __forceinline__ int zkv(int r) {
    constexpr int RPL = 128 / D, G = D / 32;
    const int x = r / RPL;
    return 4 * (x % G) + (x / G) % 4;
}

// Element offset of logical slot `slot` of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int slot) {
    return r * D + ((slot ^ zkv<D>(r)) << 3);
}

template <int D>
struct BwdGeom {
    static constexpr int SLOTS = D / 8;
    static constexpr int NQK = D / 16;  // 16-wide head-dim chunks
    static constexpr int ND = D / 32;   // 32-wide output blocks
    static constexpr int TILE = 32 * D; // elements per 32-row tile
    static constexpr int NCOPY = TILE / 512;
};

// Copy rows [r0, r0 + ROWS) of a [.., D] matrix of 16-bit elements (bf16 or
// fp16) into a swizzled LDS tile (rows >= rows_valid re-read the last valid
// row: their results are masked).  The NW waves split the 1 KiB copy
// instructions.  G and dst are byte addresses.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void copy_rows(const void *G, int r0, int rows_valid, void *dst,
                                          int wave, int lane) {
    constexpr int SLOTS = D / 8, NCOPY = ROWS * D / 512;
#pragma unroll
    for (int q0 = 0; q0 < NCOPY; q0 += NW) {
        const int q = q0 + wave;
        if (NCOPY % NW != 0 && q >= NCOPY) break;
        const int ci = q * 64 + lane;
        const int r = ci / SLOTS, p = ci % SLOTS;
        const int row = min(r0 + r, rows_valid - 1);
        const char *src = static_cast<const char *>(G) + ((int64_t)row * D + ((p ^ zkv<D>(r)) << 3)) * 2;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(static_cast<char *>(dst) + q * 1024),
                                         16, 0, 0);
    }
}

// Per-lane offsets (elements, relative to a 16-row chunk) of the two 4-row
// transposed reads that give the A fragment [32 columns of output block mb]
// x [16 rows of the chunk] with the row permutation of the B fragments.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&lo)[D / 32], int (&hi)[D / 32]) {
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
        const int row = 4 * (g >> 1) + (li >> 2);
        const int col = mb * 32 + 16 * (g & 1) + 4 * (li & 3);
        lo[mb] = row * D + (((col >> 3) ^ zkv<D>(row)) << 3) + (col & 7);
        hi[mb] = (row + 8) * D + (((col >> 3) ^ zkv<D>(row + 8)) << 3) + (col & 7);
    }
}

template <class T>
__device__ __forceinline__ typename Elem<T>::x8 read_tr8(const T *base, int lo, int hi) {
    const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + lo));
    const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + hi));
    return __builtin_bit_cast(typename Elem<T>::x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return Elem<__bf16>::mfma(a, b, c);
}
__device__ __forceinline__ f32x16_t mfma(f16x8_t a, f16x8_t b, f32x16_t c) {
    return Elem<_Float16>::mfma(a, b, c);
}

// Row of accumulator value i of lane l in a 32x32 product block.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// A staged tile's log-sum-exps in the form the exponentials take them:
// -LSE * log2(e), and -inf for a row with no allowed key (its p is then 0).
// Run by wave 0, which issued the LSE copy into LDS and has waited for it,
// once per row of the tile instead of once per score; the next barrier
// publishes it.
__device__ __forceinline__ void lse_to_neg_log2(float *l, int rows) {
    // the lane index recomputed here rather than kept live across the loop
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if (lane < rows) {
        const float x = l[lane];
        l[lane] = x == kNegInf ? kNegInf : -(x * 1.44269504088896341f);
    }
}

// ---------------------------------------------------------------- Delta

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_delta(BwdArgs a) {
    using x8_t = typename Elem<T>::x8;
    using x4_t = typename Elem<T>::x4;
    // 16 lanes (D = 128) or 8 lanes (D = 64) per row, 8 elements each.
    constexpr int LPR = D / 8;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const x8_t x = *reinterpret_cast<const x8_t *>(
            reinterpret_cast<const T *>(a.o) + row * D + part * 8);
        const x8_t y = *reinterpret_cast<const x8_t *>(
            reinterpret_cast<const T *>(a.dout) + row * D + part * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf((float)x[j], (float)y[j], acc);
    }
#pragma unroll
    for (int s = LPR / 2; s > 0; s /= 2) acc += __shfl_xor(acc, s, LPR);
    if (row < rows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------- dK, dV

// Workgroup -> (query-head split, batch * key/value head, key block), via
// the XCD-aware item order of xcd_item: the splits of one key block are
// adjacent (they read the same K and V), and within a head the key blocks
// run in ascending order.  Causal grids, where key block kt is seen by the
// query rows from kt on (the first blocks the most), use the CU-balanced
// order of xcd_item_causal instead (heaviest blocks of every head first).
// With per-batch key lengths (the key blocks past a batch entry's length
// carry no work) whole key/value heads are dealt to the XCDs round-robin
// (xcd_item_units), so every XCD gets the same share of every entry.
__device__ __forceinline__ void dkdv_block(int nkt, int nsplit, int *split, int *bkv, int *kt, bool causal,
                                           int resident, bool by_units) {
    // resident: workgroups of the kernel that fit one CU together
    int id = causal ? xcd_item_causal(nkt * nsplit, resident)
                    : (by_units ? xcd_item_units(nkt * nsplit, nkt * nsplit) : xcd_item(nkt * nsplit));
    *split = id % nsplit;
    id /= nsplit;
    *bkv = id / nkt;
    *kt = id - *bkv * nkt;
}

// Sum of the nsplit fp32 partials of dK (times the scale) and dV, rounded
// once to the element type.  Four consecutive elements per thread, in split
// order (deterministic).
template <class T>
__global__ __launch_bounds__(256) void bwd_reduce(BwdArgs a, int64_t el) {
    using x4_t = typename Elem<T>::x4;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= el) return;
    f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.nsplit; ++s) {
        sk += *reinterpret_cast<const f32x4_t *>(a.part + (int64_t)(2 * s) * el + i);
        sv += *reinterpret_cast<const f32x4_t *>(a.part + (int64_t)(2 * s + 1) * el + i);
    }
    x4_t wk, wv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        wk[j] = (T)(sk[j] * a.scale);
        wv[j] = (T)sv[j];
    }
    *reinterpret_cast<x4_t *>(reinterpret_cast<T *>(a.dk) + i) = wk;
    *reinterpret_cast<x4_t *>(reinterpret_cast<T *>(a.dv) + i) = wv;
}

template <class T, int D, int NW, int QT, bool CAUSAL, bool VL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkdv(BwdArgs a) {
    using x8_t = typename Elem<T>::x8;
    using x4_t = typename Elem<T>::x4;
    using Geo = BwdGeom<D>;
    constexpr int NQK = Geo::NQK, ND = Geo::ND, BK = 32 * NW, BQ = 32 * QT;
    static_assert(128 % BQ == 0, "a query tile lies inside one 128-row mask block");
    // Q and dO tiles of BQ rows, and the tile's LSE and Delta (BQ floats
    // each, LSE first), double-buffered.
    __shared__ __attribute__((aligned(1024))) T q_lds[2][BQ * D];
    __shared__ __attribute__((aligned(1024))) T do_lds[2][BQ * D];
    __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * BQ];
    // VL: the key block's V rows, loaded once (the V^T fragments are read
    // from here at every step instead of being held in registers).
    __shared__ __attribute__((aligned(1024))) T v_lds[VL ? BK * D : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nkt = (N + BK - 1) / BK;
    // Workgroup -> (batch, key/value head, key block, query-head split);
    // causal grids start with the key blocks that see the most query rows.
    int split, bkv, kt;
    dkdv_block(nkt, a.nsplit, &split, &bkv, &kt, CAUSAL, 2, a.key_len != nullptr);
    const int b = bkv / a.Hkv;
    const int hkv = bkv - b * a.Hkv;
    const int k0 = kt * BK, kw0 = k0 + wave * 32;

    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    const int64_t kvhead = (int64_t)bkv * N * D;
    const T *K = reinterpret_cast<const T *>(a.k) + kvhead;
    const T *V = reinterpret_cast<const T *>(a.v) + kvhead;
    const float c = a.scale_log2;
    const bool wave_live = kw0 < kv_len;  // keys >= kv_len get zero gradients

    // This wave's 32 keys as B operands: K^T and V^T fragments (lane: key
    // lane % 32, head dims 16*ks + 8*(lane/32) .. +7).
    const int key = kw0 + lane % 32;
    x8_t kf[NQK], vf[VL ? 1 : NQK];
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) {
        u32x4_t xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        if (key < N) {
            xk = *reinterpret_cast<const u32x4_t *>(K + (int64_t)key * D + ks * 16 + 8 * (lane / 32));
            if constexpr (!VL)
                xv = *reinterpret_cast<const u32x4_t *>(V + (int64_t)key * D + ks * 16 + 8 * (lane / 32));
        }
        kf[ks] = __builtin_bit_cast(x8_t, xk);
        if constexpr (!VL) vf[ks] = __builtin_bit_cast(x8_t, xv);
    }
    f32x16_t dk[ND], dv[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[mb][i] = dv[mb][i] = 0.f;

    const int rbase = (lane % 32) * D + (((lane / 32) ^ zkv<D>(lane % 32)) << 3);
    int trlo[ND], trhi[ND];
    tr_offsets<D>(lane, trlo, trhi);

    // Query tiles of BQ rows this key block can receive gradient from.
    const int qt_first = CAUSAL ? k0 / BQ : 0;
    const int nqt = (N + BQ - 1) / BQ;
    const int steps_per_head = nqt - qt_first;
    // Steps (query head g of the group, query tile) in head-major order;
    // this workgroup takes the contiguous range [s_lo, nsteps) of its split.
    // Workgroup-uniform (every wave takes part in the copies and barriers).
    const int total = k0 >= kv_len ? 0 : steps_per_head * a.group;
    const int s_lo = (int)((int64_t)total * split / a.nsplit);
    const int nsteps = (int)((int64_t)total * (split + 1) / a.nsplit);
    auto step_tile = [&](int s, int *hq, int *qt) {
        const int g = s / steps_per_head;
        *hq = b * a.H + hkv * a.group + g;
        *qt = qt_first + (s - g * steps_per_head);
    };
    auto tile_active = [&](int qt) {
        if (!a.block_mask) return true;
        return a.block_mask[(int64_t)((qt * BQ) >> 7) * a.nkb + (k0 >> 7)] != 0;
    };
    auto issue = [&](int s, int buf) {
        int hq, qt;
        step_tile(s, &hq, &qt);
        const int64_t qhead = (int64_t)hq * N * D;
        copy_rows<D, NW, BQ>(reinterpret_cast<const T *>(a.q) + qhead, qt * BQ, N, q_lds[buf], wave,
                             lane);
        copy_rows<D, NW, BQ>(reinterpret_cast<const T *>(a.dout) + qhead, qt * BQ, N, do_lds[buf],
                             wave, lane);
        // LSE and Delta of the tile's rows (4 bytes per lane; clamped rows
        // past N are masked).
        if (wave * 64 < 2 * BQ) {
            const int idx = wave * 64 + lane;  // 0 .. 2*BQ-1
            const int r = min(qt * BQ + (idx % BQ), N - 1);
            const float *src = (idx < BQ ? a.lse : a.delta) + (int64_t)hq * N + r;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(&ld_lds[buf][wave * 64]),
                                             4, 0, 0);
        }
    };
    // next active step at or after s (block mask), or nsteps
    auto next_step = [&](int s) {
        while (s < nsteps) {
            int hq, qt;
            step_tile(s, &hq, &qt);
            if (tile_active(qt)) break;
            ++s;
        }
        return s;
    };

    int s = next_step(s_lo);
    if (s < nsteps) {
        // (rows past N re-read row N-1; those keys get p = 0)
        if constexpr (VL) copy_rows<D, NW, BK>(V, k0, N, v_lds, wave, lane);
        issue(s, 0);
        if (wave == 0) {
            wait_copies();
            lse_to_neg_log2(ld_lds[0], BQ);
        }
    }
    const T *vw = VL ? v_lds + wave * 32 * D : v_lds;  // VL: this wave's 32 V rows
    int buf = 0;
    while (s < nsteps) {
        const int sn = next_step(s + 1);
        wait_copies();
        __syncthreads();
        if (sn < nsteps) issue(sn, buf ^ 1);
        int hq, qt;
        step_tile(s, &hq, &qt);
        const int qs0 = qt * BQ;
        const float *lds_l = ld_lds[buf];
#pragma unroll
        for (int hq32 = 0; hq32 < QT; ++hq32) {
            const int qs = qs0 + 32 * hq32;
            const T *Qs = q_lds[buf] + hq32 * 32 * D, *dOs = do_lds[buf] + hq32 * 32 * D;
            // this wave's keys see some query of these 32 rows
            if (wave_live && (!CAUSAL || qs + 31 >= kw0)) {
                // S = Q K^T and dP = dO V^T: D[m = query][n = key].
                f32x16_t sacc = {}, dpacc = {};
#pragma unroll
                for (int ks = 0; ks < NQK; ++ks) {
                    const x8_t qa = *reinterpret_cast<const x8_t *>(Qs + (rbase ^ (ks << 4)));
                    const x8_t da = *reinterpret_cast<const x8_t *>(dOs + (rbase ^ (ks << 4)));
                    x8_t vb;
                    if constexpr (VL)
                        vb = *reinterpret_cast<const x8_t *>(vw + (rbase ^ (ks << 4)));
                    else
                        vb = vf[ks];
                    sacc = mfma(qa, kf[ks], sacc);
                    dpacc = mfma(da, vb, dpacc);
                }
                const bool edge = (qs + 32 > N) || (kw0 + 32 > kv_len) || (CAUSAL && qs < kw0 + 31);
                // P and dS in place; this lane's 16 rows are 4 groups of 4
                // consecutive query rows: LSE and Delta as float4 LDS reads.
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int r4 = 32 * hq32 + 8 * gi + 4 * (lane >> 5);
                    const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(lds_l + r4);
                    const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(lds_l + BQ + r4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 4 * gi + j;
                        // l4: -LSE * log2(e) of the row (lse_to_neg_log2)
                        float p = fast_exp2(fmaf(sacc[i], c, l4[j]));
                        if (edge) {
                            const int qi = qs + acc_row(i, lane);
                            const bool ok = qi < N && key < kv_len && (!CAUSAL || key <= qi);
                            p = ok ? p : 0.f;
                        }
                        dpacc[i] = p * (dpacc[i] - d4[j]);
                        sacc[i] = p;
                    }
                    // VL at d = 128 sits at 256 registers: without this fence
                    // the scheduler hoists later groups' reads and spills
                    if constexpr (VL) __builtin_amdgcn_sched_barrier(0);
                }
                // dV^T += dO^T P^T and dK^T += Q^T dS^T over the two 16-row chunks.
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    x8_t pf, dsf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        pf[j] = (T)sacc[8 * h + j];
                        dsf[j] = (T)dpacc[8 * h + j];
                    }
#pragma unroll
                    for (int mb = 0; mb < ND; ++mb) {
                        const x8_t dot = read_tr8(dOs + h * 16 * D, trlo[mb], trhi[mb]);
                        const x8_t qtr = read_tr8(Qs + h * 16 * D, trlo[mb], trhi[mb]);
                        dv[mb] = mfma(dot, pf, dv[mb]);
                        dk[mb] = mfma(qtr, dsf, dk[mb]);
                    }
                }
            }
        }
        if (sn < nsteps && wave == 0) {
            wait_copies();
            lse_to_neg_log2(ld_lds[buf ^ 1], BQ);
        }
        s = sn;
        buf ^= 1;
    }

    // dK = scale * (dK^T)^T, dV: lane holds key lane % 32, head dims
    // 32*mb + 8*gg + 4*(lane/32) .. +3.  With a query-head split, fp32
    // partials (dK before the scale) go to the workspace instead.
    if (key < N && a.nsplit > 1) {
        const int64_t el = (int64_t)a.B * a.Hkv * N * D;
        float *pk = a.part + (int64_t)(2 * split) * el + kvhead + (int64_t)key * D;
        float *pv = pk + el;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                f32x4_t wk, wv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wk[j] = dk[mb][4 * gg + j];
                    wv[j] = dv[mb][4 * gg + j];
                }
                *reinterpret_cast<f32x4_t *>(pk + mb * 32 + 8 * gg + 4 * (lane / 32)) = wk;
                *reinterpret_cast<f32x4_t *>(pv + mb * 32 + 8 * gg + 4 * (lane / 32)) = wv;
            }
    } else if (key < N) {
        const float scale = a.scale;
        T *dK = reinterpret_cast<T *>(a.dk) + kvhead + (int64_t)key * D;
        T *dV = reinterpret_cast<T *>(a.dv) + kvhead + (int64_t)key * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                x4_t wk, wv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wk[j] = (T)(dk[mb][4 * gg + j] * scale);
                    wv[j] = (T)dv[mb][4 * gg + j];
                }
                *reinterpret_cast<x4_t *>(dK + mb * 32 + 8 * gg + 4 * (lane / 32)) = wk;
                *reinterpret_cast<x4_t *>(dV + mb * 32 + 8 * gg + 4 * (lane / 32)) = wv;
            }
    }
}

// dK, dV with two waves per key group (d = 128, two waves per SIMD): a
// workgroup of 8 waves owns 128 keys; waves w and w+4 hold the same 32 keys
// and take the two 32-row halves of each 64-row query tile, so each keeps only
// its K fragments and its dK^T, dV^T accumulators in registers (V fragments
// come from the key block's K/V tiles, loaded into LDS once).  The two
// partial sums of each key group are added through LDS at the end.
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(512, D == 64 ? 2 : 1) void bwd_dkdv_pair(BwdArgs a) {
    using x8_t = typename Elem<T>::x8;
    using x4_t = typename Elem<T>::x4;
    using Geo = BwdGeom<D>;
    constexpr int NQK = Geo::NQK, ND = Geo::ND, NW = 8, BK = 128, BQ = 64;
    constexpr int KV_BYTES = BK * D * 2, T_BYTES = BQ * D * 2;
    constexpr int RED_BYTES = 4 * 2 * ND * 16 * 64 * 4;  // 4 groups x (dk, dv) x 16*ND floats x 64 lanes
    constexpr int POOL = 2 * KV_BYTES + 4 * T_BYTES > RED_BYTES ? 2 * KV_BYTES + 4 * T_BYTES : RED_BYTES;
    __shared__ __attribute__((aligned(1024))) char pool[POOL];
    __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * BQ];
    T *const k_lds = reinterpret_cast<T *>(pool);
    T *const v_lds = reinterpret_cast<T *>(pool + KV_BYTES);
    auto q_lds = [&](int buf) { return reinterpret_cast<T *>(pool + 2 * KV_BYTES + buf * T_BYTES); };
    auto do_lds = [&](int buf) { return reinterpret_cast<T *>(pool + 2 * KV_BYTES + (2 + buf) * T_BYTES); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, qh = wave >> 2;
    const int N = a.N;
    const int nkt = (N + BK - 1) / BK;
    int split, bkv, kt;
    dkdv_block(nkt, a.nsplit, &split, &bkv, &kt, CAUSAL, 1, a.key_len != nullptr);
    const int b = bkv / a.Hkv;
    const int hkv = bkv - b * a.Hkv;
    const int k0 = kt * BK, kw0 = k0 + kg * 32;

    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    const int64_t kvhead = (int64_t)bkv * N * D;
    const float c = a.scale_log2;
    const bool wave_live = kw0 < kv_len;
    const int key = kw0 + lane % 32;

    // The key block's K and V rows into LDS (rows past N re-read row N-1).
    copy_rows<D, NW, BK>(reinterpret_cast<const T *>(a.k) + kvhead, k0, N, k_lds, wave, lane);
    copy_rows<D, NW, BK>(reinterpret_cast<const T *>(a.v) + kvhead, k0, N, v_lds, wave, lane);

    const int rbase = (lane % 32) * D + (((lane / 32) ^ zkv<D>(lane % 32)) << 3);
    int trlo[ND], trhi[ND];
    tr_offsets<D>(lane, trlo, trhi);
    f32x16_t dk[ND], dv[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[mb][i] = dv[mb][i] = 0.f;

    const int qt_first = CAUSAL ? k0 / BQ : 0;
    const int nqt = (N + BQ - 1) / BQ;
    const int steps_per_head = nqt - qt_first;
    // Steps in head-major order; this workgroup's split takes [s_lo, nsteps).
    const int total = k0 >= kv_len ? 0 : steps_per_head * a.group;
    const int s_lo = (int)((int64_t)total * split / a.nsplit);
    const int nsteps = (int)((int64_t)total * (split + 1) / a.nsplit);
    auto step_tile = [&](int s, int *hq, int *qt) {
        const int g = s / steps_per_head;
        *hq = b * a.H + hkv * a.group + g;
        *qt = qt_first + (s - g * steps_per_head);
    };
    auto tile_active = [&](int qt) {
        if (!a.block_mask) return true;
        return a.block_mask[(int64_t)((qt * BQ) >> 7) * a.nkb + (k0 >> 7)] != 0;
    };
    auto issue = [&](int s, int buf) {
        int hq, qt;
        step_tile(s, &hq, &qt);
        const int64_t qhead = (int64_t)hq * N * D;
        copy_rows<D, NW, BQ>(reinterpret_cast<const T *>(a.q) + qhead, qt * BQ, N, q_lds(buf), wave, lane);
        copy_rows<D, NW, BQ>(reinterpret_cast<const T *>(a.dout) + qhead, qt * BQ, N, do_lds(buf), wave,
                             lane);
        if (wave < 2) {
            const int idx = wave * 64 + lane;
            const int r = min(qt * BQ + (idx % BQ), N - 1);
            const float *src = (idx < BQ ? a.lse : a.delta) + (int64_t)hq * N + r;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(&ld_lds[buf][wave * 64]),
                                             4, 0, 0);
        }
    };
    auto next_step = [&](int s) {
        while (s < nsteps) {
            int hq, qt;
            step_tile(s, &hq, &qt);
            if (tile_active(qt)) break;
            ++s;
        }
        return s;
    };

    int s = next_step(s_lo);
    if (s < nsteps) issue(s, 0);
    wait_copies();
    if (s < nsteps && wave == 0) lse_to_neg_log2(ld_lds[0], BQ);
    __syncthreads();
    // This wave's K^T fragments (B operand of S = Q K^T), kept in registers.
    x8_t kf[NQK];
    const T *kg_k = k_lds + kg * 32 * D, *kg_v = v_lds + kg * 32 * D;
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) kf[ks] = *reinterpret_cast<const x8_t *>(kg_k + (rbase ^ (ks << 4)));

    int buf = 0;
    while (s < nsteps) {
        const int sn = next_step(s + 1);
        wait_copies();
        __syncthreads();
        if (sn < nsteps) issue(sn, buf ^ 1);
        int hq, qt;
        step_tile(s, &hq, &qt);
        const int qs = qt * BQ + 32 * qh;
        const T *Qs = q_lds(buf) + qh * 32 * D, *dOs = do_lds(buf) + qh * 32 * D;
        const float *lds_l = ld_lds[buf];
        if (wave_live && (!CAUSAL || qs + 31 >= kw0)) {
            f32x16_t sacc = {}, dpacc = {};
#pragma unroll
            for (int ks = 0; ks < NQK; ++ks) {
                const x8_t qa = *reinterpret_cast<const x8_t *>(Qs + (rbase ^ (ks << 4)));
                const x8_t da = *reinterpret_cast<const x8_t *>(dOs + (rbase ^ (ks << 4)));
                const x8_t vb = *reinterpret_cast<const x8_t *>(kg_v + (rbase ^ (ks << 4)));
                sacc = mfma(qa, kf[ks], sacc);
                dpacc = mfma(da, vb, dpacc);
            }
            const bool edge = (qs + 32 > N) || (kw0 + 32 > kv_len) || (CAUSAL && qs < kw0 + 31);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int r4 = 32 * qh + 8 * gi + 4 * (lane >> 5);
                const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(lds_l + r4);
                const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(lds_l + BQ + r4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * gi + j;
                    float p = fast_exp2(fmaf(sacc[i], c, l4[j]));  // l4: -LSE * log2(e)
                    if (edge) {
                        const int qi = qs + acc_row(i, lane);
                        const bool ok = qi < N && key < kv_len && (!CAUSAL || key <= qi);
                        p = ok ? p : 0.f;
                    }
                    dpacc[i] = p * (dpacc[i] - d4[j]);
                    sacc[i] = p;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                x8_t pf, dsf;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pf[j] = (T)sacc[8 * h + j];
                    dsf[j] = (T)dpacc[8 * h + j];
                }
#pragma unroll
                for (int mb = 0; mb < ND; ++mb) {
                    const x8_t dot = read_tr8(dOs + h * 16 * D, trlo[mb], trhi[mb]);
                    const x8_t qtr = read_tr8(Qs + h * 16 * D, trlo[mb], trhi[mb]);
                    dv[mb] = mfma(dot, pf, dv[mb]);
                    dk[mb] = mfma(qtr, dsf, dk[mb]);
                }
            }
        }
        if (sn < nsteps && wave == 0) {
            wait_copies();
            lse_to_neg_log2(ld_lds[buf ^ 1], BQ);
        }
        s = sn;
        buf ^= 1;
    }

    // Add the two halves' partial sums: the upper waves park theirs in LDS.
    wait_copies();
    __syncthreads();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(pool) + (int64_t)kg * (2 * ND * 4) * 64;
    if (qh == 1) {
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                f32x4_t xk, xv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xk[j] = dk[mb][4 * gg + j];
                    xv[j] = dv[mb][4 * gg + j];
                }
                red[((2 * mb) * 4 + gg) * 64 + lane] = xk;
                red[((2 * mb + 1) * 4 + gg) * 64 + lane] = xv;
            }
    }
    __syncthreads();
    if (qh == 0 && key < N && a.nsplit > 1) {
        // fp32 partials of this query-head split (dK before the scale)
        const int64_t el = (int64_t)a.B * a.Hkv * N * D;
        float *pk = a.part + (int64_t)(2 * split) * el + kvhead + (int64_t)key * D;
        float *pv = pk + el;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const f32x4_t xk = red[((2 * mb) * 4 + gg) * 64 + lane];
                const f32x4_t xv = red[((2 * mb + 1) * 4 + gg) * 64 + lane];
                f32x4_t wk, wv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wk[j] = dk[mb][4 * gg + j] + xk[j];
                    wv[j] = dv[mb][4 * gg + j] + xv[j];
                }
                *reinterpret_cast<f32x4_t *>(pk + mb * 32 + 8 * gg + 4 * (lane / 32)) = wk;
                *reinterpret_cast<f32x4_t *>(pv + mb * 32 + 8 * gg + 4 * (lane / 32)) = wv;
            }
    } else if (qh == 0 && key < N) {
        const float scale = a.scale;
        T *dK = reinterpret_cast<T *>(a.dk) + kvhead + (int64_t)key * D;
        T *dV = reinterpret_cast<T *>(a.dv) + kvhead + (int64_t)key * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const f32x4_t xk = red[((2 * mb) * 4 + gg) * 64 + lane];
                const f32x4_t xv = red[((2 * mb + 1) * 4 + gg) * 64 + lane];
                x4_t wk, wv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wk[j] = (T)((dk[mb][4 * gg + j] + xk[j]) * scale);
                    wv[j] = (T)(dv[mb][4 * gg + j] + xv[j]);
                }
                *reinterpret_cast<x4_t *>(dK + mb * 32 + 8 * gg + 4 * (lane / 32)) = wk;
                *reinterpret_cast<x4_t *>(dV + mb * 32 + 8 * gg + 4 * (lane / 32)) = wv;
            }
    }
}

// Sum of the nsplit_q fp32 partials of dQ, times the scale, rounded once.
template <class T>
__global__ __launch_bounds__(256) void bwd_reduce_dq(BwdArgs a, int64_t el) {
    using x4_t = typename Elem<T>::x4;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= el) return;
    f32x4_t sq = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.nsplit_q; ++s) sq += *reinterpret_cast<const f32x4_t *>(a.part_q + (int64_t)s * el + i);
    x4_t w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (T)(sq[j] * a.scale);
    *reinterpret_cast<x4_t *>(reinterpret_cast<T *>(a.dq) + i) = w;
}

// ---------------------------------------------------------------- dQ

template <class T, int D, int NW, int KT, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq(BwdArgs a) {
    using x8_t = typename Elem<T>::x8;
    using x4_t = typename Elem<T>::x4;
    using Geo = BwdGeom<D>;
    constexpr int NQK = Geo::NQK, ND = Geo::ND, BR = 32 * NW, BKT = 32 * KT;
    static_assert(128 % BKT == 0, "a key step lies inside one 128-key mask block");
    __shared__ __attribute__((aligned(1024))) T k_lds[2][KT * Geo::TILE];
    __shared__ __attribute__((aligned(1024))) T v_lds[2][KT * Geo::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nqt = (N + BR - 1) / BR;
    // (query tile, key-range split): the splits of one query tile adjacent,
    // heads and tiles in the XCD-aware order; causal grids longest first in
    // the CU-balanced order (two (d = 128) or three (d = 64) workgroups per
    // CU); with per-batch key lengths the query heads of one key/value head
    // are dealt to the XCDs round-robin (xcd_item_units).
    const int per_head = nqt * a.nsplit_q;
    const int item = CAUSAL ? xcd_item_causal(per_head, D == 128 ? 2 : 3)
                            : (a.key_len ? xcd_item_units(a.group * per_head, per_head) : xcd_item(per_head));
    const int split = item % a.nsplit_q;
    const int rest = item / a.nsplit_q;
    const int bh = rest / nqt;
    const int qt = CAUSAL ? nqt - 1 - (rest - bh * nqt) : rest - bh * nqt;
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t kvhead = (int64_t)kv_head_of(bh, a) * N * D;
    const T *Q = reinterpret_cast<const T *>(a.q) + head;
    const T *dO = reinterpret_cast<const T *>(a.dout) + head;
    const T *K = reinterpret_cast<const T *>(a.k) + kvhead;
    const T *V = reinterpret_cast<const T *>(a.v) + kvhead;
    const float c = a.scale_log2;

    const int q0 = qt * BR, wq0 = q0 + wave * 32;
    const int qrow = wq0 + lane % 32;
    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + BR);
    const int nall = (kv_end + BKT - 1) / BKT;
    // Key steps [t_lo, ntiles) of this split (all of them when unsplit).
    const int t_lo = (int)((int64_t)nall * split / a.nsplit_q);
    const int ntiles = (int)((int64_t)nall * (split + 1) / a.nsplit_q);

    // This wave's 32 query rows as B operands: Q^T and dO^T fragments.
    x8_t qf[NQK], dof[NQK];
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) {
        u32x4_t xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u};
        if (qrow < N) {
            xq = *reinterpret_cast<const u32x4_t *>(Q + (int64_t)qrow * D + ks * 16 + 8 * (lane / 32));
            xd = *reinterpret_cast<const u32x4_t *>(dO + (int64_t)qrow * D + ks * 16 + 8 * (lane / 32));
        }
        qf[ks] = __builtin_bit_cast(x8_t, xq);
        dof[ks] = __builtin_bit_cast(x8_t, xd);
    }
    float lse2 = __builtin_inff(), dl = 0.f;
    if (qrow < N) {
        const float l = a.lse[(int64_t)bh * N + qrow];
        lse2 = l == kNegInf ? __builtin_inff() : l * 1.44269504088896341f;
        dl = a.delta[(int64_t)bh * N + qrow];
    }
    f32x16_t dq[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[mb][i] = 0.f;

    const int rbase = (lane % 32) * D + (((lane / 32) ^ zkv<D>(lane % 32)) << 3);
    int trlo[ND], trhi[ND];
    tr_offsets<D>(lane, trlo, trhi);

    // Key steps of BKT keys (KT chunks of 32), skipping 128-key blocks the
    // mask turns off.
    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;
    auto next_tile = [&](int t) {
        if (mrow)
            while (t < ntiles && mrow[(t * BKT) >> 7] == 0) t = (((t * BKT) >> 7) + 1) * (128 / BKT);
        return min(t, ntiles);
    };
    auto issue = [&](int t, int buf) {
        copy_rows<D, NW, BKT>(K, t * BKT, kv_len, k_lds[buf], wave, lane);
        copy_rows<D, NW, BKT>(V, t * BKT, kv_len, v_lds[buf], wave, lane);
    };

    int t = next_tile(t_lo);
    if (t < ntiles) issue(t, 0);
    // One key step from LDS stage BUF and its KT chunks of 32 keys, both
    // compile-time indices: every LDS read of the step then has a constant
    // base, which goes into the instruction's offset field instead of an
    // address add per read (24 adds per chunk at d = 128).
    auto step = [&](auto BUF) {
        constexpr int buf = decltype(BUF)::value;
        const int tn = next_tile(t + 1);
        wait_copies();
        __syncthreads();
        if (tn < ntiles) issue(tn, buf ^ 1);
        static_for<KT>([&](auto KC) {
            constexpr int kc = decltype(KC)::value;
            const int kbase = t * BKT + 32 * kc;
            const T *Ks = k_lds[buf] + kc * Geo::TILE, *Vs = v_lds[buf] + kc * Geo::TILE;
            if (wq0 < N && kbase < kv_end && (!CAUSAL || kbase <= wq0 + 31)) {
                // S^T = K Q^T and dP^T = V dO^T: D[m = key][n = query].
                f32x16_t sacc = {}, dpacc = {};
#pragma unroll
                for (int ks = 0; ks < NQK; ++ks) {
                    const x8_t ka = *reinterpret_cast<const x8_t *>(Ks + (rbase ^ (ks << 4)));
                    const x8_t va = *reinterpret_cast<const x8_t *>(Vs + (rbase ^ (ks << 4)));
                    sacc = mfma(ka, qf[ks], sacc);
                    dpacc = mfma(va, dof[ks], dpacc);
                }
                const bool edge = (kbase + 32 > kv_len) || (CAUSAL && kbase + 31 > wq0);
                float ds[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = fast_exp2(fmaf(sacc[i], c, -lse2));
                    if (edge) {
                        const int kj = kbase + acc_row(i, lane);
                        const bool ok = kj < kv_len && (!CAUSAL || kj <= qrow);
                        p = ok ? p : 0.f;
                    }
                    ds[i] = p * (dpacc[i] - dl);
                }
                // dQ^T += K^T dS^T over the two 16-key chunks.
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    x8_t dsf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) dsf[j] = (T)ds[8 * h + j];
#pragma unroll
                    for (int mb = 0; mb < ND; ++mb) {
                        const x8_t ktr = read_tr8(Ks + h * 16 * D, trlo[mb], trhi[mb]);
                        dq[mb] = mfma(ktr, dsf, dq[mb]);
                    }
                }
            }
            // one chunk at a time: the fence keeps the compiler from
            // hoisting the next chunk's loads (which would spill)
            __builtin_amdgcn_sched_barrier(0);
        });
        t = tn;
    };
    while (t < ntiles) {
        step(IntTag<0>{});
        if (t >= ntiles) break;
        step(IntTag<1>{});
    }

    if (qrow < N && a.nsplit_q > 1) {
        // fp32 partial of this key-range split (before the scale)
        float *pq = a.part_q + ((int64_t)split * a.B * a.H * N) * D + head + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                f32x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = dq[mb][4 * gg + j];
                *reinterpret_cast<f32x4_t *>(pq + mb * 32 + 8 * gg + 4 * (lane / 32)) = w;
            }
    } else if (qrow < N) {
        const float scale = a.scale;
        T *dQ = reinterpret_cast<T *>(a.dq) + head + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = (T)(dq[mb][4 * gg + j] * scale);
                *reinterpret_cast<x4_t *>(dQ + mb * 32 + 8 * gg + 4 * (lane / 32)) = w;
            }
    }
}

template <class T, int D, bool CAUSAL>
hipError_t launch_bwd_impl(const BwdArgs &a, hipStream_t stream) {
    constexpr int NW = 4;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_delta<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkt = (a.N + 32 * NW - 1) / (32 * NW);
    // bwd_dkdv (d = 64 without the causal mask): 64 query rows per step, two
    // workgroups per CU (128 rows would spill)
    constexpr int QT = 2;
    const unsigned kgrid = (unsigned)(nkt * a.B * a.Hkv * a.nsplit);
    // d = 128: two 4-wave workgroups per CU (32 query rows per step, V read
    // from LDS) when the grid fills the CUs twice over; the two waves of a
    // SIMD then belong to different workgroups and their phases (products,
    // exponentials, transposed reads) overlap instead of meeting at one
    // barrier.  A causal grid of one round or less would pair each heavy
    // key block with a light one and leave the heavy one alone on its CU at
    // one wave per SIMD: the 8-wave pair kernel is faster there.
    if constexpr (D == 128) {
        if (kgrid >= 1024u || (!CAUSAL && kgrid >= 512u))
            hipLaunchKernelGGL((bwd_dkdv<T, D, NW, 1, CAUSAL, true>), dim3(kgrid), dim3(NW * 64), 0, stream, a);
        else
            hipLaunchKernelGGL((bwd_dkdv_pair<T, D, CAUSAL>), dim3(kgrid), dim3(512), 0, stream, a);
    } else if constexpr (CAUSAL) {
        hipLaunchKernelGGL((bwd_dkdv_pair<T, D, CAUSAL>), dim3(kgrid), dim3(512), 0, stream, a);
    } else {
        hipLaunchKernelGGL((bwd_dkdv<T, D, NW, QT, CAUSAL, false>), dim3(kgrid), dim3(NW * 64), 0, stream, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nsplit > 1) {
        const int64_t el = (int64_t)a.B * a.Hkv * a.N * D;
        hipLaunchKernelGGL((bwd_reduce<T>), dim3((unsigned)((el / 4 + 255) / 256)), dim3(256), 0, stream, a, el);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nqt = (a.N + 32 * NW - 1) / (32 * NW);
    constexpr int KT = 2;
    hipLaunchKernelGGL((bwd_dq<T, D, NW, KT, CAUSAL>), dim3((unsigned)(nqt * a.B * a.H * a.nsplit_q)),
                       dim3(NW * 64), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.nsplit_q == 1) return e;
    const int64_t el = (int64_t)a.B * a.H * a.N * D;
    hipLaunchKernelGGL((bwd_reduce_dq<T>), dim3((unsigned)((el / 4 + 255) / 256)), dim3(256), 0, stream, a, el);
    return hipGetLastError();
}

template <class T>
hipError_t launch_bwd_typed(const BwdArgs &a, int d, int causal, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_bwd_impl<T, 64, true>(a, stream) : launch_bwd_impl<T, 64, false>(a, stream);
    return causal ? launch_bwd_impl<T, 128, true>(a, stream) : launch_bwd_impl<T, 128, false>(a, stream);
}

}  // namespace

// Splits pay when a grid is too small for the GPU (one dK/dV workgroup per
// CU; few heads, few key/value heads, or short sequences).  For each of the
// dK/dV grid (B * H_kv * 128-key blocks) and the dQ grid (B * H * 128-row
// tiles): if it has fewer than 512 workgroups, the largest power of two up
// to 16 that keeps it within 1024.  Measured on B1 H2 N16384 causal: dK/dV
// split 4 and dQ split 4, 709 us; 8 and 4, 779 us; 16 and 4, 910 us; 8 and
// 8, 805 us; unsplit 1145 us.  Multi-query at 16K: 8 splits 3957 us, 16
// splits 4063 us, unsplit 10951 us.  Splitting a 512-workgroup grid made it
// slower.
static int pow2_split(int64_t base, int64_t cap) {
    if (base >= 512) return 1;
    int s = 1;
    while (s < 16 && base * s * 2 <= cap) s *= 2;
    return s;
}

// A causal grid of one round at two workgroups per CU (512 to 1023) with
// long heads (64 or more 128-key blocks) holds very unequal work: the
// heaviest key blocks see all query tiles, the lightest one.  Split in two
// it becomes two rounds of half-length items.  Measured (same box,
// alternating runs): B1 H4 N16384 d128 causal 1240 -> 1103 us, grouped
// heads B1 H16 Hkv4 N16384 3859 -> 3778 us; shorter heads (B2 H8 N4096, 32
// blocks) ran 6 % slower split and non-causal grids 4 % slower, hence both
// conditions.
static int long_causal_split(int64_t base, int blocks_per_head, bool causal) {
    return causal && base >= 512 && base < 1024 && blocks_per_head >= 64 ? 2 : 1;
}

int bwd_split(int B, int H, int Hkv, int N, bool causal) {
    if (B < 1 || H < 1 || Hkv < 1 || N < 1 || H % Hkv != 0) return 1;
    const int nb = (N + 127) / 128;
    const int64_t base = (int64_t)B * Hkv * nb;
    return max(pow2_split(base, 1024), long_causal_split(base, nb, causal));
}

int bwd_split_q(int B, int H, int N, bool causal) {
    if (B < 1 || H < 1 || N < 1) return 1;
    const int nb = (N + 127) / 128;
    const int64_t base = (int64_t)B * H * nb;
    return max(pow2_split(base, 1024), long_causal_split(base, nb, causal));
}

uint64_t bwd_workspace_bytes(int B, int H, int Hkv, int N, int d) {
    // the causal case splits at least as much as any other
    const int s = bwd_split(B, H, Hkv, N, true), sq = bwd_split_q(B, H, N, true);
    uint64_t bytes = 0;
    if (s > 1) bytes += (uint64_t)s * 2 * (uint64_t)B * Hkv * (uint64_t)N * d * sizeof(float);
    if (sq > 1) bytes += (uint64_t)sq * (uint64_t)B * H * (uint64_t)N * d * sizeof(float);
    return bytes;
}

hipError_t launch_bwd(const BwdArgs &a, int d, int causal, int f16, hipStream_t stream) {
    return f16 ? launch_bwd_typed<_Float16>(a, d, causal, stream) : launch_bwd_typed<__bf16>(a, d, causal, stream);
}

}  // namespace fa
