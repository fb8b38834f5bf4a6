// Exact attention forward, bf16 in/out, fp32 accumulation, for gfx950.
//
// The method (page "FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", ai-paper-library, Summary and Method; page
// "What is FlashAttention?", unite.ai, five-stage operating map): Q, K and V
// are cut into tiles; a tile of Q stays on chip while K/V tiles stream
// through; each K tile gives local scores that update a running row maximum
// and running row sum; the output is accumulated on chip and the N x N score
// matrix is never written out.  Disallowed keys get a -inf logit before the
// softmax (page "Ch.04 Attention optimisation: FlashAttention and sparse
// attention", mdooai.com, sparse-attention rule); whole tiles that are
// disallowed are skipped, which is the block-sparse extension of the
// FlashAttention summary page.
//
// Running statistics for one query row over key tiles 0, 1, ... (base 2,
// logits pre-multiplied by c = scale*log2(e)):
//   m'  = max(m, max_j c*s_j)          alpha = 2^(m - m')
//   p_j = 2^(c*s_j - m')               l'    = alpha*l + sum_j p_j
//   O'  = alpha*O + sum_j bf16(p_j) v_j
// and at the end O/l, LSE = (m + log2 l) * ln 2.  l sums the fp32 p_j; the
// bf16 rounding of p_j is used only as the operand of the P V product.
// When no row of a wave changes its maximum, alpha is exactly 1 and the
// rescale of O is skipped (a bit-identical no-op).
//
// gfx950 mapping.
//  * One wavefront owns MF query rows (MF = 32, or 16 for the small tiles of
//    the tile-size study); a workgroup of NW waves owns BR = MF*NW rows.
//  * Scores are computed transposed, S^T = K Q^T, on bf16 matrix-core
//    instructions (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_16x16x32_bf16), so
//    each lane holds scores of a single query row: row max and row sum are
//    in-lane reductions plus v_permlane32_swap (and v_permlane16_swap).
//  * The output is accumulated transposed too, O^T += V^T P^T, which takes P
//    straight from the score registers as the B operand (no LDS round trip).
//  * Q fragments live in VGPRs for the whole kernel.
//  * K and V tiles are copied from HBM straight into LDS with
//    global_load_lds_dwordx4 (no VGPR staging), double-buffered: the copy of
//    tile j+1 is in flight while tile j is computed.  Both are stored
//    row-major with an XOR swizzle of the 16-byte column slots.  K fragments
//    are 16-byte LDS reads; V^T fragments come from ds_read_b64_tr_b16, which
//    hands each lane one column of a 4-row block (the transpose the PV
//    product needs).  The swizzles make both read patterns bank-conflict
//    free.
#include "fa_common.h"

namespace fa {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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

// V^T fragment via ds_read_b64_tr_b16: within each 16-lane group, lane i
// points at row (i/4), columns 4*(i%4)..+3 of a 4-row x 16-column block and
// receives column i of that block (4 consecutive rows).
template <class C, int D>
__device__ __forceinline__ s16x4_t read_vt(const __bf16 *Vs, int row, int col) {
    const int off = row * D + (((col >> 3) ^ C::zv(row)) << 3) + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(Vs + off));
}

template <int D, int BC, int MF, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (MF == 32 && NW == 4) ? 2 : 1) void fwd_bf16_kernel(FwdArgs a) {
    using C = Cfg<D, BC, MF, NW>;
    using F = Frag<MF>;
    using acc_t = typename F::acc_t;

    // Two stages of [K tile | V tile]; one array so that every LDS address
    // of the second stage is the first stage's plus an immediate offset.
    __shared__ __attribute__((aligned(1024))) __bf16 smem[4 * C::TILE];
    __bf16 *const k_lds0 = smem;
    __bf16 *const v_lds0 = smem + C::TILE;
    __bf16 *const k_lds1 = smem + 2 * C::TILE;
    __bf16 *const v_lds1 = smem + 3 * C::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nqt = (N + C::BR - 1) / C::BR;
    int bh, qt;
    tile_of_block(nqt, CAUSAL, &bh, &qt);
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
    const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
    const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;
    __bf16 *O = reinterpret_cast<__bf16 *>(a.o) + head;

    const int q0 = qt * C::BR;       // first query row of the workgroup
    const int wq0 = q0 + wave * MF;  // first query row of this wave
    const int qrow = wq0 + lane % MF;

    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + C::BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    const int klast = kv_len - 1;
    // Block-sparse skipping: the mask row of this workgroup's query block is
    // scanned 64 key blocks at a time into a wave-uniform bit mask.
    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;
    int mask_chunk = -1;
    uint64_t mask_bits = 0;
    auto next_tile = [&](int t) {
        if (!mrow || t >= ntiles) return t;
        int blk = (t * BC) >> 7;
        const int blk0 = blk;
        while (blk < a.nkb) {
            const int ch = blk >> 6;
            if (ch != mask_chunk) {
                const int idx = ch * 64 + lane;
                mask_bits = __builtin_amdgcn_ballot_w64(idx < a.nkb && mrow[idx] != 0);
                mask_chunk = ch;
            }
            const uint64_t rest = mask_bits >> (blk & 63);
            if (rest) {
                blk += __builtin_ctzll(rest);
                break;
            }
            blk = (ch + 1) << 6;
        }
        if (blk == blk0) return t;
        return blk >= a.nkb ? ntiles : min(ntiles, blk * (128 / BC));
    };

    // Q fragments (B operand of S^T = K Q^T), resident for the whole kernel.
    // A negative scale is folded into Q (sign flip, exact) so that c >= 0.
    const float c = scale_factor(a.scale_log2);
    const uint32_t sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8_t qf[C::NQK];
#pragma unroll
    for (int ks = 0; ks < C::NQK; ++ks) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (qrow < N)
            x = *reinterpret_cast<const u32x4_t *>(Q + (int64_t)qrow * D + ks * F::KQK + 8 * (lane / MF));
        x ^= sign;
        qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }

    acc_t o[C::ND];
#pragma unroll
    for (int mb = 0; mb < C::ND; ++mb)
#pragma unroll
        for (int i = 0; i < F::ACC; ++i) o[mb][i] = 0.f;
    float m = kNegInf;  // running max of c*s for this lane's query (base 2)
    float l = 0.f;      // running sum of p over this lane's keys

    auto compute = [&](int t, const __bf16 *Ks, const __bf16 *Vs) {
        const int kbase = t * BC;
        if (wq0 >= N) return;
        if (CAUSAL && kbase > wq0 + MF - 1) return;  // whole tile above the diagonal

        // S^T for this tile: NKB blocks of MF keys x MF queries.
        acc_t s[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) s[kb][i] = 0.f;
            const int r = kb * MF + lane % MF;
            const __bf16 *kr = Ks + r * D;
            const int z = C::zk(r);
#pragma unroll
            for (int ks = 0; ks < C::NQK; ++ks) {
                const int slot = (ks * F::KQK + 8 * (lane / MF)) >> 3;
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(kr + ((slot ^ z) << 3));
                s[kb] = F::qk(ka, qf[ks], s[kb]);
            }
        }

        // Elementwise mask only on tiles that cross the diagonal or the end
        // of the valid keys.
        const bool edge = (kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0);
        float mx = kNegInf;
        if (edge) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) {
                    const int key = kbase + kb * MF + F::row(i, lane);
                    const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                    s[kb][i] = ok ? s[kb][i] : kNegInf;
                    mx = fmaxf(mx, s[kb][i]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) mx = fmaxf(mx, s[kb][i]);
        }
        mx = group_max<MF>(mx);
        const float m_tile = mx == kNegInf ? kNegInf : mx * c;
        const float m_new = fmaxf(m, m_tile);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        const float neg_m = -m_use;

        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) {
                const float p = fast_exp2(fmaf(s[kb][i], c, neg_m));  // exp2(-inf) = 0
                s[kb][i] = p;
                rs += p;
            }
        l = fmaf(l, alpha, rs);
        if (wave_any(m_use != m)) {
#pragma unroll
            for (int mb = 0; mb < C::ND; ++mb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) o[mb][i] *= alpha;
        }
        m = m_new;

        // O^T += V^T P^T.
        const int g = lane >> 4, li = lane & 15;
        if constexpr (MF == 32) {
            // 16-key step h of block kb: the lower half-wave holds keys
            // {0-3, 8-11}, the upper half-wave keys {4-7, 12-15} of the step
            // (score layout); V^T takes them as two 4-row transposed reads.
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x8_t pf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[kb][8 * h + j];
                    const int row = kb * 32 + h * 16 + 4 * (g >> 1) + (li >> 2);
                    const int col = 16 * (g & 1) + 4 * (li & 3);
#pragma unroll
                    for (int mb = 0; mb < C::ND; ++mb) {
                        const s16x4_t lo = read_vt<C, D>(Vs, row, mb * 32 + col);
                        const s16x4_t hi = read_vt<C, D>(Vs, row + 8, mb * 32 + col);
                        const bf16x8_t va = __builtin_bit_cast(
                            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, o[mb], 0, 0, 0);
                    }
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                bf16x4_t pf;
#pragma unroll
                for (int j = 0; j < 4; ++j) pf[j] = (__bf16)s[kb][j];
                const int row = kb * 16 + 4 * g + (li >> 2);
                const int col = 4 * (li & 3);
#pragma unroll
                for (int mb = 0; mb < C::ND; ++mb) {
                    const s16x4_t va = read_vt<C, D>(Vs, row, mb * 16 + col);
                    o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        va, __builtin_bit_cast(i16x4_t, pf), o[mb], 0, 0, 0);
                }
            }
        }
    };

    // Double-buffered main loop, unrolled by two so each half touches fixed
    // LDS buffers: wait for tile t, barrier (all waves are also done with the
    // other buffer), start copying the next tile into the other buffer,
    // compute tile t.
    int t = next_tile(0);
    if (t < ntiles) copy_tile<C, D>(K, V, k_lds0, v_lds0, t * BC, klast, wave, lane);
    while (t < ntiles) {
        int tn = next_tile(t + 1);
        wait_copies();
        __syncthreads();
        if (tn < ntiles) copy_tile<C, D>(K, V, k_lds1, v_lds1, tn * BC, klast, wave, lane);
        compute(t, k_lds0, v_lds0);
        t = tn;
        if (t >= ntiles) break;
        tn = next_tile(t + 1);
        wait_copies();
        __syncthreads();
        if (tn < ntiles) copy_tile<C, D>(K, V, k_lds0, v_lds0, tn * BC, klast, wave, lane);
        compute(t, k_lds1, v_lds1);
        t = tn;
    }

    // Epilogue: normalise, round to bf16 once, write O and LSE.
    const float l_tot = group_sum<MF>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        __bf16 *orow = O + (int64_t)qrow * D;
        if constexpr (MF == 32) {
#pragma unroll
            for (int mb = 0; mb < C::ND; ++mb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4_t w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[mb][4 * g + j] * inv);
                    *reinterpret_cast<bf16x4_t *>(orow + mb * 32 + 8 * g + 4 * (lane / 32)) = w;
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < C::ND; ++mb) {
                bf16x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[mb][j] * inv);
                *reinterpret_cast<bf16x4_t *>(orow + mb * 16 + 4 * (lane / 16)) = w;
            }
        }
        if (a.lse && lane < MF)
            a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

// ----------------------------------------------------------------------------
// Tuned kernel (BR = 128, BC = 64, MF = 32): software-pipelined over key
// tiles.  While the softmax of tile j runs on the VALU, the matrix cores
// already compute the scores of tile j+1; while they accumulate P_j V_j the
// VALU sums the row, packs P to bf16 and rescales O.  K is therefore staged
// one tile ahead of V: at iteration j the LDS holds K_{j+1}, V_j and receives
// K_{j+2}, V_{j+1}.  The interleaving is imposed with
// __builtin_amdgcn_sched_group_barrier (groups of matrix-core, LDS-read and
// VALU instructions), so one wave keeps both pipes busy on its own.

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x2, kSgMfma = 0x8, kSgDsRead = 0x100;

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_pipe(FwdArgs a) {
    constexpr int BC = 64, MF = 32, NW = 4;
    using C = Cfg<D, BC, MF, NW>;
    using acc_t = f32x16_t;
    constexpr int NQK = C::NQK, ND = C::ND;
    constexpr int ROUNDS = C::NCOPY / NW;  // copy instructions per wave per tensor
    static_assert(C::NCOPY % NW == 0, "copies must split evenly over the waves");
    constexpr int QK_MFMA = 2 * NQK;       // per tile
    constexpr int PV_MFMA = 4 * ND;        // per tile

    // [K stage 0 | K stage 1 | V stage 0 | V stage 1]
    __shared__ __attribute__((aligned(1024))) __bf16 smem[4 * C::TILE];
    __bf16 *const K0 = smem;
    __bf16 *const K1 = smem + C::TILE;
    __bf16 *const V0 = smem + 2 * C::TILE;
    __bf16 *const V1 = smem + 3 * C::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nqt = (N + C::BR - 1) / C::BR;
    int bh, qt;
    tile_of_block(nqt, CAUSAL, &bh, &qt);
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
    const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
    const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;
    __bf16 *O = reinterpret_cast<__bf16 *>(a.o) + head;

    const int q0 = qt * C::BR;
    const int wq0 = q0 + wave * MF;
    const int qrow = wq0 + lane % MF;
    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + C::BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    const int klast = kv_len - 1;
    // Tiles this wave computes form a prefix of the workgroup's sequence.
    const int wlast = wq0 >= N ? -1 : (CAUSAL ? (wq0 + MF - 1) / BC : ntiles);
    auto active = [&](int t) { return t < ntiles && t <= wlast; };

    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;
    int mask_chunk = -1;
    uint64_t mask_bits = 0;
    auto next_tile = [&](int t) {
        if (!mrow || t >= ntiles) return t;
        int blk = (t * BC) >> 7;
        const int blk0 = blk;
        while (blk < a.nkb) {
            const int ch = blk >> 6;
            if (ch != mask_chunk) {
                const int idx = ch * 64 + lane;
                mask_bits = __builtin_amdgcn_ballot_w64(idx < a.nkb && mrow[idx] != 0);
                mask_chunk = ch;
            }
            const uint64_t rest = mask_bits >> (blk & 63);
            if (rest) {
                blk += __builtin_ctzll(rest);
                break;
            }
            blk = (ch + 1) << 6;
        }
        if (blk == blk0) return t;
        return blk >= a.nkb ? ntiles : min(ntiles, blk * (128 / BC));
    };

    // Per-lane byte offsets of this wave's copy chunks inside a tile (tile
    // row 0 = key kbase); the tile base itself is a wave-uniform address.
    uint32_t koff[ROUNDS], voff[ROUNDS];
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
        const int ci = (wave + NW * i) * 64 + lane;
        const int r = ci / C::SLOTS, p = ci % C::SLOTS;
        koff[i] = (uint32_t)(r * D + ((p ^ C::zk(r)) << 3)) * 2u;
        voff[i] = (uint32_t)(r * D + ((p ^ C::zv(r)) << 3)) * 2u;
    }
    auto copy = [&](const __bf16 *G, __bf16 *dst, const uint32_t(&off)[ROUNDS], int t) {
        const int kbase = t * BC;
        const char *base = reinterpret_cast<const char *>(G + (int64_t)kbase * D);
        if (kbase + BC <= kv_len) {
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16 *>(base + off[i]),
                    (__attribute__((address_space(3))) void *)(dst + (wave + NW * i) * 512), 16, 0, 0);
        } else {
            // Last, partial tile: rows past the last valid key re-read it.
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) {
                const int r = ((wave + NW * i) * 64 + lane) / C::SLOTS;
                const int excess = max(0, kbase + r - klast);
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const __bf16 *>(base + off[i] - (uint32_t)(excess * D * 2)),
                    (__attribute__((address_space(3))) void *)(dst + (wave + NW * i) * 512), 16, 0, 0);
            }
        }
    };

    // Q fragments, sign-folded so that c >= 0.
    const float c = scale_factor(a.scale_log2);
    const uint32_t sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8_t qf[NQK];
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (qrow < N)
            x = *reinterpret_cast<const u32x4_t *>(Q + (int64_t)qrow * D + ks * 16 + 8 * (lane / 32));
        x ^= sign;
        qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }

    // LDS read offsets (elements): K fragment ks of a 32-key block, and the
    // transposed V fragment of output block mb.
    int kaddr[NQK];
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) {
        const int r = lane % 32;
        kaddr[ks] = r * D + ((((2 * ks + lane / 32)) ^ C::zk(r)) << 3);
    }
    const int g = lane >> 4, li = lane & 15;
    int vaddr[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb) {
        const int row = 4 * (g >> 1) + (li >> 2);
        const int col = mb * 32 + 16 * (g & 1) + 4 * (li & 3);
        vaddr[mb] = row * D + (((col >> 3) ^ C::zv(row)) << 3) + (col & 7);
    }

    acc_t o[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
    float m = kNegInf, l = 0.f;
    // Scores ping-pong between sA and sB across the two halves of the
    // unrolled main loop (no register copies between tiles).
    acc_t sA[2], sB[2];

    auto qk_plain = [&](acc_t (&dst)[2], const __bf16 *Ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) dst[kb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(Ks + kb * 32 * D + kaddr[ks]);
                dst[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], dst[kb], 0, 0, 0);
            }
    };

    // One pipeline step: softmax + PV of tile t (scores in s), and the
    // scores of the next tile (from Kn) into sn.  The QK products are issued
    // even when this wave has no next tile (the result is then unused): a
    // branch would split the scheduling region that interleaves the pipes.
    auto step = [&](int t, acc_t (&s)[2], acc_t (&sn)[2], const __bf16 *Kn, const __bf16 *Vs) {
        const int kbase = t * BC;
        const bool edge = (kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0);
        if (edge) {
            // Keep this a branch: the compiler would otherwise if-convert it
            // into per-element selects on every tile.
            asm volatile("" ::);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + kb * 32 + Frag<32>::row(i, lane);
                    const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                    s[kb][i] = ok ? s[kb][i] : kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = group_max<32>(mx);
        const float m_tile = mx == kNegInf ? kNegInf : mx * c;
        const float m_new = fmaxf(m, m_tile);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        const float neg_m = -m_use;
        m = m_new;

        // Phase A: QK of the next tile on the matrix cores || exponentials of
        // this tile on the VALU (masked keys: exp2(-inf) = 0).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sn[kb][i] = 0.f;
        constexpr int PER = 32 / QK_MFMA;  // exponentials per QK instruction
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(Kn + kb * 32 * D + kaddr[ks]);
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sn[kb], 0, 0, 0);
#pragma unroll
                for (int e = 0; e < PER; ++e) {
                    const int idx = (ks * 2 + kb) * PER + e;
                    s[idx >> 4][idx & 15] = fast_exp2(fmaf(s[idx >> 4][idx & 15], c, neg_m));
                }
            }
        // K reads run three instructions ahead of their products.
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 3, 0);
#pragma unroll
        for (int i = 0; i < QK_MFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            if (i + 3 < QK_MFMA) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 2 * PER, 0);
        }

        // Phase B: O^T = alpha*O^T + V^T P^T on the matrix cores || row sum,
        // bf16 packing and the rescale on the VALU.
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8_t pf;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pf[j] = (__bf16)s[kb][8 * h + j];
                    rs += s[kb][8 * h + j];
                }
#pragma unroll
                for (int mb = 0; mb < ND; ++mb) {
                    if (kb == 0 && h == 0) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
                    }
                    const __bf16 *vp = Vs + (kb * 32 + h * 16) * D + vaddr[mb];
                    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
                    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vp + 8 * D));
                    const bf16x8_t va = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, o[mb], 0, 0, 0);
                }
            }
        constexpr int VALU_B = (16 * ND + 32 + 16) / PV_MFMA + 1;
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 1);
#pragma unroll
        for (int i = 0; i < PV_MFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
            if (i + 2 < PV_MFMA) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 1);
            __builtin_amdgcn_sched_group_barrier(kSgValu, VALU_B, 1);
        }
        l = fmaf(l, alpha, rs);
    };

    int t = next_tile(0);
    int tn = next_tile(t + 1);
    if (t < ntiles) {
        copy(K, K0, koff, t);
        copy(V, V0, voff, t);
    }
    if (tn < ntiles) copy(K, K1, koff, tn);
    wait_copies();
    __syncthreads();
    if (active(t)) qk_plain(sA, K0);

    // Stage parity p: K_{tn} is read from K[1-p], V_t from V[p]; K_{tnn} is
    // copied into K[p] and V_{tn} into V[1-p].
    while (t < ntiles) {
        int tnn = next_tile(tn + 1);
        wait_copies();
        __syncthreads();
        if (tnn < ntiles) copy(K, K0, koff, tnn);
        if (tn < ntiles) copy(V, V1, voff, tn);
        if (active(t)) step(t, sA, sB, K1, V0);
        t = tn;
        tn = tnn;
        if (t >= ntiles) break;
        tnn = next_tile(tn + 1);
        wait_copies();
        __syncthreads();
        if (tnn < ntiles) copy(K, K1, koff, tnn);
        if (tn < ntiles) copy(V, V0, voff, tn);
        if (active(t)) step(t, sB, sA, K0, V1);
        t = tn;
        tn = tnn;
    }

    const float l_tot = group_sum<32>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        __bf16 *orow = O + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                bf16x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[mb][4 * gg + j] * inv);
                *reinterpret_cast<bf16x4_t *>(orow + mb * 32 + 8 * gg + 4 * (lane / 32)) = w;
            }
        if (a.lse && lane < 32)
            a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_pipe(const FwdArgs &a, hipStream_t stream) {
    const int nqt = (a.N + 127) / 128;
    hipLaunchKernelGGL((fwd_bf16_pipe<D, CAUSAL>), dim3((unsigned)(nqt * a.B * a.H)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int BC, int MF, int NW, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs &a, hipStream_t stream) {
    using C = Cfg<D, BC, MF, NW>;
    const int nqt = (a.N + C::BR - 1) / C::BR;
    const dim3 grid((unsigned)(nqt * a.B * a.H));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, MF, NW, CAUSAL>), grid, dim3(C::NT), 0, stream, a);
    return hipGetLastError();
}

// MFMA edge for a (Br, Bc) tile: 16 when either side is 16, else 32.
template <int BR, int BC>
struct Pick {
    static constexpr int MF = (BR == 16 || BC == 16) ? 16 : 32;
    static constexpr int NW = BR / MF;
};

#define FA_BF16(D, BR, BC, CAUSAL)                                             \
    Instance {                                                                 \
        D, CAUSAL, BR, BC,                                                     \
            &launch_bf16<D, BC, Pick<BR, BC>::MF, Pick<BR, BC>::NW, CAUSAL>    \
    }
#define FA_BF16_BOTH(D, BR, BC) FA_BF16(D, BR, BC, false), FA_BF16(D, BR, BC, true)
#define FA_BF16_ROW(D, BR) \
    FA_BF16_BOTH(D, BR, 16), FA_BF16_BOTH(D, BR, 32), FA_BF16_BOTH(D, BR, 64), FA_BF16_BOTH(D, BR, 128)

}  // namespace

const Instance *bf16_instances() {
    static const Instance table[] = {
        // tuned, software-pipelined shape (first match wins)
        Instance{64, 0, 128, 64, &launch_pipe<64, false>},
        Instance{64, 1, 128, 64, &launch_pipe<64, true>},
        Instance{128, 0, 128, 64, &launch_pipe<128, false>},
        Instance{128, 1, 128, 64, &launch_pipe<128, true>},
        // tile-size study shapes
        FA_BF16_ROW(128, 16),
        FA_BF16_ROW(128, 32),
        FA_BF16_BOTH(128, 64, 16), FA_BF16_BOTH(128, 64, 32), FA_BF16_BOTH(128, 64, 64), FA_BF16_BOTH(128, 64, 128),
        FA_BF16_BOTH(128, 128, 16), FA_BF16_BOTH(128, 128, 32), FA_BF16_BOTH(128, 128, 128),
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

void bf16_default_tile(int d, int *br, int *bc) {
    (void)d;
    *br = 128;
    *bc = 64;
}

}  // namespace fa
