#pragma once
// Tile-study kernel of the exact attention forward (bf16 inputs, fp32
// accumulation) for gfx950: one template, instantiated for every tile shape
// by fa_fwd_bf16.hip (bf16 output) and fa_fwd_study_modes.hip (the other
// output modes of the deviation study).  Internal header.
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
#include <type_traits>

#include "fa_bf16_tiles.h"

namespace fa {
namespace {

// MODE of the deviation study: kModeBf16 writes O rounded to bf16 (the
// library's bf16 path); kModeF32Out writes O in fp32, before its final
// rounding; kModeAcc16 rounds the running output to bf16 after every key
// tile (a model of an implementation that holds its partial output in the
// input precision between tiles, so the output is rounded once per
// rescaling step) and writes it rounded to bf16.
constexpr int kModeBf16 = 0, kModeF32Out = 1, kModeAcc16 = 2;

template <int D, int BC, int MF, int NW, bool CAUSAL, int MODE = kModeBf16>
__global__ __launch_bounds__(NW * 64, (MF == 32 && NW == 4) ? 2 : 1) void fwd_bf16_kernel(FwdArgs a) {
    using OT = typename std::conditional<MODE == kModeF32Out, float, __bf16>::type;
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
    tile_of_block(nqt, CAUSAL, 1, &bh, &qt);
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t kvhead = (int64_t)kv_head_of(bh, a) * N * D;
    const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
    const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + kvhead;
    const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + kvhead;
    OT *O = reinterpret_cast<OT *>(a.o) + head;

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
    // Largest active tile <= t (-1 if none): the same scan downwards.
    auto prev_tile = [&](int t) {
        if (!mrow || t < 0) return t;
        int blk = (t * BC) >> 7;
        const int blk0 = blk;
        while (blk >= 0) {
            const int ch = blk >> 6;
            if (ch != mask_chunk) {
                const int idx = ch * 64 + lane;
                mask_bits = __builtin_amdgcn_ballot_w64(idx < a.nkb && mrow[idx] != 0);
                mask_chunk = ch;
            }
            const int bit = blk & 63;
            const uint64_t below = bit == 63 ? ~0ull : ((1ull << (bit + 1)) - 1);
            const uint64_t rest = mask_bits & below;
            if (rest) {
                blk = ch * 64 + 63 - __builtin_clzll(rest);
                break;
            }
            blk = ch * 64 - 1;
        }
        if (blk == blk0) return t;
        return blk < 0 ? -1 : min(ntiles - 1, blk * (128 / BC) + 128 / BC - 1);
    };
    // Key tiles are visited in ascending order, or descending, or shuffled
    // when asked (the tile-order axis of the deviation study).  The loop
    // walks a cursor; tile_at maps it to a key tile.  Shuffled: cursor i is
    // the i-th visit and goes to tile (sa * i + sb) mod ntiles, where sa is
    // the smallest integer >= round(0.618 * ntiles) coprime to ntiles (so
    // the map is a permutation) and sb = ntiles / 2; tiles the block mask
    // turns off are passed over.
    const bool descending = a.order == 1, shuffled = a.order == 2;
    int sa = 1;
    const int sb = ntiles / 2;
    if (shuffled && ntiles > 1) {
        sa = max(1, (ntiles * 618 + 500) / 1000);
        for (;; ++sa) {
            int x = sa, y = ntiles;
            while (y) {
                const int r = x % y;
                x = y;
                y = r;
            }
            if (x == 1) break;
        }
    }
    auto tile_at = [&](int cur) { return shuffled ? (int)(((int64_t)sa * cur + sb) % ntiles) : cur; };
    auto next_shuffled = [&](int cur) {
        if (mrow)
            while (cur < ntiles && mrow[(tile_at(cur) * BC) >> 7] == 0) ++cur;
        return cur;
    };
    auto first_tile = [&]() {
        return shuffled ? next_shuffled(0) : descending ? prev_tile(ntiles - 1) : next_tile(0);
    };
    auto following = [&](int t) {
        return shuffled ? next_shuffled(t + 1) : descending ? prev_tile(t - 1) : next_tile(t + 1);
    };
    auto valid = [&](int t) { return t >= 0 && t < ntiles; };

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
        if constexpr (MODE == kModeAcc16) {
            // The partial output leaves the tile in bf16 (round to nearest even).
#pragma unroll
            for (int mb = 0; mb < C::ND; ++mb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) o[mb][i] = (float)(__bf16)o[mb][i];
        }
    };

    // Double-buffered main loop, unrolled by two so each half touches fixed
    // LDS buffers: wait for tile t, barrier (all waves are also done with the
    // other buffer), start copying the next tile into the other buffer,
    // compute tile t.
    int t = first_tile();
    if (valid(t)) copy_tile<C, D>(K, V, k_lds0, v_lds0, tile_at(t) * BC, klast, wave, lane);
    while (valid(t)) {
        int tn = following(t);
        wait_copies();
        __syncthreads();
        if (valid(tn)) copy_tile<C, D>(K, V, k_lds1, v_lds1, tile_at(tn) * BC, klast, wave, lane);
        compute(tile_at(t), k_lds0, v_lds0);
        t = tn;
        if (!valid(t)) break;
        tn = following(t);
        wait_copies();
        __syncthreads();
        if (valid(tn)) copy_tile<C, D>(K, V, k_lds0, v_lds0, tile_at(tn) * BC, klast, wave, lane);
        compute(tile_at(t), k_lds1, v_lds1);
        t = tn;
    }

    // Epilogue: normalise, round to bf16 once (or keep fp32), write O and LSE.
    const float l_tot = group_sum<MF>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        OT *orow = O + (int64_t)qrow * D;
        if constexpr (sizeof(OT) == 4) {
#pragma unroll
            for (int mb = 0; mb < C::ND; ++mb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) orow[mb * MF + F::row(i, lane)] = o[mb][i] * inv;
        } else if constexpr (MF == 32) {
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

template <int D, int BC, int MF, int NW, bool CAUSAL, int MODE = kModeBf16>
hipError_t launch_bf16(const FwdArgs &a, hipStream_t stream) {
    using C = Cfg<D, BC, MF, NW>;
    const int nqt = (a.N + C::BR - 1) / C::BR;
    const dim3 grid((unsigned)(nqt * a.B * a.H));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, MF, NW, CAUSAL, MODE>), grid, dim3(C::NT), 0, stream, a);
    return hipGetLastError();
}

// MFMA edge for a (Br, Bc) tile: 16 when either side is 16, else 32.
template <int BR, int BC>
struct Pick {
    static constexpr int MF = (BR == 16 || BC == 16) ? 16 : 32;
    static constexpr int NW = BR / MF;
};

}  // namespace
}  // namespace fa
