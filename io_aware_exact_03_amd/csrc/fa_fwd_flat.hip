// Exact-attention forward for gfx950 at four workgroups per CU (d = 64).
//
// The same method, recurrence and arithmetic as fwd_pipe (fa_fwd_bf16_pipe.hip:
// tiled exact attention with a running softmax, page "FlashAttention: Fast
// and Memory-Efficient Exact Attention with IO-Awareness", ai-paper-library,
// Summary and Method; five-stage map of "What is FlashAttention?", unite.ai),
// with the per-row operations in the same order, so the two give identical
// bits.  What differs is how the work is overlapped:
//
//  * fwd_pipe keeps two tiles' scores in registers (the next tile's S = K Q^T
//    runs on the matrix cores while this tile's softmax runs on the VALU),
//    which needs over 128 VGPRs at d = 64: three workgroups per CU.
//  * fwd_flat computes one tile at a time (scores, softmax, P V) in at most
//    128 VGPRs, so four workgroups (four waves per SIMD) are resident per CU
//    and the overlap of matrix-core and VALU work comes from the other waves
//    of the SIMD.  With 1024 resident workgroups a grid of 1024 or 2048
//    query tiles (B = 4, H = 16, N = 4096 block-sparse; B = 16, H = 16,
//    N = 512) runs in whole rounds instead of 1.33 or 2.67.
//
// K and V tiles still move HBM -> LDS with global_load_lds_dwordx4 through a
// ring of NSTAGE stages (two: the copy of tile t+1 is in flight while tile t
// is computed), with the stage barrier and swizzles of fwd_pipe.  Measured
// on one MI355X against fwd_pipe, bit-identical outputs: block-sparse
// B4 H16 N4096 3-7 % faster, the other d = 64 shapes 1-4 %.  At d = 128 the
// output accumulator alone takes 64 registers per lane and a one-tile kernel
// would not fit four waves per SIMD, so fwd_pipe stays there.
#include "fa_bf16_tiles.h"

namespace fa {
namespace {

// NSTAGE: depth of the K/V ring (the copies of a tile are issued NSTAGE - 1
// tiles before it is computed); OCC: workgroups resident per CU.
template <class T, int D, int BC, int NW, bool CAUSAL, int NSTAGE, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void fwd_flat(FwdArgs a) {
    using E = Elem<T>;
    using x8_t = typename E::x8;
    using x4_t = typename E::x4;
    constexpr int QW = 32, BR = QW * NW, NKB = BC / 32;
    using C = Cfg<D, BC, 32, NW>;
    using acc_t = f32x16_t;
    constexpr int NQK = C::NQK, ND = C::ND;
    constexpr int ROUNDS = C::NCOPY / NW;  // copy instructions per wave per tensor
    static_assert(C::NCOPY % NW == 0, "copies must split evenly over the waves");
    constexpr int NF = 2 * NKB;            // 8-score P fragments per tile

    constexpr int P = NSTAGE - 1;  // tiles of lookahead of the copies
    static_assert(P >= 1 && P <= 2, "2 or 3 stages");
    // Stage s: K tile at ring + 2*s*TILE, V tile right after it.
    __shared__ __attribute__((aligned(1024))) T ring[2 * NSTAGE * C::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nqt = (N + BR - 1) / BR;
    int bh, qt;
    tile_of_block(nqt, CAUSAL, OCC, &bh, &qt, !CAUSAL && a.key_len ? a.group * nqt : 0);
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t kvhead = (int64_t)kv_head_of(bh, a) * N * D;
    const T *Q = reinterpret_cast<const T *>(a.q) + head;
    const T *K = reinterpret_cast<const T *>(a.k) + kvhead;
    const T *V = reinterpret_cast<const T *>(a.v) + kvhead;
    T *O = reinterpret_cast<T *>(a.o) + head;

    const int q0 = qt * BR;
    const int wq0 = q0 + wave * QW;
    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    const int klast = kv_len - 1;
    // Tiles this wave computes form a prefix of the workgroup's sequence.
    const int wlast = wq0 >= N ? -1 : (CAUSAL ? (wq0 + QW - 1) / BC : ntiles);

    // Block-sparse skipping (BR = 128: the workgroup's rows are one query
    // block): the mask row is scanned 64 key blocks at a time into a
    // wave-uniform bit mask.
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

    // Per-lane byte offsets of this wave's copy chunks inside a tile.
    uint32_t koff[ROUNDS], voff[ROUNDS];
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
        const int ci = (wave + NW * i) * 64 + lane;
        const int r = ci / C::SLOTS, p = ci % C::SLOTS;
        koff[i] = (uint32_t)(r * D + ((p ^ C::zk(r)) << 3)) * 2u;
        voff[i] = (uint32_t)(r * D + ((p ^ C::zv(r)) << 3)) * 2u;
    }
    auto copy = [&](const T *G, T *dst, const uint32_t(&off)[ROUNDS], int t) {
        const int kbase = t * BC;
        const char *base = reinterpret_cast<const char *>(G + (int64_t)kbase * D);
        if (kbase + BC <= kv_len) {
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) lds_copy16(base, off[i], dst + (wave + NW * i) * 512);
        } else {
            // Last, partial tile: rows past the last valid key re-read it.
            // (The empty asm keeps this address arithmetic inside the
            // branch: hoisted, every full tile paid for it.)
            int over = kbase - klast;
            asm volatile("" : "+s"(over));
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) {
                const int r = ((wave + NW * i) * 64 + lane) / C::SLOTS;
                const int excess = max(0, over + r);
                lds_copy16(base, off[i] - (uint32_t)(excess * D * 2), dst + (wave + NW * i) * 512);
            }
        }
    };

    // Prologue: mask chunk, Q rows, then the first tile's copies; the Q
    // values are used only after the copies have landed.
    const int qrow = wq0 + lane % 32;
    uint8_t mask_pre = 0;
    if (mrow) mask_pre = mrow[min(lane, a.nkb - 1)];
    u32x4_t qraw[NQK];
    {
        const T *qsrc = Q + (int64_t)min(qrow, N - 1) * D + 8 * (lane / 32);
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qraw[ks] = *reinterpret_cast<const u32x4_t *>(qsrc + ks * 16);
    }
    if (mrow) {
        uint32_t mv = mask_pre;
        asm volatile("" : "+v"(mv)::"memory");
        mask_bits = __builtin_amdgcn_ballot_w64(lane < a.nkb && mv != 0);
        mask_chunk = 0;
    }
    // Issue priority from the key tiles the workgroup has left (non-causal
    // grids only): level min(3, 4 * left / scale), scale = the longest item
    // the grid can hold (N / BC tiles), or the item's own tile count under a
    // block mask (counted from the first 256 mask blocks).  By default a
    // SIMD favours its oldest wave: of four equal items started together on
    // a CU the first ends after ~60 % of the time the last one takes, the
    // next round's items start and end staggered the same way, and the CU
    // ends with one or two items left, too few to keep the VALU issue port
    // busy.  With the priority the items progress together.  Measured on
    // MI355X, bit-identical outputs: block-sparse B4 H16 N4096 -2.2 %,
    // key-padded B16 H16 N512 -2.4 %, B1 H16 N16384 d = 64 -2.3 %.  Causal
    // grids, whose work order already pairs long and short items on each
    // CU, ran 1-3 % slower with it, and do without.
    int left = 0, pscale = 1, plevel = -1;
    if constexpr (!CAUSAL) {
        left = ntiles;
        if (mrow) {
            int cnt = __builtin_popcountll(mask_bits);
            for (int ch = 1; ch < 4 && ch * 64 < a.nkb; ++ch) {
                const int idx = ch * 64 + lane;
                cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(idx < a.nkb && mrow[idx] != 0));
            }
            left = min(left, cnt * (128 / BC));
        }
        pscale = mrow ? max(left, 1) : max(1, (N + BC - 1) / BC);
    }
    auto update_priority = [&]() {
        if constexpr (!CAUSAL) {
            const int lv = min(3, 4 * left / pscale);
            if (lv != plevel) {
                plevel = lv;
                set_wave_priority(lv);
            }
        }
    };
    update_priority();
    const float c = scale_factor(a.scale_log2);
    const uint32_t sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    x8_t qf[NQK];

    const int kbase0 = (lane % 32) * D + (((lane / 32) ^ C::zk(lane % 32)) << 3);
    const int grp = lane >> 4, li = lane & 15;
    int vaddr[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb) {
        const int row = 4 * (grp >> 1) + (li >> 2);
        const int col = mb * 32 + 16 * (grp & 1) + 4 * (li & 3);
        vaddr[mb] = row * D + (((col >> 3) ^ C::zv(row)) << 3) + (col & 7);
    }

    acc_t o[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
    // m starts at the most negative finite float (see fwd_pipe): masked
    // scores give p = 0 and a row that never sees a key keeps l = 0.
    float m = -__FLT_MAX__, l = 0.f;

    // One tile: scores, running statistics, P V, in the order fwd_pipe
    // applies them to each row.
    auto compute = [&](int t, const T *Ks, const T *Vs) {
        const int kbase = t * BC;
        acc_t s[NKB];
        const acc_t zero = {};
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const x8_t ka = *reinterpret_cast<const x8_t *>(Ks + kb * 32 * D + (kbase0 ^ (ks << 4)));
                s[kb] = E::mfma(ka, qf[ks], ks == 0 ? zero : s[kb]);
            }
        const bool edge = (kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0);
        if (edge) {
            asm volatile("" ::);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + kb * 32 + Frag<32>::row(i, lane);
                    const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                    s[kb][i] = ok ? s[kb][i] : kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        const auto r = __builtin_amdgcn_permlane32_swap(f2u(mx), f2u(mx), false, false);
        const float m_new = fmaxf(fmaxf(m, u2f(r[0]) * c), u2f(r[1]) * c);
        const float alpha = fast_exp2(m - m_new);
        const float neg_m = -m_new;
        m = m_new;
        if (wave_any(alpha != 1.f)) {
            asm volatile("" ::);
#pragma unroll
            for (int mb = 0; mb < ND; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
        }
        float rs = 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int kb = f / 2, i0 = 8 * (f % 2);
            x8_t pf;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = fast_exp2(fmaf(s[kb][i0 + j], c, neg_m));
                s[kb][i0 + j] = e;
                pf[j] = (T)e;
            }
#pragma unroll
            for (int mb = 0; mb < ND; ++mb) {
                const T *vp = Vs + ((f / 2) * 32 + (f % 2) * 16) * D + vaddr[mb];
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vp + 8 * D));
                const x8_t vf = __builtin_bit_cast(x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[mb] = E::mfma(vf, pf, o[mb]);
            }
        }
        // Row sum in fwd_pipe's order: fragment by fragment, key by key.
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int j = 0; j < 8; ++j) rs += s[f / 2][8 * (f % 2) + j];
        l = fmaf(l, alpha, rs);
    };

    auto kst = [&](int st) { return ring + 2 * st * C::TILE; };
    auto vst = [&](int st) { return ring + (2 * st + 1) * C::TILE; };
    // Tile queue: tq[j] is the j-th next tile of the sequence; tq[0] is
    // computed in this iteration, tq[1..P-1] have their copies in flight.
    int tq[P + 1];
    tq[0] = next_tile(0);
#pragma unroll
    for (int j = 1; j <= P; ++j) tq[j] = next_tile(tq[j - 1] + 1);
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (tq[j] < ntiles) {
            copy(K, kst(j), koff, tq[j]);
            copy(V, vst(j), voff, tq[j]);
        }
    wait_copies();
    __syncthreads();
    {
        const uint32_t keep = qrow < N ? 0xffffffffu : 0u;
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qf[ks] = __builtin_bit_cast(x8_t, (qraw[ks] ^ sign) & keep);
    }
    // Iteration i computes tq[0] from stage i % NSTAGE and starts the
    // copies of tq[P] into stage (i + P) % NSTAGE, which the barrier shows
    // every wave is done with.  Before the barrier a wave waits for its own
    // copies of tq[0]; those of tq[1..P-1] may stay in flight.
    bool first = true;
    auto iteration = [&](auto stage_tag) {
        constexpr int u = decltype(stage_tag)::value;
        if (!first) {
            if (P > 1 && tq[P - 1] < ntiles)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * ROUNDS * (P - 1)) : "memory");
            else
                wait_copies();
            stage_barrier();
        }
        first = false;
        if (tq[P] < ntiles) {
            copy(K, kst((u + P) % NSTAGE), koff, tq[P]);
            copy(V, vst((u + P) % NSTAGE), voff, tq[P]);
        }
        if (tq[0] <= wlast) compute(tq[0], kst(u), vst(u));
        --left;
        update_priority();
#pragma unroll
        for (int j = 0; j < P; ++j) tq[j] = tq[j + 1];
        tq[P] = next_tile(tq[P] + 1);
    };
    while (true) {
        if (tq[0] >= ntiles) break;
        iteration(IntTag<0>{});
        if (tq[0] >= ntiles) break;
        iteration(IntTag<1 % NSTAGE>{});
        if constexpr (NSTAGE == 3) {
            if (tq[0] >= ntiles) break;
            iteration(IntTag<2>{});
        }
    }

    const float l_tot = group_sum<32>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        T *orow = O + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = (T)(o[mb][4 * gg + j] * inv);
                *reinterpret_cast<x4_t *>(orow + mb * 32 + 8 * gg + 4 * (lane / 32)) = w;
            }
        if (a.lse && lane < 32)
            a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

// Two stages at four workgroups per CU.  Measured against three stages at
// three per CU (48 KiB of ring per workgroup): the deeper ring was 3-7 %
// slower on the d = 64 workloads.
template <class T, int D, bool CAUSAL>
hipError_t launch_flat(const FwdArgs &a, hipStream_t stream) {
    constexpr int NW = 4, BR = 32 * NW;
    const int nqt = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_flat<T, D, 64, NW, CAUSAL, 2, 4>), dim3((unsigned)(nqt * a.B * a.H)), dim3(NW * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_flat(const FwdArgs &a, int causal, int f16, hipStream_t stream) {
    if (f16) return causal ? launch_flat<_Float16, 64, true>(a, stream) : launch_flat<_Float16, 64, false>(a, stream);
    return causal ? launch_flat<__bf16, 64, true>(a, stream) : launch_flat<__bf16, 64, false>(a, stream);
}

}  // namespace fa
