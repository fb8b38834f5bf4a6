// Tuned exact-attention forward for gfx950 (bf16 or fp16 in/out, fp32
// accumulation).
//
// Same method and running-statistics recurrence as the tile-study kernel in
// fa_fwd_bf16.hip (tiled exact attention with an online softmax: page
// "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", ai-paper-library, Summary and Method; five-stage map of
// "What is FlashAttention?", unite.ai), reorganised for throughput:
//
//  * Software pipeline over key tiles.  While the VALU exponentiates the
//    scores of tile j, the matrix cores already compute the scores of tile
//    j+1; while the matrix cores accumulate P_j V_j, the VALU packs P to
//    bf16 and sums the rows.  Each step is a fixed sequence of matrix-core
//    slots with the VALU work spread over them (see `step`), so one wave
//    keeps both pipes busy by itself.
//  * O is rescaled only when some row of the wave raised its running
//    maximum; otherwise the rescale factor is exactly 1 and the multiply is
//    skipped (a bit-identical no-op).
//  * Each wave owns 32 query rows; a workgroup of NW waves owns 32*NW.
//  * K/V tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging) through an NSTAGE-deep ring: K runs one tile ahead of V (it is
//    consumed one iteration earlier) and the copies are issued NSTAGE-1
//    tiles ahead of use.
//  * Scores are computed transposed (S^T = K Q^T) so each lane holds one
//    query row: the row max is an in-lane v_max3 chain plus one
//    v_permlane32_swap; O^T += V^T P^T takes P straight from registers.
//  * SPLIT = true (fa_fwd_ws, grids too small for the GPU): the workgroup
//    covers one share of its query tile's key tiles and writes an fp32
//    partial O and partial LSE; fwd_merge combines the shares of each row
//    by log-sum-exp.
#include "fa_bf16_tiles.h"

namespace fa {
namespace {

// VALU work of one tile for one wave, cut into chunks in dependency order:
// per 8-score fragment f (NF of them) a partial row max; the cross-lane max
// and rescale factor; per fragment two halves of exponentials and one bf16
// packing; per fragment a partial row sum.  Each chunk is assigned to the
// matrix-core slot where its estimated start falls when the total VALU time
// (fp32 op ~4 cycles, exponential ~8 cycles per wave) is spread evenly over
// the step's NS slots.
// Empty asm statements that make a value "used" where they stand: the
// compiler may not sink its computation below them (past the rescale branch
// of a step, say), which keeps the VALU work in the slot it was assigned to.
template <class T>
__device__ __forceinline__ void pin(T &x) {
    asm volatile("" : "+v"(x));
}
__device__ __forceinline__ void pin4(float &a, float &b, float &c, float &d) {
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Slot at which the V fragments of PV product pv are read (LB slots ahead;
// the first ones during the QK phase).
__host__ __device__ constexpr int vread_slot_of(int pv, int na, int lb) { return na + pv - lb; }

constexpr int kChunkMax = 0, kChunkRed = 1, kChunkExp = 2, kChunkCvt = 3, kChunkSum = 4;

template <int NF>
struct ChunkPlan {
    static constexpr int NCH = 5 * NF + 1;
    __host__ __device__ static constexpr int kind(int k) {
        return k < NF ? kChunkMax
             : k == NF ? kChunkRed
             : k < 4 * NF + 1 ? ((k - NF - 1) % 3 == 2 ? kChunkCvt : kChunkExp)
             : kChunkSum;
    }
    __host__ __device__ static constexpr int frag(int k) {
        return k < NF ? k : k == NF ? 0 : k < 4 * NF + 1 ? (k - NF - 1) / 3 : k - 4 * NF - 1;
    }
    __host__ __device__ static constexpr int half(int k) { return (k - NF - 1) % 3; }
    __host__ __device__ static constexpr int cost(int k) {
        return kind(k) == kChunkMax ? 16 : kind(k) == kChunkRed ? 48 : kind(k) == kChunkExp ? 48
             : kind(k) == kChunkCvt ? 16 : 32;
    }
    __host__ __device__ static constexpr int start(int k) {
        int c = 0;
        for (int i = 0; i < k; ++i) c += cost(i);
        return c;
    }
    __host__ __device__ static constexpr int slot(int k, int ns) { return start(k) * ns / start(NCH); }
    // Slot of the packing of fragment f.
    __host__ __device__ static constexpr int cvt_slot(int f, int ns) { return slot(NF + 1 + 3 * f + 2, ns); }
    // The PV products of fragment f occupy slots na + f*nd .. na + f*nd + nd - 1.
    __host__ __device__ static constexpr bool packed_in_time(int na, int nd, int ns) {
        for (int f = 0; f < NF; ++f)
            if (cvt_slot(f, ns) >= na + f * nd) return false;
        return true;
    }
};

template <class T, int D, int BC, int NSTAGE, int NW, bool CAUSAL, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void fwd_pipe(FwdArgs a) {
    using E = Elem<T>;
    using x8_t = typename E::x8;
    using x4_t = typename E::x4;
    constexpr int QW = 32, BR = QW * NW, NKB = BC / 32;
    using C = Cfg<D, BC, 32, NW>;
    using acc_t = f32x16_t;
    constexpr int NQK = C::NQK, ND = C::ND;
    constexpr int ROUNDS = C::NCOPY / NW;  // copy instructions per wave per tensor
    static_assert(C::NCOPY % NW == 0, "copies must split evenly over the waves");
    constexpr int P = NSTAGE - 1;          // copies run P tiles ahead
    static_assert(P >= 1 && P <= 3, "2..4 stages");
    constexpr int NA = NKB * NQK;          // QK products per tile
    constexpr int NB = NKB * 2 * ND;       // PV products per tile
    constexpr int NS = NA + NB;            // matrix-core slots per step
    constexpr int NF = 2 * NKB;            // 8-score P fragments per tile
    // K and V fragment reads run LA and LB slots ahead of their products.
    // Swept on the 16K causal workload (same box, alternating runs): LB = 1
    // +2-3 %; LA = 4, LB = 3 -0.5-1 % on the workload's data and -2 % on
    // all-zero inputs against LA = 3, LB = 2; larger distances no better.
    constexpr int LA = 4;
    constexpr int LB = 3;
    using Plan = ChunkPlan<NF>;
    // PV product pv uses fragment pv / ND; its packing must come earlier.
    static_assert(Plan::packed_in_time(NA, ND, NS), "every P fragment packed before its PV product");

    // One LDS array per K stage and per V stage.
    __shared__ __attribute__((aligned(1024))) T k_lds0[C::TILE];
    __shared__ __attribute__((aligned(1024))) T k_lds1[C::TILE];
    __shared__ __attribute__((aligned(1024))) T k_lds2[NSTAGE > 2 ? C::TILE : 1];
    __shared__ __attribute__((aligned(1024))) T k_lds3[NSTAGE > 3 ? C::TILE : 1];
    __shared__ __attribute__((aligned(1024))) T v_lds0[C::TILE];
    __shared__ __attribute__((aligned(1024))) T v_lds1[C::TILE];
    __shared__ __attribute__((aligned(1024))) T v_lds2[NSTAGE > 2 ? C::TILE : 1];
    __shared__ __attribute__((aligned(1024))) T v_lds3[NSTAGE > 3 ? C::TILE : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    const int nqt = (N + BR - 1) / BR;
    int bh, qt, split = 0;
    if constexpr (SPLIT) {
        // (query tile, key-range share): the shares of one query tile are
        // adjacent items; heads and tiles in the usual XCD-aware order, at
        // d = 128 causal in the CU-balanced order (2 resident workgroups per
        // CU: B1 H1 N32768 333 -> 313 us, B2 H2 N8192 109 -> 105 us; at
        // d = 64 it measured 1-2 % slower and is not used).
        const int item = CAUSAL && D == 128 ? xcd_item_causal(nqt * a.nsplit, 2) : xcd_item(nqt * a.nsplit);
        split = item % a.nsplit;
        const int rest = item / a.nsplit;
        bh = rest / nqt;
        const int r = rest - bh * nqt;
        qt = CAUSAL ? nqt - 1 - r : r;
    } else {
        // workgroups resident per CU: 2 at d = 128 and 3 at d = 64 with 4
        // waves (238 and 168 registers), 1 with 8 waves
        tile_of_block(nqt, CAUSAL, NW == 4 ? (D == 128 ? 2 : 3) : 1, &bh, &qt,
                      !CAUSAL && a.key_len ? a.group * nqt : 0);
    }
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
    // Key tiles [tbeg, tend) of this workgroup: all of them, or one share of
    // a key-range split.
    const int tbeg = SPLIT ? (int)((int64_t)ntiles * split / a.nsplit) : 0;
    const int tend = SPLIT ? (int)((int64_t)ntiles * (split + 1) / a.nsplit) : ntiles;
    const int klast = kv_len - 1;
    // Tiles this wave computes form a prefix of the workgroup's sequence.
    const int wlast = wq0 >= N ? -1 : (CAUSAL ? (wq0 + QW - 1) / BC : ntiles);
    auto active = [&](int t) { return t < tend && t <= wlast; };

    // Block-sparse skipping (only launched with BR = 128, where the
    // workgroup's rows are one query block): the mask row is scanned 64 key
    // blocks at a time into a wave-uniform bit mask.
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

    // Per-lane byte offsets of this wave's copy chunks inside a tile; the
    // tile base is a wave-uniform address.
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
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) {
                const int r = ((wave + NW * i) * 64 + lane) / C::SLOTS;
                const int excess = max(0, kbase + r - klast);
                lds_copy16(base, off[i] - (uint32_t)(excess * D * 2), dst + (wave + NW * i) * 512);
            }
        }
    };
    auto kstage = [&](int s) { return s == 0 ? k_lds0 : s == 1 ? k_lds1 : s == 2 ? k_lds2 : k_lds3; };
    auto vstage = [&](int s) { return s == 0 ? v_lds0 : s == 1 ? v_lds1 : s == 2 ? v_lds2 : v_lds3; };

    // Prologue loads, ordered so that their round trips overlap: the first
    // mask chunk (block-sparse), then this wave's Q rows, and only then the
    // ballot that needs the mask (it waits for the mask load alone).  The Q
    // values are not touched before the first K/V copies have been issued
    // and have landed, so the Q latency hides under the copies' latency.
    // Rows past N load row N-1 and are zeroed when the fragments are formed.
    const int qrow = wq0 + lane % 32;
    const int pre_chunk = ((tbeg * BC) >> 7) >> 6;
    uint8_t mask_pre = 0;
    if (mrow) mask_pre = mrow[min(pre_chunk * 64 + lane, a.nkb - 1)];
    u32x4_t qraw[NQK];
    {
        const T *qsrc = Q + (int64_t)min(qrow, N - 1) * D + 8 * (lane / 32);
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qraw[ks] = *reinterpret_cast<const u32x4_t *>(qsrc + ks * 16);
    }
    if (mrow) {
        // The empty asm takes the mask byte as issued by its load: the
        // compiler's wait for it lands here, after the Q loads (which the
        // memory clobber keeps above), not right after the load.
        uint32_t mv = mask_pre;
        asm volatile("" : "+v"(mv)::"memory");
        mask_bits = __builtin_amdgcn_ballot_w64(pre_chunk * 64 + lane < a.nkb && mv != 0);
        mask_chunk = pre_chunk;
    }
    // Q fragments (B operand of S^T = K Q^T), sign-folded so that c >= 0;
    // formed after the first copies (below).
    const float c = scale_factor(a.scale_log2);
    const uint32_t sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    x8_t qf[NQK];

    // LDS read offsets (elements): K fragment ks of a 32-key block, and the
    // transposed V fragment of output block mb (two 4-row reads, 8 rows apart).
    // K: row r starts at a multiple of 2*D bytes and the swizzled slot
    // (2ks + lane/32) ^ zk(r) fits in the low bits, so the element offset is
    // kbase0 ^ (16*ks): one base register instead of NQK.
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
    // m starts at the most negative finite float rather than -inf, so that
    // m - m_new and s*c - m never meet inf - inf: masked scores (-inf) still
    // give p = 0, a tile with no allowed key leaves m unchanged (alpha = 1),
    // and the first allowed key makes alpha = exp2(-huge) = 0 while O and l
    // are still 0.  Rows that never see a key keep l = 0 (LSE = -inf, O = 0).
    float m = -__FLT_MAX__, l = 0.f;
    // Scores ping-pong between sA and sB across consecutive iterations.
    acc_t sA[NKB], sB[NKB];

    auto qk_plain = [&](acc_t (&dst)[NKB], const T *Ks) {
        const acc_t zero = {};
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const x8_t ka = *reinterpret_cast<const x8_t *>(Ks + kb * 32 * D + (kbase0 ^ (ks << 4)));
                dst[kb] = E::mfma(ka, qf[ks], ks == 0 ? zero : dst[kb]);
            }
    };

    // One pipeline step: softmax + PV of tile t (scores in s), and the
    // scores of the next tile (from Kn) into sn.  The QK products are issued
    // even when this wave has no next tile (the result is then unused): a
    // branch would split the schedule below.
    //
    // Schedule.  The step is a fixed sequence of NA + NB slots, one
    // matrix-core instruction each (NA QK products of the next tile, then NB
    // PV products of this tile), separated by sched_barrier fences so the
    // compiler cannot regroup them.  The tile's VALU work, in dependency
    // order (row max, rescale factor, exponentials, bf16 packing, row sum),
    // is cut into chunks that are spread evenly over the slots
    // (chunk_slot), so the VALU works while the matrix core runs.  LDS reads
    // of K and V fragments are issued a few slots ahead of their products.
    auto step = [&](int t, acc_t (&s)[NKB], acc_t (&sn)[NKB], const T *Kn, const T *Vs) {
        const int kbase = t * BC;
        const bool edge = (kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0);
        if (edge) {
            // Keep this a branch: the compiler would otherwise if-convert it
            // into per-element selects on every tile.
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

        // The K read offsets kbase0 ^ (16 * ks) are loop-invariant; the
        // compiler keeps them in registers (238 at d = 128, still two waves
        // per SIMD), which measured 1 % faster than re-deriving them with
        // one XOR each per step.
        const int kb0 = kbase0;

        x8_t kf[NA], vf[NB], pf[NF];
        float mx = kNegInf, alpha = 1.f, neg_m = 0.f, rs = 0.f;
        bool rescale = true;

        auto kread = [&](auto A) {
            constexpr int a = decltype(A)::value, ks = a / NKB, kb = a % NKB;
            kf[a] = *reinterpret_cast<const x8_t *>(Kn + kb * 32 * D + (kb0 ^ (ks << 4)));
        };
        auto vread = [&](auto PV) {
            constexpr int pv = decltype(PV)::value, f = pv / ND, mb = pv % ND;
            const T *vp = Vs + ((f / 2) * 32 + (f % 2) * 16) * D + vaddr[mb];
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vp + 8 * D));
            vf[pv] = __builtin_bit_cast(x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // Fragment f holds scores s[f/2][8*(f%2) .. 8*(f%2)+7] of each lane.
        auto chunk = [&](auto K) {
            constexpr int k = decltype(K)::value, kind = Plan::kind(k), f = Plan::frag(k);
            constexpr int kb = f / 2, i0 = 8 * (f % 2);
            if constexpr (kind == kChunkMax) {
#pragma unroll
                for (int j = 0; j < 8; ++j) mx = fmaxf(mx, s[kb][i0 + j]);
                pin(mx);
            } else if constexpr (kind == kChunkRed) {
                // Row max over the partner lane (permlane32 swap), scaled
                // by c > 0 before the max: one three-way max, no -inf guards.
                const auto r = __builtin_amdgcn_permlane32_swap(f2u(mx), f2u(mx), false, false);
                const float m_new = fmaxf(fmaxf(m, u2f(r[0]) * c), u2f(r[1]) * c);
                alpha = fast_exp2(m - m_new);
                neg_m = -m_new;
                m = m_new;
                // O needs rescaling only when some row's maximum moved
                // (alpha = 1 exactly otherwise).
                rescale = wave_any(alpha != 1.f);
                pin(alpha);
                pin(neg_m);
            } else if constexpr (kind == kChunkExp) {
                constexpr int j0 = i0 + 4 * Plan::half(k);
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = fast_exp2(fmaf(s[kb][j0 + j], c, neg_m));
                pin4(e[0], e[1], e[2], e[3]);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[kb][j0 + j] = e[j];
            } else if constexpr (kind == kChunkCvt) {
#pragma unroll
                for (int j = 0; j < 8; ++j) pf[f][j] = (T)s[kb][i0 + j];
                pin(pf[f]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) rs += s[kb][i0 + j];
                pin(rs);
            }
        };

        static_for<NS>([&](auto G) {
            constexpr int g = decltype(G)::value;
            if constexpr (g == 0) static_for<(LA < NA ? LA : NA)>([&](auto A) { kread(A); });
            if constexpr (g < NA && g + LA < NA) kread(IntTag<g + LA>{});
            static_for<NB>([&](auto PV) {
                if constexpr (vread_slot_of(decltype(PV)::value, NA, LB) == g) vread(PV);
            });
            if constexpr (g < NA) {
                constexpr int ks = g / NKB, kb = g % NKB;
                if constexpr (ks == 0) {
                    const acc_t zero = {};
                    sn[kb] = E::mfma(kf[g], qf[ks], zero);
                } else {
                    sn[kb] = E::mfma(kf[g], qf[ks], sn[kb]);
                }
            } else {
                constexpr int pv = g - NA, f = pv / ND, mb = pv % ND;
                o[mb] = E::mfma(vf[pv], pf[f], o[mb]);
            }
            static_for<Plan::NCH>([&](auto K) {
                if constexpr (Plan::slot(decltype(K)::value, NS) == g) chunk(K);
            });
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (g == NA - 1) {
                if (rescale) {
                    // Between the phases: the first PV product of every
                    // output block follows.  A wave-uniform branch.
                    asm volatile("" ::);
#pragma unroll
                    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
                }
            }
        });
        l = fmaf(l, alpha, rs);
    };

    // ---- pipeline ---------------------------------------------------------
    // Tile sequence T[0], T[1], ... (active tiles of the workgroup); tq[j]
    // holds T[i+j] for j = 0..P at iteration i.  Iteration i computes the
    // softmax/PV of T[i] (scores already in registers) and the scores of
    // T[i+1]; it needs K(T[i+1]) in K stage (i+1)%NSTAGE and V(T[i]) in V
    // stage i%NSTAGE, and it starts the copies of K(T[i+1+P]) into K stage
    // i%NSTAGE and of V(T[i+P]) into V stage (i-1)%NSTAGE, both freed by the
    // previous iteration.
    int tq[P + 1];
    tq[0] = next_tile(tbeg);
#pragma unroll
    for (int j = 1; j <= P; ++j) tq[j] = next_tile(tq[j - 1] + 1);
#pragma unroll
    for (int j = 0; j <= P; ++j)
        if (tq[j] < tend) copy(K, kstage(j), koff, tq[j]);
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (tq[j] < tend) copy(V, vstage(j), voff, tq[j]);
    wait_copies();
    __syncthreads();
    {
        const uint32_t keep = qrow < N ? 0xffffffffu : 0u;
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qf[ks] = __builtin_bit_cast(x8_t, (qraw[ks] ^ sign) & keep);
    }
    if (active(tq[0])) qk_plain(sA, kstage(0));

    auto iteration = [&](auto stage_tag, acc_t (&s)[NKB], acc_t (&sn)[NKB]) {
        constexpr int u = decltype(stage_tag)::value;  // i % NSTAGE
        const int t_new = next_tile(tq[P] + 1);         // T[i+P+1]
        // Copies younger than those of K(T[i+1]) and V(T[i]) were issued in
        // the last P-1 iterations; they may stay in flight when complete.
        if (P > 1 && tq[P] < tend)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * ROUNDS * (P - 1)) : "memory");
        else
            wait_copies();
        stage_barrier();
        if (t_new < tend) copy(K, kstage(u), koff, t_new);
        if (tq[P] < tend) copy(V, vstage((u + NSTAGE - 1) % NSTAGE), voff, tq[P]);
        if (active(tq[0])) step(tq[0], s, sn, kstage((u + 1) % NSTAGE), vstage(u));
#pragma unroll
        for (int j = 0; j < P; ++j) tq[j] = tq[j + 1];
        tq[P] = t_new;
    };

    while (true) {
        if (tq[0] >= tend) break;
        iteration(IntTag<0>{}, sA, sB);
        if (tq[0] >= tend) break;
        iteration(IntTag<1 % NSTAGE>{}, sB, sA);
        if constexpr (NSTAGE % 2 == 1 || NSTAGE == 4) {
            // Unrolled to a multiple of both NSTAGE and 2 (score ping-pong).
            if (tq[0] >= tend) break;
            iteration(IntTag<2 % NSTAGE>{}, sA, sB);
            if (tq[0] >= tend) break;
            iteration(IntTag<3 % NSTAGE>{}, sB, sA);
            if constexpr (NSTAGE == 3) {
                if (tq[0] >= tend) break;
                iteration(IntTag<4 % NSTAGE>{}, sA, sB);
                if (tq[0] >= tend) break;
                iteration(IntTag<5 % NSTAGE>{}, sB, sA);
            }
        }
    }

    // Epilogue: normalise, round to bf16 once, write O and LSE.  A share of
    // a key-range split writes its fp32 partial O (normalised by its own
    // sum) and partial LSE instead; a share with no allowed key writes
    // O = 0, LSE = -inf, which the merge gives weight 0.
    if constexpr (SPLIT) {
        const float l_tot = group_sum<32>(l);
        if (qrow < N) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const int64_t prow = ((int64_t)split * a.B * a.H + bh) * N + qrow;
            float *orow = a.part_o + prow * D;
#pragma unroll
            for (int mb = 0; mb < ND; ++mb)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    f32x4_t w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = o[mb][4 * gg + j] * inv;
                    *reinterpret_cast<f32x4_t *>(orow + mb * 32 + 8 * gg + 4 * (lane / 32)) = w;
                }
            if (lane < 32) a.part_l[prow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
        }
        return;
    }
    {
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
}

template <class T, int D, int BC, int NSTAGE, int NW, bool CAUSAL>
hipError_t launch_pipe(const FwdArgs &a, hipStream_t stream) {
    constexpr int BR = 32 * NW;
    const int nqt = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_pipe<T, D, BC, NSTAGE, NW, CAUSAL>),
                       dim3((unsigned)(nqt * a.B * a.H)), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

// Merge of the nsplit partial results of each query row (the log-sum-exp
// combination): LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s,
// rounded once to the element type.  Shares with LSE_s = -inf carry weight
// 0; a row with no allowed key in any share gets O = 0, LSE = -inf.  D/8
// lanes per row, 8 elements each; shares added in order (deterministic).
template <class T, int D>
__global__ __launch_bounds__(256) void fwd_merge(FwdArgs a) {
    using x8_t = typename Elem<T>::x8;
    constexpr int LPR = D / 8;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    if (row >= rows) return;
    float mx = kNegInf;
    for (int s = 0; s < a.nsplit; ++s) mx = fmaxf(mx, a.part_l[(int64_t)s * rows + row]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lse = kNegInf;
    if (mx != kNegInf) {
        float wsum = 0.f;
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = __expf(a.part_l[(int64_t)s * rows + row] - mx);
            wsum += w;
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(a.part_o + ((int64_t)s * rows + row) * D + part * 8);
            const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[j] = fmaf(w, x0[j], acc[j]);
                acc[4 + j] = fmaf(w, x1[j], acc[4 + j]);
            }
        }
        const float inv = 1.f / wsum;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= inv;
        lse = mx + __logf(wsum);
    }
    x8_t w8;
#pragma unroll
    for (int j = 0; j < 8; ++j) w8[j] = (T)acc[j];
    *reinterpret_cast<x8_t *>(reinterpret_cast<T *>(a.o) + row * D + part * 8) = w8;
    if (a.lse && part == 0) a.lse[row] = lse;
}

template <class T, int D, bool CAUSAL>
hipError_t launch_split(const FwdArgs &a, hipStream_t stream) {
    constexpr int NW = 4, BR = 32 * NW;
    const int nqt = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_pipe<T, D, 64, 2, NW, CAUSAL, true>),
                       dim3((unsigned)(nqt * a.B * a.H * a.nsplit)), dim3(NW * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((fwd_merge<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <class T>
hipError_t launch_split_typed(const FwdArgs &a, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_split<T, 64, true>(a, stream) : launch_split<T, 64, false>(a, stream);
    return causal ? launch_split<T, 128, true>(a, stream) : launch_split<T, 128, false>(a, stream);
}

#define FA_PIPE(T, D, BC, NS, NW) \
    Instance{D, 0, 32 * NW, BC, &launch_pipe<T, D, BC, NS, NW, false>}, \
    Instance{D, 1, 32 * NW, BC, &launch_pipe<T, D, BC, NS, NW, true>}

// The tuned (128, 64) tile at d = 64 runs fwd_flat (fa_fwd_flat.hip), four
// workgroups per CU; the key-range split keeps fwd_pipe.
hipError_t flat_bf16(const FwdArgs &a, hipStream_t s) { return launch_fwd_flat(a, 0, 0, s); }
hipError_t flat_bf16_causal(const FwdArgs &a, hipStream_t s) { return launch_fwd_flat(a, 1, 0, s); }
hipError_t flat_f16(const FwdArgs &a, hipStream_t s) { return launch_fwd_flat(a, 0, 1, s); }
hipError_t flat_f16_causal(const FwdArgs &a, hipStream_t s) { return launch_fwd_flat(a, 1, 1, s); }

}  // namespace

const Instance *bf16_tuned_instances() {
    static const Instance table[] = {
        Instance{64, 0, 128, 64, &flat_bf16},
        Instance{64, 1, 128, 64, &flat_bf16_causal},
        FA_PIPE(__bf16, 64, 64, 2, 8),
        FA_PIPE(__bf16, 128, 64, 2, 4),
        FA_PIPE(__bf16, 128, 64, 2, 8),
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

const Instance *f16_tuned_instances() {
    static const Instance table[] = {
        Instance{64, 0, 128, 64, &flat_f16},
        Instance{64, 1, 128, 64, &flat_f16_causal},
        FA_PIPE(_Float16, 128, 64, 2, 4),
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

// A key-range split pays when the grid (B*H query tiles of 128 rows) is too
// small for the 256 CUs and a causal grid's longest tile dominates: if it
// has fewer than 512 workgroups, the largest power of two (at most 16) that
// keeps it within 1024.  (Measured on B1 H2 N16384: 4 shares 172 us,
// 8 shares 181 us, 16 shares 246 us, unsplit 299 us.)  A causal grid of
// exactly 512 tiles with long heads (64 or more query tiles) is split in two
// as well: one round pairs its heaviest and lightest tiles on the same CUs
// (same box, alternating runs: B1 H4 N16384 d128 338 -> 312 us, B2 H2
// N16384 320 -> 294 us, B1 H8 N8192 168 -> 162 us; at d = 64 B1 H8 N8192
// 119 -> 99 us, B1 H4 N16384 227 -> 179 us), while a non-causal one ran 4 %
// slower split.  Shares stay within 1024, the size of the static scratch.
int fwd_split(int B, int H, int N, bool causal) {
    if (B < 1 || H < 1 || N < 1) return 1;
    const int nqt = (N + 127) / 128;
    const int64_t base = (int64_t)B * H * nqt;
    if (base > 512 || (base == 512 && !(causal && nqt >= 64))) return 1;
    int s = 1;
    while (s < 16 && base * s * 2 <= 1024) s *= 2;
    return s;
}

uint64_t fwd_split_bytes(int B, int H, int N, int d, int s) {
    if (s <= 1) return 0;
    return (uint64_t)s * B * H * (uint64_t)N * (d + 1) * sizeof(float);
}

uint64_t fwd_workspace_bytes(int B, int H, int N, int d) {
    // the causal case splits at least as much as any other
    return fwd_split_bytes(B, H, N, d, fwd_split(B, H, N, true));
}

hipError_t launch_fwd_split(const FwdArgs &a, int d, int causal, int f16, hipStream_t stream) {
    return f16 ? launch_split_typed<_Float16>(a, d, causal, stream)
               : launch_split_typed<__bf16>(a, d, causal, stream);
}

void bf16_default_tile(int d, int block_sparse, int *br, int *bc) {
    (void)d;
    (void)block_sparse;
    *br = 128;
    *bc = 64;
}

}  // namespace fa
