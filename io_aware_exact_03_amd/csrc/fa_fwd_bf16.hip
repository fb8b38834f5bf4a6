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
//
// gfx950 mapping.  One wavefront owns MF query rows (MF = 32, or 16 for the
// small tiles of the tile-size study).  Scores are computed transposed,
// S^T = K Q^T, on bf16 matrix-core instructions (v_mfma_f32_32x32x16_bf16 /
// v_mfma_f32_16x16x32_bf16), so each lane holds scores of a single query
// row: the row max and row sum are in-lane reductions plus one (or two)
// v_permlane*_swap exchanges.  The output is accumulated transposed too,
// O^T += V^T P^T, which takes P straight from the score registers as the B
// operand (no LDS round trip).  Q fragments live in VGPRs for the whole
// kernel; K tiles are stored row-major in LDS and V tiles transposed
// (d-major) so both operands are single 16-byte LDS reads.  K/V tiles are
// double-buffered: the global loads of tile j+1 are in flight while tile j
// is being computed.
#include "fa_common.h"

namespace fa {
namespace {

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

// Position of key k inside a transposed V row.  With 32x32 tiles, one PV
// instruction consumes, in the lower half-wave, keys {0-3, 8-11} of a
// 16-key group and in the upper half-wave keys {4-7, 12-15} (that is where
// the score layout put them); swapping bits 2 and 3 of the key index makes
// each half-wave's eight keys contiguous.
template <int MF>
__device__ __forceinline__ int vt_pos(int k) {
    if constexpr (MF == 32)
        return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
    else
        return k;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

template <int D, int BC, int MF, int NW, bool CAUSAL>
struct Cfg {
    static constexpr int NT = NW * 64;
    static constexpr int BR = MF * NW;
    static constexpr int KSTR = D + 8;   // bf16 per K row in LDS (+16 B pad)
    static constexpr int VSTR = BC + 8;  // bf16 per transposed V row (+16 B)
    static constexpr int KTILE = BC * KSTR;
    static constexpr int VTILE = D * VSTR;
    static constexpr int NKB = BC / MF;  // score blocks per tile
    static constexpr int ND = D / MF;    // output blocks
    static constexpr int NQK = D / Frag<MF>::KQK;
    static constexpr int KCH = BC * D / 8;        // 16-byte chunks of a K tile
    static constexpr int VUN = (BC / 4) * (D / 8);  // 4-key x 8-dim V units
    static constexpr int KPT = (KCH + NT - 1) / NT;
    static constexpr int VPT = (VUN + NT - 1) / NT;
    // Registers that hold one prefetched tile; beyond ~48 VGPRs the tile is
    // loaded synchronously into a single buffer instead.
    static constexpr bool PREFETCH = KPT * 4 + VPT * 16 <= 48;
    static constexpr int NBUF = PREFETCH ? 2 : 1;
    static constexpr int LDS_ELEMS = NBUF * (KTILE + VTILE);
    static_assert(BC % MF == 0 && D % MF == 0, "tile must be a multiple of MF");
    static_assert(BC % 16 == 0 && 128 % BC == 0, "BC must divide the 128 mask block");
    static_assert(128 % BR == 0 || BR % 128 == 0, "BR and the mask block must nest");
};

// Per-thread staging registers of one K/V tile.
template <class C>
struct TileRegs {
    u32x4_t k[C::KPT];
    u32x4_t v[C::VPT][4];
};

// Issue the global loads of key tile `t` (rows t*BC ..) into registers.
// Rows at or past kv_len are zero so masked keys never meet non-finite data.
template <class C, int D, int BC>
__device__ __forceinline__ void load_tile(TileRegs<C> &r, const __bf16 *K,
                                          const __bf16 *V, int t, int kv_len,
                                          int tid, int first, int count) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        if (i < first || i >= first + count) continue;
        const int c = tid + i * C::NT;
        const int row = c / (D / 8), col8 = c % (D / 8);
        const int key = t * BC + row;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if ((C::KCH % C::NT == 0 || c < C::KCH) && key < kv_len)
            x = *reinterpret_cast<const u32x4_t *>(K + (int64_t)key * D + col8 * 8);
        r.k[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
        if (i < first || i >= first + count) continue;
        const int u = tid + i * C::NT;
        const int kg = u / (D / 8), col8 = u % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int key = t * BC + kg * 4 + rr;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if ((C::VUN % C::NT == 0 || u < C::VUN) && key < kv_len)
                x = *reinterpret_cast<const u32x4_t *>(V + (int64_t)key * D + col8 * 8);
            r.v[i][rr] = x;
        }
    }
}

// Write staged registers into one LDS buffer: K row-major, V transposed.
template <class C, int D, int BC, int MF>
__device__ __forceinline__ void store_tile(const TileRegs<C> &r, __bf16 *Ks,
                                           __bf16 *Vt, int tid, int first,
                                           int count) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        if (i < first || i >= first + count) continue;
        const int c = tid + i * C::NT;
        if (C::KCH % C::NT != 0 && c >= C::KCH) continue;
        const int row = c / (D / 8), col8 = c % (D / 8);
        *reinterpret_cast<u32x4_t *>(Ks + row * C::KSTR + col8 * 8) = r.k[i];
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
        if (i < first || i >= first + count) continue;
        const int u = tid + i * C::NT;
        if (C::VUN % C::NT != 0 && u >= C::VUN) continue;
        const int kg = u / (D / 8), col8 = u % (D / 8);
        const int pos = vt_pos<MF>(kg * 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dims 2w and 2w+1 of this 8-dim chunk
            const u32x2_t even = {pack_lo(r.v[i][0][w], r.v[i][1][w]),
                                  pack_lo(r.v[i][2][w], r.v[i][3][w])};
            const u32x2_t odd = {pack_hi(r.v[i][0][w], r.v[i][1][w]),
                                 pack_hi(r.v[i][2][w], r.v[i][3][w])};
            *reinterpret_cast<u32x2_t *>(Vt + (col8 * 8 + 2 * w) * C::VSTR + pos) = even;
            *reinterpret_cast<u32x2_t *>(Vt + (col8 * 8 + 2 * w + 1) * C::VSTR + pos) = odd;
        }
    }
}

template <int D, int BC, int MF, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    using C = Cfg<D, BC, MF, NW, CAUSAL>;
    using F = Frag<MF>;
    using acc_t = typename F::acc_t;

    __shared__ __attribute__((aligned(16))) __bf16 smem[C::LDS_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    const int q0 = qt * C::BR;      // first query row of the workgroup
    const int wq0 = q0 + wave * MF; // first query row of this wave
    const int qrow = wq0 + lane % MF;

    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + C::BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;
    auto next_tile = [&](int t) {
        if (mrow)
            while (t < ntiles && mrow[(t * BC) >> 7] == 0) ++t;
        return t;
    };

    // Q fragments (B operand of S^T = K Q^T), resident for the whole kernel.
    // A negative scale is folded into Q (sign flip, exact) so that c >= 0.
    const float c = fabsf(a.scale_log2);
    const uint32_t sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8_t qf[C::NQK];
#pragma unroll
    for (int ks = 0; ks < C::NQK; ++ks) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (qrow < N)
            x = *reinterpret_cast<const u32x4_t *>(Q + (int64_t)qrow * D + ks * F::KQK +
                                                   8 * (lane / MF));
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

    auto compute = [&](int t, const __bf16 *Ks, const __bf16 *Vt) {
        const int kbase = t * BC;
        if (wq0 >= N) return;
        if (CAUSAL && kbase > wq0 + MF - 1) return;  // whole tile above the diagonal

        // S^T for this tile: NKB blocks of MF keys x MF queries.
        acc_t s[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) s[kb][i] = 0.f;
            const __bf16 *kr = Ks + (kb * MF + lane % MF) * C::KSTR + 8 * (lane / MF);
#pragma unroll
            for (int ks = 0; ks < C::NQK; ++ks) {
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(kr + ks * F::KQK);
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
        if (edge) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) {
                    const float x = s[kb][i];
                    const float p = x == kNegInf ? 0.f : fast_exp2(fmaf(x, c, neg_m));
                    s[kb][i] = p;
                    rs += p;
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < F::ACC; ++i) {
                    const float p = fast_exp2(fmaf(s[kb][i], c, neg_m));
                    s[kb][i] = p;
                    rs += p;
                }
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
        if constexpr (MF == 32) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x8_t pf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[kb][8 * h + j];
                    const __bf16 *vr = Vt + (lane % 32) * C::VSTR + kb * 32 + h * 16 + 8 * (lane / 32);
#pragma unroll
                    for (int mb = 0; mb < C::ND; ++mb) {
                        const bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(vr + mb * 32 * C::VSTR);
                        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, o[mb], 0, 0, 0);
                    }
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                bf16x4_t pf;
#pragma unroll
                for (int j = 0; j < 4; ++j) pf[j] = (__bf16)s[kb][j];
                const __bf16 *vr = Vt + (lane % 16) * C::VSTR + kb * 16 + 4 * (lane / 16);
#pragma unroll
                for (int mb = 0; mb < C::ND; ++mb) {
                    const bf16x4_t va = *reinterpret_cast<const bf16x4_t *>(vr + mb * 16 * C::VSTR);
                    o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(i16x4_t, va), __builtin_bit_cast(i16x4_t, pf), o[mb], 0, 0, 0);
                }
            }
        }
    };

    __bf16 *Ks0 = smem;
    __bf16 *Vt0 = smem + C::KTILE;
    TileRegs<C> regs;
    int t = next_tile(0);
    if constexpr (C::PREFETCH) {
        __bf16 *Ks1 = smem + C::KTILE + C::VTILE;
        __bf16 *Vt1 = Ks1 + C::KTILE;
        if (t < ntiles) {
            load_tile<C, D, BC>(regs, K, V, t, kv_len, tid, 0, 1 << 20);
            store_tile<C, D, BC, MF>(regs, Ks0, Vt0, tid, 0, 1 << 20);
        }
        __syncthreads();
        int cur = 0;
        while (t < ntiles) {
            const int tn = next_tile(t + 1);
            if (tn < ntiles) load_tile<C, D, BC>(regs, K, V, tn, kv_len, tid, 0, 1 << 20);
            compute(t, cur ? Ks1 : Ks0, cur ? Vt1 : Vt0);
            if (tn < ntiles) store_tile<C, D, BC, MF>(regs, cur ? Ks0 : Ks1, cur ? Vt0 : Vt1, tid, 0, 1 << 20);
            __syncthreads();
            cur ^= 1;
            t = tn;
        }
    } else {
        // Synchronous staging, two register batches at a time.
        constexpr int STEP = 2;
        constexpr int NPASS = (C::KPT > C::VPT ? C::KPT : C::VPT);
        while (t < ntiles) {
            __syncthreads();
#pragma unroll
            for (int f = 0; f < NPASS; f += STEP) {
                load_tile<C, D, BC>(regs, K, V, t, kv_len, tid, f, STEP);
                store_tile<C, D, BC, MF>(regs, Ks0, Vt0, tid, f, STEP);
            }
            __syncthreads();
            compute(t, Ks0, Vt0);
            t = next_tile(t + 1);
        }
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

template <int D, int BC, int MF, int NW, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs &a, hipStream_t stream) {
    using C = Cfg<D, BC, MF, NW, CAUSAL>;
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
        FA_BF16_BOTH(64, 128, 64),
        FA_BF16_ROW(128, 16),
        FA_BF16_ROW(128, 32),
        FA_BF16_ROW(128, 64),
        FA_BF16_ROW(128, 128),
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
