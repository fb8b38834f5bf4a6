// Exact attention forward with fp32 inputs, outputs and arithmetic (gfx950).
//
// Same tiled method and running-statistics recurrence as the bf16 kernel
// (see fa_fwd_bf16.hip), with the two products on the fp32 matrix-core
// instruction v_mfma_f32_32x32x2_f32 and no rounding of the probabilities.
// This is the precision path of the numeric study on the page "Is Flash
// Attention Stable?" explainer (aibr.jp, section 3: the tiled kernel compared
// against an FP64 golden value at more than one precision); it is not tuned
// for speed.  K and V tiles are staged row-major in LDS (one buffer), one
// wavefront owns MF query rows (MF = 32, or 16 when Br or Bc is 16, on
// v_mfma_f32_16x16x4_f32) and computes S^T = K Q^T and O^T += V^T P^T.
// Every (Br, Bc) in {16, 32, 64, 128}^2 is built for the deviation study:
// with nothing rounded to a 16-bit type, the rescaling steps of the running
// softmax (one per key tile, so ceil(keys / Bc) of them) are among the few
// roundings left, which is the effect of tile size the study looks at.
#include "fa_common.h"

namespace fa {
namespace {

// Shapes of the two fp32 matrix-core instructions.  32x32x2: lane l feeds
// row/column l%32 at depth l/32; accumulator register i of lane l holds row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.  16x16x4: lane l feeds row/column
// l%16 at depth l/16; register i of lane l holds row 4*(l/16) + i, column
// l%16.
template <int MF>
struct F32Frag;
template <>
struct F32Frag<32> {
    using acc_t = f32x16_t;
    static constexpr int ACC = 16, DEPTH = 2, LG = 32;
    __device__ static acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
};
template <>
struct F32Frag<16> {
    using acc_t = f32x4_t;
    static constexpr int ACC = 4, DEPTH = 4, LG = 16;
    __device__ static acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 4 * (lane >> 4) + i; }
};

template <int D, int BC, int MF, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_f32_kernel(FwdArgs a) {
    using F = F32Frag<MF>;
    using acc_t = typename F::acc_t;
    constexpr int NT = NW * 64, BR = MF * NW;
    constexpr int KSTR = D + 1;  // odd stride: the rows of a K read hit distinct banks
    constexpr int VSTR = D;
    constexpr int ND = D / MF;   // output blocks
    constexpr int NKB = BC / MF; // score blocks per tile
    constexpr int NQ = D / F::DEPTH;
    static_assert(BC % MF == 0 && D % MF == 0, "tile must be a multiple of the instruction edge");
    __shared__ float Ks[BC * KSTR];
    __shared__ float Vs[BC * VSTR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.N;
    const int nqt = (N + BR - 1) / BR;
    int bh, qt;
    tile_of_block(nqt, CAUSAL, 1, &bh, &qt);
    const int b = bh / a.H;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t kvhead = (int64_t)kv_head_of(bh, a) * N * D;
    const float *Q = reinterpret_cast<const float *>(a.q) + head;
    const float *K = reinterpret_cast<const float *>(a.k) + kvhead;
    const float *V = reinterpret_cast<const float *>(a.v) + kvhead;
    float *O = reinterpret_cast<float *>(a.o) + head;

    const int q0 = qt * BR, wq0 = q0 + wave * MF, qrow = wq0 + lane % MF;
    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    // Query rows of a workgroup lie in one 128-row mask block (BR <= 128).
    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;

    const float c = scale_factor(a.scale_log2);
    const float qsign = a.scale_log2 < 0.f ? -1.f : 1.f;
    // B operand of S^T = K Q^T: lane l holds Q[qrow][DEPTH*ks + l/LG].
    float qf[NQ];
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks)
        qf[ks] = qrow < N ? qsign * Q[(int64_t)qrow * D + F::DEPTH * ks + lane / F::LG] : 0.f;

    acc_t o[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < F::ACC; ++i) o[mb][i] = 0.f;
    float m = kNegInf, l = 0.f;

    for (int t = 0; t < ntiles; ++t) {
        // Tiles of at most 128 keys lie in one 128-key mask block.
        if (mrow && mrow[(t * BC) >> 7] == 0) continue;
        const int kbase = t * BC;
        __syncthreads();
        for (int e = tid; e < BC * D; e += NT) {
            const int r = e / D, col = e % D, key = kbase + r;
            const bool ok = key < kv_len;
            Ks[r * KSTR + col] = ok ? K[(int64_t)key * D + col] : 0.f;
            Vs[r * VSTR + col] = ok ? V[(int64_t)key * D + col] : 0.f;
        }
        __syncthreads();
        if (wq0 >= N || (CAUSAL && kbase > wq0 + MF - 1)) continue;

        acc_t s[NKB];
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) s[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks)
                s[kb] = F::mma(Ks[(kb * MF + lane % MF) * KSTR + F::DEPTH * ks + lane / F::LG], qf[ks], s[kb]);
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) {
                const int key = kbase + kb * MF + F::row(i, lane);
                const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                s[kb][i] = ok ? s[kb][i] : kNegInf;
                mx = fmaxf(mx, s[kb][i]);
            }
        }
        mx = group_max<MF>(mx);
        const float m_tile = mx == kNegInf ? kNegInf : mx * c;
        const float m_new = fmaxf(m, m_tile);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) {
                const float p = fast_exp2(fmaf(s[kb][i], c, -m_use));  // exp2(-inf) = 0
                s[kb][i] = p;
                rs += p;
            }
        l = fmaf(l, alpha, rs);
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) o[mb][i] *= alpha;
        m = m_new;
        // O^T += V^T P^T.  Instruction i of score block kb takes, in lane
        // group g = l/LG, the key its score register i holds there
        // (row(i, lane)) as depth g: the lane's own P value is the B operand
        // and V at that key and the lane's output dimension the A operand.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) {
                const int key = kb * MF + F::row(i, lane);
#pragma unroll
                for (int mb = 0; mb < ND; ++mb)
                    o[mb] = F::mma(Vs[key * VSTR + mb * MF + lane % MF], s[kb][i], o[mb]);
            }
    }

    const float l_tot = group_sum<MF>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *orow = O + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int i = 0; i < F::ACC; ++i) orow[mb * MF + F::row(i, lane)] = o[mb][i] * inv;
        if (a.lse && lane < MF)
            a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

template <int D, int BR, int BC, bool CAUSAL>
hipError_t launch_f32(const FwdArgs &a, hipStream_t stream) {
    constexpr int MF = (BR == 16 || BC == 16) ? 16 : 32;
    constexpr int NW = BR / MF;
    const int nqt = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_f32_kernel<D, BC, MF, NW, CAUSAL>), dim3((unsigned)(nqt * a.B * a.H)),
                       dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

#define FA_F32(D, BR, BC) \
    Instance{D, 0, BR, BC, &launch_f32<D, BR, BC, false>}, Instance{D, 1, BR, BC, &launch_f32<D, BR, BC, true>}
#define FA_F32_ROW(D, BR) FA_F32(D, BR, 16), FA_F32(D, BR, 32), FA_F32(D, BR, 64), FA_F32(D, BR, 128)

}  // namespace

const Instance *f32_instances() {
    // The default (128, 32) first; every (Br, Bc) in {16, 32, 64, 128}^2.
    static const Instance table[] = {
        FA_F32_ROW(64, 16), FA_F32_ROW(64, 32), FA_F32_ROW(64, 64), FA_F32_ROW(64, 128),
        FA_F32_ROW(128, 16), FA_F32_ROW(128, 32), FA_F32_ROW(128, 64), FA_F32_ROW(128, 128),
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

void f32_default_tile(int d, int *br, int *bc) {
    (void)d;
    *br = 128;
    *bc = 32;
}

}  // namespace fa
