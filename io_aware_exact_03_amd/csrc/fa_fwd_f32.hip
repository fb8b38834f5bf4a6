// Exact attention forward with fp32 inputs, outputs and arithmetic (gfx950).
//
// Same tiled method and running-statistics recurrence as the bf16 kernel
// (see fa_fwd_bf16.hip), with the two products on the fp32 matrix-core
// instruction v_mfma_f32_32x32x2_f32 and no rounding of the probabilities.
// This is the precision path of the numeric study on the page "Is Flash
// Attention Stable?" explainer (aibr.jp, section 3: the tiled kernel compared
// against an FP64 golden value at more than one precision); it is not tuned
// for speed.  K and V tiles are staged row-major in LDS (one buffer), one
// wavefront owns 32 query rows and computes S^T = K Q^T and O^T += V^T P^T.
#include "fa_common.h"

namespace fa {
namespace {

constexpr int kBcF32 = 32;
constexpr int kNwF32 = 4;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNwF32 * 64) void fwd_f32_kernel(FwdArgs a) {
    constexpr int BC = kBcF32, NW = kNwF32, NT = NW * 64, BR = 32 * NW;
    constexpr int KSTR = D + 1;  // odd stride: the 32 rows of a K read hit distinct banks
    constexpr int VSTR = D;
    constexpr int ND = D / 32;
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

    const int q0 = qt * BR, wq0 = q0 + wave * 32, qrow = wq0 + lane % 32;
    int kv_len = N;
    if (a.key_len) kv_len = min(max(a.key_len[b], 0), N);
    int kv_end = kv_len;
    if (CAUSAL) kv_end = min(kv_end, q0 + BR);
    const int ntiles = (kv_end + BC - 1) / BC;
    const uint8_t *mrow = a.block_mask ? a.block_mask + (int64_t)(q0 >> 7) * a.nkb : nullptr;

    const float c = scale_factor(a.scale_log2);
    const float qsign = a.scale_log2 < 0.f ? -1.f : 1.f;
    // B operand of the 32x32x2 instruction: lane l holds Q[qrow][2*ks + l/32].
    float qf[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
        qf[ks] = qrow < N ? qsign * Q[(int64_t)qrow * D + 2 * ks + lane / 32] : 0.f;

    f32x16_t o[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
    float m = kNegInf, l = 0.f;

    for (int t = 0; t < ntiles; ++t) {
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
        if (wq0 >= N || (CAUSAL && kbase > wq0 + 31)) continue;

        f32x16_t s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(lane % 32) * KSTR + 2 * ks + lane / 32],
                                                     qf[ks], s, 0, 0, 0);
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
            s[i] = ok ? s[i] : kNegInf;
            mx = fmaxf(mx, s[i]);
        }
        mx = group_max<32>(mx);
        const float m_tile = mx == kNegInf ? kNegInf : mx * c;
        const float m_new = fmaxf(m, m_tile);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(s[i], c, -m_use));  // exp2(-inf) = 0
            s[i] = p;
            rs += p;
        }
        l = fmaf(l, alpha, rs);
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
        m = m_new;
        // O^T += V^T P^T, two keys per instruction: the lower half-wave
        // supplies key row(i, lane) and the upper half-wave the key four rows
        // further; each lane reads V at its own key and output dimension.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
#pragma unroll
            for (int mb = 0; mb < ND; ++mb)
                o[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + mb * 32 + lane % 32], s[i],
                                                             o[mb], 0, 0, 0);
        }
    }

    const float l_tot = group_sum<32>(l);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *orow = O + (int64_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < ND; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = o[mb][4 * g + j] * inv;
                *reinterpret_cast<f32x4_t *>(orow + mb * 32 + 8 * g + 4 * (lane / 32)) = w;
            }
        if (a.lse && lane < 32)
            a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs &a, hipStream_t stream) {
    constexpr int BR = 32 * kNwF32;
    const int nqt = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(nqt * a.B * a.H)),
                       dim3(kNwF32 * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

const Instance *f32_instances() {
    static const Instance table[] = {
        Instance{64, 0, 32 * kNwF32, kBcF32, &launch_f32<64, false>},
        Instance{64, 1, 32 * kNwF32, kBcF32, &launch_f32<64, true>},
        Instance{128, 0, 32 * kNwF32, kBcF32, &launch_f32<128, false>},
        Instance{128, 1, 32 * kNwF32, kBcF32, &launch_f32<128, true>},
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

void f32_default_tile(int d, int *br, int *bc) {
    (void)d;
    *br = 32 * kNwF32;
    *bc = kBcF32;
}

}  // namespace fa
