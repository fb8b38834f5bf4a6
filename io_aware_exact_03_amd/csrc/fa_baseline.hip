// Materialised ("baseline") attention for gfx950: the standard evaluation
// order that the tiled method is compared against.
//
// The page "Is Flash Attention Stable?" explainer (aibr.jp, opening dialogue
// and sections 3 and 4) measures the output deviation of FlashAttention from
// an FP64 golden value next to that of a Baseline Attention computed in the
// conventional order, at BF16.  This file is that baseline, on the same
// inputs and the same masks as the tiled kernels:
//
//   1. base_scores : S = scale * Q K^T for every (query, key) pair of every
//                    head, written to a caller workspace [B, H, N, N] (the
//                    N x N matrix the tiled method never stores); disallowed
//                    pairs are written as -inf.
//   2. base_softmax: per row, m = max_j S_ij, l = sum_j exp(S_ij - m),
//                    A_ij = exp(S_ij - m) / l written over S in place, and
//                    LSE_i = m + log l (natural log, fp32); a row with no
//                    allowed key gets A = 0 and LSE = -inf.
//   3. base_av     : O = A V, rounded once to the output type.
//
// Precision: the products run on the matrix cores with fp32 accumulation
// (bf16 x bf16, fp16 x fp16 or fp32 x fp32), like the tiled kernels.  S and
// A are held in the workspace either in fp32 or in the input type (one
// rounding each when written); the softmax computes in fp32 either way; A
// enters the A V product rounded to the input type, as P does in the tiled
// kernels.  Key tiles whose A entries are all exactly 0 (past the causal
// diagonal, past key_len, masked blocks) are skipped in A V; every other
// product is computed.  Nothing here is on the hot path; the kernels are
// plain LDS-tiled matrix-core code.
#include "fa_bf16_tiles.h"

namespace fa {
namespace {

// Matrix-core shape per input type: 32x32 output blocks, DEPTH elements of
// the contraction per instruction.  Lane l feeds row/column l%32 and depth
// elements [OFF*(l/32), OFF*(l/32) + OFF) of the instruction's DEPTH.
template <class T>
struct BaseMma;
template <>
struct BaseMma<__bf16> {
    using op_t = bf16x8_t;
    static constexpr int DEPTH = 16, OFF = 8;
    __device__ static f32x16_t mma(op_t a, op_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct BaseMma<_Float16> {
    using op_t = f16x8_t;
    static constexpr int DEPTH = 16, OFF = 8;
    __device__ static f32x16_t mma(op_t a, op_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <>
struct BaseMma<float> {
    using op_t = float;
    static constexpr int DEPTH = 2, OFF = 1;
    __device__ static f32x16_t mma(op_t a, op_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// OFF consecutive elements starting at p, converted to T (round to nearest
// even for 16-bit T); `n` of them are valid, the rest are 0.
template <class T, class S>
__device__ __forceinline__ typename BaseMma<T>::op_t load_op(const S *p, int n) {
    using op_t = typename BaseMma<T>::op_t;
    if constexpr (BaseMma<T>::OFF == 1) {
        return n > 0 ? (float)p[0] : 0.f;
    } else {
        op_t r;
        if constexpr (sizeof(S) == 2 && sizeof(T) == 2) {
            if (n >= 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0)
                return __builtin_bit_cast(op_t, *reinterpret_cast<const u32x4_t *>(p));
        } else if constexpr (sizeof(S) == 4) {
            if (n >= 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
                const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(p);
                const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(p + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[e] = (T)x0[e];
                    r[4 + e] = (T)x1[e];
                }
                return r;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = e < n ? (T)(float)p[e] : (T)0.f;
        return r;
    }
}

// Storage conversion (fp32 -> S, round to nearest even for 16-bit S).
template <class S>
__device__ __forceinline__ S to_store(float x) {
    return (S)x;
}

// Key j allowed for query i of batch entry b (the masks of include/fa.h).
struct BaseArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *key_len;
    const uint8_t *block_mask;
    void *s;  // workspace [B, H, N, N] of the intermediate type
    int B, H, N, nkb, causal;
    float scale;
};

__device__ __forceinline__ int key_limit(const BaseArgs &a, int b) {
    return a.key_len ? min(max(a.key_len[b], 0), a.N) : a.N;
}

// ---------------------------------------------------------------------------
// 1. S = scale * Q K^T.  Workgroup: one 128 x 128 block of one head, 4 waves
// of 32 query rows x 128 keys (four 32 x 32 accumulator blocks).

template <class T, class S, int D>
__global__ __launch_bounds__(256) void base_scores(BaseArgs a) {
    using M = BaseMma<T>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, nt = (N + 127) / 128;
    const int64_t id = blockIdx.x;
    const int bh = (int)(id / ((int64_t)nt * nt));
    const int rest = (int)(id - (int64_t)bh * nt * nt);
    const int qt = rest / nt, kt = rest - qt * nt;
    const int b = bh / a.H;
    const int kv_len = key_limit(a, b);
    const T *Q = reinterpret_cast<const T *>(a.q) + (int64_t)bh * N * D;
    const T *K = reinterpret_cast<const T *>(a.k) + (int64_t)bh * N * D;
    S *Sh = reinterpret_cast<S *>(a.s) + (int64_t)bh * N * N;

    const int q0 = qt * 128 + wave * 32, k0 = kt * 128;
    const bool dead = (a.causal && k0 > qt * 128 + 127) || k0 >= kv_len ||
                      (a.block_mask && a.block_mask[(int64_t)qt * a.nkb + kt] == 0);
    f32x16_t acc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[blk][i] = 0.f;
    if (!dead) {
        const int qr = min(q0 + lane % 32, N - 1);
        const int sub = M::OFF * (lane / 32);
#pragma unroll 2
        for (int ks = 0; ks < D; ks += M::DEPTH) {
            const auto qa = load_op<T>(Q + (int64_t)qr * D + ks + sub, M::OFF);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int kr = min(k0 + blk * 32 + lane % 32, N - 1);
                const auto kb = load_op<T>(K + (int64_t)kr * D + ks + sub, M::OFF);
                acc[blk] = M::mma(qa, kb, acc[blk]);
            }
        }
    }
    // Register i of lane l: query row 8*(i/4) + 4*(l/32) + i%4, key l%32.
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const int j = k0 + blk * 32 + lane % 32;
        if (j >= N) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qi = q0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (qi >= N) continue;
            const bool ok = !dead && j < kv_len && (!a.causal || j <= qi) &&
                            (!a.block_mask || a.block_mask[(int64_t)(qi >> 7) * a.nkb + (j >> 7)] != 0);
            Sh[(int64_t)qi * N + j] = to_store<S>(ok ? a.scale * acc[blk][i] : kNegInf);
        }
    }
}

// ---------------------------------------------------------------------------
// 2. Row softmax in place, fp32 arithmetic: max, then the sum of
// exp(s - max), then the normalised values; LSE = max + log(sum).

__device__ __forceinline__ float block_reduce(float x, bool is_max, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float y = __shfl_xor(x, off, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // red[] free from the previous reduction
    if ((threadIdx.x & 63) == 0) red[wave] = x;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

template <class S>
__global__ __launch_bounds__(256) void base_softmax(BaseArgs a) {
    __shared__ float red[4];
    const int N = a.N;
    const int64_t row = blockIdx.x;
    S *p = reinterpret_cast<S *>(a.s) + row * N;
    float m = kNegInf;
    for (int j = threadIdx.x; j < N; j += blockDim.x) m = fmaxf(m, (float)p[j]);
    m = block_reduce(m, true, red);
    if (m == kNegInf) {
        for (int j = threadIdx.x; j < N; j += blockDim.x) p[j] = to_store<S>(0.f);
        if (a.lse && threadIdx.x == 0) a.lse[row] = kNegInf;
        return;
    }
    float l = 0.f;
    for (int j = threadIdx.x; j < N; j += blockDim.x) l += expf((float)p[j] - m);
    l = block_reduce(l, false, red);
    for (int j = threadIdx.x; j < N; j += blockDim.x) p[j] = to_store<S>(expf((float)p[j] - m) / l);
    if (a.lse && threadIdx.x == 0) a.lse[row] = m + logf(l);
}

// ---------------------------------------------------------------------------
// 3. O = A V.  Workgroup: 128 query rows of one head, 4 waves of 32 rows x D
// outputs; 64-key steps with V staged in LDS transposed (d-major), so the B
// operand (V at 8 consecutive keys of one output column) is one contiguous
// read.  A is read straight from the workspace.

template <class T, class S, class OT, int D>
__global__ __launch_bounds__(256) void base_av(BaseArgs a) {
    using M = BaseMma<T>;
    constexpr int KS = 64;                        // keys per step
    constexpr int VP = KS + 16 / (int)sizeof(T);  // padded row of the transposed V tile
    constexpr int ND = D / 32;
    constexpr int VEC = 16 / (int)sizeof(T);      // elements per 16-byte V load
    __shared__ __attribute__((aligned(16))) T vt[D * VP];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, nqt = (N + 127) / 128;
    const int bh = blockIdx.x / nqt, qt = blockIdx.x - bh * nqt;
    const int b = bh / a.H;
    const T *V = reinterpret_cast<const T *>(a.v) + (int64_t)bh * N * D;
    const S *A = reinterpret_cast<const S *>(a.s) + (int64_t)bh * N * N;
    OT *O = reinterpret_cast<OT *>(a.o) + (int64_t)bh * N * D;

    const int q0 = qt * 128 + wave * 32;
    const int qr = min(q0 + lane % 32, N - 1);
    int kend = key_limit(a, b);
    if (a.causal) kend = min(kend, qt * 128 + 128);
    f32x16_t acc[ND];
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

    for (int k0 = 0; k0 < kend; k0 += KS) {
        // Blocks whose A entries are all 0 (masked 128-key block) add nothing.
        if (a.block_mask && a.block_mask[(int64_t)qt * a.nkb + (k0 >> 7)] == 0) continue;
        __syncthreads();
        for (int c = threadIdx.x; c < KS * (D / VEC); c += 256) {
            const int r = c / (D / VEC), col = (c - r * (D / VEC)) * VEC, key = k0 + r;
            T x[VEC];
            if (key < kend) {
                const u32x4_t raw = *reinterpret_cast<const u32x4_t *>(V + (int64_t)key * D + col);
                __builtin_memcpy(x, &raw, 16);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) x[e] = (T)0.f;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) vt[(col + e) * VP + r] = x[e];
        }
        __syncthreads();
        const int sub = M::OFF * (lane / 32);
#pragma unroll
        for (int kk = 0; kk < KS; kk += M::DEPTH) {
            const int kf = k0 + kk + sub;
            const auto aa = load_op<T>(A + (int64_t)qr * N + kf, min(M::OFF, kend - kf));
#pragma unroll
            for (int mb = 0; mb < ND; ++mb) {
                const T *vp = vt + (mb * 32 + lane % 32) * VP + kk + sub;
                typename M::op_t vb;
                if constexpr (M::OFF == 1)
                    vb = (float)vp[0];
                else
                    vb = __builtin_bit_cast(typename M::op_t, *reinterpret_cast<const u32x4_t *>(vp));
                acc[mb] = M::mma(aa, vb, acc[mb]);
            }
        }
    }
    // Register i of lane l: query row 8*(i/4) + 4*(l/32) + i%4, column l%32.
#pragma unroll
    for (int mb = 0; mb < ND; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qi = q0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (qi < N) O[(int64_t)qi * D + mb * 32 + lane % 32] = (OT)acc[mb][i];
        }
}

template <class T, class S, class OT, int D>
hipError_t launch_three(const BaseArgs &a, hipStream_t stream) {
    const int64_t nt = (a.N + 127) / 128;
    const int64_t bhn = (int64_t)a.B * a.H;
    hipLaunchKernelGGL((base_scores<T, S, D>), dim3((unsigned)(bhn * nt * nt)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((base_softmax<S>), dim3((unsigned)(bhn * a.N)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((base_av<T, S, OT, D>), dim3((unsigned)(bhn * nt)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <class T, class S, class OT>
hipError_t launch_d(const BaseArgs &a, int d, hipStream_t stream) {
    return d == 64 ? launch_three<T, S, OT, 64>(a, stream) : launch_three<T, S, OT, 128>(a, stream);
}

}  // namespace

// dtype: 0 bf16, 1 fp32, 2 fp16, 3 bf16 in / fp32 out; inter_f32: S and A
// held in fp32 (else in the input type).  The caller has validated the
// combination.
hipError_t launch_baseline(const void *q, const void *k, const void *v, void *o, float *lse,
                           const int32_t *key_len, const uint8_t *block_mask, void *ws, int B, int H,
                           int N, int d, float scale, int causal, int dtype, int inter_f32,
                           hipStream_t stream) {
    BaseArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.key_len = key_len;
    a.block_mask = block_mask;
    a.s = ws;
    a.B = B;
    a.H = H;
    a.N = N;
    a.nkb = (N + 127) / 128;
    a.causal = causal;
    a.scale = scale;
    switch (dtype) {
        case 0: return inter_f32 ? launch_d<__bf16, float, __bf16>(a, d, stream)
                                 : launch_d<__bf16, __bf16, __bf16>(a, d, stream);
        case 3: return inter_f32 ? launch_d<__bf16, float, float>(a, d, stream)
                                 : launch_d<__bf16, __bf16, float>(a, d, stream);
        case 2: return inter_f32 ? launch_d<_Float16, float, _Float16>(a, d, stream)
                                 : launch_d<_Float16, _Float16, _Float16>(a, d, stream);
        default: return launch_d<float, float, float>(a, d, stream);
    }
}

}  // namespace fa
