// C ABI of the attention library (forward and backward): argument validation (before any
// HIP call), tile selection and kernel launch.  Semantics are documented in
// include/fa.h.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "fa_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// Static scratch of fa_fwd_noalloc: the key-range split's fp32 partials
// (partial O, then partial LSE), one copy per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
__device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call there), or 0 with the HIP error in *err.
uintptr_t scratch_on_current_device(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return 0;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return 0;
    }
    uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *addr = nullptr;
    *err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !addr) {
        if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
        return 0;
    }
    // Concurrent first calls store the same address.
    g_scratch_addr[dev].store(reinterpret_cast<uintptr_t>(addr), std::memory_order_release);
    return reinterpret_cast<uintptr_t>(addr);
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// True when the byte ranges [a, a + a_bytes) and [b, b + b_bytes) intersect.
bool overlaps(const void *a, uint64_t a_bytes, const void *b, uint64_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

bool known_dtype(int dtype) {
    return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_F16 ||
           dtype == FA_DTYPE_BF16_F32OUT || dtype == FA_DTYPE_BF16_ACC16;
}

// Bytes per element of q/k/v and of o for a dtype code.
uint64_t in_elem(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }
uint64_t out_elem(int dtype) { return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_BF16_F32OUT ? 4 : 2; }

const fa::Instance *find(const fa::Instance *table, int d, int causal, int br, int bc) {
    for (const fa::Instance *e = table; e->launch; ++e)
        if (e->d == d && e->causal == causal && e->br == br && e->bc == bc) return e;
    return nullptr;
}

// Resolves (dtype, d, Br, Bc) to a built kernel.  Br = Bc = 0 selects the
// tuned default for the head size (a 128-row tile when a block mask is
// given); an explicit pair selects the tile-study kernel of that shape if
// there is one, else a tuned kernel of that shape.  Tuned tiles taller than
// one 128-token mask block do not take a block mask.
int resolve_tile(int dtype, int d, int block_sparse, int br, int bc, int causal,
                 const fa::Instance **out, int *br_out, int *bc_out, bool *study = nullptr) {
    if (study) *study = false;
    if (!known_dtype(dtype)) return FA_ERR_UNSUPPORTED_TILE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    const fa::Instance *inst = nullptr;
    if (dtype == FA_DTYPE_BF16_F32OUT || dtype == FA_DTYPE_BF16_ACC16) {
        // Output modes of the deviation study: the tile-study kernels only
        // (default (128, 64)).
        if (br == 0 && bc == 0) {
            br = 128;
            bc = 64;
        }
        inst = find(dtype == FA_DTYPE_BF16_F32OUT ? fa::bf16_f32out_instances() : fa::bf16_acc16_instances(), d,
                    causal, br, bc);
        if (inst && study) *study = true;
    } else if (dtype == FA_DTYPE_F32) {
        if (br == 0 && bc == 0) fa::f32_default_tile(d, &br, &bc);
        inst = find(fa::f32_instances(), d, causal, br, bc);
    } else if (dtype == FA_DTYPE_F16) {
        if (br == 0 && bc == 0) fa::bf16_default_tile(d, block_sparse, &br, &bc);
        inst = find(fa::f16_tuned_instances(), d, causal, br, bc);
    } else if (br == 0 && bc == 0) {
        fa::bf16_default_tile(d, block_sparse, &br, &bc);
        inst = find(fa::bf16_tuned_instances(), d, causal, br, bc);
    } else {
        inst = find(fa::bf16_instances(), d, causal, br, bc);
        if (inst && study) *study = true;
        if (!inst && (!block_sparse || br <= 128)) inst = find(fa::bf16_tuned_instances(), d, causal, br, bc);
    }
    if (!inst) return FA_ERR_UNSUPPORTED_TILE;
    if (out) *out = inst;
    *br_out = br;
    *bc_out = bc;
    return FA_OK;
}

int forward(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
            int Hkv, int N, int d, float scale, int causal, const int32_t *key_len,
            const uint8_t *block_mask, hipStream_t stream, int dtype, int br, int bc,
            int order = FA_ORDER_ASCENDING, void *workspace = nullptr, size_t workspace_bytes = 0,
            bool static_scratch = false) {
    if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
    if (B < 1 || H < 1 || N < 1 || Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!known_dtype(dtype)) return FA_ERR_UNSUPPORTED_TILE;
    // Grid size limit: B*H*ceil(N/16) workgroups at the smallest tile.
    const uint64_t groups = (uint64_t)B * (uint64_t)H * (((uint64_t)N + 15) / 16);
    if (groups >= (1ull << 31)) return FA_ERR_INVALID_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return FA_ERR_MISALIGNED;
    if ((lse && !aligned(lse, 4)) || (key_len && !aligned(key_len, 4))) return FA_ERR_MISALIGNED;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    const uint64_t bytes = (uint64_t)B * H * N * d * in_elem(dtype);
    const uint64_t o_bytes = (uint64_t)B * H * N * d * out_elem(dtype);
    const uint64_t kv_bytes = (uint64_t)B * Hkv * N * d * in_elem(dtype);
    // Outputs (o, and lse when given) must not overlap any input or each
    // other: a workgroup writing them while others still read the inputs
    // would corrupt the result silently.
    const uint64_t lse_bytes = (uint64_t)B * H * N * sizeof(float);
    const struct { const void *p; uint64_t n; } ins[] = {{q, bytes}, {k, kv_bytes}, {v, kv_bytes}};
    const struct { const void *p; uint64_t n; } outs[] = {{o, o_bytes}, {lse, lse ? lse_bytes : 0}};
    for (const auto &w : outs) {
        if (!w.p) continue;
        for (const auto &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_INVALID_ARG;
    }
    if (lse && overlaps(lse, lse_bytes, o, o_bytes)) return FA_ERR_INVALID_ARG;

    if (order != FA_ORDER_ASCENDING && order != FA_ORDER_DESCENDING && order != FA_ORDER_SHUFFLED)
        return FA_ERR_INVALID_ARG;
    int tbr = 0, tbc = 0;
    const fa::Instance *inst = nullptr;
    bool study = false;
    const int rc = resolve_tile(dtype, d, block_mask != nullptr, br, bc, causal ? 1 : 0, &inst, &tbr,
                                &tbc, &study);
    if (rc != FA_OK) return rc;
    if (order != FA_ORDER_ASCENDING && !study) return FA_ERR_UNSUPPORTED_TILE;
    // Key-range split (fa_fwd_ws): used when a workspace is given and the
    // shape gains from it; bf16/fp16 with the tuned tile only.  With the
    // static scratch (fa_fwd_noalloc) the workspace is the library's own
    // array, looked up only now that every argument has been checked.
    const bool splittable = dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16;
    const int nsplit = splittable ? fa::fwd_split(B, H, N, causal != 0) : 1;
    const uint64_t need = fa::fwd_split_bytes(B, H, N, d, nsplit);
    if (static_scratch && need > 0) {
        if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_INVALID_SHAPE;
        hipError_t e = hipSuccess;
        const uintptr_t p = scratch_on_current_device(&e);
        if (!p) {
            g_last_hip_error = (int)e;
            return FA_ERR_HIP;
        }
        workspace = reinterpret_cast<void *>(p);
        workspace_bytes = FA_NOALLOC_SCRATCH_BYTES;
    }
    const bool split = workspace && need > 0;
    if (split) {
        if (workspace_bytes < need || !aligned(workspace, 16)) return FA_ERR_INVALID_ARG;
        if (overlaps(workspace, need, q, bytes) || overlaps(workspace, need, k, kv_bytes) ||
            overlaps(workspace, need, v, kv_bytes) || overlaps(workspace, need, o, o_bytes) ||
            (lse && overlaps(workspace, need, lse, lse_bytes)))
            return FA_ERR_INVALID_ARG;
    }

    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.key_len = key_len;
    a.block_mask = block_mask;
    a.B = B;
    a.H = H;
    a.N = N;
    a.Hkv = Hkv;
    a.group = H / Hkv;
    a.nkb = (N + 127) / 128;
    a.order = order;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.nsplit = split ? nsplit : 1;
    const uint64_t rows = (uint64_t)B * H * N;
    a.part_o = split ? static_cast<float *>(workspace) : nullptr;
    a.part_l = split ? static_cast<float *>(workspace) + (uint64_t)a.nsplit * rows * d : nullptr;

    const hipError_t err = split ? fa::launch_fwd_split(a, d, causal ? 1 : 0, dtype == FA_DTYPE_F16 ? 1 : 0, stream)
                                 : inst->launch(a, stream);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return FA_ERR_HIP;
    }
    return FA_OK;
}

// Element bytes of the baseline's intermediate type, or 0 when the
// (dtype, inter_dtype) pair is not built: S and A in fp32, or in the input
// type of a 16-bit dtype.
uint64_t baseline_inter_bytes(int dtype, int inter) {
    if (dtype == FA_DTYPE_BF16_ACC16 || !known_dtype(dtype)) return 0;
    if (inter == FA_DTYPE_F32) return 4;
    if (inter == FA_DTYPE_BF16 && (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_BF16_F32OUT)) return 2;
    if (inter == FA_DTYPE_F16 && dtype == FA_DTYPE_F16) return 2;
    return 0;
}

int baseline(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
             int d, float scale, int causal, const int32_t *key_len, const uint8_t *block_mask,
             hipStream_t stream, int dtype, int inter, void *workspace, size_t workspace_bytes) {
    if (!q || !k || !v || !o || !workspace) return FA_ERR_NULL_PTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    const uint64_t ib = baseline_inter_bytes(dtype, inter);
    if (!ib) return FA_ERR_UNSUPPORTED_TILE;
    // Grids: B*H*ceil(N/128)^2 score blocks and B*H*N softmax rows.
    const uint64_t nt = ((uint64_t)N + 127) / 128, bhn = (uint64_t)B * H;
    if (bhn * nt * nt >= (1ull << 31) || bhn * N >= (1ull << 31)) return FA_ERR_INVALID_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(workspace, 16))
        return FA_ERR_MISALIGNED;
    if ((lse && !aligned(lse, 4)) || (key_len && !aligned(key_len, 4))) return FA_ERR_MISALIGNED;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    const uint64_t need = bhn * N * (uint64_t)N * ib;
    if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
    const uint64_t bytes = bhn * N * d * in_elem(dtype), o_bytes = bhn * N * d * out_elem(dtype);
    const uint64_t lse_bytes = bhn * N * sizeof(float);
    const struct { const void *p; uint64_t n; } ins[] = {{q, bytes}, {k, bytes}, {v, bytes}};
    const struct { const void *p; uint64_t n; } outs[] = {{o, o_bytes}, {lse, lse ? lse_bytes : 0},
                                                          {workspace, need}};
    for (const auto &w : outs) {
        if (!w.p) continue;
        for (const auto &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_INVALID_ARG;
        for (const auto &w2 : outs)
            if (&w2 != &w && w2.p && overlaps(w.p, w.n, w2.p, w2.n)) return FA_ERR_INVALID_ARG;
    }
    const hipError_t err = fa::launch_baseline(q, k, v, o, lse, key_len, block_mask, workspace, B, H, N, d,
                                               scale, causal ? 1 : 0, dtype, inter == FA_DTYPE_F32 ? 1 : 0,
                                               stream);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return FA_ERR_HIP;
    }
    return FA_OK;
}

int backward(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int H, int Hkv,
             int N, int d, float scale, int causal, const int32_t *key_len,
             const uint8_t *block_mask, hipStream_t stream, int dtype, void *workspace = nullptr,
             size_t workspace_bytes = 0) {
    if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return FA_ERR_NULL_PTR;
    if (B < 1 || H < 1 || N < 1 || Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED_TILE;
    const uint64_t groups = (uint64_t)B * (uint64_t)H * (((uint64_t)N + 15) / 16);
    if (groups >= (1ull << 31)) return FA_ERR_INVALID_SHAPE;
    const void *a16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : a16)
        if (!aligned(p, 16)) return FA_ERR_MISALIGNED;
    if (!aligned(lse, 4) || !aligned(delta, 4) || (key_len && !aligned(key_len, 4))) return FA_ERR_MISALIGNED;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    const uint64_t qb = (uint64_t)B * H * N * d * 2, kvb = (uint64_t)B * Hkv * N * d * 2;
    const uint64_t rb = (uint64_t)B * H * N * 4;
    // outputs and the workspace must not overlap any input or each other
    const struct { const void *p; uint64_t n; } ins[] = {{q, qb}, {k, kvb}, {v, kvb}, {o, qb}, {dout, qb},
                                                         {lse, rb}};
    // A workspace is used only when the shape gains from a query-head split
    // (fa::bwd_workspace_bytes > 0); given but too small is an error.
    const uint64_t need = fa::bwd_workspace_bytes(B, H, Hkv, N, d);
    const bool split = workspace && need > 0;
    if (split && (workspace_bytes < need || !aligned(workspace, 16))) return FA_ERR_INVALID_ARG;
    const struct { const void *p; uint64_t n; } outs[] = {{dq, qb}, {dk, kvb}, {dv, kvb}, {delta, rb},
                                                          {split ? workspace : nullptr, split ? need : 0}};
    for (const auto &w : outs) {
        if (!w.p) continue;
        for (const auto &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_INVALID_ARG;
        for (const auto &w2 : outs)
            if (&w2 != &w && w2.p && overlaps(w.p, w.n, w2.p, w2.n)) return FA_ERR_INVALID_ARG;
    }
    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.key_len = key_len;
    a.block_mask = block_mask;
    a.B = B;
    a.H = H;
    a.N = N;
    a.Hkv = Hkv;
    a.group = H / Hkv;
    a.nkb = (N + 127) / 128;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.nsplit = split ? fa::bwd_split(B, H, Hkv, N, causal != 0) : 1;
    a.nsplit_q = split ? fa::bwd_split_q(B, H, N, causal != 0) : 1;
    a.part = split && a.nsplit > 1 ? static_cast<float *>(workspace) : nullptr;
    a.part_q = nullptr;
    if (split && a.nsplit_q > 1) {
        const uint64_t kv_part = a.nsplit > 1 ? (uint64_t)a.nsplit * 2 * B * Hkv * (uint64_t)N * d : 0;
        a.part_q = static_cast<float *>(workspace) + kv_part;
    }
    const hipError_t err = fa::launch_bwd(a, d, causal ? 1 : 0, dtype == FA_DTYPE_F16 ? 1 : 0, stream);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return FA_ERR_HIP;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
           int d, float scale, int causal, const int32_t *key_len, const uint8_t *block_mask,
           hipStream_t stream) {
    return forward(q, k, v, o, lse, B, H, H, N, d, scale, causal, key_len, block_mask, stream,
                   FA_DTYPE_BF16, 0, 0);
}

int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B, int H,
               int N, int d, float scale, int causal, const int32_t *key_len,
               const uint8_t *block_mask, hipStream_t stream) {
    return forward(q, k, v, o, lse, B, H, H, N, d, scale, causal, key_len, block_mask, stream,
                   FA_DTYPE_F32, 0, 0);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int N, int d, float scale, int causal, const int32_t *key_len,
              const uint8_t *block_mask, hipStream_t stream, int dtype, int Br, int Bc) {
    return forward(q, k, v, o, lse, B, H, H, N, d, scale, causal, key_len, block_mask, stream, dtype,
                   Br, Bc);
}

int fa_fwd_study(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int N, int d, float scale, int causal, const int32_t *key_len,
                 const uint8_t *block_mask, hipStream_t stream, int dtype, int Br, int Bc,
                 int tile_order) {
    return forward(q, k, v, o, lse, B, H, H, N, d, scale, causal, key_len, block_mask, stream,
                   dtype, Br, Bc, tile_order);
}

int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int H_kv, int N, int d, float scale, int causal, const int32_t *key_len,
              const uint8_t *block_mask, hipStream_t stream, int dtype, void *workspace,
              size_t workspace_bytes) {
    return forward(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream,
                   dtype, 0, 0, FA_ORDER_ASCENDING, workspace, workspace_bytes);
}

int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                   int H_kv, int N, int d, float scale, int causal, const int32_t *key_len,
                   const uint8_t *block_mask, hipStream_t stream, int dtype) {
    return forward(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream,
                   dtype, 0, 0, FA_ORDER_ASCENDING, nullptr, 0, true);
}

size_t fa_fwd_workspace_size(int B, int H, int N, int d, int dtype) {
    if ((d != 64 && d != 128) || B < 1 || H < 1 || N < 1) return 0;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return 0;
    return (size_t)fa::fwd_workspace_bytes(B, H, N, d);
}

int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int H_kv, int N, int d, float scale, int causal, const int32_t *key_len,
               const uint8_t *block_mask, hipStream_t stream, int dtype, int Br, int Bc) {
    return forward(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream,
                   dtype, Br, Bc);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int H, int H_kv,
           int N, int d, float scale, int causal, const int32_t *key_len,
           const uint8_t *block_mask, hipStream_t stream) {
    return backward(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale, causal,
                    key_len, block_mask, stream, FA_DTYPE_BF16);
}

int fa_bwd_ex(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int H, int H_kv,
              int N, int d, float scale, int causal, const int32_t *key_len,
              const uint8_t *block_mask, hipStream_t stream, int dtype, void *workspace,
              size_t workspace_bytes) {
    return backward(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale, causal,
                    key_len, block_mask, stream, dtype, workspace, workspace_bytes);
}

int fa_fwd_baseline(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int N, int d, float scale, int causal, const int32_t *key_len,
                    const uint8_t *block_mask, hipStream_t stream, int dtype, int inter_dtype,
                    void *workspace, size_t workspace_bytes) {
    return baseline(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream, dtype,
                    inter_dtype, workspace, workspace_bytes);
}

size_t fa_fwd_baseline_workspace_size(int B, int H, int N, int dtype, int inter_dtype) {
    const uint64_t ib = baseline_inter_bytes(dtype, inter_dtype);
    if (!ib || B < 1 || H < 1 || N < 1) return 0;
    return (size_t)((uint64_t)B * H * N * (uint64_t)N * ib);
}

size_t fa_bwd_workspace_size(int B, int H, int H_kv, int N, int d) {
    if ((d != 64 && d != 128) || B < 1 || H < 1 || H_kv < 1 || N < 1 || H % H_kv != 0) return 0;
    return (size_t)fa::bwd_workspace_bytes(B, H, H_kv, N, d);
}

int fa_tile_shape(int dtype, int d, int block_sparse, int Br, int Bc, int *br_out, int *bc_out) {
    if (!br_out || !bc_out) return FA_ERR_NULL_PTR;
    return resolve_tile(dtype, d, block_sparse ? 1 : 0, Br, Bc, 0, nullptr, br_out, bc_out);
}

const char *fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL_PTR: return "null pointer argument";
        case FA_ERR_INVALID_SHAPE:
            return "invalid shape (B, H, H_kv, N must be >= 1, H a multiple of H_kv, and the grid must fit)";
        case FA_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension (d must be 64 or 128)";
        case FA_ERR_MISALIGNED: return "misaligned pointer (q/k/v/o need 16 bytes, lse/key_len 4)";
        case FA_ERR_UNSUPPORTED_TILE: return "unsupported dtype or tile shape";
        case FA_ERR_HIP: return "HIP launch error (see fa_last_hip_error)";
        case FA_ERR_INVALID_ARG:
            return "invalid argument (non-finite scale, overlapping output or unknown tile order)";
        default: return "unknown status";
    }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
