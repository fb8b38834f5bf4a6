// Internal interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a forward kernel needs, passed by value as the kernel argument.
struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;                 // may be null: no logsumexp written
    const int32_t *key_len;     // may be null
    const uint8_t *block_mask;  // may be null; ceil(N/128)^2 bytes
    int B, H, N;
    int Hkv;                    // key/value heads (H for plain multi-head attention)
    int group;                  // H / Hkv query heads per key/value head
    int nkb;                    // ceil(N/128): row length of block_mask
    int order;                  // key-tile visit order: 0 ascending, 1 descending, 2 shuffled
                                // (tile-study kernels only)
    float scale_log2;           // softmax scale * log2(e), fp32
    // Key-range split (fa_fwd_ws): nsplit workgroups per query tile, each
    // over a contiguous share of its key tiles, writing fp32 partial O
    // (normalised by its own row sum) to part_o [nsplit][B*H*N][d] and its
    // natural-log partial LSE to part_l [nsplit][B*H*N]; a merge kernel
    // combines them.  nsplit = 1: no split, part_o/part_l unused.
    int nsplit;
    float *part_o, *part_l;
};

// Key-range split the forward uses for a shape when given a workspace, and
// the workspace bytes it then needs (0 when no split is worth it).
int fwd_split(int B, int H, int N, bool causal);
uint64_t fwd_split_bytes(int B, int H, int N, int d, int nsplit);
uint64_t fwd_workspace_bytes(int B, int H, int N, int d);

// Enqueues the split forward (tuned kernel with key ranges, then the merge)
// for bf16 (f16 = 0) or fp16 (f16 = 1).
hipError_t launch_fwd_split(const FwdArgs &a, int d, int causal, int f16, hipStream_t stream);

// Enqueues the d = 64 forward at four workgroups per CU (fwd_flat) for
// bf16 (f16 = 0) or fp16 (f16 = 1); same arguments and results as the tuned
// kernel.
hipError_t launch_fwd_flat(const FwdArgs &a, int causal, int f16, hipStream_t stream);

// Enqueues the materialised baseline attention (scores to the workspace,
// row softmax in place, then A V) for dtype 0 bf16, 1 fp32, 2 fp16 or 3 bf16
// in / fp32 out; inter_f32 = 1 holds S and A in fp32, 0 in the input type.
hipError_t launch_baseline(const void *q, const void *k, const void *v, void *o, float *lse,
                           const int32_t *key_len, const uint8_t *block_mask, void *ws, int B, int H,
                           int N, int d, float scale, int causal, int dtype, int inter_f32,
                           hipStream_t stream);

// Everything the backward kernels need.
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // bf16 or fp16 [B,H,N,d] (k, v: [B,Hkv,N,d])
    const float *lse;                  // [B,H,N], natural log, from the forward
    float *delta;                      // [B,H,N] workspace: dO_i . O_i
    void *dq, *dk, *dv;                // outputs (dk, dv: [B,Hkv,N,d])
    const int32_t *key_len;
    const uint8_t *block_mask;
    int B, H, N;
    int Hkv, group;
    int nkb;
    float scale;       // softmax scale
    float scale_log2;  // scale * log2(e)
    // Splits for grids too small for the GPU (fa_bwd_ex with a workspace).
    // dK/dV: the sequence of (query head, query tile) steps of each key
    // block is cut into nsplit contiguous ranges, one workgroup each, writing
    // fp32 partial dK (before the scale) and dV to part
    // ([nsplit][2][B*Hkv*N*d], dK then dV).  dQ: the key tiles of each
    // query tile are cut into nsplit_q ranges, writing fp32 partial dQ
    // (before the scale) to part_q ([nsplit_q][B*H*N*d]).  Reduce kernels
    // add the partials.  1: no split, the buffer is unused.
    int nsplit;
    float *part;
    int nsplit_q;
    float *part_q;
};

// Splits the backward uses for a shape when given a workspace (dK/dV and
// dQ), and the workspace bytes they then need (0 when no split is worth it).
int bwd_split(int B, int H, int Hkv, int N, bool causal);
int bwd_split_q(int B, int H, int N, bool causal);
uint64_t bwd_workspace_bytes(int B, int H, int Hkv, int N, int d);

// Enqueues the backward kernels on `stream`.
hipError_t launch_bwd(const BwdArgs &a, int d, int causal, int f16, hipStream_t stream);

// Enqueues one forward pass on `stream`; returns the launch status.
using Launcher = hipError_t (*)(const FwdArgs &, hipStream_t);

// One compiled kernel instance.
struct Instance {
    int d;
    int causal;
    int br;  // query rows per workgroup tile
    int bc;  // key rows per tile
    Launcher launch;
};

// Tables of the instances each translation unit builds (terminated by an
// entry with launch == nullptr): the tuned bf16 kernels, the bf16
// tile-size-study kernels and the fp32 kernels; and the default tile per head
// size.  Tuned bf16 tiles with Br > 128 do not take a block mask.
const Instance *bf16_tuned_instances();
const Instance *f16_tuned_instances();
const Instance *bf16_instances();
const Instance *bf16_f32out_instances();
const Instance *bf16_acc16_instances();
const Instance *f32_instances();
void bf16_default_tile(int d, int block_sparse, int *br, int *bc);
void f32_default_tile(int d, int *br, int *bc);

}  // namespace fa
