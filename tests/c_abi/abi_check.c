/*
 * The attention library driven from plain C through include/fa.h alone:
 * device buffers from hipMalloc, calls on a caller-created stream, results
 * copied back and compared element by element with the FP64 oracle
 * (oracle/attn_ref.c, linked as test infrastructure).  Inputs come from a
 * seeded splitmix64 stream, rounded to bf16 on the host; the oracle gets the
 * rounded values widened to double.
 *
 *   abi_check                 every case (needs a GPU)
 *   abi_check --errors-only   only the argument checks, which return their
 *                             status before any HIP call (runs without a GPU)
 *
 * Prints one line per case and exits 0 when every case passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

/* The oracle's entry points (oracle/attn_ref.c). */
int attn_ref_f64(const double *q, const double *k, const double *v, double *o, double *lse, int64_t B,
                 int64_t H, int64_t N, int64_t d, double scale, int causal, const int32_t *key_len,
                 const uint8_t *block_mask, int64_t blk);
int attn_bwd_ref_gqa_f64(const double *q, const double *k, const double *v, const double *dout, double *dq,
                         double *dk, double *dv, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                         double scale, int causal, const int32_t *key_len, const uint8_t *block_mask,
                         int64_t blk);

static int failures = 0;

#define EXPECT(cond, ...)                                                                                    \
    do {                                                                                                     \
        if (!(cond)) {                                                                                       \
            printf("FAIL: ");                                                                                \
            printf(__VA_ARGS__);                                                                             \
            printf("\n");                                                                                    \
            ++failures;                                                                                      \
        }                                                                                                    \
    } while (0)

#define HIP_OK(call)                                                                                         \
    do {                                                                                                     \
        hipError_t e_ = (call);                                                                              \
        if (e_ != hipSuccess) {                                                                              \
            printf("FAIL: %s -> %s\n", #call, hipGetErrorString(e_));                                       \
            exit(2);                                                                                         \
        }                                                                                                    \
    } while (0)

/* splitmix64 (Steele, Lea and Flood), mapped to a uniform double in [-2, 2). */
static uint64_t rng_state;
static double uniform(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return ((double)(z >> 11) * 0x1.0p-53) * 4.0 - 2.0;
}

/* float -> bfloat16 bits, round to nearest even (finite inputs). */
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* n bf16 values on the device, their widened copy in *host. */
static void *bf16_tensor(size_t n, double **host)
{
    uint16_t *h = (uint16_t *)malloc(n * 2);
    *host = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        h[i] = to_bf16((float)uniform());
        (*host)[i] = from_bf16(h[i]);
    }
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n * 2));
    HIP_OK(hipMemcpy(d, h, n * 2, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static double *bf16_back(const void *d, size_t n)
{
    uint16_t *h = (uint16_t *)malloc(n * 2);
    HIP_OK(hipMemcpy(h, d, n * 2, hipMemcpyDeviceToHost));
    double *x = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = from_bf16(h[i]);
    free(h);
    return x;
}

/* max |a - b| over rows with a finite reference LSE; rows whose reference
 * LSE is -inf must be exactly O = 0, LSE = -inf. */
static void compare_fwd(const char *what, const double *o, const float *lse, const double *o_ref,
                        const double *lse_ref, int64_t rows, int64_t d, double tol)
{
    double eo = 0.0, el = 0.0;
    int empty_ok = 1;
    for (int64_t r = 0; r < rows; ++r) {
        if (isinf(lse_ref[r])) {
            empty_ok &= isinf(lse[r]) && lse[r] < 0;
            for (int64_t c = 0; c < d; ++c) empty_ok &= o[r * d + c] == 0.0;
            continue;
        }
        el = fmax(el, fabs((double)lse[r] - lse_ref[r]));
        for (int64_t c = 0; c < d; ++c) eo = fmax(eo, fabs(o[r * d + c] - o_ref[r * d + c]));
    }
    printf("%-44s max|dO| %.3e  max|dLSE| %.3e\n", what, eo, el);
    EXPECT(eo <= tol && el <= 1e-3 && empty_ok, "%s: dO %.3e (bar %.0e), dLSE %.3e, empty rows %s", what, eo, tol,
           el, empty_ok ? "ok" : "wrong");
}

/* One bf16 forward through fa_fwd on `stream`, against the oracle. */
static void case_fwd_bf16(hipStream_t stream, int B, int H, int N, int d, int causal, const int32_t *key_len_h,
                          const uint8_t *mask_h)
{
    const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    double *q, *k, *v;
    void *dq = bf16_tensor(n, &q), *dk = bf16_tensor(n, &k), *dv = bf16_tensor(n, &v);
    void *dout = NULL;
    float *dlse = NULL;
    int32_t *dkl = NULL;
    uint8_t *dmask = NULL;
    const int nb = (N + 127) / 128;
    HIP_OK(hipMalloc(&dout, n * 2));
    HIP_OK(hipMalloc((void **)&dlse, rows * 4));
    if (key_len_h) {
        HIP_OK(hipMalloc((void **)&dkl, (size_t)B * 4));
        HIP_OK(hipMemcpy(dkl, key_len_h, (size_t)B * 4, hipMemcpyHostToDevice));
    }
    if (mask_h) {
        HIP_OK(hipMalloc((void **)&dmask, (size_t)nb * nb));
        HIP_OK(hipMemcpy(dmask, mask_h, (size_t)nb * nb, hipMemcpyHostToDevice));
    }
    const float scale = 1.0f / sqrtf((float)d);
    const int st = fa_fwd(dq, dk, dv, dout, dlse, B, H, N, d, scale, causal, dkl, dmask, stream);
    EXPECT(st == FA_OK, "fa_fwd returned %d (%s)", st, fa_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    double *o = bf16_back(dout, n);
    float *lse = (float *)malloc(rows * 4);
    HIP_OK(hipMemcpy(lse, dlse, rows * 4, hipMemcpyDeviceToHost));
    double *o_ref = (double *)malloc(n * sizeof(double)), *lse_ref = (double *)malloc(rows * sizeof(double));
    EXPECT(attn_ref_f64(q, k, v, o_ref, lse_ref, B, H, N, d, (double)scale, causal, key_len_h, mask_h, 128) == 0,
           "oracle failed");
    char what[96];
    snprintf(what, sizeof what, "fa_fwd bf16 B%d H%d N%d d%d%s%s%s", B, H, N, d, causal ? " causal" : "",
             key_len_h ? " key_len" : "", mask_h ? " block_mask" : "");
    compare_fwd(what, o, lse, o_ref, lse_ref, (int64_t)rows, d, 2e-2);
    free(q), free(k), free(v), free(o), free(lse), free(o_ref), free(lse_ref);
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dout), hipFree(dlse), hipFree(dkl), hipFree(dmask);
}

/* fa_fwd_f32 on the default stream, against the oracle at 1e-5. */
static void case_fwd_f32(int N, int d)
{
    const size_t n = (size_t)N * d;
    float *h = (float *)malloc(n * 4 * 3);
    double *x = (double *)malloc(n * sizeof(double) * 3);
    for (size_t i = 0; i < 3 * n; ++i) {
        h[i] = (float)uniform();
        x[i] = (double)h[i];
    }
    float *dbuf = NULL, *dout = NULL, *dlse = NULL;
    HIP_OK(hipMalloc((void **)&dbuf, n * 4 * 3));
    HIP_OK(hipMalloc((void **)&dout, n * 4));
    HIP_OK(hipMalloc((void **)&dlse, (size_t)N * 4));
    HIP_OK(hipMemcpy(dbuf, h, n * 4 * 3, hipMemcpyHostToDevice));
    const float scale = 1.0f / sqrtf((float)d);
    const int st = fa_fwd_f32(dbuf, dbuf + n, dbuf + 2 * n, dout, dlse, 1, 1, N, d, scale, 0, NULL, NULL, 0);
    EXPECT(st == FA_OK, "fa_fwd_f32 returned %d", st);
    HIP_OK(hipDeviceSynchronize());
    float *of = (float *)malloc(n * 4), *lse = (float *)malloc((size_t)N * 4);
    HIP_OK(hipMemcpy(of, dout, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, (size_t)N * 4, hipMemcpyDeviceToHost));
    double *o = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) o[i] = (double)of[i];
    double *o_ref = (double *)malloc(n * sizeof(double)), *lse_ref = (double *)malloc((size_t)N * sizeof(double));
    EXPECT(attn_ref_f64(x, x + n, x + 2 * n, o_ref, lse_ref, 1, 1, N, d, (double)scale, 0, NULL, NULL, 128) == 0,
           "oracle failed");
    char what[64];
    snprintf(what, sizeof what, "fa_fwd_f32 B1 H1 N%d d%d", N, d);
    compare_fwd(what, o, lse, o_ref, lse_ref, N, d, 1e-5);
    free(h), free(x), free(of), free(lse), free(o), free(o_ref), free(lse_ref);
    hipFree(dbuf), hipFree(dout), hipFree(dlse);
}

/* fa_fwd then fa_bwd (bf16, causal) against the oracle's gradients of
 * sum(dO * O); bar 2e-2 * max(1, max|g_ref|) per gradient. */
static void case_bwd(hipStream_t stream, int B, int H, int N, int d)
{
    const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    double *q, *k, *v, *go;
    void *dq_in = bf16_tensor(n, &q), *dk_in = bf16_tensor(n, &k), *dv_in = bf16_tensor(n, &v);
    void *ddo = bf16_tensor(n, &go);
    void *dout = NULL, *gq = NULL, *gk = NULL, *gv = NULL;
    float *dlse = NULL, *ddelta = NULL;
    HIP_OK(hipMalloc(&dout, n * 2));
    HIP_OK(hipMalloc(&gq, n * 2));
    HIP_OK(hipMalloc(&gk, n * 2));
    HIP_OK(hipMalloc(&gv, n * 2));
    HIP_OK(hipMalloc((void **)&dlse, rows * 4));
    HIP_OK(hipMalloc((void **)&ddelta, rows * 4));
    const float scale = 1.0f / sqrtf((float)d);
    int st = fa_fwd(dq_in, dk_in, dv_in, dout, dlse, B, H, N, d, scale, 1, NULL, NULL, stream);
    EXPECT(st == FA_OK, "fa_fwd returned %d", st);
    st = fa_bwd(dq_in, dk_in, dv_in, dout, ddo, dlse, ddelta, gq, gk, gv, B, H, H, N, d, scale, 1, NULL, NULL,
                stream);
    EXPECT(st == FA_OK, "fa_bwd returned %d", st);
    HIP_OK(hipStreamSynchronize(stream));
    double *g[3] = {bf16_back(gq, n), bf16_back(gk, n), bf16_back(gv, n)};
    double *r[3];
    for (int i = 0; i < 3; ++i) r[i] = (double *)malloc(n * sizeof(double));
    EXPECT(attn_bwd_ref_gqa_f64(q, k, v, go, r[0], r[1], r[2], B, H, H, N, d, (double)scale, 1, NULL, NULL, 128) ==
               0,
           "oracle backward failed");
    const char *names[3] = {"dQ", "dK", "dV"};
    for (int i = 0; i < 3; ++i) {
        double err = 0.0, mx = 0.0;
        for (size_t x = 0; x < n; ++x) {
            err = fmax(err, fabs(g[i][x] - r[i][x]));
            mx = fmax(mx, fabs(r[i][x]));
        }
        const double bar = 2e-2 * fmax(1.0, mx);
        printf("fa_bwd bf16 B%d H%d N%d d%d causal %s          max err %.3e (bar %.3e)\n", B, H, N, d, names[i],
               err, bar);
        EXPECT(err <= bar, "fa_bwd %s error %.3e > %.3e", names[i], err, bar);
        free(g[i]), free(r[i]);
    }
    free(q), free(k), free(v), free(go);
    hipFree(dq_in), hipFree(dk_in), hipFree(dv_in), hipFree(ddo), hipFree(dout), hipFree(gq), hipFree(gk),
        hipFree(gv), hipFree(dlse), hipFree(ddelta);
}

/* Argument checks: each returns its status before any HIP call, so these
 * run with host pointers that are never dereferenced. */
static void case_errors(void)
{
    static _Alignas(16) uint16_t buf[4][64 * 64];
    float lse[64];
    const void *q = buf[0], *k = buf[1], *v = buf[2];
    void *o = buf[3];
    struct {
        const char *what;
        int got, want;
    } c[] = {
        {"q = NULL", fa_fwd(NULL, k, v, o, lse, 1, 1, 64, 64, 0.125f, 0, NULL, NULL, 0), FA_ERR_NULL_PTR},
        {"d = 96", fa_fwd(q, k, v, o, lse, 1, 1, 64, 96, 0.125f, 0, NULL, NULL, 0), FA_ERR_UNSUPPORTED_HEAD_DIM},
        {"N = 0", fa_fwd(q, k, v, o, lse, 1, 1, 0, 64, 0.125f, 0, NULL, NULL, 0), FA_ERR_INVALID_SHAPE},
        {"o misaligned", fa_fwd(q, k, v, (char *)o + 2, lse, 1, 1, 8, 64, 0.125f, 0, NULL, NULL, 0),
         FA_ERR_MISALIGNED},
        {"scale = NaN", fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, nanf(""), 0, NULL, NULL, 0), FA_ERR_INVALID_ARG},
        {"o overlaps q", fa_fwd(q, k, v, (void *)q, lse, 1, 1, 64, 64, 0.125f, 0, NULL, NULL, 0),
         FA_ERR_INVALID_ARG},
        {"unbuilt tile (Br, Bc) = (48, 64)",
         fa_fwd_ex(q, k, v, o, lse, 1, 1, 64, 64, 0.125f, 0, NULL, NULL, 0, FA_DTYPE_BF16, 48, 64),
         FA_ERR_UNSUPPORTED_TILE},
        {"fa_bwd H % H_kv != 0",
         fa_bwd(q, k, v, o, o, lse, lse, o, o, o, 1, 3, 2, 64, 64, 0.125f, 0, NULL, NULL, 0), FA_ERR_INVALID_SHAPE},
    };
    for (size_t i = 0; i < sizeof c / sizeof c[0]; ++i) {
        const char *s = fa_status_string(c[i].got);
        printf("argument check: %-34s -> %d (%s)\n", c[i].what, c[i].got, s ? s : "(null)");
        EXPECT(c[i].got == c[i].want, "%s: status %d, expected %d", c[i].what, c[i].got, c[i].want);
        EXPECT(s && s[0], "%s: empty status string", c[i].what);
    }
}

int main(int argc, char **argv)
{
    const int errors_only = argc > 1 && strcmp(argv[1], "--errors-only") == 0;
    case_errors();
    if (!errors_only) {
        rng_state = 20240501ull;
        hipStream_t stream;
        HIP_OK(hipStreamCreate(&stream));
        case_fwd_bf16(stream, 1, 2, 300, 64, 1, NULL, NULL);
        const int32_t key_len[2] = {200, 333};
        uint8_t mask[9] = {1, 0, 1, 1, 1, 0, 0, 1, 1};
        case_fwd_bf16(stream, 2, 2, 333, 128, 0, key_len, mask);
        case_fwd_bf16(stream, 1, 1, 1, 64, 0, NULL, NULL);
        case_fwd_f32(129, 64);
        case_bwd(stream, 1, 2, 130, 64);
        HIP_OK(hipStreamDestroy(stream));
    }
    if (failures) {
        printf("abi_check: %d failure(s)\n", failures);
        return 1;
    }
    printf("abi_check: all cases passed%s\n", errors_only ? " (argument checks only)" : "");
    return 0;
}
