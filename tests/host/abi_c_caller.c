/*
 * A plain C caller of libmrope: device buffers from the HIP runtime, the C ABI of include/mrope.h and
 * nothing else -- no Python, no torch.  It checks the library against the CPU oracle's C functions
 * (oracle/liboracle.so, test infrastructure) on one small packed batch:
 *
 *   sequence 0: 110 tokens, <image> at position 6 (the single-image prompt of the Core AI card's
 *               canvas table: start 73, amount 58);
 *   sequence 1: 50 text tokens (start 2^30, amount 0);
 *   sequence 2: 700 tokens, <image> at position 320 (its frame crosses the 512-token chunk edge).
 *
 * Q [T, 8, 256] and K [T, 2, 256] come from a seeded LCG (Box-Muller normals).  Runs:
 *   1. mrope_planes, then mrope_apply on fp32 Q/K: planes, start, amount, origin bit-exact; every
 *      rotated element within 2e-6 of the oracle relative to its pair's norm; dims 64..255 unchanged.
 *   2. mrope_apply_ids on bf16 copies: every element within one bf16 ulp of the oracle's fp32 result
 *      rounded to bf16 (nearest even), the rest bit-identical.
 *   3. A call with a NULL Q pointer: MROPE_ERR_ARG, and mrope_last_error() says why.
 * Prints one line per check and exits 0 only if all pass.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mrope.h"

/* The oracle's C entry points (oracle/mrope_oracle.c). */
void oracle_planes(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                   int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount, int32_t *origin);
void oracle_rotate(const float *x, int64_t n_tokens, int32_t n_heads, int64_t tok_stride, int64_t head_stride,
                   int32_t head_dim, int32_t rot_dim, const int32_t *planes, int64_t plane_stride, double theta,
                   float *y, double *y64);
void oracle_round_bf16(const float *x, uint16_t *out, int64_t n);

#define MARKER 248078
#define NQ 8
#define NK 2
#define HD 256
#define ROT 64
#define THETA 1e7

static int failures = 0;

#define HIP_OK(call)                                                                       \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));              \
            exit(2);                                                                       \
        }                                                                                  \
    } while (0)

static void report(const char *what, int ok, const char *detail)
{
    printf("%s %s%s%s\n", ok ? "PASS" : "FAIL", what, detail[0] ? ": " : "", detail);
    if (!ok) ++failures;
}

/* seeded inputs: a 64-bit LCG (Knuth's MMIX constants) and Box-Muller */
static uint64_t lcg_state = 20261203u;
static double lcg_uniform(void)
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return ((double)(lcg_state >> 11) + 0.5) / 9007199254740992.0;
}
static float lcg_normal(void)
{
    const double u = lcg_uniform(), v = lcg_uniform();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static int32_t lcg_text_id(void)
{
    for (;;) {
        const int32_t id = (int32_t)(lcg_uniform() * 248000.0);
        if (id != MARKER) return id;
    }
}

static uint16_t to_bf16(float x) /* input rounding of the test data (nearest even) */
{
    uint16_t b;
    oracle_round_bf16(&x, &b, 1);
    return b;
}
static float from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}
static int32_t ordered(uint16_t b) { return (b & 0x8000u) ? -(int32_t)(b & 0x7fffu) : (int32_t)(b & 0x7fffu); }

static void *dev_copy(const void *host, size_t bytes)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 4));
    if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(void)
{
    const int32_t lens[3] = {110, 50, 700}, marks[3] = {6, -1, 320};
    const int32_t n_seqs = 3;
    int32_t cu[4] = {0};
    for (int s = 0; s < n_seqs; ++s) cu[s + 1] = cu[s] + lens[s];
    const int64_t T = cu[n_seqs];

    int32_t *ids = malloc(sizeof(int32_t) * T);
    for (int s = 0; s < n_seqs; ++s)
        for (int32_t p = 0; p < lens[s]; ++p) ids[cu[s] + p] = (p == marks[s]) ? MARKER : lcg_text_id();
    const int64_t nq = T * NQ * HD, nk = T * NK * HD;
    float *q = malloc(sizeof(float) * nq), *k = malloc(sizeof(float) * nk);
    for (int64_t i = 0; i < nq; ++i) q[i] = lcg_normal();
    for (int64_t i = 0; i < nk; ++i) k[i] = lcg_normal();

    /* the oracle */
    int32_t *epl = malloc(sizeof(int32_t) * 3 * T), est[3], eam[3], eog[3];
    oracle_planes(ids, cu, n_seqs, MARKER, epl, T, est, eam, eog);
    float *eq = malloc(sizeof(float) * nq), *ek = malloc(sizeof(float) * nk);
    oracle_rotate(q, T, NQ, NQ * HD, HD, HD, ROT, epl, T, THETA, eq, NULL);
    oracle_rotate(k, T, NK, NK * HD, HD, HD, ROT, epl, T, THETA, ek, NULL);

    /* device buffers */
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int32_t *d_ids = dev_copy(ids, sizeof(int32_t) * T), *d_cu = dev_copy(cu, sizeof cu);
    float *d_q = dev_copy(q, sizeof(float) * nq), *d_k = dev_copy(k, sizeof(float) * nk);
    int32_t *d_pl, *d_st, *d_am, *d_og;
    HIP_OK(hipMalloc((void **)&d_pl, sizeof(int32_t) * 3 * T));
    HIP_OK(hipMalloc((void **)&d_st, sizeof(int32_t) * n_seqs));
    HIP_OK(hipMalloc((void **)&d_am, sizeof(int32_t) * n_seqs));
    HIP_OK(hipMalloc((void **)&d_og, sizeof(int32_t) * n_seqs));
    const size_t ws_bytes = mrope_workspace_bytes(T);
    void *d_ws;
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    char detail[256] = "";

    report("abi version", mrope_abi_version() == MROPE_ABI_VERSION, "");
    report("workspace init", mrope_workspace_init(d_ws, ws_bytes, stream) == MROPE_OK, "");

    /* 1. planes + apply, fp32 */
    int st = mrope_planes(d_ids, d_cu, n_seqs, T, MARKER, 0, NULL, NULL, NULL, d_pl, T, d_st, d_am, d_og, NULL, d_ws,
                          ws_bytes, 1u, stream);
    report("mrope_planes status", st == MROPE_OK, st == MROPE_OK ? "" : mrope_last_error());
    st = mrope_apply(d_q, NQ * HD, HD, NQ, d_k, NK * HD, HD, NK, T, HD, ROT, MROPE_F32, d_pl, T, THETA, NULL,
                     NULL, stream);
    report("mrope_apply status", st == MROPE_OK, st == MROPE_OK ? "" : mrope_last_error());
    HIP_OK(hipStreamSynchronize(stream));

    int32_t *pl = malloc(sizeof(int32_t) * 3 * T), gst[3], gam[3], gog[3];
    HIP_OK(hipMemcpy(pl, d_pl, sizeof(int32_t) * 3 * T, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gst, d_st, sizeof gst, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gam, d_am, sizeof gam, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gog, d_og, sizeof gog, hipMemcpyDeviceToHost));
    report("planes bit-exact", memcmp(pl, epl, sizeof(int32_t) * 3 * T) == 0, "");
    snprintf(detail, sizeof detail, "start %d %d %d, amount %d %d %d", gst[0], gst[1], gst[2], gam[0], gam[1],
             gam[2]);
    report("scalars bit-exact",
           !memcmp(gst, est, sizeof gst) && !memcmp(gam, eam, sizeof gam) && !memcmp(gog, eog, sizeof gog) &&
               gst[0] == 73 && gam[0] == 58 && gst[1] == MROPE_TEXT_ONLY_START && gam[1] == 0,
           detail);

    float *gq = malloc(sizeof(float) * nq), *gk = malloc(sizeof(float) * nk);
    HIP_OK(hipMemcpy(gq, d_q, sizeof(float) * nq, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gk, d_k, sizeof(float) * nk, hipMemcpyDeviceToHost));
    double worst = 0.0;
    int tail_ok = 1;
    for (int pass = 0; pass < 2; ++pass) {
        const float *got = pass ? gk : gq, *ref = pass ? ek : eq, *in = pass ? k : q;
        const int64_t rows = T * (pass ? NK : NQ);
        for (int64_t r = 0; r < rows; ++r) {
            for (int d = 0; d < ROT; ++d) {
                const int64_t i = r * HD + d, j = r * HD + (d < 32 ? d + 32 : d - 32);
                const double norm = sqrt((double)ref[i] * ref[i] + (double)ref[j] * ref[j]);
                const double err = fabs((double)got[i] - ref[i]);
                const double rel = norm > 0 ? err / norm : (err > 0 ? INFINITY : 0.0);
                if (rel > worst) worst = rel;
            }
            for (int d = ROT; d < HD; ++d)
                if (memcmp(&got[r * HD + d], &in[r * HD + d], sizeof(float))) tail_ok = 0;
        }
    }
    snprintf(detail, sizeof detail, "max pair-relative error %.3g", worst);
    report("fp32 rotation within 2e-6", worst <= 2e-6, detail);
    report("fp32 dims 64..255 unchanged", tail_ok, "");

    /* 2. the fused call on bf16 copies of the inputs */
    uint16_t *qb = malloc(2 * nq), *kb = malloc(2 * nk);
    float *qf = malloc(sizeof(float) * nq), *kf = malloc(sizeof(float) * nk);
    for (int64_t i = 0; i < nq; ++i) qf[i] = from_bf16(qb[i] = to_bf16(q[i]));
    for (int64_t i = 0; i < nk; ++i) kf[i] = from_bf16(kb[i] = to_bf16(k[i]));
    oracle_rotate(qf, T, NQ, NQ * HD, HD, HD, ROT, epl, T, THETA, eq, NULL);
    oracle_rotate(kf, T, NK, NK * HD, HD, HD, ROT, epl, T, THETA, ek, NULL);
    uint16_t *eqb = malloc(2 * nq), *ekb = malloc(2 * nk);
    oracle_round_bf16(eq, eqb, nq);
    oracle_round_bf16(ek, ekb, nk);
    void *d_qb = dev_copy(qb, 2 * nq), *d_kb = dev_copy(kb, 2 * nk);
    /* out of place first (a copy launch for dims 64..255, then the rotation launch); the in-place
       call below then starts from the same, untouched inputs */
    void *d_qo, *d_ko;
    HIP_OK(hipMalloc(&d_qo, 2 * nq));
    HIP_OK(hipMalloc(&d_ko, 2 * nk));
    st = mrope_apply_ids(d_qb, NQ * HD, HD, NQ, d_kb, NK * HD, HD, NK, T, HD, ROT, MROPE_BF16, THETA, d_qo, d_ko,
                         d_ids, d_cu, n_seqs, MARKER, 0, NULL, NULL, NULL, NULL, T, NULL, NULL, NULL, NULL, d_ws, ws_bytes,
                         3u, stream);
    report("mrope_apply_ids out of place status", st == MROPE_OK, st == MROPE_OK ? "" : mrope_last_error());
    st = mrope_apply_ids(d_qb, NQ * HD, HD, NQ, d_kb, NK * HD, HD, NK, T, HD, ROT, MROPE_BF16, THETA, NULL, NULL,
                         d_ids, d_cu, n_seqs, MARKER, 0, NULL, NULL, NULL, NULL, T, d_st, d_am, d_og, NULL, d_ws, ws_bytes,
                         2u, stream);
    report("mrope_apply_ids status", st == MROPE_OK, st == MROPE_OK ? "" : mrope_last_error());
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(qb, d_qb, 2 * nq, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(kb, d_kb, 2 * nk, hipMemcpyDeviceToHost));
    int32_t worst_ulp = 0;
    int64_t off_by_one = 0;
    for (int pass = 0; pass < 2; ++pass) {
        const uint16_t *got = pass ? kb : qb, *ref = pass ? ekb : eqb;
        const int64_t n = pass ? nk : nq;
        for (int64_t i = 0; i < n; ++i) {
            int32_t dd = ordered(got[i]) - ordered(ref[i]);
            if (dd < 0) dd = -dd;
            if ((i % HD) >= ROT && dd) dd = 1 << 20; /* the rest must be bit-identical */
            if (dd > worst_ulp) worst_ulp = dd;
            off_by_one += dd == 1;
        }
    }
    snprintf(detail, sizeof detail, "max %d ulp, %lld elements off by one", worst_ulp, (long long)off_by_one);
    report("bf16 fused rotation within 1 ulp", worst_ulp <= 1, detail);
    uint16_t *qo = malloc(2 * nq), *ko = malloc(2 * nk);
    HIP_OK(hipMemcpy(qo, d_qo, 2 * nq, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ko, d_ko, 2 * nk, hipMemcpyDeviceToHost));
    report("bf16 out of place equals in place, bit for bit", !memcmp(qo, qb, 2 * nq) && !memcmp(ko, kb, 2 * nk), "");

    /* 3. a host-detected error */
    st = mrope_apply(NULL, NQ * HD, HD, NQ, d_k, NK * HD, HD, NK, T, HD, ROT, MROPE_F32, d_pl, T, THETA, NULL, NULL,
                     stream);
    snprintf(detail, sizeof detail, "%s (%s)", mrope_status_string(st), mrope_last_error());
    report("NULL q rejected before launch", st == MROPE_ERR_ARG && mrope_last_error()[0] != 0, detail);

    printf("%s\n", failures ? "FAILED" : "ALL PASSED");
    return failures ? 1 : 0;
}
