/*
 * The host side of libmrope's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (built and
 * run by tests/test_sanitizers.py: the library's sources compiled for the host only, with the
 * sanitizers, and linked into this program).  Every entry point is called with arguments its
 * documented checks reject -- and with "nothing to do" arguments it accepts without a launch -- from
 * four threads at once, so the argument checks, the error text kept per thread, the status strings,
 * the workspace size arithmetic and the test-hook switch run under the sanitizers.  No call here
 * reaches the GPU: device pointers are aligned fake addresses that the checks never dereference.
 * Exit status 0 and "ok" on the last line when every status is the documented one.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mrope.h"

#define A ((void *)(uintptr_t)(1u << 20)) /* 256-byte aligned fake device address */
#define AT(off) ((void *)((uintptr_t)(1u << 20) + (off)))

static int failures = 0;
static pthread_mutex_t fail_lock = PTHREAD_MUTEX_INITIALIZER;

static void check(const char *what, int got, int want)
{
    const char *err = mrope_last_error();
    int bad = got != want;
    if (want != MROPE_OK && (err == NULL || err[0] == '\0' || strlen(err) > 1000)) bad = 1;
    if (bad) {
        pthread_mutex_lock(&fail_lock);
        fprintf(stderr, "FAILED: %s: status %d, want %d (%s)\n", what, got, want, err ? err : "(null)");
        ++failures;
        pthread_mutex_unlock(&fail_lock);
    }
}

static void expect(const char *what, int cond)
{
    if (!cond) {
        pthread_mutex_lock(&fail_lock);
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
        pthread_mutex_unlock(&fail_lock);
    }
}

/* ------------------------------------------------------------------------------------------ */
typedef struct {
    void *q, *k, *qo, *ko;
    int64_t qt, qh, kt, kh, n, ps;
    int32_t nq, nk, hd, rot, dt;
    const int32_t *planes;
    double theta;
} Apply;

static Apply apply_defaults(void)
{
    Apply a = {A, A, NULL, NULL, 2048, 256, 512, 256, 100, 100, 8, 2, 256, 64, MROPE_BF16, (const int32_t *)A, 1e7};
    return a;
}

static int call_apply(Apply a)
{
    return mrope_apply(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, a.n, a.hd, a.rot, a.dt, a.planes, a.ps,
                       a.theta, a.qo, a.ko, NULL);
}

#define APPLY(assign, want)                                  \
    do {                                                     \
        Apply a = apply_defaults();                          \
        assign;                                              \
        check("mrope_apply: " #assign, call_apply(a), want); \
    } while (0)

/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const int32_t *ids, *cu, *fls;
    int32_t ns, fl;
    int64_t n, ps;
    int32_t *planes;
    void *ws;
    size_t wsb;
} Planes;

static Planes planes_defaults(void)
{
    Planes p = {(const int32_t *)A, (const int32_t *)A, NULL, 4, 0, 1000, 1000, (int32_t *)A, A, 1000000};
    return p;
}

static int call_planes(Planes p)
{
    return mrope_planes(p.ids, p.cu, p.ns, p.n, 248078, p.fl, p.fls, NULL, NULL, p.planes, p.ps, NULL, NULL, NULL,
                        NULL, p.ws, p.wsb, 1u, NULL);
}

#define PLANES(assign, want)                                   \
    do {                                                       \
        Planes p = planes_defaults();                          \
        assign;                                                \
        check("mrope_planes: " #assign, call_planes(p), want); \
    } while (0)

/* ------------------------------------------------------------------------------------------ */
static int call_apply_ids(Apply a, Planes p)
{
    return mrope_apply_ids(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, a.n, a.hd, a.rot, a.dt, a.theta, a.qo, a.ko,
                           p.ids, p.cu, p.ns, 248078, p.fl, p.fls, NULL, NULL, p.planes, p.ps, NULL, NULL, NULL, NULL,
                           p.ws, p.wsb, 1u, NULL);
}

static int call_noalloc(Apply a, Planes p)
{
    return mrope_apply_ids_noalloc(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, a.n, a.hd, a.rot, a.dt, a.theta,
                                   a.qo, a.ko, p.ids, p.cu, p.ns, 248078, p.fl, p.fls, NULL, NULL, p.planes, p.ps,
                                   NULL, NULL, NULL, NULL, NULL);
}

#define IDS(assign, want)                                                 \
    do {                                                                  \
        Apply a = apply_defaults();                                       \
        Planes p = planes_defaults();                                     \
        a.n = p.n;                                                        \
        p.planes = NULL;                                                  \
        p.ps = 0;                                                         \
        assign;                                                           \
        check("mrope_apply_ids: " #assign, call_apply_ids(a, p), want);   \
    } while (0)

#define NOALLOC(assign, want)                                                 \
    do {                                                                      \
        Apply a = apply_defaults();                                           \
        Planes p = planes_defaults();                                         \
        a.n = p.n;                                                            \
        p.planes = NULL;                                                      \
        p.ps = 0;                                                             \
        assign;                                                               \
        check("mrope_apply_ids_noalloc: " #assign, call_noalloc(a, p), want); \
    } while (0)

/* ------------------------------------------------------------------------------------------ */
typedef struct {
    void *kc, *vc;
    const void *v;
    const int64_t *slots;
    int32_t bs;
    int64_t nb, cb, ct, ch, vt, vh;
} Cache;

static Cache cache_defaults(void)
{
    Cache c = {A, A, A, (const int64_t *)A, 16, 64, 8192, 512, 256, 512, 256};
    return c;
}

static int call_apply_kv(Apply a, Cache c)
{
    return mrope_apply_kv(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, c.v, c.vt, c.vh, a.n, a.hd, a.rot, a.dt,
                          a.planes, a.ps, a.theta, c.kc, c.vc, c.slots, c.bs, c.nb, c.cb, c.ct, c.ch, NULL);
}

static int call_apply_ids_kv(Apply a, Planes p, Cache c)
{
    return mrope_apply_ids_kv(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, c.v, c.vt, c.vh, a.n, a.hd, a.rot, a.dt,
                              a.theta, p.ids, p.cu, p.ns, 248078, p.fl, p.fls, NULL, NULL, NULL, 0, NULL, NULL, NULL,
                              NULL, p.ws, p.wsb, 1u, c.kc, c.vc, c.slots, c.bs, c.nb, c.cb, c.ct, c.ch, NULL);
}

static int call_decode(Apply a, Cache c, int32_t ns, const int32_t *pos, const int32_t *am)
{
    return mrope_decode(a.q, a.qt, a.qh, a.nq, a.k, a.kt, a.kh, a.nk, c.v, c.vt, c.vh, ns, pos, am, c.kc, c.vc,
                        c.slots, c.bs, c.nb, c.cb, c.ct, c.ch, a.hd, a.rot, a.dt, a.theta, NULL);
}

#define KV(assign, want)                                                                    \
    do {                                                                                    \
        Apply a = apply_defaults();                                                         \
        Planes p = planes_defaults();                                                       \
        Cache c = cache_defaults();                                                         \
        a.n = p.n;                                                                          \
        assign;                                                                             \
        check("mrope_apply_kv: " #assign, call_apply_kv(a, c), want);                       \
        check("mrope_apply_ids_kv: " #assign, call_apply_ids_kv(a, p, c), want);            \
        check("mrope_decode: " #assign, call_decode(a, c, 16, (const int32_t *)A, (const int32_t *)A), want); \
    } while (0)

static void run_cases(void)
{
    /* mrope_apply */
    APPLY(a.rot = 32, MROPE_ERR_UNSUPPORTED);
    APPLY(a.hd = 60, MROPE_ERR_UNSUPPORTED);
    APPLY(a.hd = 2048, MROPE_ERR_UNSUPPORTED);
    APPLY(a.dt = 7, MROPE_ERR_UNSUPPORTED);
    APPLY(a.nq = 65, MROPE_ERR_UNSUPPORTED);
    APPLY(a.nk = -1, MROPE_ERR_UNSUPPORTED);
    APPLY(a.n = -1, MROPE_ERR_ARG);
    APPLY(a.q = NULL, MROPE_ERR_ARG);
    APPLY(a.planes = NULL, MROPE_ERR_ARG);
    APPLY(a.ps = 99, MROPE_ERR_ARG);
    APPLY(a.theta = 0.0, MROPE_ERR_ARG);
    APPLY(a.theta = NAN, MROPE_ERR_ARG);
    APPLY(a.theta = INFINITY, MROPE_ERR_ARG);
    APPLY(a.qo = A, MROPE_ERR_ARG);
    APPLY(a.qt = -8, MROPE_ERR_ARG);
    APPLY(a.qt = INT64_MIN, MROPE_ERR_ARG);
    APPLY(a.q = AT(8), MROPE_ERR_ALIGN);
    APPLY(a.qt = 2044, MROPE_ERR_ALIGN);
    APPLY((a.dt = MROPE_F32, a.qt = 2050), MROPE_ERR_ALIGN);
    APPLY(a.n = 0, MROPE_OK);
    APPLY((a.nq = 0, a.nk = 0), MROPE_OK);

    /* mrope_planes */
    PLANES(p.ns = -1, MROPE_ERR_ARG);
    PLANES(p.n = -1, MROPE_ERR_ARG);
    PLANES(p.ns = 0, MROPE_ERR_ARG);
    PLANES(p.cu = NULL, MROPE_ERR_ARG);
    PLANES(p.ids = NULL, MROPE_ERR_ARG);
    PLANES(p.planes = NULL, MROPE_ERR_ARG);
    PLANES(p.ps = 999, MROPE_ERR_ARG);
    PLANES(p.n = (int64_t)1 << 31, MROPE_ERR_ARG);
    PLANES(p.n = INT64_MAX, MROPE_ERR_ARG);
    PLANES(p.ws = NULL, MROPE_ERR_WORKSPACE);
    PLANES(p.ws = AT(64), MROPE_ERR_WORKSPACE);
    PLANES(p.wsb = 24 * 1000, MROPE_ERR_WORKSPACE);
    PLANES(p.fl = 64, MROPE_ERR_ARG);
    PLANES(p.fl = -1, MROPE_ERR_ARG);
    PLANES(p.fl = 4097, MROPE_ERR_ARG);
    PLANES((p.ns = 0, p.n = 0, p.ws = NULL), MROPE_OK);

    /* mrope_apply_ids and its no-allocation variant */
    IDS(p.ids = NULL, MROPE_ERR_ARG);
    IDS(p.cu = NULL, MROPE_ERR_ARG);
    IDS(p.ws = NULL, MROPE_ERR_WORKSPACE);
    IDS(p.wsb = 100, MROPE_ERR_WORKSPACE);
    IDS(p.fl = 30, MROPE_ERR_ARG);
    IDS(a.rot = 32, MROPE_ERR_UNSUPPORTED);
    IDS((p.planes = (int32_t *)A, p.ps = 999), MROPE_ERR_ARG);
    IDS(a.ko = A, MROPE_ERR_ARG);
    NOALLOC((a.n = p.n = MROPE_NOALLOC_MAX_TOKENS + 1), MROPE_ERR_WORKSPACE);
    NOALLOC(p.ids = NULL, MROPE_ERR_ARG);
    NOALLOC(p.ns = 0, MROPE_ERR_ARG);
    NOALLOC(a.q = AT(8), MROPE_ERR_ALIGN);
    NOALLOC(p.fl = 30, MROPE_ERR_ARG);
    NOALLOC(a.theta = -1.0, MROPE_ERR_ARG);

    /* paged cache: mrope_apply_kv, mrope_apply_ids_kv, mrope_decode */
    KV(c.kc = NULL, MROPE_ERR_ARG);
    KV(c.slots = NULL, MROPE_ERR_ARG);
    KV(c.bs = 0, MROPE_ERR_ARG);
    KV(c.nb = -1, MROPE_ERR_ARG);
    KV(c.ct = -512, MROPE_ERR_ARG);
    KV(c.kc = AT(2), MROPE_ERR_ALIGN);
    KV(c.ch = 260, MROPE_ERR_ALIGN);
    KV(c.ch = 128, MROPE_ERR_ARG);
    KV(c.v = NULL, MROPE_ERR_ARG);
    KV(c.vc = AT(8), MROPE_ERR_ALIGN);
    KV(c.vh = 128, MROPE_ERR_ARG);
    {
        Apply a = apply_defaults();
        Cache c = cache_defaults();
        check("mrope_decode: pos NULL", call_decode(a, c, 16, NULL, (const int32_t *)A), MROPE_ERR_ARG);
        check("mrope_decode: n_seqs -1", call_decode(a, c, -1, (const int32_t *)A, (const int32_t *)A),
              MROPE_ERR_ARG);
        check("mrope_decode: nothing to do", call_decode(a, c, 0, NULL, NULL), MROPE_OK);
    }

    /* workspace, strings, hooks */
    check("mrope_workspace_init: NULL", mrope_workspace_init(NULL, 1024, NULL), MROPE_ERR_WORKSPACE);
    check("mrope_workspace_init: misaligned", mrope_workspace_init(AT(128), 1024, NULL), MROPE_ERR_WORKSPACE);
    check("mrope_workspace_init: size", mrope_workspace_init(A, 100, NULL), MROPE_ERR_WORKSPACE);
    const int64_t sizes[] = {-5, 0, 1, 511, 512, 513, (int64_t)1 << 20, ((int64_t)1 << 31) - 1};
    for (int i = 0; i < (int)(sizeof(sizes) / sizeof(sizes[0])); ++i) {
        const size_t b = mrope_workspace_bytes(sizes[i]);
        expect("mrope_workspace_bytes: a multiple of 256", b % 256 == 0);
        expect("mrope_workspace_bytes: at least the header", b >= 256);
        if (sizes[i] > 0) expect("mrope_workspace_bytes: 24 bytes a token or more", b >= 24 * (size_t)sizes[i]);
    }
    for (int code = -3; code < 12; ++code) expect("mrope_status_string", mrope_status_string(code) != NULL);
    expect("abi version", mrope_abi_version() == MROPE_ABI_VERSION);
}

static void *worker(void *arg)
{
    (void)arg;
    for (int rep = 0; rep < 20; ++rep) run_cases();
    return NULL;
}

int main(void)
{
    const int prev = mrope_set_test_hooks(MROPE_HOOK_FUSED_SCAN_FIRST);
    expect("test hooks: previous value", mrope_set_test_hooks(prev | 64) == MROPE_HOOK_FUSED_SCAN_FIRST);
    expect("test hooks: unknown bits dropped", mrope_set_test_hooks(prev) == prev);
    pthread_t th[4];
    for (int i = 0; i < 4; ++i) pthread_create(&th[i], NULL, worker, NULL);
    for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
