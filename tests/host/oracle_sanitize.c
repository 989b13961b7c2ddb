/*
 * The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (built and run by
 * tests/test_sanitizers.py with gcc -fsanitize=address,undefined): every entry point on small
 * inputs held in buffers of exactly the size each call may touch, covering the edge cases the
 * test suite feeds it -- empty batches, empty and one-token sequences, frames cut by the end of a
 * sequence, second markers, later pieces with carried origins, per-sequence frame lengths with
 * entries that describe no frame, paged slots outside the cache, and special float values for the
 * bf16 rounding.  A few results are checked against values fixed by the canvas rule, so the run
 * also fails if the build is broken.  Exit status 0 and "ok" on the last line when all is well.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's entry points (oracle/mrope_oracle.c). */
int32_t oracle_first_marker(const int32_t *ids, int32_t n, int32_t marker_id);
void oracle_frame_scalars_len(int32_t origin, int32_t frame_len, int32_t *start, int32_t *amount);
void oracle_frame_scalars(int32_t origin, int32_t *start, int32_t *amount);
void oracle_planes(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                   int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount, int32_t *origin);
int32_t oracle_seq_frame_len(const int32_t *frame_len_seq, int32_t s, int32_t frame_len);
void oracle_planes_chunk(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                         int32_t frame_len, const int32_t *frame_len_seq, const int32_t *pos_offset,
                         const int32_t *origin_in, int32_t *planes, int64_t plane_stride, int32_t *start,
                         int32_t *amount, int32_t *origin);
void oracle_inv_freq(double theta, int32_t rot_dim, float *inv_freq);
int32_t oracle_plane_of_freq(int32_t j);
void oracle_rotate(const float *x, int64_t n_tokens, int32_t n_heads, int64_t tok_stride, int64_t head_stride,
                   int32_t head_dim, int32_t rot_dim, const int32_t *planes, int64_t plane_stride, double theta,
                   float *y, double *y64);
void oracle_scatter_rows(const float *rows, int64_t n_rows, int64_t row_elems, const int64_t *slots,
                         int32_t block_size, int64_t num_blocks, float *cache);
void oracle_decode(const float *q, int32_t n_q_heads, const float *k, int32_t n_k_heads, int32_t n_seqs,
                   const int32_t *pos, const int32_t *amount, int32_t head_dim, int32_t rot_dim, double theta,
                   float *q_out, float *cache, const int64_t *slot_mapping, int32_t block_size, int64_t num_blocks,
                   int64_t cache_block_stride, int64_t cache_head_stride, int64_t cache_tok_stride, const float *v,
                   float *v_cache);
void oracle_round_bf16(const float *x, uint16_t *out, int64_t n);

#define MARKER 248078

static int failures = 0;

static void expect(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

/* malloc of exactly n elements (at least one byte, so a zero-length buffer is still a valid
   pointer whose every access is out of bounds for ASan) */
static void *exact(size_t n, size_t elem)
{
    void *p = malloc(n ? n * elem : 1);
    if (!p) {
        perror("malloc");
        exit(2);
    }
    return p;
}

static uint32_t lcg = 12345u;
static uint32_t next_u32(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return lcg;
}

/* A packed batch: lengths given, a frame of 67 tokens (<image>, 64 pads, </image>, "\n") at
   origin[s] (-1: text only), text ids elsewhere, an optional second marker. */
static int32_t *make_batch(const int32_t *lens, const int32_t *origin, const int32_t *second, int32_t n_seqs,
                           int32_t **cu_out)
{
    int32_t *cu = exact((size_t)n_seqs + 1, sizeof(int32_t));
    cu[0] = 0;
    for (int32_t s = 0; s < n_seqs; ++s) cu[s + 1] = cu[s] + lens[s];
    const int32_t total = cu[n_seqs];
    int32_t *ids = exact((size_t)total, sizeof(int32_t));
    for (int32_t t = 0; t < total; ++t) ids[t] = (int32_t)(next_u32() % 150000u);
    for (int32_t s = 0; s < n_seqs; ++s) {
        int32_t *seq = ids + cu[s];
        if (origin[s] >= 0)
            for (int32_t i = 0; i < 67 && origin[s] + i < lens[s]; ++i)
                seq[origin[s] + i] = i == 0 ? MARKER : (i <= 64 ? 248077 : (i == 65 ? 248079 : 198));
        if (second && second[s] >= 0 && second[s] < lens[s]) seq[second[s]] = MARKER;
    }
    *cu_out = cu;
    return ids;
}

static void planes_cases(void)
{
    /* empty batch: no sequences, no tokens */
    {
        int32_t cu0 = 0;
        int32_t *ids = exact(0, sizeof(int32_t));
        int32_t *pl = exact(0, sizeof(int32_t));
        int32_t *st = exact(0, sizeof(int32_t)), *am = exact(0, sizeof(int32_t));
        oracle_planes(ids, &cu0, 0, MARKER, pl, 0, st, am, NULL);
        oracle_planes_chunk(ids, &cu0, 0, MARKER, 67, NULL, NULL, NULL, pl, 0, st, am, NULL);
        free(ids), free(pl), free(st), free(am);
    }
    /* empty, one-token, cut and whole frames, a second marker, text only */
    const int32_t lens[] = {0, 1, 66, 67, 68, 300, 0, 140, 90, 5, 0};
    const int32_t orig[] = {-1, 0, 0, 0, 1, 100, -1, 73, -1, 4, -1};
    const int32_t second[] = {-1, -1, 30, -1, -1, 250, -1, 139, 7, -1, -1};
    const int32_t n = (int32_t)(sizeof(lens) / sizeof(lens[0]));
    int32_t *cu;
    int32_t *ids = make_batch(lens, orig, second, n, &cu);
    const int32_t T = cu[n];
    int32_t *pl = exact((size_t)3 * T, sizeof(int32_t));
    int32_t *st = exact((size_t)n, sizeof(int32_t)), *am = exact((size_t)n, sizeof(int32_t));
    int32_t *og = exact((size_t)n, sizeof(int32_t));
    oracle_planes(ids, cu, n, MARKER, pl, T, st, am, og);
    expect(og[5] == 100 && st[5] == 167 && am[5] == 58, "planes: scalars of a whole frame");
    expect(og[8] == 7, "planes: first marker wins in a text prompt with a stray marker");
    expect(og[0] == -1 && st[0] == (1 << 30) && am[0] == 0, "planes: empty sequence is text only");
    const int32_t b5 = cu[5];
    expect(pl[b5 + 99] == 99 && pl[T + b5 + 100] == 99 && pl[2 * T + b5 + 101] == 100,
           "planes: text, <image> and the first row");
    expect(pl[b5 + 299] == 299 - 58, "planes: after the frame");

    /* per-sequence frame lengths, pieces with carried origins */
    int32_t *fls = exact((size_t)n, sizeof(int32_t));
    int32_t *off = exact((size_t)n, sizeof(int32_t)), *oin = exact((size_t)n, sizeof(int32_t));
    const int32_t fvals[] = {65, 67, 75, 0, 64, 4097, -1, 4096, 66, 70, 0};
    for (int32_t s = 0; s < n; ++s) {
        fls[s] = fvals[s];
        off[s] = (int32_t)(next_u32() % 500u);
        oin[s] = (s % 3 == 0) ? (int32_t)(next_u32() % 400u) : -1;
    }
    oracle_planes_chunk(ids, cu, n, MARKER, 67, fls, NULL, NULL, pl, T, st, am, og);
    expect(st[7] == 73 + 4096 && am[7] == 4096 - 9, "chunk: a 4096-token frame");
    expect(st[5] == 100 + 67, "chunk: 4097 is no frame length: the call's");
    expect(st[2] == 0 + 75 && am[2] == 66, "chunk: a 75-token frame");
    expect(st[4] == 1 + 67, "chunk: 64 is no frame length: the call's");
    oracle_planes_chunk(ids, cu, n, MARKER, 70, fls, off, oin, pl, T, st, am, NULL);
    oracle_planes_chunk(ids, cu, n, MARKER, 65, NULL, off, NULL, pl, T, st, am, og);
    expect(oracle_seq_frame_len(NULL, 3, 67) == 67, "seq_frame_len: NULL array");
    free(fls), free(off), free(oin);
    free(ids), free(cu), free(pl), free(st), free(am), free(og);

    int32_t s, a;
    oracle_frame_scalars(-1, &s, &a);
    expect(s == (1 << 30) && a == 0, "frame scalars: no image");
    oracle_frame_scalars_len(6, 65, &s, &a);
    expect(s == 71 && a == 56, "frame scalars: Qwen-VL's rule");
    expect(oracle_first_marker(&s, 0, MARKER) == -1, "first marker: empty");
}

static void rotate_cases(void)
{
    float *inv = exact(32, sizeof(float));
    oracle_inv_freq(1e7, 64, inv);
    expect(inv[0] == 1.0f && inv[31] > 0.0f && inv[31] < inv[30], "inv_freq");
    free(inv);
    int32_t h = 0, w = 0;
    for (int32_t j = 0; j < 32; ++j) {
        const int32_t p = oracle_plane_of_freq(j);
        h += p == 1;
        w += p == 2;
    }
    expect(h == 11 && w == 10, "sections [11, 11, 10]");

    const int32_t dims[] = {64, 256, 72};
    for (int i = 0; i < 3; ++i) {
        const int32_t D = dims[i], H = 3;
        const int64_t Tn = 5;
        float *x = exact((size_t)(Tn * H * D), sizeof(float));
        float *y = exact((size_t)(Tn * H * D), sizeof(float));
        double *y64 = exact((size_t)(Tn * H * D), sizeof(double));
        int32_t *pl = exact((size_t)(3 * Tn), sizeof(int32_t));
        for (int64_t e = 0; e < Tn * H * D; ++e) x[e] = (float)((int32_t)(next_u32() % 2001u) - 1000) / 256.0f;
        for (int64_t e = 0; e < 3 * Tn; ++e) pl[e] = (int32_t)(next_u32() % 100000u);
        oracle_rotate(x, Tn, H, (int64_t)H * D, D, D, 64, pl, Tn, 1e7, y, y64);
        oracle_rotate(x, Tn, H, (int64_t)H * D, D, D, 64, pl, Tn, 1e7, y, NULL);
        oracle_rotate(x, 0, H, (int64_t)H * D, D, D, 64, pl, 0, 1e7, y, NULL);
        for (int64_t t = 0; t < Tn; ++t)
            for (int32_t d = 64; d < D; ++d) expect(y[t * H * D + d] == x[t * H * D + d], "rotate: pass-through dims");
        /* position 0 on every plane: the identity */
        memset(pl, 0, sizeof(int32_t) * (size_t)(3 * Tn));
        oracle_rotate(x, Tn, H, (int64_t)H * D, D, D, 64, pl, Tn, 1e7, y, NULL);
        expect(memcmp(x, y, sizeof(float) * (size_t)(Tn * H * D)) == 0, "rotate: identity at position 0");
        free(x), free(y), free(y64), free(pl);
    }
}

static void cache_cases(void)
{
    const int32_t bs = 4, H = 2, D = 64, S = 6;
    const int64_t nb = 3, row = (int64_t)H * D;
    float *rows = exact((size_t)(S * row), sizeof(float));
    float *cache = exact((size_t)(nb * bs * row), sizeof(float));
    int64_t *slots = exact((size_t)S, sizeof(int64_t));
    const int64_t sv[] = {0, 11, -1, 12, 5, 1000};
    for (int64_t e = 0; e < S * row; ++e) rows[e] = (float)e;
    for (int i = 0; i < S; ++i) slots[i] = sv[i];
    memset(cache, 0, sizeof(float) * (size_t)(nb * bs * row));
    oracle_scatter_rows(rows, S, row, slots, bs, nb, cache);
    expect(cache[11 * row] == rows[1 * row], "scatter: last slot");

    /* decode: three sequences, one slot outside the cache, with and without V */
    float *q = exact((size_t)(3 * 4 * D), sizeof(float)), *qo = exact((size_t)(3 * 4 * D), sizeof(float));
    float *k = exact((size_t)(3 * H * D), sizeof(float)), *v = exact((size_t)(3 * H * D), sizeof(float));
    float *vc = exact((size_t)(nb * bs * row), sizeof(float));
    int32_t *pos = exact(3, sizeof(int32_t)), *am = exact(3, sizeof(int32_t));
    int64_t *sl = exact(3, sizeof(int64_t));
    for (int e = 0; e < 3 * 4 * D; ++e) q[e] = (float)(e % 17) - 8.0f;
    for (int e = 0; e < 3 * H * D; ++e) k[e] = v[e] = (float)(e % 13) - 6.0f;
    for (int s = 0; s < 3; ++s) {
        pos[s] = 100 + s;
        am[s] = 58;
    }
    sl[0] = 2, sl[1] = -5, sl[2] = nb * bs - 1;
    oracle_decode(q, 4, k, H, 3, pos, am, D, 64, 1e7, qo, cache, sl, bs, nb, (int64_t)bs * row, D, row, v, vc);
    oracle_decode(q, 4, k, H, 3, pos, am, D, 64, 1e7, qo, cache, sl, bs, nb, (int64_t)bs * row, D, row, NULL, NULL);
    free(rows), free(cache), free(slots), free(q), free(qo), free(k), free(v), free(vc), free(pos), free(am), free(sl);
}

static void rounding_cases(void)
{
    const float vals[] = {0.0f, -0.0f, 1.0f, -1.5f, INFINITY, -INFINITY, NAN, 1e-40f, -1e-45f, 3.4028235e38f,
                          1.00390625f, 1.01171875f, 65504.0f};
    const int64_t n = (int64_t)(sizeof(vals) / sizeof(vals[0]));
    float *x = exact((size_t)n, sizeof(float));
    uint16_t *out = exact((size_t)n, sizeof(uint16_t));
    memcpy(x, vals, sizeof(vals));
    oracle_round_bf16(x, out, n);
    expect(out[2] == 0x3f80 && out[1] == 0x8000, "bf16: 1 and -0");
    expect(out[10] == 0x3f80, "bf16: a tie rounds to even (down)");
    expect(out[11] == 0x3f82, "bf16: a tie rounds to even (up)");
    expect(out[4] == 0x7f80, "bf16: +inf");
    oracle_round_bf16(x, out, 0);
    free(x), free(out);
}

int main(void)
{
    planes_cases();
    rotate_cases();
    cache_cases();
    rounding_cases();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
