/*
 * Canvas M-RoPE oracle: plain, slow, scalar C (C11, libm only).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library.  It shares no code, header, table or constant with the
 * HIP library, and the HIP library never calls it.
 *
 * What it computes, and where that is defined:
 *
 *   Canvas rule (planes).  "MiniCPM-V-4.7-1B — Core AI" (Hugging Face card), section "How the VLM
 *   rides the text-only engine", the canvas table and the start/amount paragraph below it; also
 *   "MiniCPM-V-4.7-1B: canvas M-RoPE on the Qwen3.5 hybrid, on Core AI" (Core AI model-zoo page),
 *   section "The canvas rule and why the gate is on the planes".  One 448x448 image makes a frame
 *   of <image>, 64 image rows (the 8x8 merged grid, row-major), </image> and one "\n".  With O the
 *   index of <image>: text before the frame (p,p,p); <image> (O,O-1,O-1); row k (O,O+k//8,O+k%8);
 *   </image> (O,O+8,O+8); the "\n" (O,O,O); from start on (p-amount) on all three planes.  start is
 *   the index after </image> and the "\n" that follows it; amount = start - (O + 9) where
 *   9 = max(H,W) + 1 over the canvas.  A prompt with no image sends start = 2^30 and amount = 0.
 *
 *   Sections.  Same card, section "What it is": three planes (T,H,W) share the rotary frequencies in
 *   interleaved sections [11, 11, 10].  The pages do not give the per-index rule; this oracle takes
 *   the model configuration's rule: frequency j uses H if j%3==1 && j<33, W if j%3==2 && j<30,
 *   else T.
 *
 *   Rotary.  Not spelled out on the pages beyond 256-dim heads with 2 KV heads (the keyCache shape
 *   in "How the VLM rides the text-only engine").  Taken from the model configuration: rotate-half
 *   over the first rot_dim (64) dims of each head, inv_freq[j] = 1 / theta^(2j/rot_dim) with
 *   theta = 1e7, and the angle formed in fp32 as the model's rotary forms it.  Dims past rot_dim
 *   pass through unchanged.
 *
 * Precision: the angle is one fp32 multiply of fl32(pos) and the fp32 inv_freq table (that is how
 * the model's own rotary forms it); everything after the angle is double: cos/sin from libm and the
 * rotation products, then one round-to-nearest-even to fp32.  The bf16 reference is that fp32 value
 * rounded to nearest even in bf16.
 *
 * Parity pins (tests that hold this file to the pages and to mathematics, not to itself) live in the
 * CPU test suite: the pages' worked example, the start/amount identity, the text-only reduction to
 * 1-D RoPE, brute-force enumeration of the 8x8 grid, closed forms of the rotation.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_TEXT_ONLY_START (1 << 30)

/* ---------------------------------------------------------------------------------------------
 * Step 1: canvas origin O = index of the first <image> marker of the sequence, or -1 when the
 * sequence has none (card "How the VLM rides the text-only engine": O is the index of <image>).
 * ------------------------------------------------------------------------------------------- */
int32_t oracle_first_marker(const int32_t *ids, int32_t n, int32_t marker_id)
{
    for (int32_t p = 0; p < n; ++p)
        if (ids[p] == marker_id)
            return p;
    return -1;
}

/* The canvas: (T,H,W) offsets from O of <image>, the 64 rows k = 0..63 (row-major over the 8x8
 * grid) and </image>, in prompt order.  Returns the number of entries (66). */
static int32_t canvas_offsets(int32_t off[][3])
{
    int32_t n = 0;
    off[n][0] = 0; off[n][1] = -1; off[n][2] = -1; ++n;            /* <image>          */
    for (int32_t k = 0; k < 64; ++k) {                              /* image row k      */
        off[n][0] = 0; off[n][1] = k / 8; off[n][2] = k % 8; ++n;
    }
    off[n][0] = 0; off[n][1] = 8; off[n][2] = 8; ++n;               /* </image>         */
    return n;
}

/* The frame: its first frame_len tokens from O, the canvas then the marker tokens that follow
 * </image> at (O, O, O).  frame_len is 67 for this model's template (<image>, 64 rows, </image>, one
 * "\n"); a run of k such tokens gives 66 + k; Qwen-VL's rule counts neither </image> nor the "\n"
 * (65).  The offsets of frame token i (0 <= i < frame_len). */
static void frame_offset(int32_t i, int32_t thw[3])
{
    int32_t off[66][3];
    int32_t n = canvas_offsets(off);
    if (i < n) {
        thw[0] = off[i][0]; thw[1] = off[i][1]; thw[2] = off[i][2];
    } else {                                                        /* marker after </image> */
        thw[0] = 0; thw[1] = 0; thw[2] = 0;
    }
}

#define ORACLE_FRAME_LEN 67

/* ---------------------------------------------------------------------------------------------
 * Step 2: frame scalars.  start = the index after the frame (</image> and the marker tokens that
 * follow it, frame_len tokens from O); amount = start - (O + 9), with 9 = max(H, W) + 1 taken over
 * the canvas of the 8x8 grid (its </image> corner included, whichever tokens the frame counts).
 * Text-only: start = 2^30, amount = 0.
 * ------------------------------------------------------------------------------------------- */
void oracle_frame_scalars_len(int32_t origin, int32_t frame_len, int32_t *start, int32_t *amount)
{
    if (origin < 0) {
        *start = ORACLE_TEXT_ONLY_START;
        *amount = 0;
        return;
    }
    int32_t off[66][3];
    int32_t n = canvas_offsets(off);
    int32_t max_hw = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (off[i][1] > max_hw) max_hw = off[i][1];
        if (off[i][2] > max_hw) max_hw = off[i][2];
    }
    *start = origin + frame_len;
    *amount = *start - (origin + max_hw + 1);
}

void oracle_frame_scalars(int32_t origin, int32_t *start, int32_t *amount)
{
    oracle_frame_scalars_len(origin, ORACLE_FRAME_LEN, start, amount);
}

/* ---------------------------------------------------------------------------------------------
 * Step 3: planes of position p (the canvas table, first matching row wins).
 * ------------------------------------------------------------------------------------------- */
static void canvas_planes_at(int32_t p, int32_t origin, int32_t start, int32_t amount, int32_t thw[3])
{
    if (origin < 0 || p < origin) {                 /* text before the frame, or no image */
        thw[0] = thw[1] = thw[2] = p;
    } else if (p >= start) {                        /* everything after the frame */
        thw[0] = thw[1] = thw[2] = p - amount;
    } else {                                        /* inside the frame */
        int32_t d[3];
        frame_offset(p - origin, d);
        thw[0] = origin + d[0];
        thw[1] = origin + d[1];
        thw[2] = origin + d[2];
    }
}

/* Planes, start, amount and origin for a packed batch.  cu_seqlens has n_seqs + 1 entries; token t
 * of the batch is position p = t - cu_seqlens[s] of sequence s.  planes is [3][plane_stride] int32
 * (T row, H row, W row).  origin may be NULL. */
void oracle_planes(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                   int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount,
                   int32_t *origin)
{
    for (int32_t s = 0; s < n_seqs; ++s) {
        int32_t b = cu_seqlens[s], n = cu_seqlens[s + 1] - cu_seqlens[s];
        int32_t o = oracle_first_marker(ids + b, n, marker_id);
        int32_t st, am;
        oracle_frame_scalars(o, &st, &am);
        start[s] = st;
        amount[s] = am;
        if (origin) origin[s] = o;
        for (int32_t p = 0; p < n; ++p) {
            int32_t thw[3];
            canvas_planes_at(p, o, st, am, thw);
            planes[0 * plane_stride + b + p] = thw[0];
            planes[1 * plane_stride + b + p] = thw[1];
            planes[2 * plane_stride + b + p] = thw[2];
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * The frame length of sequence s: frame_len_seq[s] when the caller gives one for it, else the call's
 * frame_len.  An entry of 0 means "the call's"; an entry outside [65, 4096] cannot describe a frame
 * (the canvas alone is 66 tokens with </image>, 65 without) and is replaced by the call's frame_len
 * (the GPU flags such a sequence).  frame_len_seq may be NULL.
 * ------------------------------------------------------------------------------------------- */
int32_t oracle_seq_frame_len(const int32_t *frame_len_seq, int32_t s, int32_t frame_len)
{
    int32_t f = frame_len_seq ? frame_len_seq[s] : 0;
    if (f == 0 || f < 65 || f > 4096) return frame_len;
    return f;
}

/* ---------------------------------------------------------------------------------------------
 * Planes of a later piece of each sequence (chunked prefill, a second turn: Core AI model-zoo page,
 * section "Prefill in chunks and a second turn"; Hugging Face card, section "Measured", the chunked
 * prefill and second-question paragraphs).  The tokens of sequence s continue its earlier ones:
 * token i sits at position pos_offset[s] + i.  origin_in[s] is the canvas origin found in the earlier
 * pieces (-1: none yet); the first marker of the whole sequence wins, so a marker in this piece
 * counts only when no earlier piece had one.  pos_offset / origin_in may be NULL (0 / -1).
 * frame_len: tokens from O to start (67 for this model's template; see frame_offset), for every
 * sequence whose frame_len_seq entry (NULL: none) does not give its own (oracle_seq_frame_len): a
 * packed batch may mix templates whose frames end differently.
 * ------------------------------------------------------------------------------------------- */
void oracle_planes_chunk(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                         int32_t frame_len, const int32_t *frame_len_seq, const int32_t *pos_offset,
                         const int32_t *origin_in, int32_t *planes, int64_t plane_stride, int32_t *start,
                         int32_t *amount, int32_t *origin)
{
    for (int32_t s = 0; s < n_seqs; ++s) {
        int32_t b = cu_seqlens[s], n = cu_seqlens[s + 1] - cu_seqlens[s];
        int32_t off = pos_offset ? pos_offset[s] : 0;
        int32_t o = (origin_in && origin_in[s] >= 0) ? origin_in[s] : -1;
        if (o < 0) {
            int32_t f = oracle_first_marker(ids + b, n, marker_id);
            if (f >= 0) o = off + f;
        }
        int32_t st, am;
        oracle_frame_scalars_len(o, oracle_seq_frame_len(frame_len_seq, s, frame_len), &st, &am);
        start[s] = st;
        amount[s] = am;
        if (origin) origin[s] = o;
        for (int32_t i = 0; i < n; ++i) {
            int32_t thw[3];
            canvas_planes_at(off + i, o, st, am, thw);
            planes[0 * plane_stride + b + i] = thw[0];
            planes[1 * plane_stride + b + i] = thw[1];
            planes[2 * plane_stride + b + i] = thw[2];
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Rotary frequencies: inv_freq[j] = 1 / theta^(2j/rot_dim), j = 0 .. rot_dim/2 - 1.
 * theta^(2j/rot_dim) is evaluated in double and rounded once to fp32; the reciprocal is one IEEE
 * fp32 division (the model keeps inv_freq as an fp32 buffer).
 * ------------------------------------------------------------------------------------------- */
void oracle_inv_freq(double theta, int32_t rot_dim, float *inv_freq)
{
    for (int32_t j = 0; j < rot_dim / 2; ++j) {
        float p = (float)pow(theta, (2.0 * j) / (double)rot_dim);
        inv_freq[j] = 1.0f / p;
    }
}

/* Which plane frequency j reads: 0 = T, 1 = H, 2 = W (interleaved sections [11, 11, 10]). */
int32_t oracle_plane_of_freq(int32_t j)
{
    if (j % 3 == 1 && j < 33) return 1;
    if (j % 3 == 2 && j < 30) return 2;
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Rotation of one head (x, y: head_dim floats).  For j < rot_dim/2 with h = rot_dim/2:
 *   y[j]     = x[j]     * cos(a_j) - x[j + h] * sin(a_j)
 *   y[j + h] = x[j + h] * cos(a_j) + x[j]     * sin(a_j)
 * a_j = fl32(fl32(pos_j) * inv_freq[j]), pos_j the plane that frequency j reads.  Double math,
 * one RNE rounding to fp32 per output.  Dims >= rot_dim are copied.  y64 (nullable) receives the
 * unrounded double results.
 * ------------------------------------------------------------------------------------------- */
static void rotate_head(const float *x, float *y, double *y64, int32_t head_dim, int32_t rot_dim,
                        const int32_t thw[3], const float *inv_freq)
{
    int32_t h = rot_dim / 2;
    for (int32_t j = 0; j < h; ++j) {
        float pos = (float)thw[oracle_plane_of_freq(j)];
        float a = pos * inv_freq[j];
        double c = cos((double)a), s = sin((double)a);
        double x1 = x[j], x2 = x[j + h];
        double r1 = x1 * c - x2 * s;
        double r2 = x2 * c + x1 * s;
        y[j] = (float)r1;
        y[j + h] = (float)r2;
        if (y64) {
            y64[j] = r1;
            y64[j + h] = r2;
        }
    }
    for (int32_t d = rot_dim; d < head_dim; ++d) {
        y[d] = x[d];
        if (y64) y64[d] = x[d];
    }
}

/* Rotate n_tokens x n_heads heads.  x is addressed as x[t*tok_stride + hd*head_stride + d] (float
 * elements); y (and y64 if not NULL) is dense [n_tokens][n_heads][head_dim].  planes is
 * [3][plane_stride] int32 with token t at column t. */
void oracle_rotate(const float *x, int64_t n_tokens, int32_t n_heads, int64_t tok_stride,
                   int64_t head_stride, int32_t head_dim, int32_t rot_dim, const int32_t *planes,
                   int64_t plane_stride, double theta, float *y, double *y64)
{
    float inv_freq[512];
    oracle_inv_freq(theta, rot_dim, inv_freq);
    for (int64_t t = 0; t < n_tokens; ++t) {
        int32_t thw[3] = {planes[t], planes[plane_stride + t], planes[2 * plane_stride + t]};
        for (int32_t hd = 0; hd < n_heads; ++hd) {
            int64_t o = (t * n_heads + hd) * (int64_t)head_dim;
            rotate_head(x + t * tok_stride + hd * head_stride, y + o, y64 ? y64 + o : NULL, head_dim,
                        rot_dim, thw, inv_freq);
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Paged cache write.  Row r (row_elems floats: every KV head of one token) goes to the cache slot
 * slots[r]: block slot / block_size, row slot % block_size of a cache laid out
 * [num_blocks][block_size][row_elems].  A slot < 0 or >= num_blocks * block_size writes nothing.
 * The K and V caches are the decoder's state ("How the VLM rides the text-only engine": the
 * keyCache [6, 1, 2, -1, 256]); the paging is the serving engine's layout, not the pages'.
 * ------------------------------------------------------------------------------------------- */
void oracle_scatter_rows(const float *rows, int64_t n_rows, int64_t row_elems, const int64_t *slots,
                         int32_t block_size, int64_t num_blocks, float *cache)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t slot = slots[r];
        if (slot < 0 || slot >= num_blocks * (int64_t)block_size) continue;
        const int64_t block = slot / block_size, within = slot % block_size;
        memcpy(cache + (block * block_size + within) * row_elems, rows + r * row_elems,
               sizeof(float) * (size_t)row_elems);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Decode: a generated token of sequence s sits at position pos[s]; every position from start on,
 * generated tokens included, takes p - amount on all three planes (canvas table, last row).
 * q: [n_seqs][n_q_heads][head_dim] dense, rotated into q_out (dense, same shape).
 * k: [n_seqs][n_k_heads][head_dim] dense; the rotated head is written into the paged cache copy at
 * slot_mapping[s] (block = slot / block_size, row = slot % block_size); a slot < 0 or
 * >= num_blocks * block_size skips the write.  v (nullable): [n_seqs][n_k_heads][head_dim], written
 * unrotated into v_cache at the same slot (V takes no position).
 * cache element (block, row, head, d) is at block*cache_block_stride + row*cache_tok_stride +
 * head*cache_head_stride + d (float elements), the same for both caches.
 * ------------------------------------------------------------------------------------------- */
void oracle_decode(const float *q, int32_t n_q_heads, const float *k, int32_t n_k_heads, int32_t n_seqs,
                   const int32_t *pos, const int32_t *amount, int32_t head_dim, int32_t rot_dim,
                   double theta, float *q_out, float *cache, const int64_t *slot_mapping,
                   int32_t block_size, int64_t num_blocks, int64_t cache_block_stride, int64_t cache_head_stride,
                   int64_t cache_tok_stride, const float *v, float *v_cache)
{
    float inv_freq[512];
    float y[4096];
    oracle_inv_freq(theta, rot_dim, inv_freq);
    for (int32_t s = 0; s < n_seqs; ++s) {
        int32_t plane = pos[s] - amount[s];
        int32_t thw[3] = {plane, plane, plane};
        for (int32_t hd = 0; hd < n_q_heads; ++hd) {
            int64_t o = ((int64_t)s * n_q_heads + hd) * head_dim;
            rotate_head(q + o, q_out + o, NULL, head_dim, rot_dim, thw, inv_freq);
        }
        int64_t slot = slot_mapping[s];
        if (slot < 0 || slot >= num_blocks * (int64_t)block_size) continue;
        int64_t blk = slot / block_size, row = slot % block_size;
        for (int32_t hd = 0; hd < n_k_heads; ++hd) {
            const int64_t src = ((int64_t)s * n_k_heads + hd) * head_dim;
            const int64_t dst = blk * cache_block_stride + row * cache_tok_stride + hd * cache_head_stride;
            rotate_head(k + src, y, NULL, head_dim, rot_dim, thw, inv_freq);
            memcpy(cache + dst, y, sizeof(float) * (size_t)head_dim);
            if (v) memcpy(v_cache + dst, v + src, sizeof(float) * (size_t)head_dim);
        }
    }
}

/* Round fp32 to bf16, nearest even (NaN stays a quiet NaN of the same sign). */
void oracle_round_bf16(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], sizeof u);
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7fffu + lsb) >> 16);
    }
}
