/*
 * libmrope -- canvas M-RoPE for MI355X (gfx950): position planes from token ids, and the
 * interleaved multi-section rotary embedding of Q and K, for prefill and decode.
 *
 * What is computed is defined on two pages:
 *   [card]  Hugging Face card "MiniCPM-V-4.7-1B -- Core AI" (mlboydaisuke/MiniCPM-V-4.7-1B-CoreAI):
 *           section "What it is" (three planes T, H, W in interleaved sections [11, 11, 10]) and
 *           section "How the VLM rides the text-only engine" (the canvas table; start and amount;
 *           the keyCache shape [6, 1, 2, -1, 256]: 2 KV heads of 256 dims; id layout).
 *   [zoo]   Core AI model-zoo page "MiniCPM-V-4.7-1B: canvas M-RoPE on the Qwen3.5 hybrid, on Core
 *           AI", section "The canvas rule and why the gate is on the planes".
 * Not on the pages, taken from the model configuration: rotate-half over the first 64 dims of each
 * head (32 frequencies), theta = 1e7, and frequency j reading plane H if j%3==1 && j<33, W if
 * j%3==2 && j<30, else T.
 *
 * Conventions for every entry point
 *   - Pointers to tensors are DEVICE pointers owned by the caller.  The library allocates no
 *     device memory (mrope_apply_ids_noalloc's workspace is a static device array of the library,
 *     see there).  State that crosses calls lives in the caller's workspace (see
 *     mrope_workspace_bytes); the library itself keeps only a per-thread copy of the last error
 *     text (mrope_last_error), per device the compute-unit count it sizes its grids by (read once)
 *     and the static array's address, and the process-wide test-hook flags (mrope_set_test_hooks).
 *   - Every call enqueues its work on `stream` (a hipStream_t; NULL = the null stream) and returns
 *     without synchronising.  Calls issue no memset and no allocation, so they can be captured in a
 *     HIP graph.
 *   - Arguments are checked on the host before anything is enqueued; a bad argument returns a
 *     status != MROPE_OK and enqueues nothing.  A failed launch returns MROPE_ERR_HIP.
 *     mrope_last_error() gives a one-line description of the last failure on the calling thread.
 *   - Strides are in ELEMENTS of the tensor's dtype.  Q and K element (t, h, d) is at
 *     t*tok_stride + h*head_stride + d; d is contiguous.
 *   - Data-dependent conditions (two image markers in a sequence, a frame running past the end of
 *     its sequence, a per-sequence frame length that describes no frame) are reported per sequence
 *     in the optional seq_flags array, never by a status.
 *   - Calls that share a workspace must be ordered (same stream, or synchronised); concurrent calls
 *     on one workspace race.
 */
#ifndef MROPE_H
#define MROPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MROPE_ABI_VERSION 5

typedef enum {
    MROPE_OK = 0,
    MROPE_ERR_ARG = 1,         /* NULL pointer, negative size, bad stride, bad theta, ...         */
    MROPE_ERR_ALIGN = 2,       /* Q/K/cache pointer or stride breaks 16-byte vector alignment     */
    MROPE_ERR_UNSUPPORTED = 3, /* rot_dim != 64, head_dim not in [64, 1024], head count > 64, dtype */
    MROPE_ERR_WORKSPACE = 4,   /* workspace NULL, too small or misaligned                          */
    MROPE_ERR_HIP = 5          /* the HIP runtime reported an error for a launch                   */
} mrope_status;

typedef enum {
    MROPE_F32 = 0,   /* float32 Q/K/cache */
    MROPE_BF16 = 1,  /* bfloat16 Q/K/cache */
    MROPE_F16 = 2    /* IEEE half Q/K/cache (the pages' engines keep KV state in fp16) */
} mrope_dtype;

/* seq_flags bits (optional per-sequence output of the plane-deriving calls). */
#define MROPE_SEQ_MULTI_MARKER 1u /* more than one <image> marker; planes follow the first frame */
#define MROPE_SEQ_FRAME_OVERRUN 2u /* the frame (frame_len tokens from the marker, 67 by default)
                                     runs past the end of the sequence */
#define MROPE_SEQ_BAD_FRAME_LEN 4u /* the sequence's frame_len_seq entry was neither 0 nor in
                                     [65, 4096]; the call's frame_len was used instead */

/* Text-only sequences get start = 2^30 and amount = 0 (card, start/amount paragraph). */
#define MROPE_TEXT_ONLY_START (1 << 30)

int mrope_abi_version(void);

/* Static string for a status code; never NULL. */
const char *mrope_status_string(int status);

/* Description of the last non-OK status returned on the calling thread ("" if none). */
const char *mrope_last_error(void);

/* Test and tuning hooks: not for production use.  They choose among the library's own kernels for
 * mrope_apply_ids and never change results, so the test suite can run every kernel on every input.
 * Process-wide; returns the previous value.  0 (the default) lets the library choose.
 *   MROPE_HOOK_FUSED_CHUNKED     always the chunk-per-workgroup fused kernel
 *   MROPE_HOOK_FUSED_SCAN_FIRST  always the scan-first fused kernel (8 Q + 2 K heads, no cache write)
 *   MROPE_HOOK_SCAN_FALLBACK     scan-first kernel whose rotation workgroups derive their planes
 *                                themselves instead of waiting for the scan's handover
 *   MROPE_HOOK_F32_EIGHT_LANES   fp32 with eight lanes a token (two 16-byte loads per head and lane)
 *                                instead of sixteen: mrope_apply, mrope_apply_ids, and the cache
 *                                writes of mrope_apply_kv / mrope_apply_ids_kv (then the generic
 *                                kernels, one head at a time) */
#define MROPE_HOOK_FUSED_CHUNKED 1
#define MROPE_HOOK_FUSED_SCAN_FIRST 2
#define MROPE_HOOK_SCAN_FALLBACK 4
#define MROPE_HOOK_F32_EIGHT_LANES 8
int mrope_set_test_hooks(int flags);

/* ---------------------------------------------------------------------------------------------
 * Workspace for the calls that derive planes from ids (mrope_planes, mrope_apply_ids).
 *
 * Returns the bytes needed for n_tokens packed tokens.  The workspace must be 256-byte aligned
 * device memory, zero-filled (or passed once through mrope_workspace_init) before its first use;
 * it needs no clearing between calls.  It holds a device epoch counter and room for one 64-bit
 * status word per 512-token chunk, through which a chunk hands the first marker of a sequence to
 * the chunks after it, then the planes handover of the scan-first fused kernel (24 bytes per 32
 * tokens, and 24 bytes per token for parts that hold more than one sequence): about 24.8 bytes per
 * token in all.
 *
 * Epochs.  The plane-deriving calls take an `epoch` that tags the status words they write, so a
 * call never mistakes words left by an earlier call for its own:
 *   epoch != 0  the caller's tag (low 29 bits used); it must differ from the epoch of the previous
 *               call on the same workspace (a call counter does).  No extra work.
 *   epoch == 0  the library reads a counter held in the workspace and advances it with a
 *               one-thread kernel after the scan -- use this when the call is captured in a HIP
 *               graph, whose replays would otherwise repeat one tag.
 * Device-counter tags carry bit 29, caller tags never do, so the two kinds can share a workspace.
 * ------------------------------------------------------------------------------------------- */
size_t mrope_workspace_bytes(int64_t n_tokens);

/* Zero-fill `bytes` of workspace with a kernel (no memset node) on `stream`. */
mrope_status mrope_workspace_init(void *workspace, size_t bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_planes -- canvas position planes from token ids ([card] canvas table; [zoo] canvas rule).
 *
 * ids        [n_tokens] int32, packed sequences (token t of sequence s is ids[cu_seqlens[s] + t]).
 * cu_seqlens [n_seqs + 1] int32, cu_seqlens[0] = 0, non-decreasing, cu_seqlens[n_seqs] == n_tokens
 *            (n_tokens is passed explicitly so the host never reads device memory).  Empty
 *            sequences are allowed.
 * marker_id  the <image> token id (248078 for the model's tokenizer).
 * frame_len  tokens from <image> to start: the canvas (<image>, 64 rows), then </image> and the
 *            marker tokens after it ([card] canvas table: start is the index after </image> and the
 *            markers that follow).  0 = 67, this template's one "\n"; 66 + k for a run of k such
 *            tokens; 65 for Qwen-VL's rule ([zoo] "CoreAIKit (VLChat)": +64 and 56 from the first
 *            pad).  Allowed: 0 or 65..4096.  amount = frame_len - 9 for every length.
 * frame_len_seq  [n_seqs] int32 (nullable = every sequence takes frame_len): the frame length of
 *            each sequence, for a packed batch whose prompts come from templates whose frames end
 *            differently (65, 67, 66 + k as above).  An entry of 0 takes the call's frame_len; an
 *            entry outside [65, 4096] also takes it and sets MROPE_SEQ_BAD_FRAME_LEN in seq_flags
 *            (the status stays MROPE_OK: the host never reads the array).  Everything below that
 *            names frame_len means the sequence's own.
 * pos_offset [n_seqs] int32 (nullable = all 0): position of each sequence's first token in this call
 *            within the whole sequence.  A prompt may be fed in pieces -- prefill in chunks, a second
 *            turn continuing the first ([zoo] section "Prefill in chunks and a second turn") -- and
 *            token i of sequence s then sits at position p = pos_offset[s] + i.
 * origin_in  [n_seqs] int32 (nullable = all -1): the canvas origin an earlier piece found (its
 *            `origin` output), -1 if none.  The first marker of the whole sequence wins: a marker in
 *            this piece is used only when origin_in[s] < 0.  Feeding the pieces in order, each with
 *            the previous piece's origin, gives exactly the planes of one call on the whole sequence.
 * planes     [3][plane_stride] int32 out: row 0 = T, row 1 = H, row 2 = W; plane_stride >= n_tokens.
 *            For position p of a sequence whose first marker is at O, with F = frame_len,
 *            start = O + F and amount = F - 9 (67 and 58 by default):
 *              p < O or no marker          -> (p, p, p)
 *              p == O                      -> (O, O-1, O-1)
 *              p == O+1+k, k < 64          -> (O, O + k/8, O + k%8)
 *              p == O+65 < start           -> (O, O+8, O+8)
 *              O+66 <= p < start           -> (O, O, O)
 *              p >= start                  -> (p-amount, p-amount, p-amount)
 * start, amount  [n_seqs] int32 out (nullable): start = O + frame_len, amount = frame_len - 9 for
 *            an image sequence; 2^30 and 0 for a text-only one (so far).
 * origin     [n_seqs] int32 out (nullable): O (a position in the whole sequence), or -1 when the
 *            sequence has no marker so far.
 * seq_flags  [n_seqs] int32 out (nullable): MROPE_SEQ_* bits (a marker here when origin_in >= 0
 *            counts as a second marker; "frame past the end" means past the tokens seen so far).
 * workspace  see mrope_workspace_bytes(n_tokens).
 *
 * epoch      see mrope_workspace_bytes.
 *
 * One launch (plus a one-thread kernel when epoch == 0): each 512-token chunk finds its markers with
 * wavefront ballots over 64-id loads and takes the first marker of a sequence that began in an
 * earlier chunk from its predecessors by a decoupled look-back with bounded polls (a predecessor
 * that has not published after them is evaluated from its ids), so no chunk waits without bound.
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_planes(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                          int32_t marker_id, int32_t frame_len, const int32_t *frame_len_seq,
                          const int32_t *pos_offset, const int32_t *origin_in, int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount,
                          int32_t *origin, int32_t *seq_flags, void *workspace, size_t workspace_bytes,
                          uint32_t epoch, void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_apply -- rotate Q and K heads with given planes ([card] "What it is": interleaved sections).
 *
 * q          Q heads, dtype `dtype`, element (t, h, d) at t*q_tok_stride + h*q_head_stride + d.
 * k          K heads likewise (may be NULL when n_k_heads == 0).
 * n_tokens   tokens to rotate (0 = nothing to do).
 * head_dim   dims per head, multiple of 8, 64..1024 (256 for the model).
 * rot_dim    rotated dims per head; must be 64.  For j < 32, with a_j = fl32(fl32(pos_j) *
 *            inv_freq[j]), inv_freq[j] = fl32(1 / fl32(theta^(2j/64))):
 *              y[j]    = x[j]    * cos(a_j) - x[j+32] * sin(a_j)
 *              y[j+32] = x[j+32] * cos(a_j) + x[j]    * sin(a_j)
 *            pos_j is the T, H or W plane of the token by the rule in the file header.
 * planes     [3][plane_stride] int32 (as written by mrope_planes); |plane| < 2^24.
 * theta      rotary base (1e7 for the model), > 0 and finite.
 * Precision: the angle is the fp32 product above; cos, sin and the two products of each output are
 *            double; each output is rounded to nearest-even once to fp32 and, for bf16 / fp16, once
 *            more to the 16-bit type.
 * q_out, k_out  NULL: rotate in place (dims >= rot_dim are never read or written).  Otherwise the
 *            full heads are written there, with the same strides as q / k (no aliasing with the
 *            inputs): a first launch copies dims >= rot_dim, the rotation launch writes the rest.
 *            Both NULL or both non-NULL when both head sets are present; a call with no K heads
 *            may pass q_out alone, one with no Q heads k_out alone.
 * Alignment: q, k, q_out, k_out 16-byte aligned; strides multiples of 8 (bf16, fp16) or 4 (fp32).
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_apply(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, void *k,
                         int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads, int64_t n_tokens,
                         int32_t head_dim, int32_t rot_dim, int32_t dtype, const int32_t *planes,
                         int64_t plane_stride, double theta, void *q_out, void *k_out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_apply_ids -- planes derivation and rotation fused in ONE launch (plus a one-thread kernel
 * when epoch == 0, and out of place the copy launch described under mrope_apply): ids -> first
 * marker per sequence -> planes (kept on chip) -> rotate Q and K.
 * Arguments as in mrope_planes and mrope_apply; planes_out (nullable) additionally receives the
 * planes ([3][plane_stride]).  With planes_out, an input of more than 512 tokens per resident
 * rotation workgroup (262,144 on a 256-CU MI355X; the model's head shape) runs as mrope_planes into
 * planes_out followed by mrope_apply from it: the same results, and faster at that size.
 * n_tokens must equal cu_seqlens[n_seqs].  The Q/K loads of a chunk are issued while its scan
 * runs.
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_apply_ids(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, void *k,
                             int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads, int64_t n_tokens,
                             int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta, void *q_out,
                             void *k_out, const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs,
                             int32_t marker_id, int32_t frame_len, const int32_t *frame_len_seq,
                             const int32_t *pos_offset, const int32_t *origin_in, int32_t *planes_out,
                             int64_t plane_stride, int32_t *start,
                             int32_t *amount, int32_t *origin, int32_t *seq_flags, void *workspace,
                             size_t workspace_bytes, uint32_t epoch, void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_apply_ids_noalloc -- mrope_apply_ids for callers that cannot allocate device memory or pass
 * a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors as mrope_apply_ids, without workspace, workspace_bytes and epoch.
 * The workspace is a static device array inside the library: one copy per GPU, allocated when the
 * library's code is loaded and held until the process ends (MROPE_NOALLOC_MAX_TOKENS tokens'
 * worth, about 26.0 MB).  n_tokens above MROPE_NOALLOC_MAX_TOKENS returns MROPE_ERR_WORKSPACE.
 * The call allocates nothing.  Its first call on a device looks the array up and clears it with a
 * kernel on `stream`; that first call must not be captured in a graph (MROPE_ERR_ARG if it is).
 * Each later call tags its words with the device epoch counter kept in the array, so calls and
 * graph replays need no clearing.  All calls on one GPU share the array: calls that overlap on
 * one GPU (different streams, not ordered) race.
 * ------------------------------------------------------------------------------------------- */
#define MROPE_NOALLOC_MAX_TOKENS (1 << 20)
mrope_status mrope_apply_ids_noalloc(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                                     void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads,
                                     int64_t n_tokens, int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta,
                                     void *q_out, void *k_out, const int32_t *ids, const int32_t *cu_seqlens,
                                     int32_t n_seqs, int32_t marker_id, int32_t frame_len,
                                     const int32_t *frame_len_seq, const int32_t *pos_offset,
                                     const int32_t *origin_in, int32_t *planes_out, int64_t plane_stride,
                                     int32_t *start, int32_t *amount, int32_t *origin, int32_t *seq_flags,
                                     void *stream);

/* ---------------------------------------------------------------------------------------------
 * Paged K/V cache (mrope_apply_kv, mrope_apply_ids_kv, mrope_decode).  The K and V caches are the
 * decoder's state ([card] "How the VLM rides the text-only engine": the keyCache [6, 1, 2, -1, 256],
 * 2 KV heads of 256 dims); their paging is the serving engine's layout.
 *
 * k_cache, v_cache  element (block, row, head, d) at block*cache_block_stride + row*cache_tok_stride
 *            + head*cache_head_stride + d, in elements of `dtype`; both caches use these strides.
 * slot_mapping  int64, one per token (prefill) or per sequence (decode).  The token goes to block
 *            slot / block_size, row slot % block_size.  slot < 0 or slot >= num_blocks*block_size:
 *            nothing is written for it.  Two tokens with one slot: undefined which lands.
 * A token's K heads are written whole: the first rot_dim dims rotated, the rest copied.  Its V
 * heads (as many as K heads) are copied unrotated.  The caches must not overlap q, k or v.
 * Alignment: caches 16-byte aligned, cache strides multiples of 8 (bf16, fp16) or 4 (fp32).
 * ------------------------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------------------------
 * mrope_apply_kv -- prefill rotation with the K/V cache write fused in: Q rotated in place (as
 * mrope_apply), K rotated and written whole into k_cache, V copied into v_cache, both at
 * slot_mapping[t] of each token t.  k and v are read only.  Arguments as in mrope_apply and the
 * paged-cache block above; v (n_kv_heads heads, element (t, h, d) at t*v_tok_stride +
 * h*v_head_stride + d) may be NULL together with v_cache (then only K is written).
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_apply_kv(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                            const void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_kv_heads,
                            const void *v, int64_t v_tok_stride, int64_t v_head_stride, int64_t n_tokens,
                            int32_t head_dim, int32_t rot_dim, int32_t dtype, const int32_t *planes,
                            int64_t plane_stride, double theta, void *k_cache, void *v_cache,
                            const int64_t *slot_mapping, int32_t block_size, int64_t num_blocks,
                            int64_t cache_block_stride, int64_t cache_tok_stride, int64_t cache_head_stride,
                            void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_apply_ids_kv -- mrope_apply_ids with the K/V cache write of mrope_apply_kv: ids -> planes
 * -> Q rotated in place, K rotated into k_cache, V copied into v_cache, in one launch.  The whole
 * prefill step of an attention layer's positions and cache update.
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_apply_ids_kv(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                                const void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_kv_heads,
                                const void *v, int64_t v_tok_stride, int64_t v_head_stride, int64_t n_tokens,
                                int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta,
                                const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                                int32_t frame_len, const int32_t *frame_len_seq, const int32_t *pos_offset,
                                const int32_t *origin_in, int32_t *planes_out, int64_t plane_stride, int32_t *start, int32_t *amount, int32_t *origin,
                                int32_t *seq_flags, void *workspace, size_t workspace_bytes, uint32_t epoch,
                                void *k_cache, void *v_cache, const int64_t *slot_mapping, int32_t block_size,
                                int64_t num_blocks, int64_t cache_block_stride, int64_t cache_tok_stride,
                                int64_t cache_head_stride, void *stream);

/* ---------------------------------------------------------------------------------------------
 * mrope_decode -- one generated token per sequence ([card] canvas table, last row: every position
 * from start on, generated tokens included, takes p - amount on all three planes).
 *
 * q          [n_seqs] tokens of Q heads (strides as in mrope_apply), rotated in place.
 * k          [n_seqs] tokens of new K heads (read only), written whole into k_cache at
 *            slot_mapping[s], the first rot_dim dims rotated (paged-cache block above).
 * v          nullable: [n_seqs] tokens of new V heads (n_k_heads heads, read only), copied
 *            unrotated into v_cache at the same slot.  NULL together with v_cache.
 * pos, amount  [n_seqs] int32: the token's position p and its sequence's amount; plane = p - amount.
 * slot_mapping [n_seqs] int64.
 * ------------------------------------------------------------------------------------------- */
mrope_status mrope_decode(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                          const void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads,
                          const void *v, int64_t v_tok_stride, int64_t v_head_stride, int32_t n_seqs,
                          const int32_t *pos, const int32_t *amount, void *k_cache, void *v_cache,
                          const int64_t *slot_mapping, int32_t block_size, int64_t num_blocks,
                          int64_t cache_block_stride, int64_t cache_tok_stride, int64_t cache_head_stride,
                          int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MROPE_H */
