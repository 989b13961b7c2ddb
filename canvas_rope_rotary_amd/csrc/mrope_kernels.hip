// libmrope kernels for gfx950 (CDNA4, wave64).
//
// What is computed (the pages):
//   Hugging Face card "MiniCPM-V-4.7-1B -- Core AI", section "How the VLM rides the text-only engine":
//   the canvas table (planes per position for one 448x448 image after plain text), start and amount;
//   section "What it is": three planes T, H, W sharing the rotary frequencies in interleaved sections
//   [11, 11, 10].  Core AI model-zoo page "MiniCPM-V-4.7-1B: canvas M-RoPE on the Qwen3.5 hybrid, on
//   Core AI", section "The canvas rule and why the gate is on the planes".
//
// Kernels
//   planes_kernel     ids -> first marker per sequence (ballot + decoupled look-back over 512-token
//                     chunks) -> planes, start, amount
//   apply_kernel      planes -> cos/sin on the fly -> rotate-half of Q and K (the HBM stream)
//   apply_kv_kernel   the same, with K rotated into and V copied to paged K/V caches
//   apply_any_kernel  other head counts and head dims (one workgroup per 32 tokens)
//   apply_ids_kernel  planes from ids and the rotation in one launch; a chunk's planes stay on chip
//                     (per token in LDS, or as one sequence's begin/offset/origin)
//   decode_kernel     one token per sequence: Q in place, K rotated and V copied to a paged cache
//
// Thread layout of the rotary kernels: eight lanes per token; lane pair m holds frequencies
// 8m .. 8m+7, one lane the x_j dims and its neighbour the x_{j+32} dims of every head, so the eight
// lanes of a token read or write one whole 128-byte line (bf16) per instruction.  Partners swap data
// by DPP; each sincos is evaluated once per token, and a lane applies its (cos, sin) to all heads of
// its token.  (Four lanes per token, each reading the two 64-byte halves of a line with two
// instructions, measured 25% slower on this access pattern.)
//
// Precision: the angle is one fp32 multiply (as the model's rotary forms it); cos/sin and the two
// products of each output are double (the same per-lane rate as fp32 on this chip with packed fp32
// off); each output is rounded once to fp32 and, for bf16/fp16 I/O, once more to the 16-bit type
// (nearest even).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "mrope_internal.h"
#include "mrope_math.h"

namespace mrope {
namespace {

// ------------------------------------------------------------------ the canvas rule ------------
constexpr int kGrid = 8;                      // 8x8 merged grid of one 448x448 image
constexpr int kRows = kGrid * kGrid;          // 64 image rows, row-major
constexpr int kExtent = kGrid + 1;            // largest H/W offset on the canvas (</image>) + 1
// The frame runs frame_len tokens from O to start: <image>, the rows, then </image> and the marker
// tokens after it (67 for this model's template: one "\n"; 66 + k for a run of k; 65 under
// Qwen-VL's rule, which leaves </image> and the "\n" out).  amount = start - (O + 9) = frame_len - 9.
constexpr int32_t kTextStart = 1 << 30;       // text-only prompt: start = 2^30, amount = 0
constexpr int32_t kNone = 0x7fffffff;         // "no marker"

// Planes of position p; o = the sequence's canvas origin if it lies at or before p, else kNone;
// fl = frame length (tokens from o to start).
__device__ __forceinline__ void canvas_planes(int32_t p, int32_t o, int32_t fl, int32_t &t, int32_t &h, int32_t &w)
{
    if (o == kNone) {
        t = h = w = p;
        return;
    }
    const int32_t d = p - o;
    if (d >= fl) {
        t = h = w = p - (fl - kExtent);
        return;
    }
    t = o;
    if (d == 0) {                 // <image>
        h = w = o - 1;
    } else if (d <= kRows) {      // image row k = d - 1
        h = o + ((d - 1) >> 3);
        w = o + ((d - 1) & 7);
    } else if (d == kRows + 1) {  // </image>
        h = w = o + kGrid;
    } else {                      // the "\n" after </image>
        h = w = o;
    }
}

// ------------------------------------------------------------------ workspace ------------------
// Header (256 bytes): the device epoch counter, used when the caller passes epoch 0; then one status
// word per 512-token chunk, the scan-first kernel's part records and its per-token planes of shared
// parts (ws_layout).
struct WsHeader {
    uint32_t epoch;
};

// status word of a chunk: [63:34] epoch | [33:32] flag | [31] multi | [30:0] first marker (global idx)
constexpr uint64_t kAgg = 1;   // value covers only this chunk's part of its last sequence
constexpr uint64_t kIncl = 2;  // value covers the whole sequence up to the end of this chunk
constexpr uint32_t kEpochMask = 0x1fffffffu;  // caller epochs use 29 bits ...
constexpr uint32_t kDeviceEpochBit = 0x20000000u;  // ... device-counter epochs carry bit 29 as well

__device__ __forceinline__ uint64_t status_word(uint32_t epoch, uint64_t flag, bool multi, int32_t first)
{
    return ((uint64_t)epoch << 34) | (flag << 32) | ((uint64_t)(multi ? 1u : 0u) << 31) |
           (uint64_t)((uint32_t)first & 0x7fffffffu);
}

__device__ __forceinline__ uint64_t *status_array(void *ws)
{
    return reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + kWsHeaderBytes);
}

template <typename T>
__device__ __forceinline__ T aload(const T *p)
{
    return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void astore(T *p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The epoch that tags this launch's status words: the caller's (29 bits), or the device counter's
// with bit 29 set (caller passed 0; a one-thread kernel advances the counter after the launch).
__device__ __forceinline__ uint32_t launch_epoch(const Scan &sc)
{
    if (sc.epoch) return sc.epoch & kEpochMask;
    return (aload(&static_cast<const WsHeader *>(sc.workspace)->epoch) & kEpochMask) | kDeviceEpochBit;
}

// ------------------------------------------------------------------ wave helpers ---------------
// v's value in lane r (r wave-uniform): two scalar reads, no LDS permute.
__device__ __forceinline__ int64_t lane_value(int64_t v, int r)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)v, r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)((uint64_t)v >> 32), r);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int32_t wave_min(int32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

// Numbers of entries of the non-decreasing array cu[0..n] that are <= ka and <= kb, by a 128-ary
// search of the whole wave for both keys at once: per level each lane samples two positions per key
// (four independent loads) and ballots count the samples at or below the key (one level up to 127
// sequences, two up to 16,383).
__device__ void wave_count_le2(const int32_t *cu, int32_t n, int64_t ka, int64_t kb, int lane, int32_t &ca, int32_t &cb)
{
    int32_t lo[2] = {0, 0}, hi[2] = {n + 1, n + 1};
    const int64_t key[2] = {ka, kb};
    bool done[2] = {false, false};
    int32_t res[2] = {0, 0};
    while (!(done[0] && done[1])) {
        int32_t stride[2], p0[2], p1[2];
        bool le0[2], le1[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            stride[q] = (hi[q] - lo[q] + 127) / 128;
            p0[q] = lo[q] + (2 * lane) * stride[q];
            p1[q] = p0[q] + stride[q];
        }
        // the four loads of a level go out together (clamped to valid entries, masked after)
        int32_t x0[2], x1[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            x0[q] = cu[min(p0[q], n)];
            x1[q] = cu[min(p1[q], n)];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            le0[q] = !done[q] && p0[q] < hi[q] && (int64_t)x0[q] <= key[q];
            le1[q] = !done[q] && p1[q] < hi[q] && (int64_t)x1[q] <= key[q];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (done[q]) continue;
            const int c = __builtin_popcountll(__ballot(le0[q])) + __builtin_popcountll(__ballot(le1[q]));
            if (stride[q] <= 1 || c == 0) {
                res[q] = lo[q] + c;
                done[q] = true;
                continue;
            }
            const int32_t nhi = lo[q] + c * stride[q];
            lo[q] = lo[q] + (c - 1) * stride[q] + 1;
            hi[q] = min(hi[q], nhi);
            if (lo[q] >= hi[q]) {
                res[q] = lo[q];
                done[q] = true;
            }
        }
    }
    ca = res[0];
    cb = res[1];
}

// A lower bound lo on the number of entries of the non-decreasing array cu[0..n] that are <= key,
// within 63 of it: the 128-ary search above for one key, stopped once the candidates fit one
// 64-entry window (one level up to 8,063 sequences).  A window of cu loaded from lo - 1 then holds
// the exact count's last entry.
__device__ int32_t wave_bracket_le(const int32_t *cu, int32_t n, int64_t key, int lane)
{
    int32_t lo = 0, hi = n + 1;
    while (hi - lo > 63) {
        const int32_t stride = (hi - lo + 127) / 128;
        const int32_t p0 = lo + (2 * lane) * stride, p1 = p0 + stride;
        const int32_t x0 = cu[min(p0, n)], x1 = cu[min(p1, n)];
        const int c = __builtin_popcountll(__ballot(p0 < hi && (int64_t)x0 <= key)) +
                      __builtin_popcountll(__ballot(p1 < hi && (int64_t)x1 <= key));
        if (c == 0) return lo;
        const int32_t nhi = min(hi, lo + c * stride);
        lo = lo + (c - 1) * stride + 1;
        hi = nhi;
    }
    return lo;
}

// Bits [lo, hi) of a 64-bit word, for any lo, hi (clamped to [0, 64]).
__device__ __forceinline__ uint64_t bit_range(int lo, int hi)
{
    lo = max(0, min(lo, 64));
    hi = max(0, min(hi, 64));
    if (hi <= lo) return 0;
    const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1);
    const uint64_t below_lo = (1ull << lo) - 1;  // lo < 64 here
    return upto_hi & ~below_lo;
}

// ------------------------------------------------------------------ the plane scan -------------
// A chunk of kChunk tokens is scanned by one wave: kSub coalesced loads of 64 ids, one ballot each,
// give the marker bitmask of the chunk.  Sequences come from a window of up to 64 cu_seqlens entries
// (one coalesced load; more windows when more than 64 sequences touch the chunk), and a token finds
// its sequence by a 6-step shuffle search of the window.  The first marker of a sequence that began
// in an earlier chunk comes from the decoupled look-back below.
constexpr int kChunk = 512;
constexpr int kSub = kChunk / 64;
constexpr int kWalkSeqs = 8;  // a chunk touched by up to this many sequences of a window walks them

struct ChunkMasks {
    uint64_t m[kSub];  // bit i of m[k]: token c0 + 64k + i is a marker
};

// First marker (global index, kNone if none) among chunk positions [a, b), and whether there are two.
__device__ __forceinline__ void first_in(const ChunkMasks &cm, int64_t c0, int a, int b, int32_t &first, bool &multi)
{
    first = kNone;
    int cnt = 0;
#pragma unroll
    for (int k = kSub - 1; k >= 0; --k) {
        const uint64_t m = cm.m[k] & bit_range(a - 64 * k, b - 64 * k);
        if (m) first = (int32_t)(c0 + 64 * k + __builtin_ctzll(m));
        cnt += __builtin_popcountll(m);
    }
    multi = cnt >= 2;
}

// Issue the chunk's id loads (tokens outside [from, c_end) read as a non-marker) ...
// The 8 id loads of a chunk go out back to back: every lane loads (a clamped, valid address) and
// out-of-range lanes are masked afterwards.  Loads under a per-lane condition were compiled into 8
// round trips, each waited before the next was issued.  Needs from < c_end.
__device__ __forceinline__ void issue_ids(const Scan &sc, int64_t c0, int64_t c_end, int64_t from, int lane,
                                          int32_t (&v)[kSub])
{
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
        const int64_t g = c0 + 64 * k + lane;
        v[k] = sc.ids[min(max(g, from), c_end - 1)];
    }
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
        const int64_t g = c0 + 64 * k + lane;
        if (!(g < c_end && g >= from)) v[k] = ~sc.marker;
    }
}

// ... and ballot them into the chunk's marker mask.
__device__ __forceinline__ void ballot_ids(const Scan &sc, const int32_t (&v)[kSub], ChunkMasks &cm)
{
#pragma unroll
    for (int k = 0; k < kSub; ++k) cm.m[k] = __ballot(v[k] == sc.marker);
}

__device__ __forceinline__ void load_masks(const Scan &sc, int64_t c0, int64_t c_end, int64_t from, int lane, ChunkMasks &cm)
{
    int32_t v[kSub];
    issue_ids(sc, c0, c_end, from, lane, v);
    ballot_ids(sc, v, cm);
}

// Decoupled look-back (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", 2016) over chunk status words with a (first marker, more-than-one) operator.  The wave
// reads the words of the 64 preceding chunks at once and combines everything up to the nearest
// inclusive value -- a predecessor's published inclusive word, or the chunk where the sequence
// begins.  A predecessor that has not published yet is polled a bounded number of times and then
// evaluated on the spot from its ids, so no wait is unbounded and the result never depends on which
// workgroups the hardware has scheduled.  Returns the first marker (global index) of the sequence over
// [s0_begin, chunk*kChunk) and whether that range holds more than one marker.
constexpr int kPolls = 32;

__device__ void lookback(const Scan &sc, const uint64_t *status, int64_t chunk, uint32_t ep, int lane,
                         int64_t s0_begin, int32_t &first, bool &multi)
{
    first = kNone;
    multi = false;
    const int64_t stop = max<int64_t>(s0_begin, 0) / kChunk;  // the walk always ends at or above chunk 0
    int64_t base = chunk - 1;
    while (true) {
        const int64_t idx = base - lane;
        const bool valid = idx >= stop;
        uint64_t w = 0;
        bool ready = false;
        uint64_t end_mask = 0;
        int lim = 63;
        for (int poll = 0;; ++poll) {
            if (valid && !ready) {
                w = aload(status + idx);
                ready = (uint32_t)(w >> 34) == ep && ((w >> 32) & 3u) != 0;
            }
            end_mask = __ballot(valid && ((ready && ((w >> 32) & 3u) == kIncl) || idx == stop));
            lim = end_mask ? __builtin_ctzll(end_mask) : 63;
            const bool missing = __ballot(valid && lane <= lim && !ready) != 0;
            if (!missing || poll == kPolls) break;
            __builtin_amdgcn_s_sleep(8);
        }
        const bool use = valid && lane <= lim;
        int32_t v = (use && ready) ? (int32_t)(w & 0x7fffffffu) : kNone;
        bool m = use && ready && ((w >> 31) & 1u);
        uint64_t todo = __ballot(use && !ready);
        while (todo) {  // chunks still unpublished after the polls: read their ids
            const int bsel = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int64_t cb = (base - bsel) * kChunk;
            ChunkMasks cm;
            load_masks(sc, cb, min<int64_t>(cb + kChunk, sc.n_tokens), s0_begin, lane, cm);
            int32_t f;
            bool mm;
            first_in(cm, cb, 0, kChunk, f, mm);
            if (lane == bsel) {
                v = f;
                m = mm;
            }
        }
        const uint64_t has = __ballot(use && v != kNone);
        const bool mm = __ballot(use && m) != 0;
        const int cnt = __builtin_popcountll(has) + (first != kNone ? 1 : 0);
        multi = multi || mm || cnt >= 2;
        first = min(first, wave_min(v));
        if (end_mask) return;
        base -= 64;
    }
}

// Frame length of sequence s (s < n_seqs): its own entry when the call gives one that describes a
// frame (65 .. kMaxFrameLen), else the call's; bad = the entry was neither 0 nor in that range.
__device__ __forceinline__ int32_t seq_frame_len(const Scan &sc, int32_t s, bool &bad)
{
    const int32_t f = sc.frame_lens ? sc.frame_lens[s] : 0;
    bad = f != 0 && (f < 65 || f > kMaxFrameLen);
    return (f == 0 || bad) ? sc.frame_len : f;
}

__device__ __forceinline__ void write_scalars(const Scan &sc, int32_t s, int32_t origin, bool multi, int64_t len,
                                              int32_t fl, bool bad_fl)
{
    const bool img = origin >= 0;
    if (sc.start) sc.start[s] = img ? origin + fl : kTextStart;
    if (sc.amount) sc.amount[s] = img ? fl - kExtent : 0;
    if (sc.origin) sc.origin[s] = img ? origin : -1;
    if (sc.flags)
        sc.flags[s] = (multi ? 1 : 0) | ((img && (int64_t)origin + fl > len) ? 2 : 0) | (bad_fl ? 4 : 0);
}

// Scan of one chunk by one full wave.  Publishes the chunk's status word, looks back when the
// chunk's first sequence began earlier, writes the scalars of every sequence whose last token (for
// an empty sequence: the token before it) lies in the chunk, and hands each token's planes to
// sink(k, ok, t, h, w, seq) for token chunk*kChunk + 64k + lane, where seq describes the token's
// sequence (its begin, position offset and origin; see SeqInfo).  When several workgroups scan the same
// chunk, only the owner publishes and writes scalars: device-scope stores to one address from many
// workgroups are serialized (16 writers of one status word took 3-8 us to be acknowledged, against
// 0.6 us for one).
struct NoHook {
    __device__ void operator()() const {}
};

// The sequence a token belongs to, as the scan hands it to a sink: the sequence's first token
// (global index), the position of that token in the whole sequence (pos_offset), the sequence's
// canvas origin in positions (kNone when it has no marker so far) and its frame length.  Position
// of token g: off + (g - begin).
struct SeqInfo {
    int64_t begin;
    int32_t off;
    int32_t org;
    int32_t fl;
};
struct NoSingle {
    __device__ bool operator()(int64_t, int32_t, int32_t, int32_t) const { return false; }
};

// after_issue() runs once the chunk's id and sequence-start loads are in flight, before any wait.
// single(seq_begin, pos_offset, origin, frame_len) is offered a chunk that lies in one sequence; returning true
// takes the chunk's planes over in that form (every token of the chunk is handed over), and sink is
// then not called.
template <class Sink, class Hook = NoHook, class Single = NoSingle>
__device__ void scan_chunk(const Scan &sc, uint64_t *status, int64_t chunk, uint32_t ep, int lane, bool owner,
                           Sink sink, Hook after_issue = Hook(), Single single = Single())
{
    const int64_t c0 = chunk * kChunk;
    const int64_t c_end = min<int64_t>(c0 + kChunk, sc.n_tokens);
    const int32_t n = sc.n_seqs;

    // A window of 64 sequences: lane l holds sequence win + l -- its begin W and end Wn (INT64_MAX
    // past the last sequence), position offset, carried origin and frame-length entry, all loaded in
    // one round trip.
    int32_t win;
    int64_t W, Wn;
    int32_t w_off, w_oin, w_fl;
    auto load_window = [&](int32_t at) {
        const int32_t j = at + lane;
        const int32_t w0 = sc.cu[min(j, n)], w1 = sc.cu[min(j + 1, n)];
        const int32_t js = min(j, max(n - 1, 0));
        w_off = sc.pos_offset ? sc.pos_offset[js] : 0;
        w_oin = sc.origin_in ? sc.origin_in[js] : -1;
        w_fl = sc.frame_lens ? sc.frame_lens[js] : 0;
        W = j <= n ? (int64_t)w0 : INT64_MAX;
        Wn = j < n ? (int64_t)w1 : INT64_MAX;
    };

    // id loads and the sequence search go out together
    int32_t idv[kSub];
    issue_ids(sc, c0, c_end, c0, lane, idv);
    if (n < 64) {
        // every sequence fits one window: it is loaded with the ids, and the chunk's first and last
        // sequences are counted by ballot -- one round trip instead of a search, then a window
        win = 0;
        load_window(0);
        after_issue();
    } else {
        after_issue();
        // the window starts just below the chunk's first sequence (chunk 0: at sequence 0, so
        // leading empty sequences get their scalars)
        win = c0 == 0 ? 0 : max(wave_bracket_le(sc.cu, n, c0, lane) - 1, 0);
        load_window(win);
    }
    // Every entry below the window is <= c0, so a ballot over the window counts the sequences that
    // begin at or before c0 and c_end - 1 -- unless the window's last entry is still <= c_end - 1:
    // then more than 64 sequences touch the chunk and an exact search counts them.
    int32_t cnt_first = win + __builtin_popcountll(__ballot(W <= c0));
    int32_t cnt_last = win + __builtin_popcountll(__ballot(W <= c_end - 1));
    if (__shfl(W, 63) <= c_end - 1) wave_count_le2(sc.cu, n, c0, c_end - 1, lane, cnt_first, cnt_last);
    ChunkMasks cm;
    ballot_ids(sc, idv, cm);
    // Most chunks hold no marker at all (one per image sequence): they skip the bit searches, whose
    // 64-bit VALU arithmetic is a sizeable part of a wave's instructions.
    uint64_t any_marker = 0;
#pragma unroll
    for (int k = 0; k < kSub; ++k) any_marker |= cm.m[k];
    const bool has_marker = __builtin_amdgcn_readfirstlane((uint32_t)(any_marker != 0)) != 0;
    const int32_t s_first = cnt_first - 1, s_last = cnt_last - 1;
    const bool first_ok = s_first >= 0 && s_first < n;
    int64_t s0_begin = c0;
    if (first_ok) s0_begin = (s_first - win < 64) ? __shfl(W, s_first - win) : (int64_t)sc.cu[s_first];
    const bool need_carry = first_ok && s0_begin < c0;
    const bool last_ok = s_last >= 0 && s_last < n;
    int64_t sl_begin = c_end;
    if (last_ok) sl_begin = (s_last - win < 64) ? __shfl(W, s_last - win) : (int64_t)sc.cu[s_last];
    const bool last_open = need_carry && s_last == s_first;

    // the chunk's last sequence: its part in this chunk, published before the look-back
    int32_t f_last = kNone;
    bool m_last = false;
    if (has_marker) first_in(cm, c0, (int)(max(sl_begin, c0) - c0), (int)(c_end - c0), f_last, m_last);
    if (owner && lane == 0) astore(status + chunk, status_word(ep, last_open ? kAgg : kIncl, m_last, last_ok ? f_last : kNone));

    int32_t carry = kNone;
    bool carry_multi = false;
    if (need_carry) {
        lookback(sc, status, chunk, ep, lane, s0_begin, carry, carry_multi);
        if (owner && last_open && lane == 0) {
            const bool mm = carry_multi || m_last || (carry != kNone && f_last != kNone);
            astore(status + chunk, status_word(ep, kIncl, mm, min(carry, f_last)));
        }
    }

    while (true) {
        const int32_t j = win + lane;
        int32_t f = kNone;
        bool mm = false;
        if (has_marker) first_in(cm, c0, (int)(max(min(W, c_end), c0) - c0), (int)(max(min(Wn, c_end), c0) - c0), f, mm);
        if (need_carry && j == s_first) {
            mm = mm || carry_multi || (carry != kNone && f != kNone);
            f = min(f, carry);
        }
        // the sequence's origin in its own positions: carried from an earlier piece, else found here
        const int32_t poff = j < n ? w_off : 0;
        const int32_t oin = j < n ? w_oin : -1;
        const bool bad_fl = j < n && w_fl != 0 && (w_fl < 65 || w_fl > kMaxFrameLen);
        const int32_t fl = (j < n && w_fl != 0 && !bad_fl) ? w_fl : sc.frame_len;
        int32_t oseq = f == kNone ? kNone : poff + (int32_t)(f - W);
        if (oin >= 0) {
            mm = mm || f != kNone;
            oseq = oin;
        }
        if (j < n) {
            const int64_t fin = max<int64_t>(Wn - 1, 0);
            if (owner && fin >= c0 && fin < c_end) write_scalars(sc, j, oseq == kNone ? -1 : oseq, mm, poff + (Wn - W), fl, bad_fl);
        }
        const int64_t w_lo = __shfl(W, 0), w_hi = __shfl(Wn, 63);
        if (s_first == s_last && s_first >= win && s_first - win < 64) {
            // the whole chunk lies in one sequence: no per-token search
            const int r = s_first - win;
            const int32_t orr = __shfl(oseq, r), offr = __shfl(poff, r), flr = __shfl(fl, r);
            const int64_t sb = __shfl(W, r);
            if (!single(sb, offr, orr, flr)) {
#pragma unroll
                for (int k = 0; k < kSub; ++k) {
                    const int64_t g = c0 + 64 * k + lane;
                    const bool ok = g < c_end;
                    const int32_t p = offr + (int32_t)(g - sb);
                    int32_t t = 0, h = 0, w = 0;
                    if (ok) canvas_planes(p, (orr != kNone && orr <= p) ? orr : kNone, flr, t, h, w);
                    sink(k, ok, t, h, w, SeqInfo{sb, offr, orr, flr});
                }
            }
        } else {
            // The window lanes whose sequences touch the chunk: [r_lo, r_hi].  A token belongs to the
            // last of them that begins at or before it.  A few sequences are walked in a uniform loop
            // -- each one's begin, origin, offset and frame length read from its lane into scalars,
            // every token selecting it when it begins at or before the token -- which costs two
            // instructions per sequence and token block; a chunk of many short sequences searches
            // the window per token (six dependent shuffles).  Measured on 1,048,576 ragged tokens:
            // the chunks holding 2-5 sequences ended 2.4 us after the others with the search.
            const int r_lo = max(s_first - win, 0), r_hi = min(s_last - win, 63);
            if (r_lo <= r_hi && r_hi - r_lo < kWalkSeqs) {
                int64_t sbk[kSub];
                int32_t ork[kSub], ofk[kSub], flk[kSub];
                for (int r = r_lo; r <= r_hi; ++r) {
                    const int64_t wr = lane_value(W, r);
                    const int32_t o_r = __builtin_amdgcn_readlane(oseq, r), f_r = __builtin_amdgcn_readlane(poff, r);
                    const int32_t l_r = __builtin_amdgcn_readlane(fl, r);
#pragma unroll
                    for (int k = 0; k < kSub; ++k) {
                        if (r == r_lo || c0 + 64 * k + lane >= wr) {
                            sbk[k] = wr;
                            ork[k] = o_r;
                            ofk[k] = f_r;
                            flk[k] = l_r;
                        }
                    }
                }
                const int64_t t_lo = lane_value(W, r_lo), t_hi = lane_value(Wn, r_hi);
#pragma unroll
                for (int k = 0; k < kSub; ++k) {
                    const int64_t g = c0 + 64 * k + lane;
                    const bool ok = g < c_end && g >= t_lo && g < t_hi;
                    const int32_t p = ofk[k] + (int32_t)(g - sbk[k]);
                    int32_t t = 0, h = 0, w = 0;
                    if (ok) canvas_planes(p, (ork[k] != kNone && ork[k] <= p) ? ork[k] : kNone, flk[k], t, h, w);
                    sink(k, ok, t, h, w, SeqInfo{sbk[k], ofk[k], ork[k], flk[k]});
                }
            } else {
#pragma unroll
                for (int k = 0; k < kSub; ++k) {
                    const int64_t g = c0 + 64 * k + lane;
                    int r = 0;
#pragma unroll
                    for (int step = 32; step > 0; step >>= 1)
                        if (__shfl(Wn, r + step - 1) <= g) r += step;
                    const int32_t orr = __shfl(oseq, r), offr = __shfl(poff, r), flr = __shfl(fl, r);
                    const int64_t sb = __shfl(W, r);
                    const bool ok = g < c_end && g >= w_lo && g < w_hi;
                    const int32_t p = offr + (int32_t)(g - sb);
                    int32_t t = 0, h = 0, w = 0;
                    if (ok) canvas_planes(p, (orr != kNone && orr <= p) ? orr : kNone, flr, t, h, w);
                    sink(k, ok, t, h, w, SeqInfo{sb, offr, orr, flr});
                }
            }
        }
        // the next window's first begin is this window's last end (cu[win + 64])
        if (win + 64 >= n || __shfl(Wn, 63) > c_end) break;
        win += 64;
        load_window(win);
    }
}

// ------------------------------------------------------------------ element I/O ----------------
// Element types of Q/K (the C ABI's dtype codes).
constexpr int kIoF32 = 0, kIoBF16 = 1, kIoF16 = 2;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed pair of the 16-bit type, each rounded to nearest even.
template <int IO>
__device__ __forceinline__ uint32_t pack16x2(float a, float b)
{
    const f32x2_t f = {a, b};
    if constexpr (IO == kIoBF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

// A packed pair of the 16-bit type to fp32 (exact).
template <int IO>
__device__ __forceinline__ void unpack16x2(uint32_t u, float &lo, float &hi)
{
    if constexpr (IO == kIoBF16) {
        lo = __uint_as_float(u << 16);
        hi = __uint_as_float(u & 0xffff0000u);
    } else {
        const f32x2_t f = __builtin_convertvector(__builtin_bit_cast(f16x2_t, u), f32x2_t);
        lo = f[0];
        hi = f[1];
    }
}

// 8 consecutive elements as raw 16-byte words: one for the 16-bit types, two for fp32.
template <int IO>
struct Raw8 {
    uint4 w[IO == kIoF32 ? 2 : 1];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Q, K and V chunks are read once: loads carry the non-temporal hint.  Measured on the 64 x 4096
// workload: mrope_apply 119 -> 113 us, mrope_apply_ids 124 -> 117 us back to back, and no slower
// from cold caches; marking the stores as well made both slower.
__device__ __forceinline__ uint4 load16_nt(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int IO>
__device__ __forceinline__ Raw8<IO> load8(const void *base, int64_t elem)
{
    Raw8<IO> r;
    if constexpr (IO != kIoF32) {
        r.w[0] = load16_nt(static_cast<const uint16_t *>(base) + elem);
    } else {
        const float *p = static_cast<const float *>(base) + elem;
        r.w[0] = load16_nt(p);
        r.w[1] = load16_nt(p + 4);
    }
    return r;
}

template <int IO>
__device__ __forceinline__ void store8(void *base, int64_t elem, const Raw8<IO> &r)
{
    if constexpr (IO != kIoF32) {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + elem) = r.w[0];
    } else {
        uint4 *p = reinterpret_cast<uint4 *>(static_cast<float *>(base) + elem);
        p[0] = r.w[0];
        p[1] = r.w[1];
    }
}

// A store into another buffer than the one read (a cache row, an out-of-place head) is not read
// back by the launch: it carries the non-temporal hint.  Measured on 64 x 4096 bf16 tokens: the
// fused K/V cache write 335 -> 281 us, mrope_apply_kv 328 -> 272 us; a 4,096-sequence decode step
// 7.4 -> 6.7 us (out of place: see copy_rest_kernel).  In-place stores
// take the hint only when the launch writes more in place than the memory-side cache absorbs
// (the fixed-head kernels' NTS argument, chosen by the host).
template <int IO>
__device__ __forceinline__ void store8_nt(void *base, int64_t elem, const Raw8<IO> &r)
{
    u32x4_t *p;
    if constexpr (IO != kIoF32) p = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(base) + elem);
    else p = reinterpret_cast<u32x4_t *>(static_cast<float *>(base) + elem);
#pragma unroll
    for (int i = 0; i < (IO == kIoF32 ? 2 : 1); ++i)
        __builtin_nontemporal_store((u32x4_t){r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w}, p + i);
}

// Non-temporal or plain store, chosen at compile time: with a run-time choice the compiler merges
// the two stores of the branches into one plain store (the hint is lost).
template <int IO, bool NT>
__device__ __forceinline__ void store8_as(void *base, int64_t elem, const Raw8<IO> &r)
{
    if constexpr (NT) store8_nt<IO>(base, elem, r);
    else store8<IO>(base, elem, r);
}

template <int IO>
__device__ __forceinline__ void unpack8(const Raw8<IO> &r, float (&x)[8])
{
    if constexpr (IO != kIoF32) {
        const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack16x2<IO>(u[i], x[2 * i], x[2 * i + 1]);
    } else {
        const uint32_t u[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(u[i]);
    }
}

template <int IO>
__device__ __forceinline__ Raw8<IO> pack8(const float (&y)[8])
{
    Raw8<IO> r;
    if constexpr (IO != kIoF32) {
        r.w[0] = make_uint4(pack16x2<IO>(y[0], y[1]), pack16x2<IO>(y[2], y[3]), pack16x2<IO>(y[4], y[5]),
                            pack16x2<IO>(y[6], y[7]));
    } else {
        r.w[0] = make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3]));
        r.w[1] = make_uint4(__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7]));
    }
    return r;
}

// ------------------------------------------------------------------ rotary ---------------------
// Lane layout: eight lanes per token.  Lane l = 2m + half holds the 8 consecutive dims
// [32*half + 8m, 32*half + 8m + 8) of a head: frequencies j = 8m .. 8m+7, the x_j side (half 0) or
// the x_{j+32} side (half 1).  The eight lanes of a token cover one whole 128-byte line per head
// (bf16) with one load instruction, and rotate-half partners are neighbour lanes (l, l^1), which
// swap their data with one DPP move per dword.

// Value of the neighbour lane (l ^ 1) by DPP quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t swap_pair(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ double swap_pair(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = swap_pair((uint32_t)u), hi = swap_pair((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int IO>
__device__ __forceinline__ Raw8<IO> swap_pair(const Raw8<IO> &r)
{
    Raw8<IO> o;
#pragma unroll
    for (int k = 0; k < (IO == kIoF32 ? 2 : 1); ++k)
        o.w[k] = make_uint4(swap_pair(r.w[k].x), swap_pair(r.w[k].y), swap_pair(r.w[k].z), swap_pair(r.w[k].w));
    return o;
}

// The four inverse frequencies a lane evaluates (half 0: 8m..8m+3, half 1: 8m+4..8m+7) and the
// plane each reads, 2 bits apiece.  kSelect: taken from the kernel arguments by uniform selects, for
// kernels that read them once before a token loop -- a lane-dependent index into the argument block
// is a vector memory load, and inside the loop the wait for it would also wait for the prefetched
// Q/K loads.  Otherwise (decode: one token, no prefetch) that indexed load is the cheaper form: it
// travels with the data load and needs no registers for all 32 values.
struct LaneFreq {
    float f[4];
    uint32_t sel;
    int half;
};

template <bool kSelect>
__device__ __forceinline__ LaneFreq lane_freq(const Rotary &rot, int m, int half)
{
    LaneFreq r;
    const int q = 2 * m + half;  // j0 = 4q
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (kSelect) {
            float v = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                float x = rot.inv_freq[4 * t + i];
                asm volatile("" : "+s"(x));  // keep the selects: no indexed reload of the argument block
                v = q == t ? x : v;
            }
            r.f[i] = v;
        } else {
            r.f[i] = rot.inv_freq[4 * q + i];
        }
    }
    r.sel = (uint32_t)(rot.plane_sel >> (8 * q));
    r.half = half;
    return r;
}

// (cos, sign*sin) of frequencies 8m .. 8m+7 for lane pair m.  Each lane evaluates its four and the
// pair swaps results.  ss = -sin on the x_j side and +sin on the x_{j+32} side, so every output is
// y = own*c + partner*ss.
__device__ __forceinline__ void pair_sincos(const LaneFreq &lf, int32_t pt, int32_t ph, int32_t pw, double (&c)[8],
                                            double (&ss)[8])
{
    const int half = lf.half;
    double oc[4], os[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pl = (lf.sel >> (2 * i)) & 3u;
        const int32_t pos = pl == 1u ? ph : (pl == 2u ? pw : pt);
        const float a = (float)pos * lf.f[i];
        sincos_angle(a, &os[i], &oc[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double pc = swap_pair(oc[i]), ps = swap_pair(os[i]);
        c[i] = half ? pc : oc[i];
        c[4 + i] = half ? oc[i] : pc;
        const double s_lo = half ? ps : os[i], s_hi = half ? os[i] : ps;
        ss[i] = half ? s_lo : -s_lo;
        ss[4 + i] = half ? s_hi : -s_hi;
    }
}

// One head chunk: own holds this lane's 8 dims, the partner's come by DPP.
template <int IO>
__device__ __forceinline__ Raw8<IO> rotate_chunk(const Raw8<IO> &own, const double (&c)[8], const double (&ss)[8])
{
    float x[8], p[8], y[8];
    unpack8<IO>(own, x);
    unpack8<IO>(swap_pair<IO>(own), p);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)__builtin_fma((double)x[e], c[e], (double)p[e] * ss[e]);
    return pack8<IO>(y);
}

// Copy this lane's share of the 8-element chunks of one head from dim `from` on: src at soff, dst
// at doff (element offsets of the head's dim 0).  The generic kernels' cache writes.
template <int IO>
__device__ __forceinline__ void copy_span(const void *src, int64_t soff, void *dst, int64_t doff, int from,
                                          int head_dim, int l)
{
    // up to four chunks per round trip: every load of a batch goes out before its stores (a lane
    // past the head's end reads the head's last chunk and stores nothing)
    for (int d0 = from + 8 * l; d0 - 8 * l < head_dim; d0 += 256) {
        Raw8<IO> r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = load8<IO>(src, soff + min(d0 + 64 * i, head_dim - 8));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (d0 + 64 * i < head_dim) store8_nt<IO>(dst, doff + d0 + 64 * i, r[i]);
    }
}

__device__ __forceinline__ int64_t q_off(const Heads &hd, int64_t g, int h) { return g * hd.q_tok + h * hd.q_head; }
__device__ __forceinline__ int64_t k_off(const Heads &hd, int64_t g, int h) { return g * hd.k_tok + h * hd.k_head; }

// ------------------------------------------------------------------ paged K/V cache ------------
__device__ __forceinline__ bool slot_ok(const PagedKV &pc, int64_t slot) { return slot >= 0 && slot < pc.num_slots; }

// Element offset of head h of a cache slot (0 <= slot < num_slots), the same in both caches.
__device__ __forceinline__ int64_t cache_off(const PagedKV &pc, int64_t slot, int h)
{
    int64_t blk, row;
    if (pc.bs_shift >= 0) {
        blk = slot >> pc.bs_shift;
        row = slot & (int64_t)(pc.block_size - 1);
    } else {
        blk = slot / pc.block_size;
        row = slot - blk * pc.block_size;
    }
    return blk * pc.c_block + row * pc.c_tok + h * pc.c_head;
}

__device__ __forceinline__ int64_t v_off(const PagedKV &pc, int64_t g, int h) { return g * pc.v_tok + h * pc.v_head; }

// The chunks of a token's K and V heads that a cache write copies unchanged (head_dim 256): K dims
// 64..255 (three 64-dim row segments) and all of V (four), 8 elements per lane per segment.
template <int IO, int NK>
struct CopyChunks {
    Raw8<IO> k[NK][3];
    Raw8<IO> v[NK][4];
};

template <int IO, int NK>
__device__ __forceinline__ void load_copy_chunks(const Heads &hd, const PagedKV &pc, int64_t g, int l,
                                                 CopyChunks<IO, NK> &cc)
{
#pragma unroll
    for (int h = 0; h < NK; ++h)
#pragma unroll
        for (int i = 0; i < 3; ++i) cc.k[h][i] = load8<IO>(hd.k, k_off(hd, g, h) + 64 * (i + 1) + 8 * l);
    if (pc.v) {
#pragma unroll
        for (int h = 0; h < NK; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) cc.v[h][i] = load8<IO>(pc.v, v_off(pc, g, h) + 64 * i + 8 * l);
    }
}

template <int IO, int NK>
__device__ __forceinline__ void store_copy_chunks(const PagedKV &pc, int64_t slot, int l, const CopyChunks<IO, NK> &cc)
{
#pragma unroll
    for (int h = 0; h < NK; ++h) {
        const int64_t o = cache_off(pc, slot, h);
#pragma unroll
        for (int i = 0; i < 3; ++i) store8_nt<IO>(pc.k_cache, o + 64 * (i + 1) + 8 * l, cc.k[h][i]);
        if (pc.v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) store8_nt<IO>(pc.v_cache, o + 64 * i + 8 * l, cc.v[h][i]);
        }
    }
}

template <int IO, int NQ, int NK>
__device__ __forceinline__ void load_token_fixed(const Heads &hd, int64_t g, int e0, Raw8<IO> (&qv)[NQ],
                                                 Raw8<IO> (&kv)[NK])
{
#pragma unroll
    for (int h = 0; h < NQ; ++h) qv[h] = load8<IO>(hd.q, q_off(hd, g, h) + e0);
#pragma unroll
    for (int h = 0; h < NK; ++h) kv[h] = load8<IO>(hd.k, k_off(hd, g, h) + e0);
}

// Rotate one token's chunks and store them: Q in place (or into q_out); K in place (or into k_out),
// or with KV into the cache slot (nothing when the slot is outside the cache).  The other dims of
// out-of-place heads are copied by their own launch (copy_rest_kernel).  NTS: Q and K stores (in
// place or out of place) carry the non-temporal hint; cache rows always do.
template <int IO, int NQ, int NK, bool KV, bool NTS>
__device__ __forceinline__ void rotate_token_fixed(const Heads &hd, const PagedKV &pc, int64_t slot, int64_t g, int e0,
                                                   int l, const double (&c)[8], const double (&ss)[8],
                                                   const Raw8<IO> (&qv)[NQ], const Raw8<IO> (&kv)[NK])
{
    void *qo = hd.q_out ? hd.q_out : hd.q;
#pragma unroll
    for (int h = 0; h < NQ; ++h) store8_as<IO, NTS>(qo, q_off(hd, g, h) + e0, rotate_chunk<IO>(qv[h], c, ss));
    if constexpr (KV) {
        if (slot_ok(pc, slot)) {
#pragma unroll
            for (int h = 0; h < NK; ++h) store8_nt<IO>(pc.k_cache, cache_off(pc, slot, h) + e0, rotate_chunk<IO>(kv[h], c, ss));
        }
    } else {
        void *ko = hd.k_out ? hd.k_out : hd.k;
#pragma unroll
        for (int h = 0; h < NK; ++h) store8_as<IO, NTS>(ko, k_off(hd, g, h) + e0, rotate_chunk<IO>(kv[h], c, ss));
    }
}

// Any head counts and head_dim: one head at a time.  With a cache (pc.k_cache), K heads go whole
// into the slot and V heads are copied there; slot is the token's (ignored without a cache).  Out
// of place, only the rotated dims are written here (copy_rest_kernel copies the others).
template <int IO>
__device__ __forceinline__ void rotate_token_any(const Heads &hd, const PagedKV &pc, int64_t slot, int64_t g, int e0,
                                                 int l, const double (&c)[8], const double (&ss)[8])
{
    const bool to_cache = pc.k_cache != nullptr;
    const bool cache_ok = to_cache && slot_ok(pc, slot);
    for (int hh = 0; hh < hd.nq + hd.nk; ++hh) {
        const bool isq = hh < hd.nq;
        const int h = isq ? hh : hh - hd.nq;
        const void *src = isq ? hd.q : hd.k;
        const int64_t base = isq ? q_off(hd, g, h) : k_off(hd, g, h);
        if (!isq && to_cache) {
            if (!cache_ok) continue;
            const int64_t o = cache_off(pc, slot, h);
            store8_nt<IO>(pc.k_cache, o + e0, rotate_chunk<IO>(load8<IO>(src, base + e0), c, ss));
            copy_span<IO>(src, base, pc.k_cache, o, 64, hd.head_dim, l);
            continue;
        }
        void *dst = isq ? (hd.q_out ? hd.q_out : hd.q) : (hd.k_out ? hd.k_out : hd.k);
        store8<IO>(dst, base + e0, rotate_chunk<IO>(load8<IO>(src, base + e0), c, ss));
    }
    if (cache_ok && pc.v) {
        for (int h = 0; h < hd.nk; ++h) copy_span<IO>(pc.v, v_off(pc, g, h), pc.v_cache, cache_off(pc, slot, h), 0, hd.head_dim, l);
    }
}

// ------------------------------------------------------------------ kernels --------------------
constexpr int kBlock = 256;                 // 4 waves
constexpr int kLanesPerTok = 8;
constexpr int kTokPerBlock = kBlock / kLanesPerTok;

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Fixed head counts: a grid-stride loop over 8-token groups, one group per wave per step (the grid
// is sized to the chip by the host).  Each 8-lane group prefetches its next token's planes and head
// chunks before it rotates and stores the current one, so loads stay in flight while the sincos
// and rotation math runs.  Control flow is wave-uniform.
template <int IO, int NQ, int NK, bool NTS>
__global__ __launch_bounds__(kBlock) void apply_kernel(Heads hd, Rotary rot, const int32_t *__restrict__ planes,
                                                       int64_t ps)
{
    const int tid = threadIdx.x;
    const int l = tid & 7, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 8 * m;
    const LaneFreq lf = lane_freq<true>(rot, m, half);
    const int64_t stride = (int64_t)gridDim.x * kTokPerBlock;
    int64_t G = (int64_t)blockIdx.x * kTokPerBlock + (tid >> 6) * 8;  // first token of the wave's group
    const int sub = (tid & 63) >> 3;
    int64_t g = G + sub;
    bool ok = g < hd.n_tokens;
    int32_t pt = 0, ph = 0, pw = 0;
    Raw8<IO> qv[NQ], kv[NK];
    if (ok) {
        pt = planes[g];
        ph = planes[ps + g];
        pw = planes[2 * ps + g];
        load_token_fixed<IO, NQ, NK>(hd, g, e0, qv, kv);
    }
    // Let the first token's loads land here.  Otherwise the compiler's wait counting, merging the
    // loop entry with the back edge, takes them as possibly in flight inside the loop and makes
    // every store wait for the matching prefetch load of the next token.
    wait_vm_all();
    while (G < hd.n_tokens) {
        const int64_t Gn = G + stride;
        const int64_t gn = Gn + sub;
        const bool okn = gn < hd.n_tokens;
        int32_t nt = 0, nh = 0, nw = 0;
        Raw8<IO> qn[NQ], kn[NK];
        if (okn) {
            nt = planes[gn];
            nh = planes[ps + gn];
            nw = planes[2 * ps + gn];
            load_token_fixed<IO, NQ, NK>(hd, gn, e0, qn, kn);
        }
        if (ok) {
            double c[8], ss[8];
            pair_sincos(lf, pt, ph, pw, c, ss);
            rotate_token_fixed<IO, NQ, NK, false, NTS>(hd, PagedKV{}, -1, g, e0, l, c, ss, qv, kv);
        }
        G = Gn;
        g = gn;
        ok = okn;
        pt = nt;
        ph = nh;
        pw = nw;
#pragma unroll
        for (int h = 0; h < NQ; ++h) qv[h] = qn[h];
#pragma unroll
        for (int h = 0; h < NK; ++h) kv[h] = kn[h];
    }
}

// ------------------------------------------------------------------ fp32: sixteen lanes a token --
// An fp32 head's rotated dims are 256 bytes.  In the eight-lane layout each lane loads two 16-byte
// vectors per head, and the prefetching loop over ten heads then needs about 256 VGPRs: one wave
// per SIMD.  mrope_apply in fp32 (8 Q + 2 K heads, no cache) takes sixteen lanes a token instead:
// lane l = 2m + half holds dims [32 half + 4m, 32 half + 4m + 4) -- frequencies 4m .. 4m+3, the x_j
// side (half 0) or the x_{j+32} side (half 1) -- one 16-byte vector per head, the 16-bit types'
// register budget.  Each lane evaluates two of its pair's four sincos and the pair swaps them by
// DPP, as in the eight-lane layout; every output is the same double expression, rounded once.
constexpr int kLanesW = 16;
constexpr int kTokPerBlockW = kBlock / kLanesW;

struct LaneFreq2 {
    float f[2];
    uint32_t sel;
    int half;
};

// The two inverse frequencies a lane evaluates (2q, 2q + 1 with q = 2m + half) and their planes,
// taken from the kernel arguments by uniform selects (see lane_freq).
__device__ __forceinline__ LaneFreq2 lane_freq2(const Rotary &rot, int m, int half)
{
    LaneFreq2 r;
    const int q = 2 * m + half;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float x = rot.inv_freq[2 * t + i];
            asm volatile("" : "+s"(x));
            v = q == t ? x : v;
        }
        r.f[i] = v;
    }
    r.sel = (uint32_t)(rot.plane_sel >> (4 * q));
    r.half = half;
    return r;
}

// (cos, sign*sin) of frequencies 4m .. 4m+3 for lane pair m, as pair_sincos.
__device__ __forceinline__ void pair_sincos4(const LaneFreq2 &lf, int32_t pt, int32_t ph, int32_t pw,
                                             double (&c)[4], double (&ss)[4])
{
    const int half = lf.half;
    double oc[2], os[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t pl = (lf.sel >> (2 * i)) & 3u;
        const int32_t pos = pl == 1u ? ph : (pl == 2u ? pw : pt);
        const float a = (float)pos * lf.f[i];
        sincos_angle(a, &os[i], &oc[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double pc = swap_pair(oc[i]), ps = swap_pair(os[i]);
        c[i] = half ? pc : oc[i];
        c[2 + i] = half ? oc[i] : pc;
        const double s_lo = half ? ps : os[i], s_hi = half ? os[i] : ps;
        ss[i] = half ? s_lo : -s_lo;
        ss[2 + i] = half ? s_hi : -s_hi;
    }
}

// Four fp32 dims of one head: own from this lane, the partner's by DPP.
__device__ __forceinline__ uint4 rotate4(const uint4 &own, const double (&c)[4], const double (&ss)[4])
{
    const float x[4] = {__uint_as_float(own.x), __uint_as_float(own.y), __uint_as_float(own.z), __uint_as_float(own.w)};
    const float p[4] = {__uint_as_float(swap_pair(own.x)), __uint_as_float(swap_pair(own.y)),
                        __uint_as_float(swap_pair(own.z)), __uint_as_float(swap_pair(own.w))};
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (float)__builtin_fma((double)x[e], c[e], (double)p[e] * ss[e]);
    return make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3]));
}

template <int NQ, int NK>
__device__ __forceinline__ void load_token_w(const Heads &hd, int64_t g, int e0, uint4 (&qv)[NQ], uint4 (&kv)[NK])
{
#pragma unroll
    for (int h = 0; h < NQ; ++h) qv[h] = load16_nt(static_cast<const float *>(hd.q) + q_off(hd, g, h) + e0);
#pragma unroll
    for (int h = 0; h < NK; ++h) kv[h] = load16_nt(static_cast<const float *>(hd.k) + k_off(hd, g, h) + e0);
}

template <bool NT>
__device__ __forceinline__ void store16_as(void *base, int64_t elem, const uint4 &v)
{
    float *p = static_cast<float *>(base) + elem;
    if constexpr (NT) __builtin_nontemporal_store((u32x4_t){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(p));
    else *reinterpret_cast<uint4 *>(p) = v;
}

// apply_kernel's loop for fp32 with sixteen lanes a token: 4-token groups, one per wave per step,
// each 16-lane group prefetching its next token before rotating the current one.
template <int NQ, int NK, bool NTS>
__global__ __launch_bounds__(kBlock) void apply_f32w_kernel(Heads hd, Rotary rot, const int32_t *__restrict__ planes,
                                                            int64_t ps)
{
    const int tid = threadIdx.x;
    const int l = tid & 15, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 4 * m;
    const LaneFreq2 lf = lane_freq2(rot, m, half);
    const int64_t stride = (int64_t)gridDim.x * kTokPerBlockW;
    int64_t G = (int64_t)blockIdx.x * kTokPerBlockW + (tid >> 6) * 4;  // first token of the wave's group
    const int sub = (tid & 63) >> 4;
    int64_t g = G + sub;
    bool ok = g < hd.n_tokens;
    int32_t pt = 0, ph = 0, pw = 0;
    uint4 qv[NQ], kv[NK];
    if (ok) {
        pt = planes[g];
        ph = planes[ps + g];
        pw = planes[2 * ps + g];
        load_token_w<NQ, NK>(hd, g, e0, qv, kv);
    }
    wait_vm_all();  // as in apply_kernel
    void *qo = hd.q_out ? hd.q_out : hd.q;
    void *ko = hd.k_out ? hd.k_out : hd.k;
    while (G < hd.n_tokens) {
        const int64_t Gn = G + stride;
        const int64_t gn = Gn + sub;
        const bool okn = gn < hd.n_tokens;
        int32_t nt = 0, nh = 0, nw = 0;
        uint4 qn[NQ], kn[NK];
        if (okn) {
            nt = planes[gn];
            nh = planes[ps + gn];
            nw = planes[2 * ps + gn];
            load_token_w<NQ, NK>(hd, gn, e0, qn, kn);
        }
        if (ok) {
            double c[4], ss[4];
            pair_sincos4(lf, pt, ph, pw, c, ss);
#pragma unroll
            for (int h = 0; h < NQ; ++h) store16_as<NTS>(qo, q_off(hd, g, h) + e0, rotate4(qv[h], c, ss));
#pragma unroll
            for (int h = 0; h < NK; ++h) store16_as<NTS>(ko, k_off(hd, g, h) + e0, rotate4(kv[h], c, ss));
        }
        G = Gn;
        g = gn;
        ok = okn;
        pt = nt;
        ph = nh;
        pw = nw;
#pragma unroll
        for (int h = 0; h < NQ; ++h) qv[h] = qn[h];
#pragma unroll
        for (int h = 0; h < NK; ++h) kv[h] = kn[h];
    }
}

// One token of the cache-writing path (fixed head counts, head_dim 256): every load of the token --
// its Q and K rotation chunks, K pass-through and V chunks -- goes out at once, then the math, then
// the stores (Q in place, K and V into the cache slot, nothing for a slot outside the cache).  No
// prefetch of the next token: 24 chunks a lane already keep enough bytes in flight per wave, and
// the registers of a second set would halve the waves per SIMD.
template <int IO, int NQ, int NK, bool NTS>
__device__ __forceinline__ void kv_token(const Heads &hd, const PagedKV &pc, const LaneFreq &lf, int64_t g, int e0,
                                         int l, int32_t pt, int32_t ph, int32_t pw, int64_t slot)
{
    Raw8<IO> qv[NQ], kv[NK];
    CopyChunks<IO, NK> cc;
    load_token_fixed<IO, NQ, NK>(hd, g, e0, qv, kv);
    load_copy_chunks<IO, NK>(hd, pc, g, l, cc);
    double c[8], ss[8];
    pair_sincos(lf, pt, ph, pw, c, ss);
    rotate_token_fixed<IO, NQ, NK, true, NTS>(hd, pc, slot, g, e0, l, c, ss, qv, kv);
    if (slot_ok(pc, slot)) store_copy_chunks<IO, NK>(pc, slot, l, cc);
}

// mrope_apply_kv, fixed head counts: a grid-stride loop over 8-token groups like apply_kernel.
template <int IO, int NQ, int NK, bool NTS>
__global__ __launch_bounds__(kBlock) void apply_kv_kernel(Heads hd, Rotary rot, const int32_t *__restrict__ planes,
                                                          int64_t ps, PagedKV pc)
{
    const int tid = threadIdx.x;
    const int l = tid & 7, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 8 * m;
    const LaneFreq lf = lane_freq<true>(rot, m, half);
    const int64_t stride = (int64_t)gridDim.x * kTokPerBlock;
    const int sub = (tid & 63) >> 3;
    for (int64_t G = (int64_t)blockIdx.x * kTokPerBlock + (tid >> 6) * 8; G < hd.n_tokens; G += stride) {
        const int64_t g = G + sub;
        if (g < hd.n_tokens)
            kv_token<IO, NQ, NK, NTS>(hd, pc, lf, g, e0, l, planes[g], planes[ps + g], planes[2 * ps + g], pc.slots[g]);
    }
}

// fp32 cache writes with sixteen lanes a token (fixed head counts, head_dim 256): lane l = 2m + half
// holds dims [32 half + 4m, 32 half + 4m + 4) of every rotated head, as in apply_f32w_kernel; a K
// head's pass-through dims (64..255, 48 16-byte vectors) and a V head (64 vectors) go as every
// sixteenth vector, so each instruction of a token's sixteen lanes covers 256 contiguous bytes.  Per
// lane: 8 Q + 2 K rotation vectors, 6 K pass-through and 8 V -- the 24 16-byte loads a lane of the
// 16-bit kernel issues (kv_token) -- all in flight before the math.
template <int NK>
struct CopyChunksW {
    uint4 k[NK][3];
    uint4 v[NK][4];
};

template <int NQ, int NK, bool NTS>
__device__ __forceinline__ void kv_token_w(const Heads &hd, const PagedKV &pc, const LaneFreq2 &lf, int64_t g, int e0,
                                           int l, int32_t pt, int32_t ph, int32_t pw, int64_t slot)
{
    uint4 qv[NQ], kv[NK];
    CopyChunksW<NK> cc;
    load_token_w<NQ, NK>(hd, g, e0, qv, kv);
    const float *kp = static_cast<const float *>(hd.k);
#pragma unroll
    for (int h = 0; h < NK; ++h)
#pragma unroll
        for (int i = 0; i < 3; ++i) cc.k[h][i] = load16_nt(kp + k_off(hd, g, h) + 64 + 4 * (l + 16 * i));
    if (pc.v) {
        const float *vp = static_cast<const float *>(pc.v);
#pragma unroll
        for (int h = 0; h < NK; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) cc.v[h][i] = load16_nt(vp + v_off(pc, g, h) + 4 * (l + 16 * i));
    }
    double c[4], ss[4];
    pair_sincos4(lf, pt, ph, pw, c, ss);
    void *qo = hd.q_out ? hd.q_out : hd.q;
#pragma unroll
    for (int h = 0; h < NQ; ++h) store16_as<NTS>(qo, q_off(hd, g, h) + e0, rotate4(qv[h], c, ss));
    if (!slot_ok(pc, slot)) return;
#pragma unroll
    for (int h = 0; h < NK; ++h) {
        const int64_t o = cache_off(pc, slot, h);
        store16_as<true>(pc.k_cache, o + e0, rotate4(kv[h], c, ss));
#pragma unroll
        for (int i = 0; i < 3; ++i) store16_as<true>(pc.k_cache, o + 64 + 4 * (l + 16 * i), cc.k[h][i]);
        if (pc.v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) store16_as<true>(pc.v_cache, o + 4 * (l + 16 * i), cc.v[h][i]);
        }
    }
}

// mrope_apply_kv in fp32, fixed head counts: a grid-stride loop over 4-token groups (16 tokens a
// workgroup step) like apply_kv_kernel.
template <int NQ, int NK, bool NTS>
__global__ __launch_bounds__(kBlock) void apply_kv_f32w_kernel(Heads hd, Rotary rot, const int32_t *__restrict__ planes,
                                                               int64_t ps, PagedKV pc)
{
    const int tid = threadIdx.x;
    const int l = tid & 15, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 4 * m;
    const LaneFreq2 lf = lane_freq2(rot, m, half);
    const int64_t stride = (int64_t)gridDim.x * kTokPerBlockW;
    const int sub = (tid & 63) >> 4;
    for (int64_t G = (int64_t)blockIdx.x * kTokPerBlockW + (tid >> 6) * 4; G < hd.n_tokens; G += stride) {
        const int64_t g = G + sub;
        if (g < hd.n_tokens)
            kv_token_w<NQ, NK, NTS>(hd, pc, lf, g, e0, l, planes[g], planes[ps + g], planes[2 * ps + g], pc.slots[g]);
    }
}

// Any head counts and head_dim: one token per 8-lane group, one head at a time.
template <int IO>
__global__ __launch_bounds__(kBlock) void apply_any_kernel(Heads hd, Rotary rot, const int32_t *__restrict__ planes,
                                                           int64_t ps, PagedKV pc)
{
    const int tid = threadIdx.x;
    const int l = tid & 7, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 8 * m;
    const int64_t g = (int64_t)blockIdx.x * kTokPerBlock + (tid >> 3);
    if (g >= hd.n_tokens) return;
    const int64_t slot = pc.k_cache ? pc.slots[g] : -1;
    double c[8], ss[8];
    pair_sincos(lane_freq<false>(rot, m, half), planes[g], planes[ps + g], planes[2 * ps + g], c, ss);
    rotate_token_any<IO>(hd, pc, slot, g, e0, l, c, ss);
}

// Out of place: the dims a rotation leaves unchanged (64..head_dim of every head) are copied by a
// launch of their own, shaped for a streaming copy.  Eight lanes take a head row, each every eighth
// 16-byte chunk, so an instruction of eight lanes covers 128 contiguous bytes; a 256-dim row is one
// batch of 3 chunks per lane (bf16, fp16; two batches for fp32).  Loads are unconditional (clamped
// to the last row and chunk) and go out before any store; the grid covers the rows in one pass, so
// the dispatcher balances the CUs.  Inside one token step of the rotation kernels this copy was a
// load-to-store round trip per head: 64 x 4096 bf16 tokens out of place took 542 us (4.96 TB/s),
// now 465 us (5.78 TB/s).  Two or four rows per lane took 474 and 508 us; persistent grids of 8 or
// 32 workgroups per CU, 486 and 498 us.
constexpr int kRestRows = 1;  // rows per lane and step
constexpr int kRestBatch = 3; // chunks per lane and row per batch

__global__ __launch_bounds__(kBlock) void copy_rest_kernel(const char *__restrict__ src, char *__restrict__ dst,
                                                           int64_t tok_bytes, int64_t head_bytes, int nh, int nh_shift,
                                                           int64_t n_rows, int64_t row_from, int n_chunks)
{
    const int l8 = threadIdx.x & 7;
    constexpr int kRowsPerStep = kBlock / 8 * kRestRows;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerStep;
    auto row_base = [&](int64_t row) {  // byte offset of the row's first copied chunk
        int64_t t, h;
        if (nh_shift >= 0) {
            t = row >> nh_shift;
            h = row & ((1 << nh_shift) - 1);
        } else {
            t = row / nh;
            h = row - t * nh;
        }
        return t * tok_bytes + h * head_bytes + row_from;
    };
    for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerStep + (threadIdx.x >> 3); r0 < n_rows; r0 += stride) {
        int64_t base[kRestRows];
        bool row_ok[kRestRows];
#pragma unroll
        for (int j = 0; j < kRestRows; ++j) {
            const int64_t row = r0 + (int64_t)j * (kBlock / 8);
            row_ok[j] = row < n_rows;
            base[j] = row_base(row_ok[j] ? row : n_rows - 1);
        }
        for (int c0 = l8; c0 - l8 < n_chunks; c0 += 8 * kRestBatch) {
            u32x4_t v[kRestRows][kRestBatch];
#pragma unroll
            for (int j = 0; j < kRestRows; ++j)
#pragma unroll
                for (int b = 0; b < kRestBatch; ++b)
                    v[j][b] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t *>(src + base[j] + 16 * (int64_t)min(c0 + 8 * b, n_chunks - 1)));
#pragma unroll
            for (int j = 0; j < kRestRows; ++j)
#pragma unroll
                for (int b = 0; b < kRestBatch; ++b)
                    if (row_ok[j] && c0 + 8 * b < n_chunks)
                        __builtin_nontemporal_store(v[j][b], reinterpret_cast<u32x4_t *>(dst + base[j] + 16 * (int64_t)(c0 + 8 * b)));
        }
    }
}

// One wave per chunk, four chunks per workgroup.
__global__ __launch_bounds__(kBlock) void planes_kernel(Scan sc, int64_t n_chunks)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    if (chunk >= n_chunks) return;
    const int64_t c0 = chunk * kChunk;
    scan_chunk(sc, status_array(sc.workspace), chunk, launch_epoch(sc), lane, true,
               [&](int k, bool ok, int32_t t, int32_t h, int32_t w, const SeqInfo &) {
                   if (!ok) return;
                   const int64_t g = c0 + 64 * k + lane;
                   sc.planes[g] = t;
                   sc.planes[sc.plane_stride + g] = h;
                   sc.planes[2 * sc.plane_stride + g] = w;
               });
}

// Fused: one part of a 512-token chunk per workgroup (2^part_log parts, part_log >= 1: halves for
// large inputs, down to 32-token parts for small ones; each workgroup repeats the chunk's scan, so
// more workgroups share the work and each has fewer sequential steps).  Wave 0 scans the chunk into
// LDS while waves 1-3 issue the Q/K loads of their first token (wave 0 issues its own after the
// scan), then the workgroup rotates its part 32 tokens at a time, each 8-lane group prefetching its
// next token before rotating the current one.  KV as in apply_kernel (fixed head
// counts); the generic path writes the cache when pc.k_cache is set.  W16: fp32 with sixteen lanes
// a token (apply_f32w_kernel's layout), 16 tokens a step.
template <bool W16>
__device__ __forceinline__ auto fused_lane_freq(const Rotary &rot, int m, int half)
{
    if constexpr (W16) return lane_freq2(rot, m, half);
    else return lane_freq<true>(rot, m, half);
}

template <int IO, int NQ, int NK, bool KV, bool NTS, bool W16 = false>
__global__ __launch_bounds__(kBlock) void apply_ids_kernel(Heads hd, Rotary rot, Scan sc, PagedKV pc, int part_log)
{
    static_assert(!W16 || (IO == kIoF32 && NQ > 0 && NK > 0), "sixteen lanes: fp32, fixed heads");
    constexpr int kLanes = W16 ? kLanesW : kLanesPerTok;
    constexpr int kStep = kBlock / kLanes;  // tokens a workgroup step
    __shared__ int32_t s_pl[3][kChunk];
    __shared__ uint64_t s_ok[kSub];
    __shared__ int64_t s_seq[3];  // a chunk inside one sequence: [1] = its begin; [0] = its offset | origin << 32;
                                  // [2] = its frame length
    __shared__ int32_t s_single;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l = tid & (kLanes - 1), m = l >> 1, half = l & 1;
    const int e0 = 32 * half + (W16 ? 4 : 8) * m;
    const auto lf = fused_lane_freq<W16>(rot, m, half);
    const int64_t chunk = (int64_t)(blockIdx.x >> part_log);
    const int64_t c0 = chunk * kChunk;
    const int64_t c_end = min<int64_t>(c0 + kChunk, hd.n_tokens);
    const int plen = kChunk >> part_log;
    const int64_t r0 = c0 + (int64_t)(blockIdx.x & ((1u << part_log) - 1)) * plen;  // this part: [r0, r_end)
    if (r0 >= c_end) return;  // a part past the last token (the chunk's other parts scan it)
    const int64_t r_end = min<int64_t>(r0 + plen, c_end);
    constexpr bool kFixed = NQ > 0 && NK > 0;
    constexpr int AQ = kFixed ? NQ : 1, AK = kFixed ? NK : 1;

    // Wave 0 puts the scan's loads in flight first; only then (first barrier, without a fence: no
    // wait) do the waves issue their first token's Q/K loads.  Issued the other way round, the scan's
    // first round trip queued behind all Q/K loads of the chip (7 of the scan's 11.5 us).  Wave 0
    // issues its own first token only after the scan: the scan's later waits would otherwise
    // include those loads (1 x 4096 tokens 17.8 -> 17.2 us, 4 x 4096 28.4 -> 25.7).  Issued early,
    // 8 x 32768 tokens took 122 us instead of 118: with long sequences a chunk's look-back waits on
    // its predecessors' look-backs, and each waited behind its wave 0's loads.
    int64_t g = r0 + tid / kLanes;
    using TokReg = std::conditional_t<W16, uint4, Raw8<IO>>;
    TokReg qv[AQ], kv[AK];
    auto prologue = [&]() {
        if constexpr (W16 && !KV) {
            if (g < r_end) load_token_w<AQ, AK>(hd, g, e0, qv, kv);
        } else if constexpr (kFixed && !KV) {
            if (g < r_end) load_token_fixed<IO, AQ, AK>(hd, g, e0, qv, kv);
        }
    };
    if (tid >= 64) {
        __builtin_amdgcn_s_barrier();
        prologue();
    } else {
        if (lane < kSub) s_ok[lane] = 0;
        if (lane == 0) s_single = 0;
        // A token is handed over once, in the sequence window that holds it.  A chunk inside one
        // sequence (without planes_out) is handed over as that sequence's begin, offset and origin:
        // every wave then derives its own tokens' planes, instead of wave 0 writing all 512 to LDS
        // (measured: that handover was ~4 us of the launch on 64 x 4096 tokens).
        scan_chunk(sc, status_array(sc.workspace), chunk, launch_epoch(sc), lane, r0 == c0,
                   [&](int k, bool ok, int32_t t, int32_t h, int32_t w, const SeqInfo &) {
                       const int p = 64 * k + lane;
                       const uint64_t okm = __ballot(ok);
                       if (lane == 0) s_ok[k] |= okm;
                       if (!ok) return;
                       s_pl[0][p] = t;
                       s_pl[1][p] = h;
                       s_pl[2][p] = w;
                       if (sc.planes && c0 + p >= r0 && c0 + p < r_end) {
                           const int64_t gg = c0 + p;
                           sc.planes[gg] = t;
                           sc.planes[sc.plane_stride + gg] = h;
                           sc.planes[2 * sc.plane_stride + gg] = w;
                       }
                   },
                   [&]() { __builtin_amdgcn_s_barrier(); },
                   [&](int64_t sb, int32_t off, int32_t org, int32_t fl) {
                       if (sc.planes) return false;
                       if (lane == 0) {
                           s_seq[1] = sb;
                           s_seq[0] = (int64_t)(uint32_t)off | ((int64_t)org << 32);
                           s_seq[2] = fl;
                           s_single = 1;
                       }
                       return true;
                   });
        prologue();
    }
    __syncthreads();
    wait_vm_all();  // the first token's loads: see apply_kernel

    // Wave-uniform: the chunk's planes come from its sequence (single) or from LDS per token.  A
    // single chunk wholly before the image (or in a text-only sequence) or wholly after the frame has
    // t = h = w = p - shift for a uniform shift: one add per token.
    const bool single = __builtin_amdgcn_readfirstlane(s_single) != 0;
    const int64_t seq_begin = single ? s_seq[1] : 0;
    const int64_t seq_word = single ? s_seq[0] : 0;
    const int32_t seq_off = (int32_t)(uint32_t)seq_word, seq_org = (int32_t)(seq_word >> 32);
    const int32_t seq_fl = single ? (int32_t)s_seq[2] : sc.frame_len;
    const int64_t p_c0 = single ? seq_off + (c0 - seq_begin) : 0;  // position of the chunk's first token
    const int64_t p_last = p_c0 + (c_end - 1 - c0);
    const bool before = seq_org == kNone || p_last < seq_org;
    const bool after = !before && p_c0 - seq_org >= seq_fl;
    const bool flat = single && (before || after);
    const int32_t flat_c0 = (int32_t)(p_c0 - (after ? seq_fl - kExtent : 0));
    auto planes_of = [&](int64_t gt, bool &ok, int32_t &t, int32_t &h, int32_t &w) {
        if (flat) {
            ok = true;
            t = h = w = flat_c0 + (int32_t)(gt - c0);
        } else if (single) {
            const int32_t pp = seq_off + (int32_t)(gt - seq_begin);
            ok = true;
            canvas_planes(pp, (seq_org != kNone && seq_org <= pp) ? seq_org : kNone, seq_fl, t, h, w);
        } else {
            const int p = (int)(gt - c0);
            ok = (s_ok[p >> 6] >> (p & 63)) & 1u;
            t = s_pl[0][p];
            h = s_pl[1][p];
            w = s_pl[2][p];
        }
    };

    while (g < r_end) {  // the lanes of a token stay together
        bool ok;
        int32_t pt, ph, pw;
        planes_of(g, ok, pt, ph, pw);
        const int64_t gn = g + kStep;
        double c[8], ss[8];
        if constexpr (W16 && KV) {
            if (ok) kv_token_w<AQ, AK, NTS>(hd, pc, lf, g, e0, l, pt, ph, pw, pc.slots[g]);
        } else if constexpr (W16) {
            uint4 qn[AQ], kn[AK];
            if (gn < r_end) load_token_w<AQ, AK>(hd, gn, e0, qn, kn);
            if (ok) {
                double c4[4], ss4[4];
                pair_sincos4(lf, pt, ph, pw, c4, ss4);
                void *qo = hd.q_out ? hd.q_out : hd.q;
                void *ko = hd.k_out ? hd.k_out : hd.k;
#pragma unroll
                for (int h = 0; h < AQ; ++h) store16_as<NTS>(qo, q_off(hd, g, h) + e0, rotate4(qv[h], c4, ss4));
#pragma unroll
                for (int h = 0; h < AK; ++h) store16_as<NTS>(ko, k_off(hd, g, h) + e0, rotate4(kv[h], c4, ss4));
            }
#pragma unroll
            for (int h = 0; h < AQ; ++h) qv[h] = qn[h];
#pragma unroll
            for (int h = 0; h < AK; ++h) kv[h] = kn[h];
        } else if constexpr (kFixed && KV) {
            if (ok) kv_token<IO, AQ, AK, NTS>(hd, pc, lf, g, e0, l, pt, ph, pw, pc.slots[g]);
        } else if constexpr (kFixed) {
            Raw8<IO> qn[AQ], kn[AK];
            if (gn < r_end) load_token_fixed<IO, AQ, AK>(hd, gn, e0, qn, kn);
            if (ok) {
                pair_sincos(lf, pt, ph, pw, c, ss);
                rotate_token_fixed<IO, AQ, AK, false, NTS>(hd, pc, -1, g, e0, l, c, ss, qv, kv);
            }
#pragma unroll
            for (int h = 0; h < AQ; ++h) qv[h] = qn[h];
#pragma unroll
            for (int h = 0; h < AK; ++h) kv[h] = kn[h];
        } else {
            if (ok) {
                pair_sincos(lf, pt, ph, pw, c, ss);
                rotate_token_any<IO>(hd, pc, pc.k_cache ? pc.slots[g] : -1, g, e0, l, c, ss);
            }
        }
        g = gn;
    }
}

// ------------------------------------------------------------------ scan-first fused kernel ----
// mrope_apply_ids for large inputs with the model's heads (8 Q, 2 K).  The grid holds two kinds of
// workgroups, dispatched in index order:
//   scan workgroups [0, S): one wave per 512-token chunk runs the chunk scan (ballots, look-back,
//     scalars, planes_out) and hands the planes of each 32-token part of the chunk over through the
//     workspace -- a part inside one sequence as two words (the position base, p = g + base, and the
//     sequence's canvas origin; a third, its frame length, when the call gives frame lengths per
//     sequence), any other part as its tokens' planes, three words a token -- every word tagged with
//     the launch's epoch;
//   rotation workgroups [S, S + R): one 32-token part each, shaped like mrope_apply's one-step
//     workgroups: every lane issues its token's Q/K loads, then reads the part's handover words,
//     derives its token's planes, rotates and stores.
// The scans of all chunks run first, on an otherwise idle memory system, so the rotation sees no
// scan latency beyond the first chunks'; the rotation workgroups then run on the dispatcher-balanced
// one-step grid that serves mrope_apply at this size.  A wave whose handover words are not tagged
// with this launch after a bounded number of polls scans its chunk itself (as the chunk-per-workgroup
// kernel does), so no wait depends on which workgroups the hardware has scheduled.
constexpr uint64_t kPartSingle = 1, kPartMulti = 2;
constexpr int kScanWaves = kBlock / 64;  // chunks per scan workgroup

__device__ __forceinline__ uint64_t tag_word(uint32_t ep, uint64_t kind, uint32_t v)
{
    return ((uint64_t)ep << 34) | (kind << 32) | (uint64_t)v;
}
__device__ __forceinline__ bool tagged_with(uint64_t w, uint32_t ep) { return (uint32_t)(w >> 34) == ep; }

// One wave's chunk scan with the part handover.
__device__ void sf_scan_chunk(const Scan &sc, int64_t chunk, uint32_t ep, int lane)
{
    const int64_t c0 = chunk * kChunk;
    const int64_t c_end = min<int64_t>(c0 + kChunk, sc.n_tokens);
    scan_chunk(
        sc, status_array(sc.workspace), chunk, ep, lane, true,
        [&](int k, bool ok, int32_t t, int32_t h, int32_t w, const SeqInfo &si) {
            const int64_t g = c0 + 64 * k + lane;
            if (ok && sc.planes) {
                sc.planes[g] = t;
                sc.planes[sc.plane_stride + g] = h;
                sc.planes[2 * sc.plane_stride + g] = w;
            }
            // the two 32-token parts of this 64-token block: lanes [0, 32) and [32, 64).  A part is
            // handed over as one sequence when every token of it (before the end) is delivered in
            // this call with the same sequence; otherwise its delivered tokens' planes go over one by
            // one (a part whose tokens come in several calls is written so by each).
            const int leader = lane & 32;
            const int64_t lb = __shfl(si.begin, leader);
            const int32_t lo = __shfl(si.off, leader), lg = __shfl(si.org, leader), lf = __shfl(si.fl, leader);
            const bool valid = g < c_end;
            const bool same = !valid || (ok && si.begin == lb && si.off == lo && si.org == lg);
            const uint64_t half = leader ? 0xffffffff00000000ull : 0x00000000ffffffffull;
            const bool single = (__ballot(same) & half) == half;
            if ((__ballot(ok) & half) == 0) return;
            const int64_t part = (c0 + 64 * k + leader) / kPartTokens;
            if (single) {
                if (lane == leader) {
                    astore(sc.parts + 3 * part, tag_word(ep, kPartSingle, (uint32_t)(int32_t)((int64_t)lo - lb)));
                    astore(sc.parts + 3 * part + 1, tag_word(ep, 0, (uint32_t)lg));
                    if (sc.frame_lens) astore(sc.parts + 3 * part + 2, tag_word(ep, 0, (uint32_t)lf));
                }
            } else {
                if (ok) {
                    astore(sc.tagged + 3 * g, tag_word(ep, 0, (uint32_t)t));
                    astore(sc.tagged + 3 * g + 1, tag_word(ep, 0, (uint32_t)h));
                    astore(sc.tagged + 3 * g + 2, tag_word(ep, 0, (uint32_t)w));
                }
                if (lane == leader) {
                    astore(sc.parts + 3 * part, tag_word(ep, kPartMulti, 0u));
                    astore(sc.parts + 3 * part + 1, tag_word(ep, 0, 0u));
                    if (sc.frame_lens) astore(sc.parts + 3 * part + 2, tag_word(ep, 0, 0u));
                }
            }
        },
        NoHook(),
        [&](int64_t sb, int32_t off, int32_t org, int32_t fl) {
            if (sc.planes) return false;  // planes_out is written token by token (sink)
            const int64_t p0 = c0 / kPartTokens, np = (c_end - c0 + kPartTokens - 1) / kPartTokens;
            if (lane < np) {
                uint64_t *rec = sc.parts + 3 * (p0 + lane);
                astore(rec, tag_word(ep, kPartSingle, (uint32_t)(int32_t)((int64_t)off - sb)));
                astore(rec + 1, tag_word(ep, 0, (uint32_t)org));
                if (sc.frame_lens) astore(rec + 2, tag_word(ep, 0, (uint32_t)fl));
            }
            return true;
        });
}

// The planes of this lane's token g (< n_tokens when ok) in wave's group [G, G + 8), taken from the
// part handover, or -- when it is missing after the polls, or wait is false -- from a scan of the
// chunk by this wave.
__device__ void sf_planes(const Scan &sc, uint32_t ep, int lane, int64_t G, int64_t g, bool ok, bool wait,
                          int32_t &pt, int32_t &ph, int32_t &pw)
{
    const int64_t part = G / kPartTokens;
    bool have = false;
    pt = ph = pw = 0;
    if (wait) {
        uint64_t w0 = 0, w1 = 0, w2 = 0;
        bool ready = false;
        const bool per_seq = sc.frame_lens != nullptr;
        for (int poll = 0;; ++poll) {
            w0 = aload(sc.parts + 3 * part);
            w1 = aload(sc.parts + 3 * part + 1);
            if (per_seq) w2 = aload(sc.parts + 3 * part + 2);
            ready = tagged_with(w0, ep) && tagged_with(w1, ep) && (!per_seq || tagged_with(w2, ep));
            if (ready || poll == kPolls) break;
            __builtin_amdgcn_s_sleep(8);
        }
        if (ready && ((w0 >> 32) & 3u) == kPartSingle) {
            const int32_t base = (int32_t)(uint32_t)w0, org = (int32_t)(uint32_t)w1;
            const int32_t fl = per_seq ? (int32_t)(uint32_t)w2 : sc.frame_len;
            const int32_t p = (int32_t)g + base;
            if (ok) canvas_planes(p, (org != kNone && org <= p) ? org : kNone, fl, pt, ph, pw);
            have = true;
        } else if (ready) {
            for (int poll = 0;; ++poll) {
                if (ok && !have) {
                    const uint64_t a = aload(sc.tagged + 3 * g), b = aload(sc.tagged + 3 * g + 1),
                                   c = aload(sc.tagged + 3 * g + 2);
                    if (tagged_with(a, ep) && tagged_with(b, ep) && tagged_with(c, ep)) {
                        pt = (int32_t)(uint32_t)a;
                        ph = (int32_t)(uint32_t)b;
                        pw = (int32_t)(uint32_t)c;
                        have = true;
                    }
                }
                if (__ballot(ok && !have) == 0 || poll == kPolls) break;
                __builtin_amdgcn_s_sleep(8);
            }
            have = have || !ok;
        }
    }
    if (__ballot(!have) == 0) return;
    // fallback: this wave scans the chunk (not as its owner: the scan workgroup publishes it)
    const int64_t chunk = G / kChunk, c0 = chunk * kChunk;
    const int kk = (int)((G - c0) >> 6);     // the 64-token block holding the wave's tokens
    const int src = (int)((g - c0) & 63);    // the lane that carries this lane's token there
    scan_chunk(
        sc, status_array(sc.workspace), chunk, ep, lane, false,
        [&](int k, bool tok, int32_t t, int32_t h, int32_t w, const SeqInfo &) {
            const int okv = __shfl((int)tok, src);
            const int32_t tt = __shfl(t, src), hh = __shfl(h, src), ww = __shfl(w, src);
            if (k == kk && okv) {
                pt = tt;
                ph = hh;
                pw = ww;
            }
        },
        NoHook(),
        [&](int64_t sb, int32_t off, int32_t org, int32_t fl) {
            const int32_t p = off + (int32_t)(g - sb);
            if (ok) canvas_planes(p, (org != kNone && org <= p) ? org : kNone, fl, pt, ph, pw);
            return true;
        });
}

// Block order of the scan-first grid.  The first `lead` scan workgroups come first; then each
// further scan workgroup follows the rotation workgroups of the 4 chunks (64 parts) that lie `lead`
// scan workgroups behind it, so a chunk's scan runs well before its rotation while the scans of
// later chunks overlap the rotation stream; the rotation workgroups of the last chunks close the
// grid.  The grid has n_scan + max(n_parts, 64 (n_scan - lead)) workgroups; parts past the last
// token exit at once.  With the fallback hook every rotation workgroup comes first.
constexpr int kPartsPerScanBlock = kScanWaves * (kChunk / kPartTokens);

__device__ __forceinline__ void sf_block_role(int64_t b, int64_t n_scan, int64_t lead, int64_t n_parts, bool rot_first,
                                              bool &is_scan, int64_t &idx)
{
    if (rot_first) {
        is_scan = b >= n_parts;
        idx = is_scan ? b - n_parts : b;
        return;
    }
    if (b < lead) {
        is_scan = true;
        idx = b;
        return;
    }
    const int64_t u = b - lead, ng = n_scan - lead, span = kPartsPerScanBlock + 1;
    if (u < ng * span) {
        const int64_t grp = u / span, r = u - grp * span;
        is_scan = r == kPartsPerScanBlock;
        idx = is_scan ? lead + grp : grp * kPartsPerScanBlock + r;
        return;
    }
    is_scan = false;
    idx = ng * kPartsPerScanBlock + (u - ng * span);
}

template <int IO, bool NTS, bool W16 = false>
__global__ __launch_bounds__(kBlock) void apply_ids_sf_kernel(Heads hd, Rotary rot, Scan sc, int64_t n_scan_blocks,
                                                              int64_t lead, int hooks)
{
    static_assert(!W16 || IO == kIoF32, "sixteen lanes: fp32");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const uint32_t ep = launch_epoch(sc);
    const int64_t n_parts = (hd.n_tokens + kPartTokens - 1) / kPartTokens;
    const bool rot_first = (hooks & kHookScanFallback) != 0;
    bool is_scan;
    int64_t idx;
    sf_block_role(blockIdx.x, n_scan_blocks, lead, n_parts, rot_first, is_scan, idx);
    if (is_scan) {
        const int64_t chunk = idx * kScanWaves + (tid >> 6);
        if (chunk * kChunk < hd.n_tokens) sf_scan_chunk(sc, chunk, ep, lane);
        return;
    }
    const int64_t part = idx;
    if constexpr (W16) {
        // fp32 with sixteen lanes a token (apply_f32w_kernel's layout): the part in two 16-token
        // steps, both steps' Q/K loads issued before the handover is read; each wave takes tokens
        // [G, G + 4) of a step
        const int l = tid & 15, m = l >> 1, half = l & 1;
        const int e0 = 32 * half + 4 * m;
        const int64_t G0 = part * kPartTokens + (tid >> 6) * 4;
        const int64_t g0 = G0 + ((tid & 63) >> 4);
        uint4 qv[2][8], kv[2][2];
        bool ok[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            ok[st] = g0 + 16 * st < hd.n_tokens;
            if (ok[st]) load_token_w<8, 2>(hd, g0 + 16 * st, e0, qv[st], kv[st]);
        }
        const LaneFreq2 lf = lane_freq2(rot, m, half);
        void *qo = hd.q_out ? hd.q_out : hd.q;
        void *ko = hd.k_out ? hd.k_out : hd.k;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int64_t G = G0 + 16 * st, g = g0 + 16 * st;
            if (G >= hd.n_tokens) break;  // wave-uniform
            int32_t pt, ph, pw;
            sf_planes(sc, ep, lane, G, g, ok[st], !rot_first, pt, ph, pw);
            if (ok[st]) {
                double c[4], ss[4];
                pair_sincos4(lf, pt, ph, pw, c, ss);
#pragma unroll
                for (int h = 0; h < 8; ++h) store16_as<NTS>(qo, q_off(hd, g, h) + e0, rotate4(qv[st][h], c, ss));
#pragma unroll
                for (int h = 0; h < 2; ++h) store16_as<NTS>(ko, k_off(hd, g, h) + e0, rotate4(kv[st][h], c, ss));
            }
        }
        return;
    }
    const int l = tid & 7, m = l >> 1, half = l & 1;
    const int e0 = 32 * half + 8 * m;
    const int64_t G = part * kPartTokens + (tid >> 6) * 8;  // the wave's first token
    if (G >= hd.n_tokens) return;
    const int64_t g = G + ((tid & 63) >> 3);
    const bool ok = g < hd.n_tokens;
    Raw8<IO> qv[8], kv[2];
    if (ok) load_token_fixed<IO, 8, 2>(hd, g, e0, qv, kv);
    int32_t pt, ph, pw;
    sf_planes(sc, ep, lane, G, g, ok, !rot_first, pt, ph, pw);
    if (ok) {
        const LaneFreq lf = lane_freq<true>(rot, m, half);
        double c[8], ss[8];
        pair_sincos(lf, pt, ph, pw, c, ss);
        rotate_token_fixed<IO, 8, 2, false, NTS>(hd, PagedKV{}, -1, g, e0, l, c, ss, qv, kv);
    }
}

// One work item of a decode step: an 8-element chunk of a Q rotation group (kind 0), a K rotation
// group (1), a K pass-through segment (2) or a V segment (3).  A rotation group of eight items never
// straddles two kinds, so the DPP partner of a rotation item is the item next to it.
struct DecodeItem {
    int kind, h, e, m, half;
    const void *src;
    int64_t soff;
};

__device__ __forceinline__ DecodeItem decode_item(const DecodeArgs &d, int64_t s, int it, int nrq, int n_rot, int n_k,
                                                  int kpass, int vch)
{
    DecodeItem r;
    r.m = 0;
    r.half = 0;
    if (it < n_rot) {
        const bool isq = it < nrq;
        r.kind = isq ? 0 : 1;
        r.h = (isq ? it : it - nrq) >> 3;
        const int l = it & 7;
        r.m = l >> 1;
        r.half = l & 1;
        r.e = 32 * r.half + 8 * r.m;
    } else if (it < n_k) {
        const int c = it - n_rot;
        r.kind = 2;
        r.h = c / kpass;
        r.e = 64 + (c - r.h * kpass) * 8;
    } else {
        const int c = it - n_k;
        r.kind = 3;
        r.h = c / vch;
        r.e = (c - r.h * vch) * 8;
    }
    r.src = r.kind == 0 ? d.q : (r.kind == 3 ? d.kv.v : d.k);
    r.soff = r.kind == 0 ? s * d.q_tok + r.h * d.q_head + r.e
                         : (r.kind == 3 ? s * d.kv.v_tok + r.h * d.kv.v_head + r.e : s * d.k_tok + r.h * d.k_head + r.e);
    return r;
}

// `per` lanes (a multiple of 64) per sequence, several sequences per workgroup, IPL items per lane
// and round (items base + lane + j * per).  Every lane issues all of a round's loads -- its items'
// data chunks and frequencies, the sequence's position, amount and slot -- before any math, so a
// round is one memory round trip plus the math; IPL > 1 puts more bytes in flight per lane, so
// fewer waves cover the step.
template <int IO, int IPL>
__global__ __launch_bounds__(IPL == 1 ? 1024 : 256) void decode_kernel(DecodeArgs d, Rotary rot, int per)
{
    // per is a multiple of 64, so each wave serves one sequence: its index is wave-uniform and the
    // sequence's position, amount and slot are scalar loads, issued before anything is stored.  They
    // are waited apart from the vector loads, so the sincos runs while the data chunks are in flight
    // (as vector loads issued after the chunks, they were waited together with them).
    const int32_t s = __builtin_amdgcn_readfirstlane((int32_t)(blockIdx.x * (blockDim.x / per) + threadIdx.x / per));
    if (s >= d.n_seqs) return;
    const PagedKV &pc = d.kv;
    const int nrq = d.nq * 8, nrk = d.nk * 8;
    const int kpass = (d.head_dim - 64) / 8;
    const int vch = d.head_dim / 8;
    const int n_rot = nrq + nrk, n_k = n_rot + d.nk * kpass;
    const int total = n_k + (pc.v ? d.nk * vch : 0);
    const int li = threadIdx.x % per;
    // Every rotation item of this lane sits at the same place in its group of eight (items
    // li + j * per with per a multiple of 64, groups starting at multiples of 8), so they share
    // one set of frequencies and one sincos evaluation.
    const int l8 = li & 7;
    const LaneFreq lf = lane_freq<false>(rot, l8 >> 1, l8 & 1);
    const int32_t plane = d.pos[s] - d.amount[s];
    const int64_t slot = pc.slots ? pc.slots[s] : -1;  // no slots without K heads
    DecodeItem item[IPL];
    bool live[IPL];
    Raw8<IO> x[IPL];
    auto issue = [&](int base) {
#pragma unroll
        for (int j = 0; j < IPL; ++j) {
            // an item past the last reads item 0 (always a valid chunk) and stores nothing; live and
            // dead items meet at a multiple of eight, so a live rotation item's partner is live
            const int it = base + li + j * per;
            live[j] = it < total;
            item[j] = decode_item(d, s, live[j] ? it : 0, nrq, n_rot, n_k, kpass, vch);
            x[j] = load8<IO>(item[j].src, item[j].soff);
        }
    };
    issue(0);
    // Every lane evaluates the sincos once, while the first round's chunks are in flight (a lane
    // without rotation items only wastes the arithmetic).
    double c[8], ss[8];
    pair_sincos(lf, plane, plane, plane, c, ss);
    for (int base = 0;;) {
#pragma unroll
        for (int j = 0; j < IPL; ++j) {
            const DecodeItem &r = item[j];
            if (r.kind <= 1) x[j] = rotate_chunk<IO>(x[j], c, ss);
            if (!live[j]) continue;
            if (r.kind == 0)
                store8<IO>(d.q, r.soff, x[j]);
            else if (slot_ok(pc, slot))
                store8_nt<IO>(r.kind == 3 ? pc.v_cache : pc.k_cache, cache_off(pc, slot, r.h) + r.e, x[j]);
        }
        base += per * IPL;
        if (base >= total) break;
        issue(base);
    }
}

__global__ void zero_kernel(uint32_t *p, size_t words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Scalars when the call has no tokens: every sequence keeps the origin it carries in (if any).
__global__ void text_scalars_kernel(Scan sc)
{
    const int32_t s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= sc.n_seqs) return;
    const int32_t oin = sc.origin_in ? sc.origin_in[s] : -1;
    bool bad_fl = false;
    const int32_t fl = seq_frame_len(sc, s, bad_fl);
    write_scalars(sc, s, oin >= 0 ? oin : -1, false, sc.pos_offset ? sc.pos_offset[s] : 0, fl, bad_fl);
}

// Device-counter epochs: advance the counter once the scan launch before it has finished.
__global__ void epoch_bump_kernel(WsHeader *hdr)
{
    if (threadIdx.x == 0) hdr->epoch = (hdr->epoch + 1u) & kEpochMask;
}

}  // namespace

// ------------------------------------------------------------------ launchers ------------------
hipError_t launch_workspace_init(void *ws, size_t bytes, hipStream_t stream)
{
    const size_t words = bytes / 4;
    const size_t want = (words + 255) / 256;
    const unsigned blocks = (unsigned)(want > 1024 ? 1024 : (want ? want : 1));
    if (words) zero_kernel<<<blocks, 256, 0, stream>>>(static_cast<uint32_t *>(ws), words);
    return hipGetLastError();
}

hipError_t launch_text_scalars(const Scan &s, hipStream_t stream)
{
    text_scalars_kernel<<<(s.n_seqs + 255) / 256, 256, 0, stream>>>(s);
    return hipGetLastError();
}

static hipError_t bump_if_device_epoch(const Scan &s, hipStream_t stream)
{
    if (s.epoch == 0) epoch_bump_kernel<<<1, 64, 0, stream>>>(static_cast<WsHeader *>(s.workspace));
    return hipGetLastError();
}

hipError_t launch_planes(const Scan &s, hipStream_t stream)
{
    const int64_t n_chunks = (s.n_tokens + kChunk - 1) / kChunk;
    const unsigned blocks = (unsigned)((n_chunks + kBlock / 64 - 1) / (kBlock / 64));
    planes_kernel<<<blocks, kBlock, 0, stream>>>(s, n_chunks);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : bump_if_device_epoch(s, stream);
}

// Workgroups per compute unit of the grid-stride rotary kernel (its VGPR use allows two resident).
#ifndef MROPE_APPLY_BLOCKS_PER_CU
#define MROPE_APPLY_BLOCKS_PER_CU 2
#endif
constexpr int kApplyBlocksPerCU = MROPE_APPLY_BLOCKS_PER_CU;

// Compute units of the current device, queried once per device and kept (the grid shapes depend on
// it; the attribute query costs more host time than a launch).  Racing first calls store the same
// value.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_compute_units[kMaxDevices];

static int compute_units()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int known = g_compute_units[dev].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    if (dev >= 0 && dev < kMaxDevices) g_compute_units[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// The fixed-head kernels cover the model's shape (8 Q heads, 2 KV heads); with a cache they also
// need head_dim 256, and in fp32 the sixteen-lane layout (eight lanes would carry twice the copy
// chunks a lane): with the eight-lane hook, fp32 cache writes take the generic kernels.
static bool fixed_heads(const Heads &h, const PagedKV &pc, int io)
{
    if (h.nq != 8 || h.nk != 2) return false;
    return !pc.k_cache || (h.head_dim == 256 && (io != kIoF32 || !(test_hooks() & kHookF32EightLanes)));
}

// The fixed-head kernels' Q/K stores take the non-temporal hint (the NTS template argument) out of
// place, and in place when the launch writes more than this in place: up to about there the 256 MB
// memory-side cache absorbs the written lines and plain stores are faster, beyond it the hint is.
// Measured (bf16, 8 + 2 heads; plain vs hinted): mrope_apply 109 vs 131 us at 262,144 tokens
// (335 MB written in place), 164 vs 159 us at 327,680 (419 MB), 202 vs 190 us at 393,216, 527 vs
// 498 us at 1,048,576 (fused: 531 vs 505); the fused K/V cache write (Q in place) 281 vs 323 us at
// 262,144 (268 MB), 495 vs 480 us at 393,216 (403 MB), 1,318 vs 1,281 us at 1,048,576.  fp32 at
// 262,144 tokens (671 MB): equal.  Out of place (64 x 4096 bf16) 464 vs 459 us.
constexpr int64_t kNtInplaceBytes = 352ll << 20;

template <int IO>
static bool nt_stores(const Heads &h, const PagedKV &pc)
{
    constexpr int64_t es = IO == kIoF32 ? 4 : 2;
    if (h.q_out || h.k_out) return true;
    const int64_t heads = h.nq + (pc.k_cache ? 0 : h.nk);
    return h.n_tokens * heads * 64 * es > kNtInplaceBytes;
}

// Out of place: copy dims 64..head_dim of every Q and K head (see copy_rest_kernel), for each head
// set that has an output buffer (a call with no Q heads may pass only k_out, and one with no K heads
// only q_out).  Nothing to do in place or when the heads hold only rotated dims.
template <int IO>
static hipError_t copy_rest(const Heads &h, hipStream_t st)
{
    constexpr int64_t es = IO == kIoF32 ? 4 : 2;
    const int n_chunks = (int)((h.head_dim - 64) * es / 16);
    if ((!h.q_out && !h.k_out) || n_chunks <= 0 || h.n_tokens <= 0) return hipSuccess;
    auto one = [&](const void *src, void *dst, int64_t tok, int64_t head, int nh) {
        if (nh <= 0 || !dst) return;
        const int64_t n_rows = h.n_tokens * nh;
        const int shift = (nh & (nh - 1)) == 0 ? __builtin_ctz((unsigned)nh) : -1;
        constexpr int64_t kRowsPerBlock = kBlock / 8 * kRestRows;
        const int64_t need = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
        const unsigned blocks = (unsigned)(need < (1 << 20) ? need : (1 << 20));
        copy_rest_kernel<<<blocks, kBlock, 0, st>>>(static_cast<const char *>(src), static_cast<char *>(dst), tok * es,
                                                    head * es, nh, shift, n_rows, 64 * es, n_chunks);
    };
    one(h.q, h.q_out, h.q_tok, h.q_head, h.nq);
    one(h.k, h.k_out, h.k_tok, h.k_head, h.nk);
    return hipGetLastError();
}

template <int IO>
static hipError_t apply_dispatch(const Heads &h, const Rotary &r, const int32_t *planes, int64_t ps,
                                 const PagedKV &pc, hipStream_t st)
{
    if (const hipError_t ce = copy_rest<IO>(h, st); ce != hipSuccess) return ce;
    const bool nts = nt_stores<IO>(h, pc);
    const int64_t groups = (h.n_tokens + kTokPerBlock - 1) / kTokPerBlock;
    if (fixed_heads(h, pc, IO)) {
        // Up to 16 grid-stride steps per workgroup the grid is persistent (two workgroups per CU).
        // Beyond that, one step per workgroup, many more workgroups than fit at once: the
        // dispatcher hands a freed slot the next workgroup, which balances the unequal rates of the
        // CUs.  Measured (bf16): 1,048,576 tokens 498 us with two-step workgroups, 470 us with one
        // step, 524 us persistent; 393,216 tokens 189 -> 175 us.  At 262,144 tokens (16 steps) the
        // persistent grid is 3 % faster than one-step workgroups.
        const int64_t persistent = (int64_t)compute_units() * kApplyBlocksPerCU;
        const int64_t cap = groups > 16 * persistent ? groups : persistent;
        const unsigned blocks = (unsigned)(groups < cap ? groups : cap);
        if constexpr (IO != kIoF32) {
            if (pc.k_cache) {
                // the cache-writing loop has no prefetch: one step per workgroup at every size
                // (64 x 4096 tokens: 271 -> 266 us against the persistent grid)
                const unsigned kv_blocks = (unsigned)groups;
                if (nts) apply_kv_kernel<IO, 8, 2, true><<<kv_blocks, kBlock, 0, st>>>(h, r, planes, ps, pc);
                else apply_kv_kernel<IO, 8, 2, false><<<kv_blocks, kBlock, 0, st>>>(h, r, planes, ps, pc);
                return hipGetLastError();
            }
        }
        if constexpr (IO == kIoF32) {
            if (pc.k_cache) {
                // sixteen lanes a token, one step per workgroup at every size (as the 16-bit kernel)
                const unsigned kv_blocks = (unsigned)((h.n_tokens + kTokPerBlockW - 1) / kTokPerBlockW);
                if (nts) apply_kv_f32w_kernel<8, 2, true><<<kv_blocks, kBlock, 0, st>>>(h, r, planes, ps, pc);
                else apply_kv_f32w_kernel<8, 2, false><<<kv_blocks, kBlock, 0, st>>>(h, r, planes, ps, pc);
                return hipGetLastError();
            }
            if (!(test_hooks() & kHookF32EightLanes)) {
                // sixteen lanes a token: the same grid policy over 16-token workgroup steps
                const int64_t groups_w = (h.n_tokens + kTokPerBlockW - 1) / kTokPerBlockW;
                const int64_t cap_w = groups_w > 16 * persistent ? groups_w : persistent;
                const unsigned blocks_w = (unsigned)(groups_w < cap_w ? groups_w : cap_w);
                if (nts) apply_f32w_kernel<8, 2, true><<<blocks_w, kBlock, 0, st>>>(h, r, planes, ps);
                else apply_f32w_kernel<8, 2, false><<<blocks_w, kBlock, 0, st>>>(h, r, planes, ps);
                return hipGetLastError();
            }
        }
        if (nts) apply_kernel<IO, 8, 2, true><<<blocks, kBlock, 0, st>>>(h, r, planes, ps);
        else apply_kernel<IO, 8, 2, false><<<blocks, kBlock, 0, st>>>(h, r, planes, ps);
    } else {
        apply_any_kernel<IO><<<(unsigned)groups, kBlock, 0, st>>>(h, r, planes, ps, pc);
    }
    return hipGetLastError();
}

hipError_t launch_apply(const Heads &h, const Rotary &r, const int32_t *planes, int64_t ps, const PagedKV &pc, int io,
                        hipStream_t stream)
{
    switch (io) {
    case kIoBF16: return apply_dispatch<kIoBF16>(h, r, planes, ps, pc, stream);
    case kIoF16: return apply_dispatch<kIoF16>(h, r, planes, ps, pc, stream);
    default: return apply_dispatch<kIoF32>(h, r, planes, ps, pc, stream);
    }
}

template <int IO>
static hipError_t apply_ids_dispatch(const Heads &h, const Rotary &r, const Scan &s, const PagedKV &pc, hipStream_t st)
{
    if (const hipError_t ce = copy_rest<IO>(h, st); ce != hipSuccess) return ce;
    const bool nts = nt_stores<IO>(h, pc);
    const int64_t n_chunks = (h.n_tokens + kChunk - 1) / kChunk;
    // Small inputs split each chunk over up to 16 workgroups (down to one 32-token step each) while
    // that keeps the grid within two workgroups per CU.  Larger ones split each chunk in two: with
    // one workgroup per chunk, a chunk count between one and two grids of resident workgroups left
    // slots idle or ran a partial second round, and halves let the dispatcher even the rounds out.
    // Measured (bf16, back to back): the 64 x 4096 step 116.2 -> 113.0 us (200 warm-up launches),
    // 163,840 tokens (64 sequences) 92 -> 81 us, 196,608 104 -> 99, 1,048,576 ragged 509 -> 501,
    // 8 x 32768 unchanged (118 us).  Four parts cost more than they balance (262,144 tokens: 130).
    const int64_t target = (int64_t)compute_units() * 2;
    int part_log = 0;
    while (part_log < 4 && (n_chunks << (part_log + 1)) <= target) ++part_log;
    if (part_log == 0) part_log = 1;
    const unsigned blocks = (unsigned)(n_chunks << part_log);
    if (fixed_heads(h, pc, IO)) {
        bool done = false;
        if constexpr (IO != kIoF32) {
            if (pc.k_cache) {
                if (nts) apply_ids_kernel<IO, 8, 2, true, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                else apply_ids_kernel<IO, 8, 2, true, false><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                done = true;
            }
        }
        if constexpr (IO == kIoF32) {
            if (pc.k_cache) {
                if (nts) apply_ids_kernel<IO, 8, 2, true, true, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                else apply_ids_kernel<IO, 8, 2, true, false, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                done = true;
            }
            if (!done && !(test_hooks() & kHookF32EightLanes)) {
                if (nts) apply_ids_kernel<IO, 8, 2, false, true, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                else apply_ids_kernel<IO, 8, 2, false, false, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
                done = true;
            }
        }
        if (!done && nts) apply_ids_kernel<IO, 8, 2, false, true><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
        if (!done && !nts) apply_ids_kernel<IO, 8, 2, false, false><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
    } else {
        apply_ids_kernel<IO, 0, 0, false, false><<<blocks, kBlock, 0, st>>>(h, r, s, pc, part_log);
    }
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : bump_if_device_epoch(s, st);
}

// Scan-first fused kernel (fixed heads, no cache write).  kScanLead: scan workgroups (4 chunks,
// 64 rotation workgroups each) that run ahead of the rotation.  Measured on 1,048,576 ragged tokens
// (four workgroups per CU): every scan first 485.8 us, a lead of 128 scan workgroups 484.7, 32
// 479.9, 8 479.5; the scan itself then costs nothing measurable (the same grid with no scan and
// constant planes: 478.4 us).
constexpr int64_t kScanLead = 32;

template <int IO>
static hipError_t apply_ids_sf_dispatch(const Heads &h, const Rotary &r, const Scan &s, hipStream_t st)
{
    if (const hipError_t ce = copy_rest<IO>(h, st); ce != hipSuccess) return ce;
    const int64_t n_chunks = (h.n_tokens + kChunk - 1) / kChunk;
    const int64_t n_scan = (n_chunks + kScanWaves - 1) / kScanWaves;
    const int64_t n_parts = (h.n_tokens + kPartTokens - 1) / kPartTokens;
    const int hooks = test_hooks();
    const int64_t lead = n_scan < kScanLead ? n_scan : kScanLead;
    const int64_t rot_blocks = (hooks & kHookScanFallback) ? n_parts
                                                           : std::max(n_parts, (n_scan - lead) * kPartsPerScanBlock);
    const unsigned blocks = (unsigned)(n_scan + rot_blocks);
    // Two workgroups per CU: the kernel needs 141 VGPRs (three could be resident), but more
    // concurrent 32-token parts make the HBM stream slower.  Measured on 1,048,576 ragged tokens:
    // 480 us at four workgroups per CU, 476 at three, 468 at two (mrope_apply, two by its registers:
    // 467), 680 at one.  The unused dynamic LDS holds the occupancy there.
    constexpr unsigned kOccupancyLds = 64 << 10;
    const bool nts = nt_stores<IO>(h, PagedKV{});
    if constexpr (IO == kIoF32) {
        if (!(hooks & kHookF32EightLanes)) {
            if (nts) apply_ids_sf_kernel<IO, true, true><<<blocks, kBlock, kOccupancyLds, st>>>(h, r, s, n_scan, lead, hooks);
            else apply_ids_sf_kernel<IO, false, true><<<blocks, kBlock, kOccupancyLds, st>>>(h, r, s, n_scan, lead, hooks);
            const hipError_t e = hipGetLastError();
            return e != hipSuccess ? e : bump_if_device_epoch(s, st);
        }
    }
    if (nts)
        apply_ids_sf_kernel<IO, true><<<blocks, kBlock, kOccupancyLds, st>>>(h, r, s, n_scan, lead, hooks);
    else
        apply_ids_sf_kernel<IO, false><<<blocks, kBlock, kOccupancyLds, st>>>(h, r, s, n_scan, lead, hooks);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : bump_if_device_epoch(s, st);
}

// Which fused kernel serves a call: the scan-first kernel for the model's heads from this many
// tokens on (where mrope_apply takes one-step workgroups), the chunk-per-workgroup kernel below it
// and for other shapes.
static bool use_scan_first(const Heads &h, const PagedKV &pc, int io)
{
    const int hooks = test_hooks();
    if (pc.k_cache || h.nq != 8 || h.nk != 2 || (hooks & kHookFusedChunked)) return false;
    if (hooks & (kHookFusedScanFirst | kHookScanFallback)) return true;
    const int64_t one_step_from = (int64_t)compute_units() * kApplyBlocksPerCU * 16 * kTokPerBlock;
    return h.n_tokens > one_step_from && io >= 0;
}

hipError_t launch_apply_ids(const Heads &h, const Rotary &r, const Scan &s, const PagedKV &pc, int io,
                            hipStream_t stream)
{
    if (use_scan_first(h, pc, io)) {
        switch (io) {
        case kIoBF16: return apply_ids_sf_dispatch<kIoBF16>(h, r, s, stream);
        case kIoF16: return apply_ids_sf_dispatch<kIoF16>(h, r, s, stream);
        default: return apply_ids_sf_dispatch<kIoF32>(h, r, s, stream);
        }
    }
    // With the planes wanted in memory anyway (planes_out) and past the size where mrope_apply
    // takes one step per workgroup, the scan writes planes_out and the rotation reads it back: one
    // workgroup per chunk cannot use that grid.  The scan-first kernel serves the model's heads
    // without a cache write; this route serves the cache-writing call.  Measured (bf16, before the
    // scan-first kernel): 1,048,576 ragged tokens 17.5 + 465 us against 508 us fused; 524,288
    // tokens ~243 against 261 us.
    const int64_t one_step_from = (int64_t)compute_units() * kApplyBlocksPerCU * 16 * kTokPerBlock;
    if (s.planes && fixed_heads(h, pc, io) && h.n_tokens > one_step_from) {
        const hipError_t e = launch_planes(s, stream);
        return e != hipSuccess ? e : launch_apply(h, r, s.planes, s.plane_stride, pc, io, stream);
    }
    switch (io) {
    case kIoBF16: return apply_ids_dispatch<kIoBF16>(h, r, s, pc, stream);
    case kIoF16: return apply_ids_dispatch<kIoF16>(h, r, s, pc, stream);
    default: return apply_ids_dispatch<kIoF32>(h, r, s, pc, stream);
    }
}

#ifndef MROPE_DECODE_BLOCK
#define MROPE_DECODE_BLOCK 256
#endif

template <int IO>
static void decode_launch(int ipl, unsigned blocks, unsigned threads, const DecodeArgs &d, const Rotary &r, int per,
                          hipStream_t stream)
{
    switch (ipl) {
    case 3: decode_kernel<IO, 3><<<blocks, threads, 0, stream>>>(d, r, per); break;
    case 2: decode_kernel<IO, 2><<<blocks, threads, 0, stream>>>(d, r, per); break;
    default: decode_kernel<IO, 1><<<blocks, threads, 0, stream>>>(d, r, per); break;
    }
}

hipError_t launch_decode(const DecodeArgs &d, const Rotary &r, int io, hipStream_t stream)
{
    const int items = (d.nq + d.nk) * 8 + d.nk * (d.head_dim - 64) / 8 + (d.kv.v ? d.nk * d.head_dim / 8 : 0);
    if (items == 0 || d.n_seqs == 0) return hipSuccess;
    // Items per lane: the most (up to 3) that leave less than a wave of lanes idle, with at most a
    // 256-lane workgroup per sequence (the 2- and 3-item kernels are built for 256 threads).  The
    // model's shape without V (128 items) takes 2, one wave per sequence; with V (192) 3.  Measured
    // on 4,096 sequences: 9.4 -> 8.6 us and 12.5 -> 10.4 us; 4 items per lane took 20 us.
    auto lanes = [&](int ipl) {
        const int need = (items + ipl - 1) / ipl;
        return need >= 1024 ? 1024 : (need + 63) / 64 * 64;
    };
    int ipl = 1;
    for (int c = 3; c >= 2; --c) {
        if (lanes(c) <= MROPE_DECODE_BLOCK && lanes(c) * c - items < 64) {
            ipl = c;
            break;
        }
    }
    const int per = lanes(ipl);  // lanes per sequence
    const int spb = per >= MROPE_DECODE_BLOCK ? 1 : MROPE_DECODE_BLOCK / per;  // sequences per workgroup
    const unsigned blocks = (unsigned)((d.n_seqs + spb - 1) / spb);
    const unsigned threads = (unsigned)(per * spb);
    switch (io) {
    case kIoBF16: decode_launch<kIoBF16>(ipl, blocks, threads, d, r, per, stream); break;
    case kIoF16: decode_launch<kIoF16>(ipl, blocks, threads, d, r, per, stream); break;
    default: decode_launch<kIoF32>(ipl, blocks, threads, d, r, per, stream); break;
    }
    return hipGetLastError();
}

}  // namespace mrope
