// C ABI of libmrope: argument checks, rotary constants, launches.  The entry points are declared
// and documented in include/mrope.h.
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "mrope.h"
#include "mrope_internal.h"

using namespace mrope;

namespace mrope {
// Test and tuning hooks (mrope_set_test_hooks); 0 in normal use.
static std::atomic<int> g_test_hooks{0};
int test_hooks() { return g_test_hooks.load(std::memory_order_relaxed); }
}  // namespace mrope


namespace {

thread_local char g_last_error[512] = "";

mrope_status fail(mrope_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

mrope_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return MROPE_OK;
    return fail(MROPE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rotary constants for rot_dim = 64.
//   inv_freq[j] = 1 / theta^(2j/64): the power in double rounded once to fp32, the reciprocal one
//   IEEE fp32 division -- the fp32 buffer a torch rotary builds for this theta.
//   Frequency j reads plane H if j%3==1 && j<33, W if j%3==2 && j<30, else T (three planes in
//   interleaved sections [11, 11, 10]: card "MiniCPM-V-4.7-1B -- Core AI", section "What it is").
Rotary make_rotary(double theta)
{
    Rotary r;
    r.plane_sel = 0;
    for (int j = 0; j < 32; ++j) {
        const float p = (float)std::pow(theta, (2.0 * j) / 64.0);
        r.inv_freq[j] = 1.0f / p;
        uint64_t plane = 0;
        if (j % 3 == 1 && j < 33)
            plane = 1;
        else if (j % 3 == 2 && j < 30)
            plane = 2;
        r.plane_sel |= plane << (2 * j);
    }
    return r;
}

mrope_status check_heads(void *q, int64_t q_tok, int64_t q_head, int32_t nq, void *k, int64_t k_tok, int64_t k_head,
                         int32_t nk, int64_t n_tokens, int32_t head_dim, int32_t rot_dim, int32_t dtype, void *q_out,
                         void *k_out)
{
    if (dtype != MROPE_F32 && dtype != MROPE_BF16 && dtype != MROPE_F16)
        return fail(MROPE_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if (rot_dim != 64) return fail(MROPE_ERR_UNSUPPORTED, "rot_dim must be 64 (got %d)", rot_dim);
    if (head_dim < 64 || head_dim > 1024 || head_dim % 8)
        return fail(MROPE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in [64, 1024] (got %d)", head_dim);
    if (nq < 0 || nk < 0 || nq > kMaxHeads || nk > kMaxHeads)
        return fail(MROPE_ERR_UNSUPPORTED, "head counts must be in [0, %d] (got %d, %d)", kMaxHeads, nq, nk);
    if (n_tokens < 0 || n_tokens > 0x7ffffffe) return fail(MROPE_ERR_ARG, "n_tokens out of range (%lld)", (long long)n_tokens);
    if (nq > 0 && n_tokens > 0 && !q) return fail(MROPE_ERR_ARG, "q is NULL");
    if (nk > 0 && n_tokens > 0 && !k) return fail(MROPE_ERR_ARG, "k is NULL");
    if ((q_out == nullptr) != (k_out == nullptr) && nk > 0 && nq > 0)
        return fail(MROPE_ERR_ARG, "q_out and k_out must both be NULL (in place) or both be set");
    if (q_out && nk > 0 && !k_out) return fail(MROPE_ERR_ARG, "k_out is NULL while q_out is set");
    if (k_out && nq > 0 && !q_out) return fail(MROPE_ERR_ARG, "q_out is NULL while k_out is set");
    if (q_tok < 0 || q_head < 0 || k_tok < 0 || k_head < 0) return fail(MROPE_ERR_ARG, "negative stride");
    const int64_t vec = dtype == MROPE_F32 ? 4 : 8;
    if ((nq > 0 && (q_tok % vec || q_head % vec)) || (nk > 0 && (k_tok % vec || k_head % vec)))
        return fail(MROPE_ERR_ALIGN, "strides must be multiples of %lld elements", (long long)vec);
    if ((nq > 0 && !aligned16(q)) || (nk > 0 && !aligned16(k)) || (q_out && !aligned16(q_out)) ||
        (k_out && !aligned16(k_out)))
        return fail(MROPE_ERR_ALIGN, "Q/K pointers must be 16-byte aligned");
    if (nq > 0 && q_head < head_dim && nq > 1) return fail(MROPE_ERR_ARG, "q_head_stride < head_dim");
    if (nk > 0 && k_head < head_dim && nk > 1) return fail(MROPE_ERR_ARG, "k_head_stride < head_dim");
    return MROPE_OK;
}

Heads make_heads(void *q, int64_t q_tok, int64_t q_head, int32_t nq, void *k, int64_t k_tok, int64_t k_head, int32_t nk,
                 int64_t n_tokens, int32_t head_dim, void *q_out, void *k_out)
{
    Heads h{};
    h.q = q;
    h.k = k;
    h.q_out = q_out;
    h.k_out = k_out;
    h.q_tok = q_tok;
    h.q_head = q_head;
    h.k_tok = k_tok;
    h.k_head = k_head;
    h.nq = nq;
    h.nk = nk;
    h.head_dim = head_dim;
    h.n_tokens = n_tokens;
    return h;
}

mrope_status check_scan(const int32_t *ids, const int32_t *cu, int32_t n_seqs, int64_t n_tokens, int32_t *planes,
                        int64_t plane_stride, void *ws, size_t ws_bytes, bool planes_required)
{
    if (n_seqs < 0) return fail(MROPE_ERR_ARG, "n_seqs < 0");
    if (n_tokens < 0 || n_tokens > 0x7ffffffe) return fail(MROPE_ERR_ARG, "n_tokens out of range (%lld)", (long long)n_tokens);
    if (n_seqs == 0 && n_tokens > 0) return fail(MROPE_ERR_ARG, "tokens given but no sequences");
    if (n_seqs > 0 && !cu) return fail(MROPE_ERR_ARG, "cu_seqlens is NULL");
    if (n_tokens > 0 && !ids) return fail(MROPE_ERR_ARG, "ids is NULL");
    if (planes_required && n_tokens > 0 && !planes) return fail(MROPE_ERR_ARG, "planes is NULL");
    if (planes && plane_stride < n_tokens) return fail(MROPE_ERR_ARG, "plane_stride < n_tokens");
    if (n_tokens > 0) {
        if (!ws) return fail(MROPE_ERR_WORKSPACE, "workspace is NULL");
        if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MROPE_ERR_WORKSPACE, "workspace not 256-byte aligned");
        if (ws_bytes < mrope_workspace_bytes(n_tokens))
            return fail(MROPE_ERR_WORKSPACE, "workspace too small (%zu < %zu)", ws_bytes, mrope_workspace_bytes(n_tokens));
    }
    return MROPE_OK;
}

Scan make_scan(const int32_t *ids, const int32_t *cu, int32_t n_seqs, int64_t n_tokens, int32_t marker,
               int32_t frame_len, const int32_t *frame_len_seq, const int32_t *pos_offset,
               const int32_t *origin_in, int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount,
               int32_t *origin, int32_t *flags, void *ws, uint32_t epoch)
{
    Scan s;
    s.ids = ids;
    s.cu = cu;
    s.n_seqs = n_seqs;
    s.marker = marker;
    s.n_tokens = n_tokens;
    s.planes = planes;
    s.plane_stride = plane_stride;
    s.start = start;
    s.amount = amount;
    s.origin = origin;
    s.flags = flags;
    s.pos_offset = pos_offset;
    s.origin_in = origin_in;
    s.frame_len = frame_len == 0 ? kDefaultFrameLen : frame_len;
    s.frame_lens = frame_len_seq;
    s.workspace = ws;
    const WsLayout lay = ws_layout(n_tokens);
    s.parts = ws ? reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + lay.parts) : nullptr;
    s.tagged = ws ? reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + lay.tagged) : nullptr;
    s.epoch = epoch;
    return s;
}

bool any_scalar(const Scan &s) { return s.start || s.amount || s.origin || s.flags; }

mrope_status check_frame_len(int32_t frame_len)
{
    if (frame_len != 0 && (frame_len < 65 || frame_len > kMaxFrameLen))
        return fail(MROPE_ERR_ARG, "frame_len must be 0 (67) or in [65, %d] (got %d)", kMaxFrameLen, frame_len);
    return MROPE_OK;
}

// Paged K/V cache arguments; n_kv_heads == 0 needs none of them.
mrope_status check_paged(int32_t n_kv_heads, const void *v, int64_t v_tok, int64_t v_head, void *k_cache,
                         void *v_cache, const int64_t *slots, int32_t block_size, int64_t num_blocks,
                         int64_t c_block, int64_t c_tok, int64_t c_head, int32_t head_dim, int32_t dtype)
{
    if (n_kv_heads == 0) return MROPE_OK;
    if (!k_cache || !slots) return fail(MROPE_ERR_ARG, "k_cache / slot_mapping is NULL");
    if ((v == nullptr) != (v_cache == nullptr)) return fail(MROPE_ERR_ARG, "v and v_cache must both be NULL or both set");
    if (block_size <= 0 || num_blocks < 0) return fail(MROPE_ERR_ARG, "block_size must be > 0 and num_blocks >= 0");
    if (c_block < 0 || c_tok < 0 || c_head < 0 || v_tok < 0 || v_head < 0) return fail(MROPE_ERR_ARG, "negative stride");
    if (n_kv_heads > 1 && c_head < head_dim) return fail(MROPE_ERR_ARG, "cache_head_stride < head_dim");
    if (v && n_kv_heads > 1 && v_head < head_dim) return fail(MROPE_ERR_ARG, "v_head_stride < head_dim");
    const int64_t vec = dtype == MROPE_F32 ? 4 : 8;
    if (!aligned16(k_cache) || !aligned16(v_cache) || c_block % vec || c_tok % vec || c_head % vec)
        return fail(MROPE_ERR_ALIGN, "cache pointers / strides break 16-byte alignment");
    if (v && (!aligned16(v) || v_tok % vec || v_head % vec))
        return fail(MROPE_ERR_ALIGN, "v pointer / strides break 16-byte alignment");
    return MROPE_OK;
}

PagedKV make_paged(const void *v, int64_t v_tok, int64_t v_head, void *k_cache, void *v_cache, const int64_t *slots,
                   int32_t block_size, int64_t num_blocks, int64_t c_block, int64_t c_tok, int64_t c_head)
{
    PagedKV p{};
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.v = v;
    p.v_tok = v_tok;
    p.v_head = v_head;
    p.slots = slots;
    p.block_size = block_size > 0 ? block_size : 1;
    p.num_slots = k_cache ? num_blocks * (int64_t)p.block_size : 0;
    p.bs_shift = -1;
    if ((p.block_size & (p.block_size - 1)) == 0) {
        int sh = 0;
        while ((1 << sh) < p.block_size) ++sh;
        p.bs_shift = sh;
    }
    p.c_block = c_block;
    p.c_tok = c_tok;
    p.c_head = c_head;
    return p;
}

}  // namespace

// ------------------------------------------------------------------ static scratch -------------
// The workspace of mrope_apply_ids_noalloc: a file-scope device array, one copy per GPU, held until
// the process ends.  In host code `scratch` only stands in for the symbol; the device address of a
// GPU's copy comes from hipGetSymbolAddress with that GPU current, once, and is kept per device.
// The first call on a device also clears the copy with a kernel on the caller's stream (so it must
// not be captured in a graph); later calls tag their words with the device epoch counter kept in
// the copy, so they need no clearing.
constexpr int64_t kScratchMaxTokens = 1 << 20;
constexpr size_t kScratchBytes = ws_layout(kScratchMaxTokens).total;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];  // device address of each GPU's copy; set once under the mutex

// The current device's copy of the scratch array, looked up and cleared on the first call.
mrope_status scratch_for_current_device(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return fail(MROPE_ERR_HIP, "mrope_apply_ids_noalloc: no usable current device (%d)", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
            return fail(MROPE_ERR_ARG, "mrope_apply_ids_noalloc: the first call on a device clears its scratch "
                                       "and must not be captured in a graph");
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
        const hipError_t z = launch_workspace_init(ptr, kScratchBytes, stream);
        if (z != hipSuccess) return hip_status(z, "mrope_apply_ids_noalloc scratch clear");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MROPE_OK;
}
}  // namespace

extern "C" {

int mrope_abi_version(void) { return MROPE_ABI_VERSION; }

const char *mrope_status_string(int status)
{
    switch (status) {
    case MROPE_OK: return "ok";
    case MROPE_ERR_ARG: return "invalid argument";
    case MROPE_ERR_ALIGN: return "misaligned pointer or stride";
    case MROPE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MROPE_ERR_WORKSPACE: return "bad workspace";
    case MROPE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *mrope_last_error(void) { return g_last_error; }

int mrope_set_test_hooks(int flags)
{
    const int prev = g_test_hooks.load(std::memory_order_relaxed);
    g_test_hooks.store(flags & (kHookFusedChunked | kHookFusedScanFirst | kHookScanFallback | kHookF32EightLanes),
                       std::memory_order_relaxed);
    return prev;
}

size_t mrope_workspace_bytes(int64_t n_tokens) { return ws_layout(n_tokens).total; }

mrope_status mrope_workspace_init(void *workspace, size_t bytes, void *stream)
{
    if (!workspace) return fail(MROPE_ERR_WORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(MROPE_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (bytes < kWsHeaderBytes || bytes % 8)
        return fail(MROPE_ERR_WORKSPACE, "workspace size must be >= %zu and a multiple of 8", kWsHeaderBytes);
    return hip_status(launch_workspace_init(workspace, bytes, static_cast<hipStream_t>(stream)), "mrope_workspace_init");
}

mrope_status mrope_planes(const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                          int32_t marker_id, int32_t frame_len, const int32_t *frame_len_seq,
                          const int32_t *pos_offset, const int32_t *origin_in, int32_t *planes, int64_t plane_stride, int32_t *start, int32_t *amount, int32_t *origin,
                          int32_t *seq_flags, void *workspace, size_t workspace_bytes, uint32_t epoch, void *stream)
{
    mrope_status st = check_scan(ids, cu_seqlens, n_seqs, n_tokens, planes, plane_stride, workspace, workspace_bytes, true);
    if (st != MROPE_OK) return st;
    if ((st = check_frame_len(frame_len)) != MROPE_OK) return st;
    const Scan sc = make_scan(ids, cu_seqlens, n_seqs, n_tokens, marker_id, frame_len, frame_len_seq, pos_offset, origin_in, planes,
                              plane_stride, start, amount, origin, seq_flags, workspace, epoch);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (n_tokens == 0) {
        if (n_seqs > 0 && any_scalar(sc)) return hip_status(launch_text_scalars(sc, s), "mrope_planes");
        return MROPE_OK;
    }
    return hip_status(launch_planes(sc, s), "mrope_planes");
}

mrope_status mrope_apply(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, void *k,
                         int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads, int64_t n_tokens,
                         int32_t head_dim, int32_t rot_dim, int32_t dtype, const int32_t *planes, int64_t plane_stride,
                         double theta, void *q_out, void *k_out, void *stream)
{
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                                  n_tokens, head_dim, rot_dim, dtype, q_out, k_out);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    if (n_tokens == 0 || n_q_heads + n_k_heads == 0) return MROPE_OK;
    if (!planes) return fail(MROPE_ERR_ARG, "planes is NULL");
    if (plane_stride < n_tokens) return fail(MROPE_ERR_ARG, "plane_stride < n_tokens");
    const Heads h = make_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                               n_tokens, head_dim, q_out, k_out);
    (void)hipGetLastError();
    return hip_status(launch_apply(h, make_rotary(theta), planes, plane_stride, PagedKV{}, dtype,
                                   static_cast<hipStream_t>(stream)),
                      "mrope_apply");
}

mrope_status mrope_apply_kv(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, const void *k,
                            int64_t k_tok_stride, int64_t k_head_stride, int32_t n_kv_heads, const void *v,
                            int64_t v_tok_stride, int64_t v_head_stride, int64_t n_tokens, int32_t head_dim,
                            int32_t rot_dim, int32_t dtype, const int32_t *planes, int64_t plane_stride, double theta,
                            void *k_cache, void *v_cache, const int64_t *slot_mapping, int32_t block_size,
                            int64_t num_blocks, int64_t cache_block_stride, int64_t cache_tok_stride,
                            int64_t cache_head_stride, void *stream)
{
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, const_cast<void *>(k), k_tok_stride,
                                  k_head_stride, n_kv_heads, n_tokens, head_dim, rot_dim, dtype, nullptr, nullptr);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    st = check_paged(n_kv_heads, v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping, block_size, num_blocks,
                     cache_block_stride, cache_tok_stride, cache_head_stride, head_dim, dtype);
    if (st != MROPE_OK) return st;
    if (n_tokens == 0 || n_q_heads + n_kv_heads == 0) return MROPE_OK;
    if (!planes) return fail(MROPE_ERR_ARG, "planes is NULL");
    if (plane_stride < n_tokens) return fail(MROPE_ERR_ARG, "plane_stride < n_tokens");
    const Heads h = make_heads(q, q_tok_stride, q_head_stride, n_q_heads, const_cast<void *>(k), k_tok_stride,
                               k_head_stride, n_kv_heads, n_tokens, head_dim, nullptr, nullptr);
    const PagedKV pc = n_kv_heads > 0 ? make_paged(v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping,
                                                   block_size, num_blocks, cache_block_stride, cache_tok_stride,
                                                   cache_head_stride)
                                      : PagedKV{};
    (void)hipGetLastError();
    return hip_status(launch_apply(h, make_rotary(theta), planes, plane_stride, pc, dtype,
                                   static_cast<hipStream_t>(stream)),
                      "mrope_apply_kv");
}

mrope_status mrope_apply_ids(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, void *k,
                             int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads, int64_t n_tokens,
                             int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta, void *q_out, void *k_out,
                             const int32_t *ids, const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id,
                             int32_t frame_len, const int32_t *frame_len_seq, const int32_t *pos_offset,
                             const int32_t *origin_in,
                             int32_t *planes_out, int64_t plane_stride, int32_t *start, int32_t *amount,
                             int32_t *origin, int32_t *seq_flags, void *workspace, size_t workspace_bytes,
                             uint32_t epoch, void *stream)
{
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                                  n_tokens, head_dim, rot_dim, dtype, q_out, k_out);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    st = check_scan(ids, cu_seqlens, n_seqs, n_tokens, planes_out, plane_stride, workspace, workspace_bytes, false);
    if (st != MROPE_OK) return st;
    if ((st = check_frame_len(frame_len)) != MROPE_OK) return st;
    const Scan sc = make_scan(ids, cu_seqlens, n_seqs, n_tokens, marker_id, frame_len, frame_len_seq, pos_offset, origin_in,
                              planes_out, plane_stride, start, amount, origin, seq_flags, workspace, epoch);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (n_tokens == 0) {
        if (n_seqs > 0 && any_scalar(sc)) return hip_status(launch_text_scalars(sc, s), "mrope_apply_ids");
        return MROPE_OK;
    }
    const Heads h = make_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                               n_tokens, head_dim, q_out, k_out);
    return hip_status(launch_apply_ids(h, make_rotary(theta), sc, PagedKV{}, dtype, s), "mrope_apply_ids");
}

mrope_status mrope_apply_ids_noalloc(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                                     void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads,
                                     int64_t n_tokens, int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta,
                                     void *q_out, void *k_out, const int32_t *ids, const int32_t *cu_seqlens,
                                     int32_t n_seqs, int32_t marker_id, int32_t frame_len,
                                     const int32_t *frame_len_seq, const int32_t *pos_offset, const int32_t *origin_in, int32_t *planes_out, int64_t plane_stride,
                                     int32_t *start, int32_t *amount, int32_t *origin, int32_t *seq_flags,
                                     void *stream)
{
    if (n_tokens > kScratchMaxTokens)
        return fail(MROPE_ERR_WORKSPACE, "mrope_apply_ids_noalloc takes at most %lld tokens (got %lld)",
                    (long long)kScratchMaxTokens, (long long)n_tokens);
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                                  n_tokens, head_dim, rot_dim, dtype, q_out, k_out);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    // the scratch stands in for a workspace of kScratchMaxTokens tokens: checked with a placeholder
    // address here, before anything touches the device
    const uintptr_t placeholder = 256;
    st = check_scan(ids, cu_seqlens, n_seqs, n_tokens, planes_out, plane_stride, reinterpret_cast<void *>(placeholder),
                    kScratchBytes, false);
    if (st != MROPE_OK) return st;
    if ((st = check_frame_len(frame_len)) != MROPE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    void *ws = nullptr;
    if ((st = scratch_for_current_device(s, &ws)) != MROPE_OK) return st;
    // epoch 0: the device counter in the scratch tags each call (graph replays stay distinct)
    const Scan sc = make_scan(ids, cu_seqlens, n_seqs, n_tokens, marker_id, frame_len, frame_len_seq, pos_offset, origin_in,
                              planes_out, plane_stride, start, amount, origin, seq_flags, ws, 0);
    if (n_tokens == 0) {
        if (n_seqs > 0 && any_scalar(sc)) return hip_status(launch_text_scalars(sc, s), "mrope_apply_ids_noalloc");
        return MROPE_OK;
    }
    const Heads h = make_heads(q, q_tok_stride, q_head_stride, n_q_heads, k, k_tok_stride, k_head_stride, n_k_heads,
                               n_tokens, head_dim, q_out, k_out);
    return hip_status(launch_apply_ids(h, make_rotary(theta), sc, PagedKV{}, dtype, s), "mrope_apply_ids_noalloc");
}

mrope_status mrope_apply_ids_kv(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads,
                                const void *k, int64_t k_tok_stride, int64_t k_head_stride, int32_t n_kv_heads,
                                const void *v, int64_t v_tok_stride, int64_t v_head_stride, int64_t n_tokens,
                                int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta, const int32_t *ids,
                                const int32_t *cu_seqlens, int32_t n_seqs, int32_t marker_id, int32_t frame_len,
                                const int32_t *frame_len_seq, const int32_t *pos_offset, const int32_t *origin_in, int32_t *planes_out,
                                int64_t plane_stride, int32_t *start, int32_t *amount, int32_t *origin,
                                int32_t *seq_flags, void *workspace, size_t workspace_bytes, uint32_t epoch,
                                void *k_cache, void *v_cache, const int64_t *slot_mapping, int32_t block_size,
                                int64_t num_blocks, int64_t cache_block_stride, int64_t cache_tok_stride,
                                int64_t cache_head_stride, void *stream)
{
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, const_cast<void *>(k), k_tok_stride,
                                  k_head_stride, n_kv_heads, n_tokens, head_dim, rot_dim, dtype, nullptr, nullptr);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    st = check_paged(n_kv_heads, v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping, block_size, num_blocks,
                     cache_block_stride, cache_tok_stride, cache_head_stride, head_dim, dtype);
    if (st != MROPE_OK) return st;
    st = check_scan(ids, cu_seqlens, n_seqs, n_tokens, planes_out, plane_stride, workspace, workspace_bytes, false);
    if (st != MROPE_OK) return st;
    if ((st = check_frame_len(frame_len)) != MROPE_OK) return st;
    const Scan sc = make_scan(ids, cu_seqlens, n_seqs, n_tokens, marker_id, frame_len, frame_len_seq, pos_offset, origin_in,
                              planes_out, plane_stride, start, amount, origin, seq_flags, workspace, epoch);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (n_tokens == 0) {
        if (n_seqs > 0 && any_scalar(sc)) return hip_status(launch_text_scalars(sc, s), "mrope_apply_ids_kv");
        return MROPE_OK;
    }
    const Heads h = make_heads(q, q_tok_stride, q_head_stride, n_q_heads, const_cast<void *>(k), k_tok_stride,
                               k_head_stride, n_kv_heads, n_tokens, head_dim, nullptr, nullptr);
    const PagedKV pc = n_kv_heads > 0 ? make_paged(v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping,
                                                   block_size, num_blocks, cache_block_stride, cache_tok_stride,
                                                   cache_head_stride)
                                      : PagedKV{};
    return hip_status(launch_apply_ids(h, make_rotary(theta), sc, pc, dtype, s), "mrope_apply_ids_kv");
}

mrope_status mrope_decode(void *q, int64_t q_tok_stride, int64_t q_head_stride, int32_t n_q_heads, const void *k,
                          int64_t k_tok_stride, int64_t k_head_stride, int32_t n_k_heads, const void *v,
                          int64_t v_tok_stride, int64_t v_head_stride, int32_t n_seqs, const int32_t *pos,
                          const int32_t *amount, void *k_cache, void *v_cache, const int64_t *slot_mapping,
                          int32_t block_size, int64_t num_blocks, int64_t cache_block_stride, int64_t cache_tok_stride,
                          int64_t cache_head_stride, int32_t head_dim, int32_t rot_dim, int32_t dtype, double theta,
                          void *stream)
{
    mrope_status st = check_heads(q, q_tok_stride, q_head_stride, n_q_heads, const_cast<void *>(k), k_tok_stride,
                                  k_head_stride, n_k_heads, n_seqs, head_dim, rot_dim, dtype, nullptr, nullptr);
    if (st != MROPE_OK) return st;
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(MROPE_ERR_ARG, "theta must be finite and > 0");
    if (n_seqs < 0) return fail(MROPE_ERR_ARG, "n_seqs < 0");
    st = check_paged(n_k_heads, v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping, block_size, num_blocks,
                     cache_block_stride, cache_tok_stride, cache_head_stride, head_dim, dtype);
    if (st != MROPE_OK) return st;
    if (n_seqs == 0 || n_q_heads + n_k_heads == 0) return MROPE_OK;
    if (!pos || !amount) return fail(MROPE_ERR_ARG, "pos / amount is NULL");
    DecodeArgs d{};
    d.q = q;
    d.k = k;
    d.q_tok = q_tok_stride;
    d.q_head = q_head_stride;
    d.k_tok = k_tok_stride;
    d.k_head = k_head_stride;
    d.nq = n_q_heads;
    d.nk = n_k_heads;
    d.head_dim = head_dim;
    d.n_seqs = n_seqs;
    d.pos = pos;
    d.amount = amount;
    if (n_k_heads > 0)
        d.kv = make_paged(v, v_tok_stride, v_head_stride, k_cache, v_cache, slot_mapping, block_size, num_blocks,
                          cache_block_stride, cache_tok_stride, cache_head_stride);
    (void)hipGetLastError();
    return hip_status(launch_decode(d, make_rotary(theta), dtype, static_cast<hipStream_t>(stream)), "mrope_decode");
}

}  // extern "C"
