// Internal launch interface between the C ABI (mrope_abi.hip) and the kernels (mrope_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mrope {

constexpr int kMaxHeads = 64;
constexpr int kDefaultFrameLen = 67;    // <image>, 64 rows, </image>, "\n"
constexpr int kMaxFrameLen = 4096;
constexpr int kChunkTokens = 512;       // tokens per scan chunk: one wave, eight 64-id ballots
constexpr int kPartTokens = 32;         // tokens per rotation workgroup of the scan-first fused kernel
constexpr size_t kWsHeaderBytes = 256;  // device epoch counter (+ padding)

// Workspace of the plane-deriving calls (byte offsets; every region 256-byte aligned):
//   header   the device epoch counter
//   status   one 64-bit look-back word per 512-token chunk
//   parts    three 64-bit words per 32-token part: the planes handover of the scan-first fused kernel
//   tagged   three 64-bit words per token: planes of parts that hold more than one sequence
struct WsLayout {
    size_t status, parts, tagged, total;
};

constexpr size_t ws_round(size_t b) { return (b + 255) / 256 * 256; }

constexpr WsLayout ws_layout(int64_t n_tokens)
{
    if (n_tokens < 0) n_tokens = 0;
    const size_t chunks = (size_t)((n_tokens + kChunkTokens - 1) / kChunkTokens);
    const size_t parts = (size_t)((n_tokens + kPartTokens - 1) / kPartTokens);
    WsLayout w{};
    w.status = kWsHeaderBytes;
    w.parts = w.status + ws_round(chunks * 8);
    w.tagged = w.parts + ws_round(parts * 24);
    w.total = w.tagged + ws_round((size_t)n_tokens * 24);
    return w;
}

// Rotary constants: 32 fp32 inverse frequencies and the plane each frequency reads, 2 bits per
// frequency (0 = T, 1 = H, 2 = W).
struct Rotary {
    float inv_freq[32];
    uint64_t plane_sel;
};

// Q/K heads of one call.  Element (t, h, d) of q is at q + t*q_tok + h*q_head + d (elements).
struct Heads {
    void *q;
    void *k;
    void *q_out;   // nullptr: in place
    void *k_out;
    int64_t q_tok, q_head, k_tok, k_head;
    int32_t nq, nk;
    int32_t head_dim;
    int64_t n_tokens;
};

// Plane derivation: ids + packed sequences -> planes / scalars through a workspace.
struct Scan {
    const int32_t *ids;
    const int32_t *cu;
    int32_t n_seqs;
    int32_t marker;
    int64_t n_tokens;
    int32_t *planes;     // nullable in the fused kernel
    int64_t plane_stride;
    int32_t *start;      // nullable
    int32_t *amount;     // nullable
    int32_t *origin;     // nullable
    int32_t *flags;      // nullable
    const int32_t *pos_offset;  // nullable: position of each sequence's first token here (0)
    const int32_t *origin_in;   // nullable: origin found in earlier pieces, -1 = none
    int32_t frame_len;          // tokens from <image> to start (65 .. kMaxFrameLen)
    const int32_t *frame_lens;  // nullable: per-sequence frame length (0 or out of range: frame_len)
    void *workspace;
    uint64_t *parts;     // workspace regions (see WsLayout); set by the host from n_tokens
    uint64_t *tagged;
    uint32_t epoch;      // tags this launch's status words; 0 = use (and advance) the device counter
};

// Test and tuning hooks (mrope_set_test_hooks): which fused kernel serves mrope_apply_ids, a mode
// that makes the scan-first kernel's rotation workgroups derive their planes themselves, and the
// lane layout of mrope_apply in fp32.
constexpr int kHookFusedChunked = 1;   // always the chunk-per-workgroup fused kernel
constexpr int kHookFusedScanFirst = 2; // always the scan-first fused kernel (8 Q + 2 K heads)
constexpr int kHookScanFallback = 4;   // scan-first: rotation workgroups first, no waiting
constexpr int kHookF32EightLanes = 8;  // fp32: the eight-lane (or generic cache-writing) kernels, not sixteen lanes
int test_hooks();

// Paged K/V cache destination.  Element (block, row, head, d) of either cache is at
// block*c_block + row*c_tok + head*c_head + d; slot -> (slot / block_size, slot % block_size).
struct PagedKV {
    void *k_cache;          // nullptr: no cache write
    void *v_cache;          // nullptr together with v
    const void *v;          // new V heads, element (t, h, d) at t*v_tok + h*v_head + d
    int64_t v_tok, v_head;
    const int64_t *slots;   // one per token (prefill) or per sequence (decode)
    int64_t num_slots;      // num_blocks * block_size; slots outside [0, num_slots) are skipped
    int64_t c_block, c_tok, c_head;
    int32_t block_size;
    int32_t bs_shift;       // log2(block_size) when it is a power of two, else -1
};

struct DecodeArgs {
    void *q;
    const void *k;
    int64_t q_tok, q_head, k_tok, k_head;
    int32_t nq, nk, head_dim;
    int32_t n_seqs;
    const int32_t *pos;
    const int32_t *amount;
    PagedKV kv;
};

hipError_t launch_workspace_init(void *ws, size_t bytes, hipStream_t stream);
hipError_t launch_text_scalars(const Scan &s, hipStream_t stream);
hipError_t launch_planes(const Scan &s, hipStream_t stream);
// io: the C ABI's dtype code (0 fp32, 1 bf16, 2 fp16)
// kv.k_cache == nullptr: K rotated in place (or into k_out); else K and V go to the paged caches.
hipError_t launch_apply(const Heads &h, const Rotary &r, const int32_t *planes, int64_t plane_stride,
                        const PagedKV &kv, int io, hipStream_t stream);
hipError_t launch_apply_ids(const Heads &h, const Rotary &r, const Scan &s, const PagedKV &kv, int io,
                            hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &d, const Rotary &r, int io, hipStream_t stream);

}  // namespace mrope
