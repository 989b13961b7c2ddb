// Memory-pattern reference kernels for `bench.py --mode pattern` (not part of libmrope).
//
// The in-place rotary reads and writes the first 128 bytes (64 bf16 dims) of every 512-byte head,
// ten heads a token, and nothing else.  These kernels move exactly those bytes with no rotary
// arithmetic -- reads only, writes only, and both in place -- plus dense reads, writes and copies of
// the same byte count, so the rotary kernels' times can be set against what the memory system
// sustains for their access pattern on the same chip.  Same lane map as the rotary kernels: eight
// lanes a token, lane l on bytes [16 l, 16 l + 16) of each head; non-temporal loads and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256;
constexpr int kHeads = 10;
constexpr int kHeadVec = 32;   // 16-byte vectors per 512-byte head
constexpr int kDenseVec = 4;   // 16-byte vectors per thread in the dense kernels

__device__ __forceinline__ const u32x4 *token_base(const u32x4 *buf, int64_t t, int l)
{
    return buf + t * kHeads * kHeadVec + l;
}

__global__ __launch_bounds__(kBlock) void sparse_read(const u32x4 *buf, int64_t tokens, uint32_t magic, uint32_t *sink)
{
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 8) + (threadIdx.x >> 3);
    if (t >= tokens) return;
    const u32x4 *p = token_base(buf, t, threadIdx.x & 7);
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < kHeads; ++h) acc ^= __builtin_nontemporal_load(p + h * kHeadVec);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == magic) sink[threadIdx.x & 63] = 1u;  // keeps the loads
}

__global__ __launch_bounds__(kBlock) void sparse_write(u32x4 *buf, int64_t tokens, uint32_t magic)
{
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 8) + (threadIdx.x >> 3);
    if (t >= tokens) return;
    u32x4 *p = const_cast<u32x4 *>(token_base(buf, t, threadIdx.x & 7));
    const u32x4 v = {magic, (uint32_t)t, magic, (uint32_t)t};
#pragma unroll
    for (int h = 0; h < kHeads; ++h) __builtin_nontemporal_store(v, p + h * kHeadVec);
}

__global__ __launch_bounds__(kBlock) void sparse_rw(u32x4 *buf, int64_t tokens, uint32_t magic)
{
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 8) + (threadIdx.x >> 3);
    if (t >= tokens) return;
    u32x4 *p = const_cast<u32x4 *>(token_base(buf, t, threadIdx.x & 7));
    u32x4 v[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) v[h] = __builtin_nontemporal_load(p + h * kHeadVec);
    const u32x4 m = {magic, magic, magic, magic};
#pragma unroll
    for (int h = 0; h < kHeads; ++h) __builtin_nontemporal_store(v[h] ^ m, p + h * kHeadVec);
}

__global__ __launch_bounds__(kBlock) void dense_read(const u32x4 *src, int64_t n, uint32_t magic, uint32_t *sink)
{
    const int64_t base = (int64_t)blockIdx.x * kBlock * kDenseVec + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kDenseVec; ++j)
        if (base + j * kBlock < n) acc ^= __builtin_nontemporal_load(src + base + j * kBlock);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == magic) sink[threadIdx.x & 63] = 1u;
}

__global__ __launch_bounds__(kBlock) void dense_write(u32x4 *dst, int64_t n, uint32_t magic)
{
    const int64_t base = (int64_t)blockIdx.x * kBlock * kDenseVec + threadIdx.x;
    const u32x4 v = {magic, (uint32_t)base, magic, (uint32_t)base};
#pragma unroll
    for (int j = 0; j < kDenseVec; ++j)
        if (base + j * kBlock < n) __builtin_nontemporal_store(v, dst + base + j * kBlock);
}

__global__ __launch_bounds__(kBlock) void dense_copy(const u32x4 *src, u32x4 *dst, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kBlock * kDenseVec + threadIdx.x;
    u32x4 v[kDenseVec];
#pragma unroll
    for (int j = 0; j < kDenseVec; ++j)
        if (base + j * kBlock < n) v[j] = __builtin_nontemporal_load(src + base + j * kBlock);
#pragma unroll
    for (int j = 0; j < kDenseVec; ++j)
        if (base + j * kBlock < n) __builtin_nontemporal_store(v[j], dst + base + j * kBlock);
}

// The same in-place pattern with another lane map: eight lanes on one 128-byte (token, head) piece,
// eight pieces -- consecutive in (token, head) order -- per single-wave workgroup.  Of the lane maps
// and occupancies tried for a plain read + write pass over the pattern, this one streams fastest.
__global__ __launch_bounds__(64) void sparse_rw_pieces(u32x4 *buf, int64_t pieces, uint32_t magic)
{
    const int64_t c = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 3);
    if (c >= pieces) return;
    u32x4 *p = buf + (c / kHeads) * kHeads * kHeadVec + (c % kHeads) * kHeadVec + (threadIdx.x & 7);
    const u32x4 v = __builtin_nontemporal_load(p);
    const u32x4 m = {magic, magic, magic, magic};
    __builtin_nontemporal_store(v ^ m, p);
}

// Dense copy with one 16-byte vector per lane.
__global__ __launch_bounds__(kBlock) void dense_copy_v1(const u32x4 *src, u32x4 *dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

// kind: 0 sparse read, 1 sparse write, 2 sparse read + write in place (a: [n tokens][10][512 B]);
//       3 dense read of a, 4 dense write of a, 5 dense copy a -> b (n bytes, a multiple of 16);
//       6 as 2 with a (token, head) piece per eight lanes and single-wave workgroups;
//       7 as 5 with one 16-byte vector per lane.
// sink: 64 words of device memory the read kernels may write.  Returns a hipError_t.
extern "C" int pattern_launch(int kind, void *a, void *b, int64_t n, uint32_t magic, void *sink, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n <= 0 || !a) return (int)hipErrorInvalidValue;
    if (kind < 0 || kind > 7) return (int)hipErrorInvalidValue;
    if (kind <= 2) {
        const unsigned blocks = (unsigned)((n + kBlock / 8 - 1) / (kBlock / 8));
        u32x4 *p = static_cast<u32x4 *>(a);
        if (kind == 0) sparse_read<<<blocks, kBlock, 0, s>>>(p, n, magic, static_cast<uint32_t *>(sink));
        if (kind == 1) sparse_write<<<blocks, kBlock, 0, s>>>(p, n, magic);
        if (kind == 2) sparse_rw<<<blocks, kBlock, 0, s>>>(p, n, magic);
    } else if (kind == 6) {
        const int64_t pieces = n * kHeads;
        sparse_rw_pieces<<<(unsigned)((pieces + 7) / 8), 64, 0, s>>>(static_cast<u32x4 *>(a), pieces, magic);
    } else {
        if (n % 16) return (int)hipErrorInvalidValue;
        const int64_t v = n / 16;
        const unsigned blocks = (unsigned)((v + kBlock * kDenseVec - 1) / (kBlock * kDenseVec));
        u32x4 *p = static_cast<u32x4 *>(a);
        if (kind == 3) dense_read<<<blocks, kBlock, 0, s>>>(p, v, magic, static_cast<uint32_t *>(sink));
        if (kind == 4) dense_write<<<blocks, kBlock, 0, s>>>(p, v, magic);
        if (kind == 5 || kind == 7) {
            if (!b) return (int)hipErrorInvalidValue;
            if (kind == 5) dense_copy<<<blocks, kBlock, 0, s>>>(p, static_cast<u32x4 *>(b), v);
            else dense_copy_v1<<<(unsigned)((v + kBlock - 1) / kBlock), kBlock, 0, s>>>(p, static_cast<u32x4 *>(b), v);
        }
    }
    return (int)hipGetLastError();
}
