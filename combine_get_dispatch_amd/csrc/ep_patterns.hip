// ep_patterns.hip -- measurement utilities: the memory-access patterns of the
// exchange with none of its arithmetic, layout or bookkeeping, so that each
// kernel of the path can be compared with the rate the HBM sustains for the
// pattern it must make, not only with the 8 TB/s peak.
//
//  fill    compact writes: wave w stores bytes [w KB, (w+1) KB), one 128-bit
//          non-temporal store per lane (the best write rate of the chip)
//  read    compact reads: wave w loads 4 KB at w * 4 KB
//  push    the dispatch's pattern: one wave per token loads the token's bf16
//          row, keeps the high byte of each channel (an FP8-sized row) and
//          stores it to each of the token's receive rows
//  gather  the combine's pattern: one wave per (token, 1024-channel pass)
//          loads that pass of the token's k rows, XORs them and stores the
//          pass of the token's output row; optionally at the combine's
//          residency cap (two-wave workgroups, 40 KB of LDS each)
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPushMaxPasses = 8;            // H <= 8192 channels
constexpr size_t kGatherCapLds = 40 * 1024;  // the combine's cap
constexpr int kRsrcWord3 = 0x00020000;       // buffer resource: raw 32-bit data, no swizzle
constexpr int kNonTemporal = 2;              // load cache policy: streaming

__global__ __launch_bounds__(256) void k_pattern_fill(u32x4 *__restrict__ dst, size_t nwaves) {
    const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nwaves) return;
    const uint32_t v = (uint32_t)w;
    __builtin_nontemporal_store(u32x4{v, v, v, v}, dst + w * 64 + (threadIdx.x & 63));
}

__global__ __launch_bounds__(256) void k_pattern_read(const u32x4 *__restrict__ src, size_t nwaves,
                                                      uint32_t *__restrict__ sink) {
    const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nwaves) return;
    const u32x4 *p = src + w * 256 + (threadIdx.x & 63);
    const u32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 64);
    const u32x4 c = __builtin_nontemporal_load(p + 128), d = __builtin_nontemporal_load(p + 192);
    const u32x4 x = a ^ b ^ c ^ d;
    // a value the data never makes in practice: keeps the loads, stores nothing
    if ((x.x ^ x.y ^ x.z ^ x.w) == 0x9E3779B9u) sink[0] = 1u;
}

// high bytes of 16 bf16 channels (two vectors) packed into one vector
__device__ __forceinline__ u32x4 high_bytes(u32x4 a, u32x4 b) {
    auto pack = [](uint32_t lo, uint32_t hi) {
        return (lo >> 8 & 0xFFu) | (lo >> 24 << 8) | (hi >> 8 & 0xFFu) << 16 | (hi >> 24 << 24);
    };
    return u32x4{pack(a.x, a.y), pack(a.z, a.w), pack(b.x, b.y), pack(b.z, b.w)};
}

__global__ __launch_bounds__(256) void k_pattern_push(const uint16_t *__restrict__ x, const int32_t *__restrict__ pos,
                                                      uint8_t *__restrict__ rows, int T, int k, int H,
                                                      int64_t num_rows) {
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const int np = H >> 10;
    int p = lane < k ? pos[(size_t)t * k + lane] : -1;
    if (p >= num_rows) p = -1;
    u32x4 v[kPushMaxPasses];
#pragma unroll
    for (int i = 0; i < kPushMaxPasses; ++i) {
        if (i >= np) break;
        const u32x4 *s = reinterpret_cast<const u32x4 *>(x + (size_t)t * H + i * 1024 + lane * 16);
        v[i] = high_bytes(__builtin_nontemporal_load(s), __builtin_nontemporal_load(s + 1));
    }
    for (int j = 0; j < k; ++j) {
        const int pj = __builtin_amdgcn_readlane(p, j);
        if (pj < 0) continue;
#pragma unroll
        for (int i = 0; i < kPushMaxPasses; ++i) {
            if (i >= np) break;
            __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4 *>(rows + (size_t)pj * H + i * 1024 + lane * 16));
        }
    }
}

template <int WPB>
__global__ __launch_bounds__(WPB * 64) void k_pattern_gather(const uint16_t *__restrict__ rows,
                                                             const int32_t *__restrict__ pos, uint16_t *__restrict__ out,
                                                             int T, int k, int H, int64_t num_rows) {
    const int np = H >> 10;
    const int w = blockIdx.x * WPB + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t = w / np, ps = w - t * np;
    if (t >= T) return;
    int p = lane < k ? pos[(size_t)t * k + lane] : -1;
    if (p >= num_rows) p = -1;
    // each slot's row as a buffer resource (an empty one for an unused slot,
    // which reads zeros without touching memory), so that all loads are
    // issued with no branch between them, as the combine issues them
    u32x4 r0[8], r1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int pj = j < k ? __builtin_amdgcn_readlane(p, j) : -1;
        const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(rows + (size_t)(pj < 0 ? 0 : pj) * H), 0, pj >= 0 ? H * 2 : 0, kRsrcWord3);
        const int off = (ps * 1024 + lane * 8) * 2;
        r0[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(row, off, 0, kNonTemporal));
        r1[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(row, off + 1024, 0, kNonTemporal));
    }
    u32x4 a = r0[0], b = r1[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        a ^= r0[j];
        b ^= r1[j];
    }
    u32x4 *d = reinterpret_cast<u32x4 *>(out + (size_t)t * H + ps * 1024 + lane * 8);
    __builtin_nontemporal_store(a, d);
    __builtin_nontemporal_store(b, d + 64);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP; }

}  // namespace

extern "C" {

int ep_pattern_fill(void *dst, size_t bytes, ep_stream_t stream) {
    if (bytes == 0) return EP_OK;
    if (!dst || bytes % 1024) return EP_ERR_ARG;
    if (!aligned16(dst)) return EP_ERR_ALIGN;
    const size_t nwaves = bytes / 1024;
    hipLaunchKernelGGL(k_pattern_fill, dim3((unsigned)((nwaves + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       static_cast<u32x4 *>(dst), nwaves);
    return launched();
}

int ep_pattern_read(const void *src, size_t bytes, uint32_t *sink, ep_stream_t stream) {
    if (bytes == 0) return EP_OK;
    if (!src || !sink || bytes % 4096) return EP_ERR_ARG;
    if (!aligned16(src)) return EP_ERR_ALIGN;
    const size_t nwaves = bytes / 4096;
    hipLaunchKernelGGL(k_pattern_read, dim3((unsigned)((nwaves + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(src), nwaves, sink);
    return launched();
}

int ep_pattern_push(const uint16_t *x, const int32_t *pos, void *rows, int num_tokens, int num_topk, int hidden,
                    int64_t num_rows, ep_stream_t stream) {
    if (num_tokens == 0) return EP_OK;
    if (!x || !pos || !rows || num_tokens < 0 || num_topk < 1 || num_topk > 64 || hidden < 1024 ||
        hidden % 1024 || hidden > 1024 * kPushMaxPasses || num_rows < 0)
        return EP_ERR_ARG;
    if (!aligned16(x) || !aligned16(rows)) return EP_ERR_ALIGN;
    hipLaunchKernelGGL(k_pattern_push, dim3((unsigned)((num_tokens + 3) / 4)), dim3(256), 0, (hipStream_t)stream, x,
                       pos, static_cast<uint8_t *>(rows), num_tokens, num_topk, hidden, num_rows);
    return launched();
}

int ep_pattern_gather(const uint16_t *rows, const int32_t *pos, uint16_t *out, int num_tokens, int num_topk,
                      int hidden, int64_t num_rows, int capped, ep_stream_t stream) {
    if (num_tokens == 0) return EP_OK;
    if (!rows || !pos || !out || num_tokens < 0 || num_topk < 1 || num_topk > 8 || hidden < 1024 ||
        hidden % 1024 || num_rows < 0)
        return EP_ERR_ARG;
    if (!aligned16(rows) || !aligned16(out)) return EP_ERR_ALIGN;
    const size_t nwaves = (size_t)num_tokens * (hidden / 1024);
    if (nwaves >= ((size_t)1 << 31)) return EP_ERR_ARG;
    if (capped)
        hipLaunchKernelGGL(k_pattern_gather<2>, dim3((unsigned)((nwaves + 1) / 2)), dim3(128), kGatherCapLds,
                           (hipStream_t)stream, rows, pos, out, num_tokens, num_topk, hidden, num_rows);
    else
        hipLaunchKernelGGL(k_pattern_gather<4>, dim3((unsigned)((nwaves + 3) / 4)), dim3(256), 0,
                           (hipStream_t)stream, rows, pos, out, num_tokens, num_topk, hidden, num_rows);
    return launched();
}

}  // extern "C"
