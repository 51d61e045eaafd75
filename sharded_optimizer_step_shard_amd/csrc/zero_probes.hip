// Measurement kernels (not part of the step): plain read, write and copy
// streams over a byte range, the attainable HBM rates that the step's rate
// is compared with, and the known-size traffic that calibrates hardware
// counters.  Kept apart from the step kernels so that editing a probe does
// not change the step's sources.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

namespace zs {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

template <typename T>
__device__ __forceinline__ T ld(const T *p) { return *p; }

template <typename T>
__device__ __forceinline__ void st_nt(T *p, T x) { __builtin_nontemporal_store(x, p); }

// Copy stream (also the known-size traffic that calibrates the HBM
// counters): one wave per SIMD; wave b copies 8 KiB pieces b, b + gridDim.x,
// ... with 8 non-temporal 16-byte loads in flight per lane, then their 8
// non-temporal stores.  Measured on MI355X: 5.4 TB/s (read plus written)
// against 5.0 for one plain load and store per lane in 256-lane workgroups.
// The bytes past the last full word are copied element by element.
constexpr int kCopyLanes = 64;
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopyPiece = kCopyLanes * kCopyUnroll;   // 16-byte words per piece

__global__ __launch_bounds__(kCopyLanes) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_copy_kernel(const u32x4 *src, u32x4 *dst, int64_t n16, const uint8_t *src_b,
                       uint8_t *dst_b, int64_t bytes)
{
    for (int64_t p = blockIdx.x; p * kCopyPiece < n16; p += gridDim.x) {
        u32x4 r[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = p * kCopyPiece + u * kCopyLanes + threadIdx.x;
            r[u] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = p * kCopyPiece + u * kCopyLanes + threadIdx.x;
            if (i < n16)
                st_nt(dst + i, r[u]);
        }
    }
    if (blockIdx.x == 0) {
        const int64_t b = n16 * 16 + threadIdx.x;
        if (b < bytes)
            dst_b[b] = src_b[b];
    }
}

// Read-only stream: one wave per SIMD; wave b reads 8 KiB pieces b,
// b + gridDim.x, ... with 8 non-temporal 16-byte loads in flight per lane,
// folding them by XOR into a value that is stored only if it equals
// `magic`, so the loads cannot be dropped and in practice nothing is
// written.  Of the shapes measured on MI355X (one or 4-8 loads per lane,
// plain or non-temporal, 64- or 256-lane workgroups, 1K-1M workgroups)
// this one sustained the highest rate: 7.3 TB/s against 6.6 for one plain
// load per lane in 256-lane workgroups.
constexpr int kReadLanes = 64;
constexpr int kReadUnroll = 8;
constexpr int64_t kReadPiece = kReadLanes * kReadUnroll;   // 16-byte words per piece

__global__ __launch_bounds__(kReadLanes) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_read_kernel(const u32x4 *src, int64_t n16, const uint8_t *src_b, int64_t bytes,
                       uint32_t *sink, uint32_t magic)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t p = blockIdx.x; p * kReadPiece < n16; p += gridDim.x) {
        u32x4 r[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = p * kReadPiece + u * kReadLanes + threadIdx.x;
            r[u] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            acc ^= r[u];
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (blockIdx.x == 0) {
        const int64_t b = n16 * 16 + threadIdx.x;
        if (b < bytes)
            x ^= src_b[b];
    }
    if (x == magic)
        sink[0] = x;
}

constexpr int64_t kWritePiece = kBlock;     // 16-byte words per piece (4 KiB)

// Write-only stream: workgroup b writes 4 KiB pieces b, b + gridDim.x, ...
// with one non-temporal 16-byte store per lane (the store the step kernels
// use for their state), the bytes past the last full word element by
// element.  The value written is `value` in every 32-bit word.
__global__ __launch_bounds__(kBlock) void probe_write_kernel(u32x4 *dst, int64_t n16,
                                                             uint8_t *dst_b, int64_t bytes,
                                                             uint32_t value)
{
    const u32x4 w = {value, value, value, value};
    for (int64_t p = blockIdx.x; p * kWritePiece < n16; p += gridDim.x) {
        const int64_t i = p * kWritePiece + threadIdx.x;
        if (i < n16)
            st_nt(dst + i, w);
    }
    if (blockIdx.x == 0) {
        const int64_t b = n16 * 16 + threadIdx.x;
        if (b < bytes)
            dst_b[b] = (uint8_t)value;
    }
}

// Sum streams: dst = src[0] + src[1] + ... + src[K-1] in fp32, added in that
// order.  One 64-lane workgroup per 1 KiB lane group of dst (one-shot waves
// up to 4M workgroups, a loop beyond; no occupancy cap), one non-temporal
// 16-byte load per source and one non-temporal 16-byte store per lane; the
// floats past the last full 16-byte word are summed element by element by
// the first workgroup.  With K = 1 it is a copy.  Measured on MI355X in this
// shape, 1 GiB fp32 arrays: copy, 2:1 and 3:1 streams at 0.77-0.85 of the
// 8 TB/s peak, against 0.57-0.73 for the same streams from the vendor's
// kernels; 16 sources at 0.72-0.73.
constexpr int kSumLanes = 64;
constexpr int64_t kSumMaxGroups = int64_t(1) << 22;

struct SumSources {
    const f32x4 *p[ZERO_PROBE_SUM_MAX];
};

template <int K>
__global__ __launch_bounds__(kSumLanes) void probe_sum_kernel(SumSources s, f32x4 *dst, int64_t n4,
                                                             float *dst_f, int64_t n)
{
    for (int64_t g = blockIdx.x; g * kSumLanes < n4; g += gridDim.x) {
        const int64_t i = g * kSumLanes + threadIdx.x;
        if (i < n4) {
            f32x4 x[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                x[k] = __builtin_nontemporal_load(s.p[k] + i);
            f32x4 acc = x[0];
#pragma unroll
            for (int k = 1; k < K; ++k)
                acc += x[k];
            st_nt(dst + i, acc);
        }
    }
    if (blockIdx.x == 0) {
        const int64_t j = n4 * 4 + threadIdx.x;
        if (j < n) {
            float acc = ((const float *)s.p[0])[j];
#pragma unroll
            for (int k = 1; k < K; ++k)
                acc += ((const float *)s.p[k])[j];
            dst_f[j] = acc;
        }
    }
}

}  // namespace

hipError_t launch_probe_sum(const float *const *src, int k, float *dst, int64_t n, hipStream_t s)
{
    SumSources ss{};
    for (int j = 0; j < k; ++j)
        ss.p[j] = (const f32x4 *)src[j];
    const int64_t n4 = n / 4;
    int64_t groups = (n4 + kSumLanes - 1) / kSumLanes;
    if (groups > kSumMaxGroups)
        groups = kSumMaxGroups;
    if (groups < 1)
        groups = 1;
    const dim3 grid((unsigned)groups), block(kSumLanes);
    f32x4 *d4 = (f32x4 *)dst;
    switch (k) {
#define ZS_SUM_CASE(K) \
    case K: hipLaunchKernelGGL(probe_sum_kernel<K>, grid, block, 0, s, ss, d4, n4, dst, n); break;
    ZS_SUM_CASE(1) ZS_SUM_CASE(2) ZS_SUM_CASE(3) ZS_SUM_CASE(4)
    ZS_SUM_CASE(5) ZS_SUM_CASE(6) ZS_SUM_CASE(7) ZS_SUM_CASE(8)
    ZS_SUM_CASE(9) ZS_SUM_CASE(10) ZS_SUM_CASE(11) ZS_SUM_CASE(12)
    ZS_SUM_CASE(13) ZS_SUM_CASE(14) ZS_SUM_CASE(15) ZS_SUM_CASE(16)
#undef ZS_SUM_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    int64_t pieces = (n16 + kCopyPiece - 1) / kCopyPiece;
    if (pieces > 65536)
        pieces = 65536;
    if (pieces < 1)
        pieces = 1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3((int)pieces), dim3(kCopyLanes), 0, s,
                       (const u32x4 *)src, (u32x4 *)dst, n16, (const uint8_t *)src, (uint8_t *)dst,
                       bytes);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, uint32_t magic,
                             hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    int64_t pieces = (n16 + kReadPiece - 1) / kReadPiece;
    if (pieces > 65536)
        pieces = 65536;
    if (pieces < 1)
        pieces = 1;
    hipLaunchKernelGGL(probe_read_kernel, dim3((int)pieces), dim3(kReadLanes), 0, s,
                       (const u32x4 *)src, n16, (const uint8_t *)src, bytes, sink, magic);
    return hipGetLastError();
}

hipError_t launch_probe_write(void *dst, int64_t bytes, uint32_t value, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    int64_t pieces = (n16 + kWritePiece - 1) / kWritePiece;
    if (pieces > (1 << 20))
        pieces = 1 << 20;
    if (pieces < 1)
        pieces = 1;
    hipLaunchKernelGGL(probe_write_kernel, dim3((int)pieces), dim3(kBlock), 0, s, (u32x4 *)dst, n16,
                       (uint8_t *)dst, bytes, value);
    return hipGetLastError();
}

}  // namespace zs
