// Device twin of the seeded input generator in gen.c: same definition, same
// bits for the same (seed, stream, index).  Holds no arithmetic of the
// optimizer step; it only fills input buffers on the GPU so that large
// workloads need no host mirror.  Built with -ffp-contract=off: the fp32
// operations below must round exactly as the host's SSE operations do.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

namespace {

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

__host__ __device__ __forceinline__ uint64_t key_of(uint64_t seed, uint64_t stream)
{
    return mix64(seed ^ mix64(stream + GOLDEN));
}

__device__ __forceinline__ float unif(uint64_t key, uint64_t c)
{
    uint64_t b = mix64(key + c * GOLDEN);
    return (float)(uint32_t)(b >> 40) * 0x1p-24f;
}

__device__ __forceinline__ float value_at(uint64_t key, uint64_t mkey, uint64_t i, float scale,
                                          float frac, float mult)
{
    float u0 = unif(key, 4 * i + 0);
    float u1 = unif(key, 4 * i + 1);
    float u2 = unif(key, 4 * i + 2);
    float u3 = unif(key, 4 * i + 3);
    float s = (u0 + u1) + (u2 + u3);
    float x = (s - 2.0f) * scale;
    if (frac > 0.0f && unif(mkey, i) < frac)
        x = x * mult;
    return x;
}

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ void fill_f32_kernel(float *out, uint64_t key, uint64_t mkey, int64_t start, int64_t count,
                                float scale, float frac, float mult)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
         j += (int64_t)gridDim.x * blockDim.x)
        out[j] = value_at(key, mkey, (uint64_t)(start + j), scale, frac, mult);
}

__global__ void fill_bf16_kernel(uint16_t *out, uint64_t key, uint64_t mkey, int64_t start,
                                 int64_t count, float scale, float frac, float mult)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
         j += (int64_t)gridDim.x * blockDim.x)
        out[j] = to_bf16(value_at(key, mkey, (uint64_t)(start + j), scale, frac, mult));
}

// dst[j] = prefix[src(start + j)], src(i) = i below plen, else
// mix64(key + i * GOLDEN) mod plen.
__global__ void spread_kernel(float *dst, const float *prefix, int64_t plen, uint64_t key,
                              int64_t start, int64_t count)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
         j += (int64_t)gridDim.x * blockDim.x) {
        uint64_t i = (uint64_t)(start + j);
        uint64_t src = i < (uint64_t)plen ? i : mix64(key + i * GOLDEN) % (uint64_t)plen;
        dst[j] = prefix[src];
    }
}

int grid_for(int64_t count)
{
    int64_t b = (count + 255) / 256;
    if (b > 256 * 32) b = 256 * 32;
    return b < 1 ? 1 : (int)b;
}

}  // namespace

extern "C" {

int synth_dev_fill_f32(float *out, uint64_t seed, uint64_t stream, int64_t start, int64_t count,
                       float scale, uint64_t mask_stream, float frac, float mult, hipStream_t s)
{
    if (count <= 0)
        return 0;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(count)), dim3(256), 0, s, out,
                       key_of(seed, stream), key_of(seed, mask_stream), start, count, scale, frac, mult);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_dev_fill_bf16(uint16_t *out, uint64_t seed, uint64_t stream, int64_t start, int64_t count,
                        float scale, uint64_t mask_stream, float frac, float mult, hipStream_t s)
{
    if (count <= 0)
        return 0;
    hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(count)), dim3(256), 0, s, out,
                       key_of(seed, stream), key_of(seed, mask_stream), start, count, scale, frac, mult);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_dev_spread(float *dst, const float *prefix, int64_t plen, uint64_t seed, uint64_t stream,
                     int64_t start, int64_t count, hipStream_t s)
{
    if (count <= 0)
        return 0;
    if (plen <= 0)
        return 1;
    hipLaunchKernelGGL(spread_kernel, dim3(grid_for(count)), dim3(256), 0, s, dst, prefix, plen,
                       key_of(seed, stream), start, count);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
