// Internal interface between the host API (zero_api.cpp) and the kernels
// (zero_kernels.hip).  Not installed; the public ABI is include/zero_shard.h.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "zero_shard.h"

namespace zs {

// Step constants, each formed once on the host in double (see
// make_scalars in zero_api.cpp); the kernels only combine them.
struct StepScalars {
    double b1, c1;     // beta1, 1 - beta1
    double b2, c2;     // beta2, 1 - beta2
    double bc1, bc2;   // 1 - beta1^t, 1 - beta2^t
    double eps, lr;
    double dec;        // 1 - lr * weight_decay
    double wd;         // weight_decay
};
static_assert(sizeof(StepScalars) == sizeof(zero_step_consts), "step constants layout");
static_assert(offsetof(StepScalars, bc1) == offsetof(zero_step_consts, bc1), "step constants layout");
static_assert(offsetof(StepScalars, wd) == offsetof(zero_step_consts, wd), "step constants layout");

// Reduction constants: divide by the count (N, or N * micro-batches), or
// multiply by its inverse when the count is a power of two (exact scaling,
// so the same bits as the division).  group: ranks per group of the
// two-level order (n_ranks for the flat order).
struct ReduceScalars {
    double n;
    double inv_n;
    int pow2;
    int n_ranks;
    int group;
};

struct PartialPtrs {
    const void *p[ZERO_MAX_RANKS];
};

struct StepArgs {
    PartialPtrs parts;
    ReduceScalars red;
    StepScalars k;
    float *master, *m, *v;
    const zero_chunk *chunks;
    int64_t n_chunks;
    int64_t shard_len;
    const float *acc;   // extended step: earlier micro-batches' sum, or null
    uint16_t *comp;     // pure-bf16 step: Kahan compensation (bf16), or null
    const zero_step_consts *sched;   // scheduled step: constants table, its
    const int64_t *sched_index;      // entry index and entry count
    int64_t n_sched;
};

struct ReduceArgs {
    PartialPtrs parts;
    ReduceScalars red;
    float *out;
    int64_t n;
};

struct AccArgs {
    PartialPtrs parts;
    ReduceScalars red;
    float *acc;
    int64_t n;
    int reset;
};

struct AdamArgs {
    StepScalars k;
    const float *g;
    float *master, *m, *v;
    int64_t n;
};

struct GatherArgs {
    const float *master;
    const zero_chunk *chunks;
    int64_t n_chunks;
    int64_t shard_len;
};

hipError_t launch_step(const StepArgs &a, zero_dtype gdt, hipStream_t s);
// The state layouts of the fused steps (which arrays master/m/v/comp are).
enum class StateLayout { Fp32, Bf16Moments, Kahan };

hipError_t launch_step_sched(const StepArgs &a, zero_dtype gdt, StateLayout layout, hipStream_t s);
hipError_t launch_index_advance(int64_t *index, int64_t n, hipStream_t s);
hipError_t launch_step_ex(const StepArgs &a, zero_dtype gdt, hipStream_t s);
hipError_t launch_step_m16(const StepArgs &a, zero_dtype gdt, hipStream_t s);
hipError_t launch_step_kahan(const StepArgs &a, zero_dtype gdt, hipStream_t s);
hipError_t launch_accumulate(const AccArgs &a, zero_dtype gdt, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs &a, zero_dtype gdt, hipStream_t s);
hipError_t launch_adamw(const AdamArgs &a, hipStream_t s);
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);
hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s);
hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, uint32_t magic,
                             hipStream_t s);
hipError_t launch_probe_write(void *dst, int64_t bytes, uint32_t value, hipStream_t s);
hipError_t launch_probe_sum(const float *const *src, int k, float *dst, int64_t n, hipStream_t s);

}  // namespace zs
