// Host side of libzero_shard.so: argument checks, step constants, the chunk
// table builder and the C entry points declared in include/zero_shard.h.
// Nothing here allocates device memory or keeps global state.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_internal.h"

using namespace zs;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A count outside [0, ZERO_MAX_LEN]; below the limit count * 8 fits int64.
bool bad_len(int64_t n) { return n < 0 || n > ZERO_MAX_LEN; }

// [a, a + na) and [b, b + nb) (bytes) overlap?
bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (na <= 0 || nb <= 0)
        return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

bool valid_hparams(const zero_adamw_hparams *hp)
{
    if (!hp || hp->step < 1)
        return false;
    if (!isfinite(hp->lr) || !isfinite(hp->eps) || !isfinite(hp->weight_decay))
        return false;
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return false;
    return true;
}

// Every step constant is formed here once, in double, by the same
// operations the element-wise definition uses.
StepScalars make_scalars(const zero_adamw_hparams *hp)
{
    StepScalars k;
    k.b1 = hp->beta1;
    k.c1 = 1.0 - hp->beta1;
    k.b2 = hp->beta2;
    k.c2 = 1.0 - hp->beta2;
    k.bc1 = 1.0 - pow(hp->beta1, (double)hp->step);
    k.bc2 = 1.0 - pow(hp->beta2, (double)hp->step);
    k.eps = hp->eps;
    k.lr = hp->lr;
    k.dec = 1.0 - hp->lr * hp->weight_decay;
    k.wd = hp->weight_decay;
    return k;
}

// count = N * micro_batches, the number of gradients the mean runs over.
ReduceScalars make_reduce(int n_ranks, int group = 0, int64_t micro_batches = 1)
{
    ReduceScalars r;
    const int64_t count = (int64_t)n_ranks * micro_batches;
    r.n_ranks = n_ranks;
    r.group = group > 0 ? group : n_ranks;
    r.n = (double)count;
    r.pow2 = (count & (count - 1)) == 0;
    r.inv_n = 1.0 / r.n;   // exact when the count is a power of two
    return r;
}

// Two-level order and accumulation arguments: group divides n_ranks
// (0 = one group); micro_batches >= 1; acc given exactly when there are
// earlier micro-batches.
bool valid_reduce_spec(const zero_reduce_spec *rs, int n_ranks)
{
    if (!rs)
        return false;
    if (rs->group < 0 || rs->group > n_ranks || (rs->group > 0 && n_ranks % rs->group != 0))
        return false;
    if (rs->micro_batches < 1 || (int64_t)rs->micro_batches * n_ranks > (int64_t(1) << 40))
        return false;
    return (rs->micro_batches > 1) == (rs->acc != nullptr);
}

int elem_bytes(int gdt) { return gdt == ZERO_BF16 ? 2 : 4; }   // after valid_dtype

// The INVALID checks of the partial list (null list, rank count, null
// partial); fills pp.  With n == 0 nothing is dereferenced, so null partial
// addresses are accepted (empty tensors).  Alignment and dtype are checked
// by the callers after all INVALID checks, in the order the header states.
int check_partials(const void *const *partials, int n_ranks, int64_t n, PartialPtrs &pp)
{
    if (!partials || n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
        return ZERO_ERR_INVALID;
    memset(&pp, 0, sizeof(pp));
    for (int k = 0; k < n_ranks; ++k) {
        if (!partials[k] && n > 0)
            return ZERO_ERR_INVALID;
        pp.p[k] = partials[k];
    }
    return ZERO_OK;
}

bool partials_aligned(const PartialPtrs &pp, int n_ranks)
{
    for (int k = 0; k < n_ranks; ++k)
        if (!aligned16(pp.p[k]))
            return false;
    return true;
}

// The dtype arrives as a plain int from C callers; only these values are
// converted to zero_dtype.
bool valid_dtype(int gdt) { return gdt == ZERO_BF16 || gdt == ZERO_FP32; }

int hip_status(hipError_t e) { return e == hipSuccess ? ZERO_OK : ZERO_ERR_HIP; }

// [p, p + bytes) is device memory?  Turns a stray host or freed address
// into an error code instead of a GPU memory fault.  Usually one allocation
// holds the whole range (one query).  A range built from several physical
// allocations mapped back to back (HIP's virtual memory API, allocators with
// expandable segments) is followed mapping by mapping, each one starting
// where the previous ends, up to kMaxMappings of them; a hole fails.  A
// failed query's error is cleared so it cannot surface at the caller's next
// check.
constexpr int kMaxMappings = 1 << 16;

bool in_device_alloc(const void *p, int64_t bytes)
{
    if (bytes <= 0)
        return true;
    uintptr_t at = (uintptr_t)p;
    const uintptr_t end = at + (uint64_t)bytes;
    for (int i = 0; i < kMaxMappings; ++i) {
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)at) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        const uintptr_t b0 = (uintptr_t)base, b1 = b0 + size;
        if (at < b0 || at >= b1)
            return false;
        if (end <= b1)
            return true;
        at = b1;
    }
    return false;
}

}  // namespace

extern "C" {

int zero_version(void) { return (1 << 16) | 9; }

const char *zero_strerror(int code)
{
    switch (code) {
    case ZERO_OK: return "ok";
    case ZERO_ERR_INVALID: return "invalid argument";
    case ZERO_ERR_MISALIGNED: return "base pointer not 16-byte aligned";
    case ZERO_ERR_UNSUPPORTED: return "unsupported gradient dtype";
    case ZERO_ERR_ALIAS: return "input overlaps an output";
    case ZERO_ERR_HIP: return "HIP launch error";
    case ZERO_ERR_CAPACITY: return "chunk array too small";
    case ZERO_ERR_NOT_DEVICE: return "array range is not device memory";
    default: return "unknown error code";
    }
}

}  // extern "C"

namespace zs {

// Where a scheduled step finds its constants (device table and index).
struct Schedule {
    const zero_step_consts *consts;
    int64_t n;
    const int64_t *index;
};

// The three arrays a fused step updates in place (master, m, v; or comp, m,
// v) and their element sizes in bytes.
struct StateArrays {
    const void *p[3];
    int64_t eb[3];
};

// The checks of a fused step, in the header's order, and the kernel
// arguments they have vetted (the caller sets the state pointers).  The
// constants come from hp, or, with sched given, from the device table the
// scheduled kernels read (hp is then unused).  Returns ZERO_OK with *empty
// set when there is nothing to launch.
static int prepare_fused(const void *const *partials, int n_ranks, int gdt, const StateArrays &st,
                         int64_t shard_len, const zero_chunk *d_chunks, int64_t n_chunks,
                         const zero_adamw_hparams *hp, const Schedule *sched, StepArgs &a,
                         bool *empty)
{
    *empty = true;
    int rc = check_partials(partials, n_ranks, shard_len, a.parts);
    if (rc)
        return rc;
    if (((!st.p[0] || !st.p[1] || !st.p[2]) && shard_len > 0) || bad_len(shard_len) ||
        n_chunks < 0 || n_chunks > INT32_MAX || (n_chunks > 0 && !d_chunks) ||
        (!sched && !valid_hparams(hp)))
        return ZERO_ERR_INVALID;
    if (sched && (sched->n < 0 || sched->n > INT32_MAX ||
                  (shard_len > 0 && (!sched->consts || !sched->index || sched->n < 1))))
        return ZERO_ERR_INVALID;
    if (!partials_aligned(a.parts, n_ranks) || !aligned16(st.p[0]) || !aligned16(st.p[1]) ||
        !aligned16(st.p[2]) || !aligned16(d_chunks))
        return ZERO_ERR_MISALIGNED;
    if (sched && (!aligned16(sched->consts) || ((uintptr_t)sched->index & 7u) != 0))
        return ZERO_ERR_MISALIGNED;
    if (!valid_dtype(gdt))
        return ZERO_ERR_UNSUPPORTED;
    const int64_t gb = shard_len * elem_bytes(gdt);
    const int64_t sb[3] = {shard_len * st.eb[0], shard_len * st.eb[1], shard_len * st.eb[2]};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(st.p[i], sb[i], st.p[j], sb[j]))
                return ZERO_ERR_ALIAS;
    for (int k = 0; k < n_ranks; ++k)
        for (int i = 0; i < 3; ++i)
            if (overlaps(partials[k], gb, st.p[i], sb[i]))
                return ZERO_ERR_ALIAS;
    const int64_t cb = sched ? sched->n * (int64_t)sizeof(zero_step_consts) : 0;
    if (sched && shard_len > 0)
        for (int i = 0; i < 3; ++i)
            if (overlaps(sched->consts, cb, st.p[i], sb[i]) ||
                overlaps(sched->index, 8, st.p[i], sb[i]))
                return ZERO_ERR_ALIAS;
    if (n_chunks == 0 || shard_len == 0)
        return ZERO_OK;
    for (int k = 0; k < n_ranks; ++k)
        if (!in_device_alloc(partials[k], gb))
            return ZERO_ERR_NOT_DEVICE;
    for (int i = 0; i < 3; ++i)
        if (!in_device_alloc(st.p[i], sb[i]))
            return ZERO_ERR_NOT_DEVICE;
    if (!in_device_alloc(d_chunks, n_chunks * (int64_t)sizeof(zero_chunk)))
        return ZERO_ERR_NOT_DEVICE;
    if (sched && (!in_device_alloc(sched->consts, cb) || !in_device_alloc(sched->index, 8)))
        return ZERO_ERR_NOT_DEVICE;
    a.red = make_reduce(n_ranks);
    if (sched) {
        a.sched = sched->consts;
        a.n_sched = sched->n;
        a.sched_index = sched->index;
    } else {
        a.k = make_scalars(hp);
    }
    a.chunks = d_chunks;
    a.n_chunks = n_chunks;
    a.shard_len = shard_len;
    a.acc = nullptr;
    *empty = false;
    return ZERO_OK;
}

// The 16-byte state: fp32 master, m, v.
static int prepare_step(const void *const *partials, int n_ranks, int gdt, float *master,
                        float *m, float *v, int64_t shard_len, const zero_chunk *d_chunks,
                        int64_t n_chunks, const zero_adamw_hparams *hp, StepArgs &a, bool *empty,
                        const Schedule *sched = nullptr)
{
    const StateArrays st{{master, m, v}, {4, 4, 4}};
    const int rc = prepare_fused(partials, n_ranks, gdt, st, shard_len, d_chunks, n_chunks, hp,
                                 sched, a, empty);
    a.master = master;
    a.m = m;
    a.v = v;
    a.comp = nullptr;
    return rc;
}

// The 12-byte state: fp32 master, bf16 m and v (read by the kernel as
// 16-bit patterns through the float pointers).
static int prepare_m16(const void *const *partials, int n_ranks, int gdt, float *master,
                       uint16_t *m, uint16_t *v, int64_t shard_len, const zero_chunk *d_chunks,
                       int64_t n_chunks, const zero_adamw_hparams *hp, StepArgs &a, bool *empty,
                       const Schedule *sched = nullptr)
{
    const StateArrays st{{master, m, v}, {4, 2, 2}};
    const int rc = prepare_fused(partials, n_ranks, gdt, st, shard_len, d_chunks, n_chunks, hp,
                                 sched, a, empty);
    a.master = master;
    a.m = (float *)m;
    a.v = (float *)v;
    a.comp = nullptr;
    return rc;
}

// The pure-bf16 state: compensation, m, v in bf16 (the parameters are the
// chunk destinations).
static int prepare_kahan(const void *const *partials, int n_ranks, int gdt, uint16_t *comp,
                         uint16_t *m, uint16_t *v, int64_t shard_len, const zero_chunk *d_chunks,
                         int64_t n_chunks, const zero_adamw_hparams *hp, StepArgs &a, bool *empty,
                         const Schedule *sched = nullptr)
{
    const StateArrays st{{comp, m, v}, {2, 2, 2}};
    const int rc = prepare_fused(partials, n_ranks, gdt, st, shard_len, d_chunks, n_chunks, hp,
                                 sched, a, empty);
    a.master = nullptr;
    a.m = (float *)m;
    a.v = (float *)v;
    a.comp = comp;
    return rc;
}

}  // namespace zs

extern "C" {

int zero_shard_step(const void *const *partials, int n_ranks, int gdt,
                    float *master, float *m, float *v, int64_t shard_len,
                    const zero_chunk *d_chunks, int64_t n_chunks,
                    const zero_adamw_hparams *hp, hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    int rc = prepare_step(partials, n_ranks, gdt, master, m, v, shard_len, d_chunks, n_chunks, hp,
                          a, &empty);
    if (rc || empty)
        return rc;
    return hip_status(launch_step(a, (zero_dtype)gdt, stream));
}

int zero_shard_step_buckets(const void *const *partials, int n_ranks, int gdt,
                            float *master, float *m, float *v, int64_t shard_len,
                            const zero_chunk *d_chunks, int64_t n_chunks,
                            const int64_t *first, const int64_t *count, int n_buckets,
                            const hipEvent_t *ready, const zero_adamw_hparams *hp,
                            hipStream_t stream)
{
    if (n_buckets < 0 || (n_buckets > 0 && (!first || !count)) || n_chunks < 0 ||
        n_chunks > INT32_MAX)
        return ZERO_ERR_INVALID;
    int64_t end = 0;
    for (int b = 0; b < n_buckets; ++b) {
        if (count[b] < 0 || first[b] < end || first[b] > n_chunks - count[b])
            return ZERO_ERR_INVALID;   // out of the table, overlapping or out of order
        end = first[b] + count[b];
    }
    StepArgs a{};
    bool empty;
    int rc = prepare_step(partials, n_ranks, gdt, master, m, v, shard_len, d_chunks, n_chunks, hp,
                          a, &empty);
    if (rc || empty || n_buckets == 0)
        return rc;
    if (ready) {
        for (int b = 0; b < n_buckets; ++b) {
            if (!ready[b])
                continue;
            const hipError_t e = hipEventQuery(ready[b]);
            if (e != hipSuccess && e != hipErrorNotReady) {
                (void)hipGetLastError();
                return ZERO_ERR_HIP;
            }
        }
        // hipErrorNotReady is an answer, not a failure: clear it so that the
        // launches' own status check below sees only their errors
        (void)hipGetLastError();
    }
    for (int b = 0; b < n_buckets; ++b) {
        if (count[b] == 0)
            continue;
        if (ready && ready[b] && hipStreamWaitEvent(stream, ready[b], 0) != hipSuccess)
            return ZERO_ERR_HIP;
        a.chunks = d_chunks + first[b];
        a.n_chunks = count[b];
        rc = hip_status(launch_step(a, (zero_dtype)gdt, stream));
        if (rc)
            return rc;
    }
    return ZERO_OK;
}

int zero_make_step_consts(const zero_adamw_hparams *hps, int64_t count, zero_step_consts *out)
{
    if (count < 0 || count > INT32_MAX || (count > 0 && (!hps || !out)))
        return ZERO_ERR_INVALID;
    for (int64_t i = 0; i < count; ++i)
        if (!valid_hparams(hps + i))
            return ZERO_ERR_INVALID;
    for (int64_t i = 0; i < count; ++i) {
        const StepScalars k = make_scalars(hps + i);
        memcpy(out + i, &k, sizeof(k));
    }
    return ZERO_OK;
}

int zero_shard_step_scheduled(const void *const *partials, int n_ranks, int gdt,
                              float *master, float *m, float *v, int64_t shard_len,
                              const zero_chunk *d_chunks, int64_t n_chunks,
                              const zero_step_consts *consts, int64_t n_consts,
                              const int64_t *index, hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    const Schedule sched{consts, n_consts, index};
    int rc = prepare_step(partials, n_ranks, gdt, master, m, v, shard_len, d_chunks, n_chunks,
                          nullptr, a, &empty, &sched);
    if (rc || empty)
        return rc;
    return hip_status(launch_step_sched(a, (zero_dtype)gdt, StateLayout::Fp32, stream));
}

int zero_step_index_advance(int64_t *index, int64_t n_consts, hipStream_t stream)
{
    if (!index || n_consts < 1)
        return ZERO_ERR_INVALID;
    if (((uintptr_t)index & 7u) != 0)
        return ZERO_ERR_MISALIGNED;
    if (!in_device_alloc(index, 8))
        return ZERO_ERR_NOT_DEVICE;
    return hip_status(launch_index_advance(index, n_consts, stream));
}

int zero_shard_step_ex(const void *const *partials, int n_ranks, int gdt,
                       const zero_reduce_spec *rs, float *master, float *m, float *v,
                       int64_t shard_len, const zero_chunk *d_chunks, int64_t n_chunks,
                       const zero_adamw_hparams *hp, hipStream_t stream)
{
    StepArgs a{};
    int rc = check_partials(partials, n_ranks, shard_len, a.parts);
    if (rc)
        return rc;
    if (((!master || !m || !v) && shard_len > 0) || bad_len(shard_len) || n_chunks < 0 ||
        n_chunks > INT32_MAX || (n_chunks > 0 && !d_chunks) || !valid_hparams(hp) ||
        !valid_reduce_spec(rs, n_ranks))
        return ZERO_ERR_INVALID;
    if (!partials_aligned(a.parts, n_ranks) || !aligned16(master) || !aligned16(m) ||
        !aligned16(v) || !aligned16(d_chunks) || !aligned16(rs->acc))
        return ZERO_ERR_MISALIGNED;
    if (!valid_dtype(gdt))
        return ZERO_ERR_UNSUPPORTED;
    const int64_t sb = shard_len * 4, gb = shard_len * elem_bytes(gdt);
    if (overlaps(master, sb, m, sb) || overlaps(master, sb, v, sb) || overlaps(m, sb, v, sb))
        return ZERO_ERR_ALIAS;
    for (int k = 0; k < n_ranks; ++k)
        if (overlaps(partials[k], gb, master, sb) || overlaps(partials[k], gb, m, sb) ||
            overlaps(partials[k], gb, v, sb))
            return ZERO_ERR_ALIAS;
    if (rs->acc && (overlaps(rs->acc, sb, master, sb) || overlaps(rs->acc, sb, m, sb) ||
                    overlaps(rs->acc, sb, v, sb)))
        return ZERO_ERR_ALIAS;
    if (n_chunks == 0 || shard_len == 0)
        return ZERO_OK;
    for (int k = 0; k < n_ranks; ++k)
        if (!in_device_alloc(partials[k], gb))
            return ZERO_ERR_NOT_DEVICE;
    if (!in_device_alloc(master, sb) || !in_device_alloc(m, sb) || !in_device_alloc(v, sb) ||
        !in_device_alloc(d_chunks, n_chunks * (int64_t)sizeof(zero_chunk)) ||
        (rs->acc && !in_device_alloc(rs->acc, sb)))
        return ZERO_ERR_NOT_DEVICE;
    a.red = make_reduce(n_ranks, rs->group, rs->micro_batches);
    a.k = make_scalars(hp);
    a.master = master;
    a.m = m;
    a.v = v;
    a.chunks = d_chunks;
    a.n_chunks = n_chunks;
    a.shard_len = shard_len;
    a.acc = rs->acc;
    return hip_status(launch_step_ex(a, (zero_dtype)gdt, stream));
}

int zero_shard_step_bf16_moments(const void *const *partials, int n_ranks, int gdt,
                                 float *master, uint16_t *m, uint16_t *v, int64_t shard_len,
                                 const zero_chunk *d_chunks, int64_t n_chunks,
                                 const zero_adamw_hparams *hp, hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    const int rc = prepare_m16(partials, n_ranks, gdt, master, m, v, shard_len, d_chunks,
                               n_chunks, hp, a, &empty);
    if (rc || empty)
        return rc;
    return hip_status(launch_step_m16(a, (zero_dtype)gdt, stream));
}

int zero_shard_step_kahan(const void *const *partials, int n_ranks, int gdt,
                          uint16_t *comp, uint16_t *m, uint16_t *v, int64_t shard_len,
                          const zero_chunk *d_chunks, int64_t n_chunks,
                          const zero_adamw_hparams *hp, hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    const int rc = prepare_kahan(partials, n_ranks, gdt, comp, m, v, shard_len, d_chunks,
                                 n_chunks, hp, a, &empty);
    if (rc || empty)
        return rc;
    return hip_status(launch_step_kahan(a, (zero_dtype)gdt, stream));
}

int zero_shard_step_bf16_moments_scheduled(const void *const *partials, int n_ranks, int gdt,
                                           float *master, uint16_t *m, uint16_t *v,
                                           int64_t shard_len, const zero_chunk *d_chunks,
                                           int64_t n_chunks, const zero_step_consts *consts,
                                           int64_t n_consts, const int64_t *index,
                                           hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    const Schedule sched{consts, n_consts, index};
    const int rc = prepare_m16(partials, n_ranks, gdt, master, m, v, shard_len, d_chunks,
                               n_chunks, nullptr, a, &empty, &sched);
    if (rc || empty)
        return rc;
    return hip_status(launch_step_sched(a, (zero_dtype)gdt, StateLayout::Bf16Moments, stream));
}

int zero_shard_step_kahan_scheduled(const void *const *partials, int n_ranks, int gdt,
                                    uint16_t *comp, uint16_t *m, uint16_t *v, int64_t shard_len,
                                    const zero_chunk *d_chunks, int64_t n_chunks,
                                    const zero_step_consts *consts, int64_t n_consts,
                                    const int64_t *index, hipStream_t stream)
{
    StepArgs a{};
    bool empty;
    const Schedule sched{consts, n_consts, index};
    const int rc = prepare_kahan(partials, n_ranks, gdt, comp, m, v, shard_len, d_chunks,
                                 n_chunks, nullptr, a, &empty, &sched);
    if (rc || empty)
        return rc;
    return hip_status(launch_step_sched(a, (zero_dtype)gdt, StateLayout::Kahan, stream));
}

int zero_accumulate_shard(const void *const *partials, int n_ranks, int gdt, int group,
                          int64_t n, float *acc, int reset, hipStream_t stream)
{
    AccArgs a;
    int rc = check_partials(partials, n_ranks, n, a.parts);
    if (rc)
        return rc;
    if ((!acc && n > 0) || bad_len(n) || group < 0 || group > n_ranks ||
        (group > 0 && n_ranks % group != 0))
        return ZERO_ERR_INVALID;
    if (!partials_aligned(a.parts, n_ranks) || !aligned16(acc))
        return ZERO_ERR_MISALIGNED;
    if (!valid_dtype(gdt))
        return ZERO_ERR_UNSUPPORTED;
    for (int k = 0; k < n_ranks; ++k)
        if (overlaps(partials[k], n * elem_bytes(gdt), acc, n * 4))
            return ZERO_ERR_ALIAS;
    if (n == 0)
        return ZERO_OK;
    for (int k = 0; k < n_ranks; ++k)
        if (!in_device_alloc(partials[k], n * elem_bytes(gdt)))
            return ZERO_ERR_NOT_DEVICE;
    if (!in_device_alloc(acc, n * 4))
        return ZERO_ERR_NOT_DEVICE;
    a.red = make_reduce(n_ranks, group, 1);
    a.acc = acc;
    a.n = n;
    a.reset = reset ? 1 : 0;
    return hip_status(launch_accumulate(a, (zero_dtype)gdt, stream));
}

int zero_reduce_shard(const void *const *partials, int n_ranks, int gdt, int64_t n,
                      float *grad_out, hipStream_t stream)
{
    ReduceArgs a;
    int rc = check_partials(partials, n_ranks, n, a.parts);
    if (rc)
        return rc;
    if ((!grad_out && n > 0) || bad_len(n))
        return ZERO_ERR_INVALID;
    if (!partials_aligned(a.parts, n_ranks) || !aligned16(grad_out))
        return ZERO_ERR_MISALIGNED;
    if (!valid_dtype(gdt))
        return ZERO_ERR_UNSUPPORTED;
    for (int k = 0; k < n_ranks; ++k)
        if (overlaps(partials[k], n * elem_bytes(gdt), grad_out, n * 4))
            return ZERO_ERR_ALIAS;
    if (n == 0)
        return ZERO_OK;
    for (int k = 0; k < n_ranks; ++k)
        if (!in_device_alloc(partials[k], n * elem_bytes(gdt)))
            return ZERO_ERR_NOT_DEVICE;
    if (!in_device_alloc(grad_out, n * 4))
        return ZERO_ERR_NOT_DEVICE;
    a.red = make_reduce(n_ranks);
    a.out = grad_out;
    a.n = n;
    return hip_status(launch_reduce(a, (zero_dtype)gdt, stream));
}

int zero_adamw_shard(const float *grad, float *master, float *m, float *v, int64_t n,
                     const zero_adamw_hparams *hp, hipStream_t stream)
{
    if (((!grad || !master || !m || !v) && n > 0) || bad_len(n) || !valid_hparams(hp))
        return ZERO_ERR_INVALID;
    if (!aligned16(grad) || !aligned16(master) || !aligned16(m) || !aligned16(v))
        return ZERO_ERR_MISALIGNED;
    const int64_t b = n * 4;
    if (overlaps(grad, b, master, b) || overlaps(grad, b, m, b) || overlaps(grad, b, v, b) ||
        overlaps(master, b, m, b) || overlaps(master, b, v, b) || overlaps(m, b, v, b))
        return ZERO_ERR_ALIAS;
    if (n == 0)
        return ZERO_OK;
    if (!in_device_alloc(grad, b) || !in_device_alloc(master, b) || !in_device_alloc(m, b) ||
        !in_device_alloc(v, b))
        return ZERO_ERR_NOT_DEVICE;
    AdamArgs a;
    a.k = make_scalars(hp);
    a.g = grad;
    a.master = master;
    a.m = m;
    a.v = v;
    a.n = n;
    return hip_status(launch_adamw(a, stream));
}

int zero_gather_write(const float *master, int64_t shard_len, const zero_chunk *d_chunks,
                      int64_t n_chunks, hipStream_t stream)
{
    if ((!master && shard_len > 0) || bad_len(shard_len) || n_chunks < 0 || n_chunks > INT32_MAX ||
        (n_chunks > 0 && !d_chunks))
        return ZERO_ERR_INVALID;
    if (!aligned16(master) || !aligned16(d_chunks))
        return ZERO_ERR_MISALIGNED;
    if (n_chunks == 0 || shard_len == 0)
        return ZERO_OK;
    if (!in_device_alloc(master, shard_len * 4) ||
        !in_device_alloc(d_chunks, n_chunks * (int64_t)sizeof(zero_chunk)))
        return ZERO_ERR_NOT_DEVICE;
    GatherArgs a;
    a.master = master;
    a.chunks = d_chunks;
    a.n_chunks = n_chunks;
    a.shard_len = shard_len;
    return hip_status(launch_gather(a, stream));
}

int zero_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream)
{
    if (((!src || !dst) && bytes > 0) || bad_len(bytes))
        return ZERO_ERR_INVALID;
    if (!aligned16(src) || !aligned16(dst))
        return ZERO_ERR_MISALIGNED;
    if (overlaps(src, bytes, dst, bytes))
        return ZERO_ERR_ALIAS;
    if (bytes == 0)
        return ZERO_OK;
    if (!in_device_alloc(src, bytes) || !in_device_alloc(dst, bytes))
        return ZERO_ERR_NOT_DEVICE;
    return hip_status(launch_probe_copy(src, dst, bytes, stream));
}

int zero_probe_read(const void *src, int64_t bytes, uint32_t *sink, uint32_t magic, hipStream_t stream)
{
    if (((!src || !sink) && bytes > 0) || bad_len(bytes))
        return ZERO_ERR_INVALID;
    if (!aligned16(src) || ((uintptr_t)sink & 3u) != 0)
        return ZERO_ERR_MISALIGNED;
    if (bytes == 0)
        return ZERO_OK;
    if (!in_device_alloc(src, bytes) || !in_device_alloc(sink, 4))
        return ZERO_ERR_NOT_DEVICE;
    return hip_status(launch_probe_read(src, bytes, sink, magic, stream));
}

int zero_probe_write(void *dst, int64_t bytes, uint32_t value, hipStream_t stream)
{
    if ((!dst && bytes > 0) || bad_len(bytes))
        return ZERO_ERR_INVALID;
    if (!aligned16(dst))
        return ZERO_ERR_MISALIGNED;
    if (bytes == 0)
        return ZERO_OK;
    if (!in_device_alloc(dst, bytes))
        return ZERO_ERR_NOT_DEVICE;
    return hip_status(launch_probe_write(dst, bytes, value, stream));
}

int zero_probe_sum(const float *const *src, int k, float *dst, int64_t n, hipStream_t stream)
{
    if (!src || k < 1 || k > ZERO_PROBE_SUM_MAX || n < 0 || n > ZERO_MAX_LEN / 4 || (!dst && n > 0))
        return ZERO_ERR_INVALID;
    for (int j = 0; j < k; ++j)
        if (!src[j] && n > 0)
            return ZERO_ERR_INVALID;
    if (!aligned16(dst))
        return ZERO_ERR_MISALIGNED;
    for (int j = 0; j < k; ++j)
        if (!aligned16(src[j]))
            return ZERO_ERR_MISALIGNED;
    for (int j = 0; j < k; ++j)
        if (overlaps(src[j], n * 4, dst, n * 4))
            return ZERO_ERR_ALIAS;
    if (n == 0)
        return ZERO_OK;
    if (!in_device_alloc(dst, n * 4))
        return ZERO_ERR_NOT_DEVICE;
    for (int j = 0; j < k; ++j)
        if (!in_device_alloc(src[j], n * 4))
            return ZERO_ERR_NOT_DEVICE;
    return hip_status(launch_probe_sum(src, k, dst, n, stream));
}

}  // extern "C"
