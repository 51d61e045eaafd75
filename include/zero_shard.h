/*
 * zero_shard.h -- C ABI of the ZeRO/FSDP per-rank optimizer-step library
 * for AMD Instinct MI355X (gfx950).  Library: libzero_shard.so.
 *
 * One data-parallel rank owns a contiguous segment ("shard") of the flat
 * parameter vector.  Its optimizer step has three parts:
 *
 *   1. reduce    g[i] = (p_0[i] + ... + p_{N-1}[i]) / N over the N ranks'
 *                gradient partials for this shard: the local arithmetic of
 *                the gradient reduce-scatter ("CS336 2026 Lecture 8:
 *                Parallelism Basics", Slide 8: all-reduce = reduce-scatter +
 *                all-gather; "并行策略总览：六个维度各切什么、怎么通信", data-parallel
 *                section: the full-batch gradient is the mean of the ranks'
 *                gradients).
 *   2. AdamW     on the shard's fp32 master weights and Adam moments m, v,
 *                which only this rank keeps (Lecture 8, Slides 17 and 19-20:
 *                the 16-bytes-per-parameter ledger, optimizer state sharded).
 *   3. write     the updated parameters, rounded to bf16, into this rank's
 *                slot of the full parameter buffer: the local half of the
 *                parameter all-gather (Lecture 8, Slide 20, fourth step;
 *                "并行训练优化、MoE扩展与系统瓶颈", 2.2.1 and 2.2.4).
 *
 * zero_shard_step does all three in one pass over HBM; zero_reduce_shard,
 * zero_adamw_shard and zero_gather_write do them one at a time and give the
 * same bits.  Variants of the fused pass: zero_shard_step_ex (two-level
 * reduce order, gradient accumulation), zero_shard_step_bf16_moments (fp32
 * master with bf16 m, v), zero_shard_step_kahan (pure bf16 state with a
 * compensated update, no fp32 master), zero_shard_step_buckets (one launch
 * per gradient bucket) and zero_shard_step_scheduled (step constants read
 * from device memory, for steps captured in a HIP graph).
 *
 * Arithmetic, fixed so that every result is reproducible bit for bit:
 *   - g: the partials are widened exactly to double and summed in double,
 *     rank 0 first, ranks 1..N-1 in order; the sum is divided by N in
 *     double and rounded once to fp32 (the reduced gradient shard is an
 *     fp32 tensor).
 *   - AdamW (decoupled weight decay, bias correction, eps outside the root),
 *     every operation an IEEE double operation without fused multiply-add:
 *         m' = b1 m + (1 - b1) g
 *         v' = b2 v + (1 - b2) (g g)
 *         theta' = theta (1 - lr wd) - lr (m'/(1 - b1^t)) / (sqrt(v'/(1 - b2^t)) + eps)
 *     m', v', theta' rounded once to fp32.  (1 - b1), (1 - b2), (1 - lr wd)
 *     and b^t = pow(b, t) are formed in double.
 *   - the bf16 parameter is theta' (fp32) rounded to nearest even; NaN
 *     stays NaN with its sign and the quiet bit set; overflow gives inf.
 *   Non-finite inputs propagate per IEEE; there is no clipping or skipping.
 *
 * Conventions for every entry point:
 *   - All array arguments are device pointers unless stated otherwise.
 *     The caller owns all memory.  The library never allocates or frees
 *     device memory and keeps no global mutable state; calls are re-entrant.
 *   - Kernels run on the device that `stream` belongs to (the current
 *     device for the null stream).  Every array must be accessible from that
 *     device: its own memory, or a peer's mapped with peer access or an IPC
 *     handle.  The checks confirm that an address range is device memory,
 *     not which device holds it.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without synchronising.  Device faults surface at the caller's
 *     next synchronisation, as usual for HIP.
 *   - Every check runs on the host before anything is launched; a call that
 *     returns an error has launched nothing and changed nothing.  Checks,
 *     in order: null pointers and counts (INVALID), 16-byte alignment
 *     (MISALIGNED), dtype (UNSUPPORTED), overlap of inputs with outputs
 *     (ALIAS), and finally that every array range is device memory
 *     (NOT_DEVICE, via hipMemGetAddressRange: one allocation, or up to 65,536
 *     physical allocations mapped back to back without a hole, as HIP's
 *     virtual memory API and expandable-segment allocators produce).  The chunk
 *     table lives in device memory, so the step calls cannot read its dst
 *     addresses without a device round trip; zero_check_chunks checks a
 *     host table against the arrays of a step once, before the table is
 *     used (INVALID for a malformed table, ALIAS for a dst range that
 *     overlaps a partial, a state array or another chunk's dst).  A table
 *     names each shard element at most once (tables from zero_build_chunks,
 *     and contiguous runs of their chunks, do).
 *   - `gdt` arguments are plain ints holding a zero_dtype value; any other
 *     value is UNSUPPORTED (the library converts to the enum only after the
 *     check).
 *   - Base pointers of partials, state arrays and grad arrays must be 16-byte
 *     aligned (torch allocations are).  Lengths and offsets are arbitrary.
 *   - When the element count is 0 the call does nothing and its array
 *     pointers may be NULL (an empty shard).
 *   - Element and byte counts above ZERO_MAX_LEN (2^48) are INVALID, so
 *     that no byte size the library forms can overflow int64.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the gradient partials. */
typedef enum zero_dtype {
    ZERO_BF16 = 0,   /* bfloat16, passed as 16-bit patterns */
    ZERO_FP32 = 1    /* IEEE binary32 (gradients communicated in fp32) */
} zero_dtype;

/* AdamW hyper-parameters, in double.  `step` is t >= 1, the number of this
 * update counted from 1 (bias corrections use b1^t and b2^t).
 * Requirements: finite lr, eps, weight_decay; 0 <= beta1, beta2 < 1. */
typedef struct zero_adamw_hparams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int64_t step;
} zero_adamw_hparams;

/* The constants of one step, formed on the host in double from a
 * zero_adamw_hparams (zero_make_step_consts); what the step kernels use.
 * 80 bytes. */
typedef struct zero_step_consts {
    double b1, c1;     /* beta1, 1 - beta1 */
    double b2, c2;     /* beta2, 1 - beta2 */
    double bc1, bc2;   /* 1 - beta1^t, 1 - beta2^t */
    double eps, lr;
    double dec;        /* 1 - lr * weight_decay */
    double wd;         /* weight_decay */
} zero_step_consts;

/* One chunk of a shard: shard elements [shard_off, shard_off + len), whose
 * bf16 parameters go to dst[0 .. len).  32 bytes.  Built on the host by
 * zero_build_chunks; the caller copies the table to device memory. */
typedef struct zero_chunk {
    int64_t shard_off;   /* first shard element of the chunk */
    uint16_t *dst;       /* device address of the bf16 parameter of shard_off */
    int32_t len;         /* element count, 1 .. max_chunk */
    int32_t tensor_id;   /* tensor holding shard element shard_off */
    int64_t tensor_off;  /* element offset of shard_off inside that tensor */
} zero_chunk;

/* Return codes. */
enum {
    ZERO_OK = 0,
    ZERO_ERR_INVALID = 1,      /* null pointer, bad count or length, bad hyper-parameter */
    ZERO_ERR_MISALIGNED = 2,   /* a base pointer is not 16-byte aligned */
    ZERO_ERR_UNSUPPORTED = 3,  /* unknown dtype */
    ZERO_ERR_ALIAS = 4,        /* an input array overlaps an array the call writes */
    ZERO_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
    ZERO_ERR_CAPACITY = 6,     /* caller's chunk array too small (see n_out) */
    ZERO_ERR_NOT_DEVICE = 7    /* an array range is not (wholly) device memory */
};

#define ZERO_MAX_RANKS 64
#define ZERO_MAX_LEN (((int64_t)1) << 48)   /* largest element or byte count */
/* Chunk lengths the step kernels are tuned for: 4 KiB of each partial per
 * chunk, i.e. 256 lane groups, four passes of a 64-lane wave, with either
 * partial dtype.  Measured on MI355X in one process on the same buffers:
 * bf16 partials (7B shard, N = 8) 0.727 of HBM peak with 2048 against 0.701
 * with 1024 and 0.673 with 4096; fp32 partials (ragged shard, N = 32) 0.677
 * with 1024 against 0.651 with 2048 and 0.633 with 8192. */
#define ZERO_DEFAULT_MAX_CHUNK 2048        /* bf16 partials */
#define ZERO_DEFAULT_MAX_CHUNK_FP32 1024   /* fp32 partials */
/* Launches over at most this many chunks run at a higher occupancy, which
 * suits small shards and single gradient buckets: ZERO_SMALL_LAUNCH_CHUNKS
 * for the 16-byte and extended steps (with their bucket and scheduled
 * forms), ZERO_SMALL_LAUNCH_CHUNKS_12B for the 12-byte step.  Results are
 * the same bits either way. */
#define ZERO_SMALL_LAUNCH_CHUNKS 2048
#define ZERO_SMALL_LAUNCH_CHUNKS_12B 16384

/*
 * Shard geometry and the chunk table (host only; no device calls).
 *
 * The parameters are the n_tensors tensors concatenated in order (numels[t]
 * elements each, host array), total T.  With n_ranks ranks the shard length
 * is S = ceil(T / n_ranks) and rank `rank` owns flat elements
 * [rank*S, min((rank+1)*S, T)) -- contiguous, cutting across tensor
 * boundaries; the last shards may be shorter or empty (Lecture 8,
 * Slides 19-20: each rank updates one segment of the parameters).
 *
 * Destination of the bf16 parameters, one of:
 *   tensor_dst != NULL: host array of n_tensors device pointers; element e
 *     of tensor t is written to tensor_dst[t] + e.  Chunks never cross a
 *     tensor boundary.
 *   tensor_dst == NULL: slot_dst is the device address of this rank's slot
 *     (for a flat full parameter buffer P, slot_dst = P + rank*S); shard
 *     element i is written to slot_dst + i.  Chunks may cross tensors.
 * Chunks are also cut every max_chunk elements of the shard (max_chunk a
 * positive multiple of 64, at most 2^24).
 *
 * out: host array of cap chunks, or NULL to query the count only.
 * *n_out receives the number of chunks needed, *shard_len_out receives the
 * shard length S (both may be NULL).  Returns ZERO_ERR_CAPACITY if out is
 * not NULL and cap < *n_out (nothing written beyond cap).  INVALID for a
 * negative numel, a total above ZERO_MAX_LEN, a NULL destination of a
 * non-empty tensor, rank outside [0, n_ranks) or a bad max_chunk.
 */
int zero_build_chunks(const int64_t *numels, int n_tensors, int n_ranks, int rank,
                      uint16_t *const *tensor_dst, uint16_t *slot_dst, int64_t max_chunk,
                      zero_chunk *out, int64_t cap, int64_t *n_out, int64_t *shard_len_out);

/*
 * Check a chunk table against the arrays of the step that will use it
 * (host only; no device calls, nothing dereferenced on the device).
 *
 * The parameter all-gather writes each shard element's bf16 value into its
 * slot of the full parameter buffer ("CS336 2026 Lecture 8: Parallelism
 * Basics", Slide 20, fourth step); a slot must therefore be written once
 * and must not be an input of the same step.
 *
 * chunks:      host copy of the table (n_chunks entries).
 * shard_len:   the step's shard length.
 * arrays, array_bytes: n_arrays byte ranges [arrays[i], arrays[i] +
 *              array_bytes[i]) that the step reads or writes besides the
 *              destinations: the partials, master, m, v (or comp, m, v),
 *              an accumulator.  Host arrays of device addresses and sizes.
 * Returns INVALID for a null or negative argument, a chunk with len < 1,
 * a null dst, a chunk outside [0, shard_len), or two chunks covering the
 * same shard element; then ALIAS when two chunks' destinations
 * [dst, dst + 2 len) overlap, or a destination overlaps one of the arrays.
 * O(n_chunks log n_chunks) time and O(n_chunks) host memory.
 */
int zero_check_chunks(const zero_chunk *chunks, int64_t n_chunks, int64_t shard_len,
                      const void *const *arrays, const int64_t *array_bytes, int n_arrays);

/*
 * The fused shard step: reduce + AdamW + bf16 write in one pass.
 *
 * Defined by the ZeRO lifecycle of "CS336 2026 Lecture 8: Parallelism
 * Basics", Slides 19-20: gradients are reduce-scattered to the rank that
 * owns each segment, the owner updates its segment with its own optimizer
 * state, and the updated parameters are all-gathered; "并行训练优化、MoE扩展与
 * 系统瓶颈", 2.2.1, gives the same per-rank update of a parameter shard from
 * its gradient shard and optimizer-state shard.  This call is the local
 * arithmetic of those three phases for one rank.
 *
 * partials:  host array of n_ranks device pointers; partials[k] holds rank
 *            k's gradient for this shard, shard_len elements of type gdt,
 *            read only.  1 <= n_ranks <= ZERO_MAX_RANKS.
 * master, m, v: fp32 device arrays of shard_len elements, updated in place.
 * d_chunks, n_chunks: the chunk table in device memory (from
 *            zero_build_chunks for this shard_len); chunks outside
 *            [0, shard_len) are skipped.  Shard elements no chunk covers
 *            are left untouched.
 * hp:        host pointer to the hyper-parameters of this step.
 * Errors: INVALID (null, n_ranks out of range, shard_len < 0 or above
 * ZERO_MAX_LEN, n_chunks < 0 or above INT32_MAX, bad hp), MISALIGNED,
 * UNSUPPORTED (gdt), ALIAS (a partial overlaps master, m or v, or those
 * overlap each other), NOT_DEVICE, HIP.
 */
int zero_shard_step(const void *const *partials, int n_ranks, int gdt,
                    float *master, float *m, float *v, int64_t shard_len,
                    const zero_chunk *d_chunks, int64_t n_chunks,
                    const zero_adamw_hparams *hp, hipStream_t stream);

/*
 * The fused step in buckets (ZeRO-2: "并行训练优化、MoE扩展与系统瓶颈", 2.2.4,
 * and "CS336 2026 Lecture 8: Parallelism Basics", the ZeRO-2 slides: each
 * gradient bucket is reduce-scattered as soon as it is complete, so its
 * slice of the shard can be stepped without waiting for the others).  One
 * call checks the whole shard as zero_shard_step does, then enqueues one
 * step launch per bucket on `stream`: bucket b covers chunks
 * [first[b], first[b] + count[b]) of d_chunks.  If `ready` is not NULL
 * and ready[b] is not NULL, the stream first waits for event ready[b] (for
 * example an event recorded when that bucket's gradients have arrived), so
 * the host can enqueue a whole overlapped step at once.
 * first, count, ready: host arrays of n_buckets entries.  Buckets must be
 * in increasing order, disjoint and inside the table (INVALID otherwise);
 * chunks outside every bucket are not stepped.  The result equals
 * zero_shard_step over the buckets' chunks, bit for bit.  Errors as
 * zero_shard_step; every non-NULL event is probed with hipEventQuery
 * before anything is enqueued, and an invalid one gives HIP with nothing
 * launched.  Unlike the other calls, this one enqueues several launches:
 * if the runtime reports an error at the wait or launch of bucket b (not
 * expected once the checks have passed), buckets before b are already
 * enqueued and will run, and HIP is returned.
 */
int zero_shard_step_buckets(const void *const *partials, int n_ranks, int gdt,
                            float *master, float *m, float *v, int64_t shard_len,
                            const zero_chunk *d_chunks, int64_t n_chunks,
                            const int64_t *first, const int64_t *count, int n_buckets,
                            const hipEvent_t *ready, const zero_adamw_hparams *hp,
                            hipStream_t stream);


/*
 * Extended reduce for data-parallel layouts beyond one flat group and for
 * more than one micro-batch per optimizer step.
 *
 * Two-level order (hybrid sharding, CS231n "Large-Scale Distributed
 * Training" notes, 4.4: N = M x K GPUs, sharded inside each group of K,
 * replicated across the M groups): partials m*K .. m*K+K-1 form group m;
 * each group is summed in rank order, then the group sums in group order,
 * all in double.  group = 0 or group = n_ranks is the flat order of
 * zero_shard_step; group = 1 gives the same bits too.  The shard geometry
 * then uses the K ranks of one group (zero_build_chunks with n_ranks = K),
 * while n_ranks here counts all N partials.
 *
 * Gradient accumulation ("并行训练优化、MoE扩展与系统瓶颈", 3.1: the effective
 * batch grows with the number of accumulation steps G): the gradient is the
 * mean over all N x G micro-batch gradients.  Micro-batches 0 .. G-2 go
 * through zero_accumulate_shard into an fp32 accumulator acc (after each,
 * acc = fp32(acc + that micro-batch's sum)); the step for the last one uses
 * g = fp32((acc + its sum) / (N G)).
 */
typedef struct zero_reduce_spec {
    int32_t group;          /* ranks per group of the two-level order; 0 = one group */
    int32_t micro_batches;  /* G >= 1 */
    const float *acc;       /* device, shard_len fp32: sum of micro-batches 0..G-2; NULL iff G == 1 */
} zero_reduce_spec;

/*
 * The fused shard step with the extended reduce: as zero_shard_step, with
 * g = fp32(((acc[i] if acc) + two-level sum) / (n_ranks * micro_batches)).
 * rs: host pointer.  Errors as zero_shard_step; INVALID also when group
 * does not divide n_ranks, micro_batches < 1, or acc is given iff
 * micro_batches == 1; ALIAS when acc overlaps master, m or v.
 */
int zero_shard_step_ex(const void *const *partials, int n_ranks, int gdt,
                       const zero_reduce_spec *rs, float *master, float *m, float *v,
                       int64_t shard_len, const zero_chunk *d_chunks, int64_t n_chunks,
                       const zero_adamw_hparams *hp, hipStream_t stream);

/*
 * One non-final micro-batch of gradient accumulation:
 * acc[i] = fp32((reset ? 0 : acc[i]) + two-level sum of p_0[i] .. p_{N-1}[i]),
 * i in [0, n); with reset the sum alone is rounded (a -0 sum stays -0).
 * group as in zero_reduce_spec.  acc must not overlap a partial (ALIAS).
 */
int zero_accumulate_shard(const void *const *partials, int n_ranks, int gdt, int group,
                          int64_t n, float *acc, int reset, hipStream_t stream);

/*
 * The fused step on the 12-bytes-per-parameter state ("并行训练优化、MoE扩展与
 * 系统瓶颈", 2.2.9: everything but the master weights in BF16 comes to about
 * 12 bytes per parameter): fp32 master, bf16 Adam moments m and v (16-bit
 * patterns, shard_len each, updated in place).  Reduce and AdamW as
 * zero_shard_step, with the moments widened exactly from bf16 and the new
 * m', v' rounded once, from double, to nearest-even bf16.  Moves 2N + 18
 * bytes per element (bf16 partials) instead of 2N + 26.  Errors as
 * zero_shard_step.
 */
int zero_shard_step_bf16_moments(const void *const *partials, int n_ranks, int gdt,
                                 float *master, uint16_t *m, uint16_t *v, int64_t shard_len,
                                 const zero_chunk *d_chunks, int64_t n_chunks,
                                 const zero_adamw_hparams *hp, hipStream_t stream);

/*
 * The fused step on the pure-bf16 state with a compensated update ("CS336
 * 2026 Lecture 8: Parallelism Basics", Slide 28 sizes its capacity table
 * with a pure-BF16/Kahan ledger): no fp32 master.  The bf16 parameters are
 * the weights: each chunk's dst holds the parameters of its shard elements
 * and is read and written in place.  comp, m, v: device, shard_len bf16
 * patterns each, in shard order, updated in place (comp starts at zero).
 * Per element, with g and u = mhat / (sqrt(vhat) + eps) as in
 * zero_shard_step_bf16_moments and theta the bf16 parameter:
 *   d = -lr (u + weight_decay theta),  y = d + comp,
 *   theta' = bf16(theta + y),  comp' = bf16(y - (theta' - theta)),
 * Kahan's compensated summation of the increments into theta; arithmetic
 * in double, every stored value rounded once to nearest-even bf16.  Moves
 * 2N + 16 bytes per element (bf16 partials).  The chunk table must cover
 * each shard element at most once (zero_build_chunks' tables do).  Errors
 * as zero_shard_step_bf16_moments, with comp in place of master.
 */
int zero_shard_step_kahan(const void *const *partials, int n_ranks, int gdt,
                          uint16_t *comp, uint16_t *m, uint16_t *v, int64_t shard_len,
                          const zero_chunk *d_chunks, int64_t n_chunks,
                          const zero_adamw_hparams *hp, hipStream_t stream);

/*
 * Step constants in device memory, for steps captured in a HIP graph.
 * A captured launch replays its arguments, so zero_shard_step's `hp`
 * would apply the same step t (the same bias corrections, the same lr) on
 * every replay.  Here the host forms the constants of each step of a run
 * in advance, with exactly the arithmetic of zero_shard_step, into a table
 * the caller keeps in device memory; a device counter names the entry the
 * next launch uses, so each replay applies the next step of the run.
 *
 * zero_make_step_consts (host only): out[i] = the constants of hps[i] for
 * i < count (host arrays; one entry per step, so a learning-rate schedule
 * is just a different lr per entry).  INVALID, with nothing written, if
 * count < 0, a pointer is NULL while count > 0, or any hps[i] is invalid
 * as for zero_shard_step.
 */
int zero_make_step_consts(const zero_adamw_hparams *hps, int64_t count, zero_step_consts *out);

/*
 * zero_shard_step with its constants read on the device when the kernel
 * runs: consts[*index] (consts: device array of n_consts entries, 16-byte
 * aligned; index: device int64, 8-byte aligned).  The result equals
 * zero_shard_step with the hparams that entry was made from, bit for bit.
 * If *index is outside [0, n_consts) when the kernel runs, nothing is
 * changed.  The call only reads the index; zero_step_index_advance moves it
 * on once the optimizer step is complete (after every bucket of it, when
 * the step is issued per bucket over sub-tables).
 * Errors as zero_shard_step; also INVALID for a NULL consts or index or
 * n_consts outside [1, INT32_MAX], MISALIGNED for a misaligned consts or
 * index, ALIAS when consts or the index overlaps master, m or v, and
 * NOT_DEVICE when either lies outside a device allocation.
 */
int zero_shard_step_scheduled(const void *const *partials, int n_ranks, int gdt,
                              float *master, float *m, float *v, int64_t shard_len,
                              const zero_chunk *d_chunks, int64_t n_chunks,
                              const zero_step_consts *consts, int64_t n_consts,
                              const int64_t *index, hipStream_t stream);

/*
 * The 12-byte and pure-bf16 steps with their constants read on the device,
 * as zero_shard_step_scheduled does for the 16-byte step.  Arguments as
 * zero_shard_step_bf16_moments and zero_shard_step_kahan, with consts,
 * n_consts and index in place of hp; results equal theirs bit for bit;
 * errors as zero_shard_step_scheduled.
 */
int zero_shard_step_bf16_moments_scheduled(const void *const *partials, int n_ranks, int gdt,
                                           float *master, uint16_t *m, uint16_t *v,
                                           int64_t shard_len, const zero_chunk *d_chunks,
                                           int64_t n_chunks, const zero_step_consts *consts,
                                           int64_t n_consts, const int64_t *index,
                                           hipStream_t stream);
int zero_shard_step_kahan_scheduled(const void *const *partials, int n_ranks, int gdt,
                                    uint16_t *comp, uint16_t *m, uint16_t *v, int64_t shard_len,
                                    const zero_chunk *d_chunks, int64_t n_chunks,
                                    const zero_step_consts *consts, int64_t n_consts,
                                    const int64_t *index, hipStream_t stream);

/*
 * Enqueue *index += 1 on `stream` (device int64, 8-byte aligned), applied
 * only if 0 <= *index < n_consts when it runs: the counter stops at
 * n_consts, past the last entry.  INVALID for a NULL index or
 * n_consts < 1; MISALIGNED; NOT_DEVICE; HIP.
 */
int zero_step_index_advance(int64_t *index, int64_t n_consts, hipStream_t stream);

/*
 * Reduce only: grad_out[i] = fp32((p_0[i] + ... + p_{N-1}[i]) / N),
 * i in [0, n), summed in double in rank order.  grad_out must not overlap
 * any partial (ALIAS).  n == 0 is a no-op.
 *
 * The local arithmetic of the gradient reduce-scatter: "CS336 2026 Lecture
 * 8: Parallelism Basics", Slide 8 (all-reduce = reduce-scatter +
 * all-gather), and "并行策略总览：六个维度各切什么、怎么通信", data-parallel
 * section (the full-batch gradient is the mean of the ranks' gradients,
 * because the loss is a sum over samples).
 */
int zero_reduce_shard(const void *const *partials, int n_ranks, int gdt, int64_t n,
                      float *grad_out, hipStream_t stream);

/*
 * AdamW only, from an fp32 gradient: master, m, v (n elements each) are
 * updated in place exactly as in zero_shard_step.  grad must not overlap
 * master, m or v (ALIAS).  n == 0 is a no-op.
 *
 * The optimizer state is the fp32 master copy and Adam's two moments of
 * "CS336 2026 Lecture 8: Parallelism Basics", Slide 17 (the
 * 16-bytes-per-parameter ledger); the pages name the state but not the
 * update, which is read as decoupled-weight-decay AdamW with bias
 * correction (the formula in the file comment above).
 */
int zero_adamw_shard(const float *grad, float *master, float *m, float *v, int64_t n,
                     const zero_adamw_hparams *hp, hipStream_t stream);

/*
 * bf16 write only: for every chunk c and j < c.len,
 * c.dst[j] = bf16(master[c.shard_off + j]).  master holds shard_len fp32
 * elements; chunks outside [0, shard_len) are skipped.
 *
 * The local half of the parameter all-gather: "CS336 2026 Lecture 8:
 * Parallelism Basics", Slide 20, fourth step (each rank's updated segment
 * goes back into the full bf16 parameters).
 */
int zero_gather_write(const float *master, int64_t shard_len, const zero_chunk *d_chunks,
                      int64_t n_chunks, hipStream_t stream);

/* Static description of a return code. */
const char *zero_strerror(int code);

/* Library version, (major << 16) | minor. */
int zero_version(void);

/*
 * Measurement aid, not part of the step: copies `bytes` bytes from src to
 * dst (device, 16-byte aligned, non-overlapping) with a streaming kernel.
 * Used to calibrate HBM traffic counters and the attainable copy bandwidth.
 */
int zero_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

/*
 * Measurement aid, not part of the step: reads `bytes` bytes at src (device,
 * 16-byte aligned) with a streaming kernel and writes nothing, except that
 * if the XOR of the words one lane read equals `magic` it stores that value
 * to *sink (device, 4-byte aligned, caller-owned).  Gives the attainable
 * read-only HBM rate beside the copy rate.
 * Errors: INVALID (null with bytes > 0, bytes < 0), MISALIGNED, NOT_DEVICE.
 */
int zero_probe_read(const void *src, int64_t bytes, uint32_t *sink, uint32_t magic,
                    hipStream_t stream);

/*
 * Measurement aid, not part of the step: writes `value` to every 32-bit word
 * of dst (device, 16-byte aligned; a trailing partial word gets its low
 * bytes) with the step kernels' non-temporal 16-byte stores.  Gives the
 * attainable write-only HBM rate beside the read and copy rates.
 * Errors: INVALID (null with bytes > 0, bytes < 0), MISALIGNED, NOT_DEVICE.
 */
int zero_probe_write(void *dst, int64_t bytes, uint32_t value, hipStream_t stream);

#define ZERO_PROBE_SUM_MAX 16

/*
 * Measurement aid, not part of the step: dst[i] = src[0][i] + ... +
 * src[k-1][i] for i < n, in fp32, added in that order, with one 64-lane
 * workgroup per 1 KiB of dst and non-temporal loads and stores.  k = 1 is a
 * copy.  Shows how the attainable rate of a mixed stream falls as the
 * number of arrays streamed at once grows, beside the step (which streams
 * N partials, three state arrays in place and the parameters).
 * src: k device pointers (host array of pointers), each 16-byte aligned and
 * n floats long; sources may overlap each other, not dst.  dst: device,
 * 16-byte aligned, n floats.
 * Errors: INVALID (src NULL, k outside 1..ZERO_PROBE_SUM_MAX, n < 0 or
 * above ZERO_MAX_LEN / 4, a NULL source or dst with n > 0), MISALIGNED,
 * ALIAS (dst overlaps a source), NOT_DEVICE.  n = 0 launches nothing.
 */
int zero_probe_sum(const float *const *src, int k, float *dst, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
