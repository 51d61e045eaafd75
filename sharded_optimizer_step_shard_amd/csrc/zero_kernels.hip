// HIP kernels of the ZeRO shard step for gfx950 (CDNA4, wave64).
//
// The step is a pure stream: every shard element is read once from each of
// the N gradient partials and from the fp32 master, m and v, and written
// once to master, m, v and the bf16 parameter slot.  Nothing is reused, so
// the bound is HBM bandwidth: (2N + 26) bytes per element with bf16
// partials, (4N + 26) with fp32 partials.  There is no contraction here,
// so no MFMA; the kernels are built around 16-byte per-lane accesses that
// a wave turns into fully coalesced 1 KiB requests.
//
// Work split: one workgroup (a single wave of 64 lanes) per chunk of the
// chunk table (a workgroup loops over chunks when the table is longer than
// the grid cap).  A lane handles a group of VEC consecutive elements (8
// with bf16 partials: one 16-byte load per partial; 4 with fp32 partials),
// strided by the wave width; the default 2048-element chunk is four groups
// per lane.  Groups sit on the shard's VEC-element grid, so all
// partial and state loads are 16-byte aligned; a chunk that starts or ends
// off the grid handles its first or last group element by element.
//
// Arithmetic follows the fixed evaluation order in include/zero_shard.h:
// double sums in rank order, IEEE double AdamW without contraction (the
// library is built with -ffp-contract=off), one rounding per stored value.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "zero_internal.h"

namespace zs {

constexpr int kBlock = 256;       // grid-stride kernels (unfused path)
constexpr int kStepBlock = 64;    // chunk-table kernels: one wave per workgroup
constexpr int kStepLanes = 64;    // lanes of a wave (gfx950: wave64)

// Native clang vectors: 16-byte (and 8-byte) loads and stores, and the
// non-temporal store builtin, need them rather than HIP's struct wrappers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN keeps its sign and top payload
// bits with the quiet bit set; overflow gives inf.  gfx950 converts in one
// instruction (v_cvt_pk_bf16_f32).  On MI355X its result equals, for all
// 2^32 fp32 patterns, the integer rounding (u + 0x7FFF + kept lsb) >> 16
// with NaN mapped to (u >> 16) | 0x40, which is what the oracle computes.
__device__ __forceinline__ uint32_t to_bf16(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Sum -> fp32 mean.  With N a compile-time power of two the division is a
// multiplication by the exact 1/N (same bits); otherwise the host's pow2
// flag picks it at run time.
template <int NC>
__device__ __forceinline__ float finish_reduce(double s, const ReduceScalars &r)
{
    if constexpr (NC > 0 && (NC & (NC - 1)) == 0)
        return (float)(s * r.inv_n);
    else
        return (float)(r.pow2 ? s * r.inv_n : s / r.n);
}

// Adam's moments and update direction mhat / (sqrt(vhat) + eps) for one
// element, all in double; the caller stores m1, v1 in their format.
__device__ __forceinline__ double adam_dir(float g32, double m0, double v0, double &m1, double &v1,
                                           const StepScalars &k)
{
    double g = (double)g32;
    m1 = k.b1 * m0 + k.c1 * g;
    v1 = k.b2 * v0 + k.c2 * (g * g);
    double mhat = m1 / k.bc1;
    double vhat = v1 / k.bc2;
    return mhat / (__builtin_sqrt(vhat) + k.eps);
}

// AdamW on one element: moments in and out in double (the caller stores
// them in their format), master in and out in fp32.
__device__ __forceinline__ void adamw_d(float g32, float &th, double m0, double v0, double &m1,
                                        double &v1, const StepScalars &k)
{
    double upd = adam_dir(g32, m0, v0, m1, v1, k);
    double t1 = (double)th * k.dec - k.lr * upd;
    th = (float)t1;
}

__device__ __forceinline__ void adamw(float g32, float &th, float &m, float &v, const StepScalars &k)
{
    double m1, v1;
    adamw_d(g32, th, (double)m, (double)v, m1, v1, k);
    m = (float)m1;
    v = (float)v1;
}

// double -> bf16 with a single nearest-even rounding: first round to fp32
// by round-to-odd (truncate toward zero, then set the last bit if anything
// was dropped), then round that to bf16 to nearest even.  fp32 keeps 16
// more bits than bf16 at every magnitude, subnormals included, so the odd
// bit stands in for everything below it and the second rounding is the
// correct one (Boldo & Melquiond, round-to-odd).
__device__ __forceinline__ uint32_t bf16_from_double(double d)
{
    const float f = (float)d;
    const double fd = (double)f;
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(fd) > __builtin_fabs(d))
        u -= 1;                       // rounded away from zero: one step back
    if (fd != d)
        u |= 1;                       // inexact: make it odd
    return to_bf16(__uint_as_float(u));
}

__device__ __forceinline__ double bf16_to_double(uint32_t h) { return (double)__uint_as_float(h << 16); }

// One element of the pure-bf16 step: AdamW's increment -lr (u + wd theta)
// added to the bf16 parameter by Kahan's compensated summation, the bf16
// compensation c holding the part theta has not absorbed yet:
//   y = d + c,  theta' = bf16(theta + y),  c' = bf16(y - (theta' - theta)).
// Everything in double; each stored value (theta', c', m', v') is rounded
// once to nearest-even bf16.  Bit patterns in and out.
__device__ __forceinline__ void kahan_elem(float g32, uint32_t &th, uint32_t &c, uint32_t &m,
                                           uint32_t &v, const StepScalars &k)
{
    double m1, v1;
    const double upd = adam_dir(g32, bf16_to_double(m), bf16_to_double(v), m1, v1, k);
    const double t0 = bf16_to_double(th);
    const double d = -k.lr * (upd + k.wd * t0);
    const double y = d + bf16_to_double(c);
    const uint32_t t1 = bf16_from_double(t0 + y);
    const double moved = bf16_to_double(t1) - t0;
    c = bf16_from_double(y - moved);
    th = t1;
    m = bf16_from_double(m1);
    v = bf16_from_double(v1);
}

template <typename T>
__device__ __forceinline__ T ld(const T *p) { return *p; }

// The chunk table is read-only for the whole launch; reading it through the
// constant address space lets the compiler use scalar loads for the
// (uniform) descriptor instead of one vector load per lane.
typedef __attribute__((address_space(4))) const int64_t const_i64;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const double const_f64;

__device__ __forceinline__ zero_chunk chunk_at(const zero_chunk *table, int64_t ci)
{
    const char *p = (const char *)(table + __builtin_amdgcn_readfirstlane((int)ci));
    zero_chunk c;
    c.shard_off = *(const_i64 *)(p + offsetof(zero_chunk, shard_off));
    c.dst = (uint16_t *)(uintptr_t)*(const_i64 *)(p + offsetof(zero_chunk, dst));
    c.len = *(const_i32 *)(p + offsetof(zero_chunk, len));
    c.tensor_id = *(const_i32 *)(p + offsetof(zero_chunk, tensor_id));
    c.tensor_off = *(const_i64 *)(p + offsetof(zero_chunk, tensor_off));
    return c;
}

template <typename T>
__device__ __forceinline__ void st_nt(T *p, T x) { __builtin_nontemporal_store(x, p); }

// Per gradient dtype: group width and how a 16-byte raw vector widens.
template <zero_dtype G> struct Grad;

template <> struct Grad<ZERO_BF16> {
    static constexpr int VEC = 8;
    static constexpr int BYTES = 2;
    __device__ static __forceinline__ void first(double *s, u32x4 r)
    {
        s[0] = bf16_lo(r.x); s[1] = bf16_hi(r.x); s[2] = bf16_lo(r.y); s[3] = bf16_hi(r.y);
        s[4] = bf16_lo(r.z); s[5] = bf16_hi(r.z); s[6] = bf16_lo(r.w); s[7] = bf16_hi(r.w);
    }
    __device__ static __forceinline__ void add(double *s, u32x4 r)
    {
        s[0] = s[0] + bf16_lo(r.x); s[1] = s[1] + bf16_hi(r.x);
        s[2] = s[2] + bf16_lo(r.y); s[3] = s[3] + bf16_hi(r.y);
        s[4] = s[4] + bf16_lo(r.z); s[5] = s[5] + bf16_hi(r.z);
        s[6] = s[6] + bf16_lo(r.w); s[7] = s[7] + bf16_hi(r.w);
    }
    __device__ static __forceinline__ double one(const void *p, int64_t i)
    {
        return (double)__uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
    }
};

template <> struct Grad<ZERO_FP32> {
    static constexpr int VEC = 4;
    static constexpr int BYTES = 4;
    __device__ static __forceinline__ void first(double *s, u32x4 r)
    {
        s[0] = (double)__uint_as_float(r.x); s[1] = (double)__uint_as_float(r.y);
        s[2] = (double)__uint_as_float(r.z); s[3] = (double)__uint_as_float(r.w);
    }
    __device__ static __forceinline__ void add(double *s, u32x4 r)
    {
        s[0] = s[0] + (double)__uint_as_float(r.x); s[1] = s[1] + (double)__uint_as_float(r.y);
        s[2] = s[2] + (double)__uint_as_float(r.z); s[3] = s[3] + (double)__uint_as_float(r.w);
    }
    __device__ static __forceinline__ double one(const void *p, int64_t i)
    {
        return (double)((const float *)p)[i];
    }
};

// Gradient partials are read exactly once: non-temporal loads stream them
// past the caches, which stay with the master, m and v lines that are read
// and then rewritten in place.  (Measured on MI355X: +2-4% on the 7B and
// 70B shards; non-temporal loads of the state as well cost ~15%.)
__device__ __forceinline__ u32x4 ld_raw(const void *base, int64_t byte_off)
{
    return __builtin_nontemporal_load((const u32x4 *)((const char *)base + byte_off));
}

// Sum of the N partials over one full group starting at element i0, in
// rank order.  NC > 0: N known at compile time, the loads issued in batches
// of up to BATCH before their adds (the batch changes how many loads are in
// flight, never the order of the sum); NC == 0: N at run time.
template <zero_dtype G, int NC, int BATCH = 16>
__device__ __forceinline__ void group_sum(double *s, const PartialPtrs &pp, int n_rt, int64_t i0)
{
    using GT = Grad<G>;
    const int64_t off = i0 * GT::BYTES;
    if constexpr (NC > 0) {
        constexpr int B = NC < BATCH ? NC : BATCH;
#pragma unroll
        for (int kb = 0; kb < NC; kb += B) {
            u32x4 raw[B];
#pragma unroll
            for (int j = 0; j < B; ++j)
                raw[j] = ld_raw(pp.p[kb + j], off);
            // Keep the batch's loads (and any issued before them) ahead of
            // the arithmetic: a stream kernel wants every request in flight.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (kb + j == 0)
                    GT::first(s, raw[j]);
                else
                    GT::add(s, raw[j]);
            }
        }
    } else {
        GT::first(s, ld_raw(pp.p[0], off));
#pragma unroll 4
        for (int k = 1; k < n_rt; ++k)
            GT::add(s, ld_raw(pp.p[k], off));
    }
}

template <zero_dtype G>
__device__ __forceinline__ double elem_sum(const PartialPtrs &pp, int n, int64_t i)
{
    double s = Grad<G>::one(pp.p[0], i);
    for (int k = 1; k < n; ++k)
        s = s + Grad<G>::one(pp.p[k], i);
    return s;
}

// Two-level order (hybrid sharding): ranks m*K .. m*K+K-1 form group m; the
// partials of a group are folded in rank order into t, and the group sums
// into s in group order.  K = n gives the flat fold.  K is uniform, so the
// group-boundary tests are scalar branches.
template <zero_dtype G, int VEC>
__device__ __forceinline__ void fold_two_level(double *s, double *t, u32x4 raw, int k, int K)
{
    double x[VEC];
    Grad<G>::first(x, raw);
    if (k % K == 0) {
        if (k == K) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) s[j] = t[j];
        } else if (k > K) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) s[j] = s[j] + t[j];
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) t[j] = x[j];
    } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) t[j] = t[j] + x[j];
    }
}

template <int VEC>
__device__ __forceinline__ void fold_finish(double *s, const double *t, int n, int K)
{
    if (n == K) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) s[j] = t[j];
    } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) s[j] = s[j] + t[j];
    }
}

// KC > 0: group size known at compile time, so after unrolling every group
// boundary test folds away; KC == 0: K at run time (scalar branches).
template <zero_dtype G, int NC, int KC, int BATCH = 16>
__device__ __forceinline__ void group_sum_two_level(double *s, const PartialPtrs &pp, int n_rt,
                                                    int K_rt, int64_t i0)
{
    const int K = KC > 0 ? KC : K_rt;
    using GT = Grad<G>;
    constexpr int VEC = GT::VEC;
    const int64_t off = i0 * GT::BYTES;
    double t[VEC];
    if constexpr (NC > 0) {
        constexpr int B = NC < BATCH ? NC : BATCH;
#pragma unroll
        for (int kb = 0; kb < NC; kb += B) {
            u32x4 raw[B];
#pragma unroll
            for (int j = 0; j < B; ++j)
                raw[j] = ld_raw(pp.p[kb + j], off);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < B; ++j)
                fold_two_level<G, VEC>(s, t, raw[j], kb + j, K);
        }
        fold_finish<VEC>(s, t, NC, K);
    } else {
        for (int k = 0; k < n_rt; ++k)
            fold_two_level<G, VEC>(s, t, ld_raw(pp.p[k], off), k, K);
        fold_finish<VEC>(s, t, n_rt, K);
    }
}

template <zero_dtype G>
__device__ __forceinline__ double elem_sum_two_level(const PartialPtrs &pp, int n, int K, int64_t i)
{
    double s = 0.0, t = 0.0;
    for (int k = 0; k < n; ++k) {
        const double x = Grad<G>::one(pp.p[k], i);
        if (k % K == 0) {
            if (k == K)
                s = t;
            else if (k > K)
                s = s + t;
            t = x;
        } else {
            t = t + x;
        }
    }
    return n == K ? t : s + t;
}

// VEC fp32 values (4 or 8) at a 16-byte aligned address, moved with
// 16-byte loads and non-temporal 16-byte stores.
template <int VEC> struct F32x {
    float e[VEC];
    __device__ __forceinline__ void load(const float *p)
    {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            f32x4 t = ld((const f32x4 *)p + q);
            e[4 * q + 0] = t.x; e[4 * q + 1] = t.y; e[4 * q + 2] = t.z; e[4 * q + 3] = t.w;
        }
    }
    __device__ __forceinline__ void store(float *p) const
    {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            f32x4 t = {e[4 * q + 0], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]};
            st_nt((f32x4 *)p + q, t);
        }
    }
    __device__ __forceinline__ float &operator[](int j) { return e[j]; }
};

// VEC bf16 values at an aligned address (16 bytes for VEC = 8, 8 for 4):
// the moments of the 12-byte state.
template <int VEC> struct B16x {
    uint32_t e[VEC];
    __device__ __forceinline__ void load(const uint16_t *p)
    {
        if constexpr (VEC == 8) {
            u32x4 w = ld((const u32x4 *)p);
            e[0] = w.x & 0xFFFFu; e[1] = w.x >> 16; e[2] = w.y & 0xFFFFu; e[3] = w.y >> 16;
            e[4] = w.z & 0xFFFFu; e[5] = w.z >> 16; e[6] = w.w & 0xFFFFu; e[7] = w.w >> 16;
        } else {
            u32x2 w = ld((const u32x2 *)p);
            e[0] = w.x & 0xFFFFu; e[1] = w.x >> 16; e[2] = w.y & 0xFFFFu; e[3] = w.y >> 16;
        }
    }
    __device__ __forceinline__ void store(uint16_t *p) const
    {
        if constexpr (VEC == 8) {
            u32x4 w = {e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
            st_nt((u32x4 *)p, w);
        } else {
            u32x2 w = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            st_nt((u32x2 *)p, w);
        }
    }
};

// VEC bf16 values: one 16-byte (VEC = 8) or 8-byte (VEC = 4) store when the
// destination is aligned for it, else element by element.
template <int VEC>
__device__ __forceinline__ void store_bf16(uint16_t *dst, const uint32_t *h, bool vec_ok)
{
    if (vec_ok) {
        if constexpr (VEC == 8) {
            u32x4 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            st_nt((u32x4 *)dst, w);
        } else {
            u32x2 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            st_nt((u32x2 *)dst, w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            dst[j] = (uint16_t)h[j];
    }
}

// The bf16 parameter stores of one chunk.  A destination aligned for vector
// stores gets one per lane group (store_bf16).  A misaligned one -- a tensor
// that starts at an arbitrary element, so every group of the chunk lands
// s0 elements short of an aligned slot -- would otherwise take VEC 2-byte
// stores per lane.  On a chunk whose groups are all full (it starts and ends
// on the VEC grid), the lane that owns chunk group g instead writes the
// aligned slot that straddles groups g - 1 and g: the last VEC - s0 values of
// group g - 1, which come from the previous lane by a wave shuffle (for
// lane 0, from lane 63 of the previous pass), then its own first s0 values.
// Only the chunk's first s0 elements (before its first aligned slot) and
// its last VEC - s0 are stored element by element, by the lanes that own
// them.  Every destination element is written exactly once.
template <int VEC>
struct ParamStore {
    static constexpr int W = VEC / 2;   // 32-bit words per lane group
    uint16_t *dst;
    int64_t lo, hi;
    bool vec_ok, shift;
    int s0;                             // elements before the first aligned slot
    uint32_t carry[W];                  // the previous pass's lane-63 group

    __device__ __forceinline__ ParamStore(uint16_t *d, int64_t lo_, int64_t hi_, bool ok)
        : dst(d), lo(lo_), hi(hi_), vec_ok(ok)
    {
        const int m = (int)(((uintptr_t)d >> 1) % VEC);   // elements past an aligned slot
        shift = !ok && ((uintptr_t)d & 1) == 0 && lo % VEC == 0 && hi % VEC == 0;
        s0 = VEC - m;
#pragma unroll
        for (int q = 0; q < W; ++q)
            carry[q] = 0;
    }

    // out = values [s0, s0 + VEC) of the 2 VEC values prev ++ cur (S = s0
    // known at compile time; s0 is uniform, so the switch below is scalar)
    template <int S>
    __device__ static __forceinline__ void join(uint32_t *out, const uint32_t *prev, const uint32_t *cur)
    {
        uint32_t all[2 * W];
#pragma unroll
        for (int q = 0; q < W; ++q) {
            all[q] = prev[q];
            all[W + q] = cur[q];
        }
#pragma unroll
        for (int q = 0; q < W; ++q) {
            constexpr int wq = S / 2;
            if constexpr (S % 2 == 0)
                out[q] = all[wq + q];
            else
                out[q] = (all[wq + q] >> 16) | (all[wq + q + 1] << 16);
        }
    }

    // the full group starting at shard element i0, values h[0 .. VEC)
    __device__ __forceinline__ void put(int64_t i0, const uint32_t *h)
    {
        uint16_t *d = dst + (i0 - lo);
        if (!shift) {
            store_bf16<VEC>(d, h, vec_ok);
            return;
        }
        uint32_t w[W], prev[W];
#pragma unroll
        for (int q = 0; q < W; ++q) {
            w[q] = h[2 * q] | (h[2 * q + 1] << 16);
            prev[q] = __shfl_up(w[q], 1u);
        }
        if (threadIdx.x == 0) {
#pragma unroll
            for (int q = 0; q < W; ++q)
                prev[q] = carry[q];
        }
#pragma unroll
        for (int q = 0; q < W; ++q)
            carry[q] = __shfl(w[q], kStepLanes - 1);
        if (i0 == lo) {
            for (int j = 0; j < s0; ++j)
                d[j] = (uint16_t)h[j];
        } else {
            uint32_t o[W];
            switch (s0) {
            case 1: join<1>(o, prev, w); break;
            case 2: join<2>(o, prev, w); break;
            case 3: join<3>(o, prev, w); break;
            case 4: if constexpr (VEC > 4) { join<4>(o, prev, w); break; } else { return; }
            case 5: if constexpr (VEC > 5) { join<5>(o, prev, w); break; } else { return; }
            case 6: if constexpr (VEC > 6) { join<6>(o, prev, w); break; } else { return; }
            case 7: if constexpr (VEC > 7) { join<7>(o, prev, w); break; } else { return; }
            default: return;
            }
            uint16_t *slot = d - VEC + s0;     // aligned for a VEC-element store
            if constexpr (VEC == 8)
                st_nt((u32x4 *)slot, (u32x4){o[0], o[1], o[2], o[3]});
            else
                st_nt((u32x2 *)slot, (u32x2){o[0], o[1]});
        }
        if (i0 + VEC == hi) {
            for (int j = s0; j < VEC; ++j)
                d[j] = (uint16_t)h[j];
        }
    }
};

// ---------------------------------------------------------------- fused step

// Partial loads in flight per batch (group_sum) for each fused step, from
// in-process sweeps on MI355X (bitwise-equal results): batches of 8 beat 16
// for the one-wave 16-byte step with 16 or 32 partials (70B: +1-4%, 32 fp32
// partials: +1%); the 12-byte step takes 2 with two waves per SIMD (7B:
// 0.665 -> 0.684 of peak), 8 with three and 16 with one (kM16Batch); the
// pure-bf16 step keeps 16 (smaller batches were up to 3% slower at 70B).
constexpr int kStepBatch = 8;

// EXT: the extended reduce of zero_shard_step_ex (two-level order, optional
// accumulator of earlier micro-batches, divisor N * micro-batches).
// DIV (extended step only): 1 when that divisor is a power of two (multiply
// by its exact reciprocal), 2 otherwise (divide); 0 leaves the choice to
// finish_reduce.
template <zero_dtype G, int NC, bool EXT, int KC, int DIV = 0>
__device__ __forceinline__ void step_chunk(const StepArgs &a, const zero_chunk &c,
                                           const StepScalars &k)
{
    constexpr int VEC = Grad<G>::VEC;
    if (c.len <= 0 || c.shard_off < 0 || c.shard_off > a.shard_len - c.len)
        return;
    const int n = NC > 0 ? NC : a.red.n_ranks;
    const int64_t lo = c.shard_off, hi = c.shard_off + c.len;
    const int64_t g0 = lo / VEC, g1 = (hi + VEC - 1) / VEC;
    // dst address of the first element of group g0, aligned for a vector store?
    const bool vec_ok = (((uintptr_t)c.dst - (uintptr_t)(2 * (lo - g0 * VEC))) % (2 * VEC)) == 0;
    ParamStore<VEC> ps(c.dst, lo, hi, vec_ok);

    for (int64_t g = g0 + threadIdx.x; g < g1; g += kStepBlock) {
        const int64_t i0 = g * VEC;
        uint16_t *d = c.dst + (i0 - lo);
        if (i0 >= lo && i0 + VEC <= hi) {
            double s[VEC];
            F32x<VEC> th, m, v;
            th.load(a.master + i0);
            m.load(a.m + i0);
            v.load(a.v + i0);
            if constexpr (EXT) {
                F32x<VEC> acc;
                if (a.acc)
                    acc.load(a.acc + i0);
                if constexpr (KC < 0)
                    group_sum<G, NC, kStepBatch>(s, a.parts, n, i0);
                else
                    group_sum_two_level<G, NC, KC, kStepBatch>(s, a.parts, n, a.red.group, i0);
                if (a.acc) {
#pragma unroll
                    for (int j = 0; j < VEC; ++j)
                        s[j] = (double)acc[j] + s[j];
                }
            } else {
                group_sum<G, NC, kStepBatch>(s, a.parts, n, i0);
            }
            uint32_t h[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                float gj;
                if constexpr (DIV == 1)
                    gj = (float)(s[j] * a.red.inv_n);
                else if constexpr (DIV == 2)
                    gj = (float)(s[j] / a.red.n);
                else
                    gj = finish_reduce<EXT ? 0 : NC>(s[j], a.red);
                adamw(gj, th[j], m[j], v[j], k);
                h[j] = to_bf16(th[j]);
            }
            th.store(a.master + i0);
            m.store(a.m + i0);
            v.store(a.v + i0);
            ps.put(i0, h);
        } else {
            for (int j = 0; j < VEC; ++j) {
                const int64_t i = i0 + j;
                if (i < lo || i >= hi)
                    continue;
                float gj;
                if constexpr (EXT) {
                    double e = elem_sum_two_level<G>(a.parts, n, a.red.group, i);
                    if (a.acc)
                        e = (double)a.acc[i] + e;
                    gj = finish_reduce<0>(e, a.red);
                } else {
                    gj = finish_reduce<NC>(elem_sum<G>(a.parts, n, i), a.red);
                }
                float th = a.master[i], m = a.m[i], v = a.v[i];
                adamw(gj, th, m, v, k);
                a.master[i] = th;
                a.m[i] = m;
                a.v[i] = v;
                d[j] = (uint16_t)to_bf16(th);
            }
        }
    }
}

// Resident waves per SIMD of the 12-byte and pure-bf16 steps.  Both do more
// arithmetic per byte moved than the 16-byte step (bf16 moments rounded from
// double; the compensated update on top), and when the N partials are few
// bytes per element one wave per SIMD leaves the memory pipe idle during its
// arithmetic.  Measured on MI355X (7B shard, N = 8 bf16): the 12-byte step
// 0.65 -> 0.67 of HBM peak with two waves, the pure-bf16 step 0.47 -> 0.655
// with three; with 16 partials (70B) the 12-byte step is best with one wave
// (0.725 against 0.69), the pure-bf16 step with two (0.63 -> 0.71; its
// registers allow no third).
//
// SMALL: a launch of at most ZERO_SMALL_LAUNCH_CHUNKS_12B chunks, where the
// launch's ramp and tail weigh more; there the 12-byte step with few
// partials runs three waves with batches of 8.  Measured with each launch on
// the next of enough buffer sets to keep the working set (over 2 GB) out of
// the 256 MB last-level cache (N = 8 bf16, chunks of 2048, one process, two
// waves / three): 2M-element shards 0.39 / 0.41-0.43, 4M 0.45-0.48 /
// 0.48-0.51, 8M 0.51-0.55 / 0.53-0.56, 16M 0.55-0.60 / 0.60-0.61, 32M
// 0.59-0.64 / 0.64-0.65; 128M and 256M (one buffer set) 0.64-0.69 /
// 0.67-0.68.  The pure-bf16 step gained nothing from two or four waves on
// the GPT-2 shard.
template <zero_dtype G, int NC, bool SMALL>
constexpr int kM16Waves = (NC > 0 && NC * Grad<G>::BYTES <= 16) ? (SMALL ? 3 : 2) : 1;
constexpr int kKahanWaves = 3;
// Partial-load batch of the 12-byte step: 2 with two waves per SIMD, 8 with
// three, 16 with one (more than 16 bytes of partials per element, or N known
// only at run time; at N = 16 bf16 that is every partial of a group at once).
// One wave with batches of 16 against 8, one process each on three boxes,
// 70B shard: 0.752 / 0.741 / 0.757 against 0.728 / 0.727 / 0.738; ragged fp32
// shard (32 partials): 0.687 against 0.687.
template <zero_dtype G, int NC, bool SMALL>
constexpr int kM16Batch = kM16Waves<G, NC, SMALL> == 2 ? 2
                                                       : (kM16Waves<G, NC, SMALL> == 1 ? 16 : kStepBatch);

// The step on the 12-byte state: fp32 master, bf16 m and v (in a.m, a.v
// as 16-bit patterns).  Same reduce and AdamW; the moments are read from
// bf16 and rounded back to bf16 once, from double.
template <zero_dtype G, int NC, bool SMALL>
__device__ __forceinline__ void step_chunk_m16(const StepArgs &a, const zero_chunk &c,
                                               const StepScalars &k)
{
    constexpr int VEC = Grad<G>::VEC;
    if (c.len <= 0 || c.shard_off < 0 || c.shard_off > a.shard_len - c.len)
        return;
    const int n = NC > 0 ? NC : a.red.n_ranks;
    uint16_t *const m16 = (uint16_t *)a.m, *const v16 = (uint16_t *)a.v;
    const int64_t lo = c.shard_off, hi = c.shard_off + c.len;
    const int64_t g0 = lo / VEC, g1 = (hi + VEC - 1) / VEC;
    const bool vec_ok = (((uintptr_t)c.dst - (uintptr_t)(2 * (lo - g0 * VEC))) % (2 * VEC)) == 0;
    ParamStore<VEC> ps(c.dst, lo, hi, vec_ok);
    for (int64_t g = g0 + threadIdx.x; g < g1; g += kStepBlock) {
        const int64_t i0 = g * VEC;
        uint16_t *d = c.dst + (i0 - lo);
        if (i0 >= lo && i0 + VEC <= hi) {
            double s[VEC];
            F32x<VEC> th;
            B16x<VEC> m, v;
            th.load(a.master + i0);
            m.load(m16 + i0);
            v.load(v16 + i0);
            group_sum<G, NC, kM16Batch<G, NC, SMALL>>(s, a.parts, n, i0);
            uint32_t h[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                double m1, v1;
                adamw_d(finish_reduce<NC>(s[j], a.red), th[j], bf16_to_double(m.e[j]),
                        bf16_to_double(v.e[j]), m1, v1, k);
                m.e[j] = bf16_from_double(m1);
                v.e[j] = bf16_from_double(v1);
                h[j] = to_bf16(th[j]);
            }
            th.store(a.master + i0);
            m.store(m16 + i0);
            v.store(v16 + i0);
            ps.put(i0, h);
        } else {
            for (int j = 0; j < VEC; ++j) {
                const int64_t i = i0 + j;
                if (i < lo || i >= hi)
                    continue;
                float th = a.master[i];
                double m1, v1;
                adamw_d(finish_reduce<NC>(elem_sum<G>(a.parts, n, i), a.red), th,
                        bf16_to_double(m16[i]), bf16_to_double(v16[i]), m1, v1, k);
                a.master[i] = th;
                m16[i] = (uint16_t)bf16_from_double(m1);
                v16[i] = (uint16_t)bf16_from_double(v1);
                d[j] = (uint16_t)to_bf16(th);
            }
        }
    }
}

// The pure-bf16 step: the parameters are read from and written back to
// the chunk's destination (the bf16 parameter is the only copy of the
// weight), with bf16 compensation, m and v in shard order.
template <zero_dtype G, int NC>
__device__ __forceinline__ void step_chunk_kahan(const StepArgs &a, const zero_chunk &c,
                                                 const StepScalars &k)
{
    constexpr int VEC = Grad<G>::VEC;
    if (c.len <= 0 || c.shard_off < 0 || c.shard_off > a.shard_len - c.len)
        return;
    const int n = NC > 0 ? NC : a.red.n_ranks;
    uint16_t *const m16 = (uint16_t *)a.m, *const v16 = (uint16_t *)a.v, *const c16 = a.comp;
    const int64_t lo = c.shard_off, hi = c.shard_off + c.len;
    const int64_t g0 = lo / VEC, g1 = (hi + VEC - 1) / VEC;
    const bool vec_ok = (((uintptr_t)c.dst - (uintptr_t)(2 * (lo - g0 * VEC))) % (2 * VEC)) == 0;
    for (int64_t g = g0 + threadIdx.x; g < g1; g += kStepBlock) {
        const int64_t i0 = g * VEC;
        uint16_t *d = c.dst + (i0 - lo);
        if (i0 >= lo && i0 + VEC <= hi) {
            double s[VEC];
            B16x<VEC> th, cm, m, v;
            if (vec_ok) {
                th.load(d);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    th.e[j] = d[j];
            }
            cm.load(c16 + i0);
            m.load(m16 + i0);
            v.load(v16 + i0);
            group_sum<G, NC>(s, a.parts, n, i0);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                kahan_elem(finish_reduce<NC>(s[j], a.red), th.e[j], cm.e[j], m.e[j], v.e[j], k);
            cm.store(c16 + i0);
            m.store(m16 + i0);
            v.store(v16 + i0);
            store_bf16<VEC>(d, th.e, vec_ok);
        } else {
            for (int j = 0; j < VEC; ++j) {
                const int64_t i = i0 + j;
                if (i < lo || i >= hi)
                    continue;
                uint32_t th = d[j], cm = c16[i], m = m16[i], v = v16[i];
                kahan_elem(finish_reduce<NC>(elem_sum<G>(a.parts, n, i), a.red), th, cm, m, v, k);
                d[j] = (uint16_t)th;
                c16[i] = (uint16_t)cm;
                m16[i] = (uint16_t)m;
                v16[i] = (uint16_t)v;
            }
        }
    }
}

template <zero_dtype G, int NC>
__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, kKahanWaves)))
void shard_step_kahan_kernel(StepArgs a)
{
    for (int64_t ci = blockIdx.x; ci < a.n_chunks; ci += gridDim.x)
        step_chunk_kahan<G, NC>(a, chunk_at(a.chunks, ci), a.k);
}

template <zero_dtype G, int NC, bool SMALL>
__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, kM16Waves<G, NC, SMALL>)))
void shard_step_m16_kernel(StepArgs a)
{
    for (int64_t ci = blockIdx.x; ci < a.n_chunks; ci += gridDim.x)
        step_chunk_m16<G, NC, SMALL>(a, chunk_at(a.chunks, ci), a.k);
}

// In every chunk-table kernel a workgroup (one wave) takes chunks
// blockIdx.x, blockIdx.x + gridDim.x, ...: the grid is capped so that
// work-items stay below 2^32 however long the table is.
//
// On large launches the 16-byte step keeps at most one wave per SIMD
// (waves_per_eu): with fewer concurrent streams the HBM sustains more of its
// peak on this mixed read/write stream.  Measured on MI355X with occupancy
// capped exactly by LDS reservations, one process, same buffers: 4 resident
// waves per CU beat 3 and 5-8 (7B shard 0.721 against 0.669 and
// 0.648-0.705; 70B 0.761 against 0.702 and 0.747-0.751).  Each wave still
// keeps its group's 14 (N = 8) to 22 (N = 16) 16-byte loads in flight.
//
// KC (extended step only): -1 flat rank order, 0 two-level with the group
// size at run time, > 0 two-level with that group size.
//
// W: resident waves per SIMD.  A launch of at most ZERO_SMALL_LAUNCH_CHUNKS
// chunks (a small shard, or one gradient bucket) runs two: with few
// workgroups per CU the launch's ramp and tail weigh more than the
// read/write mix.  Measured on MI355X, N = 8 bf16, chunks of 2048, one
// process, each launch on the next of enough buffer sets to keep the
// working set (over 2 GB) out of the 256 MB last-level cache, one wave
// against two: 2M-element shards 0.45 / 0.44-0.45, 4M 0.49-0.50 /
// 0.51-0.52, 8M 0.58 / 0.57-0.58, 16M 0.62-0.64 / 0.60, 32M 0.68-0.70 /
// 0.67, 64M 0.70-0.71 / 0.68; 7B gradient buckets of 4M params (2048
// chunks) 0.547 / 0.568, of 16M (8192 chunks) 0.662 / 0.652.  (Re-stepping
// one buffer set instead favours two waves up to 16M elements, 0.79 against
// 0.71 there, because part of the set then stays in that cache.)
//
// The allocation behind one wave per SIMD: with amdgpu_waves_per_eu(1, 1)
// the compiler declares 257 registers (.amdhsa_next_free_vgpr; 114 of them
// used), and 257 rounded to gfx950's granule of 8 fills more than half of
// a SIMD's 512, so only one such wave fits.  The two-wave instance declares
// 169 (176 allocated, two fit).  rocprofv3 reports the 257 as "132" (it
// counts granules of 4).
//
// The extended step picks its divisor path once per chunk, with a uniform
// branch around the whole chunk, instead of per element inside the unrolled
// loop.  On MI355X, bitwise equal, same buffers: 7B 0.696 -> 0.707 (K = 4),
// 0.648 -> 0.663 (K = 2, fold at run time), 0.697 -> 0.703 (three
// micro-batches, so divided); 70B 0.730 -> 0.740 (K = 8).
template <zero_dtype G, int NC, bool EXT, int KC = -1, int W = 1>
__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, W)))
void shard_step_kernel(StepArgs a)
{
    for (int64_t ci = blockIdx.x; ci < a.n_chunks; ci += gridDim.x) {
        if constexpr (EXT) {
            if (a.red.pow2)
                step_chunk<G, NC, EXT, KC, 1>(a, chunk_at(a.chunks, ci), a.k);
            else
                step_chunk<G, NC, EXT, KC, 2>(a, chunk_at(a.chunks, ci), a.k);
        } else {
            step_chunk<G, NC, EXT, KC>(a, chunk_at(a.chunks, ci), a.k);
        }
    }
}

// The fused steps with their constants in device memory: entry
// *a.sched_index of the table a.sched (formed on the host, as the
// launch-argument constants are).  A graph that captures this launch applies
// whichever step the index names when it replays.  An index outside the
// table leaves everything untouched.  L: the state layout (0: fp32 master,
// m, v; 1: fp32 master, bf16 m, v; 2: pure bf16 with compensation), each
// with the occupancy of its launch-argument kernel (SMALL: chosen per
// launch as for those kernels).
template <int L, zero_dtype G, int NC, bool SMALL>
constexpr int kSchedWaves = L == 0 ? (SMALL ? 2 : 1)
                                   : (L == 1 ? kM16Waves<G, NC, SMALL> : kKahanWaves);

template <int L, zero_dtype G, int NC, bool SMALL>
__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, kSchedWaves<L, G, NC, SMALL>)))
void shard_step_sched_kernel(StepArgs a)
{
    const int64_t t = *(const_i64 *)a.sched_index;
    if (t < 0 || t >= a.n_sched)
        return;
    const const_f64 *e = (const const_f64 *)(a.sched + t);
    StepScalars k;
    k.b1 = e[0]; k.c1 = e[1]; k.b2 = e[2]; k.c2 = e[3]; k.bc1 = e[4]; k.bc2 = e[5];
    k.eps = e[6]; k.lr = e[7]; k.dec = e[8]; k.wd = e[9];
    for (int64_t ci = blockIdx.x; ci < a.n_chunks; ci += gridDim.x) {
        if constexpr (L == 0)
            step_chunk<G, NC, false, -1>(a, chunk_at(a.chunks, ci), k);
        else if constexpr (L == 1)
            step_chunk_m16<G, NC, SMALL>(a, chunk_at(a.chunks, ci), k);
        else
            step_chunk_kahan<G, NC>(a, chunk_at(a.chunks, ci), k);
    }
}

// *index += 1 when 0 <= *index < n (one lane, a vector store).
__global__ __launch_bounds__(64) void step_index_advance_kernel(int64_t *index, int64_t n)
{
    if (threadIdx.x == 0) {
        const int64_t t = index[0];
        if (t >= 0 && t < n)
            index[0] = t + 1;
    }
}

// ---------------------------------------------------------------- unfused

template <zero_dtype G, int NC>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceArgs a)
{
    constexpr int VEC = Grad<G>::VEC;
    const int n = NC > 0 ? NC : a.red.n_ranks;
    const int64_t groups = a.n / VEC;
    for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * kBlock) {
        const int64_t i0 = g * VEC;
        double s[VEC];
        group_sum<G, NC>(s, a.parts, n, i0);
        F32x<VEC> out;
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            out[j] = finish_reduce<NC>(s[j], a.red);
        out.store(a.out + i0);
    }
    if (blockIdx.x == 0) {
        const int64_t i = groups * VEC + threadIdx.x;
        if (i < a.n)
            a.out[i] = finish_reduce<NC>(elem_sum<G>(a.parts, n, i), a.red);
    }
}

// One non-final micro-batch: acc = fp32((reset ? 0 : acc) + two-level sum).
// Launched like the step kernel: one wave per workgroup, at most one wave
// per SIMD; workgroup b walks spans b, b + gridDim.x, ... of kAccSpan
// consecutive elements.
constexpr int64_t kAccSpan = 2048;

template <zero_dtype G, int NC, int KC>
__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void accumulate_kernel(AccArgs a)
{
    constexpr int VEC = Grad<G>::VEC;
    constexpr int64_t GPS = kAccSpan / VEC;   // groups per span
    const int n = NC > 0 ? NC : a.red.n_ranks;
    const int64_t groups = a.n / VEC;
    for (int64_t sp = blockIdx.x; sp * GPS < groups; sp += gridDim.x) {
        const int64_t gend = (sp + 1) * GPS < groups ? (sp + 1) * GPS : groups;
        for (int64_t g = sp * GPS + threadIdx.x; g < gend; g += kStepBlock) {
            const int64_t i0 = g * VEC;
            F32x<VEC> acc;
            if (!a.reset)
                acc.load(a.acc + i0);
            double s[VEC];
            if constexpr (KC < 0)
                group_sum<G, NC>(s, a.parts, n, i0);
            else
                group_sum_two_level<G, NC, KC>(s, a.parts, n, a.red.group, i0);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                acc[j] = a.reset ? (float)s[j] : (float)((double)acc[j] + s[j]);
            acc.store(a.acc + i0);
        }
    }
    if (blockIdx.x == 0) {
        const int64_t i = groups * VEC + threadIdx.x;   // the last n % VEC elements
        if (i < a.n) {
            const double e = elem_sum_two_level<G>(a.parts, n, a.red.group, i);
            a.acc[i] = a.reset ? (float)e : (float)((double)a.acc[i] + e);
        }
    }
}

__global__ __launch_bounds__(kBlock) void adamw_kernel(AdamArgs a)
{
    const int64_t groups = a.n / 4;
    for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * kBlock) {
        const int64_t i0 = g * 4;
        F32x<4> gr, th, m, v;
        gr.load(a.g + i0);
        th.load(a.master + i0);
        m.load(a.m + i0);
        v.load(a.v + i0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            adamw(gr[j], th[j], m[j], v[j], a.k);
        th.store(a.master + i0);
        m.store(a.m + i0);
        v.store(a.v + i0);
    }
    if (blockIdx.x == 0) {
        const int64_t i = groups * 4 + threadIdx.x;
        if (i < a.n) {
            float th = a.master[i], m = a.m[i], v = a.v[i];
            adamw(a.g[i], th, m, v, a.k);
            a.master[i] = th;
            a.m[i] = m;
            a.v[i] = v;
        }
    }
}

__device__ __forceinline__ void gather_chunk(const GatherArgs &a, const zero_chunk &c)
{
    constexpr int VEC = 8;
    if (c.len <= 0 || c.shard_off < 0 || c.shard_off > a.shard_len - c.len)
        return;
    const int64_t lo = c.shard_off, hi = c.shard_off + c.len;
    const int64_t g0 = lo / VEC, g1 = (hi + VEC - 1) / VEC;
    const bool vec_ok = (((uintptr_t)c.dst - (uintptr_t)(2 * (lo - g0 * VEC))) % (2 * VEC)) == 0;
    ParamStore<VEC> ps(c.dst, lo, hi, vec_ok);
    for (int64_t g = g0 + threadIdx.x; g < g1; g += kStepBlock) {
        const int64_t i0 = g * VEC;
        uint16_t *d = c.dst + (i0 - lo);
        if (i0 >= lo && i0 + VEC <= hi) {
            F32x<VEC> th;
            th.load(a.master + i0);
            uint32_t h[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                h[j] = to_bf16(th[j]);
            ps.put(i0, h);
        } else {
            for (int j = 0; j < VEC; ++j) {
                const int64_t i = i0 + j;
                if (i >= lo && i < hi)
                    d[j] = (uint16_t)to_bf16(a.master[i]);
            }
        }
    }
}

__global__ __launch_bounds__(kStepBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gather_kernel(GatherArgs a)
{
    for (int64_t ci = blockIdx.x; ci < a.n_chunks; ci += gridDim.x)
        gather_chunk(a, chunk_at(a.chunks, ci));
}

// ---------------------------------------------------------------- launchers

static int grid_for(int64_t items)
{
    // Enough workgroups to fill 256 CUs many times over; the kernels stride.
    int64_t blocks = (items + kBlock - 1) / kBlock;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    return blocks < 1 ? 1 : (int)blocks;
}

// Chunk-table launches: one workgroup per chunk up to kMaxChunkGrid
// workgroups (kMaxChunkGrid * kStepBlock < 2^32 work-items).
constexpr int64_t kMaxChunkGrid = int64_t(1) << 22;

static unsigned chunk_grid(int64_t n_chunks)
{
    return (unsigned)(n_chunks < kMaxChunkGrid ? n_chunks : kMaxChunkGrid);
}

template <zero_dtype G, int W>
static hipError_t step_dispatch(const StepArgs &a, hipStream_t s)
{
    dim3 grid(chunk_grid(a.n_chunks)), block(kStepBlock);
    switch (a.red.n_ranks) {
    case 1: hipLaunchKernelGGL((shard_step_kernel<G, 1, false, -1, W>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((shard_step_kernel<G, 2, false, -1, W>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((shard_step_kernel<G, 4, false, -1, W>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((shard_step_kernel<G, 8, false, -1, W>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((shard_step_kernel<G, 16, false, -1, W>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((shard_step_kernel<G, 32, false, -1, W>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((shard_step_kernel<G, 64, false, -1, W>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((shard_step_kernel<G, 0, false, -1, W>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, zero_dtype gdt, hipStream_t s)
{
    const bool small = a.n_chunks <= ZERO_SMALL_LAUNCH_CHUNKS;
    if (gdt == ZERO_BF16)
        return small ? step_dispatch<ZERO_BF16, 2>(a, s) : step_dispatch<ZERO_BF16, 1>(a, s);
    return small ? step_dispatch<ZERO_FP32, 2>(a, s) : step_dispatch<ZERO_FP32, 1>(a, s);
}

template <int L, zero_dtype G, bool SMALL>
static hipError_t step_sched_dispatch(const StepArgs &a, hipStream_t s)
{
    dim3 grid(chunk_grid(a.n_chunks)), block(kStepBlock);
    switch (a.red.n_ranks) {
    case 1: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 1, SMALL>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 2, SMALL>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 4, SMALL>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 8, SMALL>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 16, SMALL>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 32, SMALL>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 64, SMALL>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((shard_step_sched_kernel<L, G, 0, SMALL>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int L>
static hipError_t step_sched_layout(const StepArgs &a, zero_dtype gdt, hipStream_t s)
{
    const bool small = a.n_chunks <= (L == 1 ? ZERO_SMALL_LAUNCH_CHUNKS_12B : ZERO_SMALL_LAUNCH_CHUNKS);
    if (gdt == ZERO_BF16)
        return small ? step_sched_dispatch<L, ZERO_BF16, true>(a, s)
                     : step_sched_dispatch<L, ZERO_BF16, false>(a, s);
    return small ? step_sched_dispatch<L, ZERO_FP32, true>(a, s)
                 : step_sched_dispatch<L, ZERO_FP32, false>(a, s);
}

hipError_t launch_step_sched(const StepArgs &a, zero_dtype gdt, StateLayout layout, hipStream_t s)
{
    switch (layout) {
    case StateLayout::Fp32: return step_sched_layout<0>(a, gdt, s);
    case StateLayout::Bf16Moments: return step_sched_layout<1>(a, gdt, s);
    case StateLayout::Kahan: return step_sched_layout<2>(a, gdt, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_index_advance(int64_t *index, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(step_index_advance_kernel, dim3(1), dim3(64), 0, s, index, n);
    return hipGetLastError();
}

// The extended step picks its fold at launch: groups of 1 or of all N ranks
// are the flat order (KC = -1); groups of 4 or 8 (GPUs per node) have
// compiled folds for N in {8, 16, 32, 64}; any other grouping runs the
// run-time fold (KC = 0).
template <zero_dtype G, int NC, int W>
static void launch_ex_n(const StepArgs &a, int K, dim3 grid, dim3 block, hipStream_t s)
{
    constexpr int K8 = (NC % 8 == 0 && NC > 8) ? 8 : 0;
    constexpr int K4 = (NC % 4 == 0 && NC > 4) ? 4 : 0;
    if (K == 1 || K == a.red.n_ranks)
        hipLaunchKernelGGL((shard_step_kernel<G, NC, true, -1, W>), grid, block, 0, s, a);
    else if (K8 == 8 && K == 8)
        hipLaunchKernelGGL((shard_step_kernel<G, NC, true, K8, W>), grid, block, 0, s, a);
    else if (K4 == 4 && K == 4)
        hipLaunchKernelGGL((shard_step_kernel<G, NC, true, K4, W>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((shard_step_kernel<G, NC, true, 0, W>), grid, block, 0, s, a);
}

template <zero_dtype G, int W>
static hipError_t step_ex_dispatch(const StepArgs &a, hipStream_t s)
{
    dim3 grid(chunk_grid(a.n_chunks)), block(kStepBlock);
    const int K = a.red.group;
    switch (a.red.n_ranks) {
    case 1: launch_ex_n<G, 1, W>(a, K, grid, block, s); break;
    case 2: launch_ex_n<G, 2, W>(a, K, grid, block, s); break;
    case 4: launch_ex_n<G, 4, W>(a, K, grid, block, s); break;
    case 8: launch_ex_n<G, 8, W>(a, K, grid, block, s); break;
    case 16: launch_ex_n<G, 16, W>(a, K, grid, block, s); break;
    case 32: launch_ex_n<G, 32, W>(a, K, grid, block, s); break;
    case 64: launch_ex_n<G, 64, W>(a, K, grid, block, s); break;
    default:
        if (K == 1 || K == a.red.n_ranks)
            hipLaunchKernelGGL((shard_step_kernel<G, 0, true, -1, W>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((shard_step_kernel<G, 0, true, 0, W>), grid, block, 0, s, a);
        break;
    }
    return hipGetLastError();
}

template <zero_dtype G, bool SMALL>
static hipError_t step_m16_dispatch(const StepArgs &a, hipStream_t s)
{
    dim3 grid(chunk_grid(a.n_chunks)), block(kStepBlock);
    switch (a.red.n_ranks) {
    case 1: hipLaunchKernelGGL((shard_step_m16_kernel<G, 1, SMALL>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((shard_step_m16_kernel<G, 2, SMALL>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((shard_step_m16_kernel<G, 4, SMALL>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((shard_step_m16_kernel<G, 8, SMALL>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((shard_step_m16_kernel<G, 16, SMALL>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((shard_step_m16_kernel<G, 32, SMALL>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((shard_step_m16_kernel<G, 64, SMALL>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((shard_step_m16_kernel<G, 0, SMALL>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <zero_dtype G>
static hipError_t step_kahan_dispatch(const StepArgs &a, hipStream_t s)
{
    const dim3 grid(chunk_grid(a.n_chunks)), block(kStepBlock);
    switch (a.red.n_ranks) {
    case 1: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 64>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((shard_step_kahan_kernel<G, 0>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_step_kahan(const StepArgs &a, zero_dtype gdt, hipStream_t s)
{
    return gdt == ZERO_BF16 ? step_kahan_dispatch<ZERO_BF16>(a, s) : step_kahan_dispatch<ZERO_FP32>(a, s);
}

hipError_t launch_step_m16(const StepArgs &a, zero_dtype gdt, hipStream_t s)
{
    const bool small = a.n_chunks <= ZERO_SMALL_LAUNCH_CHUNKS_12B;
    if (gdt == ZERO_BF16)
        return small ? step_m16_dispatch<ZERO_BF16, true>(a, s) : step_m16_dispatch<ZERO_BF16, false>(a, s);
    return small ? step_m16_dispatch<ZERO_FP32, true>(a, s) : step_m16_dispatch<ZERO_FP32, false>(a, s);
}

hipError_t launch_step_ex(const StepArgs &a, zero_dtype gdt, hipStream_t s)
{
    // the same occupancy rule as the 16-byte step (same structure); measured
    // with one accumulated micro-batch, N = 8 bf16, working set kept out of
    // the last-level cache as for the 16-byte step, one wave against two:
    // 2M-element shards 0.44 / 0.45, 4M 0.47 / 0.48, 8M 0.54-0.55 / 0.53-0.54,
    // 16M 0.60-0.64 / 0.63, 32M 0.65-0.68 / 0.66-0.67 of the bytes of the
    // step with its accumulator read; 256M 0.65-0.66 / 0.61
    const bool small = a.n_chunks <= ZERO_SMALL_LAUNCH_CHUNKS;
    if (gdt == ZERO_BF16)
        return small ? step_ex_dispatch<ZERO_BF16, 2>(a, s) : step_ex_dispatch<ZERO_BF16, 1>(a, s);
    return small ? step_ex_dispatch<ZERO_FP32, 2>(a, s) : step_ex_dispatch<ZERO_FP32, 1>(a, s);
}

template <zero_dtype G, int NC>
static void launch_acc_n(const AccArgs &a, int K, dim3 grid, dim3 block, hipStream_t s)
{
    if (K == 1 || K == a.red.n_ranks)
        hipLaunchKernelGGL((accumulate_kernel<G, NC, -1>), grid, block, 0, s, a);
    else if (NC % 8 == 0 && NC > 8 && K == 8)
        hipLaunchKernelGGL((accumulate_kernel<G, NC, (NC % 8 == 0 && NC > 8) ? 8 : 0>), grid, block, 0, s, a);
    else if (NC % 4 == 0 && NC > 4 && K == 4)
        hipLaunchKernelGGL((accumulate_kernel<G, NC, (NC % 4 == 0 && NC > 4) ? 4 : 0>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((accumulate_kernel<G, NC, 0>), grid, block, 0, s, a);
}

template <zero_dtype G>
static hipError_t accumulate_dispatch(const AccArgs &a, hipStream_t s)
{
    dim3 grid(chunk_grid((a.n + kAccSpan - 1) / kAccSpan)), block(kStepBlock);
    const int K = a.red.group;
    switch (a.red.n_ranks) {
    case 1: launch_acc_n<G, 1>(a, K, grid, block, s); break;
    case 2: launch_acc_n<G, 2>(a, K, grid, block, s); break;
    case 4: launch_acc_n<G, 4>(a, K, grid, block, s); break;
    case 8: launch_acc_n<G, 8>(a, K, grid, block, s); break;
    case 16: launch_acc_n<G, 16>(a, K, grid, block, s); break;
    case 32: launch_acc_n<G, 32>(a, K, grid, block, s); break;
    case 64: launch_acc_n<G, 64>(a, K, grid, block, s); break;
    default:
        if (K == 1 || K == a.red.n_ranks)
            hipLaunchKernelGGL((accumulate_kernel<G, 0, -1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((accumulate_kernel<G, 0, 0>), grid, block, 0, s, a);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_accumulate(const AccArgs &a, zero_dtype gdt, hipStream_t s)
{
    return gdt == ZERO_BF16 ? accumulate_dispatch<ZERO_BF16>(a, s)
                            : accumulate_dispatch<ZERO_FP32>(a, s);
}

template <zero_dtype G>
static hipError_t reduce_dispatch(const ReduceArgs &a, hipStream_t s)
{
    dim3 grid(grid_for(a.n / Grad<G>::VEC + 1)), block(kBlock);
    switch (a.red.n_ranks) {
    case 1: hipLaunchKernelGGL((reduce_kernel<G, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((reduce_kernel<G, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((reduce_kernel<G, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((reduce_kernel<G, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((reduce_kernel<G, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((reduce_kernel<G, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((reduce_kernel<G, 64>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((reduce_kernel<G, 0>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs &a, zero_dtype gdt, hipStream_t s)
{
    return gdt == ZERO_BF16 ? reduce_dispatch<ZERO_BF16>(a, s) : reduce_dispatch<ZERO_FP32>(a, s);
}

hipError_t launch_adamw(const AdamArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(a.n / 4 + 1)), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(gather_kernel, dim3(chunk_grid(a.n_chunks)), dim3(kStepBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace zs
