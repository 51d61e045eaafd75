// Shard geometry and the chunk table (zero_build_chunks): host code only,
// no device calls.  Kept in its own file because the table's cuts (chunk
// lengths, tensor boundaries) decide the step kernels' memory traffic
// together with the kernels themselves.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "zero_internal.h"

extern "C" {

int zero_build_chunks(const int64_t *numels, int n_tensors, int n_ranks, int rank,
                      uint16_t *const *tensor_dst, uint16_t *slot_dst, int64_t max_chunk,
                      zero_chunk *out, int64_t cap, int64_t *n_out, int64_t *shard_len_out)
{
    if (!numels || n_tensors < 1 || n_ranks < 1 || rank < 0 || rank >= n_ranks)
        return ZERO_ERR_INVALID;
    if (max_chunk <= 0 || max_chunk % 64 != 0 || max_chunk > (int64_t(1) << 24))
        return ZERO_ERR_INVALID;
    if (!tensor_dst && !slot_dst)
        return ZERO_ERR_INVALID;
    if (out && cap < 0)
        return ZERO_ERR_INVALID;
    int64_t total = 0;
    for (int t = 0; t < n_tensors; ++t) {
        if (numels[t] < 0 || numels[t] > ZERO_MAX_LEN - total ||
            (tensor_dst && numels[t] > 0 && !tensor_dst[t]))
            return ZERO_ERR_INVALID;
        total += numels[t];
    }
    const int64_t S = (total + n_ranks - 1) / n_ranks;
    int64_t lo = (int64_t)rank * S, hi = lo + S;
    if (lo > total) lo = total;
    if (hi > total) hi = total;

    int64_t count = 0;
    auto emit = [&](int64_t soff, int64_t len, int t, int64_t toff, uint16_t *dst) {
        if (out && count < cap) {
            zero_chunk &c = out[count];
            c.shard_off = soff;
            c.len = (int32_t)len;
            c.tensor_id = t;
            c.tensor_off = toff;
            c.dst = dst;
        }
        ++count;
    };
    if (tensor_dst) {
        // One piece per tensor that meets [lo, hi), each cut at multiples
        // of max_chunk in shard coordinates.
        int64_t a = 0;
        for (int t = 0; t < n_tensors && a < hi; ++t) {
            const int64_t b = a + numels[t];
            for (int64_t x = a > lo ? a : lo, y = b < hi ? b : hi; x < y;) {
                const int64_t soff = x - lo;
                int64_t end = lo + (soff / max_chunk + 1) * max_chunk;
                if (end > y) end = y;
                emit(soff, end - x, t, x - a, tensor_dst[t] + (x - a));
                x = end;
            }
            a = b;
        }
    } else {
        // Contiguous slot: cut only at multiples of max_chunk; record the
        // tensor holding each chunk's first element.
        int t = 0;
        int64_t a = 0;
        for (int64_t soff = 0; soff < hi - lo; soff += max_chunk) {
            const int64_t x = lo + soff;
            while (a + numels[t] <= x) {
                a += numels[t];
                ++t;
            }
            const int64_t len = (hi - x) < max_chunk ? (hi - x) : max_chunk;
            emit(soff, len, t, x - a, slot_dst + soff);
        }
    }
    if (n_out)
        *n_out = count;
    if (shard_len_out)
        *shard_len_out = S;
    if (out && count > cap)
        return ZERO_ERR_CAPACITY;
    return ZERO_OK;
}

int zero_check_chunks(const zero_chunk *chunks, int64_t n_chunks, int64_t shard_len,
                      const void *const *arrays, const int64_t *array_bytes, int n_arrays)
{
    if (n_chunks < 0 || n_chunks > INT32_MAX || (n_chunks > 0 && !chunks) || shard_len < 0 ||
        shard_len > ZERO_MAX_LEN || n_arrays < 0 || (n_arrays > 0 && (!arrays || !array_bytes)))
        return ZERO_ERR_INVALID;
    for (int i = 0; i < n_arrays; ++i)
        if (array_bytes[i] < 0 || array_bytes[i] > ZERO_MAX_LEN || (!arrays[i] && array_bytes[i] > 0))
            return ZERO_ERR_INVALID;
    typedef std::pair<uintptr_t, uintptr_t> Range;   // [first, second)
    std::vector<Range> elems, dsts;
    elems.reserve((size_t)n_chunks);
    dsts.reserve((size_t)n_chunks);
    for (int64_t i = 0; i < n_chunks; ++i) {
        const zero_chunk &c = chunks[i];
        if (c.len < 1 || c.shard_off < 0 || c.shard_off > shard_len - c.len || !c.dst)
            return ZERO_ERR_INVALID;
        const uintptr_t d = (uintptr_t)c.dst, nb = 2 * (uintptr_t)c.len;
        if (d > UINTPTR_MAX - nb)
            return ZERO_ERR_INVALID;
        elems.emplace_back((uintptr_t)c.shard_off, (uintptr_t)(c.shard_off + c.len));
        dsts.emplace_back(d, d + nb);
    }
    // every shard element in at most one chunk
    std::sort(elems.begin(), elems.end());
    for (size_t i = 1; i < elems.size(); ++i)
        if (elems[i].first < elems[i - 1].second)
            return ZERO_ERR_INVALID;
    // no two chunks write the same parameter byte
    std::sort(dsts.begin(), dsts.end());
    for (size_t i = 1; i < dsts.size(); ++i)
        if (dsts[i].first < dsts[i - 1].second)
            return ZERO_ERR_ALIAS;
    // no destination inside an array the step reads or writes: merge the
    // arrays into disjoint sorted ranges, then look each destination up
    std::vector<Range> arr;
    for (int i = 0; i < n_arrays; ++i) {
        const uintptr_t a = (uintptr_t)arrays[i], nb = (uintptr_t)array_bytes[i];
        if (nb == 0)
            continue;
        if (a > UINTPTR_MAX - nb)
            return ZERO_ERR_INVALID;
        arr.emplace_back(a, a + nb);
    }
    std::sort(arr.begin(), arr.end());
    std::vector<Range> merged;
    for (const Range &r : arr) {
        if (!merged.empty() && r.first <= merged.back().second)
            merged.back().second = std::max(merged.back().second, r.second);
        else
            merged.push_back(r);
    }
    for (const Range &d : dsts) {
        // first merged range ending after d starts
        auto it = std::upper_bound(merged.begin(), merged.end(), d.first,
                                   [](uintptr_t x, const Range &r) { return x < r.second; });
        if (it != merged.end() && it->first < d.second)
            return ZERO_ERR_ALIAS;
    }
    return ZERO_OK;
}

}  // extern "C"
