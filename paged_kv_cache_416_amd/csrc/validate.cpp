// Debug validation of the device-side contract (PKV_DEBUG_VALIDATE=1): the kernels never fault
// on bad lengths, table entries or slots, but their result is then unspecified. With the
// variable set, the host entry points copy those arrays to the host first (synchronising the
// caller's stream) and reject a violation with PKV_EINVAL before anything is launched.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"

namespace pkv {

bool debug_validate() {
    const char *v = std::getenv("PKV_DEBUG_VALIDATE");
    return v && *v && std::strcmp(v, "0") != 0;
}

namespace {

// Copies n elements of a device array to the host after the stream's earlier work.
template <class T>
int fetch(const char *fn, const char *what, const T *dev, size_t n, hipStream_t stream, std::vector<T> &host) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, dev) != hipSuccess || attr.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(PKV_EINVAL, "%s: %s is not device memory (PKV_DEBUG_VALIDATE)", fn, what);
    }
    host.resize(n);
    if (n == 0) return PKV_OK;
    int rc = hip_status(hipStreamSynchronize(stream), "PKV_DEBUG_VALIDATE stream synchronize");
    if (rc) return rc;
    return hip_status(hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost), "PKV_DEBUG_VALIDATE copy");
}

}  // namespace

int validate_device_array(const char *fn, const char *what, const void *dev) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, dev) != hipSuccess || attr.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(PKV_EINVAL, "%s: %s is not device memory (PKV_DEBUG_VALIDATE)", fn, what);
    }
    return PKV_OK;
}

int validate_step_slots(const char *fn, const int64_t *slot_mapping, const int32_t *context_lens,
                        const int32_t *block_tables, int32_t num_seqs, int32_t max_blocks, int32_t block_size,
                        hipStream_t stream) {
    std::vector<int64_t> slots;
    std::vector<int32_t> ctx, tab;
    int rc = fetch(fn, "slot_mapping", slot_mapping, static_cast<size_t>(num_seqs), stream, slots);
    if (!rc) rc = fetch(fn, "context_lens", context_lens, static_cast<size_t>(num_seqs), stream, ctx);
    if (!rc) rc = fetch(fn, "block_tables", block_tables, static_cast<size_t>(num_seqs) * max_blocks, stream, tab);
    if (rc) return rc;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (slots[s] < 0) continue;
        const int32_t t = ctx[s] - 1;  // the new token's position (lengths already checked)
        const int64_t want = t < 0 ? -1
                                   : static_cast<int64_t>(tab[static_cast<size_t>(s) * max_blocks + t / block_size]) *
                                             block_size + t % block_size;
        if (slots[s] != want)
            return fail(PKV_EINVAL,
                        "%s: slot_mapping[%d] = %lld is not the slot of position context_lens[%d] - 1 (%lld) "
                        "(PKV_DEBUG_VALIDATE)", fn, s, static_cast<long long>(slots[s]), s, static_cast<long long>(want));
    }
    return PKV_OK;
}

int validate_attention(const char *fn, const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                       const int32_t *block_tables, int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                       int32_t lmax, hipStream_t stream) {
    std::vector<int32_t> ctx, tab;
    int rc = fetch(fn, "context_lens", context_lens, static_cast<size_t>(num_seqs), stream, ctx);
    if (rc) return rc;
    if (block_tables) {
        rc = fetch(fn, "block_tables", block_tables, static_cast<size_t>(num_seqs) * max_blocks, stream, tab);
        if (rc) return rc;
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t c = ctx[s];
        if (c < 0 || c > max_context_len)
            return fail(PKV_EINVAL, "%s: context_lens[%d] = %d outside [0, max_context_len = %d] (PKV_DEBUG_VALIDATE)",
                        fn, s, c, max_context_len);
        if (!block_tables) {
            if (c > lmax)
                return fail(PKV_EINVAL, "%s: context_lens[%d] = %d exceeds lmax %d (PKV_DEBUG_VALIDATE)", fn, s, c,
                            lmax);
            continue;
        }
        const int64_t used = ceil_div(c, block_size);
        if (used > max_blocks)
            return fail(PKV_EINVAL, "%s: context_lens[%d] = %d needs %lld blocks, the table holds %d (PKV_DEBUG_VALIDATE)",
                        fn, s, c, static_cast<long long>(used), max_blocks);
        for (int64_t j = 0; j < used; ++j) {
            const int32_t b = tab[static_cast<size_t>(s) * max_blocks + j];
            if (b < 0 || b >= num_blocks)
                return fail(PKV_EINVAL, "%s: block_tables[%d][%lld] = %d outside [0, %lld) (PKV_DEBUG_VALIDATE)", fn, s,
                            static_cast<long long>(j), b, static_cast<long long>(num_blocks));
        }
    }
    return PKV_OK;
}

int validate_query_start(const char *fn, const int32_t *query_start, const int32_t *context_lens, int32_t num_seqs,
                         int32_t num_tokens, int32_t max_query_len, hipStream_t stream) {
    std::vector<int32_t> qs, ctx;
    int rc = fetch(fn, "query_start", query_start, static_cast<size_t>(num_seqs) + 1, stream, qs);
    if (rc) return rc;
    rc = fetch(fn, "context_lens", context_lens, static_cast<size_t>(num_seqs), stream, ctx);
    if (rc) return rc;
    if (qs[0] != 0) return fail(PKV_EINVAL, "%s: query_start[0] = %d, not 0 (PKV_DEBUG_VALIDATE)", fn, qs[0]);
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = qs[s + 1] - qs[s];
        if (n < 0 || n > max_query_len || n > ctx[s])
            return fail(PKV_EINVAL,
                        "%s: sequence %d has %d queries (max_query_len %d, context %d) (PKV_DEBUG_VALIDATE)", fn, s, n,
                        max_query_len, ctx[s]);
    }
    if (qs[num_seqs] > num_tokens)
        return fail(PKV_EINVAL, "%s: query_start[%d] = %d exceeds num_tokens %d (PKV_DEBUG_VALIDATE)", fn, num_seqs,
                    qs[num_seqs], num_tokens);
    return PKV_OK;
}

int validate_slots(const char *fn, const int64_t *slot_mapping, int32_t num_tokens, int64_t num_slots,
                   hipStream_t stream) {
    std::vector<int64_t> slots;
    int rc = fetch(fn, "slot_mapping", slot_mapping, static_cast<size_t>(num_tokens), stream, slots);
    if (rc) return rc;
    std::vector<int64_t> used;
    used.reserve(slots.size());
    for (int32_t i = 0; i < num_tokens; ++i) {
        if (slots[i] >= num_slots)
            return fail(PKV_EINVAL, "%s: slot_mapping[%d] = %lld outside the pool's %lld slots (PKV_DEBUG_VALIDATE)", fn,
                        i, static_cast<long long>(slots[i]), static_cast<long long>(num_slots));
        if (slots[i] >= 0) used.push_back(slots[i]);
    }
    std::sort(used.begin(), used.end());
    const auto dup = std::adjacent_find(used.begin(), used.end());
    if (dup != used.end())
        return fail(PKV_EINVAL, "%s: slot %lld appears twice in slot_mapping (PKV_DEBUG_VALIDATE)", fn,
                    static_cast<long long>(*dup));
    return PKV_OK;
}

}  // namespace pkv
