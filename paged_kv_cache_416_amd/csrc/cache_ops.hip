// Cache writes (reshape_and_cache) and copy-on-write block copies (copy_blocks).
//
// Both are byte moves: every thread moves 16-byte chunks with one vector load
// and one vector store, consecutive threads on consecutive chunks, so a wave
// touches 1 KiB of contiguous memory per instruction on each side.
#include "common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Each thread takes kWriteUnroll 16-byte chunks of (token, kv head) rows, one grid stride apart
// (consecutive lanes read consecutive chunks), with every load issued before the first store;
// chunk indices below 2^31 take 32-bit arithmetic. Token i, head h goes to block slot/B, row
// slot%B of head h (slide 11: a new token goes into the free slot of the sequence's last block).
constexpr int kWriteUnroll = 4;

template <typename I>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, int64_t key_stride_b, int64_t value_stride_b,
    char *__restrict__ k_cache, char *__restrict__ v_cache, int64_t num_slots, const int64_t *__restrict__ slots,
    int64_t total_chunks, int32_t chunks_per_row, int32_t num_kv_heads, int32_t block_size, int32_t block_shift) {
    const int32_t row_bytes = chunks_per_row * 16;
    const I per_token = static_cast<I>(chunks_per_row) * num_kv_heads;
    const I stride = static_cast<I>(gridDim.x) * kThreads;
    for (I i0 = static_cast<I>(blockIdx.x) * kThreads + threadIdx.x; i0 < total_chunks; i0 += stride * kWriteUnroll) {
        u32x4 kv[kWriteUnroll], vv[kWriteUnroll];
        int64_t slot[kWriteUnroll];
        int32_t h[kWriteUnroll], c[kWriteUnroll];
#pragma unroll
        for (int u = 0; u < kWriteUnroll; ++u) {
            const I i = i0 + u * stride;
            slot[u] = -1;
            if (i < total_chunks) {
                const I token = i / per_token;
                const int32_t rem = static_cast<int32_t>(i - token * per_token);
                h[u] = rem / chunks_per_row;
                c[u] = rem - h[u] * chunks_per_row;
                kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    key + static_cast<int64_t>(token) * key_stride_b + h[u] * row_bytes + c[u] * 16));
                vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    value + static_cast<int64_t>(token) * value_stride_b + h[u] * row_bytes + c[u] * 16));
                slot[u] = slots[token];
            }
        }
#pragma unroll
        for (int u = 0; u < kWriteUnroll; ++u) {
            // padding, a slot outside the pool, or a chunk past the end
            if (slot[u] < 0 || slot[u] >= num_slots) continue;
            const int64_t blk = block_shift >= 0 ? slot[u] >> block_shift : slot[u] / block_size;
            const int64_t off = slot[u] - blk * block_size;
            const int64_t dst = ((blk * num_kv_heads + h[u]) * block_size + off) * row_bytes + c[u] * 16;
            *reinterpret_cast<u32x4 *>(k_cache + dst) = kv[u];
            *reinterpret_cast<u32x4 *>(v_cache + dst) = vv[u];
        }
    }
}

constexpr int kMaxLayers = 16;
constexpr int kMaxPairs = 448;  // per launch: the pairs travel in the kernel arguments (about 3.8 KiB)
constexpr int kCopyUnroll = 4;

struct CopyArgs {
    char *cache[2 * kMaxLayers];  // K of layer l at 2l, V at 2l+1
    int32_t src[kMaxPairs];
    int32_t dst[kMaxPairs];
    int64_t block_bytes;
};

// grid = (slices, pairs, 2 * layers): workgroup (x, p, c) copies slice x of pair p in cache c.
// kCopyUnroll independent 16-byte loads per thread are issued before their stores: source and
// destination may alias as far as the compiler knows, so a plain loop would wait for each load
// before the next, one load in flight per thread. Loads and stores are non-temporal: nothing
// in the launch reads a byte twice.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const CopyArgs a) {
    char *base = a.cache[blockIdx.z];
    const char *src = base + a.src[blockIdx.y] * a.block_bytes;
    char *dst = base + a.dst[blockIdx.y] * a.block_bytes;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads * 16;
    for (int64_t off = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 16; off < a.block_bytes;
         off += step * kCopyUnroll) {
        u32x4 x[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (off + u * step < a.block_bytes)
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + off + u * step));
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (off + u * step < a.block_bytes)
                __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4 *>(dst + off + u * step));
    }
}

constexpr int kSwapCaches = 8;
constexpr int kSwapPairs = 224;
constexpr int kSwapUnroll = 4;

struct SwapArgs {
    const char *src[kSwapCaches];
    char *dst[kSwapCaches];
    int32_t from[kSwapPairs];
    int32_t to[kSwapPairs];
    int64_t block_bytes;
};

// grid = (slices, pairs, caches): workgroup (x, p, c) copies slice x of pair p in cache c, from
// one pool's cache to another's (either may be pinned host memory, reached over the host link:
// kSwapUnroll independent 16-byte loads per thread keep the link's long round trips overlapped).
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(const SwapArgs a) {
    const char *src = a.src[blockIdx.z] + a.from[blockIdx.y] * a.block_bytes;
    char *dst = a.dst[blockIdx.z] + a.to[blockIdx.y] * a.block_bytes;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads * 16;
    for (int64_t off = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 16; off < a.block_bytes;
         off += step * kSwapUnroll) {
        u32x4 x[kSwapUnroll];
#pragma unroll
        for (int u = 0; u < kSwapUnroll; ++u)
            if (off + u * step < a.block_bytes) x[u] = *reinterpret_cast<const u32x4 *>(src + off + u * step);
#pragma unroll
        for (int u = 0; u < kSwapUnroll; ++u)
            if (off + u * step < a.block_bytes) *reinterpret_cast<u32x4 *>(dst + off + u * step) = x[u];
    }
}

// The device-usable address of `p` if it is device memory or host memory registered with the
// runtime (pinned), with at least `bytes` of its allocation from p on; else an error code.
int reachable(const char *fn, const void *p, int64_t bytes, const char *what, int c, void **dev) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EINVAL, "%s: %s[%d] is neither device memory nor pinned host memory", fn, what, c);
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeHost && attr.type != hipMemoryTypeManaged)
        return fail(PKV_EINVAL, "%s: %s[%d] is neither device memory nor pinned host memory", fn, what, c);
    *dev = attr.type == hipMemoryTypeHost && attr.devicePointer ? attr.devicePointer : const_cast<void *>(p);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) == hipSuccess) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
        if (q < b || q - b + static_cast<uint64_t>(bytes) > size)
            return fail(PKV_EINVAL, "%s: %s[%d] holds %zu bytes from its address, the pool needs %lld", fn, what, c,
                        size - static_cast<size_t>(q - b), static_cast<long long>(bytes));
    } else {
        (void)hipGetLastError();
    }
    return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                               int64_t src_num_blocks, int64_t dst_num_blocks, int64_t block_bytes,
                               const int32_t *pairs, int32_t num_pairs, hipStream_t stream) {
    const char *fn = "pkv_swap_blocks";
    if (num_caches < 0 || num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || block_bytes <= 0)
        return fail(PKV_EINVAL, "%s: bad sizes", fn);
    if (num_pairs == 0 || num_caches == 0) return PKV_OK;
    if (!src_caches || !dst_caches || !pairs) return fail(PKV_EINVAL, "%s: NULL pointer", fn);
    if (block_bytes % 16) return fail(PKV_EINVAL, "%s: block_bytes must be a multiple of 16", fn);
    if (src_num_blocks > INT32_MAX || dst_num_blocks > INT32_MAX) return fail(PKV_EINVAL, "%s: pool too large", fn);
    {
        std::vector<char> is_dst(dst_num_blocks, 0);
        for (int32_t p = 0; p < num_pairs; ++p) {
            const int32_t s = pairs[2 * p], d = pairs[2 * p + 1];
            if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks)
                return fail(PKV_EINVAL, "%s: pair %d (%d, %d) outside the pools (%lld, %lld blocks)", fn, p, s, d,
                            (long long)src_num_blocks, (long long)dst_num_blocks);
            if (is_dst[d]) return fail(PKV_EINVAL, "%s: block %d is a destination twice", fn, d);
            is_dst[d] = 1;
        }
    }
    std::vector<const char *> src(num_caches);
    std::vector<char *> dst(num_caches);
    for (int32_t c = 0; c < num_caches; ++c) {
        if (!src_caches[c] || !dst_caches[c] || !aligned16(src_caches[c]) || !aligned16(dst_caches[c]))
            return fail(PKV_EINVAL, "%s: cache %d pointer NULL or not 16-byte aligned", fn, c);
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(src_caches[c]), d0 = reinterpret_cast<uintptr_t>(dst_caches[c]);
        const uint64_t sb = static_cast<uint64_t>(src_num_blocks * block_bytes), db = static_cast<uint64_t>(dst_num_blocks * block_bytes);
        if (s0 < d0 + db && d0 < s0 + sb)
            return fail(PKV_EINVAL, "%s: cache %d's source and destination overlap (use pkv_copy_blocks)", fn, c);
        void *ps = nullptr, *pd = nullptr;
        int rc = reachable(fn, src_caches[c], src_num_blocks * block_bytes, "src_caches", c, &ps);
        if (rc) return rc;
        rc = reachable(fn, dst_caches[c], dst_num_blocks * block_bytes, "dst_caches", c, &pd);
        if (rc) return rc;
        src[c] = static_cast<const char *>(ps);
        dst[c] = static_cast<char *>(pd);
    }
    const int64_t per_wg = static_cast<int64_t>(kThreads) * 16 * kSwapUnroll;  // 16 KiB per workgroup step
    const unsigned slices = static_cast<unsigned>(std::min<int64_t>(ceil_div(block_bytes, per_wg), 64));
    for (int32_t c0 = 0; c0 < num_caches; c0 += kSwapCaches) {
        const int32_t nc = std::min(kSwapCaches, num_caches - c0);
        for (int32_t p0 = 0; p0 < num_pairs; p0 += kSwapPairs) {
            const int32_t np = std::min(kSwapPairs, num_pairs - p0);
            SwapArgs a{};
            for (int32_t c = 0; c < nc; ++c) {
                a.src[c] = src[c0 + c];
                a.dst[c] = dst[c0 + c];
            }
            for (int32_t p = 0; p < np; ++p) {
                a.from[p] = pairs[2 * (p0 + p)];
                a.to[p] = pairs[2 * (p0 + p) + 1];
            }
            a.block_bytes = block_bytes;
            hipLaunchKernelGGL(swap_blocks_kernel, dim3(slices, np, nc), dim3(kThreads), 0, stream, a);
            int rc = hip_status(hipGetLastError(), "pkv_swap_blocks launch");
            if (rc) return rc;
        }
    }
    return PKV_OK;
}

extern "C" int pkv_reshape_and_cache(const void *key, const void *value, int64_t key_stride, int64_t value_stride,
                                     void *k_cache, void *v_cache, int64_t num_blocks, const int64_t *slot_mapping,
                                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t dtype, hipStream_t stream) {
    if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "pkv_reshape_and_cache: bad dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "pkv_reshape_and_cache: bad sizes");
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_EINVAL, "pkv_reshape_and_cache: NULL pointer");
    const int eb = elt_bytes(dtype);
    const int64_t row_bytes = static_cast<int64_t>(head_dim) * eb;
    if (row_bytes % 16) return fail(PKV_EINVAL, "pkv_reshape_and_cache: head_dim*elt must be a multiple of 16 bytes");
    if (key_stride < static_cast<int64_t>(num_kv_heads) * head_dim ||
        value_stride < static_cast<int64_t>(num_kv_heads) * head_dim)
        return fail(PKV_EINVAL, "pkv_reshape_and_cache: token stride smaller than num_kv_heads*head_dim");
    if ((key_stride * eb) % 16 || (value_stride * eb) % 16 || !aligned16(key) || !aligned16(value) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_EINVAL, "pkv_reshape_and_cache: pointers and strides must be 16-byte aligned");
    if (debug_validate()) {
        const int rc = validate_slots("pkv_reshape_and_cache", slot_mapping, num_tokens, num_blocks * block_size, stream);
        if (rc) return rc;
    }
    const int32_t cpr = static_cast<int32_t>(row_bytes / 16);
    const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * cpr;
    const int64_t want = ceil_div(total, static_cast<int64_t>(kThreads) * kWriteUnroll);
    const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
    const int32_t shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz(block_size) : -1;
    // 32-bit chunk indices while every index the grid forms stays below 2^31
    if (total + static_cast<int64_t>(grid) * kThreads * kWriteUnroll < (int64_t(1) << 31))
        hipLaunchKernelGGL(reshape_and_cache_kernel<int32_t>, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const char *>(key), static_cast<const char *>(value), key_stride * eb,
                           value_stride * eb, static_cast<char *>(k_cache), static_cast<char *>(v_cache),
                           num_blocks * block_size, slot_mapping, total, cpr, num_kv_heads, block_size, shift);
    else
        hipLaunchKernelGGL(reshape_and_cache_kernel<int64_t>, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const char *>(key), static_cast<const char *>(value), key_stride * eb,
                           value_stride * eb, static_cast<char *>(k_cache), static_cast<char *>(v_cache),
                           num_blocks * block_size, slot_mapping, total, cpr, num_kv_heads, block_size, shift);
    return hip_status(hipGetLastError(), "pkv_reshape_and_cache launch");
}

extern "C" int pkv_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers, int64_t num_blocks,
                               int64_t block_bytes, const int32_t *pairs, int32_t num_pairs, hipStream_t stream) {
    if (num_pairs < 0 || num_layers < 0 || num_blocks <= 0 || block_bytes <= 0)
        return fail(PKV_EINVAL, "pkv_copy_blocks: bad sizes");
    if (num_pairs == 0 || num_layers == 0) return PKV_OK;
    if (!k_caches || !v_caches || !pairs) return fail(PKV_EINVAL, "pkv_copy_blocks: NULL pointer");
    if (block_bytes % 16) return fail(PKV_EINVAL, "pkv_copy_blocks: block_bytes must be a multiple of 16");
    for (int32_t l = 0; l < num_layers; ++l)
        if (!k_caches[l] || !v_caches[l] || !aligned16(k_caches[l]) || !aligned16(v_caches[l]))
            return fail(PKV_EINVAL, "pkv_copy_blocks: layer %d cache pointer NULL or not 16-byte aligned", l);
    // Host check: in range, distinct destinations, no destination is also a source. Then
    // the copies are independent and may run in any order.
    {
        std::vector<char> is_src(num_blocks, 0), is_dst(num_blocks, 0);
        for (int32_t p = 0; p < num_pairs; ++p) {
            const int32_t s = pairs[2 * p], d = pairs[2 * p + 1];
            if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
                return fail(PKV_EINVAL, "pkv_copy_blocks: pair %d (%d, %d) outside [0, %lld)", p, s, d,
                            (long long)num_blocks);
            if (is_dst[d]) return fail(PKV_EINVAL, "pkv_copy_blocks: block %d is a destination twice", d);
            is_dst[d] = 1;
            is_src[s] = 1;
        }
        for (int32_t p = 0; p < num_pairs; ++p)
            if (is_src[pairs[2 * p + 1]])
                return fail(PKV_EINVAL, "pkv_copy_blocks: block %d is both a source and a destination",
                            pairs[2 * p + 1]);
    }
    const int64_t per_wg = static_cast<int64_t>(kThreads) * 16 * 4;  // ~16 KiB per workgroup
    const unsigned slices = static_cast<unsigned>(std::min<int64_t>(ceil_div(block_bytes, per_wg), 64));
    for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayers) {
        const int32_t nl = std::min(kMaxLayers, num_layers - l0);
        for (int32_t p0 = 0; p0 < num_pairs; p0 += kMaxPairs) {
            const int32_t np = std::min(kMaxPairs, num_pairs - p0);
            CopyArgs a{};
            for (int32_t l = 0; l < nl; ++l) {
                a.cache[2 * l] = static_cast<char *>(k_caches[l0 + l]);
                a.cache[2 * l + 1] = static_cast<char *>(v_caches[l0 + l]);
            }
            for (int32_t p = 0; p < np; ++p) {
                a.src[p] = pairs[2 * (p0 + p)];
                a.dst[p] = pairs[2 * (p0 + p) + 1];
            }
            a.block_bytes = block_bytes;
            hipLaunchKernelGGL(copy_blocks_kernel, dim3(slices, np, 2 * nl), dim3(kThreads), 0, stream, a);
            int rc = hip_status(hipGetLastError(), "pkv_copy_blocks launch");
            if (rc) return rc;
        }
    }
    return PKV_OK;
}
