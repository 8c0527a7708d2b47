// Streaming-read probe: the rate at which this device reads a large buffer once with the same
// 16-byte non-temporal loads the attention kernels use. It is the achievable figure that the
// attention's GB/s sits next to (the 8 TB/s HBM peak is a datasheet number), and it computes
// nothing of the method.
#include "common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Each workgroup step reads kThreads * kUnroll consecutive 16-byte chunks (32 KiB), one 4 KiB
// run per load instruction, with kUnroll loads in flight per thread; workgroups stride over
// the buffer. The chunks are XOR-folded and the fold is stored only if it equals a value no
// real buffer folds to in practice, which keeps every load live without a store per thread.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4 *__restrict__ src, int64_t n,
                                                              uint32_t *__restrict__ sink) {
    constexpr int64_t kStep = static_cast<int64_t>(kThreads) * kUnroll;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kStep + threadIdx.x; base < n;
         base += static_cast<int64_t>(gridDim.x) * kStep) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kThreads;
            x[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
    }
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == 0x9e3779b9u) sink[0] = f;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream) {
    if (!src || !sink) return fail(PKV_EINVAL, "pkv_read_probe: NULL pointer");
    if (bytes % 16 || !aligned16(src) || !aligned16(sink))
        return fail(PKV_EINVAL, "pkv_read_probe: bytes and pointers must be multiples of 16");
    if (bytes == 0) return PKV_OK;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return fail(PKV_EHIP, "pkv_read_probe: cannot read the device's compute-unit count");
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t want = (n + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const int64_t cap = static_cast<int64_t>(cus) * 8;  // up to 8 workgroups of 4 waves per CU
    const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<const u32x4 *>(src), n,
                       static_cast<uint32_t *>(sink));
    return hip_status(hipGetLastError(), "pkv_read_probe launch");
}
