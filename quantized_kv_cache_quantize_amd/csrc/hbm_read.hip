// Measurement helper: one plain read of a device buffer, for calibrating the
// HBM bandwidth a read-only kernel reaches on this GPU, next to which the
// attention kernel's bytes per second are read. Grid-stride 16-byte loads
// from 2048 workgroups of 256 threads, one load per thread and round, so the
// whole grid sweeps the buffer front to back (measured: 6.46 TB/s over 1 GiB;
// four loads per thread 8 MB apart reach 5.3 TB/s); every loaded word enters
// an XOR, and a thread stores its XOR only when it equals `key`, a run-time
// value, so no load can be dropped.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int RB = 256;         // threads per workgroup
constexpr unsigned RG = 2048;   // workgroups

__global__ __launch_bounds__(RB) void hbm_read_kernel(const uint4 *__restrict__ p, int64_t n, uint32_t key,
                                                      uint32_t *sink)
{
    const int64_t stride = (int64_t)RG * RB;
    uint32_t x = 0;
    for (int64_t i = (int64_t)blockIdx.x * RB + threadIdx.x; i < n; i += stride) {
        const uint4 v = p[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (x == key)
        *sink = x;
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_hbm_read(const void *buf, int64_t bytes, uint32_t key, uint32_t *sink, void *stream)
{
    if (bytes == 0)
        return KVQ_OK;
    if (buf == nullptr || sink == nullptr)
        return KVQ_E_NULL;
    if (bytes < 0 || bytes % 16 != 0)
        return KVQ_E_SHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return KVQ_E_ALIGN;
    hipLaunchKernelGGL(kvq::hbm_read_kernel, dim3(kvq::RG), dim3(kvq::RB), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint4 *>(buf), bytes / 16, key, sink);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_E_LAUNCH;
}
